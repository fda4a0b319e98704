// Device side of greedy tree acceptance (the target's choice per node, then
// the longest agreeing root-to-node path), shared by the acceptance launch and
// the fused verification launch (attention and acceptance in one grid).
//
// Acceptance rule: gist.science lay summary of "JetFlow ..." and the qxai.app
// commentary (drafted tokens are kept up to the first disagreement); over a
// tree the accepted path is the longest one on which every node agrees.
#pragma once
#include "jf_common.h"

namespace jf {

constexpr int kAcceptThreads = 256;
constexpr int kNoIndex = 0x7fffffff;

struct Best {
    float v;
    int i;
};

// Strict order: larger value first, then smaller index. NaN never enters.
__device__ __forceinline__ bool better(float v, int i, const Best& b) {
    return v > b.v || (v == b.v && i < b.i);
}

__device__ __forceinline__ void offer(Best& b, float v, int i) {
    if (!__builtin_isnan(v) && better(v, i, b)) {
        b.v = v;
        b.i = i;
    }
}

__device__ __forceinline__ Best merge(Best a, Best b) { return better(b.v, b.i, a) ? b : a; }

// (value, index) -> 64-bit key whose unsigned order is `better`'s order:
// high word = the float's bits mapped to an order-preserving unsigned (with -0
// read as +0), low word = ~index. An empty winner (no non-NaN value) is 0,
// below every real key.
__device__ __forceinline__ uint64_t best_key(Best b) {
    if (b.i == kNoIndex) return 0ull;
    uint32_t u = __float_as_uint(b.v == 0.f ? 0.f : b.v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint64_t)(~(uint32_t)b.i);
}

__device__ __forceinline__ int key_index(uint64_t k) { return k == 0ull ? 0 : (int)(~(uint32_t)k); }

static __device__ Best block_best(Best b, Best* scratch) {
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        Best o;
        o.v = __shfl_xor(b.v, off);
        o.i = __shfl_xor(b.i, off);
        b = merge(b, o);
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) scratch[w] = b;
    __syncthreads();
    Best r = scratch[0];
    #pragma unroll
    for (int k = 1; k < kAcceptThreads / kWave; ++k) r = merge(r, scratch[k]);
    __syncthreads();
    return r;
}

// One sequence's walk, run by a whole 256-thread workgroup (N <= 256); thread
// u holds node u's parent, draft token and ancestor words; nxt[] is the
// target's token after each node of the sequence (LDS or global).
//   mism bit u: u > 0 and draft[u] != nxt[parent[u]]
//   node v agrees along its path iff (anc[v] & mism) == 0
//   end node = the agreeing node with most path nodes, smallest index on ties
static __device__ __forceinline__ void walk_sequence(int b, int N, int p_u, int d_u, const uint64_t a_u[kAncWords],
                              const int32_t* nxt, int32_t* __restrict__ accept_len,
                              int32_t* __restrict__ accepted_nodes, int32_t* __restrict__ bonus) {
    __shared__ uint64_t mism[kAncWords];
    __shared__ uint64_t end_set[kAncWords];
    __shared__ int keys[kAcceptThreads / kWave];
    const int u = threadIdx.x;
    const int lane = u & 63, w = u >> 6;
    const size_t base = (size_t)b * N;

    bool bad = false;
    if (u > 0 && u < N) {
        const int p = (p_u < 0) ? 0 : (p_u >= N ? N - 1 : p_u);   // memory safety on broken trees
        bad = d_u != nxt[p];
    }
    const uint64_t ballot = __ballot(bad);
    if (lane == 0) mism[w] = ballot;
    __syncthreads();

    // key = (path nodes << 16) | (0xffff - node) for agreeing nodes, else 0
    unsigned key = 0;
    if (u < N) {
        bool ok = true;
        int cnt = 0;
        #pragma unroll
        for (int k = 0; k < kAncWords; ++k) {
            ok = ok && ((a_u[k] & mism[k]) == 0);
            cnt += __popcll(a_u[k]);
        }
        if (ok && cnt > 0) key = ((unsigned)cnt << 16) | (0xffffu - (unsigned)u);
    }
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const unsigned o = __shfl_xor(key, off);
        key = o > key ? o : key;
    }
    if (lane == 0) keys[w] = (int)key;
    __syncthreads();
    unsigned best = 0;
    #pragma unroll
    for (int k = 0; k < kAcceptThreads / kWave; ++k) best = (unsigned)keys[k] > best ? (unsigned)keys[k] : best;
    int v_end = 0, nodes = 1;
    if (best != 0) {
        v_end = (int)(0xffffu - (best & 0xffffu));
        nodes = (int)(best >> 16);
    }
    if (v_end >= N) v_end = 0;
    if (nodes > N) nodes = N;
    if (u == v_end) {
        #pragma unroll
        for (int k = 0; k < kAncWords; ++k) end_set[k] = a_u[k];
    }
    __syncthreads();
    if (u < N) {
        // nodes of the end node's path, in index order = root-to-end order
        const int word = u >> 6, bit = u & 63;
        const uint64_t ws = end_set[word];
        if ((ws >> bit) & 1ull) {
            int pos = __popcll(ws & ((bit ? (~0ull >> (64 - bit)) : 0ull)));
            for (int k = 0; k < word; ++k) pos += __popcll(end_set[k]);
            if (pos < N) accepted_nodes[base + pos] = u;
        }
        if (u >= nodes) accepted_nodes[base + u] = -1;
    }
    if (u == 0) {
        accept_len[b] = nodes - 1;
        bonus[b] = nxt[v_end];
    }
}

struct NodeIn {
    int p, d;
    uint64_t a[kAncWords];
};

// Thread u's node. The loads are unconditional (threads u >= N read node N - 1,
// whose values they never use: every consumer looks only at u < N), so the
// compiler counts them exactly and a later wait for them does not also wait for
// the loads issued after them.
__device__ __forceinline__ NodeIn load_node(int b, int N, const int32_t* __restrict__ parent,
                                            const int32_t* __restrict__ draft, const uint64_t* __restrict__ anc) {
    NodeIn n;
    const size_t r = (size_t)b * N + min((int)threadIdx.x, N - 1);
    n.p = parent[r];
    n.d = draft[r];
    #pragma unroll
    for (int k = 0; k < kAncWords; ++k) n.a[k] = anc ? anc[r * kAncWords + k] : 0ull;
    return n;
}


// Chunks of at most this many 16-byte vectors are scanned from registers.
constexpr int kRegChunkVecs = 16 * kAcceptThreads;

// Position (0 .. EPV-1) of the first value equal to m in a vector, or EPV.
template <typename T>
__device__ __forceinline__ int vec_first(const u32x4 r, float m) {
    constexpr int EPV = 16 / (int)sizeof(T);
    int k = EPV;
    #pragma unroll
    for (int e = EPV - 1; e >= 0; --e) k = (vec_val<T>(r, e) == m) ? e : k;
    return k;
}

// Exact, value by value (a vector that holds a signalling NaN).
template <typename T>
__device__ __forceinline__ void vec_offer(const u32x4 r, int i0, Best& b) {
    constexpr int EPV = 16 / (int)sizeof(T);
    #pragma unroll
    for (int e = 0; e < EPV; ++e) offer(b, vec_val<T>(r, e), i0 + e);
}

// The winner (largest value, smallest index; NaN never wins) of logits
// row[lo, hi), over the workgroup. Every thread returns it. 16-byte
// non-temporal loads, thread t taking vectors t, t + 256, t + 512, ...: the
// row must start on a 16-byte boundary and hi - lo must be a multiple of the
// values per vector (the acceptance plan keeps both for aligned rows). With set_n > 0, wave 0 builds the
// ancestor sets of a tree of set_n <= 64 nodes from the parent entry set_p of
// its lane (tree_set_wave) while the first loads are in flight, into set_out.
//  * Up to KR vectors per thread (the acceptance plan's chunks when rows are
//    few): every load is issued at once and the chunk stays in registers; each
//    thread takes the max of its values with v_max3 (branch-free), the
//    workgroup reduces it, and only a thread holding that max searches its
//    vectors for the first position. A signalling NaN anywhere (the only way a
//    v_max3 result is NaN) sends the chunk through the exact per-value path.
//  * Longer chunks: batches of KB vectors, two in flight; a vector is searched
//    only when its max beats the thread's best so far (indices rise within a
//    thread, so a strictly larger value is the only replacement), value by
//    value when it holds a signalling NaN.
// PATHS: 0 either path, chosen from the chunk length; 1 the in-register path
// only (the caller guarantees nvec <= KR * 256); 2 the batched path only.
template <typename T, int PATHS = 0>
__device__ __forceinline__ Best chunk_best(const T* __restrict__ row, int lo, int hi, Best* scratch, int set_p,
                                           int set_n, uint64_t& set_out) {
    __shared__ float s_max[kAcceptThreads / kWave];
    __shared__ int s_idx[kAcceptThreads / kWave];
    constexpr int EPV = 16 / (int)sizeof(T);
    constexpr int KR = kRegChunkVecs / kAcceptThreads;
    constexpr int KB = 4;
    constexpr int TH = kAcceptThreads;
    const float NEG = -__builtin_inff();
    const int nvec = (hi - lo) / EPV;
    const u32x4* vp = reinterpret_cast<const u32x4*>(row + lo);
    const int t = threadIdx.x;
    const int mine = nvec > t ? (nvec - 1 - t) / TH + 1 : 0;     // vectors t, t + TH, ... of this thread
    // every load is unconditional (past the thread's last vector it re-reads the
    // chunk's last one, which is never looked at), so the compiler counts them
    // exactly and no wait covers more than it must
    const int vlast = nvec - 1;                                  // nvec >= 1 for a non-empty chunk
    if (PATHS == 1 || (PATHS == 0 && nvec <= KR * TH)) {
        u32x4 v[KR];
        #pragma unroll
        for (int j = 0; j < KR; ++j) v[j] = __builtin_nontemporal_load(vp + min(t + j * TH, vlast));
        if (set_n > 0 && t < kWave) set_out = tree_set_wave(set_p, set_n);
        float m = NEG;
        #pragma unroll
        for (int j = 0; j < KR; ++j) {
            const float mj = vec_max<T>(v[j], m);
            m = j < mine ? mj : m;
        }
        // the workgroup's max (and whether a signalling NaN showed up) in one exchange
        const bool nan_t = m != m;
        const float wm = wave_max_f32(nan_t ? NEG : m);
        const bool wnan = __ballot(nan_t) != 0ull;
        if ((t & 63) == 0) {
            s_max[t >> 6] = wm;
            s_idx[t >> 6] = wnan ? 1 : 0;
        }
        __syncthreads();
        float M = s_max[0];
        int any_nan = s_idx[0];
        #pragma unroll
        for (int k = 1; k < TH / kWave; ++k) {
            M = fmaxf(M, s_max[k]);
            any_nan |= s_idx[k];
        }
        if (any_nan) {
            Best b{NEG, kNoIndex};
            #pragma unroll
            for (int j = 0; j < KR; ++j)
                if (j < mine) vec_offer<T>(v[j], lo + (t + j * TH) * EPV, b);
            return block_best(b, scratch);
        }
        int idx = kNoIndex;
        if (m == M) {                                   // this thread holds the max (or has nothing and M = -inf)
            #pragma unroll
            for (int j = KR - 1; j >= 0; --j) {
                if (j < mine) {
                    const int k = vec_first<T>(v[j], M);
                    idx = k < EPV ? lo + (t + j * TH) * EPV + k : idx;
                }
            }
        }
        __syncthreads();                                // every wave has read s_max / s_idx
        idx = wave_min_i32(idx);
        if ((t & 63) == 0) s_idx[t >> 6] = idx;
        __syncthreads();
        #pragma unroll
        for (int k = 0; k < TH / kWave; ++k) idx = min(idx, s_idx[k]);
        return Best{M, idx};
    }
    Best b{NEG, kNoIndex};
    u32x4 cur[KB], nxt[KB];
    auto load = [&](u32x4 (&dst)[KB], int j0) {
        #pragma unroll
        for (int j = 0; j < KB; ++j) dst[j] = __builtin_nontemporal_load(vp + min(t + (j0 + j) * TH, vlast));
    };
    auto scan = [&](const u32x4 (&src)[KB], int j0) {
        #pragma unroll
        for (int j = 0; j < KB; ++j) {
            if (j0 + j < mine) {
                // per vector: its max, and only when that beats the thread's best (or
                // nothing is recorded yet), the first position holding it
                const float m = vec_max<T>(src[j], NEG);
                const int i0 = lo + (t + (j0 + j) * TH) * EPV;
                if (m != m) {
                    vec_offer<T>(src[j], i0, b);
                } else if (m > b.v || b.i == kNoIndex) {
                    const int k = vec_first<T>(src[j], m);
                    if (k < EPV) {                      // (a vector of quiet NaNs only finds nothing)
                        b.v = m;
                        b.i = i0 + k;
                    }
                }
            }
        }
    };
    load(cur, 0);
    load(nxt, KB);
    if (set_n > 0 && t < kWave) set_out = tree_set_wave(set_p, set_n);
    for (int j0 = 0; j0 < mine; j0 += 2 * KB) {
        scan(cur, j0);
        if (j0 + 2 * KB < mine) load(cur, j0 + 2 * KB);
        scan(nxt, j0 + KB);
        if (j0 + 3 * KB < mine) load(nxt, j0 + 3 * KB);
    }
    return block_best(b, scratch);
}

// Scalar fallback for rows that are not 16-byte aligned.
template <typename T>
__device__ __forceinline__ Best chunk_best_scalar(const T* __restrict__ row, int lo, int hi, Best* scratch,
                                                  int set_p, int set_n, uint64_t& set_out) {
    if (set_n > 0 && threadIdx.x < kWave) set_out = tree_set_wave(set_p, set_n);
    Best b{-__builtin_inff(), kNoIndex};
    for (int i = lo + threadIdx.x; i < hi; i += kAcceptThreads) {
        float v;
        if constexpr (sizeof(T) == 2) v = bf16_bits_to_f32(row[i]);
        else v = row[i];
        offer(b, v, i);
    }
    return block_best(b, scratch);
}

struct AcceptArgs {
    const void* logits;
    const int32_t* draft;
    const int32_t* parent;
    const uint64_t* anc;
    int32_t* next_tokens;
    int32_t* accept_len;
    int32_t* accepted_nodes;
    int32_t* bonus;
    int* seq_count;     // [B]       (workspace, zero between calls)
    int* group_count;   // [B][groups] (workspace, zero between calls; unused when groups == 1)
    uint64_t* partial;  // [B*N*C]   chunk winners as keys (workspace)
    int N, vocab, chunks, chunk_len;
    int groups;         // arrival groups per sequence (1: every workgroup arrives on seq_count)
    uint64_t* anc_out;  // non-null: the walk builds the ancestor sets from parent (anc unused) and writes them here
    int aligned;        // rows start on 16-byte boundaries and chunk_len keeps them there
};


// Workgroup `blk` of the argmax + walk launch (one 256-thread workgroup per
// (row, chunk); the sequence's last arriver merges and walks).
template <typename T, int PATHS = 0>
__device__ __forceinline__ void accept_logits_body(const AcceptArgs& a, int blk) {
    __shared__ Best scratch[kAcceptThreads / kWave];
    __shared__ unsigned long long s_key[JF_MAX_NODES];
    __shared__ int32_t s_next[JF_MAX_NODES];
    __shared__ int last;
    const int row = blk / a.chunks, c = blk - row * a.chunks;
    const int b = row / a.N;
    const T* rp = reinterpret_cast<const T*>(a.logits) + (size_t)row * a.vocab;
    const int lo = c * a.chunk_len;
    const int hi = min(a.vocab, lo + a.chunk_len);

    // The walk's node entries are requested before the scan by every workgroup, so
    // the last one to finish already holds them. When the call builds the ancestor
    // sets and the tree has at most 64 nodes, wave 0 builds them from the parents
    // while the scan's loads are in flight (pointer doubling across its lanes).
    NodeIn nd = load_node(b, a.N, a.parent, a.draft, a.anc_out ? nullptr : a.anc);
    const bool wave_sets = a.anc_out != nullptr && a.N <= kWave;
    uint64_t early_set = 0;
    const int set_n = wave_sets ? a.N : 0;
    const Best best = a.aligned ? chunk_best<T, PATHS>(rp, lo, hi, scratch, nd.p, set_n, early_set)
                                : chunk_best_scalar<T>(rp, lo, hi, scratch, nd.p, set_n, early_set);

    // publish the chunk winner; the sequence's last workgroup to finish goes on
    const int per_seq = a.N * a.chunks;
    if (threadIdx.x == 0) {
        __hip_atomic_store(&a.partial[blk], best_key(best), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        wait_own_stores();
        // arrivals in two levels when a sequence has many workgroups: one counter per
        // group (workgroup index mod groups), then the group's last arriver on the
        // sequence counter, so no counter sees more than ~per_seq / groups + groups
        // atomics in a row
        bool closes = true;
        int expect = per_seq;
        if (a.groups > 1) {
            const int g = (blk - b * per_seq) % a.groups;
            const int members = (per_seq - g + a.groups - 1) / a.groups;
            int* gc = a.group_count + b * a.groups + g;
            const int old = arrive(gc);
            closes = (old == members - 1);
            if (closes) reset_counter(gc);
            expect = a.groups;
        }
        int is_last = 0;
        if (closes) {
            const int old = arrive(&a.seq_count[b]);
            is_last = (old == expect - 1);
            if (is_last) reset_counter(&a.seq_count[b]);
        }
        last = is_last;
    }
    __syncthreads();
    if (!last) return;

    // every load of the final phase at once: up to 4 chunk keys per thread and
    // pass (one pass covers N * C <= 1024)
    const uint64_t* pk = a.partial + (size_t)b * per_seq;
    const int u = threadIdx.x;
    if (u < a.N) s_key[u] = 0ull;
    for (int k0 = 0; k0 < per_seq; k0 += 4 * kAcceptThreads) {
        uint64_t kv[4];
        #pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k = k0 + u + j * kAcceptThreads;
            kv[j] = (k < per_seq) ? __hip_atomic_load(pk + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
        }
        __syncthreads();                    // s_key initialised (first pass) / previous pass merged
        #pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k = k0 + u + j * kAcceptThreads;
            if (k < per_seq) atomicMax(&s_key[k / a.chunks], (unsigned long long)kv[j]);
        }
    }
    __syncthreads();
    if (u < a.N) {
        const int nx = key_index(s_key[u]);
        s_next[u] = nx;
        a.next_tokens[(size_t)b * a.N + u] = nx;
    }
    __syncthreads();
    if (wave_sets) {
        // built during the scan (wave 0 holds node u in lane u); written out as well
        if (u < a.N) {
            nd.a[0] = early_set;
            a.anc_out[((size_t)b * a.N + u) * kAncWords] = early_set;
            #pragma unroll
            for (int k = 1; k < kAncWords; ++k) {
                nd.a[k] = 0ull;
                a.anc_out[((size_t)b * a.N + u) * kAncWords + k] = 0ull;
            }
        }
    } else if (a.anc_out) {
        // the ancestor sets from the parent array (pointer doubling in LDS), written out as well
        const auto sets = tree_sets_lds(nd.p, a.N);
        if (u < a.N) {
            #pragma unroll
            for (int k = 0; k < kAncWords; ++k) {
                nd.a[k] = sets[u][k];
                a.anc_out[((size_t)b * a.N + u) * kAncWords + k] = nd.a[k];
            }
        }
    }
    walk_sequence(b, a.N, nd.p, nd.d, nd.a, s_next, a.accept_len, a.accepted_nodes, a.bonus);
}


// ---------------------------------------------------------------- host side (accept.hip)

struct AcceptPlan {
    int chunks, chunk_len, groups;
    size_t off_seq, off_group, off_part, bytes;
};

AcceptPlan plan_accept(int B, int N, int vocab);

// Arguments of the logits-mode launch for a workspace laid out by plan_accept.
AcceptArgs make_accept_args(const AcceptPlan& p, int N, int vocab, const void* logits, int dtype,
                            const int32_t* draft, const int32_t* parent, const uint64_t* anc, int32_t* next_tokens,
                            int32_t* accept_len, int32_t* accepted_nodes, int32_t* bonus, void* workspace);

}  // namespace jf

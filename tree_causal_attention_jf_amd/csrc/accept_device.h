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
static __device__ void walk_sequence(int b, int N, int p_u, int d_u, const uint64_t a_u[kAncWords],
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

__device__ __forceinline__ NodeIn load_node(int b, int N, const int32_t* __restrict__ parent,
                                            const int32_t* __restrict__ draft, const uint64_t* __restrict__ anc) {
    NodeIn n{-1, 0, {0, 0, 0, 0}};
    const int u = threadIdx.x;
    if (u < N) {
        const size_t r = (size_t)b * N + u;
        n.p = parent[r];
        n.d = draft[r];
        if (anc) {
            #pragma unroll
            for (int k = 0; k < kAncWords; ++k) n.a[k] = anc[r * kAncWords + k];
        }
    }
    return n;
}


template <typename T>
__device__ __forceinline__ void scan_chunk(const T* __restrict__ row, int lo, int hi, Best& b);

// bf16: 8 values per 16-byte load; the row start must be 16-byte aligned.
// A thread visits its indices in increasing order, so a strictly larger value is
// the only thing that can replace its best (an equal one comes later and loses).
// Per 8 values: the max of the vector (v_max3 ignores NaN), and only when it beats
// the best so far, the first position holding it. A thread that has recorded
// nothing yet also takes a vector whose max equals its -inf start, so a row of
// -inf values still yields its first index.
__device__ __forceinline__ void offer8_bf16(const u32x4 r, int i0, Best& b) {
    float v[8];
    #pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[2 * e] = __uint_as_float(r[e] << 16);
        v[2 * e + 1] = __uint_as_float(r[e] & 0xffff0000u);
    }
    const float m = max3f(max3f(v[0], v[1], v[2]), max3f(v[3], v[4], v[5]), max3f(v[6], v[7], v[7]));
    if (m != m) {
        // all NaN, or a signalling NaN among them: value by value
        #pragma unroll
        for (int e = 0; e < 8; ++e) offer(b, v[e], i0 + e);
    } else if (m > b.v || (b.i == kNoIndex)) {
        int k = 7;
        #pragma unroll
        for (int e = 6; e >= 0; --e) k = (v[e] == m) ? e : k;
        b.v = m;
        b.i = i0 + k;
    }
}

template <>
__device__ __forceinline__ void scan_chunk<uint16_t>(const uint16_t* __restrict__ row, int lo, int hi, Best& b) {
    const int nvec = (hi - lo) >> 3;
    const u32x4* vp = reinterpret_cast<const u32x4*>(row + lo);
    constexpr int U = 4;
    constexpr int STEP = U * kAcceptThreads;
    int k = threadIdx.x;
    // two batches in flight: the next batch is requested before the current one is scanned
    u32x4 cur[U];
    const bool any = k + (U - 1) * kAcceptThreads < nvec;
    if (any) {
        #pragma unroll
        for (int j = 0; j < U; ++j) cur[j] = __builtin_nontemporal_load(vp + k + j * kAcceptThreads);
    }
    for (; k + (U - 1) * kAcceptThreads < nvec; k += STEP) {
        u32x4 nxt[U];
        const bool more = k + STEP + (U - 1) * kAcceptThreads < nvec;
        if (more) {
            #pragma unroll
            for (int j = 0; j < U; ++j) nxt[j] = __builtin_nontemporal_load(vp + k + STEP + j * kAcceptThreads);
        }
        #pragma unroll
        for (int j = 0; j < U; ++j) offer8_bf16(cur[j], lo + ((k + j * kAcceptThreads) << 3), b);
        if (more) {
            #pragma unroll
            for (int j = 0; j < U; ++j) cur[j] = nxt[j];
        }
    }
    for (; k < nvec; k += kAcceptThreads) offer8_bf16(__builtin_nontemporal_load(vp + k), lo + (k << 3), b);
    for (int i = lo + (nvec << 3) + threadIdx.x; i < hi; i += kAcceptThreads)
        offer(b, bf16_bits_to_f32(row[i]), i);
}

// fp32: 4 values per 16-byte load
template <>
__device__ __forceinline__ void scan_chunk<float>(const float* __restrict__ row, int lo, int hi, Best& b) {
    const int nvec = (hi - lo) >> 2;
    const f32x4* vp = reinterpret_cast<const f32x4*>(row + lo);
    constexpr int U = 4;
    int k = threadIdx.x;
    for (; k + (U - 1) * kAcceptThreads < nvec; k += U * kAcceptThreads) {
        f32x4 r[U];
        #pragma unroll
        for (int j = 0; j < U; ++j) r[j] = __builtin_nontemporal_load(vp + k + j * kAcceptThreads);
        #pragma unroll
        for (int j = 0; j < U; ++j) {
            const int i0 = lo + ((k + j * kAcceptThreads) << 2);
            #pragma unroll
            for (int e = 0; e < 4; ++e) offer(b, r[j][e], i0 + e);
        }
    }
    for (; k < nvec; k += kAcceptThreads) {
        const f32x4 r = __builtin_nontemporal_load(vp + k);
        const int i0 = lo + (k << 2);
        #pragma unroll
        for (int e = 0; e < 4; ++e) offer(b, r[e], i0 + e);
    }
    for (int i = lo + (nvec << 2) + threadIdx.x; i < hi; i += kAcceptThreads) offer(b, row[i], i);
}

// Scalar fallback for rows that are not 16-byte aligned.
template <typename T>
__device__ __forceinline__ void scan_scalar(const T* __restrict__ row, int lo, int hi, Best& b) {
    for (int i = lo + threadIdx.x; i < hi; i += kAcceptThreads) {
        float v;
        if constexpr (sizeof(T) == 2) v = bf16_bits_to_f32(row[i]);
        else v = row[i];
        offer(b, v, i);
    }
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
template <typename T>
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

    Best best{-__builtin_inff(), kNoIndex};
    if (a.aligned) scan_chunk<T>(rp, lo, hi, best);
    else scan_scalar<T>(rp, lo, hi, best);
    best = block_best(best, scratch);

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

    // every load of the final phase at once: this thread's node and up to 4
    // chunk keys per pass (one pass covers N * C <= 1024)
    NodeIn nd = load_node(b, a.N, a.parent, a.draft, a.anc_out ? nullptr : a.anc);
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
    if (a.anc_out) {
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

// Best-first construction of the draft tree from the draft head's logits.
//
// What is computed (technical summaries of "JetFlow ...", section 2, tree
// construction): the draft head emits a logits row for every node of the tree
// in one pass; a node offers its topk most likely next tokens as children,
// each scored by the node's cumulative draft log-probability plus the child's
// log-probability; a best-first expansion adds the best-scored candidate next
// until the token budget is reached. Row i of a sequence belongs to the i-th
// node to join (node 0 is the root, the last committed token). Readings:
//   * log p(t) = z_t - logsumexp(z), in fp64; NaN logits count as -inf,
//     tokens of -inf logit are never offered, a row whose largest entry is not
//     finite offers nothing;
//   * ranks inside a row: larger logit first, then the smaller token id;
//   * candidates: larger score first, then the parent that joined first, then
//     the better rank; a node whose root-to-node path holds max_path_nodes
//     nodes is not expanded; growth stops at the budget or when nothing is left.
//
// One launch:
//  1. workgroup (sequence b, row i, chunk c) reads one 32768-value chunk
//     (16384 for fp32) of row i, every 16-byte load in flight at once and held
//     in registers, and makes three passes over it: each vector's largest value
//     (packed 16-bit maxima of bf16 patterns, v_max3 for fp32); the fp64 sum of exp(z - m_t) against the thread's largest value
//     m_t (a table exponential good to 4e-14, exact at 0); the thread's sorted
//     top-k, fed only from vectors whose largest value reaches a lower bound on
//     the chunk's k-th largest (the k-th largest thread maximum of a wave, the
//     best such bound over the workgroup's waves). It publishes the chunk's
//     largest logit m_c, sum exp(z - m_c) and top-k with agent-scope atomic
//     stores and arrives on the sequence's counter (two levels when the sequence
//     has many workgroups). Only rows that can be expanded run: i < budget - 1.
//  2. the sequence's last workgroup merges each row's chunks (online logsumexp,
//     top-k), grows the tree in batches (candidates sorted, the prefix the
//     serial loop would take added at once; nodes kept in LDS), then one wave
//     finishes node by node: each selected node keeps one head (its best child
//     not yet taken) in the registers of lane node % 64; each step takes the
//     best head across the wave (DPP max of the fp64 scores, ties to the smaller
//     parent id), appends it as the next node, advances its parent's head and
//     gives the new node its first head.
// The arrival counters return to zero, so the workspace never needs clearing
// again (the same counter region as the other entry points).
#include "jf_common.h"
#include "exp_tab.h"

namespace jf {

constexpr int kBuildThreads = 256;
constexpr int kBuildVecs = 16;       // 16-byte vectors per thread per chunk (held in registers)

struct BuildArgs {
    const void* logits;         // [B, N, vocab]
    const int32_t* budget;      // [B] or NULL (N)
    int32_t* parent;            // [B, N]
    int32_t* token;             // [B, N]
    double* score;              // [B, N] or NULL
    int32_t* tree_len;          // [B]
    int* seq_count;             // [B]            workspace, zero between calls
    int* group_count;           // [B][groups]    workspace, zero between calls
    unsigned long long* rec;    // [B][N-1][chunks][rec_words] chunk records (workspace)
    int N, vocab, chunks, chunk_len, topk, cap, groups, rec_words, aligned;
};

// ---------------------------------------------------------------- packed maxima

typedef int16_t s16x2 __attribute__((ext_vector_type(2)));

// per-half signed 16-bit maximum (v_pk_max_i16)
__device__ __forceinline__ uint32_t pk_max_i16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t,
                              __builtin_elementwise_max(__builtin_bit_cast(s16x2, a), __builtin_bit_cast(s16x2, b)));
}

// ---------------------------------------------------------------- keys

// Order-preserving unsigned image of a float (-0 read as +0).
__device__ __forceinline__ uint32_t ord32(float v) {
    uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unord32(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// Chunk-local keys: larger = larger value, then smaller index; 0 = no entry.
// bf16 values keep their 16 significant bits, so value and a 16-bit index fit
// one 32-bit key; fp32 values need 64 bits.
template <typename T> struct KeyOf;
template <> struct KeyOf<uint16_t> {
    using type = uint32_t;
    __device__ static __forceinline__ type make(float v, int local) {
        return ((ord32(v) >> 16) << 16) | (uint32_t)(0xffff - local);
    }
    __device__ static __forceinline__ float value(type k) {
        const uint32_t o = k >> 16;                            // order image of the bf16 bits
        const uint32_t h = (o & 0x8000u) ? (o & 0x7fffu) : (~o & 0xffffu);
        return __uint_as_float(h << 16);
    }
    __device__ static __forceinline__ int index(type k) { return 0xffff - (int)(k & 0xffffu); }
};
template <> struct KeyOf<float> {
    using type = unsigned long long;
    __device__ static __forceinline__ type make(float v, int local) {
        return ((type)ord32(v) << 32) | (type)(0xffffffffu - (uint32_t)local);
    }
    __device__ static __forceinline__ float value(type k) { return unord32((uint32_t)(k >> 32)); }
    __device__ static __forceinline__ int index(type k) { return (int)(0xffffffffu - (uint32_t)k); }
};

template <typename K, int KT>
__device__ __forceinline__ void insert_sorted(K (&l)[KT], K x) {
    #pragma unroll
    for (int j = 0; j < KT; ++j) {
        const K hi = l[j] > x ? l[j] : x;
        x = l[j] > x ? x : l[j];
        l[j] = hi;
    }
}

// ---------------------------------------------------------------- wave reductions (DPP inside rows of 16)

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    const uint32_t lo = dpp_u32<CTRL>((uint32_t)u), hi = dpp_u32<CTRL>((uint32_t)(u >> 32));
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

__device__ __forceinline__ double maxd(double a, double b) { return a > b ? a : b; }

// Largest value of the wave (no NaN among the inputs), the same in every lane.
__device__ __forceinline__ double wave_max_f64(double v) {
    v = maxd(v, dpp_f64<kDppQuad1032>(v));
    v = maxd(v, dpp_f64<kDppQuad2301>(v));
    v = maxd(v, dpp_f64<kDppRowHalfMirror>(v));
    v = maxd(v, dpp_f64<kDppRowMirror>(v));
    return maxd(maxd(readlane_f64(v, 0), readlane_f64(v, 16)), maxd(readlane_f64(v, 32), readlane_f64(v, 48)));
}

__device__ __forceinline__ uint32_t minu(uint32_t a, uint32_t b) { return a < b ? a : b; }

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = minu(v, dpp_u32<kDppQuad1032>(v));
    v = minu(v, dpp_u32<kDppQuad2301>(v));
    v = minu(v, dpp_u32<kDppRowHalfMirror>(v));
    v = minu(v, dpp_u32<kDppRowMirror>(v));
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return minu(minu(a, b), minu(c, d));
}

template <typename K>
__device__ __forceinline__ K wave_max_key(K v) {
    #pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        K w;
        if constexpr (sizeof(K) == 4) {
            w = (K)__shfl_xor((int)v, o);
        } else {
            const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, o);
            const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), o);
            w = ((K)hi << 32) | lo;
        }
        v = v > w ? v : w;
    }
    return v;
}

// ---------------------------------------------------------------- phase 2: the tree

// Writes sequence b's tree: parent / token / score for every node, tree_len.
// s_lp / s_tok / s_cnt hold each expandable row's children (rows < rows_live).
// Run by wave 0 alone.
template <int KT>
__device__ __forceinline__ void grow_tree(const BuildArgs& a, int b, int nb, int rows_live, const double* s_lp, const int* s_tok,
                          const int* s_cnt, int n0 = 0, const double* s_nsc = nullptr, const int* s_dep = nullptr,
                          const int* s_r = nullptr) {
    const int lane = threadIdx.x;
    const int N = a.N;
    int32_t* par = a.parent + (size_t)b * N;
    int32_t* tok = a.token + (size_t)b * N;
    double* sc = a.score ? a.score + (size_t)b * N : nullptr;
    const double ninf = -__builtin_inf();

    // slot s of lane l is node s * 64 + l: its score, depth, child count, next rank,
    // head value (its best child not yet taken, -inf: none) and the head's successor
    double hs[4], hv[4], hn[4];
    int hd[4], hc[4], hr[4];
    #pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int v = s * 64 + lane;
        hs[s] = 0.0;
        hv[s] = ninf;
        hn[s] = ninf;
        hd[s] = 0;
        hr[s] = 0;
        hc[s] = (v < rows_live) ? s_cnt[v] : 0;
    }
    int n = 0;
    if (n0 > 0) {
        // continue from nodes 0 .. n0-1 already grown (their scores, depths and
        // next child ranks in LDS; their outputs already written)
        #pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int v = s * 64 + lane;
            if (v < n0) {
                hs[s] = s_nsc[v];
                hd[s] = s_dep[v];
                hr[s] = s_r[v];
                if (hd[s] < a.cap && hr[s] < hc[s]) {
                    hv[s] = hs[s] + s_lp[v * KT + hr[s]];
                    hn[s] = hr[s] + 1 < hc[s] ? s_lp[v * KT + hr[s] + 1] : ninf;
                }
            }
        }
        n = n0;
    } else if (nb >= 1) {
        if (lane == 0) {
            par[0] = -1;
            tok[0] = -1;
            if (sc) sc[0] = 0.0;
            hd[0] = 1;
            if (1 < a.cap && hc[0] > 0) {
                hv[0] = s_lp[0];
                hn[0] = hc[0] > 1 ? s_lp[1] : ninf;
            }
        }
        n = 1;
    }
    while (n < nb) {
        // best head of this lane: larger value, ties to the smaller slot (smaller node id)
        double bv = hv[0];
        int bs = 0;
        #pragma unroll
        for (int s = 1; s < 4; ++s) {
            if (hv[s] > bv) {
                bv = hv[s];
                bs = s;
            }
        }
        const double wv = wave_max_f64(bv);
        if (!(wv > ninf)) break;                                   // no candidate left (uniform)
        const unsigned long long tied = __ballot(bv == wv);
        int wp;                                                    // parent of the new node
        if (__builtin_popcountll(tied) == 1) {
            const int owner = __builtin_ctzll(tied);
            wp = __builtin_amdgcn_readlane(bs, owner) * 64 + owner;
        } else {
            wp = (int)wave_min_u32(bv == wv ? (uint32_t)(bs * 64 + lane) : 0xffffffffu);
        }
        wp = __builtin_amdgcn_readfirstlane(wp);
        const int owner = wp & 63, slot = wp >> 6;
        // the owner takes the head: the new node's token, depth; its next child becomes the head
        int nd = 0;
        if (lane == owner) {
            #pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (s == slot) {
                    const int r = hr[s];
                    tok[n] = s_tok[wp * KT + r];
                    par[n] = wp;
                    if (sc) sc[n] = wv;
                    nd = hd[s] + 1;
                    hr[s] = r + 1;
                    hv[s] = (r + 1 < hc[s]) ? hs[s] + hn[s] : ninf;
                    hn[s] = (r + 2 < hc[s]) ? s_lp[wp * KT + r + 2] : ninf;
                }
            }
        }
        nd = __builtin_amdgcn_readlane(nd, owner);
        // the new node's first head
        if (lane == (n & 63)) {
            const int ns = n >> 6;
            #pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (s == ns) {
                    hs[s] = wv;
                    hd[s] = nd;
                    hr[s] = 0;
                    if (nd < a.cap && hc[s] > 0) {                // hc = 0 for rows past rows_live
                        hv[s] = wv + s_lp[n * KT];
                        hn[s] = hc[s] > 1 ? s_lp[n * KT + 1] : ninf;
                    }
                }
            }
        }
        ++n;
    }
    // padding
    for (int v = (n > 1 ? n : 1) + lane; v < N; v += 64) {
        par[v] = 0;
        tok[v] = -1;
    }
    if (sc)
        for (int v = n + lane; v < N; v += 64) sc[v] = ninf;
    if (nb < 1 && lane == 0) {
        par[0] = -1;
        tok[0] = -1;
    }
    if (lane == 0) a.tree_len[b] = (nb >= 0 && nb <= N) ? n : -1;
}

// ---------------------------------------------------------------- growth in batches

// Wave scans over DPP: shifts inside each row of 16 lanes (row_shr 1, 2, 4, 8),
// then the row broadcasts (lane 15 of a row into the next row, lane 31 into the
// upper half). A lane whose DPP source does not exist receives the identity.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143, kDppWaveShr1 = 0x138, kDppRowRor8 = 0x128;
constexpr int kDppQuad3210 = 0x1b;

__device__ __forceinline__ int wave_incl_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr1, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr2, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr4, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr8, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowBcast15, 0xa, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowBcast31, 0xc, 0xf, false);
    return x;
}

// v moved by a DPP control; lanes the control does not reach (no source, or a
// row outside ROWS) get `fill`.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64_fill(double v, double fill) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    const unsigned long long f = (unsigned long long)__double_as_longlong(fill);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)f, (int)(uint32_t)u, CTRL, ROWS, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(f >> 32), (int)(uint32_t)(u >> 32), CTRL,
                                                              ROWS, 0xf, false);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

__device__ __forceinline__ double wave_incl_max(double x) {
    const double ni = -__builtin_inf();
    x = maxd(x, dpp_f64_fill<kDppRowShr1, 0xf>(x, ni));
    x = maxd(x, dpp_f64_fill<kDppRowShr2, 0xf>(x, ni));
    x = maxd(x, dpp_f64_fill<kDppRowShr4, 0xf>(x, ni));
    x = maxd(x, dpp_f64_fill<kDppRowShr8, 0xf>(x, ni));
    x = maxd(x, dpp_f64_fill<kDppRowBcast15, 0xa>(x, ni));
    x = maxd(x, dpp_f64_fill<kDppRowBcast31, 0xc>(x, ni));
    return x;
}

// Workgroup scans with one barrier: a DPP scan inside each wave, then the waves'
// totals through LDS. s_w has one slot per wave; every thread calls them (they
// hold a barrier), and the caller passes a barrier before reusing s_w.
__device__ __forceinline__ int block_exclusive_sum(int x, int* s_w, int* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int incl = wave_incl_sum(x);
    if (lane == 63) s_w[w] = incl;
    __syncthreads();
    int before = 0, tot = 0;
    #pragma unroll
    for (int k = 0; k < kBuildThreads / 64; ++k) {
        const int v = s_w[k];
        tot += v;
        before += k < w ? v : 0;
    }
    *total = tot;
    return before + incl - x;
}

// Exclusive prefix maximum of x over the workgroup (-inf for thread 0).
__device__ __forceinline__ double block_exclusive_max(double x, double* s_w) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const double incl = wave_incl_max(x);
    if (lane == 63) s_w[w] = incl;
    double r = dpp_f64_fill<kDppWaveShr1, 0xf>(incl, -__builtin_inf());   // the lane before (lane 0: -inf)
    __syncthreads();
    #pragma unroll
    for (int k = 0; k < kBuildThreads / 64; ++k)
        if (k < w) r = maxd(r, s_w[k]);
    return r;
}

// The value of lane (lane ^ 2^LS): DPP inside rows of 16 (quad permutations; the
// half-row mirror then a quad reversal for 4; a rotation by 8), shuffles beyond.
template <int LS>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
    if constexpr (LS == 0) return dpp_u32<kDppQuad1032>(v);
    else if constexpr (LS == 1) return dpp_u32<kDppQuad2301>(v);
    else if constexpr (LS == 2) return dpp_u32<kDppQuad3210>(dpp_u32<kDppRowHalfMirror>(v));
    else if constexpr (LS == 3) return dpp_u32<kDppRowRor8>(v);
    else return (uint32_t)__shfl_xor((int)v, 1 << LS);
}

// A register bitonic sort of one candidate per thread (thread t ends up holding
// the t-th in the loop's order: larger score first, then smaller key). Partners
// at stride 2^LS < 64 are in the same wave (xor_lane); strides 64 and 128 go
// through LDS between barriers. Branch-free compares (bitwise | and &), and the
// strides are compile-time constants, so a step is a few DPP moves, compares
// and selects.
template <int LS>
__device__ __forceinline__ void bitonic_step(double& sc, int& key, bool down, double* c_sc, int* c_key) {
    const int t = threadIdx.x;
    double ps;
    int pk;
    if constexpr (LS < 6) {
        const unsigned long long u = (unsigned long long)__double_as_longlong(sc);
        const uint32_t plo = xor_lane<LS>((uint32_t)u), phi = xor_lane<LS>((uint32_t)(u >> 32));
        ps = __longlong_as_double((long long)(((unsigned long long)phi << 32) | plo));
        pk = (int)xor_lane<LS>((uint32_t)key);
    } else {
        __syncthreads();
        c_sc[t] = sc;
        c_key[t] = key;
        __syncthreads();
        ps = c_sc[t ^ (1 << LS)];
        pk = c_key[t ^ (1 << LS)];
    }
    const bool p_first = (ps > sc) | ((ps == sc) & (pk < key));
    // the lower position of the pair keeps the first of the two when sorting into
    // the loop's order, the second otherwise
    const bool take = ((((t >> LS) & 1) == 0) == down) ? p_first : !p_first;
    sc = take ? ps : sc;
    key = take ? pk : key;
}

template <int LS>
__device__ __forceinline__ void bitonic_steps(double& sc, int& key, bool down, double* c_sc, int* c_key) {
    bitonic_step<LS>(sc, key, down, c_sc, c_key);
    if constexpr (LS > 0) bitonic_steps<LS - 1>(sc, key, down, c_sc, c_key);
}

// levels 2^1 .. P (P <= 2^MAXL, a power of two; uniform). MAXL 6 sorts inside one
// wave (no LDS, no barrier); MAXL 8 sorts the workgroup's 256 threads.
template <int MAXL>
__device__ __forceinline__ void bitonic_sort_reg(double& sc, int& key, int P, double* c_sc, int* c_key) {
    const int t = threadIdx.x;
#define JF_BITONIC_LEVEL(L) \
    if constexpr ((L) <= MAXL) \
        if ((1 << (L)) <= P) bitonic_steps<(L) - 1>(sc, key, (t & (1 << (L))) == 0, c_sc, c_key);
    JF_BITONIC_LEVEL(1)
    JF_BITONIC_LEVEL(2)
    JF_BITONIC_LEVEL(3)
    JF_BITONIC_LEVEL(4)
    JF_BITONIC_LEVEL(5)
    JF_BITONIC_LEVEL(6)
    JF_BITONIC_LEVEL(7)
    JF_BITONIC_LEVEL(8)
#undef JF_BITONIC_LEVEL
}

// Scores only fall along a path (log-probabilities are negative), so the serial
// best-first loop can be run many steps at a time: with every child not yet taken
// of every grown node sorted by the loop's own order (score, then the parent that
// joined first, then the child's rank), the loop takes c_1, c_2, ... in that order
// for as long as each c_i scores at least as well as the best child of the nodes
// c_1 .. c_{i-1} have just become (a new node joins after every existing parent, so
// on equal scores c_i still wins). Grown nodes are kept in LDS (parent, token,
// score) and written out by the caller, so no round waits on global stores.
// One round sorts the candidates (bitonic, in LDS),
// finds that prefix and grows it. Rounds go on while they add at least 4 nodes;
// the serial loop then continues from the state left in LDS. Run by the whole
// workgroup. Returns the nodes grown (>= 1 when nb >= 1).
template <int KT>
__device__ __forceinline__ int grow_batches(const BuildArgs& a, int b, int nb, int rows_live, const double* s_lp, const int* s_tok,
                            const int* s_cnt, double* s_nsc, int* s_dep, int* s_r, double* c_sc, int* c_key,
                            double* s_dtmp, int* s_itmp, int* s_isum, int* s_par, int* s_tokn, int* s_ctl) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const double ninf = -__builtin_inf();
    if (nb < 1) return 0;
    if (t == 0) {
        s_par[0] = -1;
        s_tokn[0] = -1;
        s_nsc[0] = 0.0;
        s_dep[0] = 1;
    }
    if (t < JF_MAX_NODES) s_r[t] = 0;
    __syncthreads();
    int n = 1;
    // Rounds in which every grown node and every candidate fits one lane (n <= 64,
    // M <= 64) run on wave 0 alone: the same steps with DPP scans, a one-wave
    // register sort and ballots, no workgroup barrier (one wave's LDS accesses take
    // effect in order). The other waves wait for them at one barrier.
    if (w == 0) {
        int done = 0;
        while (n < nb && n <= 64) {
            int cnt = 0;
            if (lane < n && lane < rows_live && s_dep[lane] < a.cap) cnt = max(0, s_cnt[lane] - s_r[lane]);
            const int incl = wave_incl_sum(cnt);
            const int M = __builtin_amdgcn_readlane(incl, 63);
            if (M == 0) {
                done = 1;
                break;
            }
            if (M > 64) break;                                    // a workgroup round
            const int off = incl - cnt;
            for (int j = 0; j < cnt; ++j) {
                const int key = lane * KT + s_r[lane] + j;
                c_sc[off + j] = s_nsc[lane] + s_lp[key];
                c_key[off + j] = key;
            }
            __builtin_amdgcn_wave_barrier();
            int P = 1;
            while (P < M) P <<= 1;
            double my_sc = lane < M ? c_sc[lane] : ninf;
            int my_key = lane < M ? c_key[lane] : 0x7fffffff;
            bitonic_sort_reg<6>(my_sc, my_key, P, nullptr, nullptr);
            const int m = min(M, nb - n);
            double cand = ninf, child = ninf;
            const int u = n + lane, v = my_key / KT;
            if (lane < m) {
                cand = my_sc;
                if (s_dep[v] + 1 < a.cap && u < rows_live && s_cnt[u] > 0) child = cand + s_lp[u * KT];
            }
            const double best_new = dpp_f64_fill<kDppWaveShr1, 0xf>(wave_incl_max(child), ninf);
            const unsigned long long stop = __ballot(lane < m && !(cand >= best_new));
            const int k = stop ? (int)__builtin_ctzll(stop) : m;
            if (lane < k) {
                s_par[u] = v;
                s_tokn[u] = s_tok[my_key];
                s_nsc[u] = my_sc;
                s_dep[u] = s_dep[v] + 1;
                atomicMax(&s_r[v], my_key - v * KT + 1);
            }
            __builtin_amdgcn_wave_barrier();
            n += k;
            if (k < 4) {
                done = 1;
                break;
            }
        }
        if (lane == 0) {
            s_ctl[0] = n;
            s_ctl[1] = done;
        }
    }
    __syncthreads();
    n = s_ctl[0];
    if (s_ctl[1]) return n;
    while (n < nb) {
        // candidates: node t (grown, expandable) offers its children r .. cnt-1
        int cnt_t = 0;
        if (t < n && t < rows_live && s_dep[t] < a.cap) cnt_t = max(0, s_cnt[t] - s_r[t]);
        int M = 0;
        const int off = block_exclusive_sum(cnt_t, s_isum, &M);
        if (M == 0) break;                                        // uniform
        for (int j = 0; j < cnt_t; ++j) {
            const int key = t * KT + s_r[t] + j;
            c_sc[off + j] = s_nsc[t] + s_lp[key];
            c_key[off + j] = key;
        }
        int P = 1;
        while (P < M) P <<= 1;
        __syncthreads();
        // bitonic sort into the loop's order: larger score first, then smaller key;
        // afterwards thread t holds the t-th candidate in (my_sc, my_key)
        double my_sc;
        int my_key;
        if (P <= kBuildThreads) {
            // one candidate per thread, in registers
            my_sc = t < M ? c_sc[t] : ninf;
            my_key = t < M ? c_key[t] : 0x7fffffff;
            bitonic_sort_reg<8>(my_sc, my_key, P, c_sc, c_key);
        } else {
            for (int i = M + t; i < P; i += kBuildThreads) {
                c_sc[i] = ninf;
                c_key[i] = 0x7fffffff;
            }
            __syncthreads();
            // in LDS. Pair i of a stage with stride < 128 stays in the 128-element block of
            // the wave that owns it (i = 64w + lane + 256j lies in block w + 4j), and one
            // wave's LDS accesses take effect in order: such stages follow one another with
            // only a compiler barrier. A stage with stride >= 128 mixes blocks: barriers.
            bool prev_wide = false;
            for (int ls_size = 1; (1 << ls_size) <= P; ++ls_size) {
                const int size = 1 << ls_size;
                for (int ls = ls_size - 1; ls >= 0; --ls) {           // stride 2^ls (shifts, not divisions)
                    const int stride = 1 << ls;
                    const bool wide = stride >= 128;
                    if (wide && !prev_wide) __syncthreads();
                    for (int i = t; i < P / 2; i += kBuildThreads) {
                        const int lo = ((i >> ls) << (ls + 1)) + (i & (stride - 1)), hi = lo + stride;
                        const double xs = c_sc[lo], ys = c_sc[hi];
                        const int xk = c_key[lo], yk = c_key[hi];
                        const bool y_first = ys > xs || (ys == xs && yk < xk);
                        const bool down = (lo & size) == 0;
                        if (down ? y_first : !y_first) {
                            c_sc[lo] = ys;
                            c_sc[hi] = xs;
                            c_key[lo] = yk;
                            c_key[hi] = xk;
                        }
                    }
                    if (wide) __syncthreads();
                    else __builtin_amdgcn_wave_barrier();
                    prev_wide = wide;
                }
            }
            if (!prev_wide) __syncthreads();
            my_sc = c_sc[t];
            my_key = c_key[t];
        }
        // the prefix the serial loop would take: candidate i becomes node n + i
        const int m = min(M, nb - n);
        double cand = ninf, child = ninf;
        if (t < m) {
            const int u = n + t, v = my_key / KT;
            cand = my_sc;
            if (s_dep[v] + 1 < a.cap && u < rows_live && s_cnt[u] > 0) child = cand + s_lp[u * KT];
        }
        const double best_new = block_exclusive_max(child, s_dtmp);
        // k: the first position whose candidate scores below a new node's best child
        const unsigned long long stop = __ballot(t < m && !(cand >= best_new));
        if (lane == 0) s_itmp[w] = stop ? w * 64 + __builtin_ctzll(stop) : m;
        __syncthreads();
        int k = m;
        #pragma unroll
        for (int q = 0; q < kBuildThreads / 64; ++q) k = min(k, s_itmp[q]);
        // grow them
        if (t < k) {
            const int u = n + t, key = my_key, v = key / KT;
            s_par[u] = v;
            s_tokn[u] = s_tok[key];
            s_nsc[u] = my_sc;
            s_dep[u] = s_dep[v] + 1;
            atomicMax(&s_r[v], key - v * KT + 1);
        }
        __syncthreads();
        n += k;
        if (k < 4) break;                                         // uniform
    }
    return n;
}

// ---------------------------------------------------------------- the kernel

template <typename T, int KT>
__global__ __launch_bounds__(kBuildThreads) __attribute__((amdgpu_waves_per_eu(4))) void tree_build_kernel(BuildArgs a) {
    using KO = KeyOf<T>;
    using K = typename KO::type;
    constexpr int EPV = 16 / (int)sizeof(T);                 // elements per 16-byte vector
    constexpr int kNW = kBuildThreads / kWave;
    __shared__ __attribute__((aligned(16))) double s_lp[JF_MAX_NODES * KT];   // phase 1 reuses it for keys
    __shared__ int s_tok[JF_MAX_NODES * KT];
    __shared__ int s_cnt[JF_MAX_NODES];
    __shared__ float s_m[kNW], s_tau[kNW];
    __shared__ double s_s[kNW];
    __shared__ int s_last;
    __shared__ double s_exp2[256];                            // 2^(j/256), adjusted for exp_tab_nonpos
    // growth in batches: grown nodes' scores, depths, next child ranks; candidates
    __shared__ double s_nsc[JF_MAX_NODES];
    __shared__ int s_dep[JF_MAX_NODES], s_r[JF_MAX_NODES];
    __shared__ double c_sc[JF_MAX_NODES * KT];
    __shared__ int c_key[JF_MAX_NODES * KT];
    __shared__ double s_dtmp[kNW];
    __shared__ int s_itmp[kNW], s_isum[kNW];
    __shared__ int s_par[JF_MAX_NODES], s_tokn[JF_MAX_NODES], s_ctl[2];
    static_assert(sizeof(K) * kBuildThreads * KT <= sizeof(double) * JF_MAX_NODES * KT, "key scratch");

    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int R = a.N > 1 ? a.N - 1 : 1;
    const int blk = blockIdx.x;
    const int c = blk % a.chunks;
    const int i = (blk / a.chunks) % R;
    const int b = blk / (a.chunks * R);
    const int nb = a.budget ? a.budget[b] : a.N;
    const bool nb_ok = nb >= 0 && nb <= a.N;
    const int rows_live = (nb_ok && a.cap > 1 && nb >= 2) ? nb - 1 : 0;

    if (rows_live == 0) {
        // nothing to expand: the first workgroup of the sequence writes its tree
        if (i == 0 && c == 0 && w == 0) grow_tree<KT>(a, b, nb_ok ? nb : -1, 0, s_lp, s_tok, s_cnt);
        return;
    }
    if (i >= rows_live) return;
    static_assert(kBuildThreads >= 256, "one table entry per thread");
    if (t < 256) s_exp2[t] = exp_tab_adjust(exp2((double)t / 256.0), t);   // the table exp_tab_nonpos reads
    __syncthreads();

    // ---- phase 1: one chunk of row i, kBuildVecs 16-byte vectors per thread, all
    // requested at once and held in registers, then three passes over them:
    //  (a) each vector's largest value and the thread's, m_t;
    //  (b) sum exp(z - m_t) over every value in fp64 (NaN and -inf add 0);
    //  (c) the thread's sorted top-KT, fed only from vectors whose largest value
    //      reaches tau. tau is a lower bound on the chunk's KT-th largest value:
    //      in each wave the KT-th largest of the 64 thread maxima (those are KT
    //      distinct values of the chunk), the largest over the workgroup's waves.
    const T* rp = reinterpret_cast<const T*>(a.logits) + ((size_t)b * a.N + i) * a.vocab;
    const int lo = c * a.chunk_len;
    const int hi = min(a.vocab, lo + a.chunk_len);
    constexpr float NEG = -__builtin_inff();
    constexpr uint32_t kNegWord = sizeof(T) == 2 ? 0xff80ff80u : 0xff800000u;   // -inf in each value of a word
    u32x4 v[kBuildVecs];
    if (a.aligned) {
        // every load is issued (past the chunk: the row's last chunk re-reads its last
        // vector), then vectors past the chunk are replaced by -inf
        const u32x4* vp = reinterpret_cast<const u32x4*>(rp + lo);
        const int nvec = (hi - lo) / EPV;                   // aligned: the chunk holds whole vectors
        #pragma unroll
        for (int j = 0; j < kBuildVecs; ++j) v[j] = __builtin_nontemporal_load(vp + min(j * kBuildThreads + t, nvec - 1));
        if (hi - lo < a.chunk_len) {
            #pragma unroll
            for (int j = 0; j < kBuildVecs; ++j)
                if (j * kBuildThreads + t >= nvec) v[j] = u32x4{kNegWord, kNegWord, kNegWord, kNegWord};
        }
    } else {
        #pragma unroll
        for (int j = 0; j < kBuildVecs; ++j) {
            const int e0 = (j * kBuildThreads + t) * EPV;       // chunk-local index of the vector
            uint32_t wd[4] = {kNegWord, kNegWord, kNegWord, kNegWord};
            #pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const int idx = lo + e0 + e;
                if (idx < hi) {
                    if constexpr (sizeof(T) == 2) {
                        const uint32_t x = (uint32_t)reinterpret_cast<const uint16_t*>(rp)[idx];
                        wd[e >> 1] = (wd[e >> 1] & ~(0xffffu << (16 * (e & 1)))) | (x << (16 * (e & 1)));
                    } else {
                        wd[e] = __float_as_uint(reinterpret_cast<const float*>(rp)[idx]);
                    }
                }
            }
            v[j] = u32x4{wd[0], wd[1], wd[2], wd[3]};
        }
    }
    // (a) bf16: packed 16-bit integer maxima of the bit patterns. Non-negative
    // bf16 values order like their patterns and lie above every negative pattern,
    // so when the thread's largest pattern is non-negative and not a NaN pattern it
    // is the thread's largest value; otherwise (every value negative, or a NaN with
    // the sign clear) the thread takes its maximum value by value. fp32: v_max3
    // per vector (a signalling NaN, the one input that makes it NaN, sends the
    // thread through the same value-by-value path).
    float m_t = NEG;
    bool exact_t = false;                                       // vectors are filtered value by value
    uint32_t vmp[kBuildVecs];                                   // bf16: packed per-vector maxima
    float vm[sizeof(T) == 2 ? 1 : kBuildVecs];                  // fp32: per-vector maxima
    if constexpr (sizeof(T) == 2) {
        #pragma unroll
        for (int j = 0; j < kBuildVecs; ++j)
            vmp[j] = pk_max_i16(pk_max_i16(v[j][0], v[j][1]), pk_max_i16(v[j][2], v[j][3]));
        uint32_t tp = vmp[0];
        #pragma unroll
        for (int j = 1; j < kBuildVecs; ++j) tp = pk_max_i16(tp, vmp[j]);
        const int mx = max((int)(int16_t)(tp & 0xffffu), (int)(int16_t)(tp >> 16));
        exact_t = !(mx >= 0 && mx <= 0x7f80);
        m_t = __uint_as_float((uint32_t)mx << 16);
    } else {
        #pragma unroll
        for (int j = 0; j < kBuildVecs; ++j) {
            vm[j] = vec_max<T>(v[j], NEG);
            exact_t |= vm[j] != vm[j];
        }
        #pragma unroll
        for (int j = 0; j < kBuildVecs; j += 2) m_t = max3f(vm[j], vm[j + 1], m_t);
    }
    #pragma unroll
    for (int j = 0; j < kBuildVecs; ++j) asm volatile("" : "+v"(v[j]));
    if (exact_t) {
        m_t = NEG;
        #pragma unroll
        for (int j = 0; j < kBuildVecs; ++j)
            #pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const float z = vec_val<T>(v[j], e);
                if (z > m_t) m_t = z;                           // NaN never passes
            }
    }
    // the wave's bound: KT rounds of the wave's largest thread maximum, one holder removed each round
    float tau_w, m_w;
    {
        float x = m_t;
        float mx = wave_max_f32(x);
        m_w = mx;
        #pragma unroll
        for (int r = 1; r < KT; ++r) {
            const unsigned long long hold = __ballot(x == mx);
            if (lane == (int)__builtin_ctzll(hold)) x = NEG;
            mx = wave_max_f32(x);
        }
        tau_w = mx;
    }
    if (lane == 0) {
        s_m[w] = m_w;
        s_tau[w] = tau_w;
    }
    // (b) against the thread's own largest value. (The vectors pass through an empty
    // asm between passes so each pass unpacks them again instead of the compiler
    // keeping 128 unpacked values live from the previous one.)
    #pragma unroll
    for (int j = 0; j < kBuildVecs; ++j) asm volatile("" : "+v"(v[j]));
    // Vectors from `live` on lie past the row's end in every lane (the last chunk)
    // and add nothing: skipped with a uniform branch.
    const int live = ((hi - lo + EPV - 1) / EPV + kBuildThreads - 1) / kBuildThreads;
    const double md = (m_t > NEG && m_t < __builtin_inff()) ? (double)m_t : 0.0;
    double s_a = 0.0, s_b = 0.0;
    #pragma unroll
    for (int j = 0; j < kBuildVecs; ++j) {
        if (j < live) {
            #pragma unroll
            for (int e = 0; e < EPV; e += 2) {
                s_a += exp_tab_nonpos((double)vec_val<T>(v[j], e) - md, s_exp2);
                s_b += exp_tab_nonpos((double)vec_val<T>(v[j], e + 1) - md, s_exp2);
            }
        }
    }
    double s_t = s_a + s_b;
    asm volatile("" : "+v"(s_t));                           // summed here, not sunk past pass (c)
    __syncthreads();
    float m_c = s_m[0], tau = s_tau[0];
    #pragma unroll
    for (int k = 1; k < kNW; ++k) {
        m_c = fmaxf(m_c, s_m[k]);
        tau = fmaxf(tau, s_tau[k]);
    }
    tau = fmaxf(tau, -__FLT_MAX__);                             // z >= tau: neither NaN nor -inf
    // (c)
    #pragma unroll
    for (int j = 0; j < kBuildVecs; ++j) asm volatile("" : "+v"(v[j]));
    K top[KT];
    #pragma unroll
    for (int j = 0; j < KT; ++j) top[j] = 0;
    // bf16 with tau > 0: a vector holds a value >= tau exactly when a packed max
    // against (tau's pattern - 1) in both halves changes it (negative patterns lie
    // below; a NaN pattern with the sign clear only adds a needless check)
    const bool int_hits = sizeof(T) == 2 && tau > 0.f;
    const uint32_t tt = ((__float_as_uint(tau) >> 16) - 1u) * 0x10001u;
    #pragma unroll
    for (int j = 0; j < kBuildVecs; ++j) {
        bool hit;
        if constexpr (sizeof(T) == 2) {
            if (int_hits) {
                hit = pk_max_i16(vmp[j], tt) != tt;
            } else {
                const float mj = vec_max<T>(v[j], NEG);
                hit = !(mj < tau);                              // a NaN maximum: check value by value
            }
        } else {
            hit = !(vm[j] < tau);
        }
        if (exact_t || hit) {
            u32x4 x = v[j];
            asm volatile("" : "+v"(x));                         // unpacked here, not ahead of the branch
            #pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const float z = vec_val<T>(x, e);
                if (z >= tau) insert_sorted<K, KT>(top, KO::make(z, (j * kBuildThreads + t) * EPV + e));
            }
        }
    }
    K* s_keys = reinterpret_cast<K*>(s_lp);
    #pragma unroll
    for (int j = 0; j < KT; ++j) s_keys[t * KT + j] = top[j];
    double part = (m_t > NEG && s_t > 0.0) ? s_t * exp_tab_nonpos((double)m_t - (double)m_c, s_exp2) : 0.0;
    #pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const unsigned long long u = (unsigned long long)__double_as_longlong(part);
        const uint32_t plo = (uint32_t)__shfl_xor((int)(uint32_t)u, o), phi = (uint32_t)__shfl_xor((int)(uint32_t)(u >> 32), o);
        part += __longlong_as_double((long long)(((unsigned long long)phi << 32) | plo));
    }
    if (lane == 0) s_s[w] = part;
    __syncthreads();
    if (w == 0) {
        // merge the 256 threads' lists: lane l takes threads 4l .. 4l+3, then KT rounds
        // of the wave's largest head
        K mine[KT];
        #pragma unroll
        for (int j = 0; j < KT; ++j) mine[j] = 0;
        #pragma unroll
        for (int q = 0; q < 4; ++q)
            #pragma unroll
            for (int j = 0; j < KT; ++j) insert_sorted<K, KT>(mine, s_keys[(lane * 4 + q) * KT + j]);
        unsigned long long* rec =
            a.rec + (((size_t)b * (a.N > 1 ? a.N - 1 : 1) + i) * a.chunks + c) * (size_t)a.rec_words;
        for (int r = 0; r < KT; ++r) {
            const K best = wave_max_key<K>(mine[0]);
            if (lane == 0) {
                unsigned long long word;
                if (best) word = ((unsigned long long)(uint32_t)(lo + KO::index(best)) << 32) |
                                 __float_as_uint(KO::value(best));
                else word = (0xffffffffull << 32) | __float_as_uint(-__builtin_inff());
                __hip_atomic_store(rec + 2 + r, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if (best && mine[0] == best) {              // keys are distinct: one lane pops
                #pragma unroll
                for (int j = 0; j + 1 < KT; ++j) mine[j] = mine[j + 1];
                mine[KT - 1] = 0;
            }
        }
        if (lane == 0) {
            double s_c = s_s[0];
            #pragma unroll
            for (int k = 1; k < kNW; ++k) s_c += s_s[k];
            __hip_atomic_store(rec + 0, (unsigned long long)__float_as_uint(m_c), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(rec + 1, (unsigned long long)__double_as_longlong(s_c), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            wait_own_stores();
            // arrival (two levels when the sequence has many workgroups)
            const int per_seq = rows_live * a.chunks;
            bool closes = true;
            int expect = per_seq;
            if (a.groups > 1) {
                const int g = (i * a.chunks + c) % a.groups;
                const int members = (per_seq - g + a.groups - 1) / a.groups;
                int* gc = a.group_count + b * a.groups + g;
                const int old = arrive(gc);
                closes = (old == members - 1);
                if (closes) reset_counter(gc);
                expect = per_seq < a.groups ? per_seq : a.groups;
            }
            int is_last = 0;
            if (closes) {
                const int old = arrive(&a.seq_count[b]);
                is_last = (old == expect - 1);
                if (is_last) {
                    acquire_agent();                            // the records are then read with plain loads
                    reset_counter(&a.seq_count[b]);             // after the fence, which waits for earlier stores
                }
            }
            s_last = is_last;
        }
    }
    __syncthreads();
    if (!s_last) return;

    // ---- phase 2 (the sequence's last workgroup): each row's logsumexp and children
    const unsigned long long* rb = a.rec + (size_t)b * (a.N > 1 ? a.N - 1 : 1) * a.chunks * a.rec_words;
    if (t < rows_live) {
        // row t: its chunks' records, CG at a time with every load in flight; the
        // logsumexp runs online (the sum is rescaled when a chunk holds a larger max)
        constexpr int RW = 2 + KT, CG = KT <= 4 ? 4 : 2;
        const unsigned long long* rr = rb + (size_t)t * a.chunks * a.rec_words;
        float m = -__builtin_inff();
        double s = 0.0;
        unsigned long long best[KT];
        #pragma unroll
        for (int j = 0; j < KT; ++j) best[j] = 0;
        for (int c0 = 0; c0 < a.chunks; c0 += CG) {
            unsigned long long r[CG][RW];
            #pragma unroll
            for (int q = 0; q < CG; ++q) {
                const unsigned long long* rc = rr + (size_t)min(c0 + q, a.chunks - 1) * a.rec_words;
                #pragma unroll
                for (int k = 0; k < RW; ++k) r[q][k] = rc[k];
            }
            #pragma unroll
            for (int q = 0; q < CG; ++q) {
                if (c0 + q >= a.chunks) break;
                const float mc = __uint_as_float((uint32_t)r[q][0]);
                const double scc = __longlong_as_double((long long)r[q][1]);
                if (mc > -__builtin_inff()) {
                    if (mc > m) {
                        s = (m > -__builtin_inff() ? s * exp_tab_nonpos((double)m - (double)mc, s_exp2) : 0.0) + scc;
                        m = mc;
                    } else {
                        s += scc * exp_tab_nonpos((double)mc - (double)m, s_exp2);
                    }
                }
                #pragma unroll
                for (int j = 0; j < KT; ++j) {
                    const unsigned long long e = r[q][2 + j];
                    const float ev = __uint_as_float((uint32_t)e);
                    const uint32_t etok = (uint32_t)(e >> 32);
                    // global key: value, then the smaller token id
                    const unsigned long long key = ev > -__builtin_inff()
                                                       ? (((unsigned long long)ord32(ev) << 32) | (0xffffffffu - etok))
                                                       : 0ull;
                    insert_sorted<unsigned long long, KT>(best, key);
                }
            }
        }
        int cnt = 0;
        if (m > -__builtin_inff() && m < __builtin_inff()) {
            const double lse = (double)m + log(s);
            #pragma unroll
            for (int j = 0; j < KT; ++j) {
                if (j < a.topk && best[j]) {
                    s_lp[t * KT + j] = (double)unord32((uint32_t)(best[j] >> 32)) - lse;
                    s_tok[t * KT + j] = (int)(0xffffffffu - (uint32_t)best[j]);
                    cnt = j + 1;
                }
            }
        }
        s_cnt[t] = cnt;
    }
    __syncthreads();
    const int n0 = grow_batches<KT>(a, b, nb, rows_live, s_lp, s_tok, s_cnt, s_nsc, s_dep, s_r, c_sc, c_key, s_dtmp,
                                    s_itmp, s_isum, s_par, s_tokn, s_ctl);
    // the batches' nodes (the serial loop writes its own, all past n0)
    {
        int32_t* par = a.parent + (size_t)b * a.N;
        int32_t* tok = a.token + (size_t)b * a.N;
        double* sc = a.score ? a.score + (size_t)b * a.N : nullptr;
        for (int v = t; v < n0; v += kBuildThreads) {
            par[v] = s_par[v];
            tok[v] = s_tokn[v];
            if (sc) sc[v] = s_nsc[v];
        }
    }
    if (w == 0) grow_tree<KT>(a, b, nb, rows_live, s_lp, s_tok, s_cnt, n0, s_nsc, s_dep, s_r);
}

// ---------------------------------------------------------------- host side

struct BuildPlan {
    int chunks, chunk_len, groups, rec_words, kt;
    size_t off_group, off_rec, bytes;
};

static size_t align_up_b(size_t x, size_t a) { return (x + a - 1) / a * a; }

BuildPlan plan_build(int B, int N, int vocab, int topk, int dtype) {
    BuildPlan p{};
    p.kt = topk <= 1 ? 1 : topk <= 2 ? 2 : topk <= 4 ? 4 : 8;
    const int epv = dtype == JF_BF16 ? 8 : 4;
    p.chunk_len = kBuildThreads * kBuildVecs * epv;          // 32768 bf16 / 16384 fp32 values
    p.chunks = (vocab + p.chunk_len - 1) / p.chunk_len;
    p.rec_words = 2 + p.kt;
    const int R = N > 1 ? N - 1 : 1;
    const int per_seq = R * p.chunks;
    int groups = 1;
    if (per_seq >= 160 && B > 0) {
        groups = per_seq / 16 < 16 ? per_seq / 16 : 16;
        const int room = (kMaxCounters - B) / B;
        if (groups > room) groups = room;
        if (groups < 2) groups = 1;
    }
    p.groups = groups;
    p.off_group = (size_t)B * 4;
    p.off_rec = kCounterBytes;
    p.bytes = p.off_rec + align_up_b((size_t)B * R * p.chunks * p.rec_words * 8, 256);
    return p;
}

size_t build_workspace_bytes(int B, int N, int vocab, int topk, int dtype) {
    return plan_build(B, N, vocab, topk, dtype).bytes;
}

template <typename T, int KT>
static void launch_build_t(const BuildArgs& a, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((tree_build_kernel<T, KT>), dim3(grid), dim3(kBuildThreads), 0, stream, a);
}

hipError_t launch_build(int B, int N, int vocab, const void* logits, int dtype, int topk, int cap,
                        const int32_t* budget, int32_t* parent, int32_t* token, double* score, int32_t* tree_len,
                        void* workspace, hipStream_t stream) {
    const BuildPlan p = plan_build(B, N, vocab, topk, dtype);
    char* ws = static_cast<char*>(workspace);
    BuildArgs a{};
    a.logits = logits;
    a.budget = budget;
    a.parent = parent;
    a.token = token;
    a.score = score;
    a.tree_len = tree_len;
    a.seq_count = reinterpret_cast<int*>(ws);
    a.group_count = reinterpret_cast<int*>(ws + p.off_group);
    a.rec = reinterpret_cast<unsigned long long*>(ws + p.off_rec);
    a.N = N;
    a.vocab = vocab;
    a.chunks = p.chunks;
    a.chunk_len = p.chunk_len;
    a.topk = topk;
    a.cap = cap;
    a.groups = p.groups;
    a.rec_words = p.rec_words;
    const int epv = dtype == JF_BF16 ? 8 : 4;
    a.aligned = (vocab % epv == 0) && ((reinterpret_cast<uintptr_t>(logits) & 15) == 0);
    const int R = N > 1 ? N - 1 : 1;
    const long grid = (long)B * R * p.chunks;
    if (grid <= 0) return hipSuccess;
    if (dtype == JF_BF16) {
        switch (p.kt) {
            case 1: launch_build_t<uint16_t, 1>(a, (int)grid, stream); break;
            case 2: launch_build_t<uint16_t, 2>(a, (int)grid, stream); break;
            case 4: launch_build_t<uint16_t, 4>(a, (int)grid, stream); break;
            default: launch_build_t<uint16_t, 8>(a, (int)grid, stream); break;
        }
    } else {
        switch (p.kt) {
            case 1: launch_build_t<float, 1>(a, (int)grid, stream); break;
            case 2: launch_build_t<float, 2>(a, (int)grid, stream); break;
            case 4: launch_build_t<float, 4>(a, (int)grid, stream); break;
            default: launch_build_t<float, 8>(a, (int)grid, stream); break;
        }
    }
    return hipGetLastError();
}

}  // namespace jf

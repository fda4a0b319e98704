// Greedy tree acceptance: the target's choice per node (first index of the
// row's largest logit) and the longest agreeing root-to-node path.
//
// Acceptance rule: gist.science lay summary of "JetFlow ..." and the qxai.app
// commentary (drafted tokens are kept up to the first disagreement); over a
// tree the accepted path is the longest one on which every node agrees.
//
// Logits mode runs as ONE launch. The vocabulary of each row is cut into C
// chunks; workgroup (row, chunk) streams its chunk with 16-byte loads and
// keeps the best (value, index) pair. The last chunk of a row to finish
// (agent-scope counter) merges the C pairs and writes next_tokens[row]; the
// last row of a sequence to finish then runs the walk for that sequence. All
// counters return to zero, so the workspace never needs clearing again.
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

__device__ Best block_best(Best b, Best* scratch) {
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

// One sequence's walk, run by a whole 256-thread workgroup (N <= 256).
//   mism bit u: u > 0 and draft[u] != next[parent[u]]
//   node v agrees along its path iff (anc[v] & mism) == 0
//   end node = the agreeing node with most path nodes, smallest index on ties
__device__ void walk_sequence(int b, int N, const int32_t* __restrict__ draft,
                              const int32_t* __restrict__ parent, const uint64_t* __restrict__ anc,
                              const int32_t* __restrict__ next, int32_t* __restrict__ accept_len,
                              int32_t* __restrict__ accepted_nodes, int32_t* __restrict__ bonus) {
    __shared__ uint64_t mism[kAncWords];
    __shared__ uint64_t end_set[kAncWords];
    __shared__ int keys[kAcceptThreads / kWave];
    const int u = threadIdx.x;
    const int lane = u & 63, w = u >> 6;
    const size_t base = (size_t)b * N;

    bool bad = false;
    if (u > 0 && u < N) {
        int p = parent[base + u];
        p = (p < 0) ? 0 : (p >= N ? N - 1 : p);     // memory safety on broken trees
        bad = draft[base + u] != next[base + p];
    }
    const uint64_t ballot = __ballot(bad);
    if (lane == 0) mism[w] = ballot;
    __syncthreads();

    // key = (path nodes << 16) | (0xffff - node) for agreeing nodes, else 0
    unsigned key = 0;
    uint64_t mine[kAncWords] = {0, 0, 0, 0};
    if (u < N) {
        bool ok = true;
        int cnt = 0;
        #pragma unroll
        for (int k = 0; k < kAncWords; ++k) {
            mine[k] = anc[(base + u) * kAncWords + k];
            ok = ok && ((mine[k] & mism[k]) == 0);
            cnt += __popcll(mine[k]);
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
        for (int k = 0; k < kAncWords; ++k) end_set[k] = mine[k];
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
        bonus[b] = next[base + v_end];
    }
}

// ids mode: next_tokens = target_ids, then the walk. One workgroup per sequence.
__global__ __launch_bounds__(kAcceptThreads) void accept_ids_kernel(
    int N, const int32_t* __restrict__ target_ids, const int32_t* __restrict__ draft,
    const int32_t* __restrict__ parent, const uint64_t* __restrict__ anc, int32_t* __restrict__ next_tokens,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ accepted_nodes, int32_t* __restrict__ bonus) {
    const int b = blockIdx.x;
    if (threadIdx.x < N) next_tokens[(size_t)b * N + threadIdx.x] = target_ids[(size_t)b * N + threadIdx.x];
    walk_sequence(b, N, draft, parent, anc, target_ids, accept_len, accepted_nodes, bonus);
}

template <typename T>
__device__ __forceinline__ void scan_chunk(const T* __restrict__ row, int lo, int hi, Best& b);

// bf16: 8 values per 16-byte load; the row start must be 16-byte aligned
template <>
__device__ __forceinline__ void scan_chunk<uint16_t>(const uint16_t* __restrict__ row, int lo, int hi, Best& b) {
    const int nvec = (hi - lo) >> 3;
    const u32x4* vp = reinterpret_cast<const u32x4*>(row + lo);
    constexpr int U = 4;
    int k = threadIdx.x;
    for (; k + (U - 1) * kAcceptThreads < nvec; k += U * kAcceptThreads) {
        u32x4 r[U];
        #pragma unroll
        for (int j = 0; j < U; ++j) r[j] = __builtin_nontemporal_load(vp + k + j * kAcceptThreads);
        #pragma unroll
        for (int j = 0; j < U; ++j) {
            const int i0 = lo + ((k + j * kAcceptThreads) << 3);
            #pragma unroll
            for (int e = 0; e < 4; ++e) {
                offer(b, bf16_bits_to_f32(r[j][e] & 0xffffu), i0 + 2 * e);
                offer(b, bf16_bits_to_f32(r[j][e] >> 16), i0 + 2 * e + 1);
            }
        }
    }
    for (; k < nvec; k += kAcceptThreads) {
        const u32x4 r = __builtin_nontemporal_load(vp + k);
        const int i0 = lo + (k << 3);
        #pragma unroll
        for (int e = 0; e < 4; ++e) {
            offer(b, bf16_bits_to_f32(r[e] & 0xffffu), i0 + 2 * e);
            offer(b, bf16_bits_to_f32(r[e] >> 16), i0 + 2 * e + 1);
        }
    }
    for (int i = lo + (nvec << 3) + threadIdx.x; i < hi; i += kAcceptThreads)
        offer(b, bf16_bits_to_f32(row[i]), i);
}

// fp32: 4 values per 16-byte load
template <>
__device__ __forceinline__ void scan_chunk<float>(const float* __restrict__ row, int lo, int hi, Best& b) {
    const int nvec = (hi - lo) >> 2;
    const f32x4* vp = reinterpret_cast<const f32x4*>(row + lo);
    int k = threadIdx.x;
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
    int* row_count;     // [B*N]   (workspace, zero between calls)
    int* seq_count;     // [B]     (workspace, zero between calls)
    Best* partial;      // [B*N*C] (workspace)
    int N, vocab, chunks, chunk_len;
    int aligned;        // rows start on 16-byte boundaries and chunk_len keeps them there
};

template <typename T>
__global__ __launch_bounds__(kAcceptThreads) void accept_logits_kernel(AcceptArgs a) {
    __shared__ Best scratch[kAcceptThreads / kWave];
    __shared__ int last;
    const int blk = blockIdx.x;
    const int row = blk / a.chunks, c = blk - row * a.chunks;
    const int b = row / a.N;
    const T* rp = reinterpret_cast<const T*>(a.logits) + (size_t)row * a.vocab;
    const int lo = c * a.chunk_len;
    const int hi = min(a.vocab, lo + a.chunk_len);

    Best best{-__builtin_inff(), kNoIndex};
    if (a.aligned) scan_chunk<T>(rp, lo, hi, best);
    else scan_scalar<T>(rp, lo, hi, best);
    best = block_best(best, scratch);

    if (a.chunks > 1) {
        if (threadIdx.x == 0) a.partial[blk] = best;
        __threadfence();
        __syncthreads();
        if (threadIdx.x == 0) {
            const int old = arrive(&a.row_count[row]);
            last = (old == a.chunks - 1);
            if (last) reset_counter(&a.row_count[row]);
        }
        __syncthreads();
        if (!last) return;
        __threadfence();
        // merge the row's chunk winners (order-independent: `better` is a strict total order)
        Best m{-__builtin_inff(), kNoIndex};
        for (int k = threadIdx.x; k < a.chunks; k += kAcceptThreads) {
            const Best p = a.partial[(size_t)row * a.chunks + k];
            if (p.i != kNoIndex) m = merge(m, p);
        }
        best = block_best(m, scratch);
    }
    if (threadIdx.x == 0) a.next_tokens[row] = (best.i == kNoIndex) ? 0 : best.i;

    // sequence completion: the last finished row of sequence b runs the walk
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const int old = arrive(&a.seq_count[b]);
        last = (old == a.N - 1);
        if (last) reset_counter(&a.seq_count[b]);
    }
    __syncthreads();
    if (!last) return;
    __threadfence();
    walk_sequence(b, a.N, a.draft, a.parent, a.anc, a.next_tokens, a.accept_len, a.accepted_nodes, a.bonus);
}

// ---------------------------------------------------------------- host side

struct AcceptPlan {
    int chunks, chunk_len;
    size_t off_row, off_seq, off_part, bytes;
};

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

AcceptPlan plan_accept(int B, int N, int vocab) {
    AcceptPlan p{};
    const long rows = (long)B * N;
    const int min_chunk = 4096;                        // >= 16 values per thread
    int chunks = (int)((2048 + rows - 1) / (rows > 0 ? rows : 1));   // aim for ~2048 workgroups
    const int max_chunks = (vocab + min_chunk - 1) / min_chunk;
    chunks = chunks < 1 ? 1 : chunks;
    chunks = chunks > max_chunks ? max_chunks : chunks;
    chunks = chunks < 1 ? 1 : chunks;
    int len = (vocab + chunks - 1) / chunks;
    len = (len + 7) / 8 * 8;                          // keeps 16-byte alignment of every chunk
    chunks = (vocab + len - 1) / len;
    p.chunks = chunks;
    p.chunk_len = len;
    p.off_row = 0;
    p.off_seq = align_up((size_t)rows * 4, 256);
    p.off_part = p.off_seq + align_up((size_t)B * 4, 256);
    p.bytes = p.off_part + align_up((size_t)rows * chunks * sizeof(Best), 256);
    return p;
}

hipError_t launch_accept(int B, int N, int vocab, const void* logits, int dtype, const int32_t* target_ids,
                         const int32_t* draft, const int32_t* parent, const uint64_t* anc, int32_t* next_tokens,
                         int32_t* accept_len, int32_t* accepted_nodes, int32_t* bonus, void* workspace,
                         hipStream_t stream) {
    if (B == 0) return hipSuccess;
    if (target_ids) {
        hipLaunchKernelGGL(accept_ids_kernel, dim3(B), dim3(kAcceptThreads), 0, stream, N, target_ids, draft,
                           parent, anc, next_tokens, accept_len, accepted_nodes, bonus);
        return hipGetLastError();
    }
    const AcceptPlan p = plan_accept(B, N, vocab);
    char* ws = static_cast<char*>(workspace);
    AcceptArgs a;
    a.logits = logits;
    a.draft = draft;
    a.parent = parent;
    a.anc = anc;
    a.next_tokens = next_tokens;
    a.accept_len = accept_len;
    a.accepted_nodes = accepted_nodes;
    a.bonus = bonus;
    a.row_count = reinterpret_cast<int*>(ws + p.off_row);
    a.seq_count = reinterpret_cast<int*>(ws + p.off_seq);
    a.partial = reinterpret_cast<Best*>(ws + p.off_part);
    a.N = N;
    a.vocab = vocab;
    a.chunks = p.chunks;
    a.chunk_len = p.chunk_len;
    const size_t elt = dtype == JF_BF16 ? 2 : 4;
    a.aligned = ((reinterpret_cast<uintptr_t>(logits) % 16) == 0) && (((size_t)vocab * elt) % 16 == 0);
    const dim3 grid((unsigned)((long)B * N * p.chunks));
    if (dtype == JF_BF16)
        hipLaunchKernelGGL(accept_logits_kernel<uint16_t>, grid, dim3(kAcceptThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(accept_logits_kernel<float>, grid, dim3(kAcceptThreads), 0, stream, a);
    return hipGetLastError();
}

size_t accept_workspace_bytes(int B, int N, int vocab) { return plan_accept(B, N, vocab).bytes; }

}  // namespace jf

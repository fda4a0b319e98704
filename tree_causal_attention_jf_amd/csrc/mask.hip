// Ancestor bitset of a batch of draft trees.
//
// Definition ("JetFlow ..." gist.science technical summary, section 2,
// tree-causal attention mask): node i sees the nodes on its root-to-i path,
// itself included. Encoded as 256 bits per node (4 x uint64, node j = bit
// j % 64 of word j / 64).
//
// One workgroup per tree, one thread per node. The path sets are built by
// pointer doubling in LDS: after round k a node holds every node within
// distance < 2^k above it and a pointer to its 2^k-th ancestor, so
// ceil(log2 N) <= 8 rounds cover any tree of up to 256 nodes.
#include "jf_common.h"

namespace jf {

__global__ __launch_bounds__(256) void ancestor_mask_kernel(const int32_t* __restrict__ parent, int N,
                                                            uint64_t* __restrict__ anc,
                                                            int32_t* __restrict__ depth,
                                                            int32_t* __restrict__ bad_tree) {
    __shared__ uint64_t set[2][JF_MAX_NODES][kAncWords];
    __shared__ int16_t up[2][JF_MAX_NODES];
    __shared__ int any_bad;
    const int b = blockIdx.x;
    const int i = threadIdx.x;
    if (i == 0) any_bad = 0;
    __syncthreads();

    int p = -1;
    if (i < N) {
        p = parent[(size_t)b * N + i];
        const bool ok = (i == 0) ? (p == -1) : (p >= 0 && p < i);
        if (!ok) {
            any_bad = 1;     // benign race: every writer stores 1
            p = -1;          // a broken link is read as a root
        }
        #pragma unroll
        for (int w = 0; w < kAncWords; ++w) set[0][i][w] = (w == (i >> 6)) ? (1ull << (i & 63)) : 0ull;
        up[0][i] = (int16_t)p;
    }
    __syncthreads();

    int cur = 0;
    for (int round = 0; round < 8; ++round) {
        int more = 0;
        if (i < N) {
            const int j = up[cur][i];
            uint64_t s[kAncWords];
            #pragma unroll
            for (int w = 0; w < kAncWords; ++w) s[w] = set[cur][i][w];
            int jj = -1;
            if (j >= 0) {
                #pragma unroll
                for (int w = 0; w < kAncWords; ++w) s[w] |= set[cur][j][w];
                jj = up[cur][j];
            }
            #pragma unroll
            for (int w = 0; w < kAncWords; ++w) set[cur ^ 1][i][w] = s[w];
            up[cur ^ 1][i] = (int16_t)jj;
            more = (jj >= 0);
        }
        cur ^= 1;
        if (!__syncthreads_or(more)) break;
    }

    if (i < N) {
        const size_t row = (size_t)b * N + i;
        int cnt = 0;
        #pragma unroll
        for (int w = 0; w < kAncWords; ++w) {
            const uint64_t v = set[cur][i][w];
            anc[row * kAncWords + w] = v;
            cnt += __popcll(v);
        }
        if (depth) depth[row] = cnt;
    }
    if (i == 0 && bad_tree) bad_tree[b] = any_bad;
}

hipError_t launch_ancestor_mask(const int32_t* parent, int B, int N, uint64_t* anc, int32_t* depth,
                                int32_t* bad_tree, hipStream_t stream) {
    hipLaunchKernelGGL(ancestor_mask_kernel, dim3(B), dim3(256), 0, stream, parent, N, anc, depth, bad_tree);
    return hipGetLastError();
}

}  // namespace jf

// Append each sequence's accepted path to its paged KV cache.
//
// What is computed: the target keeps the drafted tokens up to its first
// disagreement (lay summary and qxai.app commentary), and the prefix the next
// step attends to lives in a paged KV cache ("JetFlow ..." gist.science
// technical summary, section 3). Node 0 of a tree is the last committed token,
// whose K/V was computed together with the tree, so prefix token
// prefix_len[b] + i of sequence b receives the K and V of node
// accepted_nodes[b, i], for i = 0 .. accept_len[b].
//
// One workgroup per (path position i, sequence b). Each workgroup first checks
// its whole sequence -- the length, every path entry, and every page slot the
// new tokens land in -- so that a sequence is committed entirely or not at
// all, then copies one token's K and V rows (Hkv x D elements each) with
// 16-byte loads and stores.
#include "jf_common.h"

namespace jf {

constexpr int kCommitThreads = 256;

__global__ __launch_bounds__(kCommitThreads) void commit_kernel(
    const char* __restrict__ k_tree, const char* __restrict__ v_tree, const int32_t* __restrict__ accept_len,
    const int32_t* __restrict__ accepted_nodes, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ prefix_len, char* __restrict__ k_pages, char* __restrict__ v_pages,
    int32_t* __restrict__ new_prefix_len, int N, int Hkv, int row_bytes, int num_pages, int max_pages) {
    const int i = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    const int L = prefix_len[b];
    const int a = accept_len[b];
    const bool head_ok = L >= 0 && a >= 0 && a < N;
    int bad = head_ok ? 0 : 1;
    if (head_ok) {
        // path entries 0..a (a < N <= 256: one per thread)
        if (t <= a) {
            const int n = accepted_nodes[(size_t)b * N + t];
            if (n < 0 || n >= N) bad = 1;
        }
        // page slots of tokens L..L+a: at most 17, one per thread
        const long first = (long)L / JF_PAGE_SIZE, last = ((long)L + a) / JF_PAGE_SIZE;
        const long slot = first + t;
        if (slot <= last) {
            if (slot >= max_pages) {
                bad = 1;
            } else {
                const int pid = block_table[(size_t)b * max_pages + slot];
                if (pid < 0 || pid >= num_pages) bad = 1;
            }
        }
    }
    const bool ok = !__syncthreads_or(bad);
    if (i == 0 && t == 0) new_prefix_len[b] = ok ? L + a + 1 : -1;
    if (!ok || i > a) return;

    const int n = accepted_nodes[(size_t)b * N + i];
    const long pos = (long)L + i;
    const size_t page = (size_t)block_table[(size_t)b * max_pages + pos / JF_PAGE_SIZE];
    const int in_page = (int)(pos % JF_PAGE_SIZE);
    const int cpr = row_bytes / 16;                       // 16-byte chunks per row
    const size_t src = ((size_t)b * N + n) * Hkv * row_bytes;
    for (int c = t; c < Hkv * cpr; c += kCommitThreads) {
        const int h = c / cpr, part = c - h * cpr;
        const size_t s_off = src + (size_t)h * row_bytes + (size_t)part * 16;
        const size_t d_off = ((page * Hkv + h) * JF_PAGE_SIZE + in_page) * (size_t)row_bytes + (size_t)part * 16;
        *reinterpret_cast<u32x4*>(k_pages + d_off) = *reinterpret_cast<const u32x4*>(k_tree + s_off);
        *reinterpret_cast<u32x4*>(v_pages + d_off) = *reinterpret_cast<const u32x4*>(v_tree + s_off);
    }
}

hipError_t launch_commit(const jf_attn_shape& s, const void* k_tree, const void* v_tree, const int32_t* accept_len,
                         const int32_t* accepted_nodes, const int32_t* block_table, const int32_t* prefix_len,
                         void* k_pages, void* v_pages, int32_t* new_prefix_len, hipStream_t stream) {
    const int elt = s.dtype == JF_BF16 ? 2 : 4;
    hipLaunchKernelGGL(commit_kernel, dim3((unsigned)s.N, (unsigned)s.B), dim3(kCommitThreads), 0, stream,
                       static_cast<const char*>(k_tree), static_cast<const char*>(v_tree), accept_len,
                       accepted_nodes, block_table, prefix_len, static_cast<char*>(k_pages),
                       static_cast<char*>(v_pages), new_prefix_len, s.N, s.Hkv, s.D * elt, s.num_pages,
                       s.max_pages_per_seq);
    return hipGetLastError();
}

}  // namespace jf

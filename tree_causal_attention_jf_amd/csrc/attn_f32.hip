// Tree-causal attention over a paged prefix, fp32 inputs, fp32 arithmetic.
//
// Same operation as the bf16 kernel ("JetFlow ..." gist.science technical
// summary, section 2 mask, section 3 paged verification), computed entirely
// in fp32 with vector FMAs: the small-model / exact-check path.
//
// One workgroup per (sequence, KV head, 64 packed query rows); 4 threads per
// row, each holding a quarter of the head dimension of q and of the output.
// Keys stream through LDS in tiles of 32 (two pages, then the tree); per tile
// the 32 scores are formed with a 4-lane shuffle reduction, the online
// softmax is updated once, and the values are accumulated.
#include "jf_common.h"

namespace jf {

struct AttnF32Args {
    const float* q;
    const float* kp;
    const float* vp;
    const int32_t* block_table;
    const int32_t* prefix_len;
    const float* kt;
    const float* vt;
    const uint64_t* anc;
    float* out;
    float* lse;
    int B, N, Hq, Hkv, G, num_pages, max_pages, max_prefix, rows, nrb;
    float scale_log2;
};

constexpr int kF32Rows = 64;
constexpr int kF32Keys = 32;

template <int D>
__global__ __launch_bounds__(256) void tree_attn_f32_kernel(AttnF32Args a) {
    constexpr int DP = D / 4;
    __shared__ __attribute__((aligned(16))) float Ks[kF32Keys][D];
    __shared__ __attribute__((aligned(16))) float Vs[kF32Keys][D];
    __shared__ int s_bad;

    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int rb = lid % a.nrb;
    const int kvh = (lid / a.nrb) % a.Hkv;
    const int b = lid / (a.nrb * a.Hkv);
    const int tid = threadIdx.x;
    const int part = tid & 3;
    const int row = rb * kF32Rows + (tid >> 2);
    const bool row_ok = row < a.rows;
    const int node = row_ok ? row / a.G : 0;
    const int head = kvh * a.G + (row_ok ? row % a.G : 0);

    int L = a.prefix_len[b];
    bool bad = (L < 0 || L > a.max_prefix);
    if (bad) L = 0;
    if (tid == 0) s_bad = 0;

    float qv[DP], ov[DP];
    const float* qp = a.q + (((long)b * a.N + node) * a.Hq + head) * D + part * DP;
    #pragma unroll
    for (int i = 0; i < DP; ++i) {
        qv[i] = row_ok ? qp[i] : 0.f;
        ov[i] = 0.f;
    }
    uint64_t ancw[kAncWords] = {0, 0, 0, 0};
    if (row_ok) {
        #pragma unroll
        for (int k = 0; k < kAncWords; ++k) ancw[k] = a.anc[((long)b * a.N + node) * kAncWords + k];
    }
    float m_run = -__builtin_inff(), l_run = 0.f;
    const int n_pre = (L + kF32Keys - 1) / kF32Keys;
    const int n_tree = (a.N + kF32Keys - 1) / kF32Keys;
    __syncthreads();

    for (int it = 0; it < n_pre + n_tree; ++it) {
        const bool tree = it >= n_pre;
        const int t0 = tree ? (it - n_pre) * kF32Keys : it * kF32Keys;
        const int limit = tree ? a.N : L;
        // stage 32 keys x D of K and V (zero outside the valid range)
        for (int e = tid; e < kF32Keys * D / 4; e += 256) {
            const int k = e / (D / 4), c = e % (D / 4);
            const int t = t0 + k;
            f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
            if (t < limit) {
                long off;
                if (tree) {
                    off = (((long)b * a.N + t) * a.Hkv + kvh) * D;
                } else {
                    int page = a.block_table[(long)b * a.max_pages + (t >> 4)];
                    if (page < 0 || page >= a.num_pages) {
                        s_bad = 1;
                        page = 0;
                    }
                    off = (((long)page * a.Hkv + kvh) * kPage + (t & 15)) * D;
                }
                kv = *reinterpret_cast<const f32x4*>((tree ? a.kt : a.kp) + off + 4 * c);
                vv = *reinterpret_cast<const f32x4*>((tree ? a.vt : a.vp) + off + 4 * c);
            }
            *reinterpret_cast<f32x4*>(&Ks[k][4 * c]) = kv;
            *reinterpret_cast<f32x4*>(&Vs[k][4 * c]) = vv;
        }
        __syncthreads();
        float s[kF32Keys];
        float mx = -__builtin_inff();
        const uint64_t mw = tree ? (t0 < 64 ? ancw[0] : t0 < 128 ? ancw[1] : t0 < 192 ? ancw[2] : ancw[3]) : 0ull;
        #pragma unroll
        for (int k = 0; k < kF32Keys; ++k) {
            float dot = 0.f;
            #pragma unroll
            for (int i = 0; i < DP; ++i) dot = __builtin_fmaf(qv[i], Ks[k][part * DP + i], dot);
            dot += __shfl_xor(dot, 1);
            dot += __shfl_xor(dot, 2);
            const int t = t0 + k;
            bool vis = t < limit;
            if (tree) vis = vis && ((mw >> ((t0 + k) & 63)) & 1ull);
            s[k] = vis ? dot * a.scale_log2 : -__builtin_inff();
            mx = fmaxf(mx, s[k]);
        }
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);
        l_run *= alpha;
        #pragma unroll
        for (int i = 0; i < DP; ++i) ov[i] *= alpha;
        #pragma unroll
        for (int k = 0; k < kF32Keys; ++k) {
            const float p = exp2f(s[k] - m_use);
            l_run += p;
            #pragma unroll
            for (int i = 0; i < DP; ++i) ov[i] = __builtin_fmaf(p, Vs[k][part * DP + i], ov[i]);
        }
        m_run = m_new;
        __syncthreads();
    }
    bad = bad || s_bad;
    if (!row_ok) return;
    const float NANF = __builtin_nanf("");
    const float inv = bad ? NANF : 1.f / l_run;
    float* op = a.out + (((long)b * a.N + node) * a.Hq + head) * D + part * DP;
    #pragma unroll
    for (int i = 0; i < DP; ++i) op[i] = ov[i] * inv;
    if (a.lse && part == 0)
        a.lse[((long)b * a.N + node) * a.Hq + head] = bad ? NANF : (m_run + log2f(l_run)) * 0.69314718055994530942f;
}

hipError_t launch_attention_f32(const jf_attn_shape& s, int max_prefix, const void* q, const void* k_pages,
                                const void* v_pages, const int32_t* block_table, const int32_t* prefix_len,
                                const void* k_tree, const void* v_tree, const uint64_t* anc, void* out,
                                float* lse, hipStream_t stream) {
    AttnF32Args a;
    a.q = static_cast<const float*>(q);
    a.kp = static_cast<const float*>(k_pages);
    a.vp = static_cast<const float*>(v_pages);
    a.block_table = block_table;
    a.prefix_len = prefix_len;
    a.kt = static_cast<const float*>(k_tree);
    a.vt = static_cast<const float*>(v_tree);
    a.anc = anc;
    a.out = static_cast<float*>(out);
    a.lse = lse;
    a.B = s.B;
    a.N = s.N;
    a.Hq = s.Hq;
    a.Hkv = s.Hkv;
    a.G = s.Hq / s.Hkv;
    a.num_pages = s.num_pages;
    a.max_pages = s.max_pages_per_seq;
    a.max_prefix = max_prefix;
    a.rows = a.G * s.N;
    a.nrb = (a.rows + kF32Rows - 1) / kF32Rows;
    a.scale_log2 = s.sm_scale * 1.44269504088896340736f;
    const long grid = (long)s.B * s.Hkv * a.nrb;
    if (grid == 0) return hipSuccess;
    if (s.D == 128)
        hipLaunchKernelGGL(tree_attn_f32_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(tree_attn_f32_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace jf

// Tree-causal attention over a paged prefix, bf16 inputs, gfx950 matrix cores.
//
// What is computed ("JetFlow ..." gist.science technical summary: section 2,
// tree-causal attention mask; section 3, verification over a paged KV cache):
// for node i of sequence b and query head h,
//   out[b,i,h] = softmax_j(sm_scale * q[b,i,h] . k_j) v_j
// over the L_b prefix keys plus the tree keys j that lie on the root-to-i path
// (bit j of anc[b,i]); KV head = h / G with G = Hq / Hkv.
//
// Work decomposition
//   * GQA packing: the G*N query rows that share one KV head form one matrix
//     (row r = node * G + g), so every K/V tile is staged once per KV head.
//   * A workgroup owns RB = 32 * NW consecutive rows (NW waves, 32 rows per
//     wave) of one (sequence, KV head) and a contiguous run of prefix pages
//     (a "split"). The split that owns the last prefix page also runs the tree
//     block. Splits of one row block are merged in the same launch by the last
//     one to finish (agent-scope counter), in split order.
//   * Workgroup ids are remapped so that the row blocks and splits of one KV
//     head land on one XCD and share its L2.
//
// Per 64-key tile, per wave (32 query rows):
//   S^T[key, row] = K_tile Q^T         8 (D=128) v_mfma_f32_32x32x16_bf16 per 32 keys
//   online softmax in fp32 per row (exp2 with the scale folded into log2 e)
//   O^T[d, row]  += V_tile^T P^T       P is rounded to bf16 for the product
// With S^T in the matrix-core output layout each lane owns one query row and
// 16 keys per 32-key block, so the 256-bit ancestor bitset of that row's node
// sits in the lane's registers and masking is a per-register bit test.
//
// LDS layout (16-byte chunks, XOR-swizzled so the matrix-operand reads are
// bank-conflict free):
//   K  [64 keys][D]   chunk c of key k stored at chunk c ^ (k & 7)
//   V^T[D][64 keys]   keys permuted inside each 16-key group so one 16-byte
//                     read gives a lane the 8 keys its P^T registers hold;
//                     chunk c of row d stored at c ^ ((d ^ (d >> 3)) & 7)
// Global -> register -> LDS staging is double buffered: the loads of tile t+1
// are in flight while tile t is multiplied.
#include "jf_common.h"

namespace jf {

constexpr int kKeyTile = 64;
constexpr int kMaxPagesPerSplit = 1024;

struct AttnArgs {
    const uint16_t* q;
    const uint16_t* kp;
    const uint16_t* vp;
    const int32_t* block_table;
    const int32_t* prefix_len;
    const uint16_t* kt;
    const uint16_t* vt;
    const uint64_t* anc;
    uint16_t* out;
    float* lse;
    int* counters;     // [items]                       zero between calls
    float* part_ml;    // [items][splits][RB][2]        (m in log2 units, l)
    float* part_o;     // [items][splits][RB][D]        unnormalised
    int B, N, Hq, Hkv, G, num_pages, max_pages, max_prefix;
    int rows;          // G * N
    int nrb;           // row blocks per (sequence, KV head)
    int splits;        // splits per row block in the grid
    int pps;           // prefix pages per split (multiple of 4)
    float scale_log2;  // sm_scale * log2(e)
};

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

template <int D, int NW>
struct Tile {
    static constexpr int T = NW * kWave;          // threads
    static constexpr int CPR = D / 8;             // 16-byte chunks per key row
    static constexpr int KCH = kKeyTile * CPR / T;                   // K chunks per thread
    static constexpr int VUNITS = (kKeyTile / 4) * CPR;              // 4-key x 8-d units
    static constexpr int VU = (VUNITS + T - 1) / T;                  // V units per thread
    static constexpr int K_BYTES = kKeyTile * D * 2;
    static constexpr int V_BYTES = D * kKeyTile * 2;
    static constexpr int BUF_BYTES = K_BYTES + V_BYTES;
    static_assert(kKeyTile * CPR % T == 0, "K tile must split evenly over threads");
};

// Byte offset of 16-byte chunk c of key k in the K tile.
template <int D>
__device__ __forceinline__ int k_off(int k, int c) {
    return k * (D * 2) + ((c ^ (k & 7)) << 4);
}

__device__ __forceinline__ int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }

// Byte offset of 16-byte chunk c of row d in the V^T tile (64 keys = 128 bytes per row).
__device__ __forceinline__ int vt_off(int d, int c) { return d * (kKeyTile * 2) + ((c ^ vt_swz(d)) << 4); }

template <int D, int NW>
struct Stage {
    u32x4 k[Tile<D, NW>::KCH];
    u32x4 v[Tile<D, NW>::VU][4];
};

// Element offset (within k_pages/v_pages or k_tree/v_tree) of key `key` of a
// tile, or -1 when that key is outside the tile's valid range.
struct TileSrc {
    bool tree;
    int t0;        // prefix: first token of the tile; tree: first node
    int limit;     // prefix: one past the last valid token; tree: N
};

template <int D>
__device__ __forceinline__ long key_elem(const AttnArgs& a, const TileSrc& src, int key, int b, int kvh,
                                         int p_begin, const int* s_pages) {
    const int t = src.t0 + key;
    if (t >= src.limit) return -1;
    if (src.tree) return (((long)b * a.N + t) * a.Hkv + kvh) * D;
    const int page = s_pages[(t >> 4) - p_begin];
    return (((long)page * a.Hkv + kvh) * kPage + (t & 15)) * D;
}

template <int D, int NW>
__device__ __forceinline__ void load_tile(const AttnArgs& a, const TileSrc& src, int b, int kvh, int p_begin,
                                          const int* s_pages, Stage<D, NW>& st) {
    using TL = Tile<D, NW>;
    const uint16_t* kb = src.tree ? a.kt : a.kp;
    const uint16_t* vb = src.tree ? a.vt : a.vp;
    const int tid = threadIdx.x;
    #pragma unroll
    for (int i = 0; i < TL::KCH; ++i) {
        const int id = tid + i * TL::T;
        const int key = id / TL::CPR, c = id % TL::CPR;
        const long e = key_elem<D>(a, src, key, b, kvh, p_begin, s_pages);
        st.k[i] = e >= 0 ? ld16(kb + e + c * 8) : u32x4{0, 0, 0, 0};
    }
    #pragma unroll
    for (int i = 0; i < TL::VU; ++i) {
        const int uid = tid + i * TL::T;
        const int kg = uid / TL::CPR, dc = uid % TL::CPR;
        #pragma unroll
        for (int j = 0; j < 4; ++j) {
            long e = -1;
            if (uid < TL::VUNITS) e = key_elem<D>(a, src, 4 * kg + j, b, kvh, p_begin, s_pages);
            st.v[i][j] = e >= 0 ? ld16(vb + e + dc * 8) : u32x4{0, 0, 0, 0};
        }
    }
}

template <int D, int NW>
__device__ __forceinline__ void store_tile(char* buf, const Stage<D, NW>& st) {
    using TL = Tile<D, NW>;
    const int tid = threadIdx.x;
    #pragma unroll
    for (int i = 0; i < TL::KCH; ++i) {
        const int id = tid + i * TL::T;
        const int key = id / TL::CPR, c = id % TL::CPR;
        *reinterpret_cast<u32x4*>(buf + k_off<D>(key, c)) = st.k[i];
    }
    char* vbuf = buf + TL::K_BYTES;
    #pragma unroll
    for (int i = 0; i < TL::VU; ++i) {
        const int uid = tid + i * TL::T;
        if (uid >= TL::VUNITS) continue;
        const int kg = uid / TL::CPR, dc = uid % TL::CPR;
        // keys 4kg..4kg+3 go to positions 16*(kg/4) + 4*qq, with the two middle
        // 4-key groups of each 16-key block swapped (matches the P^T registers)
        const int q4 = kg & 3;
        const int qq = ((q4 & 1) << 1) | (q4 >> 1);
        const int chunk = 2 * (kg >> 2) + (qq >> 1);
        const int half = (qq & 1) * 8;
        #pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t r0 = st.v[i][0][m], r1 = st.v[i][1][m], r2 = st.v[i][2][m], r3 = st.v[i][3][m];
            const int d0 = 8 * dc + 2 * m;
            // even element of the pair: low halves; odd: high halves
            u32x2 lo = {(r0 & 0xffffu) | (r1 << 16), (r2 & 0xffffu) | (r3 << 16)};
            u32x2 hi = {(r0 >> 16) | (r1 & 0xffff0000u), (r2 >> 16) | (r3 & 0xffff0000u)};
            *reinterpret_cast<u32x2*>(vbuf + vt_off(d0, chunk) + half) = lo;
            *reinterpret_cast<u32x2*>(vbuf + vt_off(d0 + 1, chunk) + half) = hi;
        }
    }
}

__device__ __forceinline__ uint64_t pick_word(const uint64_t w[4], int i) {
    return i == 0 ? w[0] : i == 1 ? w[1] : i == 2 ? w[2] : w[3];
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 2) void tree_attn_bf16_kernel(AttnArgs a) {
    using TL = Tile<D, NW>;
    constexpr int RB = NW * 32;
    constexpr int DCH = D / 16;     // k-steps of the QK product
    constexpr int DT = D / 32;      // 32-wide d tiles of O^T
    __shared__ __attribute__((aligned(16))) char lds[2][TL::BUF_BYTES];
    __shared__ int s_pages[kMaxPagesPerSplit];
    __shared__ unsigned long long s_union[kAncWords];
    __shared__ int s_last;

    // ---- which (sequence, KV head, split, row block) this workgroup owns
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int rb = lid % a.nrb;
    int t1 = lid / a.nrb;
    const int s = t1 % a.splits;
    t1 /= a.splits;
    const int kvh = t1 % a.Hkv;
    const int b = t1 / a.Hkv;
    const int item = (b * a.Hkv + kvh) * a.nrb + rb;

    int L = a.prefix_len[b];
    bool bad = (L < 0 || L > a.max_prefix);
    if (bad) L = 0;
    const int npages = (L + kPage - 1) / kPage;
    int n_act = (npages + a.pps - 1) / a.pps;
    if (n_act < 1) n_act = 1;
    if (s >= n_act) return;                                   // uniform: the whole workgroup leaves
    const int p_begin = s * a.pps;
    const int p_end = min(npages, p_begin + a.pps);
    const int tok_begin = p_begin * kPage;
    const int tok_end = min(L, p_end * kPage);
    const bool has_tree = (s == n_act - 1);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int hf = lane >> 5, l32 = lane & 31;
    const int row = rb * RB + w * 32 + l32;
    const bool row_ok = row < a.rows;
    const int node = row_ok ? row / a.G : 0;
    const int head = kvh * a.G + (row_ok ? row % a.G : 0);

    // ---- Q rows of this wave -> registers (B operand: lane = row, 8 d values per k-step)
    bf16x8 qreg[DCH];
    {
        const uint16_t* qp = a.q + (((long)b * a.N + node) * a.Hq + head) * D + 8 * hf;
        #pragma unroll
        for (int c = 0; c < DCH; ++c) {
            const u32x4 v = row_ok ? ld16(qp + 16 * c) : u32x4{0, 0, 0, 0};
            qreg[c] = __builtin_bit_cast(bf16x8, v);
        }
    }
    uint64_t ancw[kAncWords] = {0, 0, 0, 0};
    if (tid < kAncWords) s_union[tid] = 0;
    __syncthreads();
    if (has_tree && row_ok) {
        #pragma unroll
        for (int k = 0; k < kAncWords; ++k) ancw[k] = a.anc[((long)b * a.N + node) * kAncWords + k];
        if (row % a.G == 0) {
            #pragma unroll
            for (int k = 0; k < kAncWords; ++k)
                if (ancw[k]) atomicOr(&s_union[k], (unsigned long long)ancw[k]);
        }
    }
    int my_bad = 0;
    for (int i = tid; i < p_end - p_begin; i += TL::T) {
        int pid = a.block_table[(long)b * a.max_pages + p_begin + i];
        if (pid < 0 || pid >= a.num_pages) {
            my_bad = 1;
            pid = 0;
        }
        s_pages[i] = pid;
    }
    bad = __syncthreads_or(my_bad) || bad;

    // ---- tile list: prefix tiles, then the non-empty tree tiles
    const int n_pre = (tok_end - tok_begin + kKeyTile - 1) / kKeyTile;
    int tree_list = 0, n_tree = 0;   // up to 4 tile ids, 2 bits each
    if (has_tree) {
        for (int tt = 0; tt * kKeyTile < a.N; ++tt) {
            if (s_union[tt]) {
                tree_list |= tt << (2 * n_tree);
                ++n_tree;
            }
        }
    }
    const int n_tiles = n_pre + n_tree;

    auto tile_src = [&](int it) {
        TileSrc src;
        if (it < n_pre) {
            src.tree = false;
            src.t0 = tok_begin + it * kKeyTile;
            src.limit = tok_end;
        } else {
            src.tree = true;
            src.t0 = ((tree_list >> (2 * (it - n_pre))) & 3) * kKeyTile;
            src.limit = a.N;
        }
        return src;
    };

    f32x16 oacc[DT];
    #pragma unroll
    for (int i = 0; i < DT; ++i) oacc[i] = f32x16{};
    const float NEG = -__builtin_inff();
    float m_run = NEG;
    float l_run = 0.f;

    Stage<D, NW> stage;
    if (n_tiles > 0) {
        load_tile<D, NW>(a, tile_src(0), b, kvh, p_begin, s_pages, stage);
        store_tile<D, NW>(lds[0], stage);
    }
    __syncthreads();

    for (int it = 0; it < n_tiles; ++it) {
        const TileSrc src = tile_src(it);
        if (it + 1 < n_tiles) load_tile<D, NW>(a, tile_src(it + 1), b, kvh, p_begin, s_pages, stage);
        const char* kbuf = lds[it & 1];
        const char* vbuf = kbuf + TL::K_BYTES;

        // S^T = K Q^T for two 32-key halves
        f32x16 sacc[2] = {f32x16{}, f32x16{}};
        #pragma unroll
        for (int c = 0; c < DCH; ++c) {
            #pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int key = h2 * 32 + l32;
                const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kbuf + k_off<D>(key, 2 * c + hf));
                sacc[h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qreg[c], sacc[h2], 0, 0, 0);
            }
        }
        // register r of half h2 holds key h2*32 + 8*(r/4) + 4*hf + r%4 of the tile
        if (src.tree) {
            const int tt = src.t0 / kKeyTile;
            const int left = a.N - src.t0;
            uint64_t mw = pick_word(ancw, tt);
            if (left < 64) mw &= (1ull << left) - 1ull;
            mw >>= 4 * hf;
            const uint32_t lo = (uint32_t)mw, hi = (uint32_t)(mw >> 32);
            #pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int sh = 8 * (r >> 2) + (r & 3);
                if (!((lo >> sh) & 1u)) sacc[0][r] = NEG;
                if (!((hi >> sh) & 1u)) sacc[1][r] = NEG;
            }
        } else if (src.t0 + kKeyTile > src.limit) {
            const int nvalid = src.limit - src.t0 - 4 * hf;
            #pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kk = 8 * (r >> 2) + (r & 3);
                if (kk >= nvalid) sacc[0][r] = NEG;
                if (kk + 32 >= nvalid) sacc[1][r] = NEG;
            }
        }
        // online softmax (log2 domain)
        float mx = NEG;
        #pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(sacc[0][r], sacc[1][r]));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx * a.scale_log2);
        const float m_use = (m_new == NEG) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float rs = 0.f;
        uint32_t pk[2][8];
        #pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            #pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[h2][r], a.scale_log2, -m_use));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[h2][r + 1], a.scale_log2, -m_use));
                rs += p0 + p1;
                pk[h2][r >> 1] = pack_bf16x2(p0, p1);
            }
        }
        l_run = l_run * alpha + rs;
        m_run = m_new;
        #pragma unroll
        for (int i = 0; i < DT; ++i) oacc[i] *= alpha;

        // O^T += V^T P^T, 16 keys per step
        #pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            const int h2 = kc >> 1, o4 = (kc & 1) * 4;
            const u32x4 pw = {pk[h2][o4], pk[h2][o4 + 1], pk[h2][o4 + 2], pk[h2][o4 + 3]};
            const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
            #pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int d = dt * 32 + l32;
                const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vbuf + vt_off(d, 2 * kc + hf));
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, oacc[dt], 0, 0, 0);
            }
        }
        if (it + 1 < n_tiles) store_tile<D, NW>(lds[(it + 1) & 1], stage);
        __syncthreads();
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float NANF = __builtin_nanf("");
    const float LN2 = 0.69314718055994530942f;

    if (n_act == 1) {
        if (row_ok) {
            const float inv = bad ? NANF : 1.f / l_tot;
            uint16_t* op = a.out + (((long)b * a.N + node) * a.Hq + head) * D + 4 * hf;
            #pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                #pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const u32x2 v = {pack_bf16x2(oacc[dt][4 * rq] * inv, oacc[dt][4 * rq + 1] * inv),
                                     pack_bf16x2(oacc[dt][4 * rq + 2] * inv, oacc[dt][4 * rq + 3] * inv)};
                    *reinterpret_cast<u32x2*>(op + dt * 32 + 8 * rq) = v;
                }
            }
            if (a.lse && hf == 0)
                a.lse[((long)b * a.N + node) * a.Hq + head] = bad ? NANF : (m_run + __log2f(l_tot)) * LN2;
        }
        return;
    }

    // ---- several splits: publish this split's partial result
    {
        const long pr = ((long)item * a.splits + s) * RB + (row - rb * RB);
        float* po = a.part_o + pr * D + 4 * hf;
        #pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            #pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const f32x4 v = {oacc[dt][4 * rq], oacc[dt][4 * rq + 1], oacc[dt][4 * rq + 2], oacc[dt][4 * rq + 3]};
                *reinterpret_cast<f32x4*>(po + dt * 32 + 8 * rq) = v;
            }
        }
        if (hf == 0) {
            a.part_ml[pr * 2 + 0] = bad ? NANF : m_run;
            a.part_ml[pr * 2 + 1] = bad ? NANF : l_tot;
        }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const int old = arrive(&a.counters[item]);
        s_last = (old == n_act - 1);
        if (s_last) reset_counter(&a.counters[item]);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    // ---- last split to finish: merge all splits of this row block, in split order
    {
        constexpr int TPR = TL::T / RB;            // threads per row (2)
        constexpr int DPT = D / TPR;               // d values per thread
        const int rl = tid / TPR, part = tid % TPR;
        const int grow = rb * RB + rl;
        if (grow < a.rows) {
            const long base = (long)item * a.splits * RB + rl;   // + sp * RB
            float M = NEG;
            for (int sp = 0; sp < n_act; ++sp) M = fmaxf(M, a.part_ml[(base + (long)sp * RB) * 2]);
            const float M_use = (M == NEG) ? 0.f : M;
            float acc[DPT];
            #pragma unroll
            for (int i = 0; i < DPT; ++i) acc[i] = 0.f;
            float Ls = 0.f;
            for (int sp = 0; sp < n_act; ++sp) {
                const long pr = base + (long)sp * RB;
                const float wgt = __builtin_amdgcn_exp2f(a.part_ml[pr * 2] - M_use);
                Ls += wgt * a.part_ml[pr * 2 + 1];
                const f32x4* src = reinterpret_cast<const f32x4*>(a.part_o + pr * D + part * DPT);
                #pragma unroll
                for (int i = 0; i < DPT / 4; ++i) {
                    const f32x4 v = src[i];
                    acc[4 * i] += wgt * v[0];
                    acc[4 * i + 1] += wgt * v[1];
                    acc[4 * i + 2] += wgt * v[2];
                    acc[4 * i + 3] += wgt * v[3];
                }
            }
            const int gnode = grow / a.G, ghead = kvh * a.G + grow % a.G;
            const float inv = 1.f / Ls;
            uint16_t* op = a.out + (((long)b * a.N + gnode) * a.Hq + ghead) * D + part * DPT;
            #pragma unroll
            for (int i = 0; i < DPT / 8; ++i) {
                const u32x4 v = {pack_bf16x2(acc[8 * i] * inv, acc[8 * i + 1] * inv),
                                 pack_bf16x2(acc[8 * i + 2] * inv, acc[8 * i + 3] * inv),
                                 pack_bf16x2(acc[8 * i + 4] * inv, acc[8 * i + 5] * inv),
                                 pack_bf16x2(acc[8 * i + 6] * inv, acc[8 * i + 7] * inv)};
                *reinterpret_cast<u32x4*>(op + 8 * i) = v;
            }
            if (a.lse && part == 0) a.lse[((long)b * a.N + gnode) * a.Hq + ghead] = (M + __log2f(Ls)) * LN2;
        }
    }
}

// ---------------------------------------------------------------- host side

struct AttnPlanBf16 {
    int nw, rb, nrb, items, splits, pps;
    long grid;
    size_t off_cnt, off_ml, off_o, bytes;
};

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

static int env_int(const char* name, int dflt) {
    const char* v = getenv(name);
    if (!v || !*v) return dflt;
    return atoi(v);
}

AttnPlanBf16 plan_attention_bf16(const jf_attn_shape& s, int max_prefix) {
    AttnPlanBf16 p{};
    const long rows = (long)(s.Hq / s.Hkv) * s.N;
    p.nw = rows <= 64 ? 2 : 4;
    p.rb = 32 * p.nw;
    p.nrb = (int)((rows + p.rb - 1) / p.rb);
    p.items = s.B * s.Hkv * p.nrb;
    const int max_pages = (max_prefix + kPage - 1) / kPage;
    // enough workgroups to cover 256 CUs several times; splits of whole 64-key tiles
    const int target = env_int("JF_TARGET_WG", 1024);
    int splits = p.items > 0 ? (target + p.items - 1) / p.items : 1;
    const int max_splits = max_pages > 0 ? (max_pages + 3) / 4 : 1;
    splits = splits < 1 ? 1 : (splits > max_splits ? max_splits : splits);
    const int forced = env_int("JF_SPLITS", 0);
    if (forced > 0) splits = forced < max_splits ? forced : max_splits;
    int pps = max_pages > 0 ? (max_pages + splits - 1) / splits : 4;
    pps = (pps + 3) / 4 * 4;
    if (pps > kMaxPagesPerSplit) pps = kMaxPagesPerSplit;
    splits = max_pages > 0 ? (max_pages + pps - 1) / pps : 1;
    p.splits = splits;
    p.pps = pps;
    p.grid = (long)p.items * splits;
    if (splits > 1) {
        p.off_cnt = 0;
        p.off_ml = align256((size_t)p.items * 4);
        p.off_o = p.off_ml + align256((size_t)p.items * splits * p.rb * 2 * 4);
        p.bytes = p.off_o + align256((size_t)p.items * splits * p.rb * s.D * 4);
    }
    return p;
}

template <int D, int NW>
static hipError_t launch_bf16_t(const AttnArgs& a, long grid, hipStream_t stream) {
    hipLaunchKernelGGL((tree_attn_bf16_kernel<D, NW>), dim3((unsigned)grid), dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_attention_bf16(const jf_attn_shape& s, int max_prefix, const void* q, const void* k_pages,
                                 const void* v_pages, const int32_t* block_table, const int32_t* prefix_len,
                                 const void* k_tree, const void* v_tree, const uint64_t* anc, void* out,
                                 float* lse, void* workspace, hipStream_t stream) {
    const AttnPlanBf16 p = plan_attention_bf16(s, max_prefix);
    if (p.grid == 0) return hipSuccess;
    AttnArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.kp = static_cast<const uint16_t*>(k_pages);
    a.vp = static_cast<const uint16_t*>(v_pages);
    a.block_table = block_table;
    a.prefix_len = prefix_len;
    a.kt = static_cast<const uint16_t*>(k_tree);
    a.vt = static_cast<const uint16_t*>(v_tree);
    a.anc = anc;
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    char* ws = static_cast<char*>(workspace);
    a.counters = p.splits > 1 ? reinterpret_cast<int*>(ws + p.off_cnt) : nullptr;
    a.part_ml = p.splits > 1 ? reinterpret_cast<float*>(ws + p.off_ml) : nullptr;
    a.part_o = p.splits > 1 ? reinterpret_cast<float*>(ws + p.off_o) : nullptr;
    a.B = s.B;
    a.N = s.N;
    a.Hq = s.Hq;
    a.Hkv = s.Hkv;
    a.G = s.Hq / s.Hkv;
    a.num_pages = s.num_pages;
    a.max_pages = s.max_pages_per_seq;
    a.max_prefix = max_prefix;
    a.rows = a.G * s.N;
    a.nrb = p.nrb;
    a.splits = p.splits;
    a.pps = p.pps;
    a.scale_log2 = s.sm_scale * 1.44269504088896340736f;
    if (s.D == 128) return p.nw == 2 ? launch_bf16_t<128, 2>(a, p.grid, stream) : launch_bf16_t<128, 4>(a, p.grid, stream);
    return p.nw == 2 ? launch_bf16_t<64, 2>(a, p.grid, stream) : launch_bf16_t<64, 4>(a, p.grid, stream);
}

size_t attention_bf16_workspace_bytes(const jf_attn_shape& s, int max_prefix) {
    return plan_attention_bf16(s, max_prefix).bytes;
}

}  // namespace jf

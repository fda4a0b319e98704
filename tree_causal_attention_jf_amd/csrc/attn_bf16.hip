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
//   * A workgroup owns RB = 32 * RW * RPW rows of one (sequence, KV head) and
//     a contiguous run of prefix pages (a "split"). The split that owns the
//     last prefix page also runs the tree block, unless splits are short: then
//     the tree block gets a split of its own, so that it does not add a round
//     (and a full memory latency) to the last prefix split.
//   * Its RW * KW waves form RW row groups (32 rows each) times KW key groups:
//     key group k multiplies tiles k, k + KW, k + 2 KW, ... of the split, so
//     small row counts still keep many tiles in flight per workgroup. Key
//     groups are merged in LDS at the end.
//   * Splits of one row block are merged in the same launch by the last one
//     to finish: partials are written through to device scope, one thread per
//     workgroup bumps an agent-scope counter, and the last arriver invalidates
//     its caches and merges the partials in split order.
//   * Schedules. One sequence: every (KV head, row block) gets the same number
//     of equal page ranges, and workgroup ids are remapped so that one KV
//     head's row blocks and splits land on one XCD and share its L2. Batches of
//     2..64 sequences: each workgroup plans from the prefix lengths themselves
//     (the host knows only the longest). A sequence with more than 1.5x the
//     mean work per CU is cut into ceil(work / mean) pieces, or, when that fits
//     one round of CUs but the rest would not, into a head and a tail; units
//     (sequence, piece, KV head) are ranked by piece size and dealt round robin
//     to the XCDs, a unit's row blocks together (only those that hold rows of
//     the tree), so that every XCD list-schedules its own longest-first share.
//
// Data movement: 64-key tiles of K and V go from HBM straight into a 4-tile
// LDS ring with global_load_lds_dwordx4 (16 bytes per lane, no staging
// registers), rounds of KW tiles ahead of the ones being multiplied; each wave
// counts its own transfers with vmcnt and a barrier publishes a round to all
// waves. Rows are stored as they are in the cache (key-major), 16-byte chunks
// XOR-swizzled per key so that the matrix-operand reads are bank-conflict free.
// A one-round ring's prefix split (the few-row plans of budget-16 steps) requests
// its round as soon as its page ids have landed, while the rest of the set-up runs.
//
// Per tile, per wave (32 query rows):
//   S^T[key, row] = K_tile Q^T     (A = K rows via ds_read_b128, B = Q in registers)
//   online softmax in fp32 per row (exp2 with the scale folded into log2 e;
//   the running max is only moved when it grows by more than 2^8, so the
//   output accumulators are rarely rescaled)
//   O^T[d, row]  += V^T P^T        (A = V^T via ds_read_b64_tr_b16, which
//                                   transposes 4 keys x 16 d per 16 lanes;
//                                   B = P^T in registers, rounded to bf16)
// In the matrix-core output layout each lane owns one query row and 16 keys
// per 32-key block, so the 256-bit ancestor bitset of that row's node sits in
// the lane's registers and masking is a per-register bit test.
//
// The same body also runs inside the verification launch (tree_verify_bf16_kernel
// below): attention workgroups first, then the acceptance workgroups (argmax over
// the target logits and the walk) in the same grid. There the workgroups that run
// tree tiles may build the ancestor bitsets from the parent array themselves.
#include "jf_common.h"
#include "accept_device.h"

namespace jf {

constexpr int kKeyTile = 64;
constexpr int kRing = 4;                 // LDS tile buffers
constexpr int kMaxPagesPerSplit = 1024;
constexpr int kMaxSplits = 64;
constexpr int kMaxTreePages = JF_MAX_NODES / 16 + 1;   // pages a paged tree of up to 256 nodes spans
constexpr int kMaxBalanced = 64;         // batches planned from their prefix lengths inside the kernel (one wave)
constexpr int kMinTail = 8;              // balanced: smallest tail piece (tiles) of the head-and-tail rule

struct AttnArgs {
    const uint16_t* q;
    const uint16_t* kp;
    const uint16_t* vp;
    const int32_t* block_table;
    const int32_t* prefix_len;
    const uint16_t* kt;
    const uint16_t* vt;
    const uint64_t* anc;
    const int32_t* parent_sets;   // non-null: tree WGs build the ancestor words from this parent array
    uint16_t* out;
    float* lse;
    int* counters;     // [items]                       zero between calls
    float* part_ml;    // [items][splits][RB][4]        (m in log2 units, l, row scale r, unused)
    float* part_o;     // [items][splits] x [RB][D]     fp16 of O / r: in the MFMA layout (frag_half_off)
                       //                               with one key group, else row-major (half_off)
    uint32_t part_ml_bytes, part_o_bytes;
    int B, N, Hq, Hkv, G, num_pages, max_pages, max_prefix;
    int rows;          // G * N
    int nrb;           // row blocks per (sequence, KV head)
    int splits;        // splits per row block in the grid
    int pps;           // prefix pages per split (multiple of 4; per sequence when balanced)
    int balanced;      // 1: per-sequence pieces, units dealt longest first to the XCDs (2 <= B <= kMaxBalanced)
    int tree_tiles;    // 64-key tiles of the tree (for the balanced plan's work estimate)
    int cus;           // compute units of the device (ditto)
    int forced;        // balanced: every sequence takes `splits` pieces (tuning and tests)
    float cut;         // balanced: a sequence is cut when its work exceeds cut x the mean per CU
    float ht_frac;     // balanced: head size of the head-and-tail rule, x the mean per CU (0: off)
    const int32_t* tree_len;  // [B] nodes of each tree (NULL: all N); rows of later nodes are not written
    int paged_tree;    // 1: node j's K/V is cached token prefix_len[b] + j (kt / vt unused)
    int tree_split;    // 1: split splits-1 runs the tree tiles alone, the others the prefix
    float scale_log2;  // sm_scale * log2(e)
};

template <int D>
struct Geo {
    static constexpr int ROW_BYTES = D * 2;
    static constexpr int CPR = D / 8;                       // 16-byte chunks per key row
    static constexpr int ROWS_PER_KB = 1024 / ROW_BYTES;    // key rows per 1 KB transfer
    static constexpr int TILE_BYTES = kKeyTile * ROW_BYTES; // one of K or V
    static constexpr int KB_PER_TILE = TILE_BYTES / 1024;
    static constexpr int BUF_BYTES = 2 * TILE_BYTES;        // K then V
    static constexpr int XFER_PER_TILE = 2 * KB_PER_TILE;   // 1 KB transfers per tile
};

// Chunk swizzles for gfx950's 64-bank LDS, where one access cycle serves 256
// bytes (16 lanes of a 16-byte read):
//  K is read 16 keys at a time at one logical chunk (QK operand): the 16 keys
//    must land on 16 distinct 16-byte bank groups;
//  V is read 4 consecutive keys x 2 adjacent chunks per 16 lanes, two such
//    groups (chunk pairs 0-1 and 2-3 of a 4-chunk block) per 32 lanes
//    (transposing PV operand): the 4 keys x 4 chunks must be distinct.
// Rows are 256 bytes (D = 128, one row per bank window) or 128 bytes (D = 64,
// two rows per window, so the low key bit picks the half).
template <int D>
__device__ __forceinline__ int swz_k(int key) {
    return D == 128 ? (key & 15) : ((key >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int key) {
    return D == 128 ? ((key & 3) << 2) : (((key >> 1) & 1) << 2);
}

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// One 16-byte-per-lane transfer from global memory into LDS at lds_base + 16 * lane.
__device__ __forceinline__ void dma16(uint32_t lds_base, const void* gptr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(gptr)
                 : "memory", "m0");
}

// A pointer the compiler may not prove wave-uniform (it is, by construction) in scalar registers.
template <typename P>
__device__ __forceinline__ P* uniform_ptr(P* p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
    return reinterpret_cast<P*>(((uint64_t)hi << 32) | lo);
}

// The same from a wave-uniform base (scalar registers) plus a per-lane 32-bit byte offset.
__device__ __forceinline__ void dma16_s(uint32_t lds_base, const void* sbase, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}


// max of a value over lanes i and i ^ 32 (swap of the two half-waves)
__device__ __forceinline__ float max_halves(float x) {
    const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

struct TileSrc {
    bool tree;
    int t0;        // prefix: first token of the tile; tree: first node
    int limit;     // prefix: one past the last valid token; tree: N
};

// Per-lane byte offsets, inside one page of one KV head, of the chunks a lane
// moves in transfer kb (0 .. TPP-1) of that page: K and V differ only in the
// swizzle. A page is TPP = 16 * ROW_BYTES / 1024 consecutive 1 KB transfers.
template <int D>
struct PageLanes {
    static constexpr int TPP = kPage * Geo<D>::ROW_BYTES / 1024;
    uint32_t k[TPP], v[TPP];
};

template <int D>
__device__ __forceinline__ PageLanes<D> page_lanes(int lane) {
    using Gm = Geo<D>;
    PageLanes<D> pl;
    const int rsub = lane / Gm::CPR, pc = lane % Gm::CPR;
    #pragma unroll
    for (int kb = 0; kb < PageLanes<D>::TPP; ++kb) {
        const int row = kb * Gm::ROWS_PER_KB + rsub;     // key within the page (and, mod 16, the tile)
        pl.k[kb] = (uint32_t)(row * D + ((pc ^ swz_k<D>(row)) << 3)) * 2u;
        pl.v[kb] = (uint32_t)(row * D + ((pc ^ swz_v<D>(row)) << 3)) * 2u;
    }
    return pl;
}

// Issue this wave's share (transfers first .. first + CNT - 1 of a round) of
// the transfers of one round of KW tiles into LDS starting at `buf`. Tile j of
// the round goes to buf + j * BUF_BYTES; K transfers first, then V; the TPP
// transfers of one page are consecutive and never split between waves.
//  * Full prefix tile: one page id (read from LDS, wave-uniform) gives a
//    scalar base; the lane part is the fixed PageLanes offset.
//  * Tree tile, or the tile that crosses the end of the prefix: per-lane
//    addresses. Keys beyond the valid range are fetched from a valid key
//    instead (tree: the last node; prefix: the tile's first key); the softmax
//    masks them, and they are finite, so a zero weight times them stays zero.
// A round slot past the last tile re-fetches the last tile (the slot is never
// multiplied), which keeps every wave's transfer count per round fixed for
// the vmcnt bookkeeping.
template <int D, int CNT, typename SrcFn>
__device__ __forceinline__ void issue_round(const uint16_t* kp, const uint16_t* vp, const uint16_t* kt,
                                            const uint16_t* vt, int N, int Hkv, SrcFn tile_src, int round_first_tile,
                                            int n_tiles, int b, int kvh, const int* s_pages,
                                            const PageLanes<D>& pl, uint32_t buf, int first, int lane,
                                            const int* s_tp, int tok0) {
    using Gm = Geo<D>;
    constexpr int TPP = PageLanes<D>::TPP;
    static_assert(CNT % TPP == 0, "a wave moves whole pages");
    first = __builtin_amdgcn_readfirstlane(first);       // wave index based: uniform
    const int rsub = lane / Gm::CPR, pc = lane % Gm::CPR;
    #pragma unroll
    for (int g = 0; g < CNT / TPP; ++g) {
        const int i0 = first + g * TPP;                  // wave-uniform transfer index in the round
        const int j = i0 / Gm::XFER_PER_TILE;
        const int ii0 = i0 % Gm::XFER_PER_TILE;
        const bool isv = ii0 >= Gm::KB_PER_TILE;
        const int pq = (isv ? ii0 - Gm::KB_PER_TILE : ii0) / TPP;   // page of the tile
        const int it = min(round_first_tile + j, n_tiles - 1);
        const TileSrc src = tile_src(it);
        const uint32_t lds0 = buf + j * Gm::BUF_BYTES + ii0 * 1024;
        if (!src.tree && src.t0 + kKeyTile <= src.limit) {
            // prefix tiles start on page boundaries; s_pages[k] = page of the split's k-th 16 tokens
            const int page = __builtin_amdgcn_readfirstlane(s_pages[it * (kKeyTile / kPage) + pq]);
            const uint16_t* base = (isv ? vp : kp) + ((long)page * Hkv + kvh) * (kPage * D);
            base = uniform_ptr(base);                    // wave-uniform by construction
            #pragma unroll
            for (int kb = 0; kb < TPP; ++kb)
                dma16_s(__builtin_amdgcn_readfirstlane(lds0 + kb * 1024), base, isv ? pl.v[kb] : pl.k[kb]);
        } else {
            #pragma unroll
            for (int kb = 0; kb < TPP; ++kb) {
                const int row = pq * kPage + kb * Gm::ROWS_PER_KB + rsub;     // key within the tile
                const int c = pc ^ (isv ? swz_v<D>(row) : swz_k<D>(row));
                const uint16_t* gp;
                if (src.tree) {
                    const int t = min(src.t0 + row, src.limit - 1);    // nodes past the tree: its last node
                    if (tok0 >= 0) {
                        // paged tree: node t is cached token tok0 + t; s_tp lists the pages from tok0's on
                        const int tok = tok0 + t;
                        const int page = s_tp[(tok >> 4) - (tok0 >> 4)];
                        gp = (isv ? vp : kp) + (((long)page * Hkv + kvh) * kPage + (tok & 15)) * D + c * 8;
                    } else {
                        gp = (isv ? vt : kt) + (((long)b * N + t) * Hkv + kvh) * D + c * 8;
                    }
                } else {
                    int t = src.t0 + row;
                    if (t >= src.limit) t = src.t0;
                    const int page = s_pages[(t >> 4) - (src.t0 >> 4) + it * (kKeyTile / kPage)];
                    gp = (isv ? vp : kp) + (((long)page * Hkv + kvh) * kPage + (t & 15)) * D + c * 8;
                }
                dma16(__builtin_amdgcn_readfirstlane(lds0 + kb * 1024), gp);
            }
        }
    }
}

// One prefix tile into LDS at `buf`, K transfers then V, with the tile's four
// page ids in lanes 0..3 of `pages` (already checked): the same transfers as a
// round's share for that tile, for a wave that requests its tile before the
// page list is in LDS.
template <int D>
__device__ __forceinline__ void issue_tile_own_pages(const uint16_t* kp, const uint16_t* vp, int Hkv, int kvh,
                                                     const TileSrc& src, int pages, const PageLanes<D>& pl,
                                                     uint32_t buf, int lane) {
    using Gm = Geo<D>;
    constexpr int TPP = PageLanes<D>::TPP;
    const int rsub = lane / Gm::CPR, pc = lane % Gm::CPR;
    const bool full = src.t0 + kKeyTile <= src.limit;
    #pragma unroll
    for (int ii0 = 0; ii0 < Gm::XFER_PER_TILE; ii0 += TPP) {
        const bool isv = ii0 >= Gm::KB_PER_TILE;
        const int pq = (isv ? ii0 - Gm::KB_PER_TILE : ii0) / TPP;   // page of the tile
        const uint32_t lds0 = buf + ii0 * 1024;
        if (full) {
            const int page = __builtin_amdgcn_readlane(pages, pq);
            const uint16_t* base = uniform_ptr((isv ? vp : kp) + ((long)page * Hkv + kvh) * (kPage * D));
            #pragma unroll
            for (int kb = 0; kb < TPP; ++kb)
                dma16_s(__builtin_amdgcn_readfirstlane(lds0 + kb * 1024), base, isv ? pl.v[kb] : pl.k[kb]);
        } else {
            #pragma unroll
            for (int kb = 0; kb < TPP; ++kb) {
                const int row = pq * kPage + kb * Gm::ROWS_PER_KB + rsub;     // key within the tile
                const int c = pc ^ (isv ? swz_v<D>(row) : swz_k<D>(row));
                int t = src.t0 + row;
                if (t >= src.limit) t = src.t0;
                const int page = __shfl(pages, (t >> 4) - (src.t0 >> 4));
                const uint16_t* gp = (isv ? vp : kp) + (((long)page * Hkv + kvh) * kPage + (t & 15)) * D + c * 8;
                dma16(__builtin_amdgcn_readfirstlane(lds0 + kb * 1024), gp);
            }
        }
    }
}

// The tree tiles of a workgroup that runs the tree alone (its own split) in a
// one-round ring, requested before anything else: their addresses depend on
// no loaded value (the tree's K/V are the separate [B, N, Hkv, D] arrays). Wave
// w moves tree tile w into ring slot w, only the transfers that hold tree keys
// (a transfer that straddles the tree's end re-reads its last key); the value
// rows of skipped transfers are zeroed, so that their zero weights multiply
// finite values (key rows are left as they are: their scores are masked
// before they are used). The caller waits with vmcnt(0) before the products.
template <int D>
__device__ __forceinline__ void issue_tree_tiles(const uint16_t* kt, const uint16_t* vt, int N, int Hkv, int b,
                                                 int kvh, int nt, uint32_t ring0, char* ring, int w, int lane) {
    using Gm = Geo<D>;
    if (w >= nt) return;                                      // wave-uniform
    const int t0 = w * kKeyTile;
    const int nrows = min(kKeyTile, N - t0);
    const int rsub = lane / Gm::CPR, pc = lane % Gm::CPR;
    const uint32_t buf = ring0 + w * Gm::BUF_BYTES;
    #pragma unroll
    for (int ii = 0; ii < Gm::XFER_PER_TILE; ++ii) {
        const bool isv = ii >= Gm::KB_PER_TILE;
        const int row0 = (isv ? ii - Gm::KB_PER_TILE : ii) * Gm::ROWS_PER_KB;
        if (row0 < nrows) {                                   // uniform
            const int row = min(row0 + rsub, nrows - 1);
            const int c = pc ^ (isv ? swz_v<D>(row) : swz_k<D>(row));
            const uint16_t* gp = (isv ? vt : kt) + (((long)b * N + t0 + row) * Hkv + kvh) * D + c * 8;
            dma16(__builtin_amdgcn_readfirstlane(buf + ii * 1024), gp);
        }
    }
    const int zr0 = (nrows + Gm::ROWS_PER_KB - 1) / Gm::ROWS_PER_KB * Gm::ROWS_PER_KB;
    char* vz = ring + w * Gm::BUF_BYTES + Gm::TILE_BYTES + zr0 * Gm::ROW_BYTES;
    const int zbytes = (kKeyTile - zr0) * Gm::ROW_BYTES;
    for (int off = lane * 16; off < zbytes; off += kWave * 16) *reinterpret_cast<u32x4*>(vz + off) = u32x4{0, 0, 0, 0};
}

// Wait until at most `pending` later rounds of this wave's transfers are in flight.
template <int DPR>
__device__ __forceinline__ void wait_rounds(int pending) {
    if (pending >= 2) wait_vm<2 * DPR>();
    else if (pending == 1) wait_vm<DPR>();
    else wait_vm<0>();
}

// The 256-bit ancestor bitset of a lane's node, as a register vector (a
// variable index into it selects between registers instead of spilling).
typedef unsigned long long u64x4 __attribute__((ext_vector_type(4)));

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4 ds_read_tr(const char* lds_ptr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(lds_ptr));
}

// Running state of one wave: 32 query rows, one lane pair per row.
template <int D>
struct RowState {
    f32x16 o[D / 32];    // O^T accumulators: lane = row, register = d
    float m;             // reference max (log2 units), equal in both half-waves
    float l;             // partial sum of this half-wave's keys
};

// x = keep ? x : -inf, bitwise (keep is all ones or zero), in x's own register
__device__ __forceinline__ float keep_or_neg(float x, uint32_t keep) {
    float y;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(y) : "v"(keep), "0"(x), "s"(0xff800000u));
    return y;
}

// all ones when bit `sh` of w is set, else zero
__device__ __forceinline__ uint32_t bit_mask(uint32_t w, int sh) {
    return (uint32_t)__builtin_amdgcn_sbfe((int)w, sh, 1);
}

// Multiply one 64-key tile into a wave's running state.
// Multiply one 64-key tile into the running state of a wave's RPW row blocks
// (32 query rows each). Every K and V operand read from LDS feeds the product
// of each row block, so RPW = 2 halves the LDS traffic per product and gives the
// wave two independent chains to interleave.
template <int D, int RPW>
__device__ __forceinline__ void tile_product(RowState<D>* st, const char* kbuf, const char* vbuf,
                                             const bf16x8 (*qreg)[D / 16], const TileSrc& src, const u64x4* ancw,
                                             int N, float scale_log2, const int* v_off, int hf, int l32) {
    using Gm = Geo<D>;
    constexpr int DCH = D / 16;
    constexpr int DT = D / 32;
    const float NEG = -__builtin_inff();
    // S^T = K Q^T for two 32-key halves, per row block. The ragged prefix tail
    // starts the accumulators at -inf for keys past the prefix end (their rows
    // were redirected to a valid finite key, so -inf + finite stays -inf); every
    // other tile starts from the inline zero. Only the first k-step differs, so
    // both paths leave their scores in the same MFMA result registers.
    f32x16 sacc[RPW][2];
    auto kfrag = [&](int c, int h2) {
        const int key = h2 * 32 + l32;
        return *reinterpret_cast<const bf16x8*>(kbuf + key * Gm::ROW_BYTES + (((2 * c + hf) ^ swz_k<D>(key)) << 4));
    };
    // K operands one k-step ahead: the reads of step c + 1 are issued before the
    // products of step c, so the LDS latency hides behind two products instead of
    // standing between every pair (the asm keeps each step's products below the
    // next step's reads; it reads the step's own operands, so the wait for them
    // lands there and lets the newer reads stay in flight)
    bf16x8 kf[DCH][2];
    kf[0][0] = kfrag(0, 0);
    kf[0][1] = kfrag(0, 1);
    if constexpr (DCH > 1) {
        kf[1][0] = kfrag(1, 0);
        kf[1][1] = kfrag(1, 1);
    }
    asm volatile("" : "+v"(kf[0][0]), "+v"(kf[0][1])::"memory");
    {
        if (!src.tree && src.t0 + kKeyTile > src.limit) {
            const int nvalid = src.limit - src.t0 - 4 * hf;
            f32x16 b0, b1;
            #pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kk = 8 * (r >> 2) + (r & 3);
                b0[r] = kk < nvalid ? 0.f : NEG;
                b1[r] = kk + 32 < nvalid ? 0.f : NEG;
            }
            #pragma unroll
            for (int blk = 0; blk < RPW; ++blk) {
                sacc[blk][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0][0], qreg[blk][0], b0, 0, 0, 0);
                sacc[blk][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0][1], qreg[blk][0], b1, 0, 0, 0);
            }
        } else {
            #pragma unroll
            for (int blk = 0; blk < RPW; ++blk) {
                sacc[blk][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0][0], qreg[blk][0], f32x16{}, 0, 0, 0);
                sacc[blk][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0][1], qreg[blk][0], f32x16{}, 0, 0, 0);
            }
        }
    }
    #pragma unroll
    for (int c = 1; c < DCH; ++c) {
        if (c + 1 < DCH) {
            kf[c + 1][0] = kfrag(c + 1, 0);
            kf[c + 1][1] = kfrag(c + 1, 1);
        }
        asm volatile("" : "+v"(kf[c][0]), "+v"(kf[c][1])::"memory");
        #pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            #pragma unroll
            for (int blk = 0; blk < RPW; ++blk)
                sacc[blk][h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[c][h2], qreg[blk][c], sacc[blk][h2], 0, 0, 0);
        }
    }
    uint32_t pk[RPW][2][8];
    #pragma unroll
    for (int blk = 0; blk < RPW; ++blk) {
        // register r of half h2 holds key h2*32 + 8*(r/4) + 4*hf + r%4 of the tile
        // masked scores become -inf in place (same registers), so the unmasked path
        // needs no copies where the paths meet
        if (src.tree) {
            const int tt = src.t0 / kKeyTile;
            const int left = N - src.t0;
            uint64_t mw = ancw[blk][tt];
            if (left < 64) mw &= (1ull << left) - 1ull;
            mw >>= 4 * hf;
            const uint32_t lo = (uint32_t)mw, hi = (uint32_t)(mw >> 32);
            #pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int sh = 8 * (r >> 2) + (r & 3);
                sacc[blk][0][r] = keep_or_neg(sacc[blk][0][r], bit_mask(lo, sh));
                sacc[blk][1][r] = keep_or_neg(sacc[blk][1][r], bit_mask(hi, sh));
            }
        }
        // online softmax (log2 domain), lazy rescale
        float mxa = NEG, mxb = NEG;
        #pragma unroll
        for (int r = 0; r < 16; r += 2) {
            mxa = max3f(mxa, sacc[blk][0][r], sacc[blk][1][r]);
            mxb = max3f(mxb, sacc[blk][0][r + 1], sacc[blk][1][r + 1]);
        }
        const float mx = max_halves(fmaxf(mxa, mxb)) * scale_log2;
        RowState<D>& sb = st[blk];
        // move the reference max only when some row's max grew by more than 2^8
        if (__builtin_amdgcn_ballot_w64(mx > sb.m + 8.f)) {
            const float m_new = fmaxf(sb.m, mx);
            // a row with no visible key yet keeps m = -inf (its l and O are 0): rescaling
            // against 0 instead of -inf gives alpha = 0, not exp2(-inf + inf) = NaN
            const float alpha = __builtin_amdgcn_exp2f(sb.m - (m_new == NEG ? 0.f : m_new));
            sb.l *= alpha;
            #pragma unroll
            for (int i = 0; i < DT; ++i) sb.o[i] *= alpha;
            sb.m = m_new;
        }
        const float m_use = (sb.m == NEG) ? 0.f : sb.m;
        // the row sum adds the bf16-rounded weights that the P.V product uses, two
        // per v_dot2_f32_bf16
        float rs = 0.f;
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        #pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            #pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[blk][h2][r], scale_log2, -m_use));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[blk][h2][r + 1], scale_log2, -m_use));
                pk[blk][h2][r >> 1] = pack_bf16x2(p0, p1);
                rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[blk][h2][r >> 1]), ones, rs, false);
            }
        }
        sb.l += rs;
    }
    // O^T += V^T P^T, 16 keys per step (two transposing reads give the 8 keys of a lane)
    #pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
        const int h2 = kc >> 1, o4 = (kc & 1) * 4;
        bf16x8 pb[RPW];
        #pragma unroll
        for (int blk = 0; blk < RPW; ++blk) {
            const u32x4 pw = {pk[blk][h2][o4], pk[blk][h2][o4 + 1], pk[blk][h2][o4 + 2], pk[blk][h2][o4 + 3]};
            pb[blk] = __builtin_bit_cast(bf16x8, pw);
        }
        #pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const char* vp0 = vbuf + v_off[dt] + kc * 16 * Gm::ROW_BYTES;
            const u32x2 lo2 = __builtin_bit_cast(u32x2, ds_read_tr(vp0));
            const u32x2 hi2 = __builtin_bit_cast(u32x2, ds_read_tr(vp0 + 8 * Gm::ROW_BYTES));
            const u32x4 vw = {lo2[0], lo2[1], hi2[0], hi2[1]};
            #pragma unroll
            for (int blk = 0; blk < RPW; ++blk)
                st[blk].o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vw), pb[blk],
                                                                        st[blk].o[dt], 0, 0, 0);
        }
    }
}

// Byte offset of float4 chunk c of row r in a [rows][D] fp32 LDS array,
// chunk-swizzled so that 8 consecutive rows at one chunk hit distinct banks.
template <int D>
__device__ __forceinline__ int merge_off(int r, int c) {
    return r * (D * 4) + ((c ^ (r & 7)) << 4);
}

// Byte offset, inside one split's [RB][D] fp16 partial, of the k-th 16 bytes
// that a lane of the tile loop's MFMA layout holds (one key group: lane = row
// r % 32 + 32 hf of its 32-row block, holding the row's chunks 2j + hf, j = 0 ..
// D/8 - 1; store k packs chunks 4k + hf and 4k + 2 + hf). One store instruction
// writes one contiguous 1 KB block (the hand-off stores write through to
// memory, where partial lines cost extra transactions), and the last arriver,
// which merges in the same layout, reads it back the same way.
template <int D>
__device__ __forceinline__ uint32_t frag_half_off(int r, int hf, int k) {
    return (uint32_t)((((r >> 5) * (D / 16) + k) * 64 + (r & 31) + 32 * hf) * 16);
}

// Byte offset, inside one split's [RB][D] fp16 partial, of the 16 bytes that
// thread `part` of row r's TPR threads (consecutive lanes) writes in its k-th
// store: chunks 2k * TPR + part and (2k + 1) * TPR + part of the row (4 values
// each). One store instruction puts a row's TPR threads side by side, so with
// TPR = 8 it writes the row's whole 128-byte lines.
template <int D, int TPR>
__device__ __forceinline__ uint32_t half_off(int r, int part, int k) {
    return (uint32_t)(r * (D * 2) + (k * TPR + part) * 16);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    const _Float16 a = (_Float16)lo, b = (_Float16)hi;            // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ f32x4 unpack_f16x4(uint32_t w0, uint32_t w1) {
    return f32x4{(float)__builtin_bit_cast(_Float16, (uint16_t)(w0 & 0xffffu)),
                 (float)__builtin_bit_cast(_Float16, (uint16_t)(w0 >> 16)),
                 (float)__builtin_bit_cast(_Float16, (uint16_t)(w1 & 0xffffu)),
                 (float)__builtin_bit_cast(_Float16, (uint16_t)(w1 >> 16))};
}

// Largest value over each aligned group of TPR (4 or 8) consecutive lanes, in
// every lane of the group (DPP quad permutations, then the half-row mirror).
template <int TPR>
__device__ __forceinline__ float group_max(float v) {
    static_assert(TPR == 4 || TPR == 8, "row groups of 4 or 8 lanes");
    v = fmaxf(v, __uint_as_float(dpp_u32<kDppQuad1032>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_u32<kDppQuad2301>(__float_as_uint(v))));
    if constexpr (TPR == 8) v = fmaxf(v, __uint_as_float(dpp_u32<kDppRowHalfMirror>(__float_as_uint(v))));
    return v;
}

// OR of a value over the whole wave (DPP inside rows of 16, then readlane).
__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v) {
    v |= dpp_u32<kDppQuad1032>(v);
    v |= dpp_u32<kDppQuad2301>(v);
    v |= dpp_u32<kDppRowHalfMirror>(v);
    v |= dpp_u32<kDppRowMirror>(v);
    return (uint32_t)(__builtin_amdgcn_readlane((int)v, 0) | __builtin_amdgcn_readlane((int)v, 16) |
                      __builtin_amdgcn_readlane((int)v, 32) | __builtin_amdgcn_readlane((int)v, 48));
}

// Workgroup `bid` of an attention grid of `nblk` workgroups (the attention
// launch, or the attention part of the fused verification launch).
template <int D, int RW, int KW, int RPW>
__device__ __forceinline__ void tree_attn_bf16_body(const AttnArgs& a, const unsigned bid, const unsigned nblk) {
    using Gm = Geo<D>;
    // Split partials are written as fp16 of O / r, r the row's largest |O| (values
    // in [-1, 1]: no overflow, 2^-11 of r per value), half the bytes of fp32 for
    // the last arriver to read: after the key-group merge in row-major order
    // (half_off), without key groups in the MFMA layout (frag_half_off)
    constexpr bool kHalfPart = KW > 1;
    constexpr int NW = RW * KW;
    constexpr int T = NW * 64;
    constexpr int RB = RW * 32 * RPW;                // rows per workgroup: RW waves x RPW blocks of 32
    static_assert(RPW == 1 || KW == 1, "several row blocks per wave only without key groups");
    constexpr int DCH = D / 16;                      // k-steps of the QK product
    constexpr int DT = D / 32;                       // 32-wide d tiles of O^T
    constexpr int RING_R = kRing / KW;               // rounds the ring holds
    constexpr int DPR = KW * Gm::XFER_PER_TILE / NW; // transfers per wave per round
    static_assert(kRing % KW == 0 && (KW * Gm::XFER_PER_TILE) % NW == 0, "bad wave split");
    static_assert(KW == 1 || KW * RB * D * 4 <= kRing * Gm::BUF_BYTES, "key-group merge must fit the ring");
    __shared__ __attribute__((aligned(1024))) char ring[kRing * Gm::BUF_BYTES];
    __shared__ int s_pages[kMaxPagesPerSplit];
    __shared__ float s_ml[KW][RB][2];
    __shared__ unsigned long long s_union[kAncWords];
    __shared__ int s_last;
    __shared__ int s_plan[5];
    __shared__ int s_epi[6];
    __shared__ int s_tpages[kMaxTreePages];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);     // wave index: uniform

    // ---- which (sequence, KV head, split, row block) this workgroup owns
    int rb, s, kvh, b, pps;
    if (a.balanced) {
        // Balanced schedule, planned alike by every workgroup from the prefix (and
        // tree) lengths. The mean is the work per CU (prefix tiles + tree tiles, over
        // the row blocks that hold rows of the tree; the others exit at once). Two
        // rules cut sequences into pieces:
        //  * equal pieces: a sequence whose work exceeds `cut` x the mean is cut into
        //    ceil(work / mean) pieces (at most `splits`) of equal page counts;
        //  * head and tail, used instead when the equal pieces fit the CUs in one round
        //    (so nothing else would take over the CUs the short sequences free) and
        //    the tails do not: a sequence at least kMinTail tiles above ht_frac x the
        //    mean keeps a head of that many prefix tiles (at least half its pages)
        //    and hands the rest, with its tree tiles, to a tail piece. Tails rank low,
        //    so they start on the CUs that the short sequences free first, and end
        //    beside the heads instead of after them.
        // Units (sequence, piece, KV head) are ranked by piece size, largest first,
        // and dealt round robin to the XCDs; a unit's row blocks that hold rows of
        // the tree (which read the same K/V pages) run one after another on one XCD.
        // Each XCD starts its workgroups in id order as its CUs free up, so it
        // list-schedules its own longest-first share. Ids past the units are idle.
        if (w == 0) {
            const bool in = lane < a.B;
            const int Lm = in ? a.prefix_len[lane] : 0;
            int nbm = (a.tree_len && in) ? a.tree_len[lane] : a.N;
            if (nbm < 0 || nbm > a.N) nbm = a.N;       // a bad length computes every row (as NaN)
            const int pg = (in && Lm > 0 && Lm <= a.max_prefix) ? (Lm + kPage - 1) / kPage : 0;
            const int ttl = min(a.tree_tiles, (nbm + kKeyTile - 1) / kKeyTile);
            const int tiles = (pg + 3) / 4 + ttl;
            const int live = min(a.nrb, (nbm * a.G + RB - 1) / RB);        // row blocks with rows
            int tot = in ? tiles * live : 0;
            #pragma unroll
            for (int o = 32; o > 0; o >>= 1) tot += __shfl_xor(tot, o);
            const float mean = (float)tot * (float)a.Hkv / (float)a.cus;
            int n = 1;
            if (a.forced) n = a.splits;
            else if (mean > 0.f && live > 0 && (float)tiles > a.cut * mean)
                n = min(a.splits, (int)ceilf((float)tiles / mean));
            n = min(n, max(1, pg / (4 * KW)));                            // a full round of tiles per piece
            n = max(n, (pg + kMaxPagesPerSplit - 1) / kMaxPagesPerSplit);  // (the host keeps this <= splits)
            int pp = (pg + n - 1) / n;
            pp = max(4, (pp + 3) / 4 * 4);
            n = in ? max(1, (pg + pp - 1) / pp) : 0;
            // head and tail: head pages h, a multiple of 4 and at least half the prefix,
            // so that the two pieces [0, h) and [h, pg) are the splits of h pages each
            const int T = (int)(a.ht_frac * mean + 0.5f);
            const int h = max(4 * T, (pg + 7) / 8 * 4);
            const bool cut2 = in && !a.forced && a.ht_frac > 0.f && live > 0 && tiles - T >= kMinTail &&
                              h < pg && h >= 4 * KW && h <= kMaxPagesPerSplit;
            int wgs = in ? (cut2 ? 2 : 1) * live * a.Hkv : 0;     // workgroups with head and tail pieces
            int wgs_eq = in ? n * live * a.Hkv : 0;                // with equal pieces
            int big = pg > kMaxPagesPerSplit;                      // must be cut however long the others are
            #pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                wgs += __shfl_xor(wgs, o);
                wgs_eq += __shfl_xor(wgs_eq, o);
                big |= __shfl_xor(big, o);
            }
            // (256-row blocks only: the 128-row plans measured slower with it)
            const bool ht = KW == 1 && a.ht_frac > 0.f && !a.forced && !big && wgs_eq <= a.cus && wgs > a.cus;
            // a sequence's pieces in two groups of equal keys (pieces of one group are
            // consecutive in the ranking): na pieces of key ka, then nb of key kb
            int na = n, ka = in ? min(pp, pg) : -1, nb = 0, kb = -1;
            if (ht && in) {
                na = 1;
                if (cut2) {
                    pp = h;
                    ka = h;
                    nb = 1;
                    kb = (pg - h) + 4 * ttl;
                } else {
                    pp = max(4, (pg + 3) / 4 * 4);
                    ka = pg + 4 * ttl;
                }
            }
            // units ranked before each group: larger keys first, ties by sequence,
            // then group (the loop index is uniform: lane j's values are read into
            // scalar registers; without tails, one group per sequence: the shorter loop)
            int offa = 0, offb = 0;
            if (ht) {
                for (int j = 0; j < a.B; ++j) {
                    const int kaj = __builtin_amdgcn_readlane(ka, j), kbj = __builtin_amdgcn_readlane(kb, j);
                    const int naj = __builtin_amdgcn_readlane(na, j), nbj = __builtin_amdgcn_readlane(nb, j);
                    offa += ((kaj > ka || (kaj == ka && j < lane)) ? naj : 0) +
                            ((kbj > ka || (kbj == ka && j < lane)) ? nbj : 0);
                    offb += ((kaj > kb || (kaj == kb && j <= lane)) ? naj : 0) +
                            ((kbj > kb || (kbj == kb && j < lane)) ? nbj : 0);
                }
            } else {
                for (int j = 0; j < a.B; ++j) {
                    const int kaj = __builtin_amdgcn_readlane(ka, j), naj = __builtin_amdgcn_readlane(na, j);
                    offa += (kaj > ka || (kaj == ka && j < lane)) ? naj : 0;
                }
            }
            const int x = bid % kNumXcd, slot = bid / kNumXcd;
            const int loa = offa * a.Hkv, lob = offb * a.Hkv;
            const int lv = in ? live : 0;
            bool mine_a, mine_b;
            int u, rbp;
            if (__ballot(in && lv < a.nrb) == 0) {
                // every row block holds rows: unit (slot / nrb) * 8 + x, row block slot % nrb
                u = (slot / a.nrb) * kNumXcd + x;
                rbp = slot % a.nrb;
                mine_a = in && u >= loa && u < loa + na * a.Hkv;
                mine_b = in && u >= lob && u < lob + nb * a.Hkv;
            } else {
                // Trees of ragged lengths: XCD x runs its units (u = x mod 8, in rank
                // order) one after another, each with its live row blocks only, and
                // workgroup id 8 k + x takes XCD x's k-th live slot. Row blocks past a
                // sequence's tree get no workgroup, and ids past the last live slot are idle.
                auto on_x = [&](int v) { return v > x ? (v - x + kNumXcd - 1) / kNumXcd : 0; };  // units u < v on x
                const int wa = (on_x(loa + na * a.Hkv) - on_x(loa)) * lv;     // slots of each group on XCD x
                const int wb = (on_x(lob + nb * a.Hkv) - on_x(lob)) * lv;
                int sa = 0, sb = 0;                                            // slots of the groups ranked before
                for (int j = 0; j < a.B; ++j) {
                    const int loaj = __builtin_amdgcn_readlane(loa, j), lobj = __builtin_amdgcn_readlane(lob, j);
                    const int waj = __builtin_amdgcn_readlane(wa, j), wbj = __builtin_amdgcn_readlane(wb, j);
                    sa += (loaj < loa ? waj : 0) + (lobj < loa ? wbj : 0);
                    sb += (loaj < lob ? waj : 0) + (lobj < lob ? wbj : 0);
                }
                mine_a = in && slot >= sa && slot < sa + wa;
                mine_b = in && slot >= sb && slot < sb + wb;
                const int lo = mine_a ? loa : lob;
                const int local = slot - (mine_a ? sa : sb);
                // the group's (local / lv)-th unit on XCD x, and its row block
                u = lo + ((x - lo) % kNumXcd + kNumXcd) % kNumXcd + (local / max(lv, 1)) * kNumXcd;
                rbp = local % max(lv, 1);
            }
            if (mine_a || mine_b) {
                const int lo = mine_a ? loa : lob;
                s_plan[0] = lane;
                s_plan[1] = (mine_a ? 0 : na) + (u - lo) / a.Hkv;
                s_plan[2] = (u - lo) % a.Hkv;
                s_plan[3] = pp;
                s_plan[4] = rbp;
            }
            if (__ballot(mine_a || mine_b) == 0 && lane == 0) s_plan[0] = -1;
        }
        __syncthreads();
        b = __builtin_amdgcn_readfirstlane(s_plan[0]);
        if (b < 0) return;                             // idle id (whole workgroup)
        s = __builtin_amdgcn_readfirstlane(s_plan[1]);
        kvh = __builtin_amdgcn_readfirstlane(s_plan[2]);
        pps = __builtin_amdgcn_readfirstlane(s_plan[3]);
        rb = __builtin_amdgcn_readfirstlane(s_plan[4]);
    } else {
        // ids remapped so that one KV head's row blocks and splits share an XCD
        const int lid = xcd_remap(bid, nblk);
        rb = lid % a.nrb;
        int t1 = lid / a.nrb;
        s = t1 % a.splits;
        t1 /= a.splits;
        kvh = t1 % a.Hkv;
        b = t1 / a.Hkv;
        pps = a.pps;
    }
    int item = (b * a.Hkv + kvh) * a.nrb + rb;
    const int rw = w % RW, kw = w / RW;
    const int hf = lane >> 5, l32 = lane & 31;
    // the lane's row in each of the wave's row blocks
    int rloc[RPW], node[RPW], head[RPW];
    bool row_ok[RPW];
    #pragma unroll
    for (int blk = 0; blk < RPW; ++blk) {
        rloc[blk] = (rw * RPW + blk) * 32 + l32;    // row within the workgroup's rows
        const int row = rb * RB + rloc[blk];
        row_ok[blk] = row < a.rows;
        node[blk] = row_ok[blk] ? row / a.G : 0;
        head[blk] = kvh * a.G + (row_ok[blk] ? row % a.G : 0);
    }

    // ---- every global read of the set-up is issued at once: the prefix length,
    // this split's block-table entries (the page range does not depend on the
    // length), the rows' ancestor words and, last, the wave's Q rows: the page list
    // and the tree-tile union need the first ones before the first tiles are
    // requested, Q only once the first tile has landed
    constexpr int PPT = (kMaxPagesPerSplit + T - 1) / T;
    // with tree_split, the last split slot holds no prefix pages
    const bool tree_wg = a.tree_split && s == a.splits - 1;
    // a one-round ring's tree-only workgroup requests its tree tiles first (when
    // they all fit the round and live in the separate tree arrays)
    const int n_tree_tiles = (a.N + kKeyTile - 1) / kKeyTile;
    const bool early_tree = RING_R == 1 && tree_wg && !a.paged_tree && a.tree_len == nullptr && n_tree_tiles <= KW;
    const int p_begin = tree_wg ? 0 : s * pps;
    const int p_avail = tree_wg ? 0 : min(pps, a.max_pages - p_begin);
    // Every load of the set-up is unconditional (an index past the end is clamped,
    // an absent array replaced by prefix_len, a valid address) and its value is
    // selected where it is used: the compiler then counts the loads exactly, and a
    // wait for one of them never also waits for every load issued after it.
    // (one-round rings with one tile per wave: this wave's four page ids of the
    // split's first round, in lanes 0..3, first of all)
    int own_pages = 0;
    if constexpr (RING_R == 1 && RW == 1)
        own_pages = *(p_avail > 0 ? a.block_table + (long)b * a.max_pages + p_begin +
                                        min(4 * kw + min(lane, 3), p_avail - 1)
                                  : a.prefix_len + b);
    int L = a.prefix_len[b];
    const int nb_raw = *(a.tree_len ? a.tree_len + b : a.prefix_len + b);
    // when this launch builds the ancestor words itself: the parent of node `lane`
    // (trees of at most 64 nodes: every wave builds them alone) or of node tid
    const int par_idx = a.N <= kWave ? lane : tid;
    const int par_raw = *(a.parent_sets ? a.parent_sets + (long)b * a.N + min(par_idx, a.N - 1) : a.prefix_len + b);
    int pid[PPT];
    #pragma unroll
    for (int k = 0; k < PPT; ++k) {
        const int i = tid + k * T;
        pid[k] = *(p_avail > 0 ? a.block_table + (long)b * a.max_pages + p_begin + min(i, p_avail - 1)
                               : a.prefix_len + b);
    }
    // rows past the end read node 0 (a valid address): the loads stay unconditional,
    // so the compiler's wait for the ancestor words does not have to cover the Q
    // loads issued after them. Such a row computes node 0's prefix attention (its
    // ancestor words are cleared below) and is never written out.
    u64x4 ancw[RPW];
    #pragma unroll
    for (int blk = 0; blk < RPW; ++blk) {
        #pragma unroll
        for (int k = 0; k < kAncWords; ++k) ancw[blk][k] = a.anc[((long)b * a.N + node[blk]) * kAncWords + k];
    }
    asm volatile("" ::: "memory");                 // keep the Q loads behind the ones above
    bf16x8 qreg[RPW][DCH];
    #pragma unroll
    for (int blk = 0; blk < RPW; ++blk) {
        const uint16_t* qp = a.q + (((long)b * a.N + node[blk]) * a.Hq + head[blk]) * D + 8 * hf;
        #pragma unroll
        for (int c = 0; c < DCH; ++c) qreg[blk][c] = __builtin_bit_cast(bf16x8, ld16(qp + 16 * c));
    }
    // (the tree tiles go out after the set-up loads: a wait for one of those loads
    // then never has to wait for the tiles too, which are newer)
    if (early_tree)
        issue_tree_tiles<D>(a.kt, a.vt, a.N, a.Hkv, b, kvh, n_tree_tiles,
                            (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)ring), ring, w, lane);
    int nb = a.tree_len ? nb_raw : a.N;
    const int par_own = (a.parent_sets && par_idx < a.N) ? par_raw : -1;
    bool bad = (L < 0 || L > a.max_prefix);
    if (bad) L = 0;
    if (nb < 0 || nb > a.N) {                       // a bad tree length: every row of the sequence is NaN
        bad = true;
        nb = a.N;
    }
    if (rb * RB >= nb * a.G) {                      // uniform: no row of the block is a node of the tree
        if (early_tree) wait_vm<0>();               // (never with early tree tiles; kept safe regardless)
        return;
    }
    // rows of nodes past the tree's length are not computed into the output
    #pragma unroll
    for (int blk = 0; blk < RPW; ++blk) {
        row_ok[blk] = row_ok[blk] && node[blk] < nb;
        if (!row_ok[blk]) ancw[blk] = u64x4{0, 0, 0, 0};
    }
    const int npages = (L + kPage - 1) / kPage;
    // splits that hold work: the prefix splits, and the tree either in the last of
    // them or (tree_split) in its own slot, splits - 1
    const int n_pre_splits = (npages + pps - 1) / pps;
    int n_act;
    bool has_tree;
    if (a.tree_split) {
        n_act = n_pre_splits + 1;
        if (!tree_wg && s >= n_pre_splits) return;            // uniform: the whole workgroup leaves
        has_tree = tree_wg;
    } else {
        n_act = n_pre_splits < 1 ? 1 : n_pre_splits;
        if (s >= n_act) return;
        has_tree = (s == n_act - 1);
    }
    const int p_end = tree_wg ? 0 : min(npages, p_begin + pps);
    const int tok_begin = p_begin * kPage;
    const int tok_end = tree_wg ? 0 : min(L, p_end * kPage);
    // A prefix split of a one-round ring with one tile per wave (and no tree tiles)
    // requests its round here, once its page ids and lengths have landed, so that
    // the tiles move while the rest of the set-up runs. Every set-up load but Q's is
    // waited for first: the compiler's own waits do not count the transfers, so a
    // later wait for one of those loads would also wait for the round.
    bool early_pre = false;
    if constexpr (RING_R == 1 && RW == 1) {
        early_pre = !has_tree && !a.paged_tree && p_end > p_begin;
        if (early_pre) {
            asm volatile("" ::"v"(par_raw), "v"(own_pages));
            #pragma unroll
            for (int k = 0; k < PPT; ++k) asm volatile("" ::"v"(pid[k]));
            #pragma unroll
            for (int k = 0; k < kAncWords; ++k) asm volatile("" ::"v"(ancw[0][k]));
            const int n_pre0 = (tok_end - tok_begin + kKeyTile - 1) / kKeyTile;
            if (kw < n_pre0) {                          // wave-uniform
                const int pv = (own_pages < 0 || own_pages >= a.num_pages) ? 0 : own_pages;
                const TileSrc src{false, tok_begin + kw * kKeyTile, tok_end};
                issue_tile_own_pages<D>(a.kp, a.vp, a.Hkv, kvh, src, pv, page_lanes<D>(lane),
                                        (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)ring) +
                                            kw * Gm::BUF_BYTES,
                                        lane);
            }
        }
    }
    if (a.parent_sets && has_tree) {
        // the ancestor words come from the parent array (the loads above read a
        // buffer this launch writes, and are discarded): pointer doubling across the
        // wave's lanes for trees of at most 64 nodes, else in LDS
        if (a.N <= kWave) {
            const uint64_t set = tree_set_wave(par_own, a.N);
            #pragma unroll
            for (int blk = 0; blk < RPW; ++blk) {
                const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)set, node[blk]);
                const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(set >> 32), node[blk]);
                ancw[blk] = u64x4{row_ok[blk] ? (((uint64_t)hi << 32) | lo) : 0ull, 0, 0, 0};
            }
        } else {
            const auto sets = tree_sets_lds(par_own, a.N);
            #pragma unroll
            for (int blk = 0; blk < RPW; ++blk) {
                #pragma unroll
                for (int k = 0; k < kAncWords; ++k) ancw[blk][k] = row_ok[blk] ? sets[node[blk]][k] : 0ull;
            }
        }
    }
    if (!has_tree) {
        #pragma unroll
        for (int blk = 0; blk < RPW; ++blk) ancw[blk] = u64x4{0, 0, 0, 0};
    }

    if (tid < kAncWords) s_union[tid] = 0;
    __syncthreads();
    // union of the block's ancestor sets, for the words the tree has: OR over the
    // wave's rows (DPP, no LDS; both half-waves hold the same rows and rows past the
    // end hold zero), then one LDS atomic per word and wave. Tree tiles requested
    // early need no union (every tile is run).
    if (has_tree && kw == 0 && !early_tree) {
        #pragma unroll
        for (int k = 0; k < kAncWords; ++k) {
            if (k * 64 < a.N) {                         // uniform
                uint64_t u = ancw[0][k];
                #pragma unroll
                for (int blk = 1; blk < RPW; ++blk) u |= ancw[blk][k];
                const unsigned long long word = ((unsigned long long)wave_or_u32((uint32_t)(u >> 32)) << 32) |
                                                wave_or_u32((uint32_t)u);
                if (lane == 0 && word) atomicOr(&s_union[k], word);
            }
        }
    }
    int my_bad = 0;
    // paged tree: the pages holding cached tokens L .. L + nb - 1 (at most kMaxTreePages)
    if (a.paged_tree && has_tree && nb > 0) {
        const int first = L / kPage, count = (L + nb - 1) / kPage - first + 1;
        if (tid < count) {
            const int slot = first + tid;
            int v = slot < a.max_pages ? a.block_table[(long)b * a.max_pages + slot] : -1;
            if (v < 0 || v >= a.num_pages) {
                my_bad = 1;
                v = 0;
            }
            s_tpages[tid] = v;
        }
    }
    #pragma unroll
    for (int k = 0; k < PPT; ++k) {
        const int i = tid + k * T;
        if (i < p_end - p_begin) {
            int v = pid[k];
            if (v < 0 || v >= a.num_pages) {
                my_bad = 1;
                v = 0;
            }
            s_pages[i] = v;
        }
    }
    // the coordinates only the epilogue needs go to LDS and are read back there,
    // rather than held in registers through the tile loop
    if (tid == 0) {
        s_epi[0] = item;
        s_epi[1] = s;
        s_epi[2] = rb;
        s_epi[3] = n_act;
        s_epi[4] = n_pre_splits;
        s_epi[5] = nb;
    }
    bad = __syncthreads_or(my_bad) || bad;

    // ---- tile list: prefix tiles, then the non-empty tree tiles
    const int n_pre = (tok_end - tok_begin + kKeyTile - 1) / kKeyTile;
    int tree_list = 0, n_tree = 0;   // up to 4 tile ids, 2 bits each
    if (early_tree) {
        // every tree tile, in order, as issued (a tile no row has an ancestor in
        // contributes zero weights)
        tree_list = 0xe4;
        n_tree = n_tree_tiles;
    } else if (has_tree) {
        for (int tt = 0; tt * kKeyTile < a.N; ++tt) {
            if (s_union[tt]) {
                tree_list |= tt << (2 * n_tree);
                ++n_tree;
            }
        }
    }
    const int n_tiles = n_pre + n_tree;
    const int n_rounds = (n_tiles + KW - 1) / KW;
    const int N = a.N;
    auto tile_src = [=](int it) {
        TileSrc src;
        if (it < n_pre) {
            src.tree = false;
            src.t0 = tok_begin + it * kKeyTile;
            src.limit = tok_end;
        } else {
            src.tree = true;
            src.t0 = ((tree_list >> (2 * (it - n_pre))) & 3) * kKeyTile;
            src.limit = nb;
        }
        return src;
    };

    const uint32_t ring0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)ring);
    const int tree_tok0 = a.paged_tree ? L : -1;      // paged tree: cached token of node 0
    const uint16_t* const g_kp = a.kp;
    const uint16_t* const g_vp = a.vp;
    const uint16_t* const g_kt = a.kt;
    const uint16_t* const g_vt = a.vt;
    const int Hkv = a.Hkv;
    const float scale_log2 = a.scale_log2;

    // per-lane LDS offsets (within one V tile) of the transposing PV operand reads:
    // in 16-lane group g16, lane x reads key 16*kc + 8*rd + 4*hf + x/4 at
    // d = 32*dt + 16*(g16&1) + 4*(x&3); it receives keys 4*hf + {0..3} (+8*rd)
    // at d = 32*dt + lane%32, which is the A operand of the 32x32x16 product
    const int x16 = lane & 15, g16 = lane >> 4;
    int v_off[DT];
    #pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        const int key = 4 * hf + (x16 >> 2);
        const int d = 32 * dt + 16 * (g16 & 1) + 4 * (x16 & 3);
        v_off[dt] = key * Gm::ROW_BYTES + (((d >> 3) ^ swz_v<D>(key)) << 4) + ((d >> 2) & 1) * 8;
    }

    const PageLanes<D> pl = page_lanes<D>(lane);

    RowState<D> st[RPW];
    const float NEG = -__builtin_inff();
    #pragma unroll
    for (int blk = 0; blk < RPW; ++blk) {
        #pragma unroll
        for (int i = 0; i < DT; ++i) st[blk].o[i] = f32x16{};
        st[blk].m = NEG;
        st[blk].l = 0.f;
    }

    if constexpr (RING_R >= 2) {
        // every load the compiler issued (Q, anc, page table) has landed: from here on
        // the only vector-memory traffic is the tile ring, counted by hand. (Issuing the
        // prologue rounds before this wait, beside the Q loads, measured slower for the
        // multi-round rings.)
        __builtin_amdgcn_s_waitcnt(0);
        // prologue: RING_R - 1 rounds in flight
        #pragma unroll
        for (int p = 0; p < RING_R - 1; ++p)
            if (p < n_rounds)
                issue_round<D, DPR>(g_kp, g_vp, g_kt, g_vt, N, Hkv, tile_src, p * KW, n_tiles, b, kvh, s_pages, pl,
                                    ring0 + p * KW * Gm::BUF_BYTES, w * DPR, lane, s_tpages, tree_tok0);
    }
    // (a one-round ring issues each round and waits for all of it, which also covers
    // the set-up loads still landing from before its first round)
    for (int r = 0; r < n_rounds; ++r) {
        if constexpr (RING_R >= 2) {
            wait_rounds<DPR>(min(n_rounds - 1 - r, RING_R - 2));
            __syncthreads();      // round r is in LDS for every wave; the buffers of round r-1 are free
            if (r + RING_R - 1 < n_rounds)
                issue_round<D, DPR>(g_kp, g_vp, g_kt, g_vt, N, Hkv, tile_src, (r + RING_R - 1) * KW, n_tiles, b, kvh, s_pages, pl,
                                    ring0 + ((r + RING_R - 1) % RING_R) * KW * Gm::BUF_BYTES, w * DPR, lane,
                                    s_tpages, tree_tok0);
        } else {
            __syncthreads();      // every wave is done with the previous round
            if (!((early_tree || early_pre) && r == 0))
                issue_round<D, DPR>(g_kp, g_vp, g_kt, g_vt, N, Hkv, tile_src, r * KW, n_tiles, b, kvh, s_pages, pl,
                                    ring0, w * DPR, lane, s_tpages, tree_tok0);
            wait_vm<0>();
            __syncthreads();
        }
        const int it = r * KW + kw;
        if (it < n_tiles) {
            const char* kbuf = ring + ((r % RING_R) * KW + kw) * Gm::BUF_BYTES;
            tile_product<D, RPW>(st, kbuf, kbuf + Gm::TILE_BYTES, qreg, tile_src(it), ancw, N, scale_log2, v_off, hf,
                                 l32);
        }
    }

    item = __builtin_amdgcn_readfirstlane(s_epi[0]);
    s = __builtin_amdgcn_readfirstlane(s_epi[1]);
    rb = __builtin_amdgcn_readfirstlane(s_epi[2]);
    n_act = __builtin_amdgcn_readfirstlane(s_epi[3]);
    const int n_pre_e = __builtin_amdgcn_readfirstlane(s_epi[4]);
    const int nb_e = __builtin_amdgcn_readfirstlane(s_epi[5]);
    const float NANF = __builtin_nanf("");
    const float LN2 = 0.69314718055994530942f;
    float* mo = reinterpret_cast<float*>(ring);      // key-group merge area (reuses the ring)

    // ---- one row block's result, as (m, l, unnormalised O) per row
    // (one key group: the split's fp16 partial as stored, and its m, l and row
    // scale, kept for the merge if this workgroup arrives last)
    u32x4 hp[RPW][D / 16];
    float own_m[RPW], own_l[RPW], own_r[RPW];
    if constexpr (KW == 1) {
        #pragma unroll
        for (int blk = 0; blk < RPW; ++blk) {
            const RowState<D>& sb = st[blk];
            const float l_tot = sb.l + __shfl_xor(sb.l, 32);
            // opaque copies: the output offset is formed here, not shared with the Q
            // offset of the set-up and kept live (64-bit) through the tile loop
            int nd = node[blk], hd = head[blk], h2f = hf;
            asm volatile("" : "+v"(nd), "+v"(hd), "+v"(h2f));
            if (n_act == 1) {
                if (row_ok[blk]) {
                    const float inv = bad ? NANF : 1.f / l_tot;
                    uint16_t* op = a.out + (((long)b * a.N + nd) * a.Hq + hd) * D + 4 * h2f;
                    #pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        #pragma unroll
                        for (int rq = 0; rq < 4; ++rq) {
                            const u32x2 v = {pack_bf16x2(sb.o[dt][4 * rq] * inv, sb.o[dt][4 * rq + 1] * inv),
                                             pack_bf16x2(sb.o[dt][4 * rq + 2] * inv, sb.o[dt][4 * rq + 3] * inv)};
                            *reinterpret_cast<u32x2*>(op + dt * 32 + 8 * rq) = v;
                        }
                    }
                    if (a.lse && h2f == 0)
                        a.lse[((long)b * a.N + nd) * a.Hq + hd] = bad ? NANF : (sb.m + __log2f(l_tot)) * LN2;
                }
                continue;
            }
            const uint32_t psplit = ((uint32_t)item * a.splits + s) * RB;
            const uint32_t pr = psplit + rloc[blk];
            const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.part_o, a.part_o_bytes);
            // the row's scale: its largest |O| over both half-waves' 64 values each
            float r = 0.f;
            #pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                #pragma unroll
                for (int i = 0; i < 16; ++i) r = fmaxf(r, fabsf(sb.o[dt][i]));
            }
            r = fmaxf(r, __shfl_xor(r, 32));
            const float rinv = r > 0.f ? 1.f / r : 0.f;
            // store k: chunks j = 2k and 2k + 1 of the lane (O registers dt = j / 4,
            // 4 (j % 4) .. 4 (j % 4) + 3)
            #pragma unroll
            for (int k = 0; k < D / 16; ++k) {
                const int d0 = (2 * k) >> 2, q0 = 4 * ((2 * k) & 3), d1 = (2 * k + 1) >> 2, q1 = 4 * ((2 * k + 1) & 3);
                hp[blk][k] = u32x4{pack_f16x2(sb.o[d0][q0] * rinv, sb.o[d0][q0 + 1] * rinv),
                                   pack_f16x2(sb.o[d0][q0 + 2] * rinv, sb.o[d0][q0 + 3] * rinv),
                                   pack_f16x2(sb.o[d1][q1] * rinv, sb.o[d1][q1 + 1] * rinv),
                                   pack_f16x2(sb.o[d1][q1 + 2] * rinv, sb.o[d1][q1 + 3] * rinv)};
                st16(ro, psplit * (D * 2) + frag_half_off<D>(rloc[blk], h2f, k), __builtin_bit_cast(f32x4, hp[blk][k]));
            }
            own_m[blk] = bad ? NANF : sb.m;
            own_l[blk] = bad ? NANF : l_tot;
            own_r[blk] = r;
            if (h2f == 0)
                st16(make_rsrc(a.part_ml, a.part_ml_bytes), pr * 16, f32x4{own_m[blk], own_l[blk], r, 0.f});
        }
        if (n_act == 1) return;
    } else {
        // merge the KW key groups through LDS (one row block per wave)
        constexpr int TPR = T / RB;                 // threads per row
        constexpr int CPT = D / 4 / TPR;            // float4 chunks per thread
        const RowState<D>& st0 = st[0];
        const float l_tot = st0.l + __shfl_xor(st0.l, 32);
        __syncthreads();                               // every wave is done with the ring
        {
            char* mk = reinterpret_cast<char*>(mo) + kw * RB * D * 4;
            #pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                #pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const f32x4 v = {st0.o[dt][4 * rq], st0.o[dt][4 * rq + 1], st0.o[dt][4 * rq + 2], st0.o[dt][4 * rq + 3]};
                    *reinterpret_cast<f32x4*>(mk + merge_off<D>(rloc[0], dt * 8 + 2 * rq + hf)) = v;
                }
            }
            if (hf == 0) {
                s_ml[kw][rloc[0]][0] = st0.m;
                s_ml[kw][rloc[0]][1] = l_tot;
            }
        }
        __syncthreads();
        const int rl = tid / TPR, part = tid % TPR;
        const int grow = rb * RB + rl;
        float M = NEG;
        #pragma unroll
        for (int k = 0; k < KW; ++k) M = fmaxf(M, s_ml[k][rl][0]);
        const float M_use = (M == NEG) ? 0.f : M;
        float wk[KW];
        float Ls = 0.f;
        #pragma unroll
        for (int k = 0; k < KW; ++k) {
            wk[k] = __builtin_amdgcn_exp2f(s_ml[k][rl][0] - M_use);
            Ls += wk[k] * s_ml[k][rl][1];
        }
        // the thread's chunks are part, part + TPR, ...: each pass over c reads and
        // writes whole lines
        f32x4 acc[CPT];
        #pragma unroll
        for (int c = 0; c < CPT; ++c) {
            acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
            #pragma unroll
            for (int k = 0; k < KW; ++k)
                acc[c] += wk[k] * *reinterpret_cast<const f32x4*>(reinterpret_cast<const char*>(mo) + k * RB * D * 4 +
                                                                  merge_off<D>(rl, c * TPR + part));
        }
        if (n_act == 1) {
            if (grow < a.rows && grow / a.G < nb_e) {
                const int gnode = grow / a.G, ghead = kvh * a.G + grow % a.G;
                const float inv = bad ? NANF : 1.f / Ls;
                uint16_t* op = a.out + (((long)b * a.N + gnode) * a.Hq + ghead) * D + part * 4;
                #pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    const u32x2 v = {pack_bf16x2(acc[c][0] * inv, acc[c][1] * inv),
                                     pack_bf16x2(acc[c][2] * inv, acc[c][3] * inv)};
                    *reinterpret_cast<u32x2*>(op + 4 * TPR * c) = v;
                }
                if (a.lse && part == 0)
                    a.lse[((long)b * a.N + gnode) * a.Hq + ghead] = bad ? NANF : (M + __log2f(Ls)) * LN2;
            }
            return;
        }
        const uint32_t psplit = ((uint32_t)item * a.splits + s) * RB;
        const uint32_t pr = psplit + rl;
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.part_o, a.part_o_bytes);
        static_assert(CPT % 2 == 0, "fp16 partials pair a thread's chunks");
        float r = 0.f;
        #pragma unroll
        for (int c = 0; c < CPT; ++c)
            r = fmaxf(r, fmaxf(fmaxf(fabsf(acc[c][0]), fabsf(acc[c][1])), fmaxf(fabsf(acc[c][2]), fabsf(acc[c][3]))));
        r = group_max<TPR>(r);
        const float rinv = r > 0.f ? 1.f / r : 0.f;
        #pragma unroll
        for (int k = 0; k < CPT / 2; ++k) {
            const f32x4 x = acc[2 * k] * rinv, y = acc[2 * k + 1] * rinv;
            const u32x4 h = {pack_f16x2(x[0], x[1]), pack_f16x2(x[2], x[3]), pack_f16x2(y[0], y[1]),
                             pack_f16x2(y[2], y[3])};
            st16(ro, psplit * (D * 2) + half_off<D, TPR>(rl, part, k), __builtin_bit_cast(f32x4, h));
        }
        if (part == 0) {
            const f32x4 ml = {bad ? NANF : M, bad ? NANF : Ls, r, 0.f};
            st16(make_rsrc(a.part_ml, a.part_ml_bytes), pr * 16, ml);
        }
    }

    // ---- several splits: this split's partial is published; the last one merges
    wait_own_stores();
    __syncthreads();
    if (tid == 0) {
        const int old = arrive(&a.counters[item]);
        s_last = (old == n_act - 1);
        if (s_last) {
            acquire_agent();                   // before the reset: the fence waits for earlier stores
            reset_counter(&a.counters[item]);
        }
    }
    __syncthreads();
    if (!s_last) return;

    {
        if constexpr (kHalfPart) {
        constexpr int TPR = T / RB;                // threads per row
        constexpr int CPT = D / 4 / TPR;           // float4 chunks per thread (CPT / 2 16-byte loads per split)
        // splits per batch: every split's loads at once within the in-flight budget
        constexpr int INFLIGHT = NW <= 4 ? 64 : 32;
        constexpr int SB0 = INFLIGHT / (CPT / 2 + 1) > 1 ? INFLIGHT / (CPT / 2 + 1) : 1;
        constexpr int SB = SB0 > 16 ? 16 : SB0;
        const int rl = tid / TPR, part = tid % TPR;
        const int grow = rb * RB + rl;
        const uint32_t base = (uint32_t)item * a.splits * RB;        // + slot * RB
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.part_o, a.part_o_bytes);
        const __amdgpu_buffer_rsrc_t rml = make_rsrc(a.part_ml, a.part_ml_bytes);
        const bool out_ok = grow < a.rows && grow / a.G < nb_e;
        const int gnode = out_ok ? grow / a.G : 0, ghead = kvh * a.G + (out_ok ? grow % a.G : 0);
        float M = NEG;
        f32x4 acc[CPT];
        #pragma unroll
        for (int c = 0; c < CPT; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        float Ls = 0.f;
        for (int sp0 = 0; sp0 < n_act; sp0 += SB) {
            u32x4 v[SB][CPT / 2];
            f32x4 ml[SB];
            #pragma unroll
            for (int j = 0; j < SB; ++j) {
                const int kk = sp0 + j;
                if (kk < n_act) {                      // uniform: slots past the last split load nothing
                    const int slot = (a.tree_split && kk >= n_pre_e) ? a.splits - 1 : kk;
                    const uint32_t ps = base + (uint32_t)slot * RB;
                    #pragma unroll
                    for (int k = 0; k < CPT / 2; ++k)
                        v[j][k] = __builtin_bit_cast(u32x4, ld16(ro, ps * (D * 2) + half_off<D, TPR>(rl, part, k)));
                    ml[j] = ld16(rml, (ps + rl) * 16);
                } else {
                    #pragma unroll
                    for (int k = 0; k < CPT / 2; ++k) v[j][k] = u32x4{0u, 0u, 0u, 0u};
                    ml[j] = f32x4{NEG, 0.f, 0.f, 0.f};
                }
            }
            float mb = NEG;
            #pragma unroll
            for (int j = 0; j < SB; ++j) mb = fmaxf(mb, ml[j][0]);
            const float Mn = fmaxf(M, mb);
            const float Mn_use = (Mn == NEG) ? 0.f : Mn;
            const float sc = __builtin_amdgcn_exp2f(M - Mn_use);                          // M = -inf -> 0
            Ls *= sc;
            #pragma unroll
            for (int c = 0; c < CPT; ++c) acc[c] *= sc;
            #pragma unroll
            for (int j = 0; j < SB; ++j) {
                if (sp0 + j < n_act) {                 // uniform: no work for slots past the last split
                    const float wgt = __builtin_amdgcn_exp2f(ml[j][0] - Mn_use);
                    Ls += wgt * ml[j][1];
                    const float wr = wgt * ml[j][2];                                      // weight x row scale
                    #pragma unroll
                    for (int k = 0; k < CPT / 2; ++k) {
                        acc[2 * k] += wr * unpack_f16x4(v[j][k][0], v[j][k][1]);
                        acc[2 * k + 1] += wr * unpack_f16x4(v[j][k][2], v[j][k][3]);
                    }
                }
            }
            M = Mn;
        }
        if (out_ok) {
            const float inv = 1.f / Ls;
            uint16_t* op = a.out + (((long)b * a.N + gnode) * a.Hq + ghead) * D + part * 4;
            #pragma unroll
            for (int c = 0; c < CPT; ++c) {                   // acc[c] is chunk c * TPR + part
                const u32x2 o = {pack_bf16x2(acc[c][0] * inv, acc[c][1] * inv),
                                 pack_bf16x2(acc[c][2] * inv, acc[c][3] * inv)};
                *reinterpret_cast<u32x2*>(op + 4 * TPR * c) = o;
            }
            if (a.lse && part == 0)
                a.lse[((long)b * a.N + gnode) * a.Hq + ghead] = (M + __log2f(Ls)) * LN2;
        }
        } else {
        // One key group: every lane merges its own row's chunks in the tile loop's
        // layout, as the splits stored them. This workgroup's own partial comes from
        // registers (the fp16 values it stored, so the result does not depend on
        // which split arrives last); the others' are loaded, every split's loads of a
        // batch at once.
        constexpr int NK = D / 16;                 // 16-byte pieces of a lane's partial
        constexpr int SB = 32 / (NK + 1) > 1 ? 32 / (NK + 1) : 1;    // splits per batch
        const int own_kk = (a.tree_split && s == a.splits - 1) ? n_pre_e : s;
        const uint32_t base = (uint32_t)item * a.splits * RB;        // + slot * RB
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.part_o, a.part_o_bytes);
        const __amdgpu_buffer_rsrc_t rml = make_rsrc(a.part_ml, a.part_ml_bytes);
        #pragma unroll
        for (int blk = 0; blk < RPW; ++blk) {
            float M = NEG;
            f32x4 acc[D / 8];
            #pragma unroll
            for (int c = 0; c < D / 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
            float Ls = 0.f;
            for (int sp0 = 0; sp0 < n_act; sp0 += SB) {
                u32x4 v[SB][NK];
                f32x4 ml[SB];
                #pragma unroll
                for (int j = 0; j < SB; ++j) {
                    const int kk = sp0 + j;
                    if (kk == own_kk) {                // uniform
                        #pragma unroll
                        for (int k = 0; k < NK; ++k) v[j][k] = hp[blk][k];
                        ml[j] = f32x4{own_m[blk], own_l[blk], own_r[blk], 0.f};
                    } else if (kk < n_act) {           // uniform: slots past the last split load nothing
                        const int slot = (a.tree_split && kk >= n_pre_e) ? a.splits - 1 : kk;
                        const uint32_t ps = base + (uint32_t)slot * RB;
                        #pragma unroll
                        for (int k = 0; k < NK; ++k)
                            v[j][k] = __builtin_bit_cast(u32x4, ld16(ro, ps * (D * 2) + frag_half_off<D>(rloc[blk], hf, k)));
                        ml[j] = ld16(rml, (ps + rloc[blk]) * 16);
                    } else {
                        #pragma unroll
                        for (int k = 0; k < NK; ++k) v[j][k] = u32x4{0u, 0u, 0u, 0u};
                        ml[j] = f32x4{NEG, 0.f, 0.f, 0.f};
                    }
                }
                float mb = NEG;
                #pragma unroll
                for (int j = 0; j < SB; ++j) mb = fmaxf(mb, ml[j][0]);
                const float Mn = fmaxf(M, mb);
                const float Mn_use = (Mn == NEG) ? 0.f : Mn;
                const float sc = __builtin_amdgcn_exp2f(M - Mn_use);                      // M = -inf -> 0
                Ls *= sc;
                #pragma unroll
                for (int c = 0; c < D / 8; ++c) acc[c] *= sc;
                #pragma unroll
                for (int j = 0; j < SB; ++j) {
                    if (sp0 + j < n_act) {             // uniform: no work for slots past the last split
                        const float wgt = __builtin_amdgcn_exp2f(ml[j][0] - Mn_use);
                        Ls += wgt * ml[j][1];
                        const float wr = wgt * ml[j][2];                                  // weight x row scale
                        #pragma unroll
                        for (int k = 0; k < NK; ++k) {
                            acc[2 * k] += wr * unpack_f16x4(v[j][k][0], v[j][k][1]);
                            acc[2 * k + 1] += wr * unpack_f16x4(v[j][k][2], v[j][k][3]);
                        }
                    }
                }
                M = Mn;
            }
            if (row_ok[blk]) {
                // opaque copies, as for the direct store above
                int nd = node[blk], hd = head[blk], h2f = hf;
                asm volatile("" : "+v"(nd), "+v"(hd), "+v"(h2f));
                const float inv = 1.f / Ls;
                uint16_t* op = a.out + (((long)b * a.N + nd) * a.Hq + hd) * D + 4 * h2f;
                #pragma unroll
                for (int c = 0; c < D / 8; ++c) {               // acc[c]: d = 8c + 4 hf .. + 3
                    const u32x2 o = {pack_bf16x2(acc[c][0] * inv, acc[c][1] * inv),
                                     pack_bf16x2(acc[c][2] * inv, acc[c][3] * inv)};
                    *reinterpret_cast<u32x2*>(op + 8 * c) = o;
                }
                if (a.lse && h2f == 0)
                    a.lse[((long)b * a.N + nd) * a.Hq + hd] = (M + __log2f(Ls)) * LN2;
            }
        }
        }
    }
}

template <int D, int RW, int KW, int RPW>
__global__ __launch_bounds__(RW * KW * 64) void tree_attn_bf16_kernel(AttnArgs a) {
    tree_attn_bf16_body<D, RW, KW, RPW>(a, blockIdx.x, gridDim.x);
}

// ---------------------------------------------------------------- host side

struct AttnPlanBf16 {
    int rw, kw, rpw, rb, nrb, items, splits, pps, balanced, forced, tree_split, cus;
    long grid;
    size_t off_cnt, fill_bytes, off_ml, off_o, bytes;
};

// Zero the counters past the fixed region (a kernel, so that the call can be
// captured in a graph).
__global__ void zero_words(int* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

static int env_int(const char* name, int dflt) {
    const char* v = getenv(name);
    if (!v || !*v) return dflt;
    return atoi(v);
}

AttnPlanBf16 plan_attention_bf16(const jf_attn_shape& s, int max_prefix, int ragged) {
    AttnPlanBf16 p{};
    const long rows = (long)(s.Hq / s.Hkv) * s.N;
    // few rows -> key groups keep several tiles in flight per workgroup
    if (rows <= 64) { p.rw = 1; p.kw = 4; }
    else if (rows <= 128) { p.rw = 4; p.kw = 2; }
    else {
        // 256-row blocks (8 waves, one key group) when they give the chip enough
        // items; 128-row blocks with two key groups when 256-row blocks would leave
        // fewer items than a quarter of the CUs (one sequence: the items then need
        // many splits, each merged through fp32 partials) or when the budgets are
        // ragged (128-row blocks waste half as many padding rows). Measured: the
        // draft head's pass (1 x 256 nodes, 8192 prefix) 62.3 -> 55.4 us, ragged
        // budgets U{16..256} x 8 99.5 -> 90.3 us; batches of full trees lose
        // (budget 256 x 8: 131.5 -> 137.6 us; prefix 32768 x 4: 517 -> 588 us).
        const long items8 = (long)s.B * s.Hkv * ((rows + 255) / 256);
        if (ragged || items8 * 4 < 256) { p.rw = 4; p.kw = 2; }
        else { p.rw = 8; p.kw = 1; }
    }
    p.rpw = 1;
    {
        // Few rows but many tiles per workgroup: streaming the prefix sets the time.
        // Then one 64-row block (both row groups share every K/V tile read) with two
        // key groups (a second round of tiles in flight while one is consumed) beats
        // 32-row blocks with four key groups, which read each tile twice and drain
        // the ring every round. Measured at 16 tree nodes x 4 heads per KV head:
        // batch 8 x 16384 prefix 157 -> 104 us; at batch 1 x 2048 (2 tiles per
        // workgroup) the four key groups stay ahead (15.2 vs 19.8 us).
        const long pages = (max_prefix + kPage - 1) / kPage;
        const long tiles_per_wg = (long)s.B * s.Hkv * ((rows + 31) / 32) * ((pages + 3) / 4) / 256;
        if (rows <= 64 && tiles_per_wg >= env_int(s.B >= 2 ? "JF_STREAM_TILES" : "JF_STREAM_TILES1",
                                                  s.B >= 2 ? 8 : 32)) { p.rw = 2; p.kw = 2; }
    }
    // tuning override: JF_RW = 1, 2, 4 or 8 row groups (key groups follow)
    switch (env_int("JF_RW", 0)) {
        case 1: p.rw = 1; p.kw = 4; break;
        case 2: p.rw = 2; p.kw = 2; break;
        case 4: p.rw = 4; p.kw = 2; break;
        case 8: p.rw = 8; p.kw = 1; break;
        default: break;
    }
    // 256-row blocks as 4 waves x 2 row blocks (instead of 8 waves x 1): JF_RPW=2
    if (p.rw == 8 && env_int("JF_RPW", 1) == 2) { p.rw = 4; p.kw = 1; p.rpw = 2; }
    p.rb = 32 * p.rw * p.rpw;
    p.nrb = (int)((rows + p.rb - 1) / p.rb);
    p.items = s.B * s.Hkv * p.nrb;
    const int max_pages = (max_prefix + kPage - 1) / kPage;
    // one workgroup per CU (the LDS ring takes most of it): aim at filling 256 CUs
    const int target = env_int("JF_TARGET_WG", 256);
    p.cus = target > 0 ? target : 256;
    // at least one full round of tiles per split
    const int min_pages = 4 * p.kw;
    // one workgroup per CU: never more workgroups than the target (a second wave of
    // a few workgroups would double the time). One sequence in 256-row blocks: aim at
    // 7/8 of the target, which leaves CUs free for stragglers (measured for 256-node
    // trees: prefix 8192 62.5 -> 58.3 us, 4096 45.3 -> 43.1 us; batches gain nothing)
    const int target_split = (s.B == 1 && p.rw == 8 && env_int("JF_TARGET_WG", 0) <= 0) ? target * 7 / 8 : target;
    int splits = p.items > 0 ? target_split / p.items : 1;
    int max_splits = max_pages > 0 ? (max_pages + min_pages - 1) / min_pages : 1;
    if (max_splits > kMaxSplits) max_splits = kMaxSplits;
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
    // split partials are addressed with 32-bit buffer offsets
    while (splits > 1 && (size_t)p.items * splits * p.rb * s.D * 4 >= (size_t)0xffffff00u) {
        splits = (splits + 1) / 2;
        pps = (max_pages + splits - 1) / splits;
        pps = (pps + 3) / 4 * 4;
        if (pps > kMaxPagesPerSplit) pps = kMaxPagesPerSplit;
        splits = (max_pages + pps - 1) / pps;
        p.splits = splits;
        p.pps = pps;
        p.grid = (long)p.items * splits;
    }
    // batches of 2..kMaxBalanced sequences: the kernel cuts each sequence into pieces
    // from the actual lengths (the host knows only the longest) and deals the
    // pieces out longest first; partial slots for up to max(splits, 2) pieces
    if (s.B >= 2 && s.B <= kMaxBalanced && env_int("JF_BALANCED", 1)) {
        int smax = splits > 1 ? splits : (max_splits >= 2 ? 2 : 1);
        if ((size_t)p.items * smax * p.rb * s.D * 4 >= (size_t)0xffffff00u) smax = splits;
        p.balanced = 1;
        p.forced = forced > 0 ? 1 : 0;
        p.splits = splits = smax;
        const long units = (long)s.B * s.Hkv * smax;
        p.grid = (units + kNumXcd - 1) / kNumXcd * kNumXcd * p.nrb;
    }
    // short splits (a few rounds each): the tree tiles get a split of their own instead
    // of adding a round (and a full memory latency) to the last prefix split
    if (!p.balanced && splits > 1 && p.pps / 4 <= 8 * p.kw && env_int("JF_TREE_SPLIT", 1) &&
        (size_t)p.items * (splits + 1) * p.rb * s.D * 4 < (size_t)0xffffff00u) {
        // room for the tree's split within the target: fewer, longer prefix splits
        while (forced <= 0 && splits > 1 && (long)p.items * (splits + 1) > target) {
            int fewer = splits - 1;
            int longer = (max_pages + fewer - 1) / fewer;
            longer = (longer + 3) / 4 * 4;
            if (longer > kMaxPagesPerSplit) break;          // splits already as long as they may be
            fewer = (max_pages + longer - 1) / longer;
            if (fewer >= splits) break;
            splits = fewer;
            pps = longer;
        }
        p.pps = pps;
        p.tree_split = 1;
        splits += 1;
        p.splits = splits;
        p.grid = (long)p.items * splits;
    }
    // one sequence whose tree tiles ride on the last prefix split: count them as pages
    // when sizing the splits, so the last split takes that many fewer prefix pages and
    // no split runs longer than the others (draft head's pass, 1 x 256 nodes over 8192:
    // 32 + 4 tree tiles on the last of four splits -> 33 tiles on each)
    if (!p.balanced && !p.tree_split && splits > 1 && env_int("JF_TREE_PAGES", 1)) {
        const int tree_pages = 4 * ((s.N + kKeyTile - 1) / kKeyTile);
        int even = (max_pages + tree_pages + splits - 1) / splits;
        even = (even + 3) / 4 * 4;
        if (even <= kMaxPagesPerSplit && (max_pages + even - 1) / even == splits) {
            pps = even;
            p.pps = pps;
        }
    }
    if (splits > 1) {
        // counters: the fixed region of every workspace (self-cleaning), extended past
        // it, and zero-filled before the launch, only for more than kMaxCounters items
        p.off_cnt = 0;
        p.fill_bytes = p.items > kMaxCounters ? align256((size_t)(p.items - kMaxCounters) * 4) : 0;
        p.off_ml = kCounterBytes + p.fill_bytes;
        p.off_o = p.off_ml + align256((size_t)p.items * splits * p.rb * 4 * 4);
        // fp16 partials: O / r with r the row's largest |O|
        p.bytes = p.off_o + align256((size_t)p.items * splits * p.rb * s.D * 2);
    }
    return p;
}

template <int D, int RW, int KW, int RPW>
static hipError_t launch_bf16_t(const AttnArgs& a, long grid, hipStream_t stream) {
    hipLaunchKernelGGL((tree_attn_bf16_kernel<D, RW, KW, RPW>), dim3((unsigned)grid), dim3(RW * KW * 64), 0, stream, a);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_bf16_d(const AttnPlanBf16& p, const AttnArgs& a, hipStream_t stream) {
    if (p.rpw == 2) return launch_bf16_t<D, 4, 1, 2>(a, p.grid, stream);
    if (p.rw == 1) return launch_bf16_t<D, 1, 4, 1>(a, p.grid, stream);
    if (p.rw == 2) return launch_bf16_t<D, 2, 2, 1>(a, p.grid, stream);
    if (p.rw == 4) return launch_bf16_t<D, 4, 2, 1>(a, p.grid, stream);
    return launch_bf16_t<D, 8, 1, 1>(a, p.grid, stream);
}

// Kernel arguments of one attention call under plan p.
static AttnArgs make_attn_args(const AttnPlanBf16& p, const jf_attn_shape& s, int max_prefix, const void* q,
                               const void* k_pages, const void* v_pages, const int32_t* block_table,
                               const int32_t* prefix_len, const void* k_tree, const void* v_tree,
                               const uint64_t* anc, void* out, float* lse, void* workspace,
                               const int32_t* tree_len, int paged_tree) {
    AttnArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.kp = static_cast<const uint16_t*>(k_pages);
    a.vp = static_cast<const uint16_t*>(v_pages);
    a.block_table = block_table;
    a.prefix_len = prefix_len;
    a.kt = static_cast<const uint16_t*>(k_tree);
    a.vt = static_cast<const uint16_t*>(v_tree);
    a.anc = anc;
    a.parent_sets = nullptr;
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    char* ws = static_cast<char*>(workspace);
    a.counters = p.splits > 1 ? reinterpret_cast<int*>(ws + p.off_cnt) : nullptr;
    a.part_ml = p.splits > 1 ? reinterpret_cast<float*>(ws + p.off_ml) : nullptr;
    a.part_o = p.splits > 1 ? reinterpret_cast<float*>(ws + p.off_o) : nullptr;
    a.part_ml_bytes = (uint32_t)(p.off_o - p.off_ml);
    a.part_o_bytes = (uint32_t)(p.bytes - p.off_o);
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
    a.balanced = p.balanced;
    a.forced = p.forced;
    a.tree_tiles = (s.N + kKeyTile - 1) / kKeyTile;
    a.cus = p.cus;
    {
        const char* v = getenv("JF_BAL_CUT");
        a.cut = (v && *v) ? (float)atof(v) : 1.5f;
        const char* f = getenv("JF_BAL_HT");
        a.ht_frac = (f && *f) ? (float)atof(f) : 1.1f;
    }
    a.tree_split = p.tree_split;
    a.tree_len = tree_len;
    a.paged_tree = paged_tree;
    a.scale_log2 = s.sm_scale * 1.44269504088896340736f;
    return a;
}

// Counters past the fixed region (more than kMaxCounters items with splits) are
// zero-filled by a small kernel before the attention launch.
static void fill_counters(const AttnPlanBf16& p, void* workspace, hipStream_t stream) {
    if (p.splits > 1 && p.fill_bytes > 0) {
        const int n = (int)(p.fill_bytes / 4);
        hipLaunchKernelGGL(zero_words, dim3((n + 255) / 256), dim3(256), 0, stream,
                           reinterpret_cast<int*>(static_cast<char*>(workspace) + kCounterBytes), n);
    }
}

hipError_t launch_attention_bf16(const jf_attn_shape& s, int max_prefix, const void* q, const void* k_pages,
                                 const void* v_pages, const int32_t* block_table, const int32_t* prefix_len,
                                 const void* k_tree, const void* v_tree, const uint64_t* anc, void* out,
                                 float* lse, void* workspace, hipStream_t stream, const int32_t* tree_len,
                                 int paged_tree) {
    const AttnPlanBf16 p = plan_attention_bf16(s, max_prefix, paged_tree);
    if (p.grid == 0) return hipSuccess;
    const AttnArgs a = make_attn_args(p, s, max_prefix, q, k_pages, v_pages, block_table, prefix_len, k_tree,
                                      v_tree, anc, out, lse, workspace, tree_len, paged_tree);
    fill_counters(p, workspace, stream);
    return s.D == 128 ? launch_bf16_d<128>(p, a, stream) : launch_bf16_d<64>(p, a, stream);
}

// ---------------------------------------------------------------- fused verification

// Attention and acceptance in one grid: workgroups [0, attn_grid) run the
// attention body, the rest (one per logits row and vocabulary chunk) the
// argmax + walk. The two parts share nothing but the launch: neither waits
// for the other, so on a chip with more CUs than the attention grid fills they
// run side by side instead of one after the other. Needs 256-thread attention
// workgroups (four waves), the acceptance workgroup size.
template <int D, int RW, int KW, int RPW>
__global__ __launch_bounds__(RW * KW * 64) void tree_verify_bf16_kernel(AttnArgs a, AcceptArgs c,
                                                                         unsigned attn_grid) {
    static_assert(RW * KW * 64 == kAcceptThreads, "the two parts share the workgroup size");
    if (blockIdx.x < attn_grid) tree_attn_bf16_body<D, RW, KW, RPW>(a, blockIdx.x, attn_grid);
    else accept_logits_body<uint16_t>(c, (int)(blockIdx.x - attn_grid));
}

template <int D, int RW, int KW, int RPW>
static hipError_t launch_verify_t(const AttnArgs& a, const AcceptArgs& c, long attn_grid, long accept_grid,
                                  hipStream_t stream) {
    hipLaunchKernelGGL((tree_verify_bf16_kernel<D, RW, KW, RPW>), dim3((unsigned)(attn_grid + accept_grid)),
                       dim3(RW * KW * 64), 0, stream, a, c, (unsigned)attn_grid);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_verify_d(const AttnPlanBf16& p, const AttnArgs& a, const AcceptArgs& c, long accept_grid,
                                  hipStream_t stream) {
    if (p.rpw == 2) return launch_verify_t<D, 4, 1, 2>(a, c, p.grid, accept_grid, stream);
    if (p.rw == 1) return launch_verify_t<D, 1, 4, 1>(a, c, p.grid, accept_grid, stream);
    return launch_verify_t<D, 2, 2, 1>(a, c, p.grid, accept_grid, stream);
}

bool verify_fusable(const jf_attn_shape& s, int max_prefix, int logits_dtype) {
    if (s.dtype != JF_BF16 || logits_dtype != JF_BF16 || s.B == 0) return false;
    const AttnPlanBf16 p = plan_attention_bf16(s, max_prefix, 0);
    return p.grid > 0 && p.rw * p.kw == 4 && (p.rpw == 1 || p.rpw == 2);
}

hipError_t launch_verify_bf16(const jf_attn_shape& s, int max_prefix, const void* q, const void* k_pages,
                              const void* v_pages, const int32_t* block_table, const int32_t* prefix_len,
                              const void* k_tree, const void* v_tree, const uint64_t* anc, void* out, float* lse,
                              void* attn_workspace, int vocab, const void* logits, const int32_t* draft,
                              const int32_t* parent, int32_t* next_tokens, int32_t* accept_len,
                              int32_t* accepted_nodes, int32_t* bonus, void* accept_workspace,
                              int anc_from_parent, hipStream_t stream) {
    const AttnPlanBf16 p = plan_attention_bf16(s, max_prefix, 0);
    AttnArgs a = make_attn_args(p, s, max_prefix, q, k_pages, v_pages, block_table, prefix_len, k_tree,
                                v_tree, anc, out, lse, attn_workspace, nullptr, 0);
    const AcceptPlan ap = plan_accept(s.B, s.N, vocab);
    AcceptArgs c = make_accept_args(ap, s.N, vocab, logits, JF_BF16, draft, parent, anc, next_tokens,
                                    accept_len, accepted_nodes, bonus, accept_workspace);
    if (anc_from_parent) {
        // both parts build the ancestor sets from parent themselves; the acceptance
        // part also writes them to anc
        a.parent_sets = parent;
        c.anc_out = const_cast<uint64_t*>(anc);
    }
    const long accept_grid = (long)s.B * s.N * ap.chunks;
    fill_counters(p, attn_workspace, stream);
    return s.D == 128 ? launch_verify_d<128>(p, a, c, accept_grid, stream)
                      : launch_verify_d<64>(p, a, c, accept_grid, stream);
}

void attention_bf16_plan(const jf_attn_shape& s, int max_prefix, int ragged, int32_t* out) {
    const AttnPlanBf16 p = plan_attention_bf16(s, max_prefix, ragged);
    out[0] = p.rb;
    out[1] = p.kw;
    out[2] = p.rpw;
    out[3] = p.splits;
    out[4] = p.pps;
    out[5] = p.balanced;
    out[6] = p.tree_split;
    out[7] = (int32_t)p.grid;
}

// Enough for the plan of jf_tree_attention and that of the ragged entry point.
size_t attention_bf16_workspace_bytes(const jf_attn_shape& s, int max_prefix) {
    const size_t a = plan_attention_bf16(s, max_prefix, 0).bytes, b = plan_attention_bf16(s, max_prefix, 1).bytes;
    return a > b ? a : b;
}

}  // namespace jf

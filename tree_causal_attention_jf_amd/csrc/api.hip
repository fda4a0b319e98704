// C ABI of libjf_tree: argument checks, workspace sizing and launches.
// Every check here runs on the host before any HIP call, so a rejected call
// touches neither the device nor the caller's buffers.
#include <math.h>

#include <mutex>

#include "jf_common.h"

namespace jf {
hipError_t launch_ancestor_mask(const int32_t* parent, int B, int N, uint64_t* anc, int32_t* depth,
                                int32_t* bad_tree, hipStream_t stream);
hipError_t launch_attention_bf16(const jf_attn_shape& s, int max_prefix, const void* q, const void* k_pages,
                                 const void* v_pages, const int32_t* block_table, const int32_t* prefix_len,
                                 const void* k_tree, const void* v_tree, const uint64_t* anc, void* out,
                                 float* lse, void* workspace, hipStream_t stream, const int32_t* tree_len = nullptr,
                                 int paged_tree = 0);
hipError_t launch_attention_f32(const jf_attn_shape& s, int max_prefix, const void* q, const void* k_pages,
                                const void* v_pages, const int32_t* block_table, const int32_t* prefix_len,
                                const void* k_tree, const void* v_tree, const uint64_t* anc, void* out,
                                float* lse, hipStream_t stream);
size_t attention_bf16_workspace_bytes(const jf_attn_shape& s, int max_prefix);
hipError_t launch_accept(int B, int N, int vocab, const void* logits, int dtype, const int32_t* target_ids,
                         const int32_t* draft, const int32_t* parent, const uint64_t* anc, int32_t* next_tokens,
                         int32_t* accept_len, int32_t* accepted_nodes, int32_t* bonus, void* workspace,
                         hipStream_t stream);
size_t accept_workspace_bytes(int B, int N, int vocab);
hipError_t launch_verify_bf16(const jf_attn_shape& s, int max_prefix, const void* q, const void* k_pages,
                              const void* v_pages, const int32_t* block_table, const int32_t* prefix_len,
                              const void* k_tree, const void* v_tree, const uint64_t* anc, void* out, float* lse,
                              void* attn_workspace, int vocab, const void* logits, const int32_t* draft,
                              const int32_t* parent, int32_t* next_tokens, int32_t* accept_len,
                              int32_t* accepted_nodes, int32_t* bonus, void* accept_workspace,
                              int anc_from_parent, hipStream_t stream);
bool verify_fusable(const jf_attn_shape& s, int max_prefix, int logits_dtype);
void attention_bf16_plan(const jf_attn_shape& s, int max_prefix, int ragged, int32_t* out);
hipError_t launch_commit(const jf_attn_shape& s, const void* k_tree, const void* v_tree, const int32_t* accept_len,
                         const int32_t* accepted_nodes, const int32_t* block_table, const int32_t* prefix_len,
                         void* k_pages, void* v_pages, int32_t* new_prefix_len, hipStream_t stream);
size_t build_workspace_bytes(int B, int N, int vocab, int topk, int dtype);
hipError_t launch_build(int B, int N, int vocab, const void* logits, int dtype, int topk, int cap,
                        const int32_t* budget, int32_t* parent, int32_t* token, double* score, int32_t* tree_len,
                        void* workspace, hipStream_t stream);
}  // namespace jf

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

jf_status check_attn_shape(const jf_attn_shape* s, int32_t max_prefix_len) {
    if (!s) return JF_ERR_NULL;
    if (s->dtype != JF_F32 && s->dtype != JF_BF16) return JF_ERR_DTYPE;
    if (s->B < 0 || s->B > JF_MAX_BATCH || s->N < 1 || s->N > JF_MAX_NODES || s->Hq < 1 || s->Hkv < 1 ||
        s->Hq % s->Hkv != 0)
        return JF_ERR_SHAPE;
    if (s->num_pages < 0 || s->max_pages_per_seq < 0) return JF_ERR_SHAPE;
    if (s->D != 64 && s->D != 128) return JF_ERR_UNSUPPORTED;
    if (s->page_size != JF_PAGE_SIZE) return JF_ERR_UNSUPPORTED;
    if (max_prefix_len < 0 || (long)max_prefix_len > (long)s->max_pages_per_seq * JF_PAGE_SIZE) return JF_ERR_SHAPE;
    if (max_prefix_len > 0 && s->num_pages < 1) return JF_ERR_SHAPE;
    if (!(s->sm_scale > 0.f) || !isfinite(s->sm_scale)) return JF_ERR_SHAPE;
    // index arithmetic inside the kernels: grid and row counts fit 32 bits
    const long rows = (long)(s->Hq / s->Hkv) * s->N;
    if ((long)s->B * s->Hkv * ((rows + 63) / 64) * ((max_prefix_len / 64) + 1) > 0x7fffffffL) return JF_ERR_SHAPE;
    // work units (64-key tiles per sequence and KV head) counted in 32 bits per sequence
    if ((long)s->B * ((max_prefix_len + 63) / 64 + (s->N + 63) / 64) > 0x7fffffffL / s->Hkv) return JF_ERR_SHAPE;
    return JF_OK;
}

}  // namespace

extern "C" {

const char* jf_status_string(jf_status s) {
    switch (s) {
        case JF_OK: return "ok";
        case JF_ERR_NULL: return "a required pointer is NULL";
        case JF_ERR_SHAPE: return "a size is out of range or inconsistent";
        case JF_ERR_DTYPE: return "unknown dtype code";
        case JF_ERR_UNSUPPORTED: return "unsupported configuration (head dim must be 64 or 128, page size 16)";
        case JF_ERR_WORKSPACE: return "workspace missing or too small";
        case JF_ERR_LAUNCH: return "kernel launch failed";
        case JF_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case JF_ERR_SCRATCH:
            return "the call needs more scratch than the fixed array of jf_tree_verify_noalloc holds "
                   "(JF_NOALLOC_SCRATCH_BYTES); use jf_tree_verify with caller workspaces";
        default: return "unknown status";
    }
}

const char* jf_version(void) { return "0.1.0"; }

jf_status jf_build_ancestor_mask(const int32_t* parent, int32_t B, int32_t N, uint64_t* anc, int32_t* depth,
                                 int32_t* bad_tree, hipStream_t stream) {
    if (B < 0 || N < 1 || N > JF_MAX_NODES) return JF_ERR_SHAPE;
    if (!parent || !anc) return JF_ERR_NULL;
    if (B == 0) return JF_OK;
    return jf::launch_ancestor_mask(parent, B, N, anc, depth, bad_tree, stream) == hipSuccess ? JF_OK
                                                                                              : JF_ERR_LAUNCH;
}

size_t jf_tree_attention_workspace_bytes(const jf_attn_shape* s, int32_t max_prefix_len) {
    if (check_attn_shape(s, max_prefix_len) != JF_OK) return 0;
    if (s->dtype == JF_F32) return 0;
    return jf::attention_bf16_workspace_bytes(*s, max_prefix_len);
}

// Host checks of jf_tree_attention (nothing is launched).
static jf_status check_attention_call(const jf_attn_shape* s, int32_t max_prefix_len, const void* q,
                                      const void* k_pages, const void* v_pages, const int32_t* block_table,
                                      const int32_t* prefix_len, const void* k_tree, const void* v_tree,
                                      const uint64_t* anc, const void* out, const void* workspace,
                                      size_t workspace_bytes) {
    const jf_status st = check_attn_shape(s, max_prefix_len);
    if (st != JF_OK) return st;
    if (!q || !prefix_len || !k_tree || !v_tree || !anc || !out) return JF_ERR_NULL;
    if (max_prefix_len > 0 && (!k_pages || !v_pages || !block_table)) return JF_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(k_tree) || !aligned16(v_tree) ||
        !aligned16(out))
        return JF_ERR_ALIGN;
    const size_t need = jf_tree_attention_workspace_bytes(s, max_prefix_len);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return JF_ERR_WORKSPACE;
        if (!aligned16(workspace)) return JF_ERR_ALIGN;
    }
    return JF_OK;
}

jf_status jf_tree_attention_plan(const jf_attn_shape* s, int32_t max_prefix_len, int32_t* plan) {
    const jf_status st = check_attn_shape(s, max_prefix_len);
    if (st != JF_OK) return st;
    if (!plan) return JF_ERR_NULL;
    if (s->dtype != JF_BF16) return JF_ERR_UNSUPPORTED;
    jf::attention_bf16_plan(*s, max_prefix_len, 0, plan);
    return JF_OK;
}

jf_status jf_tree_attention_paged_tree_plan(const jf_attn_shape* s, int32_t max_prefix_len, int32_t* plan) {
    const jf_status st = check_attn_shape(s, max_prefix_len);
    if (st != JF_OK) return st;
    if (!plan) return JF_ERR_NULL;
    if (s->dtype != JF_BF16) return JF_ERR_UNSUPPORTED;
    jf::attention_bf16_plan(*s, max_prefix_len, 1, plan);
    return JF_OK;
}

jf_status jf_tree_attention(const jf_attn_shape* s, int32_t max_prefix_len, const void* q, const void* k_pages,
                            const void* v_pages, const int32_t* block_table, const int32_t* prefix_len,
                            const void* k_tree, const void* v_tree, const uint64_t* anc, void* out, float* lse,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const jf_status st = check_attention_call(s, max_prefix_len, q, k_pages, v_pages, block_table, prefix_len,
                                              k_tree, v_tree, anc, out, workspace, workspace_bytes);
    if (st != JF_OK) return st;
    if (s->B == 0) return JF_OK;
    hipError_t e;
    if (s->dtype == JF_BF16)
        e = jf::launch_attention_bf16(*s, max_prefix_len, q, k_pages, v_pages, block_table, prefix_len, k_tree,
                                      v_tree, anc, out, lse, workspace, stream);
    else
        e = jf::launch_attention_f32(*s, max_prefix_len, q, k_pages, v_pages, block_table, prefix_len, k_tree,
                                     v_tree, anc, out, lse, stream);
    return e == hipSuccess ? JF_OK : JF_ERR_LAUNCH;
}

jf_status jf_tree_attention_paged_tree(const jf_attn_shape* s, int32_t max_prefix_len, const void* q,
                                       const void* k_pages, const void* v_pages, const int32_t* block_table,
                                       const int32_t* prefix_len, const int32_t* tree_len, const uint64_t* anc,
                                       void* out, float* lse, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
    const jf_status st = check_attn_shape(s, max_prefix_len);
    if (st != JF_OK) return st;
    if (s->dtype != JF_BF16) return JF_ERR_UNSUPPORTED;
    if (!q || !k_pages || !v_pages || !block_table || !prefix_len || !anc || !out) return JF_ERR_NULL;
    if (s->num_pages < 1 || s->max_pages_per_seq < 1) return JF_ERR_SHAPE;   // the tree itself is cached
    if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(out)) return JF_ERR_ALIGN;
    const size_t need = jf_tree_attention_workspace_bytes(s, max_prefix_len);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return JF_ERR_WORKSPACE;
        if (!aligned16(workspace)) return JF_ERR_ALIGN;
    }
    if (s->B == 0) return JF_OK;
    const hipError_t e = jf::launch_attention_bf16(*s, max_prefix_len, q, k_pages, v_pages, block_table, prefix_len,
                                                   nullptr, nullptr, anc, out, lse, workspace, stream, tree_len, 1);
    return e == hipSuccess ? JF_OK : JF_ERR_LAUNCH;
}

size_t jf_tree_accept_workspace_bytes(int32_t B, int32_t N, int32_t vocab) {
    if (B < 0 || N < 1 || N > JF_MAX_NODES || vocab < 1) return 0;
    return jf::accept_workspace_bytes(B, N, vocab);
}

// Host checks of jf_tree_accept (nothing is launched).
static jf_status check_accept_call(int32_t B, int32_t N, int32_t vocab, const void* target_logits,
                                   int32_t logits_dtype, const int32_t* target_ids, const int32_t* draft_tokens,
                                   const int32_t* parent, const uint64_t* anc, const int32_t* next_tokens,
                                   const int32_t* accept_len, const int32_t* accepted_nodes,
                                   const int32_t* bonus_token, const void* workspace, size_t workspace_bytes) {
    if (B < 0 || N < 1 || N > JF_MAX_NODES || vocab < 1) return JF_ERR_SHAPE;
    if ((target_logits == nullptr) == (target_ids == nullptr)) return JF_ERR_SHAPE;
    if (!draft_tokens || !parent || !anc || !next_tokens || !accept_len || !accepted_nodes || !bonus_token)
        return JF_ERR_NULL;
    if (target_logits) {
        if (logits_dtype != JF_F32 && logits_dtype != JF_BF16) return JF_ERR_DTYPE;
        const size_t need = jf::accept_workspace_bytes(B, N, vocab);
        if (!workspace || workspace_bytes < need) return JF_ERR_WORKSPACE;
        if (!aligned16(workspace)) return JF_ERR_ALIGN;
        if ((long)B * N * ((vocab + 4095) / 4096) > 0x7fffffffL) return JF_ERR_SHAPE;
        if (B > JF_WORKSPACE_COUNTER_BYTES / 4) return JF_ERR_SHAPE;   // one counter per sequence
    }
    return JF_OK;
}

jf_status jf_tree_accept(int32_t B, int32_t N, int32_t vocab, const void* target_logits, int32_t logits_dtype,
                         const int32_t* target_ids, const int32_t* draft_tokens, const int32_t* parent,
                         const uint64_t* anc, int32_t* next_tokens, int32_t* accept_len, int32_t* accepted_nodes,
                         int32_t* bonus_token, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const jf_status st = check_accept_call(B, N, vocab, target_logits, logits_dtype, target_ids, draft_tokens,
                                           parent, anc, next_tokens, accept_len, accepted_nodes, bonus_token,
                                           workspace, workspace_bytes);
    if (st != JF_OK) return st;
    if (B == 0) return JF_OK;
    const hipError_t e = jf::launch_accept(B, N, vocab, target_logits, logits_dtype, target_ids, draft_tokens,
                                           parent, anc, next_tokens, accept_len, accepted_nodes, bonus_token,
                                           workspace, stream);
    return e == hipSuccess ? JF_OK : JF_ERR_LAUNCH;
}

jf_status jf_tree_verify(const jf_attn_shape* s, int32_t max_prefix_len, const void* q, const void* k_pages,
                         const void* v_pages, const int32_t* block_table, const int32_t* prefix_len,
                         const void* k_tree, const void* v_tree, uint64_t* anc, int32_t anc_from_parent,
                         void* out, float* lse, void* attn_workspace, size_t attn_workspace_bytes, int32_t vocab,
                         const void* target_logits, int32_t logits_dtype, const int32_t* draft_tokens,
                         const int32_t* parent, int32_t* next_tokens, int32_t* accept_len,
                         int32_t* accepted_nodes, int32_t* bonus_token, void* accept_workspace,
                         size_t accept_workspace_bytes, hipStream_t stream) {
    jf_status st = check_attention_call(s, max_prefix_len, q, k_pages, v_pages, block_table, prefix_len, k_tree,
                                        v_tree, anc, out, attn_workspace, attn_workspace_bytes);
    if (st != JF_OK) return st;
    if (!target_logits) return JF_ERR_NULL;
    if (anc_from_parent != 0 && anc_from_parent != 1) return JF_ERR_SHAPE;
    st = check_accept_call(s->B, s->N, vocab, target_logits, logits_dtype, nullptr, draft_tokens, parent, anc,
                           next_tokens, accept_len, accepted_nodes, bonus_token, accept_workspace,
                           accept_workspace_bytes);
    if (st != JF_OK) return st;
    const size_t attn_need = jf_tree_attention_workspace_bytes(s, max_prefix_len);
    if (attn_need > 0) {
        const char* a0 = static_cast<const char*>(attn_workspace);
        const char* c0 = static_cast<const char*>(accept_workspace);
        const size_t acc_need = jf::accept_workspace_bytes(s->B, s->N, vocab);
        if (a0 < c0 + acc_need && c0 < a0 + attn_need) return JF_ERR_WORKSPACE;
    }
    if (s->B == 0) return JF_OK;
    hipError_t e;
    if (jf::verify_fusable(*s, max_prefix_len, logits_dtype)) {
        e = jf::launch_verify_bf16(*s, max_prefix_len, q, k_pages, v_pages, block_table, prefix_len, k_tree, v_tree,
                                   anc, out, lse, attn_workspace, vocab, target_logits, draft_tokens, parent,
                                   next_tokens, accept_len, accepted_nodes, bonus_token, accept_workspace,
                                   anc_from_parent, stream);
    } else {
        e = anc_from_parent ? jf::launch_ancestor_mask(parent, s->B, s->N, anc, nullptr, nullptr, stream)
                            : hipSuccess;
        if (e == hipSuccess)
            e = s->dtype == JF_BF16
                ? jf::launch_attention_bf16(*s, max_prefix_len, q, k_pages, v_pages, block_table, prefix_len,
                                            k_tree, v_tree, anc, out, lse, attn_workspace, stream)
                : jf::launch_attention_f32(*s, max_prefix_len, q, k_pages, v_pages, block_table, prefix_len,
                                           k_tree, v_tree, anc, out, lse, stream);
        if (e == hipSuccess)
            e = jf::launch_accept(s->B, s->N, vocab, target_logits, logits_dtype, nullptr, draft_tokens, parent,
                                  anc, next_tokens, accept_len, accepted_nodes, bonus_token, accept_workspace,
                                  stream);
    }
    return e == hipSuccess ? JF_OK : JF_ERR_LAUNCH;
}

jf_status jf_commit_accepted(const jf_attn_shape* s, const void* k_tree, const void* v_tree,
                             const int32_t* accept_len, const int32_t* accepted_nodes, const int32_t* block_table,
                             const int32_t* prefix_len, void* k_pages, void* v_pages, int32_t* new_prefix_len,
                             hipStream_t stream) {
    if (!s) return JF_ERR_NULL;
    if (s->dtype != JF_F32 && s->dtype != JF_BF16) return JF_ERR_DTYPE;
    if (s->B < 0 || s->B > JF_MAX_BATCH || s->N < 1 || s->N > JF_MAX_NODES || s->Hkv < 1 || s->num_pages < 0 ||
        s->max_pages_per_seq < 0)
        return JF_ERR_SHAPE;
    if (s->D != 64 && s->D != 128) return JF_ERR_UNSUPPORTED;
    if (s->page_size != JF_PAGE_SIZE) return JF_ERR_UNSUPPORTED;
    if (!k_tree || !v_tree || !accept_len || !accepted_nodes || !block_table || !prefix_len || !k_pages || !v_pages ||
        !new_prefix_len)
        return JF_ERR_NULL;
    if (!aligned16(k_tree) || !aligned16(v_tree) || !aligned16(k_pages) || !aligned16(v_pages)) return JF_ERR_ALIGN;
    if (new_prefix_len == prefix_len) return JF_ERR_SHAPE;   // read by every workgroup while one writes
    if (s->B == 0) return JF_OK;
    const hipError_t e = jf::launch_commit(*s, k_tree, v_tree, accept_len, accepted_nodes, block_table, prefix_len,
                                           k_pages, v_pages, new_prefix_len, stream);
    return e == hipSuccess ? JF_OK : JF_ERR_LAUNCH;
}

namespace {
bool build_shape_ok(int32_t B, int32_t N, int32_t vocab, int32_t topk) {
    return B >= 0 && B <= JF_MAX_BATCH && B <= JF_WORKSPACE_COUNTER_BYTES / 4 && N >= 1 && N <= JF_MAX_NODES &&
           vocab >= 1 && topk >= 1 && topk <= JF_MAX_TOPK &&
           (long)B * (N > 1 ? N - 1 : 1) * ((vocab + 16383) / 16384) <= 0x7fffffffL;
}
}  // namespace

size_t jf_build_tree_workspace_bytes(int32_t B, int32_t N, int32_t vocab, int32_t topk, int32_t logits_dtype) {
    if (!build_shape_ok(B, N, vocab, topk) || (logits_dtype != JF_F32 && logits_dtype != JF_BF16)) return 0;
    return jf::build_workspace_bytes(B, N, vocab, topk, logits_dtype);
}

jf_status jf_build_tree(int32_t B, int32_t N, int32_t vocab, const void* draft_logits, int32_t logits_dtype,
                        int32_t topk, int32_t max_path_nodes, const int32_t* budget, int32_t* parent,
                        int32_t* token, double* score, int32_t* tree_len, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
    if (!build_shape_ok(B, N, vocab, topk) || max_path_nodes < 1) return JF_ERR_SHAPE;
    if (logits_dtype != JF_F32 && logits_dtype != JF_BF16) return JF_ERR_DTYPE;
    if (!draft_logits || !parent || !token || !tree_len) return JF_ERR_NULL;
    const size_t need = jf::build_workspace_bytes(B, N, vocab, topk, logits_dtype);
    if (!workspace || workspace_bytes < need) return JF_ERR_WORKSPACE;
    if (!aligned16(workspace)) return JF_ERR_ALIGN;
    if (B == 0) return JF_OK;
    const hipError_t e = jf::launch_build(B, N, vocab, draft_logits, logits_dtype, topk, max_path_nodes, budget,
                                          parent, token, score, tree_len, workspace, stream);
    return e == hipSuccess ? JF_OK : JF_ERR_LAUNCH;
}

}  // extern "C"

// ---------------------------------------------------------------- verification without allocation

namespace {

// The fixed scratch of jf_tree_verify_noalloc: its acceptance workspace, then its
// attention workspace, each starting with its own counter region. Every GPU the
// library is loaded on holds one copy (zero-initialised with the code object)
// until the process ends.
static __device__ __align__(256) char scratch[JF_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, once looked up

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Zero the counter regions of both workspaces (a kernel, not a memset, so the
// call can be captured into a graph).
__global__ void clear_counter_regions(int* accept_counters, int* attn_counters) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < jf::kMaxCounters) {
        accept_counters[i] = 0;
        if (attn_counters) attn_counters[i] = 0;
    }
}

// Device address of `scratch` on device `dev` (looked up once per device, with
// that device current). The array's name is a host-side stand-in, never passed
// to a kernel.
hipError_t scratch_on_device(int dev, char** out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = static_cast<char*>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

jf_status jf_tree_verify_noalloc(const jf_attn_shape* s, int32_t max_prefix_len, const void* q,
                                 const void* k_pages, const void* v_pages, const int32_t* block_table,
                                 const int32_t* prefix_len, const void* k_tree, const void* v_tree, uint64_t* anc,
                                 int32_t anc_from_parent, void* out, float* lse, int32_t vocab,
                                 const void* target_logits, int32_t logits_dtype, const int32_t* draft_tokens,
                                 const int32_t* parent, int32_t* next_tokens, int32_t* accept_len,
                                 int32_t* accepted_nodes, int32_t* bonus_token, hipStream_t stream) {
    // the host checks of jf_tree_verify, with workspaces of the required sizes
    // standing in for the fixed array (nothing is launched or looked up before
    // the call is known to be valid)
    jf_status st = check_attention_call(s, max_prefix_len, q, k_pages, v_pages, block_table, prefix_len, k_tree,
                                        v_tree, anc, out, reinterpret_cast<void*>(256), ~(size_t)0);
    if (st != JF_OK) return st;
    if (!target_logits) return JF_ERR_NULL;
    if (anc_from_parent != 0 && anc_from_parent != 1) return JF_ERR_SHAPE;
    st = check_accept_call(s->B, s->N, vocab, target_logits, logits_dtype, nullptr, draft_tokens, parent, anc,
                           next_tokens, accept_len, accepted_nodes, bonus_token, reinterpret_cast<void*>(256),
                           ~(size_t)0);
    if (st != JF_OK) return st;
    const size_t acc_need = jf::accept_workspace_bytes(s->B, s->N, vocab);
    const size_t attn_need = jf_tree_attention_workspace_bytes(s, max_prefix_len);
    const size_t attn_off = align256(acc_need);
    if (attn_off + attn_need > (size_t)JF_NOALLOC_SCRATCH_BYTES) return JF_ERR_SCRATCH;
    if (s->B == 0) return JF_OK;

    int dev = -1;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return JF_ERR_LAUNCH;
    char* base = nullptr;
    if (scratch_on_device(dev, &base) != hipSuccess) return JF_ERR_LAUNCH;
    char* acc_ws = base;
    char* attn_ws = attn_need > 0 ? base + attn_off : nullptr;
    hipLaunchKernelGGL(clear_counter_regions, dim3((jf::kMaxCounters + 255) / 256), dim3(256), 0, stream,
                       reinterpret_cast<int*>(acc_ws), reinterpret_cast<int*>(attn_ws));
    if (hipGetLastError() != hipSuccess) return JF_ERR_LAUNCH;
    return jf_tree_verify(s, max_prefix_len, q, k_pages, v_pages, block_table, prefix_len, k_tree, v_tree, anc,
                          anc_from_parent, out, lse, attn_ws, attn_need, vocab, target_logits, logits_dtype,
                          draft_tokens, parent, next_tokens, accept_len, accepted_nodes, bonus_token, acc_ws,
                          acc_need, stream);
}

}  // extern "C"

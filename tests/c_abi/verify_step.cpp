// One verification step driven through the C ABI alone (no Python, no torch):
// device buffers from hipMalloc, inputs from a fixed integer hash, then
//   jf_build_ancestor_mask + jf_tree_attention + jf_tree_accept
// against jf_tree_verify with the ancestor bitsets built inside the call.
// The two must agree bit for bit (outputs, log-sum-exp, acceptance, bitsets).
// Prints one line per check; exit status 0 when everything agrees.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "jf_tree.h"

#define CHECK_HIP(x)                                                                   \
    do {                                                                               \
        hipError_t e_ = (x);                                                           \
        if (e_ != hipSuccess) {                                                        \
            std::printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
            return 2;                                                                  \
        }                                                                              \
    } while (0)
#define CHECK_JF(x)                                                                    \
    do {                                                                               \
        jf_status s_ = (x);                                                            \
        if (s_ != JF_OK) {                                                             \
            std::printf("%s returned %s\n", #x, jf_status_string(s_));                \
            return 3;                                                                  \
        }                                                                              \
    } while (0)

static uint32_t hash32(uint32_t x) {
    x ^= x >> 16; x *= 0x7feb352dU; x ^= x >> 15; x *= 0x846ca68bU; x ^= x >> 16;
    return x;
}

// bf16 bits of a value in [-scale, scale) drawn from the hash (round to nearest even)
static uint16_t bf16_from(uint32_t h, float scale) {
    const float v = ((float)(h & 0xffffff) / 16777216.0f * 2.0f - 1.0f) * scale;
    uint32_t u;
    std::memcpy(&u, &v, 4);
    return (uint16_t)((u + 0x7fff + ((u >> 16) & 1)) >> 16);
}

template <typename T>
static T* upload(const std::vector<T>& h) {
    T* d = nullptr;
    if (hipMalloc(&d, h.size() * sizeof(T) + 16) != hipSuccess) return nullptr;
    if (hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess) return nullptr;
    return d;
}

template <typename T>
static std::vector<T> download(const T* d, size_t n) {
    std::vector<T> h(n);
    if (hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost) != hipSuccess) h.clear();
    return h;
}

int main() {
    const int B = 2, N = 16, Hq = 8, Hkv = 2, D = 128, V = 3000, P = 16;
    const int lens[B] = {100, 37};
    const int max_prefix = 100, max_pages = (max_prefix + 15) / 16;
    // paged prefix: page ids dealt backwards from the pool
    std::vector<int32_t> table(B * max_pages, 0), plen(lens, lens + B);
    int next_page = P - 1;
    for (int b = 0; b < B; ++b)
        for (int p = 0; p < (lens[b] + 15) / 16; ++p) table[b * max_pages + p] = next_page--;
    std::vector<uint16_t> q((size_t)B * N * Hq * D), kp((size_t)P * Hkv * 16 * D), vp(kp.size()),
        kt((size_t)B * N * Hkv * D), vt(kt.size()), logits((size_t)B * N * V);
    uint32_t seed = 1;
    for (auto& x : q) x = bf16_from(hash32(seed++), 1.0f);
    for (auto& x : kp) x = bf16_from(hash32(seed++), 1.0f);
    for (auto& x : vp) x = bf16_from(hash32(seed++), 1.0f);
    for (auto& x : kt) x = bf16_from(hash32(seed++), 1.0f);
    for (auto& x : vt) x = bf16_from(hash32(seed++), 1.0f);
    for (auto& x : logits) x = bf16_from(hash32(seed++), 3.0f);
    // a random recursive tree per sequence; every node's first child agrees with the target
    std::vector<int32_t> parent(B * N), draft(B * N, -1);
    for (int b = 0; b < B; ++b) {
        parent[b * N] = -1;
        for (int i = 1; i < N; ++i) parent[b * N + i] = (int)(hash32(seed++) % (uint32_t)i);
        std::vector<int> first(N, -1);
        for (int i = 1; i < N; ++i) {
            const int p = parent[b * N + i];
            draft[b * N + i] = (int)(hash32(seed++) % V);
            if (first[p] < 0) {
                first[p] = i;
                logits[((size_t)b * N + p) * V + draft[b * N + i]] = 0x4120;    // 10.0 in bf16: the row's max
            } else if (draft[b * N + i] == draft[b * N + first[p]]) {
                draft[b * N + i] = (draft[b * N + i] + 1) % V;                 // only the first child agrees
            }
        }
    }

    jf_attn_shape s = {B, N, Hq, Hkv, D, 16, P, max_pages, JF_BF16, 0.08838834764831845f};
    const size_t ws_attn = jf_tree_attention_workspace_bytes(&s, max_prefix);
    const size_t ws_acc = jf_tree_accept_workspace_bytes(B, N, V);
    void *wa = nullptr, *wc = nullptr;
    CHECK_HIP(hipMalloc(&wa, ws_attn + 256));
    CHECK_HIP(hipMalloc(&wc, ws_acc + 256));
    CHECK_HIP(hipMemset(wa, 0, ws_attn + 256));          // counter regions start at zero
    CHECK_HIP(hipMemset(wc, 0, ws_acc + 256));

    uint16_t *dq = upload(q), *dkp = upload(kp), *dvp = upload(vp), *dkt = upload(kt), *dvt = upload(vt);
    uint16_t* dlog = upload(logits);
    int32_t *dtab = upload(table), *dplen = upload(plen), *dpar = upload(parent), *ddraft = upload(draft);
    if (!dq || !dkp || !dvp || !dkt || !dvt || !dlog || !dtab || !dplen || !dpar || !ddraft) return 2;
    uint64_t *anc1 = nullptr, *anc2 = nullptr;
    uint16_t *out1 = nullptr, *out2 = nullptr;
    float *lse1 = nullptr, *lse2 = nullptr;
    int32_t *nx1, *nx2, *al1, *al2, *nd1, *nd2, *bo1, *bo2;
    CHECK_HIP(hipMalloc(&anc1, (size_t)B * N * 32));
    CHECK_HIP(hipMalloc(&anc2, (size_t)B * N * 32));
    CHECK_HIP(hipMalloc(&out1, q.size() * 2));
    CHECK_HIP(hipMalloc(&out2, q.size() * 2));
    CHECK_HIP(hipMalloc(&lse1, (size_t)B * N * Hq * 4));
    CHECK_HIP(hipMalloc(&lse2, (size_t)B * N * Hq * 4));
    for (int32_t** p : {&nx1, &nx2, &nd1, &nd2}) CHECK_HIP(hipMalloc(p, (size_t)B * N * 4));
    for (int32_t** p : {&al1, &al2, &bo1, &bo2}) CHECK_HIP(hipMalloc(p, (size_t)B * 4));

    // three calls
    CHECK_JF(jf_build_ancestor_mask(dpar, B, N, anc1, nullptr, nullptr, nullptr));
    CHECK_JF(jf_tree_attention(&s, max_prefix, dq, dkp, dvp, dtab, dplen, dkt, dvt, anc1, out1, lse1, wa, ws_attn,
                               nullptr));
    CHECK_JF(jf_tree_accept(B, N, V, dlog, JF_BF16, nullptr, ddraft, dpar, anc1, nx1, al1, nd1, bo1, wc, ws_acc,
                            nullptr));
    // one call, bitsets built from the parents
    CHECK_JF(jf_tree_verify(&s, max_prefix, dq, dkp, dvp, dtab, dplen, dkt, dvt, anc2, 1, out2, lse2, wa, ws_attn,
                            V, dlog, JF_BF16, ddraft, dpar, nx2, al2, nd2, bo2, wc, ws_acc, nullptr));
    CHECK_HIP(hipDeviceSynchronize());

    int bad = 0;
    auto same = [&](const char* what, const void* a, const void* b, size_t bytes) {
        std::vector<char> x(bytes), y(bytes);
        const bool copied = hipMemcpy(x.data(), a, bytes, hipMemcpyDeviceToHost) == hipSuccess &&
                            hipMemcpy(y.data(), b, bytes, hipMemcpyDeviceToHost) == hipSuccess;
        const bool ok = copied && std::memcmp(x.data(), y.data(), bytes) == 0;
        std::printf("%s: %s\n", what, ok ? "identical" : "DIFFERENT");
        bad += !ok;
    };
    same("ancestor bitsets", anc1, anc2, (size_t)B * N * 32);
    same("attention output", out1, out2, q.size() * 2);
    same("log-sum-exp", lse1, lse2, (size_t)B * N * Hq * 4);
    same("next tokens", nx1, nx2, (size_t)B * N * 4);
    same("accepted nodes", nd1, nd2, (size_t)B * N * 4);
    same("accept lengths", al1, al2, (size_t)B * 4);
    same("bonus tokens", bo1, bo2, (size_t)B * 4);
    const std::vector<int32_t> al = download(al2, B);
    const std::vector<uint16_t> o = download(out2, q.size());
    int finite = 1;
    for (uint16_t x : o) finite &= ((x & 0x7f80) != 0x7f80);
    std::printf("outputs finite: %s\n", finite ? "yes" : "NO");
    // the accepted path is the chain of first children from the root
    for (int b = 0; b < B; ++b) {
        int v = 0, len = 0;
        for (bool more = true; more;) {
            more = false;
            for (int i = 1; i < N; ++i)
                if (parent[b * N + i] == v) { v = i; ++len; more = true; break; }
        }
        std::printf("sequence %d: accept_len %d (first-child chain %d)\n", b, al.size() ? al[b] : -1, len);
        bad += (al.size() == 0 || al[b] != len);
    }
    bad += !finite;
    std::printf("%s\n", bad ? "FAILED" : "ok");
    return bad ? 1 : 0;
}

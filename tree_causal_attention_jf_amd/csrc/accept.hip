// Greedy tree acceptance: the target's choice per node (first index of the
// row's largest logit) and the longest agreeing root-to-node path.
//
// Acceptance rule: gist.science lay summary of "JetFlow ..." and the qxai.app
// commentary (drafted tokens are kept up to the first disagreement); over a
// tree the accepted path is the longest one on which every node agrees.
//
// Logits mode runs as ONE launch. The vocabulary of each row is cut into C
// chunks; workgroup (row, chunk) streams its chunk with 16-byte loads and
// publishes its winner as one order-preserving 64-bit key (value, then the
// smaller index). The last of a sequence's N * C workgroups to finish (one
// agent-scope counter per sequence) merges the keys with LDS atomic max, writes
// next_tokens, and runs the walk from LDS. The counters return to zero, so the
// workspace never needs clearing again.
#include "accept_device.h"

namespace jf {

__global__ __launch_bounds__(kAcceptThreads) void accept_ids_kernel(
    int N, const int32_t* __restrict__ target_ids, const int32_t* __restrict__ draft,
    const int32_t* __restrict__ parent, const uint64_t* __restrict__ anc, int32_t* __restrict__ next_tokens,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ accepted_nodes, int32_t* __restrict__ bonus) {
    const int b = blockIdx.x;
    const NodeIn nd = load_node(b, N, parent, draft, anc);
    if (threadIdx.x < N) next_tokens[(size_t)b * N + threadIdx.x] = target_ids[(size_t)b * N + threadIdx.x];
    walk_sequence(b, N, nd.p, nd.d, nd.a, target_ids + (size_t)b * N, accept_len, accepted_nodes, bonus);
}


// PATHS 1: every chunk fits in registers; 2: chunks are scanned in batches
// (one instantiation each, so neither carries the other's registers)
template <typename T, int PATHS>
__global__ __launch_bounds__(kAcceptThreads) void accept_logits_kernel(AcceptArgs a) {
    accept_logits_body<T, PATHS>(a, blockIdx.x);
}

// ---------------------------------------------------------------- host side

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

AcceptPlan plan_accept(int B, int N, int vocab) {
    AcceptPlan p{};
    const long rows = (long)B * N;
    // >= 128 values (4 batches of 4 loads) per thread: every workgroup of a sequence
    // arrives on that sequence's one counter, so fewer, longer chunks contend less
    // (16 rows x 151936: 304 workgroups 10.6 us, 80 workgroups 9.4 us)
    const int min_chunk = 32768;
    int chunks = (int)((1024 + rows - 1) / (rows > 0 ? rows : 1));   // aim for ~1024 workgroups
    const int max_chunks = (vocab + min_chunk - 1) / min_chunk;
    chunks = chunks < 1 ? 1 : chunks;
    chunks = chunks > max_chunks ? max_chunks : chunks;
    chunks = chunks < 1 ? 1 : chunks;
    int len = (vocab + chunks - 1) / chunks;
    len = (len + 7) / 8 * 8;                          // keeps 16-byte alignment of every chunk
    chunks = (vocab + len - 1) / len;
    p.chunks = chunks;
    p.chunk_len = len;
    p.off_seq = 0;                                     // B <= kMaxCounters (host check)
    // two-level arrival for sequences with many workgroups, while the group counters
    // fit the fixed counter region beside the B sequence counters (every group has
    // at least one member). Measured: 256 workgroups per sequence 60.8 -> 56.3 us;
    // at 80 the extra level costs more (9.25 -> 10.05 us) than the contention it saves.
    const int per_seq = N * chunks;
    int groups = 1;
    if (per_seq >= 160 && B > 0) {
        groups = per_seq / 16 < 16 ? per_seq / 16 : 16;
        const int room = (kMaxCounters - B) / B;
        if (groups > room) groups = room;
        if (groups < 2) groups = 1;
    }
    p.groups = groups;
    p.off_group = (size_t)B * 4;
    p.off_part = kCounterBytes;
    p.bytes = p.off_part + align_up((size_t)rows * chunks * 8, 256);
    return p;
}

AcceptArgs make_accept_args(const AcceptPlan& p, int N, int vocab, const void* logits, int dtype,
                            const int32_t* draft, const int32_t* parent, const uint64_t* anc, int32_t* next_tokens,
                            int32_t* accept_len, int32_t* accepted_nodes, int32_t* bonus, void* workspace) {
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
    a.seq_count = reinterpret_cast<int*>(ws + p.off_seq);
    a.group_count = reinterpret_cast<int*>(ws + p.off_group);
    a.groups = p.groups;
    a.partial = reinterpret_cast<uint64_t*>(ws + p.off_part);
    a.N = N;
    a.vocab = vocab;
    a.chunks = p.chunks;
    a.chunk_len = p.chunk_len;
    const size_t elt = dtype == JF_BF16 ? 2 : 4;
    a.aligned = ((reinterpret_cast<uintptr_t>(logits) % 16) == 0) && (((size_t)vocab * elt) % 16 == 0);
    a.anc_out = nullptr;
    return a;
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
    const AcceptArgs a = make_accept_args(p, N, vocab, logits, dtype, draft, parent, anc, next_tokens, accept_len,
                                          accepted_nodes, bonus, workspace);
    const dim3 grid((unsigned)((long)B * N * p.chunks));
    const int epv = dtype == JF_BF16 ? 8 : 4;
    const bool in_regs = (p.chunk_len + epv - 1) / epv <= kRegChunkVecs;
    if (dtype == JF_BF16) {
        if (in_regs) hipLaunchKernelGGL((accept_logits_kernel<uint16_t, 1>), grid, dim3(kAcceptThreads), 0, stream, a);
        else hipLaunchKernelGGL((accept_logits_kernel<uint16_t, 2>), grid, dim3(kAcceptThreads), 0, stream, a);
    } else {
        if (in_regs) hipLaunchKernelGGL((accept_logits_kernel<float, 1>), grid, dim3(kAcceptThreads), 0, stream, a);
        else hipLaunchKernelGGL((accept_logits_kernel<float, 2>), grid, dim3(kAcceptThreads), 0, stream, a);
    }
    return hipGetLastError();
}

size_t accept_workspace_bytes(int B, int N, int vocab) { return plan_accept(B, N, vocab).bytes; }

}  // namespace jf

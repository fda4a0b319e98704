/*
 * jf_tree.h -- C ABI of the MI355X (gfx950) tree-causal attention and greedy
 * tree-acceptance library (libjf_tree.so).
 *
 * The operations come from "JetFlow: Breaking the Scaling Ceiling of
 * Speculative Decoding with Parallel Tree Drafting" as summarised on the
 * gist.science pages:
 *   - section 2 (method), tree-causal attention mask: each draft-tree node
 *     attends to the input prefix and to its own ancestors in the tree (and,
 *     on our reading, itself), never to descendants or unrelated siblings;
 *   - section 3 (contributions): the tree is verified in one target pass over
 *     a paged KV cache;
 *   - lay summary / qxai.app commentary: the target keeps the drafted tokens
 *     up to the first disagreement.
 *
 * Conventions shared by every entry point
 *   - Every array argument is a DEVICE pointer owned by the caller. The
 *     library never allocates, frees or keeps a pointer after returning.
 *     Scratch memory comes from the caller's `workspace`.
 *   - Every call is asynchronous on `stream` and never synchronises.
 *   - A host-checkable argument error returns a non-zero jf_status before any
 *     launch; nothing is written. Errors that only the device can see (an
 *     invalid tree, an out-of-range page id or prefix length) are reported as
 *     described for each call.
 *   - Trees: N nodes numbered in creation order, 1 <= N <= 256,
 *     parent[0] = -1 and 0 <= parent[i] < i for i > 0. Node 0 is the last
 *     committed token; nodes 1..N-1 are drafts.
 *   - Ancestor bitset `anc`: uint64 [B, N, 4]; node j is bit (j % 64) of word
 *     (j / 64); row i has the bits of every node on the root-to-i path,
 *     i itself included. Bits >= N are zero.
 *   - Thread safety: the library keeps no mutable global state besides the
 *     per-device address of the fixed scratch array of jf_tree_verify_noalloc
 *     (looked up once per device, under a lock). Two calls in flight at the
 *     same time must not share a workspace.
 */
#ifndef JF_TREE_H
#define JF_TREE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t jf_status;
enum {
    JF_OK = 0,
    JF_ERR_NULL = 1,         /* a required pointer is NULL                      */
    JF_ERR_SHAPE = 2,        /* a size is out of range or inconsistent          */
    JF_ERR_DTYPE = 3,        /* unknown dtype code                              */
    JF_ERR_UNSUPPORTED = 4,  /* valid but not implemented (e.g. D not 64/128)   */
    JF_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than required         */
    JF_ERR_LAUNCH = 6,       /* the HIP runtime refused a launch                */
    JF_ERR_ALIGN = 7,        /* a pointer is not 16-byte aligned                */
    JF_ERR_SCRATCH = 8       /* jf_tree_verify_noalloc: the call needs more than
                                JF_NOALLOC_SCRATCH_BYTES of scratch             */
};

/* Element types of floating-point arrays. */
enum { JF_F32 = 0, JF_BF16 = 1 };

/* Longest tree the 256-bit ancestor bitset can describe. */
#define JF_MAX_NODES 256
#define JF_PAGE_SIZE 16
/* Most sequences one jf_tree_attention call takes (its work schedule is
 * formed on the device from all B prefix lengths). */
#define JF_MAX_BATCH 1024
/* children a node may offer in jf_build_tree */
#define JF_MAX_TOPK 8
/* Size of the counter region at the start of every workspace (see the
 * workspace notes of jf_tree_attention and jf_tree_accept). */
#define JF_WORKSPACE_COUNTER_BYTES 4096
/* Size of the fixed device array jf_tree_verify_noalloc takes its scratch
 * from (32 MiB on every GPU the library is loaded on). */
#define JF_NOALLOC_SCRATCH_BYTES 33554432

/* Human-readable name of a status code (static string, never NULL). */
const char* jf_status_string(jf_status s);

/* Library version, e.g. "0.1.0" (static string). */
const char* jf_version(void);

/*
 * jf_build_ancestor_mask -- the per-node ancestor bitset of a batch of trees
 * (section 2, tree-causal attention mask).
 *
 *   parent    int32  [B, N]     parent of each node (see Trees above)
 *   anc       uint64 [B, N, 4]  out: ancestor-or-self bitset
 *   depth     int32  [B, N]     out, nullable: nodes on the root-to-node path
 *                               (root = 1) = popcount of the row of anc
 *   bad_tree  int32  [B]        out, nullable: 1 if that sequence's parent
 *                               array breaks the tree rules, else 0
 *
 * For a flagged sequence, every parent entry that breaks the rules is read
 * as -1 (a root), so anc/depth stay well defined but do not describe the
 * intended tree. Host errors: JF_ERR_NULL (parent or anc NULL),
 * JF_ERR_SHAPE (B < 0, N < 1 or N > 256). B = 0 is a no-op.
 */
jf_status jf_build_ancestor_mask(const int32_t* parent, int32_t B, int32_t N,
                                 uint64_t* anc, int32_t* depth, int32_t* bad_tree,
                                 hipStream_t stream);

/* Shape of one tree-attention call. */
typedef struct {
    int32_t B;                 /* sequences, 0..JF_MAX_BATCH                        */
    int32_t N;                 /* tree nodes per sequence, 1..256                  */
    int32_t Hq;                /* query heads                                      */
    int32_t Hkv;               /* KV heads; Hq % Hkv == 0; head h reads KV head h / (Hq/Hkv) */
    int32_t D;                 /* head dimension: 64 or 128                        */
    int32_t page_size;         /* tokens per KV page: must be 16                   */
    int32_t num_pages;         /* pages in the pool: page ids are in [0, num_pages) */
    int32_t max_pages_per_seq; /* columns of block_table                           */
    int32_t dtype;             /* JF_BF16 or JF_F32, for q, pages, tree K/V and out */
    float sm_scale;            /* score scale, usually 1/sqrt(D)                   */
} jf_attn_shape;

/*
 * Bytes of workspace jf_tree_attention needs for this shape and prefix bound
 * (0 when the call needs none: fp32, a grid without split prefixes, or an
 * invalid shape); enough for jf_tree_attention_paged_tree's plan of the same
 * shape as well.
 *
 * Workspace contract (both jf_tree_attention and jf_tree_accept): the first
 * JF_WORKSPACE_COUNTER_BYTES bytes are arrival counters. They must be zero
 * before the first call (e.g. allocate with a zeroing allocator) and every
 * call leaves them zero again; the rest is scratch that a call writes before
 * it reads. So one workspace, sized for the largest call, can be reused by
 * calls of any shape and by both entry points without clearing, provided the
 * calls do not run at the same time (calls on one stream never do).
 */
size_t jf_tree_attention_workspace_bytes(const jf_attn_shape* s, int32_t max_prefix_len);

/*
 * jf_tree_attention_plan -- the launch plan jf_tree_attention would use for a
 * bf16 call of this shape (for tuning, tests and capacity planning; nothing is
 * launched). plan: int32 [8], host memory, receives
 *   [0] query rows per workgroup (packed GQA rows: node * G + head in group)
 *   [1] key groups (waves that take alternate key tiles of one row block)
 *   [2] 32-row blocks per wave
 *   [3] splits per row block (prefix page ranges merged in the same launch;
 *       includes the tree's own split when [6] is 1)
 *   [4] prefix pages per split
 *   [5] 1 when the batch schedule is planned on the device from the prefix
 *       lengths (2 to 64 sequences), else 0
 *   [6] 1 when the tree tiles run in a split of their own, else 0
 *   [7] workgroups launched
 * Host errors: those of jf_tree_attention's shape checks, JF_ERR_NULL (plan
 * NULL), JF_ERR_UNSUPPORTED (fp32: one workgroup per 64 rows, no plan).
 */
jf_status jf_tree_attention_plan(const jf_attn_shape* s, int32_t max_prefix_len, int32_t* plan);

/*
 * jf_tree_attention_paged_tree_plan -- the launch plan jf_tree_attention_paged_tree
 * would use for a bf16 call of this shape: the same fields as
 * jf_tree_attention_plan. Ragged budgets take 128-row blocks wherever
 * jf_tree_attention would take 256-row ones (half the padding rows of a
 * partly filled tree). Same host errors as jf_tree_attention_plan.
 */
jf_status jf_tree_attention_paged_tree_plan(const jf_attn_shape* s, int32_t max_prefix_len, int32_t* plan);

/*
 * jf_tree_attention -- tree-causal attention over a paged prefix
 * (section 2 mask; section 3 paged verification).
 *
 *   s               host: shape (above)
 *   max_prefix_len  host: upper bound on prefix_len[b]; sizes the grid.
 *                   0 <= max_prefix_len <= max_pages_per_seq * page_size
 *   q               [B, N, Hq, D]         queries of the tree nodes
 *   k_pages,v_pages [num_pages, Hkv, page_size, D]  paged prefix cache
 *   block_table     int32 [B, max_pages_per_seq]: prefix token t of sequence b
 *                   is slot t % page_size of page block_table[b, t / page_size]
 *   prefix_len      int32 [B]            prefix tokens of each sequence (may be 0)
 *   k_tree,v_tree   [B, N, Hkv, D]       K/V of the tree nodes themselves
 *   anc             uint64 [B, N, 4]     ancestor bitset (jf_build_ancestor_mask)
 *   out             [B, N, Hq, D]        out, same dtype as q
 *   lse             float [B, N, Hq]     out, nullable: natural-log log-sum-exp
 *                                        of the scaled scores of each row
 *   workspace       see jf_tree_attention_workspace_bytes
 *
 * Row (b, i, h) is softmax(sm_scale * q . k) over the L_b prefix keys and the
 * tree keys j with bit j set in anc[b, i], times the matching values, with
 * head h using KV head h / (Hq / Hkv). bf16 inputs use bf16 matrix cores
 * with fp32 accumulation and an fp32 softmax; fp32 inputs are computed in
 * fp32 throughout. Page slots at or beyond L_b and pages not in the table are
 * never read into the result. If prefix_len[b] is outside
 * [0, max_prefix_len] or a page id it needs is outside [0, num_pages), every
 * output row of sequence b (and its lse) is set to NaN.
 *
 * Host errors: JF_ERR_NULL, JF_ERR_SHAPE (including B > JF_MAX_BATCH),
 * JF_ERR_DTYPE, JF_ERR_UNSUPPORTED (D not 64/128, page_size not 16),
 * JF_ERR_ALIGN (q, pages, tree K/V, out or workspace not 16-byte aligned),
 * JF_ERR_WORKSPACE, JF_ERR_LAUNCH.
 */
jf_status jf_tree_attention(const jf_attn_shape* s, int32_t max_prefix_len,
                            const void* q, const void* k_pages, const void* v_pages,
                            const int32_t* block_table, const int32_t* prefix_len,
                            const void* k_tree, const void* v_tree, const uint64_t* anc,
                            void* out, float* lse,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * jf_tree_attention_paged_tree -- jf_tree_attention for ragged tree budgets
 * whose tree K/V are already in the paged cache, right after the prefix (the
 * verification pass over a paged KV cache, technical summary section 3, with
 * per-sequence budgets).
 *
 * As jf_tree_attention, except:
 *   - sequence b has tree_len[b] nodes (int32 [B], 0..N; NULL: N for all):
 *     nodes 0..tree_len[b]-1 of q / anc are its tree, later ones are padding
 *     and their output rows (and lse) are not written;
 *   - the K/V of node j is cached token prefix_len[b] + j, so block_table
 *     must list the pages of prefix_len[b] + tree_len[b] tokens; there are no
 *     k_tree / v_tree arguments;
 *   - max_prefix_len bounds prefix_len (the tree's tokens not included);
 *   - bf16 only (JF_ERR_UNSUPPORTED for fp32).
 * anc for a padding node must not set bits of real nodes other than 0 (e.g.
 * parent 0, as jf_build_ancestor_mask gives it); jf_tree_accept never accepts
 * a padding node whose draft token is -1. A tree_len[b] outside [0, N], or a
 * tree page that is not listed, sets every row of sequence b to NaN. Same
 * workspace (jf_tree_attention_workspace_bytes) and host errors as
 * jf_tree_attention, plus JF_ERR_SHAPE when num_pages or max_pages_per_seq
 * is 0.
 */
jf_status jf_tree_attention_paged_tree(const jf_attn_shape* s, int32_t max_prefix_len,
                                       const void* q, const void* k_pages, const void* v_pages,
                                       const int32_t* block_table, const int32_t* prefix_len,
                                       const int32_t* tree_len, const uint64_t* anc,
                                       void* out, float* lse,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Bytes of workspace jf_tree_accept needs in logits mode (ids mode needs
 * none). Same workspace contract as jf_tree_attention: the two entry points
 * may share one workspace.
 */
size_t jf_tree_accept_workspace_bytes(int32_t B, int32_t N, int32_t vocab);

/*
 * jf_tree_accept -- greedy tree acceptance (lay summary: keep the drafted
 * tokens up to the first disagreement; in a tree, the longest agreeing
 * root-to-node path).
 *
 *   target_logits   [B, N, vocab] of logits_dtype, or NULL   (logits mode)
 *   target_ids      int32 [B, N], or NULL                    (ids mode)
 *                   exactly one of the two must be given
 *   draft_tokens    int32 [B, N]   draft token of each node; column 0 unused
 *   parent          int32 [B, N]
 *   anc             uint64 [B, N, 4] (jf_build_ancestor_mask)
 *   next_tokens     int32 [B, N]   out: target's token after each node =
 *                   first index of the row's largest logit (NaN never wins,
 *                   an all-NaN row gives 0), or a copy of target_ids
 *   accept_len      int32 [B]      out: accepted draft tokens (path nodes - 1)
 *   accepted_nodes  int32 [B, N]   out: root..end of the accepted path, then -1
 *   bonus_token     int32 [B]      out: next_tokens at the end of the path
 *
 * Node u > 0 agrees when draft_tokens[u] == next_tokens[parent[u]]. The
 * accepted path is the longest root-to-node path whose nodes all agree; ties
 * go to the smallest end-node index. Results for a sequence whose parent
 * array is not a valid tree are unspecified (memory-safe).
 *
 * Host errors: JF_ERR_NULL, JF_ERR_SHAPE (B < 0, N outside 1..256,
 * vocab < 1, both or neither of logits/ids, B > JF_MAX_BATCH in logits
 * mode), JF_ERR_DTYPE, JF_ERR_WORKSPACE (logits mode), JF_ERR_LAUNCH.
 */
jf_status jf_tree_accept(int32_t B, int32_t N, int32_t vocab,
                         const void* target_logits, int32_t logits_dtype,
                         const int32_t* target_ids,
                         const int32_t* draft_tokens, const int32_t* parent, const uint64_t* anc,
                         int32_t* next_tokens, int32_t* accept_len, int32_t* accepted_nodes,
                         int32_t* bonus_token,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * jf_tree_verify -- one tree-verification step: jf_tree_attention and
 * jf_tree_accept (logits mode) together (technical summaries, section 3:
 * tree verification over a paged KV cache; lay summary: keep the drafted
 * tokens up to the first disagreement).
 *
 * Arguments as in those two calls: the attention arguments with the
 * attention workspace (size from jf_tree_attention_workspace_bytes), then
 * vocab, target_logits (required) with logits_dtype, draft_tokens, parent,
 * the four acceptance outputs and the acceptance workspace (size from
 * jf_tree_accept_workspace_bytes). The results are exactly those of
 * jf_tree_attention followed by jf_tree_accept.
 *
 *   anc              uint64 [B, N, 4]: with anc_from_parent = 0, the ancestor
 *                    bitsets (input, from jf_build_ancestor_mask); with
 *                    anc_from_parent = 1, an output: the call builds the
 *                    bitsets from parent itself (section 2, tree-causal mask)
 *                    and writes them here, exactly as jf_build_ancestor_mask
 *                    writes them (depth and bad_tree are not produced; the
 *                    tree rules are read the same way, so a broken parent
 *                    entry counts as a root). Then no separate mask launch is
 *                    needed before the call.
 *
 * With bf16 attention, bf16 logits and a plan whose attention workgroups
 * have four waves (few query rows per KV head, as at budget 16), both run in
 * one launch and side by side on the chip; otherwise the two launches follow
 * each other on the stream. The two workspaces must not overlap: each keeps
 * the rules of its own call (counter region zeroed once, left zero).
 *
 * Host errors: those of jf_tree_attention and of jf_tree_accept, plus
 * JF_ERR_NULL (target_logits NULL), JF_ERR_SHAPE (anc_from_parent not 0 or
 * 1) and JF_ERR_WORKSPACE (overlapping workspaces).
 */
jf_status jf_tree_verify(const jf_attn_shape* s, int32_t max_prefix_len, const void* q, const void* k_pages,
                         const void* v_pages, const int32_t* block_table, const int32_t* prefix_len,
                         const void* k_tree, const void* v_tree, uint64_t* anc, int32_t anc_from_parent,
                         void* out, float* lse, void* attn_workspace, size_t attn_workspace_bytes, int32_t vocab,
                         const void* target_logits, int32_t logits_dtype, const int32_t* draft_tokens,
                         const int32_t* parent, int32_t* next_tokens, int32_t* accept_len,
                         int32_t* accepted_nodes, int32_t* bonus_token, void* accept_workspace,
                         size_t accept_workspace_bytes, hipStream_t stream);

/*
 * jf_tree_verify_noalloc -- jf_tree_verify for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc. It takes no workspace arguments; both
 * workspaces are carved from a fixed device array of the library
 * (JF_NOALLOC_SCRATCH_BYTES, 32 MiB per GPU, held from the library's load on
 * that GPU until the process ends). The call itself allocates nothing and
 * frees nothing.
 *
 * Arguments, results and host errors are those of jf_tree_verify without the
 * two workspaces, plus JF_ERR_SCRATCH when the acceptance workspace (rounded
 * up to 256 bytes) and the attention workspace together exceed
 * JF_NOALLOC_SCRATCH_BYTES (e.g. batch 32 with 64-node trees at 32q/4kv); the
 * sizes come from jf_tree_accept_workspace_bytes and
 * jf_tree_attention_workspace_bytes. Every call first clears the counter
 * regions of both workspaces with a small kernel on `stream`, so the
 * contents left by an earlier call never matter; JF_ERR_LAUNCH when the
 * array's address on the stream's device cannot be looked up.
 *
 * All calls on one GPU share that GPU's array: two calls in flight at the
 * same time on one GPU (on different streams, or from different threads)
 * race and give undefined results. Calls on one stream never overlap.
 */
jf_status jf_tree_verify_noalloc(const jf_attn_shape* s, int32_t max_prefix_len, const void* q,
                                 const void* k_pages, const void* v_pages, const int32_t* block_table,
                                 const int32_t* prefix_len, const void* k_tree, const void* v_tree, uint64_t* anc,
                                 int32_t anc_from_parent, void* out, float* lse, int32_t vocab,
                                 const void* target_logits, int32_t logits_dtype, const int32_t* draft_tokens,
                                 const int32_t* parent, int32_t* next_tokens, int32_t* accept_len,
                                 int32_t* accepted_nodes, int32_t* bonus_token, hipStream_t stream);

/*
 * jf_commit_accepted -- append each sequence's accepted path to its paged KV
 * cache, the step after acceptance (lay summary: the target keeps the drafted
 * tokens up to its first disagreement; technical summary, section 3: the
 * prefix the next step attends to lives in a paged KV cache).
 *
 *   s               shape: B, N, Hkv, D, page_size, num_pages,
 *                   max_pages_per_seq and dtype as for jf_tree_attention
 *                   (Hq and sm_scale are not used)
 *   k_tree,v_tree   [B, N, Hkv, D]             K/V of the tree nodes
 *   accept_len      int32 [B]                  from jf_tree_accept
 *   accepted_nodes  int32 [B, N]               from jf_tree_accept
 *   block_table     int32 [B, max_pages_per_seq]
 *   prefix_len      int32 [B]                  prefix tokens before the call
 *   k_pages,v_pages [num_pages, Hkv, 16, D]    in/out
 *   new_prefix_len  int32 [B]                  out: prefix_len[b] + accept_len[b] + 1,
 *                                              or -1 if sequence b was not committed;
 *                                              must not overlap prefix_len
 *
 * Node 0 is the last committed token, whose K/V was computed with the tree,
 * so the path's accept_len[b] + 1 nodes are appended: prefix token
 * prefix_len[b] + i receives the K/V of node accepted_nodes[b, i]. The bonus
 * token has no K/V yet. A sequence is committed only when prefix_len[b] >= 0,
 * 0 <= accept_len[b] < N, its path entries are node ids in [0, N), and every
 * page its new tokens land in is listed (table slot below max_pages_per_seq,
 * page id in [0, num_pages)); otherwise nothing of it is written and
 * new_prefix_len[b] = -1. No other page slot is touched. Asynchronous on
 * `stream`; allocates nothing.
 *
 * Host errors: JF_ERR_NULL, JF_ERR_SHAPE (B outside 0..JF_MAX_BATCH, N outside
 * 1..256, Hkv < 1, negative page counts, new_prefix_len == prefix_len),
 * JF_ERR_DTYPE, JF_ERR_UNSUPPORTED (D not 64/128, page_size not 16),
 * JF_ERR_ALIGN (tree K/V or pages not 16-byte aligned), JF_ERR_LAUNCH.
 */
jf_status jf_commit_accepted(const jf_attn_shape* s, const void* k_tree, const void* v_tree,
                             const int32_t* accept_len, const int32_t* accepted_nodes,
                             const int32_t* block_table, const int32_t* prefix_len,
                             void* k_pages, void* v_pages, int32_t* new_prefix_len,
                             hipStream_t stream);


/*
 * jf_build_tree -- best-first construction of the draft tree (technical
 * summaries, section 2, tree construction: the draft head emits logits for
 * the whole tree in one pass, nodes are ranked by cumulative draft
 * log-probability, and a best-first expansion grows the tree to the budget).
 *
 *   draft_logits    [B, N, vocab] of logits_dtype (JF_BF16 or JF_F32). Row i
 *                   of sequence b is the draft head's output at the i-th node
 *                   to join the tree (node 0: the root, the last committed
 *                   token). Rows at or past budget[b] - 1 are never read.
 *   topk            1..JF_MAX_TOPK children offered per node: its topk most
 *                   likely tokens, larger logit first, ties to the smaller id
 *   max_path_nodes  >= 1; a node whose root-to-node path holds this many nodes
 *                   offers no children
 *   budget          int32 [B] nodes per tree, or NULL (N for every sequence)
 *   parent, token   int32 [B, N] out: the tree in join order. Node 0 has parent
 *                   -1 and token -1. Nodes at or past tree_len[b] are padding:
 *                   parent 0, token -1 (as jf_tree_attention_paged_tree and
 *                   jf_tree_accept expect them)
 *   score           float64 [B, N] out, nullable: each node's cumulative draft
 *                   log-probability (root 0, padding -inf)
 *   tree_len        int32 [B] out: nodes grown, at most budget[b]; fewer when no
 *                   candidate is left; -1 for a budget outside [0, N]
 *
 * A child's log-probability is its logit minus the row's logsumexp, in fp64.
 * NaN logits count as -inf; tokens of -inf logit are never offered; a row
 * whose largest entry is not finite offers nothing. The best candidate joins
 * next: larger score first, then the candidate whose parent joined first, then
 * the better-ranked child. Workspace: jf_build_tree_workspace_bytes, same
 * contract as jf_tree_attention (may be shared with the other entry points,
 * not between calls in flight at once). Asynchronous on `stream`.
 *
 * Host errors: JF_ERR_NULL, JF_ERR_SHAPE (B outside 0..JF_MAX_BATCH, N outside
 * 1..256, vocab < 1, topk outside 1..JF_MAX_TOPK, max_path_nodes < 1),
 * JF_ERR_DTYPE, JF_ERR_WORKSPACE, JF_ERR_ALIGN (workspace not 16-byte
 * aligned), JF_ERR_LAUNCH.
 */
size_t jf_build_tree_workspace_bytes(int32_t B, int32_t N, int32_t vocab, int32_t topk, int32_t logits_dtype);
jf_status jf_build_tree(int32_t B, int32_t N, int32_t vocab, const void* draft_logits, int32_t logits_dtype,
                        int32_t topk, int32_t max_path_nodes, const int32_t* budget,
                        int32_t* parent, int32_t* token, double* score, int32_t* tree_len,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* JF_TREE_H */

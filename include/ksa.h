/*
 * ksa.h -- C ABI of libksa: one decode step of block top-k sparse attention
 * over a GQA KV cache, the vote-union (LessIsMore-style) shared token
 * selection, and dense decode attention for comparison, on AMD MI355X
 * (gfx950).
 *
 * Pages the operations follow (cited by page and section):
 *   Kinetics explainer (news.43u.com.cn), section 五: block top-k attention --
 *     history tokens are cut into fixed-size blocks, each block is summarised
 *     by its mean key, the K' blocks most relevant to the query are chosen
 *     and attention runs over their tokens only; the method works with a
 *     paged KV cache.
 *   Kinetics explainer, section 四: dense attention over every history token.
 *   LessIsMore explainer (techwalker.com), section 二: each query head gets
 *     the same number of votes, the per-token vote totals rank the tokens and
 *     one ranked set serves every head; 75 % of the token budget goes to voted
 *     history and 25 % to the most recent tokens.
 *   LessIsMore explainer, section 五: a selection layer scores every token
 *     for every head, aggregates the heads' picks, appends the most recent
 *     tokens; sparse layers attend only that set, which is shared by all
 *     heads of a GQA group (one KV read per group).
 *
 * Conventions for every entry point
 *   - Buffer pointers are DEVICE pointers (hipMalloc'd or torch CUDA memory)
 *     owned by the caller; the problem and selection structs are HOST memory
 *     read during the call only.
 *   - Every call enqueues its kernels on `stream` (a hipStream_t; NULL is the
 *     default stream) and returns without synchronising.  The library never
 *     allocates, frees or synchronises device memory and keeps no pointer
 *     after a call returns (ksa_sparse_decode_noalloc uses a device array of
 *     the library's own instead of a workspace).  Calls on different streams with disjoint outputs
 *     and workspaces may run concurrently.
 *   - Arguments are validated on the host before any launch.  On any status
 *     other than KSA_OK nothing is launched and no output is written, except
 *     KSA_ERR_HIP, which reports a failed launch (hipGetLastError).
 *   - Index buffers are device data and are not validated: out-of-range or
 *     duplicate indices are undefined behaviour.  NaN/Inf inputs are not
 *     supported.
 *   - Workspaces: a call that needs one takes `workspace` (device memory,
 *     16-byte aligned, contents irrelevant) of at least ksa_workspace_bytes()
 *     bytes; it is scratch for that call only.  Concurrent calls need
 *     distinct workspaces.  (An attention workspace starts with one 8-byte
 *     arrival word per split row, tagged per call, so it needs no clearing.)
 *   - Ranking ties are broken by the lowest index everywhere; every index
 *     list is written in ascending order.
 *   - No C++ exception crosses this interface.
 *
 * Layouts (row-major, last dimension contiguous):
 *   q          [B, Hq, D]            KV dtype
 *   k, v       [B, Hkv, T_cap, D]    KV dtype; token t of sequence b, KV head g
 *   summaries  [B, Hkv, NB_cap, D]   KV dtype, NB_cap = ceil(T_cap / Bs)
 *   out        [B, Hq, D]            fp32
 *   lse        [B, Hq]               fp32, natural log (nullable)
 * Query head h reads KV head h / (Hq / Hkv).  Block j of a sequence covers
 * tokens [j*Bs, min((j+1)*Bs, T)); NB = ceil(T / Bs).
 */
#ifndef KSA_H
#define KSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KSA_OK = 0,
  KSA_ERR_INVALID_ARGUMENT = 1, /* a size, pointer or parameter is out of range */
  KSA_ERR_UNSUPPORTED = 2,      /* valid, but outside what this library handles */
  KSA_ERR_WORKSPACE_TOO_SMALL = 3,
  KSA_ERR_HIP = 4               /* a HIP launch failed */
} ksa_status;

typedef enum { KSA_F32 = 0, KSA_BF16 = 1 } ksa_dtype;

/* One decode step's shape.  T counts the valid cached tokens, the token being
 * decoded included (its K/V are appended before the call).  Every sequence of
 * the batch has the same T (the uniform-workload setting of the Kinetics news
 * page, section on the Qwen3-0.6B throughput gain).
 * Supported by this library: D in {64, 128}; G = Hq/Hkv in {1, 2, 4, 8};
 * dtype fp32 or bf16; B*Hkv*T_cap*D < 2^40; B*Hkv <= 16384. */
typedef struct {
  int32_t batch;        /* B >= 1 */
  int32_t num_q_heads;  /* Hq >= 1, a multiple of Hkv */
  int32_t num_kv_heads; /* Hkv >= 1 */
  int32_t head_dim;     /* D */
  int32_t seq_len;      /* T, 1 <= T <= T_cap */
  int32_t max_seq_len;  /* T_cap: token stride of k and v */
  int32_t block_size;   /* Bs >= 1 (block top-k calls only; ignored elsewhere) */
  ksa_dtype dtype;      /* element type of q, k, v and summaries */
  float sm_scale;       /* softmax scale; <= 0 means 1/sqrt(D) */
} ksa_problem;

typedef enum { KSA_SEL_BLOCKS = 0, KSA_SEL_TOKENS = 1, KSA_SEL_HEAD_TOKENS = 2 } ksa_sel_kind;

/* What ksa_sparse_decode attends.
 *   BLOCKS: idx is [B, Hkv, count] int32 -- for each (sequence, KV head) the
 *           ids of `count` distinct blocks < NB, ascending (the output of
 *           ksa_select_topk); all G query heads of the group attend them.
 *   TOKENS: idx is [B, count] int32 -- for each sequence `count` distinct
 *           token ids < T, ascending (the output of ksa_vote_select); every
 *           query head of the sequence attends them.
 *   HEAD_TOKENS: idx is [B, Hq, count] int32 -- a list per query head
 *           (distinct, ascending, < T; the output of ksa_vote_select_per_head);
 *           the per-head-sets ablation, which reads K/V once per query head
 *           rather than once per group. */
typedef struct {
  ksa_sel_kind kind;
  const int32_t* idx; /* device pointer */
  int32_t count;      /* >= 1 */
} ksa_selection;

/* ---------------------------------------------------------------------
 * ksa_block_summaries -- mean key of each block (Kinetics explainer,
 * section 五: every block is represented by its average).
 * For blocks j in [first_block, first_block + num_blocks) of every
 * (sequence, KV head): summaries[b,g,j,:] = mean over the block's n_j valid
 * tokens of k[b,g,t,:], summed in fp64 in token order, divided by n_j in
 * fp64, rounded once to nearest-even in the KV dtype.  Other blocks are not
 * touched.  A decode step refreshes only the block holding token T-1
 * (first_block = (T-1)/Bs, num_blocks = 1); a rebuild passes (0, NB).
 * Requires 0 <= first_block, num_blocks >= 1, first_block + num_blocks <= NB.
 * Needs no workspace. */
ksa_status ksa_block_summaries(const ksa_problem* problem, const void* k, void* summaries,
                               int32_t first_block, int32_t num_blocks, void* stream);

/* ---------------------------------------------------------------------
 * ksa_select_topk -- choose the K' most relevant blocks per (sequence, KV
 * head) (Kinetics explainer, section 五).
 * Relevance of block j to KV group g: the sum over the group's query heads h
 * of q_h . summaries[b,g,j,:], accumulated in fp32; the k_eff = min(top_k, NB)
 * blocks ranked first by (relevance desc, j asc) are written to
 * block_idx [B, Hkv, k_eff] int32 in ascending order.
 * block_scores (nullable) [B, Hkv, NB] fp32 receives sm_scale * relevance / G,
 * the mean attention logit of the group against the summary.
 * top_k >= 1.  NB must not exceed 15360.  workspace: ksa_workspace_bytes(
 * problem, KSA_OP_SELECT_TOPK, top_k) bytes (B*Hkv*NB*4: one key per block). */
ksa_status ksa_select_topk(const ksa_problem* problem, const void* q, const void* summaries,
                           int32_t top_k, int32_t* block_idx, float* block_scores,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------
 * ksa_sparse_decode -- softmax attention of every query head over the
 * selected tokens only (Kinetics explainer, section 五, for BLOCKS; the
 * LessIsMore explainer, section 五, for TOKENS): for head h of group g,
 * out[b,h,:] = sum_t p_t v[b,g,t,:], p = softmax_t(sm_scale * q_h . k[b,g,t,:])
 * over the selected tokens t < T, accumulated in fp32; lse[b,h] = log of the
 * softmax denominator plus the max logit (natural log).  Tokens of a
 * selected block at or past T are skipped.
 * workspace: ksa_workspace_bytes(problem, KSA_OP_SPARSE_BLOCKS or
 * KSA_OP_SPARSE_TOKENS, sel->count) bytes. */
ksa_status ksa_sparse_decode(const ksa_problem* problem, const void* q, const void* k,
                             const void* v, const ksa_selection* sel, float* out, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the device array behind ksa_sparse_decode_noalloc, one per GPU. */
#define KSA_NOALLOC_SCRATCH_BYTES (4u << 20)

/* ksa_sparse_decode_noalloc -- ksa_sparse_decode for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * layouts and results (bit for bit) as ksa_sparse_decode, without the
 * workspace: the call's scratch (the partial states and arrival words of
 * rows split over several workgroups) lives in a library-owned device array
 * of KSA_NOALLOC_SCRATCH_BYTES on each GPU, created with the library and held
 * until the process ends; its address is looked up once per device on the
 * first call.  The call allocates nothing and needs nothing cleared (arrival
 * words carry a per-call tag).  Every call on a GPU shares that GPU's array:
 * calls that may overlap on one GPU (other streams, or graph replays running
 * concurrently) race and give undefined results; calls ordered on one
 * stream are safe.  `stream` must belong to the current device, else
 * KSA_ERR_INVALID_ARGUMENT.  A call needs scratch only when its rows are
 * split: when there are fewer than 256 rows (at most ~2.2 MB then, for
 * lists of up to 2048 entries), or when a row's list has more than 2048
 * entries (staged 2048 at a time).  A call whose scratch would exceed the
 * array (ksa_workspace_bytes(problem, KSA_OP_SPARSE_BLOCKS, _TOKENS or
 * _HEAD_TOKENS, sel->count) > KSA_NOALLOC_SCRATCH_BYTES) returns
 * KSA_ERR_UNSUPPORTED before touching the device. */
ksa_status ksa_sparse_decode_noalloc(const ksa_problem* problem, const void* q, const void* k,
                                     const void* v, const ksa_selection* sel, float* out,
                                     float* lse, void* stream);

/* ---------------------------------------------------------------------
 * ksa_vote_select -- the shared token set of the vote-union variant
 * (LessIsMore explainer, sections 二 and 五), per sequence b, with
 * N = token_budget and W = recent_window (the pages use W = N/4):
 *   if T <= N: token_idx[b] = 0..T-1 and no vote is taken;
 *   else, with history C = [0, T-W) and Kv = N - W:
 *     every query head h (all Hq of them) picks the first Kv tokens of C by
 *       (q_h . k[b,h/G,t,:] desc, t asc), scores accumulated in fp32;
 *     votes[b,t] = number of heads that picked t (0 for t >= T-W);
 *     the first Kv tokens of C by (votes desc, t asc), ascending, are
 *       followed by T-W, ..., T-1.
 * token_idx: [B, min(N, T)] int32.  votes (nullable): [B, T] uint8 (needs
 * Hq <= 255); all zero when T <= N.
 * Requires 0 <= W <= N, N >= 1.  T - W must not exceed 2^21.
 * workspace: ksa_workspace_bytes(problem, KSA_OP_VOTE_SELECT, token_budget). */
ksa_status ksa_vote_select(const ksa_problem* problem, const void* q, const void* k,
                           int32_t token_budget, int32_t recent_window, int32_t* token_idx,
                           uint8_t* votes, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------
 * ksa_dense_decode -- exact softmax attention of every query head over all T
 * cached tokens (Kinetics explainer, section 四); the comparison baseline.
 * Outputs as ksa_sparse_decode.
 * workspace: ksa_workspace_bytes(problem, KSA_OP_DENSE, 0) bytes. */
ksa_status ksa_dense_decode(const ksa_problem* problem, const void* q, const void* k,
                            const void* v, float* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------
 * ksa_block_topk_decode -- one whole decode step of block top-k attention
 * (Kinetics explainer, section 五) in a single launch, one workgroup per
 * (sequence, KV head):
 *   1. if refresh_last_block != 0: the summary of block (T-1)/Bs is
 *      recomputed and written to summaries, exactly as
 *      ksa_block_summaries(first_block = (T-1)/Bs, num_blocks = 1) does; the
 *      other blocks' summaries are read as given;
 *   2. the blocks are ranked as in ksa_select_topk(top_k) (same fp32
 *      relevance, same ties); the k_eff = min(top_k, NB) ids are written,
 *      ascending, to block_idx [B, Hkv, k_eff] int32 when it is not NULL;
 *   3. out [B, Hq, D] fp32 and lse [B, Hq] fp32 (nullable) are the attention
 *      of ksa_sparse_decode over those blocks.
 * summaries and block_idx are bitwise those of the three separate calls; out
 * and lse differ from ksa_sparse_decode's only in the fp32 order of the final
 * merge (and not at all when both run one workgroup of 8 waves per row, e.g.
 * B*Hkv = 512, Hq/Hkv = 2 on MI355X).  Results are bitwise repeatable.  One
 * workgroup serves each (sequence, KV head) row, so the call is meant for
 * batches with at least a few hundred such rows.
 * Limits (else KSA_ERR_UNSUPPORTED): NB <= 4096, k_eff <= 2048,
 * k_eff * Bs < 2^30, and Bs <= 64 when refresh_last_block is set.
 * Needs no workspace. */
ksa_status ksa_block_topk_decode(const ksa_problem* problem, const void* q, const void* k,
                                 const void* v, void* summaries, int32_t top_k,
                                 int32_t refresh_last_block, int32_t* block_idx, float* out,
                                 float* lse, void* stream);

/* ksa_block_topk_decode_varlen -- ksa_block_topk_decode on the contiguous
 * cache with one length per sequence (the batches of unequal lengths a
 * paged cache also serves, Kinetics news page on the uniform workload and
 * Kinetics explainer, section 五): sequence b holds T_b = seq_lens[b] tokens
 * (device [B] int32; not validated, clamped into [1, T] with T the problem's
 * seq_len, which must be the longest length), so NB_b = ceil(T_b / Bs) and
 * k_eff_b = min(top_k, NB_b).  For every (sequence, KV head) the refresh
 * rewrites block (T_b - 1) / Bs, the ranking covers blocks [0, NB_b) and the
 * attention covers the tokens below T_b of the chosen blocks.  block_idx
 * [B, Hkv, min(top_k, NB)] (NB from T) holds each row's k_eff_b ascending
 * ids, then -1.  With every T_b = T it is ksa_block_topk_decode bit for bit.
 * seq_lens NULL or misaligned: KSA_ERR_INVALID_ARGUMENT.  Same layouts,
 * limits and (no) workspace as ksa_block_topk_decode. */
ksa_status ksa_block_topk_decode_varlen(const ksa_problem* problem, const int32_t* seq_lens,
                                        const void* q, const void* k, const void* v,
                                        void* summaries, int32_t top_k,
                                        int32_t refresh_last_block, int32_t* block_idx,
                                        float* out, float* lse, void* stream);

/* ---------------------------------------------------------------------
 * Paged KV cache with one length per sequence (Kinetics explainer, section
 * 五: block top-k attention works with a paged cache, the attention blocks
 * being its pages).
 * K and V live in pools of pages; a page holds block_size consecutive tokens
 * of one sequence for every KV head:
 *   k_pool, v_pool  [num_pages, Hkv, Bs, D]   KV dtype
 * Logical block j of sequence b (tokens [j*Bs, (j+1)*Bs)) is page
 * block_table[b * max_blocks + j]; sequence b holds T_b = seq_lens[b]
 * tokens, NB_b = ceil(T_b / Bs) blocks.  Summaries stay per sequence:
 *   summaries  [B, Hkv, max_blocks, D]
 * In the problem struct, seq_len is the longest T_b (it sizes launches and
 * workspaces) and max_seq_len must equal max_blocks * Bs.  The table and the
 * lengths are device data and are not validated: a page id >= num_pages for
 * a block < NB_b is undefined behaviour; every kernel clamps a length into
 * [1, T] with T the problem's seq_len, since launches, workspaces and
 * outputs (votes [B, T], token_idx, block_scores) are sized from T.
 * num_pages * Hkv * Bs must stay below 2^31. */
typedef struct {
  const int32_t* block_table; /* device [B, max_blocks] int32 */
  const int32_t* seq_lens;    /* device [B] int32 */
  int32_t max_blocks;         /* >= 1: row stride of block_table */
  int32_t num_pages;          /* >= 1: pages in each pool */
} ksa_paged_kv;

/* ksa_paged_block_summaries -- ksa_block_summaries on a paged cache: for
 * every (sequence, KV head), the blocks j in [first_block, first_block +
 * num_blocks) with j < NB_b get their mean key (same arithmetic, n_j counted
 * against T_b).  first_block = -1 with num_blocks = 1 selects each
 * sequence's own newest block (T_b - 1) / Bs (the decode-step refresh).
 * Requires num_blocks >= 1 and first_block + num_blocks <= max_blocks (or the
 * -1 form).  Needs no workspace. */
ksa_status ksa_paged_block_summaries(const ksa_problem* problem, const ksa_paged_kv* paged,
                                     const void* k_pool, void* summaries, int32_t first_block,
                                     int32_t num_blocks, void* stream);

/* ksa_paged_block_topk_decode -- ksa_block_topk_decode on a paged cache with
 * per-sequence lengths: each row uses its own T_b, NB_b and
 * k_eff_b = min(top_k, NB_b).  block_idx (nullable) is [B, Hkv, top_k]
 * int32: the k_eff_b ids ascending, then -1.  When every T_b equals T,
 * summaries, ids, out and lse are bitwise those of ksa_block_topk_decode on
 * the same tokens stored contiguously.  Same limits as
 * ksa_block_topk_decode, with NB = max_blocks.  Needs no workspace. */
ksa_status ksa_paged_block_topk_decode(const ksa_problem* problem, const ksa_paged_kv* paged,
                                       const void* q, const void* k_pool, const void* v_pool,
                                       void* summaries, int32_t top_k, int32_t refresh_last_block,
                                       int32_t* block_idx, float* out, float* lse, void* stream);

/* ksa_paged_dense_decode -- ksa_dense_decode on a paged cache: every query
 * head of sequence b attends its T_b tokens.
 * workspace: ksa_workspace_bytes(problem, KSA_OP_PAGED_DENSE, 0) bytes. */
ksa_status ksa_paged_dense_decode(const ksa_problem* problem, const ksa_paged_kv* paged,
                                  const void* q, const void* k_pool, const void* v_pool, float* out,
                                  float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* ksa_paged_vote_select -- ksa_vote_select on a paged cache with
 * per-sequence lengths: sequence b votes over its own history [0, T_b - W)
 * when T_b > N, else takes all of [0, T_b).  token_idx is [B, min(N, T)]
 * int32 (T the longest sequence), each row ascending and padded with -1;
 * votes (nullable) is [B, T] uint8, zero past each sequence's history.
 * Same limits as ksa_vote_select, with T the longest sequence.
 * workspace: ksa_workspace_bytes(problem, KSA_OP_VOTE_SELECT, token_budget). */
ksa_status ksa_paged_vote_select(const ksa_problem* problem, const ksa_paged_kv* paged,
                                 const void* q, const void* k_pool, int32_t token_budget,
                                 int32_t recent_window, int32_t* token_idx, uint8_t* votes,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* ksa_paged_sparse_decode -- ksa_sparse_decode on a paged cache with
 * per-sequence lengths, for BLOCKS (logical block ids [B, Hkv, count], e.g.
 * ksa_paged_block_topk_decode's), TOKENS (token ids [B, count], e.g.
 * ksa_paged_vote_select's) and HEAD_TOKENS (token ids [B, Hq, count], e.g.
 * ksa_paged_vote_select_per_head's); negative entries are padding and are
 * skipped, as are tokens at or past T_b.  workspace: ksa_workspace_bytes(
 * problem, KSA_OP_SPARSE_BLOCKS, _TOKENS or _HEAD_TOKENS, sel->count). */
ksa_status ksa_paged_sparse_decode(const ksa_problem* problem, const ksa_paged_kv* paged,
                                   const void* q, const void* k_pool, const void* v_pool,
                                   const ksa_selection* sel, float* out, float* lse,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------
 * Selection variants (the ablations the pages report) and a quality signal.
 *
 * ksa_select_topk_ex -- ksa_select_topk with options:
 *   aggregate KSA_AGG_SUM ranks a block by the group's summed relevance (the
 *     method, as ksa_select_topk); KSA_AGG_MAX by its largest single-head
 *     relevance max_h q_h . summaries[b,g,j,:] (block_scores then holds
 *     sm_scale * that maximum);
 *   force_last_block != 0 always keeps block (T-1)/Bs (the local block,
 *     Kinetics explainer, section 五, local attention) and ranks the others
 *     for the remaining k_eff - 1 places.
 * Same outputs, limits and workspace as ksa_select_topk. */
typedef enum { KSA_AGG_SUM = 0, KSA_AGG_MAX = 1 } ksa_group_agg;
typedef struct {
  int32_t top_k;             /* >= 1 */
  ksa_group_agg aggregate;
  int32_t force_last_block;
} ksa_select_options;
ksa_status ksa_select_topk_ex(const ksa_problem* problem, const void* q, const void* summaries,
                              const ksa_select_options* options, int32_t* block_idx,
                              float* block_scores, void* workspace, size_t workspace_bytes,
                              void* stream);

/* ksa_paged_select_topk_ex -- ksa_select_topk_ex for a paged cache with
 * per-sequence lengths (the summaries of ksa_paged_block_summaries,
 * [B, Hkv, max_blocks, D]): row (b, g) ranks its own NB_b blocks and keeps
 * k_eff_b = min(top_k, NB_b); block_idx is [B, Hkv, top_k] int32, the ids
 * ascending, then -1.  force_last_block keeps each row's own newest block
 * (T_b - 1)/Bs.  block_scores (nullable) is [B, Hkv, NB] (NB from the
 * problem's T, the longest sequence); entries past a row's NB_b are not
 * written.  The ids feed ksa_paged_sparse_decode (KSA_SEL_BLOCKS).  Same
 * limits and workspace as ksa_select_topk (NB from the problem's T). */
ksa_status ksa_paged_select_topk_ex(const ksa_problem* problem, const ksa_paged_kv* paged,
                                    const void* q, const void* summaries,
                                    const ksa_select_options* options, int32_t* block_idx,
                                    float* block_scores, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* ksa_vote_select_heads -- ksa_vote_select where only the listed query heads
 * vote (voting_heads: host array of num_voting distinct heads < Hq, read
 * during the call).  One head is the random-head ablation of the LessIsMore
 * explainer, section 五 (one head's picks serve every head); all Hq heads is
 * ksa_vote_select.  votes then counts the listed heads' picks only.
 * Same outputs, limits and workspace as ksa_vote_select. */
ksa_status ksa_vote_select_heads(const ksa_problem* problem, const void* q, const void* k,
                                 int32_t token_budget, int32_t recent_window,
                                 const int32_t* voting_heads, int32_t num_voting,
                                 int32_t* token_idx, uint8_t* votes, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* ksa_paged_vote_select_heads -- ksa_vote_select_heads on a paged cache with
 * per-sequence lengths (the outputs of ksa_paged_vote_select, from the listed
 * heads' picks only).  Same limits and workspace as ksa_paged_vote_select. */
/* ksa_paged_vote_select_per_head -- ksa_vote_select_per_head on a paged cache
 * with per-sequence lengths: token_idx [B, Hq, min(N, T)] (T the longest
 * sequence), every row ascending; a sequence no longer than N gives all its
 * T_b tokens, then -1.  Same limits and workspace as ksa_paged_vote_select. */
ksa_status ksa_paged_vote_select_per_head(const ksa_problem* problem, const ksa_paged_kv* paged,
                                          const void* q, const void* k_pool,
                                          int32_t token_budget, int32_t recent_window,
                                          int32_t* token_idx, void* workspace,
                                          size_t workspace_bytes, void* stream);

ksa_status ksa_paged_vote_select_heads(const ksa_problem* problem, const ksa_paged_kv* paged,
                                       const void* q, const void* k_pool, int32_t token_budget,
                                       int32_t recent_window, const int32_t* voting_heads,
                                       int32_t num_voting, int32_t* token_idx, uint8_t* votes,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* ksa_vote_select_per_head -- the per-head-sets ablation (LessIsMore
 * explainer, section 五: each head keeps its own set): every query head h
 * keeps its own first Kv = N - W history tokens by (q_h . k desc, t asc),
 * ascending, followed by the W most recent tokens; token_idx is
 * [B, Hq, min(N, T)] int32 (all tokens when T <= N), for ksa_sparse_decode
 * with KSA_SEL_HEAD_TOKENS.  Same limits and workspace as ksa_vote_select. */
ksa_status ksa_vote_select_per_head(const ksa_problem* problem, const void* q, const void* k,
                                    int32_t token_budget, int32_t recent_window,
                                    int32_t* token_idx, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* ksa_attention_recall -- the share of each query head's dense softmax mass
 * that a selection covers (the attention recall the LessIsMore explainer,
 * sections 四 and 五, judges selections by): with lse_selected from
 * ksa_sparse_decode (or a decode step) and lse_dense from ksa_dense_decode on
 * the same queries and scale, recall[i] = exp(lse_selected[i] - lse_dense[i])
 * = sum over the selected tokens of the dense softmax weights.  count >= 1
 * fp32 entries each ([B, Hq] arrays).  Needs no workspace. */
ksa_status ksa_attention_recall(const float* lse_selected, const float* lse_dense, float* recall,
                                int32_t count, void* stream);

/* ---------------------------------------------------------------------
 * ksa_vote_layer_decode -- a token-selection layer of the LessIsMore
 * schedule (LessIsMore explainer, section 五: full-attention layers first,
 * then selection layers that compute the full score matrix, let every head
 * pick, pool and rank the picks and append the most recent tokens, and
 * sparse layers that attend only that set).  In one call:
 *   out, lse   = ksa_dense_decode (the layer attends every token);
 *   token_idx, votes = ksa_vote_select(token_budget, recent_window) on the
 *                same queries, the set the following sparse layers attend.
 * For bf16, D = 128 and G in {4, 8} the vote's per-head scores are the
 * dense attention's own logits (MFMA), so K is read once for both; other
 * shapes run the dense attention and the vote's scoring as two passes.
 * token_idx and votes are bitwise those of ksa_vote_select.
 * workspace: ksa_workspace_bytes(problem, KSA_OP_VOTE_LAYER, token_budget). */
ksa_status ksa_vote_layer_decode(const ksa_problem* problem, const void* q, const void* k,
                                 const void* v, int32_t token_budget, int32_t recent_window,
                                 float* out, float* lse, int32_t* token_idx, uint8_t* votes,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* ksa_paged_vote_layer_decode -- ksa_vote_layer_decode on a paged cache with
 * per-sequence lengths (the selection layer of the schedule above over the
 * block-table layout the Kinetics explainer's section 五 says block sparsity
 * fits):
 *   out, lse   = ksa_paged_dense_decode (sequence b attends its T_b tokens);
 *   token_idx, votes = ksa_paged_vote_select(token_budget, recent_window).
 * For bf16, D = 128 and G in {4, 8} the paged dense walk writes the vote's
 * keys from its own logits (K read once); other shapes run the two passes.
 * token_idx and votes are bitwise those of ksa_paged_vote_select, out and
 * lse those of ksa_paged_dense_decode.  Same limits as those two calls.
 * workspace: ksa_workspace_bytes(problem, KSA_OP_PAGED_VOTE_LAYER,
 * token_budget). */
ksa_status ksa_paged_vote_layer_decode(const ksa_problem* problem, const ksa_paged_kv* paged,
                                       const void* q, const void* k_pool, const void* v_pool,
                                       int32_t token_budget, int32_t recent_window, float* out,
                                       float* lse, int32_t* token_idx, uint8_t* votes,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* Operations for ksa_workspace_bytes. */
enum {
  KSA_OP_SELECT_TOPK = 0,    /* param: top_k */
  KSA_OP_SPARSE_BLOCKS = 1,  /* param: selection count (blocks per row) */
  KSA_OP_SPARSE_TOKENS = 2,  /* param: selection count (tokens per sequence) */
  KSA_OP_VOTE_SELECT = 3,    /* param: token_budget */
  KSA_OP_DENSE = 4,          /* param: unused */
  KSA_OP_PAGED_DENSE = 5,    /* param: unused */
  KSA_OP_VOTE_LAYER = 6,     /* param: token_budget */
  KSA_OP_SPARSE_HEAD_TOKENS = 7, /* param: selection count (tokens per query head) */
  KSA_OP_PAGED_VOTE_LAYER = 8    /* param: token_budget */
};

/* Workspace bytes a call needs for this problem; a pure host function of its
 * arguments (no device query).  Returns 0 when the call needs none, and
 * SIZE_MAX when the arguments are invalid. */
size_t ksa_workspace_bytes(const ksa_problem* problem, int32_t op, int32_t param);

/* Static, NUL-terminated description of a status code. */
const char* ksa_status_string(ksa_status status);

/* Library version, "major.minor.patch". */
const char* ksa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KSA_H */

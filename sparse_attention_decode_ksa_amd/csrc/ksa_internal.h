// ksa_internal.h -- shapes, launch plans and launcher declarations shared by
// the host side of libksa (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ksa.h"

namespace ksa {

// Problem shape with derived sizes.
struct Dims {
  int B, Hq, Hkv, G, D, T, Tcap, Bs, NB, NBcap;
  int dtype;    // KSA_F32 or KSA_BF16
  float scale;  // softmax scale
};

inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

constexpr int kMaxRows = 16384;  // B * Hkv: the top-k grid's row count stays far below 2^31

// Elements one lane moves in one 16-byte load.
inline int elems_per_lane(int dtype) { return dtype == KSA_F32 ? 4 : 8; }
// Lanes that together hold one token row of D elements.
inline int lanes_per_token(const Dims& d) { return d.D / elems_per_lane(d.dtype); }
// Token rows one wave covers with one 16-byte load per lane.
inline int slots_per_wave(const Dims& d) { return 64 / lanes_per_token(d); }

// 16-byte loads per lane per chunk for K (and again for V) in the attention
// kernels; a chunk is slots_per_wave * kLoadsPerChunk tokens.
#ifndef KSA_ATTN_LOADS
#define KSA_ATTN_LOADS 4
#endif
constexpr int kLoadsPerChunk = KSA_ATTN_LOADS;
// index entries a workgroup stages in LDS
constexpr int kIdxStage = 2048;
inline int chunk_tokens(const Dims& d) { return slots_per_wave(d) * kLoadsPerChunk; }

// Attention launch: `splits` workgroups of `nw` waves per (sequence, KV
// head) row; each workgroup covers `cps` chunks of the row's token list.
struct AttnPlan {
  int nw, splits, cps, chunk;
};
// kind: 0 = selected blocks, 1 = shared token list, 2 = dense range
AttnPlan plan_attention(const Dims& d, int kind, int64_t tokens_per_row);
size_t attention_workspace_bytes(const Dims& d, const AttnPlan& p);
// Bytes of the per-row arrival words at the start of a split plan's
// workspace (8 bytes a row, rounded up to 256).
inline size_t arrival_bytes(size_t rows) { return (rows * 8 + 255) & ~(size_t)255; }

// A paged cache (device table and lengths, see ksa_paged_kv).
struct PagedKv {
  const int32_t* table;
  const int32_t* seq_lens;
  int max_blocks;
  int num_pages;
};

// Attention over a row-wise token list.  kind: 0 = selected blocks,
// 1 = shared token list, 2 = dense range [0, T), 3 = dense over a paged
// cache (`paged` given; d.T is the longest sequence).
// Order keys of the raw logits the dense MFMA body writes for the vote.
struct VoteKeys {
  uint32_t* keys;  // [B, Hq, kstride]
  int kstride;
  int hist;        // tokens t < hist get keys
  // paged dense (kind 3): each sequence's own history instead, T_b - window
  // when T_b > budget, else none
  int budget = 0, window = 0;
};
// kind 4 (a token list per query head) takes d with Hkv = Hq and G = 1 and
// kv_div = the real G: row (b, h) reads KV head h / kv_div.
hipError_t launch_attention(const Dims& d, int kind, const void* q, const void* k, const void* v,
                            const int32_t* idx, int count, float* out, float* lse,
                            void* workspace, const AttnPlan& plan, hipStream_t stream,
                            const PagedKv* paged = nullptr, const VoteKeys* vote_keys = nullptr,
                            int kv_div = 1);

// recall[i] = exp(lse_sel[i] - lse_dense[i]) for i < n.
hipError_t launch_attention_recall(const float* lse_sel, const float* lse_dense, float* recall,
                                   int n, hipStream_t stream);

hipError_t launch_block_summaries(const Dims& d, const void* k, void* summaries, int first_block,
                                  int num_blocks, hipStream_t stream);
// Paged: blocks [first, first + num) below each sequence's NB_b, or each
// sequence's newest block when first_block < 0.
hipError_t launch_paged_block_summaries(const Dims& d, const PagedKv& p, const void* k_pool,
                                        void* summaries, int first_block, int num_blocks,
                                        hipStream_t stream);

constexpr int kSelectMaxBlocks = 15360;  // a row's keys fit the registers of one top-k workgroup
size_t select_workspace_bytes(const Dims& d);
// Selection variants (the ablations): rank a block by its largest head
// instead of the group's sum; always keep one block (its key made maximal).
struct SelectVariant {
  int agg_max = 0;
  int forced_block = -1;      // with seq_lens: >= 0 forces each row's own newest block
  const int32_t* seq_lens = nullptr;  // per-sequence lengths (a paged cache), or uniform d.T
  int id_stride = 0;          // with seq_lens: ids per row in block_idx (-1 past k_eff_b)
};
hipError_t launch_select_topk(const Dims& d, const void* q, const void* summaries, int keff,
                              int32_t* block_idx, float* block_scores, void* workspace,
                              hipStream_t stream, const SelectVariant& var = SelectVariant());

// Whole decode step in one launch (refresh + select + attend per row).
constexpr int kStepMaxBlocks = 4096;  // blocks per row whose keys the step keeps in LDS
constexpr int kStepMaxBs = 64;        // largest block size the step refreshes
hipError_t launch_block_topk_decode(const Dims& d, const void* q, const void* k, const void* v,
                                    void* summaries, int keff, int refresh, int32_t* block_idx,
                                    float* out, float* lse, hipStream_t stream,
                                    const PagedKv* paged = nullptr,
                                    const int32_t* seq_lens = nullptr);

// Vote-union selection.
struct VotePlan {
  int hist;        // C = T - W history tokens (candidates)
  int words;       // 32-token words per head bitmask
  int kstride;     // uint32 keys per head row (hist rounded up to a multiple of 4)
  int kv;          // N - W picks per head
  size_t keys_off, bits_off, votes_off, vhist_off, total;
};
VotePlan plan_vote(const Dims& d, int N, int W);
// The query heads that vote (bit h of w[h / 32]); every head by default.
struct HeadMask {
  uint32_t w[8] = {~0u, ~0u, ~0u, ~0u, ~0u, ~0u, ~0u, ~0u};
};
hipError_t launch_vote_select(const Dims& d, const void* q, const void* k, int N, int W,
                              int32_t* token_idx, uint8_t* votes, void* workspace,
                              const VotePlan& plan, hipStream_t stream,
                              const HeadMask& voting = HeadMask());
// The vote after the keys are in the workspace (per-head picks, tally, set).
hipError_t launch_vote_finish(const Dims& d, int N, int W, int32_t* token_idx, uint8_t* votes,
                              void* workspace, const VotePlan& plan, hipStream_t stream,
                              const HeadMask& voting = HeadMask());
// T <= N: the whole context, no vote.
hipError_t launch_vote_all(const Dims& d, int32_t* token_idx, uint8_t* votes, hipStream_t stream);
// The vote on a paged cache with per-sequence lengths (d.T the longest):
// token_idx [B, min(N, T)], -1 past a sequence shorter than N.
hipError_t launch_paged_vote_select(const Dims& d, const PagedKv& p, const void* q,
                                    const void* k_pool, int N, int W, int32_t* token_idx,
                                    uint8_t* votes, void* workspace, const VotePlan& plan,
                                    hipStream_t stream, const HeadMask& voting = HeadMask());
// The same vote from keys already in the workspace (written by the paged
// dense walk with VoteKeys{budget N, window W}).
hipError_t launch_paged_vote_finish(const Dims& d, const PagedKv& p, int N, int W,
                                    int32_t* token_idx, uint8_t* votes, void* workspace,
                                    const VotePlan& plan, hipStream_t stream);
// Per-head sets: every head's own picks plus the window, token_idx [B, Hq, min(N, T)].
// paged: K is a page pool and every sequence has its own length (d.T the
// longest); token_idx is [B, Hq, min(N, T)], rows of short sequences -1 padded.
hipError_t launch_vote_per_head(const Dims& d, const void* q, const void* k, int N, int W,
                                int32_t* token_idx, void* workspace, const VotePlan& plan,
                                hipStream_t stream, const PagedKv* paged = nullptr);
// Whether dense attention of this shape runs the MFMA body (and can emit the
// vote's keys while it attends).
inline bool dense_emits_vote_keys(const Dims& d) {
  return d.dtype == KSA_BF16 && d.D == 128 && (d.G == 4 || d.G == 8);
}

}  // namespace ksa

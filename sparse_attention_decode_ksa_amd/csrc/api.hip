// api.hip -- the extern "C" entry points of libksa (declared in
// include/ksa.h): host-side argument validation, workspace sizing and launch
// selection.  Validation is pure host code that runs before any HIP call, so
// an invalid call launches nothing and writes nothing.
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <new>

#include "ksa_internal.h"

namespace ksa {
namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 40;

bool supported_shape(const ksa_problem& p) {
  if (p.head_dim != 64 && p.head_dim != 128) return false;
  const int G = p.num_q_heads / p.num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return false;
  if ((int64_t)p.batch * p.num_kv_heads * (int64_t)p.max_seq_len * p.head_dim >= kMaxElems)
    return false;
  if ((int64_t)p.batch * p.num_kv_heads > kMaxRows) return false;
  return true;
}

// Checks the fields every call uses; INVALID for impossible shapes,
// UNSUPPORTED for valid ones outside this library.
ksa_status check_problem(const ksa_problem* p, bool needs_block_size) {
  if (!p) return KSA_ERR_INVALID_ARGUMENT;
  if (p->batch < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1 || p->head_dim < 1)
    return KSA_ERR_INVALID_ARGUMENT;
  if (p->num_q_heads % p->num_kv_heads != 0) return KSA_ERR_INVALID_ARGUMENT;
  if (p->seq_len < 1 || p->max_seq_len < p->seq_len) return KSA_ERR_INVALID_ARGUMENT;
  if (needs_block_size && p->block_size < 1) return KSA_ERR_INVALID_ARGUMENT;
  if (p->dtype != KSA_F32 && p->dtype != KSA_BF16) return KSA_ERR_INVALID_ARGUMENT;
  if (!(p->sm_scale == p->sm_scale) || isinf(p->sm_scale)) return KSA_ERR_INVALID_ARGUMENT;
  if (!supported_shape(*p)) return KSA_ERR_UNSUPPORTED;
  return KSA_OK;
}

Dims make_dims(const ksa_problem& p) {
  Dims d;
  d.B = p.batch;
  d.Hq = p.num_q_heads;
  d.Hkv = p.num_kv_heads;
  d.G = p.num_q_heads / p.num_kv_heads;
  d.D = p.head_dim;
  d.T = p.seq_len;
  d.Tcap = p.max_seq_len;
  d.Bs = p.block_size >= 1 ? p.block_size : 1;
  d.NB = ceil_div(d.T, d.Bs);
  d.NBcap = ceil_div(d.Tcap, d.Bs);
  d.dtype = p.dtype;
  d.scale = p.sm_scale > 0.f ? p.sm_scale : 1.0f / sqrtf((float)p.head_dim);
  return d;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }
bool aligned4(const void* ptr) { return ((uintptr_t)ptr & 3u) == 0; }

ksa_status from_hip(hipError_t e) { return e == hipSuccess ? KSA_OK : KSA_ERR_HIP; }

size_t workspace_for(const ksa_problem& p, int32_t op, int32_t param) {
  const Dims d = make_dims(p);
  switch (op) {
    case KSA_OP_SELECT_TOPK:
      return select_workspace_bytes(d);
    case KSA_OP_SPARSE_BLOCKS:
      return attention_workspace_bytes(d, plan_attention(d, 0, (int64_t)param * d.Bs));
    case KSA_OP_SPARSE_TOKENS:
      return attention_workspace_bytes(d, plan_attention(d, 1, param));
    case KSA_OP_VOTE_SELECT:
      // bound over every recent_window: W = 0 has the most candidates
      return plan_vote(d, param, 0).total;
    case KSA_OP_DENSE:
      return attention_workspace_bytes(d, plan_attention(d, 2, d.T));
    case KSA_OP_PAGED_DENSE:
      return attention_workspace_bytes(d, plan_attention(d, 3, (int64_t)d.NB * d.Bs));
    case KSA_OP_SPARSE_HEAD_TOKENS: {
      Dims dh = d;
      dh.Hkv = d.Hq;
      dh.G = 1;
      return attention_workspace_bytes(dh, plan_attention(dh, 4, param));
    }
    case KSA_OP_VOTE_LAYER:
      // the vote's workspace (bound over every window), then the dense partials
      return ((plan_vote(d, param, 0).total + 255) & ~(size_t)255) +
             attention_workspace_bytes(d, plan_attention(d, 2, d.T));
    case KSA_OP_PAGED_VOTE_LAYER:
      return ((plan_vote(d, param, 0).total + 255) & ~(size_t)255) +
             attention_workspace_bytes(d, plan_attention(d, 3, (int64_t)d.NB * d.Bs));
    default:
      return SIZE_MAX;
  }
}

// The paged-cache description: pointers, strides and the pool's row count
// (page ids are int32 row offsets: num_pages * Hkv * Bs < 2^31).
ksa_status check_paged(const ksa_problem& p, const ksa_paged_kv* pg, PagedKv* out) {
  if (!pg || !pg->block_table || !pg->seq_lens || !aligned4(pg->block_table) ||
      !aligned4(pg->seq_lens))
    return KSA_ERR_INVALID_ARGUMENT;
  if (pg->max_blocks < 1 || pg->num_pages < 1) return KSA_ERR_INVALID_ARGUMENT;
  if ((int64_t)pg->max_blocks * p.block_size != p.max_seq_len) return KSA_ERR_INVALID_ARGUMENT;
  if ((int64_t)pg->num_pages * p.num_kv_heads * p.block_size >= ((int64_t)1 << 31))
    return KSA_ERR_UNSUPPORTED;
  out->table = pg->block_table;
  out->seq_lens = pg->seq_lens;
  out->max_blocks = pg->max_blocks;
  out->num_pages = pg->num_pages;
  return KSA_OK;
}

// The voting heads as a bitmask: num_voting distinct heads < Hq (and < 256).
ksa_status head_mask(const ksa_problem& p, const int32_t* voting_heads, int32_t num_voting,
                     HeadMask* mask) {
  if (!voting_heads || num_voting < 1 || num_voting > p.num_q_heads)
    return KSA_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < 8; ++i) mask->w[i] = 0u;
  for (int32_t i = 0; i < num_voting; ++i) {
    const int32_t h = voting_heads[i];
    if (h < 0 || h >= p.num_q_heads || h > 255) return KSA_ERR_INVALID_ARGUMENT;
    if ((mask->w[h >> 5] >> (h & 31)) & 1u) return KSA_ERR_INVALID_ARGUMENT;  // listed twice
    mask->w[h >> 5] |= 1u << (h & 31);
  }
  return KSA_OK;
}

}  // namespace
}  // namespace ksa

// ---------------------------------------------------------------- no-allocation scratch
// Split-row scratch (partial states and arrival words) of
// ksa_sparse_decode_noalloc: one array per GPU the library runs on, held
// until the process ends, shared by every such call on that GPU.  Rows are
// split when there are fewer than 256 of them (at most ~2.2 MB of scratch
// for lists of up to 2048 entries) or when a list outgrows the 2048-entry
// LDS stage; calls needing more than the array are refused.  On the host,
// `scratch` names a
// stand-in, not a device address: kernels get the address that
// hipGetSymbolAddress returns for the device, found once per device.
static __device__ __align__(256) unsigned char scratch[KSA_NOALLOC_SCRATCH_BYTES];

namespace ksa {
namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];

// The scratch of the device `stream` runs on, which must be the current
// device (hipGetSymbolAddress resolves the symbol on the current device).
ksa_status noalloc_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return KSA_ERR_HIP;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return KSA_ERR_HIP;
    if (sdev != dev) return KSA_ERR_INVALID_ARGUMENT;
  }
  if (dev < 0 || dev >= kMaxScratchDevices) return KSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KSA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KSA_OK;
}

// ksa_sparse_decode, with the workspace size check delegated: workspace_for
// receives the bytes the call needs and returns whether `workspace` holds
// them (the no-allocation entry point supplies its own scratch there).
template <typename WorkspaceFor>
ksa_status sparse_decode(const ksa_problem* problem, const void* q, const void* k, const void* v,
                         const ksa_selection* sel, float* out, float* lse, void* stream,
                         WorkspaceFor workspace_for) {
  if (!sel) return KSA_ERR_INVALID_ARGUMENT;
  const bool blocks = sel->kind == KSA_SEL_BLOCKS;
  if (!blocks && sel->kind != KSA_SEL_TOKENS && sel->kind != KSA_SEL_HEAD_TOKENS)
    return KSA_ERR_INVALID_ARGUMENT;
  ksa_status st = check_problem(problem, blocks);
  if (st != KSA_OK) return st;
  const Dims d = make_dims(*problem);
  if (!q || !k || !v || !out || !sel->idx) return KSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned4(out) || !aligned4(sel->idx) ||
      (lse && !aligned4(lse)))
    return KSA_ERR_INVALID_ARGUMENT;
  if (sel->count < 1) return KSA_ERR_INVALID_ARGUMENT;
  if (blocks && sel->count > d.NB) return KSA_ERR_INVALID_ARGUMENT;
  if (!blocks && sel->count > d.T) return KSA_ERR_INVALID_ARGUMENT;
  if (blocks && (int64_t)sel->count * d.Bs > INT32_MAX / 2) return KSA_ERR_UNSUPPORTED;
  if (sel->kind == KSA_SEL_HEAD_TOKENS) {  // rows are query heads, each its own group
    Dims dh = d;
    dh.Hkv = d.Hq;
    dh.G = 1;
    const AttnPlan plan = plan_attention(dh, 4, sel->count);
    void* workspace = nullptr;
    st = workspace_for(attention_workspace_bytes(dh, plan), &workspace);
    if (st != KSA_OK) return st;
    return from_hip(launch_attention(dh, 4, q, k, v, sel->idx, sel->count, out, lse, workspace,
                                     plan, (hipStream_t)stream, nullptr, nullptr, d.G));
  }
  const int64_t ltot = blocks ? (int64_t)sel->count * d.Bs : sel->count;
  const AttnPlan plan = plan_attention(d, blocks ? 0 : 1, ltot);
  void* workspace = nullptr;
  st = workspace_for(attention_workspace_bytes(d, plan), &workspace);
  if (st != KSA_OK) return st;
  return from_hip(launch_attention(d, blocks ? 0 : 1, q, k, v, sel->idx, sel->count, out, lse,
                                   workspace, plan, (hipStream_t)stream));
}

}  // namespace
}  // namespace ksa

using namespace ksa;

extern "C" {

const char* ksa_version(void) { return "0.1.0"; }

const char* ksa_status_string(ksa_status status) {
  switch (status) {
    case KSA_OK: return "KSA_OK: success";
    case KSA_ERR_INVALID_ARGUMENT: return "KSA_ERR_INVALID_ARGUMENT: an argument is out of range";
    case KSA_ERR_UNSUPPORTED: return "KSA_ERR_UNSUPPORTED: valid arguments outside what this library handles";
    case KSA_ERR_WORKSPACE_TOO_SMALL: return "KSA_ERR_WORKSPACE_TOO_SMALL: workspace smaller than ksa_workspace_bytes()";
    case KSA_ERR_HIP: return "KSA_ERR_HIP: a HIP kernel launch failed";
    default: return "unknown ksa_status";
  }
}

size_t ksa_workspace_bytes(const ksa_problem* problem, int32_t op, int32_t param) {
  const bool blocks = op == KSA_OP_SELECT_TOPK || op == KSA_OP_SPARSE_BLOCKS ||
                      op == KSA_OP_PAGED_DENSE || op == KSA_OP_PAGED_VOTE_LAYER;
  if (check_problem(problem, blocks) != KSA_OK) return SIZE_MAX;
  if (op < KSA_OP_SELECT_TOPK || op > KSA_OP_PAGED_VOTE_LAYER) return SIZE_MAX;
  if (op != KSA_OP_DENSE && op != KSA_OP_PAGED_DENSE && param < 1) return SIZE_MAX;
  return workspace_for(*problem, op, param);
}

ksa_status ksa_block_summaries(const ksa_problem* problem, const void* k, void* summaries,
                               int32_t first_block, int32_t num_blocks, void* stream) {
  ksa_status st = check_problem(problem, true);
  if (st != KSA_OK) return st;
  const Dims d = make_dims(*problem);
  if (!k || !summaries || !aligned16(k) || !aligned16(summaries)) return KSA_ERR_INVALID_ARGUMENT;
  if (first_block < 0 || num_blocks < 1 || (int64_t)first_block + num_blocks > d.NB)
    return KSA_ERR_INVALID_ARGUMENT;
  return from_hip(launch_block_summaries(d, k, summaries, first_block, num_blocks,
                                         (hipStream_t)stream));
}

ksa_status ksa_select_topk(const ksa_problem* problem, const void* q, const void* summaries,
                           int32_t top_k, int32_t* block_idx, float* block_scores, void* workspace,
                           size_t workspace_bytes, void* stream) {
  ksa_status st = check_problem(problem, true);
  if (st != KSA_OK) return st;
  const Dims d = make_dims(*problem);
  if (!q || !summaries || !block_idx || top_k < 1) return KSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(summaries) || !aligned4(block_idx) ||
      (block_scores && !aligned4(block_scores)))
    return KSA_ERR_INVALID_ARGUMENT;
  if (d.NB > kSelectMaxBlocks) return KSA_ERR_UNSUPPORTED;
  const size_t need = workspace_for(*problem, KSA_OP_SELECT_TOPK, top_k);
  if (workspace_bytes < need) return KSA_ERR_WORKSPACE_TOO_SMALL;
  if (need && (!workspace || !aligned16(workspace))) return KSA_ERR_INVALID_ARGUMENT;
  const int keff = top_k < d.NB ? top_k : d.NB;
  return from_hip(launch_select_topk(d, q, summaries, keff, block_idx, block_scores, workspace,
                                     (hipStream_t)stream));
}

ksa_status ksa_sparse_decode(const ksa_problem* problem, const void* q, const void* k,
                             const void* v, const ksa_selection* sel, float* out, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return sparse_decode(problem, q, k, v, sel, out, lse, stream,
                       [&](size_t need, void** ws) -> ksa_status {
                         if (workspace_bytes < need) return KSA_ERR_WORKSPACE_TOO_SMALL;
                         if (need && (!workspace || !aligned16(workspace)))
                           return KSA_ERR_INVALID_ARGUMENT;
                         *ws = workspace;
                         return KSA_OK;
                       });
}

ksa_status ksa_sparse_decode_noalloc(const ksa_problem* problem, const void* q, const void* k,
                                     const void* v, const ksa_selection* sel, float* out,
                                     float* lse, void* stream) {
  return sparse_decode(problem, q, k, v, sel, out, lse, stream,
                       [&](size_t need, void** ws) -> ksa_status {
                         if (need > (size_t)KSA_NOALLOC_SCRATCH_BYTES) return KSA_ERR_UNSUPPORTED;
                         if (need == 0) return KSA_OK;
                         return noalloc_scratch((hipStream_t)stream, ws);
                       });
}

ksa_status ksa_vote_select(const ksa_problem* problem, const void* q, const void* k,
                           int32_t token_budget, int32_t recent_window, int32_t* token_idx,
                           uint8_t* votes, void* workspace, size_t workspace_bytes, void* stream) {
  ksa_status st = check_problem(problem, false);
  if (st != KSA_OK) return st;
  const Dims d = make_dims(*problem);
  if (!q || !k || !token_idx) return KSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned4(token_idx)) return KSA_ERR_INVALID_ARGUMENT;
  if (token_budget < 1 || recent_window < 0 || recent_window > token_budget)
    return KSA_ERR_INVALID_ARGUMENT;
  if (d.Hq > 255) return KSA_ERR_UNSUPPORTED;  // vote counts are bytes
  if (d.T > token_budget && (d.T - recent_window) > (1 << 21)) return KSA_ERR_UNSUPPORTED;
  const VotePlan plan = plan_vote(d, token_budget, recent_window);
  if (workspace_bytes < plan.total) return KSA_ERR_WORKSPACE_TOO_SMALL;
  if (plan.total && (!workspace || !aligned16(workspace))) return KSA_ERR_INVALID_ARGUMENT;
  return from_hip(launch_vote_select(d, q, k, token_budget, recent_window, token_idx, votes,
                                     workspace, plan, (hipStream_t)stream));
}

ksa_status ksa_dense_decode(const ksa_problem* problem, const void* q, const void* k,
                            const void* v, float* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream) {
  ksa_status st = check_problem(problem, false);
  if (st != KSA_OK) return st;
  const Dims d = make_dims(*problem);
  if (!q || !k || !v || !out) return KSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned4(out) || (lse && !aligned4(lse)))
    return KSA_ERR_INVALID_ARGUMENT;
  const AttnPlan plan = plan_attention(d, 2, d.T);
  const size_t need = attention_workspace_bytes(d, plan);
  if (workspace_bytes < need) return KSA_ERR_WORKSPACE_TOO_SMALL;
  if (need && (!workspace || !aligned16(workspace))) return KSA_ERR_INVALID_ARGUMENT;
  return from_hip(launch_attention(d, 2, q, k, v, nullptr, 0, out, lse, workspace, plan,
                                   (hipStream_t)stream));
}

namespace {
// ksa_block_topk_decode with an optional length per sequence
ksa_status block_topk_decode(const ksa_problem* problem, const int32_t* seq_lens, const void* q,
                             const void* k, const void* v, void* summaries, int32_t top_k,
                             int32_t refresh_last_block, int32_t* block_idx, float* out,
                             float* lse, void* stream) {
  ksa_status st = check_problem(problem, true);
  if (st != KSA_OK) return st;
  const Dims d = make_dims(*problem);
  if (!q || !k || !v || !summaries || !out || top_k < 1) return KSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(summaries) || !aligned4(out) ||
      (lse && !aligned4(lse)) || (block_idx && !aligned4(block_idx)))
    return KSA_ERR_INVALID_ARGUMENT;
  const int keff = top_k < d.NB ? top_k : d.NB;
  if (d.NB > kStepMaxBlocks || keff > kIdxStage) return KSA_ERR_UNSUPPORTED;
  if ((int64_t)keff * d.Bs > INT32_MAX / 2) return KSA_ERR_UNSUPPORTED;
  if (refresh_last_block && d.Bs > kStepMaxBs) return KSA_ERR_UNSUPPORTED;
  return from_hip(launch_block_topk_decode(d, q, k, v, summaries, keff, refresh_last_block, block_idx,
                                           out, lse, (hipStream_t)stream, nullptr, seq_lens));
}
}  // namespace

ksa_status ksa_block_topk_decode(const ksa_problem* problem, const void* q, const void* k,
                                 const void* v, void* summaries, int32_t top_k,
                                 int32_t refresh_last_block, int32_t* block_idx, float* out,
                                 float* lse, void* stream) {
  return block_topk_decode(problem, nullptr, q, k, v, summaries, top_k, refresh_last_block,
                           block_idx, out, lse, stream);
}

ksa_status ksa_block_topk_decode_varlen(const ksa_problem* problem, const int32_t* seq_lens,
                                        const void* q, const void* k, const void* v,
                                        void* summaries, int32_t top_k,
                                        int32_t refresh_last_block, int32_t* block_idx,
                                        float* out, float* lse, void* stream) {
  if (!problem) return KSA_ERR_INVALID_ARGUMENT;
  if (!seq_lens || !aligned4(seq_lens)) return KSA_ERR_INVALID_ARGUMENT;
  return block_topk_decode(problem, seq_lens, q, k, v, summaries, top_k, refresh_last_block,
                           block_idx, out, lse, stream);
}

ksa_status ksa_paged_block_summaries(const ksa_problem* problem, const ksa_paged_kv* paged,
                                     const void* k_pool, void* summaries, int32_t first_block,
                                     int32_t num_blocks, void* stream) {
  ksa_status st = check_problem(problem, true);
  if (st != KSA_OK) return st;
  PagedKv pk;
  st = check_paged(*problem, paged, &pk);
  if (st != KSA_OK) return st;
  const Dims d = make_dims(*problem);
  if (!k_pool || !summaries || !aligned16(k_pool) || !aligned16(summaries))
    return KSA_ERR_INVALID_ARGUMENT;
  const bool newest = first_block == -1 && num_blocks == 1;
  if (!newest &&
      (first_block < 0 || num_blocks < 1 || (int64_t)first_block + num_blocks > pk.max_blocks))
    return KSA_ERR_INVALID_ARGUMENT;
  return from_hip(launch_paged_block_summaries(d, pk, k_pool, summaries, first_block, num_blocks,
                                               (hipStream_t)stream));
}

ksa_status ksa_paged_block_topk_decode(const ksa_problem* problem, const ksa_paged_kv* paged,
                                       const void* q, const void* k_pool, const void* v_pool,
                                       void* summaries, int32_t top_k, int32_t refresh_last_block,
                                       int32_t* block_idx, float* out, float* lse, void* stream) {
  ksa_status st = check_problem(problem, true);
  if (st != KSA_OK) return st;
  PagedKv pk;
  st = check_paged(*problem, paged, &pk);
  if (st != KSA_OK) return st;
  const Dims d = make_dims(*problem);
  if (!q || !k_pool || !v_pool || !summaries || !out || top_k < 1) return KSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(summaries) ||
      !aligned4(out) || (lse && !aligned4(lse)) || (block_idx && !aligned4(block_idx)))
    return KSA_ERR_INVALID_ARGUMENT;
  const int keff_max = top_k < pk.max_blocks ? top_k : pk.max_blocks;
  if (pk.max_blocks > kStepMaxBlocks || keff_max > kIdxStage) return KSA_ERR_UNSUPPORTED;
  if ((int64_t)keff_max * d.Bs > INT32_MAX / 2) return KSA_ERR_UNSUPPORTED;
  if (refresh_last_block && d.Bs > kStepMaxBs) return KSA_ERR_UNSUPPORTED;
  return from_hip(launch_block_topk_decode(d, q, k_pool, v_pool, summaries, top_k,
                                           refresh_last_block, block_idx, out, lse,
                                           (hipStream_t)stream, &pk));
}

ksa_status ksa_paged_dense_decode(const ksa_problem* problem, const ksa_paged_kv* paged,
                                  const void* q, const void* k_pool, const void* v_pool, float* out,
                                  float* lse, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  ksa_status st = check_problem(problem, true);
  if (st != KSA_OK) return st;
  PagedKv pk;
  st = check_paged(*problem, paged, &pk);
  if (st != KSA_OK) return st;
  const Dims d = make_dims(*problem);
  if (!q || !k_pool || !v_pool || !out) return KSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned4(out) ||
      (lse && !aligned4(lse)))
    return KSA_ERR_INVALID_ARGUMENT;
  const AttnPlan plan = plan_attention(d, 3, (int64_t)d.NB * d.Bs);
  const size_t need = attention_workspace_bytes(d, plan);
  if (workspace_bytes < need) return KSA_ERR_WORKSPACE_TOO_SMALL;
  if (need && (!workspace || !aligned16(workspace))) return KSA_ERR_INVALID_ARGUMENT;
  return from_hip(launch_attention(d, 3, q, k_pool, v_pool, nullptr, 0, out, lse, workspace, plan,
                                   (hipStream_t)stream, &pk));
}

ksa_status ksa_select_topk_ex(const ksa_problem* problem, const void* q, const void* summaries,
                              const ksa_select_options* options, int32_t* block_idx,
                              float* block_scores, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (!options) return KSA_ERR_INVALID_ARGUMENT;
  if (options->aggregate != KSA_AGG_SUM && options->aggregate != KSA_AGG_MAX)
    return KSA_ERR_INVALID_ARGUMENT;
  ksa_status st = check_problem(problem, true);
  if (st != KSA_OK) return st;
  const Dims d = make_dims(*problem);
  const int32_t top_k = options->top_k;
  if (!q || !summaries || !block_idx || top_k < 1) return KSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(summaries) || !aligned4(block_idx) ||
      (block_scores && !aligned4(block_scores)))
    return KSA_ERR_INVALID_ARGUMENT;
  if (d.NB > kSelectMaxBlocks) return KSA_ERR_UNSUPPORTED;
  const size_t need = workspace_for(*problem, KSA_OP_SELECT_TOPK, top_k);
  if (workspace_bytes < need) return KSA_ERR_WORKSPACE_TOO_SMALL;
  if (need && (!workspace || !aligned16(workspace))) return KSA_ERR_INVALID_ARGUMENT;
  const int keff = top_k < d.NB ? top_k : d.NB;
  SelectVariant var;
  var.agg_max = options->aggregate == KSA_AGG_MAX ? 1 : 0;
  var.forced_block = options->force_last_block ? (d.T - 1) / d.Bs : -1;
  return from_hip(launch_select_topk(d, q, summaries, keff, block_idx, block_scores, workspace,
                                     (hipStream_t)stream, var));
}

ksa_status ksa_paged_select_topk_ex(const ksa_problem* problem, const ksa_paged_kv* paged,
                                    const void* q, const void* summaries,
                                    const ksa_select_options* options, int32_t* block_idx,
                                    float* block_scores, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  if (!options) return KSA_ERR_INVALID_ARGUMENT;
  if (options->aggregate != KSA_AGG_SUM && options->aggregate != KSA_AGG_MAX)
    return KSA_ERR_INVALID_ARGUMENT;
  ksa_status st = check_problem(problem, true);
  if (st != KSA_OK) return st;
  PagedKv pk;
  st = check_paged(*problem, paged, &pk);
  if (st != KSA_OK) return st;
  const Dims d = make_dims(*problem);
  const int32_t top_k = options->top_k;
  if (!q || !summaries || !block_idx || top_k < 1) return KSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(summaries) || !aligned4(block_idx) ||
      (block_scores && !aligned4(block_scores)))
    return KSA_ERR_INVALID_ARGUMENT;
  if (d.NB > kSelectMaxBlocks) return KSA_ERR_UNSUPPORTED;
  const size_t need = workspace_for(*problem, KSA_OP_SELECT_TOPK, top_k);
  if (workspace_bytes < need) return KSA_ERR_WORKSPACE_TOO_SMALL;
  if (need && (!workspace || !aligned16(workspace))) return KSA_ERR_INVALID_ARGUMENT;
  SelectVariant var;
  var.agg_max = options->aggregate == KSA_AGG_MAX ? 1 : 0;
  var.forced_block = options->force_last_block ? 0 : -1;  // each row's own newest block
  var.seq_lens = pk.seq_lens;
  var.id_stride = top_k;
  return from_hip(launch_select_topk(d, q, summaries, top_k, block_idx, block_scores, workspace,
                                     (hipStream_t)stream, var));
}

ksa_status ksa_paged_vote_select_heads(const ksa_problem* problem, const ksa_paged_kv* paged,
                                       const void* q, const void* k_pool, int32_t token_budget,
                                       int32_t recent_window, const int32_t* voting_heads,
                                       int32_t num_voting, int32_t* token_idx, uint8_t* votes,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  ksa_status st = check_problem(problem, true);
  if (st != KSA_OK) return st;
  PagedKv pk;
  st = check_paged(*problem, paged, &pk);
  if (st != KSA_OK) return st;
  HeadMask mask;
  st = head_mask(*problem, voting_heads, num_voting, &mask);
  if (st != KSA_OK) return st;
  const Dims d = make_dims(*problem);
  if (!q || !k_pool || !token_idx) return KSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned4(token_idx)) return KSA_ERR_INVALID_ARGUMENT;
  if (token_budget < 1 || recent_window < 0 || recent_window > token_budget)
    return KSA_ERR_INVALID_ARGUMENT;
  if (d.Hq > 255) return KSA_ERR_UNSUPPORTED;
  if (d.T > token_budget && (d.T - recent_window) > (1 << 21)) return KSA_ERR_UNSUPPORTED;
  const VotePlan plan = plan_vote(d, token_budget, recent_window);
  if (workspace_bytes < plan.total) return KSA_ERR_WORKSPACE_TOO_SMALL;
  if (plan.total && (!workspace || !aligned16(workspace))) return KSA_ERR_INVALID_ARGUMENT;
  return from_hip(launch_paged_vote_select(d, pk, q, k_pool, token_budget, recent_window, token_idx,
                                           votes, workspace, plan, (hipStream_t)stream, mask));
}

ksa_status ksa_vote_select_heads(const ksa_problem* problem, const void* q, const void* k,
                                 int32_t token_budget, int32_t recent_window,
                                 const int32_t* voting_heads, int32_t num_voting,
                                 int32_t* token_idx, uint8_t* votes, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  ksa_status st = check_problem(problem, false);
  if (st != KSA_OK) return st;
  HeadMask mask;
  st = head_mask(*problem, voting_heads, num_voting, &mask);
  if (st != KSA_OK) return st;
  const Dims d = make_dims(*problem);
  if (!q || !k || !token_idx) return KSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned4(token_idx)) return KSA_ERR_INVALID_ARGUMENT;
  if (token_budget < 1 || recent_window < 0 || recent_window > token_budget)
    return KSA_ERR_INVALID_ARGUMENT;
  if (d.Hq > 255) return KSA_ERR_UNSUPPORTED;
  if (d.T > token_budget && (d.T - recent_window) > (1 << 21)) return KSA_ERR_UNSUPPORTED;
  const VotePlan plan = plan_vote(d, token_budget, recent_window);
  if (workspace_bytes < plan.total) return KSA_ERR_WORKSPACE_TOO_SMALL;
  if (plan.total && (!workspace || !aligned16(workspace))) return KSA_ERR_INVALID_ARGUMENT;
  return from_hip(launch_vote_select(d, q, k, token_budget, recent_window, token_idx, votes,
                                     workspace, plan, (hipStream_t)stream, mask));
}

ksa_status ksa_attention_recall(const float* lse_selected, const float* lse_dense, float* recall,
                                int32_t count, void* stream) {
  if (!lse_selected || !lse_dense || !recall || count < 1) return KSA_ERR_INVALID_ARGUMENT;
  if (!aligned4(lse_selected) || !aligned4(lse_dense) || !aligned4(recall))
    return KSA_ERR_INVALID_ARGUMENT;
  return from_hip(launch_attention_recall(lse_selected, lse_dense, recall, count,
                                          (hipStream_t)stream));
}

ksa_status ksa_vote_layer_decode(const ksa_problem* problem, const void* q, const void* k,
                                 const void* v, int32_t token_budget, int32_t recent_window,
                                 float* out, float* lse, int32_t* token_idx, uint8_t* votes,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  ksa_status st = check_problem(problem, false);
  if (st != KSA_OK) return st;
  const Dims d = make_dims(*problem);
  if (!q || !k || !v || !out || !token_idx) return KSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned4(out) || !aligned4(token_idx) ||
      (lse && !aligned4(lse)))
    return KSA_ERR_INVALID_ARGUMENT;
  if (token_budget < 1 || recent_window < 0 || recent_window > token_budget)
    return KSA_ERR_INVALID_ARGUMENT;
  if (d.Hq > 255) return KSA_ERR_UNSUPPORTED;
  if (d.T > token_budget && (d.T - recent_window) > (1 << 21)) return KSA_ERR_UNSUPPORTED;
  const VotePlan vplan = plan_vote(d, token_budget, recent_window);
  const size_t voff = (vplan.total + 255) & ~(size_t)255;
  const AttnPlan aplan = plan_attention(d, 2, d.T);
  const size_t need = voff + attention_workspace_bytes(d, aplan);
  if (workspace_bytes < need) return KSA_ERR_WORKSPACE_TOO_SMALL;
  if (need && (!workspace || !aligned16(workspace))) return KSA_ERR_INVALID_ARGUMENT;
  const hipStream_t s = (hipStream_t)stream;
  void* aws = (char*)workspace + voff;
  if (d.T <= token_budget) {
    hipError_t e = launch_attention(d, 2, q, k, v, nullptr, 0, out, lse, aws, aplan, s);
    if (e != hipSuccess) return KSA_ERR_HIP;
    return from_hip(launch_vote_all(d, token_idx, votes, s));
  }
  if (dense_emits_vote_keys(d)) {
    VoteKeys vk;
    vk.keys = (uint32_t*)((char*)workspace + vplan.keys_off);
    vk.kstride = vplan.kstride;
    vk.hist = vplan.hist;
    hipError_t e = launch_attention(d, 2, q, k, v, nullptr, 0, out, lse, aws, aplan, s, nullptr, &vk);
    if (e != hipSuccess) return KSA_ERR_HIP;
    return from_hip(launch_vote_finish(d, token_budget, recent_window, token_idx, votes, workspace,
                                       vplan, s));
  }
  hipError_t e = launch_attention(d, 2, q, k, v, nullptr, 0, out, lse, aws, aplan, s);
  if (e != hipSuccess) return KSA_ERR_HIP;
  return from_hip(launch_vote_select(d, q, k, token_budget, recent_window, token_idx, votes,
                                     workspace, vplan, s));
}

ksa_status ksa_paged_vote_layer_decode(const ksa_problem* problem, const ksa_paged_kv* paged,
                                       const void* q, const void* k_pool, const void* v_pool,
                                       int32_t token_budget, int32_t recent_window, float* out,
                                       float* lse, int32_t* token_idx, uint8_t* votes,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  ksa_status st = check_problem(problem, true);
  if (st != KSA_OK) return st;
  PagedKv pk;
  st = check_paged(*problem, paged, &pk);
  if (st != KSA_OK) return st;
  const Dims d = make_dims(*problem);
  if (!q || !k_pool || !v_pool || !out || !token_idx) return KSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned4(out) ||
      !aligned4(token_idx) || (lse && !aligned4(lse)))
    return KSA_ERR_INVALID_ARGUMENT;
  if (token_budget < 1 || recent_window < 0 || recent_window > token_budget)
    return KSA_ERR_INVALID_ARGUMENT;
  if (d.Hq > 255) return KSA_ERR_UNSUPPORTED;
  if (d.T > token_budget && (d.T - recent_window) > (1 << 21)) return KSA_ERR_UNSUPPORTED;
  const VotePlan vplan = plan_vote(d, token_budget, recent_window);
  const size_t voff = (vplan.total + 255) & ~(size_t)255;
  const AttnPlan aplan = plan_attention(d, 3, (int64_t)d.NB * d.Bs);
  const size_t need = voff + attention_workspace_bytes(d, aplan);
  if (workspace_bytes < need) return KSA_ERR_WORKSPACE_TOO_SMALL;
  if (need && (!workspace || !aligned16(workspace))) return KSA_ERR_INVALID_ARGUMENT;
  const hipStream_t s = (hipStream_t)stream;
  void* aws = (char*)workspace + voff;
  if (dense_emits_vote_keys(d) && d.T > token_budget) {
    // the paged dense walk writes each sequence's vote keys as it attends
    VoteKeys vk;
    vk.keys = (uint32_t*)((char*)workspace + vplan.keys_off);
    vk.kstride = vplan.kstride;
    vk.hist = vplan.hist;
    vk.budget = token_budget;
    vk.window = recent_window;
    hipError_t e = launch_attention(d, 3, q, k_pool, v_pool, nullptr, 0, out, lse, aws, aplan, s,
                                    &pk, &vk);
    if (e != hipSuccess) return KSA_ERR_HIP;
    return from_hip(launch_paged_vote_finish(d, pk, token_budget, recent_window, token_idx, votes,
                                             workspace, vplan, s));
  }
  hipError_t e = launch_attention(d, 3, q, k_pool, v_pool, nullptr, 0, out, lse, aws, aplan, s, &pk);
  if (e != hipSuccess) return KSA_ERR_HIP;
  return from_hip(launch_paged_vote_select(d, pk, q, k_pool, token_budget, recent_window, token_idx,
                                           votes, workspace, vplan, s));
}

ksa_status ksa_vote_select_per_head(const ksa_problem* problem, const void* q, const void* k,
                                    int32_t token_budget, int32_t recent_window,
                                    int32_t* token_idx, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  ksa_status st = check_problem(problem, false);
  if (st != KSA_OK) return st;
  const Dims d = make_dims(*problem);
  if (!q || !k || !token_idx) return KSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned4(token_idx)) return KSA_ERR_INVALID_ARGUMENT;
  if (token_budget < 1 || recent_window < 0 || recent_window > token_budget)
    return KSA_ERR_INVALID_ARGUMENT;
  if (d.Hq > 255) return KSA_ERR_UNSUPPORTED;
  if (d.T > token_budget && (d.T - recent_window) > (1 << 21)) return KSA_ERR_UNSUPPORTED;
  const VotePlan plan = plan_vote(d, token_budget, recent_window);
  if (workspace_bytes < plan.total) return KSA_ERR_WORKSPACE_TOO_SMALL;
  if (plan.total && (!workspace || !aligned16(workspace))) return KSA_ERR_INVALID_ARGUMENT;
  return from_hip(launch_vote_per_head(d, q, k, token_budget, recent_window, token_idx, workspace,
                                       plan, (hipStream_t)stream));
}

ksa_status ksa_paged_vote_select_per_head(const ksa_problem* problem, const ksa_paged_kv* paged,
                                          const void* q, const void* k_pool,
                                          int32_t token_budget, int32_t recent_window,
                                          int32_t* token_idx, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  ksa_status st = check_problem(problem, true);
  if (st != KSA_OK) return st;
  PagedKv pk;
  st = check_paged(*problem, paged, &pk);
  if (st != KSA_OK) return st;
  const Dims d = make_dims(*problem);
  if (!q || !k_pool || !token_idx) return KSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned4(token_idx)) return KSA_ERR_INVALID_ARGUMENT;
  if (token_budget < 1 || recent_window < 0 || recent_window > token_budget)
    return KSA_ERR_INVALID_ARGUMENT;
  if (d.Hq > 255) return KSA_ERR_UNSUPPORTED;
  if (d.T > token_budget && (d.T - recent_window) > (1 << 21)) return KSA_ERR_UNSUPPORTED;
  const VotePlan plan = plan_vote(d, token_budget, recent_window);
  if (workspace_bytes < plan.total) return KSA_ERR_WORKSPACE_TOO_SMALL;
  if (plan.total && (!workspace || !aligned16(workspace))) return KSA_ERR_INVALID_ARGUMENT;
  return from_hip(launch_vote_per_head(d, q, k_pool, token_budget, recent_window, token_idx,
                                       workspace, plan, (hipStream_t)stream, &pk));
}

ksa_status ksa_paged_vote_select(const ksa_problem* problem, const ksa_paged_kv* paged,
                                 const void* q, const void* k_pool, int32_t token_budget,
                                 int32_t recent_window, int32_t* token_idx, uint8_t* votes,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  ksa_status st = check_problem(problem, true);
  if (st != KSA_OK) return st;
  PagedKv pk;
  st = check_paged(*problem, paged, &pk);
  if (st != KSA_OK) return st;
  const Dims d = make_dims(*problem);
  if (!q || !k_pool || !token_idx) return KSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned4(token_idx)) return KSA_ERR_INVALID_ARGUMENT;
  if (token_budget < 1 || recent_window < 0 || recent_window > token_budget)
    return KSA_ERR_INVALID_ARGUMENT;
  if (d.Hq > 255) return KSA_ERR_UNSUPPORTED;
  if (d.T > token_budget && (d.T - recent_window) > (1 << 21)) return KSA_ERR_UNSUPPORTED;
  const VotePlan plan = plan_vote(d, token_budget, recent_window);
  if (workspace_bytes < plan.total) return KSA_ERR_WORKSPACE_TOO_SMALL;
  if (plan.total && (!workspace || !aligned16(workspace))) return KSA_ERR_INVALID_ARGUMENT;
  return from_hip(launch_paged_vote_select(d, pk, q, k_pool, token_budget, recent_window, token_idx,
                                           votes, workspace, plan, (hipStream_t)stream));
}

ksa_status ksa_paged_sparse_decode(const ksa_problem* problem, const ksa_paged_kv* paged,
                                   const void* q, const void* k_pool, const void* v_pool,
                                   const ksa_selection* sel, float* out, float* lse,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!sel) return KSA_ERR_INVALID_ARGUMENT;
  const bool blocks = sel->kind == KSA_SEL_BLOCKS;
  if (!blocks && sel->kind != KSA_SEL_TOKENS && sel->kind != KSA_SEL_HEAD_TOKENS)
    return KSA_ERR_INVALID_ARGUMENT;
  ksa_status st = check_problem(problem, true);
  if (st != KSA_OK) return st;
  PagedKv pk;
  st = check_paged(*problem, paged, &pk);
  if (st != KSA_OK) return st;
  const Dims d = make_dims(*problem);
  if (!q || !k_pool || !v_pool || !out || !sel->idx) return KSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned4(out) ||
      !aligned4(sel->idx) || (lse && !aligned4(lse)))
    return KSA_ERR_INVALID_ARGUMENT;
  if (sel->count < 1) return KSA_ERR_INVALID_ARGUMENT;
  if (blocks && sel->count > pk.max_blocks) return KSA_ERR_INVALID_ARGUMENT;
  if (!blocks && sel->count > d.Tcap) return KSA_ERR_INVALID_ARGUMENT;
  if (blocks && (int64_t)sel->count * d.Bs > INT32_MAX / 2) return KSA_ERR_UNSUPPORTED;
  if (sel->kind == KSA_SEL_HEAD_TOKENS) {  // rows are query heads, each its own group
    Dims dh = d;
    dh.Hkv = d.Hq;
    dh.G = 1;
    const AttnPlan plan = plan_attention(dh, 6, sel->count);
    const size_t need = attention_workspace_bytes(dh, plan);
    if (workspace_bytes < need) return KSA_ERR_WORKSPACE_TOO_SMALL;
    if (need && (!workspace || !aligned16(workspace))) return KSA_ERR_INVALID_ARGUMENT;
    return from_hip(launch_attention(dh, 6, q, k_pool, v_pool, sel->idx, sel->count, out, lse,
                                     workspace, plan, (hipStream_t)stream, &pk, nullptr, d.G));
  }
  const int kind = blocks ? 3 : 5;
  const int64_t ltot = blocks ? (int64_t)sel->count * d.Bs : sel->count;
  const AttnPlan plan = plan_attention(d, kind, ltot);
  const size_t need = attention_workspace_bytes(d, plan);
  if (workspace_bytes < need) return KSA_ERR_WORKSPACE_TOO_SMALL;
  if (need && (!workspace || !aligned16(workspace))) return KSA_ERR_INVALID_ARGUMENT;
  return from_hip(launch_attention(d, kind, q, k_pool, v_pool, sel->idx, sel->count, out, lse,
                                   workspace, plan, (hipStream_t)stream, &pk));
}

}  // extern "C"

// Host-side argument checks and workspace layout (pure C++17).
#include "plan.h"

#include <cstdint>

namespace dspark {
namespace {

inline bool aligned(const void* p, std::size_t a) {
  return (reinterpret_cast<std::uintptr_t>(p) % a) == 0;
}

inline std::size_t round_up(std::size_t x, std::size_t a) { return (x + a - 1) / a * a; }

constexpr uint32_t kKnownFlags = DSPARK_CHECK_INPUTS;

// A workspace given to a call: present, large enough, 256-byte aligned.
inline int check_workspace(const void* ws, std::size_t have, std::size_t need) {
  if (need == 0) return DSPARK_OK;
  if (ws == nullptr || have < need) return DSPARK_ERR_WORKSPACE;
  if (!aligned(ws, kWsAlign)) return DSPARK_ERR_ALIGN;
  return DSPARK_OK;
}

// The optional fragment-packed W2: bf16 weights only, 16-byte aligned, at
// least as large as the layout for (V, rank).
inline int check_w2_packed(const void* w2p, std::size_t bytes, int32_t wdtype, int32_t V, int32_t rank) {
  if (w2p == nullptr) return DSPARK_OK;
  if (wdtype != DSPARK_W_BF16) return DSPARK_ERR_DTYPE;
  if (!aligned(w2p, 16)) return DSPARK_ERR_ALIGN;
  if (bytes < w2_packed_bytes(V, rank)) return DSPARK_ERR_WORKSPACE;
  return DSPARK_OK;
}

// Schedule-side shape checks shared by the top-K schedule and the cutoff.
inline int check_schedule_dims(int32_t R, int32_t gamma) {
  if (R < 0 || gamma < 1) return DSPARK_ERR_SHAPE;
  if (gamma > DSPARK_MAX_GAMMA) return DSPARK_ERR_UNSUPPORTED;
  const int64_t per_thread = (static_cast<int64_t>(R) + 1023) / 1024 * gamma;
  if (per_thread > DSPARK_SCHED_KEYS_PER_THREAD) return DSPARK_ERR_UNSUPPORTED;
  return DSPARK_OK;
}

// The head of a draft or verify call: the RNN head runs on the 16-row path
// only (bf16 weights, R <= 64).
inline int check_head(int32_t head, int32_t act, int32_t R, int32_t wdtype) {
  if (head == DSPARK_HEAD_MARKOV) return DSPARK_OK;
  if (head != DSPARK_HEAD_RNN) return DSPARK_ERR_UNSUPPORTED;
  if (act != DSPARK_ACT_IDENTITY && act != DSPARK_ACT_TANH) return DSPARK_ERR_UNSUPPORTED;
  if (seg_rows_for(R, wdtype) != kSegSmall) return DSPARK_ERR_UNSUPPORTED;
  return DSPARK_OK;
}

}  // namespace

int check_dims(int32_t R, int32_t gamma, int32_t V, int32_t rank, int32_t wdtype) {
  if (wdtype != DSPARK_W_F32 && wdtype != DSPARK_W_BF16) return DSPARK_ERR_DTYPE;
  if (R < 0 || gamma < 1 || V < 1 || rank < 1) return DSPARK_ERR_SHAPE;
  if (gamma > DSPARK_MAX_GAMMA || V > DSPARK_MAX_VOCAB) return DSPARK_ERR_UNSUPPORTED;
  if (rank < 8 || rank > DSPARK_MAX_RANK || rank % 8 != 0) return DSPARK_ERR_UNSUPPORTED;
  // request index is kept in 24 bits by the kernels' composite keys; the
  // [R, gamma, V] logits must be addressable with 64-bit offsets (always).
  if (R > (1 << 24)) return DSPARK_ERR_UNSUPPORTED;
  return DSPARK_OK;
}

int plan_draft(const dspark_draft_args* a, DraftPlan* plan) {
  if (a == nullptr || plan == nullptr) return DSPARK_ERR_NULL;
  if (a->struct_size != sizeof(dspark_draft_args)) return DSPARK_ERR_ABI;
  int st = check_dims(a->R, a->gamma, a->V, a->rank, a->wdtype);
  if (st != DSPARK_OK) return st;
  if ((a->flags & ~kKnownFlags) != 0) return DSPARK_ERR_UNSUPPORTED;
  st = check_head(a->head, a->act, a->R, a->wdtype);
  if (st != DSPARK_OK) return st;
  plan->check = (a->flags & DSPARK_CHECK_INPUTS) != 0;
  plan->seg_rows = seg_rows_for(a->R, a->wdtype);
  plan->n_seg = (a->V + plan->seg_rows - 1) / plan->seg_rows;
  const std::size_t rows = static_cast<std::size_t>(record_rows(plan->seg_rows, a->R));
  plan->part_off = kHeaderBytes;
  plan->total = kHeaderBytes + round_up(rows * plan->n_seg * kRecFloats * sizeof(float), kWsAlign);
  if (a->head == DSPARK_HEAD_RNN && plan->seg_rows == kSegSmall) {
    plan->ap_off = plan->total;
    plan->total += round_up(w2_packed_bytes(a->rank, a->rank), kWsAlign);
  }
  return DSPARK_OK;
}

int validate_draft(const dspark_draft_args* a, DraftPlan* plan) {
  int st = plan_draft(a, plan);
  if (st != DSPARK_OK) return st;
  if (a->R == 0) return DSPARK_OK;
  if (!a->U || !a->W1 || !a->W2 || !a->anchor || !a->temp || !a->u_draft || !a->y ||
      !a->q_tok || !a->q_stats)
    return DSPARK_ERR_NULL;
  if (!aligned(a->U, 16) || !aligned(a->W1, 16) || !aligned(a->W2, 16)) return DSPARK_ERR_ALIGN;
  if (!aligned(a->anchor, 4) || !aligned(a->temp, 4) || !aligned(a->u_draft, 4) ||
      !aligned(a->y, 4) || !aligned(a->q_tok, 4) || !aligned(a->q_stats, 8))
    return DSPARK_ERR_ALIGN;
  st = check_w2_packed(a->W2_packed, a->W2_packed_bytes, a->wdtype, a->V, a->rank);
  if (st != DSPARK_OK) return st;
  if (a->head == DSPARK_HEAD_RNN) {
    if (!a->A || !a->h) return DSPARK_ERR_NULL;
    if (!aligned(a->A, 16) || !aligned(a->h, 16)) return DSPARK_ERR_ALIGN;
  }
  return check_workspace(a->workspace, a->workspace_bytes, plan->total);
}

int plan_verify(const dspark_verify_args* a, VerifyPlan* plan) {
  if (a == nullptr || plan == nullptr) return DSPARK_ERR_NULL;
  if (a->struct_size != sizeof(dspark_verify_args)) return DSPARK_ERR_ABI;
  int st = check_dims(a->R, a->gamma, a->V, a->rank, a->wdtype);
  if (st != DSPARK_OK) return st;
  const int64_t max_rows = static_cast<int64_t>(a->R) * (a->gamma + 1);
  if (a->n_rows < a->R || a->n_rows > max_rows) return DSPARK_ERR_SHAPE;
  if ((a->flags & ~kKnownFlags) != 0) return DSPARK_ERR_UNSUPPORTED;
  st = check_head(a->head, DSPARK_ACT_IDENTITY, a->R, a->wdtype);
  if (st != DSPARK_OK) return st;
  plan->check = (a->flags & DSPARK_CHECK_INPUTS) != 0;
  plan->seg_rows = seg_rows_for(a->R, a->wdtype);
  plan->n_seg = (a->V + plan->seg_rows - 1) / plan->seg_rows;
  plan->n_chunks = (a->V + kChunk - 1) / kChunk;
  std::size_t off = kHeaderBytes;
  plan->vpart_off = off;
  off = round_up(off + static_cast<std::size_t>(a->n_rows) * plan->n_chunks * kChunkFloats * sizeof(float),
                 kWsAlign);
  plan->rsinfo_off = off;
  off = round_up(off + static_cast<std::size_t>(a->R) * 4 * sizeof(int32_t), kWsAlign);
  plan->rsstats_off = off;
  off = round_up(off + static_cast<std::size_t>(a->R) * 4 * sizeof(float), kWsAlign);
  const std::size_t rows = static_cast<std::size_t>(record_rows(plan->seg_rows, a->R));
  plan->rpart_off = off;
  off = round_up(off + rows * plan->n_seg * kRecFloats * sizeof(float), kWsAlign);
  if (plan->seg_rows == kSegWide) {
    plan->rcount_off = off;
    off = round_up(off + sizeof(int32_t), kWsAlign);
    plan->rlist_off = off;
    off = round_up(off + static_cast<std::size_t>(a->R) * kResidualEntryBytes, kWsAlign);
  }
  plan->total = off;
  return DSPARK_OK;
}

int validate_verify(const dspark_verify_args* a, VerifyPlan* plan) {
  int st = plan_verify(a, plan);
  if (st != DSPARK_OK) return st;
  if (a->R == 0) return DSPARK_OK;
  if (!a->target || !a->row_offsets || !a->U || !a->W1 || !a->W2 || !a->anchor || !a->temp ||
      !a->y || !a->q_tok || !a->q_stats || !a->u_accept || !a->u_final || !a->n_accept ||
      !a->out_tok || !a->p_tok)
    return DSPARK_ERR_NULL;
  if (!aligned(a->target, 16) || !aligned(a->U, 16) || !aligned(a->W1, 16) || !aligned(a->W2, 16))
    return DSPARK_ERR_ALIGN;
  if (!aligned(a->row_offsets, 4) || !aligned(a->anchor, 4) || !aligned(a->temp, 4) ||
      !aligned(a->y, 4) || !aligned(a->q_tok, 4) || !aligned(a->q_stats, 8) ||
      !aligned(a->u_accept, 4) || !aligned(a->u_final, 4) || !aligned(a->n_accept, 4) ||
      !aligned(a->out_tok, 4) || !aligned(a->p_tok, 4))
    return DSPARK_ERR_ALIGN;
  st = check_w2_packed(a->W2_packed, a->W2_packed_bytes, a->wdtype, a->V, a->rank);
  if (st != DSPARK_OK) return st;
  if (a->head == DSPARK_HEAD_RNN) {
    if (!a->h) return DSPARK_ERR_NULL;
    if (!aligned(a->h, 16)) return DSPARK_ERR_ALIGN;
  }
  return check_workspace(a->workspace, a->workspace_bytes, plan->total);
}

int validate_pack_w2(const dspark_pack_w2_args* a) {
  if (a == nullptr) return DSPARK_ERR_NULL;
  if (a->struct_size != sizeof(dspark_pack_w2_args)) return DSPARK_ERR_ABI;
  const int st = check_dims(0, 1, a->V, a->rank, DSPARK_W_BF16);
  if (st != DSPARK_OK) return st;
  if (!a->W2 || !a->W2_packed) return DSPARK_ERR_NULL;
  if (!aligned(a->W2, 16) || !aligned(a->W2_packed, 16)) return DSPARK_ERR_ALIGN;
  if (a->W2_packed_bytes < w2_packed_bytes(a->V, a->rank)) return DSPARK_ERR_WORKSPACE;
  return DSPARK_OK;
}

int plan_schedule(const dspark_schedule_args* a, std::size_t* bytes) {
  if (a == nullptr || bytes == nullptr) return DSPARK_ERR_NULL;
  if (a->struct_size != sizeof(dspark_schedule_args)) return DSPARK_ERR_ABI;
  const int st = check_schedule_dims(a->R, a->gamma);
  if (st != DSPARK_OK) return st;
  if ((a->flags & ~kKnownFlags) != 0) return DSPARK_ERR_UNSUPPORTED;
  *bytes = (a->flags & DSPARK_CHECK_INPUTS) ? kHeaderBytes : 0;
  return DSPARK_OK;
}

int plan_cutoff(const dspark_cutoff_args* a, std::size_t* bytes) {
  if (a == nullptr || bytes == nullptr) return DSPARK_ERR_NULL;
  if (a->struct_size != sizeof(dspark_cutoff_args)) return DSPARK_ERR_ABI;
  if (a->conf_min != a->conf_min) return DSPARK_ERR_SHAPE;
  const int st = check_schedule_dims(a->R, a->gamma);
  if (st != DSPARK_OK) return st;
  if ((a->flags & ~kKnownFlags) != 0) return DSPARK_ERR_UNSUPPORTED;
  *bytes = (a->flags & DSPARK_CHECK_INPUTS) ? kHeaderBytes : 0;
  return DSPARK_OK;
}

int validate_schedule(const dspark_schedule_args* a) {
  std::size_t need = 0;
  const int st = plan_schedule(a, &need);
  if (st != DSPARK_OK) return st;
  if (a->R == 0) return DSPARK_OK;
  if (!a->c || !a->anchor || !a->y || !a->a || !a->l || !a->row_offsets || !a->row_req ||
      !a->row_pos || !a->row_tok)
    return DSPARK_ERR_NULL;
  if (!aligned(a->c, 4) || !aligned(a->anchor, 4) || !aligned(a->y, 4) || !aligned(a->a, 4) ||
      !aligned(a->l, 4) || !aligned(a->row_offsets, 4) || !aligned(a->row_req, 4) ||
      !aligned(a->row_pos, 4) || !aligned(a->row_tok, 4) ||
      (a->expected_tokens && !aligned(a->expected_tokens, 4)))
    return DSPARK_ERR_ALIGN;
  return check_workspace(a->workspace, a->workspace_bytes, need);
}

int validate_cutoff(const dspark_cutoff_args* a) {
  std::size_t need = 0;
  const int st = plan_cutoff(a, &need);
  if (st != DSPARK_OK) return st;
  if (a->R == 0) return DSPARK_OK;
  if (!a->c || !a->anchor || !a->y || !a->a || !a->l || !a->row_offsets || !a->row_req || !a->row_pos ||
      !a->row_tok)
    return DSPARK_ERR_NULL;
  if (!aligned(a->c, 4) || !aligned(a->anchor, 4) || !aligned(a->y, 4) || !aligned(a->a, 4) ||
      !aligned(a->l, 4) || !aligned(a->row_offsets, 4) || !aligned(a->row_req, 4) ||
      !aligned(a->row_pos, 4) || !aligned(a->row_tok, 4) ||
      (a->expected_tokens && !aligned(a->expected_tokens, 4)))
    return DSPARK_ERR_ALIGN;
  return check_workspace(a->workspace, a->workspace_bytes, need);
}

int validate_capacity(const dspark_capacity_args* a) {
  if (a == nullptr) return DSPARK_ERR_NULL;
  if (a->struct_size != sizeof(dspark_capacity_args)) return DSPARK_ERR_ABI;
  if (a->R < 0 || a->gamma < 1) return DSPARK_ERR_SHAPE;
  if (a->gamma > DSPARK_MAX_GAMMA) return DSPARK_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(a->R) * a->gamma > DSPARK_CAPACITY_MAX_CANDIDATES) return DSPARK_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(a->n_sps) < static_cast<int64_t>(a->R) + 1) return DSPARK_ERR_SHAPE;
  if (!a->sps || !a->K || (a->R > 0 && !a->a_lag)) return DSPARK_ERR_NULL;
  if (!aligned(a->sps, 4) || !aligned(a->K, 4) || (a->a_lag && !aligned(a->a_lag, 4)) ||
      (a->expected && !aligned(a->expected, 8)) || (a->theta && !aligned(a->theta, 8)))
    return DSPARK_ERR_ALIGN;
  return DSPARK_OK;
}

int validate_sts_fit(const dspark_sts_fit_args* a) {
  if (a == nullptr) return DSPARK_ERR_NULL;
  if (a->struct_size != sizeof(dspark_sts_fit_args)) return DSPARK_ERR_ABI;
  if (a->N < 0 || a->gamma < 1) return DSPARK_ERR_SHAPE;
  if (a->gamma > DSPARK_MAX_GAMMA) return DSPARK_ERR_UNSUPPORTED;
  if (!a->tau || (a->N > 0 && (!a->z || !a->n_acc))) return DSPARK_ERR_NULL;
  if (!aligned(a->tau, 4) || (a->z && !aligned(a->z, 4)) || (a->n_acc && !aligned(a->n_acc, 4)))
    return DSPARK_ERR_ALIGN;
  return DSPARK_OK;
}

int validate_sts_apply(const dspark_sts_apply_args* a) {
  if (a == nullptr) return DSPARK_ERR_NULL;
  if (a->struct_size != sizeof(dspark_sts_apply_args)) return DSPARK_ERR_ABI;
  if (a->R < 0 || a->gamma < 1) return DSPARK_ERR_SHAPE;
  if (a->gamma > DSPARK_MAX_GAMMA) return DSPARK_ERR_UNSUPPORTED;
  if (a->R == 0) return DSPARK_OK;
  if (!a->z || !a->tau || !a->c) return DSPARK_ERR_NULL;
  if (!aligned(a->z, 4) || !aligned(a->tau, 4) || !aligned(a->c, 4)) return DSPARK_ERR_ALIGN;
  return DSPARK_OK;
}

int64_t schedule_rows(int32_t R, int32_t gamma, int64_t K) {
  if (R < 0 || gamma < 1) return -1;
  const int64_t n = static_cast<int64_t>(R) * gamma;
  int64_t kc = K < 0 ? 0 : K;
  if (kc > n) kc = n;
  return static_cast<int64_t>(R) + kc;
}

const char* status_string(int status) {
  switch (status) {
    case DSPARK_OK: return "ok";
    case DSPARK_ERR_NULL: return "a required pointer is NULL";
    case DSPARK_ERR_SHAPE: return "a size argument is out of range";
    case DSPARK_ERR_DTYPE: return "unknown weight dtype";
    case DSPARK_ERR_ALIGN: return "a pointer is not aligned as required";
    case DSPARK_ERR_WORKSPACE: return "workspace missing or too small";
    case DSPARK_ERR_UNSUPPORTED: return "arguments outside the library's supported limits";
    case DSPARK_ERR_ABI: return "struct_size does not match this library's ABI";
    case DSPARK_ERR_HIP: return "HIP runtime error or kernel launch failure";
    case DSPARK_ERR_INPUT: return "a device input check found a value outside the contract";
    default: return "unknown status";
  }
}

}  // namespace dspark

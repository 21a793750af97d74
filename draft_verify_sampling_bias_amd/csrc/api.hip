// C ABI of libdspark: host-side checks, workspace carve-up and kernel
// launches on the caller's stream.  No allocation, no synchronisation.

#include <hip/hip_runtime.h>

#include "device_info.h"
#include "dspark.h"
#include "launchers.h"
#include "plan.h"

using namespace dspark;

namespace {

inline int hip_status(hipError_t e) { return e == hipSuccess ? DSPARK_OK : DSPARK_ERR_HIP; }

template <typename T>
inline T* ws_at(void* ws, std::size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// The input-check pass of a call made with DSPARK_CHECK_INPUTS: writes the
// error word at the start of the workspace.
inline CheckParams check_params(void* ws) {
  CheckParams c{};
  c.err = ws_at<uint32_t>(ws, 0);
  return c;
}

// Schedule calls: the check of c (confidence) and of the token ids copied
// into the verify rows.
template <typename A>
int schedule_check(const A* a, hipStream_t s) {
  CheckParams c = check_params(a->workspace);
  c.ids[0] = a->anchor;
  c.n_ids[0] = a->R;
  c.ids[1] = a->y;
  c.n_ids[1] = static_cast<int64_t>(a->R) * a->gamma;
  c.V = 0x7fffffff;  // the schedule knows no vocabulary size: ids are checked for >= 0 only
  c.conf = a->c;
  c.n_conf = static_cast<int64_t>(a->R) * a->gamma;
  return hip_status(launch_input_check(c, s));
}

}  // namespace

extern "C" {

int dspark_abi_version(void) { return DSPARK_ABI_VERSION; }

const char* dspark_status_string(int status) { return status_string(status); }

int64_t dspark_schedule_rows(int32_t R, int32_t gamma, int64_t K) { return schedule_rows(R, gamma, K); }

int dspark_draft_workspace_size(const dspark_draft_args* args, size_t* bytes) {
  if (bytes == nullptr) return DSPARK_ERR_NULL;
  DraftPlan plan;
  const int st = plan_draft(args, &plan);
  if (st != DSPARK_OK) return st;
  *bytes = plan.total;
  return DSPARK_OK;
}

int dspark_verify_workspace_size(const dspark_verify_args* args, size_t* bytes) {
  if (bytes == nullptr) return DSPARK_ERR_NULL;
  VerifyPlan plan;
  const int st = plan_verify(args, &plan);
  if (st != DSPARK_OK) return st;
  *bytes = plan.total;
  return DSPARK_OK;
}

int dspark_schedule_workspace_size(const dspark_schedule_args* args, size_t* bytes) {
  return plan_schedule(args, bytes);
}

int dspark_cutoff_workspace_size(const dspark_cutoff_args* args, size_t* bytes) {
  return plan_cutoff(args, bytes);
}

int dspark_check(const void* workspace, void* stream, uint32_t* bits) {
  if (workspace == nullptr) return DSPARK_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t word = 0;
  // enqueued behind the calls that wrote the word, then waited for
  if (hipMemcpyAsync(&word, workspace, sizeof(word), hipMemcpyDeviceToHost, s) != hipSuccess) return DSPARK_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return DSPARK_ERR_HIP;
  if (bits != nullptr) *bits = word;
  return word == 0 ? DSPARK_OK : DSPARK_ERR_INPUT;
}

int dspark_draft_block(const dspark_draft_args* a) {
  DraftPlan plan;
  int st = validate_draft(a, &plan);
  if (st != DSPARK_OK || a->R == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(a->stream);

  TileParams tp{};
  tp.W1 = a->W1;
  tp.W2 = a->W2;
  tp.V = a->V;
  tp.rank = a->rank;
  tp.R = a->R;
  tp.seg_rows = plan.seg_rows;
  tp.n_seg = plan.n_seg;
  tp.temp = a->temp;
  tp.U_stride = static_cast<int64_t>(a->gamma) * a->V;
  tp.part = ws_at<float>(a->workspace, plan.part_off);
  // the fragment-packed W2 is the 16-row path's layout only
  tp.w2p = (plan.seg_rows == kSegSmall) ? static_cast<const uint16_t*>(a->W2_packed) : nullptr;

  FinishParams fp{};
  fp.part = tp.part;
  fp.seg_rows = plan.seg_rows;
  fp.n_seg = plan.n_seg;
  fp.V = a->V;
  fp.rank = a->rank;
  fp.R = a->R;
  fp.gamma = a->gamma;
  fp.W1 = a->W1;
  fp.W2 = a->W2;
  fp.U_stride = tp.U_stride;
  fp.temp = a->temp;
  fp.u_draft = a->u_draft;
  fp.y = a->y;
  fp.q_tok = a->q_tok;
  fp.q_stats = a->q_stats;

  uint32_t* err = ws_at<uint32_t>(a->workspace, 0);
  if (plan.check) {
    CheckParams c = check_params(a->workspace);
    c.ids[0] = a->anchor;
    c.n_ids[0] = a->R;
    c.V = a->V;
    c.unif[0] = a->u_draft;
    c.n_unif[0] = static_cast<int64_t>(a->R) * a->gamma;
    st = hip_status(launch_input_check(c, s));
    if (st != DSPARK_OK) return st;
  }

  // RNN head: the state of each position is computed first; the fused bias
  // kernel and the finish then read it instead of W1[prev]
  const bool rnn = a->head == DSPARK_HEAD_RNN;
  RnnStateParams rp{};
  if (rnn) {
    rp.R = a->R;
    rp.gamma = a->gamma;
    rp.V = a->V;
    rp.rank = a->rank;
    rp.act = a->act;
    rp.W1 = static_cast<const uint16_t*>(a->W1);
    rp.A = static_cast<const uint16_t*>(a->A);
    rp.anchor = a->anchor;
    rp.y = a->y;
    rp.h = a->h;
    tp.h_stride = static_cast<int64_t>(a->gamma) * a->rank;
    fp.hstate = a->h;
  }

  // the RNN head's state of position k + 1: z = A h_k by the fused bias
  // kernel of position k (as extra segments of its walk), act(z + W1[y_k])
  // by the finish of position k, when that finish can (the state kernel then
  // runs for k = 0 only)
  const bool fused = rnn && draft_finish_fuses_state(fp, a->wdtype);
  if (fused) {
    fp.A = static_cast<const uint16_t*>(a->A);
    fp.act = a->act;
    if (tp.w2p != nullptr) {
      // A in the fused kernel's fragment-packed layout, like W2
      dspark_pack_w2_args pk{};
      pk.struct_size = sizeof(pk);
      pk.W2 = a->A;
      pk.V = a->rank;
      pk.rank = a->rank;
      pk.W2_packed = ws_at<uint16_t>(a->workspace, plan.ap_off);
      pk.W2_packed_bytes = w2_packed_bytes(a->rank, a->rank);
      pk.stream = a->stream;
      st = hip_status(launch_pack_w2(pk, s));
      if (st != DSPARK_OK) return st;
      tp.ap = static_cast<const uint16_t*>(pk.W2_packed);
    }
  }
  const int cu = current_cu_count();
  for (int k = 0; k < a->gamma; ++k) {
    // prev = anchor for the first position, the token drafted just before otherwise
    tp.prev_base = (k == 0) ? a->anchor : a->y + (k - 1);
    tp.prev_stride = (k == 0) ? 1 : a->gamma;
    tp.U_base = a->U + static_cast<int64_t>(k) * a->V;
    if (rnn) {
      rp.k = k;
      if (k == 0 || !fused) {
        st = hip_status(launch_rnn_state(rp, s));
        if (st != DSPARK_OK) return st;
      }
      tp.h_base = a->h + static_cast<int64_t>(k) * a->rank;
      // fused: this position's kernel also computes A h into the next state row
      const bool next = fused && k + 1 < a->gamma;
      tp.n_seg_a = next ? (a->rank + kSegSmall - 1) / kSegSmall : 0;
      tp.A = static_cast<const uint16_t*>(a->A);
      tp.z_out = next ? a->h + static_cast<int64_t>(k + 1) * a->rank : nullptr;
    }
    hipEvent_t e0 = a->prof_events ? static_cast<hipEvent_t>(a->prof_events[2 * k]) : nullptr;
    hipEvent_t e1 = a->prof_events ? static_cast<hipEvent_t>(a->prof_events[2 * k + 1]) : nullptr;
    st = hip_status(launch_bias_tile(tp, a->wdtype, false, cu, s, e0, e1));
    if (st != DSPARK_OK) return st;
    fp.prev_base = tp.prev_base;
    fp.prev_stride = tp.prev_stride;
    fp.U_base = tp.U_base;
    fp.k = k;
    // a call without the checks still rewrites the error word (first finish)
    fp.err_clear = (k == 0 && !plan.check) ? err : nullptr;
    st = hip_status(launch_draft_finish(fp, a->wdtype, s));
    if (st != DSPARK_OK) return st;
  }
  return DSPARK_OK;
}

int dspark_schedule(const dspark_schedule_args* a) {
  int st = validate_schedule(a);
  if (st != DSPARK_OK || a->R == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(a->stream);
  if (a->flags & DSPARK_CHECK_INPUTS) {
    st = schedule_check(a, s);
    if (st != DSPARK_OK) return st;
  }
  return hip_status(launch_schedule(*a, s));
}

size_t dspark_w2_packed_bytes(int32_t V, int32_t rank) {
  if (check_dims(0, 1, V, rank, DSPARK_W_BF16) != DSPARK_OK) return 0;
  return w2_packed_bytes(V, rank);
}

int dspark_pack_w2(const dspark_pack_w2_args* a) {
  const int st = validate_pack_w2(a);
  if (st != DSPARK_OK) return st;
  return hip_status(launch_pack_w2(*a, static_cast<hipStream_t>(a->stream)));
}

int dspark_schedule_cutoff(const dspark_cutoff_args* a) {
  int st = validate_cutoff(a);
  if (st != DSPARK_OK || a->R == 0) return st;
  if (a->flags & DSPARK_CHECK_INPUTS) {
    st = schedule_check(a, static_cast<hipStream_t>(a->stream));
    if (st != DSPARK_OK) return st;
  }
  dspark_schedule_args s{};
  s.struct_size = sizeof(s);
  s.R = a->R;
  s.gamma = a->gamma;
  s.K = 0;  // not read by the cutoff
  s.c = a->c;
  s.anchor = a->anchor;
  s.y = a->y;
  s.a = a->a;
  s.l = a->l;
  s.row_offsets = a->row_offsets;
  s.row_req = a->row_req;
  s.row_pos = a->row_pos;
  s.row_tok = a->row_tok;
  s.expected_tokens = a->expected_tokens;
  s.stream = a->stream;
  return hip_status(launch_schedule_cutoff(s, a->conf_min, static_cast<hipStream_t>(a->stream)));
}

int dspark_capacity(const dspark_capacity_args* a) {
  const int st = validate_capacity(a);
  if (st != DSPARK_OK) return st;
  return hip_status(launch_capacity(*a, static_cast<hipStream_t>(a->stream)));
}

int dspark_sts_fit(const dspark_sts_fit_args* a) {
  const int st = validate_sts_fit(a);
  if (st != DSPARK_OK) return st;
  return hip_status(launch_sts_fit(*a, static_cast<hipStream_t>(a->stream)));
}

int dspark_sts_apply(const dspark_sts_apply_args* a) {
  const int st = validate_sts_apply(a);
  if (st != DSPARK_OK || a->R == 0) return st;
  return hip_status(launch_sts_apply(*a, static_cast<hipStream_t>(a->stream)));
}

int dspark_verify(const dspark_verify_args* a) {
  VerifyPlan plan;
  int st = validate_verify(a, &plan);
  if (st != DSPARK_OK || a->R == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(a->stream);

  VerifyParams vp{};
  vp.R = a->R;
  vp.gamma = a->gamma;
  vp.V = a->V;
  vp.rank = a->rank;
  vp.n_chunks = plan.n_chunks;
  vp.seg_rows = plan.seg_rows;
  vp.n_seg = plan.n_seg;
  vp.n_rows = a->n_rows;
  vp.target = a->target;
  vp.row_offsets = a->row_offsets;
  vp.U = a->U;
  vp.W1 = a->W1;
  vp.W2 = a->W2;
  vp.anchor = a->anchor;
  vp.temp = a->temp;
  vp.y = a->y;
  vp.q_tok = a->q_tok;
  vp.q_stats = a->q_stats;
  vp.u_accept = a->u_accept;
  vp.u_final = a->u_final;
  vp.n_accept = a->n_accept;
  vp.out_tok = a->out_tok;
  vp.p_tok = a->p_tok;
  vp.vpart = ws_at<float>(a->workspace, plan.vpart_off);
  vp.rs_info = ws_at<int32_t>(a->workspace, plan.rsinfo_off);
  vp.rs_stats = ws_at<float>(a->workspace, plan.rsstats_off);
  vp.rpart = ws_at<float>(a->workspace, plan.rpart_off);
  if (a->head == DSPARK_HEAD_RNN) vp.hstate = a->h;
  if (plan.seg_rows == kSegWide) {
    vp.rs_count = ws_at<int32_t>(a->workspace, plan.rcount_off);
    vp.rs_list = ws_at<ResidualEntry>(a->workspace, plan.rlist_off);
  }
  if (plan.check) {
    CheckParams c = check_params(a->workspace);
    c.ids[0] = a->anchor;
    c.n_ids[0] = a->R;
    c.ids[1] = a->y;
    c.n_ids[1] = static_cast<int64_t>(a->R) * a->gamma;
    c.V = a->V;
    c.unif[0] = a->u_accept;
    c.n_unif[0] = static_cast<int64_t>(a->R) * a->gamma;
    c.unif[1] = a->u_final;
    c.n_unif[1] = a->R;
    c.offsets = a->row_offsets;
    c.R = a->R;
    c.gamma = a->gamma;
    c.n_rows = a->n_rows;
    st = hip_status(launch_input_check(c, s));
    if (st != DSPARK_OK) return st;
  } else {
    vp.err_clear = ws_at<uint32_t>(a->workspace, 0);
  }

  st = hip_status(launch_verify_stats(vp, s));
  if (st != DSPARK_OK) return st;
  st = hip_status(launch_verify_finish(vp, s));
  if (st != DSPARK_OK) return st;

  // residual pass: rebuild q for the rejected position and sum max(0, p - q)
  TileParams tp{};
  tp.W1 = a->W1;
  tp.W2 = a->W2;
  tp.V = a->V;
  tp.rank = a->rank;
  tp.R = a->R;
  tp.seg_rows = plan.seg_rows;
  tp.n_seg = plan.n_seg;
  tp.temp = a->temp;
  tp.rs_info = vp.rs_info;
  tp.rs_stats = vp.rs_stats;
  tp.rs_count = vp.rs_count;
  tp.rs_list = vp.rs_list;
  tp.U = a->U;
  tp.target = a->target;
  tp.u_rows = static_cast<int64_t>(a->R) * a->gamma;
  tp.t_rows = a->n_rows;
  tp.part = vp.rpart;
  tp.w2p = (plan.seg_rows == kSegSmall) ? static_cast<const uint16_t*>(a->W2_packed) : nullptr;
  tp.h_base = vp.hstate;  // residual mode: row urow of the states
  st = hip_status(launch_bias_tile(tp, a->wdtype, true, current_cu_count(), s));
  if (st != DSPARK_OK) return st;
  return hip_status(launch_residual_finish(vp, a->wdtype, s));
}

}  // extern "C"

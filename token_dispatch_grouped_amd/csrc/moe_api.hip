// C ABI of the MoE expert-layer forward: host-side validation, then launches.
// Every check runs before anything is enqueued, so an invalid call touches no
// output ("Paralelismo de especialistas", section "Sobrescrevendo os planos":
// errors are raised before anything is sharded).
#include <limits.h>

#include "moe_internal.h"

namespace {

using moe::kMaxExperts;

moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// Shape checks shared by the layer steps. `need_dims` adds d/d_ff/local-range checks.
moe_status check_shape(const moe_shape* s, bool need_dims) {
  if (s == nullptr) return MOE_EINVAL;
  if (s->T < 0 || s->E < 1 || s->k < 1 || s->k > s->E) return MOE_EINVAL;
  if (s->T * static_cast<int64_t>(s->k) > INT32_MAX) return MOE_EINVAL;
  if (s->E > kMaxExperts) return MOE_EUNSUPPORTED;
  if (need_dims) {
    if (s->d <= 0 || s->d_ff <= 0 || s->d % 8 != 0 || s->d_ff % 8 != 0) return MOE_EINVAL;
    if (s->e_begin < 0 || s->e_end > s->E || s->e_begin >= s->e_end) return MOE_EINVAL;
  }
  return MOE_OK;
}

bool valid_dtype(moe_dtype dt) { return dt == MOE_F32 || dt == MOE_BF16; }

size_t elem_bytes(moe_dtype dt) { return dt == MOE_BF16 ? 2 : 4; }

int64_t n_max_of(const moe_shape* s) {
  const int64_t e_loc = s->e_end - s->e_begin;
  return s->T * (s->k < e_loc ? s->k : e_loc);
}

constexpr size_t kWsAlign = 256;
size_t align_up(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }
// workspace of moe_grouped_gemm_backward: x_perm [N_max, d], gu and d_gu [N_max, 2 d_ff], and dY in
// 32-column blocks [N_max, d]
size_t backward_ws(const moe_shape* s, size_t* off_gu, size_t* off_dgu, size_t* off_dyb = nullptr) {
  const size_t n = static_cast<size_t>(n_max_of(s));
  const size_t xp = align_up(n * static_cast<size_t>(s->d) * 2);
  const size_t g = align_up(n * static_cast<size_t>(s->d_ff) * 2 * 2);
  if (off_gu) *off_gu = xp;
  if (off_dgu) *off_dgu = xp + g;
  if (off_dyb) *off_dyb = xp + 2 * g;
  return 2 * xp + 2 * g;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: unsupported shape";
    case MOE_EHIP: return "MOE_EHIP: HIP launch failed";
  }
  return "unknown moe_status";
}

moe_status moe_expert_range(int32_t E, int32_t ep, int32_t rank, int32_t* e_begin, int32_t* e_end) {
  if (e_begin == nullptr || e_end == nullptr) return MOE_EINVAL;
  if (E < 1 || ep < 1 || E % ep != 0 || rank < 0) return MOE_EINVAL;
  const int32_t per = E / ep;
  const int32_t r = rank % ep;
  *e_begin = r * per;
  *e_end = (r + 1) * per;
  return MOE_OK;
}

moe_status moe_route_topk(const moe_shape* s, const float* logits, int32_t* topk_idx, float* topk_w,
                          hipStream_t stream) {
  const moe_status st = check_shape(s, false);
  if (st != MOE_OK) return st;
  if (s->T == 0) return MOE_OK;
  if (logits == nullptr || topk_idx == nullptr || topk_w == nullptr) return MOE_EINVAL;
  if (s->T * static_cast<int64_t>(s->E) > (int64_t{1} << 40)) return MOE_EUNSUPPORTED;
  return from_hip(moe::launch_route_topk(logits, topk_idx, topk_w, s->T, s->E, s->k, stream));
}

size_t moe_dispatch_workspace_bytes(const moe_shape* s) {
  if (check_shape(s, false) != MOE_OK) return 0;
  return moe::dispatch_workspace_bytes(s->T, s->k, s->E);
}

moe_status moe_dispatch(const moe_shape* s, moe_dtype dt, const void* x, const int32_t* topk_idx,
                        int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pair_pos,
                        void* x_perm, void* workspace, hipStream_t stream) {
  const moe_status st = check_shape(s, true);
  if (st != MOE_OK) return st;
  if (!valid_dtype(dt)) return MOE_EINVAL;
  if (counts == nullptr || offsets == nullptr) return MOE_EINVAL;
  if (s->T > 0 && (x == nullptr || topk_idx == nullptr || perm == nullptr || pair_pos == nullptr ||
                   x_perm == nullptr))
    return MOE_EINVAL;
  if (moe::dispatch_workspace_bytes(s->T, s->k, s->E) > 0 && workspace == nullptr) return MOE_EINVAL;
  return from_hip(moe::launch_dispatch(x, static_cast<size_t>(s->d) * elem_bytes(dt), topk_idx, counts,
                                       offsets, perm, pair_pos, x_perm, workspace, s->T, s->k, s->E,
                                       s->e_begin, s->e_end, n_max_of(s), stream));
}

moe_status moe_dispatch_indices(const moe_shape* s, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                                int32_t* perm, int32_t* pair_pos, void* workspace, hipStream_t stream) {
  const moe_status st = check_shape(s, true);
  if (st != MOE_OK) return st;
  if (counts == nullptr || offsets == nullptr) return MOE_EINVAL;
  if (s->T > 0 && (topk_idx == nullptr || perm == nullptr || pair_pos == nullptr)) return MOE_EINVAL;
  if (moe::dispatch_workspace_bytes(s->T, s->k, s->E) > 0 && workspace == nullptr) return MOE_EINVAL;
  return from_hip(moe::launch_dispatch(nullptr, 0, topk_idx, counts, offsets, perm, pair_pos, nullptr, workspace,
                                       s->T, s->k, s->E, s->e_begin, s->e_end, n_max_of(s), stream));
}

size_t moe_dispatch_debug_word_offset(void) { return moe::dispatch_debug_word_offset(); }

moe_status moe_dispatch_indices_noalloc(const moe_shape* s, const int32_t* topk_idx, int32_t* counts,
                                        int32_t* offsets, int32_t* perm, int32_t* pair_pos, hipStream_t stream) {
  const moe_status st = check_shape(s, true);
  if (st != MOE_OK) return st;
  if (counts == nullptr || offsets == nullptr) return MOE_EINVAL;
  if (s->T > 0 && (topk_idx == nullptr || perm == nullptr || pair_pos == nullptr)) return MOE_EINVAL;
  if (moe::dispatch_workspace_bytes(s->T, s->k, s->E) > moe::kDispatchScratchBytes) return MOE_EUNSUPPORTED;
  void* ws = nullptr;
  if (moe::dispatch_scratch(&ws) != hipSuccess) return MOE_EHIP;
  return from_hip(moe::launch_dispatch(nullptr, 0, topk_idx, counts, offsets, perm, pair_pos, nullptr, ws, s->T,
                                       s->k, s->E, s->e_begin, s->e_end, n_max_of(s), stream));
}

size_t moe_grouped_gemm_workspace_bytes(const moe_shape* s, moe_dtype dt) {
  // the gathered rows' blocked copy of moe_grouped_gemm_gather(_save), when it pays
  if (s == nullptr || dt != MOE_BF16 || s->e_end <= s->e_begin) return 0;
  const int64_t n_max = n_max_of(s);
  if (!moe::grouped_gemm_blocked_rows(n_max, s->e_end - s->e_begin, s->d, s->d_ff)) return 0;
  return moe::blocked_rows_workspace_bytes(n_max, s->d);
}

moe_status moe_grouped_gemm(const moe_shape* s, moe_dtype dt, const void* x_perm,
                            const int32_t* offsets, const void* w_gate_up, const void* w_down, void* h,
                            void* y, void* workspace, hipStream_t stream) {
  (void)workspace;
  const moe_status st = check_shape(s, true);
  if (st != MOE_OK) return st;
  if (!valid_dtype(dt)) return MOE_EINVAL;
  if (s->T == 0) return MOE_OK;
  if (x_perm == nullptr || offsets == nullptr || w_gate_up == nullptr || w_down == nullptr ||
      h == nullptr || y == nullptr)
    return MOE_EINVAL;
  const int e_loc = s->e_end - s->e_begin;
  const int64_t n_max = n_max_of(s);
  // Per-expert weights are addressed through 32-bit buffer offsets (with one
  // K step of slack for the tail); larger experts are not supported.
  const int64_t eb = static_cast<int64_t>(elem_bytes(dt));
  if ((static_cast<int64_t>(s->d) + 64) * 2 * s->d_ff * eb > INT32_MAX ||
      (static_cast<int64_t>(s->d_ff) + 64) * s->d * eb > INT32_MAX)
    return MOE_EUNSUPPORTED;
  if (dt == MOE_BF16)
    return from_hip(moe::launch_grouped_gemm_bf16(x_perm, offsets, w_gate_up, w_down, h, y, s->d,
                                                  s->d_ff, s->e_begin, e_loc, n_max, s->T, s->k,
                                                  s->E, stream));
  return from_hip(moe::launch_grouped_gemm_f32(
      static_cast<const float*>(x_perm), offsets, static_cast<const float*>(w_gate_up),
      static_cast<const float*>(w_down), static_cast<float*>(h), static_cast<float*>(y), s->d, s->d_ff,
      s->e_begin, e_loc, n_max, stream));
}

}  // extern "C"

namespace {

// moe_grouped_gemm_gather, and with gu != nullptr moe_grouped_gemm_gather_save
moe_status gemm_gather(const moe_shape* s, moe_dtype dt, const void* x, const int32_t* perm, const int32_t* offsets,
                       const void* w_gate_up, const void* w_down, void* h, void* y, void* gu, void* workspace,
                       hipStream_t stream) {
  const moe_status st = check_shape(s, true);
  if (st != MOE_OK) return st;
  if (!valid_dtype(dt)) return MOE_EINVAL;
  if (s->T == 0) return MOE_OK;
  if (x == nullptr || perm == nullptr || offsets == nullptr || w_gate_up == nullptr || w_down == nullptr ||
      h == nullptr || y == nullptr)
    return MOE_EINVAL;
  // Only the pipelined bf16 kernel gathers rows in its loads: K in whole 32-wide
  // stages, and x addressed through 32-bit buffer offsets.
  if (dt != MOE_BF16 || s->d % 32 != 0 || s->d_ff % 32 != 0) return MOE_EUNSUPPORTED;
  if (s->T * static_cast<int64_t>(s->d) * 2 + 64 > INT32_MAX) return MOE_EUNSUPPORTED;
  if ((static_cast<int64_t>(s->d) + 64) * 2 * s->d_ff * 2 > INT32_MAX ||
      (static_cast<int64_t>(s->d_ff) + 64) * s->d * 2 > INT32_MAX)
    return MOE_EUNSUPPORTED;
  // the blocked copy of the gathered rows, when the workspace is there for it
  void* a_blk = moe_grouped_gemm_workspace_bytes(s, dt) > 0 ? workspace : nullptr;
  return from_hip(moe::launch_grouped_gemm_gather(x, perm, offsets, w_gate_up, w_down, h, y, gu, s->d, s->d_ff,
                                                  s->e_begin, s->e_end - s->e_begin, n_max_of(s), s->T, s->k,
                                                  a_blk, stream));
}

}  // namespace

extern "C" {

moe_status moe_grouped_gemm_gather(const moe_shape* s, moe_dtype dt, const void* x, const int32_t* perm,
                                   const int32_t* offsets, const void* w_gate_up, const void* w_down, void* h,
                                   void* y, void* workspace, hipStream_t stream) {
  return gemm_gather(s, dt, x, perm, offsets, w_gate_up, w_down, h, y, nullptr, workspace, stream);
}

moe_status moe_grouped_gemm_gather_save(const moe_shape* s, moe_dtype dt, const void* x, const int32_t* perm,
                                        const int32_t* offsets, const void* w_gate_up, const void* w_down, void* h,
                                        void* y, void* gu, void* workspace, hipStream_t stream) {
  if (s != nullptr && s->T > 0 && gu == nullptr) return MOE_EINVAL;
  return gemm_gather(s, dt, x, perm, offsets, w_gate_up, w_down, h, y, gu, workspace, stream);
}

moe_status moe_combine(const moe_shape* s, moe_dtype dt, const void* y, const int32_t* pair_pos,
                       const float* topk_w, void* out, hipStream_t stream) {
  const moe_status st = check_shape(s, true);
  if (st != MOE_OK) return st;
  if (!valid_dtype(dt)) return MOE_EINVAL;
  if (s->T == 0) return MOE_OK;
  if (y == nullptr || pair_pos == nullptr || topk_w == nullptr || out == nullptr) return MOE_EINVAL;
  return from_hip(moe::launch_combine(y, pair_pos, topk_w, out, s->T, s->k, s->d, n_max_of(s),
                                      dt == MOE_BF16, stream));
}

// ------------------------------------------------------------------ backward

moe_status moe_combine_backward(const moe_shape* s, moe_dtype dt, const void* d_out, const void* y,
                                const int32_t* pair_pos, const float* topk_w, void* d_y, float* d_topk_w,
                                hipStream_t stream) {
  const moe_status st = check_shape(s, true);
  if (st != MOE_OK) return st;
  if (!valid_dtype(dt)) return MOE_EINVAL;
  if (s->T == 0) return MOE_OK;
  if (d_out == nullptr || y == nullptr || pair_pos == nullptr || topk_w == nullptr || d_y == nullptr ||
      d_topk_w == nullptr)
    return MOE_EINVAL;
  return from_hip(moe::launch_combine_backward(d_out, y, pair_pos, topk_w, d_y, d_topk_w, s->T, s->k, s->d,
                                               n_max_of(s), dt == MOE_BF16, stream));
}

size_t moe_grouped_gemm_backward_workspace_bytes(const moe_shape* s, moe_dtype dt) {
  if (check_shape(s, true) != MOE_OK || dt != MOE_BF16) return 0;
  return backward_ws(s, nullptr, nullptr);
}

}  // extern "C"

namespace {

// moe_grouped_gemm_backward (saved == nullptr: [G | U] recomputed into the
// workspace) and moe_grouped_gemm_backward_saved ([G | U] read from saved)
moe_status gemm_backward(const moe_shape* s, moe_dtype dt, const void* x, const int32_t* perm,
                         const int32_t* offsets, const void* w_gate_up, const void* w_down, const void* h,
                         const void* saved, const void* d_y, void* d_x_perm, void* d_w_gate_up, void* d_w_down,
                         void* workspace, hipStream_t stream) {
  const moe_status st = check_shape(s, true);
  if (st != MOE_OK) return st;
  if (!valid_dtype(dt)) return MOE_EINVAL;
  if (offsets == nullptr || w_gate_up == nullptr || w_down == nullptr || d_w_gate_up == nullptr ||
      d_w_down == nullptr)
    return MOE_EINVAL;
  // with no tokens only the (zero) weight gradients are written
  if (s->T > 0 && (x == nullptr || perm == nullptr || h == nullptr || d_y == nullptr || d_x_perm == nullptr ||
                   workspace == nullptr))
    return MOE_EINVAL;
  // the pipelined bf16 kernels only: K in whole 32-wide stages
  if (dt != MOE_BF16 || s->d % 32 != 0 || s->d_ff % 32 != 0) return MOE_EUNSUPPORTED;
  const int64_t n_max = n_max_of(s);
  // 32-bit buffer offsets: the widest activation block of an expert, x, and a weight matrix
  const int64_t widest = s->d > 2 * static_cast<int64_t>(s->d_ff) ? s->d : 2 * static_cast<int64_t>(s->d_ff);
  if (n_max * 2 * widest + 64 > INT32_MAX || s->T * static_cast<int64_t>(s->d) * 2 + 64 > INT32_MAX ||
      (static_cast<int64_t>(s->d) + 64) * 2 * s->d_ff * 2 > INT32_MAX ||
      (static_cast<int64_t>(s->d_ff) + 64) * s->d * 2 > INT32_MAX)
    return MOE_EUNSUPPORTED;
  const int e_loc = s->e_end - s->e_begin;
  const int d = s->d, d_ff = s->d_ff;
  size_t off_gu = 0, off_dgu = 0, off_dyb = 0;
  backward_ws(s, &off_gu, &off_dgu, &off_dyb);
  char* ws = static_cast<char*>(workspace);
  void* x_perm = ws;
  const void* gu = saved != nullptr ? saved : static_cast<const void*>(ws + off_gu);
  void* d_gu = ws + off_dgu;
  void* d_y_blk = ws + off_dyb;
  hipError_t e = hipSuccess;
  if (n_max > 0) {
    // the rows of the local pairs, then (unless the forward kept them) their gate/up pre-activations
    e = moe::launch_gather_rows(x, static_cast<size_t>(d) * 2, perm, offsets, x_perm, s->k, s->e_begin, s->e_end,
                                n_max, stream);
    if (e == hipSuccess && saved == nullptr)
      e = moe::launch_grouped_gemm_plain(x_perm, w_gate_up, ws + off_gu, offsets, s->e_begin, e_loc, d, 2 * d_ff,
                                         2 * d_ff, n_max,
                                         moe::grouped_gemm_grid(n_max, e_loc, (2 * d_ff + 255) / 256), stream);
    // [dG | dU] from dH = dY @ W_dn^T and [G | U]; dY read, and [dG | dU] written, in 32-column
    // blocks of N_max rows (the layout the products read fastest)
    if (e == hipSuccess) e = moe::launch_to_blocked(d_y, d_y_blk, offsets, s->e_begin, s->e_end, d, n_max, stream);
    if (e == hipSuccess)
      e = moe::launch_grouped_gemm_nt(d_y_blk, w_down, d_gu, gu, offsets, s->e_begin, e_loc, d, d_ff, 2 * d_ff,
                                      n_max, true, moe::grouped_gemm_grid(n_max, e_loc, (d_ff + 255) / 256), stream);
    // dX_perm = [dG | dU] @ W_gu^T
    if (e == hipSuccess)
      e = moe::launch_grouped_gemm_nt(d_gu, w_gate_up, d_x_perm, nullptr, offsets, s->e_begin, e_loc, 2 * d_ff, d,
                                      d, n_max, false, moe::grouped_gemm_grid(n_max, e_loc, (d + 255) / 256), stream);
  }
  // weight gradients over each expert's rows (an expert without rows gets zeros)
  const int cus = moe::device_cu_count();
  auto tn_grid = [&](int M, int N) {
    const int64_t tiles = static_cast<int64_t>(e_loc) * ((M + 255) / 256) * ((N + 255) / 256);
    int64_t g = tiles < cus ? tiles : cus;
    if (g > 8) g &= ~int64_t{7};
    return static_cast<int>(g < 1 ? 1 : g);
  };
  if (e == hipSuccess)
    e = moe::launch_grouped_gemm_tn(h, d_y, d_w_down, offsets, s->e_begin, e_loc, d_ff, d, n_max, false,
                                    tn_grid(d_ff, d), stream);
  if (e == hipSuccess)
    e = moe::launch_grouped_gemm_tn(x_perm, d_gu, d_w_gate_up, offsets, s->e_begin, e_loc, d, 2 * d_ff, n_max, true,
                                    tn_grid(d, 2 * d_ff), stream);
  return from_hip(e);
}

}  // namespace

extern "C" {

moe_status moe_grouped_gemm_backward(const moe_shape* s, moe_dtype dt, const void* x, const int32_t* perm,
                                     const int32_t* offsets, const void* w_gate_up, const void* w_down,
                                     const void* h, const void* d_y, void* d_x_perm, void* d_w_gate_up,
                                     void* d_w_down, void* workspace, hipStream_t stream) {
  return gemm_backward(s, dt, x, perm, offsets, w_gate_up, w_down, h, nullptr, d_y, d_x_perm, d_w_gate_up, d_w_down,
                       workspace, stream);
}

moe_status moe_grouped_gemm_backward_saved(const moe_shape* s, moe_dtype dt, const void* x, const int32_t* perm,
                                           const int32_t* offsets, const void* w_gate_up, const void* w_down,
                                           const void* h, const void* gu, const void* d_y, void* d_x_perm,
                                           void* d_w_gate_up, void* d_w_down, void* workspace, hipStream_t stream) {
  if (s != nullptr && s->T > 0 && gu == nullptr) return MOE_EINVAL;
  return gemm_backward(s, dt, x, perm, offsets, w_gate_up, w_down, h, gu, d_y, d_x_perm, d_w_gate_up, d_w_down,
                       workspace, stream);
}

moe_status moe_dispatch_backward(const moe_shape* s, moe_dtype dt, const void* d_x_perm, const int32_t* pair_pos,
                                 void* d_x, hipStream_t stream) {
  const moe_status st = check_shape(s, true);
  if (st != MOE_OK) return st;
  if (!valid_dtype(dt)) return MOE_EINVAL;
  if (s->T == 0) return MOE_OK;
  if (d_x_perm == nullptr || pair_pos == nullptr || d_x == nullptr) return MOE_EINVAL;
  return from_hip(moe::launch_combine(d_x_perm, pair_pos, nullptr, d_x, s->T, s->k, s->d, n_max_of(s),
                                     dt == MOE_BF16, stream));
}

moe_status moe_route_topk_backward(const moe_shape* s, const int32_t* topk_idx, const float* topk_w,
                                   const float* d_topk_w, float* d_logits, hipStream_t stream) {
  const moe_status st = check_shape(s, false);
  if (st != MOE_OK) return st;
  if (s->T == 0) return MOE_OK;
  if (topk_idx == nullptr || topk_w == nullptr || d_topk_w == nullptr || d_logits == nullptr) return MOE_EINVAL;
  if (s->T * static_cast<int64_t>(s->E) > (int64_t{1} << 40)) return MOE_EUNSUPPORTED;
  return from_hip(moe::launch_route_topk_backward(topk_idx, topk_w, d_topk_w, d_logits, s->T, s->E, s->k, stream));
}

}  // extern "C"

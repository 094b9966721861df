// C ABI of the library (declared in include/qgemm.h). Every entry point
// checks its arguments on the host, before any HIP call, and only then
// enqueues work on the caller's stream. Nothing here allocates device memory.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <cmath>

#include "qg_internal.h"
#include "qgemm.h"

namespace {

constexpr int64_t kMaxKN = int64_t(1) << 20;
constexpr int64_t kMaxM = int64_t(1) << 24;
constexpr int64_t kMaxElems = int64_t(1) << 31;
constexpr int64_t kSmallMaxM = 16;   // above this, the library's own plan is the prefill kernel

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

qg_status check_kn(int64_t K, int64_t N) {
  if (K <= 0 || N <= 0 || K % 128 != 0 || N % 16 != 0) return QG_ERR_SHAPE;
  if (K > kMaxKN || N > kMaxKN || K * N >= kMaxElems) return QG_ERR_SHAPE;
  return QG_OK;
}

qg_status check_mkn(int64_t M, int64_t K, int64_t N) {
  const qg_status s = check_kn(K, N);
  if (s != QG_OK) return s;
  if (M < 0 || M > kMaxM || M * K >= kMaxElems || M * N >= kMaxElems) return QG_ERR_SHAPE;
  return QG_OK;
}

// NULL first, then alignment, over a list of pointers.
qg_status check_ptrs(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (p == nullptr) return QG_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return QG_ERR_ALIGN;
  return QG_OK;
}

qg_status from_hip(hipError_t e) { return e == hipSuccess ? QG_OK : QG_ERR_HIP; }

bool s_bf16(qg_dtype d) { return d == QG_BF16 || d == QG_BF16_CBM; }
// Scale dtypes the GEMM entry points take: logical or column-block-major.
bool gemm_scale_dtype(qg_dtype d) {
  return d == QG_F16 || d == QG_BF16 || d == QG_F16_CBM || d == QG_BF16_CBM;
}
bool s_cbm(qg_dtype d) { return d == QG_F16_CBM || d == QG_BF16_CBM; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

qg_status rtn_scales(int bits, const void* W, qg_dtype w_dt, int64_t K, int64_t N, void* scales,
                     void* stream) {
  qg_status s = check_kn(K, N);
  if (s != QG_OK) return s;
  if (w_dt != QG_F32 && w_dt != QG_BF16) return QG_ERR_DTYPE;
  if ((s = check_ptrs({W, scales})) != QG_OK) return s;
  return from_hip(qg::launch_rtn_scales(bits, W, w_dt == QG_BF16, K, N, scales, as_stream(stream)));
}

qg_status pack_to_grid(int bits, const void* W, qg_dtype w_dt, const void* scales, qg_dtype s_dt,
                       int64_t K, int64_t N, void* packed, void* stream) {
  qg_status s = check_kn(K, N);
  if (s != QG_OK) return s;
  if (w_dt != QG_F32 && w_dt != QG_BF16) return QG_ERR_DTYPE;
  if (s_dt != QG_F16 && s_dt != QG_BF16) return QG_ERR_DTYPE;
  if ((s = check_ptrs({W, scales, packed})) != QG_OK) return s;
  return from_hip(qg::launch_pack_to_grid(bits, W, w_dt == QG_BF16, scales, s_dt == QG_BF16, K, N,
                                          packed, as_stream(stream)));
}

qg_status prepack(int bits, const int8_t* codes, int64_t K, int64_t N, void* packed, void* stream) {
  qg_status s = check_kn(K, N);
  if (s != QG_OK) return s;
  if ((s = check_ptrs({codes, packed})) != QG_OK) return s;
  return from_hip(qg::launch_prepack(bits, codes, K, N, packed, as_stream(stream)));
}

qg_status unpack(int bits, const void* packed, int64_t K, int64_t N, int8_t* codes, void* stream) {
  qg_status s = check_kn(K, N);
  if (s != QG_OK) return s;
  if ((s = check_ptrs({packed, codes})) != QG_OK) return s;
  return from_hip(qg::launch_unpack(bits, packed, K, N, codes, as_stream(stream)));
}

// The GEMM's argument checks other than the workspace (shape, scale dtype,
// pointers), in the order the entry points report them.
qg_status gemm_check(const void* x, const void* packed, const void* scales, qg_dtype s_dt,
                     const void* out, int64_t M, int64_t K, int64_t N) {
  qg_status s = check_mkn(M, K, N);
  if (s != QG_OK) return s;
  if (!gemm_scale_dtype(s_dt)) return QG_ERR_DTYPE;
  if ((s = check_ptrs({packed, scales})) != QG_OK) return s;
  if (M == 0) return QG_OK;
  return check_ptrs({x, out});
}

qg_status gemm(int bits, bool x_f16, const void* x, const void* packed, const void* scales,
               qg_dtype s_dt, void* out, int64_t M, int64_t K, int64_t N, void* ws,
               size_t ws_bytes, int nbw, int wk, int splits, void* stream) {
  qg_status s = gemm_check(x, packed, scales, s_dt, out, M, K, N);
  if (s != QG_OK || M == 0) return s;
  const bool explicit_plan = (nbw != 0 || wk != 0 || splits != 0);
  if (!explicit_plan && (M == 1 || qg::gemv_rows_fits(M, K, N))) {   // GEMV: no workspace
    qg::GroupArgs g;
    g.count = 1;
    g.item[0].n = (int)N;
    g.item[0].packed = static_cast<const char*>(packed);
    g.item[0].scales = static_cast<const uint16_t*>(scales);
    g.item[0].out = static_cast<uint16_t*>(out);
    qg::gemv_group(&g);
    return from_hip(qg::launch_gemv(bits, x, x_f16, g, s_bf16(s_dt), s_cbm(s_dt), M, K,
                                    as_stream(stream)));
  }
  if (M > kSmallMaxM && !explicit_plan) {
    qg::PrefillPlan pp;
    if (!qg::make_prefill_plan(M, K, N, &pp)) return QG_ERR_SHAPE;
    const size_t need = qg::prefill_workspace(bits, pp, K);
    if (need > 0) {
      if (ws == nullptr || ws_bytes < need) return QG_ERR_WORKSPACE;
      if (!aligned16(ws)) return QG_ERR_ALIGN;
    }
    return from_hip(qg::launch_gemm_prefill(bits, pp, x, x_f16, packed, scales, s_bf16(s_dt),
                                            s_cbm(s_dt), out,
                                            M, K, N, ws, as_stream(stream)));
  }
  qg::SmallPlan plan;
  if (!qg::make_small_plan(bits, M, K, N, nbw, wk, splits, &plan)) return QG_ERR_PLAN;
  const size_t need = qg::small_plan_workspace(plan, M, N);
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need) return QG_ERR_WORKSPACE;
    if (!aligned16(ws)) return QG_ERR_ALIGN;
  }
  qg::GroupArgs g;
  g.count = 1;
  g.item[0].n = (int)N;
  g.item[0].packed = static_cast<const char*>(packed);
  g.item[0].scales = static_cast<const uint16_t*>(scales);
  g.item[0].out = static_cast<uint16_t*>(out);
  qg::small_plan_group(plan, &g);
  return from_hip(qg::launch_gemm_small(bits, plan, x, x_f16, g, s_bf16(s_dt), s_cbm(s_dt), M, K, ws,
                                        as_stream(stream)));
}

// Grouped GEMMs sharing x, M and K: checks every item, then one launch of the
// small-M kernel over all of them (M <= 16), or one prefill launch per item.
constexpr int64_t kMaxCounters = 65536 / 4;   // 32-bit arrival counters at the workspace start

qg_status grouped_plan(int bits, int64_t M, int64_t K, const qg_group_item* items, int count,
                       qg::SmallPlan* plan, qg::GroupArgs* g) {
  if (items == nullptr) return QG_ERR_NULL;
  if (count < 1 || count > qg::GroupArgs::kMax) return QG_ERR_SHAPE;
  int64_t ntot = 0;
  for (int i = 0; i < count; ++i) {
    const qg_status s = check_mkn(M, K, items[i].N);
    if (s != QG_OK) return s;
    ntot += items[i].N;
  }
  qg_status s = check_mkn(M, K, ntot);
  if (s != QG_OK) return s;
  if (M > kSmallMaxM) return QG_OK;
  if (M == 0) return QG_OK;
  if (M == 1 || qg::gemv_rows_fits(M, K, ntot)) {   // GEMV: one workgroup per column block
    g->count = count;
    for (int i = 0; i < count; ++i) {
      g->item[i].n = (int)items[i].N;
      g->item[i].packed = static_cast<const char*>(items[i].packed_w);
      g->item[i].scales = static_cast<const uint16_t*>(items[i].scales);
      g->item[i].out = static_cast<uint16_t*>(items[i].out);
    }
    qg::gemv_group(g);
    return QG_OK;
  }
  if (!qg::make_small_plan(bits, M, K, ntot, 0, 0, 0, plan)) return QG_ERR_SHAPE;
  g->count = count;
  for (int i = 0; i < count; ++i) {
    g->item[i].n = (int)items[i].N;
    g->item[i].packed = static_cast<const char*>(items[i].packed_w);
    g->item[i].scales = static_cast<const uint16_t*>(items[i].scales);
    g->item[i].out = static_cast<uint16_t*>(items[i].out);
  }
  qg::small_plan_group(*plan, g);
  if (plan->splits > 1 && (int64_t)g->wg_total * plan->row_blocks > kMaxCounters)
    return QG_ERR_SHAPE;
  if (!qg::small_plan_partials_fit(*plan, g->n_total)) return QG_ERR_SHAPE;
  return QG_OK;
}

size_t grouped_workspace(int bits, int64_t M, int64_t K, const qg_group_item* items, int count) {
  if (bits != 4 && bits != 8) return 0;
  qg::SmallPlan plan;
  qg::GroupArgs g;
  if (grouped_plan(bits, M, K, items, count, &plan, &g) != QG_OK || M == 0) return 0;
  if (M == 1 || qg::gemv_rows_fits(M, K, g.n_total)) return 0;
  if (M > kSmallMaxM) {
    qg::PrefillPlan pp;
    if (!qg::make_prefill_plan(M, K, items[0].N, &pp)) return 0;
    return qg::prefill_workspace(bits, pp, K);   // depends on M and K only
  }
  return qg::small_plan_workspace(plan, M, g.n_total);
}

qg_status gemm_grouped(int bits, bool x_f16, const void* x, const qg_group_item* items, int count,
                       qg_dtype s_dt, int64_t M, int64_t K, void* ws, size_t ws_bytes,
                       void* stream) {
  if (!gemm_scale_dtype(s_dt)) return QG_ERR_DTYPE;
  qg::SmallPlan plan;
  qg::GroupArgs g;
  qg_status s = grouped_plan(bits, M, K, items, count, &plan, &g);
  if (s != QG_OK) return s;
  for (int i = 0; i < count; ++i)
    if ((s = check_ptrs({items[i].packed_w, items[i].scales})) != QG_OK) return s;
  if (M == 0) return QG_OK;
  if ((s = check_ptrs({x})) != QG_OK) return s;
  for (int i = 0; i < count; ++i)
    if ((s = check_ptrs({items[i].out})) != QG_OK) return s;
  const size_t need = grouped_workspace(bits, M, K, items, count);
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need) return QG_ERR_WORKSPACE;
    if (!aligned16(ws)) return QG_ERR_ALIGN;
  }
  if (M > kSmallMaxM) {
    for (int i = 0; i < count; ++i) {
      qg::PrefillPlan pp;
      if (!qg::make_prefill_plan(M, K, items[i].N, &pp)) return QG_ERR_SHAPE;
      s = from_hip(qg::launch_gemm_prefill(bits, pp, x, x_f16, items[i].packed_w, items[i].scales,
                                           s_bf16(s_dt), s_cbm(s_dt), items[i].out, M, K,
                                           items[i].N, ws,
                                           as_stream(stream)));
      if (s != QG_OK) return s;
    }
    return QG_OK;
  }
  if (M == 1 || qg::gemv_rows_fits(M, K, g.n_total))
    return from_hip(qg::launch_gemv(bits, x, x_f16, g, s_bf16(s_dt), s_cbm(s_dt), M, K,
                                    as_stream(stream)));
  return from_hip(qg::launch_gemm_small(bits, plan, x, x_f16, g, s_bf16(s_dt), s_cbm(s_dt), M, K, ws,
                                        as_stream(stream)));
}

qg_status dequant(int bits, const void* packed, const void* scales, qg_dtype s_dt, int64_t K,
                  int64_t N, void* out, qg_dtype out_dt, void* stream) {
  qg_status s = check_kn(K, N);
  if (s != QG_OK) return s;
  if (s_dt != QG_F16 && s_dt != QG_BF16) return QG_ERR_DTYPE;
  if (out_dt != QG_F16 && out_dt != QG_BF16) return QG_ERR_DTYPE;
  if ((s = check_ptrs({packed, scales, out})) != QG_OK) return s;
  return from_hip(qg::launch_dequant(bits, packed, scales, s_dt == QG_BF16, out, out_dt == QG_F16,
                                     K, N, as_stream(stream)));
}

qg_status fake_quant(int bits, const void* W, qg_dtype w_dt, const void* scales, qg_dtype s_dt,
                     int64_t K, int64_t N, void* out, qg_dtype out_dt, void* stream) {
  qg_status s = check_kn(K, N);
  if (s != QG_OK) return s;
  if (w_dt != QG_F32 && w_dt != QG_BF16) return QG_ERR_DTYPE;
  if (s_dt != QG_F16 && s_dt != QG_BF16) return QG_ERR_DTYPE;
  if (out_dt != QG_BF16 && out_dt != QG_F16 && out_dt != QG_F32) return QG_ERR_DTYPE;
  if ((s = check_ptrs({W, scales, out})) != QG_OK) return s;
  const int kind = out_dt == QG_BF16 ? 0 : (out_dt == QG_F16 ? 1 : 2);
  return from_hip(qg::launch_fake_quant(bits, W, w_dt == QG_BF16, scales, s_dt == QG_BF16, out,
                                        kind, K, N, as_stream(stream)));
}

size_t workspace_bytes(int bits, int64_t M, int64_t K, int64_t N, int nbw, int wk, int splits) {
  if ((bits != 4 && bits != 8) || check_mkn(M, K, N) != QG_OK || M == 0) return 0;
  const bool own = nbw == 0 && wk == 0 && splits == 0;
  if (own && (M == 1 || qg::gemv_rows_fits(M, K, N))) return 0;   // GEMV
  if (M > kSmallMaxM && own) {                                  // prefill kernel
    qg::PrefillPlan pp;
    if (!qg::make_prefill_plan(M, K, N, &pp)) return 0;
    return qg::prefill_workspace(bits, pp, K);
  }
  qg::SmallPlan plan;
  if (!qg::make_small_plan(bits, M, K, N, nbw, wk, splits, &plan)) return 0;
  return qg::small_plan_workspace(plan, M, N);
}

constexpr int64_t kSwaMaxPairs = 65536 / 4;   // arrival counters at the workspace start

qg_status swa_check(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t D, int64_t S_max,
                    int64_t window, int64_t chunk, int64_t heads, qg::SwaPlan* plan) {
  if (B < 0 || B > kMaxM || T < 1 || T > 16 || D != 128 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return QG_ERR_SHAPE;
  if (S_max < T || window < 0 || chunk < 0 || chunk % 32 != 0 || chunk > (int64_t(1) << 20))
    return QG_ERR_SHAPE;
  if (heads < 0 || heads > 8) return QG_ERR_SHAPE;
  if (Hq > 4096 || S_max * Hkv * D * 2 >= kMaxElems || T * Hq * D * 2 >= kMaxElems)
    return QG_ERR_SHAPE;
  if (!qg::make_swa_plan(B, T, Hq, Hkv, S_max, window, chunk, heads, plan)) return QG_ERR_SHAPE;
  if (plan->nchunks > 1 && B * Hq > kSwaMaxPairs) return QG_ERR_SHAPE;
  if ((int64_t)plan->grid >= kMaxElems) return QG_ERR_SHAPE;
  return QG_OK;
}

size_t swa_workspace_bytes(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t D,
                           int64_t S_max, int64_t window, int64_t chunk, int64_t heads) {
  qg::SwaPlan plan;
  if (swa_check(B, T, Hq, Hkv, D, S_max, window, chunk, heads, &plan) != QG_OK || B == 0)
    return 0;
  return qg::swa_workspace(plan, B, Hq);
}

qg_status swa_attention(const void* q, const void* k, const void* v, const int32_t* seq_lens,
                        void* out, int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t D,
                        int64_t S_max, int64_t window, float scale, int64_t chunk,
                        int64_t heads, void* ws, size_t ws_bytes, void* stream) {
  qg::SwaPlan plan;
  qg_status s = swa_check(B, T, Hq, Hkv, D, S_max, window, chunk, heads, &plan);
  if (s != QG_OK) return s;
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY) return QG_ERR_SHAPE;
  if (B == 0) return QG_OK;
  if ((s = check_ptrs({q, k, v, out})) != QG_OK) return s;
  if (seq_lens == nullptr) return QG_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(seq_lens) & 3u) != 0) return QG_ERR_ALIGN;
  const size_t need = qg::swa_workspace(plan, B, Hq);
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need) return QG_ERR_WORKSPACE;
    if (!aligned16(ws)) return QG_ERR_ALIGN;
  }
  return from_hip(qg::launch_swa_attention(plan, q, k, v, seq_lens, out, T, Hq, Hkv, S_max, scale,
                                           ws, as_stream(stream)));
}

}  // namespace

extern "C" {

const char* qg_status_str(qg_status s) {
  switch (s) {
    case QG_OK: return "QG_OK";
    case QG_ERR_NULL: return "QG_ERR_NULL: a required pointer is NULL";
    case QG_ERR_SHAPE: return "QG_ERR_SHAPE: K must be a positive multiple of 128, N of 16, within limits";
    case QG_ERR_ALIGN: return "QG_ERR_ALIGN: pointers must be 16-byte aligned";
    case QG_ERR_DTYPE: return "QG_ERR_DTYPE: unsupported dtype for this argument";
    case QG_ERR_WORKSPACE: return "QG_ERR_WORKSPACE: workspace missing or too small";
    case QG_ERR_HIP: return "QG_ERR_HIP: the HIP runtime reported an error";
    case QG_ERR_PLAN: return "QG_ERR_PLAN: unsupported tiling plan";
  }
  return "unknown qg_status";
}

size_t qg_packed_bytes(int bits, int64_t K, int64_t N) {
  if (check_kn(K, N) != QG_OK) return 0;
  if (bits == 4) return (size_t)(K * N / 2);
  if (bits == 8) return (size_t)(K * N);
  return 0;
}

size_t qg_scale_bytes(int64_t K, int64_t N) {
  if (check_kn(K, N) != QG_OK) return 0;
  return (size_t)(K / 128 * N * 2);
}

size_t qg_workspace_bytes(int bits, int64_t M, int64_t K, int64_t N) {
  return workspace_bytes(bits, M, K, N, 0, 0, 0);
}

size_t qg_workspace_bytes_plan(int bits, int64_t M, int64_t K, int64_t N, int cols_per_wave,
                               int k_waves, int splits) {
  return workspace_bytes(bits, M, K, N, cols_per_wave, k_waves, splits);
}

qg_status qg_rtn_scales_w4(const void* W, qg_dtype w_dt, int64_t K, int64_t N, void* scales,
                           void* stream) {
  return rtn_scales(4, W, w_dt, K, N, scales, stream);
}

qg_status qg_rtn_scales_w8(const void* W, qg_dtype w_dt, int64_t K, int64_t N, void* scales,
                           void* stream) {
  return rtn_scales(8, W, w_dt, K, N, scales, stream);
}

qg_status qg_pack_to_grid_w4(const void* W, qg_dtype w_dt, const void* scales, qg_dtype s_dt,
                             int64_t K, int64_t N, void* packed_w, void* stream) {
  return pack_to_grid(4, W, w_dt, scales, s_dt, K, N, packed_w, stream);
}

qg_status qg_pack_to_grid_w8(const void* W, qg_dtype w_dt, const void* scales, qg_dtype s_dt,
                             int64_t K, int64_t N, void* packed_w, void* stream) {
  return pack_to_grid(8, W, w_dt, scales, s_dt, K, N, packed_w, stream);
}

qg_status qg_prepack_w4(const int8_t* codes, int64_t K, int64_t N, void* packed_w, void* stream) {
  return prepack(4, codes, K, N, packed_w, stream);
}

qg_status qg_unpack_w4(const void* packed_w, int64_t K, int64_t N, int8_t* codes, void* stream) {
  return unpack(4, packed_w, K, N, codes, stream);
}

qg_status qg_prepack_w8(const int8_t* codes, int64_t K, int64_t N, void* packed_w, void* stream) {
  return prepack(8, codes, K, N, packed_w, stream);
}

qg_status qg_unpack_w8(const void* packed_w, int64_t K, int64_t N, int8_t* codes, void* stream) {
  return unpack(8, packed_w, K, N, codes, stream);
}

qg_status qgemm_w4a16(const void* x, const void* packed_w, const void* scales, qg_dtype s_dt,
                      void* out, int64_t M, int64_t K, int64_t N, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return gemm(4, false, x, packed_w, scales, s_dt, out, M, K, N, workspace, workspace_bytes, 0,
              0, 0, stream);
}

qg_status qgemm_w8a16(const void* x, const void* packed_w, const void* scales, qg_dtype s_dt,
                      void* out, int64_t M, int64_t K, int64_t N, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return gemm(8, false, x, packed_w, scales, s_dt, out, M, K, N, workspace, workspace_bytes, 0,
              0, 0, stream);
}

size_t qg_noalloc_scratch_bytes(void) { return qg::kScratchBytes; }

qg_status qgemm_w4a16_noalloc(const void* x, const void* packed_w, const void* scales,
                              qg_dtype s_dt, void* out, int64_t M, int64_t K, int64_t N,
                              void* stream) {
  // Every check of qgemm_w4a16 first, on the host; then the workspace this
  // call would need against the fixed scratch (QG_ERR_WORKSPACE beyond it);
  // only then any HIP call.
  const qg_status s = gemm_check(x, packed_w, scales, s_dt, out, M, K, N);
  if (s != QG_OK || M == 0) return s;
  const size_t need = workspace_bytes(4, M, K, N, 0, 0, 0);
  if (need > qg::kScratchBytes) return QG_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && qg::scratch_for_stream(as_stream(stream), &ws) != hipSuccess) return QG_ERR_HIP;
  return gemm(4, false, x, packed_w, scales, s_dt, out, M, K, N, ws, need, 0, 0, 0, stream);
}

qg_status qgemm_w4a16_plan(const void* x, const void* packed_w, const void* scales, qg_dtype s_dt,
                           void* out, int64_t M, int64_t K, int64_t N, void* workspace,
                           size_t workspace_bytes, int cols_per_wave, int k_waves, int splits,
                           void* stream) {
  return gemm(4, false, x, packed_w, scales, s_dt, out, M, K, N, workspace, workspace_bytes,
              cols_per_wave, k_waves, splits, stream);
}

qg_status qgemm_w8a16_plan(const void* x, const void* packed_w, const void* scales, qg_dtype s_dt,
                           void* out, int64_t M, int64_t K, int64_t N, void* workspace,
                           size_t workspace_bytes, int cols_per_wave, int k_waves, int splits,
                           void* stream) {
  return gemm(8, false, x, packed_w, scales, s_dt, out, M, K, N, workspace, workspace_bytes,
              cols_per_wave, k_waves, splits, stream);
}

qg_status qgemm_w4f16(const void* x, const void* packed_w, const void* scales, qg_dtype s_dt,
                      void* out, int64_t M, int64_t K, int64_t N, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return gemm(4, true, x, packed_w, scales, s_dt, out, M, K, N, workspace, workspace_bytes, 0, 0,
              0, stream);
}

qg_status qgemm_w8f16(const void* x, const void* packed_w, const void* scales, qg_dtype s_dt,
                      void* out, int64_t M, int64_t K, int64_t N, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return gemm(8, true, x, packed_w, scales, s_dt, out, M, K, N, workspace, workspace_bytes, 0, 0,
              0, stream);
}

qg_status qgemm_w4f16_plan(const void* x, const void* packed_w, const void* scales, qg_dtype s_dt,
                           void* out, int64_t M, int64_t K, int64_t N, void* workspace,
                           size_t workspace_bytes, int cols_per_wave, int k_waves, int splits,
                           void* stream) {
  return gemm(4, true, x, packed_w, scales, s_dt, out, M, K, N, workspace, workspace_bytes,
              cols_per_wave, k_waves, splits, stream);
}

qg_status qgemm_w8f16_plan(const void* x, const void* packed_w, const void* scales, qg_dtype s_dt,
                           void* out, int64_t M, int64_t K, int64_t N, void* workspace,
                           size_t workspace_bytes, int cols_per_wave, int k_waves, int splits,
                           void* stream) {
  return gemm(8, true, x, packed_w, scales, s_dt, out, M, K, N, workspace, workspace_bytes,
              cols_per_wave, k_waves, splits, stream);
}

qg_status qg_dequant_w4(const void* packed_w, const void* scales, qg_dtype s_dt, int64_t K,
                        int64_t N, void* out, qg_dtype out_dt, void* stream) {
  return dequant(4, packed_w, scales, s_dt, K, N, out, out_dt, stream);
}

qg_status qg_dequant_w8(const void* packed_w, const void* scales, qg_dtype s_dt, int64_t K,
                        int64_t N, void* out, qg_dtype out_dt, void* stream) {
  return dequant(8, packed_w, scales, s_dt, K, N, out, out_dt, stream);
}

qg_status qg_fake_quant_w4(const void* W, qg_dtype w_dt, const void* scales, qg_dtype s_dt,
                           int64_t K, int64_t N, void* out, qg_dtype out_dt, void* stream) {
  return fake_quant(4, W, w_dt, scales, s_dt, K, N, out, out_dt, stream);
}

qg_status qg_fake_quant_w8(const void* W, qg_dtype w_dt, const void* scales, qg_dtype s_dt,
                           int64_t K, int64_t N, void* out, qg_dtype out_dt, void* stream) {
  return fake_quant(8, W, w_dt, scales, s_dt, K, N, out, out_dt, stream);
}

size_t qg_workspace_bytes_grouped(int bits, int64_t M, int64_t K, const qg_group_item* items,
                                  int count) {
  return grouped_workspace(bits, M, K, items, count);
}

qg_status qgemm_w4a16_grouped(const void* x, const qg_group_item* items, int count, qg_dtype s_dt,
                              int64_t M, int64_t K, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return gemm_grouped(4, false, x, items, count, s_dt, M, K, workspace, workspace_bytes, stream);
}

qg_status qgemm_w8a16_grouped(const void* x, const qg_group_item* items, int count, qg_dtype s_dt,
                              int64_t M, int64_t K, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return gemm_grouped(8, false, x, items, count, s_dt, M, K, workspace, workspace_bytes, stream);
}

qg_status qgemm_w4f16_grouped(const void* x, const qg_group_item* items, int count, qg_dtype s_dt,
                              int64_t M, int64_t K, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return gemm_grouped(4, true, x, items, count, s_dt, M, K, workspace, workspace_bytes, stream);
}

qg_status qgemm_w8f16_grouped(const void* x, const qg_group_item* items, int count, qg_dtype s_dt,
                              int64_t M, int64_t K, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return gemm_grouped(8, true, x, items, count, s_dt, M, K, workspace, workspace_bytes, stream);
}

size_t qg_swa_workspace_bytes(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t D,
                              int64_t S_max, int64_t window) {
  return swa_workspace_bytes(B, T, Hq, Hkv, D, S_max, window, 0, 0);
}

qg_status qg_swa_attention(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* seq_lens, void* out, int64_t B, int64_t T, int64_t Hq,
                           int64_t Hkv, int64_t D, int64_t S_max, int64_t window, float scale,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return swa_attention(q, k_cache, v_cache, seq_lens, out, B, T, Hq, Hkv, D, S_max, window,
                       scale, 0, 0, workspace, workspace_bytes, stream);
}

size_t qg_swa_workspace_bytes_plan(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t D,
                                   int64_t S_max, int64_t window, int64_t chunk,
                                   int64_t heads) {
  return swa_workspace_bytes(B, T, Hq, Hkv, D, S_max, window, chunk, heads);
}

qg_status qg_swa_attention_plan(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* seq_lens, void* out, int64_t B, int64_t T,
                                int64_t Hq, int64_t Hkv, int64_t D, int64_t S_max,
                                int64_t window, float scale, int64_t chunk, int64_t heads,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return swa_attention(q, k_cache, v_cache, seq_lens, out, B, T, Hq, Hkv, D, S_max, window,
                       scale, chunk, heads, workspace, workspace_bytes, stream);
}

qg_status qg_prepack_scales(const void* scales, qg_dtype s_dt, int64_t K, int64_t N, void* out,
                            void* stream) {
  qg_status s = check_kn(K, N);
  if (s != QG_OK) return s;
  if (s_dt != QG_F16 && s_dt != QG_BF16) return QG_ERR_DTYPE;
  if ((s = check_ptrs({scales, out})) != QG_OK) return s;
  return from_hip(qg::launch_prepack_scales(scales, K, N, out, as_stream(stream)));
}

qg_status qg_read_stream(const void* src, size_t bytes, int workgroups, void* sink, void* stream) {
  if (bytes == 0 || bytes % 16 != 0 || bytes >= (size_t(1) << 40)) return QG_ERR_SHAPE;
  if (workgroups < 1 || workgroups > 65536) return QG_ERR_SHAPE;
  const qg_status s = check_ptrs({src, sink});
  if (s != QG_OK) return s;
  return from_hip(qg::launch_read_stream(src, (int64_t)bytes, workgroups, sink, as_stream(stream)));
}

}  // extern "C"

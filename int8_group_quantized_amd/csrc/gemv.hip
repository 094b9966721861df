// Decode GEMV (M = 1) of the group-quantized GEMM, and its 2-16-row form for
// narrow verification shapes:
//   out[n] = bf16( sum_g s[g, n] * sum_{k in g} x[k] * q[k, n] )
// (arXiv 2607.04244, QAD paragraph: the served weight is s (.) W_q; group of
// 128 along K per the drafter-PTQ paragraph; INT8 variant per the W8A16
// model card.)
//
// One token streams the whole weight once: the kernel is bound by HBM, and on
// MI355X what separates it from a plain read of the same bytes is work that
// waits on the data. Loads retire in issue order, so a wavefront's tiles
// become usable late and in a clump; anything queued behind them (a staging
// barrier, a long dependent chain) spills past the last byte. So:
//   * a workgroup owns one 16-column block; its WK wavefronts split K, each
//     taking GW groups per round. A wavefront issues every load of a round
//     up front, per group: its x slice, its scales, its code tile(s);
//   * no LDS staging and no barrier before compute: x of one group is a
//     single 16-byte load per lane into the A operand, row r holding the
//     group's K slice r % 4 (32 values), so each K step j of the tile is an
//     independent 16x16x32 product whose row j is that step's partial sum.
//     The four partials (the diagonal of four products) and the INT4 offset
//     partials (one product of the same A with the constant 136, rows 0..3)
//     are added in the same order, so an all-zero code column cancels to
//     exactly 0; the group's fp32 scale is applied with one FMA;
//   * the scale of the lane's column is a 2-byte load per group (either
//     scale order), issued with the group's other loads;
//   * wavefronts that split K are summed through LDS in wave order after
//     one barrier (deterministic); lanes 0..15 store the 16 outputs;
//   * the scale order is a template parameter and the round loop exits on a
//     scalar test of the next round's first group: with the order chosen by
//     a runtime branch inside the loop, the same arithmetic measured 6.12
//     against 5.90 us (gate/up) and 4.98 against 4.89 us (down).
// Workgroups are dealt to the eight XCDs round-robin; each XCD gets a
// contiguous run of column blocks, so the four blocks sharing a 128-byte scale
// line are read by one XCD's L2.
#include "qg_device.h"
#include "qg_internal.h"

namespace qg {
namespace {

constexpr int kGW = kGemvGroups;   // groups per wavefront per round

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemv_rsrc(const void* base, int bytes) {
  // Raw buffer resource: loads at or past `bytes` return zeros, no access.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ uint32_t gemv_opaque(uint32_t m) {
  asm volatile("" : "+v"(m));   // keep the INT4 constant in a register (one AND-OR per pair)
  return m;
}

template <int BITS, bool SBF, bool XH, bool GR, int WK, bool SCBM>
__global__ __launch_bounds__(64 * WK) void gemv_kernel(const uint16_t* __restrict__ x, int G,
                                                       const GroupArgs ga) {
  using A = Act<XH>;
  constexpr int TB = (BITS == 4) ? 1024 : 2048;   // bytes per 16 x 128 tile
  constexpr int TW = TB / 1024;                   // 16-byte loads per lane per tile
  constexpr int aux = (BITS == 4) ? 2 : 0;        // INT4 tiles stream with the nontemporal hint
  __shared__ float red[WK > 1 ? (WK - 1) * 16 : 1];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, lq = lane >> 4;

  int b = blockIdx.x;
  const int nwg = gridDim.x;
  const int b8 = nwg / 8 * 8;
  if (b < b8) b = (b % 8) * (nwg / 8) + b / 8;
  int item = 0;
  if constexpr (GR) {
    for (int i = 1; i < ga.count; ++i)
      if (b >= ga.item[i].wg_first) item = i;
  }
  const GroupItem& it = ga.item[item];
  const int N = it.n;
  const int cb = b - (GR ? it.wg_first : 0);
  const char* __restrict__ packed = it.packed;
  const uint16_t* __restrict__ scales = it.scales;
  uint16_t* __restrict__ out = it.out;
  const uint32_t magic = gemv_opaque(A::kMagic);
  const u32x4 off = {A::kOffset, A::kOffset, A::kOffset, A::kOffset};
  // A operand: lane (row l16, K slice lq) takes elements 32 (l16 % 4) + 8 lq .. + 8
  const int xoff = (32 * (l16 & 3) + 8 * lq) * 2;

  float acc = 0.0f;
  for (int r = 0;; ++r) {
    const int g0 = (r * WK + wave) * kGW;
    if (g0 >= G) break;                           // wave-uniform: later rounds are empty too
    const int wn = min(kGW, G - g0);              // groups of this wavefront this round
    const __amdgpu_buffer_rsrc_t xr = gemv_rsrc(x + (int64_t)g0 * kGroup, wn * kGroup * 2);
    const __amdgpu_buffer_rsrc_t tr = gemv_rsrc(packed + ((int64_t)cb * G + g0) * TB, wn * TB);
    const __amdgpu_buffer_rsrc_t sr =
        SCBM ? gemv_rsrc(scales + ((int64_t)cb * G + g0) * 16, wn * 32)
             : gemv_rsrc(scales + (int64_t)g0 * N + cb * 16, ((wn - 1) * N + 16) * 2);
    const int sstride = SCBM ? 16 : N;

    u32x4 xa[kGW];
    u32x4 t[kGW][TW];
    uint32_t sb[kGW];
    // Every load of the round goes out before the first multiply, group by
    // group (x, scale, tile): loads retire in issue order, so this order
    // makes each group usable as early as its own bytes allow (measured
    // against the scheduler's own interleaving and against x / scales /
    // tiles issued as three blocks: 6.09 vs 6.15 / 6.35 us for the decode
    // gate/up GEMV).
#pragma unroll
    for (int d = 0; d < kGW; ++d) {
      xa[d] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, xoff + d * 256, 0, 0));
      sb[d] = __builtin_amdgcn_raw_buffer_load_b16(sr, (d * sstride + l16) * 2, 0, 0);
#pragma unroll
      for (int v = 0; v < TW; ++v)
        t[d][v] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(tr, lane * (TB / 64) + d * TB + 16 * v, 0, aux));
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int d = 0; d < kGW; ++d) {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      f32x4 p[4];
      if constexpr (BITS == 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) p[j] = A::mma(xa[d], int4_word_to_act(t[d][0][j], magic), z);
      } else {
        p[0] = A::mma(xa[d], int8_words_to_act<A>(t[d][0][0], t[d][0][1]), z);
        p[1] = A::mma(xa[d], int8_words_to_act<A>(t[d][0][2], t[d][0][3]), z);
        p[2] = A::mma(xa[d], int8_words_to_act<A>(t[d][1][0], t[d][1][1]), z);
        p[3] = A::mma(xa[d], int8_words_to_act<A>(t[d][1][2], t[d][1][3]), z);
      }
      float part = ((p[0][0] + p[1][1]) + p[2][2]) + p[3][3];
      if constexpr (BITS == 4) {
        const f32x4 bias = A::mma(xa[d], off, z);
        part -= ((bias[0] + bias[1]) + bias[2]) + bias[3];
      }
      const float sv = scale_to_f32(sb[d], SBF);
      acc = fmaf(d < wn ? sv : 0.0f, part, acc);
    }
  }

  if constexpr (WK > 1) {
    if (wave > 0 && lq == 0) red[(wave - 1) * 16 + l16] = acc;
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < WK - 1; ++w) acc += red[w * 16 + l16];
  }
  if (lq == 0) out[cb * 16 + l16] = A::out(acc);
}

// The same structure for 2-16 rows (a verification block), where the shape
// is narrow (at most 512 column blocks, at most 40 groups): every 16-row A
// operand is fully used, so x of a group is four 16-byte loads per lane
// (rows past M read as zeros), the four K steps chain into one product, and
// the INT4 offset is the same chain with the constant 136 (exact cancellation
// for all-zero code columns). x is re-read from L2 by every column block;
// that costs less than staging it behind a barrier while the column blocks
// are few (wide shapes use the staged small-M kernel).
template <int BITS, bool SBF, bool XH, bool GR, int WK, bool SCBM>
__global__ __launch_bounds__(64 * WK) void gemv_rows_kernel(const uint16_t* __restrict__ x, int M,
                                                            int K, const GroupArgs ga) {
  using A = Act<XH>;
  constexpr int TB = (BITS == 4) ? 1024 : 2048;
  constexpr int TW = TB / 1024;
  constexpr int aux = (BITS == 4) ? 2 : 0;
  __shared__ f32x4 red[WK > 1 ? (WK - 1) * 64 : 1];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, lq = lane >> 4;

  int b = blockIdx.x;
  const int nwg = gridDim.x;
  const int b8 = nwg / 8 * 8;
  if (b < b8) b = (b % 8) * (nwg / 8) + b / 8;
  int item = 0;
  if constexpr (GR) {
    for (int i = 1; i < ga.count; ++i)
      if (b >= ga.item[i].wg_first) item = i;
  }
  const GroupItem& it = ga.item[item];
  const int N = it.n;
  const int cb = b - (GR ? it.wg_first : 0);
  const char* __restrict__ packed = it.packed;
  const uint16_t* __restrict__ scales = it.scales;
  uint16_t* __restrict__ out = it.out;
  const int G = K >> 7;
  const uint32_t magic = gemv_opaque(A::kMagic);
  const u32x4 off = {A::kOffset, A::kOffset, A::kOffset, A::kOffset};
  // A operand: lane (row l16, K slice lq); rows >= M lie past the resource
  // (M rows of K values) and read as zeros.
  const __amdgpu_buffer_rsrc_t xr = gemv_rsrc(x, M * K * 2);
  const int xrow = l16 * K * 2 + 16 * lq;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int r = 0;; ++r) {
    const int g0 = (r * WK + wave) * kGW;
    if (g0 >= G) break;                           // wave-uniform: later rounds are empty too
    const int wn = min(kGW, G - g0);
    const __amdgpu_buffer_rsrc_t tr = gemv_rsrc(packed + ((int64_t)cb * G + g0) * TB, wn * TB);
    const __amdgpu_buffer_rsrc_t sr =
        SCBM ? gemv_rsrc(scales + ((int64_t)cb * G + g0) * 16, wn * 32)
             : gemv_rsrc(scales + (int64_t)g0 * N + cb * 16, ((wn - 1) * N + 16) * 2);
    const int sstride = SCBM ? 16 : N;

    u32x4 xa[kGW][4];
    u32x4 t[kGW][TW];
    uint32_t sb[kGW];
#pragma unroll
    for (int d = 0; d < kGW; ++d) {
      // groups past this wavefront's last read x as zeros too
      const int xo = (d < wn) ? xrow + (g0 + d) * kGroup * 2 : 0x7FFFFFF0;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xa[d][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 xr, (d < wn) ? xo + 64 * j : xo, 0, 0));
      sb[d] = __builtin_amdgcn_raw_buffer_load_b16(sr, (d * sstride + l16) * 2, 0, 0);
#pragma unroll
      for (int v = 0; v < TW; ++v)
        t[d][v] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(tr, lane * (TB / 64) + d * TB + 16 * v, 0, aux));
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int d = 0; d < kGW; ++d) {
      f32x4 p = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BITS == 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) p = A::mma(xa[d][j], int4_word_to_act(t[d][0][j], magic), p);
        f32x4 bias = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) bias = A::mma(xa[d][j], off, bias);
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] -= bias[e];
      } else {
        p = A::mma(xa[d][0], int8_words_to_act<A>(t[d][0][0], t[d][0][1]), p);
        p = A::mma(xa[d][1], int8_words_to_act<A>(t[d][0][2], t[d][0][3]), p);
        p = A::mma(xa[d][2], int8_words_to_act<A>(t[d][1][0], t[d][1][1]), p);
        p = A::mma(xa[d][3], int8_words_to_act<A>(t[d][1][2], t[d][1][3]), p);
      }
      const float sv = d < wn ? scale_to_f32(sb[d], SBF) : 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(sv, p[e], acc[e]);
    }
  }

  if constexpr (WK > 1) {
    if (wave > 0) red[(wave - 1) * 64 + lane] = acc;
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < WK - 1; ++w) {
      const f32x4 o = red[w * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += o[e];
    }
  }
  // C layout: lane holds column l16, rows 4 lq + e
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = 4 * lq + e;
    if (row < M) out[(int64_t)row * N + cb * 16 + l16] = A::out(acc[e]);
  }
}

template <int BITS, bool SBF, bool XH, bool GR, bool SCBM>
hipError_t launch_wk(int wk, const void* x, const GroupArgs& g, int64_t M, int64_t K,
                     hipStream_t st) {
  const auto* xp = static_cast<const uint16_t*>(x);
  const int m = (int)M, k = (int)K, G = (int)(K / kGroup);
  const dim3 grid((unsigned)g.wg_total);
  if (M == 1) {
    switch (wk) {
      case 1: gemv_kernel<BITS, SBF, XH, GR, 1, SCBM><<<grid, 64, 0, st>>>(xp, G, g); break;
      case 2: gemv_kernel<BITS, SBF, XH, GR, 2, SCBM><<<grid, 128, 0, st>>>(xp, G, g); break;
      case 4: gemv_kernel<BITS, SBF, XH, GR, 4, SCBM><<<grid, 256, 0, st>>>(xp, G, g); break;
      case 8: gemv_kernel<BITS, SBF, XH, GR, 8, SCBM><<<grid, 512, 0, st>>>(xp, G, g); break;
      case 16: gemv_kernel<BITS, SBF, XH, GR, 16, SCBM><<<grid, 1024, 0, st>>>(xp, G, g); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (wk) {
      case 1: gemv_rows_kernel<BITS, SBF, XH, GR, 1, SCBM><<<grid, 64, 0, st>>>(xp, m, k, g); break;
      case 2: gemv_rows_kernel<BITS, SBF, XH, GR, 2, SCBM><<<grid, 128, 0, st>>>(xp, m, k, g); break;
      case 4: gemv_rows_kernel<BITS, SBF, XH, GR, 4, SCBM><<<grid, 256, 0, st>>>(xp, m, k, g); break;
      case 8: gemv_rows_kernel<BITS, SBF, XH, GR, 8, SCBM><<<grid, 512, 0, st>>>(xp, m, k, g); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

template <int BITS, bool SBF, bool XH>
hipError_t launch_gr(int wk, const void* x, const GroupArgs& g, bool s_cbm, int64_t M, int64_t K,
                     hipStream_t st) {
  if (g.count > 1)
    return s_cbm ? launch_wk<BITS, SBF, XH, true, true>(wk, x, g, M, K, st)
                 : launch_wk<BITS, SBF, XH, true, false>(wk, x, g, M, K, st);
  return s_cbm ? launch_wk<BITS, SBF, XH, false, true>(wk, x, g, M, K, st)
               : launch_wk<BITS, SBF, XH, false, false>(wk, x, g, M, K, st);
}

}  // namespace

hipError_t launch_gemv(int bits, const void* x, bool x_f16, const GroupArgs& g, bool s_bf16,
                       bool s_cbm, int64_t M, int64_t K, hipStream_t st) {
  const int wk = gemv_k_waves(K);
  if (M < 1 || M > 16 || (M > 1 && wk > 8)) return hipErrorInvalidValue;
#define QG_GV(B, S, H) \
  if (bits == B && s_bf16 == S && x_f16 == H) return launch_gr<B, S, H>(wk, x, g, s_cbm, M, K, st);
  QG_GV(4, false, false) QG_GV(4, true, false) QG_GV(8, false, false) QG_GV(8, true, false)
  QG_GV(4, false, true) QG_GV(4, true, true) QG_GV(8, false, true) QG_GV(8, true, true)
#undef QG_GV
  return hipErrorInvalidValue;
}

}  // namespace qg

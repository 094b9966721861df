// Small-M group-quantized GEMM (decode M = 1, verification blocks M <= 16):
//   out[m, n] = bf16( sum_g s[g, n] * sum_{k in g} x[m, k] * q[k, n] )
// (arXiv 2607.04244, QAD paragraph: the served weight is s (.) W_q; group of
// 128 along K per the drafter-PTQ paragraph; INT8 variant per the W8A16
// model card.)
//
// The path is HBM-bound: 0.5 (INT4) or 1 (INT8) byte per weight streams once
// from memory. Each wavefront owns `NBW` 16-column blocks and a slice of the
// K groups. Per group it
//   1. loads its packed tile(s) with one 16-byte load per lane per 1 KiB
//      (fully coalesced: a tile is 1 KiB contiguous, lane l reads bytes
//      16l..16l+15),
//   2. loads the matching 16 x 128 slice of x (bf16, L2-resident),
//   3. expands codes in registers to exact bf16 integers and runs four
//      16x16x32 bf16 matrix-core ops, giving the group's fp32 partial sums
//      for 16 rows x 16 columns (rows >= M are zero-filled),
//   4. multiplies by the group's fp32 scale and adds into the accumulator.
// The matrix cores carry the contraction because the vector ALUs cannot: at
// M = 16 the path needs ~1.8e14 multiply-adds/s to keep pace with HBM, twice
// the fp32 vector peak, while the 16-row matrix op matches M = 16 exactly.
//
// INT4 codes expand as 128 + u with u = q + 8 (one AND-OR per pair). The bias
// 136 * sum_k x[m, k] is the same 16x16x32 product with every code equal to
// 136, evaluated in the same order; subtracting it gives sum x*q. A column
// whose codes are all zero yields bit-identical sums on both sides, so it
// comes out exactly 0.
//
// Reductions are deterministic: `WK` wavefronts of a workgroup that split K
// are summed through LDS in wave order; `splits` workgroups along K write
// fp32 partials, and whichever arrives last sums them in split order.
#include "qg_device.h"
#include "qg_internal.h"

namespace qg {
namespace {

constexpr int kMaxCounters = kCounterBytes / sizeof(uint32_t);

template <int BITS, int NBW, int WK, int U>
__global__ __launch_bounds__(256) void gemm_small_kernel(
    const uint16_t* __restrict__ x, const u32x4* __restrict__ packed,
    const uint16_t* __restrict__ scales, int s_bf16, uint16_t* __restrict__ out,
    uint32_t* __restrict__ counters, float* __restrict__ partials, int M, int K, int N,
    int splits, int gps) {
  constexpr int WN = 4 / WK;                 // wavefronts along N in a workgroup
  constexpr int TU4 = (BITS == 4) ? 1 : 2;   // 16-byte words per lane per tile
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wn = wave % WN;
  const int wk = wave / WN;
  const int G = K >> 7;
  const int NB = N >> 4;
  const int cb0 = (blockIdx.x * WN + wn) * NBW;
  const int nvalid = min(NBW, NB - cb0);     // column blocks this wave owns (may be <= 0)
  const int split = blockIdx.y;
  const int row0 = blockIdx.z * 16;
  const int g_end = min(G, (split + 1) * gps);
  const int l16 = lane & 15;                 // A row / C column of this lane
  const int lq = lane >> 4;                  // K slice (A, B) / row quad (C)
  const bool row_ok = row0 + l16 < M;
  const uint16_t* xrow = x + (int64_t)(row0 + l16) * K + 8 * lq;
  const bool sbf = s_bf16 != 0;

  f32x4 acc[NBW];
#pragma unroll
  for (int c = 0; c < NBW; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nvalid > 0) {
    for (int g0 = split * gps + wk; g0 < g_end; g0 += U * WK) {
      u32x4 xa[U][4];
      u32x4 wt[U][NBW][TU4];
      float sc[U][NBW];
      // Issue every load of the chunk before any arithmetic.
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int g = g0 + u * WK;
        if (g < g_end) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            xa[u][j] = row_ok ? *reinterpret_cast<const u32x4*>(xrow + (int64_t)g * 128 + 32 * j)
                              : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
          for (int c = 0; c < NBW; ++c) {
            if (c < nvalid) {
              const int64_t t = (int64_t)(cb0 + c) * G + g;
#pragma unroll
              for (int v = 0; v < TU4; ++v) wt[u][c][v] = packed[(t * 64 + lane) * TU4 + v];
              sc[u][c] = scale_to_f32(scales[(int64_t)g * N + (cb0 + c) * 16 + l16], sbf);
            }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int g = g0 + u * WK;
        if (g >= g_end) break;
        bf16x8 a[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = __builtin_bit_cast(bf16x8, xa[u][j]);
        f32x4 bias = {0.f, 0.f, 0.f, 0.f};
        if constexpr (BITS == 4) {
          const bf16x8 b136 = bias136_bf16x8();
#pragma unroll
          for (int j = 0; j < 4; ++j) bias = mfma16x16x32(a[j], b136, bias);
        }
#pragma unroll
        for (int c = 0; c < NBW; ++c) {
          if (c < nvalid) {
            f32x4 p = {0.f, 0.f, 0.f, 0.f};
            if constexpr (BITS == 4) {
#pragma unroll
              for (int j = 0; j < 4; ++j)
                p = mfma16x16x32(a[j], int4_word_to_biased_bf16(wt[u][c][0][j]), p);
            } else {
              p = mfma16x16x32(a[0], int8_words_to_bf16(wt[u][c][0][0], wt[u][c][0][1]), p);
              p = mfma16x16x32(a[1], int8_words_to_bf16(wt[u][c][0][2], wt[u][c][0][3]), p);
              p = mfma16x16x32(a[2], int8_words_to_bf16(wt[u][c][1][0], wt[u][c][1][1]), p);
              p = mfma16x16x32(a[3], int8_words_to_bf16(wt[u][c][1][2], wt[u][c][1][3]), p);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[c][e] = fmaf(sc[u][c], p[e] - bias[e], acc[c][e]);
          }
        }
      }
    }
  }

  // Wavefronts that split K inside the workgroup: reduce through LDS.
  if constexpr (WK > 1) {
    __shared__ f32x4 red[WK - 1][WN][NBW][64];
    if (wk > 0) {
#pragma unroll
      for (int c = 0; c < NBW; ++c) red[wk - 1][wn][c][lane] = acc[c];
    }
    __syncthreads();
    if (wk == 0) {
#pragma unroll
      for (int w = 0; w < WK - 1; ++w) {
#pragma unroll
        for (int c = 0; c < NBW; ++c) {
          const f32x4 o = red[w][wn][c][lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[c][e] += o[e];
        }
      }
    }
  }

  // C layout of the 16x16 result: lane holds column l16, rows 4*lq + e.
  if (splits == 1) {
    if (wk == 0) {
#pragma unroll
      for (int c = 0; c < NBW; ++c) {
        if (c < nvalid) {
          const int n = (cb0 + c) * 16 + l16;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = row0 + 4 * lq + e;
            if (row < M) out[(int64_t)row * N + n] = f32_to_bf16_bits(acc[c][e]);
          }
        }
      }
    }
    return;
  }

  if (wk == 0) {
#pragma unroll
    for (int c = 0; c < NBW; ++c) {
      if (c < nvalid) {
        const int n = (cb0 + c) * 16 + l16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = row0 + 4 * lq + e;
          if (row < M) partials[((int64_t)split * M + row) * N + n] = acc[c][e];
        }
      }
    }
  }
  // Publish this workgroup's partials device-wide, then count arrivals.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  __shared__ uint32_t s_last;
  const uint32_t cidx = blockIdx.z * gridDim.x + blockIdx.x;
  if (threadIdx.x == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(&counters[cidx], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == (uint32_t)splits - 1u) ? 1u : 0u;
  }
  __syncthreads();
  if (s_last == 0u) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (wk == 0) {
#pragma unroll
    for (int c = 0; c < NBW; ++c) {
      if (c < nvalid) {
        const int n = (cb0 + c) * 16 + l16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = row0 + 4 * lq + e;
          if (row < M) {
            float sum = 0.0f;
            for (int sp = 0; sp < splits; ++sp) sum += partials[((int64_t)sp * M + row) * N + n];
            out[(int64_t)row * N + n] = f32_to_bf16_bits(sum);
          }
        }
      }
    }
  }
  if (threadIdx.x == 0) counters[cidx] = 0u;   // ready for the next call
}

template <int BITS, int NBW, int WK>
hipError_t launch_variant(const SmallPlan& p, const void* x, const void* packed,
                          const void* scales, bool s_bf16, void* out, int64_t M, int64_t K,
                          int64_t N, void* ws, hipStream_t st) {
  constexpr int U = (NBW >= 4) ? 2 : 4;
  const dim3 grid((unsigned)p.wgs_n, (unsigned)p.splits, (unsigned)p.row_blocks);
  uint32_t* counters = nullptr;
  float* partials = nullptr;
  if (p.splits > 1) {
    counters = static_cast<uint32_t*>(ws);
    partials = reinterpret_cast<float*>(static_cast<char*>(ws) + kCounterBytes);
  }
  gemm_small_kernel<BITS, NBW, WK, U><<<grid, 256, 0, st>>>(
      static_cast<const uint16_t*>(x), static_cast<const u32x4*>(packed),
      static_cast<const uint16_t*>(scales), s_bf16 ? 1 : 0, static_cast<uint16_t*>(out),
      counters, partials, (int)M, (int)K, (int)N, p.splits, p.gps);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const SmallPlan& p, const void* x, const void* packed, const void* scales,
                       bool s_bf16, void* out, int64_t M, int64_t K, int64_t N, void* ws,
                       hipStream_t st) {
#define QG_V(NBW, WK)                                                                       \
  if (p.nbw == NBW && p.wk == WK)                                                           \
    return launch_variant<BITS, NBW, WK>(p, x, packed, scales, s_bf16, out, M, K, N, ws, st);
  QG_V(1, 1) QG_V(1, 2) QG_V(1, 4)
  QG_V(2, 1) QG_V(2, 2) QG_V(2, 4)
  QG_V(4, 1) QG_V(4, 2) QG_V(4, 4)
#undef QG_V
  return hipErrorInvalidValue;
}

}  // namespace

bool make_small_plan(int bits, int64_t M, int64_t K, int64_t N, int nbw, int wk, int splits,
                     SmallPlan* plan) {
  (void)bits;
  const int64_t NB = N / kTileCols;
  const int64_t G = K / kGroup;
  SmallPlan p;
  p.row_blocks = (int)((M + 15) / 16);
  if (nbw == 0) nbw = (M > 16) ? 2 : 1;
  if (wk == 0) wk = (M > 16) ? 1 : 4;
  if (nbw != 1 && nbw != 2 && nbw != 4) return false;
  if (wk != 1 && wk != 2 && wk != 4) return false;
  const int64_t wn = 4 / wk;
  p.nbw = nbw;
  p.wk = wk;
  p.wgs_n = (int)((NB + wn * nbw - 1) / (wn * nbw));
  if (splits == 0) {
    if (M > 16) {
      splits = 1;
    } else {
      // Aim for ~1024 workgroups (4 per compute unit), at least 4 groups each.
      const int64_t want = (1024 + p.wgs_n - 1) / p.wgs_n;
      const int64_t cap = G / 4 > 1 ? G / 4 : 1;
      splits = (int)(want < cap ? want : cap);
      if (splits < 1) splits = 1;
    }
  }
  if (splits < 1 || splits > G) return false;
  p.gps = (int)((G + splits - 1) / splits);
  p.splits = (int)((G + p.gps - 1) / p.gps);   // no empty split
  if (p.splits > 65535 || p.row_blocks > 65535) return false;
  if (p.splits > 1 && (int64_t)p.wgs_n * p.row_blocks > kMaxCounters) return false;
  *plan = p;
  return true;
}

size_t small_plan_workspace(const SmallPlan& p, int64_t M, int64_t N) {
  if (p.splits <= 1) return 0;
  return (size_t)kCounterBytes + (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float);
}

hipError_t launch_gemm_small(int bits, const SmallPlan& p, const void* x, const void* packed,
                             const void* scales, bool s_bf16, void* out, int64_t M, int64_t K,
                             int64_t N, void* ws, hipStream_t st) {
  if (bits == 4) return launch_bits<4>(p, x, packed, scales, s_bf16, out, M, K, N, ws, st);
  return launch_bits<8>(p, x, packed, scales, s_bf16, out, M, K, N, ws, st);
}

}  // namespace qg

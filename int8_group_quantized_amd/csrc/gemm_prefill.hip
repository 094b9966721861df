// Large-M group-quantized GEMM (prefill, e.g. the 8,192-token Long setting
// of the speed paragraph of arXiv 2607.04244):
//   out[m, n] = bf16( sum_g s[g, n] * sum_{k in g} x[m, k] * q[k, n] )
//
// At M = 8192 the product is a dense contraction (~2,000 flop per HBM byte),
// so the kernel is bound by the bf16 matrix cores, not by memory:
//   * a workgroup computes a 128 x 128 output tile with four wavefronts, each
//     a 64 x 64 sub-tile as a 4 x 4 grid of 16x16 blocks;
//   * the K loop steps one scale group (128) at a time. x for the group
//     (128 rows x 128 K, 32 KiB of bf16) is staged in LDS with direct
//     global->LDS loads, double-buffered, in the lane order of the
//     16x16x32 A operand, so each wavefront reads its fragments with
//     conflict-free 16-byte LDS reads; one barrier per group;
//   * the packed weight tiles are already in B-operand order, so each
//     wavefront loads its four 1 KiB (INT8: 2 KiB) column-block tiles of the
//     next group straight into registers while the current group computes;
//   * per group, each 16x16 block runs a four-instruction 16x16x32 chain
//     into a scratch accumulator that is then scaled by the group's fp32
//     scale and added to the running fp32 total (exact products, fp32 sums,
//     as in the decode kernel). INT4 codes expand to 128 + u; the bias
//     136 * sum x is one more chain per 16-row block, evaluated with the
//     same instruction and operand order, so zero-code columns cancel to 0.
// Tiles are mapped so that each XCD (workgroups are dealt to the eight XCDs
// round-robin) walks a contiguous run of tiles with the column tile fastest:
// the 128-row x slice it is working on stays in that XCD's L2 while the
// packed weight streams past.
#include "qg_device.h"
#include "qg_internal.h"

namespace qg {
namespace {

constexpr int kBM = 128;             // rows per workgroup tile
constexpr int kBNB = 8;              // 16-column blocks per workgroup tile (128 columns)
constexpr int kThreads = 256;        // four wavefronts, 2 x 2 over the tile
constexpr int kRowBlocks = kBM / 16;
constexpr int kXcds = 8;

__device__ __forceinline__ bf16x8 int4_to_biased(uint32_t w, uint32_t magic) {
  const u32x4 r = {(w & 0x000F000Fu) | magic, ((w >> 4) & 0x000F000Fu) | magic,
                   ((w >> 8) & 0x000F000Fu) | magic, ((w >> 12) & 0x000F000Fu) | magic};
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ uint32_t opaque_bias_magic() {
  uint32_t m = 0x43004300u;
  asm volatile("" : "+v"(m));
  return m;
}

template <int BITS, bool SBF>
__global__ __launch_bounds__(kThreads, 2) void gemm_prefill_kernel(
    const uint16_t* __restrict__ x, const char* __restrict__ packed,
    const uint16_t* __restrict__ scales, uint16_t* __restrict__ out, int M, int K, int N,
    int tiles_n, int tiles) {
  constexpr int TB = (BITS == 4) ? 1024 : 2048;   // bytes per packed tile
  constexpr int TW = TB / 1024;                   // 16-byte words per lane per tile
  // LDS: two buffers of [row block 8][K step 4][lane 64] 16-byte words.
  __shared__ u32x4 xs[2][kRowBlocks * 4 * 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1;        // which 64-row half
  const int wn = wave & 1;         // which 64-column half
  const int l16 = lane & 15;
  const int lq = lane >> 4;
  const int G = K >> 7;
  const int NB = N >> 4;

  // XCD-aware tile order: workgroup b runs on XCD b % 8; give each XCD a
  // contiguous range of tiles (identity on the ragged tail).
  int t = blockIdx.x;
  const int t8 = tiles / kXcds * kXcds;
  if (t < t8) t = (t % kXcds) * (t8 / kXcds) + t / kXcds;
  const int tm = t / tiles_n;
  const int tn = t - tm * tiles_n;
  const int m0 = tm * kBM;
  const int cb_base = tn * kBNB + wn * 4;          // this wave's first column block

  int cb[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) cb[c] = min(cb_base + c, NB - 1);   // clamped for loads

  const uint32_t magic = opaque_bias_magic();

  // x staging: each wave fills 8 of the 32 (row block, K step) blocks of a
  // group; lane l of a block holds row 16*rb + l%16, K 32*j + 8*(l/16) .. +7.
  // Rows past M are clamped to M - 1 (their outputs are never stored).
  auto stage_x = [&](int g, int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int blk = wave * 8 + i;               // = rb * 4 + j
      const int rb = blk >> 2;
      const int j = blk & 3;
      const int row = min(m0 + rb * 16 + l16, M - 1);
      const uint16_t* src = x + (int64_t)row * K + (int64_t)g * 128 + 32 * j + 8 * lq;
      __builtin_amdgcn_global_load_lds(
          src, (__attribute__((address_space(3))) void*)(&xs[buf][blk * 64]), 16, 0, 0);
    }
  };
  auto load_b = [&](int g, u32x4 (&bt)[4][TW], uint32_t (&sc)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const char* tp = packed + ((int64_t)cb[c] * G + g) * TB + lane * (TB / 64);
#pragma unroll
      for (int v = 0; v < TW; ++v) bt[c][v] = *reinterpret_cast<const u32x4*>(tp + 16 * v);
      sc[c] = scales[(int64_t)g * N + cb[c] * 16 + l16];
    }
  };

  f32x4 acc[4][4];   // [column block][row block]
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[c][r] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 bcur[4][TW], bnext[4][TW];
  uint32_t scur[4], snext[4];
  stage_x(0, 0);
  load_b(0, bcur, scur);

  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    // This group's x and weights have landed (direct-to-LDS loads count in
    // the vector-memory counter), and every wave is done with the other
    // buffer, which the next group overwrites.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (g + 1 < G) {
      stage_x(g + 1, buf ^ 1);
      load_b(g + 1, bnext, snext);
    }

    // A fragments of this wave's four row blocks, all four K steps.
    bf16x8 a[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        a[r][j] = __builtin_bit_cast(bf16x8, xs[buf][((wm * 4 + r) * 4 + j) * 64 + lane]);

    f32x4 bias[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      bias[r] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (BITS == 4) {
        const bf16x8 b136 = bias136_bf16x8();
#pragma unroll
        for (int j = 0; j < 4; ++j) bias[r] = mfma16x16x32(a[r][j], b136, bias[r]);
      }
    }

#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x8 bw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (BITS == 4) {
          bw[j] = int4_to_biased(bcur[c][0][j], magic);
        } else {
          const u32x4& w = bcur[c][j >> 1];
          bw[j] = int8_words_to_bf16(w[(j & 1) * 2], w[(j & 1) * 2 + 1]);
        }
      }
      const float s = SBF ? bf16_bits_to_f32(scur[c]) : f16_bits_to_f32(scur[c]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) p = mfma16x16x32(a[r][j], bw[j], p);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[c][r][e] = fmaf(s, p[e] - bias[r][e], acc[c][r][e]);
      }
    }

#pragma unroll
    for (int c = 0; c < 4; ++c) {
      scur[c] = snext[c];
#pragma unroll
      for (int v = 0; v < TW; ++v) bcur[c][v] = bnext[c][v];
    }
  }

  // C layout of a 16x16 block: lane holds column l16, rows 4*lq + e.
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (cb_base + c >= NB) continue;
    const int n = (cb_base + c) * 16 + l16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wm * 64 + r * 16 + 4 * lq + e;
        if (row < M) out[(int64_t)row * N + n] = f32_to_bf16_bits(acc[c][r][e]);
      }
    }
  }
}

}  // namespace

bool make_prefill_plan(int64_t M, int64_t K, int64_t N, PrefillPlan* plan) {
  (void)K;
  const int64_t tiles_m = (M + kBM - 1) / kBM;
  const int64_t tiles_n = (N / kTileCols + kBNB - 1) / kBNB;
  const int64_t tiles = tiles_m * tiles_n;
  if (tiles > 0x7FFFFFFF) return false;
  plan->tiles_n = (int)tiles_n;
  plan->tiles = (int)tiles;
  return true;
}

hipError_t launch_gemm_prefill(int bits, const PrefillPlan& p, const void* x, const void* packed,
                               const void* scales, bool s_bf16, void* out, int64_t M, int64_t K,
                               int64_t N, hipStream_t st) {
  const dim3 grid((unsigned)p.tiles);
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* wp = static_cast<const char*>(packed);
  const auto* sp = static_cast<const uint16_t*>(scales);
  auto* op = static_cast<uint16_t*>(out);
  const int m = (int)M, k = (int)K, n = (int)N;
  if (bits == 4) {
    if (s_bf16) gemm_prefill_kernel<4, true><<<grid, kThreads, 0, st>>>(xp, wp, sp, op, m, k, n, p.tiles_n, p.tiles);
    else        gemm_prefill_kernel<4, false><<<grid, kThreads, 0, st>>>(xp, wp, sp, op, m, k, n, p.tiles_n, p.tiles);
  } else {
    if (s_bf16) gemm_prefill_kernel<8, true><<<grid, kThreads, 0, st>>>(xp, wp, sp, op, m, k, n, p.tiles_n, p.tiles);
    else        gemm_prefill_kernel<8, false><<<grid, kThreads, 0, st>>>(xp, wp, sp, op, m, k, n, p.tiles_n, p.tiles);
  }
  return hipGetLastError();
}

}  // namespace qg

// Large-M group-quantized GEMM (prefill, e.g. the 8,192-token Long setting
// of the speed paragraph of arXiv 2607.04244):
//   out[m, n] = bf16( sum_g s[g, n] * sum_{k in g} x[m, k] * q[k, n] )
//
// At M = 8192 the product is a dense contraction (~2,000 flop per HBM byte):
// the bound is the bf16 matrix core, and what keeps the kernel from it is
// (a) the per-CU load path (about 55 bytes per clock), (b) the vector ALU
// work of unpacking codes and applying the per-group scale, and (c) waiting.
//   * A workgroup of WN wavefronts computes a 64 x (64 WN) output tile; each
//     wavefront a 64 x 64 sub-tile as a 2 x 2 grid of 32x32 blocks, with
//     32x32x16 products: each one does twice the work of a 16x16x32 product
//     on the same operand registers (half the matrix instructions and
//     operand reads per group; measured 3-5% faster than 4 x 4 blocks of
//     16x16, outputs bit-identical). Two or more workgroups share a CU, so
//     while one waits at its barrier the other keeps the matrix core busy.
//   * The K loop steps one scale group (128) at a time through a ring of
//     LDS stages. A stage holds the group's x (64 rows, in the lane order of
//     the 16x16x32 A operand), the 4 WN packed weight tiles (in the 16x16x32
//     B-operand lane order of the packed format), the group's scales and the
//     64 negated INT4 offsets. The 32x32x16 operands are read from the same
//     layout with their own per-lane offsets: lane L takes row (column)
//     32 h + L % 32 and K slice 16 s + 8 (L / 32) of step s, which the
//     16x16 order holds in row (column) block 2 h + (L % 32) / 16, lane
//     L % 16 + 16 (2 (s % 2) + L / 32), word s / 2. Every byte arrives by a buffer load straight into LDS whose
//     per-lane offset is fixed for the whole K loop (the group enters as the
//     scalar offset, so a stage costs no address arithmetic; 4% faster than
//     per-load 64-bit addresses at 8192 x 2560 x 19456), and every
//     wavefront issues the same number of them per stage, so "this stage
//     has landed" is one vmcnt wait with a constant count and one barrier.
//   * INT4 codes expand to bf16 128 + u with one and-or per pair; the
//     offset 136 * sum_k x is computed once per (row, group) by a small
//     pre-pass (a 16x16x32 chain over constant B) and stored negated, and it
//     seeds each block's chain of products. The group total then leaves the
//     matrix core as sum x * q, and one fma per element applies the fp32
//     scale into the fp32 running sum (exact products, fp32 sums).
// Tiles are mapped so that each XCD (workgroups are dealt to the eight XCDs
// round-robin) walks its own rows of tiles in panels of eight column tiles:
// the x slices and weight tiles of the workgroups resident on an XCD at one
// time stay in that XCD's L2.
#include "qg_device.h"
#include "qg_internal.h"

namespace qg {
namespace {

constexpr int kBM = kPrefillRows;            // rows per workgroup tile
constexpr int kXcds = 8;
constexpr int kPanel = 8;                    // column tiles per panel of the tile walk
constexpr int kXBytes = kBM * kGroup * 2;    // one group of x for the tile: 16 KiB

// One ring stage: x [16 blocks of 1 KiB], the 4 WN weight tiles, and per
// wavefront 256 bytes of side data (64 scales, then 64 / WN negated offsets).
template <int BITS, int WN, int NST>
struct Stage {
  static constexpr int kTile = (BITS == 4) ? 1024 : 2048;   // packed bytes per 16 x 128 tile
  static constexpr int kB = kXBytes;                        // offset of the weight tiles
  static constexpr int kSide = kB + 4 * WN * kTile;         // offset of the side data
  static constexpr int kBytes = kSide + 256 * WN;
  static constexpr int kXLoads = 16 / WN;
  static constexpr int kBLoads = 4 * kTile / 1024;
  static constexpr int kLoads = kXLoads + kBLoads + (BITS == 4 ? 2 : 1);   // loads per wavefront per stage
  static constexpr int kRowsPerWave = kBM / WN;             // offsets loaded by one wavefront
};

typedef __attribute__((address_space(3))) void* lds_ptr;

// A buffer resource over [base, base + bytes); loads past the end read zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t prefill_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// One 16-byte-per-lane buffer load straight into LDS: lane l's bytes land at
// dst + 16 l.
__device__ __forceinline__ void to_lds(__amdgpu_buffer_rsrc_t r, char* dst, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)dst, 16, voff, soff, 0, 0);
}

// The INT4 expansion constant in a vector register (so the mask takes the
// one scalar slot of the AND-OR); the empty asm emits no instruction.
__device__ __forceinline__ uint32_t opaque_magic(uint32_t m) {
  asm volatile("" : "+v"(m));
  return m;
}

// Where one wavefront's share of every stage comes from. The per-lane byte
// offsets are fixed for the whole K loop; group g enters only through the
// scalar offset of each load. Wavefront w loads 16 / WN x blocks (row block,
// K step), its four weight tiles (one 1 KiB piece per load), the scales of
// its 64 columns (lanes 0-7) and, INT4 only, the negated offsets of its
// 64 / WN rows (lanes 8..). Rows past M re-read row M - 1 and columns past N
// the last block: both are computed but never stored.
template <int BITS, int WN, int NST>
struct StageSrc {
  using S = Stage<BITS, WN, NST>;
  __amdgpu_buffer_rsrc_t xr, cr, sr, br;
  int xo[S::kXLoads], co[S::kBLoads], so, bo;
  int sstep, bstep;   // scale and offset bytes per group

  __device__ __forceinline__ StageSrc(const uint16_t* x, const char* packed, const uint16_t* scales,
                                      const float* nbias, int wave, int lane, int m0, int cb0,
                                      int M, int K, int N, int NB, int G, int Mp, int scbm) {
    const int rows = min(M - m0, kBM);
    xr = prefill_rsrc(x + (int64_t)m0 * K, (int64_t)rows * K * 2);
#pragma unroll
    for (int i = 0; i < S::kXLoads; ++i) {
      const int blk = wave * S::kXLoads + i;   // = row block * 4 + K step
      xo[i] = min(16 * (blk >> 2) + (lane & 15), rows - 1) * K * 2 + 64 * (blk & 3) + 16 * (lane >> 4);
    }
    const int ncb = min(4 * WN, NB - cb0);
    cr = prefill_rsrc(packed + (int64_t)cb0 * G * S::kTile, (int64_t)ncb * G * S::kTile);
#pragma unroll
    for (int i = 0; i < S::kBLoads; ++i) {
      const int piece = wave * S::kBLoads + i;
      const int cbl = min(piece / (S::kTile / 1024), ncb - 1);
      co[i] = cbl * G * S::kTile + (piece % (S::kTile / 1024)) * 1024 + lane * 16;
    }
    // Logical scales: row g of [G, N]; column-block-major: the run of the
    // column's 16-wide block (qg_prepack_scales).
    const int col = min(cb0 * 16 + 64 * wave + 8 * (lane & 7), N - 8);
    sr = prefill_rsrc(scales, (int64_t)G * N * 2);
    so = scbm ? ((col >> 4) * G * 16 + (col & 15)) * 2 : col * 2;
    sstep = scbm ? 32 : N * 2;
    br = prefill_rsrc(nbias, (int64_t)G * Mp * 4);
    bo = (m0 + S::kRowsPerWave * wave + 4 * max(lane - 8, 0)) * 4;
    bstep = Mp * 4;
  }

  __device__ __forceinline__ void fill(char* st, int g, int wave, int lane) const {
#pragma unroll
    for (int i = 0; i < S::kXLoads; ++i)
      to_lds(xr, st + (wave * S::kXLoads + i) * 1024, xo[i], g * (kGroup * 2));
#pragma unroll
    for (int i = 0; i < S::kBLoads; ++i)
      to_lds(cr, st + S::kB + (wave * S::kBLoads + i) * 1024, co[i], g * S::kTile);
    constexpr int kBiasLanes = (BITS == 4) ? S::kRowsPerWave / 4 : 0;
    if (lane < 8) to_lds(sr, st + S::kSide + 256 * wave, so, g * sstep);
    else if (lane < 8 + kBiasLanes) to_lds(br, st + S::kSide + 256 * wave, bo, g * bstep);
  }
};

template <int BITS, bool SBF, bool XH, int WN, int NST>
__global__ __launch_bounds__(64 * WN) __attribute__((amdgpu_waves_per_eu(2))) void gemm_prefill_kernel(
    const uint16_t* __restrict__ x, const char* __restrict__ packed,
    const uint16_t* __restrict__ scales, const float* __restrict__ nbias,
    uint16_t* __restrict__ out, int M, int K, int N, int Mp, int tiles_n, int tiles, int scbm) {
  using S = Stage<BITS, WN, NST>;
  using A = Act<XH>;
  extern __shared__ u32x4 smem[];
  char* const lds = reinterpret_cast<char*>(smem);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // column quarter / half
  const int l16 = lane & 15;
  const int G = K >> 7;
  const int NB = N >> 4;

  // XCD-aware tile order: workgroup b runs on XCD b % 8; give each XCD a
  // contiguous range of tiles (identity on the ragged tail). When that range
  // is whole tile rows, walk it in panels of kPanel column tiles, so the
  // workgroups resident on one XCD at a time (~8 rows x 8 columns of tiles)
  // share both their x slices and their weight tiles in that XCD's L2
  // (measured +4% at 8192 x 2560 x 19456).
  int t = blockIdx.x;
  const int t8 = tiles / kXcds * kXcds;
  const int per = t8 / kXcds;
  int tm, tn;
  if (t < t8 && per % tiles_n == 0) {
    const int xcd = t % kXcds, i = t / kXcds;
    const int rows_x = per / tiles_n;
    const int full = tiles_n / kPanel;
    if (i < full * kPanel * rows_x) {
      const int pn = i / (rows_x * kPanel), j = i - pn * rows_x * kPanel;
      tm = xcd * rows_x + j / kPanel;
      tn = pn * kPanel + j % kPanel;
    } else {   // the last, narrower panel
      const int j = i - full * kPanel * rows_x, wt = tiles_n - full * kPanel;
      tm = xcd * rows_x + j / wt;
      tn = full * kPanel + j % wt;
    }
  } else {
    if (t < t8) t = (t % kXcds) * per + t / kXcds;
    tm = t / tiles_n;
    tn = t - tm * tiles_n;
  }
  const int m0 = tm * kBM;
  const int cb0 = tn * 4 * WN;

  const uint32_t magic = opaque_magic(A::kMagic);

  f32x16 acc[2][2];   // [32-column half][32-row half]
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[c][r][i] = 0.0f;
  // Per-lane stage offsets of the 32x32x16 operands (see the header).
  const int hb = (lane & 31) >> 4;                          // 16-block within a 32-half
  const int lp = ((lane & 15) + 16 * (lane >> 5)) * 16;     // piece of the even K16 steps
  const int a_off = hb * 4096 + lp;

  const StageSrc<BITS, WN, NST> src(x, packed, scales, nbias, wave, lane, m0, cb0, M, K, N, NB, G, Mp,
                                   scbm);
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < G) src.fill(lds + s * S::kBytes, s, wave, lane);

  int cur = 0;   // ring slot of group g
  for (int g = 0; g < G; ++g) {
    // Group g's stage has landed once only the loads of later stages (if
    // any were issued) are outstanding; the barrier then publishes every
    // wavefront's part and tells that all of them are done with the slot
    // that the load below overwrites.
    if (NST == 3 && g + 1 < G)
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(S::kLoads) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    const int ahead = g + NST - 1;
    if (ahead < G) {
      const int slot = (cur == 0) ? NST - 1 : cur - 1;
      src.fill(lds + slot * S::kBytes, ahead, wave, lane);
    }
    const char* st = lds + cur * S::kBytes;
    cur = (cur == NST - 1) ? 0 : cur + 1;

    // A operand of step s for row half R: x rows 32 R + L % 32, K 16 s + 8 (L / 32).
    u32x4 a[2][8];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8)
        a[r][s8] = *reinterpret_cast<const u32x4*>(st + a_off + r * 8192 + (s8 >> 1) * 1024 +
                                                   (s8 & 1) * 512);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      // B operand of step s for column half c: codes of column 32 c + L % 32.
      u32x4 bw[8];
      if constexpr (BITS == 4) {
        const char* tp = st + S::kB + (wave * 4 + 2 * c + hb) * 1024 + lp;
        const u32x4 we = *reinterpret_cast<const u32x4*>(tp);
        const u32x4 wo = *reinterpret_cast<const u32x4*>(tp + 512);
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) bw[s8] = int4_word_to_act((s8 & 1) ? wo[s8 >> 1] : we[s8 >> 1], magic);
      } else {
        const char* tp = st + S::kB + (wave * 4 + 2 * c + hb) * 2048 + 2 * lp;
        const u32x4 e0 = *reinterpret_cast<const u32x4*>(tp);
        const u32x4 e1 = *reinterpret_cast<const u32x4*>(tp + 16);
        const u32x4 o0 = *reinterpret_cast<const u32x4*>(tp + 1024);
        const u32x4 o1 = *reinterpret_cast<const u32x4*>(tp + 1040);
        bw[0] = int8_words_to_act<A>(e0[0], e0[1]);
        bw[1] = int8_words_to_act<A>(o0[0], o0[1]);
        bw[2] = int8_words_to_act<A>(e0[2], e0[3]);
        bw[3] = int8_words_to_act<A>(o0[2], o0[3]);
        bw[4] = int8_words_to_act<A>(e1[0], e1[1]);
        bw[5] = int8_words_to_act<A>(o1[0], o1[1]);
        bw[6] = int8_words_to_act<A>(e1[2], e1[3]);
        bw[7] = int8_words_to_act<A>(o1[2], o1[3]);
      }
      const uint32_t sraw =
          *reinterpret_cast<const uint16_t*>(st + S::kSide + 256 * wave + (32 * c + (lane & 31)) * 2);
      const float sc = SBF ? bf16_bits_to_f32(sraw) : f16_bits_to_f32(sraw);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        // INT4: the chain starts from the rows' negated offsets (C layout of a
        // 32x32 block: lane L holds rows 8 (i / 4) + 4 (L / 32) + i % 4).
        f32x16 p;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 sd = f32x4{0.f, 0.f, 0.f, 0.f};
          if constexpr (BITS == 4) {
            const int rr = 32 * r + 8 * q4 + 4 * (lane >> 5);
            sd = *reinterpret_cast<const f32x4*>(st + S::kSide + 256 * (rr / S::kRowsPerWave) + 128 +
                                                 4 * (rr % S::kRowsPerWave));
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) p[4 * q4 + e] = sd[e];
        }
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) p = A::mma32(a[r][s8], bw[s8], p);
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[c][r][i] = fmaf(sc, p[i], acc[c][r][i]);
      }
    }
  }



  // C layout of a 32x32 block: lane L holds column L % 32, rows 8 (i / 4) + 4 (L / 32) + i % 4.
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int cb = cb0 + wave * 4 + 2 * c + hb;
    if (cb >= NB) continue;
    const int n = cb * 16 + l16;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = m0 + 32 * r + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        if (row < M) out[(int64_t)row * N + n] = A::out(acc[c][r][i]);
      }
    }
  }
}

// Negated INT4 offsets: nbias[g * Mp + m] = -(c * sum_{k in g} x[m, k]) with
// c = 136 (bf16 activations) or 1032 (fp16),
// formed by a 16x16x32 chain (four K steps of 32, from zero); the main
// kernel's chains of products start from it. One wavefront per (16-row block, run of
// kBiasGroups groups), all of its x loads issued before the first multiply;
// rows from M to Mp repeat row M - 1.
constexpr int kBiasGroups = 4;

template <bool XH>
__global__ __launch_bounds__(256) void prefill_bias_kernel(const uint16_t* __restrict__ x,
                                                           float* __restrict__ nbias, int M, int K,
                                                           int Mp, int units) {
  const int lane = threadIdx.x & 63;
  const int u = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (u >= units) return;
  const int RB = Mp >> 4;
  const int G = K >> 7;
  const int gc = u / RB;
  const int rb = u - gc * RB;
  const int row = min(rb * 16 + (lane & 15), M - 1);
  const uint16_t* src = x + (int64_t)row * K + 8 * (lane >> 4);
  using A = Act<XH>;
  u32x4 a[kBiasGroups][4];
#pragma unroll
  for (int i = 0; i < kBiasGroups; ++i) {
    const int g = min(gc * kBiasGroups + i, G - 1);   // past G: re-read, not stored
#pragma unroll
    for (int j = 0; j < 4; ++j)
      a[i][j] = *reinterpret_cast<const u32x4*>(src + g * kGroup + 32 * j);
  }
  const u32x4 off = {A::kOffset, A::kOffset, A::kOffset, A::kOffset};
#pragma unroll
  for (int i = 0; i < kBiasGroups; ++i) {
    const int g = gc * kBiasGroups + i;
    f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) p = A::mma(a[i][j], off, p);
    if (g < G && (lane & 15) == 0)
      *reinterpret_cast<f32x4*>(nbias + (int64_t)g * Mp + rb * 16 + 4 * (lane >> 4)) = -p;
  }
}

template <int BITS, bool SBF, bool XH, int WN, int NST>
void launch_main(const PrefillPlan& p, const uint16_t* x, const char* w, const uint16_t* s,
                 const float* nb, uint16_t* out, int M, int K, int N, int scbm, hipStream_t st) {
  gemm_prefill_kernel<BITS, SBF, XH, WN, NST>
      <<<dim3((unsigned)p.tiles), 64 * WN, NST * Stage<BITS, WN, NST>::kBytes, st>>>(
          x, w, s, nb, out, M, K, N, (int)p.mp, p.tiles_n, p.tiles, scbm);
}

template <int BITS, bool SBF, bool XH>
void launch_bits(const PrefillPlan& p, const uint16_t* x, const char* w, const uint16_t* s,
                 const float* nb, uint16_t* out, int M, int K, int N, int scbm, hipStream_t st) {
  if (p.wn == 4) launch_main<BITS, SBF, XH, 4, 2>(p, x, w, s, nb, out, M, K, N, scbm, st);
  else           launch_main<BITS, SBF, XH, 2, 2>(p, x, w, s, nb, out, M, K, N, scbm, st);
}

}  // namespace

hipError_t launch_gemm_prefill(int bits, const PrefillPlan& p, const void* x, bool x_f16,
                               const void* packed, const void* scales, bool s_bf16, bool s_cbm,
                               void* out, int64_t M, int64_t K, int64_t N, void* ws,
                               hipStream_t st) {
  const int scbm = s_cbm ? 1 : 0;
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* wp = static_cast<const char*>(packed);
  const auto* sp = static_cast<const uint16_t*>(scales);
  auto* op = static_cast<uint16_t*>(out);
  const int m = (int)M, k = (int)K, n = (int)N;
  if (bits == 4) {
    // The offsets sit after the arrival counters, which stay untouched.
    float* nb = reinterpret_cast<float*>(static_cast<char*>(ws) + kCounterBytes);
    const int units = (int)(p.mp / 16 * ((K / kGroup + kBiasGroups - 1) / kBiasGroups));
    const dim3 bgrid((unsigned)((units + 3) / 4));
    if (x_f16) prefill_bias_kernel<true><<<bgrid, 256, 0, st>>>(xp, nb, m, k, (int)p.mp, units);
    else       prefill_bias_kernel<false><<<bgrid, 256, 0, st>>>(xp, nb, m, k, (int)p.mp, units);
    if (x_f16) {
      if (s_bf16) launch_bits<4, true, true>(p, xp, wp, sp, nb, op, m, k, n, scbm, st);
      else        launch_bits<4, false, true>(p, xp, wp, sp, nb, op, m, k, n, scbm, st);
    } else {
      if (s_bf16) launch_bits<4, true, false>(p, xp, wp, sp, nb, op, m, k, n, scbm, st);
      else        launch_bits<4, false, false>(p, xp, wp, sp, nb, op, m, k, n, scbm, st);
    }
  } else {
    if (x_f16) {
      if (s_bf16) launch_bits<8, true, true>(p, xp, wp, sp, nullptr, op, m, k, n, scbm, st);
      else        launch_bits<8, false, true>(p, xp, wp, sp, nullptr, op, m, k, n, scbm, st);
    } else {
      if (s_bf16) launch_bits<8, true, false>(p, xp, wp, sp, nullptr, op, m, k, n, scbm, st);
      else        launch_bits<8, false, false>(p, xp, wp, sp, nullptr, op, m, k, n, scbm, st);
    }
  }
  return hipGetLastError();
}

}  // namespace qg

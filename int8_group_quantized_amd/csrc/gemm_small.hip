// Small-M group-quantized GEMM (decode M = 1, verification blocks M <= 16):
//   out[m, n] = bf16( sum_g s[g, n] * sum_{k in g} x[m, k] * q[k, n] )
// (arXiv 2607.04244, QAD paragraph: the served weight is s (.) W_q; group of
// 128 along K per the drafter-PTQ paragraph; INT8 variant per the W8A16
// model card.)
//
// The path is HBM-bound: 0.5 (INT4) or 1 (INT8) byte per weight streams once
// from memory. With about one wavefront per SIMD, every vector instruction a
// wavefront issues costs four cycles of its SIMD, so the kernel is built to
// keep loads in flight and to spend as few vector instructions per 1 KiB tile
// as the arithmetic allows:
//   * a wavefront owns NBW 16-column blocks and a contiguous run of K groups,
//     walked in batches of D groups held in two register buffers: while one
//     batch is multiplied the next is being fetched. Each tile is one
//     16-byte buffer load per lane (a tile is contiguous, so the load is a
//     fully coalesced 1 KiB transaction) through a per-wavefront buffer
//     resource that covers exactly the wavefront's remaining groups, so a
//     fetch past the last group returns zeros without touching memory. The
//     loop body is therefore straight-line code with no redundant traffic,
//     and the wait counters keep a fixed number of loads in flight;
//   * the workgroup stages its slice of x in LDS with direct global->LDS
//     loads, in the lane order of the matrix-core A operand, with rows >= M
//     stored as zeros (MR = 16) or read from a zero block (MR = 1), so each
//     group is four unconditional 16-byte LDS reads at immediate offsets.
//     The scales of the workgroup's column blocks follow in one sweep of
//     16-byte direct loads. The staging loads go out before the weight
//     tiles, so waiting for them does not wait for the tiles;
//   * codes expand in registers to exact bf16 integers (seven ALU ops per
//     eight INT4 codes, twelve per eight INT8 codes); four 16x16x32 bf16
//     matrix-core ops give a group's fp32 partial sums for 16 rows x 16
//     columns, and the group's fp32 scale is applied with one FMA per output.
// The matrix cores carry the contraction because the vector ALUs cannot: at
// M = 16 the path needs ~1.8e14 multiply-adds/s to keep pace with HBM, twice
// the fp32 vector peak, and the 16-row matrix op fits M = 16 exactly; M = 1
// uses the same op with one live row (its cost hides under the loads).
//
// INT4 codes expand as 128 + u with u = q + 8 (one AND-OR per pair). The bias
// 136 * sum_k x[m, k] is the same 16x16x32 product with every code equal to
// 136, evaluated with the same instruction and operand order as the code
// product, so a column whose codes are all zero cancels to exactly 0.
//
// Reductions are deterministic: WK wavefronts of a workgroup that split K are
// summed through LDS in wave order; `splits` workgroups along K publish fp32
// partials with device-coherent stores, count arrivals with one atomic, and
// the last to arrive sums the partials in split order (no whole-cache flush
// or invalidate is needed: the partials never sit in a non-coherent cache).
#include <algorithm>

#include "qg_device.h"
#include "qg_internal.h"

namespace qg {
namespace {


// Device-coherent (agent scope: sc1, past the per-XCD L2) 16-byte accesses
// for the split-K partials, through a buffer resource whose range check turns
// an offset at or past 2^31 into a zero read.
constexpr int kCoherent = 16;
constexpr uint32_t kNoRead = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(float* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(p, 0, (int)bytes, 0x00020000);
}

// The INT4 expansion constant held in a vector register the optimiser cannot
// fold back into a literal, so the compiler selects one AND-OR per pair (a
// three-operand vector op may read only one scalar or constant operand, and
// the mask takes that slot). The empty asm emits no instruction.
__device__ __forceinline__ uint32_t opaque_magic(uint32_t m) {
  asm volatile("" : "+v"(m));
  return m;
}

// s_waitcnt immediate (gfx9 encoding) for "at most n vector-memory loads
// outstanding, all LDS operations done". Issued through the builtin so that
// the compiler's own wait-count tracking sees it.
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// Raw buffer resource (no stride, no swizzle): loads at byte offsets at or
// past num_records return zeros and make no memory access.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}

template <int BITS>
struct Tile {
  static constexpr int bytes = (BITS == 4) ? 1024 : 2048;
  static constexpr int words = bytes / 1024;   // 16-byte words per lane
  // Cache policy of the tile loads: INT4 tiles, read exactly once, stream
  // with the nontemporal hint (measured 2-3% faster at M = 1 and 16); the
  // same hint made the INT8 M = 16 gate/up GEMM 12.9 -> 16.5 µs, so INT8
  // tiles load with the default policy.
  static constexpr int aux = (BITS == 4) ? 2 : 0;
};

// Groups per batch: two batches of D x NBW tiles stay in registers, and a
// batch's tiles of one column block sit within the 4 KiB immediate-offset
// reach of a load instruction.
template <int BITS, int NBW, int MR>
struct Batch {
  // Two column blocks at M = 1 (five groups per wavefront in the decode
  // plans) take batches of three so that two batches cover them exactly.
  static constexpr int D = (BITS == 4) ? (NBW == 1 ? 4 : (NBW == 2 ? (MR == 1 ? 3 : 2) : 1))
                                       : (NBW == 4 ? 1 : 2);
};

template <int BITS, bool SBF, bool XH, bool GR, int MR, int NBW, int WN, int WK>
__global__ __launch_bounds__(64 * WN * WK, 2) void gemm_small_kernel(
    const uint16_t* __restrict__ x, uint32_t* __restrict__ counters,
    float* __restrict__ partials, int M, int K, int splits, int gps, int sg, int scbm,
    const GroupArgs ga) {
  constexpr int NT = 64 * WN * WK;
  constexpr int NW = WN * WK;
  constexpr int TB = Tile<BITS>::bytes;
  constexpr int TW = Tile<BITS>::words;
  constexpr int D = Batch<BITS, NBW, MR>::D;
  constexpr int XG = (MR == 1) ? 16 : 256;   // LDS 16-byte words of x per group
  constexpr int CBW = WN * NBW;               // column blocks of the workgroup
  using A = Act<XH>;
  extern __shared__ u32x4 smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % WN;
  const int wk = wave / WN;
  // The GEMM of the group this workgroup belongs to (a scalar search over at
  // most 16 prefix entries); a single GEMM is item 0, read at fixed offsets.
  int item = 0;
  if constexpr (GR) {
    for (int i = 1; i < ga.count; ++i)
      if ((int)blockIdx.x >= ga.item[i].wg_first) item = i;
  }
  const GroupItem& it = ga.item[item];
  const int N = it.n;
  const int wg0 = GR ? it.wg_first : 0;
  const int colp = GR ? it.col_first : 0;
  const char* packed = it.packed;
  const uint16_t* scales = it.scales;
  uint16_t* out = it.out;
  const int G = K >> 7;
  const int NB = N >> 4;
  const int cb0 = (((int)blockIdx.x - wg0) * WN + wn) * NBW;
  const int nvalid = min(NBW, NB - cb0);     // column blocks this wave owns (may be <= 0)
  const int split = blockIdx.y;
  const int row0 = blockIdx.z * 16;
  const int mrows = min(16, M - row0);       // live rows in this 16-row block
  const int wg_g0 = split * gps;             // first group of the workgroup
  const int wg_gn = min(G, wg_g0 + gps) - wg_g0;
  const int l16 = lane & 15;                 // A row / C column of this lane
  const int lq = lane >> 4;                  // K slice (A, B) / row quad (C)
  u32x4* xs = smem;                          // [sg][XG] x fragments, then a zero block (MR == 1)
  // The scales of the workgroup's column blocks and groups follow: 32 bytes
  // (16 columns) per (column block, group), [CBW][sn] order.
  u32x4* ss = smem + sg * XG + 16;
  const uint32_t magic = opaque_magic(A::kMagic);

  int cb[NBW];
#pragma unroll
  for (int c = 0; c < NBW; ++c) cb[c] = min(cb0 + c, NB - 1);   // clamped: stays in range
  const int lane_off = lane * (TB / 64);
  // x fragment address of this lane for stage group 0, and its per-group step
  // (in 16-byte words); with MR == 1 only lanes of row 0 read data, the rest
  // read the zero block.
  const int xa_lane = (MR == 1) ? ((l16 == 0) ? lq : sg * XG) : lane;
  const int xa_step = (MR == 1) ? ((l16 == 0) ? XG : 0) : XG;

  f32x4 acc[NBW];
#pragma unroll
  for (int c = 0; c < NBW; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  {
    // One stage: the workgroup's whole K range is staged at once.
    constexpr int s0 = 0;
    const int sn = wg_gn;
    const int per = (sn + WK - 1) / WK;
    const int w_lo = min(sn, wk * per);
    const int w_n = min(sn, w_lo + per) - w_lo;   // may be 0 for trailing waves
    const int g_first = wg_g0 + s0 + w_lo;
    const int nbatch = (w_n + D - 1) / D;

    u32x4 ta[D][NBW][TW], tb[D][NBW][TW];
    const uint16_t* ssc = reinterpret_cast<const uint16_t*>(ss);
    // Batch b: groups g_first + b*D + d of each column block, through a
    // resource that ends at the wavefront's last group (later ones read 0).
    auto load_batch = [&](int b, u32x4 (&t)[D][NBW][TW]) {
      const int i0 = min(b * D, w_n);
      const int left = w_n - i0;                      // groups still in range
#pragma unroll
      for (int c = 0; c < NBW; ++c) {
        const __amdgpu_buffer_rsrc_t r =
            make_rsrc(packed + ((int64_t)cb[c] * G + g_first + i0) * TB, left * TB);
#pragma unroll
        for (int d = 0; d < D; ++d) {
#pragma unroll
          for (int v = 0; v < TW; ++v)
            t[d][c][v] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, lane_off + d * TB + 16 * v, 0,
                                                      Tile<BITS>::aux));
        }
      }
    };
    auto compute_batch = [&](int b, const u32x4 (&t)[D][NBW][TW]) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int i = b * D + d;                      // wave-relative group
        const bool live = i < w_n;
        const int gl = w_lo + min(i, w_n - 1);        // stage-relative group
        const u32x4* xp = xs + xa_lane + gl * xa_step;
        u32x4 a[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = xp[j * (XG / 4)];
        f32x4 bias = {0.f, 0.f, 0.f, 0.f};
        if constexpr (BITS == 4) {
          const u32x4 off = {A::kOffset, A::kOffset, A::kOffset, A::kOffset};
#pragma unroll
          for (int j = 0; j < 4; ++j) bias = A::mma(a[j], off, bias);
        }
#pragma unroll
        for (int c = 0; c < NBW; ++c) {
          f32x4 p = {0.f, 0.f, 0.f, 0.f};
          if constexpr (BITS == 4) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              p = A::mma(a[j], int4_word_to_act(t[d][c][0][j], magic), p);
          } else {
            p = A::mma(a[0], int8_words_to_act<A>(t[d][c][0][0], t[d][c][0][1]), p);
            p = A::mma(a[1], int8_words_to_act<A>(t[d][c][0][2], t[d][c][0][3]), p);
            p = A::mma(a[2], int8_words_to_act<A>(t[d][c][1][0], t[d][c][1][1]), p);
            p = A::mma(a[3], int8_words_to_act<A>(t[d][c][1][2], t[d][c][1][3]), p);
          }
          const uint32_t sbits = ssc[((wn * NBW + c) * sn + gl) * 16 + l16];
          const float sv = SBF ? bf16_bits_to_f32(sbits) : f16_bits_to_f32(sbits);
          const float scale = live ? sv : 0.0f;
          if constexpr (MR == 1) {
            // One live row: only element 0 of the lanes holding rows 0..3 is
            // ever stored, so the other three rows are not accumulated.
            acc[c][0] = fmaf(scale, p[0] - bias[0], acc[c][0]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[c][e] = fmaf(scale, p[e] - bias[e], acc[c][e]);
          }
        }
      }
    };

    {
      // Stage x with direct global->LDS loads: one wavefront instruction fills
      // one contiguous 1 KiB block of the layout (lane l -> 16 bytes at l*16).
      // Slots of rows >= M are written with zeros by the lanes that skip the
      // load, so no slot is written twice.
      const int total = sn * XG;                      // 16-byte words to fill
      // Zero slots first (rows >= M, and the zero block that rows >= 1 read
      // when MR == 1), then the direct loads, so no LDS write follows a
      // direct load that might still be landing.
      if constexpr (MR == 16) {
        if (mrows < 16)
          for (int e = tid; e < total; e += NT)
            if ((e & 15) >= mrows) xs[e] = u32x4{0u, 0u, 0u, 0u};
      } else {
        if (tid < 16) xs[sg * XG + tid] = u32x4{0u, 0u, 0u, 0u};
      }
      for (int w0 = wave * 64; w0 < total; w0 += NW * 64) {
        const int e = w0 + lane;
        int g, j, q, r;
        if constexpr (MR == 1) {
          g = e >> 4; j = (e >> 2) & 3; q = e & 3; r = 0;
        } else {
          g = e >> 8; j = (e >> 6) & 3; q = (e >> 4) & 3; r = e & 15;
        }
        if (e < total && r < mrows) {
          const uint16_t* src = x + (int64_t)(row0 + r) * K + (int64_t)(wg_g0 + s0 + g) * 128 +
                                32 * j + 8 * q;
          __builtin_amdgcn_global_load_lds(
              src, (__attribute__((address_space(3))) void*)(xs + w0), 16, 0, 0);
        }
      }
      // The scales, 16 bytes (8 columns) per lane: one sweep per workgroup
      // instead of a load per tile in every wavefront.
      const int stotal = CBW * sn * 2;
      for (int w0 = wave * 64; w0 < stotal; w0 += NW * 64) {
        const int e = w0 + lane;
        if (e < stotal) {
          const int cc = e / (2 * sn);
          const int rem = e - cc * 2 * sn;
          const int cbw = min(((int)blockIdx.x - wg0) * CBW + cc, NB - 1);
          // Logical scales: row g of [G, N]; column-block-major: the
          // block's run of G groups x 16 columns.
          const int gg = wg_g0 + s0 + (rem >> 1);
          const uint16_t* src = scbm ? scales + ((int64_t)cbw * G + gg) * 16 + 8 * (rem & 1)
                                     : scales + (int64_t)gg * N + cbw * 16 + 8 * (rem & 1);
          __builtin_amdgcn_global_load_lds(
              src, (__attribute__((address_space(3))) void*)(ss + w0), 16, 0, 0);
        }
      }
    }
    // The first tile batches go out after the staging loads (the empty asm
    // keeps the compiler from hoisting them); waiting until no more than
    // their count is outstanding then waits for the staging only, and the
    // zero slots written through LDS are complete before the barrier.
    // A fetch past the wavefront's last group reads zeros without touching
    // memory but still occupies the address unit like a real one, so one and
    // two batches (the common decode and verification shapes) take
    // straight-line paths that issue nothing beyond them; longer runs use the
    // pairwise pipeline, whose last pair fetches ahead past the end. Each
    // path has static wait counts (a load issued on only some paths would
    // make the compiler drain every load before each use).
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    constexpr int LB = D * NBW * TW;                  // loads per batch
    if (nbatch <= 1) {
      if (nbatch == 1) {
        load_batch(0, ta);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(LB));
      } else {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
      }
      asm volatile("s_barrier" ::: "memory");
      if (nbatch == 1) compute_batch(0, ta);
    } else if (nbatch == 2) {
      load_batch(0, ta);
      load_batch(1, tb);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * LB));
      asm volatile("s_barrier" ::: "memory");
      compute_batch(0, ta);
      __builtin_amdgcn_sched_barrier(0);
      compute_batch(1, tb);
    } else {
      load_batch(0, ta);
      load_batch(1, tb);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * LB));
      asm volatile("s_barrier" ::: "memory");
      int b = 0;
      for (; b + 1 < nbatch; b += 2) {
        compute_batch(b, ta);
        __builtin_amdgcn_sched_barrier(0);
        load_batch(b + 2, ta);
        __builtin_amdgcn_sched_barrier(0);
        compute_batch(b + 1, tb);
        __builtin_amdgcn_sched_barrier(0);
        load_batch(b + 3, tb);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (b < nbatch) compute_batch(b, ta);
    }
  }

  // Wavefronts that split K inside the workgroup: reduce through LDS (the x
  // slice is dead by now, so its space is reused after a barrier).
  if constexpr (WK > 1) {
    __syncthreads();
    f32x4* red = reinterpret_cast<f32x4*>(smem);       // [WK-1][WN][NBW][64]
    if (wk > 0) {
#pragma unroll
      for (int c = 0; c < NBW; ++c) red[(((wk - 1) * WN + wn) * NBW + c) * 64 + lane] = acc[c];
    }
    __syncthreads();
    if (wk == 0) {
      for (int w = 0; w < WK - 1; ++w) {
#pragma unroll
        for (int c = 0; c < NBW; ++c) {
          const f32x4 o = red[((w * WN + wn) * NBW + c) * 64 + lane];
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
            const int r = 4 * lq + e;
            if (r < mrows) out[(int64_t)(row0 + r) * N + n] = A::out(acc[c][e]);
          }
        }
      }
    }
    return;
  }

  // Partials in the accumulators' own lane order: 16-byte word
  // ((split * row blocks + row block) * NBT + column block) * 64 + lane holds
  // this lane's acc (column l16, rows 4 lq .. +3 of the 16-row block; NBT =
  // column blocks of all GEMMs of the call), so every store and every merge
  // load of a wavefront moves 1 KB of consecutive bytes.
  const uint32_t nbt = (uint32_t)ga.n_total >> 4;
  const uint32_t split_bytes = gridDim.z * nbt * 1024u;
  const __amdgpu_buffer_rsrc_t rp = part_rsrc(partials, splits * split_bytes);
  uint32_t poff[NBW];
#pragma unroll
  for (int c = 0; c < NBW; ++c)
    poff[c] = ((blockIdx.z * nbt + (uint32_t)(colp >> 4) + (uint32_t)(cb0 + (c < nvalid ? c : 0))) *
                   64u + (uint32_t)lane) * 16u;
  if (wk == 0) {
#pragma unroll
    for (int c = 0; c < NBW; ++c) {
      if (c < nvalid)
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{__float_as_uint(acc[c][0]), __float_as_uint(acc[c][1]),
                  __float_as_uint(acc[c][2]), __float_as_uint(acc[c][3])},
            rp, poff[c] + split * split_bytes, 0, kCoherent);
    }
  }
  // The coherent stores must have completed before the arrival is counted.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  __shared__ uint32_t s_last;
  const uint32_t cidx = blockIdx.z * gridDim.x + blockIdx.x;
  if (tid == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(&counters[cidx], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == (uint32_t)splits - 1u) ? 1u : 0u;
  }
  __syncthreads();
  if (s_last == 0u) return;
  if (wk == 0) {
    // Sum the partials in split order. The loads of U splits for all of the
    // lane's outputs are issued before any is added, so the merge costs one
    // memory round trip per U splits instead of one per load. One-block
    // wavefronts (the library's split-K plans, five or six splits) take all
    // splits in one round trip (M = 16 down GEMM 2% faster); wider ones keep
    // four, since the larger merge's registers slowed the M = 1 gate/up
    // kernel, which shares the instantiation, by 13%.
    constexpr int U = (NBW == 1) ? 8 : 4;
    f32x4 sum[NBW];
#pragma unroll
    for (int c = 0; c < NBW; ++c) sum[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sp0 = 0; sp0 < splits; sp0 += U) {
      u32x4 v[U][NBW];
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int c = 0; c < NBW; ++c)
          v[u][c] = __builtin_amdgcn_raw_buffer_load_b128(
              rp, (sp0 + u < splits && c < nvalid) ? poff[c] + (sp0 + u) * split_bytes : kNoRead,
              0, kCoherent);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int c = 0; c < NBW; ++c) {
#pragma unroll
          for (int e = 0; e < 4; ++e) sum[c][e] += __uint_as_float(v[u][c][e]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < NBW; ++c) {
      if (c < nvalid) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * lq + e < mrows)
            out[(int64_t)(row0 + 4 * lq + e) * N + (cb0 + c) * 16 + l16] = A::out(sum[c][e]);
      }
    }
  }
  if (tid == 0)   // ready for the next call on this workspace
    __hip_atomic_store(&counters[cidx], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int BITS, bool SBF, bool XH, bool GR, int MR, int NBW, int WN, int WK>
hipError_t launch_variant(const SmallPlan& p, const void* x, const GroupArgs& g, bool s_cbm,
                          int64_t M, int64_t K, void* ws, hipStream_t st) {
  const dim3 grid((unsigned)g.wg_total, (unsigned)p.splits, (unsigned)p.row_blocks);
  uint32_t* counters = nullptr;
  float* partials = nullptr;
  if (p.splits > 1) {
    counters = static_cast<uint32_t*>(ws);
    partials = reinterpret_cast<float*>(static_cast<char*>(ws) + kCounterBytes);
  }
  const size_t lds = small_plan_lds_bytes(p, M);
  gemm_small_kernel<BITS, SBF, XH, GR, MR, NBW, WN, WK><<<grid, 64 * WN * WK, lds, st>>>(
      static_cast<const uint16_t*>(x), counters, partials, (int)M, (int)K, p.splits, p.gps,
      p.sg, s_cbm ? 1 : 0, g);
  return hipGetLastError();
}

template <int BITS, bool SBF, bool XH, int MR>
hipError_t launch_shape(const SmallPlan& p, const void* x, const GroupArgs& g, bool s_cbm,
                        int64_t M, int64_t K, void* ws, hipStream_t st) {
  if (g.count > 1) {
    // Groups always take the library's own plan, which uses these shapes
    // (M = 1: one or two column blocks per wavefront, four K-wavefronts;
    // 2-16 rows: wide, long-K and the rest).
#define QG_G(NBW, WN, WK)                                                                    \
    if (p.nbw == NBW && p.wn == WN && p.wk == WK)                                            \
      return launch_variant<BITS, SBF, XH, true, MR, NBW, WN, WK>(p, x, g, s_cbm, M, K, ws, st);
    QG_G(1, 1, 4) QG_G(2, 1, 4) QG_G(2, 4, 1) QG_G(2, 3, 2) QG_G(1, 4, 1)
#undef QG_G
    return hipErrorInvalidValue;
  }
#define QG_V(NBW, WN, WK)                                                                    \
  if (p.nbw == NBW && p.wn == WN && p.wk == WK)                                              \
    return launch_variant<BITS, SBF, XH, false, MR, NBW, WN, WK>(p, x, g, s_cbm, M, K, ws, st);
  QG_V(1, 4, 1) QG_V(1, 2, 2) QG_V(1, 1, 4) QG_V(1, 1, 8)
  QG_V(2, 4, 1) QG_V(2, 3, 2) QG_V(2, 1, 4)
  QG_V(4, 4, 1) QG_V(4, 1, 4)
#undef QG_V
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_small(int bits, const SmallPlan& p, const void* x, bool x_f16,
                             const GroupArgs& g, bool s_bf16, bool s_cbm, int64_t M, int64_t K,
                             void* ws, hipStream_t st) {
#define QG_B(B, S, H, R)                                                                  \
  if (bits == B && s_bf16 == S && x_f16 == H && p.mr == R)                                \
    return launch_shape<B, S, H, R>(p, x, g, s_cbm, M, K, ws, st);
  QG_B(4, false, false, 1) QG_B(4, false, false, 16) QG_B(4, true, false, 1) QG_B(4, true, false, 16)
  QG_B(8, false, false, 1) QG_B(8, false, false, 16) QG_B(8, true, false, 1) QG_B(8, true, false, 16)
  QG_B(4, false, true, 1) QG_B(4, false, true, 16) QG_B(4, true, true, 1) QG_B(4, true, true, 16)
  QG_B(8, false, true, 1) QG_B(8, false, true, 16) QG_B(8, true, true, 1) QG_B(8, true, true, 16)
#undef QG_B
  return hipErrorInvalidValue;
}

}  // namespace qg

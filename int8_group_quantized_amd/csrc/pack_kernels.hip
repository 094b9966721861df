// Elementwise, HBM-bound kernels around the packed layout:
//   rtn_scales     per-group RTN scale from the weights
//                  (W8A16 model card: RTN, symmetric, group = 128)
//   pack_to_grid   the fixed-grid quantizer Q_s + packing
//                  (arXiv 2607.04244, QAD paragraph: updated bf16 weights
//                  rounded back onto the frozen grid)
//   prepack/unpack reorder logical codes into / out of the packed tiles
//   fake_quant     the fixed-grid fake quantizer s (.) Q_s(W) of QAD's
//                  forward pass, one rounding into bf16, fp16 or fp32
//   dequant        the dense weight s (.) W_q in bf16 or fp16
//                  (arXiv 2607.04244, QAD paragraph: the student starts from
//                  the dequantized weights; README "Stage 2": the dense
//                  dequantized twin used for finetuning and calibration)
//
// Thread mapping for the tile kernels: one thread per (tile, lane), i.e. per
// 16 packed bytes (INT4) or 32 (INT8). A thread's 32 codes share one column
// and one group, hence one scale. Packed stores are 16-byte vector stores,
// contiguous across the wavefront (one 1 KiB or 2 KiB tile per wave);
// pack_to_grid stages its workgroup's weight block in LDS first.
#include "qg_device.h"
#include "qg_internal.h"

namespace qg {
namespace {

template <bool W_BF16>
__device__ __forceinline__ float load_weight(const void* W, int64_t idx) {
  if constexpr (W_BF16) {
    return bf16_bits_to_f32(static_cast<const uint16_t*>(W)[idx]);
  } else {
    return static_cast<const float*>(W)[idx];
  }
}

// Nibble position (within a 32-bit word) of element i of an 8-deep slice.
__device__ __forceinline__ constexpr int nibble_of(int i) { return (i >> 1) + 4 * (i & 1); }

// scales[g, n] for every (g, n): max |W[128g .. 128g+127, n]| / divisor.
template <int BITS, bool W_BF16>
__global__ __launch_bounds__(256) void rtn_scales_kernel(const void* __restrict__ W,
                                                         uint16_t* __restrict__ scales,
                                                         int K, int N) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int g = blockIdx.y;
  if (n >= N) return;
  float amax = 0.0f;
  const int64_t base = (int64_t)g * kGroup * N + n;
#pragma unroll 8
  for (int r = 0; r < kGroup; ++r) {
    float a = fabsf(load_weight<W_BF16>(W, base + (int64_t)r * N));
    a = (a != a) ? 0.0f : a;          // NaN weights count as 0
    amax = fmaxf(amax, a);
  }
  const float s = amax / (BITS == 4 ? 7.0f : 127.0f);   // IEEE division
  scales[(int64_t)g * N + n] = (BITS == 4) ? f32_to_f16_bits(s) : f32_to_bf16_bits(s);
}

// The 32 logical values of one (tile, lane), in element order: q[j*8 + i] is
// k = 128g + 32j + 8*(lane/16) + i, column 16*nb + lane%16.
template <int BITS>
__device__ __forceinline__ void store_lane_codes(void* packed, int64_t out_u4, const int (&q)[32]) {
  u32x4* dst = static_cast<u32x4*>(packed) + out_u4;
  if constexpr (BITS == 4) {
    u32x4 w = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) word |= (uint32_t)((q[8 * j + i] + 8) & 15) << (4 * nibble_of(i));
      w[j] = word;
    }
    dst[0] = w;
  } else {
    uint32_t words[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo |= (uint32_t)(q[8 * j + i] & 0xFF) << (8 * i);
        hi |= (uint32_t)(q[8 * j + 4 + i] & 0xFF) << (8 * i);
      }
      words[2 * j] = lo;
      words[2 * j + 1] = hi;
    }
    dst[0] = u32x4{words[0], words[1], words[2], words[3]};
    dst[1] = u32x4{words[4], words[5], words[6], words[7]};
  }
}

// Q_s + packing. A workgroup owns one group (128 rows) of four column
// blocks (64 columns): it first stages that block of W in LDS as fp32 with
// 16-byte loads (whole cache lines, a quarter of the load instructions of
// per-element loads), then each wavefront packs one column block, a lane
// reading its 32 codes down one column. LDS rows are padded to 66 words so
// the four row quads of a lane group read 16 banks apart.
constexpr int kPackRowW = 66;

template <int BITS, bool W_BF16, bool S_BF16>
__global__ __launch_bounds__(256) void pack_to_grid_kernel(const void* __restrict__ W,
                                                           const uint16_t* __restrict__ scales,
                                                           void* __restrict__ packed, int K, int N) {
  __shared__ float tw[kGroup * kPackRowW];
  const int G = K / kGroup;
  const int NB = N / kTileCols;
  const int g = blockIdx.y;
  const int col0 = blockIdx.x * 64;
  const int ncols = min(64, N - col0);            // a multiple of 16
  const int tid = threadIdx.x;
  const int64_t row_base = (int64_t)g * kGroup;
  if constexpr (W_BF16) {
    // 8 lanes per 128-byte row, 32 rows per pass.
    const int ch = tid & 7;
    if (8 * ch < ncols) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int r = (tid >> 3) + 32 * p;
        const u32x4 v = *reinterpret_cast<const u32x4*>(
            static_cast<const uint16_t*>(W) + (row_base + r) * N + col0 + 8 * ch);
        float* d = tw + r * kPackRowW + 8 * ch;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          *reinterpret_cast<float2*>(d + 2 * e) =
              float2{bf16_bits_to_f32(v[e] & 0xFFFFu), bf16_bits_to_f32(v[e] >> 16)};
        }
      }
    }
  } else {
    // 16 lanes per 256-byte row, 16 rows per pass.
    const int ch = tid & 15;
    if (4 * ch < ncols) {
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int r = (tid >> 4) + 16 * p;
        const float4 v = *reinterpret_cast<const float4*>(
            static_cast<const float*>(W) + (row_base + r) * N + col0 + 4 * ch);
        float* d = tw + r * kPackRowW + 4 * ch;
        *reinterpret_cast<float2*>(d) = float2{v.x, v.y};
        *reinterpret_cast<float2*>(d + 2) = float2{v.z, v.w};
      }
    }
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  const int nb = blockIdx.x * 4 + wave;
  if (nb >= NB) return;
  const int cw = 16 * wave + (lane & 15);           // column within the block of 64
  const float s = scale_to_f32(scales[(int64_t)g * N + col0 + cw], S_BF16);
  const float lo = (BITS == 4) ? -8.0f : -127.0f;
  const float hi = (BITS == 4) ? 7.0f : 127.0f;
  const int r0 = 8 * (lane >> 4);
  int q[32];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      q[8 * j + i] = quantize_to_grid(tw[(r0 + 32 * j + i) * kPackRowW + cw], s, lo, hi);
  }
  const int64_t lane_u4 = ((int64_t)nb * G + g) * 64 + lane;
  store_lane_codes<BITS>(packed, (BITS == 4) ? lane_u4 : 2 * lane_u4, q);
}

// prepack / unpack move int8 codes [K, N] (row-major) to and from the
// packed tiles through LDS, one workgroup per group of 64 columns, so the
// code array is read or written with 16-byte row accesses (a lane's 32
// codes run down one column: one byte per row). LDS rows are 68 bytes, so
// the four row quads of a lane group sit 8 banks apart.
constexpr int kCodeRowB = 68;

template <int BITS>
__global__ __launch_bounds__(256) void prepack_kernel(const int8_t* __restrict__ codes,
                                                      void* __restrict__ packed, int K, int N) {
  __shared__ uint32_t tc[kGroup * kCodeRowB / 4];
  unsigned char* tb = reinterpret_cast<unsigned char*>(tc);
  const int G = K / kGroup;
  const int NB = N / kTileCols;
  const int g = blockIdx.y;
  const int col0 = blockIdx.x * 64;
  const int ncols = min(64, N - col0);            // a multiple of 16
  const int tid = threadIdx.x;
  const int ch = tid & 3;
  if (16 * ch < ncols) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int r = (tid >> 2) + 64 * p;
      const u32x4 v = *reinterpret_cast<const u32x4*>(codes + ((int64_t)g * kGroup + r) * N + col0 +
                                                      16 * ch);
      uint32_t* d = tc + (r * kCodeRowB + 16 * ch) / 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) d[e] = v[e];
    }
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  const int nb = blockIdx.x * 4 + wave;
  if (nb >= NB) return;
  const int cw = 16 * wave + (lane & 15);
  const int r0 = 8 * (lane >> 4);
  int q[32];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int i = 0; i < 8; ++i) q[8 * j + i] = (int8_t)tb[(r0 + 32 * j + i) * kCodeRowB + cw];
  }
  const int64_t lane_u4 = ((int64_t)nb * G + g) * 64 + lane;
  store_lane_codes<BITS>(packed, (BITS == 4) ? lane_u4 : 2 * lane_u4, q);
}

template <int BITS>
__global__ __launch_bounds__(256) void unpack_kernel(const void* __restrict__ packed,
                                                     int8_t* __restrict__ codes, int K, int N) {
  __shared__ uint32_t tc[kGroup * kCodeRowB / 4];
  unsigned char* tb = reinterpret_cast<unsigned char*>(tc);
  const int G = K / kGroup;
  const int NB = N / kTileCols;
  const int g = blockIdx.y;
  const int col0 = blockIdx.x * 64;
  const int ncols = min(64, N - col0);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int nb = blockIdx.x * 4 + wave;
  if (nb < NB) {
    const int64_t lane_u4 = ((int64_t)nb * G + g) * 64 + lane;
    const u32x4* src = static_cast<const u32x4*>(packed) + ((BITS == 4) ? lane_u4 : 2 * lane_u4);
    int q[32];
    if constexpr (BITS == 4) {
      const u32x4 w = src[0];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[8 * j + i] = (int)((w[j] >> (4 * nibble_of(i))) & 15u) - 8;
      }
    } else {
      const u32x4 a = src[0], b = src[1];
      const uint32_t words[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[8 * j + i] = (int8_t)(words[2 * j + (i >> 2)] >> (8 * (i & 3)));
      }
    }
    const int cw = 16 * wave + (lane & 15);
    const int r0 = 8 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int i = 0; i < 8; ++i) tb[(r0 + 32 * j + i) * kCodeRowB + cw] = (unsigned char)q[8 * j + i];
    }
  }
  __syncthreads();
  const int ch = tid & 3;
  if (16 * ch < ncols) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int r = (tid >> 2) + 64 * p;
      const uint32_t* d = tc + (r * kCodeRowB + 16 * ch) / 4;
      *reinterpret_cast<u32x4*>(codes + ((int64_t)g * kGroup + r) * N + col0 + 16 * ch) =
          u32x4{d[0], d[1], d[2], d[3]};
    }
  }
}

// Dense dequantization: out[k, n] = round(s[g, n] * q[k, n]) in bf16 or fp16
// (OH), k in group g. The product of the decoded scale and the integer code
// is exact in fp32 (at most 11 + 8 significant bits), so the one rounding is
// the RNE conversion to the output format. A workgroup takes one group and
// eight column blocks (128 x 128 outputs): each wavefront expands two tiles
// into an LDS block, then the workgroup writes whole 256-byte row segments.
constexpr int kDqCols = 128;                 // columns per workgroup
constexpr int kDqStride = kDqCols + 8;       // LDS row stride (16-bit), spreads banks

template <int BITS, bool SBF, bool OH>
__global__ __launch_bounds__(256) void dequant_kernel(const void* __restrict__ packed,
                                                      const uint16_t* __restrict__ scales,
                                                      uint16_t* __restrict__ out, int K, int N) {
  __shared__ uint16_t blk[kGroup * kDqStride];
  constexpr int TB = (BITS == 4) ? 1024 : 2048;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l16 = lane & 15;
  const int lq = lane >> 4;
  const int G = K / kGroup;
  const int NB = N / kTileCols;
  const int g = blockIdx.y;
  const int cb0 = blockIdx.x * (kDqCols / kTileCols);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int cbl = wave * 2 + h;
    const int cb = cb0 + cbl;
    if (cb >= NB) break;
    const char* tp = static_cast<const char*>(packed) + ((int64_t)cb * G + g) * TB + lane * (TB / 64);
    const uint32_t sb = scales[(int64_t)g * N + cb * 16 + l16];
    const float s = SBF ? bf16_bits_to_f32(sb) : f16_bits_to_f32(sb);
    int q[32];
    if constexpr (BITS == 4) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(tp);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) q[8 * j + i] = (int)((w[j] >> (4 * nibble_of(i))) & 15u) - 8;
    } else {
      const u32x4 a = reinterpret_cast<const u32x4*>(tp)[0], b = reinterpret_cast<const u32x4*>(tp)[1];
      const uint32_t words[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) q[8 * j + i] = (int8_t)(words[2 * j + (i >> 2)] >> (8 * (i & 3)));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // The empty asm keeps the fp32 product and the conversion apart: the
        // backend would otherwise fold them into one mixed-precision fused
        // multiply-add with a +0 addend, which turns -0 (s = 0, q < 0) into +0.
        float v = s * (float)q[8 * j + i];
        asm volatile("" : "+v"(v));
        blk[(32 * j + 8 * lq + i) * kDqStride + cbl * 16 + l16] = OH ? f32_to_f16_bits(v) : f32_to_bf16_bits(v);
      }
  }
  __syncthreads();
  // 128 rows x 16 pieces of 8 columns; pieces past N are skipped.
  const int n0 = cb0 * kTileCols;
#pragma unroll
  for (int m = 0; m < (kGroup * kDqCols / 8) / 256; ++m) {
    const int c = m * 256 + threadIdx.x;
    const int row = c >> 4;
    const int piece = c & 15;
    const int n = n0 + piece * 8;
    if (n < N) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(&blk[row * kDqStride + piece * 8]);
      *reinterpret_cast<u32x4*>(out + (int64_t)(g * kGroup + row) * N + n) = v;
    }
  }
}

// Fake quantization: out[k, n] = s[g, n] * Q_s(W[k, n]) with the codes of
// pack_to_grid (IEEE division, ties to even, clamp), the product exact in
// fp32 and one rounding into OUT (0 bf16, 1 fp16, 2 fp32). A thread takes 8
// consecutive weights of one row (N is a multiple of 16) and their 8 scales.
template <int BITS, bool W_BF16, bool S_BF16, int OUT>
__global__ __launch_bounds__(256) void fake_quant_kernel(const void* __restrict__ W,
                                                         const uint16_t* __restrict__ scales,
                                                         void* __restrict__ out, int K, int N) {
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (e0 >= (int64_t)K * N) return;
  const int64_t k = e0 / N;
  const int n = (int)(e0 - k * N);
  const int g = (int)(k / kGroup);
  constexpr float lo = (BITS == 4) ? -8.0f : -127.0f;
  constexpr float hi = (BITS == 4) ? 7.0f : 127.0f;
  float w[8];
  if constexpr (W_BF16) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(W) + e0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[2 * i] = bf16_bits_to_f32(v[i] & 0xFFFFu);
      w[2 * i + 1] = bf16_bits_to_f32(v[i] >> 16);
    }
  } else {
    const float* src = static_cast<const float*>(W) + e0;
    const f32x4 a = *reinterpret_cast<const f32x4*>(src), b = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { w[i] = a[i]; w[4 + i] = b[i]; }
  }
  const u32x4 sv = *reinterpret_cast<const u32x4*>(scales + (int64_t)g * N + n);
  float r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t sb = (i & 1) ? (sv[i >> 1] >> 16) : (sv[i >> 1] & 0xFFFFu);
    const float s = S_BF16 ? bf16_bits_to_f32(sb) : f16_bits_to_f32(sb);
    r[i] = s * (float)quantize_to_grid(w[i], s, lo, hi);
    asm volatile("" : "+v"(r[i]));   // keep the product and the rounding apart
  }
  if constexpr (OUT == 2) {
    float* dst = static_cast<float*>(out) + e0;
    *reinterpret_cast<f32x4*>(dst) = f32x4{r[0], r[1], r[2], r[3]};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{r[4], r[5], r[6], r[7]};
  } else {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t a = OUT == 1 ? f32_to_f16_bits(r[2 * i]) : f32_to_bf16_bits(r[2 * i]);
      const uint32_t b = OUT == 1 ? f32_to_f16_bits(r[2 * i + 1]) : f32_to_bf16_bits(r[2 * i + 1]);
      o[i] = a | (b << 16);
    }
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + e0) = o;
  }
}


// Scales [G, N] -> column-block-major [N/16][G][16]: a thread moves the 8
// scales (16 bytes) at row g, columns 8p .. 8p+7 to their block's run.
// Reads walk the rows contiguously; writes are whole 16-byte pieces.
__global__ __launch_bounds__(256) void prepack_scales_kernel(const u32x4* __restrict__ in,
                                                             u32x4* __restrict__ out, int G,
                                                             int N) {
  const int64_t piece = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int per_row = N / 8;
  if (piece >= (int64_t)G * per_row) return;
  const int g = (int)(piece / per_row);
  const int c8 = (int)(piece - (int64_t)g * per_row);   // 8-column piece within the row
  const int cb = c8 >> 1;                              // 16-column block
  out[((int64_t)cb * G + g) * 2 + (c8 & 1)] = in[piece];
}

}  // namespace

hipError_t launch_rtn_scales(int bits, const void* W, bool w_bf16, int64_t K, int64_t N,
                             void* scales, hipStream_t st) {
  const dim3 grid((unsigned)((N + 255) / 256), (unsigned)(K / kGroup));
  auto* s = static_cast<uint16_t*>(scales);
  if (bits == 4) {
    if (w_bf16) rtn_scales_kernel<4, true><<<grid, 256, 0, st>>>(W, s, (int)K, (int)N);
    else        rtn_scales_kernel<4, false><<<grid, 256, 0, st>>>(W, s, (int)K, (int)N);
  } else {
    if (w_bf16) rtn_scales_kernel<8, true><<<grid, 256, 0, st>>>(W, s, (int)K, (int)N);
    else        rtn_scales_kernel<8, false><<<grid, 256, 0, st>>>(W, s, (int)K, (int)N);
  }
  return hipGetLastError();
}

hipError_t launch_pack_to_grid(int bits, const void* W, bool w_bf16, const void* scales,
                               bool s_bf16, int64_t K, int64_t N, void* packed, hipStream_t st) {
  const dim3 grid((unsigned)((N / kTileCols + 3) / 4), (unsigned)(K / kGroup));
  const auto* s = static_cast<const uint16_t*>(scales);
  const int k = (int)K, n = (int)N;
#define QG_PACK(B, WB, SB) pack_to_grid_kernel<B, WB, SB><<<grid, 256, 0, st>>>(W, s, packed, k, n)
  if (bits == 4) {
    if (w_bf16) { if (s_bf16) QG_PACK(4, true, true);  else QG_PACK(4, true, false); }
    else        { if (s_bf16) QG_PACK(4, false, true); else QG_PACK(4, false, false); }
  } else {
    if (w_bf16) { if (s_bf16) QG_PACK(8, true, true);  else QG_PACK(8, true, false); }
    else        { if (s_bf16) QG_PACK(8, false, true); else QG_PACK(8, false, false); }
  }
#undef QG_PACK
  return hipGetLastError();
}

hipError_t launch_prepack(int bits, const int8_t* codes, int64_t K, int64_t N, void* packed,
                          hipStream_t st) {
  const dim3 grid((unsigned)((N / kTileCols + 3) / 4), (unsigned)(K / kGroup));
  if (bits == 4) prepack_kernel<4><<<grid, 256, 0, st>>>(codes, packed, (int)K, (int)N);
  else           prepack_kernel<8><<<grid, 256, 0, st>>>(codes, packed, (int)K, (int)N);
  return hipGetLastError();
}

hipError_t launch_prepack_scales(const void* scales, int64_t K, int64_t N, void* out,
                                 hipStream_t st) {
  const int64_t G = K / kGroup;
  const int64_t pieces = G * (N / 8);
  prepack_scales_kernel<<<(unsigned)((pieces + 255) / 256), 256, 0, st>>>(
      static_cast<const u32x4*>(scales), static_cast<u32x4*>(out), (int)G, (int)N);
  return hipGetLastError();
}

hipError_t launch_unpack(int bits, const void* packed, int64_t K, int64_t N, int8_t* codes,
                         hipStream_t st) {
  const dim3 grid((unsigned)((N / kTileCols + 3) / 4), (unsigned)(K / kGroup));
  if (bits == 4) unpack_kernel<4><<<grid, 256, 0, st>>>(packed, codes, (int)K, (int)N);
  else           unpack_kernel<8><<<grid, 256, 0, st>>>(packed, codes, (int)K, (int)N);
  return hipGetLastError();
}

hipError_t launch_dequant(int bits, const void* packed, const void* scales, bool s_bf16, void* out,
                          bool out_f16, int64_t K, int64_t N, hipStream_t st) {
  const dim3 grid((unsigned)((N / kTileCols + 7) / 8), (unsigned)(K / kGroup));
  const auto* sp = static_cast<const uint16_t*>(scales);
  auto* op = static_cast<uint16_t*>(out);
  const int k = (int)K, n = (int)N;
#define QG_D(B, S, H)                                                         \
  if (bits == B && s_bf16 == S && out_f16 == H)                               \
    dequant_kernel<B, S, H><<<grid, 256, 0, st>>>(packed, sp, op, k, n);
  QG_D(4, false, false) QG_D(4, false, true) QG_D(4, true, false) QG_D(4, true, true)
  QG_D(8, false, false) QG_D(8, false, true) QG_D(8, true, false) QG_D(8, true, true)
#undef QG_D
  return hipGetLastError();
}

hipError_t launch_fake_quant(int bits, const void* W, bool w_bf16, const void* scales, bool s_bf16,
                             void* out, int out_kind, int64_t K, int64_t N, hipStream_t st) {
  const int64_t threads = K * N / 8;
  const dim3 grid((unsigned)((threads + 255) / 256));
  const auto* sp = static_cast<const uint16_t*>(scales);
  const int k = (int)K, n = (int)N;
#define QG_F(B, WB, SB, O)                                                        \
  if (bits == B && w_bf16 == WB && s_bf16 == SB && out_kind == O)                 \
    fake_quant_kernel<B, WB, SB, O><<<grid, 256, 0, st>>>(W, sp, out, k, n);
#define QG_F3(B, WB, SB) QG_F(B, WB, SB, 0) QG_F(B, WB, SB, 1) QG_F(B, WB, SB, 2)
  QG_F3(4, false, false) QG_F3(4, false, true) QG_F3(4, true, false) QG_F3(4, true, true)
  QG_F3(8, false, false) QG_F3(8, false, true) QG_F3(8, true, false) QG_F3(8, true, true)
#undef QG_F3
#undef QG_F
  return hipGetLastError();
}

}  // namespace qg

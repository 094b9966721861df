// Drafter attention with a symmetric sliding window over a full KV cache, for
// one draft block of up to 16 queries per sequence (gfx950).
//
// "Quantize the Target, Quantize the Drafter" (arXiv 2607.04244), Drafter SWA
// paragraph: the drafter's mask-token queries attend bidirectionally, so the
// window (1,024 or 2,048 tokens) is symmetric around each query; it exists
// only inside the attention kernel, the KV cache keeps every position, and a
// sequence within the window size falls back to full attention. The drafter
// setup paragraph fixes the block at 16 tokens. Window reading: W // 2
// positions to each side of the query; the block's queries sit at the last T
// cache positions; W = 0 is full attention.
//
// Work split. A workgroup owns one (sequence, query head, chunk of keys); its
// four wavefronts take 32-key steps of the chunk in turn and keep an online
// softmax each. Query heads that share a KV head are dealt to the same XCD
// (workgroup i runs on XCD i % 8), so their K/V rows come from one L2. For
// long spans with many sequences a second kernel (below) gives one workgroup
// all query heads of a KV head over a single stream of its K/V rows.
//
// Both products run on the bf16 matrix core (16x16x32), transposed so that
// no probability ever leaves the registers:
//   S^T = K Q^T   A = K rows (16 keys x 32 dims per lane-row), B = Q^T;
//                 the result holds, per lane, one query (lane % 16) and four
//                 keys 4(lane / 16) + e of a 16-key block;
//   O^T = V^T P^T B = P^T straight from those registers (two 16-key blocks
//                 give the 8 keys a lane supplies), A = V^T read from a
//                 per-wavefront LDS copy of the step's 32 value rows with
//                 gfx950's transposing LDS read: in each group of 16 lanes,
//                 lane s names four consecutive 16-bit values (row s of a
//                 16 x 4 block) and lane t receives element t % 4 of block
//                 rows t / 4 + 4e, e < 4.
// P is split into a bf16 high part and the bf16 rounding of the remainder,
// so P V is accumulated with ~2^-18 relative error in P (two instructions
// per block) instead of bf16's 2^-9.
//
// Chunks of one (sequence, head) are combined deterministically: each
// workgroup writes (max, sum, unnormalised output) with device-coherent
// stores, counts its arrival, and the last arrival merges the chunks in
// chunk order and writes the bf16 output.

#include "qg_internal.h"
#include "qg_device.h"

#include <cmath>

namespace qg {
namespace {

constexpr int kD = 128;                        // head dimension
constexpr int kRowBytes = kD * 2;
constexpr int kVRowBytes = kRowBytes + 32;        // a value row + pad (rows 8 banks apart)
constexpr int kVStageBytes = 32 * kVRowBytes;      // one step: 32 value rows
constexpr int kWaves = 4;
constexpr int kWavesLds = kWaves * kVStageBytes;
constexpr int kQRow = kRowBytes + 16;          // a query row in LDS + pad (rows 4 banks apart)
constexpr int kQLds = 16 * kQRow;
constexpr int kOFloats = 16 * kD;                  // one chunk's O[16][128]
constexpr int kPartFloats = kSwaPartFloats;       // O[16][128], then max[16], sum[16]
static_assert(kPartFloats == kOFloats + 32, "chunk record layout");
constexpr int kMaxChunks = kSwaMaxChunks;   // merge table of maxima and sums in LDS (128 B per chunk)
static_assert(kMaxChunks * 128 <= kWavesLds, "merge table exceeds the LDS stage area");
static_assert(kMaxChunks * 8 % (64 * kWaves) == 0, "merge table loads");
constexpr int kCoherent = 16;                  // sc1: bypass the per-XCD L2

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ float xmax(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask));
}

// QLDS: the block's queries are loaded once per workgroup into LDS and each
// step reads the Q^T operand from there (short chunks: measured 9.3 -> 8.7 us
// at batch 1, window 1,024, 106 keys per chunk); otherwise each wavefront
// loads it into registers (long chunks, where the per-step LDS reads cost
// more than the duplicate loads: batch 8, window 2,048: 16.3 vs 18.4 us).
template <bool QLDS>
__global__ __launch_bounds__(256, 2) void swa_attention_kernel(
    const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* seq_lens,
    uint16_t* out, uint32_t* counters, float* partials, int T, int Hq, int Hkv, int S_max,
    int window, float scale_log2, int chunk, int nchunks, int units) {
  extern __shared__ __align__(16) char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = Hq / Hkv;
  const int xcd = blockIdx.x & 7;
  const int m = blockIdx.x >> 3;
  const int u = (m / G) * 8 + xcd;
  if (u >= units) return;
  const int hg = m % G;
  const int c = u % nchunks;
  const int kvh = (u / nchunks) % Hkv;
  const int b = u / (nchunks * Hkv);
  const int h = kvh * G + hg;

  const int S = min(max(seq_lens[b], T), S_max);
  const bool full = window == 0 || S <= window;
  const int half = window >> 1;
  const int p0 = S - T;                          // position of query 0
  const int lo_u = full ? 0 : max(0, p0 - half);
  const int hi_u = full ? S : min(S, p0 + T + half);
  // The sequence's own span is divided evenly among the chunks (a short
  // sequence or a window cut by the cache end leaves no chunk empty).
  const int per = min(chunk, (hi_u - lo_u + nchunks - 1) / nchunks);
  const int k0 = min(lo_u + c * per, hi_u);
  const int k1 = min(k0 + per, hi_u);

  const int tok = lane & 15;                     // this lane's query (column)
  const int g = lane >> 4;                       // this lane's key / dim quarter
  int vlo = 0, vhi = 0;                          // visible keys of the query, in this chunk
  if (tok < T) {
    const int p = p0 + tok;
    vlo = max(full ? 0 : max(0, p - half), k0);
    vhi = min(full ? S : min(S, p + half + 1), k1);
  }

  // Q^T operand: query tok, dims 32j + 8g .. +7.
  const uint32_t kv_seq_bytes = (uint32_t)S * (uint32_t)Hkv * kRowBytes;
  const uint16_t* kb_ = k + (size_t)b * S_max * Hkv * kD;
  const uint16_t* vb_ = v + (size_t)b * S_max * Hkv * kD;
  const __amdgpu_buffer_rsrc_t rk = rsrc(kb_, kv_seq_bytes);
  const __amdgpu_buffer_rsrc_t rv = rsrc(vb_, kv_seq_bytes);
  u32x4 bq[4];
  char* const qlds = lds + kWavesLds;   // QLDS: query t's row at t * kQRow (rows past T zero)
  {
    const __amdgpu_buffer_rsrc_t rq = rsrc(q + ((size_t)b * T * Hq + h) * kD,
                                           (uint32_t)(T * Hq * kRowBytes));
    if constexpr (QLDS) {
      const int qt = tid >> 4;
      *reinterpret_cast<u32x4*>(qlds + qt * kQRow + 16 * (tid & 15)) =
          ld16(rq, qt < T ? (uint32_t)(qt * Hq * kRowBytes + 16 * (tid & 15)) : 0x80000000u);
      __syncthreads();
    } else {
      const uint32_t qoff = (uint32_t)(tok * Hq * kRowBytes + 16 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j) bq[j] = ld16(rq, tok < T ? qoff + 64 * j : 0x80000000u);
    }
  }
  // Q^T operand: query tok, dims 32j + 8g .. +7.
  auto qop = [&](int j) -> u32x4 {
    if constexpr (QLDS)
      return *reinterpret_cast<const u32x4*>(qlds + tok * kQRow + 64 * j + 16 * g);
    else
      return bq[j];
  };

  const int nsteps = k1 > k0 ? (k1 - k0 + 31) >> 5 : 0;
  char* vst = lds + wave * kVStageBytes;
  const uint32_t row_stride = (uint32_t)Hkv * kRowBytes;
  // K operand rows: key key0 + 16 kb + tok, dims 32j + 8g; value rows for the
  // LDS stage: key key0 + 4r + g, 16-byte piece tok.
  const uint32_t k_lane = (uint32_t)tok * row_stride + kvh * kRowBytes + 16 * g;
  const uint32_t v_lane = (uint32_t)g * row_stride + kvh * kRowBytes + 16 * tok;

  u32x4 kc[2][4], vn[8];
  auto load_k = [&](u32x4 (&dst)[2][4], int key0) {
    const uint32_t base = (uint32_t)key0 * row_stride + k_lane;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[kb][j] = ld16(rk, base + kb * 16 * row_stride + 64 * j);
  };
  auto load_v = [&](int key0) {
    const uint32_t base = (uint32_t)key0 * row_stride + v_lane;
#pragma unroll
    for (int r = 0; r < 8; ++r) vn[r] = ld16(rv, base + 4 * r * row_stride);
  };
  auto stage_v = [&]() {
#pragma unroll
    for (int r = 0; r < 8; ++r)
      *reinterpret_cast<u32x4*>(vst + (4 * r + g) * kVRowBytes + 16 * tok) = vn[r];
  };

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  int s = wave;
  if (s < nsteps) {
    load_k(kc, k0 + 32 * s);
    load_v(k0 + 32 * s);
    stage_v();
  }
  // V^T operand of lane (tok, g): dim 16 db + tok of keys 4g .. 4g+3 and
  // 16 + 4g .. +3. Through the transposing read, lane s of the group names
  // key k0 + s / 4, dims 16 db + 4 (s % 4) .. +3 (8 bytes), and receives
  // keys k0 .. k0+3 of dim 16 db + s.
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s* lds_v4s;
  const char* vt0 = vst + (4 * g + (tok >> 2)) * kVRowBytes + 8 * (tok & 3);
  const char* vt1 = vt0 + 16 * kVRowBytes;
  for (; s < nsteps; s += kWaves) {
    const int key0 = k0 + 32 * s;
    const bool more = s + kWaves < nsteps;
    // Scores for two 16-key blocks; the next step's rows are requested once
    // these products have their operands (a fetch issued before them made
    // the products wait on it).
    f32x4 acc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kc[kb][j]),
                                                          __builtin_bit_cast(bf16x8, qop(j)),
                                                          acc[kb], 0, 0, 0);
    }
    u32x4 kn[2][4];
    if (more) {
      load_k(kn, key0 + 32 * kWaves);
      load_v(key0 + 32 * kWaves);
    }
    float sc[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = key0 + 16 * kb + 4 * g + e;
        sc[kb][e] = (key >= vlo && key < vhi) ? acc[kb][e] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, sc[kb][e]);
      }
    }
    mx = xmax(xmax(mx, 16), 32);
    const float m_new = fmaxf(m_run, mx);
    const float ms = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - ms);
    float pv[8];
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pv[i] = __builtin_amdgcn_exp2f(sc[i >> 2][i & 3] - ms);
      psum += pv[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    u32x4 phi, plo;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t hw = pack_bf16x2(pv[2 * w], pv[2 * w + 1]);
      phi[w] = hw;
      plo[w] = pack_bf16x2(pv[2 * w] - bf16_bits_to_f32(hw & 0xFFFFu),
                           pv[2 * w + 1] - bf16_bits_to_f32(hw >> 16));
    }
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const v4s r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(vt0 + 32 * db));
      const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(vt1 + 32 * db));
      const u32x2 w0 = __builtin_bit_cast(u32x2, r0), w1 = __builtin_bit_cast(u32x2, r1);
      const u32x4 av = {w0[0], w0[1], w1[0], w1[1]};
      f32x4 od = o[db] * alpha;
      od = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                   __builtin_bit_cast(bf16x8, phi), od, 0, 0, 0);
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                      __builtin_bit_cast(bf16x8, plo), od, 0, 0,
                                                      0);
    }
    if (more) {
      // The LDS reads above precede these writes in this wavefront's LDS queue.
      stage_v();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) kc[kb][j] = kn[kb][j];
    }
  }
  // Sum the lane-partial row sums of a query over the four key quarters.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  // Merge the four wavefronts in LDS (each reuses its own stage area):
  // part[16][128] unnormalised output, then max[16], sum[16].
  float* part = reinterpret_cast<float*>(vst);
#pragma unroll
  for (int db = 0; db < 8; ++db)
    *reinterpret_cast<f32x4*>(part + tok * kD + 16 * db + 4 * g) = o[db];
  if (g == 0) {
    part[16 * kD + tok] = m_run;
    part[16 * kD + 16 + tok] = l_run;
  }
  __syncthreads();
  const int rt = tid >> 4;                         // query of this thread
  const int d0 = (tid & 15) * 8;                   // its 8 dims
  float wm[kWaves];
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    wm[w] = reinterpret_cast<const float*>(lds + w * kVStageBytes)[16 * kD + rt];
    M = fmaxf(M, wm[w]);
  }
  const float Ms = M == -INFINITY ? 0.0f : M;
  float L = 0.0f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float* pw = reinterpret_cast<const float*>(lds + w * kVStageBytes);
    const float f = __builtin_amdgcn_exp2f(wm[w] - Ms);
    L += f * pw[16 * kD + 16 + rt];
    const f32x4 a = *reinterpret_cast<const f32x4*>(pw + rt * kD + d0);
    const f32x4 bb = *reinterpret_cast<const f32x4*>(pw + rt * kD + d0 + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += f * a[e];
      acc[4 + e] += f * bb[e];
    }
  }
  uint16_t* orow = out + (((size_t)b * T + rt) * Hq + h) * kD + d0;
  auto store_out = [&](const float (&x)[8], float l) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(x[2 * e] * inv, x[2 * e + 1] * inv);
    *reinterpret_cast<u32x4*>(orow) = w;
  };
  if (nchunks == 1) {
    if (rt < T) store_out(acc, L);
    return;
  }

  // Split across workgroups: publish this chunk, count the arrival. The
  // region of one (sequence, head) holds every chunk's O[16][128], then every
  // chunk's max[16] and sum[16], so the merge reads the maxima in one sweep.
  // A chunk's O is stored thread-major: 16-byte word 256 j + tid holds this
  // thread's dims d0 + 4 j .. +3, so each store and each merge load of a
  // wavefront moves 1 KB of consecutive bytes.
  const size_t pbase = ((size_t)(b * Hq + h) * nchunks) * kPartFloats;
  const uint32_t ml0 = (uint32_t)(nchunks * kOFloats * sizeof(float));
  const __amdgpu_buffer_rsrc_t rp =
      rsrc(partials + pbase, (uint32_t)(nchunks * kPartFloats * sizeof(float)));
  {
    const uint32_t off = (uint32_t)((c * kOFloats + 4 * tid) * sizeof(float));
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(acc[0]), __float_as_uint(acc[1]),
                                                 __float_as_uint(acc[2]), __float_as_uint(acc[3])},
                                           rp, off, 0, kCoherent);
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(acc[4]), __float_as_uint(acc[5]),
                                                 __float_as_uint(acc[6]), __float_as_uint(acc[7])},
                                           rp, off + 4096, 0, kCoherent);
    if ((tid & 15) == 0) {
      const uint32_t moff = ml0 + (uint32_t)((c * 32 + rt) * sizeof(float));
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(M), rp, moff, 0, kCoherent);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(L), rp, moff + 64, 0, kCoherent);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  __shared__ uint32_t s_last;
  const int cidx = b * Hq + h;
  if (tid == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(&counters[cidx], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (uint32_t)nchunks - 1u ? 1u : 0u;
  }
  __syncthreads();
  if (s_last == 0u) return;

  // Last arrival: merge every chunk in chunk order. Maxima and sums of all
  // chunks go to LDS in one sweep of 16-byte loads; the outputs follow in
  // batches of eight chunks whose loads are all in flight together (a slot
  // past the last chunk reads zeros through the buffer range check).
  float* ml = reinterpret_cast<float*>(lds);
  constexpr int kBatch = 8;
  u32x4 a[kBatch], bb[kBatch];
  auto issue = [&](int c0) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const uint32_t off = c0 + i < nchunks
                               ? (uint32_t)(((c0 + i) * kOFloats + 4 * tid) * sizeof(float))
                               : 0x80000000u;
      a[i] = __builtin_amdgcn_raw_buffer_load_b128(rp, off, 0, kCoherent);
      bb[i] = __builtin_amdgcn_raw_buffer_load_b128(rp, off + 4096, 0, kCoherent);
    }
  };
  // The first batch of outputs and the whole table of maxima and sums are in
  // flight together.
  u32x4 mlv[kMaxChunks * 8 / (64 * kWaves)];
  constexpr int kMlPer = kMaxChunks * 8 / (64 * kWaves);
  __syncthreads();                                 // the wavefront merge above is done
#pragma unroll
  for (int j = 0; j < kMlPer; ++j) {
    const int i = tid + j * 64 * kWaves;
    mlv[j] = __builtin_amdgcn_raw_buffer_load_b128(
        rp, i < nchunks * 8 ? ml0 + 16 * i : 0x80000000u, 0, kCoherent);
    if (j == 0) issue(0);
  }
#pragma unroll
  for (int j = 0; j < kMlPer; ++j) {
    const int i = tid + j * 64 * kWaves;
    if (i < nchunks * 8) *reinterpret_cast<u32x4*>(ml + 4 * i) = mlv[j];
  }
  __syncthreads();
  float Mx = -INFINITY;
  for (int cc = 0; cc < nchunks; ++cc) Mx = fmaxf(Mx, ml[cc * 32 + rt]);
  const float Mxs = Mx == -INFINITY ? 0.0f : Mx;
  float tot[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float Lt = 0.0f;
  for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
    if (c0 > 0) issue(c0);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int cc = min(c0 + i, nchunks - 1);
      const float f = c0 + i < nchunks ? __builtin_amdgcn_exp2f(ml[cc * 32 + rt] - Mxs) : 0.0f;
      Lt += f * ml[cc * 32 + 16 + rt];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        tot[e] += f * __uint_as_float(a[i][e]);
        tot[4 + e] += f * __uint_as_float(bb[i][e]);
      }
    }
  }
  if (rt < T) store_out(tot, Lt);
  if (tid == 0)   // ready for the next call on this workspace
    __hip_atomic_store(&counters[cidx], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// ---- Query heads of one KV head over a shared K/V ring in LDS ----
//
// Grouped-query attention: the query heads of a group read the same key and
// value rows. This kernel gives one workgroup a (sequence, KV head, group of
// WV query heads, chunk of keys), one wavefront per query head, and fetches
// every 64-key step's K and V rows (32 KB) once for the whole group, straight
// into an LDS ring of kRing slots by buffer loads. One more wavefront only
// issues those loads (32 per step, 1 KB each): it waits for a step with a
// constant vmcnt count and meets the others at one barrier per step. The
// wavefronts that compute issue no memory loads inside the loop, so no wait
// the compiler places before their LDS reads can stall on the ring. A row's 16-byte pieces are stored
// XOR-swizzled by the row index, so the K operand reads (16 rows, one piece
// each) and the transposing V^T reads (16 rows, 8 bytes each) hit distinct
// banks. Each wavefront keeps its head's online softmax over the whole chunk,
// so no merge runs between wavefronts; chunks merge through partial records
// of the one-head kernel's size (O, maxima, sums per chunk and head, here in
// the accumulators' lane order), with one arrival count per head group.
constexpr int kRing = 2;                          // slots: the step computed, the next one loading
constexpr int kRingKeys = 64;                     // keys per step
constexpr int kRingSlot = 2 * kRingKeys * kRowBytes;   // K rows, then V rows, of one step
constexpr int kRingLds = kRing * kRingSlot;
constexpr int kRingMaxChunks = kSwaRingMaxChunks;   // merge table: 128 B per chunk and wavefront
static_assert(kRingMaxChunks * 8 <= 128, "merge table loads: two 16-byte words per lane");
static_assert(8 * kRingMaxChunks * 128 <= kRingLds, "merge tables exceed the ring");

// Byte offset of piece p (16 bytes) of row r in a block of swizzled 256-byte rows.
__device__ __forceinline__ int swz(int r, int p) { return r * kRowBytes + ((p ^ (r & 15)) << 4); }

typedef __attribute__((address_space(3))) void* ring_lds_ptr;
__device__ __forceinline__ void ring_to_lds(__amdgpu_buffer_rsrc_t r, char* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (ring_lds_ptr)dst, 16, voff, 0, 0, 0);
}

template <int WV>
__global__ __launch_bounds__(64 * (WV + 1), 2) void swa_ring_kernel(
    const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* seq_lens,
    uint16_t* out, uint32_t* counters, float* partials, int T, int Hq, int Hkv, int S_max,
    int window, float scale_log2, int chunk, int nchunks, int units) {
  extern __shared__ __align__(16) char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool loader = wave == WV;                       // the last wavefront fetches
  const int G = Hq / Hkv;
  const int NG = G / WV;                                // head groups per KV head
  const int u = blockIdx.x;
  if (u >= units) return;
  const int c = u % nchunks;
  const int grp = (u / nchunks) % NG;
  const int kvh = (u / (nchunks * NG)) % Hkv;
  const int b = u / (nchunks * NG * Hkv);
  const int h = kvh * G + grp * WV + (loader ? 0 : wave);   // this wavefront's query head

  const int S = min(max(seq_lens[b], T), S_max);
  const bool full = window == 0 || S <= window;
  const int half = window >> 1;
  const int p0 = S - T;
  const int lo_u = full ? 0 : max(0, p0 - half);
  const int hi_u = full ? S : min(S, p0 + T + half);
  const int per = min(chunk, (hi_u - lo_u + nchunks - 1) / nchunks);
  const int k0 = min(lo_u + c * per, hi_u);
  const int k1 = min(k0 + per, hi_u);
  const int nsteps = k1 > k0 ? (k1 - k0 + kRingKeys - 1) / kRingKeys : 0;

  const int tok = lane & 15;
  const int g = lane >> 4;
  constexpr float kLazy = 8.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (loader) {
    // Loads of one step: instruction i (0..31) fills rows 4 (i % 16) .. +3 of
    // K (i < 16) or V; lane L lands at row 4 (i % 16) + L / 16, slot position
    // L % 16, which holds source piece (L % 16) ^ row. Rows past the sequence
    // read zeros (steps past the chunk's end fill slots no step reads).
    const uint32_t kv_seq_bytes = (uint32_t)S * (uint32_t)Hkv * kRowBytes;
    const __amdgpu_buffer_rsrc_t rk = rsrc(k + (size_t)b * S_max * Hkv * kD, kv_seq_bytes);
    const __amdgpu_buffer_rsrc_t rv = rsrc(v + (size_t)b * S_max * Hkv * kD, kv_seq_bytes);
    const uint32_t row_stride = (uint32_t)Hkv * kRowBytes;
    const int lrow = lane >> 4;
    const int lpiece = lane & 15;
    auto issue_step = [&](int st) {
      char* slot = lds + (st % kRing) * kRingSlot;
      const int key0 = k0 + kRingKeys * st;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int row = 4 * (i & 15) + lrow;
        const uint32_t voff = (uint32_t)(key0 + row) * row_stride + kvh * kRowBytes +
                              16 * (lpiece ^ (row & 15));
        ring_to_lds(i < 16 ? rk : rv,
                    slot + (i < 16 ? 0 : kRingKeys * kRowBytes) + (i & 15) * 1024,
                    key0 + row < S ? voff : 0x80000000u);
      }
    };
#pragma unroll
    for (int st = 0; st < kRing - 1; ++st) issue_step(st);
#pragma unroll 1
    for (int s = 0; s < nsteps; ++s) {
      // step s has landed: only the next kRing - 2 steps' loads may be out
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((kRing - 2) * 32) : "memory");
      issue_step(s + kRing - 1);                     // into the slot step s - 1 used
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    int vlo = 0, vhi = 0;
    if (tok < T) {
      const int p = p0 + tok;
      vlo = max(full ? 0 : max(0, p - half), k0);
      vhi = min(full ? S : min(S, p + half + 1), k1);
    }
    // Keys every query of the block sees: steps inside need no mask (rows
    // past T score against a zero query and are never stored).
    const int fast_lo = max(full ? 0 : max(0, p0 + T - 1 - half), k0);
    const int fast_hi = min(full ? S : min(S, p0 + half + 1), k1);
    // Q^T operand: query tok, dims 32 j + 8 g .. +7.
    u32x4 bq[4];
    {
      const __amdgpu_buffer_rsrc_t rq = rsrc(q + ((size_t)b * T * Hq + h) * kD,
                                             (uint32_t)(T * Hq * kRowBytes));
      const uint32_t qoff = (uint32_t)(tok * Hq * kRowBytes + 16 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j) bq[j] = ld16(rq, tok < T ? qoff + 64 * j : 0x80000000u);
    }
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s* lds_v4s;
    // V^T reads: rows 4 g + tok / 4 and +16, byte 32 db + 8 (tok % 4) of the row.
    const int vrow = 4 * g + (tok >> 2);
    const int vsub = 8 * (tok & 1);
    const int vpc = (tok & 3) >> 1;
#pragma unroll 1
    for (int s = 0; s < nsteps; ++s) {
      // this wavefront's reads of step s - 1 are done before its slot is refilled
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      const char* slot = lds + (s % kRing) * kRingSlot;
      const int key0 = k0 + kRingKeys * s;
      f32x4 acc[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 kv = *reinterpret_cast<const u32x4*>(slot + swz(16 * kb + tok, 4 * j + g));
          acc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv),
                                                            __builtin_bit_cast(bf16x8, bq[j]),
                                                            acc[kb], 0, 0, 0);
        }
      }
      float sc[4][4];
      float mx = -INFINITY;
      if (key0 >= fast_lo && key0 + kRingKeys <= fast_hi) {   // wave-uniform
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sc[kb][e] = acc[kb][e] * scale_log2;
            mx = fmaxf(mx, sc[kb][e]);
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = key0 + 16 * kb + 4 * g + e;
            sc[kb][e] = (key >= vlo && key < vhi) ? acc[kb][e] * scale_log2 : -INFINITY;
            mx = fmaxf(mx, sc[kb][e]);
          }
      }
      mx = xmax(xmax(mx, 16), 32);
      // The exponent reference moves only when a query's maximum passes it
      // by more than kLazy (log2 units): probabilities stay at most 2^kLazy,
      // which the two-part bf16 P carries to the same relative precision.
      if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazy) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.0f : m_new));
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 8; ++db) o[db] *= alpha;
      }
      const float ms = m_run == -INFINITY ? 0.0f : m_run;
      // Each 32-key half: P^T operand from this lane's 8 scores (keys
      // 16 kb + 4 g + e of its two 16-key blocks), then O^T += V^T P^T.
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float pv[8];
        float psum = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(sc[2 * hh + (e >> 2)][e & 3] - ms);
          psum += pv[e];
        }
        l_run += psum;
        u32x4 phi, plo;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t hw = pack_bf16x2(pv[2 * w], pv[2 * w + 1]);
          phi[w] = hw;
          plo[w] = pack_bf16x2(pv[2 * w] - bf16_bits_to_f32(hw & 0xFFFFu),
                               pv[2 * w + 1] - bf16_bits_to_f32(hw >> 16));
        }
        const char* vs = slot + kRingKeys * kRowBytes;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const int pc = 2 * db + vpc;
          const v4s r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4s)(vs + swz(32 * hh + vrow, pc) + vsub));
          const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4s)(vs + swz(32 * hh + vrow + 16, pc) + vsub));
          const u32x2 w0 = __builtin_bit_cast(u32x2, r0), w1 = __builtin_bit_cast(u32x2, r1);
          const u32x4 av = {w0[0], w0[1], w1[0], w1[1]};
          const f32x4 od = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, phi), o[db], 0, 0, 0);
          o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, plo), od, 0, 0, 0);
        }
      }
    }
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
  }

  const size_t pstride = (size_t)nchunks * kPartFloats;
  const uint32_t ml0 = (uint32_t)(nchunks * kOFloats * sizeof(float));
  if (nchunks == 1) {
    if (!loader && tok < T) {
      const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
      uint16_t* orow = out + (((size_t)b * T + tok) * Hq + h) * kD + 4 * g;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        u32x2 w;
        w[0] = pack_bf16x2(o[db][0] * inv, o[db][1] * inv);
        w[1] = pack_bf16x2(o[db][2] * inv, o[db][3] * inv);
        *reinterpret_cast<u32x2*>(orow + 16 * db) = w;
      }
    }
    return;
  }

  // This chunk's record for the head, in the accumulators' own layout:
  // 16-byte word 64 db + lane holds o[db] of that lane (query lane % 16,
  // dims 16 db + 4 (lane / 16) .. +3), so every store and every merge load
  // moves 1 KB of consecutive bytes; then max[16] and sum[16].
  if (!loader) {
    const __amdgpu_buffer_rsrc_t rp =
        rsrc(partials + (size_t)(b * Hq + h) * pstride, (uint32_t)(pstride * sizeof(float)));
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint32_t off = (uint32_t)((c * kOFloats + 4 * (64 * db + lane)) * sizeof(float));
      __builtin_amdgcn_raw_buffer_store_b128(
          u32x4{__float_as_uint(o[db][0]), __float_as_uint(o[db][1]), __float_as_uint(o[db][2]),
                __float_as_uint(o[db][3])}, rp, off, 0, kCoherent);
    }
    if (g == 0) {
      const uint32_t moff = ml0 + (uint32_t)((c * 32 + tok) * sizeof(float));
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m_run), rp, moff, 0, kCoherent);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l_run), rp, moff + 64, 0, kCoherent);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  __shared__ uint32_t s_last;
  const int cidx = (b * Hkv + kvh) * NG + grp;
  if (tid == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(&counters[cidx], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (uint32_t)nchunks - 1u ? 1u : 0u;
  }
  __syncthreads();
  if (s_last == 0u) return;

  if (!loader) {
    // Last arrival: each wavefront merges its head's chunks in chunk order,
    // every lane the same words it stored. The maxima and sums of all chunks
    // go to the wavefront's own LDS area; the first batch of words is in
    // flight with them.
    const __amdgpu_buffer_rsrc_t rp =
        rsrc(partials + (size_t)(b * Hq + h) * pstride, (uint32_t)(pstride * sizeof(float)));
    float* ml = reinterpret_cast<float*>(lds + wave * (kRingMaxChunks * 128));
    constexpr int kB = 2;                              // chunks per load batch
    u32x4 a[kB][8];
    auto issue = [&](int c0) {
#pragma unroll
      for (int j = 0; j < kB; ++j)
#pragma unroll
        for (int db = 0; db < 8; ++db)
          a[j][db] = __builtin_amdgcn_raw_buffer_load_b128(
              rp, c0 + j < nchunks
                      ? (uint32_t)(((c0 + j) * kOFloats + 4 * (64 * db + lane)) * sizeof(float))
                      : 0x80000000u,
              0, kCoherent);
    };
    {
      // nchunks * 8 16-byte words, at most 128: two per lane
      const u32x4 t0 = __builtin_amdgcn_raw_buffer_load_b128(
          rp, lane < nchunks * 8 ? ml0 + 16 * lane : 0x80000000u, 0, kCoherent);
      const u32x4 t1 = __builtin_amdgcn_raw_buffer_load_b128(
          rp, lane + 64 < nchunks * 8 ? ml0 + 16 * (lane + 64) : 0x80000000u, 0, kCoherent);
      issue(0);
      if (lane < nchunks * 8) *reinterpret_cast<u32x4*>(ml + 4 * lane) = t0;
      if (lane + 64 < nchunks * 8) *reinterpret_cast<u32x4*>(ml + 4 * (lane + 64)) = t1;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    float Mx = -INFINITY;
    for (int cc = 0; cc < nchunks; ++cc) Mx = fmaxf(Mx, ml[cc * 32 + tok]);
    const float Mxs = Mx == -INFINITY ? 0.0f : Mx;
    f32x4 tot[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) tot[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float Lt = 0.0f;
    for (int c0 = 0; c0 < nchunks; c0 += kB) {
      if (c0 > 0) issue(c0);
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        const int cc = min(c0 + j, nchunks - 1);
        const float f = c0 + j < nchunks ? __builtin_amdgcn_exp2f(ml[cc * 32 + tok] - Mxs) : 0.0f;
        Lt += f * ml[cc * 32 + 16 + tok];
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
          for (int x = 0; x < 4; ++x) tot[db][x] += f * __uint_as_float(a[j][db][x]);
      }
    }
    if (tok < T) {
      const float inv = Lt > 0.0f ? 1.0f / Lt : 0.0f;
      uint16_t* orow = out + (((size_t)b * T + tok) * Hq + h) * kD + 4 * g;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        u32x2 w;
        w[0] = pack_bf16x2(tot[db][0] * inv, tot[db][1] * inv);
        w[1] = pack_bf16x2(tot[db][2] * inv, tot[db][3] * inv);
        *reinterpret_cast<u32x2*>(orow + 16 * db) = w;
      }
    }
  }
  if (tid == 0)   // ready for the next call on this workspace
    __hip_atomic_store(&counters[cidx], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_swa_attention(const SwaPlan& p, const void* q, const void* k, const void* v,
                                const int32_t* seq_lens, void* out, int64_t T, int64_t Hq,
                                int64_t Hkv, int64_t S_max, float scale, void* ws,
                                hipStream_t st) {
  uint32_t* counters = nullptr;
  float* partials = nullptr;
  if (p.nchunks > 1) {
    counters = static_cast<uint32_t*>(ws);
    partials = reinterpret_cast<float*>(static_cast<char*>(ws) + kCounterBytes);
  }
  const float scale_log2 = (float)((double)scale * 1.4426950408889634);
  if (p.ring > 0) {
    void (*rk)(const uint16_t*, const uint16_t*, const uint16_t*, const int32_t*, uint16_t*,
               uint32_t*, float*, int, int, int, int, int, float, int, int, int) = nullptr;
    switch (p.ring) {
      case 2: rk = swa_ring_kernel<2>; break;
      case 3: rk = swa_ring_kernel<3>; break;
      case 4: rk = swa_ring_kernel<4>; break;
      case 5: rk = swa_ring_kernel<5>; break;
      case 6: rk = swa_ring_kernel<6>; break;
      case 8: rk = swa_ring_kernel<8>; break;
      default: return hipErrorInvalidValue;
    }
    if (p.nchunks > kRingMaxChunks) return hipErrorInvalidValue;
    rk<<<p.grid, 64 * (p.ring + 1), kRingLds, st>>>(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
        static_cast<const uint16_t*>(v), seq_lens, static_cast<uint16_t*>(out), counters,
        partials, (int)T, (int)Hq, (int)Hkv, (int)S_max, p.window, scale_log2, p.chunk,
        p.nchunks, p.units);
    return hipGetLastError();
  }
  auto kernel = p.q_lds ? swa_attention_kernel<true> : swa_attention_kernel<false>;
  kernel<<<p.grid, 64 * kWaves, kWavesLds + (p.q_lds ? kQLds : 0), st>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), seq_lens, static_cast<uint16_t*>(out), counters, partials,
      (int)T, (int)Hq, (int)Hkv, (int)S_max, p.window, scale_log2, p.chunk, p.nchunks, p.units);
  return hipGetLastError();
}

}  // namespace qg

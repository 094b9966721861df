/*
 * qgemm.h -- weight-only group-quantized matrix multiply for AMD Instinct
 * MI355X (gfx950), C ABI.
 *
 * What is computed
 *   A quantized Linear y = x . W with W stored as integer codes W_q and one
 *   scale per group of 128 consecutive input features per output column; the
 *   effective weight is the dequantized s (.) W_q ("Quantize the Target,
 *   Quantize the Drafter", arXiv 2607.04244, QAD method paragraph; group-wise
 *   symmetric INT4 with group size 128, drafter-PTQ calibration paragraph).
 *   INT4 codes with fp16 scales serve the W4A16 target and drafter (same
 *   paper; the quickstart of the Qwen3.5-4B-DFlash-GPTQ-W4A16 model card);
 *   INT8 codes with bf16 scales are the W8A16 variant (Qwen3.5-4B-DFlash-W8A16
 *   model card, "What changed vs upstream" table). The fixed-grid quantizer
 *   Q_s puts updated weights back on the frozen grid (QAD method paragraph:
 *   at packing time the updated bf16 weights are rounded onto the same grid,
 *   giving new codes under the original scales).
 *
 * Conventions shared by every entry point
 *   - Logical layouts are row-major and contiguous:
 *       x[M,K] bf16 (fp16 for the *f16 GEMMs), out[M,N] likewise,
 *       W[K,N], codes[K,N] int8,
 *       scales[K/128, N] (fp16 or bf16); the GEMM entry points also
 *       take the column-block-major order of qg_prepack_scales.
 *     A PyTorch Linear weight is [N,K]; transpose it before packing.
 *   - K must be a positive multiple of 128 and N a positive multiple of 16,
 *     else QG_ERR_SHAPE. M may be 0 (nothing is launched). Limits:
 *     K, N <= 2^20, M <= 2^24, and M*K, M*N, K*N each < 2^31.
 *   - Every pointer is a DEVICE pointer owned by the caller, 16-byte aligned
 *     (else QG_ERR_ALIGN), non-NULL when its size is non-zero (else
 *     QG_ERR_NULL). Outputs must not alias inputs. The library allocates no
 *     device memory and frees nothing.
 *   - stream is a hipStream_t (NULL = the default stream). Calls enqueue work
 *     on it and return without waiting. Argument checks run on the host
 *     before any HIP call; on any error nothing is enqueued and no output is
 *     touched. A failed launch returns QG_ERR_HIP. No C++ exception crosses
 *     this interface.
 *   - Identical inputs give bit-identical outputs: no reduction depends on
 *     the order in which workgroups finish.
 *
 * Packed-weight layout (the pages name only the container, "compressed-
 * tensors pack-quantized", with no bit layout, so this one is the library's
 * own). Codes are cut into tiles of 16 output columns x 128 K (one group).
 * Tile t = (n/16) * (K/128) + k/128. Inside a tile, lane l in [0,64) owns
 * column 16*(n/16) + l%16 and, for K step j in [0,4) and element i in [0,8),
 * k = 128*(k/128) + 32*j + 8*(l/16) + i -- the B-operand order of the
 * 16x16x32 bf16 matrix-core instruction.
 *   INT4: tile = 1024 bytes; lane l's K step j is the little-endian 32-bit
 *         word at byte 1024*t + 16*l + 4*j; element i is the nibble at bits
 *         4*p..4*p+3 with p = i/2 + 4*(i%2); the nibble holds q + 8.
 *   INT8: tile = 2048 bytes; element i of K step j of lane l is the byte at
 *         2048*t + 32*l + 8*j + i, holding q in two's complement.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QG_OK = 0,
  QG_ERR_NULL = 1,      /* a required pointer is NULL                      */
  QG_ERR_SHAPE = 2,     /* K, N or M outside the rules above               */
  QG_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned                */
  QG_ERR_DTYPE = 4,     /* unsupported dtype enum for that argument        */
  QG_ERR_WORKSPACE = 5, /* workspace missing or smaller than required      */
  QG_ERR_HIP = 6,       /* the HIP runtime reported an error at launch     */
  QG_ERR_PLAN = 7       /* an explicit tiling plan is not supported        */
} qg_status;

/* Element types. The *_CBM values name scales (fp16 or bf16) stored
 * column-block-major by qg_prepack_scales; only the GEMM entry points accept
 * them (every other entry point returns QG_ERR_DTYPE). */
typedef enum {
  QG_BF16 = 0, QG_F16 = 1, QG_F32 = 2, QG_F16_CBM = 3, QG_BF16_CBM = 4
} qg_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* qg_status_str(qg_status s);

/* Bytes of packed codes for a [K,N] weight: K*N/2 (bits=4) or K*N (bits=8);
 * 0 for an invalid shape or bit width. */
size_t qg_packed_bytes(int bits, int64_t K, int64_t N);

/* Bytes of the [K/128, N] scale array (2 bytes per scale). */
size_t qg_scale_bytes(int64_t K, int64_t N);

/* Workspace the GEMM needs for this shape; 0 when the chosen plan needs
 * none (always 0 at M = 1, the decode GEMV, and at M = 2..16 for shapes of
 * at most 40 groups and 512 column blocks, the 2-16-row GEMV). The first
 * 65536 bytes of a workspace hold arrival counters: they must
 * be zero before the first call that uses the workspace, and every completed
 * call leaves them zero again. The rest holds fp32 split-K partial sums
 * (the small-M kernel: M <= 16, or any M under an explicit plan) or, for
 * INT4 with M > 16 on the library's plan, the per-row, per-group activation
 * sums that remove the code offset; it needs no initial value. Calls that share
 * one workspace must not overlap in time (use one stream or distinct
 * workspaces). The same sizes apply to the fp16-activation entry points. */
size_t qg_workspace_bytes(int bits, int64_t M, int64_t K, int64_t N);

/* RTN scale choice from the weights, no calibration data (W8A16 model card:
 * RTN, symmetric, group = 128, "pure RTN on the weights").
 *   W        [K,N], w_dt = QG_F32 or QG_BF16
 *   scales   [K/128,N] out: fp16 max|w|/7 (w4) or bf16 max|w|/127 (w8),
 *            fp32 division rounded to nearest even; NaN weights count as 0. */
qg_status qg_rtn_scales_w4(const void* W, qg_dtype w_dt, int64_t K, int64_t N,
                           void* scales, void* stream);
qg_status qg_rtn_scales_w8(const void* W, qg_dtype w_dt, int64_t K, int64_t N,
                           void* scales, void* stream);

/* Fixed-grid quantizer Q_s plus packing (QAD method paragraph of arXiv
 * 2607.04244: updated bf16 weights rounded back onto the frozen grid).
 *   W        [K,N], w_dt = QG_F32 or QG_BF16
 *   scales   [K/128,N], s_dt = QG_F16 or QG_BF16 -- inputs, never recomputed
 *   packed_w out, qg_packed_bytes(bits,K,N) bytes in the layout above
 * code = clamp(rne(W / s), lo, hi) with IEEE fp32 division; (lo,hi) = (-8,7)
 * for w4 and (-127,127) for w8; s == 0 or a NaN quotient gives 0; an
 * infinite quotient saturates. */
qg_status qg_pack_to_grid_w4(const void* W, qg_dtype w_dt, const void* scales,
                             qg_dtype s_dt, int64_t K, int64_t N,
                             void* packed_w, void* stream);
qg_status qg_pack_to_grid_w8(const void* W, qg_dtype w_dt, const void* scales,
                             qg_dtype s_dt, int64_t K, int64_t N,
                             void* packed_w, void* stream);

/* Reorder logical int8 codes [K,N] into the packed layout, and back.
 * prepack_w4 stores the low 4 bits of q + 8, so codes outside [-8,7] do not
 * survive the round trip; prepack_w8 stores q unchanged. unpack is the exact
 * inverse of prepack on in-range codes. */
qg_status qg_prepack_w4(const int8_t* codes, int64_t K, int64_t N,
                        void* packed_w, void* stream);
qg_status qg_unpack_w4(const void* packed_w, int64_t K, int64_t N,
                       int8_t* codes, void* stream);
qg_status qg_prepack_w8(const int8_t* codes, int64_t K, int64_t N,
                        void* packed_w, void* stream);
qg_status qg_unpack_w8(const void* packed_w, int64_t K, int64_t N,
                       int8_t* codes, void* stream);

/* out[M,N] = bf16_rne( x[M,K] . (s (.) W_q) ), fp32 accumulation.
 *   x         bf16 [M,K]
 *   packed_w  qg_packed_bytes(bits,K,N) bytes (from pack_to_grid or prepack)
 *   scales    [K/128,N]; s_dt = QG_F16 or QG_BF16
 *   out       bf16 [M,N]
 *   workspace qg_workspace_bytes(bits,M,K,N) bytes (may be NULL when 0);
 *             see qg_workspace_bytes for the zero-counter rule.
 * Products of activations and codes are exact; each group of 128 is summed
 * in fp32, multiplied by its fp32 scale and added to an fp32 accumulator.
 * INT4 codes enter the product as 136 + q and the offset 136 * sum x of each
 * group is removed in fp32: for M <= 16 both sums use the same instruction
 * and order, so an all-zero code column gives exactly 0; for M > 16 the
 * offset seeds the accumulation, leaving fp32 rounding of that cancellation.
 * Supported domain: |x| < 1e30. */
qg_status qgemm_w4a16(const void* x, const void* packed_w, const void* scales,
                      qg_dtype s_dt, void* out, int64_t M, int64_t K, int64_t N,
                      void* workspace, size_t workspace_bytes, void* stream);
qg_status qgemm_w8a16(const void* x, const void* packed_w, const void* scales,
                      qg_dtype s_dt, void* out, int64_t M, int64_t K, int64_t N,
                      void* workspace, size_t workspace_bytes, void* stream);

/* The same GEMMs with an explicit tiling plan, for tests and tuning.
 *   cols_per_wave  16-column blocks per wavefront: 1, 2 or 4
 *   k_waves        wavefronts of a workgroup that split K: 1, 2, 4 or 8 with
 *                  cols_per_wave 1; 1, 2 or 4 with cols_per_wave 2; 1 or 4
 *                  with cols_per_wave 4. A workgroup has 4 wavefronts, 6
 *                  (three along N) for cols_per_wave 2 with k_waves 2, or 8
 *                  when k_waves is 8
 *   splits         workgroups that split K (>= 1, at most K/128)
 * Any argument 0 takes the library's choice. Unsupported values give
 * QG_ERR_PLAN. workspace must cover qg_workspace_bytes_plan(). */
qg_status qgemm_w4a16_plan(const void* x, const void* packed_w,
                           const void* scales, qg_dtype s_dt, void* out,
                           int64_t M, int64_t K, int64_t N, void* workspace,
                           size_t workspace_bytes, int cols_per_wave,
                           int k_waves, int splits, void* stream);
qg_status qgemm_w8a16_plan(const void* x, const void* packed_w,
                           const void* scales, qg_dtype s_dt, void* out,
                           int64_t M, int64_t K, int64_t N, void* workspace,
                           size_t workspace_bytes, int cols_per_wave,
                           int k_waves, int splits, void* stream);
size_t qg_workspace_bytes_plan(int bits, int64_t M, int64_t K, int64_t N,
                               int cols_per_wave, int k_waves, int splits);

/* The W4A16 / W8A16 GEMMs with fp16 activations and fp16 output (the pages
 * serve the target with INT4 weights and FP16 activations: adaptfm-quant-
 * dflash README, "Stage 2: Target Model"; QAD paper, serving setup).
 *   x    fp16 [M,K];  out  fp16 [M,N], fp32 -> fp16 round to nearest even
 *        (values beyond the fp16 range become +-Inf).
 * Everything else -- packed weights, scales, workspace, plans, errors -- is
 * as for qgemm_w4a16 / qgemm_w8a16. INT4 codes enter as 1032 + q in fp16. */
qg_status qgemm_w4f16(const void* x, const void* packed_w, const void* scales,
                      qg_dtype s_dt, void* out, int64_t M, int64_t K, int64_t N,
                      void* workspace, size_t workspace_bytes, void* stream);
qg_status qgemm_w8f16(const void* x, const void* packed_w, const void* scales,
                      qg_dtype s_dt, void* out, int64_t M, int64_t K, int64_t N,
                      void* workspace, size_t workspace_bytes, void* stream);
qg_status qgemm_w4f16_plan(const void* x, const void* packed_w,
                           const void* scales, qg_dtype s_dt, void* out,
                           int64_t M, int64_t K, int64_t N, void* workspace,
                           size_t workspace_bytes, int cols_per_wave,
                           int k_waves, int splits, void* stream);
qg_status qgemm_w8f16_plan(const void* x, const void* packed_w,
                           const void* scales, qg_dtype s_dt, void* out,
                           int64_t M, int64_t K, int64_t N, void* workspace,
                           size_t workspace_bytes, int cols_per_wave,
                           int k_waves, int splits, void* stream);

/* Dense dequantized weight W[k,n] = s[k/128, n] * q[k,n] (QAD paper, QAD
 * paragraph: the student is initialised from the dequantized weights
 * s (.) W_q; adaptfm-quant-dflash README, Stage 2: the dense dequantized
 * bf16 twin used for drafter finetuning and calibration).
 *   packed_w  qg_packed_bytes(bits,K,N) bytes
 *   scales    [K/128,N]; s_dt = QG_F16 or QG_BF16
 *   out       [K,N] row-major, out_dt = QG_BF16 or QG_F16
 * s * q is exact in fp32; the one rounding is to out_dt, nearest even
 * (+-Inf beyond its range). */
qg_status qg_dequant_w4(const void* packed_w, const void* scales, qg_dtype s_dt,
                        int64_t K, int64_t N, void* out, qg_dtype out_dt,
                        void* stream);
qg_status qg_dequant_w8(const void* packed_w, const void* scales, qg_dtype s_dt,
                        int64_t K, int64_t N, void* out, qg_dtype out_dt,
                        void* stream);

/* Fixed-grid fake quantizer of QAD's forward pass (QAD paper, QAD method
 * paragraph: the student's weights W pass through Q_s under the frozen
 * scales, trained with a straight-through estimator).
 *   W      [K,N], w_dt = QG_F32 or QG_BF16
 *   scales [K/128,N], s_dt = QG_F16 or QG_BF16
 *   out    [K,N], out_dt = QG_BF16, QG_F16 or QG_F32
 * out = s * clamp(rne(W / s), lo, hi): the codes of qg_pack_to_grid_w4/w8
 * (same division, rounding and special cases), the product exact in fp32,
 * one rounding to nearest even into out_dt. The straight-through estimator
 * passes the gradient through Q_s unchanged, so the backward pass is the
 * identity on the incoming gradient and has no entry point of its own. */
qg_status qg_fake_quant_w4(const void* W, qg_dtype w_dt, const void* scales,
                           qg_dtype s_dt, int64_t K, int64_t N, void* out,
                           qg_dtype out_dt, void* stream);
qg_status qg_fake_quant_w8(const void* W, qg_dtype w_dt, const void* scales,
                           qg_dtype s_dt, int64_t K, int64_t N, void* out,
                           qg_dtype out_dt, void* stream);

/* Grouped launch: several GEMMs that share x, M and K, each with its own
 * packed weight, scales, output and N -- a drafter layer set, or the K/V
 * projections of all drafter layers that the pages' fused-KV path computes
 * from one input (Qwen3.5-4B-DFlash-W8A16 model card, "Required vLLM
 * patches", the fused K+V buffer across the 5 layers) -- in one kernel launch
 * for M <= 16, which saves the per-launch fixed cost of the small shapes
 * (for M > 16 the items run as consecutive prefill launches).
 *   items     HOST array of count descriptors (1 <= count <= 16), read during
 *             the call only; each N a positive multiple of 16
 *   x, M, K   shared input (bf16, or fp16 for the *f16 variants)
 *   workspace qg_workspace_bytes_grouped(...) bytes, same rules as above
 * Each item's output equals what the single GEMM computes on it, bit for
 * bit when the single call and the group pick the same tiling plan; the
 * group's plan is chosen for the summed N, which must also meet the limits
 * of one N. Errors as for qgemm_w4a16, plus QG_ERR_NULL for items == NULL
 * and QG_ERR_SHAPE for a count out of range. */
typedef struct {
  const void* packed_w;   /* qg_packed_bytes(bits, K, N) bytes */
  const void* scales;     /* [K/128, N] */
  void* out;              /* [M, N] */
  int64_t N;
} qg_group_item;

size_t qg_workspace_bytes_grouped(int bits, int64_t M, int64_t K,
                                  const qg_group_item* items, int count);
qg_status qgemm_w4a16_grouped(const void* x, const qg_group_item* items, int count,
                              qg_dtype s_dt, int64_t M, int64_t K, void* workspace,
                              size_t workspace_bytes, void* stream);
qg_status qgemm_w8a16_grouped(const void* x, const qg_group_item* items, int count,
                              qg_dtype s_dt, int64_t M, int64_t K, void* workspace,
                              size_t workspace_bytes, void* stream);
qg_status qgemm_w4f16_grouped(const void* x, const qg_group_item* items, int count,
                              qg_dtype s_dt, int64_t M, int64_t K, void* workspace,
                              size_t workspace_bytes, void* stream);
qg_status qgemm_w8f16_grouped(const void* x, const qg_group_item* items, int count,
                              qg_dtype s_dt, int64_t M, int64_t K, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Drafter attention with a symmetric sliding window over a full KV cache
 * ("Quantize the Target, Quantize the Drafter", arXiv 2607.04244, Drafter SWA
 * paragraph: a fixed window of 1,024 or 2,048 tokens, symmetric around each
 * query because the drafter's mask-token queries attend bidirectionally,
 * applied only inside the attention kernel while the cache keeps every
 * position, and full attention for sequences within the window size; the
 * drafter setup paragraph fixes a draft block at 16 tokens).
 *
 * For each sequence b, its block of T queries sits at cache positions
 * S_b - T .. S_b - 1, where S_b = seq_lens[b] counts every cache entry of the
 * sequence, the block's own T included. Query t at position p attends to the
 * cache positions j < S_b with |p - j| <= window / 2 (integer division), or
 * to all j < S_b when window == 0 or S_b <= window:
 *   out[b,t,h,:] = sum_j softmax_j(scale * q[b,t,h,:] . k[b,j,h/G,:]) v[b,j,h/G,:]
 * with G = Hq / Hkv query heads per KV head.
 *   q         DEVICE bf16 [B, T, Hq, D]
 *   k_cache,
 *   v_cache   DEVICE bf16 [B, S_max, Hkv, D]; rows at or past seq_lens[b]
 *             are never read
 *   seq_lens  DEVICE int32 [B]; each must lie in [T, S_max] (values outside
 *             are clamped into that range, never read out of bounds)
 *   out       DEVICE bf16 [B, T, Hq, D] (must not alias the inputs)
 *   D         must be 128; 1 <= T <= 16; Hq % Hkv == 0, Hq <= 4096; window >= 0
 *   scale     the softmax scale (1/sqrt(D) in the usual model), finite
 *   workspace qg_swa_workspace_bytes(...) bytes, 16-byte aligned (NULL when
 *             that is 0); its first 64 KiB are arrival counters that must be
 *             zero before the first call and are left zero by every call;
 *             calls that overlap on one workspace race
 * Softmax and sums in fp32 on the matrix core (probabilities carried as a
 * bf16 pair, ~2^-18 relative), one rounding to bf16 at the end; identical
 * inputs give identical bits. Errors: QG_ERR_NULL, QG_ERR_ALIGN (tensors 16
 * bytes, seq_lens 4), QG_ERR_SHAPE (sizes above, S_max * Hkv * D * 2 or
 * T * Hq * D * 2 at or past 2^31 bytes, more than 16384 (sequence, head)
 * pairs for a call that needs the workspace), QG_ERR_WORKSPACE; nothing is
 * launched on error. B == 0 is a no-op. */
size_t qg_swa_workspace_bytes(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t D,
                              int64_t S_max, int64_t window);
qg_status qg_swa_attention(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* seq_lens, void* out, int64_t B, int64_t T,
                           int64_t Hq, int64_t Hkv, int64_t D, int64_t S_max,
                           int64_t window, float scale, void* workspace,
                           size_t workspace_bytes, void* stream);
/* The same with the work split chosen by the caller, for tests and tuning.
 *   chunk  keys per workgroup: a multiple of 32, or 0 for the library's own
 *   heads  query heads per workgroup: 0 lets the library choose; 1 runs one
 *          query head per workgroup; 2, 3, 4, 5, 6 or 8 (a divisor of
 *          Hq / Hkv) runs that many heads of one KV head per workgroup over
 *          one shared stream of its K/V rows, with at most 16 chunks
 * Results match qg_swa_attention's to the summation order of the chunks.
 * Errors as qg_swa_attention, plus QG_ERR_SHAPE for a heads value outside
 * that list or a split with too many chunks; the workspace size depends on
 * both values, and qg_swa_workspace_bytes_plan returns 0 for a split that
 * cannot run. */
size_t qg_swa_workspace_bytes_plan(int64_t B, int64_t T, int64_t Hq, int64_t Hkv,
                                   int64_t D, int64_t S_max, int64_t window,
                                   int64_t chunk, int64_t heads);
qg_status qg_swa_attention_plan(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* seq_lens, void* out, int64_t B, int64_t T,
                                int64_t Hq, int64_t Hkv, int64_t D, int64_t S_max,
                                int64_t window, float scale, int64_t chunk, int64_t heads,
                                void* workspace, size_t workspace_bytes, void* stream);

/* qgemm_w4a16 for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It takes no workspace argument: the split-K partials, arrival counters
 * and prefill INT4 offsets go to the library's fixed scratch buffer, a
 * device array of qg_noalloc_scratch_bytes() (8 MiB) that every GPU the
 * library runs on holds until the process ends. The call allocates and
 * frees nothing. Arguments, checks, results and errors are those of
 * qgemm_w4a16 with the workspace omitted, plus QG_ERR_WORKSPACE when
 * qg_workspace_bytes(4, M, K, N) exceeds the scratch (e.g. a prefill past
 * about 27,000 rows at K = 9728), and QG_ERR_HIP when the scratch address
 * cannot be obtained. The first call on a device also enqueues, on stream,
 * the clearing of the scratch's arrival counters (every later call leaves
 * them at zero). All calls on one GPU share that GPU's scratch: calls that
 * may overlap in time on one GPU (concurrent streams, or graphs replayed
 * on several streams) race and must be ordered by the caller. */
size_t qg_noalloc_scratch_bytes(void);
qg_status qgemm_w4a16_noalloc(const void* x, const void* packed_w, const void* scales,
                              qg_dtype s_dt, void* out, int64_t M, int64_t K, int64_t N,
                              void* stream);

/* Column-block-major scales: a storage order of the same scales, prepared
 * once at load time like the packed codes. The logical scales[K/128, N]
 * (group g, column n) become cbm[N/16][K/128][16] with
 *   cbm[((n / 16) * (K / 128) + g) * 16 + n % 16] = scales[g * N + n],
 * so the scales of one 16-column block for every group are one contiguous
 * run (the layout is the library's own; the pages fix none). A small-M GEMM
 * workgroup then reads its scales as one run instead of gathering one piece
 * per group from rows N * 2 bytes apart, which delays its first multiply
 * (about 0.3 µs of the 8 µs decode GEMV on MI355X). Pass the result to the
 * GEMM entry points with s_dt = QG_F16_CBM or QG_BF16_CBM; their outputs
 * are bit-identical to those with the logical scales.
 *   scales  [K/128, N] logical, s_dt = QG_F16 or QG_BF16
 *   out     K/128 * N elements of s_dt (not in place)
 * K and N follow the shape rules above. */
qg_status qg_prepack_scales(const void* scales, qg_dtype s_dt, int64_t K, int64_t N,
                            void* out, void* stream);

/* Read-stream probe: a measurement aid, not a step of the method. Reads
 * [src, src + bytes) once with 16-byte nontemporal vector loads over
 * `workgroups` workgroups of 256 threads (grid stride, four loads in flight
 * per thread)
 * and discards the data; a launch over a buffer that the 256 MB Infinity
 * Cache cannot hold measures the rate at which this GPU streams `bytes` from
 * HBM in one launch, the ceiling the HBM-bound entry points are reported
 * against beside the 8 TB/s figure.
 *   src         bytes bytes; bytes a positive multiple of 16, below 2^40
 *   workgroups  1 .. 65536
 *   sink        4 bytes, written only when the XOR of the 32-bit words one
 *               thread reads equals 0x9E3779B9 (the value then stored), so the
 *               loads cannot be optimised away; otherwise untouched
 * src and sink follow the pointer rules above (QG_ERR_NULL, QG_ERR_ALIGN);
 * a bad size or workgroup count is QG_ERR_SHAPE. */
qg_status qg_read_stream(const void* src, size_t bytes, int workgroups, void* sink,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */

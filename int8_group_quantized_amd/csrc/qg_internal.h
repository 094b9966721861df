// Host-side launchers behind the C ABI (one per kernel family). Arguments
// are already validated by the ABI layer when these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qgemm.h"

namespace qg {

constexpr int kGroup = 128;                 // K extent of one scale group
constexpr int kTileCols = 16;               // output columns per packed tile
constexpr uint32_t kCounterBytes = 65536;   // arrival counters at a workspace's start
constexpr int kPrefillRows = 64;            // rows of a prefill tile
constexpr int kGemvGroups = 5;              // groups per decode-GEMV wavefront per round
constexpr int kSwaMaxChunks = 256;          // key chunks one (sequence, head) may have
constexpr int kSwaRingMaxChunks = 16;       // the same for the shared-ring kernel (merge table)
constexpr int kSwaPartFloats = 16 * 128 + 32;   // a chunk's record: O[16][128], max[16], sum[16]

// Small-M tiling: each wavefront covers `nbw` 16-column blocks; `wk`
// wavefronts of a 4-wave workgroup split the K range of the workgroup;
// `splits` workgroups split K across the grid (fp32 partials + a last-arrival
// reduction). Rows are covered 16 at a time (grid z).
// Several GEMMs that share x, M and K (a layer's Linear set, or the K/V
// projections of every drafter layer), run by one launch of the small-M
// kernel: item i owns column workgroups [wg_first, next item's wg_first) and
// columns [col_first, col_first + n) of the concatenated split-K partials. A
// single GEMM is a group of one. The items are stored as an array of structs
// so that a group of one reads only the first 40 bytes of the table.
struct GroupItem {
  const char* packed = nullptr;
  const uint16_t* scales = nullptr;
  uint16_t* out = nullptr;
  int n = 0;
  int wg_first = 0;
  int col_first = 0;
  int pad = 0;
};

struct GroupArgs {
  static constexpr int kMax = 16;
  int count = 0;
  int n_total = 0;
  int wg_total = 0;
  int pad = 0;
  GroupItem item[kMax];
};

struct SmallPlan {
  int bits = 4;
  int mr = 16;        // 1: single-row layout of x in LDS; 16: rows padded to 16
  int nbw = 1;
  int wn = 4;         // wavefronts along N in a workgroup
  int wk = 1;
  int splits = 1;
  int gps = 1;        // scale groups per split (one workgroup's K range)
  int sg = 1;         // groups per LDS stage of x
  int wgs_n = 1;      // workgroups along N
  int row_blocks = 1; // 16-row blocks along M
};

// Large-M (prefill) tiling: 128 x 128 output tiles, one workgroup each.
struct PrefillPlan {
  int wn = 4;         // wavefronts per workgroup = 64-column sub-tiles per tile
  int tiles_n = 1;    // 64 * wn-column tiles along N
  int tiles = 1;      // total tiles (= workgroups)
  int64_t mp = 64;    // M rounded up to the 64-row tile
};

bool make_prefill_plan(int64_t M, int64_t K, int64_t N, PrefillPlan* plan);
// Workspace bytes of the prefill path (INT4: counters area + negated offsets).
size_t prefill_workspace(int bits, const PrefillPlan& p, int64_t K);
// s_cbm: scales column-block-major (qg_prepack_scales) instead of [K/128, N].
hipError_t launch_gemm_prefill(int bits, const PrefillPlan& p, const void* x, bool x_f16,
                               const void* packed, const void* scales, bool s_bf16, bool s_cbm,
                               void* out, int64_t M, int64_t K, int64_t N, void* ws,
                               hipStream_t st);

bool make_small_plan(int bits, int64_t M, int64_t K, int64_t N, int nbw, int wk,
                     int splits, SmallPlan* plan);
size_t small_plan_workspace(const SmallPlan& p, int64_t M, int64_t N);
// False when the split partials of a plan over n_total columns would pass
// 2^31 bytes.
bool small_plan_partials_fit(const SmallPlan& p, int64_t n_total);
size_t small_plan_lds_bytes(const SmallPlan& p, int64_t M);

hipError_t launch_rtn_scales(int bits, const void* W, bool w_bf16, int64_t K,
                             int64_t N, void* scales, hipStream_t st);
hipError_t launch_pack_to_grid(int bits, const void* W, bool w_bf16,
                               const void* scales, bool s_bf16, int64_t K,
                               int64_t N, void* packed, hipStream_t st);
hipError_t launch_prepack(int bits, const int8_t* codes, int64_t K, int64_t N,
                          void* packed, hipStream_t st);
hipError_t launch_unpack(int bits, const void* packed, int64_t K, int64_t N,
                         int8_t* codes, hipStream_t st);
// out_kind: 0 bf16, 1 fp16, 2 fp32.
hipError_t launch_fake_quant(int bits, const void* W, bool w_bf16, const void* scales,
                             bool s_bf16, void* out, int out_kind, int64_t K, int64_t N,
                             hipStream_t st);
hipError_t launch_dequant(int bits, const void* packed, const void* scales, bool s_bf16,
                          void* out, bool out_f16, int64_t K, int64_t N, hipStream_t st);
// Fills the group's workgroup prefixes for plan p (wgs_n is per item there).
void small_plan_group(const SmallPlan& p, GroupArgs* g);
hipError_t launch_gemm_small(int bits, const SmallPlan& p, const void* x, bool x_f16,
                             const GroupArgs& g, bool s_bf16, bool s_cbm, int64_t M, int64_t K,
                             void* workspace, hipStream_t st);
// Decode GEMV (gemv.hip): the library's own plan for M = 1, and for 2-16
// rows where gemv_rows_fits (K of at most 40 groups, at most 512 column
// blocks over all items). One workgroup per 16-column block (of every item
// of the group), gemv_k_waves(K) wavefronts splitting K; no workspace.
int gemv_k_waves(int64_t K);
bool gemv_rows_fits(int64_t M, int64_t K, int64_t n_total);
void gemv_group(GroupArgs* g);
hipError_t launch_gemv(int bits, const void* x, bool x_f16, const GroupArgs& g, bool s_bf16,
                       bool s_cbm, int64_t M, int64_t K, hipStream_t st);
// Logical scales [K/128, N] -> column-block-major [N/16][K/128][16] (16-bit).
hipError_t launch_prepack_scales(const void* scales, int64_t K, int64_t N, void* out,
                                 hipStream_t st);

// Drafter sliding-window attention (swa_attention.hip): one workgroup per
// (sequence, query head, chunk of `chunk` keys); `units` = sequences x KV heads
// x chunks; `window` is 0 when no sequence can exceed it.
struct SwaPlan {
  int window = 0;
  int chunk = 128;
  int nchunks = 1;
  int units = 0;
  int grid = 0;
  bool q_lds = false;   // queries staged once per workgroup in LDS (short chunks)
  int ring = 0;         // > 0: that many query heads of one KV head per workgroup
                        // over a shared K/V ring (units then count sequence x KV
                        // head x head group x chunk); 0: one query head each
};
// chunk: keys per workgroup, 0 for the library's choice; heads: query heads
// per workgroup, 0 for the library's choice, 1 for the one-head kernel, 2-6
// or 8 (dividing Hq / Hkv) for the shared-ring kernel. False when no plan fits.
bool make_swa_plan(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t S_max, int64_t window,
                   int64_t chunk, int64_t heads, SwaPlan* p);
size_t swa_workspace(const SwaPlan& p, int64_t B, int64_t Hq);
hipError_t launch_swa_attention(const SwaPlan& p, const void* q, const void* k, const void* v,
                                const int32_t* seq_lens, void* out, int64_t T, int64_t Hq,
                                int64_t Hkv, int64_t S_max, float scale, void* ws,
                                hipStream_t st);

// The fixed scratch buffer of the no-allocation entry point (scratch.hip):
// kScratchBytes of device memory per GPU, held for the life of the process.
// Returns its device address on the stream's device (taken once per device
// with hipGetSymbolAddress) and, on that device's first use, enqueues on st
// the clearing of its arrival counters.
constexpr size_t kScratchBytes = size_t(8) << 20;
hipError_t scratch_for_stream(hipStream_t st, void** ptr);

// Read-stream probe (read_probe.hip): reads bytes (a multiple of 16) at src
// once over `workgroups` workgroups of 256 threads; stores kReadProbeMark to
// sink only when a thread's XOR of what it read equals it.
constexpr uint32_t kReadProbeMark = 0x9E3779B9u;
hipError_t launch_read_stream(const void* src, int64_t bytes, int workgroups, void* sink,
                              hipStream_t st);

}  // namespace qg

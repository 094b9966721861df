// Host-side planning of the kernel launches: tile and split choices and the
// workspace each plan needs. Plain C++ (no device code), shared by the
// library and by a host-only build of the argument checks.
#include <algorithm>
#include <cmath>

#include "qg_internal.h"

namespace qg {
namespace {

constexpr int kMaxCounters = kCounterBytes / sizeof(uint32_t);
constexpr int64_t kLdsAuto = 80 * 1024;     // LDS per workgroup the library's own plans use
constexpr int64_t kLdsMax = 160 * 1024;     // LDS a workgroup may have (explicit plans)
constexpr int kCUs = 256;                   // MI355X compute units (plan heuristic only)

// Small-M tilings the library instantiates: (cols per wave, waves along N,
// waves along K).
bool shape_supported(int nbw, int wn, int wk) {
  static const int ok[][3] = {{1, 4, 1}, {1, 2, 2}, {1, 1, 4}, {1, 1, 8},
                              {2, 4, 1}, {2, 3, 2}, {2, 1, 4}, {4, 4, 1}, {4, 1, 4}};
  for (const auto& s : ok)
    if (s[0] == nbw && s[1] == wn && s[2] == wk) return true;
  return false;
}

// LDS bytes per staged group: x fragments (rows padded to 16 unless M == 1)
// and the 16 scales of each of the workgroup's column blocks.
int64_t lds_per_group(int wn, int nbw, int mr) {
  return (mr == 1 ? 256 : 4096) + (int64_t)wn * nbw * 32;
}

}  // namespace

// ---- small-M kernel (M <= 16) ----

size_t small_plan_lds_bytes(const SmallPlan& p, int64_t M) {
  (void)M;
  const size_t stage = (size_t)p.sg * (size_t)lds_per_group(p.wn, p.nbw, p.mr) + 256;
  const size_t red = (size_t)(p.wk - 1) * p.wn * p.nbw * 64 * 16;
  return stage > red ? stage : red;
}

bool make_small_plan(int bits, int64_t M, int64_t K, int64_t N, int nbw, int wk, int splits,
                     SmallPlan* plan) {
  const int64_t NB = N / kTileCols;
  const int64_t G = K / kGroup;
  SmallPlan p;
  p.bits = bits;
  p.mr = (M == 1) ? 1 : 16;
  p.row_blocks = (int)((M + 15) / 16);
  const bool own = (nbw == 0 && wk == 0 && splits == 0);
  if (own) {
    // The library's own plan for 2-16 rows (one row runs the decode GEMV),
    // from sweeps of the verification shapes on MI355X: wide N shares each
    // staged x group between eight column blocks (two per wavefront), long K
    // splits across workgroups of four column blocks (about 16 INT4 or 13
    // INT8 groups each), and the rest use four K-wavefronts per column block.
    // Wide INT4 shapes instead take six column blocks over six wavefronts,
    // two along K (K = 2560, N = 19456: 9.8 against 10.25 us; INT8 13.7
    // against 13.0, so INT8 keeps eight blocks along N).
    if (NB >= 1024) {
      nbw = 2; wk = (bits == 4) ? 2 : 1; splits = 1;
    } else if (G >= 40) {
      const int per = bits == 4 ? 16 : 13;
      nbw = 1; wk = 1; splits = (int)((G + per - 1) / per);
    } else {
      nbw = 1; wk = 4;
    }
  }
  if (nbw == 0) nbw = 1;
  if (wk == 0) {
    // Enough column-block waves to fill the chip without splitting K, else
    // waves that split K inside a workgroup.
    wk = (NB >= 1024) ? 1 : (NB >= 128 ? 4 : 8);
  }
  const int wn = (wk >= 8) ? 1 : ((nbw >= 2 && wk == 4) ? 1 : ((nbw == 2 && wk == 2) ? 3 : 4 / wk));
  if (!shape_supported(nbw, wn, wk)) return false;
  p.nbw = nbw;
  p.wk = wk;
  p.wn = wn;
  p.wgs_n = (int)((NB + (int64_t)wn * nbw - 1) / ((int64_t)wn * nbw));
  // The workgroup stages x and the scales for its whole K range at once.
  // The library's plans split K across workgroups so that this fits two
  // workgroups per CU; explicit plans may use up to a CU's LDS.
  const int64_t per_group = lds_per_group(wn, nbw, p.mr);
  if (splits == 0) {
    // The own plan may use up to a CU's LDS; other plans keep two
    // workgroups per CU.
    const int64_t fit = ((own ? kLdsMax - 512 : kLdsAuto - 256)) / per_group;
    splits = (int)((G + fit - 1) / fit);
  } else if (own) {
    const int64_t fit = (kLdsMax - 512) / per_group;
    splits = (int)std::max<int64_t>(splits, (G + fit - 1) / fit);
  }
  if (splits < 1 || splits > G) return false;
  p.gps = (int)((G + splits - 1) / splits);
  p.splits = (int)((G + p.gps - 1) / p.gps);   // no empty split
  p.sg = p.gps;
  if (p.splits > 65535 || p.row_blocks > 65535) return false;
  if (p.splits > 1 && (int64_t)p.wgs_n * p.row_blocks > kMaxCounters) return false;
  if (!small_plan_partials_fit(p, N)) return false;
  if ((int64_t)small_plan_lds_bytes(p, M) > kLdsMax) return false;
  *plan = p;
  return true;
}

size_t small_plan_workspace(const SmallPlan& p, int64_t M, int64_t N) {
  (void)M;
  if (p.splits <= 1) return 0;
  // Every split keeps whole 16-row blocks (the accumulators' lane order).
  return (size_t)kCounterBytes +
         (size_t)p.splits * (size_t)p.row_blocks * 16 * (size_t)N * sizeof(float);
}

bool small_plan_partials_fit(const SmallPlan& p, int64_t n_total) {
  // The split partials are addressed with 32-bit byte offsets below 2^31.
  return p.splits <= 1 || (int64_t)p.splits * p.row_blocks * 16 * n_total * 4 < (int64_t(1) << 31);
}

void small_plan_group(const SmallPlan& p, GroupArgs* g) {
  const int per = p.wn * p.nbw;                      // column blocks per workgroup
  int wg = 0, col = 0;
  for (int i = 0; i < g->count; ++i) {
    g->item[i].wg_first = wg;
    g->item[i].col_first = col;
    wg += (g->item[i].n / kTileCols + per - 1) / per;
    col += g->item[i].n;
  }
  g->wg_total = wg;
  g->n_total = col;
}

// ---- decode GEMV (M = 1) ----

int gemv_k_waves(int64_t K) {
  // Enough wavefronts that each takes about kGemvGroups groups (the decode shapes:
  // K = 2560 -> 4, K = 9728 -> 16), rounded up to a power of two, at most 16.
  const int64_t want = (K / kGroup + kGemvGroups - 1) / kGemvGroups;
  int wk = 1;
  while (wk < want && wk < 16) wk *= 2;
  return wk;
}

bool gemv_rows_fits(int64_t M, int64_t K, int64_t n_total) {
  // Measured on the verification shapes (M = 16): the fused QKV projection
  // (224 column blocks, 20 groups) runs 5.8 -> 4.9 us with x loaded per
  // wavefront; the gate/up projection (1216 blocks) and the down projection
  // (76 groups) are faster staged.
  return M >= 2 && M <= 16 && K / kGroup <= 40 && n_total / kTileCols <= 512;
}

void gemv_group(GroupArgs* g) {
  int wg = 0, col = 0;
  for (int i = 0; i < g->count; ++i) {
    g->item[i].wg_first = wg;
    g->item[i].col_first = col;
    wg += g->item[i].n / kTileCols;
    col += g->item[i].n;
  }
  g->wg_total = wg;
  g->n_total = col;
}

// ---- prefill (M > 16) ----

// Tile width: 256 columns (four wavefronts, two workgroups per CU) unless
// 128 columns (two wavefronts, three per CU) fills the last round of
// workgroups better.
bool make_prefill_plan(int64_t M, int64_t K, int64_t N, PrefillPlan* plan) {
  const int64_t tiles_m = (M + kPrefillRows - 1) / kPrefillRows;
  const int64_t NB = N / kTileCols;
  double best = -1.0;
  for (int wn : {4, 2}) {
    const int64_t tiles = tiles_m * ((NB + 4 * wn - 1) / (4 * wn));
    const int64_t slots = (int64_t)kCUs * (wn == 4 ? 2 : 3);
    const int64_t rounds = (tiles + slots - 1) / slots;
    // useful fraction of the occupied slot-rounds, with the narrower tile's
    // extra x traffic priced at 15%
    const double eff = (double)tiles / (double)(rounds * slots) * (wn == 4 ? 1.0 : 0.85);
    if (tiles > 0x7FFFFFFF) return false;
    if (eff > best + 1e-9) {
      best = eff;
      plan->wn = wn;
      plan->tiles_n = (int)((NB + 4 * wn - 1) / (4 * wn));
      plan->tiles = (int)tiles;
    }
  }
  plan->mp = tiles_m * kPrefillRows;
  if (plan->mp * (K / kGroup) > 0x7FFFFFFF) return false;
  return true;
}

size_t prefill_workspace(int bits, const PrefillPlan& p, int64_t K) {
  if (bits != 4) return 0;
  return (size_t)kCounterBytes + (size_t)p.mp * (size_t)(K / kGroup) * sizeof(float);
}

// ---- drafter attention ----

bool make_swa_plan(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t S_max, int64_t window,
                   int64_t chunk_req, int64_t heads_req, SwaPlan* p) {
  const int64_t w = window >= S_max ? 0 : window;   // a window past every sequence is no window
  // Longest key span of any sequence: the whole cache without a window; else
  // a sequence within the window (full attention, at most W keys) or the
  // block plus W / 2 keys before its first query.
  const int64_t span = w == 0 ? S_max : std::min<int64_t>(S_max, std::max<int64_t>(w, T + w / 2));
  // Key span of a sequence longer than the window: the block plus W / 2 keys
  // before its first query; the chunk count is sized for it (a shorter
  // sequence's full-attention span then takes more steps per wavefront).
  const int64_t typ = w == 0 ? S_max : std::min<int64_t>(S_max, T + w / 2);
  const int64_t G = Hq / Hkv;
  auto ring_ok = [&](int64_t h) {
    return (h == 2 || h == 3 || h == 4 || h == 5 || h == 6 || h == 8) && G % h == 0;
  };
  int64_t ring = 0;
  if (heads_req > 1) {
    if (!ring_ok(heads_req)) return false;
    ring = heads_req;
  } else if (heads_req == 0 && chunk_req == 0) {
    // The shared-ring kernel reads each K/V row once for up to eight query
    // heads; it pays off on long spans once there are 16 or more (sequence,
    // KV head, head group) units to split into chunks (MI355X, 20 query over
    // 4 KV heads, full attention over 8,208 keys: batch 4 30 us against 39
    // us for one head per workgroup, batch 8 38 against 67, batch 16 63
    // against 173, batch 32 114 against 278; batch 2 equal, windowed spans
    // and batch 1 faster one head each).
    int64_t h = 0;
    for (int64_t c : {8, 6, 5, 4, 3, 2})
      if (h == 0 && ring_ok(c)) h = c;
    const int64_t groups = h > 0 ? B * Hkv * (G / h) : 0;
    if (h > 0 && typ >= 4096 && groups >= 16 && groups <= 256) ring = h;
  }
  int64_t n = 1;
  if (ring > 0) {
    // About 256 workgroups, at least 512 keys per chunk.
    const int64_t groups = B * Hkv * (G / ring);
    n = std::max<int64_t>(1, std::min<int64_t>(256 / std::max<int64_t>(1, groups), typ / 512));
    n = std::min<int64_t>(n, kSwaRingMaxChunks);
  } else {
    // Chunk count: each extra chunk adds its partial to the cross-workgroup
    // merge, fewer chunks leave each workgroup more keys to stream. Sweeps of
    // the drafter's Long-context shapes on MI355X: at batch 1 the best counts
    // grow about as the cube root of the span (5 chunks for 528 keys, 6-7 for
    // 1,040, ~9-12 for 8,208); with 128 or more query heads in the call a
    // windowed span is fastest unsplit, and longer spans want at most about
    // two workgroups per CU. A chunk shorter than about one 32-key step per
    // wavefront saves less than its merge costs.
    const int64_t heads = std::max<int64_t>(1, B * Hq);
    if (!(heads >= 128 && typ <= 2048)) {
      n = (int64_t)std::llround(0.6 * std::cbrt((double)typ));
      n = std::min<int64_t>(n, std::max<int64_t>(1, 512 / heads));
      n = std::max<int64_t>(1, std::min<int64_t>(n, typ / 96));   // >= 96 keys per chunk
    }
  }
  int64_t chunk = (span + n - 1) / n;
  chunk = (chunk + 31) / 32 * 32;
  if (chunk_req > 0) chunk = chunk_req;
  p->window = (int)w;
  p->chunk = (int)chunk;
  p->nchunks = (int)((span + chunk - 1) / chunk);
  p->ring = (int)ring;
  if (p->nchunks > (ring > 0 ? kSwaRingMaxChunks : kSwaMaxChunks)) return false;
  if (ring > 0) {
    const int64_t units = B * Hkv * (G / ring) * p->nchunks;
    if (units >= (1 << 24)) return false;
    p->units = (int)units;
    p->grid = (int)units;
    p->q_lds = false;
    return true;
  }
  const int64_t units = B * Hkv * p->nchunks;
  const int64_t grid = 8 * G * ((units + 7) / 8);
  if (units >= (1 << 24) || grid > 0x7FFFFFFF) return false;
  p->units = (int)units;
  p->grid = (int)grid;
  // At most two 32-key steps per wavefront in a typical chunk: the queries
  // go through LDS once per workgroup.
  p->q_lds = (typ + p->nchunks - 1) / p->nchunks <= 2 * 4 * 32;
  return true;
}

size_t swa_workspace(const SwaPlan& p, int64_t B, int64_t Hq) {
  if (p.nchunks <= 1) return 0;
  return (size_t)kCounterBytes + (size_t)B * Hq * p.nchunks * kSwaPartFloats * sizeof(float);
}

}  // namespace qg

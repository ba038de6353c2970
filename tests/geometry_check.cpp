// Host-side bounds check of the balance launches (count, plan, reroute).
//
// For one shape and layer count it walks every workgroup and every thread of
// each launch with the kernels' own index functions (ultraep_geometry.h) and
// checks every global index against the buffer it addresses, with the
// buffers sized by the library itself (ultraep_workspace_bytes,
// ultraep_plan_bytes, ultraep_plan_field); it also checks that the tile-base
// workgroups write every (tile, expert) base exactly once, that the
// histogram sum reads every expert column of every row exactly once, and that
// the planner's LDS tables fit the allocation ultraep_create accepted.
// Indices that depend on the data (a pair's instance, a layout row) are
// guarded inside the kernels and are not walked here.
//
// Usage: geometry_check E R S D L T k [plant]
//   plant (optional) replaces one index function by a plausible mistake, to
//   show that the walk catches it: "sum-row" (the histogram sum's batch
//   without its clamp to the last row), "scan-row" (the same in the tile-base
//   scan), "scan-ew" (experts per tile-base workgroup not capped at E),
//   "local-first" (the planner's early first batch of the local takes loaded
//   also for ranks without tiles), "xcd-tail" (the reroute's XCD block order
//   applied also to the blocks past the last whole group of eight).
// Exit status: 0 every index in bounds, 1 a violation (printed), 2 usage or
// a shape the library refuses.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "ultraep.h"
#include "ultraep_geometry.h"

using namespace ultraep;

namespace {

long fails = 0;
std::string plant;

void fail(const char* what, long long a, long long b, long long c = 0) {
  if (fails++ < 12) std::fprintf(stderr, "out of bounds: %s (%lld, %lld, %lld)\n", what, a, b, c);
}

int32_t sum_row_x(int32_t tb, int u, int32_t nch, int32_t ntiles) {
  return plant == "sum-row" ? tb + u * nch : sum_row(tb, u, nch, ntiles);
}
int32_t scan_row_x(int32_t tb, int u, int32_t ntiles) {
  return plant == "scan-row" ? tb + u : scan_row(tb, u, ntiles);
}
bool local_prefetch_x(int32_t tpr) { return plant == "local-first" ? true : local_prefetch(tpr); }
int64_t xcd_block_x(int64_t g, int64_t n) {
  return plant == "xcd-tail" ? (g % kXcds) * (n / kXcds) + g / kXcds : xcd_block(g, n);
}
PlanGrid plan_grid_x(int32_t E, int32_t ntiles) {
  if (plant != "scan-ew") return plan_grid(E, ntiles);
  PlanGrid g;
  const int64_t ew = ntiles > 0 ? (16ll * kPlanThreads) / ntiles : E;
  g.scan_ew = static_cast<int32_t>(ew < 1 ? 1 : ew);
  g.scan_wgs = ntiles > 0 ? (E + g.scan_ew - 1) / g.scan_ew : 0;
  return g;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc < 8) {
    std::fprintf(stderr, "usage: %s E R S D L T k [plant]\n", argv[0]);
    return 2;
  }
  const int32_t E = std::atoi(argv[1]), R = std::atoi(argv[2]), S = std::atoi(argv[3]),
                D = std::atoi(argv[4]), L = std::atoi(argv[5]);
  const int64_t T = std::atoll(argv[6]);
  const int32_t k = std::atoi(argv[7]);
  if (argc > 8) plant = argv[8];

  ultraep_ctx* ctx = nullptr;
  if (ultraep_create(E, R, S, D, nullptr, &ctx) != ULTRAEP_OK) return 2;
  size_t ws_bytes = 0, plan_bytes = 0;
  if (ultraep_workspace_bytes(ctx, L, T, k, &ws_bytes) != ULTRAEP_OK) return 2;
  if (ultraep_plan_bytes(ctx, &plan_bytes) != ULTRAEP_OK) return 2;
  size_t off[ULTRAEP_PLAN_NUM_FIELDS], len[ULTRAEP_PLAN_NUM_FIELDS];
  for (int f = 0; f < ULTRAEP_PLAN_NUM_FIELDS; ++f)
    if (ultraep_plan_field(ctx, f, &off[f], &len[f]) != ULTRAEP_OK) return 2;

  const int32_t M = E / R, P = R * (M + S), ndom = R / D, n_inst = E + R * S;
  const int32_t TK = static_cast<int32_t>(T * k), N = R * TK;
  const int32_t tpr = static_cast<int32_t>(tiles_per_rank(TK));
  const int32_t ntiles = static_cast<int32_t>(ntiles_of(R, TK));
  const int32_t hs = hist_stride(E);
  const int64_t pairs = static_cast<int64_t>(L) * N;
  // the workspace: 16-bit histograms in the first half, int32 tile bases in
  // the second (as launch_balance splits it)
  const int64_t ws_words = static_cast<int64_t>(ws_bytes / 4);
  const int64_t hist_entries = 2 * (static_cast<int64_t>(L) * ntiles * E);  // uint16 entries of the first half
  const int64_t tbase_at = static_cast<int64_t>(L) * ntiles * E;            // int32 word where the bases start
  if (2 * tbase_at > ws_words) fail("workspace halves", 2 * tbase_at, ws_words);
  const int64_t rec_words = static_cast<int64_t>(plan_bytes / 4);

  // ---- count: one workgroup per (layer, tile) ----
  for (int64_t blk = 0; blk < static_cast<int64_t>(L) * ntiles; ++blk) {
    const int32_t layer = static_cast<int32_t>(blk / ntiles), tile = static_cast<int32_t>(blk % ntiles);
    const TileSpan sp = tile_span(layer, tile, N, TK, tpr);
    if (sp.n < 1 || sp.n > kTile) fail("count tile size", blk, sp.n);
    if (sp.first < 0 || sp.first + sp.n > pairs) fail("count ids", blk, sp.first, sp.n);
    if (sp.first != static_cast<int64_t>(layer) * N + sp.tile0) fail("tile start", blk, sp.first);
    const int64_t row = static_cast<int64_t>(layer) * ntiles + tile;
    if ((row + 1) * hs > hist_entries) fail("count histogram row", blk, row);
  }
  // the tiles of a layer cover its pairs exactly once, rank by rank
  {
    std::vector<unsigned char> seen(static_cast<size_t>(N), 0);
    for (int32_t tile = 0; tile < ntiles; ++tile) {
      const TileSpan sp = tile_span(0, tile, N, TK, tpr);
      if (sp.tile0 / (TK > 0 ? TK : 1) != tile / tpr) fail("tile straddles ranks", tile, sp.tile0);
      for (int32_t i = 0; i < sp.n; ++i) seen[static_cast<size_t>(sp.tile0 + i)]++;
    }
    for (int32_t n = 0; n < N; ++n)
      if (seen[static_cast<size_t>(n)] != 1) {
        fail("pair not covered once by the tiles", n, seen[static_cast<size_t>(n)]);
        break;
      }
  }

  // ---- plan launch: per layer 1 planner + scan_wgs tile-base workgroups ----
  const PlanGrid g = plan_grid_x(E, ntiles);
  const PlanRounds pr = plan_rounds_of(ndom);
  const PlanTables tb = plan_tables(E, R, S, D, P, ndom, pr.items);
  const int64_t lds_words = tb.off[kT_end];
  if (4 * lds_words > 160 * 1024) fail("planner LDS beyond 160 KiB", lds_words, 0);
  if (lds_words < kPlanThreads) fail("tile-base partials beyond the LDS allocation", lds_words, 0);
  if (tb.off[kT_rmask] % 2 != 0) fail("64-bit rank masks misaligned", tb.off[kT_rmask], 0);
  for (int i = 0; i < kT_end; ++i)
    if (tb.off[i + 1] < tb.off[i]) fail("LDS tables out of order", i, tb.off[i]);
  if (ntiles > 0) {
    if (g.scan_ew < 1 || g.scan_ew > E || g.scan_ew > kPlanThreads)
      fail("experts per tile-base workgroup", g.scan_ew, E);
    if (static_cast<int64_t>(g.scan_wgs) * g.scan_ew < E) fail("tile-base workgroups cover E", g.scan_wgs, g.scan_ew);
  }
  const bool scan_ok = ntiles == 0 || (g.scan_ew >= 1 && g.scan_ew <= kPlanThreads);
  const uint32_t grid = static_cast<uint32_t>(L) * static_cast<uint32_t>(1 + g.scan_wgs);
  // layer 0's coverage: tile bases written, histogram entries summed
  std::vector<int32_t> written(static_cast<size_t>(ntiles) * E, 0);
  std::vector<int32_t> read_cols(static_cast<size_t>(ntiles) * E, 0);
  for (uint32_t blk = 0; blk < grid; ++blk) {
    const PlanRole role = plan_role(blk, g.scan_wgs);
    if (role.layer < 0 || role.layer >= L) fail("plan layer", blk, role.layer);
    const int64_t hbase = static_cast<int64_t>(role.layer) * ntiles * hs;  // uint16 entries
    const int64_t bbase = tbase_at + static_cast<int64_t>(role.layer) * ntiles * E;
    if (role.role > 0) {
      if (!scan_ok) continue;
      for (int tid = 0; tid < kPlanThreads; ++tid) {
        const ScanThread th = scan_thread(tid, role.role, g.scan_ew, ntiles, E);
        if (!th.act) continue;
        if (th.e < 0 || th.e >= E) fail("tile-base expert", blk, tid, th.e);
        for (int q = 0; q < th.ch; ++q)
          if (q * g.scan_ew + th.el >= kPlanThreads) fail("tile-base partial", blk, tid, q);
        for (int pass = 0; pass < 2; ++pass)
          for (int32_t t = th.t0; t < th.t1; t += kScanBatch)
            for (int u = 0; u < kScanBatch; ++u) {
              const int32_t row = scan_row_x(t, u, ntiles);
              if (row < 0 || row >= ntiles) {
                fail("tile-base histogram row", blk, tid, row);
                continue;
              }
              const int64_t at = hbase + static_cast<int64_t>(row) * hs + th.e;
              if (at < 0 || at >= hist_entries) fail("tile-base histogram entry", blk, tid, at);
              if (pass == 1 && t + u < th.t1) {
                const int64_t w = bbase + static_cast<int64_t>(t + u) * E + th.e;
                if (w < tbase_at || w >= ws_words) fail("tile base write", blk, tid, w);
                if (role.layer == 0) written[static_cast<size_t>(t + u) * E + th.e]++;
              }
            }
      }
      continue;
    }
    // the planner: the histogram sum (16-byte form when the layer's rows
    // allow it on a 256-byte aligned workspace)
    const bool vec = sum_vector_form(hs, static_cast<uintptr_t>(2 * hbase));
    const int W = vec ? 4 : 1;
    const int B = vec ? sum_batch(hs, ntiles) : 32;
    for (int tid = 0; tid < kPlanThreads; ++tid) {
      const SumThread th = sum_thread(tid, hs, W, ntiles);
      if (!th.act) continue;
      if ((th.q + 1) * 2 * W > hs) fail("histogram sum column", blk, tid, th.q);
      for (int32_t t = th.ch; t < ntiles; t += B * th.nch)
        for (int u = 0; u < B; ++u) {
          const int32_t row = sum_row_x(t, u, th.nch, ntiles);
          if (row < 0 || row >= ntiles) {
            fail("histogram sum row", blk, tid, row);
            continue;
          }
          const int64_t at = hbase + static_cast<int64_t>(row) * hs + 2 * W * th.q;
          if (at < 0 || at + 2 * W > hist_entries) fail("histogram sum entry", blk, tid, at);
          if (role.layer == 0 && t + u * th.nch < ntiles)
            for (int i = 0; i < 2 * W; ++i)
              if (2 * W * th.q + i < E) read_cols[static_cast<size_t>(row) * E + 2 * W * th.q + i]++;
        }
    }
    if (role.layer == 0)
      for (size_t i = 0; i < read_cols.size(); ++i)
        if (read_cols[i] != 1) {
          fail("histogram entry not summed once", static_cast<long long>(i), read_cols[i]);
          break;
        }
    // the local takes: column e of rank r's tile rows, for every instance
    for (int32_t r = 0; r < R; ++r) {
      const int32_t t1 = (r + 1) * tpr;
      for (int32_t t0 = r * tpr; t0 < t1; t0 += kLocalBatch)
        for (int u = 0; u < kLocalBatch; ++u) {
          const int32_t row = local_row(t0, u, t1);
          if (row < r * tpr || row >= t1 || row >= ntiles) fail("local take row", r, row);
          if (hbase + static_cast<int64_t>(row + 1) * hs > hist_entries) fail("local take entry", r, row);
        }
    }
    // the early first batch of the local takes: thread tid loads rank
    // tid / S's rows for slot tid and rank tid / M's for master tid (any
    // expert column: the experts are not known yet)
    if (local_prefetch_x(tpr))
      for (int tid = 0; tid < kPlanThreads; ++tid)
        for (int which = 0; which < 2; ++which) {
          if (which == 0 ? (tid >= R * S) : (tid >= E)) continue;
          const int32_t r = which == 0 ? tid / S : tid / (E / R);
          for (int u = 0; u < kLocalBatch; ++u) {
            const int32_t row = local_row(r * tpr, u, (r + 1) * tpr);
            if (row < r * tpr || row >= (r + 1) * tpr || row < 0 || row >= ntiles)
              fail("local take first batch row", tid, r, row);
            else if (hbase + static_cast<int64_t>(row + 1) * hs > hist_entries)
              fail("local take first batch entry", tid, r, row);
          }
        }
    // the plan record: every field the planner writes, at the extents its
    // loops use, inside the record of its layer
    const int64_t want[ULTRAEP_PLAN_NUM_FIELDS] = {ULTRAEP_HDR_WORDS, E, E, R * S, R * S, P, P + 1,
                                                   E + 1, n_inst, n_inst, n_inst, R, R, n_inst};
    for (int f = 0; f < ULTRAEP_PLAN_NUM_FIELDS; ++f) {
      if (static_cast<int64_t>(len[f]) != want[f]) fail("plan field length", f, len[f], want[f]);
      if (off[f] % 16 != 0) fail("plan field alignment", f, off[f]);
      if (static_cast<int64_t>(off[f] / 4 + len[f]) > rec_words) fail("plan field end", f, off[f], len[f]);
      if (f + 1 < ULTRAEP_PLAN_NUM_FIELDS && off[f] / 4 + len[f] > off[f + 1] / 4) fail("plan fields overlap", f, 0);
    }
  }
  if (ntiles > 0 && scan_ok)
    for (size_t i = 0; i < written.size(); ++i)
      if (written[i] != 1) {
        fail("tile base not written once", static_cast<long long>(i), written[i]);
        break;
      }

  // ---- reroute: one workgroup per (layer, tile), as count, in the XCD
  // order: every (layer, tile) taken by exactly one workgroup ----
  const int64_t nrb = static_cast<int64_t>(L) * ntiles;
  std::vector<int> taken(static_cast<size_t>(nrb), 0);
  for (int64_t g = 0; g < nrb; ++g) {
    const int64_t blk = xcd_block_x(g, nrb);
    if (blk < 0 || blk >= nrb) {
      fail("reroute block order", g, blk);
      continue;
    }
    ++taken[static_cast<size_t>(blk)];
    const int32_t layer = static_cast<int32_t>(blk / ntiles), tile = static_cast<int32_t>(blk % ntiles);
    const TileSpan sp = tile_span(layer, tile, N, TK, tpr);
    if (sp.first + sp.n > pairs) fail("reroute pairs", blk, sp.first);
    const int64_t b = tbase_at + (static_cast<int64_t>(layer) * ntiles + tile) * E;
    if (b < tbase_at || b + E > ws_words) fail("reroute tile bases", blk, b);
  }
  for (int64_t i = 0; i < nrb; ++i)
    if (taken[static_cast<size_t>(i)] != 1) {
      fail("reroute tile not taken once", i, taken[static_cast<size_t>(i)]);
      break;
    }

  ultraep_destroy(ctx);
  if (fails) {
    std::fprintf(stderr, "%ld violations\n", fails);
    return 1;
  }
  std::printf("ok E=%d R=%d S=%d D=%d L=%d T=%lld k=%d: %u plan workgroups, %d tiles per layer\n", E,
              R, S, D, L, static_cast<long long>(T), k, grid, ntiles);
  return 0;
}

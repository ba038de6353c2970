// Index arithmetic of the balance launches' global-memory and LDS accesses:
// where each workgroup's tile of pairs lies, how the plan launch splits into
// one planner and several tile-base workgroups per layer, which histogram
// rows and expert columns each of their threads reads, and where each LDS
// table of the planner starts.  The kernels and a host-side bounds check
// (tests/geometry_check.cpp, which walks every workgroup and thread of a
// launch) call the same functions, so the check cannot drift from the
// kernels.  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ultraep {

// Pairs handled by one count / reroute workgroup.
constexpr int kTile = 8192;
// The plan solver runs in one workgroup of 16 waves per layer; the tile-base
// workgroups of the same launch have the same size.
constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;

// Tiles never straddle two ranks: each rank's TK = T*k pairs split into
// ceil(TK / kTile) tiles, the last one ragged, so a tile's pairs all come
// from one rank's tokens.
__host__ __device__ inline int64_t tiles_per_rank(int64_t TK) { return (TK + kTile - 1) / kTile; }
__host__ __device__ inline int64_t ntiles_of(int64_t R, int64_t TK) { return R * tiles_per_rank(TK); }

// Entries per tile histogram row (16-bit counts, rows of an even length so
// the planner can read two experts per 32-bit word).
__host__ __device__ inline int32_t hist_stride(int32_t E) { return (E + 1) & ~1; }

// Where tile `tile` of a layer lies: tiles are numbered rank by rank, TK
// pairs per rank in tiles of kTile (the last one of a rank ragged).
struct TileSpan {
  int64_t first;  // index of the first pair in the [L][N] arrays
  int32_t tile0;  // index of the first pair inside the layer
  int32_t n;      // pairs in the tile
};

__host__ __device__ inline TileSpan tile_span(int64_t layer, int32_t tile, int32_t N, int32_t TK,
                                              int32_t tpr) {
  const int32_t r = tile / tpr, q = tile % tpr;
  const int32_t tile0 = r * TK + q * kTile;
  const int32_t rest = TK - q * kTile;
  return {layer * N + tile0, tile0, rest < kTile ? rest : kTile};
}

// Workgroups of one launch are handed to the 8 XCDs in turn (workgroup g to
// XCD g % 8), and each XCD has its own L2.  The reroute kernels take their
// (layer, tile) from xcd_block, which gives the workgroups of one XCD
// consecutive tiles: neighbouring tiles write the two ends of the same
// layout runs, so the lines they share meet in one L2 instead of going to
// HBM twice as partial lines.  A bijection on [0, n): the first 8*(n/8)
// blocks are regrouped, the n % 8 last ones keep their index.
constexpr int kXcds = 8;

__host__ __device__ inline int64_t xcd_block(int64_t g, int64_t n) {
  const int64_t per = n / kXcds;
  if (g >= per * kXcds) return g;
  return (g % kXcds) * per + g / kXcds;
}

// ---- the plan launch -------------------------------------------------------
// Per layer, one planner workgroup (role 0) and scan_wgs tile-base workgroups
// (roles 1..scan_wgs), each of the latter covering scan_ew experts: enough
// workgroups that each thread's run of tiles is about one batch of loads, at
// most one per expert (so scan_ew never exceeds E).
struct PlanGrid {
  int32_t scan_ew;
  int32_t scan_wgs;
};

__host__ __device__ inline PlanGrid plan_grid(int32_t E, int32_t ntiles) {
  const int64_t ew = ntiles > 0 ? (16ll * kPlanThreads) / ntiles : E;
  PlanGrid g;
  g.scan_ew = static_cast<int32_t>(ew < 1 ? 1 : (ew > E ? E : ew));
  g.scan_wgs = ntiles > 0 ? (E + g.scan_ew - 1) / g.scan_ew : 0;
  return g;
}

struct PlanRole {
  int32_t layer;
  int32_t role;  // 0: planner; r > 0: tile bases of experts [(r-1)*scan_ew, r*scan_ew)
};

__host__ __device__ inline PlanRole plan_role(uint32_t block, int32_t scan_wgs) {
  const int32_t group = 1 + scan_wgs;
  return {static_cast<int32_t>(block / group), static_cast<int32_t>(block % group)};
}

// Thread tid of a tile-base workgroup: expert e (column el of the group),
// tile chunk ch of nch, and its run of tiles [t0, t1).
struct ScanThread {
  int32_t e, el, ch, t0, t1;
  bool act;
};

__host__ __device__ inline ScanThread scan_thread(int tid, int32_t role, int32_t ew, int32_t ntiles,
                                                  int32_t E) {
  ScanThread s;
  const int nch = kPlanThreads / ew;
  s.el = tid % ew;
  s.ch = tid / ew;
  s.e = (role - 1) * ew + s.el;
  s.act = s.ch < nch && s.e < E && ntiles > 0;
  const int clen = (ntiles + nch - 1) / nch;
  const int a = s.ch * clen;
  s.t0 = a < ntiles ? a : ntiles;
  s.t1 = s.t0 + clen < ntiles ? s.t0 + clen : ntiles;
  return s;
}

// Loads of the tile-base scan go in batches of kScanBatch rows; a batch's
// rows past the run repeat the last tile (they are masked afterwards).
constexpr int kScanBatch = 16;
__host__ __device__ inline int32_t scan_row(int32_t tb, int u, int32_t ntiles) {
  return tb + u < ntiles - 1 ? tb + u : ntiles - 1;
}

// Thread tid of the planner's histogram sum reads W 32-bit words (2W
// experts) at word column q of the rows ch, ch + nch, ... (nq = hs / 2W
// word columns per row).
struct SumThread {
  int32_t q, ch, nch;
  bool act;
};

__host__ __device__ inline SumThread sum_thread(int tid, int32_t hs, int W, int32_t ntiles) {
  SumThread s;
  const int nq = hs / (2 * W);
  s.nch = kPlanThreads / nq;
  s.q = tid % nq;
  s.ch = tid / nq;
  s.act = s.ch < s.nch && ntiles > 0;
  return s;
}

// Row of load u of the batch starting at row tb (rows past the last repeat it).
__host__ __device__ inline int32_t sum_row(int32_t tb, int u, int32_t nch, int32_t ntiles) {
  const int32_t row = tb + u * nch;
  return row < ntiles - 1 ? row : ntiles - 1;
}

// The histogram sum's 16-byte form (W = 4) needs rows of a multiple of 8
// entries on a 16-byte aligned base; its batch size follows from the rows a
// thread reads.
__host__ __device__ inline bool sum_vector_form(int32_t hs, uintptr_t base) {
  return hs % 8 == 0 && (base & 15) == 0;
}
__host__ __device__ inline int sum_batch(int32_t hs, int32_t ntiles) {
  const int per = kPlanThreads / (hs / 8);
  const int rows = (ntiles + per - 1) / per;
  return rows <= 4 ? 4 : rows <= 8 ? 8 : 16;
}

// Rows of rank r's tiles (the local takes read column e of each), loaded
// kLocalBatch at a time; rows past the rank's last repeat it.
constexpr int kLocalBatch = 8;
__host__ __device__ inline int32_t local_row(int32_t t0, int u, int32_t t1) {
  return t0 + u < t1 - 1 ? t0 + u : t1 - 1;
}

// The planner loads the first batch of every local take early: thread tid
// for slot tid (rank tid / S) and for master tid (rank tid / M), before it
// knows which experts those instances hold.  A rank without tiles (a layer
// of no tokens) has no rows, and then nothing is loaded.
__host__ __device__ inline bool local_prefetch(int32_t tpr) { return tpr > 0; }

// Grid quotas per probe round: enough (quota, domain) items for one probe
// wave per SIMD.  More probe waves than SIMDs only share issue slots: the
// probes of a round run in lock step, and the first one usually succeeds.
struct PlanRounds {
  int32_t G;      // grid quotas per round
  int32_t items;  // (quota, domain) probes per round
};

__host__ __device__ inline PlanRounds plan_rounds_of(int32_t ndom) {
  constexpr int kSimds = 4;
  const int32_t G = ndom < kSimds ? kSimds / ndom : 1;
  return {G, G * ndom};
}

// ---- the planner's LDS tables ---------------------------------------------
// Word offsets of the planner's tables inside its dynamic LDS allocation
// (16-byte aligned), in carving order.  The 64-bit rank masks come first so
// they are naturally aligned for 64-bit LDS atomics.  The tile-base
// workgroups use only the first kPlanThreads words.
enum PlanTable {
  kT_rmask = 0,  // [E] 64-bit: domain ranks holding a replica of e
  kT_c,          // [E] pairs per expert
  kT_H,          // [R] home loads
  kT_part,       // [kPlanThreads] unused by the planner: it keeps the allocation large
                 // enough for the tile-base workgroups' partials (its first kPlanThreads words)
  kT_dom,        // [ndom] domain loads
  kT_scal,       // [kPlanScalars]
  kT_ok,         // [items] probe outcomes
  kT_res,        // [2][items][D*S] hosted expert, then its quota
  kT_mq,         // [E] master quotas
  kT_iptr,       // [E+1]
  kT_pload,      // [P+1]
  kT_slotE,      // [R*S]
  kT_slotQ,      // [R*S]
  kT_instp,      // [E+R*S]
  kT_iq,         // [E+R*S+1]
  kT_iex,        // [E+R*S]
  kT_end,
};
constexpr int kPlanScalars = 16;

struct PlanTables {
  int64_t off[kT_end + 1];  // word offset of each table; off[kT_end] = words in all
};

__host__ __device__ inline PlanTables plan_tables(int E, int R, int S, int D, int P, int ndom,
                                                  int items) {
  const int64_t ni = static_cast<int64_t>(E) + static_cast<int64_t>(R) * S;
  const int64_t len[kT_end] = {2ll * E, E, R, kPlanThreads, ndom, kPlanScalars, items,
                               2ll * items * D * S, E, E + 1ll, P + 1ll, static_cast<int64_t>(R) * S,
                               static_cast<int64_t>(R) * S, ni, ni + 1, ni};
  PlanTables t;
  int64_t at = 0;
  for (int i = 0; i < kT_end; ++i) {
    t.off[i] = at;
    at += len[i];
  }
  t.off[kT_end] = at;
  return t;
}

}  // namespace ultraep

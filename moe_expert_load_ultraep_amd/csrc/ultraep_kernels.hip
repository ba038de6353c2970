// gfx950 (CDNA4) kernels of the exact-load expert rebalancing path.
//
// Sources, cited by page title and section:
//   [README] "UltraEP" project README (mirror kd.iw.mk/studio-dots-ai/UltraEP)
//   [NEWS]   "Xiaohongshu's UltraEP Balances MoE Experts in 300 µs, Reaching
//            94.3% of Ideal" (news.hamidun.com)
//
// Nothing here is a dense contraction, so no MFMA: the count, reroute,
// layout, permute and fold kernels are HBM-streaming kernels built around
// wave64 ballots, LDS-privatised counters and 16-byte vector accesses, and
// the plan solver is a latency-bound single-workgroup kernel that keeps all
// of its state in LDS and registers.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ultraep_device.h"
#include "ultraep_internal.h"

namespace ultraep {
namespace {

// Lanes of the wave holding the same value v: every lane ORs its lane bit
// into an LDS word owned by its value, then reads the word back.  Each half
// of the wave ORs into its own 32-bit half of the 64-bit word (half the
// bytes of a 64-bit OR, and equal values of the two halves do not collide);
// the word read back holds lanes 0-31 in its low half.  LDS operations of
// one wave complete in program order, so the read sees all of this
// instruction's ORs; the caller clears the word (one lane per group) before
// the next use.  Every lane must be active.
__device__ __forceinline__ uint64_t match_peers_lds(unsigned long long* words, uint32_t v,
                                                    int lane) {
  atomicOr(reinterpret_cast<uint32_t*>(words) + 2 * v + (lane >> 5), 1u << (lane & 31));
  return __atomic_load_n(&words[v], __ATOMIC_RELAXED);
}

// A tile of kTile pairs worked on by W waves: wave q owns the stretch of
// kWavePairs pairs from q * kWavePairs, in kChunks chunks of 64.
template <int W>
struct TileShape {
  static constexpr int kWaves = W;
  static constexpr int kThreads = 64 * W;
  static constexpr int kWavePairs = kTile / W;
  static constexpr int kChunks = kWavePairs / 64;
  static_assert(kChunks * 64 * W == kTile, "tile must split into whole chunks");
};

// The tiling of one launch: N = R*TK pairs per layer, tpr tiles per rank,
// ntiles = R*tpr tiles per layer.
struct Tiling {
  int32_t N, TK, tpr, ntiles;
};

// Expert ids of one wave's stretch of a tile: chunk c, lane l holds pair
// base + 64c + l.  Every load is issued unconditionally through one buffer
// resource over the tile (one offset register for all chunks; loads past the
// tile read 0 and are masked afterwards), so all C loads are in flight
// together instead of one round trip per chunk.  Ids outside [0, E) and
// padding become E.
template <int C>
__device__ __forceinline__ void load_tile_ids(const int32_t* __restrict__ src, int base,
                                              int n_here, int lane, int32_t E,
                                              uint32_t (&v)[C]) {
  const __amdgpu_buffer_rsrc_t r = row_rsrc(src, static_cast<uint32_t>(n_here) * 4u);
  uint32_t raw[C];
#pragma unroll
  for (int c = 0; c < C; ++c)
    raw[c] = __builtin_amdgcn_raw_buffer_load_b32(r, (base + c * 64 + lane) * 4, 0, kNonTemporal);
#pragma unroll
  for (int c = 0; c < C; ++c)
    v[c] = (base + c * 64 + lane < n_here && raw[c] < static_cast<uint32_t>(E)) ? raw[c]
                                                                                 : static_cast<uint32_t>(E);
}

// Exclusive scan of a[0, n) by the calling wave alone (a[n] receives the
// total): each lane sums a contiguous run, the lanes scan their sums, and
// each lane writes its run's prefixes.  For the short arrays of a tile's
// runs and the planner's offsets one wave is enough, where a scan across the
// workgroup would need two more barriers.  The caller synchronises
// afterwards.  With COUNT, each
// value x (a run length below 2^16) is taken as x + 2^16 [x > 0], so the
// prefixes hold the offset in the low half and the non-empty runs before
// in the high half.
template <bool COUNT = false>
__device__ void wave_exclusive_scan(int32_t* a, int n) {
  const int lane = lane_id();
  const int per = (n + 63) / 64;
  const int b = min(lane * per, n), en = min(b + per, n);
  auto val = [](int32_t x) { return COUNT ? x + (x > 0 ? 1 << 16 : 0) : x; };
  int32_t s = 0;
  for (int i = b; i < en; ++i) s += val(a[i]);
  const int32_t inc = wave_inclusive_scan(s);
  int32_t run = inc - s;
  for (int i = b; i < en; ++i) {
    const int32_t v = val(a[i]);
    a[i] = run;
    run += v;
  }
  if (lane == 63) a[n] = inc;
}

// ------------------------------------------------------------------------
// count: per-tile expert histogram ([README] intro: exact post-gating load)
// ------------------------------------------------------------------------
// One workgroup of 16 waves per (layer, tile of kTile pairs).  Each wave
// loads its 512-pair stretch with all loads in flight at once and adds each
// valid id to an LDS counter.  The order of the additions does not matter
// here, so a plain LDS atomic per pair is the cheapest form: equal ids in one
// wave instruction only serialise inside the LDS, they cost no VALU work.
// Lanes 8q..8q+7 add into copy q of the counters (kCountCopies copies, rows
// of E + 1 words so the copies of one expert fall in different banks): with
// top-8 routing those lanes hold one token's 8 distinct experts, so a hot
// expert's atomics in one instruction hit 8 different words instead of one.
// The copies are summed when the row is written.
// A tile holds at most kTile pairs, so its counts are stored as 16-bit
// values, rows of hist_stride(E) entries: the planner reads every row, and
// half the bytes is half its wait.
using CountTile = TileShape<16>;
constexpr int kCountCopies = 8;

__global__ __launch_bounds__(CountTile::kThreads) void count_kernel(
    const int32_t* __restrict__ idx, int32_t N, int32_t TK, int32_t tpr, int32_t E, int32_t ntiles,
    uint16_t* __restrict__ hist) {
  using T = CountTile;
  extern __shared__ __align__(16) int32_t s_cnt[];
  const int64_t blk = blockIdx.x;
  const int32_t layer = static_cast<int32_t>(blk / ntiles);
  const int32_t tile = static_cast<int32_t>(blk % ntiles);
  for (int i = threadIdx.x; i < kCountCopies * (E + 1); i += T::kThreads) s_cnt[i] = 0;
  const TileSpan sp = tile_span(layer, tile, N, TK, tpr);
  const int32_t* src = idx + sp.first;
  const int n_here = sp.n;
  uint32_t v[T::kChunks];
  load_tile_ids(src, (threadIdx.x >> 6) * T::kWavePairs, n_here, lane_id(), E, v);
  __syncthreads();
  int32_t* mine = s_cnt + (lane_id() / (64 / kCountCopies)) * (E + 1);
#pragma unroll
  for (int c = 0; c < T::kChunks; ++c)
    if (v[c] < static_cast<uint32_t>(E)) atomicAdd(&mine[v[c]], 1);
  __syncthreads();
  uint16_t* dst = hist + (static_cast<int64_t>(layer) * ntiles + tile) * hist_stride(E);
  for (int i = threadIdx.x; i < hist_stride(E); i += T::kThreads) {
    int32_t n = 0;
    if (i < E)
#pragma unroll
      for (int q = 0; q < kCountCopies; ++q) n += s_cnt[q * (E + 1) + i];
    dst[i] = static_cast<uint16_t>(n);
  }
}

// ------------------------------------------------------------------------
// plan: quota solver, one workgroup per layer
// ------------------------------------------------------------------------
struct PlanParams {
  int32_t E, R, S, D, M, P, ndom, n_inst;
  int32_t N, ntiles, tpr;
  int32_t eps_num, eps_den, allow_zero;
  int32_t thr_num, thr_den;
  int32_t min_tokens;
  int32_t lean;
  int32_t rec_words;
  int32_t G, items;  // grid quotas per probe round, (quota, domain) items per round
  int32_t scan_wgs;  // workgroups per layer that build the tile ordinal bases
  int32_t scan_ew;   // experts per scan workgroup
  int32_t off[ULTRAEP_PLAN_NUM_FIELDS];
  int32_t len[ULTRAEP_PLAN_NUM_FIELDS];
};

enum Scalar {
  kTotal = 0, kQmax, kFloor, kQlb, kTol, kK, kWin, kReplicas, kCmax, kScalars = kPlanScalars
};

struct PlanLds {
  int32_t* c;      // [E]
  int32_t* H;      // [R]
  int32_t* dom;    // [ndom]
  int32_t* scal;   // [kScalars]
  int32_t* ok;     // [items]
  int32_t* res;    // [2][items][D*S]  hosted expert, then its quota
  int32_t* mq;     // [E]
  unsigned long long* rmask;  // [E] domain ranks (bit r % D) holding a replica of e
  int32_t* iptr;   // [E+1]
  int32_t* pload;  // [P+1]
  int32_t* slotE;  // [R*S]
  int32_t* slotQ;  // [R*S]
  int32_t* instp;  // [E+R*S] physical expert of each instance entry
  int32_t* iq;     // [E+R*S+1] its quota, then the exclusive prefix of the quotas
  int32_t* iex;    // [E+R*S] its expert
};

__host__ __device__ inline size_t plan_lds_words(int E, int R, int S, int D, int P, int ndom,
                                                 int items) {
  return static_cast<size_t>(plan_tables(E, R, S, D, P, ndom, items).off[kT_end]);
}

__device__ inline PlanLds carve(int32_t* lds, const PlanParams& a) {
  const PlanTables t = plan_tables(a.E, a.R, a.S, a.D, a.P, a.ndom, a.items);
  PlanLds L;
  L.rmask = reinterpret_cast<unsigned long long*>(lds + t.off[kT_rmask]);
  L.c = lds + t.off[kT_c];
  L.H = lds + t.off[kT_H];
  L.dom = lds + t.off[kT_dom];
  L.scal = lds + t.off[kT_scal];
  L.ok = lds + t.off[kT_ok];
  L.res = lds + t.off[kT_res];
  L.mq = lds + t.off[kT_mq];
  L.iptr = lds + t.off[kT_iptr];
  L.pload = lds + t.off[kT_pload];
  L.slotE = lds + t.off[kT_slotE];
  L.slotQ = lds + t.off[kT_slotQ];
  L.instp = lds + t.off[kT_instp];
  L.iq = lds + t.off[kT_iq];
  L.iex = lds + t.off[kT_iex];
  return L;
}

// One feasibility probe: can domain d be brought to at most Q with the
// greedy placement?  Runs on one wave; lane l plays rank d*D + l and holds
// that rank's M queued pieces and S hosted replicas in registers.  On success
// the hosted (expert, quota) lists go to res_e / res_q ([D][S]).
//
// The pages describe a quota-driven scheduler that replicates hot experts to
// idle ranks and merges cold ones ([NEWS] "How balancing in 300 microseconds
// works"; [README] "Replication planning": a master may be required to keep
// part of its load) without giving its steps; this build's greedy:
//  shed    a rank above Q gives up its excess from its hottest experts first
//          (pairs desc, id asc), each master keeping one pair unless zero
//          master quota is allowed;
//  pop     the largest queued piece (ties: lowest expert id);
//  fit     the receiver with the least spare that still takes it whole
//          (ties: lowest rank);
//  chain   else, if a shedding rank could host it, the roomiest receiver is
//          filled and the rest goes to the rank of the largest such queued
//          piece, which sheds that much more of its own expert;
//  fill    else the roomiest receiver (most spare, ties: lowest rank) is
//          filled and the rest queued;
//  fail    else.
// Each step fills a slot, so at most D*S steps run.
//
// Two implementations of the same greedy follow.  greedy_probe_packed folds
// each selection's value and its tie-break (lane, queue index) into one
// 32-bit key, so a pick is one wave reduction; it needs every piece below
// 2^(26 - log2 MMAX) pairs and Q below 2^25.  greedy_probe makes the same
// picks with a value reduction followed by a ballot for the lowest tied
// lane, for any size.

// shed: the pieces rank r (lane) queues at quota Q and the room left on each
// of its experts; false when some rank of the domain cannot shed enough.
template <int MMAX>
__device__ bool shed_pieces(int32_t Q, bool act, int r, int32_t Hr, const PlanParams& a,
                            const PlanLds& L, int32_t (&pa)[MMAX], int32_t (&room)[MMAX]) {
  const int M = a.M;
  const int32_t mt = a.min_tokens;
#pragma unroll
  for (int j = 0; j < MMAX; ++j) {
    pa[j] = 0;
    room[j] = 0;
  }
  bool fail = false;
  if (act && Hr > Q) {
    int32_t ce[MMAX];
#pragma unroll
    for (int j = 0; j < MMAX; ++j) ce[j] = j < M ? L.c[r * M + j] : 0;
    int32_t X = Hr - Q;
    uint32_t used = 0;
    for (int step = 0; step < M; ++step) {
      int bj = 0;
      int32_t bc = -1;
#pragma unroll
      for (int j = 0; j < MMAX; ++j)
        if (j < M && !((used >> j) & 1u) && ce[j] > bc) {
          bc = ce[j];
          bj = j;
        }
      used |= 1u << bj;
      const int32_t keep = (bc > 0 && !a.allow_zero) ? 1 : 0;
      const int32_t avail = bc - keep;
      int32_t t = min(X, avail);
      // a piece is never below the minimum: raised to it when the expert
      // has room (the rank then ends below Q), else not shed
      if (t < mt) t = (X > 0 && avail >= mt) ? mt : 0;
      if (t > 0) {
#pragma unroll
        for (int j = 0; j < MMAX; ++j)
          if (j == bj) {
            pa[j] = t;
            room[j] = avail - t;
          }
        X -= t;
      }
    }
    fail = X > 0;
  }
  return ballot(fail) == 0;
}

template <int MMAX, int SMAX>
__device__ bool greedy_probe(int32_t Q, int d, const PlanParams& a, const PlanLds& L,
                             int32_t* res_e, int32_t* res_q) {
  const int lane = lane_id();
  const int D = a.D, M = a.M, S = a.S;
  const int32_t mt = a.min_tokens;
  const bool act = lane < D;
  const int r = d * D + lane;
  const int32_t Hr = act ? L.H[r] : 0;
  int32_t pa[MMAX], room[MMAX];
  if (!shed_pieces<MMAX>(Q, act, r, Hr, a, L, pa, room)) return false;

  int32_t spare = act ? max(0, Q - Hr) : 0;
  int32_t nh = act ? 0 : S;  // filled slots; inactive lanes look full
  int32_t he[SMAX], hq[SMAX];
#pragma unroll
  for (int s = 0; s < SMAX; ++s) {
    he[s] = -1;
    hq[s] = 0;
  }
  // place x pairs of expert e on the lane `who` (branch-free selects)
  auto place = [&](int who, int32_t e, int32_t x) {
    const bool me = lane == who;
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
      const bool here = me && s == nh;
      he[s] = here ? e : he[s];
      hq[s] = here ? x : hq[s];
    }
    nh += me ? 1 : 0;
  };

  const int max_steps = D * S + 1;
  for (int step = 0; step <= max_steps; ++step) {
    // pop the largest piece (ties: lowest expert id = lowest lane, lowest j)
    uint32_t mya = 0;
    int myj = 0;
#pragma unroll
    for (int j = 0; j < MMAX; ++j) {
      const bool bigger = static_cast<uint32_t>(pa[j]) > mya;
      mya = bigger ? static_cast<uint32_t>(pa[j]) : mya;
      myj = bigger ? j : myj;
    }
    const uint32_t amax = wave_max(mya);
    if (amax == 0) {
      if (act) {
#pragma unroll
        for (int s = 0; s < SMAX; ++s)
          if (s < S) {
            res_e[lane * S + s] = he[s];
            res_q[lane * S + s] = hq[s];
          }
      }
      return true;
    }
    const int owner = lowest_lane(ballot(mya == amax));
    const int jsel = static_cast<int>(readlane(static_cast<uint32_t>(myj), owner));
    const int32_t e = (d * D + owner) * M + jsel;
    int32_t amt = static_cast<int32_t>(amax);
#pragma unroll
    for (int j = 0; j < MMAX; ++j) pa[j] = (lane == owner && j == jsel) ? 0 : pa[j];
    bool hosts = false;
#pragma unroll
    for (int s = 0; s < SMAX; ++s) hosts |= (he[s] == e);
    const bool elig = lane != owner && nh < S && !hosts;

    // One key serves both receiver choices: a receiver that takes the whole
    // piece gets the top bit and the inverted spare (the largest key is the
    // tightest fit, ties to the lowest lane); otherwise the key is the spare
    // itself (the largest key is the roomiest receiver).
    // (a receiver needs a spare of at least the minimum; a whole piece is
    // never below it, so a fit always has that much)
    const uint32_t key = (elig && spare >= mt)
                             ? (spare >= amt ? (0x80000000u | (0x7FFFFFFFu - static_cast<uint32_t>(spare)))
                                             : static_cast<uint32_t>(spare))
                             : 0u;
    // donor: largest queued piece on an eligible rank with room for the
    // minimum more
    uint32_t dbest = 0;
    int dj = 0;
#pragma unroll
    for (int j = 0; j < MMAX; ++j) {
      const bool cand = !a.lean && elig && pa[j] > 0 && room[j] >= mt && static_cast<uint32_t>(pa[j]) > dbest;
      dbest = cand ? static_cast<uint32_t>(pa[j]) : dbest;
      dj = cand ? j : dj;
    }
    const uint32_t kmax = wave_max(key);
    const uint32_t dmax = wave_max(dbest);
    if (kmax & 0x80000000u) {  // fit
      const int rr = lowest_lane(ballot(key == kmax));
      spare -= lane == rr ? amt : 0;
      place(rr, e, amt);
      continue;
    }
    const uint32_t rmax = kmax;  // roomiest receiver's spare (0: none)
    // the roomiest receiver's part leaves at least the minimum queued and
    // is not placed below it
    int32_t part = min(static_cast<int32_t>(rmax), amt - mt);
    part = part < mt ? 0 : part;
    if (dmax > 0) {              // chain through the donor's rank
      const int dl = lowest_lane(ballot(dbest == dmax));
      const int djs = static_cast<int>(readlane(static_cast<uint32_t>(dj), dl));
      if (part > 0) {
        const int r2 = lowest_lane(ballot(key == rmax));
        place(r2, e, part);
        spare -= lane == r2 ? part : 0;
        amt -= part;
      }
      int32_t myroom = 0;
#pragma unroll
      for (int j = 0; j < MMAX; ++j) myroom = j == djs ? room[j] : myroom;
      const int32_t droom = static_cast<int32_t>(readlane(static_cast<uint32_t>(myroom), dl));
      int32_t x = min(amt, droom);
      if (amt - x > 0 && amt - x < mt) x = amt - mt;  // what stays queued is at least mt
      if (x < mt) return false;
      place(dl, e, x);
#pragma unroll
      for (int j = 0; j < MMAX; ++j) {
        const bool here = lane == dl && j == djs;
        pa[j] += here ? x : 0;
        room[j] -= here ? x : 0;
      }
      amt -= x;
    } else if (part > 0) {  // fill the roomiest receiver
      const int r2 = lowest_lane(ballot(key == rmax));
      place(r2, e, part);
      spare -= lane == r2 ? part : 0;
      amt -= part;
    } else {
      return false;
    }
    if (amt > 0) {
#pragma unroll
      for (int j = 0; j < MMAX; ++j) pa[j] = (lane == owner && j == jsel) ? amt : pa[j];
    }
  }
  return false;
}

constexpr int ilog2_c(int x) { return x <= 1 ? 0 : 1 + ilog2_c(x / 2); }

// MIN: a minimum above one pair per replica is in force.  Without it the
// step is compiled without the minimum's rules (each one is then a no-op),
// so the common case keeps the shortest dependent chain.  LEAN: no chain
// step (no queued piece serves as donor).
template <int MMAX, int SMAX, bool MIN, bool LEAN>
__device__ bool greedy_probe_packed(int32_t Q, int d, const PlanParams& a, const PlanLds& L,
                                    int32_t* res_e, int32_t* res_q) {
  // queue keys: pairs << TB | (TMASK - (lane * MMAX + j)); the largest key
  // is the largest piece, ties to the lowest expert id (lane, then j)
  constexpr int TB = 6 + ilog2_c(MMAX);
  constexpr uint32_t TMASK = (1u << TB) - 1;
  // receiver keys: (fit ? 2^25 | (2^25 - 1 - spare) : spare) << 6 | (63 - lane)
  constexpr uint32_t kFitBit = 1u << 25;
  const int lane = lane_id();
  const int D = a.D, M = a.M, S = a.S;
  const int32_t mt = MIN ? a.min_tokens : 1;
  const bool act = lane < D;
  const int r = d * D + lane;
  const int32_t Hr = act ? L.H[r] : 0;
  int32_t pa[MMAX], room[MMAX];
  if (!shed_pieces<MMAX>(Q, act, r, Hr, a, L, pa, room)) return false;

  const uint32_t tie0 = TMASK - static_cast<uint32_t>(lane * MMAX);
  // the pieces are kept as their queue keys (0: none), so a step's keys
  // need no packing
  uint32_t qk[MMAX];
#pragma unroll
  for (int j = 0; j < MMAX; ++j)
    qk[j] = pa[j] > 0 ? (static_cast<uint32_t>(pa[j]) << TB) | (tie0 - j) : 0u;
  int32_t spare = act ? max(0, Q - Hr) : 0;
  int32_t nh = act ? 0 : S;  // filled slots; inactive lanes look full
  // hosted replicas, newest first, each as the queue index (lane * MMAX + j
  // inside the domain) of its expert's master, which names the expert
  int32_t ht[SMAX], hq[SMAX];
#pragma unroll
  for (int s = 0; s < SMAX; ++s) {
    ht[s] = -1;
    hq[s] = 0;
  }
  const uint32_t rl = static_cast<uint32_t>(63 - lane);

  // One reduction stage per step: the receiver key, the donor key and the
  // queue's key after the pop are reduced together.  The next pop key is
  // then known without another reduction: a fit leaves the queue as the pop
  // left it; a chain grows the donor's piece (its key grows by the pairs
  // added, the tie bits stay) and may re-queue the rest of the popped piece
  // under its own tie bits; a fill re-queues the rest.  Keys are unique, so
  // the popped entry is the one whose key equals the pop key.
  //
  // The three outcomes share one update.  The receiver (lane kl) takes
  // r_amt pairs: the whole piece on a fit, else its whole spare (0 when no
  // rank has spare); the donor (lane dl, chains only) takes x more; the
  // rest goes back to the owner's queue entry.  Receiver and donor are
  // different ranks (a rank with spare queued nothing), so each lane places
  // at most one replica per step, and the step has no branch but the exit
  // and the rare failure.  A rank that queues a piece has no spare, so the
  // popped piece's own rank is never a receiver; it is kept out of the
  // donors explicitly.
  uint32_t mk = 0;
#pragma unroll
  for (int j = 0; j < MMAX; ++j) mk = max(mk, qk[j]);
  uint32_t km = wave_max_bcast(mk);
  int guard = D * S + 1;  // every step fills a slot
  while (km != 0) {
    if (--guard < 0) return false;
    const uint32_t own_tie = km & TMASK;
    const int32_t t = static_cast<int32_t>(TMASK - own_tie);
    const int32_t amt = static_cast<int32_t>(km >> TB);
    bool hosts = false;
#pragma unroll
    for (int s = 0; s < SMAX; ++s) hosts |= ht[s] == t;
    const bool elig = !hosts && nh < S;
    const uint32_t core = spare >= amt ? (kFitBit | (kFitBit - 1 - static_cast<uint32_t>(spare)))
                                       : static_cast<uint32_t>(spare);
    // receivers need a spare of at least the minimum (a whole piece is never
    // below it), donors room for the minimum more
    const uint32_t key = (elig && (MIN ? spare >= mt : spare > 0)) ? (core << 6) | rl : 0u;
    const bool delig = !LEAN && elig && lane != t / MMAX;
    uint32_t dk = 0, qn = 0;
    bool popped[MMAX];
#pragma unroll
    for (int j = 0; j < MMAX; ++j) {
      popped[j] = qk[j] == km;
      const uint32_t kj = popped[j] ? 0u : qk[j];
      qn = max(qn, kj);
      if constexpr (!LEAN) dk = max(dk, (delig && (MIN ? room[j] >= mt : room[j] > 0)) ? kj : 0u);
    }
    uint32_t kmax = key, dmax = dk, knext = qn;
    if constexpr (LEAN)
      wave_max2_bcast(kmax, knext);
    else
      wave_max3_bcast(kmax, dmax, knext);
    const bool fit = (kmax & (kFitBit << 6)) != 0;
    // the receiver's lane, none (64) when no rank has spare
    const int kl = kmax != 0 ? 63 - static_cast<int>(kmax & 63) : 64;
    int32_t r_amt, x = 0;
    int dl = 0, djs = 0;
    if constexpr (!LEAN) {
      const uint32_t dt = TMASK - (dmax & TMASK);
      dl = static_cast<int>(dt / MMAX) & 63;
      djs = static_cast<int>(dt % MMAX);
    }
    int32_t droom = 0;
    if constexpr (!LEAN) {
      int32_t myroom = room[0];
#pragma unroll
      for (int j = 1; j < MMAX; ++j) myroom = j == djs ? room[j] : myroom;
      droom = static_cast<int32_t>(readlane(static_cast<uint32_t>(myroom), dl));
    }
    if constexpr (MIN) {
      // without a fit the roomiest receiver takes its spare, but leaves at
      // least the minimum queued and takes nothing below it; the donor's
      // part is cut so that what stays queued is 0 or at least the minimum
      // (bitwise logic: short-circuit tests let the compiler sink the donor
      // and queue reductions behind the receiver's)
      if (fit) {
        r_amt = amt;
      } else {
        r_amt = min(static_cast<int32_t>(kmax >> 6), amt - mt);
        r_amt = r_amt >= mt ? r_amt : 0;
        const int32_t rest = amt - r_amt;
        if (dmax > 0) {
          // the donor takes the rest when it has room for all of it, else
          // at most rest - mt (what stays queued is at least the minimum)
          x = droom >= rest ? rest : min(droom, rest - mt);
          if (x < mt) return false;
        } else if (r_amt == 0) {
          return false;
        }
      }
    } else {
      // the receiver takes the whole piece on a fit, else its whole spare
      if (!fit && kmax == 0 && dmax == 0) return false;
      r_amt = fit ? amt : static_cast<int32_t>(kmax >> 6);
      if constexpr (!LEAN) x = (!fit && dmax > 0) ? min(amt - r_amt, droom) : 0;
    }
    const int32_t left = amt - r_amt - x;
    const bool rcv = lane == kl, don = !LEAN && lane == dl;
    // (the receiver, when there is one, is never the donor; dl names some
    // lane even when no donor is taken, x then being 0)
    const int32_t give = rcv ? r_amt : (don ? x : 0);
    const bool put = give > 0;
#pragma unroll
    for (int s = SMAX - 1; s > 0; --s) {
      ht[s] = put ? ht[s - 1] : ht[s];
      hq[s] = put ? hq[s - 1] : hq[s];
    }
    ht[0] = put ? t : ht[0];
    hq[0] = put ? give : hq[0];
    nh += put ? 1 : 0;
    spare -= rcv ? r_amt : 0;
    const uint32_t requeue = left > 0 ? (static_cast<uint32_t>(left) << TB) | own_tie : 0u;
    const uint32_t xs = static_cast<uint32_t>(x) << TB;
#pragma unroll
    for (int j = 0; j < MMAX; ++j) {
      const bool dj = don && j == djs;
      qk[j] = popped[j] ? requeue : qk[j] + (dj ? xs : 0u);
      room[j] -= dj ? x : 0;
    }
    // a fit leaves dmax at most knext (the donor's piece is still queued)
    km = __builtin_amdgcn_readfirstlane(static_cast<int>(max(max(knext, dmax + xs), requeue)));
  }
  // hosted lists in arrival order (slot s holds the s-th replica placed)
  if (act) {
#pragma unroll
    for (int s = 0; s < SMAX; ++s)
      if (s < S) {
        int32_t tt = -1, qq = 0;
#pragma unroll
        for (int p = 0; p < SMAX; ++p)
          if (p == nh - 1 - s) {
            tt = ht[p];
            qq = hq[p];
          }
        res_e[lane * S + s] = tt >= 0 ? (d * D + tt / MMAX) * M + tt % MMAX : -1;
        res_q[lane * S + s] = tt >= 0 ? qq : 0;
      }
  }
  return true;
}

// Tile ordinal bases for the experts of tile-base workgroup `role` (see
// scan_thread) of one layer: base[t][e]
// = number of pairs of e in tiles before t.  Thread (el, ch) sums a
// contiguous run of tiles of one expert, the runs are scanned in LDS, and the
// run is re-read and written out as running prefixes.  Loads go in batches
// of 16 with clamped indices so each batch is one round trip.
__device__ void tile_base_scan(const uint16_t* __restrict__ hist, int32_t* __restrict__ base,
                               int32_t ntiles, int32_t E, int32_t role, int32_t ew, int32_t* part) {
  const int32_t hs = hist_stride(E);
  constexpr int B = kScanBatch;
  const int tid = threadIdx.x;
  const ScanThread th = scan_thread(tid, role, ew, ntiles, E);
  const int e = th.e;
  int32_t sum = 0;
  if (th.act) {
    for (int tb = th.t0; tb < th.t1; tb += B) {
      int32_t x[B];
#pragma unroll
      for (int u = 0; u < B; ++u) x[u] = hist[static_cast<int64_t>(scan_row(tb, u, ntiles)) * hs + e];
#pragma unroll
      for (int u = 0; u < B; ++u)
        if (tb + u < th.t1) sum += x[u];
    }
  }
  part[tid] = sum;
  __syncthreads();
  if (th.act) {
    int32_t run = 0;
    for (int q = 0; q < th.ch; ++q) run += part[q * ew + th.el];
    for (int tb = th.t0; tb < th.t1; tb += B) {
      int32_t x[B];
#pragma unroll
      for (int u = 0; u < B; ++u) x[u] = hist[static_cast<int64_t>(scan_row(tb, u, ntiles)) * hs + e];
#pragma unroll
      for (int u = 0; u < B; ++u)
        if (tb + u < th.t1) {
          base[static_cast<int64_t>(tb + u) * E + e] = run;
          run += x[u];
        }
    }
  }
}

// Pairs per expert of one layer: c[e] += the sum of column e over the tile
// histogram rows.  Thread (q, ch) reads W 32-bit words (2W experts) of rows
// ch, ch + nch, ..., so each batch of loads reads whole rows; a batch of B
// loads is issued before any is used (B no larger than a thread's rows
// need: the loads past the last row repeat it).  W = 4 (16-byte loads, half
// the batches of W = 1) needs rows of a multiple of 8 entries on a 16-byte
// aligned base.  The chunk sums meet in LDS.
template <int W, int B>
__device__ void sum_hist_rows(const uint16_t* __restrict__ H, int hs, int ntiles, int E, int32_t* c) {
  const SumThread th = sum_thread(threadIdx.x, hs, W, ntiles);
  if (!th.act) return;
  const int q = th.q, nch = th.nch;
  int32_t sum[2 * W];
#pragma unroll
  for (int i = 0; i < 2 * W; ++i) sum[i] = 0;
  for (int tb = th.ch; tb < ntiles; tb += B * nch) {
    uint32_t x[B][W];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int64_t row = sum_row(tb, u, nch, ntiles);
      if constexpr (W == 4) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(H + row * hs + 8 * q);
        x[u][0] = v.x; x[u][1] = v.y; x[u][2] = v.z; x[u][3] = v.w;
      } else {
        x[u][0] = reinterpret_cast<const uint32_t*>(H)[row * (hs / 2) + q];
      }
    }
    // rows past the last are masked to zero, not skipped: a load whose
    // value is used only under a condition may be sunk into that branch and
    // issued after the others have been waited for
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const uint32_t keep = tb + u * nch < ntiles ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const uint32_t v = x[u][w] & keep;
        sum[2 * w] += static_cast<int32_t>(v & 0xFFFFu);
        sum[2 * w + 1] += static_cast<int32_t>(v >> 16);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 2 * W; ++i) {
    const int e = 2 * W * q + i;
    if (sum[i] && e < E) atomicAdd(&c[e], sum[i]);
  }
}

// One launch per batch of layers: workgroup 0 of each layer's group solves
// the plan; the other scan_wgs workgroups build the tile ordinal bases the
// reroute kernel needs, on other CUs, while the plan is being solved.
template <int MMAX, int SMAX>
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const uint16_t* __restrict__ hist,
                                                            int32_t* __restrict__ tile_base,
                                                            int32_t* __restrict__ plans,
                                                            PlanParams a) {
  extern __shared__ __align__(16) int32_t lds[];
  const PlanRole pr = plan_role(blockIdx.x, a.scan_wgs);
  const int layer = pr.layer;
  const int E = a.E, R = a.R, S = a.S, D = a.D, M = a.M, P = a.P;
  const int32_t hs = hist_stride(E);
  const uint16_t* H = hist + static_cast<int64_t>(layer) * a.ntiles * hs;
  if (pr.role > 0) {
    tile_base_scan(H, tile_base + static_cast<int64_t>(layer) * a.ntiles * E, a.ntiles, E, pr.role,
                   a.scan_ew, lds);
    return;
  }
  const PlanLds L = carve(lds, a);
  const int tid = threadIdx.x;
  // the wave index is uniform: kept in a scalar register, so the probe's
  // per-item values (quota, domain, popped expert) stay scalar too
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = lane_id();
  int32_t* rec = plans + static_cast<int64_t>(layer) * a.rec_words;

  if (tid < kScalars) L.scal[tid] = 0;
  for (int d = tid; d < a.ndom; d += kPlanThreads) L.dom[d] = 0;

  // -- phase 0: pairs per expert = sum of the tile histograms.
  for (int e = tid; e < E; e += kPlanThreads) L.c[e] = 0;
  __syncthreads();
  if (sum_vector_form(hs, reinterpret_cast<uintptr_t>(H))) {
    const int batch = sum_batch(hs, a.ntiles);
    if (batch == 4)
      sum_hist_rows<4, 4>(H, hs, a.ntiles, E, L.c);
    else if (batch == 8)
      sum_hist_rows<4, 8>(H, hs, a.ntiles, E, L.c);
    else
      sum_hist_rows<4, 16>(H, hs, a.ntiles, E, L.c);
  } else {
    sum_hist_rows<1, 32>(H, hs, a.ntiles, E, L.c);
  }
  __syncthreads();
  // -- phase 1: home loads, total, grid (wave 0, wave reductions only: LDS
  // atomics on one address would be serialised lane by lane).
  if (wave == 0) {
    uint32_t total = 0, qmax = 0, floor = 0, cmax = 0;
    for (int e0 = 0; e0 < E; e0 += 64)
      cmax = max(cmax, wave_max(e0 + lane < E ? static_cast<uint32_t>(L.c[e0 + lane]) : 0u));
    // domain loads by LDS atomics (L.dom starts at zero): one instruction
    // per 64 ranks instead of a serial sum per domain
    // (when a domain spans whole waves of ranks, its load is the wave sums
    // of its ranks, added by one lane, instead of 64 atomics on one word)
    const bool wide = D % 64 == 0;
    for (int r0 = 0; r0 < R; r0 += 64) {
      const int r = r0 + lane;
      int32_t h = 0;
      if (r < R) {
        for (int j = 0; j < M; ++j) h += L.c[r * M + j];
        L.H[r] = h;
        if (!wide) atomicAdd(&L.dom[r / D], h);
      }
      const uint32_t hsum = wave_sum(static_cast<uint32_t>(h));
      if (wide && lane == 0) L.dom[r0 / D] += static_cast<int32_t>(hsum);
      total += hsum;
      qmax = max(qmax, wave_max(static_cast<uint32_t>(h)));
    }
    for (int d0 = 0; d0 < a.ndom; d0 += 64) {
      const int d = d0 + lane;
      const uint32_t dl = d < a.ndom ? static_cast<uint32_t>(L.dom[d]) : 0u;
      floor = max(floor, wave_max((dl + D - 1) / D));
    }
    if (lane == 0) {
      // lowest quota aimed at: the early-stop target times the mean (at
      // least the domain floor, at most the max home load)
      // (64-bit division is a long software sequence: both quotients take
      // the 32-bit form whenever their operands fit, as they do for the
      // default target and tolerance)
      const uint64_t tden = static_cast<uint64_t>(R) * a.thr_den;
      const uint64_t qnum = static_cast<uint64_t>(total) * a.thr_num + tden - 1;
      const uint64_t eden = static_cast<uint64_t>(R) * a.eps_den;
      const uint64_t enum_ = static_cast<uint64_t>(total) * a.eps_num;
      const int64_t qmean = static_cast<int64_t>(
          (qnum >> 32) == 0 && (tden >> 32) == 0 ? static_cast<uint32_t>(qnum) / static_cast<uint32_t>(tden)
                                                 : qnum / tden);
      const int64_t qlb64 = min(max(qmean, static_cast<int64_t>(floor)), static_cast<int64_t>(qmax));
      const int32_t qlb = static_cast<int32_t>(qlb64);
      const int64_t tol64 = static_cast<int64_t>(
          (enum_ >> 32) == 0 && (eden >> 32) == 0 ? static_cast<uint32_t>(enum_) / static_cast<uint32_t>(eden)
                                                  : enum_ / eden);
      const int32_t tol = static_cast<int32_t>(tol64 < 1 ? 1 : tol64);
      L.scal[kTotal] = static_cast<int32_t>(total);
      L.scal[kQmax] = static_cast<int32_t>(qmax);
      L.scal[kFloor] = static_cast<int32_t>(floor);
      L.scal[kQlb] = qlb;
      L.scal[kTol] = tol;
      L.scal[kK] = static_cast<int32_t>(qmax) > qlb ? (static_cast<int32_t>(qmax) - qlb + tol - 1) / tol : 0;
      L.scal[kReplicas] = 0;
      L.scal[kCmax] = static_cast<int32_t>(cmax);
    }
  } else {
    // meanwhile the other waves write what is already final (the counts and
    // the padding between the record's fields: fixed values, so a record is
    // a pure function of its inputs) and set up the master quotas, so these
    // stores are long done when the kernel ends
    const int t1 = tid - 64, n1 = kPlanThreads - 64;
    for (int e = t1; e < E; e += n1) {
      rec[a.off[ULTRAEP_PLAN_COUNTS] + e] = L.c[e];
      L.mq[e] = L.c[e];
      L.rmask[e] = 0;
    }
    // (unrolled, so the field offsets come in with one batch of scalar
    // loads instead of a dependent load per field)
#pragma unroll
    for (int f = 0; f < ULTRAEP_PLAN_NUM_FIELDS; ++f) {
      const int end = f + 1 < ULTRAEP_PLAN_NUM_FIELDS ? a.off[f + 1] : a.rec_words;
      for (int wd = a.off[f] + a.len[f] + t1; wd < end; wd += n1) rec[wd] = 0;
    }
  }
  __syncthreads();
  const int32_t qlb = L.scal[kQlb], tol = L.scal[kTol], K = L.scal[kK], qmax = L.scal[kQmax];
  const int32_t cmax = L.scal[kCmax];

  // -- phase 2: probe rounds; each wave takes (grid quota, domain) items.
  const bool no_moves = (S == 0 || D == 1);
  int32_t winner = no_moves ? K : -1;
  int32_t wg0 = 0, rounds = 0;
  for (int32_t g0 = 0; winner < 0; g0 += a.G) {
    ++rounds;
    for (int item = wave; item < a.items; item += kPlanWaves) {
      const int32_t g = g0 + item / a.ndom;
      const int d = item % a.ndom;
      bool okv = false;
      if (g <= K) {
        const int32_t Q = g < K ? qlb + g * tol : qmax;
        int32_t* re = L.res + static_cast<size_t>(item) * D * S;
        int32_t* rq = L.res + static_cast<size_t>(a.items + item) * D * S;
        constexpr uint32_t kPieceLimit = 1u << (26 - ilog2_c(MMAX));
        const bool packed = static_cast<uint32_t>(cmax) < kPieceLimit && Q < (1 << 25);
        if (!packed)
          okv = greedy_probe<MMAX, SMAX>(Q, d, a, L, re, rq);
        else if (a.lean)
          okv = a.min_tokens > 1 ? greedy_probe_packed<MMAX, SMAX, true, true>(Q, d, a, L, re, rq)
                                 : greedy_probe_packed<MMAX, SMAX, false, true>(Q, d, a, L, re, rq);
        else
          okv = a.min_tokens > 1 ? greedy_probe_packed<MMAX, SMAX, true, false>(Q, d, a, L, re, rq)
                                 : greedy_probe_packed<MMAX, SMAX, false, false>(Q, d, a, L, re, rq);
      }
      if (lane == 0) L.ok[item] = okv ? 1 : 0;
    }
    __syncthreads();
    if (tid == 0) {
      int32_t w = -1;
      for (int gg = 0; gg < a.G && w < 0 && g0 + gg <= K; ++gg) {
        bool all = true;
        for (int d = 0; d < a.ndom; ++d) all = all && L.ok[gg * a.ndom + d];
        if (all) w = g0 + gg;
      }
      L.scal[kWin] = w;
    }
    __syncthreads();
    winner = L.scal[kWin];
    wg0 = g0;
    __syncthreads();
  }

  // -- phase 3: the plan record.  One thread per slot (there are at most
  // kPlanThreads) takes its hosted expert and quota from the winning probe,
  // records them, and takes the quota off the master's (L.mq starts as the
  // counts) and marks the slot's rank in the expert's mask.
  // The same thread later places the slot's instance and that of master
  // tid, whose local takes need the counts of the expert in its rank's
  // tiles: the first kLocalBatch of those are loaded here, and their latency
  // passes while the offsets are built.
  static_assert(ULTRAEP_MAX_TOTAL_SLOTS <= kPlanThreads && ULTRAEP_MAX_EXPERTS <= kPlanThreads,
                "one thread per slot and per master");
  int32_t slot_e = -1, slot_q = 0;
  int32_t xs[kLocalBatch], xm[kLocalBatch];
  {
    const int s = tid;
    int32_t e = -1, q = 0;
    if (s < R * S && !no_moves) {
      const int r = s / S, j = s % S, d = r / D, lr = r % D;
      const int item = (winner - wg0) * a.ndom + d;
      e = L.res[static_cast<size_t>(item) * D * S + lr * S + j];
      q = L.res[static_cast<size_t>(a.items + item) * D * S + lr * S + j];
    }
    q = e >= 0 ? q : 0;
    slot_e = e;
    slot_q = q;
    {
      const bool pf = local_prefetch(a.tpr);
      const int rs = S > 0 ? s / S : 0, rm = tid / M;
#pragma unroll
      for (int u = 0; u < kLocalBatch; ++u) {
        xs[u] = pf && e >= 0 ? H[static_cast<int64_t>(local_row(rs * a.tpr, u, (rs + 1) * a.tpr)) * hs + e] : 0;
        xm[u] = pf && tid < E ? H[static_cast<int64_t>(local_row(rm * a.tpr, u, (rm + 1) * a.tpr)) * hs + tid] : 0;
      }
    }
    if (s < R * S) {
      L.slotE[s] = e;
      L.slotQ[s] = q;
      rec[a.off[ULTRAEP_PLAN_SLOT_EXPERT] + s] = e;
      rec[a.off[ULTRAEP_PLAN_SLOT_QUOTA] + s] = q;
      if (e >= 0) {
        atomicSub(&L.mq[e], q);
        atomicOr(&L.rmask[e], 1ull << ((s / S) % D));
      }
    }
    const uint32_t filled = __builtin_popcountll(ballot(e >= 0));
    if (lane == 0 && filled) atomicAdd(&L.scal[kReplicas], static_cast<int32_t>(filled));
  }
  __syncthreads();
  // physical loads (recorded as they are written: the scan below turns them
  // into offsets) and rank loads, both from the final quotas
  for (int p = tid; p < P; p += kPlanThreads) {
    const int r = p / (M + S), j = p % (M + S);
    const int32_t q = j < M ? L.mq[r * M + j] : L.slotQ[r * S + (j - M)];
    L.pload[p] = q;
    rec[a.off[ULTRAEP_PLAN_PHYS_LOAD] + p] = q;
  }
  for (int e = tid; e < E; e += kPlanThreads) {
    L.iptr[e] = 1 + __builtin_popcountll(L.rmask[e]);
    rec[a.off[ULTRAEP_PLAN_MASTER_QUOTA] + e] = L.mq[e];
  }
  for (int r = tid; r < R; r += kPlanThreads) {
    int32_t s = 0;
    for (int j = 0; j < M; ++j) s += L.mq[r * M + j];
    for (int j = 0; j < S; ++j) s += L.slotQ[r * S + j];
    rec[a.off[ULTRAEP_PLAN_RANK_AFTER] + r] = s;
    rec[a.off[ULTRAEP_PLAN_RANK_BEFORE] + r] = L.H[r];
  }
  __syncthreads();
  // pload -> phys_off, instance counts -> inst_ptr: one wave each, so the
  // two scans run side by side and need no barrier but the one after them
  if (wave == 0) wave_exclusive_scan(L.pload, P);
  if (wave == 1) wave_exclusive_scan(L.iptr, E);
  __syncthreads();

  // instances of e in ascending physical id = ascending rank inside e's
  // domain.  One thread per master or filled slot places its instance: the
  // index is e's first index + e's instances on lower ranks (the set bits of
  // e's rank mask below its own); its local take is min(quota, pairs of e
  // from its rank's tiles).  Then the quota ends and first rows come from
  // one scan of the instances' quotas.
  int32_t* inst_phys = rec + a.off[ULTRAEP_PLAN_INST_PHYS];
  int32_t* inst_end = rec + a.off[ULTRAEP_PLAN_INST_END];
  int32_t* inst_base = rec + a.off[ULTRAEP_PLAN_INST_BASE];
  int32_t* inst_local = rec + a.off[ULTRAEP_PLAN_INST_LOCAL];
  for (int e = tid; e <= E; e += kPlanThreads) rec[a.off[ULTRAEP_PLAN_INST_PTR] + e] = L.iptr[e];
  for (int p = tid; p <= P; p += kPlanThreads) rec[a.off[ULTRAEP_PLAN_PHYS_OFF] + p] = L.pload[p];
  // unused instance entries get fixed values
  for (int i = L.iptr[E] + tid; i < a.n_inst; i += kPlanThreads) {
    inst_phys[i] = -1;
    inst_end[i] = 0;
    inst_base[i] = 0;
    inst_local[i] = 0;
  }
  // thread tid places master tid and the instance of slot tid
  auto place = [&](int e, int r, int p, int32_t q, const int32_t (&x0)[kLocalBatch]) {
    const int home = e / M;
    const uint64_t in_domain = D == 64 ? ~0ull : ((1ull << D) - 1);
    const uint64_t m = (L.rmask[e] | (1ull << (home % D))) & in_domain;
    const int i = L.iptr[e] + __builtin_popcountll(m & ((1ull << (r % D)) - 1));
    L.instp[i] = p;
    L.iq[i] = q;
    L.iex[i] = e;
    inst_phys[i] = p;
    // pairs of e from rank r's tiles: the first batch came in early, the
    // rest (ranks of more than kLocalBatch tiles) eight loads at a time
    const int t0 = r * a.tpr, t1 = t0 + a.tpr;
    int32_t own = 0;
#pragma unroll
    for (int u = 0; u < kLocalBatch; ++u) own += t0 + u < t1 ? x0[u] : 0;
    for (int tb = t0 + kLocalBatch; tb < t1; tb += kLocalBatch) {
      int32_t x[kLocalBatch];
#pragma unroll
      for (int u = 0; u < kLocalBatch; ++u) x[u] = H[static_cast<int64_t>(local_row(tb, u, t1)) * hs + e];
#pragma unroll
      for (int u = 0; u < kLocalBatch; ++u) own += tb + u < t1 ? x[u] : 0;
    }
    inst_local[i] = min(q, own);
  };
  if (tid < E) {
    const int r = tid / M;
    place(tid, r, r * (M + S) + tid % M, L.mq[tid], xm);
  }
  if (tid < R * S && slot_e >= 0) {
    const int r = tid / S;
    place(slot_e, r, r * (M + S) + M + tid % S, slot_q, xs);
  }
  __syncthreads();
  // quota ends and first rows: the instances' quotas are scanned once across
  // all experts (e's instances are contiguous), so each instance's end is
  // its inclusive prefix minus the prefix at e's first instance
  const int n_used = L.iptr[E];
  if (wave == 0) wave_exclusive_scan(L.iq, n_used);
  __syncthreads();
  for (int i = tid; i < n_used; i += kPlanThreads) {
    const int e = L.iex[i];
    const int32_t q = L.iq[i + 1] - L.iq[i];
    const int32_t end = L.iq[i + 1] - L.iq[L.iptr[e]];
    inst_end[i] = end;
    inst_base[i] = L.pload[L.instp[i]] - (end - q);
  }
  if (tid < kHeaderWords) {
    int32_t v = 0;
    const int32_t total = L.scal[kTotal];
    switch (tid) {
      case ULTRAEP_HDR_MAGIC: v = static_cast<int32_t>(ULTRAEP_PLAN_MAGIC); break;
      case ULTRAEP_HDR_E: v = E; break;
      case ULTRAEP_HDR_R: v = R; break;
      case ULTRAEP_HDR_S: v = S; break;
      case ULTRAEP_HDR_D: v = D; break;
      case ULTRAEP_HDR_M: v = M; break;
      case ULTRAEP_HDR_P: v = P; break;
      case ULTRAEP_HDR_N: v = a.N; break;
      case ULTRAEP_HDR_TOTAL: v = total; break;
      case ULTRAEP_HDR_DROPPED: v = a.N - total; break;
      case ULTRAEP_HDR_Q_STAR: v = winner < K ? qlb + winner * tol : qmax; break;
      case ULTRAEP_HDR_Q_LB: v = qlb; break;
      case ULTRAEP_HDR_Q_MAX: v = qmax; break;
      case ULTRAEP_HDR_TOL: v = tol; break;
      case ULTRAEP_HDR_GRID_INDEX: v = winner; break;
      case ULTRAEP_HDR_FLOOR: v = L.scal[kFloor]; break;
      case ULTRAEP_HDR_REPLICAS: v = L.scal[kReplicas]; break;
      case ULTRAEP_HDR_ROUNDS: v = rounds; break;
      default: v = 0; break;
    }
    rec[a.off[ULTRAEP_PLAN_HEADER] + tid] = v;
  }
}

// ------------------------------------------------------------------------
// reroute: replica and layout row of every pair ([README] Interface,
// "Forward and backward": reroute expands logical routing to replicas)
// ------------------------------------------------------------------------
// Same tiling as count.  A pair's ordinal among its expert's pairs is the
// tile's base (from the plan launch's scan workgroups) + the pairs of earlier
// waves in the tile + the pair's rank inside its wave, which the wave tracks
// with groups of equal ids (found through LDS lane masks) and per-wave LDS
// counters, so no sort is needed and the result does not depend on
// scheduling.
//
// With LAYOUT the kernel also writes the inverse index and permuted weights.
// Inside one tile, the pairs that land on one instance have consecutive
// ordinals, so they fill one contiguous run of layout rows.  Each pair's
// weight and index are first placed at its run's slot in LDS; the runs are
// then written out with consecutive lanes on consecutive rows, instead of
// one 4-byte scatter per pair.  The staged weights reuse the words of the
// grouping masks and the indices are 16-bit, which keeps the tables (about
// 65 KiB at E = 128, 77 KiB at E = 256) small enough for two 16-wave
// workgroups per CU.
struct RerouteLds {
  unsigned long long* peers;  // [waves][E+1] lane masks for grouping equal ids (pass 1)
  i32x4* inst;     // [n_inst] per instance: quota end, physical expert, first
                   // layout row, then (LAYOUT) staging slot minus layout row
                   // of its run; one 16-byte read per instance in pass 2
  uint32_t* bits;  // LAYOUT: [kTile / 32] bit j set where a non-empty run starts at slot j
  int32_t* cntw;   // [waves][E]: per-wave counters, then per-wave ordinal bases
  int32_t* tcnt;   // [E] the tile's ordinal base of e
  uint32_t* ek;    // [E] first instance of e holding ordinals of this tile | last instance << 16
  int32_t* iptr;   // [E+1]
  int32_t* roff;   // LAYOUT: [n_inst+1] run offsets inside the staging area | runs
                   // before with pairs << 16
  int32_t* nr;     // LAYOUT: [n_inst] staging slot minus layout row of the q-th non-empty run
  float* wst;      // [kTile] staged slot's routing weight (pass 2; shares its
                   // words with peers, which pass 1 is done with)
  uint16_t* sn;    // [kTile] staged slot's pair index inside the tile
};

// Words of the region that holds peers, and with the layout also the staged
// weights.  A multiple of 4 words, so the instance records after it are
// 16-byte aligned.
__host__ __device__ inline size_t reroute_shared_words(int E, bool layout, int waves) {
  const size_t peers = 2ull * waves * (E + 1);
  return layout && peers < static_cast<size_t>(kTile) ? kTile : peers;
}

__host__ __device__ inline size_t reroute_lds_bytes(int E, int n_inst, bool layout, int waves) {
  size_t words = reroute_shared_words(E, layout, waves) + 4ull * n_inst + static_cast<size_t>(waves) * E +
                 2ull * E + (E + 1);
  if (layout) words += kTile / 32 + (n_inst + 1) + n_inst + kTile / 2;
  return 4 * words;
}

// Two 16-wave workgroups per CU need at most 64 VGPRs per lane.
template <bool LAYOUT, int W>
__global__ __launch_bounds__(TileShape<W>::kThreads)
__attribute__((amdgpu_waves_per_eu(W == 16 ? 8 : 1))) void reroute_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ w, int32_t N, int32_t TK, int32_t tpr,
    int32_t E, int32_t ntiles, const int32_t* __restrict__ tile_base, const int32_t* __restrict__ plans,
    int32_t rec_words, int32_t off_iptr, int32_t off_iend, int32_t off_iphys, int32_t off_ibase,
    int32_t n_inst, int32_t* __restrict__ phys_idx, int32_t* __restrict__ pos,
    int32_t* __restrict__ inv, float* __restrict__ w_perm) {
  using T = TileShape<W>;
  constexpr int NT = T::kThreads;
  extern __shared__ __align__(16) int32_t lds[];
  RerouteLds S;
  {
    int32_t* q = lds;
    S.peers = reinterpret_cast<unsigned long long*>(q);
    S.wst = reinterpret_cast<float*>(q);
    q += reroute_shared_words(E, LAYOUT, W);
    S.inst = reinterpret_cast<i32x4*>(q); q += 4 * n_inst;
    if (LAYOUT) {
      S.bits = reinterpret_cast<uint32_t*>(q); q += kTile / 32;
    }
    S.cntw = q; q += W * E;
    S.tcnt = q; q += E;
    S.ek = reinterpret_cast<uint32_t*>(q); q += E;
    S.iptr = q; q += E + 1;
    if (LAYOUT) {
      S.roff = q; q += n_inst + 1;
      S.nr = q; q += n_inst;
      S.sn = reinterpret_cast<uint16_t*>(q);
    }
  }
  const int64_t blk = xcd_block(blockIdx.x, gridDim.x);
  const int32_t layer = static_cast<int32_t>(blk / ntiles);
  const int32_t tile = static_cast<int32_t>(blk % ntiles);
  const int32_t* plan = plans + static_cast<int64_t>(layer) * rec_words;
  const int64_t lb = static_cast<int64_t>(layer) * N;
  const TileSpan span = tile_span(layer, tile, N, TK, tpr);
  const int64_t first = span.first;
  const int n_here = span.n;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int base = wave * T::kWavePairs;
  const int32_t* tb = tile_base + (static_cast<int64_t>(layer) * ntiles + tile) * E;

  uint32_t v[T::kChunks];
  load_tile_ids(idx + first, base, n_here, lane, E, v);
  for (int i = threadIdx.x; i < W * (E + 1); i += NT) S.peers[i] = 0;
  for (int i = threadIdx.x; i < W * E; i += NT) S.cntw[i] = 0;
  for (int i = threadIdx.x; i <= E; i += NT) S.iptr[i] = plan[off_iptr + i];
  for (int i = threadIdx.x; i < n_inst; i += NT)
    S.inst[i] = i32x4{plan[off_iend + i], plan[off_iphys + i], plan[off_ibase + i], 0};
  if (LAYOUT)
    for (int i = threadIdx.x; i < kTile / 32; i += NT) S.bits[i] = 0;
  for (int e = threadIdx.x; e < E; e += NT) S.tcnt[e] = tb[e];
  __syncthreads();

  // pass 1: rank of each pair among the wave's earlier pairs of its expert.
  // Afterwards v[c] holds the pair's expert id (E for an invalid one) in its
  // low 11 bits and its rank in the wave above them.
  int32_t* my = S.cntw + wave * E;
  unsigned long long* mw = S.peers + wave * (E + 1);
#pragma unroll
  for (int c = 0; c < T::kChunks; ++c) {
    const uint64_t peers = match_peers_lds(mw, v[c], lane);
    const bool valid = v[c] < static_cast<uint32_t>(E);
    const int32_t old = valid ? my[v[c]] : 0;
    if (lane == lowest_lane(peers)) {
      if (valid) my[v[c]] = old + __builtin_popcountll(peers);
      mw[v[c]] = 0;
    }
    const uint32_t lr = static_cast<uint32_t>(old + count_below(peers));
    v[c] = (lr << 11) | (valid ? v[c] : static_cast<uint32_t>(E));
  }
  __syncthreads();
  // with the layout, the packed values wait out the steps up to pass 2 in
  // the staging words (pass 1 is done with its lane masks), so they hold no
  // registers meanwhile; the registers take the pairs' weights instead (one
  // coalesced load per chunk), which arrive while the runs are set up.  The
  // weights come through one buffer resource over the tile (one offset
  // register for all chunks; loads past the tile read 0 and are not used).
  float wl[LAYOUT ? T::kChunks : 1];
  if (LAYOUT) {
#pragma unroll
    for (int c = 0; c < T::kChunks; ++c) reinterpret_cast<uint32_t*>(S.wst)[c * NT + threadIdx.x] = v[c];
    const __amdgpu_buffer_rsrc_t r_w = row_rsrc(w + first, static_cast<uint32_t>(n_here) * 4u);
#pragma unroll
    for (int c = 0; c < T::kChunks; ++c)
      wl[c] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(r_w, (base + c * 64 + lane) * 4, 0, kNonTemporal));
  }
  for (int e = threadIdx.x; e < E; e += NT) {
    const int32_t b0 = S.tcnt[e];
    // counts are read eight at a time before their bases are written: the
    // reads then go out back to back instead of one round trip per wave
    constexpr int kGroup = W < 8 ? W : 8;
    int32_t run = b0;
#pragma unroll
    for (int q0 = 0; q0 < W; q0 += kGroup) {
      int32_t t[kGroup];
#pragma unroll
      for (int q = 0; q < kGroup; ++q) t[q] = S.cntw[(q0 + q) * E + e];
#pragma unroll
      for (int q = 0; q < kGroup; ++q) {
        S.cntw[(q0 + q) * E + e] = run;
        run += t[q];
      }
    }
    // k: the instance where the tile's ordinals of e start (the first whose
    // quota end passes b0); a pair's instance is then at most a few steps
    // further.  With the layout, the same walk sets up the runs: instance i
    // holds the tile's ordinals [max(start_i, b0), min(end_i, b1)) of
    // [b0, b1).  The scan below sums the run lengths (low half) and the
    // non-empty runs (high half) together; the first ordinal waits in the
    // record's fourth word.  The next end is read ahead, so the walk takes
    // one LDS round trip per instance.
    const int i0 = S.iptr[e], last = S.iptr[e + 1] - 1;
    int k = -1;
    int32_t start = 0, end = S.inst[i0].x;
    for (int i = i0; i <= last; ++i) {
      const int32_t next = i < last ? S.inst[i + 1].x : 0;
      if (k < 0 && (b0 < end || i == last)) k = i;
      if (LAYOUT) {
        const int32_t lo = max(start, b0), len = max(0, min(end, run) - lo);
        S.roff[i] = len | (len > 0 ? 1 << 16 : 0);
        S.inst[i].w = lo;
      } else if (k >= 0) {
        break;
      }
      start = end;
      end = next;
    }
    S.ek[e] = static_cast<uint32_t>(k) | (static_cast<uint32_t>(last) << 16);
  }
  if (LAYOUT) {
    // instance entries beyond the plan's used ones are empty runs
    for (int i = S.iptr[E] + threadIdx.x; i < n_inst; i += NT) {
      S.roff[i] = 0;
      S.inst[i].w = 0;
    }
  }
  __syncthreads();

  if (LAYOUT) {
    if (wave == 0) wave_exclusive_scan(S.roff, n_inst);
    __syncthreads();
    // the fourth word becomes staging slot minus layout row of each run;
    // a non-empty run (the q-th) also marks its first slot and files the
    // same offset under q
    for (int i = threadIdx.x; i < n_inst; i += NT) {
      const int32_t r0 = S.roff[i];
      const int off = r0 & 0xFFFF, q = r0 >> 16, len = (S.roff[i + 1] - r0) & 0xFFFF;
      const int32_t d = off - S.inst[i].z - S.inst[i].w;
      S.inst[i].w = d;
      // (the bounds only matter for a corrupted plan record)
      if (len > 0 && off < kTile && q < n_inst) {
        S.nr[q] = d;
        atomicOr(&S.bits[off >> 5], 1u << (off & 31));
      }
    }
    __syncthreads();
  }

  // pass 2: instance, physical expert and layout row of each pair; with the
  // layout, each pair's weight and index go to its run's slot
  if (LAYOUT) {
#pragma unroll
    for (int c = 0; c < T::kChunks; ++c) v[c] = reinterpret_cast<const uint32_t*>(S.wst)[c * NT + threadIdx.x];
    __syncthreads();
  }
  // phys and pos go out non-temporally: each wave store is whole lines and
  // nothing here reads them back, so they need not stay in L2 (the scattered
  // layout stores below keep the default policy, under which their partial
  // lines merge in L2)
  const __amdgpu_buffer_rsrc_t r_phys = row_rsrc(phys_idx + first, static_cast<uint32_t>(n_here) * 4u);
  const __amdgpu_buffer_rsrc_t r_pos = row_rsrc(pos + first, static_cast<uint32_t>(n_here) * 4u);
#pragma unroll
  for (int c = 0; c < T::kChunks; ++c) {
    const int i = base + c * 64 + lane;
    int32_t p = -1, row = -1;
    const int e = static_cast<int>(v[c] & 0x7FFu);
    if (e < E) {
      const int32_t o = my[e] + static_cast<int32_t>(v[c] >> 11);
      const uint32_t ek = S.ek[e];
      int k = static_cast<int>(ek & 0xFFFFu);
      const int last = static_cast<int>(ek >> 16);
      i32x4 rec = S.inst[k];
      while (k < last && o >= rec.x) rec = S.inst[++k];
      p = rec.y;
      row = rec.z + o;
      if (LAYOUT) {
        const int32_t sl = row + rec.w;
        if (sl >= 0 && sl < kTile) {
          S.sn[sl] = static_cast<uint16_t>(i);
          S.wst[sl] = wl[c];
        }
      }
    }
    __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(p), r_phys, i * 4, 0, kNonTemporal);
    __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(row), r_pos, i * 4, 0, kNonTemporal);
  }
  if (LAYOUT) {
    __syncthreads();
    // write the staged slots in order: consecutive threads take consecutive
    // slots, which are consecutive layout rows inside each run.  A wave's 64
    // slots are one aligned block b (lane = slot - 64 b), and a slot's run
    // is the q-th non-empty one, q + 1 being the run starts at or before
    // it: the starts in blocks before b (each wave scans the blocks' start
    // counts itself, two blocks a lane) plus those in b up to the lane.
    // A tile holds at most n_here valid pairs; the checks only matter for a
    // corrupted plan record.
    constexpr int kPer = kTile / NT;
    static_assert(kTile / 64 == 128, "two 64-slot blocks per lane");
    const int nt = min(S.roff[n_inst] & 0xFFFF, n_here);
    const int32_t tile0 = span.tile0;
    const uint64_t upto = (2ull << lane) - 1;  // lanes 0..lane (all for lane 63)
    const unsigned long long* bits64 = reinterpret_cast<const unsigned long long*>(S.bits);
    const int c0 = __builtin_popcountll(bits64[2 * lane]), c1 = __builtin_popcountll(bits64[2 * lane + 1]);
    const int incl = wave_inclusive_scan(c0 + c1);
    const int before_even = incl - c0 - c1, before_odd = incl - c1;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int j = u * NT + static_cast<int>(threadIdx.x);
      const int b = __builtin_amdgcn_readfirstlane(j >> 6);
      const int pb = static_cast<int>(readlane(static_cast<uint32_t>((b & 1) ? before_odd : before_even), b >> 1));
      if (j < nt) {
        const int q = min(pb + __builtin_popcountll(bits64[b] & upto) - 1, n_inst - 1);
        const int n = S.sn[j];
        const int32_t row = j - S.nr[q];
        if (n < n_here && row >= 0 && row < N) {
          inv[lb + row] = tile0 + n;
          w_perm[lb + row] = S.wst[j];
        }
      }
    }
  }
}

// ------------------------------------------------------------------------
// reroute, locality first ([README] "Replication planning": locality-aware
// per-rank quota decomposition; reroute interleave)
// ------------------------------------------------------------------------
// A tile's pairs all come from one source rank r (tiles never straddle
// ranks).  Pass 1 is the same grouping as reroute_kernel and gives every
// pair its ordinal o among its expert's pairs; t = o - (pairs of e from ranks
// before r) is its place in rank r's block of e.  If e has an instance on
// rank r and t is below that instance's local take a_L, the pair is local
// (row t of that instance).  Otherwise it is pool pair u = (pool pairs of e
// from ranks before r) + t - a_L.  The pool fills the remaining quotas
// rho_i = quota_i - a_i either contiguously in instance order, or
// (INTERLEAVE) round by round: in round tau every instance with rho_i > tau
// takes the next pool pair, in instance order.  Before round tau there are
// F(tau) = sum_i min(rho_i, tau) pool pairs, so pool pair u is in the round
// tau with F(tau) <= u < F(tau + 1), at place s = u - F(tau) among the
// instances with rho_i > tau.  F is linear between consecutive rho values:
// e's instances sorted by rho, each with F at its rho and the number of
// instances whose rho is at least as large, give tau and s with one search
// and one division.
//
// From one tile an instance receives its pool pairs in consecutive rows.
// With A_i(u) the pool pairs before u that instance i takes,
// clamp(u - pool start of i, 0, rho_i) for the contiguous fill and
// min(rho_i, tau(u)) + [rho_i > tau(u) and fewer than s(u) instances before
// i have rho > tau(u)] for the interleave, the tile's pool pairs [u0, u1) of
// e put A_i(u1) - A_i(u0) pairs on instance i from row A_i(u0) of its pool
// part.  With LAYOUT those runs, and the local run, are staged in LDS as in
// reroute_kernel and written out with consecutive lanes on consecutive rows.
//
// Pass 2 is bound by LDS traffic, so the set-up steps pack what it reads:
// per expert one 8-word record, per instance one packed entry (for the
// interleave, the instances of the phase where the tile's pool pairs of e
// start, in round-robin order, so a pair needs one division and one entry),
// and per run the offset from layout row to staging slot.  A pair whose pool
// index lies past that phase (the tile straddles a change in the number of
// instances still taking pairs) finds its phase among the later ones the
// tile reaches, whose headers and instance lists come from a small per-tile
// pool; only if that pool is full does it take the general search.  The
// tables stay small enough at E = 128 (about 73 KiB, 76 KiB with the
// interleave's phase pool) for two 16-wave workgroups per CU.
struct LocalLds {
  unsigned long long* peers;  // [waves][E+1] lane masks (pass 1)
  uint32_t* park;  // [kTile] the packed pair values between the passes
                   // (shares its words with peers)
  float* wst;      // [kTile] LAYOUT: the staged slots' routing weights (pass 2;
                   // shares its words with peers and park)
  uint16_t* sn;    // [kTile] LAYOUT: the staged slots' pair indices in the tile
                   // (with the weights gathered instead of staged, sn takes
                   // the words of wst)
  int32_t* cntw;   // [waves][E] per-wave counters, then per-wave bases of t
  int32_t* er;     // [E][8] per expert: set-up words (kEr*), then the record of pass 2
  int32_t* al;     // INTERLEAVE: [n_inst][2] the phase's instances (its words are ipool and ie)
  int32_t* ipool;  // [n4] the plan's cumulative quota ends, then (contiguous
                   // fill) the pool pairs before the instance
  int32_t* ie;     // [n4] expert of the instance
  int32_t* pi;     // !INTERLEAVE: [n_inst][4] packed instances (its words are ie, lev, fv, act)
  int32_t* lev;    // [n4] INTERLEAVE: e's rho values ascending (in e's instance entries)
  int32_t* fv;     // [n4] INTERLEAVE: F at that value
  int32_t* act;    // [n4] INTERLEAVE: e's instances whose rho is at least that value
  int32_t* iphys;  // [n4]
  int32_t* irow;   // [n4] first layout row of the instance
  int32_t* ia;     // [n4] local take
  int32_t* irho;   // [n4] remaining quota after the local take
  int32_t* iptr;   // [E+1]
  int32_t* roff;   // [n_inst+E+1] LAYOUT: run lengths, then their offsets in the
                   // staging area | non-empty runs before << 16 (instance i's
                   // pool run at i, e's local run at n_inst + e)
  int32_t* ro0;    // [n_inst+E] LAYOUT: first layout row of the run, then
                   // staging slot minus layout row
  int32_t* phdr;   // INTERLEAVE: [kPhaseHeaders][4] later phases the tile reaches
  int32_t* pent;   // INTERLEAVE: [kPhaseEntries][2] their instances, in order
  int32_t* pcnt;   // INTERLEAVE: [4] headers and entries handed out
};

// The tile's pool for the interleave's later phases: a tile's pool pairs of
// an expert reach past the first phase only where the number of instances
// still taking pairs changes inside the tile, which few (tile, expert) pairs
// do.  Without room a pair takes the general search.
constexpr int kPhaseHeaders = 32;
constexpr int kPhaseEntries = 160;

// Set-up words of an expert's record: the tile's ordinal base of e, then
// its pairs in the tile; pairs of e from ranks before r; pool pairs of e
// from ranks before r; e's instance on rank r (or -1).
constexpr int kErWords = 8;
constexpr int kErCount = 0, kErBlk = 1, kErPool = 2, kErLoc = 3;

__host__ __device__ inline int local_n4(int n_inst) { return (n_inst + 3) & ~3; }

// The write-out's words: the start bits of the tile's slots and one offset
// per run.  The words free after pass 2 (per-wave bases, expert records,
// the interleave's phase pool and the instance tables) usually hold them.
__host__ __device__ inline size_t local_wo_words(int E, int n_inst) {
  return kTile / 32 + static_cast<size_t>(n_inst) + E;
}
__host__ __device__ inline size_t local_dead_words(int E, int n_inst, bool interleave, int waves) {
  return static_cast<size_t>(waves) * E + static_cast<size_t>(kErWords) * E +
         (interleave ? 4 * kPhaseHeaders + 2 * kPhaseEntries + 4 : 0) + 9ull * local_n4(n_inst);
}

// gather: the write-out reads the weights from w instead of LDS, which
// frees the words of the staged weights for the pair indices.
__host__ __device__ inline size_t local_lds_bytes(int E, int n_inst, bool layout, bool interleave,
                                                  int waves, bool gather = false) {
  const size_t n4 = static_cast<size_t>(local_n4(n_inst));
  // the shared region also parks the packed pair values between the passes
  size_t words = reroute_shared_words(E, true, waves) + static_cast<size_t>(waves) * E +
                 static_cast<size_t>(kErWords) * E + 9 * n4 + (E + 1);
  if (interleave) words += 4 * kPhaseHeaders + 2 * kPhaseEntries + 4;
  if (layout) {
    words += (gather ? 0 : kTile / 2) + 2ull * (n_inst + E) + 1;
    // the write-out's own words, 16-byte aligned at the end, when the words
    // freed after pass 2 are too few
    if (local_dead_words(E, n_inst, interleave, waves) < local_wo_words(E, n_inst))
      words = ((words + 3) & ~size_t{3}) + ((local_wo_words(E, n_inst) + 3) & ~size_t{3});
  }
  return 4 * words;
}

// Where the write-out's start bits and per-run offsets go: the words of the
// per-wave bases and the expert and instance tables (done with after pass
// 2; they start 16-byte aligned), or past the end of the allocation when
// those are too few (small shapes only).
__host__ __device__ inline int32_t* local_wo_base(int32_t* lds, int E, int n_inst, bool interleave,
                                                  int waves, bool gather) {
  const size_t shared = reroute_shared_words(E, true, waves) + (gather ? 0 : kTile / 2);
  if (local_dead_words(E, n_inst, interleave, waves) >= local_wo_words(E, n_inst)) return lds + shared;
  return lds + local_lds_bytes(E, n_inst, true, interleave, waves, gather) / 4 -
         ((local_wo_words(E, n_inst) + 3) & ~size_t{3});
}

// Round and place of pool pair u of the expert whose sorted tables are the
// entries [i0, i1), searching from entry j (whose F is at most u's).  A u at
// or past the end of the pool gives the last round and place 0.
__device__ inline void interleave_round(const LocalLds& S_, int i0, int i1, int j, int32_t u,
                                        int32_t* tau, int32_t* s) {
  while (j < i1 && S_.fv[j] <= u) ++j;
  if (j == i1) {
    *tau = S_.lev[i1 - 1];
    *s = 0;
    return;
  }
  const int32_t lam0 = j > i0 ? S_.lev[j - 1] : 0;
  const int32_t f0 = j > i0 ? S_.fv[j - 1] : 0;
  const int32_t a = max(S_.act[j], 1);
  const int32_t off = u - f0;
  *tau = lam0 + off / a;
  *s = off % a;
}

// Two 16-wave workgroups per CU need at most 64 VGPRs per lane (8 waves per
// SIMD).
// Lanes that share one expert's record set-up in the locality reroute: the
// largest power of two, at most 16, with every expert's lanes in one pass
// of the workgroup (at least one lane; more experts then take more passes).
__host__ __device__ inline int records_lanes(int E, int threads) {
  int g = 1;
  while (2 * g <= 16 && static_cast<int64_t>(E) * 2 * g <= threads) g *= 2;
  return g;
}

// Per expert, G lanes together: the tile's runs and the packed record of
// pass 2.  Record words 0-3: local take, pool offset (contiguous: u = t +
// it; interleave: the place x counted from the tile's first pool pair = t +
// it), then contiguous: first instance and end of e's instances;
// interleave: the bound on x inside the phase, and phase entry base | phase
// instances << 16.  Words 4-6: local instance's physical expert and first
// row, and (interleave) u - x.  The loops over e's instances take G
// instances at a time; a first match is the lowest set bit of the
// segment's ballot, and a count of earlier instances the set bits below
// the lane, so the G lanes agree on every value without a reduction.  The
// tile's later interleave phases (rare) are set up by the segment's first
// lane alone.
template <bool INTERLEAVE, bool LAYOUT, int NT, int G>
__device__ __forceinline__ void local_records(const LocalLds& S_, int32_t* er, int E, int n_inst) {
  constexpr int EPI = NT / G;
  const int lane = lane_id();
  const int sub = lane & (G - 1), seg = lane & ~(G - 1);
  const uint32_t segmask = (1u << G) - 1, below = (1u << sub) - 1;
  auto bits = [&](bool pred) { return static_cast<uint32_t>(ballot(pred) >> seg) & segmask; };
  for (int e0 = 0; e0 < E; e0 += EPI) {
    const int e = e0 + static_cast<int>(threadIdx.x) / G;
    if (e >= E) continue;  // whole segments
    const int i0 = S_.iptr[e], i1 = S_.iptr[e + 1];
    int32_t* rec = er + e * kErWords;
    const int32_t t0 = S_.cntw[e], t1 = t0 + rec[kErCount];
    const int32_t pbase = rec[kErPool];
    const int L = rec[kErLoc];
    const int32_t aL = L >= 0 ? S_.ia[L] : 0;
    const int32_t u0 = pbase + max(t0, aL) - aL, u1 = pbase + max(t1, aL) - aL;
    if (LAYOUT && sub == 0) {
      S_.roff[n_inst + e] = L >= 0 ? max(0, min(t1, aL) - t0) : 0;
      S_.ro0[n_inst + e] = L >= 0 ? S_.irow[L] + t0 : 0;
    }
    int32_t w2, w3, w6 = 0, w7 = -1;
    if (!INTERLEAVE) {
      // the first instance whose pool range ends past u0 (the pool ends
      // grow with the instance), else the last
      int k = i1 - 1;
      for (int g0 = i0; g0 < i1 - 1; g0 += G) {
        const int kk = g0 + sub;
        const uint32_t hit = bits(kk < i1 - 1 && u0 < S_.ipool[kk] + S_.irho[kk]);
        if (hit) {
          k = g0 + __builtin_ctz(hit);
          break;
        }
      }
      w2 = k;
      w3 = i1;
      for (int i = i0 + sub; i < i1; i += G) {
        const int32_t a = S_.ia[i], r = S_.irho[i], pl0 = S_.ipool[i];
        if (LAYOUT) {
          const int32_t a0 = min(max(u0 - pl0, 0), r);
          const int32_t a1 = min(max(u1 - pl0, 0), r);
          S_.roff[i] = a1 - a0;
          S_.ro0[i] = S_.irow[i] + a + a0;
        }
        i32x4 ent;
        ent.x = S_.iphys[i];
        ent.y = S_.irow[i] + a - pl0;  // row = this + u
        ent.z = pl0 + r;                // end of the instance's pool range
        ent.w = 0;
        *reinterpret_cast<i32x4*>(S_.pi + 4 * i) = ent;
      }
    } else {
      // the first level whose F exceeds u0 (F grows with the level)
      int j = i1;
      for (int g0 = i0; g0 < i1; g0 += G) {
        const int jj = g0 + sub;
        const uint32_t hit = bits(jj < i1 && S_.fv[jj] > u0);
        if (hit) {
          j = g0 + __builtin_ctz(hit);
          break;
        }
      }
      const int32_t lam0 = j > i0 ? S_.lev[j - 1] : 0;
      const int32_t f0 = j > i0 ? S_.fv[j - 1] : 0;
      // the tile's first pool pair of e is round lam0 + q0, place r0 of the
      // phase; a later pool pair u of the tile is x = u - u0 + r0 places
      // further (x < kTile + 64, small enough for a float quotient)
      int n = 0, q0 = 0, r0 = 0;
      if (j < i1) {
        const int32_t a = max(S_.act[j], 1);
        q0 = (u0 - f0) / a;
        r0 = (u0 - f0) - q0 * a;
        for (int g0 = i0; g0 < i1; g0 += G) {
          const int i = g0 + sub;
          const bool take = i < i1 && S_.irho[i] > lam0;
          const uint32_t b = bits(take);
          if (take) {
            i32x2 ent;
            ent.x = S_.iphys[i] | (i << 16);
            ent.y = S_.irow[i] + S_.ia[i] + lam0 + q0;  // row = this + x / a
            *reinterpret_cast<i32x2*>(S_.al + 2 * (i0 + n + __builtin_popcount(b & below))) = ent;
          }
          n += __builtin_popcount(b);
        }
      }
      w2 = j < i1 ? S_.fv[j] - u0 + r0 : 0;  // x below this: in the phase
      w3 = i0 | (n << 16);
      w6 = u0 - r0;                           // u = x + this
      // the later phases the tile's pool pairs of e reach (up to the first
      // whose end is at or past u1): a header {x bound, x at the phase
      // start, instances | first entry << 8, rounds before the phase} and
      // the phase's instances in order, from the tile's pool
      if (sub == 0 && j < i1 && S_.fv[j] < u1) {
        int jl = j + 1;
        while (jl < i1 - 1 && S_.fv[jl] < u1) ++jl;
        const int nh = jl - j;
        int ne = 0;
        for (int jj = j + 1; jj <= jl; ++jj) ne += S_.act[jj];
        const int hb = atomicAdd(&S_.pcnt[0], nh);
        const int eb = atomicAdd(&S_.pcnt[1], ne);
        if (hb + nh <= kPhaseHeaders && eb + ne <= kPhaseEntries) {
          int ep = eb;
          for (int jj = j + 1; jj <= jl; ++jj) {
            const int32_t lamp = S_.lev[jj - 1];
            i32x4 h;
            h.x = S_.fv[jj] - w6;
            h.y = S_.fv[jj - 1] - w6;
            h.z = S_.act[jj] | (ep << 8);
            h.w = lamp;
            *reinterpret_cast<i32x4*>(S_.phdr + 4 * (hb + jj - j - 1)) = h;
            for (int i = i0; i < i1; ++i) {
              if (S_.irho[i] > lamp) {
                i32x2 ent;
                ent.x = S_.iphys[i] | (i << 16);
                ent.y = S_.irow[i] + S_.ia[i];
                *reinterpret_cast<i32x2*>(S_.pent + 2 * ep) = ent;
                ++ep;
              }
            }
          }
          w7 = hb | (nh << 16);
        }
      }
      if (LAYOUT) {
        int32_t tau0, s0, tau1, s1;
        interleave_round(S_, i0, i1, j, u0, &tau0, &s0);
        interleave_round(S_, i0, i1, j, u1, &tau1, &s1);
        int32_t p0 = 0, p1 = 0;  // instances before i still taking in round tau0 / tau1
        for (int g0 = i0; g0 < i1; g0 += G) {
          const int i = g0 + sub;
          const bool on = i < i1;
          const int32_t r = on ? S_.irho[i] : 0;
          const uint32_t b0 = bits(on && r > tau0), b1 = bits(on && r > tau1);
          if (on) {
            const int32_t c0 = p0 + __builtin_popcount(b0 & below), c1 = p1 + __builtin_popcount(b1 & below);
            const int32_t a0 = min(r, tau0) + (r > tau0 && c0 < s0 ? 1 : 0);
            const int32_t a1 = min(r, tau1) + (r > tau1 && c1 < s1 ? 1 : 0);
            S_.roff[i] = a1 - a0;
            S_.ro0[i] = S_.irow[i] + S_.ia[i] + a0;
          }
          p0 += __builtin_popcount(b0);
          p1 += __builtin_popcount(b1);
        }
      }
    }
    if (sub == 0) {
      i32x4 lo, hi;
      lo.x = aL;
      lo.y = pbase - aL - w6;  // u (contiguous) or x (interleave) = t + this
      lo.z = w2;
      lo.w = w3;
      hi.x = L >= 0 ? S_.iphys[L] : -1;
      hi.y = L >= 0 ? S_.irow[L] : 0;
      hi.z = w6;
      hi.w = w7;
      *reinterpret_cast<i32x4*>(rec) = lo;
      *reinterpret_cast<i32x4*>(rec + 4) = hi;
    }
  }
}

template <bool INTERLEAVE, bool LAYOUT, int W, bool GATHER = false>
__global__ __launch_bounds__(TileShape<W>::kThreads)
__attribute__((amdgpu_waves_per_eu(W == 16 ? 8 : 1))) void reroute_local_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ w, int32_t N, int32_t TK,
    int32_t tpr, int32_t E, int32_t M, int32_t S, int32_t ntiles,
    const int32_t* __restrict__ tile_base, const int32_t* __restrict__ plans, int32_t rec_words,
    int32_t off_iptr, int32_t off_iend, int32_t off_iphys, int32_t off_ibase, int32_t off_ilocal,
    int32_t n_inst, int32_t* __restrict__ phys_idx, int32_t* __restrict__ pos,
    int32_t* __restrict__ inv, float* __restrict__ w_perm) {
  constexpr bool gather_w = GATHER;
  using T = TileShape<W>;
  constexpr int NT = T::kThreads;
  extern __shared__ __align__(16) int32_t lds[];
  LocalLds S_;
  const int n4 = local_n4(n_inst);
  {
    // the record arrays first: every offset up to the per-instance arrays is
    // a multiple of four words, so the packed entries are 16-byte aligned
    int32_t* q = lds;
    S_.peers = reinterpret_cast<unsigned long long*>(q);
    S_.park = reinterpret_cast<uint32_t*>(q);
    S_.wst = reinterpret_cast<float*>(q);
    S_.sn = reinterpret_cast<uint16_t*>(q);
    q += reroute_shared_words(E, true, W);
    if (LAYOUT && !gather_w) {
      S_.sn = reinterpret_cast<uint16_t*>(q);
      q += kTile / 2;
    }
    S_.cntw = q; q += W * E;
    S_.er = q; q += kErWords * E;
    if (INTERLEAVE) {
      S_.phdr = q; q += 4 * kPhaseHeaders;
      S_.pent = q; q += 2 * kPhaseEntries;
      S_.pcnt = q; q += 4;
    }
    S_.al = q;
    S_.ipool = q; q += n4;
    S_.ie = q; q += n4;
    S_.pi = S_.ie;
    S_.lev = q; q += n4;
    S_.fv = q; q += n4;
    S_.act = q; q += n4;
    S_.iphys = q; q += n4;
    S_.irow = q; q += n4;
    S_.ia = q; q += n4;
    S_.irho = q; q += n4;
    S_.iptr = q; q += E + 1;
    if (LAYOUT) {
      S_.roff = q; q += n_inst + E + 1;
      S_.ro0 = q; q += n_inst + E;
    }
  }
  const int64_t blkid = xcd_block(blockIdx.x, gridDim.x);
  const int32_t layer = static_cast<int32_t>(blkid / ntiles);
  const int32_t tile = static_cast<int32_t>(blkid % ntiles);
  const int32_t src_rank = tile / tpr;
  const int32_t* plan = plans + static_cast<int64_t>(layer) * rec_words;
  const int64_t lb = static_cast<int64_t>(layer) * N;
  const TileSpan span = tile_span(layer, tile, N, TK, tpr);
  const int64_t first = span.first;
  const int n_here = span.n;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int base = wave * T::kWavePairs;
  const int32_t* tb = tile_base + (static_cast<int64_t>(layer) * ntiles + tile) * E;
  const int32_t* rb = tile_base + (static_cast<int64_t>(layer) * ntiles + src_rank * tpr) * E;
  const int PS = M + S;
  int32_t* er = S_.er;

  uint32_t v[T::kChunks];
  load_tile_ids(idx + first, base, n_here, lane, E, v);
  for (int i = threadIdx.x; i < W * (E + 1); i += NT) S_.peers[i] = 0;
  for (int i = threadIdx.x; i < W * E; i += NT) S_.cntw[i] = 0;
  for (int i = threadIdx.x; i <= E; i += NT) S_.iptr[i] = plan[off_iptr + i];
  if (INTERLEAVE && threadIdx.x < 4) S_.pcnt[threadIdx.x] = 0;
  for (int e = threadIdx.x; e < E; e += NT) {
    er[e * kErWords + kErCount] = tb[e];
    er[e * kErWords + kErBlk] = rb[e];
    er[e * kErWords + kErPool] = rb[e];
    er[e * kErWords + kErLoc] = -1;
  }
  for (int i = threadIdx.x; i < n_inst; i += NT) {
    S_.iphys[i] = plan[off_iphys + i];
    S_.irow[i] = plan[off_ibase + i];
    S_.ia[i] = plan[off_ilocal + i];
    S_.ipool[i] = plan[off_iend + i];
  }
  __syncthreads();

  // expert of each instance; pass 1: rank of each pair among the wave's
  // earlier pairs of its expert.  Afterwards v[c] holds the pair's expert id
  // (E for an invalid one) in its low 11 bits and its rank in the wave above
  // them (E <= 1024 and a wave's pairs number at most kTile).
  for (int e = threadIdx.x; e < E; e += NT)
    for (int i = S_.iptr[e]; i < S_.iptr[e + 1]; ++i) S_.ie[i] = e;
  int32_t* my = S_.cntw + wave * E;
  unsigned long long* mw = S_.peers + wave * (E + 1);
#pragma unroll
  for (int c = 0; c < T::kChunks; ++c) {
    const uint64_t peers = match_peers_lds(mw, v[c], lane);
    const bool valid = v[c] < static_cast<uint32_t>(E);
    const int32_t old = valid ? my[v[c]] : 0;
    if (lane == lowest_lane(peers)) {
      if (valid) my[v[c]] = old + __builtin_popcountll(peers);
      mw[v[c]] = 0;
    }
    const uint32_t lr = static_cast<uint32_t>(old + count_below(peers));
    v[c] = (lr << 11) | (valid ? v[c] : static_cast<uint32_t>(E));
  }
  __syncthreads();
  // the packed values wait out the set-up steps in the staging area (pass 1
  // is done with its lane masks; pass 2 reloads them before any staging),
  // so they hold no registers meanwhile
#pragma unroll
  for (int c = 0; c < T::kChunks; ++c) S_.park[c * NT + threadIdx.x] = v[c];

  // per instance: its first row and remaining quota; per expert: each
  // wave's first t and the tile's pairs of e
  const int n_used = S_.iptr[E];
  for (int i = threadIdx.x; i < n_used; i += NT) {
    const int e = S_.ie[i];
    const int32_t start = i > S_.iptr[e] ? S_.ipool[i - 1] : 0;
    S_.irow[i] += start;  // phys_off of the instance
    S_.irho[i] = S_.ipool[i] - start - S_.ia[i];
  }
  for (int e = threadIdx.x; e < E; e += NT) {
    const int32_t b0 = er[e * kErWords + kErCount] - er[e * kErWords + kErBlk];
    int32_t run = b0;
#pragma unroll
    for (int q = 0; q < W; ++q) {
      const int32_t x = S_.cntw[q * E + e];
      S_.cntw[q * E + e] = run;
      run += x;
    }
    er[e * kErWords + kErCount] = run - b0;
  }
  __syncthreads();

  // per instance: pool pairs before it (contiguous fill), the instance on
  // rank r and the local pairs of ranks before r, and the sorted interleave
  // tables
  for (int i = threadIdx.x; i < n_used; i += NT) {
    const int e = S_.ie[i];
    const int i0 = S_.iptr[e], i1 = S_.iptr[e + 1];
    if (!INTERLEAVE) {
      int32_t pool = 0;
      for (int j = i0; j < i; ++j) pool += S_.irho[j];
      S_.ipool[i] = pool;
    }
    const int h = S_.iphys[i] / PS;
    if (h == src_rank) er[e * kErWords + kErLoc] = i;
    // the last instance below rank r holds the local takes of ranks before r
    if (h < src_rank && (i + 1 == i1 || S_.iphys[i + 1] / PS >= src_rank)) {
      int32_t before = 0;
      for (int j = i0; j <= i; ++j) before += S_.ia[j];
      er[e * kErWords + kErPool] = er[e * kErWords + kErBlk] - before;
    }
    if (INTERLEAVE) {
      const int32_t rho = S_.irho[i];
      int ord = 0, ge = 0;
      int32_t f = 0;
      for (int j = i0; j < i1; ++j) {
        const int32_t x = S_.irho[j];
        ord += (x < rho || (x == rho && j < i)) ? 1 : 0;
        ge += x >= rho ? 1 : 0;
        f += min(x, rho);
      }
      S_.lev[i0 + ord] = rho;
      S_.fv[i0 + ord] = f;
      S_.act[i0 + ord] = ge;
    }
  }
  __syncthreads();

  // per expert: the tile's runs and the packed record of pass 2, several
  // lanes per expert (local_records)
  switch (records_lanes(E, NT)) {
    case 16: local_records<INTERLEAVE, LAYOUT, NT, 16>(S_, er, E, n_inst); break;
    case 8: local_records<INTERLEAVE, LAYOUT, NT, 8>(S_, er, E, n_inst); break;
    case 4: local_records<INTERLEAVE, LAYOUT, NT, 4>(S_, er, E, n_inst); break;
    case 2: local_records<INTERLEAVE, LAYOUT, NT, 2>(S_, er, E, n_inst); break;
    default: local_records<INTERLEAVE, LAYOUT, NT, 1>(S_, er, E, n_inst); break;
  }
  if (LAYOUT) {
    // instance entries beyond the plan's used ones are empty runs
    for (int i = n_used + threadIdx.x; i < n_inst; i += NT) {
      S_.roff[i] = 0;
      S_.ro0[i] = 0;
    }
    __syncthreads();
    if (wave == 0) wave_exclusive_scan<true>(S_.roff, n_inst + E);
    __syncthreads();
    for (int r = threadIdx.x; r < n_inst + E; r += NT) S_.ro0[r] = (S_.roff[r] & 0xFFFF) - S_.ro0[r];
  }
  __syncthreads();

#pragma unroll
  for (int c = 0; c < T::kChunks; ++c) v[c] = S_.park[c * NT + threadIdx.x];
  // each pair's routing weight, one coalesced load per chunk, issued here
  // so that they are in flight behind the LDS work of pass 2 (through one
  // buffer resource over the tile: one offset register for all chunks;
  // loads past the tile read 0 and are not used)
  float wl[LAYOUT ? T::kChunks : 1];
  if (LAYOUT && !gather_w) {
    const __amdgpu_buffer_rsrc_t r_w = row_rsrc(w + first, static_cast<uint32_t>(n_here) * 4u);
#pragma unroll
    for (int c = 0; c < T::kChunks; ++c)
      wl[c] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(r_w, (base + c * 64 + lane) * 4, 0, kNonTemporal));
  }
  __syncthreads();

  // pass 2: instance, physical expert and layout row of each pair.  The
  // tile's stretches of phys_idx and pos are written through buffer
  // resources sized to the tile (stores past it are dropped), which keeps
  // the eight chunks' addresses out of vector registers.  Interleaved pool
  // pairs past the tile's first phase of their expert are left to a second
  // loop, which keeps the rare paths out of the unrolled one.
  const __amdgpu_buffer_rsrc_t r_phys = row_rsrc(phys_idx + first, static_cast<uint32_t>(n_here) * 4u);
  const __amdgpu_buffer_rsrc_t r_pos = row_rsrc(pos + first, static_cast<uint32_t>(n_here) * 4u);
  uint32_t later = 0;
#pragma unroll
  for (int c = 0; c < T::kChunks; ++c) {
    const int i = base + c * 64 + lane;
    int32_t p = -1, row = -1;
    int run = -1;
    const int e = static_cast<int>(v[c] & 0x7FFu);
    if (e < E) {
      const int32_t t = my[e] + static_cast<int32_t>(v[c] >> 11);
      const i32x4 lo = *reinterpret_cast<const i32x4*>(er + e * kErWords);
      if (t < lo.x) {
        const i32x4 hi = *reinterpret_cast<const i32x4*>(er + e * kErWords + 4);
        p = hi.x;
        row = hi.y + t;
        run = n_inst + e;
      } else if (!INTERLEAVE) {
        const int32_t u = t + lo.y;
        int k = lo.z;
        while (k < lo.w - 1 && u >= S_.pi[4 * k + 2]) ++k;
        const i32x4 ent = *reinterpret_cast<const i32x4*>(S_.pi + 4 * k);
        p = ent.x;
        row = ent.y + u;
        run = k;
      } else {
        const int32_t x = t + lo.y;
        if (x < lo.z) {
          // the phase of the tile's first pool pair of e, as nearly always:
          // x / a from a float reciprocal (x < 2^14, a <= 64: the estimate
          // is within one of the quotient, and the remainder fixes it)
          const int32_t a = max(lo.w >> 16, 1);
          int32_t q = static_cast<int32_t>(static_cast<float>(x) *
                                           __builtin_amdgcn_rcpf(static_cast<float>(a)));
          int32_t r = x - q * a;
          if (r < 0) {
            --q;
            r += a;
          } else if (r >= a) {
            ++q;
            r -= a;
          }
          const i32x2 ent = *reinterpret_cast<const i32x2*>(S_.al + 2 * ((lo.w & 0xFFFF) + r));
          p = ent.x & 0xFFFF;
          row = ent.y + q;
          run = ent.x >> 16;
        } else {
          later |= 1u << c;
        }
      }
    }
    if (!(later >> c & 1u)) {
      if (LAYOUT && run >= 0) {
        const int32_t sl = row + S_.ro0[run];
        if (sl >= 0 && sl < kTile) {
          S_.sn[sl] = static_cast<uint16_t>(i);
          if (!gather_w) S_.wst[sl] = wl[c];
        }
      }
      __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(p), r_phys, i * 4, 0, kNonTemporal);
      __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(row), r_pos, i * 4, 0, kNonTemporal);
    }
  }
  if (INTERLEAVE && later != 0u) {
#pragma unroll
    for (int c = 0; c < T::kChunks; ++c) {
      if (later >> c & 1u) {
        const int i = base + c * 64 + lane;
        const int e = static_cast<int>(v[c] & 0x7FFu);
        const int32_t t = my[e] + static_cast<int32_t>(v[c] >> 11);
        const i32x4 lo = *reinterpret_cast<const i32x4*>(er + e * kErWords);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(er + e * kErWords + 4);
        const int32_t x = t + lo.y;
        int32_t p = -1, row = -1;
        int run = -1;
        if (hi.w >= 0) {
          // a later phase from the tile's pool: d = x - (x at its start) is
          // below kTile + 64 as well
          const int hb = hi.w & 0xFFFF, he = hb + (hi.w >> 16);
          for (int h = hb; h < he; ++h) {
            const i32x4 hd = *reinterpret_cast<const i32x4*>(S_.phdr + 4 * h);
            if (x < hd.x) {
              const int32_t a = max(hd.z & 0xFF, 1);
              const int32_t d = x - hd.y;
              int32_t q = static_cast<int32_t>(static_cast<float>(d) *
                                               __builtin_amdgcn_rcpf(static_cast<float>(a)));
              int32_t r = d - q * a;
              if (r < 0) {
                --q;
                r += a;
              } else if (r >= a) {
                ++q;
                r -= a;
              }
              const i32x2 ent = *reinterpret_cast<const i32x2*>(S_.pent + 2 * ((hd.z >> 8) + r));
              p = ent.x & 0xFFFF;
              row = ent.y + hd.w + q;
              run = ent.x >> 16;
              break;
            }
          }
        }
        if (run < 0) {
          // the general search (the tile's pool was full)
          const int i0 = lo.w & 0xFFFF, i1 = S_.iptr[e + 1];
          int32_t tau, s;
          interleave_round(S_, i0, i1, i0, x + hi.z, &tau, &s);
          int k = i1 - 1;
          for (int y = i0; y < i1; ++y) {
            if (S_.irho[y] > tau) {
              if (s == 0) {
                k = y;
                break;
              }
              --s;
            }
          }
          p = S_.iphys[k];
          row = S_.irow[k] + S_.ia[k] + tau;
          run = k;
        }
        if (LAYOUT) {
          const int32_t sl = row + S_.ro0[run];
          if (sl >= 0 && sl < kTile) {
            S_.sn[sl] = static_cast<uint16_t>(i);
            if (!gather_w) S_.wst[sl] = wl[c];
          }
        }
        __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(p), r_phys, i * 4, 0, kNonTemporal);
        __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(row), r_pos, i * 4, 0, kNonTemporal);
      }
    }
  }
  if (LAYOUT) {
    __syncthreads();
    // the staged slots in order: consecutive threads take consecutive slots,
    // which are consecutive layout rows inside each run.  A slot's run is
    // the q-th non-empty one, q + 1 being the run starts at or before it.
    // Pass 2 is done with the per-wave bases and the expert and instance
    // tables, so their words take the start bits of the slots (cleared, then
    // set by one atomic OR per non-empty run) and each non-empty run's
    // staging offset filed under q.  Then a wave's 64 slots are one aligned
    // block: q is the starts in the blocks before (each wave scans the
    // blocks' start counts itself, two blocks a lane) plus those in the
    // block up to the lane.  The checks only matter for a corrupted plan
    // record.
    constexpr int kPer = kTile / NT;
    static_assert(kTile / 64 == 128, "two 64-slot blocks per lane");
    const int nruns = n_inst + E;
    uint32_t* sbits = reinterpret_cast<uint32_t*>(local_wo_base(lds, E, n_inst, INTERLEAVE, W, gather_w));
    int32_t* nr = reinterpret_cast<int32_t*>(sbits) + kTile / 32;
    for (int d = threadIdx.x; d < kTile / 32; d += NT) sbits[d] = 0;
    for (int r = threadIdx.x; r < nruns; r += NT) {
      const int32_t r0 = S_.roff[r];
      const int q = r0 >> 16;
      if (((S_.roff[r + 1] - r0) & 0xFFFF) > 0 && q < nruns) nr[q] = S_.ro0[r];
    }
    __syncthreads();
    for (int r = threadIdx.x; r < nruns; r += NT) {
      const int32_t r0 = S_.roff[r];
      const int off = r0 & 0xFFFF;
      if (((S_.roff[r + 1] - r0) & 0xFFFF) > 0 && off < kTile) atomicOr(&sbits[off >> 5], 1u << (off & 31));
    }
    __syncthreads();
    const int nt = min(S_.roff[nruns] & 0xFFFF, n_here);
    const int32_t tile0 = span.tile0;
    const uint64_t upto = (2ull << lane) - 1;  // lanes 0..lane (all for lane 63)
    const unsigned long long* bits64 = reinterpret_cast<const unsigned long long*>(sbits);
    const int c0 = __builtin_popcountll(bits64[2 * lane]), c1 = __builtin_popcountll(bits64[2 * lane + 1]);
    const int incl = wave_inclusive_scan(c0 + c1);
    const int before_even = incl - c0 - c1, before_odd = incl - c1;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int j = u * NT + static_cast<int>(threadIdx.x);
      const int b = __builtin_amdgcn_readfirstlane(j >> 6);
      const int pb = static_cast<int>(readlane(static_cast<uint32_t>((b & 1) ? before_odd : before_even), b >> 1));
      if (j < nt) {
        const int q = min(pb + __builtin_popcountll(bits64[b] & upto) - 1, nruns - 1);
        const int n = S_.sn[j];
        const int32_t row = j - nr[q];
        if (n < n_here && row >= 0 && row < N) {
          inv[lb + row] = tile0 + n;
          w_perm[lb + row] = gather_w ? w[first + n] : S_.wst[j];
        }
      }
    }
  }
}

// ------------------------------------------------------------------------
// layout: inverse index and permuted weights
// ------------------------------------------------------------------------
__global__ __launch_bounds__(256) void layout_kernel(const int32_t* __restrict__ pos,
                                                     const float* __restrict__ w, int32_t L,
                                                     int32_t N, int32_t* __restrict__ inv,
                                                     float* __restrict__ w_perm) {
  // 64-bit index: N may come within a stride of 2^31
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int32_t layer = 0; layer < L; ++layer) {
    const int64_t lb = static_cast<int64_t>(layer) * N;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < N; i += stride) {
      const int32_t p = __builtin_nontemporal_load(pos + lb + i);
      const float wt = __builtin_nontemporal_load(w + lb + i);
      if (p >= 0 && p < N) {
        inv[lb + p] = static_cast<int32_t>(i);
        w_perm[lb + p] = wt;
      }
    }
  }
}

// ------------------------------------------------------------------------
// permute: bf16 rows into the layout order
// ------------------------------------------------------------------------
// One wave per 1 KiB chunk of an output row (64 lanes x one 16-byte vector):
// the row's source token is one uniform load, and the chunk moves with one
// load and one store per lane.  Every row is addressed through its own
// buffer resource whose size is the row's byte length, or 0 for a row that
// must be zero-filled: loads past the size return zeros and stores past it
// are dropped, so ragged row tails and invalid rows need no per-lane
// branches.  Loads and stores are non-temporal (each row is streamed once).
// Launch-shape sweeps on a full-size segment (H = 4096, 66,191 rows) put the
// 1 KiB chunk per wave first: 170 us of kernel time against 173 us for 2 KiB
// chunks (two rounds of one vector), 179 us for 2 KiB in one round, 183 us
// for 4 KiB, 185 us for the whole row per wave (four rounds of two vectors),
// 195 us for the whole row in one round, and 252 us for 512-byte chunks of
// 8-byte vectors.  A row's chunks are neighbouring waves, so the row's
// source bytes are requested together; many small independent streams keep
// more of HBM's channels busy than a few deep ones.
constexpr int kPermThreads = 256;
constexpr int kPermChunk = 64;  // 16-byte vectors per wave

__host__ __device__ inline int32_t perm_chunks(int32_t H8) { return (H8 + kPermChunk - 1) / kPermChunk; }

__device__ __forceinline__ int32_t perm_token(int32_t n, int32_t k, int64_t hidden_rows) {
  const int32_t t = n >= 0 ? n / k : -1;
  return t < hidden_rows ? t : -1;
}

__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t* __restrict__ phys_off, const int32_t* __restrict__ inv, int32_t k,
    const u32x4* __restrict__ hidden, int64_t hidden_rows, int32_t H8, int32_t p_begin,
    int32_t p_end, u32x4* __restrict__ out, int64_t cap) {
  const int32_t seg0 = phys_off[p_begin];
  const int64_t rows = min(static_cast<int64_t>(phys_off[p_end] - seg0), cap);
  const int lane = lane_id();
  const uint32_t rowb = static_cast<uint32_t>(H8) * 16u;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (kPermThreads / 64);
  const int32_t nch = perm_chunks(H8);
  // wave-uniform values go through readfirstlane so the buffer resources
  // built from them live in scalar registers
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  for (int64_t item = static_cast<int64_t>(blockIdx.x) * (kPermThreads / 64) + wv; item < rows * nch;
       item += nwaves) {
    const int64_t row = item / nch;
    const int32_t c0 = static_cast<int32_t>(item - row * nch) * kPermChunk;
    const int32_t t = __builtin_amdgcn_readfirstlane(perm_token(inv[seg0 + row], k, hidden_rows));
    const __amdgpu_buffer_rsrc_t src =
        row_rsrc(hidden + static_cast<int64_t>(t < 0 ? 0 : t) * H8, t < 0 ? 0u : rowb);
    const __amdgpu_buffer_rsrc_t dst = row_rsrc(out + row * H8, rowb);
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(src, (c0 + lane) * 16, 0, kNonTemporal);
    __builtin_amdgcn_raw_buffer_store_b128(x, dst, (c0 + lane) * 16, 0, kNonTemporal);
  }
}

// ------------------------------------------------------------------------
// fold: replica gradients into masters ([README] "Performance Tuning",
// "Expert communication": deterministic, non-atomic reduction)
// ------------------------------------------------------------------------
// blockIdx.y picks a slot of the range; only the lowest in-range slot of an
// expert does that expert's work, so each master is written by exactly one
// set of workgroups and the sum order (master, then slots ascending) is
// fixed.  blockIdx.x strides over the elements.
constexpr int kFoldThreads = 256;
constexpr int kFoldMaxReps = 64;
constexpr int kFoldVecs = 4;  // 16-byte vectors in flight per lane and stream
constexpr int kFoldScan = 4;  // 64-slot chunks of the range wave 0 loads at once
constexpr int kFoldPtrs = (ULTRAEP_MAX_EXPERTS + kFoldThreads - 1) / kFoldThreads;

__global__ __launch_bounds__(kFoldThreads) void fold_kernel(
    const int32_t* __restrict__ slot_expert, int32_t E, float* const* __restrict__ masters,
    const float* __restrict__ reps, int64_t numel, int32_t slot_begin, int32_t slot_end) {
  __shared__ int32_t s_list[kFoldMaxReps];
  __shared__ int32_t s_n;
  __shared__ float* s_mptr[ULTRAEP_MAX_EXPERTS];
  const int32_t s0 = slot_begin + static_cast<int32_t>(blockIdx.y);
  const int32_t nsl = slot_end - slot_begin;
  // The loads that wait on nothing go out first and together: this slot's
  // expert, the experts of the range's first slots (wave 0) and every master
  // pointer.  e's replicas in the range are the slots whose expert is e, in
  // ascending slot id (the order the fold sums them), so the list is one
  // ballot away and the master's address one LDS read, where a walk of e's
  // instances had cost two more dependent loads and the pointer one.
  const int32_t e = slot_expert[s0];
  int32_t se[kFoldScan];
  if (threadIdx.x < 64) {
#pragma unroll
    for (int c = 0; c < kFoldScan; ++c)
      se[c] = c * 64 < nsl ? slot_expert[slot_begin + min(c * 64 + static_cast<int32_t>(threadIdx.x), nsl - 1)] : -1;
  }
  float* mp[kFoldPtrs];
#pragma unroll
  for (int c = 0; c < kFoldPtrs; ++c)
    mp[c] = c * kFoldThreads < E ? masters[min(c * kFoldThreads + static_cast<int32_t>(threadIdx.x), E - 1)]
                                 : nullptr;
  if (e < 0 || e >= E) return;
  // Whenever this workgroup does e's work, its own slot s0 is the first
  // replica summed (the lowest of e's slots in the range), so the first
  // round of s0's gradient is loaded before the list is known: those loads
  // wait only on the slot's expert (an empty slot loads nothing).
  const int64_t n4 = numel / 4;
  const f32x4* r4 = reinterpret_cast<const f32x4*>(reps);
  const bool rvec = (numel % 4 == 0) && ((reinterpret_cast<uintptr_t>(reps) & 15) == 0);
  const int64_t span = static_cast<int64_t>(kFoldVecs) * kFoldThreads;
  const int64_t i00 = static_cast<int64_t>(blockIdx.x) * span + threadIdx.x;
  f32x4 g0[kFoldVecs], a0[kFoldVecs];
  if (rvec) {
    const f32x4* rq = r4 + static_cast<int64_t>(s0 - slot_begin) * n4;
#pragma unroll
    for (int u = 0; u < kFoldVecs; ++u) {
      const int64_t i = i00 + static_cast<int64_t>(u) * kFoldThreads;
      g0[u] = i < n4 ? __builtin_nontemporal_load(rq + i) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
#pragma unroll
  for (int c = 0; c < kFoldPtrs; ++c) {
    const int32_t x = c * kFoldThreads + static_cast<int32_t>(threadIdx.x);
    if (x < E) s_mptr[x] = mp[c];
  }
  if (threadIdx.x < 64) {
    // the range's slots of expert e, kept in order; the workgroups of the
    // lowest of them do e's work
    const int lane = threadIdx.x;
    int n = 0;
    bool first = true;
    for (int32_t b = 0; b < nsl; b += kFoldScan * 64) {
      if (b > 0) {
#pragma unroll
        for (int c = 0; c < kFoldScan; ++c)
          se[c] = b + c * 64 < nsl ? slot_expert[slot_begin + min(b + c * 64 + lane, nsl - 1)] : -1;
      }
#pragma unroll
      for (int c = 0; c < kFoldScan; ++c) {
        const int32_t i = b + c * 64 + lane;
        const int32_t s = (i < nsl && se[c] == e) ? i : -1;
        const uint64_t mk = ballot(s >= 0);
        if (n == 0 && mk != 0)
          first = static_cast<int32_t>(readlane(static_cast<uint32_t>(s), lowest_lane(mk))) == s0 - slot_begin;
        const int at = n + count_below(mk);
        if (s >= 0 && at < kFoldMaxReps) s_list[at] = s;
        n += __builtin_popcountll(mk);
      }
    }
    if (lane == 0) s_n = first ? n : 0;
  }
  __syncthreads();
  float* m = s_mptr[e];
  const bool vec = rvec && ((reinterpret_cast<uintptr_t>(m) & 15) == 0);
  if (vec && m != nullptr) {
    const f32x4* m4 = reinterpret_cast<const f32x4*>(m);
#pragma unroll
    for (int u = 0; u < kFoldVecs; ++u) {
      const int64_t i = i00 + static_cast<int64_t>(u) * kFoldThreads;
      a0[u] = i < n4 ? __builtin_nontemporal_load(m4 + i) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  const int n = min(s_n, kFoldMaxReps);
  if (n == 0 || m == nullptr) return;

  const int64_t tstride = static_cast<int64_t>(gridDim.x) * kFoldThreads;
  if (vec) {
    // each thread takes kFoldVecs 16-byte vectors a block-width apart, and
    // every load of a replica round is issued before any add or store (the
    // masters and the replica gradients are distinct buffers)
    // (rounds step by a workgroup-uniform base b0.  When the grid covers
    // the job in one round, the stores are written through at device
    // scope, from one buffer resource over the round's vectors (those past
    // the end are dropped), so little is left dirty in the L2s for the
    // write-back at the kernel's end: 1 us less at two 32 MiB masters.  With
    // more rounds per workgroup the same measured 2% slower than plain
    // non-temporal global stores, which those keep.)
    f32x4* m4 = reinterpret_cast<f32x4*>(m);
    const int64_t b00 = i00 - threadIdx.x;
    const int64_t step = static_cast<int64_t>(gridDim.x) * span;
    for (int64_t b0 = b00; b0 < n4; b0 += step) {
      const int64_t i0 = b0 + threadIdx.x;
      f32x4 acc[kFoldVecs];
      if (b0 == b00) {
#pragma unroll
        for (int u = 0; u < kFoldVecs; ++u) acc[u] = a0[u];
      } else {
#pragma unroll
        for (int u = 0; u < kFoldVecs; ++u) {
          const int64_t i = i0 + static_cast<int64_t>(u) * kFoldThreads;
          acc[u] = i < n4 ? __builtin_nontemporal_load(m4 + i) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      for (int q = 0; q < n; ++q) {
        f32x4 g[kFoldVecs];
        if (q == 0 && b0 == b00) {
          // s_list[0] is s0: its first round is already loaded
#pragma unroll
          for (int u = 0; u < kFoldVecs; ++u) g[u] = g0[u];
        } else {
          const f32x4* rq = r4 + static_cast<int64_t>(s_list[q]) * n4;
#pragma unroll
          for (int u = 0; u < kFoldVecs; ++u) {
            const int64_t i = i0 + static_cast<int64_t>(u) * kFoldThreads;
            g[u] = i < n4 ? __builtin_nontemporal_load(rq + i) : f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
#pragma unroll
        for (int u = 0; u < kFoldVecs; ++u) {
          acc[u].x += g[u].x;
          acc[u].y += g[u].y;
          acc[u].z += g[u].z;
          acc[u].w += g[u].w;
        }
      }
      if (step >= n4) {
        const __amdgpu_buffer_rsrc_t dst =
            row_rsrc(m4 + b0, static_cast<uint32_t>((n4 - b0 < span ? n4 - b0 : span) * 16));
#pragma unroll
        for (int u = 0; u < kFoldVecs; ++u)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[u]), dst,
                                                 (threadIdx.x + u * kFoldThreads) * 16, 0, kStreamStore);
      } else {
#pragma unroll
        for (int u = 0; u < kFoldVecs; ++u) {
          const int64_t i = i0 + static_cast<int64_t>(u) * kFoldThreads;
          if (i < n4) __builtin_nontemporal_store(acc[u], m4 + i);
        }
      }
    }
  } else {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kFoldThreads + threadIdx.x; i < numel;
         i += tstride) {
      float acc = m[i];
      for (int q = 0; q < n; ++q) acc += reps[static_cast<int64_t>(s_list[q]) * numel + i];
      m[i] = acc;
    }
  }
}

template <int MMAX, int SMAX>
hipError_t launch_plan_t(const PlanParams& pp, int32_t L, size_t lds, const uint16_t* hist,
                         int32_t* tbase, int32_t* plans, hipStream_t st) {
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&plan_kernel<MMAX, SMAX>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  const uint32_t grid = static_cast<uint32_t>(L) * static_cast<uint32_t>(1 + pp.scan_wgs);
  plan_kernel<MMAX, SMAX><<<dim3(grid), dim3(kPlanThreads), lds, st>>>(hist, tbase, plans, pp);
  return hipGetLastError();
}

template <int SMAX>
hipError_t launch_plan_m(int M, const PlanParams& pp, int32_t L, size_t lds, const uint16_t* hist,
                         int32_t* tbase, int32_t* plans, hipStream_t st) {
  if (M <= 2) return launch_plan_t<2, SMAX>(pp, L, lds, hist, tbase, plans, st);
  if (M <= 4) return launch_plan_t<4, SMAX>(pp, L, lds, hist, tbase, plans, st);
  if (M <= 8) return launch_plan_t<8, SMAX>(pp, L, lds, hist, tbase, plans, st);
  return launch_plan_t<16, SMAX>(pp, L, lds, hist, tbase, plans, st);
}

void plan_rounds(const Shape& sh, int32_t* G, int32_t* items) {
  const PlanRounds pr = plan_rounds_of(sh.ndom);
  *G = pr.G;
  *items = pr.items;
}

// Waves per reroute workgroup: the most whose per-wave grouping tables still
// fit one CU's LDS.  With 16 waves one workgroup fills a CU's four SIMDs four
// waves deep, which hides the LDS round trips of the per-pair passes.
constexpr size_t kLdsBytes = 160 * 1024;

int reroute_waves(const Shape& sh, bool layout) {
  for (int waves : {16, 8})
    if (reroute_lds_bytes(sh.E, sh.n_inst, layout, waves) <= kLdsBytes) return waves;
  return 4;
}

template <bool LAYOUT, int W>
hipError_t launch_reroute(const Shape& sh, int64_t blocks, const int32_t* idx, const float* w,
                          const Tiling& tl, const int32_t* tbase, const int32_t* plans,
                          int32_t* phys_idx, int32_t* pos, int32_t* inv, float* w_perm,
                          hipStream_t st) {
  const size_t rl = reroute_lds_bytes(sh.E, sh.n_inst, LAYOUT, W);
  const void* fn = reinterpret_cast<const void*>(&reroute_kernel<LAYOUT, W>);
  if (rl > 65536) {
    const hipError_t e =
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(rl));
    if (e != hipSuccess) return e;
  }
  reroute_kernel<LAYOUT, W><<<dim3(static_cast<uint32_t>(blocks)), dim3(TileShape<W>::kThreads),
                              rl, st>>>(
      idx, w, tl.N, tl.TK, tl.tpr, sh.E, tl.ntiles, tbase, plans, sh.lay.words, sh.lay.off[ULTRAEP_PLAN_INST_PTR],
      sh.lay.off[ULTRAEP_PLAN_INST_END], sh.lay.off[ULTRAEP_PLAN_INST_PHYS],
      sh.lay.off[ULTRAEP_PLAN_INST_BASE], sh.n_inst, phys_idx, pos, inv, w_perm);
  return hipGetLastError();
}

template <bool LAYOUT>
hipError_t launch_reroute_w(const Shape& sh, int64_t blocks, const int32_t* idx, const float* w,
                            const Tiling& tl, const int32_t* tbase,
                            const int32_t* plans, int32_t* phys_idx, int32_t* pos, int32_t* inv,
                            float* w_perm, hipStream_t st) {
  switch (reroute_waves(sh, LAYOUT)) {
    case 16:
      return launch_reroute<LAYOUT, 16>(sh, blocks, idx, w, tl, tbase, plans, phys_idx, pos,
                                        inv, w_perm, st);
    case 8:
      return launch_reroute<LAYOUT, 8>(sh, blocks, idx, w, tl, tbase, plans, phys_idx, pos,
                                       inv, w_perm, st);
    default:
      return launch_reroute<LAYOUT, 4>(sh, blocks, idx, w, tl, tbase, plans, phys_idx, pos,
                                       inv, w_perm, st);
  }
}

// Waves per locality workgroup, as for reroute_kernel; 0 when even four
// waves' tables do not fit (then the layout is left to layout_kernel).
int local_waves(const Shape& sh, bool layout) {
  for (int waves : {16, 8, 4})
    if (local_lds_bytes(sh.E, sh.n_inst, layout, true, waves) <= kLdsBytes) return waves;
  return 0;
}

// Two 16-wave workgroups share a CU when each needs at most this much LDS
// (measured: 77.4 KiB does, 78.6 KiB does not).
constexpr size_t kTwoPerCu = 78 * 1024;

// Gather the weights in the write-out only where that is what lets two
// workgroups share a CU; staged weights are cheaper otherwise.
bool local_gather(const Shape& sh, bool interleave) {
  return local_lds_bytes(sh.E, sh.n_inst, true, interleave, 16, false) > kTwoPerCu &&
         local_lds_bytes(sh.E, sh.n_inst, true, interleave, 16, true) <= kTwoPerCu;
}

template <bool INTERLEAVE, bool LAYOUT, int W, bool GATHER = false>
hipError_t launch_reroute_local_w(const Shape& sh, int64_t blocks, const int32_t* idx, const float* w,
                                  const Tiling& tl, const int32_t* tbase, const int32_t* plans,
                                  int32_t* phys_idx, int32_t* pos, int32_t* inv, float* w_perm,
                                  hipStream_t st) {
  const size_t rl = local_lds_bytes(sh.E, sh.n_inst, LAYOUT, INTERLEAVE, W, GATHER);
  const void* fn = reinterpret_cast<const void*>(&reroute_local_kernel<INTERLEAVE, LAYOUT, W, GATHER>);
  if (rl > 65536) {
    const hipError_t e =
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(rl));
    if (e != hipSuccess) return e;
  }
  reroute_local_kernel<INTERLEAVE, LAYOUT, W, GATHER>
      <<<dim3(static_cast<uint32_t>(blocks)), dim3(TileShape<W>::kThreads), rl, st>>>(
          idx, w, tl.N, tl.TK, tl.tpr, sh.E, sh.M, sh.S, tl.ntiles, tbase, plans, sh.lay.words,
          sh.lay.off[ULTRAEP_PLAN_INST_PTR], sh.lay.off[ULTRAEP_PLAN_INST_END],
          sh.lay.off[ULTRAEP_PLAN_INST_PHYS], sh.lay.off[ULTRAEP_PLAN_INST_BASE],
          sh.lay.off[ULTRAEP_PLAN_INST_LOCAL], sh.n_inst, phys_idx, pos, inv, w_perm);
  return hipGetLastError();
}

// With inv non-null the layout is fused; the caller checks that it fits.
template <bool INTERLEAVE, bool LAYOUT>
hipError_t launch_reroute_local(const Shape& sh, int64_t blocks, const int32_t* idx, const float* w,
                                const Tiling& tl, const int32_t* tbase, const int32_t* plans,
                                int32_t* phys_idx, int32_t* pos, int32_t* inv, float* w_perm,
                                hipStream_t st) {
  if (LAYOUT && local_gather(sh, INTERLEAVE))
    return launch_reroute_local_w<INTERLEAVE, LAYOUT, 16, true>(sh, blocks, idx, w, tl, tbase, plans,
                                                                phys_idx, pos, inv, w_perm, st);
  switch (local_waves(sh, LAYOUT)) {
    case 16:
      return launch_reroute_local_w<INTERLEAVE, LAYOUT, 16>(sh, blocks, idx, w, tl, tbase, plans,
                                                            phys_idx, pos, inv, w_perm, st);
    case 8:
      return launch_reroute_local_w<INTERLEAVE, LAYOUT, 8>(sh, blocks, idx, w, tl, tbase, plans,
                                                           phys_idx, pos, inv, w_perm, st);
    case 4:
      return launch_reroute_local_w<INTERLEAVE, LAYOUT, 4>(sh, blocks, idx, w, tl, tbase, plans,
                                                           phys_idx, pos, inv, w_perm, st);
    default:
      return hipErrorInvalidConfiguration;
  }
}

}  // namespace

size_t rerouting_lds_bytes(const Shape& sh, bool layout) {
  const size_t a = reroute_lds_bytes(sh.E, sh.n_inst, layout, reroute_waves(sh, layout));
  // the locality kernel without the layout always has a fitting shape when
  // this is within bounds; with it, it is used only where it fits
  const int lw = local_waves(sh, false);
  const size_t b = local_lds_bytes(sh.E, sh.n_inst, false, true, lw > 0 ? lw : 4);
  return a > b ? a : b;
}

size_t plan_lds_bytes(const Shape& sh) {
  int32_t G, items;
  plan_rounds(sh, &G, &items);
  return 4 * plan_lds_words(sh.E, sh.R, sh.S, sh.D, sh.P, sh.ndom, items);
}

hipError_t launch_balance(const Shape& sh, int32_t L, const int32_t* idx, const float* w,
                          int32_t TK, int32_t* ws, int32_t* plans, int32_t* phys_idx, int32_t* pos,
                          int32_t* inv, float* w_perm, hipStream_t st) {
  if (L <= 0) return hipSuccess;
  const int32_t N = sh.R * TK;
  const int32_t ntiles = static_cast<int32_t>(ntiles_of(sh.R, TK));
  const Tiling tl{N, TK, static_cast<int32_t>(tiles_per_rank(TK)), ntiles};
  const int64_t blocks = static_cast<int64_t>(L) * ntiles;
  // the 16-bit histograms take the first half of the histogram region
  uint16_t* hist = reinterpret_cast<uint16_t*>(ws);
  int32_t* tbase = ws + static_cast<int64_t>(L) * ntiles * sh.E;
  if (blocks > 0) {
    hipLaunchKernelGGL(count_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(CountTile::kThreads),
                       sizeof(int32_t) * kCountCopies * (sh.E + 1), st, idx, N, TK, tl.tpr, sh.E, ntiles,
                       hist);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  PlanParams pp{};
  pp.E = sh.E; pp.R = sh.R; pp.S = sh.S; pp.D = sh.D; pp.M = sh.M; pp.P = sh.P;
  pp.ndom = sh.ndom; pp.n_inst = sh.n_inst; pp.N = N; pp.ntiles = ntiles; pp.tpr = tl.tpr;
  pp.eps_num = sh.eps_num; pp.eps_den = sh.eps_den; pp.allow_zero = sh.allow_zero;
  pp.thr_num = sh.thr_num; pp.thr_den = sh.thr_den; pp.min_tokens = sh.min_tokens; pp.lean = sh.lean;
  pp.rec_words = sh.lay.words;
  plan_rounds(sh, &pp.G, &pp.items);
  {
    const PlanGrid g = plan_grid(sh.E, ntiles);
    pp.scan_ew = g.scan_ew;
    pp.scan_wgs = g.scan_wgs;
  }
  for (int f = 0; f < ULTRAEP_PLAN_NUM_FIELDS; ++f) {
    pp.off[f] = sh.lay.off[f];
    pp.len[f] = sh.lay.len[f];
  }
  const size_t lds = plan_lds_bytes(sh);
  hipError_t e;
  if (sh.S <= 2)
    e = launch_plan_m<2>(sh.M, pp, L, lds, hist, tbase, plans, st);
  else if (sh.S <= 4)
    e = launch_plan_m<4>(sh.M, pp, L, lds, hist, tbase, plans, st);
  else
    e = launch_plan_m<8>(sh.M, pp, L, lds, hist, tbase, plans, st);
  if (e != hipSuccess) return e;
  if (blocks > 0) {
    if (sh.reroute_mode != ULTRAEP_REROUTE_RANGES) {
      const bool il = sh.reroute_mode == ULTRAEP_REROUTE_INTERLEAVE;
      if (inv != nullptr && local_waves(sh, true) > 0) {
        e = il ? launch_reroute_local<true, true>(sh, blocks, idx, w, tl, tbase, plans, phys_idx,
                                                  pos, inv, w_perm, st)
               : launch_reroute_local<false, true>(sh, blocks, idx, w, tl, tbase, plans, phys_idx,
                                                   pos, inv, w_perm, st);
      } else {
        e = il ? launch_reroute_local<true, false>(sh, blocks, idx, w, tl, tbase, plans, phys_idx,
                                                   pos, nullptr, nullptr, st)
               : launch_reroute_local<false, false>(sh, blocks, idx, w, tl, tbase, plans, phys_idx,
                                                    pos, nullptr, nullptr, st);
        if (e == hipSuccess && inv != nullptr) e = launch_layout(L, N, pos, w, inv, w_perm, st);
      }
    } else if (inv != nullptr) {
      e = launch_reroute_w<true>(sh, blocks, idx, w, tl, tbase, plans, phys_idx, pos, inv,
                                 w_perm, st);
    } else {
      e = launch_reroute_w<false>(sh, blocks, idx, w, tl, tbase, plans, phys_idx, pos,
                                  nullptr, nullptr, st);
    }
  }
  return e;
}

hipError_t launch_layout(int32_t L, int32_t N, const int32_t* pos, const float* w, int32_t* inv,
                         float* w_perm, hipStream_t st) {
  const int64_t total = static_cast<int64_t>(L) * N;
  if (total <= 0) return hipSuccess;
  const int64_t want = (static_cast<int64_t>(N) + 255) / 256;
  const uint32_t blocks = static_cast<uint32_t>(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(layout_kernel, dim3(blocks), dim3(256), 0, st, pos, w, L, N, inv, w_perm);
  return hipGetLastError();
}

hipError_t launch_permute(const Shape& sh, const int32_t* plan, const int32_t* inv, int32_t k,
                          const uint16_t* hidden, int64_t hidden_rows, int32_t H, int32_t p_begin,
                          int32_t p_end, uint16_t* out, int64_t cap, hipStream_t st) {
  if (cap <= 0 || p_begin == p_end) return hipSuccess;
  const int64_t want = (cap * perm_chunks(H / 8) + kPermThreads / 64 - 1) / (kPermThreads / 64);  // one chunk per wave
  const uint32_t blocks = static_cast<uint32_t>(want < (1 << 20) ? want : (1 << 20));
  hipLaunchKernelGGL(permute_kernel, dim3(blocks), dim3(kPermThreads), 0, st,
                     plan + sh.lay.off[ULTRAEP_PLAN_PHYS_OFF], inv, k,
                     reinterpret_cast<const u32x4*>(hidden), hidden_rows, H / 8, p_begin, p_end,
                     reinterpret_cast<u32x4*>(out), cap);
  return hipGetLastError();
}

hipError_t launch_fold(const Shape& sh, const int32_t* plan, float* const* masters,
                       const float* reps, int64_t numel, int32_t slot_begin, int32_t slot_end,
                       hipStream_t st) {
  const int32_t nslots = slot_end - slot_begin;
  if (nslots <= 0 || numel <= 0) return hipSuccess;
  const int64_t per_block = static_cast<int64_t>(kFoldThreads) * 4 * kFoldVecs;
  const int64_t want = (numel + per_block - 1) / per_block;
  const uint32_t bx = static_cast<uint32_t>(want < 2048 ? want : 2048);
  hipLaunchKernelGGL(fold_kernel, dim3(bx, static_cast<uint32_t>(nslots)), dim3(kFoldThreads), 0, st,
                     plan + sh.lay.off[ULTRAEP_PLAN_SLOT_EXPERT], sh.E, masters, reps, numel, slot_begin,
                     slot_end);
  return hipGetLastError();
}

}  // namespace ultraep

/*
 * ultraep.h -- C ABI of the MI355X (gfx950) exact-load expert rebalancing path.
 *
 * One call sequence per MoE layer and microbatch, after gating:
 *
 *   ultraep_balance          count the exact load per expert, solve the quota
 *                            plan, and give every (token, k) pair its replica
 *                            and its row in the replica-contiguous layout
 *   ultraep_balance_static   the same without a caller workspace (for callers
 *                            that cannot allocate)
 *   ultraep_dispatch_layout  the layout's inverse index and permuted weights
 *   ultraep_permute          gather bf16 hidden rows into the layout
 *   ultraep_combine          after the experts: each token's k output rows,
 *                            weighted, back to the token (unweighted: the
 *                            backward of ultraep_permute)
 *   ultraep_combine_backward gradients of combine: expert-output rows and the
 *                            routing weights in logical (token, k) order
 *   ultraep_weight_sync_plan the relay schedule of the master -> replica copies
 *   ultraep_weight_sync      copy master weights into the replica slots
 *   ultraep_fold_grads       fold replica gradients back into their masters
 *
 * Sources, cited by page title and section:
 *   [README]  "UltraEP" project README (mirror kd.iw.mk/studio-dots-ai/UltraEP)
 *   [NEWS]    "Xiaohongshu's UltraEP Balances MoE Experts in 300 µs, Reaching
 *             94.3% of Ideal" (news.hamidun.com)
 *   [WEEKLY]  "UltraEP: Real-Time Load Balancing for Large-Scale MoE Training
 *             and Inference" (aikit weekly)
 *
 * Conventions (all calls):
 *   - R logical EP ranks with T tokens each; token g = r*T + t (rank-major).
 *     top-k routing is int32 topk_idx[L][R*T][k]; pair n = g*k + j, N = R*T*k
 *     pairs per layer (N < 2^31).  Ids outside [0, E) are dropped pairs.
 *   - E experts, M = E/R masters per rank; expert e lives on rank e / M.
 *   - S redundant slots per rank ([README] Interface, "Initialization": every
 *     rank reserves the same number of redundant-expert slots); slot id
 *     s = r*S + j.  Replicas stay within a scale-up domain of D consecutive
 *     ranks ([README] principles, "Topology-aware replication").
 *   - Physical experts P = R*(M+S), rank-major: p = r*(M+S) + j; j < M is the
 *     master of expert r*M + j, j >= M is slot j-M of rank r.  A rank's
 *     physical experts [r*(M+S), (r+1)*(M+S)) are its receive segment.
 *   - Load is counted in pairs.
 *   - Device pointers are caller-owned (any device allocator); the library
 *     allocates no device memory and keeps no device state ([README]
 *     principles: no dynamic allocation at runtime), except the fixed static
 *     workspace of ultraep_balance_static.  The context is host
 *     memory, immutable after create, usable from several streams at once
 *     as long as each call gets its own workspace and outputs.
 *   - Every call is ordered on the given stream (a hipStream_t passed as
 *     void*, NULL = the null stream), never synchronises the host, and reads
 *     data-dependent sizes from the device plan, so the sequence can be
 *     captured in a HIP graph ([README] design principles: graph capture
 *     is supported).
 *   - Return value: ULTRAEP_OK or a negative status (below).  Argument checks
 *     happen on the host before anything is launched; on error nothing is
 *     launched and outputs are untouched.  Data-dependent conditions that
 *     cannot be reported synchronously are recorded in the plan header.
 */
#ifndef ULTRAEP_H
#define ULTRAEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define ULTRAEP_OK 0
#define ULTRAEP_EINVAL (-1)       /* bad argument: shape rules, null pointer, range */
#define ULTRAEP_EUNSUPPORTED (-2) /* legal but beyond this build's limits or alignment */
#define ULTRAEP_ELAUNCH (-3)      /* a HIP launch or runtime call failed */
#define ULTRAEP_EWORKSPACE (-4)   /* workspace smaller than ultraep_workspace_bytes */
#define ULTRAEP_ESCRATCH (-5)     /* ultraep_balance_static: more than the static workspace */

/* Limits of this build. */
#define ULTRAEP_MAX_EXPERTS 1024      /* E */
#define ULTRAEP_MAX_MASTERS 16        /* M = E/R */
#define ULTRAEP_MAX_SLOTS 8           /* S */
#define ULTRAEP_MAX_DOMAIN 64         /* D: one rank per lane of a wave64 */
#define ULTRAEP_MAX_TOTAL_SLOTS 1024  /* R*S */
#define ULTRAEP_MAX_TOPK 64           /* k */

typedef struct ultraep_ctx ultraep_ctx;

/* Planning options ([README] "Performance Tuning", "Replication planning").
 * eps_num/eps_den: the balancing tolerance eps (default 1/100, the pages'
 *   default 0.01).  The quota grid steps by floor(total*eps/R), at least 1.
 * allow_zero_master: 0 (default) = a master with load keeps at least one
 *   pair; 1 = a master may give all of its load to replicas.
 * threshold_num/threshold_den: the early-stop target of the balancing search
 *   (the pages' default 1.0; 0/0 means 1/1), read as the lowest max/mean the
 *   plan aims at: the quota grid starts at min(max(ceil(total * threshold /
 *   R), domain floor), max home load).  Must be >= 1 (num >= den >= 1) and
 *   at most 64.
 * reroute_mode: which pairs an instance serves ([README] "Replication
 *   planning": locality-aware per-rank quota decomposition; reroute
 *   interleave).  ULTRAEP_REROUTE_RANGES (0, default): instance i of an
 *   expert serves the contiguous range [start_i, end_i) of the expert's
 *   pairs in pair order.  ULTRAEP_REROUTE_LOCAL (1): instance i first
 *   serves the first INST_LOCAL[i] pairs of its expert whose tokens live on
 *   its own rank; the expert's other pairs, in pair order, fill the
 *   instances' remaining quotas contiguously in instance order.
 *   ULTRAEP_REROUTE_INTERLEAVE (2): as LOCAL, but the remaining pairs are
 *   dealt round by round: in round t every instance with more than t pairs
 *   still to take gets the next one, in instance order.  In modes 1 and 2 an
 *   instance's layout rows hold its local pairs (pair order), then the rest
 *   (in the order dealt), and a fused layout is written by a scatter pass.
 * min_tokens_per_replica ([README] "Replication planning": the minimal load
 *   allocated to a replica; 0 means 1): m, a rule of the greedy (step 3 of
 *   ultraep_balance), so every replica serves at least m pairs and every
 *   rank still ends at Q* or below.  Every amount the greedy moves is at
 *   least m: a shed piece below m is raised to m when its expert has room
 *   for m (the rank then ends below Q) and is not shed when it has not;
 *   only receivers with spare >= m and donors with room >= m more take part
 *   of a piece; a split leaves at least m queued (the roomiest receiver
 *   takes min(spare, piece - m), skipped in a chain when below m; the
 *   donor's part is cut so that 0 or at least m stays queued); a placement
 *   below m fails the probe.  m = 1 is the plain greedy.
 * replica_lean (the pages' EP64 table, [README] "Tests", reaches max/mean
 *   1.01 with few replicas; their planner's rule is not given): 1 plans
 *   without the chain step of the greedy (step 3 of ultraep_balance): only
 *   ranks with spare take replicas, a piece that fits no receiver goes in
 *   part to the roomiest one and the rest is queued again.  On large domains
 *   this needs about a third fewer replicas at the same quota; small domains
 *   may need a higher quota.  0 (default) keeps the chain. */
#define ULTRAEP_REROUTE_RANGES 0
#define ULTRAEP_REROUTE_LOCAL 1
#define ULTRAEP_REROUTE_INTERLEAVE 2
typedef struct ultraep_options {
  int32_t eps_num;
  int32_t eps_den;
  int32_t allow_zero_master;
  int32_t threshold_num;
  int32_t threshold_den;
  int32_t reroute_mode;
  int32_t min_tokens_per_replica;
  int32_t replica_lean; /* 0 (default) or 1 */
} ultraep_options;

/* Weight-distribution plan of ultraep_weight_sync_plan ([README]
 * "Performance Tuning", "Expert communication": the plan mode is direct,
 * adaptive or forced relay; adaptive relay needs a minimum replica count per
 * expert and a minimum fan-out gain and uses at most a maximum number of
 * relays; plans are direct when the scale-up domain has at most 8 GPUs).
 * NULL options mean: adaptive, min_replicas 4, max_relays 8, min_gain 2,
 * domain_gpus = D. */
#define ULTRAEP_RELAY_DIRECT 0
#define ULTRAEP_RELAY_ADAPTIVE 1
#define ULTRAEP_RELAY_FORCE 2
typedef struct ultraep_relay_options {
  int32_t mode;         /* ULTRAEP_RELAY_* */
  int32_t min_replicas; /* adaptive: relay only experts with at least this many replicas */
  int32_t max_relays;   /* at most this many relays per expert (>= 1 to relay at all) */
  int32_t min_gain;     /* adaptive: relay only if replicas >= min_gain * relayed fan-out */
  int32_t domain_gpus;  /* GPUs of the scale-up domain; <= 8 forces direct */
  int32_t reserved[3];  /* must be zero */
} ultraep_relay_options;

/* Create a planning context for E experts over R ranks with S redundant slots
 * per rank and scale-up domains of D ranks ([README] Interface,
 * "Initialization": one manager per EP group with a fixed number of
 * redundant slots per rank).
 * Rules: E % R == 0, R % D == 0, 1 <= E <= ULTRAEP_MAX_EXPERTS,
 * E/R <= ULTRAEP_MAX_MASTERS, 0 <= S <= ULTRAEP_MAX_SLOTS,
 * 1 <= D <= ULTRAEP_MAX_DOMAIN, R*S <= ULTRAEP_MAX_TOTAL_SLOTS (EINVAL for a
 * broken rule, EUNSUPPORTED beyond a limit).  Within these limits every
 * kernel's per-workgroup tables fit one CU's 160 KiB of LDS; the check is
 * still made and fails with EUNSUPPORTED.
 * opt may be NULL (defaults).  *out receives a host object the caller frees
 * with ultraep_destroy.  No HIP call is made. */
int ultraep_create(int32_t E, int32_t R, int32_t slots_per_rank, int32_t D,
                   const ultraep_options* opt, ultraep_ctx** out);

/* Free a context (NULL is accepted). */
int ultraep_destroy(ultraep_ctx* ctx);

/* Bytes of one layer's plan record (a multiple of 256).  Plan records of L
 * layers are laid out back to back.  The record is int32 words; the offset
 * and length of each field are given by ultraep_plan_field. */
int ultraep_plan_bytes(const ultraep_ctx* ctx, size_t* out);

/* Plan record fields.  All int32. */
enum ultraep_plan_field_id {
  ULTRAEP_PLAN_HEADER = 0,       /* [64] see ULTRAEP_HDR_* */
  ULTRAEP_PLAN_COUNTS = 1,       /* [E] pairs routed to each expert */
  ULTRAEP_PLAN_MASTER_QUOTA = 2, /* [E] pairs the master keeps */
  ULTRAEP_PLAN_SLOT_EXPERT = 3,  /* [R*S] expert replicated into slot s, -1 = empty */
  ULTRAEP_PLAN_SLOT_QUOTA = 4,   /* [R*S] pairs served by slot s (0 if empty) */
  ULTRAEP_PLAN_PHYS_LOAD = 5,    /* [P] pairs per physical expert */
  ULTRAEP_PLAN_PHYS_OFF = 6,     /* [P+1] exclusive prefix of PHYS_LOAD: layout rows */
  ULTRAEP_PLAN_INST_PTR = 7,     /* [E+1] CSR: expert e's instances are [ptr[e], ptr[e+1]) */
  ULTRAEP_PLAN_INST_PHYS = 8,    /* [E+R*S] physical id of each instance, ascending per expert */
  ULTRAEP_PLAN_INST_END = 9,     /* [E+R*S] cumulative end of the instance's ordinal range */
  ULTRAEP_PLAN_INST_BASE = 10,   /* [E+R*S] layout row of ordinal o is INST_BASE + o */
  ULTRAEP_PLAN_RANK_BEFORE = 11, /* [R] home load before balancing */
  ULTRAEP_PLAN_RANK_AFTER = 12,  /* [R] load after balancing */
  ULTRAEP_PLAN_INST_LOCAL = 13,  /* [E+R*S] pairs the instance takes from its own rank's tokens:
                                    min(its quota, pairs of its expert from its host rank) */
  ULTRAEP_PLAN_NUM_FIELDS = 14
};

/* Header words (ULTRAEP_PLAN_HEADER). */
enum ultraep_header_word {
  ULTRAEP_HDR_MAGIC = 0,      /* 0x55455031 */
  ULTRAEP_HDR_E = 1,
  ULTRAEP_HDR_R = 2,
  ULTRAEP_HDR_S = 3,
  ULTRAEP_HDR_D = 4,
  ULTRAEP_HDR_M = 5,
  ULTRAEP_HDR_P = 6,
  ULTRAEP_HDR_N = 7,          /* pairs in the layer */
  ULTRAEP_HDR_TOTAL = 8,      /* valid pairs = layout rows */
  ULTRAEP_HDR_DROPPED = 9,    /* pairs with an id outside [0, E) */
  ULTRAEP_HDR_Q_STAR = 10,    /* the quota the plan reached (max rank load) */
  ULTRAEP_HDR_Q_LB = 11,      /* first grid quota */
  ULTRAEP_HDR_Q_MAX = 12,     /* max home load (always reachable) */
  ULTRAEP_HDR_TOL = 13,       /* grid step */
  ULTRAEP_HDR_GRID_INDEX = 14,/* index of Q_STAR on the grid */
  ULTRAEP_HDR_FLOOR = 15,     /* max over domains of ceil(domain load / D) */
  ULTRAEP_HDR_REPLICAS = 16,  /* filled slots */
  ULTRAEP_HDR_ROUNDS = 17,    /* probe rounds the device solver ran (diagnostic only) */
  ULTRAEP_HDR_WORDS = 64
};

#define ULTRAEP_PLAN_MAGIC 0x55455031

/* Offset (bytes from the start of a record) and element count of a field. */
int ultraep_plan_field(const ultraep_ctx* ctx, int32_t field, size_t* offset_bytes, size_t* count);

/* Workspace bytes ultraep_balance needs for L layers of R*T*k pairs (per-tile
 * expert histograms and per-tile ordinal bases).  The workspace is scratch:
 * nothing in it must be initialised, and ultraep_balance leaves in it nothing
 * the other calls read. */
int ultraep_workspace_bytes(const ultraep_ctx* ctx, int32_t L, int64_t T, int32_t k, size_t* out);

/* Balance L layers ([README] Interface, "Forward and backward":
 * update_placement plans from the exact post-gating load, reroute expands
 * logical routing to physical replicas; [NEWS] "How balancing in 300
 * microseconds works": a quota-driven scheduler right after gating).
 *
 * In:  topk_idx  int32 [L][R*T][k]
 *      topk_w    fp32  [L][R*T][k] routing weights, or NULL (see layout below)
 * Out: plans     L plan records (ultraep_plan_bytes each)
 *      phys_idx  int32 [L][N]  physical expert of each pair, -1 if dropped
 *      pos       int32 [L][N]  layout row of each pair, -1 if dropped
 *      inv       int32 [L][N]  optional: inv[pos[n]] = n         } the dispatch
 *      w_perm    fp32  [L][N]  optional: w_perm[pos[n]] = w[n]   } layout
 * topk_w, inv and w_perm are given together or all NULL.  Given, the layout
 * is written by the same kernel that reroutes (rows [0, total) of each layer;
 * ultraep_dispatch_layout computes the same from pos separately).
 *
 * Per layer:
 *  1. c[e] = number of pairs with id e.
 *  2. Quota grid: Q_lb = max over domains of ceil(domain load / D) (never
 *     below ceil(total * threshold / R), never above Q_max), step
 *     tol = max(1, floor(total*eps/R)), up to the max home load Q_max;
 *     Q* = the first grid quota the greedy reaches.
 *  3. The greedy, per domain: ranks above Q shed their excess from their
 *     hottest experts first (pairs desc, id asc), each master keeping one
 *     pair unless allow_zero_master; the largest shed piece (ties: lower id)
 *     goes whole to the tightest receiver that fits (least spare, then lowest
 *     rank); if none fits and another shedding rank could host it, the
 *     roomiest receiver is filled and the rest is swapped onto that rank,
 *     which sheds as much more of its own largest queued expert (ties: lower
 *     id); otherwise the roomiest receiver (most spare, then lowest rank) is
 *     filled and the rest queued.  A receiver needs a free slot and must not
 *     already host the expert.  Slot index = arrival order on the rank.
 *  4. Instances of expert e: its master and replicas in ascending physical
 *     id; instance i serves ordinals [start_i, end_i) where ordinal o(n) is
 *     the number of earlier pairs (lower n) with the same expert.
 *  5. phys_idx[n] = the instance's physical id; pos[n] = phys_off[p] +
 *     o(n) - start_i.  So the layout lists pairs by (physical expert, n).
 * The result is deterministic and identical on every run.
 *
 * Errors: EINVAL for null pointers (when L*N > 0), only some of topk_w /
 * inv / w_perm given, L < 0, T < 0, k outside [1, min(E, ULTRAEP_MAX_TOPK)];
 * EUNSUPPORTED when N >= 2^31 or a pointer is not 4-byte aligned;
 * EWORKSPACE when workspace_bytes is short. */
int ultraep_balance(const ultraep_ctx* ctx, int32_t L, const int32_t* topk_idx,
                    const float* topk_w, int64_t T, int32_t k, void* workspace,
                    size_t workspace_bytes, void* plans, int32_t* phys_idx, int32_t* pos,
                    int32_t* inv, float* w_perm, void* stream);

/* Allocation-free ultraep_balance, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments (less the workspace), results and errors
 * as ultraep_balance; the workspace is a static device buffer of
 * ULTRAEP_STATIC_WORKSPACE_BYTES that every device the library runs on holds
 * from the time the library's code is loaded there until the process ends.
 * Its device address is looked up once per device, on the first call with
 * that device current; the call runs on the device current on the calling
 * thread, and the stream must belong to it.
 * Limit: ultraep_workspace_bytes(L, T, k) must not exceed
 * ULTRAEP_STATIC_WORKSPACE_BYTES (32 MiB: e.g. 64 layers of the E = 128,
 * R = 64, 8192 x top-8 shape, or 61 layers of E = 256, R = 64, 4096 x
 * top-8); a larger call fails with ULTRAEP_ESCRATCH before anything is
 * launched.
 * Sharing: all calls on one device use the same buffer, which keeps the last
 * call's contents (nothing in it needs clearing: a call reads only words it
 * wrote itself).  Two calls that overlap in time on one device race (two
 * streams, or two host threads without ordering between them); order them
 * on one stream.  No hipMalloc, hipFree or other allocating call is made. */
#define ULTRAEP_STATIC_WORKSPACE_BYTES (32u << 20)
int ultraep_balance_static(const ultraep_ctx* ctx, int32_t L, const int32_t* topk_idx,
                           const float* topk_w, int64_t T, int32_t k, void* plans,
                           int32_t* phys_idx, int32_t* pos, int32_t* inv, float* w_perm,
                           void* stream);

/* Inverse index and permuted routing weights of the dispatch layout
 * ([README] Interface, "Forward and backward": tokens are dispatched to the
 * physical experts that reroute produced).
 * In:  pos [L][N] from ultraep_balance, topk_w fp32 [L][R*T][k]
 * Out: inv [L][N]: inv[pos[n]] = n;  w_perm [L][N]: w_perm[pos[n]] = topk_w[n].
 * Only rows [0, total) of each layer are written (total is in the plan
 * header); pos entries outside [0, N) are ignored.
 * Errors: EINVAL (null pointers with L*N > 0, L < 0, T < 0, bad k),
 * EUNSUPPORTED (N >= 2^31, pointers not 4-byte aligned). */
int ultraep_dispatch_layout(const ultraep_ctx* ctx, int32_t L, int64_t T, int32_t k,
                            const int32_t* pos, const float* topk_w, int32_t* inv,
                            float* w_perm, void* stream);

/* Gather the bf16 hidden rows of physical experts [p_begin, p_end) of one
 * layer into the layout order (one rank's receive segment when the range is
 * [r*(M+S), (r+1)*(M+S))): the one-GPU form of the dispatch that follows
 * reroute ([README] Interface, "Forward and backward": the tokens are
 * dispatched to the physical experts reroute chose, before the grouped
 * expert GEMM; principles, "Self-contained codebase": UltraEP itself is
 * independent of the token dispatcher, so this build supplies the row
 * movement the dispatch needs).
 * In:  plan (one record), inv [N] of that layer, hidden [hidden_rows][H] bf16
 *      (raw 16-bit patterns, never converted)
 * Out: out [rows][H] with rows = phys_off[p_end] - phys_off[p_begin]; row i is
 *      hidden[inv[phys_off[p_begin] + i] / k].  Rows at or beyond
 *      out_capacity_rows are not written (the caller sizes out from the plan
 *      or from a bound); a row whose inv entry is negative or names a token
 *      at or beyond hidden_rows is written as zeros.
 * Errors: EINVAL (null pointers, H <= 0, k outside [1, 64], bad range
 *      0 <= p_begin <= p_end <= P, out_capacity_rows < 0); EUNSUPPORTED
 *      (H % 8 != 0 or hidden/out not 16-byte aligned: rows move as 16-byte
 *      vectors). */
int ultraep_permute(const ultraep_ctx* ctx, const void* plan, const int32_t* inv, int32_t k,
                    const uint16_t* hidden, int64_t hidden_rows, int32_t H, int32_t p_begin,
                    int32_t p_end, uint16_t* out, int64_t out_capacity_rows, void* stream);

/* Fold replica gradients into their masters ([README] Interface, "Forward and
 * backward": grad_reduce reduces replica weight gradients into the master
 * experts' gradients; "Performance Tuning", "Expert communication":
 * deterministic, non-atomic reduction).
 * For every expert e with a replica in slots [slot_begin, slot_end):
 *   master_grads[e][i] += the replicas' grads, added one after another in
 *   fp32 in ascending slot order.
 * In:  plan (one record); master_grads: DEVICE array of E device pointers
 *      (entries of experts without a replica in the range may be NULL; a NULL
 *      entry of a touched expert is skipped); replica_grads fp32
 *      [slot_end - slot_begin][numel], slot s at row s - slot_begin.
 * Out: the touched masters, in place.  Masters may not alias replica_grads.
 * Errors: EINVAL (null pointers, numel < 0, bad slot range
 *      0 <= slot_begin <= slot_end <= R*S).  Any alignment works; 16-byte
 *      aligned buffers with numel % 4 == 0 take the vector path. */
int ultraep_fold_grads(const ultraep_ctx* ctx, const void* plan, float* const* master_grads,
                       const float* replica_grads, int64_t numel, int32_t slot_begin,
                       int32_t slot_end, void* stream);

/* Combine: bring each token's k expert outputs back to the token, weighted
 * by its routing weights ([README] Interface, "Forward and backward": the
 * experts run on the dispatched rows, then combine returns their outputs to
 * the tokens).  With topk_w NULL the rows are summed unweighted, which is the
 * backward of ultraep_permute: a token's gradient is the sum of the gradients
 * of its k dispatched rows.
 * For every token g in [token_begin, token_end):
 *   out[g - token_begin] = sum over j of w[g*k + j] * rows[pos[g*k + j]]
 * summed in fp32 in ascending j and rounded to bf16 (nearest even); pairs
 * whose pos is outside [0, layout_rows) (dropped pairs) add nothing.
 * In:  pos [.][k] int32 of the layer (from ultraep_balance), topk_w fp32
 *      [.][k] or NULL, rows [layout_rows][H] bf16 in layout order (the expert
 *      outputs; layout_rows = total of the layer's plan, or N).
 * Out: out [token_end - token_begin][H] bf16.
 * Errors: EINVAL (null pointers, H <= 0, k outside [1, min(E, 64)], bad token
 *      range, layout_rows < 0); EUNSUPPORTED (H % 8 != 0, layout_rows >= 2^31,
 *      rows/out not 16-byte aligned, pos/topk_w not 4-byte aligned). */
int ultraep_combine(const ultraep_ctx* ctx, const int32_t* pos, const float* topk_w, int32_t k,
                    const uint16_t* rows, int64_t layout_rows, int32_t H, int64_t token_begin,
                    int64_t token_end, uint16_t* out, void* stream);

/* Backward of ultraep_combine ([README] Interface, "Forward and backward":
 * reroute gathers the gradients of the physical replicas back to the logical
 * experts).  For every pair n = g*k + j of the tokens [token_begin, token_end)
 * with pos[n] in [0, layout_rows):
 *   grad_rows[pos[n]]     = w[n] * grad_out[g - token_begin]   (bf16, nearest even)
 *   grad_topk_w[(g - token_begin)*k + j] = <grad_out[g - token_begin], rows[pos[n]]>
 * the dot product summed in fp32 (each lane over its columns in order, then
 * across the wave in a fixed order); a dropped pair gets weight gradient 0
 * and writes no row.  The weight gradients come back in logical (token, k)
 * order, the order of topk_w.
 * In:  pos, topk_w, rows as for ultraep_combine; grad_out
 *      [token_end - token_begin][H] bf16.
 * Out: grad_rows [layout_rows][H] bf16 (only the rows the range's pairs point
 *      to are written), grad_topk_w [token_end - token_begin][k] fp32.
 * Errors: as ultraep_combine, and EINVAL for a NULL topk_w, grad_out,
 *      grad_rows or grad_topk_w with a non-empty range. */
int ultraep_combine_backward(const ultraep_ctx* ctx, const int32_t* pos, const float* topk_w,
                             int32_t k, const uint16_t* rows, int64_t layout_rows, int32_t H,
                             const uint16_t* grad_out, int64_t token_begin, int64_t token_end,
                             uint16_t* grad_rows, float* grad_topk_w, void* stream);

/* The relay schedule of the plan's replica slots (see ultraep_relay_options).
 * Reading of the pages' switches: an expert with n replicas either copies
 * all of them from its master in one stage (fan-out n) or names its m
 * lowest-physical-id replicas relays, which copy from the master in stage 1,
 * while the i-th of the others (i >= m, ascending physical id) copies from
 * relay (i - m) mod m in stage 2; m is the smallest value in
 * [1, min(max_relays, n - 1)] minimising the critical fan-out
 * m + ceil((n - m) / m).  Relay is used under FORCE (n >= 2), or under
 * ADAPTIVE when n >= min_replicas and n >= min_gain * that fan-out, and never
 * when domain_gpus <= 8.
 * In:  plan (one record from ultraep_balance).
 * Out: relay int32 [2][R*S]: relay[s] = -1 (copy from the master), a slot
 *      id (copy from that relay slot) or -2 (empty slot); relay[R*S + s] =
 *      the stage, 1 or 2 (0 for an empty slot).
 * Errors: EINVAL (null pointers, mode outside 0..2, negative counts, reserved
 *      fields not zero); EUNSUPPORTED (pointers not 4-byte aligned). */
int ultraep_weight_sync_plan(const ultraep_ctx* ctx, const void* plan, const ultraep_relay_options* opt,
                             int32_t* relay, void* stream);

/* weight_sync: copy master weights into the redundant slots of the plan
 * ([README] Interface, "Forward and backward": weight_sync materialises the
 * plan by distributing master weights to the replica slots; "Initialization":
 * redundant weight buffers of expert_fc1_numel / expert_fc2_numel elements,
 * one call per tensor).
 * For every slot s in [slot_begin, slot_end) that holds expert e:
 *   replica_weights[s - slot_begin][0, numel) = master_weights[e][0, numel)
 * as a bit copy (any 16-bit element type).  Each source is read once per call
 * and written to all of its target slots.  With relay (from
 * ultraep_weight_sync_plan) the copy runs in its two stages, stage-2 slots
 * copying from their relay slots; the result is the same bits.
 * In:  plan (one record); master_weights: DEVICE array of E device pointers
 *      (entries of experts without a replica in the range may be NULL; a
 *      NULL entry of a touched expert leaves its slots untouched);
 *      relay NULL or the [2][R*S] table (then the range must be all slots,
 *      [0, R*S), since relays may sit anywhere).
 * Out: replica_weights [slot_end - slot_begin][numel]; empty slots untouched.
 * Errors: EINVAL (null pointers, numel < 0, bad slot range, relay with a
 *      partial range); EUNSUPPORTED (master table not 8-byte aligned).  Any
 *      data alignment works; 16-byte aligned buffers with numel % 8 == 0
 *      take the vector path. */
int ultraep_weight_sync(const ultraep_ctx* ctx, const void* plan, const uint16_t* const* master_weights,
                        uint16_t* replica_weights, int64_t numel, int32_t slot_begin, int32_t slot_end,
                        const int32_t* relay, void* stream);

/* Human-readable name of a status code (static storage). */
const char* ultraep_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ULTRAEP_H */

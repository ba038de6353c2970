// Internal interface between the C ABI (ultraep_abi.hip) and the gfx950
// kernels (ultraep_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ultraep.h"
#include "ultraep_geometry.h"

namespace ultraep {

constexpr int kHeaderWords = ULTRAEP_HDR_WORDS;

struct PlanLayout {
  int32_t off[ULTRAEP_PLAN_NUM_FIELDS];  // word offset of each field
  int32_t len[ULTRAEP_PLAN_NUM_FIELDS];  // elements of each field
  int32_t words;                         // record words, a multiple of 64 (256 bytes)
};

struct Shape {
  int32_t E, R, S, D, M, P, ndom;
  int32_t n_inst;                        // E + R*S instance entries
  int32_t eps_num, eps_den, allow_zero;
  int32_t thr_num, thr_den;              // early-stop target of the quota search
  int32_t reroute_mode;                  // ULTRAEP_REROUTE_*
  int32_t min_tokens;                    // minimum pairs per replica (>= 1)
  int32_t lean;                          // 1: the greedy without its chain step
  PlanLayout lay;
};

// Launchers.  All work is queued on `st`; none of them synchronises.
// ws: 2*L*ntiles*E int32 (tile histograms, tile ordinal bases); TK = T*k
// pairs per rank, N = R*TK per layer.  With inv non-null the dispatch
// layout (inv, w_perm from w) is written too.
hipError_t launch_balance(const Shape& sh, int32_t L, const int32_t* idx, const float* w,
                          int32_t TK, int32_t* ws, int32_t* plans, int32_t* phys_idx, int32_t* pos,
                          int32_t* inv, float* w_perm, hipStream_t st);
hipError_t launch_layout(int32_t L, int32_t N, const int32_t* pos, const float* w,
                         int32_t* inv, float* w_perm, hipStream_t st);
hipError_t launch_permute(const Shape& sh, const int32_t* plan, const int32_t* inv, int32_t k,
                          const uint16_t* hidden, int64_t hidden_rows, int32_t H,
                          int32_t p_begin, int32_t p_end, uint16_t* out, int64_t cap,
                          hipStream_t st);
hipError_t launch_fold(const Shape& sh, const int32_t* plan, float* const* masters,
                       const float* reps, int64_t numel, int32_t slot_begin, int32_t slot_end,
                       hipStream_t st);

// Combine (w null: unweighted sum) and its backward over tokens [g0, g1).
hipError_t launch_combine(const int32_t* pos, const float* w, int32_t k, const uint16_t* rows,
                          int64_t layout_rows, int32_t H, int64_t g0, int64_t g1, uint16_t* out,
                          hipStream_t st);
hipError_t launch_combine_backward(const int32_t* pos, const float* w, int32_t k,
                                   const uint16_t* rows, int64_t layout_rows, int32_t H,
                                   const uint16_t* grad_out, int64_t g0, int64_t g1,
                                   uint16_t* grad_rows, float* grad_w, hipStream_t st);

// weight_sync: the relay table [2][R*S] and the copy (relay may be null).
hipError_t launch_relay_plan(const Shape& sh, const int32_t* plan, int32_t mode, int32_t min_replicas,
                             int32_t max_relays, int32_t min_gain, int32_t domain_gpus, int32_t* relay,
                             hipStream_t st);
hipError_t launch_weight_sync(const Shape& sh, const int32_t* plan, const uint16_t* const* masters,
                              uint16_t* reps, int64_t numel, int32_t slot_begin, int32_t slot_end,
                              const int32_t* relay, hipStream_t st);

// Bytes of dynamic LDS the plan solver / reroute kernel need for this shape.
size_t plan_lds_bytes(const Shape& sh);
size_t rerouting_lds_bytes(const Shape& sh, bool layout);

}  // namespace ultraep

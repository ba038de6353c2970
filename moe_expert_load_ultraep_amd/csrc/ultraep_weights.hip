// gfx950 kernels of weight_sync: master expert weights into the redundant
// slots the plan filled ([README] Interface, "Forward and backward":
// weight_sync materialises the plan by distributing master weights to the
// replica slots), and the relay plan that stages that distribution
// ([README] "Performance Tuning", "Expert communication": direct, adaptive
// or forced relay, at most a maximum number of relays, a minimum fan-out
// gain and a minimum replica count; direct for small scale-up domains).
//
// The copy is HBM-bound: every source (a master, or a relay slot in the
// second stage) is read once per call by one leader workgroup per element
// chunk, which writes it to all of the source's target slots in the range.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ultraep_device.h"
#include "ultraep_internal.h"

namespace ultraep {
namespace {

constexpr int kSyncThreads = 256;
constexpr int kSyncUnroll = 4;
constexpr int kSyncMaxTargets = 64;  // replicas of one expert <= ranks of its domain - 1 < 64
constexpr int kRelayThreads = 1024;

__device__ __forceinline__ int replica_slot(int32_t p, int32_t M, int32_t S) {
  const int32_t P1 = M + S;
  const int32_t r = p / P1, j = p % P1;
  return j >= M ? r * S + (j - M) : -1;
}

// One workgroup: slots start empty (-2, stage 0); then each expert walks its
// instances in ascending physical id, decides direct or relay and fills its
// replicas' source and stage.
__global__ __launch_bounds__(kRelayThreads) void relay_plan_kernel(
    const int32_t* __restrict__ slot_expert, const int32_t* __restrict__ inst_ptr,
    const int32_t* __restrict__ inst_phys, int32_t E, int32_t nslots, int32_t M, int32_t S,
    int32_t mode, int32_t min_replicas, int32_t max_relays, int32_t min_gain, int32_t domain_gpus,
    int32_t* __restrict__ src, int32_t* __restrict__ stage) {
  for (int s = threadIdx.x; s < nslots; s += kRelayThreads) {
    src[s] = -2;
    stage[s] = 0;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kRelayThreads) {
    const int i0 = inst_ptr[e], i1 = inst_ptr[e + 1];
    int n = 0;
    for (int i = i0; i < i1; ++i) n += replica_slot(inst_phys[i], M, S) >= 0 ? 1 : 0;
    bool relay = false;
    int m = 0;
    if (mode != ULTRAEP_RELAY_DIRECT && domain_gpus > 8 && n >= 2 && max_relays >= 1) {
      int best = 0;
      const int mmax = min(max_relays, n - 1);
      for (int c = 1; c <= mmax; ++c) {
        const int cost = c + (n - c + c - 1) / c;
        if (m == 0 || cost < best) {
          best = cost;
          m = c;
        }
      }
      relay = mode == ULTRAEP_RELAY_FORCE ||
              (n >= min_replicas && static_cast<int64_t>(n) >= static_cast<int64_t>(min_gain) * best);
    }
    int q = 0;  // replica rank in ascending physical id
    for (int i = i0; i < i1; ++i) {
      const int s = replica_slot(inst_phys[i], M, S);
      if (s < 0 || s >= nslots) continue;
      if (!relay || q < m) {
        src[s] = -1;
        stage[s] = 1;
      } else {
        // the relay of this replica: replica number (q - m) mod m
        const int want = (q - m) % m;
        int seen = 0, rs = -1;
        for (int i2 = i0; i2 < i1 && rs < 0; ++i2) {
          const int s2 = replica_slot(inst_phys[i2], M, S);
          if (s2 < 0) continue;
          if (seen == want) rs = s2;
          ++seen;
        }
        src[s] = rs;
        stage[s] = 2;
      }
      ++q;
    }
  }
}

// blockIdx.y = slot of the range; blockIdx.x strides over element chunks.
// The slot's source is its expert's master (relay table null, or source -1)
// or a relay slot; only the lowest slot of the range with that source in
// this stage does the work, for all of the source's targets in the range.
__global__ __launch_bounds__(kSyncThreads) void weight_sync_kernel(
    const int32_t* __restrict__ slot_expert, const int32_t* __restrict__ inst_ptr,
    const int32_t* __restrict__ inst_phys, int32_t M, int32_t S,
    const int32_t* __restrict__ relay_src, const int32_t* __restrict__ relay_stage, int32_t want_stage,
    const uint16_t* const* __restrict__ masters, uint16_t* __restrict__ reps, int64_t numel,
    int32_t slot_begin, int32_t slot_end) {
  __shared__ int32_t s_tgt[kSyncMaxTargets];
  __shared__ int32_t s_n;
  const int32_t s0 = slot_begin + static_cast<int32_t>(blockIdx.y);
  const int32_t e = slot_expert[s0];
  if (e < 0) return;
  const int32_t my_src = relay_src ? relay_src[s0] : -1;
  const int32_t my_stage = relay_src ? relay_stage[s0] : 1;
  if (my_stage != want_stage) return;
  if (threadIdx.x == 0) {
    int n = 0;
    bool leader = true;
    for (int i = inst_ptr[e]; i < inst_ptr[e + 1]; ++i) {
      const int s = replica_slot(inst_phys[i], M, S);
      if (s < slot_begin || s >= slot_end) continue;
      const int32_t ssrc = relay_src ? relay_src[s] : -1;
      const int32_t sst = relay_src ? relay_stage[s] : 1;
      if (ssrc != my_src || sst != my_stage) continue;
      if (s < s0) leader = false;
      if (n < kSyncMaxTargets) s_tgt[n++] = s;
    }
    s_n = leader ? n : 0;
  }
  __syncthreads();
  const int n = s_n;
  if (n == 0) return;
  const uint16_t* src = my_src < 0 ? masters[e] : reps + static_cast<int64_t>(my_src - slot_begin) * numel;
  if (src == nullptr) return;
  bool vec = (numel % 8) == 0 && (reinterpret_cast<uintptr_t>(src) % 16) == 0 &&
             (reinterpret_cast<uintptr_t>(reps) % 16) == 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kSyncThreads;
  if (vec) {
    const u32x4* sv = reinterpret_cast<const u32x4*>(src);
    const int64_t nv = numel / 8;
    for (int64_t b = static_cast<int64_t>(blockIdx.x) * kSyncThreads + threadIdx.x; b < nv;
         b += stride * kSyncUnroll) {
      u32x4 x[kSyncUnroll];
#pragma unroll
      for (int u = 0; u < kSyncUnroll; ++u) {
        const int64_t i = b + u * stride;
        if (i < nv) x[u] = __builtin_nontemporal_load(sv + i);
      }
      for (int t = 0; t < n; ++t) {
        u32x4* dv = reinterpret_cast<u32x4*>(reps + static_cast<int64_t>(s_tgt[t] - slot_begin) * numel);
#pragma unroll
        for (int u = 0; u < kSyncUnroll; ++u) {
          const int64_t i = b + u * stride;
          if (i < nv) __builtin_nontemporal_store(x[u], dv + i);
        }
      }
    }
  } else {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kSyncThreads + threadIdx.x; i < numel; i += stride) {
      const uint16_t x = src[i];
      for (int t = 0; t < n; ++t) reps[static_cast<int64_t>(s_tgt[t] - slot_begin) * numel + i] = x;
    }
  }
}

}  // namespace

hipError_t launch_relay_plan(const Shape& sh, const int32_t* plan, int32_t mode, int32_t min_replicas,
                             int32_t max_relays, int32_t min_gain, int32_t domain_gpus, int32_t* relay,
                             hipStream_t st) {
  const int32_t nslots = sh.R * sh.S;
  hipLaunchKernelGGL(relay_plan_kernel, dim3(1), dim3(kRelayThreads), 0, st,
                     plan + sh.lay.off[ULTRAEP_PLAN_SLOT_EXPERT], plan + sh.lay.off[ULTRAEP_PLAN_INST_PTR],
                     plan + sh.lay.off[ULTRAEP_PLAN_INST_PHYS], sh.E, nslots, sh.M, sh.S, mode, min_replicas,
                     max_relays, min_gain, domain_gpus, relay, relay + nslots);
  return hipGetLastError();
}

hipError_t launch_weight_sync(const Shape& sh, const int32_t* plan, const uint16_t* const* masters,
                              uint16_t* reps, int64_t numel, int32_t slot_begin, int32_t slot_end,
                              const int32_t* relay, hipStream_t st) {
  const int32_t nslots = slot_end - slot_begin;
  if (nslots <= 0 || numel <= 0) return hipSuccess;
  const int64_t per_block = static_cast<int64_t>(kSyncThreads) * 8 * kSyncUnroll;
  const int64_t want = (numel + per_block - 1) / per_block;
  const uint32_t bx = static_cast<uint32_t>(want < 2048 ? want : 2048);
  const int32_t all = sh.R * sh.S;
  for (int32_t stg = 1; stg <= (relay ? 2 : 1); ++stg) {
    hipLaunchKernelGGL(weight_sync_kernel, dim3(bx, static_cast<uint32_t>(nslots)), dim3(kSyncThreads), 0, st,
                       plan + sh.lay.off[ULTRAEP_PLAN_SLOT_EXPERT], plan + sh.lay.off[ULTRAEP_PLAN_INST_PTR],
                       plan + sh.lay.off[ULTRAEP_PLAN_INST_PHYS], sh.M, sh.S, relay,
                       relay ? relay + all : nullptr, stg, masters, reps, numel, slot_begin, slot_end);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ultraep

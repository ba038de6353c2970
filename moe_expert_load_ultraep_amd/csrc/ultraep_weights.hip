// gfx950 kernels of weight_sync: master expert weights into the redundant
// slots the plan filled ([README] Interface, "Forward and backward":
// weight_sync materialises the plan by distributing master weights to the
// replica slots), and the relay plan that stages that distribution
// ([README] "Performance Tuning", "Expert communication": direct, adaptive
// or forced relay, at most a maximum number of relays, a minimum fan-out
// gain and a minimum replica count; direct for small scale-up domains).
//
// The copy is HBM-bound: every source (a master, or a relay slot in the
// second stage) is read once per call, each element chunk by one
// workgroup, which writes it to all of the source's target slots in the
// range.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ultraep_device.h"
#include "ultraep_internal.h"

namespace ultraep {
namespace {

constexpr int kSyncThreads = 256;
constexpr int kSyncUnroll = 4;
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

// One launch per stage, a 1-D grid over element chunks.  Every workgroup
// first groups the filled slots of the range that copy in this stage by
// their source, in LDS: a slot's key is its expert (it copies from the
// master) or E + its relay slot (it copies from that relay, in stage 2).
// Then it moves its chunks of every group's source to all of that group's
// targets, so each source is read once per call and no workgroup of the
// launch sits idle.  The grouping reads the range's slot entries in one
// parallel round and the groups' master pointers in another.

__global__ __launch_bounds__(kSyncThreads) void weight_sync_kernel(
    const int32_t* __restrict__ slot_expert, int32_t E, const int32_t* __restrict__ relay_src,
    const int32_t* __restrict__ relay_stage, int32_t want_stage, const uint16_t* const* __restrict__ masters,
    uint16_t* __restrict__ reps, int64_t numel, int32_t slot_begin, int32_t slot_end) {
  // tables sized to the range (sync_lds_bytes): the groups' source pointers
  // first (8-byte aligned), then range slot -> key or -1, key -> slots and
  // then their first place, slots grouped by key, group -> key, group starts
  extern __shared__ __align__(16) int32_t lds[];
  __shared__ int32_t s_ng;
  const int nslots = slot_end - slot_begin;
  const int nkeys = E + slot_end;  // relay keys name slots below slot_end
  const uint16_t** s_gsrc = reinterpret_cast<const uint16_t**>(lds);
  int32_t* s_key = lds + 2 * nslots;
  int32_t* s_cnt = s_key + nslots;
  int32_t* s_order = s_cnt + nkeys;
  int32_t* s_gkey = s_order + nslots;
  int32_t* s_gbeg = s_gkey + nslots;
  const int tid = threadIdx.x;
  for (int k = tid; k < nkeys; k += kSyncThreads) s_cnt[k] = 0;
  __syncthreads();
  for (int i = tid; i < nslots; i += kSyncThreads) {
    const int32_t s = slot_begin + i;
    const int32_t e = slot_expert[s];
    const int32_t src = relay_src ? relay_src[s] : -1;
    const int32_t stg = relay_src ? relay_stage[s] : 1;
    const int32_t key = (e >= 0 && e < E && stg == want_stage && src < slot_end) ? (src < 0 ? e : E + src) : -1;
    s_key[i] = key;
    if (key >= 0) atomicAdd(&s_cnt[key], 1);
  }
  __syncthreads();
  if (tid < 64) {
    // keys in ascending order: each non-empty one is a group, its slots a
    // run of s_order; s_cnt becomes the run's first place
    const int lane = tid;
    const int per = (nkeys + 63) / 64;
    const int b = min(lane * per, nkeys), en = min(b + per, nkeys);
    int32_t slots = 0, groups = 0;
    for (int k = b; k < en; ++k) {
      slots += s_cnt[k];
      groups += s_cnt[k] > 0 ? 1 : 0;
    }
    const int32_t packed = wave_inclusive_scan((groups << 16) | slots);
    int32_t place = (packed - ((groups << 16) | slots)) & 0xFFFF;
    int32_t g = (packed - ((groups << 16) | slots)) >> 16;
    for (int k = b; k < en; ++k) {
      const int32_t c = s_cnt[k];
      if (c > 0) {
        s_gkey[g] = k;
        s_gbeg[g] = place;
        ++g;
      }
      s_cnt[k] = place;
      place += c;
    }
    if (lane == 63) {
      s_ng = packed >> 16;
      s_gbeg[packed >> 16] = packed & 0xFFFF;
    }
  }
  __syncthreads();
  const int ng = s_ng;
  // sources of the groups (one parallel round), and the slots into their runs
  for (int g = tid; g < ng; g += kSyncThreads) {
    const int32_t k = s_gkey[g];
    s_gsrc[g] = k < E ? masters[k] : reps + static_cast<int64_t>(k - E - slot_begin) * numel;
  }
  for (int i = tid; i < nslots; i += kSyncThreads) {
    const int32_t key = s_key[i];
    // (the order of slots inside a group only changes the store order)
    if (key >= 0) s_order[atomicAdd(&s_cnt[key], 1)] = slot_begin + i;
  }
  __syncthreads();

  const int64_t nv = numel / 8;
  const bool reps_vec = (numel % 8) == 0 && (reinterpret_cast<uintptr_t>(reps) % 16) == 0;
  for (int g = 0; g < ng; ++g) {
    const uint16_t* src = s_gsrc[g];
    if (src == nullptr) continue;  // a touched expert without a master pointer: its slots stay
    const int t0 = s_gbeg[g], t1 = s_gbeg[g + 1];
    if (reps_vec && (reinterpret_cast<uintptr_t>(src) % 16) == 0) {
      // kSyncUnroll 16-byte vectors a block-width apart per thread and
      // chunk, all loaded before any store
      const u32x4* sv = reinterpret_cast<const u32x4*>(src);
      const int64_t span = static_cast<int64_t>(kSyncUnroll) * kSyncThreads;
      for (int64_t c0 = static_cast<int64_t>(blockIdx.x) * span + tid; c0 < nv;
           c0 += static_cast<int64_t>(gridDim.x) * span) {
        u32x4 x[kSyncUnroll];
#pragma unroll
        for (int u = 0; u < kSyncUnroll; ++u) {
          const int64_t i = c0 + static_cast<int64_t>(u) * kSyncThreads;
          if (i < nv) x[u] = __builtin_nontemporal_load(sv + i);
        }
        for (int t = t0; t < t1; ++t) {
          u32x4* dv = reinterpret_cast<u32x4*>(reps + static_cast<int64_t>(s_order[t] - slot_begin) * numel);
#pragma unroll
          for (int u = 0; u < kSyncUnroll; ++u) {
            const int64_t i = c0 + static_cast<int64_t>(u) * kSyncThreads;
            if (i < nv) __builtin_nontemporal_store(x[u], dv + i);
          }
        }
      }
    } else {
      for (int64_t i = static_cast<int64_t>(blockIdx.x) * kSyncThreads + tid; i < numel;
           i += static_cast<int64_t>(gridDim.x) * kSyncThreads) {
        const uint16_t x = src[i];
        for (int t = t0; t < t1; ++t) reps[static_cast<int64_t>(s_order[t] - slot_begin) * numel + i] = x;
      }
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

// Dynamic LDS of weight_sync_kernel: per range slot a group's source
// pointer (2 words) and 4 words of tables, one word per key, and one more
// group start (at most 33 KiB at the limits of the build).
size_t sync_lds_bytes(int32_t E, int32_t slot_begin, int32_t slot_end) {
  const size_t nslots = static_cast<size_t>(slot_end - slot_begin);
  return 4 * (6 * nslots + static_cast<size_t>(E) + static_cast<size_t>(slot_end) + 1);
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
    hipLaunchKernelGGL(weight_sync_kernel, dim3(bx), dim3(kSyncThreads), sync_lds_bytes(sh.E, slot_begin, slot_end),
                       st,
                       plan + sh.lay.off[ULTRAEP_PLAN_SLOT_EXPERT], sh.E, relay, relay ? relay + all : nullptr,
                       stg, masters, reps, numel, slot_begin, slot_end);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ultraep

// gfx950 kernels of the combine step and of the gradient gathers of the
// backward pass ([README] Interface, "Forward and backward": after the
// experts, combine returns each token's k expert outputs to the token,
// weighted by its routing probabilities; in the backward pass reroute gathers
// the gradients of the physical replicas back to the logical experts).
//
// All three are HBM-streaming gathers over the dispatch layout: one wave per
// token, every row of the token addressed through its own buffer resource
// (size 0 for a dropped pair, so it reads as zeros and its stores vanish),
// 16-byte accesses, fp32 arithmetic, bf16 results rounded to nearest even.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ultraep_device.h"
#include "ultraep_internal.h"

namespace ultraep {
namespace {

constexpr int kCombThreads = 256;
constexpr int kCombWaves = kCombThreads / 64;
constexpr int kRowsInFlight = 4;    // rows of one token loaded together
constexpr int kChunksInFlight = 2;  // 16-byte column chunks per lane per row

// y[t] = sum_j w[g, j] * rows[pos[g*k + j]] for g = g0 + t (w = 1 when not
// WEIGHTED).  Column chunks are the outer loop so each chunk's fp32
// accumulators stay in registers while the k rows stream through; the rows
// of a token are summed in ascending j.
template <bool WEIGHTED>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(
    const int32_t* __restrict__ pos, const float* __restrict__ w, int32_t k,
    const u32x4* __restrict__ rows, int64_t layout_rows, int32_t H8, int64_t g0, int64_t ntok,
    u32x4* __restrict__ out) {
  const int lane = lane_id();
  const uint32_t rowb = static_cast<uint32_t>(H8) * 16u;
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kCombWaves;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * kCombWaves + wv; t < ntok; t += nwaves) {
    const int64_t n0 = (g0 + t) * k;
    // lane j < k holds pair j's layout row (-1 when dropped) and weight
    int32_t pj = -1;
    float wj = 0.f;
    if (lane < k) {
      const int32_t p = pos[n0 + lane];
      pj = (p >= 0 && p < layout_rows) ? p : -1;
      if (WEIGHTED) wj = w[n0 + lane];
    }
    const __amdgpu_buffer_rsrc_t dst = row_rsrc(out + t * H8, rowb);
    for (int c0 = 0; c0 < H8; c0 += 64 * kChunksInFlight) {
      float acc[kChunksInFlight][8];
#pragma unroll
      for (int u = 0; u < kChunksInFlight; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[u][e] = 0.f;
      for (int j0 = 0; j0 < k; j0 += kRowsInFlight) {
        u32x4 x[kRowsInFlight][kChunksInFlight];
#pragma unroll
        for (int r = 0; r < kRowsInFlight; ++r) {
          const int j = j0 + r;
          const int32_t p = static_cast<int32_t>(readlane(static_cast<uint32_t>(pj), j < k ? j : 0));
          const bool live = j < k && p >= 0;
          const __amdgpu_buffer_rsrc_t src =
              row_rsrc(rows + static_cast<int64_t>(live ? p : 0) * H8, live ? rowb : 0u);
#pragma unroll
          for (int u = 0; u < kChunksInFlight; ++u)
            x[r][u] = __builtin_amdgcn_raw_buffer_load_b128(src, (c0 + u * 64 + lane) * 16, 0,
                                                             kNonTemporal);
        }
#pragma unroll
        for (int r = 0; r < kRowsInFlight; ++r) {
          const int j = j0 + r;
          const float wt = WEIGHTED ? readlane_f(wj, j < k ? j : 0) : 1.f;
          if (j < k) {
#pragma unroll
            for (int u = 0; u < kChunksInFlight; ++u)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                acc[u][2 * q] += wt * bf16_lo(x[r][u][q]);
                acc[u][2 * q + 1] += wt * bf16_hi(x[r][u][q]);
              }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kChunksInFlight; ++u) {
        u32x4 y;
#pragma unroll
        for (int q = 0; q < 4; ++q) y[q] = pack_bf16(acc[u][2 * q], acc[u][2 * q + 1]);
        __builtin_amdgcn_raw_buffer_store_b128(y, dst, (c0 + u * 64 + lane) * 16, 0, kNonTemporal);
      }
    }
  }
}

// For each pair n = g*k + j of the tokens: grad_rows[pos[n]] = w[n] * dy[t]
// (bf16) and grad_w[t*k + j] = <dy[t], rows[pos[n]]> (fp32: each lane sums
// its columns in order, then the wave sums the lanes in a fixed order).  The
// rows of a token go in groups of kRowsInFlight: one pass over the columns
// loads the gradient chunk once for the group's rows, and the group's dot
// products are reduced together at its end.  The gradient row is re-read per
// group from L2; expert-output rows are read once, gradient rows written once.
__global__ __launch_bounds__(kCombThreads) void combine_backward_kernel(
    const int32_t* __restrict__ pos, const float* __restrict__ w, int32_t k,
    const u32x4* __restrict__ rows, int64_t layout_rows, int32_t H8, const u32x4* __restrict__ dy,
    int64_t g0, int64_t ntok, u32x4* __restrict__ grad_rows, float* __restrict__ grad_w) {
  const int lane = lane_id();
  const uint32_t rowb = static_cast<uint32_t>(H8) * 16u;
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kCombWaves;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * kCombWaves + wv; t < ntok; t += nwaves) {
    const int64_t n0 = (g0 + t) * k;
    int32_t pj = -1;
    float wj = 0.f;
    if (lane < k) {
      const int32_t p = pos[n0 + lane];
      pj = (p >= 0 && p < layout_rows) ? p : -1;
      wj = w[n0 + lane];
    }
    const __amdgpu_buffer_rsrc_t gsrc = row_rsrc(dy + t * H8, rowb);
    for (int j0 = 0; j0 < k; j0 += kRowsInFlight) {
      __amdgpu_buffer_rsrc_t xsrc[kRowsInFlight], gdst[kRowsInFlight];
      float wt[kRowsInFlight], dot[kRowsInFlight];
#pragma unroll
      for (int r = 0; r < kRowsInFlight; ++r) {
        const int j = j0 + r;
        const int32_t p = static_cast<int32_t>(readlane(static_cast<uint32_t>(pj), j < k ? j : 0));
        const bool live = j < k && p >= 0;
        const int64_t row = live ? p : 0;
        xsrc[r] = row_rsrc(rows + row * H8, live ? rowb : 0u);
        gdst[r] = row_rsrc(grad_rows + row * H8, live ? rowb : 0u);
        wt[r] = readlane_f(wj, j < k ? j : 0);
        dot[r] = 0.f;
      }
      for (int c0 = 0; c0 < H8; c0 += 64 * kChunksInFlight) {
        u32x4 g[kChunksInFlight], x[kRowsInFlight][kChunksInFlight];
#pragma unroll
        for (int u = 0; u < kChunksInFlight; ++u)
          g[u] = __builtin_amdgcn_raw_buffer_load_b128(gsrc, (c0 + u * 64 + lane) * 16, 0, 0);
#pragma unroll
        for (int r = 0; r < kRowsInFlight; ++r)
#pragma unroll
          for (int u = 0; u < kChunksInFlight; ++u)
            x[r][u] = __builtin_amdgcn_raw_buffer_load_b128(xsrc[r], (c0 + u * 64 + lane) * 16, 0,
                                                            kNonTemporal);
#pragma unroll
        for (int r = 0; r < kRowsInFlight; ++r)
#pragma unroll
          for (int u = 0; u < kChunksInFlight; ++u) {
            u32x4 d;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float glo = bf16_lo(g[u][q]), ghi = bf16_hi(g[u][q]);
              dot[r] += glo * bf16_lo(x[r][u][q]);
              dot[r] += ghi * bf16_hi(x[r][u][q]);
              d[q] = pack_bf16(wt[r] * glo, wt[r] * ghi);
            }
            __builtin_amdgcn_raw_buffer_store_b128(d, gdst[r], (c0 + u * 64 + lane) * 16, 0,
                                                   kNonTemporal);
          }
      }
#pragma unroll
      for (int r = 0; r < kRowsInFlight; ++r) {
        const int j = j0 + r;
        const float sum = wave_sum_f32(dot[r]);
        const int32_t p = static_cast<int32_t>(readlane(static_cast<uint32_t>(pj), j < k ? j : 0));
        if (lane == 0 && j < k) grad_w[t * k + j] = p >= 0 ? sum : 0.f;
      }
    }
  }
}

uint32_t comb_blocks(int64_t ntok) {
  const int64_t want = (ntok + kCombWaves - 1) / kCombWaves;
  return static_cast<uint32_t>(want < (1 << 20) ? want : (1 << 20));
}

}  // namespace

hipError_t launch_combine(const int32_t* pos, const float* w, int32_t k, const uint16_t* rows,
                          int64_t layout_rows, int32_t H, int64_t g0, int64_t g1, uint16_t* out,
                          hipStream_t st) {
  const int64_t ntok = g1 - g0;
  if (ntok <= 0) return hipSuccess;
  const auto* r = reinterpret_cast<const u32x4*>(rows);
  auto* o = reinterpret_cast<u32x4*>(out);
  if (w != nullptr)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(comb_blocks(ntok)), dim3(kCombThreads), 0, st, pos,
                       w, k, r, layout_rows, H / 8, g0, ntok, o);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(comb_blocks(ntok)), dim3(kCombThreads), 0, st,
                       pos, w, k, r, layout_rows, H / 8, g0, ntok, o);
  return hipGetLastError();
}

hipError_t launch_combine_backward(const int32_t* pos, const float* w, int32_t k,
                                   const uint16_t* rows, int64_t layout_rows, int32_t H,
                                   const uint16_t* grad_out, int64_t g0, int64_t g1,
                                   uint16_t* grad_rows, float* grad_w, hipStream_t st) {
  const int64_t ntok = g1 - g0;
  if (ntok <= 0) return hipSuccess;
  hipLaunchKernelGGL(combine_backward_kernel, dim3(comb_blocks(ntok)), dim3(kCombThreads), 0, st, pos,
                     w, k, reinterpret_cast<const u32x4*>(rows), layout_rows, H / 8,
                     reinterpret_cast<const u32x4*>(grad_out), g0, ntok,
                     reinterpret_cast<u32x4*>(grad_rows), grad_w);
  return hipGetLastError();
}

}  // namespace ultraep

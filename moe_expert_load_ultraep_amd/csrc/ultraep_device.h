// wave64 and buffer helpers shared by the gfx950 kernels (device code
// only; internal, not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ultraep {
namespace {

// ------------------------------------------------------------------------
// wave64 helpers
// ------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Number of set bits of m in lanes below the calling lane.
__device__ __forceinline__ int count_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ uint32_t readlane(uint32_t v, int l) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), l));
}

// Wave-wide max / min of an unsigned value; every lane must be active.  The
// butterfly inside each 16-lane row uses DPP (quad swaps, half-row and row
// mirrors); the four row results are combined through scalar registers.
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  x = max(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
  x = max(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
  x = max(x, dpp<0x141>(x));  // row_half_mirror
  x = max(x, dpp<0x140>(x));  // row_mirror
  return max(max(readlane(x, 0), readlane(x, 16)), max(readlane(x, 32), readlane(x, 48)));
}

// Wave-wide max left in lane 63 and returned through one read-lane: the row
// maxima are combined by DPP row broadcasts (lane 15 into rows 1 and 3, then
// lane 31 into rows 2 and 3) instead of four read-lanes and scalar maxima,
// which shortens the dependent chain.  Every lane must be active.
// Rows outside ROWS read 0, the identity of an unsigned max, which lets the
// compiler fold the move into the max as one DPP instruction.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_rows(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROWS, 0xF, false));
}

__device__ __forceinline__ uint32_t wave_max_bcast(uint32_t x) {
  x = max(x, dpp<0xB1>(x));             // quad_perm [1,0,3,2]
  x = max(x, dpp<0x4E>(x));             // quad_perm [2,3,0,1]
  x = max(x, dpp<0x141>(x));            // row_half_mirror
  x = max(x, dpp<0x140>(x));            // row_mirror: every lane holds its row's max
  x = max(x, dpp_rows<0x142, 0xA>(x));  // row_bcast:15 -> rows 1, 3
  x = max(x, dpp_rows<0x143, 0xC>(x));  // row_bcast:31 -> rows 2, 3
  return readlane(x, 63);
}

// Three independent wave maxima, as wave_max_bcast, with each DPP stage
// issued for all three values before the next stage: the stages of one
// value depend on each other, so interleaving fills the DPP hazard slots
// with the other values' work instead of wait states.
__device__ __forceinline__ void wave_max3_bcast(uint32_t& a, uint32_t& b, uint32_t& c) {
#define ULTRAEP_MAX3(F) a = max(a, F(a)); b = max(b, F(b)); c = max(c, F(c))
  ULTRAEP_MAX3(dpp<0xB1>);
  ULTRAEP_MAX3(dpp<0x4E>);
  ULTRAEP_MAX3(dpp<0x141>);
  ULTRAEP_MAX3(dpp<0x140>);
  ULTRAEP_MAX3((dpp_rows<0x142, 0xA>));
  ULTRAEP_MAX3((dpp_rows<0x143, 0xC>));
#undef ULTRAEP_MAX3
  a = readlane(a, 63);
  b = readlane(b, 63);
  c = readlane(c, 63);
}

// Two independent wave maxima, interleaved as wave_max3_bcast.
__device__ __forceinline__ void wave_max2_bcast(uint32_t& a, uint32_t& b) {
#define ULTRAEP_MAX2(F) a = max(a, F(a)); b = max(b, F(b))
  ULTRAEP_MAX2(dpp<0xB1>);
  ULTRAEP_MAX2(dpp<0x4E>);
  ULTRAEP_MAX2(dpp<0x141>);
  ULTRAEP_MAX2(dpp<0x140>);
  ULTRAEP_MAX2((dpp_rows<0x142, 0xA>));
  ULTRAEP_MAX2((dpp_rows<0x143, 0xC>));
#undef ULTRAEP_MAX2
  a = readlane(a, 63);
  b = readlane(b, 63);
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return readlane(x, 0) + readlane(x, 16) + readlane(x, 32) + readlane(x, 48);
}

__device__ __forceinline__ int lowest_lane(uint64_t m) { return __builtin_ctzll(m); }

// Inclusive scan across the wave's lanes, all in DPP (no LDS round trip):
// inside each 16-lane row by row shifts of 1, 2, 4 and 8 lanes (a lane
// whose source lies before its row adds 0), then the row totals are carried
// by row broadcasts (lane 15 into row 1 and lane 47 into row 3, then lane 31
// into rows 2 and 3).  Every lane must be active.
__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t x) {
  uint32_t v = static_cast<uint32_t>(x);
  v += dpp<0x111>(v);               // row_shr:1
  v += dpp<0x112>(v);               // row_shr:2
  v += dpp<0x114>(v);               // row_shr:4
  v += dpp<0x118>(v);               // row_shr:8
  v += dpp_rows<0x142, 0xA>(v);     // row_bcast:15 -> rows 1, 3
  v += dpp_rows<0x143, 0xC>(v);     // row_bcast:31 -> rows 2, 3
  return static_cast<int32_t>(v);
}

// Aligned segments of N lanes (N a power of two, at most 16, so a segment
// never crosses a 16-lane row), for work that N lanes share: an inclusive
// scan (row shifts, each added only where the source lane is in the
// segment), and the segment's sum and minimum in every lane (the quad swaps
// and half-row and row mirrors of wave_max).  Every lane of a segment must
// be active together.
template <int N>
__device__ __forceinline__ int32_t segment_inclusive_scan(int32_t x, int sub) {
  static_assert(N >= 1 && N <= 16 && (N & (N - 1)) == 0, "segments of 1, 2, 4, 8 or 16 lanes");
  uint32_t v = static_cast<uint32_t>(x), y;
  if constexpr (N > 1) { y = dpp<0x111>(v); v += sub >= 1 ? y : 0u; }
  if constexpr (N > 2) { y = dpp<0x112>(v); v += sub >= 2 ? y : 0u; }
  if constexpr (N > 4) { y = dpp<0x114>(v); v += sub >= 4 ? y : 0u; }
  if constexpr (N > 8) { y = dpp<0x118>(v); v += sub >= 8 ? y : 0u; }
  return static_cast<int32_t>(v);
}

template <int N>
__device__ __forceinline__ int32_t segment_sum(int32_t x) {
  uint32_t v = static_cast<uint32_t>(x);
  if constexpr (N > 1) v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  if constexpr (N > 2) v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  if constexpr (N > 4) v += dpp<0x141>(v);  // row_half_mirror
  if constexpr (N > 8) v += dpp<0x140>(v);  // row_mirror
  return static_cast<int32_t>(v);
}

template <int N>
__device__ __forceinline__ int32_t segment_min(int32_t x) {
  if constexpr (N > 1) x = min(x, static_cast<int32_t>(dpp<0xB1>(static_cast<uint32_t>(x))));
  if constexpr (N > 2) x = min(x, static_cast<int32_t>(dpp<0x4E>(static_cast<uint32_t>(x))));
  if constexpr (N > 4) x = min(x, static_cast<int32_t>(dpp<0x141>(static_cast<uint32_t>(x))));
  if constexpr (N > 8) x = min(x, static_cast<int32_t>(dpp<0x140>(static_cast<uint32_t>(x))));
  return x;
}

// 16-byte vectors as native clang vectors (the nontemporal builtins take
// these, not HIP's struct vector types).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

// Wave-wide fp32 sum in one fixed order (the same butterfly inside each row,
// then rows 0 + 1 + 2 + 3), so repeated runs give identical bits.
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

__device__ __forceinline__ float wave_sum_f32(float x) {
  x += dppf<0xB1>(x);
  x += dppf<0x4E>(x);
  x += dppf<0x141>(x);
  x += dppf<0x140>(x);
  return ((readlane_f(x, 0) + readlane_f(x, 16)) + readlane_f(x, 32)) + readlane_f(x, 48);
}

// bf16 <-> fp32: a bf16 is the top half of an fp32; fp32 -> bf16 rounds to
// nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __builtin_bit_cast(float, v & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// ------------------------------------------------------------------------
// raw buffer resources
// ------------------------------------------------------------------------
// A row addressed through its own buffer resource: loads at or past `bytes`
// return zeros and stores there are dropped, so ragged row tails and rows
// that must read as zero need no per-lane branches.
constexpr int kBufferWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)
constexpr int kNonTemporal = 2;           // cache policy bit: non-temporal
// Non-temporal stores written through at device scope (the sc1 bit): the
// L2s keep no dirty lines of them for the write-back at the kernel's end.
// Used where a streaming kernel's workgroups each store once, at its end;
// as the form of every store of a long copy, or of 4-byte scatters, it
// measured slower than plain non-temporal global stores.
constexpr int kStreamStore = kNonTemporal | 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           kBufferWord3);
}

}  // namespace
}  // namespace ultraep

// device.hpp -- gfx950 device helpers for the Lamport mailbox kernels.
//
// Mailbox protocol (vLLM DSpark drafter pages, "drafter.comm" module prose): a 16 B
// fragment of four 32-bit words is published once none of its words is the
// sentinel, the BF16 pair (+0, -0) = 0x80000000; writers send clean words, so a
// fragment torn into single-word writes is never mistaken for a published one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace arn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kSentinel = 0x80000000u;
constexpr int kHidden = 7168;     // BF16 columns per row
constexpr int kRowWords = 3584;   // 32-bit words per row
constexpr int kRowFrags = 896;    // 16 B fragments per row
constexpr int kRowBytes = 14336;  // bytes per row

// Cache-policy bits of a gfx950 buffer instruction: sc0 = 1, nt = 2, sc1 = 16.
// sc1 alone is the device (agent) scope: the access is coherent across the eight
// XCDs' L2s, which is what a poll needs when its producer runs concurrently.
enum : int { kPolPlain = 0, kPolNT = 2, kPolDevice = 16, kPolDeviceNT = 18 };

// Minimum waves per SIMD asked of the compiler for each consumer workgroup size
// (0 = no request).
#ifndef ARNORM_WPE_896
#define ARNORM_WPE_896 0
#endif
#ifndef ARNORM_WPE_448
#define ARNORM_WPE_448 0
#endif
#ifndef ARNORM_WPE_256
#define ARNORM_WPE_256 0
#endif

// Device status word: bit 0 set when a poll gave up (ARNORM_TIMEOUT).  Set with a
// vector atomic OR by any kernel; taken by status_take_kernel, which swaps it with 0 in
// one device atomic and leaves the old value in g_status_taken for the host to copy.  The
// library is one translation unit, so these are their only definitions.
__device__ unsigned int g_status;
__device__ unsigned int g_status_taken;

__global__ void __launch_bounds__(64) status_take_kernel() {
  if (threadIdx.x == 0) g_status_taken = atomicExch(&g_status, 0u);
}

// Buffer resource over `bytes` bytes at `base` (raw buffer: stride 0; the gfx9
// data-format word).  Accesses past `bytes` read 0 and drop their stores.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

template <int POL>
__device__ inline u32x4 buf_load(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, POL);
}

template <int POL>
__device__ inline void buf_store(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)byte_off, 0, POL);
}

// Streaming (non-temporal) 16 B load of an input read once.
__device__ inline u32x4 nt_load(const u32x4 *p) { return __builtin_nontemporal_load(p); }

// One re-read of a fragment for a poll loop: four relaxed device-scope atomic
// loads, which the compiler may neither hoist out of the loop nor merge, and which
// read through to the device-coherent level.
__device__ inline u32x4 load_fragment_coherent(const uint32_t *p) {
  u32x4 v;
  v.x = __hip_atomic_load(p + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v.y = __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v.z = __hip_atomic_load(p + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v.w = __hip_atomic_load(p + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v;
}

// drafter.comm, `clean`: the sentinel pair becomes (+0, +0); every other word is
// sent unchanged.
__device__ inline uint32_t clean(uint32_t w) { return w == kSentinel ? 0u : w; }
__device__ inline u32x4 clean4(u32x4 v) {
  return u32x4{clean(v.x), clean(v.y), clean(v.z), clean(v.w)};
}

__device__ inline bool published(u32x4 v) {
  return v.x != kSentinel && v.y != kSentinel && v.z != kSentinel && v.w != kSentinel;
}

__device__ inline u32x4 sentinel4() { return u32x4{kSentinel, kSentinel, kSentinel, kSentinel}; }

// BF16 lanes of a word -> FP32 (exact: the BF16 pattern is the FP32 high half).
__device__ inline float lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two FP32 values -> one word of BF16 (lo in the low half), round-to-nearest-even:
// a single v_cvt_pk_bf16_f32 on gfx950.
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Sum over the 64 lanes of a wave by an XOR butterfly: every lane ends with the same
// bits (each step adds a commutative pair), so the result does not depend on the lane.
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// A lane's value read by every lane (v_readlane_b32), bit for bit.
__device__ inline float lane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// DPP move of v within rows of 16 lanes; CTRL is the gfx9 DPP control word.
template <int CTRL>
__device__ inline float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// The same sum with DPP moves instead of LDS-pipe shuffles: the 16 lanes of a row
// exchange across quads (quad_perm [1,0,3,2] and [2,3,0,1]), half rows (row_half_mirror)
// and rows (row_mirror), each step adding a commutative pair, so every lane of a row
// holds that row's sum; the four row sums are then read out and added in row order.
// Fewer cycles than the butterfly (its LDS-pipe shuffles, each a round trip, become
// VALU moves), which matters where a row's sum sits on a chain of dependent steps.
__device__ inline float wave_sum_dpp(float v) {
  v = v + dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  v = v + dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  v = v + dpp_f32<0x141>(v);  // row_half_mirror
  v = v + dpp_f32<0x140>(v);  // row_mirror
  return (lane_f32(v, 0) + lane_f32(v, 16)) + (lane_f32(v, 32) + lane_f32(v, 48));
}

}  // namespace arn

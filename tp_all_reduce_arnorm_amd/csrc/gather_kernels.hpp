// gather_kernels.hpp -- the sentinel-cleaning Gather for gfx950.
//
// Method: vLLM DSpark drafter pages, "drafter.comm" (module prose, Gather entry and
// kernel): rank r's [M, S] shard of 32-bit words lands, cleaned, at columns r*S .. of
// the [cap, TP*S] mailbox rows; the reader polls every fragment of its rows and either
// copies them to a dense output and re-arms them, or leaves them published for a later
// reader.  One-GPU stand-in: the ranks' shards are pushed by gather_push calls on the
// same GPU, the pages' push-then-poll kernel is split into two kernels.
#pragma once

#include "device.hpp"

namespace arn {

// gather_push: grid (x, M, nslots); shard row m of slot s is F = S/4 contiguous
// fragments, written to row m at word offset (rank + s) * S.
template <int POL>
__global__ void __launch_bounds__(256)
gather_push_kernel(const u32x4 *__restrict__ shard, uint8_t *__restrict__ box, uint32_t frags,
                   uint32_t M, uint32_t row_bytes, uint32_t first_col_bytes) {
  const uint32_t m = blockIdx.y, s = blockIdx.z;
  const u32x4 *src = shard + ((size_t)s * M + m) * frags;
  const __amdgpu_buffer_rsrc_t dst =
      make_rsrc(box + (size_t)m * row_bytes + first_col_bytes + (size_t)s * frags * 16u, frags * 16u);
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < frags; i += gridDim.x * 256u)
    buf_store<POL>(clean4(nt_load(src + i)), dst, i * 16u);
}

// gather_poll: grid (ctas, M); workgroup `cta` of row m takes fragments
// cta*256 + t, strided by ctas*256, over the row's TP*S/4 fragments.
template <int POL_LD, int POL_ST>
__global__ void __launch_bounds__(256)
gather_poll_kernel(uint8_t *__restrict__ box, u32x4 *__restrict__ out, uint32_t row_frags,
                   int copy, uint64_t spin_limit) {
  const uint32_t m = blockIdx.y;
  uint8_t *row = box + (size_t)m * row_frags * 16u;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(row, row_frags * 16u);
  // Waiting must not steal the producers' bandwidth: a wave with unpublished fragments
  // watches one witness (the fragment of its lowest waiting lane; every lane loads the
  // same 16 B) and its lanes re-read their own fragments only once that is published.
  // The loop trip count is uniform per wave (the step is a multiple of 64).
  const int lane = threadIdx.x & 63;
  for (uint32_t base = blockIdx.x * 256u + (threadIdx.x & ~63u); base < row_frags; base += gridDim.x * 256u) {
    const uint32_t i = base + lane;
    const bool mine = i < row_frags;
    u32x4 w = buf_load<POL_LD>(r, mine ? i * 16u : 0x80000000u);
    bool ok = !mine || published(w);
    bool gave_up = false;
    for (uint64_t polls = 0;; ++polls) {
      const uint64_t waiting = __ballot(!ok);
      if (waiting == 0) break;
      if (polls >= spin_limit) {
        if (!ok) atomicOr(&g_status, 1u);
        gave_up = true;
        break;
      }
      const int wl = __ffsll((unsigned long long)waiting) - 1;
      const uint32_t *wp = reinterpret_cast<const uint32_t *>(row + (size_t)(base + wl) * 16u);
      if (!published(load_fragment_coherent(wp))) {
        __builtin_amdgcn_s_sleep(8);
        continue;
      }
      asm volatile("" ::: "memory");
      if (!ok) {
        w = buf_load<POL_LD>(r, i * 16u);
        ok = published(w);
      }
    }
    (void)gave_up;
    if (copy && mine && ok) {
      nt_store(w, out + (size_t)m * row_frags + i);
      buf_store<POL_ST>(sentinel4(), r, i * 16u);
    }
  }
}

}  // namespace arn

// gather_kernels.hpp -- the sentinel-cleaning Gather for gfx950.
//
// Method: vLLM DSpark drafter pages, "drafter.comm" (module prose, Gather entry and
// kernel): rank r's [M, S] shard of 32-bit words lands, cleaned, at columns r*S .. of
// the [cap, TP*S] mailbox rows; the reader polls every fragment of its rows and either
// copies them to a dense output and re-arms them, or leaves them published for a later
// reader.  One-GPU stand-in: the ranks' shards are pushed on the same GPU, by
// gather_push calls followed by gather_poll, or by the producer workgroups of one
// gather_push_poll launch ahead of its pollers.
#pragma once

#include "device.hpp"

namespace arn {

// One producer workgroup's share of a cleaned copy: fragments chunk*256 + t, strided
// by chunks*256, of `frags` contiguous source fragments into the buffer at dst.
// SRC_NT: read the source with non-temporal loads (the separate push kernels), else with
// the default policy (the producers of a one-launch call; see gather_push_poll_kernel).
template <int POL, bool SRC_NT = true>
__device__ __forceinline__ void push_frags(const u32x4 *__restrict__ src, uint8_t *dst, uint32_t frags,
                                           uint32_t chunk, uint32_t chunks) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(dst, frags * 16u);
  for (uint32_t i = chunk * 256u + threadIdx.x; i < frags; i += chunks * 256u)
    buf_store<POL>(clean4(SRC_NT ? nt_load(src + i) : src[i]), r, i * 16u);
}

// gather_push: slot s's shard rows [M, F] (F = S/4 fragments a row) are one contiguous range
// of n = M*F fragments, taken in blocks of 256 by a grid of ceil(n/256) x nslots workgroups:
// workgroup (b, s), thread t copies fragment i = b*256 + t, row m = i / F, column j = i % F,
// to row m of the mailbox at word offset (rank + s) * S + 4j.  No lane idles for a width that
// is not a multiple of 1024 words (a workgroup per row and chunk of 256 fragments left 32 of
// 256 lanes without work at S=896, and 255 at S=4).  The block's buffer resource spans the
// rows its fragments fall in, so it is uniform per workgroup, and a block within one row
// (every block when F is a multiple of 256) needs no per-lane division.  Measured at TP=8
// with gather_poll, µs per call, per row / flat (medians of 3): S=4 M=1000 5.50 / 4.04,
// M=70000 166.1 / 15.2; S=36 M=4096 13.54 / 6.84; S=896 M=300 7.84 / 7.94, M=1200 26.97 /
// 26.20, M=2400 52.44 / 51.93, M=4 and 32 within 0.01; S=10240 M=4 3.98 / 3.95, M=205 50.26 /
// 50.02.
template <int POL>
__global__ void __launch_bounds__(256)
gather_push_kernel(const u32x4 *__restrict__ shard, uint8_t *__restrict__ box, uint32_t frags, uint32_t n,
                   uint32_t row_bytes, uint32_t first_col_bytes) {
  const uint32_t s = blockIdx.y, first = blockIdx.x * 256u;
  const uint32_t cnt = n - first < 256u ? n - first : 256u;  // fragments of this block
  const uint32_t m0 = first / frags, c0 = first - m0 * frags;
  const bool one_row = c0 + cnt <= frags;
  const uint32_t rows = one_row ? 1u : (first + cnt - 1u) / frags - m0 + 1u;
  uint8_t *base = box + (size_t)m0 * row_bytes + first_col_bytes + (size_t)s * frags * 16u;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(base, (rows - 1u) * row_bytes + frags * 16u);
  if (threadIdx.x >= cnt) return;
  const uint32_t i = first + threadIdx.x;
  const uint32_t m = one_row ? m0 : i / frags, j = i - m * frags;
  buf_store<POL>(clean4(nt_load(shard + (size_t)s * n + i)), r, (m - m0) * row_bytes + j * 16u);
}

// The poll of a flat range of n fragments (the rows < M of a mailbox are one contiguous
// block, and so are those of `out`), with copy and re-arm.  Workgroup w of W takes blocks
// w, w + W, ... of 256*U fragments; in block b thread t owns fragments b*256*U + u*256 + t
// (u < U), issues their U loads together, then waits on its pending ones.  Each block gets
// a buffer resource of its own, so the range may span more than a resource's 4 GiB; lanes
// past the range end load out of range (0) and store nothing.  The block loop is uniform
// per workgroup.
//
// Waiting must not steal the producers' bandwidth: a wave with unpublished fragments
// watches one witness (the first pending fragment of its lowest waiting lane; every lane
// loads the same 16 B) and its lanes re-read their own pending fragments only once that is
// published; a small range (poll_all) re-reads every pending fragment on each pass
// instead, so the data arrives with the news.  The copy is stored with the cache policy
// POL_CP through a buffer resource per block.  Device scope (sc1) measured best: with the
// default policy the one-slot read at M=4096, width 7168 fetched 2 MB more than the 58.7
// MB it reads (1.0135 x its algorithmic bytes in all; 1.0004 with sc1) and took 31.6-31.8
// against 29.3-30.2 us from HBM; TP=8 Gathers at M=4 (one launch) 2.72-2.74 against
// 2.55-2.58 us, logits at M=4 (the pair) 4.20-4.21 against 3.97-3.98, the two-shot call at
// M=4 5.03-5.05 against 4.91-4.92.  A non-temporal store was slower (35.0 against 32.0 us
// at M=4096).
template <int POL_LD, int POL_ST, int POL_CP, int U>
__device__ __forceinline__ void poll_range(uint8_t *box, u32x4 *out, uint64_t n, uint32_t w, uint32_t W, int copy,
                                           uint64_t spin_limit, int poll_all) {
  constexpr uint32_t kBlk = 256u * U;
  const uint64_t nblk = (n + kBlk - 1) / kBlk;
  for (uint64_t b = w; b < nblk; b += W) {
    const uint64_t first = b * kBlk;
    const uint32_t cnt = (uint32_t)(n - first < kBlk ? n - first : kBlk);
    uint8_t *blk = box + first * 16u;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(blk, cnt * 16u);
    uint32_t idx[U];
    u32x4 v[U];
    uint32_t pend = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      idx[u] = u * 256u + threadIdx.x;
      v[u] = buf_load<POL_LD>(r, idx[u] < cnt ? idx[u] * 16u : 0x80000000u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (idx[u] < cnt && !published(v[u])) pend |= 1u << u;
    for (uint64_t polls = 0;; ++polls) {
      const uint64_t waiting = __ballot(pend != 0);
      if (waiting == 0) break;
      if (polls >= spin_limit) {
        if (pend) atomicOr(&g_status, 1u);
        break;
      }
      if (poll_all) {
        __builtin_amdgcn_s_sleep(1);
      } else {
        uint32_t first_pending = 0;
#pragma unroll
        for (int u = U - 1; u >= 0; --u)
          if ((pend >> u) & 1u) first_pending = idx[u];
        const uint32_t wi = __shfl(first_pending, __ffsll((unsigned long long)waiting) - 1, 64);
        if (!published(load_fragment_coherent(reinterpret_cast<const uint32_t *>(blk + (size_t)wi * 16u)))) {
          __builtin_amdgcn_s_sleep(8);
          continue;
        }
      }
      asm volatile("" ::: "memory");
#pragma unroll
      for (int u = 0; u < U; ++u)
        if ((pend >> u) & 1u) {
          v[u] = buf_load<POL_LD>(r, idx[u] * 16u);
          if (published(v[u])) pend &= ~(1u << u);
        }
    }
    if (copy) {
      const __amdgpu_buffer_rsrc_t o = make_rsrc(out + first, cnt * 16u);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (idx[u] < cnt && !((pend >> u) & 1u)) {
          buf_store<POL_CP>(v[u], o, idx[u] * 16u);
          buf_store<POL_ST>(sentinel4(), r, idx[u] * 16u);
        }
    }
  }
}

// gather_poll: the M rows < M as one range of n fragments, U fragments per thread in
// flight; the grid (at most 1024 workgroups) is resident at once.
template <int POL_LD, int POL_ST, int POL_CP, int U>
__global__ void __launch_bounds__(256)
gather_poll_kernel(uint8_t *__restrict__ box, u32x4 *__restrict__ out, uint64_t n, int copy, uint64_t spin_limit,
                   int poll_all) {
  poll_range<POL_LD, POL_ST, POL_CP, U>(box, out, n, blockIdx.x, gridDim.x, copy, spin_limit, poll_all);
}

// gather_push_poll in one launch, as the pages' Gather kernel pushes its shard and then
// polls the gathered row: workgroups [0, producers) push every rank's shard rows (the
// lowest ids, dispatched first), the rest poll the M gathered rows.
//
// The producers work by block of the gathered range, as the pollers do: producer b writes
// the range's fragments b*256 .. b*256+255, each from the rank and row it belongs to, and
// with the automatic poll layout (one fragment per thread while the range has at most 1024
// blocks, so a poller each) poller b polls exactly those.  `producers` is
// the block count rounded up to a multiple of 8 (the padding ids end at once), so that
// producer b and poller b, whose ids then agree mod 8, sit on one XCD (workgroup ids go to
// the eight XCDs in turn).  Measured at TP=8, µs per call, a producer per (rank, row) / per
// block: S=896 M=1 2.63-2.65 / 2.63-2.64, M=4 2.85-2.86 / 2.63, M=8 3.00-3.01 / 2.73-2.74,
// M=16 3.10-3.12 / 2.89-2.92; S=448 M=8 2.90-2.94 / 2.75-2.77, M=32 3.25-3.26 / 3.02;
// S=10240 M=1 2.79-2.80 / 2.80.  Without the padding, S=896 M=1 (7 blocks) took 2.72.
struct GatherStepArgs {
  const u32x4 *shard;  // [TP, M, F]
  uint8_t *box;        // [cap, TP*F*16 B]
  u32x4 *out;          // [M, TP*F]
  uint32_t frags;      // F = S/4 fragments of one rank's row
  uint32_t M;
  uint32_t producers;  // producer workgroups: ceil(M*TP*F / 256) rounded up to a multiple of 8
  uint32_t pollers;    // poller workgroups (poll_range over the M gathered rows)
  int copy;
  uint64_t spin_limit;
  int poll_all;
  uint32_t poll_delay;  // s_sleep(1) steps (64 cycles each) before a poller's first pass
};

template <int TP, int U, int POL_PUSH, int POL_LD, int POL_ST, int POL_CP>
__global__ void __launch_bounds__(256) gather_push_poll_kernel(GatherStepArgs a) {
  const uint32_t row_frags = TP * a.frags;
  const uint32_t n = a.M * row_frags;  // the gathered range: the host keeps it within 32 MiB
  if (blockIdx.x < a.producers) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i >= n) return;
    // fragment i of the gathered rows: row m, rank s's shard, its fragment j
    const uint32_t m = i / row_frags, c = i - m * row_frags, s = c / a.frags, j = c - s * a.frags;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(a.box, n * 16u);
    // the shard rows with the default cache policy: a caller's rows, just written, are
    // usually still in the last-level cache (non-temporal loads fetched them from HBM:
    // S=896 M=600 13.03 against 11.81 us, M=1000 22.56 / 20.31, logits M=64 16.82 / 14.63;
    // the same within 0.02 up to 8 MiB)
    buf_store<POL_PUSH>(clean4(a.shard[((size_t)s * a.M + m) * a.frags + j]), r, i * 16u);
    return;
  }
  // wait about as long as the producers' stores take: polling lines while they are written
  // slows the stores
  for (uint32_t i = 0; i < a.poll_delay; ++i) __builtin_amdgcn_s_sleep(1);
  poll_range<POL_LD, POL_ST, POL_CP, U>(a.box, a.out, n, blockIdx.x - a.producers, a.pollers, a.copy, a.spin_limit,
                                a.poll_all);
}

}  // namespace arn

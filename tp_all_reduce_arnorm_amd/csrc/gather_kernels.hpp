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
template <int POL>
__device__ __forceinline__ void push_frags(const u32x4 *__restrict__ src, uint8_t *dst, uint32_t frags,
                                           uint32_t chunk, uint32_t chunks) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(dst, frags * 16u);
  for (uint32_t i = chunk * 256u + threadIdx.x; i < frags; i += chunks * 256u)
    buf_store<POL>(clean4(nt_load(src + i)), r, i * 16u);
}

// gather_push: a 1-D grid of chunks * M * nslots workgroups, id = (s * M + m) * chunks + c;
// shard row m of slot s is F = S/4 contiguous fragments, written to row m at word offset
// (rank + s) * S, chunk c taking fragments c*256 + t, strided by chunks*256.
template <int POL>
__global__ void __launch_bounds__(256)
gather_push_kernel(const u32x4 *__restrict__ shard, uint8_t *__restrict__ box, uint32_t frags,
                   uint32_t M, uint32_t row_bytes, uint32_t first_col_bytes, uint32_t chunks) {
  const uint32_t sm = blockIdx.x / chunks, c = blockIdx.x - sm * chunks;  // sm = s * M + m
  const uint32_t s = sm / M, m = sm - s * M;
  push_frags<POL>(shard + (size_t)sm * frags, box + (size_t)m * row_bytes + first_col_bytes + (size_t)s * frags * 16u,
                  frags, c, chunks);
}

// The poll of one row's fragments by workgroup `cta` of `ctas` (cta*256 + t, strided by
// ctas*256), with copy and re-arm.  The copy is stored with the default cache policy, as
// the ArNorm consumer stores its rows: the last-level cache keeps it for the next reader
// (a non-temporal store made the one-slot read at M=4096, width 7168, 35.0 against
// 32.0 us from HBM, and changed nothing at small M).  Waiting must not steal the producers' bandwidth: a
// wave with unpublished fragments watches one witness (the fragment of its lowest
// waiting lane; every lane loads the same 16 B) and its lanes re-read their own
// fragments only once that is published; a small grid (poll_all) re-reads every
// pending fragment on each pass instead, so the data arrives with the news.  The loop
// trip count is uniform per wave (the step is a multiple of 64).
template <int POL_LD, int POL_ST>
__device__ __forceinline__ void poll_row(uint8_t *row, u32x4 *out_row, uint32_t row_frags, uint32_t cta,
                                         uint32_t ctas, int copy, uint64_t spin_limit, int poll_all) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(row, row_frags * 16u);
  const int lane = threadIdx.x & 63;
  for (uint32_t base = cta * 256u + (threadIdx.x & ~63u); base < row_frags; base += ctas * 256u) {
    const uint32_t i = base + lane;
    const bool mine = i < row_frags;
    u32x4 w = buf_load<POL_LD>(r, mine ? i * 16u : 0x80000000u);
    bool ok = !mine || published(w);
    for (uint64_t polls = 0;; ++polls) {
      const uint64_t waiting = __ballot(!ok);
      if (waiting == 0) break;
      if (polls >= spin_limit) {
        if (!ok) atomicOr(&g_status, 1u);
        break;
      }
      if (poll_all) {
        __builtin_amdgcn_s_sleep(1);
      } else {
        const int wl = __ffsll((unsigned long long)waiting) - 1;
        const uint32_t *wp = reinterpret_cast<const uint32_t *>(row + (size_t)(base + wl) * 16u);
        if (!published(load_fragment_coherent(wp))) {
          __builtin_amdgcn_s_sleep(8);
          continue;
        }
      }
      asm volatile("" ::: "memory");
      if (!ok) {
        w = buf_load<POL_LD>(r, i * 16u);
        ok = published(w);
      }
    }
    if (copy && mine && ok) {
      out_row[i] = w;
      buf_store<POL_ST>(sentinel4(), r, i * 16u);
    }
  }
}

// poll_row with U fragments per thread in flight, for a grid too large to give every
// fragment a thread of its own: workgroup `cta` of `ctas` takes blocks of 256*U
// fragments (blk + u*256 + t), strided by ctas*256*U, issues the U loads of a thread
// together, and waits on the thread's pending ones as poll_row does (the witness of a
// wave is the first pending fragment of its lowest waiting lane).  The block loop is
// uniform per workgroup; lanes past the row end load out of range (0) and store nothing.
template <int POL_LD, int POL_ST, int U>
__device__ __forceinline__ void poll_row_batch(uint8_t *row, u32x4 *out_row, uint32_t row_frags, uint32_t cta,
                                               uint32_t ctas, int copy, uint64_t spin_limit, int poll_all) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(row, row_frags * 16u);
  for (uint32_t blk = cta * 256u * U; blk < row_frags; blk += ctas * 256u * U) {
    uint32_t idx[U];
    u32x4 w[U];
    uint32_t pend = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      idx[u] = blk + u * 256u + threadIdx.x;
      w[u] = buf_load<POL_LD>(r, idx[u] < row_frags ? idx[u] * 16u : 0x80000000u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (idx[u] < row_frags && !published(w[u])) pend |= 1u << u;
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
        uint32_t first = 0;
#pragma unroll
        for (int u = U - 1; u >= 0; --u)
          if ((pend >> u) & 1u) first = idx[u];
        const uint32_t wi = __shfl(first, __ffsll((unsigned long long)waiting) - 1, 64);
        if (!published(load_fragment_coherent(reinterpret_cast<const uint32_t *>(row + (size_t)wi * 16u)))) {
          __builtin_amdgcn_s_sleep(8);
          continue;
        }
      }
      asm volatile("" ::: "memory");
#pragma unroll
      for (int u = 0; u < U; ++u)
        if ((pend >> u) & 1u) {
          w[u] = buf_load<POL_LD>(r, idx[u] * 16u);
          if (published(w[u])) pend &= ~(1u << u);
        }
    }
    if (copy) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (idx[u] < row_frags && !((pend >> u) & 1u)) {
          out_row[idx[u]] = w[u];
          buf_store<POL_ST>(sentinel4(), r, idx[u] * 16u);
        }
    }
  }
}

// gather_poll: a 1-D grid of ctas * M workgroups, id = m * ctas + cta; U fragments per
// thread in flight.
template <int POL_LD, int POL_ST, int U>
__global__ void __launch_bounds__(256)
gather_poll_kernel(uint8_t *__restrict__ box, u32x4 *__restrict__ out, uint32_t row_frags, uint32_t ctas,
                   int copy, uint64_t spin_limit, int poll_all) {
  const uint32_t m = blockIdx.x / ctas, cta = blockIdx.x - m * ctas;
  if constexpr (U == 1)
    poll_row<POL_LD, POL_ST>(box + (size_t)m * row_frags * 16u, out + (size_t)m * row_frags, row_frags, cta, ctas,
                             copy, spin_limit, poll_all);
  else
    poll_row_batch<POL_LD, POL_ST, U>(box + (size_t)m * row_frags * 16u, out + (size_t)m * row_frags, row_frags, cta,
                                      ctas, copy, spin_limit, poll_all);
}

// gather_push_poll in one launch, as the pages' Gather kernel pushes its shard and then
// polls the gathered row: workgroups [0, TP*M*per_row) are the producers of every rank's
// shard rows (the lowest ids, dispatched first), the rest poll the M gathered rows.
struct GatherStepArgs {
  const u32x4 *shard;  // [TP, M, F]
  uint8_t *box;        // [cap, TP*F*16 B]
  u32x4 *out;          // [M, TP*F]
  uint32_t frags;      // F = S/4 fragments of one rank's row
  uint32_t M;
  uint32_t per_row;    // producer workgroups per (rank, row)
  uint32_t ctas;       // poller workgroups per row
  int copy;
  uint64_t spin_limit;
  int poll_all;
};

template <int TP, int U, int POL_PUSH, int POL_LD, int POL_ST>
__global__ void __launch_bounds__(256) gather_push_poll_kernel(GatherStepArgs a) {
  const uint32_t row_frags = TP * a.frags;
  const uint32_t producers = TP * a.M * a.per_row;
  if (blockIdx.x < producers) {
    const uint32_t sm = blockIdx.x / a.per_row, chunk = blockIdx.x - sm * a.per_row;  // sm = s * M + m
    const uint32_t s = sm / a.M, m = sm - s * a.M;
    push_frags<POL_PUSH>(a.shard + (size_t)sm * a.frags, a.box + ((size_t)m * row_frags + (size_t)s * a.frags) * 16u,
                         a.frags, chunk, a.per_row);
    return;
  }
  const uint32_t c = blockIdx.x - producers, m = c / a.ctas, cta = c - m * a.ctas;
  if constexpr (U == 1)
    poll_row<POL_LD, POL_ST>(a.box + (size_t)m * row_frags * 16u, a.out + (size_t)m * row_frags, row_frags, cta,
                             a.ctas, a.copy, a.spin_limit, a.poll_all);
  else
    poll_row_batch<POL_LD, POL_ST, U>(a.box + (size_t)m * row_frags * 16u, a.out + (size_t)m * row_frags, row_frags,
                                      cta, a.ctas, a.copy, a.spin_limit, a.poll_all);
}

}  // namespace arn

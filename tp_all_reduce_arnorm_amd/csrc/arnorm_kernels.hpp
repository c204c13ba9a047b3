// arnorm_kernels.hpp -- the ArNorm producer and consumer kernels for gfx950.
//
// Method: vLLM DSpark drafter pages, "drafter.comm" (module prose, ArNorm entry and
// kernel), in the one-GPU stand-in of the two-shot page (owners = 1: TP local slots
// of one mailbox play the ranks).  The pages' design (one 8-CTA cluster per row,
// 112 threads of 8 columns, sums of squares exchanged through distributed shared
// memory, a multicast push) is NVIDIA prior art.  Here one workgroup owns a whole row,
// so the row's sum of squares never leaves the CU (per-thread FMA chains, a wave64
// butterfly or DPP sum, the wave sums added through LDS in wave order); at small M a row may
// instead be split over 7 or 14 workgroups, which exchange their parts through a
// sentinel-armed norm box, itself a small Lamport mailbox (reduce_row, K > 1).
#pragma once

#include "device.hpp"

namespace arn {

// ---------------------------------------------------------------------------------
// lamport_arm: fill `nfrag` fragments and `ntail` trailing words with the sentinel.
__global__ void __launch_bounds__(256)
arm_kernel(u32x4 *__restrict__ buf, size_t nfrag, uint32_t *__restrict__ tail, int ntail,
           uint32_t sentinel) {
  const u32x4 v = u32x4{sentinel, sentinel, sentinel, sentinel};
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nfrag; i += stride) buf[i] = v;
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = sentinel;
}

// ---------------------------------------------------------------------------------
// arnorm_push: slot s = blockIdx.y of the nslots pushed; each slot's M rows are one
// contiguous block of `frags` fragments in both the partial rows and the mailbox.
// U fragments per thread per step, loads first, so a wave has U x 1 KB in flight.  The
// partial rows are read non-temporally (SRC_NT) or with the default policy.
template <int U, int POL, bool SRC_NT>
__global__ void __launch_bounds__(256)
push_kernel(const u32x4 *__restrict__ partial, uint8_t *__restrict__ first_slot,
            size_t slot_stride_bytes, uint32_t frags) {
  const uint32_t s = blockIdx.y;
  const u32x4 *src = partial + (size_t)s * frags;
  const __amdgpu_buffer_rsrc_t dst = make_rsrc(first_slot + s * slot_stride_bytes, frags * 16u);
  const uint32_t step = gridDim.x * 256u * U;
  for (uint32_t base = blockIdx.x * 256u * U + threadIdx.x; base < frags; base += step) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t i = base + u * 256u;
      if (i < frags) v[u] = SRC_NT ? nt_load(src + i) : src[i];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t i = base + u * 256u;
      if (i < frags) buf_store<POL>(clean4(v[u]), dst, i * 16u);
    }
  }
}

// ---------------------------------------------------------------------------------
// arnorm_reduce_norm: one workgroup of NT threads per row (blockIdx.x); thread t owns
// fragments t, t + NT, ... (< 896), NF of them, so every wave instruction touches
// 1 KB of contiguous row.  Every access is a buffer instruction on a per-row resource
// of 14336 bytes, so the hot path has no branch: a fragment past the row end, the own
// slot of the fused form (a resource of 0 bytes) and the re-arm of a fragment whose
// poll timed out (offset kOffNone) are out of range, read as 0 and store nothing.
// All TP slot loads of a thread, its residual and gamma loads are in flight together.
struct ReduceArgs {
  const uint8_t *partial;   // [M, 14336 B] (FUSED only)
  const uint8_t *residual;  // [M, 14336 B] (RES only)
  const uint8_t *gamma;     // [14336 B]
  uint8_t *out;             // [M, 14336 B]
  uint8_t *res_out;         // [M, 14336 B]
  uint8_t *box;             // mailbox[parity]: [TP, cap, 14336 B]
  size_t slot_stride;       // cap * 14336 bytes
  uint32_t *nbox;           // norm_box[parity]: [cap, 256 words] (split rows only)
  uint32_t rows;            // M
  int rank;                 // own slot (FUSED only)
  int poll_all;             // later poll passes re-read every slot (small grids) instead of a witness
  float eps;
  uint64_t spin_limit;
  uint32_t poll_delay;      // s_sleep(1) steps (64 cycles each) before the first poll pass
};

constexpr int kNormBoxRowWords = 256;  // a row's inbox block: [K readers][K writers], K <= 14

constexpr uint32_t kOffNone = 0x80000000u;  // an offset past every resource

// Threads of a workgroup that owns one of a row's K parts (K divides 896): the part's
// 896 / K fragments, one per thread, rounded up to whole wave64s (K = 4: 224 -> 256,
// K = 8: 112 -> 128; the lanes past the part idle).  K = 1 is not a split.
constexpr int split_threads(int K) { return (kRowFrags / K + 63) / 64 * 64; }

// Occupancy target (waves per SIMD) asked of the compiler for a workgroup size.
constexpr int reduce_occupancy(int nt) {
  return nt == 896 ? ARNORM_WPE_896 : nt == 448 ? ARNORM_WPE_448 : nt == 256 ? ARNORM_WPE_256 : 0;
}

// K = workgroups per row.  K = 1: one workgroup of NT threads owns the whole row
// (fragments t, t + NT, ...).  K > 1 (small M, a grid small enough to be resident at
// once): workgroup k of the row owns fragments k*P .. k*P + P - 1 (P = 896 / K), one per
// thread (threads t >= P idle: their offsets are out of range), so each CU moves 1/K of
// the row; the row's sum of squares is then
// exchanged through the sentinel-armed norm box, itself a small Lamport mailbox: each
// workgroup writes its part into slot k of every peer's inbox, polls its own inbox,
// adds the K parts in workgroup order and re-arms its inbox.  A part is a sum of FMA
// products started from +0, so it is never -0, the sentinel word.
//
// `it` counts the rows a workgroup has done before this one (a whole-row workgroup may
// loop over rows): the wave sums alternate between two LDS buffers by its parity, so a
// wave that starts the next row cannot overwrite sums that a slower wave of the same
// workgroup is still reading (between two uses of one buffer every wave has passed the
// other row's barrier).
template <int TP, bool RES, bool FUSED, int NT, int K, int POL_LD, int POL_ST, int POL_IN, int POL_IO>
__device__ __forceinline__ void reduce_row(const ReduceArgs &a, const uint32_t row, const uint32_t k,
                                           const uint32_t it = 0) {
  constexpr int NF = K > 1 ? 1 : (kRowFrags + NT - 1) / NT;  // fragments per thread
  constexpr int NW = NT / 64;
  static_assert(NT % 64 == 0 && NW <= 16, "wave64 workgroups of at most 16 waves");
  static_assert(K == 1 || (kRowFrags % K == 0 && NT == split_threads(K) && K * K <= kNormBoxRowWords),
                "a split row is K parts of 896 / K fragments");
  constexpr uint32_t NP = K > 1 ? kRowFrags / K : kRowFrags;  // fragments of this workgroup's part
  __shared__ float wave_sums_buf[2][NW];
  __shared__ float row_total;
  float *wave_sums = wave_sums_buf[it & 1];

  const int t = threadIdx.x;
  const size_t row_off = (size_t)row * kRowBytes;
  const uint32_t base = k * NP;  // first fragment of this workgroup's part of the row
  uint32_t off[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f)
    off[f] = (K > 1 && NT > (int)NP && (uint32_t)t >= NP) ? kOffNone : (uint32_t)(base + t + f * NT) * 16u;

  const __amdgpu_buffer_rsrc_t gam = make_rsrc(a.gamma, kRowBytes);
  const __amdgpu_buffer_rsrc_t resr = make_rsrc(RES ? a.residual + row_off : nullptr, RES ? kRowBytes : 0);
  const __amdgpu_buffer_rsrc_t part = make_rsrc(FUSED ? a.partial + row_off : nullptr, FUSED ? kRowBytes : 0);
  const __amdgpu_buffer_rsrc_t rout = make_rsrc(a.res_out + row_off, kRowBytes);
  const __amdgpu_buffer_rsrc_t nout = make_rsrc(a.out + row_off, kRowBytes);
  __amdgpu_buffer_rsrc_t slot[TP];
#pragma unroll
  for (int s = 0; s < TP; ++s) {
    const bool own = FUSED && s == a.rank;
    slot[s] = make_rsrc(a.box + s * a.slot_stride + row_off, own ? 0u : (uint32_t)kRowBytes);
  }

  // In a launch that also holds the producers, wait about as long as their stores take
  // before the first poll pass: re-reading lines while they are written slows the stores.
  for (uint32_t i = 0; i < a.poll_delay; ++i) __builtin_amdgcn_s_sleep(1);

  // issue every load: gamma (L2-resident), residual, own partial, the TP slots
  u32x4 g[NF], res[NF], mine[NF], raw[TP][NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) g[f] = buf_load<kPolPlain>(gam, off[f]);
  if constexpr (RES) {
#pragma unroll
    for (int f = 0; f < NF; ++f) res[f] = buf_load<POL_IN>(resr, off[f]);
  }
  if constexpr (FUSED) {
#pragma unroll
    for (int f = 0; f < NF; ++f) mine[f] = buf_load<POL_IN>(part, off[f]);
  }
  // A whole-row workgroup's odd waves issue their slot loads from the last slot down
  // (the order of the sum does not change): the TP streams of a row then start at both
  // ends at once.  TP=8, M=4096 from HBM: 185.6-187.1 against 187.5-189.0 us over six
  // alternations on one box, the call as it runs unchanged; a rotation by wave index
  // was slower right after the push.
  if (K == 1 && ((t >> 6) & 1)) {
#pragma unroll
    for (int s = TP - 1; s >= 0; --s)
#pragma unroll
      for (int f = 0; f < NF; ++f) raw[s][f] = buf_load<POL_LD>(slot[s], off[f]);
  } else {
#pragma unroll
    for (int s = 0; s < TP; ++s)
#pragma unroll
      for (int f = 0; f < NF; ++f) raw[s][f] = buf_load<POL_LD>(slot[s], off[f]);
  }
  if constexpr (FUSED) {
#pragma unroll
    for (int s = 0; s < TP; ++s)
#pragma unroll
      for (int f = 0; f < NF; ++f) raw[s][f] = (s == a.rank) ? clean4(mine[f]) : raw[s][f];
  }

  // later poll passes, only while a producer is still writing.  Waiting must not steal
  // the producer's bandwidth: each wave watches one witness fragment (the first pending
  // one of its lowest waiting lane; every lane loads the same 16 B, one request) and only
  // when that is published do its lanes re-read all their slots together.  Re-reading a
  // published fragment is exact: it cannot change before this thread re-arms it.
  uint32_t pending = 0;  // bit s * NF + f: slot s of fragment f not yet published
#pragma unroll
  for (int s = 0; s < TP; ++s)
#pragma unroll
    for (int f = 0; f < NF; ++f)
      if (!published(raw[s][f])) pending |= 1u << (s * NF + f);
  uint32_t timed_out = 0;  // bit f: fragment f gave up
  if (__any(pending != 0)) {
    const int lane = t & 63;
    for (uint64_t polls = 0;; ++polls) {
      const uint64_t waiting = __ballot(pending != 0);
      if (waiting == 0) break;
      if (polls >= a.spin_limit) {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          uint32_t frag_bits = 0;
#pragma unroll
          for (int s = 0; s < TP; ++s) frag_bits |= 1u << (s * NF + f);
          if (pending & frag_bits) timed_out |= 1u << f;
        }
        if (pending) atomicOr(&g_status, 1u);
        break;
      }
      if (a.poll_all) {
        // a small grid: every pass re-reads all slots, so the data arrives with the news
        __builtin_amdgcn_s_sleep(1);
      } else {
        const int wl = __ffsll((unsigned long long)waiting) - 1;
        const int wbit = __shfl(__ffs(pending) - 1, wl, 64);  // s * NF + f of the witness
        const int ws = wbit / NF, wf = wbit % NF;
        const uint32_t *wp = reinterpret_cast<const uint32_t *>(
            a.box + ws * a.slot_stride + row_off + (size_t)(base + (t - lane + wl) + wf * NT) * 16u);
        if (!published(load_fragment_coherent(wp))) {
          __builtin_amdgcn_s_sleep(8);
          continue;
        }
      }
      asm volatile("" ::: "memory");
#pragma unroll
      for (int s = 0; s < TP; ++s)
#pragma unroll
        for (int f = 0; f < NF; ++f) raw[s][f] = buf_load<POL_LD>(slot[s], off[f]);
      if constexpr (FUSED) {
#pragma unroll
        for (int s = 0; s < TP; ++s)
#pragma unroll
          for (int f = 0; f < NF; ++f) raw[s][f] = (s == a.rank) ? clean4(mine[f]) : raw[s][f];
      }
      pending = 0;
#pragma unroll
      for (int s = 0; s < TP; ++s)
#pragma unroll
        for (int f = 0; f < NF; ++f)
          if (!published(raw[s][f])) pending |= 1u << (s * NF + f);
    }
  }

  // re-arm every slot read; a fragment that timed out is left for lamport_arm
#pragma unroll
  for (int s = 0; s < TP; ++s)
#pragma unroll
    for (int f = 0; f < NF; ++f) buf_store<POL_ST>(sentinel4(), slot[s], (timed_out >> f) & 1u ? kOffNone : off[f]);

  // rank-order sum, one BF16 rounding; residual add, one rounding; sum of squares
  float sq = 0.0f;
  u32x4 nres[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float lo = lo_f32(raw[0][f][j]);
      float hi = hi_f32(raw[0][f][j]);
#pragma unroll
      for (int s = 1; s < TP; ++s) {
        lo = lo + lo_f32(raw[s][f][j]);
        hi = hi + hi_f32(raw[s][f][j]);
      }
      uint32_t w = pack_bf16x2(lo, hi);
      if constexpr (RES) w = pack_bf16x2(lo_f32(w) + lo_f32(res[f][j]), hi_f32(w) + hi_f32(res[f][j]));
      nres[f][j] = w;
      sq = __builtin_fmaf(lo_f32(w), lo_f32(w), sq);
      sq = __builtin_fmaf(hi_f32(w), hi_f32(w), sq);
    }
    buf_store<POL_IO>(nres[f], rout, off[f]);
  }

  // the row's sum of squares: a wave sum, then wave sums in wave order.  A split row
  // (small M: the sum is on the call's chain of dependent steps) takes the DPP sum,
  // 0.15-0.2 us less per call at TP=8, M=1..8; a whole row keeps the butterfly, which
  // measured 0.5 points of 8 TB/s better at M=4096 from HBM (76.0 against 75.5 %).
  if constexpr (K > 1) sq = wave_sum_dpp(sq); else sq = wave_sum(sq);
  if ((t & 63) == 0) wave_sums[t >> 6] = sq;
  __syncthreads();
  float total = wave_sums[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) total = total + wave_sums[w];
  if constexpr (K > 1) {
    // `total` is this workgroup's part; wave 0 exchanges it with the row's K workgroups
    if (t < 64) {
      uint32_t *inbox = a.nbox + (size_t)row * kNormBoxRowWords;  // [reader][writer]
      if (t < K) __hip_atomic_store(inbox + t * K + k, __float_as_uint(total), __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
      uint32_t v = kSentinel;
      if (t < K) v = __hip_atomic_load(inbox + k * K + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (uint64_t polls = 0;; ++polls) {
        if (__ballot(t < K && v == kSentinel) == 0) break;
        if (polls >= a.spin_limit) {
          if (t == 0) atomicOr(&g_status, 1u);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
        if (t < K && v == kSentinel)
          v = __hip_atomic_load(inbox + k * K + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      float sum = lane_f32(__uint_as_float(v), 0);
#pragma unroll
      for (int j = 1; j < K; ++j) sum = sum + lane_f32(__uint_as_float(v), j);
      if (t < K && v != kSentinel)
        __hip_atomic_store(inbox + k * K + t, kSentinel, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (t == 0) row_total = sum;
    }
    __syncthreads();
    total = row_total;
  }
  const float rstd = 1.0f / sqrtf(total / (float)kHidden + a.eps);  // IEEE div and sqrt

#pragma unroll
  for (int f = 0; f < NF; ++f) {
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = nres[f][j];
      o[j] = pack_bf16x2((lo_f32(w) * rstd) * lo_f32(g[f][j]), (hi_f32(w) * rstd) * hi_f32(g[f][j]));
    }
    buf_store<POL_IO>(o, nout, off[f]);
  }
}

// K = 1: a grid of at most M workgroups, each taking rows blockIdx.x, blockIdx.x +
// gridDim.x, ... in turn.  The host caps the grid at what the GPU holds at once with room
// left beside it, so that a consumer launched before its producer (on another stream)
// never waits on a row whose workgroup could not be dispatched.
//
// K > 1: the workgroups come in blocks of 8 * K: workgroup c = 8 * K * b + 8 * k + j
// serves row 8 * b + j, part k (ids past the last row end at once).  The dispatcher hands
// workgroup ids to the eight XCDs in turn, so a row's K workgroups, whose ids agree mod 8,
// share one XCD and its L2 for the norm-box exchange; placement only, the results do not
// depend on it.  Measured at TP=8, push + consumer, us per call (rows split 4 ways, spread
// / one XCD per row): M=32 5.71-5.74 / 5.64-5.66, M=48 6.31-6.33 / 6.19-6.21, M=64
// 7.23-7.25 / 6.97-7.00, M=96 and 128 unchanged.  Deadlock freedom: with workgroups
// dispatched in id order, every workgroup of the lowest unfinished block has been
// dispatched (every lower id has finished), and a block (8 * K workgroups of at most 256
// threads) is resident at once many times over.
template <int TP, bool RES, bool FUSED, int NT, int K, int POL_LD, int POL_ST, int POL_IN, int POL_IO>
__global__ void __launch_bounds__(NT, reduce_occupancy(NT)) reduce_norm_kernel(ReduceArgs a) {
  if constexpr (K == 1) {
    uint32_t it = 0;
    for (uint32_t row = blockIdx.x; row < a.rows; row += gridDim.x, ++it)
      reduce_row<TP, RES, FUSED, NT, 1, POL_LD, POL_ST, POL_IN, POL_IO>(a, row, 0, it);
  } else {
    const uint32_t c = blockIdx.x, b = c / (8u * K), w = c - b * 8u * K;
    const uint32_t row = 8u * b + (w & 7u);
    if (row >= a.rows) return;  // a padding id of the last block
    reduce_row<TP, RES, FUSED, NT, K, POL_LD, POL_ST, POL_IN, POL_IO>(a, row, w >> 3);
  }
}

// ---------------------------------------------------------------------------------
// arnorm_push_reduce_norm in one launch: the pages' ArNorm kernel pushes a rank's row
// and then polls every slot, with no kernel boundary between a producer and its
// reader.  The one-GPU stand-in of such a call puts every rank's push in the same grid:
// workgroups [0, TP * per_slot) are the producers (per_slot of them per slot, the
// lowest workgroup ids, which the dispatcher places first), the others are the row
// consumers, split K ways (896/K threads each), which poll until the producers' stores
// land, re-arm and reduce.
//
// Consumer layout: the consumers come in blocks of 8 * K.  Consumer c = 8 * K * b + 8 * k +
// j serves row 8 * b + j, part k (ids past the last row end at once).  The dispatcher
// hands workgroup ids to the eight XCDs in turn, so a row's K workgroups, whose ids then
// agree mod 8, share one XCD and its L2 for the norm-box exchange.  Placement only: the
// results do not depend on it.  A block's rows interleave in id order, so the argument
// that the lowest unfinished row has all its workgroups dispatched needs the block (8 * K
// workgroups of at most 256 threads) resident at once, which any GPU of this family holds
// many times over.
struct StepArgs {
  ReduceArgs r;
  const u32x4 *partials;  // [TP, M, 896]
  uint32_t frags;         // M * 896: one slot's fragments, one block in the mailbox
  uint32_t per_slot;      // producer workgroups per slot
};

template <int TP, bool RES, int K, int U, int POL_PUSH, int POL_LD, int POL_ST, int POL_IN, int POL_IO>
__global__ void __launch_bounds__(split_threads(K)) push_reduce_kernel(StepArgs a) {
  constexpr int NT = split_threads(K);
  const uint32_t producers = TP * a.per_slot;
  if (blockIdx.x < producers) {
    const uint32_t s = blockIdx.x / a.per_slot, p = blockIdx.x - s * a.per_slot;
    const u32x4 *src = a.partials + (size_t)s * a.frags;
    const __amdgpu_buffer_rsrc_t dst = make_rsrc(a.r.box + s * a.r.slot_stride, a.frags * 16u);
    // The partial rows are read with the default cache policy: a caller's rows, just
    // written by the step before, are usually still in the last-level cache.  Non-temporal
    // loads fetched them from HBM, and from M=55 a few producers then ended late enough to
    // cost 0.4-1.2 us per call (TP=8, medians of 3 alternations, non-temporal / default: M=55
    // 5.78 / 5.37, M=59 6.66 / 5.64, M=62 6.98 / 5.80, M=63 6.76 / 5.83, M=64 6.28 / 5.88;
    // M=1..56 within 0.02).
    for (uint32_t i0 = p * NT * U + threadIdx.x; i0 < a.frags; i0 += a.per_slot * NT * U) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t i = i0 + u * NT;
        if (i < a.frags) v[u] = src[i];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t i = i0 + u * NT;
        if (i < a.frags) buf_store<POL_PUSH>(clean4(v[u]), dst, i * 16u);
      }
    }
    return;
  }
  const uint32_t c = blockIdx.x - producers;
  const uint32_t b = c / (8u * K), w = c - b * 8u * K;
  const uint32_t row = 8u * b + (w & 7u);
  if (row >= a.frags / kRowFrags) return;  // a padding id of the last block
  reduce_row<TP, RES, false, NT, K, POL_LD, POL_ST, POL_IN, POL_IO>(a.r, row, w >> 3);
}

}  // namespace arn

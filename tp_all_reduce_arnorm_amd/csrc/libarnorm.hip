// libarnorm.hip -- the C ABI declared in include/arnorm.h: argument validation, launch
// geometry and dispatch to the gfx950 kernels.  One translation unit, so the device
// status word has a single definition per device.
#include <algorithm>
#include <atomic>
#include <cstdint>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>

#include "arnorm.h"
#include "arnorm_kernels.hpp"
#include "gather_kernels.hpp"
#include "twoshot_kernels.hpp"

// The norm box of arnorm_push_reduce_norm_static: 64 rows of 256 words (64 KiB), one
// parity, on every device the library runs on, held until the process ends.  Host code
// never uses this name as an address: each device's own address comes from
// hipGetSymbolAddress (static_scratch below).
constexpr int kScratchRows = 64;
static __device__ __align__(256) uint32_t scratch[kScratchRows * arn::kNormBoxRowWords];

namespace {

using arn::u32x4;

// The device address of `scratch` on the current device: looked up with
// hipGetSymbolAddress on a device's first call, with that device current, and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint32_t *g_scratch_ptr[kMaxDevices] = {};

int static_scratch(uint32_t **ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ARNORM_HIP_ERROR;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return ARNORM_HIP_ERROR;
    g_scratch_ptr[dev] = static_cast<uint32_t *>(p);
  }
  *ptr = g_scratch_ptr[dev];
  return ARNORM_OK;
}

std::atomic<uint64_t> g_spin_limit{uint64_t(1) << 22};
std::atomic<int> g_reduce_threads{0};
std::atomic<int> g_reduce_split{0};
std::atomic<int> g_poll_frags{0};  // Gather polls: fragments per thread in flight, 0 = automatic
std::atomic<int> g_poll_mode{0};   // Gather polls: 0 = automatic, 1 = re-read all, 2 = witness

// Cache policies (gfx950 cache bits, see device.hpp).  Slot reads, re-arm writes and
// pushes are device-scope coherent (sc1); the re-arm writes are also non-temporal
// (nothing reads the sentinel back until the next push of that parity overwrites it);
// the residual (and the own partial of the fused form), read once, is non-temporal
// (TP=8, M=4096: 84 against 83.4 % of 8 TB/s right after the push, 75.2 against 74.3 %
// from HBM).  Measured on MI355X at TP=8, M=4096: the non-temporal re-arm took the
// consumer from 201 to 169 us, while a non-temporal slot read slowed it (183 us) and a
// non-temporal push slowed the small-M calls.  The ArNorm output rows (out, residual_out)
// and the polls' copies (Gather out, the two-shot read) are stored at device scope too:
// against the default policy, the consumer at M=4096 from HBM 186.2-186.7 against
// 188.0-188.6 us (right after the push unchanged, 165.9-167.3 against 166.6-166.8), the
// ArNorm call at M=64 6.74-6.81 against 6.91-6.93 us and at M=8 4.92 against 4.96; the
// copies as in poll_range.  The macros let a build measure other choices.
#ifndef ARNORM_POL_POLL
#define ARNORM_POL_POLL 16
#endif
#ifndef ARNORM_POL_REARM
#define ARNORM_POL_REARM 18
#endif
#ifndef ARNORM_POL_PUSH
#define ARNORM_POL_PUSH 16
#endif
#ifndef ARNORM_POL_IN
#define ARNORM_POL_IN 2
#endif
#ifndef ARNORM_POL_IO
#define ARNORM_POL_IO 16
#endif
#ifndef ARNORM_POL_COPY
#define ARNORM_POL_COPY 16
#endif
// Producer kernel (arnorm_push, twoshot_push) layout: 2 fragments per thread while a
// slot's rows total at most ARNORM_PUSH_SMALL_BYTES, else one fragment per thread with
// up to ARNORM_PUSH_MAX_GRID workgroups per slot (larger pushes loop).  The small layout
// reads the partial rows with the default cache policy, the large one non-temporally:
// measured at TP=8 (us, default / non-temporal), the call at M=64 as the pair 6.90-6.95 /
// 7.11-7.19 (M=16 unchanged), the push of 8 slots at M=4096 142.3-142.9 / 133.5-133.8
// from HBM and the call there 325.9-327.0 / 307.0-312.9.  Measured on
// MI355X at TP=8.  Small: us per call of the pair push + consumer, graph-replayed,
// fragments per thread 1 / 2 / 4 / 8: M=16 5.12 / 5.12-5.13 / 5.21-5.22 / 5.47, M=32
// 5.74 / 5.53-5.54 / 5.63 / 5.80, M=64 7.36 / 7.29-7.30 / 7.53 / 7.50.  Large: the push of
// 8 slots at M=4096, us from HBM / right after the consumer / push + consumer as the
// call repeats: 4 per thread, at most 1024 workgroups 134.4-134.7 / 155.2-157.4 /
// 320.0-323.8; 2 per thread, 7168 workgroups 128.5-128.8 / 150.9-151.5 / 316.0-316.9;
// 1 per thread, 14336 workgroups 134.1-134.2 / 144.7-145.4 / 309.8-310.2; 1 per thread,
// at most 8192 131.3-131.7 / 147.4-148.1 / 312.2-312.6, at most 4096 134.1-134.6 /
// 157.9-158.6 / 322.7-323.0.
#ifndef ARNORM_PUSH_U
#define ARNORM_PUSH_U 1
#endif
#ifndef ARNORM_PUSH_U_SMALL
#define ARNORM_PUSH_U_SMALL 2
#endif
#ifndef ARNORM_PUSH_SMALL_BYTES
#define ARNORM_PUSH_SMALL_BYTES (1u << 20)
#endif
#ifndef ARNORM_PUSH_MAX_GRID
#define ARNORM_PUSH_MAX_GRID 16384
#endif
// Rows split over 7 workgroups when a norm box is given and M <= ARNORM_SPLIT7_MAX_M,
// over 4 up to ARNORM_SPLIT4_MAX_M, else one workgroup per row.  Measured on MI355X at
// TP=8, us per call (graph replay; arnorm_push_reduce_norm, so one launch up to M=9, the
// pair above), rows split 1 / 4 / 7 ways: M=8 6.42 / 5.07-5.20 / 4.88-4.96, M=16 6.43-6.48
// / 5.25-5.31 / 5.06-5.11, M=32 6.73-6.76 / 5.73-5.75 / 5.54-5.59, M=48 7.15-7.17 /
// 6.34-6.36 / 6.74-6.81, M=64 7.82-8.35 / 7.03-7.07 / 7.32-7.45, M=96 11.20-11.22 /
// 10.52-10.54 / 10.81-10.88, M=128 12.84-12.85 / 12.62-12.63 / 13.24-13.29, M=192 17.54-17.58
// / 17.77-17.80, M=256 21.41-21.45 / 21.98-22.03 (14 ways was slower than 7 everywhere,
// 8 slower than 7 and 4).  Measured again with the rows of a split on one XCD (4 / 7 ways):
// M=32 5.57-5.60 / 5.41-5.42, M=33 5.61-5.67 / 5.58-5.62, M=34 5.64-5.72 / 5.89-5.93, M=36
// 5.77-5.81 / 6.11-6.18, M=40 5.90-5.92 / 6.27-6.28, M=48 6.14-6.15 / 6.58-6.63: 7 ways
// while an XCD's 32 CUs hold its rows' workgroups (4 rows of 7 each up to M=32).  At M=33,
// with the one launch's poll delay and a row on one XCD there too, 4 / 7 ways: one launch
// 4.68-4.69 / 4.93-4.95, the pair 5.67-5.70 / 5.92-5.96; so 4 from M=33.  And 1 way / 4 ways: M=120 12.18-12.22 / 12.00-12.02, M=128 12.52-12.64 /
// 12.40-12.49, M=130 12.74-12.79 / 13.48-13.50, M=136 13.04-13.09 / 13.93-13.96, M=160
// 14.82-14.92 / 15.62-15.67, M=192 17.31-17.32 / 17.73-17.76: 4 ways up to M=128.
#ifndef ARNORM_SPLIT7_MAX_M
#define ARNORM_SPLIT7_MAX_M 32
#endif
#ifndef ARNORM_SPLIT4_MAX_M
#define ARNORM_SPLIT4_MAX_M 128
#endif
// arnorm_push_reduce_norm, one-launch form: fragments per producer thread per step.
#ifndef ARNORM_STEP_PUSH_U
#define ARNORM_STEP_PUSH_U 2
#endif
// arnorm_push_reduce_norm, one-launch form: a row's consumer workgroups are placed on one
// XCD (push_reduce_kernel), at every M, and rows split the automatic K ways (7, or 4 from
// M=34).  Measured on MI355X at TP=8 with the poll delay below, us per call, HIP-graph
// replay, medians of 3 alternations on one box (fresh buffers each time).  One XCD per row
// against spread rows (workgroup c serving row c / K, part c % K): M=1 3.74 / 3.89, M=2
// 3.82 / 3.94, M=4 3.83-3.84 / 3.91, M=5 3.83 / 3.98, M=6 3.88 / 3.99, M=8 3.89 / 4.00;
// up to M=64 against one XCD per row only to M=8: M=12 4.07 / 4.11, M=16 4.11 / 4.16, M=24
// 4.35 / 4.33, M=32 4.45 / 4.49, M=40 4.95 / 4.96, M=48 5.10 / 5.22, M=64 6.59 / 6.68.
// Without the delay, spread rows had won from M=4 (4.14-4.35 against 4.21-4.44) and 8 ways
// had beaten 7 at M=5..9; with it, 7 / 8 ways on spread rows, two runs: M=4 3.95-3.96 /
// 4.06, M=5 4.00-4.02 / 4.07-4.09, M=6 4.03 / 4.10-4.11, M=7 4.03 / 4.09-4.12, M=8
// 4.02-4.05 / 4.11-4.13, M=9 4.10 / 4.17-4.19.
// The re-arm stores inside the one-launch calls (ArNorm, the Gather and the two-shot
// call), whose pollers re-read lines while their producers write them: device scope
// without the non-temporal bit.  ArNorm, before the poll delay, on six boxes: the
// consumers spread with these re-arms against one XCD per row with non-temporal ones,
// M=2 4.25-4.31 / 4.10-4.16, M=4 4.34-4.38 / 4.11-4.33 on five boxes (4.43 / 4.59 on the
// sixth), M=8 4.90-5.06 / 4.74-4.97, M=9 5.00-5.10 / 4.86-5.03, M=5..7 mixed, -0.25..+0.12.
// The others against ARNORM_POL_REARM (medians of 4 alternations on one box, us per call): Gathers at TP=8, S=896, M=4 2.54 / 2.28, M=16
// 2.77 / 2.38, M=32 3.29 / 2.99; logits at M=1 2.68 / 2.34; the context-projection gather
// (S=448, M=64) 3.25 / 2.97; the two-shot call at M=1 4.50 / 4.09, M=4 4.91 / 4.53, M=8
// 4.70 / 4.29.  The launches that run after their producer (the pair of ArNorm launches,
// gather_poll, twoshot_reduce and twoshot_read) keep ARNORM_POL_REARM: the ArNorm pair at
// M=12..128 measured the same with either, and the M=4096 kernels faster with it.
#ifndef ARNORM_POL_REARM_STEP
#define ARNORM_POL_REARM_STEP 16
#endif
// Fragments per thread in flight in a Gather poll whose grid is capped below a thread
// per fragment.
#ifndef ARNORM_POLL_U
#define ARNORM_POLL_U 4
#endif
// A consumer grid whose TP slots of rows < M total at most this many bytes re-reads all
// of them on every later poll pass (the data arrives with the news); a larger one
// watches one witness fragment per wave, so that waiting does not starve the producer.
#ifndef ARNORM_POLL_ALL_MAX_BYTES
#define ARNORM_POLL_ALL_MAX_BYTES (1u << 20)
#endif
// arnorm_push_reduce_norm runs as one launch (with a norm box) up to ARNORM_STEP_MAX_M rows
// whose TP slots total at most ARNORM_STEP_MAX_BYTES, in a grid of at most
// ARNORM_STEP_MAX_GRID workgroups (the limit that binds at TP <= 8), else as the pair.  Its consumers wait
// ARNORM_STEP_POLL_DELAY s_sleep steps of 64 cycles (ARNORM_STEP_POLL_DELAY_SPLIT4 and its ramp
// for rows split 4 or 2 ways) before their first poll pass, about as long as the producers' stores take
// to land: polling the lines while they are written slowed the stores.  Measured at TP=8,
// us per call, medians of 2 (delay 0 / 16 / 24 / 32 / 48 steps): M=1 3.81 / 3.96-3.98 /
// 3.69 / 3.89 / 4.32, M=4 4.22-4.25 / 3.98-4.05 / 4.12 / 4.32-4.33 / 4.75-4.76, M=8
// 4.86-4.90 / 4.51-4.54 / 4.17-4.18 / 4.39-4.40 / 4.81, M=16 5.44 / 4.73 / 4.30 / 4.51 /
// 4.94-4.95, M=32 6.80-6.81 / 5.18 / 4.56 / 4.77 / 5.20; split 4 ways M=34 6.26-6.27 / - /
// 5.28-5.30 / 4.79-4.80 / 5.22, M=40 6.56 / - / 5.56 / 4.95 / 5.36-5.37, M=64 7.85-7.88 / - /
// 6.84-6.86 / 6.61-6.62 / 6.31-6.38; the pair at M=32 5.38, M=40 5.90, M=64 6.75-6.79.
// On a second box, delay 0 / 24 / 32: TP=8 M=4 4.10-4.11 / 3.96 / 4.16, M=40 6.54 / 5.52-5.53
// / 4.96-4.97, M=64 7.83-7.85 / 6.83-6.85 / 6.66-6.67; TP=4 M=16 4.60-4.67 / 3.76-3.85 /
// 3.97-4.06; TP=2 M=4 3.78-3.83 / 3.53 / 3.74.  Finer, on two more boxes (delay 16 / 18 / 20 /
// 22 / 24): M=1 4.06-4.11 / 3.82-3.98 / 3.70-3.74 / 3.75-3.76 / 3.78-3.83, M=4 4.07-4.16 /
// 3.87-3.90 / 3.84-3.89 / 3.92-3.94 / 3.96-3.99, M=8 4.47-4.55 / 4.44 / 4.08-4.16 / 4.08 /
// 4.12-4.14, M=16 4.58-4.64 / 4.48-4.54 / 4.08-4.13 / 4.11-4.16 / 4.15-4.22.  Too short a
// delay falls off a cliff (16 to 18 here); 22 keeps a margin above it.  Rows split 4 ways
// wait one step more per two rows above ARNORM_STEP_POLL_DELAY_RAMP_M (M=64: 40 steps).
// With the producers' default-policy loads, medians of 3 alternations, constant delay 32 /
// 36: M=40 4.90 / 4.99, M=48 5.15 / 5.14, M=56 5.66 / 5.34, M=64 6.36 / 5.85; the ramp of one
// step per row (M=64: 48 steps) / this one, medians of 4: M=56 5.41 / 5.34, M=60 5.67 /
// 5.59, M=64 5.88 / 5.67, M=33..51 within 0.03.  The ramp ends at ARNORM_STEP_POLL_DELAY_RAMP_END
// rows: above it a constant 40 steps measured best or within 0.15 us (one launch, medians of
// 3, the ramp continued / constant 24 / 32 / 40): M=65 6.34 / 6.74 / 6.45 / 6.33, M=80 7.12 /
// 7.41 / 7.20 / 7.02, M=96 8.83 / 8.89 / 8.83 / 8.77, M=112 10.58 / 9.90 / 9.96 / 9.91, M=128
// 12.08 / 11.64 / 11.45 / 11.40.  The one launch beats the pair up to M=128 (the pair: M=65
// 7.57, M=80 9.02, M=96 10.46, M=112 11.50, M=128 12.48), and with rows split 4 ways up to
// ARNORM_STEP_SPLIT4_MAX_M also above, where the pair takes whole rows (one launch / the
// pair, medians of 3: M=129 11.32 / 12.79, M=144 12.60 / 13.63, M=160 14.05 / 15.02, M=192
// 16.68 / 17.32, M=224 18.54 / 19.26, M=256 20.63 / 21.25; the pair with 4-way rows was
// slower still, M=192 17.65), and then with rows split 2 ways (448-thread workgroups)
// (one launch / the pair: M=257 20.04 / 23.64, M=300 22.68 / 25.79, M=384 28.56 / 30.85,
// M=448 33.29 / 34.46, M=512 38.02 / 38.65) while its grid holds at most
// ARNORM_STEP_MAX_GRID workgroups (TP=8: M <= 562, TP=4: M <= 936, TP=2: M <= 1024).  Past
// about 6000 workgroups the one launch fell behind the pair, by a margin that grew with M
// and at a size that moved between boxes; below it, it won on every box (µs per call,
// medians of 3, calls chained through residual_out, one launch / the pair; TP=8, 10 M
// workgroups: M=513 39.06-39.36 / 42.14-42.19, M=544 41.56-42.10 / 43.92-44.02, M=560
// 42.83-43.98 / 44.46-44.62, M=576 (5760) 44.01-44.14 / 45.42-45.66, M=600 50.12 / 46.85 and
// M=608 46.06 / 47.75 on two boxes, M=640 53.2 / 49.6-49.9, M=1024 89.8-90.4 / 74.9-75.1;
// TP=4, 6 M workgroups: M=513 22.21 / 25.17, M=768 31.20 / 33.42, M=896 (5376) 36.41-37.66 /
// 38.61-38.64, M=1024 (6144) 47.79 / 42.96 and 41.98 / 42.71 on two boxes; TP=2, 4 M
// workgroups: M=513 13.62 / 15.58, M=1024 24.52 / 26.12).  Consumers that watch one witness
// per wave instead of re-reading every slot left that loss as it was (TP=8 M=640 53.24, M=1024
// 90.62).  The workgroup count stands in for an edge it does not cause: producers of 4
// fragments per thread (TP=8: 6 M workgroups) lost from the same M=640 (54.09 against 49.82).  From about M=100 at TP=8 the grid is larger than what the GPU holds at once,
// which the dispatch order allows (producers wait on nothing, and a row's consumers come in
// one block).
#ifndef ARNORM_STEP_MAX_BYTES
#define ARNORM_STEP_MAX_BYTES (64u << 20)
#endif
#ifndef ARNORM_STEP_MAX_M
#define ARNORM_STEP_MAX_M 1024
#endif
#ifndef ARNORM_STEP_MAX_GRID
#define ARNORM_STEP_MAX_GRID 5632
#endif
#ifndef ARNORM_STEP_SPLIT4_MAX_M
#define ARNORM_STEP_SPLIT4_MAX_M 256
#endif
#ifndef ARNORM_STEP_SPLIT2_MAX_M
#define ARNORM_STEP_SPLIT2_MAX_M 1024
#endif
#ifndef ARNORM_STEP_POLL_DELAY
#define ARNORM_STEP_POLL_DELAY 22
#endif
#ifndef ARNORM_STEP_POLL_DELAY_SPLIT4
#define ARNORM_STEP_POLL_DELAY_SPLIT4 32
#endif
#ifndef ARNORM_STEP_POLL_DELAY_RAMP_M
#define ARNORM_STEP_POLL_DELAY_RAMP_M 48
#endif
#ifndef ARNORM_STEP_POLL_DELAY_RAMP_END
#define ARNORM_STEP_POLL_DELAY_RAMP_END 64
#endif
// gather_push_poll runs as one launch when the gathered rows total at most this many
// bytes, its pollers waiting ARNORM_GATHER_STEP_POLL_DELAY s_sleep steps (8 more above 2
// MiB, 16 more above 4 MiB, 8 more above 8 MiB) and then re-reading every pending fragment per pass, else as the pair
// gather_push + gather_poll.  Measured on MI355X at TP=8 (HIP-graph replay, us per call,
// medians of 2, the pair / one launch with delay 0 / 16 / 24 / 32): S=896 M=4 3.50 / 2.33-2.36
// / 2.27-2.28 / 2.49 / 2.70, M=32 3.66-3.72 / 2.70-2.71 / 2.43 / 2.64-2.65 / 2.86, M=64 (1.84
// MB) 4.16 / 5.47-5.56 / 2.66-2.68 / 2.87-2.89 / 3.08-3.10; S=10240 M=1 3.53 / 2.39-2.40 /
// 2.32 / 2.53 / 2.74, M=4 3.97 / 3.69-3.76 / 2.57 / 2.77-2.78 / 2.99, M=8 (2.6 MB) 4.48 /
// 5.68-5.73 / 3.45-3.47 / 3.13-3.14 / 3.35-3.37, M=16 (5.2 MB) 5.81 / - / 5.35 / 4.66 / 4.62,
// M=32 (10.5 MB) 8.50 / - / 8.32 / 8.49 / 8.60.  Finer, on two boxes (delay 10 / 12 / 14 /
// 16): S=896 M=4 2.20 / 2.17-2.19 / 2.23 / 2.25-2.29, M=32 2.73 / 2.35-2.39 / 2.38-2.39 /
// 2.43-2.44; logits M=4 2.74-2.75 / 2.43-2.48 / 2.51-2.52 / 2.55-2.57: 14 keeps a margin above
// the cliff at 10.  Above 8 MiB, medians of 3 on one box, the pair / one launch with 22 / 30
// / 38 more steps: S=896 M=300 (8.6 MB) 7.86 / 6.59 / 6.65 / 6.72, M=400 9.89 / 8.71 / 8.84 /
// 9.03, M=600 15.25 / 13.04 / 13.13 / 13.19, M=1000 22.76 / 22.55 / 22.68 / 22.83; logits M=26
// 7.79 / 6.29 / 6.43 / 6.65, M=48 13.53 / 12.01 / 12.08 / 12.20, M=64 17.39 / 16.85 / 16.98 /
// 17.10.  Above 32 MiB, with the producers' default-policy loads (the pair / one launch,
// medians of 3): S=896 M=1200 (34.4 MB) 26.99 / 25.21, M=1600 34.73 / 34.25, M=2340 51.20 /
// 50.37, M=3600 (103 MB) 77.00 / 83.09, but the drafter's logits rows (S=10240) gain nothing
// there: M=103 25.47 / 24.53, M=128 30.87 / 31.51, M=160 39.18 / 39.38, M=192 47.35 / 46.95,
// M=204 50.10-50.19 / 51.97-52.23 on two boxes.  (At S=896 the pair's push leaves 32 of each
// 256 lanes idle, 224 fragments to a row.)  So the limit stays at 32 MiB.
#ifndef ARNORM_GATHER_STEP_MAX_BYTES
#define ARNORM_GATHER_STEP_MAX_BYTES (32u << 20)
#endif
#ifndef ARNORM_GATHER_STEP_POLL_DELAY
#define ARNORM_GATHER_STEP_POLL_DELAY 14
#endif
static_assert(ARNORM_GATHER_STEP_MAX_BYTES <= (1u << 30), "the one-launch Gather range is one buffer resource");
// Steps of the one-launch Gather's poll delay for a gathered range of `bytes`.
uint32_t gather_step_delay(uint64_t bytes) {
  return bytes <= (2u << 20)   ? ARNORM_GATHER_STEP_POLL_DELAY
         : bytes <= (4u << 20) ? ARNORM_GATHER_STEP_POLL_DELAY + 8
         : bytes <= (8u << 20) ? ARNORM_GATHER_STEP_POLL_DELAY + 16
                               : ARNORM_GATHER_STEP_POLL_DELAY + 8;
}
// twoshot_push_reduce_read runs as one launch when the TP slots of rows < M total at
// most this many bytes, its owners and readers waiting ARNORM_TWOSHOT_STEP_POLL_DELAY
// s_sleep steps (6 more above 2 MiB of slots) and then re-reading every pending fragment on
// each poll pass, else as its three launches.  Measured at TP=8, width 7168, with the re-arms of ARNORM_POL_REARM_STEP
// (us per call, medians of 2, three launches / one launch with delay 0 / 16 / 24 / 32):
// M=1 - / 4.04-4.06 / 3.86-3.87 / 4.07 / 4.27-4.29, M=4 6.22-6.29 / 4.44-4.45 / 4.05-4.06 /
// 4.26-4.27 / 4.47-4.48, M=16 6.43-6.44 / 4.75 / 4.29-4.30 / 4.50-4.51 / 4.71-4.72, M=32
// 6.84-6.87 / 6.65 / 4.82-4.83 / 4.99-5.00 / 5.20-5.22, M=48 7.48-7.54 / 7.94-7.95 / 5.59-5.63
// / 5.72-5.77 / 5.93-5.98, M=64 8.17-8.23 / 7.51 / 6.47-6.68 / 6.69-6.74 / 6.91-6.97, M=96
// 11.45 / - / 11.53 / 11.19 / 11.09, M=128 13.19 / - / 13.43 / 13.27 / 13.23.  Finer, on two
// boxes (delay 4 / 6 / 8 / 10 / 12): M=1 3.91 / 3.77-3.81 / 3.68-3.70 / 3.69-3.70 / 3.74-3.75,
// M=4 4.03-4.06 / 3.92-3.95 / 3.86-3.89 / 3.87-3.89 / 3.91-3.95, M=16 4.26-4.28 / 4.20 /
// 4.12-4.14 / 4.13-4.14 / 4.16-4.17.  Above 2 MiB (M=18 at TP=8) 16 steps: medians of 3 on
// one box, delay 10 / 16 / 24: M=16 4.13 / 4.25 / 4.47, M=20 4.43 / 4.37 / 4.58, M=24 4.93 /
// 4.50 / 4.70, M=28 5.43 / 4.67 / 4.84, M=32 5.74 / 4.82 / 4.97, M=40 6.01 / 5.33 / 5.44, M=48
// 6.07 / 5.67 / 5.73, M=56 6.14 / 6.20 / 6.41, M=64 6.82 / 6.53 / 6.71, M=73 7.38 / 7.19 / 7.34.
// Above 8 MiB, with the producers' default-policy loads, three launches / one launch with
// 16 / 24 / 32 steps: M=74 10.17 / 9.78 / 9.12 / 8.94, M=75 - / 7.86 / 8.01 / 8.23, M=80 10.14
// / 8.18 / 8.37 / 8.61, M=96 11.15 / 9.48 / 9.63 / 9.85, M=128 13.11 / 12.22 / 12.39 / 12.60,
// M=160 - / 15.12 / 15.00 / 15.12, M=224 - / 19.45 / 19.50 / 19.62, M=292 - / 23.54 / 23.59 /
// 23.76 (M=74 is slower than its neighbours at every delay).  Above 32 MiB (M=293), three
// launches / one launch with 16 steps, medians of 3: M=300 27.19 / 24.32, M=400 33.92 /
// 30.53, M=600 (68.8 MB) 49.06 / 45.79, M=1000 (115 MB) 75.97 / 78.02; the limit sits at 64
// MiB (M=585 at TP=8), below that loss.
#ifndef ARNORM_TWOSHOT_STEP_MAX_BYTES
#define ARNORM_TWOSHOT_STEP_MAX_BYTES (64u << 20)
#endif
#ifndef ARNORM_TWOSHOT_STEP_POLL_DELAY
#define ARNORM_TWOSHOT_STEP_POLL_DELAY 10
#endif
// Steps of the one-launch two-shot call's poll delay for TP slots of `bytes` (rows < M).
uint32_t twoshot_step_delay(uint64_t bytes) {
  return bytes <= (2u << 20) ? ARNORM_TWOSHOT_STEP_POLL_DELAY : ARNORM_TWOSHOT_STEP_POLL_DELAY + 6;
}
// The one-launch two-shot call places an owner workgroup and the reader of the same
// fragments on one XCD always, and their producers too from this many blocks of 256
// fragments per slot (below it, the producers of a few blocks would crowd a few XCDs while
// the others idle).  Measured at TP=8, width 7168, us per call (spread as before / owner
// and reader aligned / everything aligned), blocks = 3.5 M: M=1 4.74-4.81 / 4.56-4.61 /
// 4.89-4.92, M=2 4.89-4.90 / 4.68-4.70 / 4.99-5.02, M=4 5.23-5.25 / 5.02 / 5.61-5.62, M=6
// 5.32-5.34 / 5.15-5.17 / 5.88-5.93, M=7 5.45-5.48 / 5.22-5.26 / 4.91-4.93, M=8
// 5.98-6.00 / 5.75-5.77 / 4.94-4.96, M=9 5.04-5.11 / 5.16-5.18 / 5.06-5.09.
#ifndef ARNORM_TWOSHOT_ALIGN_PRODUCERS_MIN
#define ARNORM_TWOSHOT_ALIGN_PRODUCERS_MIN 24
#endif
constexpr int kPolPoll = ARNORM_POL_POLL;
constexpr int kPolRearm = ARNORM_POL_REARM;
constexpr int kPolRearmStep = ARNORM_POL_REARM_STEP;  // re-arms inside the one-launch calls
constexpr int kPolPush = ARNORM_POL_PUSH;
constexpr int kPolIn = ARNORM_POL_IN;  // the caller's rows read once (residual, own partial)
constexpr int kPolIO = ARNORM_POL_IO;  // the caller's output rows
constexpr int kPolCopy = ARNORM_POL_COPY;  // a poll's copy of the rows it read

// Up to this many rows a whole-row consumer gets one workgroup per row without asking
// the runtime for the resident grid (any GPU of this family holds that many at once).
#ifndef ARNORM_WHOLE_ROW_LOOP_MIN_ROWS
#define ARNORM_WHOLE_ROW_LOOP_MIN_ROWS 128
#endif
constexpr int kWholeRowLoopMinRows = ARNORM_WHOLE_ROW_LOOP_MIN_ROWS;

bool aligned16(const void *p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// hipLaunchKernel with the kernel's own parameter types, so every argument is passed
// exactly as the kernel declares it, and `lds` bytes of dynamic LDS per workgroup;
// returns the launch status.
template <typename... KArgs, typename... Args>
int launch_lds(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t stream, Args &&...args) {
  std::tuple<KArgs...> values(std::forward<Args>(args)...);
  void *argv[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
  std::apply([&](auto &...v) {
    int i = 0;
    ((argv[i++] = static_cast<void *>(&v)), ...);
  }, values);
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, lds, stream);
  return e == hipSuccess ? ARNORM_OK : ARNORM_HIP_ERROR;
}

template <typename... KArgs, typename... Args>
int launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream, Args &&...args) {
  return launch_lds(kernel, grid, block, 0, stream, std::forward<Args>(args)...);
}

// Dynamic LDS (unused by the kernel) that keeps the two-shot owner's reduce, 256-thread
// workgroups of 45 VGPRs that would otherwise fill all 32 wave slots of a CU, to at most
// 7 workgroups per CU of gfx950's 160 KB, 28 slots.  The owner keeps one fragment per
// thread over the whole range (a grid capped at half the GPU measured 10 % slower at
// M=4096), so a producer launched after it on another stream gets in only while that grid
// leaves room: measured at TP=8, width 7168, up to M=448 (1568 workgroups), not at M=512
// (1792, every CU full) or above, where the owner is served in order only (its producer
// first, or the polls give up at the spin limit).  The LDS costs nothing measurable
// (M=4096 from HBM: 173.0-175.7 against 171.5-172.7 us without).
#ifndef ARNORM_OWNER_LDS_BYTES
#define ARNORM_OWNER_LDS_BYTES (22u * 1024u)
#endif

// Shape and argument checks shared by arnorm_push / arnorm_reduce_norm.
int check_box(int parities, int tp, int cap, int parity, int M) {
  if (tp < 2 || tp > 8) return ARNORM_NOT_SERVED;
  if (cap < 1 || parities < 1) return ARNORM_BAD_ARG;
  if (parity < 0 || parity >= parities) return ARNORM_BAD_ARG;
  if (M < 1 || M > cap) return ARNORM_NOT_SERVED;
  // one slot's M rows form one buffer range; keep it inside 2 GiB
  if ((uint64_t)M * arn::kRowBytes >= (uint64_t(1) << 31)) return ARNORM_NOT_SERVED;
  return ARNORM_OK;
}

int check_gather(int tp, int cap, int S, int M) {
  if (tp < 2 || tp > 8) return ARNORM_NOT_SERVED;
  if (cap < 1) return ARNORM_BAD_ARG;
  if (S < 4 || S % 4 != 0) return ARNORM_NOT_SERVED;
  if (M < 1 || M > cap) return ARNORM_NOT_SERVED;
  if ((uint64_t)tp * S * 4 >= (uint64_t(1) << 31)) return ARNORM_NOT_SERVED;
  return ARNORM_OK;
}

int check_twoshot(int parities, int cap, int width, int parity, int M) {
  if (width < 8 || width % 8 != 0) return ARNORM_NOT_SERVED;
  if (cap < 1 || parities < 1) return ARNORM_BAD_ARG;
  if (parity < 0 || parity >= parities) return ARNORM_BAD_ARG;
  if (M < 1 || M > cap) return ARNORM_NOT_SERVED;
  if ((uint64_t)M * width * 2 >= (uint64_t(1) << 31)) return ARNORM_NOT_SERVED;
  return ARNORM_OK;
}

// A row-block poll with copy (the Gather consumer): rows < M of `box`, row_frags
// fragments each, as one range; the grid resident at once.
int launch_poll(uint8_t *box, u32x4 *out, uint32_t row_frags, int M, int copy, hipStream_t stream);

uint8_t *parity_base(int32_t *mailbox, int parity, int tp, int cap) {
  return reinterpret_cast<uint8_t *>(mailbox) + (size_t)parity * tp * cap * arn::kRowBytes;
}

// Half of the workgroups of `kernel` (nt threads each) that the current device holds at
// once: compute units x max(1, workgroups per CU / 2), from the occupancy the compiled
// kernel allows.  A polling grid of that size is resident at once with room beside it on
// every CU, so a producer launched after it on another stream always gets in.  (A
// polling grid that fills the GPU exactly does not leave that room: the two-shot owner's
// reduce, 7 workgroups per CU at most, let a producer in at 1568 workgroups and kept it
// out at 1792 = 7 x 256.)  Cached per device and kernel; 0 if the runtime cannot tell.
uint32_t half_resident_grid(const void *kernel, int nt) {
  static std::mutex mu;
  static std::map<std::pair<int, const void *>, uint32_t> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(dev, kernel);
  const auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, nt, 0) != hipSuccess || cus < 1)
    return 0;
  const uint32_t grid = (uint32_t)cus * (uint32_t)std::max(1, per_cu / 2);
  cache.emplace(key, grid);
  return grid;
}

// A whole-row consumer: min(M, half_resident_grid) workgroups, each looping over rows
// (one 896-thread workgroup per CU).  Measured at TP=8, M=4096 (us from HBM / right after
// the push / push + consumer as the call repeats): 256 workgroups 187.7 / 167.1 /
// 305.4-305.9, 512 (two per CU, the GPU full) 187.9-190.5 / 167.8-168.5 / 309.0-311.9,
// 448 194.5-194.9 / 178.5-179.2 / 318.3-318.7, 384 208.7-209.8 / 198.4-198.5 / 338.6-338.8,
// one workgroup per row (4096, not resident) 183.5-186.8 / 169.3-170.8 / 307.8-316.2.
template <int TP, bool RES, bool FUSED, int NT>
int launch_reduce(const arn::ReduceArgs &a, int M, hipStream_t stream) {
  auto kernel = arn::reduce_norm_kernel<TP, RES, FUSED, NT, 1, kPolPoll, kPolRearm, kPolIn, kPolIO>;
  uint32_t grid = (uint32_t)M;
  if (M > kWholeRowLoopMinRows) {
    const uint32_t cap = half_resident_grid(reinterpret_cast<const void *>(kernel), NT);
    if (cap == 0) return ARNORM_HIP_ERROR;
    grid = std::min(grid, cap);
  }
  return launch(kernel, dim3(grid), dim3(NT), stream, a);
}

template <int TP, bool RES, bool FUSED, int K>
int launch_reduce_split(const arn::ReduceArgs &a, int M, hipStream_t stream) {
  constexpr int NT = arn::split_threads(K);
  return launch(arn::reduce_norm_kernel<TP, RES, FUSED, NT, K, kPolPoll, kPolRearm, kPolIn, kPolIO>,
                dim3((M + 7) / 8 * 8 * K), dim3(NT),
                stream, a);
}

template <int TP, bool RES, bool FUSED>
int launch_reduce_nt(const arn::ReduceArgs &a, int M, int threads, int split, hipStream_t stream) {
  if (split == 4) return launch_reduce_split<TP, RES, FUSED, 4>(a, M, stream);
  if (split == 7) return launch_reduce_split<TP, RES, FUSED, 7>(a, M, stream);
  if (split == 8) return launch_reduce_split<TP, RES, FUSED, 8>(a, M, stream);
  if (split == 14) return launch_reduce_split<TP, RES, FUSED, 14>(a, M, stream);
  switch (threads) {
    case 896: return launch_reduce<TP, RES, FUSED, 896>(a, M, stream);
    case 448: return launch_reduce<TP, RES, FUSED, 448>(a, M, stream);
    case 256: return launch_reduce<TP, RES, FUSED, 256>(a, M, stream);
    default: return ARNORM_BAD_ARG;
  }
}

template <int TP>
int launch_reduce_tp(const arn::ReduceArgs &a, bool res, bool fused, int M, int threads, int split,
                     hipStream_t stream) {
  if (fused)
    return res ? launch_reduce_nt<TP, true, true>(a, M, threads, split, stream)
               : launch_reduce_nt<TP, false, true>(a, M, threads, split, stream);
  return res ? launch_reduce_nt<TP, true, false>(a, M, threads, split, stream)
             : launch_reduce_nt<TP, false, false>(a, M, threads, split, stream);
}

// Workgroup size of the consumer when a row is one workgroup.
int reduce_threads(int M) {
  const int forced = g_reduce_threads.load(std::memory_order_relaxed);
  if (forced) return forced;
  (void)M;
  return 896;
}

// Workgroups per row: more than one only with a norm box and a grid small enough to be
// resident at once (every workgroup of a row waits on its peers' parts).
#ifndef ARNORM_SPLIT_MAX_GRID
#define ARNORM_SPLIT_MAX_GRID 1024
#endif
constexpr int kSplitMaxGrid = ARNORM_SPLIT_MAX_GRID;
int reduce_split(int M, bool have_box) {
  if (!have_box) return 1;
  int k = g_reduce_split.load(std::memory_order_relaxed);
  if (k == 0) k = M <= ARNORM_SPLIT7_MAX_M ? 7 : M <= ARNORM_SPLIT4_MAX_M ? 4 : 1;
  if (k > 1 && M * k > kSplitMaxGrid) k = 1;
  return k;
}

// The layout of a Gather poll over n fragments (the rows < M as one range): U fragments
// per thread in flight and the number of workgroups.  One fragment per thread while that
// takes at most 1024 workgroups of 256 threads, else ARNORM_POLL_U in flight per thread
// over at most 1024 workgroups.  1024 workgroups of 256 threads are a quarter of what
// 256 CUs hold, so the whole grid is resident at once and a producer running beside it
// on another stream still finds room (a cap of 2048, the full machine, starved a
// concurrent producer at M=512: the poll spun to its limit and the push ran after).
// Measured for the one-slot read at M=4096, width 7168 (a copy and re-arm of 58.7 MB, us
// from HBM): this layout 31.0-31.7, one row per workgroup (the layout before, not resident
// above 1024 rows) 32.0-32.2; a probe doing only the copy and re-arm, one fragment per
// thread over the whole range (14,336 workgroups, not resident), 29.7-31.0.
constexpr uint32_t kPollMaxGrid = 1024;
struct PollLayout {
  int u;
  uint32_t grid;
};
PollLayout poll_layout(uint64_t n) {
  int u = g_poll_frags.load(std::memory_order_relaxed);
  if (u == 0) u = n <= (uint64_t)kPollMaxGrid * 256u ? 1 : ARNORM_POLL_U;
  const uint64_t blocks = (n + 256u * u - 1) / (256u * u);
  return {u, (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>(blocks, kPollMaxGrid))};
}
int poll_mode(int automatic) {
  const int mode = g_poll_mode.load(std::memory_order_relaxed);
  return mode == 0 ? automatic : mode == 1 ? 1 : 0;
}

int launch_poll(uint8_t *box, u32x4 *out, uint32_t row_frags, int M, int copy, hipStream_t stream) {
  const uint64_t n = (uint64_t)M * row_frags;
  const int poll_all = poll_mode(n * 16u <= ARNORM_POLL_ALL_MAX_BYTES);
  const uint64_t spin = g_spin_limit.load(std::memory_order_relaxed);
  const PollLayout l = poll_layout(n);
  if (l.u == 1)
    return launch(arn::gather_poll_kernel<kPolPoll, kPolRearm, kPolCopy, 1>, dim3(l.grid), dim3(256), stream, box,
                  out, n,
                  copy ? 1 : 0, spin, poll_all);
  return launch(arn::gather_poll_kernel<kPolPoll, kPolRearm, kPolCopy, ARNORM_POLL_U>, dim3(l.grid), dim3(256), stream,
                box,
                out, n, copy ? 1 : 0, spin, poll_all);
}

// The producer kernel over `frags` fragments per slot of nslots slots.
int launch_push(const void *partial, uint8_t *first, size_t slot_stride, uint32_t frags, int nslots,
                hipStream_t stream) {
  const bool small = (uint64_t)frags * 16u <= ARNORM_PUSH_SMALL_BYTES;
  const uint32_t per_wg = 256u * (small ? ARNORM_PUSH_U_SMALL : ARNORM_PUSH_U);
  const dim3 grid(std::max(1u, std::min((frags + per_wg - 1) / per_wg, (uint32_t)ARNORM_PUSH_MAX_GRID)),
                  (unsigned)nslots);
  const u32x4 *src = reinterpret_cast<const u32x4 *>(partial);
  if (small)
    return launch(arn::push_kernel<ARNORM_PUSH_U_SMALL, kPolPush, false>, grid, dim3(256), stream, src, first,
                  slot_stride, frags);
  return launch(arn::push_kernel<ARNORM_PUSH_U, kPolPush, true>, grid, dim3(256), stream, src, first, slot_stride,
                frags);
}

// The block of a caller's norm box int32 [parities, cap, 256] that a call of this parity uses.
uint32_t *norm_box_block(int32_t *norm_box, int parity, int cap) {
  return reinterpret_cast<uint32_t *>(norm_box) + (size_t)parity * cap * arn::kNormBoxRowWords;
}

// arnorm_reduce_norm after its argument checks; nbox is the norm box's block of this
// call's parity (int32 [rows >= M, 256]) or NULL.
int reduce_norm_launch(const uint16_t *partial, const uint16_t *residual, const uint16_t *gamma, uint16_t *out,
                       uint16_t *residual_out, int32_t *mailbox, uint32_t *nbox, int tp, int cap, int parity, int rank,
                       int M, float eps, hipStream_t stream) {
  arn::ReduceArgs a;
  a.partial = reinterpret_cast<const uint8_t *>(partial);
  a.residual = reinterpret_cast<const uint8_t *>(residual);
  a.gamma = reinterpret_cast<const uint8_t *>(gamma);
  a.out = reinterpret_cast<uint8_t *>(out);
  a.res_out = reinterpret_cast<uint8_t *>(residual_out);
  a.box = parity_base(mailbox, parity, tp, cap);
  a.slot_stride = (size_t)cap * arn::kRowBytes;
  a.rows = (uint32_t)M;
  a.rank = partial ? rank : -1;
  a.poll_delay = 0;
  a.eps = eps;
  a.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  a.poll_all = (uint64_t)tp * M * arn::kRowBytes <= ARNORM_POLL_ALL_MAX_BYTES;
  const bool res = residual != nullptr;
  const bool fused = partial != nullptr;
  const int threads = reduce_threads(M);
  const int split = reduce_split(M, nbox != nullptr);
  a.nbox = nbox;
  switch (tp) {
    case 2: return launch_reduce_tp<2>(a, res, fused, M, threads, split, stream);
    case 3: return launch_reduce_tp<3>(a, res, fused, M, threads, split, stream);
    case 4: return launch_reduce_tp<4>(a, res, fused, M, threads, split, stream);
    case 5: return launch_reduce_tp<5>(a, res, fused, M, threads, split, stream);
    case 6: return launch_reduce_tp<6>(a, res, fused, M, threads, split, stream);
    case 7: return launch_reduce_tp<7>(a, res, fused, M, threads, split, stream);
    case 8: return launch_reduce_tp<8>(a, res, fused, M, threads, split, stream);
  }
  return ARNORM_NOT_SERVED;
}

// arnorm_push_reduce_norm after its argument checks; nbox is the norm box's block of this
// call's parity (int32 [rows >= M, 256]) or NULL.
int push_reduce_norm_launch(const uint16_t *partials, const uint16_t *residual, const uint16_t *gamma,
                            uint16_t *out, uint16_t *residual_out, int32_t *mailbox, uint32_t *nbox, int parities,
                            int tp, int cap, int parity, int M, float eps, hipStream_t stream) {
  // One launch where its consumers, re-reading every slot on each poll pass after the
  // delay below, beat the pair (see ARNORM_STEP_MAX_BYTES).  Rows split 7 ways beat 14 (M=4:
  // 3.80-3.82 against 3.96 us) and one workgroup per row (4.98 us, 4.70 at M=1 against 3.71).
  int K = nbox != nullptr ? reduce_split(M, true) : 1;
  // the automatic split takes whole rows above ARNORM_SPLIT4_MAX_M (the pair's crossover);
  // the one launch keeps rows split 4 ways up to ARNORM_STEP_SPLIT4_MAX_M, then 2 ways up to
  // ARNORM_STEP_SPLIT2_MAX_M.  Its 2-way rows may pass the split grid's cap, which leaves room
  // for a producer on another stream: in one launch the producers come first and a row's
  // workgroups in one block, so the dispatch order guarantees progress at any grid size.
  if (nbox != nullptr && K == 1 && g_reduce_split.load(std::memory_order_relaxed) == 0) {
    if (M <= ARNORM_STEP_SPLIT4_MAX_M && M * 4 <= kSplitMaxGrid)
      K = 4;
    else if (M <= ARNORM_STEP_SPLIT2_MAX_M)
      K = 2;
  }
  const int U = ARNORM_STEP_PUSH_U;
  const uint32_t nt = arn::split_threads(K);
  // Workgroups of at most 128 threads (rows split 7 ways) come in an even number of
  // producers per slot (an extra one finds no fragments and ends).  With an odd count, from
  // M=14 the call paid most of a poll round trip more: TP=8, medians of 3 alternations, odd
  // / rounded up to even, M=14 4.12 / 3.99, M=15 4.16 / 3.98, M=18 4.32 / 4.07, M=22 4.66 /
  // 4.17, M=23 4.71 / 4.15, M=26 4.75 / 4.24, M=27 4.77 / 4.23, M=30 5.02 / 4.40, M=31 5.17 /
  // 4.48 (two more boxes: M=30 5.08, 4.81 / 4.39, 4.47), the other row counts within 0.02.
  // Rows split 4 ways (256 threads) keep the count: there rounding moved the slow row counts
  // about (M=39 4.87 / 5.41, M=47 5.09 / 5.74, M=61 6.31 / 6.07, measured while the producers
  // read their rows with non-temporal loads).
  const uint64_t frags = (uint64_t)M * arn::kRowFrags;
  uint64_t per_slot = (frags + nt * U - 1) / (nt * U);
  if (nt <= 128) per_slot += per_slot & 1u;
  const uint64_t grid_wgs = tp * per_slot + (uint64_t)(M + 7) / 8 * 8 * K;
  const bool one_launch = K > 1 && M <= ARNORM_STEP_MAX_M &&
                          (uint64_t)tp * M * arn::kRowBytes <= ARNORM_STEP_MAX_BYTES &&
                          grid_wgs <= ARNORM_STEP_MAX_GRID;
  if (!one_launch) {
    // the same call as two launches: every rank's push, then the consumer
    const int rc = arnorm_push(partials, mailbox, parities, tp, cap, parity, 0, tp, M, stream);
    if (rc != ARNORM_OK) return rc;
    return reduce_norm_launch(nullptr, residual, gamma, out, residual_out, mailbox, nbox, tp, cap, parity, 0, M, eps,
                              stream);
  }

  arn::StepArgs a;
  a.r.partial = nullptr;
  a.r.residual = reinterpret_cast<const uint8_t *>(residual);
  a.r.gamma = reinterpret_cast<const uint8_t *>(gamma);
  a.r.out = reinterpret_cast<uint8_t *>(out);
  a.r.res_out = reinterpret_cast<uint8_t *>(residual_out);
  a.r.box = parity_base(mailbox, parity, tp, cap);
  a.r.slot_stride = (size_t)cap * arn::kRowBytes;
  a.r.nbox = nbox;
  a.r.rows = (uint32_t)M;
  a.r.rank = -1;
  a.r.eps = eps;
  a.r.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  a.r.poll_all = 1;
  a.r.poll_delay = K != 4 && K != 2 ? ARNORM_STEP_POLL_DELAY
                          : ARNORM_STEP_POLL_DELAY_SPLIT4 +
                                (M > ARNORM_STEP_POLL_DELAY_RAMP_M
                                     ? ((M < ARNORM_STEP_POLL_DELAY_RAMP_END ? M : ARNORM_STEP_POLL_DELAY_RAMP_END) -
                                        ARNORM_STEP_POLL_DELAY_RAMP_M + 1) / 2
                                     : 0);
  a.partials = reinterpret_cast<const u32x4 *>(partials);
  a.frags = (uint32_t)frags;
  // The residual rows are read with the default cache policy here, so that a residual buffer
  // read again unchanged stays in the last-level cache (with non-temporal reads it came from
  // HBM on every call: TP=8, one residual buffer for every call, M=64 6.09 against 5.77 us,
  // M=128 13.44 / 11.77, M=256 24.89 / 21.08, M=512 44.73 / 38.71; M=1..16 and the drafter
  // step the same).  Rows that the previous call stored as its residual_out are still in
  // that cache and read from it with either policy (calls chained that way, M=16..512, within
  // 0.05 us).  The pair and the M=4096 consumer keep kPolIn.
  a.per_slot = (uint32_t)per_slot;
  const dim3 grid((uint32_t)grid_wgs);
  const bool res = residual != nullptr;
#define ARNORM_STEP_LAUNCH_K(TPV, KV)                                                                              \
  return res ? launch(arn::push_reduce_kernel<TPV, true, KV, ARNORM_STEP_PUSH_U, kPolPush, kPolPoll, kPolRearmStep,  \
                                              arn::kPolPlain, kPolIO>,                                             \
                      grid, dim3(nt), stream, a)                                                                   \
             : launch(arn::push_reduce_kernel<TPV, false, KV, ARNORM_STEP_PUSH_U, kPolPush, kPolPoll, kPolRearmStep, \
                                              kPolIn, kPolIO>,                                                     \
                      grid, dim3(nt), stream, a);
#define ARNORM_STEP_LAUNCH(TPV)                                                                                   \
  case TPV:                                                                                                      \
    if (K == 2) {                                                                                                \
      ARNORM_STEP_LAUNCH_K(TPV, 2)                                                                               \
    }                                                                                                            \
    if (K == 4) {                                                                                                \
      ARNORM_STEP_LAUNCH_K(TPV, 4)                                                                               \
    }                                                                                                            \
    if (K == 7) {                                                                                                \
      ARNORM_STEP_LAUNCH_K(TPV, 7)                                                                               \
    }                                                                                                            \
    if (K == 8) {                                                                                                \
      ARNORM_STEP_LAUNCH_K(TPV, 8)                                                                               \
    }                                                                                                            \
    ARNORM_STEP_LAUNCH_K(TPV, 14)
  switch (tp) {
    ARNORM_STEP_LAUNCH(2)
    ARNORM_STEP_LAUNCH(3)
    ARNORM_STEP_LAUNCH(4)
    ARNORM_STEP_LAUNCH(5)
    ARNORM_STEP_LAUNCH(6)
    ARNORM_STEP_LAUNCH(7)
    ARNORM_STEP_LAUNCH(8)
  }
#undef ARNORM_STEP_LAUNCH
#undef ARNORM_STEP_LAUNCH_K
  return ARNORM_NOT_SERVED;
}

}  // namespace

extern "C" {

int lamport_arm(int32_t *buf, size_t words, uint32_t sentinel, hipStream_t stream) {
  if (!aligned16(buf)) return ARNORM_BAD_ARG;
  if (words == 0) return ARNORM_OK;
  const size_t nfrag = words / 4;
  const int ntail = (int)(words % 4);
  const size_t want = (nfrag + 255) / 256;
  const unsigned blocks = (unsigned)std::max<size_t>(1, std::min<size_t>(want, 8192));
  return launch(arn::arm_kernel, dim3(blocks), dim3(256), stream, reinterpret_cast<u32x4 *>(buf), nfrag,
                reinterpret_cast<uint32_t *>(buf) + nfrag * 4, ntail, sentinel);
}

int arnorm_push(const uint16_t *partial, int32_t *mailbox, int parities, int tp, int cap, int parity,
                int rank, int nslots, int M, hipStream_t stream) {
  int rc = check_box(parities, tp, cap, parity, M);
  if (rc != ARNORM_OK) return rc;
  if (rank < 0 || nslots < 1 || rank + nslots > tp) return ARNORM_BAD_ARG;
  if (!aligned16(partial) || !aligned16(mailbox)) return ARNORM_BAD_ARG;
  uint8_t *first = parity_base(mailbox, parity, tp, cap) + (size_t)rank * cap * arn::kRowBytes;
  return launch_push(partial, first, (size_t)cap * arn::kRowBytes, (uint32_t)M * arn::kRowFrags, nslots, stream);
}

int arnorm_reduce_norm(const uint16_t *partial, const uint16_t *residual, const uint16_t *gamma, uint16_t *out,
                       uint16_t *residual_out, int32_t *mailbox, int32_t *norm_box, int parities, int tp, int cap,
                       int parity, int rank, int M, float eps, hipStream_t stream) {
  int rc = check_box(parities, tp, cap, parity, M);
  if (rc != ARNORM_OK) return rc;
  if (partial && (rank < 0 || rank >= tp)) return ARNORM_BAD_ARG;
  if ((partial && !aligned16(partial)) || (residual && !aligned16(residual))) return ARNORM_BAD_ARG;
  if (!aligned16(gamma) || !aligned16(out) || !aligned16(residual_out) || !aligned16(mailbox))
    return ARNORM_BAD_ARG;
  if (norm_box && (!aligned16(norm_box) || norm_box == mailbox)) return ARNORM_BAD_ARG;
  const void *outs[3] = {out, residual_out, norm_box};
  const void *ins[4] = {partial, residual, gamma, mailbox};
  for (const void *o : outs)
    for (const void *i : ins)
      if (o && o == i && !(o == residual_out && i == residual)) return ARNORM_BAD_ARG;
  if (norm_box && (static_cast<void *>(norm_box) == out || static_cast<void *>(norm_box) == residual_out))
    return ARNORM_BAD_ARG;
  if (out == residual_out) return ARNORM_BAD_ARG;

  return reduce_norm_launch(partial, residual, gamma, out, residual_out, mailbox,
                            norm_box ? norm_box_block(norm_box, parity, cap) : nullptr, tp, cap, parity, rank, M, eps,
                            stream);
}

int arnorm_push_reduce_norm(const uint16_t *partials, const uint16_t *residual, const uint16_t *gamma,
                            uint16_t *out, uint16_t *residual_out, int32_t *mailbox, int32_t *norm_box, int parities,
                            int tp, int cap, int parity, int M, float eps, hipStream_t stream) {
  int rc = check_box(parities, tp, cap, parity, M);
  if (rc != ARNORM_OK) return rc;
  // every check of both halves first, so that a call launches all of its work or none
  if (!aligned16(partials) || (residual && !aligned16(residual))) return ARNORM_BAD_ARG;
  if (!aligned16(gamma) || !aligned16(out) || !aligned16(residual_out) || !aligned16(mailbox)) return ARNORM_BAD_ARG;
  if (norm_box && !aligned16(norm_box)) return ARNORM_BAD_ARG;
  const void *outs[3] = {out, residual_out, norm_box};
  const void *ins[4] = {partials, residual, gamma, mailbox};
  for (const void *o : outs)
    for (const void *i : ins)
      if (o && o == i && !(o == residual_out && i == residual)) return ARNORM_BAD_ARG;
  if (out == residual_out) return ARNORM_BAD_ARG;
  if (norm_box && (static_cast<void *>(norm_box) == out || static_cast<void *>(norm_box) == residual_out))
    return ARNORM_BAD_ARG;
  return push_reduce_norm_launch(partials, residual, gamma, out, residual_out, mailbox,
                                 norm_box ? norm_box_block(norm_box, parity, cap) : nullptr, parities, tp, cap, parity,
                                 M, eps, stream);
}

int arnorm_push_reduce_norm_static(const uint16_t *partials, const uint16_t *residual, const uint16_t *gamma,
                                   uint16_t *out, uint16_t *residual_out, int32_t *mailbox, int parities, int tp,
                                   int cap, int parity, int M, float eps, hipStream_t stream) {
  int rc = check_box(parities, tp, cap, parity, M);
  if (rc != ARNORM_OK) return rc;
  if (!aligned16(partials) || (residual && !aligned16(residual))) return ARNORM_BAD_ARG;
  if (!aligned16(gamma) || !aligned16(out) || !aligned16(residual_out) || !aligned16(mailbox)) return ARNORM_BAD_ARG;
  const void *outs[2] = {out, residual_out};
  const void *ins[4] = {partials, residual, gamma, mailbox};
  for (const void *o : outs)
    for (const void *i : ins)
      if (o == i && !(o == residual_out && i == residual)) return ARNORM_BAD_ARG;
  if (out == residual_out) return ARNORM_BAD_ARG;
  if (M > kScratchRows) return ARNORM_TOO_LARGE;
  uint32_t *nbox = nullptr;
  rc = static_scratch(&nbox);
  if (rc != ARNORM_OK) return rc;
  // the rows this call uses start armed, whatever an earlier call (a timed-out one
  // included) left there; a fill kernel, not a memset, so that the call stays capturable
  const size_t nfrag = (size_t)M * arn::kNormBoxRowWords / 4;
  rc = launch(arn::arm_kernel, dim3((unsigned)((nfrag + 255) / 256)), dim3(256), stream,
              reinterpret_cast<u32x4 *>(nbox), nfrag, nbox + nfrag * 4, 0, (uint32_t)arn::kSentinel);
  if (rc != ARNORM_OK) return rc;
  return push_reduce_norm_launch(partials, residual, gamma, out, residual_out, mailbox, nbox, parities, tp, cap,
                                 parity, M, eps, stream);
}

int gather_push(const int32_t *shard, int32_t *mailbox, int tp, int cap, int S, int rank, int nslots, int M,
                hipStream_t stream) {
  int rc = check_gather(tp, cap, S, M);
  if (rc != ARNORM_OK) return rc;
  if (rank < 0 || nslots < 1 || rank + nslots > tp) return ARNORM_BAD_ARG;
  if (!aligned16(shard) || !aligned16(mailbox)) return ARNORM_BAD_ARG;
  const uint32_t frags = (uint32_t)S / 4;
  const uint64_t n = (uint64_t)M * frags;  // one slot's fragments
  if (n > 0xFFFFFF00u) return ARNORM_NOT_SERVED;  // a grid row of at most 2^32 - 256 threads
  return launch(arn::gather_push_kernel<kPolPush>, dim3((uint32_t)((n + 255) / 256), (uint32_t)nslots), dim3(256),
                stream, reinterpret_cast<const u32x4 *>(shard), reinterpret_cast<uint8_t *>(mailbox), frags,
                (uint32_t)n, (uint32_t)tp * S * 4u, (uint32_t)rank * S * 4u);
}

int gather_poll(int32_t *mailbox, int32_t *out, int tp, int cap, int S, int M, int copy, hipStream_t stream) {
  int rc = check_gather(tp, cap, S, M);
  if (rc != ARNORM_OK) return rc;
  if (!aligned16(mailbox) || (copy && !aligned16(out))) return ARNORM_BAD_ARG;
  if (copy && static_cast<void *>(out) == static_cast<void *>(mailbox)) return ARNORM_BAD_ARG;
  return launch_poll(reinterpret_cast<uint8_t *>(mailbox), reinterpret_cast<u32x4 *>(out), (uint32_t)tp * S / 4, M,
                     copy, stream);
}

int gather_push_poll(const int32_t *shard, int32_t *mailbox, int32_t *out, int tp, int cap, int S, int M, int copy,
                     hipStream_t stream) {
  int rc = check_gather(tp, cap, S, M);
  if (rc != ARNORM_OK) return rc;
  if (!aligned16(shard) || !aligned16(mailbox) || (copy && !aligned16(out))) return ARNORM_BAD_ARG;
  if (copy && (static_cast<void *>(out) == static_cast<void *>(mailbox) ||
               static_cast<const void *>(out) == static_cast<const void *>(shard)))
    return ARNORM_BAD_ARG;
  const uint32_t frags = (uint32_t)S / 4;
  if ((uint64_t)M * tp * S * 4 > ARNORM_GATHER_STEP_MAX_BYTES) {
    // a larger grid: the same call as the pair of launches
    rc = gather_push(shard, mailbox, tp, cap, S, 0, tp, M, stream);
    if (rc != ARNORM_OK) return rc;
    return gather_poll(mailbox, out, tp, cap, S, M, copy, stream);
  }
  arn::GatherStepArgs a;
  a.shard = reinterpret_cast<const u32x4 *>(shard);
  a.box = reinterpret_cast<uint8_t *>(mailbox);
  a.out = reinterpret_cast<u32x4 *>(out);
  a.frags = frags;
  a.M = (uint32_t)M;
  const uint32_t n = (uint32_t)M * tp * frags;
  a.producers = ((n + 255) / 256 + 7) / 8 * 8;
  const PollLayout l = poll_layout(n);
  a.pollers = l.grid;
  a.copy = copy ? 1 : 0;
  a.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  a.poll_all = poll_mode(1);
  a.poll_delay = gather_step_delay((uint64_t)n * 16u);
  const dim3 grid(a.producers + a.pollers);
#define ARNORM_GATHER_STEP(T)                                                                                      \
  case T:                                                                                                          \
    if (l.u == 1)                                                                                                  \
      return launch(arn::gather_push_poll_kernel<T, 1, kPolPush, kPolPoll, kPolRearmStep, kPolCopy>, grid,         \
                    dim3(256),                                                                                     \
                    stream, a);                                                                                    \
    return launch(arn::gather_push_poll_kernel<T, ARNORM_POLL_U, kPolPush, kPolPoll, kPolRearmStep, kPolCopy>,     \
                  grid, dim3(256), stream, a);
  switch (tp) {
    ARNORM_GATHER_STEP(2)
    ARNORM_GATHER_STEP(3)
    ARNORM_GATHER_STEP(4)
    ARNORM_GATHER_STEP(5)
    ARNORM_GATHER_STEP(6)
    ARNORM_GATHER_STEP(7)
    ARNORM_GATHER_STEP(8)
  }
#undef ARNORM_GATHER_STEP
  return ARNORM_NOT_SERVED;
}

int twoshot_push(const uint16_t *partial, int32_t *recv, int parities, int tp, int cap, int width, int parity,
                 int rank, int nslots, int M, hipStream_t stream) {
  if (tp < 2 || tp > 8) return ARNORM_NOT_SERVED;
  int rc = check_twoshot(parities, cap, width, parity, M);
  if (rc != ARNORM_OK) return rc;
  if (rank < 0 || nslots < 1 || rank + nslots > tp) return ARNORM_BAD_ARG;
  if (!aligned16(partial) || !aligned16(recv)) return ARNORM_BAD_ARG;
  const size_t row_bytes = (size_t)width * 2;
  uint8_t *first = reinterpret_cast<uint8_t *>(recv) + ((size_t)parity * tp + rank) * cap * row_bytes;
  return launch_push(partial, first, (size_t)cap * row_bytes, (uint32_t)((size_t)M * row_bytes / 16), nslots,
                     stream);
}

int twoshot_reduce(int32_t *recv, int32_t *gather, int parities, int tp, int cap, int width, int parity, int M,
                   hipStream_t stream) {
  if (tp < 2 || tp > 8) return ARNORM_NOT_SERVED;
  int rc = check_twoshot(parities, cap, width, parity, M);
  if (rc != ARNORM_OK) return rc;
  if (!aligned16(recv) || !aligned16(gather) || recv == gather) return ARNORM_BAD_ARG;
  const size_t row_bytes = (size_t)width * 2;
  arn::TwoShotArgs a;
  a.recv = reinterpret_cast<uint8_t *>(recv) + (size_t)parity * tp * cap * row_bytes;
  a.gather = reinterpret_cast<uint8_t *>(gather) + (size_t)parity * cap * row_bytes;
  a.slot_stride = (size_t)cap * row_bytes;
  a.frags = (uint32_t)((size_t)M * row_bytes / 16);
  a.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  a.poll_all = (uint64_t)tp * a.frags * 16u <= ARNORM_POLL_ALL_MAX_BYTES;
  const dim3 grid(std::max(1u, std::min((a.frags + 255) / 256, 16384u)));
  const size_t lds = ARNORM_OWNER_LDS_BYTES;
  switch (tp) {
#define ARNORM_OWNER(T)                                                                                             \
  case T:                                                                                                           \
    return launch_lds(arn::twoshot_reduce_kernel<T, kPolPoll, kPolRearm, kPolPush>, grid, dim3(256), lds, stream, a);
    ARNORM_OWNER(2)
    ARNORM_OWNER(3)
    ARNORM_OWNER(4)
    ARNORM_OWNER(5)
    ARNORM_OWNER(6)
    ARNORM_OWNER(7)
    ARNORM_OWNER(8)
#undef ARNORM_OWNER
  }
  return ARNORM_NOT_SERVED;
}

int twoshot_read(int32_t *gather, uint16_t *out, int parities, int cap, int width, int parity, int M,
                 hipStream_t stream) {
  int rc = check_twoshot(parities, cap, width, parity, M);
  if (rc != ARNORM_OK) return rc;
  if (!aligned16(gather) || !aligned16(out)) return ARNORM_BAD_ARG;
  if (static_cast<void *>(out) == static_cast<void *>(gather)) return ARNORM_BAD_ARG;
  const size_t row_bytes = (size_t)width * 2;
  return launch_poll(reinterpret_cast<uint8_t *>(gather) + (size_t)parity * cap * row_bytes,
                     reinterpret_cast<u32x4 *>(out), (uint32_t)(row_bytes / 16), M, 1, stream);
}

int twoshot_push_reduce_read(const uint16_t *partial, int32_t *recv, int32_t *gather, uint16_t *out, int parities,
                             int tp, int cap, int width, int parity, int M, hipStream_t stream) {
  if (tp < 2 || tp > 8) return ARNORM_NOT_SERVED;
  int rc = check_twoshot(parities, cap, width, parity, M);
  if (rc != ARNORM_OK) return rc;
  if (!aligned16(partial) || !aligned16(recv) || !aligned16(gather) || !aligned16(out)) return ARNORM_BAD_ARG;
  const void *p = partial, *r = recv, *g = gather, *o = out;
  if (r == g || o == g || o == r || o == p) return ARNORM_BAD_ARG;
  const size_t row_bytes = (size_t)width * 2;
  const uint32_t frags = (uint32_t)((size_t)M * row_bytes / 16);
  if ((uint64_t)tp * frags * 16u > ARNORM_TWOSHOT_STEP_MAX_BYTES) {
    rc = twoshot_push(partial, recv, parities, tp, cap, width, parity, 0, tp, M, stream);
    if (rc == ARNORM_OK) rc = twoshot_reduce(recv, gather, parities, tp, cap, width, parity, M, stream);
    if (rc == ARNORM_OK) rc = twoshot_read(gather, out, parities, cap, width, parity, M, stream);
    return rc;
  }
  arn::TwoShotStepArgs a;
  a.r.recv = reinterpret_cast<uint8_t *>(recv) + (size_t)parity * tp * cap * row_bytes;
  a.r.gather = reinterpret_cast<uint8_t *>(gather) + (size_t)parity * cap * row_bytes;
  a.r.slot_stride = (size_t)cap * row_bytes;
  a.r.frags = frags;
  a.r.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  a.r.poll_all = 1;
  a.partial = reinterpret_cast<const u32x4 *>(partial);
  a.out = reinterpret_cast<u32x4 *>(out);
  a.per_slot = a.red_ctas = a.read_ctas = (frags + 255) / 256;
  a.red_span = (a.red_ctas + 7) / 8 * 8;
  a.prod_span = a.per_slot >= ARNORM_TWOSHOT_ALIGN_PRODUCERS_MIN ? (a.per_slot + 7) / 8 * 8 : a.per_slot;
  a.poll_delay = twoshot_step_delay((uint64_t)tp * frags * 16u);
  const dim3 grid(tp * a.prod_span + a.red_span + a.read_ctas);
  switch (tp) {
#define ARNORM_TWOSHOT_STEP(T)                                                                                      \
  case T:                                                                                                           \
    return launch(arn::twoshot_step_kernel<T, kPolPush, kPolPoll, kPolRearmStep, kPolPush, kPolCopy>, grid,          \
                  dim3(256),                                                                                        \
                  stream, a);
    ARNORM_TWOSHOT_STEP(2)
    ARNORM_TWOSHOT_STEP(3)
    ARNORM_TWOSHOT_STEP(4)
    ARNORM_TWOSHOT_STEP(5)
    ARNORM_TWOSHOT_STEP(6)
    ARNORM_TWOSHOT_STEP(7)
    ARNORM_TWOSHOT_STEP(8)
#undef ARNORM_TWOSHOT_STEP
  }
  return ARNORM_NOT_SERVED;
}

int arnorm_set_spin_limit(uint64_t polls) {
  if (polls == 0) return ARNORM_BAD_ARG;
  g_spin_limit.store(polls, std::memory_order_relaxed);
  return ARNORM_OK;
}

uint64_t arnorm_get_spin_limit(void) { return g_spin_limit.load(std::memory_order_relaxed); }

int arnorm_set_reduce_split(int workgroups_per_row) {
  const int k = workgroups_per_row;
  if (k != 0 && k != 1 && k != 4 && k != 7 && k != 8 && k != 14) return ARNORM_BAD_ARG;
  g_reduce_split.store(k, std::memory_order_relaxed);
  return ARNORM_OK;
}

int arnorm_set_poll(int frags_per_thread, int mode) {
  if (frags_per_thread != 0 && frags_per_thread != 1 && frags_per_thread != ARNORM_POLL_U) return ARNORM_BAD_ARG;
  if (mode < 0 || mode > 2) return ARNORM_BAD_ARG;
  g_poll_frags.store(frags_per_thread, std::memory_order_relaxed);
  g_poll_mode.store(mode, std::memory_order_relaxed);
  return ARNORM_OK;
}

int arnorm_set_reduce_threads(int threads) {
  if (threads != 0 && threads != 896 && threads != 448 && threads != 256) return ARNORM_BAD_ARG;
  g_reduce_threads.store(threads, std::memory_order_relaxed);
  return ARNORM_OK;
}

int arnorm_status(int *status, hipStream_t stream) {
  if (status == nullptr) return ARNORM_BAD_ARG;
  // The swap is one device atomic, so a timeout that a kernel on another stream records
  // at any moment lands either in this read or in the next one, never in neither.  The
  // mutex keeps two host threads from sharing the one g_status_taken word between the
  // swap and its copy.
  static std::mutex mu;
  std::lock_guard<std::mutex> lock(mu);
  if (hipStreamSynchronize(stream) != hipSuccess) return ARNORM_HIP_ERROR;
  if (launch(arn::status_take_kernel, dim3(1), dim3(64), stream) != ARNORM_OK) return ARNORM_HIP_ERROR;
  unsigned int v = 0;
  if (hipMemcpyFromSymbolAsync(&v, HIP_SYMBOL(arn::g_status_taken), sizeof(v), 0, hipMemcpyDeviceToHost, stream) !=
          hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return ARNORM_HIP_ERROR;
  *status = v ? ARNORM_TIMEOUT : ARNORM_OK;
  return ARNORM_OK;
}

const char *arnorm_strerror(int code) {
  switch (code) {
    case ARNORM_OK: return "ok";
    case ARNORM_NOT_SERVED: return "shape not served (use the stock collective)";
    case ARNORM_BAD_ARG: return "bad argument";
    case ARNORM_HIP_ERROR: return "HIP runtime error";
    case ARNORM_TIMEOUT: return "poll timed out (re-arm the mailbox)";
    case ARNORM_TOO_LARGE: return "more rows than the library's static scratch holds";
  }
  return "unknown code";
}

}  // extern "C"

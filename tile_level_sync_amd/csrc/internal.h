// Definitions shared by the host runtime and the gfx950 kernels: workspace
// layout, kernel parameter blocks and the tile-configuration table.
#pragma once

#include <stdint.h>
#include <stddef.h>

namespace tls {

// ---------------------------------------------------------------------------
// Workspace layout.  The control block sits at offset 0, each hot word on its
// own 128-byte line (the L2 line size).  Then come three fixed flag regions,
// one u32 per flag, each flag on its own 128-byte line so that a polled flag
// and a posted neighbour never share a line:
//   * row counters (RowSync), kMaxRowCounters slots; they count up from zero
//     within a launch and are cleared by its last workgroup;
//   * split-K arrival counters, kMaxSplitCounters slots, likewise cleared by
//     the last workgroup;
//   * tile flags (TileSync / Conv2DTileSync), kMaxTileFlags slots, holding
//     the epoch of the call that last completed the tile; never cleared.
// The regions sit at fixed offsets and hold nothing else, so whatever shapes
// and policies share a workspace, a flag only ever holds a count of its own
// kind or an epoch (monotone per workspace): never stale data of another
// region.  After them (from kFixedBytes): the optional order table, split
// partial sums and the intermediate buffer, laid out per call.
// ---------------------------------------------------------------------------
constexpr uint32_t kLine = 128;                  // bytes
constexpr uint32_t kFlagStride = kLine / 4;      // u32 elements between flags

constexpr int kNumQueues = 8;  // one work queue per XCD (gfx950 has 8)
constexpr int kMaxPhases = 3;  // stages of the longest chain (self-attention)

struct Ctl {
  uint32_t work;            // next work item (global atomic work counter)
  uint32_t pad0[31];
  uint32_t done;            // workgroups that have left the loop
  uint32_t pad1[31];
  uint32_t epoch;           // last completed sync-policy call (TileSync flag value)
  uint32_t status;          // 0 = ok, 1 = a wait expired
  uint32_t status_item;     // work item of the expired wait
  uint32_t status_kind;     // 0 producer side, 1 consumer side
  uint32_t abort;           // set with status: remaining tiles are skipped
  uint32_t pad2[27];
  uint32_t qnext[kMaxPhases * kNumQueues][32];  // per-XCD queue counters: [phase * 8 + queue][0]
  uint32_t fillnext;        // next chunk of the sentinel ring slot re-filled at exit
  uint32_t pad3[31];
};
static_assert(sizeof(Ctl) == (4 + kMaxPhases * kNumQueues) * kLine, "Ctl layout");

constexpr size_t kCtlBytes = 4096;
constexpr uint32_t kNoItem = 0xFFFFFFFFu;
constexpr uint32_t kMaxRowCounters = 8192;
constexpr size_t kRowCntOffset = kCtlBytes;
static_assert(sizeof(Ctl) <= kCtlBytes, "Ctl size");
constexpr uint32_t kMaxSplitCounters = 16384;
constexpr size_t kSplitCntOffset = kRowCntOffset + (size_t)kMaxRowCounters * kLine;
constexpr uint32_t kMaxTileFlags = 32768;
constexpr size_t kTileFlagOffset = kSplitCntOffset + (size_t)kMaxSplitCounters * kLine;
constexpr size_t kFixedBytes = kTileFlagOffset + (size_t)kMaxTileFlags * kLine;

enum : uint32_t { kStatusOk = 0, kStatusTimeout = 1 };

// Size of the static device array that serves as the workspace of the
// allocation-free MLP entry point: the fixed regions above plus split
// partials and the intermediate of the call (the GPT-3 slice needs at most
// about 40 MiB, at M = 512 with its K-split partials).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;

constexpr uint32_t kDefaultPollLimit = 1u << 20;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// Policies as the kernels see them.
// ---------------------------------------------------------------------------
enum Policy : int32_t {
  kSerial = 0,     // no flags: two stream-ordered launches
  kTileSync = 1,
  kRowSync = 2,
  kConvTileSync = 3,
  kSentinel = 4,
  kStrided = 5,    // self-attention stage 1 -> 2: one counter per head group
};

enum Act : int32_t { kGeluErf = 0, kGeluTanh = 1, kActNone = 2, kRelu = 3 };

// ---------------------------------------------------------------------------
// Scheduler parameters shared by the chain kernels (see sched.h).
// ---------------------------------------------------------------------------
struct SchedParams {
  int32_t sched;                   // 0 global counter, 1 per-XCD queues
  int32_t first_phase, last_phase; // queues: phases this launch drains
  uint32_t t_begin, t_end;         // global: item range of this launch
  uint32_t base[kMaxPhases];       // first item of each phase (stage)
  int32_t rows[kMaxPhases];        // tile rows of each phase's grid
  int32_t cols[kMaxPhases];        // tile columns of each phase's grid
  int32_t col_major[kMaxPhases];   // a queue lists its slab column by column
  int32_t slab_rows;               // queues slab rows (1) or columns (0)
  uint32_t qcount[kMaxPhases][kNumQueues];  // items per queue and phase
  uint32_t qstart[kMaxPhases][kNumQueues];  // offset of a queue's list in `order` (table mode)
  const uint32_t* order;           // optional order table
  Ctl* ctl;
};

// First items of a global-counter launch (sched.h, claim_first / sweep_first):
// the i-th first claim on XCD x takes item base + x + 8 i while
// i < ceil((n - x) / 8), through ctl->qnext[x][0]; the shared counter starts
// after them.  The workgroup that draws shared counter value sweep_at runs
// whatever the per-XCD counters still hold before its own item.  n = 0: off.
struct FirstItems {
  uint32_t n;
  uint32_t base;
  uint32_t sweep_at;
  uint32_t skip;  // test knob: workgroups with an odd block index take no first item
};

// Optional per-item trace: one record per work item, at the item's index,
// written by thread 0 with ordinary vector stores.  Times are ticks of the
// constant-rate realtime counter (s_memrealtime; its rate is the device's
// wall-clock rate).  Layout mirrors chain_trace_rec of the C ABI.
struct TraceRec {
  uint32_t item;
  uint16_t wg;       // workgroup (blockIdx.x)
  uint16_t hw;       // XCD << 8 | SE << 5 | SH << 4 | CU
  uint64_t t_start;  // item taken
  uint64_t t_ready;  // first dependency wait returned (t_start if there is none)
  uint64_t t_end;    // item done (after its final barrier)
};
static_assert(sizeof(TraceRec) == 32, "trace record layout");

// ---------------------------------------------------------------------------
// MLP kernel parameters.
// ---------------------------------------------------------------------------
struct MlpParams {
  const void* X;            // [M,H]
  const void* W1;           // [H,F]
  const void* W2;           // [F,H]
  void* Z;                  // [M,F] intermediate
  void* Y;                  // [M,H]
  float* zdbg;              // optional [M,F] fp32 activation
  int32_t M, H, F;
  int32_t mt;               // row tiles
  int32_t nt1, nt2;         // producer / consumer column tiles
  uint32_t P, C;            // producer / consumer work items (tiles x K splits)
  int32_t ks1, ks2;         // K splits of a producer / consumer tile (1 = none)
  float* part1;             // split partials (register images), producer tiles
  float* part2;             // split partials, consumer tiles
  uint32_t part1_bytes, part2_bytes;
  uint32_t* splitcnt;       // split arrivals: producer tiles, then consumer tiles
  SchedParams sp;
  Ctl* ctl;
  uint32_t* tileflags;      // TileSync: one flag (epoch) per producer tile
  uint32_t* rowcnt;         // RowSync: mt counters
  int32_t policy;
  int32_t act;
  uint32_t poll_limit;
  int32_t skip_producer;
  uint32_t delay;
  uint32_t light_acquire;  // intermediate 128-byte aligned: light acquire after a poll
  void* zfill;              // sentinel ring: the slot the next call consumes (refilled at exit)
  uint32_t fill_bytes;      // its size (0 = no ring)
  TraceRec* trace;          // optional per-item records (null = off)
  uint32_t trace_cap;
  int32_t bf16;             // operands, intermediate and output are bf16 (else fp16)
};

// ---------------------------------------------------------------------------
// Conv-pair kernel parameters (implicit GEMM over NHWC pixels).
// ---------------------------------------------------------------------------
struct ConvParams {
  const void* X;            // [N,Hh,Ww,C]
  const void* Wa;           // [R,S,C,K]
  const void* Wb;           // [R,S,K,K]
  void* Z;                  // [N,Hh,Ww,K] intermediate
  void* Y;                  // [N,Hh,Ww,K]
  float* zdbg;              // optional [npix,K] fp32 activation
  int32_t N, Hh, Ww, C, K, R, S, pad;
  int32_t npix;             // N * Hh * Ww
  int32_t mt;               // pixel tiles
  int32_t nt1, nt2;         // producer / consumer channel tiles
  uint32_t P, Cn;           // producer / consumer work items (tiles x K splits)
  int32_t ks1, ks2;         // K splits of a producer / consumer tile (1 = none)
  float* part1;             // split partials (register images)
  float* part2;
  uint32_t part1_bytes, part2_bytes;
  uint32_t* splitcnt;       // split arrivals: producer tiles, then consumer tiles
  SchedParams sp;
  Ctl* ctl;
  uint32_t* tileflags;
  uint32_t* rowcnt;
  int32_t act;
  uint32_t poll_limit;
  int32_t skip_producer;
  uint32_t delay;
  uint32_t light_acquire;  // intermediate 128-byte aligned: light acquire after a poll
  void* zfill;              // sentinel ring: the slot the next call consumes (refilled at exit)
  uint32_t fill_bytes;      // its size (0 = no ring)
  TraceRec* trace;          // optional per-item trace (nullptr = off)
  uint32_t trace_cap;
  int32_t bf16;             // operands, intermediate and output in bf16 (else fp16)
  FirstItems first;         // first items through the per-XCD counters (sched.h)
};

// ---------------------------------------------------------------------------
// Self-attention chain (three stages): XQKV = X Wqkv; per head the fused
// softmax(scale Q S2^T) S3 into XDot; Y = XDot W2.  Hs = heads * 128.
// ---------------------------------------------------------------------------
struct SaParams {
  const void* X;            // [M,H]
  const void* Wqkv;         // [H,3 Hs]
  const void* W2;           // [Hs,H]
  void* QKV;                // [M,3 Hs] intermediate
  void* Dot;                // [M,Hs] intermediate
  void* Y;                  // [M,H]
  int32_t M, H, heads, Hs;
  float scale_log2e;        // softmax scale times log2(e)
  uint32_t P1, P2;          // items of stages 1 and 2 (stage 3 follows)
  uint32_t T1;              // stage-1 tiles
  int32_t ks1;              // K splits of a stage-1 tile below tail_begin (1 = none)
  uint32_t tail_begin;      // first stage-1 tile split ks_tail ways (T1: none)
  int32_t ks_tail;          // K splits of a tile from tail_begin on
  float* part1;             // split partials (register images) of stage-1 tiles
  uint32_t part1_bytes;
  uint32_t* splitcnt;       // split arrivals per stage-1 tile, then per stage-2 (block, head)
  int32_t ks2;              // key splits of a stage-2 item (1 = none)
  int32_t nkb;              // key blocks of 64 (ceil(M / 64))
  float* part2;             // stage-2 split partials (register images: O, max, sum)
  uint32_t part2_bytes;
  int32_t mt1, nc1;         // stage 1 grid: M/128 rows x 3 heads columns
  int32_t nq;               // stage 2 query blocks (M/256)
  int32_t nc3;              // stage 3 columns (H/128)
  SchedParams sp;
  Ctl* ctl;
  uint32_t* sem;            // StridedSync: one counter per head (row-counter region)
  uint32_t* flags1;         // TileSync: XQKV tile flags (epochs)
  uint32_t* flags2;         // XDot tile flags (query block, head) (epochs)
  int32_t policy;           // kSerial, kStrided or kTileSync for stage 1 -> 2
  uint32_t poll_limit;
  int32_t skip_producer;
  uint32_t delay;
  uint32_t light_acquire;
  TraceRec* trace;          // optional per-item trace (nullptr = off)
  uint32_t trace_cap;
  int32_t bf16;             // 1: X, Wqkv, W2, XQKV, XDot and Y are bf16
};

// ---------------------------------------------------------------------------
// Attention-chain kernel parameters: rows of all heads stacked, Q/K/V/O are
// [B*heads*S, d], the scores Sc are [B*heads*S, S].
// ---------------------------------------------------------------------------
struct AttnParams {
  const void* Q;
  const void* K;
  const void* V;
  void* Sc;
  void* O;
  int32_t B, heads, S, d;
  float scale;
  int32_t rows;             // row tiles: B * heads * S / 128
  int32_t ntj;              // producer key tiles per row: S / 128
  uint32_t P, Cn;
  SchedParams sp;
  Ctl* ctl;
  uint32_t* tileflags;
  uint32_t* rowcnt;
  uint32_t poll_limit;
  int32_t skip_producer;
  uint32_t delay;
  uint32_t light_acquire;  // intermediate 128-byte aligned: light acquire after a poll
  void* zfill;              // sentinel ring: the slot the next call consumes (refilled at exit)
  uint32_t fill_bytes;      // its size (0 = no ring)
  TraceRec* trace;          // optional per-item trace (nullptr = off)
  uint32_t trace_cap;
  int32_t bf16;             // Q, K, V, the scores and O in bf16 (else fp16)
  FirstItems first;         // first items through the per-XCD counters (sched.h)
};

// Conv tile configurations: BM output pixels x BN output channels, NS ring
// stages, WM x WN waves, K steps of BK channels of one tap (0 = 64).
struct ConvCfg {
  int bm, bn, ns, wm, wn, bk;
  constexpr int kstep() const { return bk ? bk : 64; }
};
constexpr int kNumConvCfgs = 11;
constexpr ConvCfg kConvCfgs[kNumConvCfgs] = {
    {128, 64, 3, 2, 2},   // 0
    {256, 64, 3, 4, 1},   // 1
    {128, 128, 3, 2, 2},  // 2: K multiple of 128
    {64, 64, 4, 2, 2},    // 3: the automatic choice (long reductions, smaller batches)
    {128, 64, 2, 2, 2},   // 4: short reductions over many pixels (three workgroups per CU)
    {64, 64, 3, 2, 2},    // 5
    {64, 64, 2, 2, 2},    // 6
    {128, 128, 2, 2, 2},  // 7: K multiple of 128, two workgroups per CU
    {128, 64, 3, 2, 2, 32},  // 8: K steps of 32 channels, four workgroups per CU
    {128, 64, 4, 2, 2, 32},  // 9: K steps of 32, three steps in flight, three per CU
    {64, 64, 4, 2, 2, 32},   // 10: K steps of 32
};

// Tile configurations of the MLP chain: producer BM x BN1, consumer BM x BN2,
// K step BK, NS LDS stages (of the A operand), WM x WN waves of 64 lanes,
// NSB stages of the B operand (0 = NS).  The kernel table in chain_mlp.h
// lists the same configurations.
struct MlpCfg {
  int bm, bn1, bn2, bk, ns, wm, wn, nsb;
};
constexpr int kNumMlpCfgs = 19;
constexpr MlpCfg kMlpCfgs[kNumMlpCfgs] = {
    {64, 64, 64, 64, 4, 2, 2},     // 0: smallest tile; any H, F multiple of 64
    {128, 128, 128, 64, 4, 2, 2},  // 1
    {256, 128, 128, 64, 3, 2, 2},  // 2
    {128, 64, 64, 64, 3, 2, 2},    // 3: more tiles at small M
    {64, 128, 128, 64, 3, 2, 2},   // 4: more row tiles at small M
    {256, 256, 256, 64, 2, 2, 2},  // 5: one wave per SIMD, 128 x 128 per wave
    {256, 128, 128, 64, 3, 4, 2},  // 6: 8 waves
    {128, 128, 128, 64, 4, 2, 4},  // 7: 8 waves
    {256, 192, 192, 64, 2, 2, 2},  // 8: F = 32 x 192 and H = 64 x 192 fill 256 CUs
    {128, 192, 192, 64, 3, 2, 2},  // 9
    {64, 192, 192, 64, 4, 2, 2},   // 10
    {128, 256, 256, 64, 3, 2, 2},  // 11
    {256, 192, 192, 64, 2, 4, 2},  // 12: 8 waves
    {256, 256, 256, 32, 4, 2, 4},  // 13: 8 waves, K steps of 32, 3 steps in flight
    {256, 192, 192, 32, 4, 2, 2},  // 14
    {128, 192, 192, 32, 5, 2, 2},  // 15
    {256, 256, 256, 32, 4, 2, 2},  // 16
    {256, 192, 192, 64, 3, 2, 2, 2},  // 17: split ring, A three slots deep, B two (144 KB)
    {256, 192, 192, 64, 3, 4, 2, 2},  // 18: the same with 8 waves
};

// ---------------------------------------------------------------------------
// Conv2DTileSync halo range (host and device).  For a "same" convolution
// (stride 1, 2 * pad = R - 1 = S - 1) output pixel m (flattened n, p, q) reads
// input pixels whose flattened index lies in [m - pad*Ww - pad,
// m + pad*Ww + pad]; a tile of bm consecutive output pixels therefore reads
// the producer pixel tiles first..last below.  The interval may include
// pixels of a neighbouring image row or image that the window does not touch,
// so the range is a superset of the exact read set: waiting on it is safe.
// ---------------------------------------------------------------------------
__host__ __device__ inline void conv_dep_range(int64_t tile, int64_t npix, int64_t Ww,
                                               int64_t bm, int64_t pad, int64_t* first,
                                               int64_t* last) {
  const int64_t m0 = tile * bm;
  int64_t m1 = m0 + bm - 1;
  if (m1 > npix - 1) m1 = npix - 1;
  int64_t lo = m0 - pad * Ww - pad;
  int64_t hi = m1 + pad * Ww + pad;
  if (lo < 0) lo = 0;
  if (hi > npix - 1) hi = npix - 1;
  *first = lo / bm;
  *last = hi / bm;
}

// Columns [slab_begin(q), slab_begin(q + 1)) of an nt-column tile grid belong
// to queue q (XCD q): each weight panel is read by one XCD only.
__host__ __device__ inline uint32_t slab_begin(int q, int nt) {
  return (uint32_t)(q * nt / kNumQueues);
}

}  // namespace tls

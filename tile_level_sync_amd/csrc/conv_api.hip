// C ABI of the conv-pair chain: argument checks, tile choice, workspace
// layout, scheduling and launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <vector>

#include "internal.h"
#include "runtime_internal.h"

namespace tls {

hipError_t conv_launch(int cfg, const ConvParams& p, int policy, int grid, hipStream_t s);
hipError_t conv_occupancy(int cfg, int* blocks);
bool conv_bf16_cfg(int cfg);

namespace {

constexpr int kConvOccKeyBase = 200;

// 64 x 64 tiles with a four-stage ring, except for a short reduction over
// many pixels (64 channels, at least 32768 pixels: the 56 x 56 x 64 pair at
// batch 32), which takes 128 x 64 tiles with a two-stage ring: there a tile
// has only 9 K steps, each short, so it is bound by load latency, and the
// 48 KB footprint lets three workgroups share a CU and hide it (4-12 %
// faster than the three-stage 128 x 64 and 128 x 128 tiles, 25 % faster than
// 64 x 64).  With 128 channels or more (18 or more K steps) and on smaller
// batches the deeper ring wins: Conv2DTileSync on the 14 x 14 x 256 pair at
// batch 8 27 vs 31 us.  The same 128 x 64 tile with K steps of 32 channels
// and a four-stage ring (18 steps, three in flight, the same 48 KB) runs the
// 56 x 56 x 64 pair at batch 32 another 3-7 % faster (Conv2DTileSync 38.0 vs
// 40.3 us, serial 56.2 vs 59.5; medians of two interleaved sweeps on two
// boxes), and takes its place.  Between the two, 128 channels over at least 16384
// pixels (the 28 x 28 x 128 pair at batch 32: 18 K steps, 392 tiles) take
// 128 x 64 tiles with a three-stage ring: Conv2DTileSync 37.7 vs 43.2 us,
// serial 47.3 vs 54.2 (medians, interleaved), while the same pair at batch 8
// and the 56 x 56 x 64 pair at batch 8 stay faster on 64 x 64.
int conv_auto_cfg(int64_t npix, int K) {
  if (K <= 64 && npix >= 32768) return 9;
  if (K > 64 && K <= 128 && npix >= 16384) return 0;
  return 3;
}

// Automatic K split: the largest power of two S <= 8 with tiles * S within
// the 512 resident workgroups of the automatic 64 x 64 tile (two per CU on
// 256 CUs) and at least 16 K steps per split.  A conv tile's time is set by
// its per-step latency, so a second resident item per CU nearly halves the
// time to drain the tiles, while splits shorter than 16 steps spend more on
// the prologue and the partial reduction than they save.  Measured on the
// ResNet-38 pairs (Conv2DTileSync, median us, S = 1 / 2 / 4 / 8): 7x7x512 at
// batch 32 (200 tiles) 67.5 / 51.9 / 53.7 / 69.1, at batch 8 54.2 / 40.3 /
// 38.4 / 45.8, at batch 1 51.7 / 37.0 / 31.9 / 36.4; 14x14x256 at batch 32
// 45.7 / 52.7 / 64.9, at batch 1 32.2 / 27.4 / 27.4; 28x28x128 at batch 1
// 22.5 / 23.0.  Device independent on purpose: the split fixes the summation
// order of the result.
constexpr int64_t kConvSplitSlots = 512;
int conv_auto_split(int64_t tiles, int64_t ksteps) {
  int s = 1;
  while (s < 8 && tiles * s * 2 <= kConvSplitSlots && ksteps % (2 * s) == 0 &&
         ksteps / (2 * s) >= 16)
    s *= 2;
  return s;
}

struct ConvPlan {
  int cfg;
  int64_t mt;
  int nt;
  int ks1, ks2;
  uint32_t tiles;  // per conv
  uint32_t P, C;   // work items
};

struct ConvLayout {
  size_t tileflags, order, part1, part2, z, total;
};

ConvLayout conv_layout(int64_t npix, int K, const ConvPlan& pl, bool z_in_ws) {
  const ConvCfg& c = kConvCfgs[pl.cfg];
  ConvLayout L;
  L.tileflags = kTileFlagOffset;
  L.order = kFixedBytes;
  L.part1 = align_up(L.order + (size_t)(pl.P + pl.C) * 4, 256);
  L.part2 = align_up(L.part1 + (pl.ks1 > 1 ? (size_t)pl.tiles * pl.ks1 * c.bm * c.bn * 4 : 0), 256);
  L.z = align_up(L.part2 + (pl.ks2 > 1 ? (size_t)pl.tiles * pl.ks2 * c.bm * c.bn * 4 : 0), 256);
  L.total = align_up(L.z + (z_in_ws ? (size_t)npix * K * 2 : 0), 256);
  return L;
}

// Kernel policy for a conv call (TILESYNC is read as the halo-aware
// Conv2DTileSync: plain per-tile flags would ignore the halo).
int conv_kernel_policy(int policy) {
  return policy == CHAIN_TILESYNC ? (int)kConvTileSync : policy;
}

chain_status conv_check(const chain_conv_args* a, ConvPlan* out) {
  if (!a || !a->X || !a->Wa || !a->Wb || !a->Y) return CHAIN_EINVAL;
  if (!aligned16(a->X) || !aligned16(a->Wa) || !aligned16(a->Wb) || !aligned16(a->Y))
    return CHAIN_EINVAL;
  if ((a->z_out && !aligned16(a->z_out)) || (a->z_debug_f32 && !aligned16(a->z_debug_f32)))
    return CHAIN_EINVAL;
  if (a->N <= 0 || a->Hh <= 0 || a->Ww <= 0 || a->C <= 0 || a->K <= 0 || a->R <= 0 ||
      a->S <= 0 || a->pad < 0 || a->stride <= 0)
    return CHAIN_EINVAL;
  if (a->stride != 1 || 2 * a->pad != a->R - 1 || 2 * a->pad != a->S - 1)
    return CHAIN_EUNSUPPORTED;
  if (a->C % 64 || a->K % 64 || a->Hh >= 32768 || a->Ww >= 32768) return CHAIN_EUNSUPPORTED;
  const int64_t npix = (int64_t)a->N * a->Hh * a->Ww;
  const int64_t lim = (int64_t)1 << 31;
  if (npix * a->C * 2 >= lim || npix * a->K * 2 >= lim ||
      (int64_t)a->R * a->S * std::max(a->C, a->K) * a->K * 2 >= lim)
    return CHAIN_EUNSUPPORTED;
  if (a->dtype != CHAIN_F16 && a->dtype != CHAIN_BF16) return CHAIN_EUNSUPPORTED;
  if (a->act < CHAIN_ACT_GELU_ERF || a->act > CHAIN_ACT_RELU) return CHAIN_EINVAL;
  switch (a->policy) {
    case CHAIN_STREAM_SERIAL:
    case CHAIN_TILESYNC:
    case CHAIN_CONV2D_TILESYNC:
    case CHAIN_ROWSYNC:
    case CHAIN_SENTINEL:
      break;
    default:
      return CHAIN_EUNSUPPORTED;
  }
  if (a->order < CHAIN_ORDER_XCD || a->order > CHAIN_ORDER_STRIDED || a->order_stride < 0)
    return CHAIN_EINVAL;
  if (a->grid < 0 || a->debug_skip_producer < 0) return CHAIN_EINVAL;
  if (a->debug_first_skip < 0 || a->debug_first_skip > 1) return CHAIN_EINVAL;
  if (a->tile_cfg < 0 || a->tile_cfg > kNumConvCfgs) return CHAIN_EINVAL;
  const int cfg = a->tile_cfg == 0 ? conv_auto_cfg(npix, a->K) : a->tile_cfg - 1;
  if (a->K % kConvCfgs[cfg].bn) return CHAIN_EUNSUPPORTED;
  if (a->dtype == CHAIN_BF16 && !conv_bf16_cfg(cfg)) return CHAIN_EUNSUPPORTED;
  const int64_t mt = (npix + kConvCfgs[cfg].bm - 1) / kConvCfgs[cfg].bm;
  if (a->policy == CHAIN_ROWSYNC && mt > (int64_t)kMaxRowCounters) return CHAIN_EUNSUPPORTED;
  if ((a->policy == CHAIN_TILESYNC || a->policy == CHAIN_CONV2D_TILESYNC) &&
      mt * (a->K / kConvCfgs[cfg].bn) > (int64_t)kMaxTileFlags)
    return CHAIN_EUNSUPPORTED;
  if (a->split_k1 < 0 || a->split_k1 > 16 || a->split_k2 < 0 || a->split_k2 > 16)
    return CHAIN_EINVAL;
  ConvPlan pl;
  pl.cfg = cfg;
  pl.mt = mt;
  pl.nt = a->K / kConvCfgs[cfg].bn;
  pl.tiles = (uint32_t)(mt * pl.nt);
  const int bk = kConvCfgs[cfg].kstep();
  const int64_t kt1 = (int64_t)a->R * a->S * a->C / bk, kt2 = (int64_t)a->R * a->S * a->K / bk;
  pl.ks1 = a->split_k1 ? a->split_k1 : conv_auto_split(pl.tiles, kt1);
  pl.ks2 = a->split_k2 ? a->split_k2 : conv_auto_split(pl.tiles, kt2);
  if (kt1 % pl.ks1 || kt2 % pl.ks2) return CHAIN_EUNSUPPORTED;
  pl.P = pl.tiles * (uint32_t)pl.ks1;
  pl.C = pl.tiles * (uint32_t)pl.ks2;
  const int64_t lim32 = (int64_t)1 << 32;  // partial buffers: 32-bit byte offsets
  const int64_t tile_bytes = (int64_t)kConvCfgs[cfg].bm * kConvCfgs[cfg].bn * 4;
  if ((int64_t)pl.tiles * pl.ks1 * tile_bytes >= lim32 ||
      (int64_t)pl.tiles * pl.ks2 * tile_bytes >= lim32)
    return CHAIN_EUNSUPPORTED;
  if ((pl.ks1 > 1 || pl.ks2 > 1) && 2 * (int64_t)pl.tiles > (int64_t)kMaxSplitCounters)
    return CHAIN_EUNSUPPORTED;
  if (chain_status rs = ring_validate(a->z_ring, a->ring_slots, a->policy, a->z_out))
    return rs;
  if (a->trace && (!aligned16(a->trace) || (uint64_t)a->trace_capacity < (uint64_t)pl.P + pl.C))
    return CHAIN_EINVAL;
  *out = pl;
  return CHAIN_OK;
}

// Scheduler parameters and order table of a call.  The default order runs
// as one global counter here: per-XCD row slabs measured 4-9 % slower for
// every policy of the conv pair.  The interleaved order places each consumer
// row of pixel tiles one producer row after the last producer tile its 3x3
// halo reads (conv_dep_range), so that no consumer is handed out before a
// producer it reads.
chain_status conv_sched_plan(const chain_conv_args* a, const ConvPlan& pl, SchedParams* sp,
                             std::vector<uint32_t>* tab) {
  const int order = a->order == CHAIN_ORDER_XCD ? CHAIN_ORDER_ROW_MAJOR : a->order;
  const int64_t npix = (int64_t)a->N * a->Hh * a->Ww;
  std::vector<int> dep_last((size_t)pl.mt);
  for (int64_t c = 0; c < pl.mt; ++c) {
    int64_t first = 0, last = 0;
    conv_dep_range(c, npix, a->Ww, kConvCfgs[pl.cfg].bm, a->pad, &first, &last);
    dep_last[(size_t)c] = (int)last;
  }
  const int rows[2] = {(int)pl.mt, (int)pl.mt};
  const int cols[2] = {pl.nt * pl.ks1, pl.nt * pl.ks2};
  return plan_sched_phases(sp, order, a->order_seed,
                           a->order_stride ? a->order_stride : kDefaultOrderStride, 2, rows,
                           cols, nullptr, true, a->policy == CHAIN_STREAM_SERIAL,
                           dep_last.data(), tab);
}

}  // namespace
}  // namespace tls

using namespace tls;

extern "C" {

chain_status chain_conv_dep_range(int64_t tile, int64_t N, int64_t Hh, int64_t Ww, int64_t bm,
                                  int R, int S, int pad, int64_t* first, int64_t* last) {
  if (!first || !last || N <= 0 || Hh <= 0 || Ww <= 0 || bm <= 0 || R <= 0 || S <= 0 || pad < 0)
    return CHAIN_EINVAL;
  if (2 * pad != R - 1 || 2 * pad != S - 1) return CHAIN_EUNSUPPORTED;
  const int64_t npix = N * Hh * Ww;
  const int64_t tiles = (npix + bm - 1) / bm;
  if (tile < 0 || tile >= tiles) return CHAIN_EINVAL;
  conv_dep_range(tile, npix, Ww, bm, pad, first, last);
  return CHAIN_OK;
}

size_t chain_conv_workspace_bytes(int N, int Hh, int Ww, int C, int K, int R, int S, int pad,
                                  int stride, int policy, int dtype, int tile_cfg) {
  chain_conv_args a;
  std::memset(&a, 0, sizeof(a));
  static const char dummy[16] __attribute__((aligned(16))) = {0};
  a.X = a.Wa = a.Wb = dummy;
  a.Y = (void*)dummy;
  a.N = N; a.Hh = Hh; a.Ww = Ww; a.C = C; a.K = K; a.R = R; a.S = S;
  a.pad = pad; a.stride = stride; a.policy = policy; a.dtype = dtype;
  a.tile_cfg = tile_cfg < 0 ? 0 : tile_cfg + 1;
  ConvPlan pl;
  if (conv_check(&a, &pl) != CHAIN_OK) return 0;
  const int64_t npix = (int64_t)N * Hh * Ww;
  return conv_layout(npix, K, pl, true).total;
}

chain_status chain_conv_plan(int N, int Hh, int Ww, int C, int K, int tile_cfg, chain_plan* out) {
  if (!out) return CHAIN_EINVAL;
  chain_conv_args a;
  std::memset(&a, 0, sizeof(a));
  static const char dummy[16] __attribute__((aligned(16))) = {0};
  a.X = a.Wa = a.Wb = dummy;
  a.Y = (void*)dummy;
  a.N = N; a.Hh = Hh; a.Ww = Ww; a.C = C; a.K = K; a.R = 3; a.S = 3;
  a.pad = 1; a.stride = 1; a.policy = CHAIN_CONV2D_TILESYNC; a.dtype = CHAIN_F16;
  a.tile_cfg = tile_cfg < 0 ? 0 : tile_cfg + 1;
  ConvPlan pl;
  const chain_status st = conv_check(&a, &pl);
  if (st != CHAIN_OK) return st;
  out->tile_cfg = pl.cfg;
  out->row_tiles = pl.mt;
  out->prod_col_tiles = pl.nt;
  out->cons_col_tiles = pl.nt;
  out->producer_tiles = pl.tiles;
  out->consumer_tiles = pl.tiles;
  out->split_k1 = pl.ks1;
  out->split_k2 = pl.ks2;
  return CHAIN_OK;
}

chain_status chain_conv_ex(const chain_conv_args* a) {
  ConvPlan pl;
  chain_status st = conv_check(a, &pl);
  if (st != CHAIN_OK) return st;
  const int cfg = pl.cfg;
  const hipStream_t stream = (hipStream_t)a->stream;
  const int64_t npix = (int64_t)a->N * a->Hh * a->Ww;
  const int64_t mt = pl.mt;
  const int nt = pl.nt;
  const uint32_t P = pl.P, C = pl.C;  // work items (tiles x K splits)

  int dev = 0;
  if ((st = current_device(&dev)) != CHAIN_OK) return st;
  int cus = 0;
  if ((st = device_cus(dev, &cus)) != CHAIN_OK) return st;
  int occ = 0;
  if ((st = kernel_occupancy(dev, kConvOccKeyBase + cfg, conv_occupancy, cfg, &occ)) != CHAIN_OK)
    return st;
  if (occ <= 0) return CHAIN_EUNSUPPORTED;

  const ConvLayout L = conv_layout(npix, a->K, pl, a->z_out == nullptr && a->z_ring == nullptr);
  void* ws = a->workspace;
  if (ws) {
    if (!aligned16(ws)) return CHAIN_EINVAL;
    if (a->workspace_bytes < L.total) return CHAIN_ENOMEM;
  } else if ((st = library_workspace(dev, L.total, &ws)) != CHAIN_OK) {
    return st;
  }
  char* base = (char*)ws;

  ConvParams p;
  std::memset(&p, 0, sizeof(p));
  {
    std::vector<uint32_t> tab;
    if ((st = conv_sched_plan(a, pl, &p.sp, &tab)) != CHAIN_OK) return st;
    if ((st = install_order(&p.sp, tab, ws, L.order, stream)) != CHAIN_OK) return st;
  }
  p.X = a->X;
  p.Wa = a->Wa;
  p.Wb = a->Wb;
  const size_t zbytes = (size_t)npix * a->K * 2;
  p.Z = a->z_out ? a->z_out : (void*)(base + L.z);
  bool prime = a->policy == CHAIN_SENTINEL;
  if (a->z_ring) {
    const RingPick r = ring_pick(a->z_ring, a->ring_slots, a->ring_index, zbytes);
    p.Z = r.z;
    p.zfill = r.zfill;
    p.fill_bytes = r.fill_bytes;
    prime = r.prime;
  }
  p.Y = a->Y;
  p.zdbg = a->z_debug_f32;
  p.trace = (TraceRec*)a->trace;
  p.trace_cap = a->trace ? a->trace_capacity : 0u;
  p.bf16 = a->dtype == CHAIN_BF16 ? 1 : 0;
  p.N = a->N;
  p.Hh = a->Hh;
  p.Ww = a->Ww;
  p.C = a->C;
  p.K = a->K;
  p.R = a->R;
  p.S = a->S;
  p.pad = a->pad;
  p.npix = (int32_t)npix;
  p.mt = (int32_t)mt;
  p.nt1 = nt;
  p.nt2 = nt;
  p.P = P;
  p.Cn = C;
  p.ks1 = pl.ks1;
  p.ks2 = pl.ks2;
  p.part1 = (float*)(base + L.part1);
  p.part2 = (float*)(base + L.part2);
  p.part1_bytes = (uint32_t)(L.part2 - L.part1);
  p.part2_bytes = (uint32_t)(L.z - L.part2);
  p.splitcnt = (uint32_t*)(base + kSplitCntOffset);
  p.ctl = (Ctl*)base;
  p.tileflags = (uint32_t*)(base + L.tileflags);
  p.rowcnt = (uint32_t*)(base + kRowCntOffset);
  p.act = a->act == CHAIN_ACT_GELU_ERF ? (int)kRelu : a->act;
  p.poll_limit = a->poll_limit ? a->poll_limit : kDefaultPollLimit;
  p.skip_producer = a->debug_skip_producer - 1;
  p.delay = a->debug_delay;
  // Whole 128-byte lines per tile (row strides are multiples of 128 bytes).
  p.light_acquire = ((uintptr_t)p.Z % 128u) == 0 ? 1u : 0u;
  const int kpol = conv_kernel_policy(a->policy);

  const int slots = cus * occ;
  if (prime) {  // a ring slot after the first was filled by the call before
    if ((st = fill_u32(p.Z, 0xFFFFFFFFu, zbytes, stream)) != CHAIN_OK) return st;
  }
  // With the default order (the shared counter, no table) a launch's first
  // claims go to the eight per-XCD counters: producer items [0, nfirst) as
  // first items, the shared counter from nfirst on, and the workgroup that
  // draws value P sweeps the per-XCD counters before its own item.
  const bool spread = p.sp.sched == 0 && p.sp.order == nullptr;
  auto first_items = [&](int grid, uint32_t begin, uint32_t end) {
    set_first_items(&p.sp, &p.first, spread && begin == 0, grid, begin, end, P,
                    a->debug_first_skip != 0);
  };
  hipError_t e;
  if (a->policy == CHAIN_STREAM_SERIAL) {
    const int g1 = a->grid ? a->grid : std::min<int>((int)P, slots);
    first_items(g1, 0, P);
    p.sp.first_phase = p.sp.last_phase = 0;
    e = conv_launch(cfg, p, kpol, g1, stream);
    if (e != hipSuccess) return hip_fail(e);
    first_items(0, P, P + C);
    p.sp.first_phase = p.sp.last_phase = 1;
    e = conv_launch(cfg, p, kpol, a->grid ? a->grid : std::min<int>((int)C, slots), stream);
    if (e != hipSuccess) return hip_fail(e);
  } else {
    const int g = a->grid ? a->grid : std::min<int>((int)(P + C), slots);
    first_items(g, p.sp.t_begin, p.sp.t_end);
    e = conv_launch(cfg, p, kpol, g, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  return finish_call(ws, stream);
}

chain_status chain_conv_order(const chain_conv_args* a, uint32_t* items, size_t capacity,
                              size_t* count) {
  if (!count) return CHAIN_EINVAL;
  ConvPlan pl;
  chain_status st = conv_check(a, &pl);
  if (st != CHAIN_OK) return st;
  SchedParams sp;
  std::vector<uint32_t> tab, seq;
  if ((st = conv_sched_plan(a, pl, &sp, &tab)) != CHAIN_OK) return st;
  order_sequence(sp, tab, &seq);
  return export_sequence(seq, items, capacity, count);
}

chain_status chain_conv(const void* X, const void* Wa, const void* Wb, void* Y, int N, int Hh,
                        int Ww, int C, int K, int R, int S, int pad, int stride, int policy) {
  chain_conv_args a;
  std::memset(&a, 0, sizeof(a));
  a.X = X; a.Wa = Wa; a.Wb = Wb; a.Y = Y;
  a.N = N; a.Hh = Hh; a.Ww = Ww; a.C = C; a.K = K; a.R = R; a.S = S;
  a.pad = pad; a.stride = stride; a.policy = policy;
  return chain_conv_ex(&a);
}

}  // extern "C"

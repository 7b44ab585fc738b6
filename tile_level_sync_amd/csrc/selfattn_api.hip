// C ABI of the three-stage self-attention chain: argument checks, workspace
// layout, scheduling and launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>

#include "internal.h"
#include "runtime_internal.h"

namespace tls {

hipError_t selfattn_launch(const SaParams& p, int grid, hipStream_t s);
hipError_t selfattn_occupancy(int, int* blocks);

namespace {

constexpr int kSaOccKey = 400;
constexpr int64_t kGlobalOrderMinM = 1024;
// Stage 1 and 3 tiles (the kernel's SaT), head dimension, queries per stage-2 item.
constexpr int kRowTile = 128, kColTile = 128, kD = 128, kBQ = 256;

// Automatic K split of stage 1 (the XQKV projection), when its 128 x 128
// tiles fit one wave of the chip (kSplitTarget, the MI355X CU count): the S
// of 1 to 4 that finishes the tiles soonest, in rounds of one item per
// workgroup, ceil(tiles * S / 256) rounds of 1 / S of a tile each, the
// smaller S on a tie, and only if that is at most two thirds of the unsplit
// rounds (the partials and the reductions cost the rest: at M = 640, four
// splits in three rounds, 0.75, measured 14 % slower than none); S divides
// the K steps and leaves each split at least 16 (1024 of K).  On the GPT-3
// shard: 4 up to M = 128, 3 at M = 256 (216 items, one round of a third) and
// at M = 512 (432 items, two rounds of a third, 4.5 % faster than one
// unsplit round), none at M = 640 and 768.  When the tiles fill more
// than one wave, the same rule splits only the tiles past the last whole wave
// (the tail, last in item order): at M = 2048 576 tiles are 2.25 waves of
// 114 us items, and the quarter wave after the two whole ones holds up every
// head's attention stage; split four ways it becomes a wave of quarter-length
// items.  Shape only, so the bits of XQKV do not depend on the policy, the
// order or the device.
constexpr int64_t kSplitTarget = 256;
int sa_auto_split(int64_t tiles, int64_t ksteps) {
  int best = 1;
  int64_t best_rounds = (tiles + kSplitTarget - 1) / kSplitTarget;  // rounds of whole tiles
  for (int s = 2; s <= 4; ++s) {
    if (ksteps % s || ksteps / s < 16) continue;
    const int64_t rounds = (tiles * s + kSplitTarget - 1) / kSplitTarget;
    if (rounds * best < best_rounds * s) {  // rounds / s < best_rounds / best
      best = s;
      best_rounds = rounds;
    }
  }
  const int64_t unsplit = (tiles + kSplitTarget - 1) / kSplitTarget;
  return 3 * best_rounds <= 2 * best * unsplit ? best : 1;
}

// Automatic key split of stage 2 (the fused dot product): when its (query
// block, head) items do not fill the chip, the largest S of 4, 3, 2 that
// keeps items * S within one wave, leaves each split at least 8 key blocks
// (512 keys: below that the merge costs more than the extra CUs give back)
// and gives every split a non-empty range.  Shape only, like the stage-1
// split.
constexpr int kMinKeyBlocksPerSplit = 8;
bool sa_keys_split_ok(int64_t nkb, int s) {
  const int64_t per = (nkb + s - 1) / s;
  return (s - 1) * per < nkb;  // the last split starts below the last key block
}
int sa_auto_split2(int64_t pairs, int64_t nkb) {
  for (int s = 4; s >= 2; --s)
    if (pairs * s <= kSplitTarget && nkb / s >= kMinKeyBlocksPerSplit && sa_keys_split_ok(nkb, s))
      return s;
  return 1;
}

// Register image of one stage-2 split: 17 chunks of 16 bytes per thread of
// 512 (the 16 chunks of O^T, then the running max and sum).
constexpr int64_t kSaPart2Bytes = 17 * 512 * 16;

struct SaPlan {
  int mt, nq, nc1, nc3, ks1, nkb, ks2;
  uint32_t T1, P1, pairs, P2, P3;
  uint32_t tail_begin;  // first tile split ks_tail ways (T1: no tail split)
  int ks_tail;
  // Partial register images of stage 1: uniform splits or the tail's.
  uint32_t part1_images() const {
    return ks1 > 1 ? T1 * (uint32_t)ks1 : (ks_tail > 1 ? (T1 - tail_begin) * (uint32_t)ks_tail : 0u);
  }
};

SaPlan sa_plan(const chain_selfattn_args* a) {
  SaPlan pl;
  pl.mt = (int)((a->M + kRowTile - 1) / kRowTile);  // ragged M: the last tiles are partial
  pl.nq = (int)((a->M + kBQ - 1) / kBQ);
  pl.nc1 = 3 * a->heads;
  pl.nc3 = (int)(a->H / kColTile);
  pl.T1 = (uint32_t)pl.mt * pl.nc1;
  pl.ks1 = a->split_k1                    ? a->split_k1
           : pl.T1 <= (uint32_t)kSplitTarget ? sa_auto_split(pl.T1, a->H / 64)
                                             : 1;
  pl.tail_begin = pl.T1;
  pl.ks_tail = 1;
  if (!a->split_k1 && pl.ks1 == 1 && pl.T1 > kSplitTarget && pl.T1 % kSplitTarget) {
    const uint32_t tail = pl.T1 % kSplitTarget;
    const int s = sa_auto_split(tail, a->H / 64);
    if (s > 1) {
      pl.tail_begin = pl.T1 - tail;
      pl.ks_tail = s;
    }
  }
  pl.P1 = pl.tail_begin * (uint32_t)pl.ks1 + (pl.T1 - pl.tail_begin) * (uint32_t)pl.ks_tail;
  pl.nkb = (int)((a->M + 63) / 64);
  pl.pairs = (uint32_t)pl.nq * a->heads;
  pl.ks2 = a->split_keys ? a->split_keys : sa_auto_split2(pl.pairs, pl.nkb);
  pl.P2 = pl.pairs * (uint32_t)pl.ks2;
  pl.P3 = (uint32_t)pl.mt * pl.nc3;
  return pl;
}

struct SaLayout {
  size_t order, part1, part2, qkv, dot, total;
};

SaLayout sa_layout(int64_t M, int64_t Hs, const SaPlan& pl, bool qkv_in_ws, bool dot_in_ws) {
  SaLayout L;
  L.order = kFixedBytes;
  L.part1 = align_up(L.order + (size_t)(pl.P1 + pl.P2 + pl.P3) * 4, 256);
  L.part2 = align_up(L.part1 + (size_t)pl.part1_images() * kRowTile * kColTile * 4, 256);
  L.qkv = align_up(L.part2 + (pl.ks2 > 1 ? (size_t)pl.P2 * kSaPart2Bytes : 0), 256);
  L.dot = align_up(L.qkv + (qkv_in_ws ? (size_t)M * 3 * Hs * 2 : 0), 256);
  L.total = align_up(L.dot + (dot_in_ws ? (size_t)M * Hs * 2 : 0), 256);
  return L;
}

chain_status sa_check(const chain_selfattn_args* a) {
  if (!a || !a->X || !a->Wqkv || !a->W2 || !a->Y) return CHAIN_EINVAL;
  if (!aligned16(a->X) || !aligned16(a->Wqkv) || !aligned16(a->W2) || !aligned16(a->Y))
    return CHAIN_EINVAL;
  if ((a->qkv_out && !aligned16(a->qkv_out)) || (a->dot_out && !aligned16(a->dot_out)))
    return CHAIN_EINVAL;
  if (a->M <= 0 || a->H <= 0 || a->heads <= 0 || a->d <= 0) return CHAIN_EINVAL;
  if (!(a->scale > 0.0f) || !std::isfinite(a->scale)) return CHAIN_EINVAL;
  if (a->d != kD || a->H % kColTile) return CHAIN_EUNSUPPORTED;
  if (a->dtype != CHAIN_F16 && a->dtype != CHAIN_BF16) return CHAIN_EUNSUPPORTED;
  const int64_t Hs = (int64_t)a->heads * a->d;
  const int64_t lim = (int64_t)1 << 31;
  if (a->M * a->H * 2 >= lim || a->H * 3 * Hs * 2 >= lim || a->M * 3 * Hs * 2 >= lim ||
      Hs * a->H * 2 >= lim)
    return CHAIN_EUNSUPPORTED;
  switch (a->policy) {
    case CHAIN_STREAM_SERIAL:
    case CHAIN_STRIDEDSYNC:
    case CHAIN_TILESYNC:
      break;
    default:
      return CHAIN_EUNSUPPORTED;
  }
  if (a->order != CHAIN_ORDER_XCD && a->order != CHAIN_ORDER_ROW_MAJOR &&
      a->order != CHAIN_ORDER_INTERLEAVED)
    return CHAIN_EINVAL;
  if (a->grid < 0 || a->debug_skip_producer < 0) return CHAIN_EINVAL;
  const int64_t mt = (a->M + kRowTile - 1) / kRowTile, nq = (a->M + kBQ - 1) / kBQ;
  if (a->heads > (int64_t)kMaxRowCounters) return CHAIN_EUNSUPPORTED;
  if (mt * 3 * a->heads + nq * a->heads > (int64_t)kMaxTileFlags) return CHAIN_EUNSUPPORTED;
  if (a->split_k1 < 0 || a->split_k1 > 16) return CHAIN_EINVAL;
  if (a->split_keys < 0 || a->split_keys > 16) return CHAIN_EINVAL;
  const SaPlan pl = sa_plan(a);
  if ((a->H / 64) % pl.ks1) return CHAIN_EUNSUPPORTED;
  if (pl.part1_images() > 0 &&
      ((int64_t)pl.T1 > (int64_t)kMaxSplitCounters ||
       (int64_t)pl.part1_images() * kRowTile * kColTile * 4 >= ((int64_t)1 << 32)))
    return CHAIN_EUNSUPPORTED;
  if (a->trace && (!aligned16(a->trace) ||
                   (uint64_t)a->trace_capacity < (uint64_t)pl.P1 + pl.P2 + pl.P3))
    return CHAIN_EINVAL;
  if (pl.ks2 > 1) {
    if (!sa_keys_split_ok(pl.nkb, pl.ks2)) return CHAIN_EUNSUPPORTED;  // an empty split
    if ((int64_t)pl.T1 + pl.pairs > (int64_t)kMaxSplitCounters ||
        (int64_t)pl.P2 * kSaPart2Bytes >= ((int64_t)1 << 32))
      return CHAIN_EUNSUPPORTED;
  }
  return CHAIN_OK;
}

int sa_kernel_policy(int policy) {
  switch (policy) {
    case CHAIN_STRIDEDSYNC:
      return kStrided;
    case CHAIN_TILESYNC:
      return kTileSync;
    default:
      return kSerial;
  }
}

}  // namespace
}  // namespace tls

using namespace tls;

extern "C" {

size_t chain_selfattn_workspace_bytes(int64_t M, int64_t H, int heads, int d, int policy,
                                      int dtype) {
  chain_selfattn_args a;
  std::memset(&a, 0, sizeof(a));
  static const char dummy[16] __attribute__((aligned(16))) = {0};
  a.X = a.Wqkv = a.W2 = dummy;
  a.Y = (void*)dummy;
  a.M = M; a.H = H; a.heads = heads; a.d = d; a.scale = 1.0f; a.policy = policy;
  a.dtype = dtype;
  if (sa_check(&a) != CHAIN_OK) return 0;
  const int64_t Hs = (int64_t)heads * d;
  return sa_layout(M, Hs, sa_plan(&a), true, true).total;
}

chain_status chain_selfattn_plan(int64_t M, int64_t H, int heads, int d, int split_k1,
                                 int split_keys, chain_selfattn_plan_info* out) {
  if (!out) return CHAIN_EINVAL;
  chain_selfattn_args a;
  std::memset(&a, 0, sizeof(a));
  static const char dummy[16] __attribute__((aligned(16))) = {0};
  a.X = a.Wqkv = a.W2 = dummy;
  a.Y = (void*)dummy;
  a.M = M; a.H = H; a.heads = heads; a.d = d; a.scale = 1.0f;
  a.policy = CHAIN_STRIDEDSYNC;
  a.dtype = CHAIN_F16;
  a.split_k1 = split_k1;
  a.split_keys = split_keys;
  const chain_status st = sa_check(&a);
  if (st != CHAIN_OK) return st;
  const SaPlan pl = sa_plan(&a);
  out->row_tile = kRowTile;
  out->col_tile = kColTile;
  out->row_tiles = pl.mt;
  out->stage1_tiles = pl.T1;
  out->split_k1 = pl.ks1;
  out->split_keys = pl.ks2;
  out->query_blocks = pl.nq;
  out->key_blocks = pl.nkb;
  out->stage1_items = pl.P1;
  out->stage2_items = pl.P2;
  out->stage3_items = pl.P3;
  out->tail_tiles = pl.T1 - pl.tail_begin;
  out->split_k_tail = pl.ks_tail;
  out->reserved = 0;
  return CHAIN_OK;
}

chain_status chain_selfattn_ex(const chain_selfattn_args* a) {
  chain_status st = sa_check(a);
  if (st != CHAIN_OK) return st;
  const hipStream_t stream = (hipStream_t)a->stream;
  const int64_t Hs = (int64_t)a->heads * a->d;
  const SaPlan pl = sa_plan(a);
  const int mt = pl.mt, nq = pl.nq, nc3 = pl.nc3, nc1 = pl.nc1;
  const uint32_t P1 = pl.P1, P2 = pl.P2, P3 = pl.P3;

  int dev = 0;
  if ((st = current_device(&dev)) != CHAIN_OK) return st;
  int cus = 0;
  if ((st = device_cus(dev, &cus)) != CHAIN_OK) return st;
  int occ = 0;
  if ((st = kernel_occupancy(dev, kSaOccKey, selfattn_occupancy, 0, &occ)) != CHAIN_OK)
    return st;
  if (occ <= 0) return CHAIN_EUNSUPPORTED;

  const SaLayout L = sa_layout(a->M, Hs, pl, a->qkv_out == nullptr, a->dot_out == nullptr);
  void* ws = a->workspace;
  if (ws) {
    if (!aligned16(ws)) return CHAIN_EINVAL;
    if (a->workspace_bytes < L.total) return CHAIN_ENOMEM;
  } else if ((st = library_workspace(dev, L.total, &ws)) != CHAIN_OK) {
    return st;
  }
  char* base = (char*)ws;

  SaParams p;
  std::memset(&p, 0, sizeof(p));
  // Stage 1 lists a head group's tiles (three slices, every row; the K
  // splits of a tile as adjacent columns) before the next group; stage 2
  // likewise head by head; stage 3 row by row.  Queues take column slabs, so
  // a head's groups stay on one XCD.  With a split tail, stage 1's items are
  // one row in item order (the tail's splits last).
  const bool tail = pl.tail_begin < pl.T1;
  const int rows[3] = {tail ? 1 : mt, nq, mt},
            cols[3] = {tail ? (int)P1 : nc1 * pl.ks1, a->heads * pl.ks2, nc3},
            colmaj[3] = {tail ? 0 : 1, 1, 0};
  // From M = 1024 on the default order runs as one global counter: 2.5-4.5 %
  // faster there under every policy; the per-XCD queues win 4-10 % below.
  const int order = a->order == CHAIN_ORDER_XCD && a->M >= kGlobalOrderMinM ? CHAIN_ORDER_ROW_MAJOR
                                                                            : a->order;
  if ((st = setup_sched_phases(&p.sp, order, a->order_seed, kDefaultOrderStride, 3, rows, cols,
                               colmaj, false, ws, L.order, stream,
                               a->policy == CHAIN_STREAM_SERIAL)) != CHAIN_OK)
    return st;
  p.X = a->X;
  p.Wqkv = a->Wqkv;
  p.W2 = a->W2;
  p.QKV = a->qkv_out ? a->qkv_out : (void*)(base + L.qkv);
  p.Dot = a->dot_out ? a->dot_out : (void*)(base + L.dot);
  p.Y = a->Y;
  p.M = (int32_t)a->M;
  p.H = (int32_t)a->H;
  p.heads = a->heads;
  p.Hs = (int32_t)Hs;
  p.scale_log2e = a->scale * 1.4426950408889634f;
  p.P1 = P1;
  p.P2 = P2;
  p.T1 = pl.T1;
  p.ks1 = pl.ks1;
  p.tail_begin = pl.tail_begin;
  p.ks_tail = pl.ks_tail;
  p.part1 = (float*)(base + L.part1);
  p.part1_bytes = (uint32_t)(L.part2 - L.part1);
  p.ks2 = pl.ks2;
  p.nkb = pl.nkb;
  p.part2 = (float*)(base + L.part2);
  p.part2_bytes = (uint32_t)(L.qkv - L.part2);
  p.splitcnt = (uint32_t*)(base + kSplitCntOffset);
  p.mt1 = mt;
  p.nc1 = nc1;
  p.nq = nq;
  p.nc3 = nc3;
  p.ctl = (Ctl*)base;
  p.sem = (uint32_t*)(base + kRowCntOffset);
  p.flags1 = (uint32_t*)(base + kTileFlagOffset);
  p.flags2 = p.flags1 + (size_t)pl.T1 * kFlagStride;
  p.policy = sa_kernel_policy(a->policy);
  p.poll_limit = a->poll_limit ? a->poll_limit : kDefaultPollLimit;
  p.skip_producer = a->debug_skip_producer - 1;
  p.delay = a->debug_delay;
  p.trace = (TraceRec*)a->trace;
  p.trace_cap = a->trace ? a->trace_capacity : 0u;
  p.bf16 = a->dtype == CHAIN_BF16 ? 1 : 0;
  // Whole 128-byte lines per tile in both intermediates.
  p.light_acquire =
      ((uintptr_t)p.QKV % 128u) == 0 && ((uintptr_t)p.Dot % 128u) == 0 ? 1u : 0u;

  const int slots = cus * occ;
  hipError_t e;
  if (a->policy == CHAIN_STREAM_SERIAL) {
    const uint32_t begin[3] = {0, P1, P1 + P2}, end[3] = {P1, P1 + P2, P1 + P2 + P3};
    for (int ph = 0; ph < 3; ++ph) {
      p.sp.t_begin = begin[ph];
      p.sp.t_end = end[ph];
      p.sp.first_phase = p.sp.last_phase = ph;
      const int g = a->grid ? a->grid : std::min<int>((int)(end[ph] - begin[ph]), slots);
      e = selfattn_launch(p, g, stream);
      if (e != hipSuccess) return hip_fail(e);
    }
  } else {
    e = selfattn_launch(p, a->grid ? a->grid : std::min<int>((int)(P1 + P2 + P3), slots),
                        stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  return finish_call(ws, stream);
}

chain_status chain_selfattn(const void* X, const void* Wqkv, const void* W2, void* Y, int64_t M,
                            int64_t H, int heads, int d, float scale, int policy) {
  chain_selfattn_args a;
  std::memset(&a, 0, sizeof(a));
  a.X = X;
  a.Wqkv = Wqkv;
  a.W2 = W2;
  a.Y = Y;
  a.M = M;
  a.H = H;
  a.heads = heads;
  a.d = d;
  a.scale = scale;
  a.policy = policy;
  return chain_selfattn_ex(&a);
}

}  // extern "C"

// C ABI of the MLP chain: argument checks, tile choice, workspace layout,
// order table and launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <vector>

#include "internal.h"
#include "runtime_internal.h"

namespace tls {

hipError_t mlp_launch(int cfg, const MlpParams& p, int grid, hipStream_t s);
bool mlp_bf16_cfg(int cfg);
hipError_t mlp_occupancy(int cfg, int* blocks);
int mlp_lds_bytes(int cfg);

namespace {

constexpr int kMlpOccKeyBase = 100;
constexpr int64_t kGlobalOrderMaxM = 128;

// Automatic tile choice for the MLP chain (shape only, never the policy, so
// every policy computes the same bits).
int mlp_auto_cfg(int64_t M, int64_t H, int64_t F) {
  auto fits = [&](int c) {
    return F % kMlpCfgs[c].bn1 == 0 && H % kMlpCfgs[c].bn2 == 0;
  };
  // Measured on MI355X for the GPT-3 slice (H = 12288, F = 6144): 8-wave
  // 128 x 128 up to M = 384 (also for the smallest batches, where 64 x 64
  // tiles measured slower with every policy; at M = 384 4-6 % ahead of
  // 256 x 128) and 256 x 128 up to M = 512 (with the K splits below);
  // above, tiles 192 wide so that the column
  // counts (F / 192 = 32, H / 192 = 64) times the row tiles fill the 256 CUs
  // in whole waves: 128 x 192 up to M = 1024, 256 x 192 above with four waves
  // and the split ring (A three slots deep, B two): 4-10 % fewer cycles than
  // the two-stage 256 x 192 tiles at M = 2048 (part of it is given back as a
  // lower clock under the heavier MFMA load).
  const int prefs[4] = {M <= 384 ? 7 : (M <= 512 ? 6 : (M <= 1024 ? 9 : 17)), 7, 1, 0};
  for (int c : prefs)
    if (fits(c)) return c;
  return 0;  // 64 x 64 divides every accepted H, F
}

// Automatic K split of one GEMM of the chain: the largest power of two S
// (at most 4) with tiles * S within `target` work items, S dividing the K
// steps and each split at least 16 K steps (1024 of K).  The target is one
// wave of the chip (kSplitTarget, the MI355X CU count), and one and a half
// waves for the producer GEMM of tiles of at most 128 x 128, whose short
// items leave the tail of the wave to the consumers that follow them.  On
// the GPT-3 slice that is (4, 2) for the two GEMMs at M <= 128, where the
// chain only streams the weights and needs more loads in flight, (4, 1) at
// M = 256 (3-12 % ahead of (2, 1) on four boxes, interleaved), (2, 1) at
// M = 384 and 512, none above.  8 or more splits measured slower: the
// partial tiles they write and read back cost more than the parallelism
// gains.  Device independent on purpose: the split fixes the summation order,
// hence the bits of the result.
constexpr int64_t kSplitTarget = 256;
constexpr int64_t kSplitTargetSmallProducer = 384;
int mlp_auto_split(int64_t tiles, int64_t ksteps, int64_t target) {
  for (int s = 4; s >= 2; s /= 2)
    if (tiles * s <= target && ksteps % s == 0 && ksteps / s >= 16) return s;
  return 1;
}

struct MlpPlan {
  int cfg;
  int64_t mt, nt1, nt2;
  int ks1, ks2;
  uint32_t ptiles, ctiles;  // tiles
  uint32_t P, C;            // work items
};

struct MlpLayout {
  size_t tileflags, order, splitcnt, part1, part2, z, total;
};

MlpLayout mlp_layout(int64_t M, int64_t F, const MlpPlan& pl, bool z_in_ws) {
  const MlpCfg& c = kMlpCfgs[pl.cfg];
  MlpLayout L;
  L.tileflags = kTileFlagOffset;
  L.splitcnt = kSplitCntOffset;
  L.order = kFixedBytes;
  L.part1 = align_up(L.order + (size_t)(pl.P + pl.C) * 4, 256);
  L.part2 = align_up(
      L.part1 + (pl.ks1 > 1 ? (size_t)pl.ptiles * pl.ks1 * c.bm * c.bn1 * 4 : 0), 256);
  L.z = align_up(L.part2 + (pl.ks2 > 1 ? (size_t)pl.ctiles * pl.ks2 * c.bm * c.bn2 * 4 : 0),
                 256);
  L.total = align_up(L.z + (z_in_ws ? (size_t)M * F * 2 : 0), 256);
  return L;
}

chain_status mlp_check(const chain_mlp_args* a, MlpPlan* out) {
  if (!a || !a->X || !a->W1 || !a->W2 || !a->Y) return CHAIN_EINVAL;
  if (!aligned16(a->X) || !aligned16(a->W1) || !aligned16(a->W2) || !aligned16(a->Y))
    return CHAIN_EINVAL;
  if ((a->z_out && !aligned16(a->z_out)) || (a->z_debug_f32 && !aligned16(a->z_debug_f32)))
    return CHAIN_EINVAL;
  if (a->M <= 0 || a->H <= 0 || a->F <= 0) return CHAIN_EINVAL;
  if (a->H % 64 || a->F % 64) return CHAIN_EUNSUPPORTED;
  const int64_t lim = (int64_t)1 << 31;
  if (a->M * a->H * 2 >= lim || a->H * a->F * 2 >= lim || a->M * a->F * 2 >= lim)
    return CHAIN_EUNSUPPORTED;
  if (a->dtype != CHAIN_F16 && a->dtype != CHAIN_BF16) return CHAIN_EUNSUPPORTED;
  if (a->act < CHAIN_ACT_GELU_ERF || a->act > CHAIN_ACT_RELU) return CHAIN_EINVAL;
  switch (a->policy) {
    case CHAIN_STREAM_SERIAL:
    case CHAIN_TILESYNC:
    case CHAIN_ROWSYNC:
    case CHAIN_SENTINEL:
      break;
    default:
      return CHAIN_EUNSUPPORTED;
  }
  if (a->order < CHAIN_ORDER_XCD || a->order > CHAIN_ORDER_STRIDED || a->order_stride < 0)
    return CHAIN_EINVAL;
  if (a->grid < 0) return CHAIN_EINVAL;
  if (a->tile_cfg < 0 || a->tile_cfg > kNumMlpCfgs) return CHAIN_EINVAL;
  if (a->debug_skip_producer < 0) return CHAIN_EINVAL;
  if (a->split_k1 < 0 || a->split_k1 > 16 || a->split_k2 < 0 || a->split_k2 > 16)
    return CHAIN_EINVAL;
  int cfg = a->tile_cfg == 0 ? mlp_auto_cfg(a->M, a->H, a->F) : a->tile_cfg - 1;
  const MlpCfg& c = kMlpCfgs[cfg];
  if (a->F % c.bn1 || a->H % c.bn2) return CHAIN_EUNSUPPORTED;
  if (a->dtype == CHAIN_BF16 && !mlp_bf16_cfg(cfg)) return CHAIN_EUNSUPPORTED;
  const int64_t mt = (a->M + c.bm - 1) / c.bm;
  if (a->policy == CHAIN_ROWSYNC && mt > (int64_t)kMaxRowCounters) return CHAIN_EUNSUPPORTED;
  MlpPlan pl;
  pl.cfg = cfg;
  pl.mt = mt;
  pl.nt1 = a->F / c.bn1;
  pl.nt2 = a->H / c.bn2;
  const int64_t kt1 = a->H / c.bk, kt2 = a->F / c.bk;
  const bool small_tile = c.bm * c.bn1 <= 128 * 128;
  pl.ks1 = a->split_k1 ? a->split_k1
                       : mlp_auto_split(mt * pl.nt1, kt1,
                                        small_tile ? kSplitTargetSmallProducer : kSplitTarget);
  pl.ks2 = a->split_k2 ? a->split_k2 : mlp_auto_split(mt * pl.nt2, kt2, kSplitTarget);
  if (kt1 % pl.ks1 || kt2 % pl.ks2) return CHAIN_EUNSUPPORTED;
  pl.ptiles = (uint32_t)(mt * pl.nt1);
  pl.ctiles = (uint32_t)(mt * pl.nt2);
  pl.P = pl.ptiles * (uint32_t)pl.ks1;
  pl.C = pl.ctiles * (uint32_t)pl.ks2;
  const int64_t lim32 = (int64_t)1 << 32;  // partial buffers: 32-bit byte offsets
  if ((int64_t)pl.ptiles * pl.ks1 * c.bm * c.bn1 * 4 >= lim32 ||
      (int64_t)pl.ctiles * pl.ks2 * c.bm * c.bn2 * 4 >= lim32)
    return CHAIN_EUNSUPPORTED;
  if ((pl.ks1 > 1 || pl.ks2 > 1) && (int64_t)pl.ptiles + pl.ctiles > (int64_t)kMaxSplitCounters)
    return CHAIN_EUNSUPPORTED;
  if (a->policy == CHAIN_TILESYNC && pl.ptiles > kMaxTileFlags) return CHAIN_EUNSUPPORTED;
  if (chain_status rs = ring_validate(a->z_ring, a->ring_slots, a->policy, a->z_out))
    return rs;
  if (a->trace && (!aligned16(a->trace) || (uint64_t)a->trace_capacity < (uint64_t)pl.P + pl.C))
    return CHAIN_EINVAL;
  *out = pl;
  return CHAIN_OK;
}

// Scheduler parameters and order table of a call.  The K splits of a tile
// are adjacent items of its row: column slabs and orders treat them as extra
// columns.  At M <= 128 (one row of tiles, the weights streamed once) the
// default order runs as one global counter: 4-6 % faster than the per-XCD
// column slabs, which win from M = 512 on.
chain_status mlp_sched_plan(const chain_mlp_args* a, const MlpPlan& pl, SchedParams* sp,
                            std::vector<uint32_t>* tab) {
  const int order = a->order == CHAIN_ORDER_XCD && a->M <= kGlobalOrderMaxM ? CHAIN_ORDER_ROW_MAJOR
                                                                            : a->order;
  const int rows[2] = {(int)pl.mt, (int)pl.mt};
  const int cols[2] = {(int)(pl.nt1 * pl.ks1), (int)(pl.nt2 * pl.ks2)};
  return plan_sched_phases(sp, order, a->order_seed,
                           a->order_stride ? a->order_stride : kDefaultOrderStride, 2, rows,
                           cols, nullptr, false, a->policy == CHAIN_STREAM_SERIAL, nullptr, tab);
}

}  // namespace

// Workspace bytes a chain_mlp_ex call with these arguments needs (its plan,
// splits and whether the intermediate lives in the workspace).
chain_status mlp_workspace_need(const chain_mlp_args* a, size_t* need) {
  MlpPlan pl;
  chain_status st = mlp_check(a, &pl);
  if (st != CHAIN_OK) return st;
  *need = mlp_layout(a->M, a->F, pl, a->z_out == nullptr && a->z_ring == nullptr).total;
  return CHAIN_OK;
}

}  // namespace tls

using namespace tls;

extern "C" {

int chain_num_tile_cfgs(void) { return kNumMlpCfgs; }

chain_status chain_tile_cfg_info(int cfg, chain_tile_info* out) {
  if (cfg < 0 || cfg >= kNumMlpCfgs || !out) return CHAIN_EINVAL;
  out->bm = kMlpCfgs[cfg].bm;
  out->bn1 = kMlpCfgs[cfg].bn1;
  out->bn2 = kMlpCfgs[cfg].bn2;
  out->bk = kMlpCfgs[cfg].bk;
  out->threads = 64 * kMlpCfgs[cfg].wm * kMlpCfgs[cfg].wn;
  out->lds_bytes = mlp_lds_bytes(cfg);
  return CHAIN_OK;
}

chain_status chain_mlp_plan(int64_t M, int64_t H, int64_t F, int dtype, int tile_cfg,
                            chain_plan* out) {
  if (!out) return CHAIN_EINVAL;
  chain_mlp_args a;
  std::memset(&a, 0, sizeof(a));
  static const char dummy[16] __attribute__((aligned(16))) = {0};
  a.X = a.W1 = a.W2 = dummy;
  a.Y = (void*)dummy;
  a.M = M;
  a.H = H;
  a.F = F;
  a.dtype = dtype;
  a.tile_cfg = tile_cfg < 0 ? 0 : tile_cfg + 1;
  a.policy = CHAIN_TILESYNC;
  MlpPlan pl;
  chain_status st = mlp_check(&a, &pl);
  if (st != CHAIN_OK) return st;
  out->tile_cfg = pl.cfg;
  out->row_tiles = pl.mt;
  out->prod_col_tiles = pl.nt1;
  out->cons_col_tiles = pl.nt2;
  out->producer_tiles = pl.ptiles;
  out->consumer_tiles = pl.ctiles;
  out->split_k1 = pl.ks1;
  out->split_k2 = pl.ks2;
  return CHAIN_OK;
}

size_t chain_mlp_workspace_bytes(int64_t M, int64_t H, int64_t F, int policy, int dtype,
                                 int tile_cfg) {
  chain_mlp_args a;
  std::memset(&a, 0, sizeof(a));
  static const char dummy[16] __attribute__((aligned(16))) = {0};
  a.X = a.W1 = a.W2 = dummy;
  a.Y = (void*)dummy;
  a.M = M;
  a.H = H;
  a.F = F;
  a.dtype = dtype;
  a.tile_cfg = tile_cfg < 0 ? 0 : tile_cfg + 1;
  a.policy = policy;
  MlpPlan pl;
  if (mlp_check(&a, &pl) != CHAIN_OK) return 0;
  return mlp_layout(M, F, pl, true).total;
}

chain_status chain_mlp_ex(const chain_mlp_args* a) {
  MlpPlan pl;
  chain_status st = mlp_check(a, &pl);
  if (st != CHAIN_OK) return st;
  const int cfg = pl.cfg;
  const hipStream_t stream = (hipStream_t)a->stream;
  const int64_t mt = pl.mt, nt1 = pl.nt1, nt2 = pl.nt2;
  const uint32_t P = pl.P, C = pl.C;  // work items (tiles x K splits)

  int dev = 0;
  if ((st = current_device(&dev)) != CHAIN_OK) return st;
  int cus = 0;
  if ((st = device_cus(dev, &cus)) != CHAIN_OK) return st;
  int occ = 0;
  if ((st = kernel_occupancy(dev, kMlpOccKeyBase + cfg, mlp_occupancy, cfg, &occ)) != CHAIN_OK)
    return st;
  if (occ <= 0) return CHAIN_EUNSUPPORTED;

  const MlpLayout L = mlp_layout(a->M, a->F, pl, a->z_out == nullptr && a->z_ring == nullptr);
  void* ws = a->workspace;
  if (ws) {
    if (!aligned16(ws)) return CHAIN_EINVAL;
    if (a->workspace_bytes < L.total) return CHAIN_ENOMEM;
  } else if ((st = library_workspace(dev, L.total, &ws)) != CHAIN_OK) {
    return st;
  }
  char* base = (char*)ws;

  MlpParams p;
  std::memset(&p, 0, sizeof(p));
  {
    std::vector<uint32_t> tab;
    if ((st = mlp_sched_plan(a, pl, &p.sp, &tab)) != CHAIN_OK) return st;
    if ((st = install_order(&p.sp, tab, ws, L.order, stream)) != CHAIN_OK) return st;
  }
  p.X = a->X;
  p.W1 = a->W1;
  p.W2 = a->W2;
  const size_t zbytes = (size_t)a->M * a->F * 2;
  p.Z = a->z_out ? a->z_out : (void*)(base + L.z);
  p.bf16 = a->dtype == CHAIN_BF16 ? 1 : 0;
  p.trace = (TraceRec*)a->trace;
  p.trace_cap = a->trace ? a->trace_capacity : 0u;
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
  p.M = (int32_t)a->M;
  p.H = (int32_t)a->H;
  p.F = (int32_t)a->F;
  p.mt = (int32_t)mt;
  p.nt1 = (int32_t)nt1;
  p.nt2 = (int32_t)nt2;
  p.P = P;
  p.C = C;
  p.ks1 = pl.ks1;
  p.ks2 = pl.ks2;
  p.part1 = (float*)(base + L.part1);
  p.part2 = (float*)(base + L.part2);
  p.part1_bytes = (uint32_t)(L.part2 - L.part1);
  p.part2_bytes = (uint32_t)(L.z - L.part2);
  p.splitcnt = (uint32_t*)(base + L.splitcnt);
  p.ctl = (Ctl*)base;
  p.tileflags = (uint32_t*)(base + L.tileflags);
  p.rowcnt = (uint32_t*)(base + kRowCntOffset);
  p.policy = a->policy;
  p.act = a->act;
  p.poll_limit = a->poll_limit ? a->poll_limit : kDefaultPollLimit;
  p.skip_producer = a->debug_skip_producer - 1;
  p.delay = a->debug_delay;
  // Whole 128-byte lines per tile (row strides are multiples of 128 bytes).
  p.light_acquire = ((uintptr_t)p.Z % 128u) == 0 ? 1u : 0u;

  const int slots = cus * occ;
  if (prime) {
    // Every element of Z starts as 0xFFFF (sentinel guide, 4.6.4.2: the buffer
    // is initialised before the consumer loads it; here by a kernel earlier in
    // the same stream).  A ring slot after the first was filled by the call
    // before (sentinel_refill).
    if ((st = fill_u32(p.Z, 0xFFFFFFFFu, zbytes, stream)) != CHAIN_OK) return st;
  }
  hipError_t e;
  if (a->policy == CHAIN_STREAM_SERIAL) {
    p.sp.t_begin = 0;
    p.sp.t_end = P;
    p.sp.first_phase = p.sp.last_phase = 0;
    int g1 = a->grid ? a->grid : std::min<int>((int)P, slots);
    e = mlp_launch(cfg, p, g1, stream);
    if (e != hipSuccess) return hip_fail(e);
    p.sp.t_begin = P;
    p.sp.t_end = P + C;
    p.sp.first_phase = p.sp.last_phase = 1;
    int g2 = a->grid ? a->grid : std::min<int>((int)C, slots);
    e = mlp_launch(cfg, p, g2, stream);
    if (e != hipSuccess) return hip_fail(e);
  } else {
    int g = a->grid ? a->grid : std::min<int>((int)(P + C), slots);
    e = mlp_launch(cfg, p, g, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  return finish_call(ws, stream);
}

chain_status chain_mlp_order(const chain_mlp_args* a, uint32_t* items, size_t capacity,
                             size_t* count) {
  if (!count) return CHAIN_EINVAL;
  MlpPlan pl;
  chain_status st = mlp_check(a, &pl);
  if (st != CHAIN_OK) return st;
  SchedParams sp;
  std::vector<uint32_t> tab, seq;
  if ((st = mlp_sched_plan(a, pl, &sp, &tab)) != CHAIN_OK) return st;
  order_sequence(sp, tab, &seq);
  return export_sequence(seq, items, capacity, count);
}

chain_status chain_mlp(const void* X, const void* W1, const void* W2, void* Y, int64_t M,
                       int64_t H, int64_t F, int policy) {
  chain_mlp_args a;
  std::memset(&a, 0, sizeof(a));
  a.X = X;
  a.W1 = W1;
  a.W2 = W2;
  a.Y = Y;
  a.M = M;
  a.H = H;
  a.F = F;
  a.policy = policy;
  a.dtype = CHAIN_F16;
  a.act = CHAIN_ACT_GELU_ERF;
  return chain_mlp_ex(&a);
}

}  // extern "C"

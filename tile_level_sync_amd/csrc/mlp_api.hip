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
hipError_t mlp_occupancy(int cfg, int* blocks);
int mlp_lds_bytes(int cfg);

namespace {

constexpr int kMlpOccKeyBase = 100;

// Automatic tile choice for the MLP chain (shape only, never the policy, so
// every policy computes the same bits).
int mlp_auto_cfg(int64_t M, int64_t H, int64_t F) {
  auto fits = [&](int c) {
    return F % kMlpCfgs[c].bn1 == 0 && H % kMlpCfgs[c].bn2 == 0;
  };
  // Measured on MI355X for the GPT-3 slice (H = 12288, F = 6144): 128 x 128
  // with 8 waves up to M = 512; above, tiles 192 wide so that the column
  // counts (F / 192 = 32, H / 192 = 64) times the row tiles fill the 256 CUs
  // in whole waves: 128 x 192 up to M = 1024, 256 x 192 (8 waves) above.
  const int prefs[3] = {M <= 512 ? 7 : (M <= 1024 ? 9 : 12), 7, 1};
  if (M <= 64) return 0;
  for (int c : prefs)
    if (fits(c)) return c;
  return 0;  // 64 x 64 divides every accepted H, F
}

struct MlpLayout {
  size_t tileflags, order, z, total;
};

MlpLayout mlp_layout(int64_t M, int64_t F, uint32_t P, uint32_t C, bool z_in_ws) {
  MlpLayout L;
  L.tileflags = kTileFlagOffset;
  L.order = align_up(L.tileflags + (size_t)P * kLine, 256);
  L.z = align_up(L.order + (size_t)(P + C) * 4, 256);
  L.total = align_up(L.z + (z_in_ws ? (size_t)M * F * 2 : 0), 256);
  return L;
}

chain_status mlp_check(const chain_mlp_args* a, int* cfg_out) {
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
  if (a->dtype != CHAIN_F16) return CHAIN_EUNSUPPORTED;
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
  if (a->order != CHAIN_ORDER_XCD && a->order != CHAIN_ORDER_ROW_MAJOR &&
      a->order != CHAIN_ORDER_INTERLEAVED)
    return CHAIN_EINVAL;
  if (a->grid < 0) return CHAIN_EINVAL;
  if (a->tile_cfg < 0 || a->tile_cfg > kNumMlpCfgs) return CHAIN_EINVAL;
  if (a->debug_skip_producer < 0) return CHAIN_EINVAL;
  int cfg = a->tile_cfg == 0 ? mlp_auto_cfg(a->M, a->H, a->F) : a->tile_cfg - 1;
  if (a->F % kMlpCfgs[cfg].bn1 || a->H % kMlpCfgs[cfg].bn2) return CHAIN_EUNSUPPORTED;
  const int64_t mt = (a->M + kMlpCfgs[cfg].bm - 1) / kMlpCfgs[cfg].bm;
  if (a->policy == CHAIN_ROWSYNC && mt > (int64_t)kMaxRowCounters) return CHAIN_EUNSUPPORTED;
  *cfg_out = cfg;
  return CHAIN_OK;
}

}  // namespace
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
  int cfg = 0;
  chain_status st = mlp_check(&a, &cfg);
  if (st != CHAIN_OK) return st;
  const MlpCfg& c = kMlpCfgs[cfg];
  out->tile_cfg = cfg;
  out->row_tiles = (M + c.bm - 1) / c.bm;
  out->prod_col_tiles = F / c.bn1;
  out->cons_col_tiles = H / c.bn2;
  out->producer_tiles = out->row_tiles * out->prod_col_tiles;
  out->consumer_tiles = out->row_tiles * out->cons_col_tiles;
  return CHAIN_OK;
}

size_t chain_mlp_workspace_bytes(int64_t M, int64_t H, int64_t F, int policy, int dtype,
                                 int tile_cfg) {
  chain_plan pl;
  if (chain_mlp_plan(M, H, F, dtype, tile_cfg, &pl) != CHAIN_OK) return 0;
  (void)policy;
  return mlp_layout(M, F, (uint32_t)pl.producer_tiles, (uint32_t)pl.consumer_tiles, true).total;
}

chain_status chain_mlp_ex(const chain_mlp_args* a) {
  int cfg = 0;
  chain_status st = mlp_check(a, &cfg);
  if (st != CHAIN_OK) return st;
  const MlpCfg& c = kMlpCfgs[cfg];
  const hipStream_t stream = (hipStream_t)a->stream;
  const int64_t mt = (a->M + c.bm - 1) / c.bm;
  const int64_t nt1 = a->F / c.bn1, nt2 = a->H / c.bn2;
  const uint32_t P = (uint32_t)(mt * nt1), C = (uint32_t)(mt * nt2);

  int dev = 0;
  if ((st = current_device(&dev)) != CHAIN_OK) return st;
  int cus = 0;
  if ((st = device_cus(dev, &cus)) != CHAIN_OK) return st;
  int occ = 0;
  if ((st = kernel_occupancy(dev, kMlpOccKeyBase + cfg, mlp_occupancy, cfg, &occ)) != CHAIN_OK)
    return st;
  if (occ <= 0) return CHAIN_EUNSUPPORTED;

  const MlpLayout L = mlp_layout(a->M, a->F, P, C, a->z_out == nullptr);
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
  if ((st = setup_sched(&p.sp, a->order, a->order_seed, (int)mt, (int)nt1, (int)nt2, false, ws,
                        L.order, stream, 100 + (uint64_t)cfg)) != CHAIN_OK)
    return st;
  p.X = a->X;
  p.W1 = a->W1;
  p.W2 = a->W2;
  p.Z = a->z_out ? a->z_out : (void*)(base + L.z);
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
  if (a->policy == CHAIN_SENTINEL) {
    // Every element of Z starts as 0xFFFF (sentinel guide, 4.6.4.2: the buffer
    // is initialised before the consumer loads it; here by a kernel earlier in
    // the same stream).
    if ((st = fill_u32(p.Z, 0xFFFFFFFFu, (size_t)a->M * a->F * 2, stream)) != CHAIN_OK)
      return st;
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

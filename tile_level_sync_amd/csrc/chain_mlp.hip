// MLP chain: instances of the fp16 tile configurations 0-8, and the
// dispatch of a call to the translation unit that holds its kernel.
#include "chain_mlp.h"

namespace tls {

TLS_MLP_UNIT(f16a, TLS_MLP_CFGS_A, 0)

static bool in_b(int cfg) {
  switch (cfg) {
#define X(i, bm, bn1, bn2, bk, ns, wm, wn, nsb) \
  case i:                                   \
    return true;
    TLS_MLP_CFGS_B(X)
#undef X
    default:
      return false;
  }
}

static bool in_a(int cfg) {
  switch (cfg) {
#define X(i, bm, bn1, bn2, bk, ns, wm, wn, nsb) \
  case i:                              \
    return true;
    TLS_MLP_CFGS_A(X)
#undef X
    default:
      return false;
  }
}

hipError_t mlp_launch(int cfg, const MlpParams& p, int grid, hipStream_t s) {
  if (p.bf16) return mlp_launch_bf16(cfg, p, grid, s);
  if (in_a(cfg)) return mlp_launch_f16a(cfg, p, grid, s);
  return in_b(cfg) ? mlp_launch_f16b(cfg, p, grid, s) : mlp_launch_f16c(cfg, p, grid, s);
}

hipError_t mlp_occupancy(int cfg, int* blocks) {
  if (in_a(cfg)) return mlp_occupancy_f16a(cfg, blocks);
  return in_b(cfg) ? mlp_occupancy_f16b(cfg, blocks) : mlp_occupancy_f16c(cfg, blocks);
}

bool mlp_bf16_cfg(int cfg) {
  switch (cfg) {
#define X(i, bm, bn1, bn2, bk, ns, wm, wn, nsb) \
  case i:                              \
    return true;
    TLS_MLP_BF16_CFGS(X)
#undef X
    default:
      return false;
  }
}

int mlp_lds_bytes(int cfg) {
  switch (cfg) {
#define X(i, bm, bn1, bn2, bk, ns, wm, wn, nsb) \
  case i:                              \
    return MlpShapes<bm, bn1, bn2, bk, ns, wm, wn, false, nsb>::SMEM;
    TLS_MLP_CFGS(X)
#undef X
    default:
      return 0;
  }
}

}  // namespace tls

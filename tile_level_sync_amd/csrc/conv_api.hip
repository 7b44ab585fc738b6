// C ABI of the conv-pair chain.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "runtime_internal.h"

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

chain_status chain_conv_ex(const chain_conv_args* a) {
  if (!a) return CHAIN_EINVAL;
  return CHAIN_EUNSUPPORTED;
}

chain_status chain_conv(const void* X, const void* Wa, const void* Wb, void* Y, int N, int Hh,
                        int Ww, int C, int K, int R, int S, int pad, int stride, int policy) {
  chain_conv_args a = {};
  a.X = X; a.Wa = Wa; a.Wb = Wb; a.Y = Y;
  a.N = N; a.Hh = Hh; a.Ww = Ww; a.C = C; a.K = K; a.R = R; a.S = S;
  a.pad = pad; a.stride = stride; a.policy = policy;
  return chain_conv_ex(&a);
}

size_t chain_conv_workspace_bytes(int, int, int, int, int, int, int, int, int, int, int, int) {
  return 0;
}

}  // extern "C"

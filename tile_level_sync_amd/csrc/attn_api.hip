// C ABI of the attention-score chain.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "runtime_internal.h"

using namespace tls;

extern "C" {

chain_status chain_attn_ex(const chain_attn_args* a) {
  if (!a) return CHAIN_EINVAL;
  return CHAIN_EUNSUPPORTED;
}

chain_status chain_attn(const void* Q, const void* K, const void* V, void* O, int B, int heads,
                        int S, int d, float scale, int policy) {
  chain_attn_args a = {};
  a.Q = Q; a.K = K; a.V = V; a.O = O;
  a.B = B; a.heads = heads; a.S = S; a.d = d; a.scale = scale; a.policy = policy;
  return chain_attn_ex(&a);
}

size_t chain_attn_workspace_bytes(int, int, int, int, int, int, int) { return 0; }

}  // extern "C"

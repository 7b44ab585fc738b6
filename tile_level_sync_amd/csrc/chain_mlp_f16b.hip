// MLP chain: instances of the fp16 tile configurations 9-16.
#include "chain_mlp.h"

namespace tls {
TLS_MLP_UNIT(f16b, TLS_MLP_CFGS_B, 0)
}  // namespace tls

// MLP chain: instances of the fp16 tile configurations 17-18 (split rings).
#include "chain_mlp.h"

namespace tls {
TLS_MLP_UNIT(f16c, TLS_MLP_CFGS_C, 0)
}  // namespace tls

// MLP chain: bf16 instances (the configurations the automatic plan picks).
#include "chain_mlp.h"

namespace tls {
TLS_MLP_UNIT(bf16, TLS_MLP_BF16_CFGS, 1)
}  // namespace tls

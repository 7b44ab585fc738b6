"""CPU oracle for the dependent tile-GEMM chains (test infrastructure only).

This package is the slow, plain reference that the HIP path is checked against.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product path (``tile_level_sync_amd``) never
imports, calls or links anything here, and nothing here imports the product.

Sources followed (cited per function):

* "A Framework for Fine-Grained Synchronization of Dependent GPU Kernels"
  (Jangda et al., arXiv 2305.13450), below "the cuSync paper": the MLP block
  (Fig. "Architecture of two building blocks of GPT models" (a)), the
  ResNet-38 conv pairs (Table "Input/output image size, kernel size ...") and
  the dependency definitions of TileSync / RowSync / Conv2DTileSync
  (section "Synchronization Policies"), and the three-kernel self-attention
  block with StridedSync (Fig. "Architecture of two building blocks of GPT
  models" (b), section "Self-Attention").
* "CUDA Programming Guide, 4.6 Fine-Grained Synchronization", below "the
  sentinel guide": producer canonicalisation (4.6.4.3 Producer Rules).

Arithmetic is carried out in float64 on the exact (fp16-representable) input
values; a value is rounded to fp16 only where the chain stores it in fp16
(the intermediate and the output).  Every function here is pinned by the
``-m "not gpu"`` tests against closed forms, brute force or an independent
library routine; none is "parity unpinned".
"""

from .common import (rne_fp16, canon_nan_fp16, normwise_rel_err, rne_bf16, bf16_bits,
                     bf16_values)
from .mlp import gelu_erf, gelu_tanh, mlp_chain, mlp_chain_rows, mlp_chain_bf16
from .conv import conv2d_nhwc, conv_chain, conv_chain_bf16
from .attn import (softmax_rows, attn_chain, attn_chain_rows, attn_chain_bf16,
                   attn_chain_bf16_rows)
from .deps import (mlp_consumer_deps, conv_consumer_deps, attn_consumer_deps,
                   toy_example_deps, selfattn_stage2_deps, strided_group)
from .selfattn import selfattn_chain, selfattn_rows, selfattn_chain_bf16, selfattn_rows_bf16

__all__ = [
    "rne_fp16", "canon_nan_fp16", "normwise_rel_err", "rne_bf16", "bf16_bits", "bf16_values",
    "gelu_erf", "gelu_tanh", "mlp_chain", "mlp_chain_rows", "mlp_chain_bf16",
    "conv2d_nhwc", "conv_chain", "conv_chain_bf16",
    "softmax_rows", "attn_chain", "attn_chain_rows", "attn_chain_bf16", "attn_chain_bf16_rows",
    "mlp_consumer_deps", "conv_consumer_deps", "attn_consumer_deps",
    "toy_example_deps", "selfattn_stage2_deps", "strided_group",
    "selfattn_chain", "selfattn_rows", "selfattn_chain_bf16", "selfattn_rows_bf16",
]

"""Allocation-free MLP entry point (chain_mlp_noalloc): its workspace is the
library's static device array.  Its output must equal chain_mlp_ex's bit for
bit (same plan, so the same summation order) and the oracle's within the fp16
bar, on consecutive calls through the shared array, the second one smaller."""

import ctypes

import numpy as np
import pytest

import oracle
import tile_level_sync_amd as tls
from tile_level_sync_amd import inputs
from tests.gpu_util import TOL_FP16, bits, note, to_dev, to_np, torch_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("pol", ["serial", "tilesync", "rowsync", "sentinel"])
def test_noalloc_matches_chain_mlp_ex_on_consecutive_calls(pol):
    torch = torch_dev()
    shapes = [(512, 1024, 2048, 51), (200, 512, 768, 52)]  # second call smaller, ragged M
    for (M, H, F, seed) in shapes:
        Xn, W1n, W2n = inputs.mlp_inputs(M, H, F, seed=seed)
        Yr = oracle.mlp_chain(Xn, W1n, W2n)[2]
        X, W1, W2 = map(to_dev, (Xn, W1n, W2n))
        ws = torch.zeros(tls.chain_mlp_workspace_bytes(M, H, F, policy=pol), dtype=torch.uint8,
                         device="cuda")
        ref = tls.chain_mlp(X, W1, W2, policy=pol, workspace=ws, check=True).clone()
        note("noalloc policy=%s M=%d H=%d F=%d" % (pol, M, H, F))
        Y = tls.chain_mlp(X, W1, W2, policy=pol, noalloc=True, check=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(Y), bits(ref))
        assert oracle.normwise_rel_err(to_np(Y), Yr) <= TOL_FP16


def test_noalloc_argument_errors():
    """Rejected on the host before any device work: a caller workspace, an
    order that needs a table, and a call larger than the static array."""
    torch = torch_dev()
    lib = tls.load()
    a = tls.chain_mlp_args()
    a.X = a.W1 = a.W2 = a.Y = 1 << 16  # never dereferenced: every case is rejected first
    a.M, a.H, a.F = 256, 512, 768
    a.policy = tls.POLICIES["tilesync"]
    a.workspace = 1 << 16
    assert lib.chain_mlp_noalloc(ctypes.byref(a)) == tls.CHAIN_EINVAL
    a.workspace = None
    a.order_seed = 3
    assert lib.chain_mlp_noalloc(ctypes.byref(a)) == tls.CHAIN_EUNSUPPORTED
    a.order_seed = 0
    a.order = tls.ORDERS["interleaved"]
    assert lib.chain_mlp_noalloc(ctypes.byref(a)) == tls.CHAIN_EUNSUPPORTED
    a.order = 0
    a.M, a.H, a.F = 8192, 4096, 4096  # the intermediate alone is 64 MiB
    assert lib.chain_mlp_noalloc(ctypes.byref(a)) == tls.CHAIN_ESCRATCH
    assert "static scratch" in lib.chain_strerror(tls.CHAIN_ESCRATCH).decode()

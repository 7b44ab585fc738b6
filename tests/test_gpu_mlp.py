"""MLP chain on the GPU through the C ABI: parity with the oracle, exactness,
bit-equality across policies and tile orders, race and watchdog checks."""

import numpy as np
import pytest

import oracle
import tile_level_sync_amd as tls
from tile_level_sync_amd import inputs
from tests.gpu_util import TOL_FP16, TOL_FP32_PRE, bits, note, to_dev, to_np, torch_dev

pytestmark = pytest.mark.gpu

POLICIES = ["serial", "tilesync", "rowsync", "sentinel"]


def _run(X, W1, W2, policy, **kw):
    torch = torch_dev()
    M, H = X.shape
    F = W1.shape[1]
    z = torch.empty((M, F), dtype=torch.float16, device="cuda")
    zd = torch.empty((M, F), dtype=torch.float32, device="cuda") if kw.pop("dbg", False) else None
    Y = tls.chain_mlp(X, W1, W2, policy=policy, z_out=z, z_debug=zd, check=True, **kw)
    torch.cuda.synchronize()
    return Y, z, zd


def test_tiny_config_all_policies():
    """X[64x256] W1[256x1024] W2[1024x256], N(0, 0.02), seed 0."""
    torch_dev()
    Xn, W1n, W2n = inputs.tiny_mlp_inputs(seed=0)
    G, Zr, Yr = oracle.mlp_chain(Xn, W1n, W2n)
    X, W1, W2 = map(to_dev, (Xn, W1n, W2n))
    ref_bits = None
    for pol in POLICIES:
        note("tiny mlp policy=%s" % pol)
        Y, z, zd = _run(X, W1, W2, pol, dbg=True)
        assert oracle.normwise_rel_err(to_np(zd), G) <= TOL_FP32_PRE, pol
        assert oracle.normwise_rel_err(to_np(z), Zr) <= TOL_FP16, pol
        assert oracle.normwise_rel_err(to_np(Y), Yr) <= TOL_FP16, pol
        if ref_bits is None:
            ref_bits = bits(Y)
        np.testing.assert_array_equal(bits(Y), ref_bits, err_msg=pol)


@pytest.mark.parametrize("cfg", list(range(19)))
def test_ragged_multi_tile_each_config(cfg):
    """M not a multiple of any tile height; several tiles in every dimension."""
    torch_dev()
    tc = tls.tile_configs()[cfg]
    M, H, F = (300, 768, 1536) if tc["bn1"] % 3 == 0 else (300, 512, 768)
    Xn, W1n, W2n = inputs.mlp_inputs(M, H, F, seed=1, x_sigma=1.0, w_sigma=0.05)
    G, Zr, Yr = oracle.mlp_chain(Xn, W1n, W2n)
    X, W1, W2 = map(to_dev, (Xn, W1n, W2n))
    ref = None
    for pol in POLICIES:
        note("ragged mlp cfg=%d policy=%s" % (cfg, pol))
        Y, z, zd = _run(X, W1, W2, pol, tile_cfg=cfg, dbg=True)
        assert oracle.normwise_rel_err(to_np(zd), G) <= TOL_FP32_PRE
        assert oracle.normwise_rel_err(to_np(Y), Yr) <= TOL_FP16
        if ref is None:
            ref = bits(Y)
        np.testing.assert_array_equal(bits(Y), ref, err_msg=pol)


def test_exact_small_integers_bit_exact():
    """Entries in {-2..2}/16 keep every fp32 sum exact: the GPU result must
    equal the oracle bit for bit (identity activation)."""
    torch_dev()
    M, H, F = 192, 512, 768
    Xn = inputs.small_int_fp16((M, H), 5, 0)
    W1n = inputs.small_int_fp16((H, F), 5, 1)
    W2n = inputs.small_int_fp16((F, H), 5, 2)
    G, Zr, Yr = oracle.mlp_chain(Xn, W1n, W2n, act="none")
    X, W1, W2 = map(to_dev, (Xn, W1n, W2n))
    for cfg in (0, 1, 2):
        for pol in ("serial", "tilesync"):
            note("exact ints cfg=%d policy=%s" % (cfg, pol))
            Y, z, zd = _run(X, W1, W2, pol, tile_cfg=cfg, act="none", dbg=True)
            np.testing.assert_array_equal(to_np(zd), G.astype(np.float32))
            np.testing.assert_array_equal(bits(z), Zr.view(np.uint16))
            np.testing.assert_array_equal(to_np(Y).astype(np.float64), Yr.astype(np.float64))


def test_closed_forms_zero_and_identity():
    torch_dev()
    M, H = 128, 256
    W1n = np.eye(H, dtype=np.float16)
    W2n = np.eye(H, dtype=np.float16)
    Xn = inputs.normal_fp16((M, H), 1.5, 3, 0)
    X, W1, W2 = map(to_dev, (Xn, W1n, W2n))
    note("closed forms identity")
    Y, z, _ = _run(X, W1, W2, "rowsync")
    # identity weights: Z = RNE(GeLU(X)) elementwise, Y = Z
    Zexp = oracle.rne_fp16(oracle.gelu_erf(Xn.astype(np.float64)))
    assert oracle.normwise_rel_err(to_np(z), Zexp) <= 1e-3
    np.testing.assert_array_equal(to_np(Y).astype(np.float64), to_np(z).astype(np.float64))
    note("closed forms zero input")
    Y0, z0, _ = _run(to_dev(np.zeros_like(Xn)), W1, W2, "tilesync")
    assert not np.any(to_np(Y0)) and not np.any(to_np(z0))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_order_permutations_bit_identical(seed):
    torch_dev()
    M, H, F = 256, 512, 1024
    Xn, W1n, W2n = inputs.mlp_inputs(M, H, F, seed=4)
    X, W1, W2 = map(to_dev, (Xn, W1n, W2n))
    note("order seed=%d reference" % seed)
    ref, _, _ = _run(X, W1, W2, "serial", tile_cfg=3)
    for pol in ("serial", "tilesync", "rowsync", "sentinel"):
        for order in ("xcd", "row_major", "interleaved", "col_major", "strided"):
            note("order seed=%d policy=%s order=%s" % (seed, pol, order))
            Y, _, _ = _run(X, W1, W2, pol, tile_cfg=3, order=order, order_seed=seed)
            np.testing.assert_array_equal(bits(Y), bits(ref))


@pytest.mark.parametrize("grid", [1, 3])
@pytest.mark.parametrize("order", ["interleaved", "col_major", "strided"])
def test_few_workgroups_every_order_completes(grid, order):
    """One or three persistent workgroups walk the whole order: each consumer
    is handed out after every producer it reads, so no wait can block the
    only workgroups there are (a wrong order would end in CHAIN_ETIMEOUT)."""
    torch_dev()
    M, H, F = 256, 512, 768
    Xn, W1n, W2n = inputs.mlp_inputs(M, H, F, seed=6)
    X, W1, W2 = map(to_dev, (Xn, W1n, W2n))
    ref, _, _ = _run(X, W1, W2, "serial", tile_cfg=3)
    for pol in ("tilesync", "rowsync", "sentinel"):
        note("few workgroups grid=%d order=%s policy=%s" % (grid, order, pol))
        Y, _, _ = _run(X, W1, W2, pol, tile_cfg=3, order=order, grid=grid, poll_limit=200000,
                       order_stride=5)
        np.testing.assert_array_equal(bits(Y), bits(ref))


def test_repeated_calls_and_workspace_reuse():
    """Many calls with changing shapes and policies through one workspace:
    epochs advance, row counters reset, results stay identical."""
    torch = torch_dev()
    shapes = [(64, 256, 1024), (200, 512, 768), (64, 256, 1024)]
    data = [tuple(map(to_dev, inputs.mlp_inputs(*s, seed=7))) for s in shapes]
    need = max(tls.chain_mlp_workspace_bytes(*s, tile_cfg=0) for s in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    refs = [tls.chain_mlp(*d, policy="serial", tile_cfg=0, workspace=ws, check=True).clone()
            for d in data]
    for it in range(4):
        for pol in ("tilesync", "rowsync", "sentinel", "serial"):
            for d, r in zip(data, refs):
                note("reuse it=%d policy=%s M=%d" % (it, pol, d[0].shape[0]))
                Y = tls.chain_mlp(*d, policy=pol, tile_cfg=0, workspace=ws, check=True)
                torch.cuda.synchronize()
                np.testing.assert_array_equal(bits(Y), bits(r))


@pytest.mark.parametrize("pol", ["tilesync", "rowsync"])
def test_poison_and_delay_detect_early_reads(pol):
    """Z pre-filled with 0xFFFF (NaN) and producers delayed: a consumer that
    read Z before its producer finished would leave NaN/garbage in Y."""
    torch = torch_dev()
    M, H, F = 256, 512, 1024
    Xn, W1n, W2n = inputs.mlp_inputs(M, H, F, seed=8)
    X, W1, W2 = map(to_dev, (Xn, W1n, W2n))
    ref, _, _ = _run(X, W1, W2, "serial", tile_cfg=3)
    for seed in (0, 5):
        z = torch.full((M, F), -1, dtype=torch.int16, device="cuda").view(torch.float16)
        note("poison policy=%s seed=%d" % (pol, seed))
        Y = tls.chain_mlp(X, W1, W2, policy=pol, tile_cfg=3, z_out=z, order_seed=seed,
                          debug_delay=2, check=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(Y), bits(ref))


def test_split_ring_tilesync_waits_for_whole_rows():
    """The 256 x 192 split-ring tile (configuration 17) runs TileSync with a
    wait for every tile flag of the consumer's row before its main loop: Z
    poisoned with 0xFFFF and producers delayed must still give the serialised
    bits; a producer tile that never posts makes the wait expire
    (CHAIN_ETIMEOUT), and the next call works."""
    torch = torch_dev()
    M, H, F = 300, 768, 1536
    Xn, W1n, W2n = inputs.mlp_inputs(M, H, F, seed=14, x_sigma=1.0, w_sigma=0.05)
    X, W1, W2 = map(to_dev, (Xn, W1n, W2n))
    ref, _, _ = _run(X, W1, W2, "serial", tile_cfg=17)
    for seed, delay in ((0, 2), (3, 4)):
        z = torch.full((M, F), -1, dtype=torch.int16, device="cuda").view(torch.float16)
        note("split-ring tilesync poison seed=%d delay=%d" % (seed, delay))
        Y = tls.chain_mlp(X, W1, W2, policy="tilesync", tile_cfg=17, z_out=z, order_seed=seed,
                          debug_delay=delay, check=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(Y), bits(ref))
    note("split-ring tilesync watchdog")
    with pytest.raises(tls.ChainError) as ei:
        tls.chain_mlp(X, W1, W2, policy="tilesync", tile_cfg=17, debug_skip_producer=1,
                      poll_limit=2000, check=True)
    assert ei.value.status == tls.CHAIN_ETIMEOUT
    note("split-ring tilesync recovery")
    Y = tls.chain_mlp(X, W1, W2, policy="tilesync", tile_cfg=17, check=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(Y), bits(ref))


@pytest.mark.parametrize("cfg", [8, 3, 1])
def test_sentinel_delayed_producers_every_ring_depth(cfg):
    """Sentinel policy with delayed producers on two-, three- and four-stage
    rings (tiles 256x192, 128x64, 128x128): consumers load chunks before their
    producers store them and re-poll them, through the check at the stage
    boundary (two stages) or the one started inside the step before (three or
    more).  Y is bit-equal to the serialised pair on every call."""
    torch_dev()
    M, H, F = 256, 768, 1536
    Xn, W1n, W2n = inputs.mlp_inputs(M, H, F, seed=12)
    X, W1, W2 = map(to_dev, (Xn, W1n, W2n))
    ref, _, _ = _run(X, W1, W2, "serial", tile_cfg=cfg)
    for delay in (1, 3):
        for seed in (0, 7):
            note("sentinel delayed cfg=%d delay=%d seed=%d" % (cfg, delay, seed))
            Y, _, _ = _run(X, W1, W2, "sentinel", tile_cfg=cfg, debug_delay=delay,
                           order_seed=seed)
            np.testing.assert_array_equal(bits(Y), bits(ref))


@pytest.mark.parametrize("cfg,splits", [(3, (2, 3)), (3, (8, 4)), (7, (4, 2)), (12, (2, 6))])
def test_split_k_parity_and_bit_equality(cfg, splits):
    """K split producer and consumer tiles with the deterministic in-order
    reduction: oracle parity, identical bits under every policy and order."""
    torch_dev()
    tc = tls.tile_configs()[cfg]
    M, H, F = (300, 768, 1536) if tc["bn1"] % 3 == 0 else (300, 512, 768)
    Xn, W1n, W2n = inputs.mlp_inputs(M, H, F, seed=11, x_sigma=1.0, w_sigma=0.05)
    G, Zr, Yr = oracle.mlp_chain(Xn, W1n, W2n)
    X, W1, W2 = map(to_dev, (Xn, W1n, W2n))
    ref = None
    for pol in POLICIES:
        for order, seed in (("xcd", 0), ("interleaved", 3)):
            note("split cfg=%d splits=%s policy=%s order=%s" % (cfg, splits, pol, order))
            Y, z, zd = _run(X, W1, W2, pol, tile_cfg=cfg, dbg=True, split_k=splits, order=order,
                            order_seed=seed, debug_delay=1)
            assert oracle.normwise_rel_err(to_np(zd), G) <= TOL_FP32_PRE
            assert oracle.normwise_rel_err(to_np(Y), Yr) <= TOL_FP16
            if ref is None:
                ref = bits(Y)
            np.testing.assert_array_equal(bits(Y), ref, err_msg="%s %s" % (pol, order))


@pytest.mark.parametrize("M", [1, 5, 33, 130])
@pytest.mark.parametrize("cfg,splits", [(7, (4, 2)), (6, (4, 2)), (17, (2, 2))])
def test_split_k_small_batches(M, cfg, splits):
    """Batches smaller than the tile through the split-K path: a partial moves
    only the chunks of rows inside the output (the others' offsets fall past
    the buffer), so every row of Z and Y must still match the oracle, with
    identical bits under every policy, for row counts that end inside a
    thread's four-row chunk, a wave's rows and a second row tile."""
    torch_dev()
    tc = tls.tile_configs()[cfg]
    H, F = (768, 1536) if tc["bn1"] % 3 == 0 else (1024, 2048)
    Xn, W1n, W2n = inputs.mlp_inputs(M, H, F, seed=M, x_sigma=1.0, w_sigma=0.05)
    G, Zr, Yr = oracle.mlp_chain(Xn, W1n, W2n)
    X, W1, W2 = map(to_dev, (Xn, W1n, W2n))
    ref = None
    for pol in POLICIES:
        note("split small batch M=%d cfg=%d splits=%s policy=%s" % (M, cfg, splits, pol))
        Y, z, zd = _run(X, W1, W2, pol, tile_cfg=cfg, dbg=True, split_k=splits)
        assert oracle.normwise_rel_err(to_np(zd), G) <= TOL_FP32_PRE, pol
        assert oracle.normwise_rel_err(to_np(z), Zr) <= TOL_FP16, pol
        assert oracle.normwise_rel_err(to_np(Y), Yr) <= TOL_FP16, pol
        if ref is None:
            ref = bits(Y)
        np.testing.assert_array_equal(bits(Y), ref, err_msg=pol)


def test_split_k_exact_small_integers():
    torch_dev()
    M, H, F = 192, 512, 768
    Xn = inputs.small_int_fp16((M, H), 6, 0)
    W1n = inputs.small_int_fp16((H, F), 6, 1)
    W2n = inputs.small_int_fp16((F, H), 6, 2)
    G, Zr, Yr = oracle.mlp_chain(Xn, W1n, W2n, act="none")
    X, W1, W2 = map(to_dev, (Xn, W1n, W2n))
    for pol in ("serial", "rowsync", "tilesync"):
        note("split exact ints policy=%s" % pol)
        Y, z, zd = _run(X, W1, W2, pol, tile_cfg=0, act="none", dbg=True, split_k=(4, 3))
        np.testing.assert_array_equal(to_np(zd), G.astype(np.float32))
        np.testing.assert_array_equal(to_np(Y).astype(np.float64), Yr.astype(np.float64))


@pytest.mark.parametrize("pol", ["tilesync", "rowsync", "sentinel"])
def test_split_k_missing_split_times_out_then_recovers(pol):
    torch = torch_dev()
    M, H, F = 128, 512, 768
    Xn, W1n, W2n = inputs.mlp_inputs(M, H, F, seed=4)
    X, W1, W2 = map(to_dev, (Xn, W1n, W2n))
    note("split watchdog policy=%s" % pol)
    with pytest.raises(tls.ChainError) as ei:
        tls.chain_mlp(X, W1, W2, policy=pol, tile_cfg=3, split_k=(4, 2), debug_skip_producer=5,
                      poll_limit=2000, check=True)
    assert ei.value.status == tls.CHAIN_ETIMEOUT
    ref = tls.chain_mlp(X, W1, W2, policy="serial", tile_cfg=3, split_k=(4, 2), check=True).clone()
    Y = tls.chain_mlp(X, W1, W2, policy=pol, tile_cfg=3, split_k=(4, 2), check=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(Y), bits(ref))


def test_split_k_argument_errors():
    torch = torch_dev()
    X, W1, W2 = map(to_dev, inputs.mlp_inputs(64, 512, 768, seed=1))
    for splits in ((3, 1), (1, 5), (32, 1)):
        with pytest.raises(tls.ChainError):
            tls.chain_mlp(X, W1, W2, tile_cfg=0, split_k=splits)


@pytest.mark.parametrize("pol", ["tilesync", "rowsync"])
@pytest.mark.parametrize("offset", [0, 16, 80])
def test_intermediate_alignment_selects_acquire(pol, offset):
    """z_out 128-byte aligned (light acquire after a poll) or not (full
    agent-scope acquire): poisoned, delayed producers, both bit-equal to the
    stream-serialised result."""
    torch = torch_dev()
    M, H, F = 256, 512, 1024
    Xn, W1n, W2n = inputs.mlp_inputs(M, H, F, seed=9)
    X, W1, W2 = map(to_dev, (Xn, W1n, W2n))
    ref, _, _ = _run(X, W1, W2, "serial", tile_cfg=3)
    flat = torch.full((M * F + 128,), -1, dtype=torch.int16, device="cuda").view(torch.float16)
    z = flat[offset // 2: offset // 2 + M * F].view(M, F)
    assert z.data_ptr() % 128 == offset % 128
    for seed in (0, 3):
        flat.view(torch.int16).fill_(-1)
        note("alignment policy=%s offset=%d seed=%d" % (pol, offset, seed))
        Y = tls.chain_mlp(X, W1, W2, policy=pol, tile_cfg=3, z_out=z, order_seed=seed,
                          debug_delay=2, check=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(Y), bits(ref))


@pytest.mark.parametrize("pol", ["tilesync", "rowsync"])
@pytest.mark.parametrize("where", ["z_out", "workspace"])
def test_alternating_inputs_reuse_one_intermediate(pol, where):
    """Two different inputs in turn through one workspace and one 128-byte
    aligned intermediate (the light acquire): a consumer that read a line of
    the previous call's Z still held in some cache would mix the two chains.
    Every Y must equal the oracle's and, bit for bit, the serial result of
    its own input computed in a fresh workspace."""
    torch = torch_dev()
    M, H, F = 512, 1024, 2048
    data, refs, oref = [], [], []
    for seed in (21, 22):
        Xn, W1n, W2n = inputs.mlp_inputs(M, H, F, seed=seed)
        oref.append(oracle.mlp_chain(Xn, W1n, W2n)[2])
        d = tuple(map(to_dev, (Xn, W1n, W2n)))
        data.append(d)
        ws0 = torch.zeros(tls.chain_mlp_workspace_bytes(M, H, F, policy="serial", tile_cfg=3),
                          dtype=torch.uint8, device="cuda")
        refs.append(tls.chain_mlp(*d, policy="serial", tile_cfg=3, workspace=ws0,
                                  check=True).clone())
    ws = torch.zeros(tls.chain_mlp_workspace_bytes(M, H, F, policy=pol, tile_cfg=3),
                     dtype=torch.uint8, device="cuda")
    z = torch.empty((M, F), dtype=torch.float16, device="cuda") if where == "z_out" else None
    assert z is None or z.data_ptr() % 128 == 0
    for it in range(6):
        i = it % 2
        note("alternating inputs policy=%s where=%s call=%d" % (pol, where, it))
        Y = tls.chain_mlp(*data[i], policy=pol, tile_cfg=3, workspace=ws, z_out=z,
                          debug_delay=1 if it >= 4 else 0, check=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(Y), bits(refs[i]), err_msg="call %d" % it)
        assert oracle.normwise_rel_err(to_np(Y), oref[i]) <= TOL_FP16


def test_flags_never_alias_other_regions_of_a_shared_workspace():
    """A caller workspace used first by a shape with few tiles and a large
    intermediate (filled with positive values that would read as reached
    epochs), then by a shape with many more tiles: the flags live in their own
    fixed region, so delayed producers are still waited for."""
    torch = torch_dev()
    XA, W1A, W2A = map(to_dev, inputs.mlp_inputs(2048, 256, 4096, seed=12, x_sigma=4.0,
                                                 w_sigma=0.5))
    XB, W1B, W2B = map(to_dev, inputs.mlp_inputs(128, 512, 4096, seed=13))
    need = max(tls.chain_mlp_workspace_bytes(2048, 256, 4096, policy="serial", tile_cfg=1),
               tls.chain_mlp_workspace_bytes(128, 512, 4096, policy="tilesync", tile_cfg=0))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    tls.chain_workspace_reset(ws)
    ref = tls.chain_mlp(XB, W1B, W2B, policy="serial", tile_cfg=0, workspace=ws, split_k=(1, 1),
                        check=True).clone()
    for rep in range(2):
        note("workspace regions rep=%d" % rep)
        tls.chain_mlp(XA, W1A, W2A, policy="serial", tile_cfg=1, workspace=ws, check=True)
        Y = tls.chain_mlp(XB, W1B, W2B, policy="tilesync", tile_cfg=0, workspace=ws,
                          debug_delay=3, split_k=(1, 1), check=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(Y), bits(ref))


@pytest.mark.parametrize("pol", ["tilesync", "rowsync", "sentinel"])
def test_watchdog_reports_timeout_then_recovers(pol):
    """A producer tile that never posts (host knob) makes its consumers'
    bounded waits expire: the call reports CHAIN_ETIMEOUT instead of hanging,
    and the next call works."""
    torch = torch_dev()
    Xn, W1n, W2n = inputs.tiny_mlp_inputs(seed=0)
    X, W1, W2 = map(to_dev, (Xn, W1n, W2n))
    note("watchdog policy=%s" % pol)
    with pytest.raises(tls.ChainError) as ei:
        tls.chain_mlp(X, W1, W2, policy=pol, tile_cfg=0, debug_skip_producer=3,
                      poll_limit=2000, check=True)
    assert ei.value.status == tls.CHAIN_ETIMEOUT
    item, kind = tls.chain_last_timeout()
    assert kind == 1
    note("watchdog recovery policy=%s" % pol)
    ref = tls.chain_mlp(X, W1, W2, policy="serial", tile_cfg=0, check=True).clone()
    Y = tls.chain_mlp(X, W1, W2, policy=pol, tile_cfg=0, check=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(Y), bits(ref))


def test_argument_errors():
    torch = torch_dev()
    X = torch.zeros((64, 256), dtype=torch.float16, device="cuda")
    W1 = torch.zeros((256, 1024), dtype=torch.float16, device="cuda")
    W2 = torch.zeros((1024, 256), dtype=torch.float16, device="cuda")
    with pytest.raises(tls.ChainError) as ei:
        tls.chain_mlp(X, W1, W2, policy="conv2d_tilesync")
    assert ei.value.status == tls.CHAIN_EUNSUPPORTED
    Xb = torch.zeros((64, 200), dtype=torch.float16, device="cuda")
    W1b = torch.zeros((200, 1024), dtype=torch.float16, device="cuda")
    W2b = torch.zeros((1024, 200), dtype=torch.float16, device="cuda")
    with pytest.raises(tls.ChainError) as ei:
        tls.chain_mlp(Xb, W1b, W2b)
    assert ei.value.status == tls.CHAIN_EUNSUPPORTED


@pytest.mark.parametrize("M", inputs.GPT3_MS)
def test_gpt3_slice_sampled_rows(M):
    """GPT-3 MLP slice at full size: every policy bit-identical; sampled rows
    (including the first and last of every row tile) against the oracle."""
    torch = torch_dev()
    H, F = inputs.GPT3_H, inputs.GPT3_F
    W1n, W2n = inputs.mlp_weights(H, F, seed=0)
    Xn = inputs.mlp_x(M, H, seed=0)
    X, W1, W2 = map(to_dev, (Xn, W1n, W2n))
    plan = tls.chain_mlp_plan(M, H, F)
    bm = tls.tile_configs()[plan["tile_cfg"]]["bm"]
    rows = sorted({0, M - 1} | {r for t in range(0, M, bm) for r in (t, min(t + bm - 1, M - 1))}
                  | set(np.random.default_rng(M).integers(0, M, 8).tolist()))
    G, Zr, Yr = oracle.mlp_chain_rows(Xn, W1n, W2n, rows)
    ref = None
    for pol in POLICIES:
        note("gpt3 M=%d policy=%s" % (M, pol))
        zd = torch.empty((M, F), dtype=torch.float32, device="cuda") if pol == "tilesync" else None
        Y = tls.chain_mlp(X, W1, W2, policy=pol, z_debug=zd, check=True)
        torch.cuda.synchronize()
        Yh = to_np(Y)
        assert oracle.normwise_rel_err(Yh[rows], Yr) <= TOL_FP16, pol
        if zd is not None:
            assert oracle.normwise_rel_err(to_np(zd)[rows], G) <= TOL_FP32_PRE
        if ref is None:
            ref = Yh.view(np.uint16).copy()
        np.testing.assert_array_equal(Yh.view(np.uint16), ref, err_msg=pol)


@pytest.mark.parametrize("slots", [2, 3])
def test_sentinel_ring_matches_flag_policy(slots):
    """Sentinel buffer rotation: five calls through a ring, each with its own
    X and a ragged M.  Every Y and every intermediate is bit-equal to the
    TileSync call's, and after call i the slot call i + 1 consumes holds the
    sentinel everywhere (it was refilled inside call i)."""
    torch = torch_dev()
    M, H, F = 200, 512, 1024
    _, W1n, W2n = inputs.mlp_inputs(M, H, F, seed=3)
    W1, W2 = to_dev(W1n), to_dev(W2n)
    ring = tls.SentinelRing(M, F, slots=slots)
    ring.buf.fill_(0)  # nothing of it is the sentinel before the first call
    for i in range(5):
        note("sentinel ring slots=%d call %d" % (slots, i))
        X = to_dev(inputs.mlp_x(M, H, seed=10 + i))
        ref, zref, _ = _run(X, W1, W2, "tilesync", tile_cfg=1)
        Y = tls.chain_mlp(X, W1, W2, policy="sentinel", tile_cfg=1, ring=ring, check=True)
        torch.cuda.synchronize()
        assert ring.index == i + 1
        np.testing.assert_array_equal(bits(Y), bits(ref))
        np.testing.assert_array_equal(bits(ring.slot(i)), bits(zref))
        nxt = bits(ring.slot(i + 1))
        assert (nxt == 0xFFFF).all(), "slot of call %d not refilled" % (i + 1)


def test_sentinel_ring_timeout_still_refills_next_slot():
    """A call whose producer tile never stores times out, yet the slot of the
    next call is refilled in full, so the next call is correct."""
    torch = torch_dev()
    M, H, F = 128, 512, 768
    X, W1, W2 = map(to_dev, inputs.mlp_inputs(M, H, F, seed=4))
    ref, _, _ = _run(X, W1, W2, "serial", tile_cfg=3)
    ring = tls.SentinelRing(M, F, slots=2)
    Y = tls.chain_mlp(X, W1, W2, policy="sentinel", tile_cfg=3, ring=ring, check=True)
    np.testing.assert_array_equal(bits(Y), bits(ref))
    note("sentinel ring watchdog")
    with pytest.raises(tls.ChainError) as ei:
        tls.chain_mlp(X, W1, W2, policy="sentinel", tile_cfg=3, ring=ring, debug_skip_producer=2,
                      poll_limit=2000, check=True)
    assert ei.value.status == tls.CHAIN_ETIMEOUT
    assert ring.index == 2
    assert (bits(ring.slot(2)) == 0xFFFF).all()
    Y = tls.chain_mlp(X, W1, W2, policy="sentinel", tile_cfg=3, ring=ring, check=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(Y), bits(ref))


def test_sentinel_ring_shape_mismatch():
    torch_dev()
    X, W1, W2 = map(to_dev, inputs.mlp_inputs(64, 256, 1024, seed=1))
    ring = tls.SentinelRing(64, 512, slots=2)
    with pytest.raises(ValueError):
        tls.chain_mlp(X, W1, W2, policy="sentinel", ring=ring)
    assert ring.index == 0


@pytest.mark.parametrize("pol", ["serial", "tilesync", "rowsync"])
def test_trace_records_every_item_once(pol):
    """The optional trace: one record per work item, at its index; times
    ordered within a record; a workgroup's items do not overlap and its
    producer items come before its consumer items; Y unchanged by tracing."""
    torch = torch_dev()
    from tile_level_sync_amd import trace
    M, H, F = 384, 1024, 2048
    X, W1, W2 = map(to_dev, inputs.mlp_inputs(M, H, F, seed=9))
    plan = tls.chain_mlp_plan(M, H, F)
    P = plan["producer_tiles"] * plan["split_k1"]
    n = tls.mlp_work_items(M, H, F)
    ref, _, _ = _run(X, W1, W2, pol)
    buf = tls.trace_buffer(n + 3)
    note("trace policy=%s items=%d" % (pol, n))
    Y = tls.chain_mlp(X, W1, W2, policy=pol, trace=buf, check=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(Y), bits(ref))
    r = trace.decode(buf)
    assert len(r) == n
    np.testing.assert_array_equal(r["item"], np.arange(n))
    assert (r["t_start"] <= r["t_ready"]).all() and (r["t_ready"] <= r["t_end"]).all()
    assert (r["t_ready"][:P] == r["t_start"][:P]).all()
    for wg in np.unique(r["wg"]):
        w = np.sort(r[r["wg"] == wg], order="t_start")
        assert (w["t_start"][1:] >= w["t_end"][:-1]).all(), wg
        kinds = (w["item"] >= P).astype(int)
        assert (np.diff(kinds) >= 0).all(), wg  # producers first
    s = trace.summarize(r, P, tls.trace_clock_khz(),
                        n_cu=torch.cuda.get_device_properties(0).multi_processor_count)
    assert 0.0 < s["busy_frac"] <= 1.0 and 0.0 <= s["tail_idle_frac"] < 1.0
    if pol == "serial":
        assert s["producer_consumer_gap_us"] >= 0.0


def test_trace_capacity_too_small():
    torch_dev()
    X, W1, W2 = map(to_dev, inputs.mlp_inputs(128, 512, 768, seed=1))
    n = tls.mlp_work_items(128, 512, 768)
    with pytest.raises(tls.ChainError):
        tls.chain_mlp(X, W1, W2, trace=tls.trace_buffer(n - 1))


def _bf16_dev(bits):
    torch = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(
        torch.bfloat16)


def _bits16(t):
    torch = torch_dev()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("M,H,F,cfg", [(64, 256, 1024, None), (300, 512, 768, None),
                                       (200, 1024, 2048, 1), (300, 768, 1536, 17)])
def test_bf16_all_policies(M, H, F, cfg):
    """bf16 storage, fp32 accumulation: the fp32 activation within 1e-3 of the
    oracle, the bf16 intermediate and output within 2e-2 (two bf16 ulps are
    2^-6 = 1.6e-2), Y and Z bit-identical under every policy."""
    torch = torch_dev()
    Xb, W1b, W2b = inputs.mlp_inputs_bf16(M, H, F, seed=11, x_sigma=1.0, w_sigma=0.05)
    G, Zb, Yb = oracle.mlp_chain_bf16(Xb, W1b, W2b)
    X, W1, W2 = map(_bf16_dev, (Xb, W1b, W2b))
    ref = None
    for pol in POLICIES:
        note("bf16 M=%d H=%d F=%d cfg=%s policy=%s" % (M, H, F, cfg, pol))
        z = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
        zd = torch.empty((M, F), dtype=torch.float32, device="cuda")
        Y = tls.chain_mlp(X, W1, W2, policy=pol, z_out=z, z_debug=zd, tile_cfg=cfg, check=True)
        torch.cuda.synchronize()
        assert Y.dtype == torch.bfloat16
        assert oracle.normwise_rel_err(to_np(zd), G) <= TOL_FP32_PRE, pol
        assert oracle.normwise_rel_err(oracle.bf16_values(_bits16(z)),
                                       oracle.bf16_values(Zb)) <= TOL_FP16, pol
        assert oracle.normwise_rel_err(oracle.bf16_values(_bits16(Y)),
                                       oracle.bf16_values(Yb)) <= TOL_FP16, pol
        if ref is None:
            ref = (_bits16(Y), _bits16(z))
        np.testing.assert_array_equal(_bits16(Y), ref[0], err_msg=pol)
        np.testing.assert_array_equal(_bits16(z), ref[1], err_msg=pol)


def test_bf16_gpt3_slice_sampled_rows():
    torch = torch_dev()
    M, H, F = 256, 12288, 6144
    Xb, W1b, W2b = inputs.mlp_inputs_bf16(M, H, F, seed=12)
    X, W1, W2 = map(_bf16_dev, (Xb, W1b, W2b))
    rows = np.array([0, 1, 77, 128, 255])
    _, _, Yr = oracle.mlp_chain_bf16(Xb[rows], W1b, W2b)
    outs = {}
    for pol in ("serial", "tilesync", "rowsync"):
        note("bf16 gpt3 M=256 policy=%s" % pol)
        Y = tls.chain_mlp(X, W1, W2, policy=pol, check=True)
        torch.cuda.synchronize()
        outs[pol] = _bits16(Y)
        assert oracle.normwise_rel_err(oracle.bf16_values(outs[pol][rows]),
                                       oracle.bf16_values(Yr)) <= TOL_FP16, pol
    for pol in outs:
        np.testing.assert_array_equal(outs[pol], outs["serial"], err_msg=pol)


def test_bf16_sentinel_ring():
    torch = torch_dev()
    M, H, F = 128, 512, 1024
    Xb, W1b, W2b = inputs.mlp_inputs_bf16(M, H, F, seed=13, w_sigma=0.05)
    X, W1, W2 = map(_bf16_dev, (Xb, W1b, W2b))
    ref = _bits16(tls.chain_mlp(X, W1, W2, policy="tilesync", check=True))
    ring = tls.SentinelRing(M, F, slots=2)
    for i in range(3):
        note("bf16 sentinel ring call %d" % i)
        Y = tls.chain_mlp(X, W1, W2, policy="sentinel", ring=ring, check=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_bits16(Y), ref)


def test_bf16_unsupported_tile_config():
    torch_dev()
    X, W1, W2 = map(_bf16_dev, inputs.mlp_inputs_bf16(256, 512, 768, seed=1))
    with pytest.raises(tls.ChainError) as ei:
        tls.chain_mlp(X, W1, W2, tile_cfg=2)  # 256x128, 4 waves: no bf16 instance
    assert ei.value.status == tls.CHAIN_EUNSUPPORTED

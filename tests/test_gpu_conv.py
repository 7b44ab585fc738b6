"""Conv-pair chain on the GPU through the C ABI: parity with the oracle,
closed forms (delta and shifted-delta filters), exactness, bit-equality
across policies and tile orders, watchdog."""

import numpy as np
import pytest

import oracle
import tile_level_sync_amd as tls
from tile_level_sync_amd import inputs
from tests.gpu_util import TOL_FP16, TOL_FP32_PRE, bits, note, to_dev, to_np, torch_dev

pytestmark = pytest.mark.gpu

POLICIES = ["serial", "conv2d_tilesync", "rowsync", "sentinel"]


def _run(X, Wa, Wb, policy, dbg=False, **kw):
    torch = torch_dev()
    N, Hh, Ww, _ = X.shape
    K = Wa.shape[3]
    z = torch.empty((N, Hh, Ww, K), dtype=torch.float16, device="cuda")
    zd = torch.empty((N, Hh, Ww, K), dtype=torch.float32, device="cuda") if dbg else None
    Y = tls.chain_conv(X, Wa, Wb, policy=policy, z_out=z, z_debug=zd, check=True, **kw)
    torch.cuda.synchronize()
    return Y, z, zd


@pytest.mark.parametrize("cfg", list(range(11)))
def test_small_pair_all_policies(cfg):
    torch_dev()
    C = K = 128 if cfg in (2, 7) else 64
    Xn, Wan, Wbn = inputs.conv_inputs(2, 11, 9, C, K, seed=3)  # 198 pixels: ragged tiles
    G, Zr, Yr = oracle.conv_chain(Xn, Wan, Wbn)
    X, Wa, Wb = map(to_dev, (Xn, Wan, Wbn))
    ref = None
    for pol in POLICIES:
        note("conv small cfg=%d policy=%s" % (cfg, pol))
        Y, z, zd = _run(X, Wa, Wb, pol, dbg=True, tile_cfg=cfg)
        assert oracle.normwise_rel_err(to_np(zd), G) <= TOL_FP32_PRE, pol
        assert oracle.normwise_rel_err(to_np(z), Zr) <= TOL_FP16, pol
        assert oracle.normwise_rel_err(to_np(Y), Yr) <= TOL_FP16, pol
        if ref is None:
            ref = bits(Y)
        np.testing.assert_array_equal(bits(Y), ref, err_msg=pol)


def test_channel_change_pair():
    torch_dev()
    Xn, Wan, Wbn = inputs.conv_inputs(1, 10, 12, 64, 128, seed=4)
    G, Zr, Yr = oracle.conv_chain(Xn, Wan, Wbn)
    X, Wa, Wb = map(to_dev, (Xn, Wan, Wbn))
    for pol in ("serial", "conv2d_tilesync"):
        note("conv 64->128 policy=%s" % pol)
        Y, z, zd = _run(X, Wa, Wb, pol, dbg=True)
        assert oracle.normwise_rel_err(to_np(Y), Yr) <= TOL_FP16


def test_delta_filters_give_relu_exactly():
    torch_dev()
    C = 64
    Xn = inputs.normal_fp16((2, 7, 8, C), 1.0, 5, 0)
    D = np.zeros((3, 3, C, C), np.float16)
    D[1, 1] = np.eye(C, dtype=np.float16)
    X, Dd = to_dev(Xn), to_dev(D)
    note("conv delta filters")
    Y, z, _ = _run(X, Dd, Dd, "conv2d_tilesync")
    relu = np.where(Xn < 0, np.float16(0), Xn).astype(np.float64)
    np.testing.assert_array_equal(to_np(z).astype(np.float64), relu)
    np.testing.assert_array_equal(to_np(Y).astype(np.float64), relu)


@pytest.mark.parametrize("r,s", [(0, 0), (2, 2), (0, 2), (2, 1)])
def test_shifted_delta_pins_halo_and_padding(r, s):
    torch_dev()
    C = 64
    Xn = np.abs(inputs.normal_fp16((2, 9, 7, C), 1.0, 6, 0))  # nonnegative: ReLU is the identity
    D = np.zeros((3, 3, C, C), np.float16)
    D[r, s] = np.eye(C, dtype=np.float16)
    I = np.zeros((3, 3, C, C), np.float16)
    I[1, 1] = np.eye(C, dtype=np.float16)
    X, Dd, Id = to_dev(Xn), to_dev(D), to_dev(I)
    note("conv shifted delta r=%d s=%d" % (r, s))
    Y, _, _ = _run(X, Dd, Id, "rowsync", tile_cfg=0)
    exp = oracle.conv2d_nhwc(Xn, D)
    np.testing.assert_array_equal(to_np(Y).astype(np.float64), exp)


def test_exact_small_integers():
    torch_dev()
    Xn = inputs.small_int_fp16((1, 8, 9, 64), 7, 0)
    Wan = inputs.small_int_fp16((3, 3, 64, 64), 7, 1)
    Wbn = inputs.small_int_fp16((3, 3, 64, 64), 7, 2)
    G, Zr, Yr = oracle.conv_chain(Xn, Wan, Wbn)
    X, Wa, Wb = map(to_dev, (Xn, Wan, Wbn))
    for pol in ("serial", "conv2d_tilesync", "sentinel"):
        note("conv exact ints policy=%s" % pol)
        Y, z, zd = _run(X, Wa, Wb, pol, dbg=True)
        np.testing.assert_array_equal(to_np(zd), G.astype(np.float32))
        np.testing.assert_array_equal(to_np(z).astype(np.float64), Zr.astype(np.float64))
        np.testing.assert_array_equal(to_np(Y).astype(np.float64), Yr.astype(np.float64))


@pytest.mark.parametrize("seed", [1, 2])
@pytest.mark.parametrize("ch,cfg", [(64, None), (128, 0)])
def test_orders_bit_identical(seed, ch, cfg):
    """Every order and seed gives the serial bits; at 128 channels with
    128 x 64 tiles there are two channel tiles, so column-major and strided
    differ from row-major."""
    torch_dev()
    Xn, Wan, Wbn = inputs.conv_inputs(2, 16, 16, ch, ch, seed=8)
    X, Wa, Wb = map(to_dev, (Xn, Wan, Wbn))
    ref, _, _ = _run(X, Wa, Wb, "serial", tile_cfg=cfg)
    for pol in ("serial", "conv2d_tilesync", "rowsync", "sentinel"):
        for order in ("xcd", "row_major", "interleaved", "col_major", "strided"):
            note("conv order ch=%d seed=%d policy=%s order=%s" % (ch, seed, pol, order))
            Y, _, _ = _run(X, Wa, Wb, pol, order=order, order_seed=seed, debug_delay=1,
                           tile_cfg=cfg)
            np.testing.assert_array_equal(bits(Y), bits(ref))


@pytest.mark.parametrize("grid", [1, 3])
def test_interleaved_order_with_halo_longer_than_a_tile(grid):
    """64 x 64 images with 64-pixel tiles: the 3x3 halo (65 flattened pixels)
    reaches two producer tiles ahead.  With one or three workgroups walking
    the interleaved order, a consumer handed out before a producer it reads
    would wait forever (here: CHAIN_ETIMEOUT); the order lists it after them."""
    torch_dev()
    Xn, Wan, Wbn = inputs.conv_inputs(2, 64, 64, 64, 64, seed=12)
    assert tls.chain_conv_plan(2, 64, 64, 64, 64)["tile_cfg"] == 3
    X, Wa, Wb = map(to_dev, (Xn, Wan, Wbn))
    ref, _, _ = _run(X, Wa, Wb, "serial")
    for pol in ("conv2d_tilesync", "rowsync", "sentinel"):
        note("conv interleaved grid=%d policy=%s" % (grid, pol))
        Y, _, _ = _run(X, Wa, Wb, pol, order="interleaved", grid=grid, poll_limit=200000)
        np.testing.assert_array_equal(bits(Y), bits(ref))


@pytest.mark.parametrize("pol", ["conv2d_tilesync", "rowsync", "sentinel"])
def test_watchdog(pol):
    torch = torch_dev()
    Xn, Wan, Wbn = inputs.conv_inputs(1, 8, 8, 64, 64, seed=2)
    X, Wa, Wb = map(to_dev, (Xn, Wan, Wbn))
    note("conv watchdog policy=%s" % pol)
    with pytest.raises(tls.ChainError) as ei:
        tls.chain_conv(X, Wa, Wb, policy=pol, debug_skip_producer=0, poll_limit=2000, check=True)
    assert ei.value.status == tls.CHAIN_ETIMEOUT
    ref = tls.chain_conv(X, Wa, Wb, policy="serial", check=True).clone()
    Y = tls.chain_conv(X, Wa, Wb, policy=pol, check=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(Y), bits(ref))


def test_resnet_layer_full_size():
    """Batch 32, 56x56, 64 -> 64 -> 64 channels: whole output against the oracle."""
    torch_dev()
    Xn, Wan, Wbn = inputs.resnet_pair_inputs(batch=32, seed=0)
    G, Zr, Yr = oracle.conv_chain(Xn, Wan, Wbn)
    X, Wa, Wb = map(to_dev, (Xn, Wan, Wbn))
    ref = None
    for pol in POLICIES:
        note("resnet 32x56x56x64 policy=%s" % pol)
        Y, z, zd = _run(X, Wa, Wb, pol, dbg=(pol == "conv2d_tilesync"))
        assert oracle.normwise_rel_err(to_np(Y), Yr) <= TOL_FP16, pol
        if zd is not None:
            assert oracle.normwise_rel_err(to_np(zd), G) <= TOL_FP32_PRE
        if ref is None:
            ref = bits(Y)
        np.testing.assert_array_equal(bits(Y), ref, err_msg=pol)


@pytest.mark.parametrize("batch", [1, 8, 32])
@pytest.mark.parametrize("side,channels", inputs.RESNET38_PAIRS[1:])
def test_resnet38_pairs(side, channels, batch):
    """The deeper ResNet-38 layer pairs (28x28x128, 14x14x256, 7x7x512) at
    batch 1, 8 and 32: the whole output against the oracle, identical bits
    under every policy."""
    torch_dev()
    Xn, Wan, Wbn = inputs.resnet_pair_inputs(batch, seed=2, side=side, channels=channels)
    G, Zr, Yr = oracle.conv_chain(Xn, Wan, Wbn)
    X, Wa, Wb = map(to_dev, (Xn, Wan, Wbn))
    ref = None
    for pol in POLICIES:
        note("resnet38 %dx%dx%d batch=%d policy=%s" % (side, side, channels, batch, pol))
        Y, z, zd = _run(X, Wa, Wb, pol, dbg=(pol == "rowsync"))
        assert oracle.normwise_rel_err(to_np(Y), Yr) <= TOL_FP16, pol
        if zd is not None:
            assert oracle.normwise_rel_err(to_np(zd), G) <= TOL_FP32_PRE
        if ref is None:
            ref = bits(Y)
        np.testing.assert_array_equal(bits(Y), ref, err_msg=pol)


@pytest.mark.parametrize("pol", ["conv2d_tilesync", "rowsync"])
def test_alternating_inputs_reuse_one_intermediate(pol):
    """Two different images in turn through one workspace and one aligned
    intermediate (light acquire): each Y bit-equal to its own serial result
    and within tolerance of the oracle."""
    torch = torch_dev()
    data, refs, oref = [], [], []
    for seed in (31, 32):
        Xn, Wan, Wbn = inputs.conv_inputs(4, 28, 28, 64, 64, seed=seed)
        oref.append(oracle.conv_chain(Xn, Wan, Wbn)[2])
        d = tuple(map(to_dev, (Xn, Wan, Wbn)))
        data.append(d)
        ws0 = torch.zeros(tls.chain_conv_workspace_bytes(4, 28, 28, 64, 64, policy="serial"),
                          dtype=torch.uint8, device="cuda")
        refs.append(tls.chain_conv(*d, policy="serial", workspace=ws0, check=True).clone())
    ws = torch.zeros(tls.chain_conv_workspace_bytes(4, 28, 28, 64, 64, policy=pol),
                     dtype=torch.uint8, device="cuda")
    z = torch.empty((4, 28, 28, 64), dtype=torch.float16, device="cuda")
    assert z.data_ptr() % 128 == 0
    for it in range(6):
        i = it % 2
        note("conv alternating inputs policy=%s call=%d" % (pol, it))
        Y = tls.chain_conv(*data[i], policy=pol, workspace=ws, z_out=z,
                           debug_delay=1 if it >= 4 else 0, check=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(Y), bits(refs[i]), err_msg="call %d" % it)
        assert oracle.normwise_rel_err(to_np(Y), oref[i]) <= TOL_FP16


@pytest.mark.parametrize("cfg,splits,ch", [(0, (3, 3), 64), (3, (9, 1), 64), (2, (2, 6), 128),
                                           (3, (1, 3), 128)])
def test_split_k_parity_and_bit_equality(cfg, splits, ch):
    """K split over taps x channel blocks with the in-order reduction: oracle
    parity and identical bits under every policy and tile order."""
    torch_dev()
    Xn, Wan, Wbn = inputs.conv_inputs(2, 11, 9, ch, ch, seed=5)
    G, Zr, Yr = oracle.conv_chain(Xn, Wan, Wbn)
    X, Wa, Wb = map(to_dev, (Xn, Wan, Wbn))
    ref = None
    for pol in POLICIES:
        for order, seed in (("xcd", 0), ("interleaved", 2)):
            note("conv split cfg=%d splits=%s policy=%s order=%s" % (cfg, splits, pol, order))
            Y, z, zd = _run(X, Wa, Wb, pol, dbg=True, tile_cfg=cfg, split_k=splits, order=order,
                            order_seed=seed, debug_delay=1)
            assert oracle.normwise_rel_err(to_np(zd), G) <= TOL_FP32_PRE, pol
            assert oracle.normwise_rel_err(to_np(Y), Yr) <= TOL_FP16, pol
            if ref is None:
                ref = bits(Y)
            np.testing.assert_array_equal(bits(Y), ref, err_msg="%s %s" % (pol, order))


@pytest.mark.parametrize("pol", ["conv2d_tilesync", "rowsync", "sentinel"])
def test_split_k_missing_split_times_out(pol):
    torch = torch_dev()
    Xn, Wan, Wbn = inputs.conv_inputs(1, 8, 8, 64, 64, seed=2)
    X, Wa, Wb = map(to_dev, (Xn, Wan, Wbn))
    note("conv split watchdog policy=%s" % pol)
    with pytest.raises(tls.ChainError) as ei:
        tls.chain_conv(X, Wa, Wb, policy=pol, tile_cfg=3, split_k=(3, 3), debug_skip_producer=1,
                       poll_limit=2000, check=True)
    assert ei.value.status == tls.CHAIN_ETIMEOUT
    ref = tls.chain_conv(X, Wa, Wb, policy="serial", tile_cfg=3, split_k=(3, 3), check=True).clone()
    Y = tls.chain_conv(X, Wa, Wb, policy=pol, tile_cfg=3, split_k=(3, 3), check=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(Y), bits(ref))


def test_sentinel_ring_matches_flag_policy():
    """Sentinel buffer rotation on the conv pair: four calls through a ring of
    three slots, each with its own X (ragged pixel tiles).  Y and the
    intermediate are bit-equal to Conv2DTileSync's, and the slot of the next
    call holds the sentinel everywhere once a call has ended."""
    torch = torch_dev()
    N, Hh, Ww, C = 2, 11, 9, 64
    _, Wan, Wbn = inputs.conv_inputs(N, Hh, Ww, C, C, seed=3)
    Wa, Wb = to_dev(Wan), to_dev(Wbn)
    ring = tls.SentinelRing(N * Hh * Ww, C, slots=3)
    ring.buf.fill_(0)
    for i in range(4):
        note("conv sentinel ring call %d" % i)
        X = to_dev(inputs.conv_inputs(N, Hh, Ww, C, C, seed=20 + i)[0])
        ref, zref, _ = _run(X, Wa, Wb, "conv2d_tilesync", tile_cfg=0)
        Y = tls.chain_conv(X, Wa, Wb, policy="sentinel", tile_cfg=0, ring=ring, check=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(Y), bits(ref))
        np.testing.assert_array_equal(bits(ring.slot(i)).reshape(-1), bits(zref).reshape(-1))
        assert (bits(ring.slot(i + 1)) == 0xFFFF).all()


@pytest.mark.parametrize("pol", ["serial", "conv2d_tilesync", "rowsync"])
def test_trace_records_every_item_once(pol):
    """The optional per-item trace of the conv pair: one record per work item
    at its index, times ordered within a record, a workgroup's items disjoint
    in time with its producer items first; Y unchanged by tracing."""
    torch = torch_dev()
    from tile_level_sync_amd import trace
    N, Hh, Ww, C = 2, 28, 28, 128
    X, Wa, Wb = map(to_dev, inputs.conv_inputs(N, Hh, Ww, C, C, seed=14))
    plan = tls.chain_conv_plan(N, Hh, Ww, C, C)
    P = plan["producer_tiles"] * plan["split_k1"]
    n = tls.conv_work_items(N, Hh, Ww, C, C)
    ref, _, _ = _run(X, Wa, Wb, pol)
    buf = tls.trace_buffer(n + 3)
    note("conv trace policy=%s items=%d" % (pol, n))
    Y = tls.chain_conv(X, Wa, Wb, policy=pol, trace=buf, check=True)
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
        assert (np.diff((w["item"] >= P).astype(int)) >= 0).all(), wg
    s = trace.summarize(r, P, tls.trace_clock_khz(),
                        n_cu=torch.cuda.get_device_properties(0).multi_processor_count)
    assert 0.0 < s["busy_frac"] <= 1.0 and 0.0 <= s["tail_idle_frac"] < 1.0
    if pol == "serial":
        assert s["producer_consumer_gap_us"] >= 0.0


def test_trace_capacity_too_small():
    torch_dev()
    X, Wa, Wb = map(to_dev, inputs.conv_inputs(1, 8, 8, 64, 64, seed=1))
    n = tls.conv_work_items(1, 8, 8, 64, 64)
    with pytest.raises(tls.ChainError):
        tls.chain_conv(X, Wa, Wb, trace=tls.trace_buffer(n - 1))


def _bf16_dev(bits16):
    torch = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(bits16).view(np.int16)).to("cuda").view(
        torch.bfloat16)


def _bits16(t):
    torch = torch_dev()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("N,Hh,Ww,C,cfg", [(2, 11, 9, 64, None), (2, 11, 9, 64, 3),
                                           (1, 14, 14, 128, None), (32, 56, 56, 64, None),
                                           (2, 11, 9, 128, 0), (32, 28, 28, 128, None)])
def test_bf16_pair_all_policies(N, Hh, Ww, C, cfg):
    """bf16 storage, fp32 accumulation: the fp32 ReLU output within 1e-3 of
    the oracle, the bf16 intermediate and output within 2e-2, every policy
    bit-equal (whole outputs, ragged tiles in the first cases)."""
    torch = torch_dev()
    Xb, Wab, Wbb = inputs.conv_inputs_bf16(N, Hh, Ww, C, C, seed=13, w_sigma=0.05)
    G, Zb, Yb = oracle.conv_chain_bf16(Xb, Wab, Wbb)
    X, Wa, Wb = map(_bf16_dev, (Xb, Wab, Wbb))
    ref = None
    for pol in POLICIES:
        note("conv bf16 %dx%dx%dx%d cfg=%s policy=%s" % (N, Hh, Ww, C, cfg, pol))
        z = torch.empty((N, Hh, Ww, C), dtype=torch.bfloat16, device="cuda")
        zd = torch.empty((N, Hh, Ww, C), dtype=torch.float32, device="cuda")
        Y = tls.chain_conv(X, Wa, Wb, policy=pol, tile_cfg=cfg, z_out=z, z_debug=zd, check=True)
        torch.cuda.synchronize()
        assert Y.dtype == torch.bfloat16
        assert oracle.normwise_rel_err(to_np(zd), G) <= TOL_FP32_PRE, pol
        assert oracle.normwise_rel_err(oracle.bf16_values(_bits16(z)),
                                       oracle.bf16_values(Zb)) <= TOL_FP16, pol
        assert oracle.normwise_rel_err(oracle.bf16_values(_bits16(Y)),
                                       oracle.bf16_values(Yb)) <= TOL_FP16, pol
        if ref is None:
            ref = _bits16(Y)
        np.testing.assert_array_equal(_bits16(Y), ref, err_msg=pol)


def test_bf16_rejected_where_no_instance_exists():
    torch_dev()
    Xb, Wab, Wbb = inputs.conv_inputs_bf16(1, 8, 8, 64, 64, seed=1)
    X, Wa, Wb = map(_bf16_dev, (Xb, Wab, Wbb))
    with pytest.raises(tls.ChainError) as ei:
        tls.chain_conv(X, Wa, Wb, tile_cfg=1)  # 256 x 64, three stages: fp16 only
    assert ei.value.status == tls.CHAIN_EUNSUPPORTED


@pytest.mark.parametrize("pol", POLICIES)
def test_first_items_left_to_the_sweep(pol):
    """With the default order a launch's first producer items come from eight
    per-XCD counters.  The test knob makes every odd workgroup take none, so
    their share stays in those counters until the workgroup that draws the
    first consumer value (under serial: the producer launch's end) runs it
    before its own item.  Y bit-equal to the call without the knob, every
    item traced exactly once, a workgroup's producer items before its
    consumer items."""
    torch = torch_dev()
    from tile_level_sync_amd import trace
    N, Hh, Ww, C = 4, 28, 28, 64
    X, Wa, Wb = map(to_dev, inputs.conv_inputs(N, Hh, Ww, C, C, seed=17, w_sigma=0.05))
    plan = tls.chain_conv_plan(N, Hh, Ww, C, C)
    P = plan["producer_tiles"] * plan["split_k1"]
    n = tls.conv_work_items(N, Hh, Ww, C, C)
    note("conv first items policy=%s reference" % pol)
    ref, _, _ = _run(X, Wa, Wb, pol)
    for rep in range(2):
        note("conv first items left to the sweep policy=%s call %d" % (pol, rep))
        buf = tls.trace_buffer(n)
        Y = tls.chain_conv(X, Wa, Wb, policy=pol, debug_first_skip=True, trace=buf, check=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(Y), bits(ref))
        r = trace.decode(buf)
        np.testing.assert_array_equal(np.sort(r["item"]), np.arange(n))
        for wg in np.unique(r["wg"]):
            w = np.sort(r[r["wg"] == wg], order="t_start")
            assert (w["t_start"][1:] >= w["t_end"][:-1]).all(), wg
            assert (np.diff((w["item"] >= P).astype(int)) >= 0).all(), wg

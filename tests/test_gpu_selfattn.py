"""Three-stage self-attention chain on the GPU through the C ABI: parity of
every stage with the oracle, identical bits under every policy and order,
watchdog on both dependencies, sampled rows at the GPT-3 shard size."""

import numpy as np
import pytest

import oracle
import tile_level_sync_amd as tls
from tile_level_sync_amd import inputs
from tests.gpu_util import TOL_FP16, bits, note, to_dev, to_np, torch_dev

pytestmark = pytest.mark.gpu

POLICIES = ["serial", "stridedsync", "tilesync"]


def _run(X, Wqkv, W2, heads, policy, scale, **kw):
    torch = torch_dev()
    M, H = X.shape
    Hs = W2.shape[0]
    q = torch.empty((M, 3 * Hs), dtype=torch.float16, device="cuda")
    dt = torch.empty((M, Hs), dtype=torch.float16, device="cuda")
    Y = tls.chain_selfattn(X, Wqkv, W2, policy=policy, heads=heads, scale=scale, qkv_out=q,
                           dot_out=dt, check=True, **kw)
    torch.cuda.synchronize()
    return Y, q, dt


@pytest.mark.parametrize("M,H,heads", [(256, 256, 2), (512, 384, 3)])
def test_small_all_policies(M, H, heads):
    torch_dev()
    scale = float(np.float32(1.0 / np.sqrt(128.0)))
    Xn, Wq, W2n = inputs.selfattn_inputs(M, H, heads, seed=1, w_sigma=0.05)
    Qr, Dr, Yr = oracle.selfattn_chain(Xn, Wq, W2n, heads, 128, scale)
    X, Wqkv, W2 = map(to_dev, (Xn, Wq, W2n))
    ref = None
    for pol in POLICIES:
        note("selfattn M=%d H=%d heads=%d policy=%s" % (M, H, heads, pol))
        Y, q, dt = _run(X, Wqkv, W2, heads, pol, scale)
        assert oracle.normwise_rel_err(to_np(q), Qr) <= TOL_FP16, pol
        assert oracle.normwise_rel_err(to_np(dt), Dr) <= TOL_FP16, pol
        assert oracle.normwise_rel_err(to_np(Y), Yr) <= TOL_FP16, pol
        if ref is None:
            ref = bits(Y)
        np.testing.assert_array_equal(bits(Y), ref, err_msg=pol)


def test_zero_query_slice_gives_token_mean():
    torch_dev()
    M, H, heads = 256, 256, 2
    Xn, Wq, W2n = inputs.selfattn_inputs(M, H, heads, seed=2, w_sigma=0.05)
    Wq[:, :heads * 128] = 0
    Qr, Dr, Yr = oracle.selfattn_chain(Xn, Wq, W2n, heads, 128, 0.1)
    note("selfattn zero queries")
    Y, q, dt = _run(*map(to_dev, (Xn, Wq, W2n)), heads, "stridedsync", 0.1)
    assert oracle.normwise_rel_err(to_np(dt), Dr) <= 2e-3
    assert oracle.normwise_rel_err(to_np(Y), Yr) <= TOL_FP16


@pytest.mark.parametrize("seed", [1, 2])
def test_orders_bit_identical(seed):
    torch_dev()
    M, H, heads = 512, 256, 4
    Xn, Wq, W2n = inputs.selfattn_inputs(M, H, heads, seed=3, w_sigma=0.05)
    X, Wqkv, W2 = map(to_dev, (Xn, Wq, W2n))
    ref, _, _ = _run(X, Wqkv, W2, heads, "serial", 0.1)
    for pol in POLICIES:
        for order in ("xcd", "row_major", "interleaved"):
            note("selfattn order seed=%d policy=%s order=%s" % (seed, pol, order))
            Y, _, _ = _run(X, Wqkv, W2, heads, pol, 0.1, order=order, order_seed=seed,
                           debug_delay=2)
            np.testing.assert_array_equal(bits(Y), bits(ref))


@pytest.mark.parametrize("pol", ["stridedsync", "tilesync"])
@pytest.mark.parametrize("stage", [1, 2])
def test_watchdog_both_dependencies(pol, stage):
    torch = torch_dev()
    M, H, heads = 256, 256, 2
    Xn, Wq, W2n = inputs.selfattn_inputs(M, H, heads, seed=4, w_sigma=0.05)
    X, Wqkv, W2 = map(to_dev, (Xn, Wq, W2n))
    p1 = tls.chain_selfattn_plan(M, H, heads)["stage1_items"]
    skip = 1 if stage == 1 else p1 + 1
    note("selfattn watchdog policy=%s stage=%d" % (pol, stage))
    with pytest.raises(tls.ChainError) as ei:
        tls.chain_selfattn(X, Wqkv, W2, policy=pol, heads=heads, debug_skip_producer=skip,
                           poll_limit=2000, check=True)
    assert ei.value.status == tls.CHAIN_ETIMEOUT
    ref = tls.chain_selfattn(X, Wqkv, W2, policy="serial", heads=heads, check=True).clone()
    Y = tls.chain_selfattn(X, Wqkv, W2, policy=pol, heads=heads, check=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(Y), bits(ref))


@pytest.mark.parametrize("M", [256, 1024, 2048])
def test_gpt3_shard_sampled_rows(M):
    """H = 12288, 12 heads of 128: XQKV in full, XDot and Y at sampled rows
    against the oracle; the policies bit-identical."""
    torch_dev()
    H, heads = 12288, inputs.GPT3_SA_HEADS
    scale = float(np.float32(1.0 / np.sqrt(128.0)))
    Xn, Wq, W2n = inputs.selfattn_inputs(M, H, heads, seed=0)
    X, Wqkv, W2 = map(to_dev, (Xn, Wq, W2n))
    rows = sorted(set([0, 1, M // 2, M - 1] + list(np.random.default_rng(M).integers(0, M, 4))))
    Qr, Dr, Yr = oracle.selfattn_rows(Xn, Wq, W2n, heads, 128, scale, rows, return_qkv=True)
    ref = None
    for pol in POLICIES:
        note("selfattn gpt3 M=%d policy=%s" % (M, pol))
        Y, q, dt = _run(X, Wqkv, W2, heads, pol, scale)
        assert oracle.normwise_rel_err(to_np(q), Qr) <= TOL_FP16, pol
        assert oracle.normwise_rel_err(to_np(dt)[rows], Dr) <= TOL_FP16, pol
        assert oracle.normwise_rel_err(to_np(Y)[rows], Yr) <= TOL_FP16, pol
        if ref is None:
            ref = bits(Y)
        np.testing.assert_array_equal(bits(Y), ref, err_msg=pol)


@pytest.mark.parametrize("split", [0, 1, 2, 4])
def test_stage1_split_parity_and_bit_equality(split):
    """Stage 1 with its K split in 2 or 4 (and the automatic choice, 2 here:
    12 tiles, 32 K steps): every stage within tolerance of the oracle, Y and
    XQKV bit-identical across the policies and a seeded order."""
    torch_dev()
    M, H, heads = 256, 2048, 2
    scale = float(np.float32(1.0 / np.sqrt(128.0)))
    Xn, Wq, W2n = inputs.selfattn_inputs(M, H, heads, seed=5, w_sigma=0.02)
    Qr, Dr, Yr = oracle.selfattn_chain(Xn, Wq, W2n, heads, 128, scale)
    X, Wqkv, W2 = map(to_dev, (Xn, Wq, W2n))
    ref = refq = None
    for pol in POLICIES:
        for order in ("xcd", "interleaved"):
            note("selfattn split=%d policy=%s order=%s" % (split, pol, order))
            Y, q, dt = _run(X, Wqkv, W2, heads, pol, scale, split_k=split, order=order,
                            order_seed=3 if order == "interleaved" else 0, debug_delay=2)
            assert oracle.normwise_rel_err(to_np(q), Qr) <= TOL_FP16, pol
            assert oracle.normwise_rel_err(to_np(dt), Dr) <= TOL_FP16, pol
            assert oracle.normwise_rel_err(to_np(Y), Yr) <= TOL_FP16, pol
            if ref is None:
                ref, refq = bits(Y), bits(q)
            np.testing.assert_array_equal(bits(Y), ref, err_msg=pol)
            np.testing.assert_array_equal(bits(q), refq, err_msg=pol)


@pytest.mark.parametrize("pol", ["stridedsync", "tilesync"])
def test_stage1_missing_split_times_out_then_recovers(pol):
    torch = torch_dev()
    M, H, heads = 256, 2048, 2
    X, Wqkv, W2 = map(to_dev, inputs.selfattn_inputs(M, H, heads, seed=6, w_sigma=0.02))
    note("selfattn split watchdog policy=%s" % pol)
    with pytest.raises(tls.ChainError) as ei:
        tls.chain_selfattn(X, Wqkv, W2, policy=pol, heads=heads, split_k=4,
                           debug_skip_producer=5, poll_limit=2000, check=True)
    assert ei.value.status == tls.CHAIN_ETIMEOUT
    ref = tls.chain_selfattn(X, Wqkv, W2, policy="serial", heads=heads, split_k=4,
                             check=True).clone()
    Y = tls.chain_selfattn(X, Wqkv, W2, policy=pol, heads=heads, split_k=4, check=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(Y), bits(ref))


def test_stage1_split_argument_errors():
    torch_dev()
    X, Wqkv, W2 = map(to_dev, inputs.selfattn_inputs(256, 2048, 2, seed=1))
    for s in (3, 17, -1):  # 3 does not divide 32 K steps; 17 and -1 out of range
        with pytest.raises(tls.ChainError):
            tls.chain_selfattn(X, Wqkv, W2, heads=2, split_k=s)


@pytest.mark.parametrize("M,heads", [(1, 2), (40, 2), (200, 3), (300, 2), (700, 1)])
def test_ragged_token_counts(M, heads):
    """Any number of tokens: partial row tiles and query blocks, and a last
    key block whose tail is masked.  Every stage against the oracle, all
    policies bit-identical."""
    torch_dev()
    H = 384
    scale = float(np.float32(1.0 / np.sqrt(128.0)))
    Xn, Wq, W2n = inputs.selfattn_inputs(M, H, heads, seed=7, w_sigma=0.05)
    Qr, Dr, Yr = oracle.selfattn_chain(Xn, Wq, W2n, heads, 128, scale)
    X, Wqkv, W2 = map(to_dev, (Xn, Wq, W2n))
    ref = None
    for pol in POLICIES:
        note("selfattn ragged M=%d heads=%d policy=%s" % (M, heads, pol))
        Y, q, dt = _run(X, Wqkv, W2, heads, pol, scale)
        assert oracle.normwise_rel_err(to_np(q), Qr) <= TOL_FP16, pol
        assert oracle.normwise_rel_err(to_np(dt), Dr) <= TOL_FP16, pol
        assert oracle.normwise_rel_err(to_np(Y), Yr) <= TOL_FP16, pol
        if ref is None:
            ref = bits(Y)
        np.testing.assert_array_equal(bits(Y), ref, err_msg=pol)


def test_one_token_is_a_projection_chain():
    """With a single token the softmax is 1 on itself: XDot_h = S3_h of that
    token, rounded once more to fp16 (a closed form on the GPU's own XQKV)."""
    torch_dev()
    M, H, heads = 1, 256, 2
    Xn, Wq, W2n = inputs.selfattn_inputs(M, H, heads, seed=8, w_sigma=0.05)
    X, Wqkv, W2 = map(to_dev, (Xn, Wq, W2n))
    note("selfattn one token")
    Y, q, dt = _run(X, Wqkv, W2, heads, "stridedsync", 0.3)
    Hs = heads * 128
    np.testing.assert_array_equal(bits(dt), bits(q[:, 2 * Hs:].contiguous()))


@pytest.mark.parametrize("split", [2, 3, 16])
def test_stage2_key_split_parity_and_bit_equality(split):
    """Stage 2 with its keys split in contiguous ranges of 64-key blocks (1000
    tokens: 16 blocks, the last one ragged; 16 splits of one block each):
    every stage within tolerance of the oracle, Y and XDot bit-identical
    across the policies and a seeded order with delays (the merge runs in
    split order whichever split finishes last)."""
    torch_dev()
    M, H, heads = 1000, 256, 2
    scale = float(np.float32(1.0 / np.sqrt(128.0)))
    Xn, Wq, W2n = inputs.selfattn_inputs(M, H, heads, seed=9, w_sigma=0.05)
    Qr, Dr, Yr = oracle.selfattn_chain(Xn, Wq, W2n, heads, 128, scale)
    X, Wqkv, W2 = map(to_dev, (Xn, Wq, W2n))
    ref = refd = None
    for pol in POLICIES:
        for order in ("xcd", "interleaved"):
            note("selfattn key split=%d policy=%s order=%s" % (split, pol, order))
            Y, q, dt = _run(X, Wqkv, W2, heads, pol, scale, split_keys=split, order=order,
                            order_seed=5 if order == "interleaved" else 0, debug_delay=2)
            assert oracle.normwise_rel_err(to_np(q), Qr) <= TOL_FP16, pol
            assert oracle.normwise_rel_err(to_np(dt), Dr) <= TOL_FP16, pol
            assert oracle.normwise_rel_err(to_np(Y), Yr) <= TOL_FP16, pol
            if ref is None:
                ref, refd = bits(Y), bits(dt)
            np.testing.assert_array_equal(bits(Y), ref, err_msg=pol)
            np.testing.assert_array_equal(bits(dt), refd, err_msg=pol)


def test_stage2_key_split_with_stage1_split():
    """Both splits at once (stage 1 in 4, stage 2 in 2): the two kinds of
    arrival counters share one array without overlapping."""
    torch_dev()
    M, H, heads = 512, 2048, 2
    scale = float(np.float32(1.0 / np.sqrt(128.0)))
    Xn, Wq, W2n = inputs.selfattn_inputs(M, H, heads, seed=10, w_sigma=0.02)
    Qr, Dr, Yr = oracle.selfattn_chain(Xn, Wq, W2n, heads, 128, scale)
    X, Wqkv, W2 = map(to_dev, (Xn, Wq, W2n))
    ref = None
    for pol in POLICIES:
        for _ in range(2):  # the counters are cleared for the next call
            note("selfattn both splits policy=%s" % pol)
            Y, q, dt = _run(X, Wqkv, W2, heads, pol, scale, split_k=4, split_keys=2)
            assert oracle.normwise_rel_err(to_np(dt), Dr) <= TOL_FP16, pol
            assert oracle.normwise_rel_err(to_np(Y), Yr) <= TOL_FP16, pol
            if ref is None:
                ref = bits(Y)
            np.testing.assert_array_equal(bits(Y), ref, err_msg=pol)


@pytest.mark.parametrize("pol", ["stridedsync", "tilesync"])
def test_stage2_missing_key_split_times_out_then_recovers(pol):
    torch = torch_dev()
    M, H, heads = 1024, 256, 2
    X, Wqkv, W2 = map(to_dev, inputs.selfattn_inputs(M, H, heads, seed=11, w_sigma=0.05))
    p1 = tls.chain_selfattn_plan(M, H, heads, split_keys=4)["stage1_items"]
    note("selfattn key split watchdog policy=%s" % pol)
    with pytest.raises(tls.ChainError) as ei:
        tls.chain_selfattn(X, Wqkv, W2, policy=pol, heads=heads, split_keys=4,
                           debug_skip_producer=p1 + 1, poll_limit=2000, check=True)
    assert ei.value.status == tls.CHAIN_ETIMEOUT
    ref = tls.chain_selfattn(X, Wqkv, W2, policy="serial", heads=heads, split_keys=4,
                             check=True).clone()
    Y = tls.chain_selfattn(X, Wqkv, W2, policy=pol, heads=heads, split_keys=4, check=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(Y), bits(ref))


def test_stage2_key_split_argument_errors():
    torch_dev()
    X, Wqkv, W2 = map(to_dev, inputs.selfattn_inputs(1000, 256, 2, seed=1))
    # 17 and -1 out of range; 5 splits of 16 key blocks (4 per split) leave the
    # fifth empty
    for s in (17, -1, 5):
        with pytest.raises(tls.ChainError):
            tls.chain_selfattn(X, Wqkv, W2, heads=2, split_keys=s)
    X1, Wq1, W21 = map(to_dev, inputs.selfattn_inputs(100, 256, 2, seed=1))
    with pytest.raises(tls.ChainError):  # 3 splits of 2 key blocks
        tls.chain_selfattn(X1, Wq1, W21, heads=2, split_keys=3)


@pytest.mark.parametrize("pol", POLICIES)
def test_trace_records_every_item_once(pol):
    """The optional per-item trace of the three-stage chain: one record per
    work item (stage 1, 2, 3 in turn) at its index, times ordered, a
    workgroup's items disjoint in time and in stage order; Y unchanged by
    tracing."""
    torch = torch_dev()
    from tile_level_sync_amd import trace
    M, H, heads = 512, 384, 3
    X, Wqkv, W2 = map(to_dev, inputs.selfattn_inputs(M, H, heads, seed=16, w_sigma=0.05))
    plan = tls.chain_selfattn_plan(M, H, heads)
    P1, P2 = plan["stage1_items"], plan["stage2_items"]
    n = tls.selfattn_work_items(M, H, heads)
    ref, _, _ = _run(X, Wqkv, W2, heads, pol, 0.1)
    buf = tls.trace_buffer(n + 3)
    note("selfattn trace policy=%s items=%d" % (pol, n))
    Y = tls.chain_selfattn(X, Wqkv, W2, policy=pol, heads=heads, scale=0.1, trace=buf,
                           check=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(Y), bits(ref))
    r = trace.decode(buf)
    assert len(r) == n
    np.testing.assert_array_equal(r["item"], np.arange(n))
    assert (r["t_start"] <= r["t_ready"]).all() and (r["t_ready"] <= r["t_end"]).all()
    assert (r["t_ready"][:P1] == r["t_start"][:P1]).all()
    stage = np.where(r["item"] < P1, 0, np.where(r["item"] < P1 + P2, 1, 2))
    for wg in np.unique(r["wg"]):
        sel = r["wg"] == wg
        order = np.argsort(r["t_start"][sel], kind="stable")
        w = r[sel][order]
        assert (w["t_start"][1:] >= w["t_end"][:-1]).all(), wg
        assert (np.diff(stage[sel][order]) >= 0).all(), wg
    s = trace.summarize(r, P1, tls.trace_clock_khz(),
                        n_cu=torch.cuda.get_device_properties(0).multi_processor_count)
    assert 0.0 < s["busy_frac"] <= 1.0


def _bf16_dev(bits16):
    torch = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(bits16).view(np.int16)).to("cuda").view(
        torch.bfloat16)


def _bits16(t):
    torch = torch_dev()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _run_bf16(X, Wqkv, W2, heads, policy, scale, **kw):
    torch = torch_dev()
    M, H = X.shape
    Hs = W2.shape[0]
    q = torch.empty((M, 3 * Hs), dtype=torch.bfloat16, device="cuda")
    dt = torch.empty((M, Hs), dtype=torch.bfloat16, device="cuda")
    Y = tls.chain_selfattn(X, Wqkv, W2, policy=policy, heads=heads, scale=scale, qkv_out=q,
                           dot_out=dt, check=True, **kw)
    torch.cuda.synchronize()
    assert Y.dtype == torch.bfloat16
    return _bits16(Y), _bits16(q), _bits16(dt)


@pytest.mark.parametrize("M,H,heads,kw", [(256, 256, 2, {}),
                                          (1000, 256, 2, {"split_keys": 3, "split_k": 2})])
def test_bf16_all_policies(M, H, heads, kw):
    """bf16 storage: XQKV, XDot and Y within 2e-2 of the bf16 oracle under
    every policy (whole outputs; 1000 tokens: a ragged last tile and key
    block, stage 1 split along K and stage 2 along the keys), all three
    bit-equal across the policies."""
    torch_dev()
    scale = float(np.float32(1.0 / np.sqrt(128.0)))
    Xb, Wqb, W2b = inputs.selfattn_inputs_bf16(M, H, heads, seed=11, w_sigma=0.05)
    Qr, Dr, Yr = oracle.selfattn_chain_bf16(Xb, Wqb, W2b, heads, 128, scale)
    X, Wqkv, W2 = map(_bf16_dev, (Xb, Wqb, W2b))
    ref = None
    for pol in POLICIES:
        note("selfattn bf16 M=%d H=%d heads=%d %s policy=%s" % (M, H, heads, kw, pol))
        got = _run_bf16(X, Wqkv, W2, heads, pol, scale, **kw)
        for g, r, name in zip(got, (Yr, Qr, Dr), ("Y", "XQKV", "XDot")):
            assert oracle.normwise_rel_err(oracle.bf16_values(g),
                                           oracle.bf16_values(r)) <= TOL_FP16, (pol, name)
        if ref is None:
            ref = got
        for g, r in zip(got, ref):
            np.testing.assert_array_equal(g, r, err_msg=pol)


def test_bf16_gpt3_shard_sampled_rows():
    """H = 12288, 12 heads of 128, M = 2048 in bf16: XDot and Y at sampled
    rows against the bf16 oracle; the policies bit-identical."""
    torch_dev()
    M, H, heads = 2048, 12288, inputs.GPT3_SA_HEADS
    scale = float(np.float32(1.0 / np.sqrt(128.0)))
    Xb, Wqb, W2b = inputs.selfattn_inputs_bf16(M, H, heads, seed=0)
    X, Wqkv, W2 = map(_bf16_dev, (Xb, Wqb, W2b))
    rows = sorted(set([0, 1, M // 2, M - 1] + list(np.random.default_rng(M).integers(0, M, 4))))
    Dr, Yr = oracle.selfattn_rows_bf16(Xb, Wqb, W2b, heads, 128, scale, rows)
    ref = None
    for pol in POLICIES:
        note("selfattn bf16 gpt3 M=%d policy=%s" % (M, pol))
        Y, _, dt = _run_bf16(X, Wqkv, W2, heads, pol, scale)
        assert oracle.normwise_rel_err(oracle.bf16_values(dt[rows]),
                                       oracle.bf16_values(Dr)) <= TOL_FP16, pol
        assert oracle.normwise_rel_err(oracle.bf16_values(Y[rows]),
                                       oracle.bf16_values(Yr)) <= TOL_FP16, pol
        if ref is None:
            ref = Y
        np.testing.assert_array_equal(Y, ref, err_msg=pol)

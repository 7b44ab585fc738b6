"""Attention-score chain on the GPU through the C ABI: parity with the
oracle, uniform and one-hot softmax, bit-equality across policies and orders,
watchdog, sampled heads at the full sizes."""

import numpy as np
import pytest

import oracle
import tile_level_sync_amd as tls
from tile_level_sync_amd import inputs
from tests.gpu_util import TOL_FP16, bits, note, to_dev, to_np, torch_dev

pytestmark = pytest.mark.gpu

POLICIES = ["serial", "tilesync", "rowsync", "sentinel"]


def _run(Q, K, V, policy, scale, s_out=False, **kw):
    torch = torch_dev()
    B, Hh, S, _ = Q.shape
    sc = torch.empty((B, Hh, S, S), dtype=torch.float16, device="cuda") if s_out else None
    O = tls.chain_attn(Q, K, V, policy=policy, scale=scale, s_out=sc, check=True, **kw)
    torch.cuda.synchronize()
    return O, sc


@pytest.mark.parametrize("scale", [1.0, 1.0 / np.sqrt(128.0)])
def test_small_all_policies(scale):
    torch_dev()
    scale = float(np.float32(scale))
    Qn, Kn, Vn = inputs.attn_inputs(2, 3, 256, 128, seed=1)
    A, Scr, P, Or = oracle.attn_chain(Qn, Kn, Vn, scale)
    Q, K, V = map(to_dev, (Qn, Kn, Vn))
    ref = None
    for pol in POLICIES:
        note("attn small scale=%.4f policy=%s" % (scale, pol))
        O, sc = _run(Q, K, V, pol, scale, s_out=True)
        assert oracle.normwise_rel_err(to_np(sc), Scr) <= TOL_FP16, pol
        assert oracle.normwise_rel_err(to_np(O), Or) <= TOL_FP16, pol
        if ref is None:
            ref = bits(O)
        np.testing.assert_array_equal(bits(O), ref, err_msg=pol)


def test_zero_queries_give_column_mean():
    torch_dev()
    _, Kn, Vn = inputs.attn_inputs(1, 2, 128, 128, seed=2)
    Qn = np.zeros_like(Kn)
    _, _, _, Or = oracle.attn_chain(Qn, Kn, Vn, 1.0)
    note("attn zero queries")
    O, _ = _run(*map(to_dev, (Qn, Kn, Vn)), "rowsync", 1.0)
    assert oracle.normwise_rel_err(to_np(O), Or) <= 2e-3


def test_dominant_key_one_hot():
    torch_dev()
    S, d = 128, 128
    Qn = np.zeros((1, 1, S, d), np.float16)
    Kn = np.zeros((1, 1, S, d), np.float16)
    Vn = inputs.normal_fp16((1, 1, S, d), 1.0, 4, 2)
    Qn[..., 0] = 1.0
    Kn[0, 0, 77, 0] = 200.0
    note("attn one-hot")
    O, _ = _run(*map(to_dev, (Qn, Kn, Vn)), "tilesync", 1.0)
    np.testing.assert_array_equal(to_np(O)[0, 0], np.broadcast_to(Vn[0, 0, 77], (S, d)))


@pytest.mark.parametrize("seed", [1, 2])
def test_orders_bit_identical(seed):
    torch_dev()
    Qn, Kn, Vn = inputs.attn_inputs(1, 4, 512, 128, seed=3)
    Q, K, V = map(to_dev, (Qn, Kn, Vn))
    ref, _ = _run(Q, K, V, "serial", 0.125)
    for pol in ("serial", "tilesync", "rowsync", "sentinel"):
        for order in ("xcd", "row_major", "interleaved", "col_major", "strided"):
            note("attn order seed=%d policy=%s order=%s" % (seed, pol, order))
            O, _ = _run(Q, K, V, pol, 0.125, order=order, order_seed=seed, debug_delay=1)
            np.testing.assert_array_equal(bits(O), bits(ref))


@pytest.mark.parametrize("pol", ["tilesync", "rowsync", "sentinel"])
def test_watchdog(pol):
    torch = torch_dev()
    Qn, Kn, Vn = inputs.attn_inputs(1, 2, 256, 128, seed=4)
    Q, K, V = map(to_dev, (Qn, Kn, Vn))
    note("attn watchdog policy=%s" % pol)
    with pytest.raises(tls.ChainError) as ei:
        tls.chain_attn(Q, K, V, policy=pol, debug_skip_producer=1, poll_limit=2000, check=True)
    assert ei.value.status == tls.CHAIN_ETIMEOUT
    ref = tls.chain_attn(Q, K, V, policy="serial", check=True).clone()
    O = tls.chain_attn(Q, K, V, policy=pol, check=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(O), bits(ref))


@pytest.mark.parametrize("B,S", [(1, 512), (1, 1024), (4, 512), (4, 1024)])
def test_full_size_sampled_heads(B, S):
    """96 heads, d = 128: policies bit-identical; sampled (batch, head, rows)
    against the oracle."""
    torch_dev()
    Qn, Kn, Vn = inputs.attn_inputs(B, 96, S, 128, seed=0)
    Q, K, V = map(to_dev, (Qn, Kn, Vn))
    rng = np.random.default_rng(S + B)
    ref = None
    for pol in POLICIES:
        note("attn B=%d S=%d policy=%s" % (B, S, pol))
        O, _ = _run(Q, K, V, pol, 1.0)
        Oh = to_np(O)
        if ref is None:
            ref = Oh.view(np.uint16).copy()
            for _ in range(3):
                b, h = int(rng.integers(B)), int(rng.integers(96))
                rows = sorted(set([0, S - 1, 127, 128] + rng.integers(0, S, 6).tolist()))
                _, _, _, Orow = oracle.attn_chain_rows(Qn, Kn, Vn, b, h, rows, 1.0)
                assert oracle.normwise_rel_err(Oh[b, h, rows], Orow) <= TOL_FP16
        np.testing.assert_array_equal(Oh.view(np.uint16), ref, err_msg=pol)


@pytest.mark.parametrize("pol", ["rowsync", "tilesync"])
def test_alternating_inputs_reuse_one_score_buffer(pol):
    """Two different inputs in turn through one workspace and one aligned
    score buffer (light acquire): each O bit-equal to its own serial result
    and within tolerance of the oracle."""
    torch = torch_dev()
    B, Hh, S, d = 1, 8, 512, 128
    data, refs, oref = [], [], []
    for seed in (41, 42):
        Qn, Kn, Vn = inputs.attn_inputs(B, Hh, S, d, seed=seed)
        oref.append(oracle.attn_chain(Qn, Kn, Vn, scale=1.0)[3])
        dd = tuple(map(to_dev, (Qn, Kn, Vn)))
        data.append(dd)
        refs.append(_run(*dd, "serial", 1.0)[0].clone())
    ws = torch.zeros(tls.chain_attn_workspace_bytes(B, Hh, S, d, policy=pol),
                     dtype=torch.uint8, device="cuda")
    sc = torch.empty((B, Hh, S, S), dtype=torch.float16, device="cuda")
    assert sc.data_ptr() % 128 == 0
    for it in range(6):
        i = it % 2
        note("attn alternating inputs policy=%s call=%d" % (pol, it))
        O = tls.chain_attn(*data[i], policy=pol, scale=1.0, workspace=ws, s_out=sc,
                           debug_delay=1 if it >= 4 else 0, check=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(O), bits(refs[i]), err_msg="call %d" % it)
        assert oracle.normwise_rel_err(to_np(O), oref[i]) <= TOL_FP16


def test_sentinel_ring_matches_flag_policy():
    """Sentinel buffer rotation on the attention chain: three calls through a
    ring of two score buffers.  O and the scores are bit-equal to RowSync's;
    the next call's slot holds the sentinel once a call has ended."""
    torch = torch_dev()
    B, Hh, S, d = 1, 3, 256, 128
    ring = tls.SentinelRing(B * Hh * S, S, slots=2)
    ring.buf.fill_(0)
    for i in range(3):
        note("attn sentinel ring call %d" % i)
        Q, K, V = map(to_dev, inputs.attn_inputs(B, Hh, S, d, seed=30 + i))
        ref, scref = _run(Q, K, V, "rowsync", 1.0, s_out=True)
        O = tls.chain_attn(Q, K, V, policy="sentinel", scale=1.0, ring=ring, check=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(O), bits(ref))
        np.testing.assert_array_equal(bits(ring.slot(i)).reshape(-1), bits(scref).reshape(-1))
        assert (bits(ring.slot(i + 1)) == 0xFFFF).all()


def _wide_shape():
    """B, heads, S with at least two score-row blocks per workgroup slot (two
    per CU): consumers start while producers still run."""
    torch = torch_dev()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    B, S = 2, 1024
    heads = -(-2 * cus * 128 // (B * S))
    return B, heads, S


def test_tilesync_with_waiting_consumers():
    """Producers delayed (debug_delay) so that consumers find rows incomplete
    and wait on the row's key-block flags; O bit-identical to the serialised
    launches and sampled rows within tolerance of the oracle."""
    torch_dev()
    B, heads, S = _wide_shape()
    scale = float(np.float32(1.0 / np.sqrt(128.0)))
    Qn, Kn, Vn = inputs.attn_inputs(B, heads, S, 128, seed=12)
    Q, K, V = map(to_dev, (Qn, Kn, Vn))
    note("attn wide serial B=%d heads=%d S=%d" % (B, heads, S))
    ref, _ = _run(Q, K, V, "serial", scale)
    ref = bits(ref)
    for delay in (0, 4):
        note("attn wide tilesync delay=%d" % delay)
        O, _ = _run(Q, K, V, "tilesync", scale, debug_delay=delay)
        np.testing.assert_array_equal(bits(O), ref)
    rows = [0, 511, 1023]
    for b, h in ((0, 0), (B - 1, heads - 1)):
        Or = oracle.attn_chain_rows(Qn, Kn, Vn, b, h, rows, scale)[3]
        assert oracle.normwise_rel_err(to_np(O)[b, h][rows], Or) <= TOL_FP16


def test_tilesync_wide_watchdog_then_recovers():
    torch = torch_dev()
    B, heads, S = _wide_shape()
    Q, K, V = map(to_dev, inputs.attn_inputs(B, heads, S, 128, seed=13))
    note("attn wide tilesync watchdog")
    with pytest.raises(tls.ChainError) as ei:
        tls.chain_attn(Q, K, V, policy="tilesync", debug_skip_producer=B * heads * S // 128 - 1,
                       poll_limit=2000, check=True)
    assert ei.value.status == tls.CHAIN_ETIMEOUT
    ref = tls.chain_attn(Q, K, V, policy="serial", check=True).clone()
    O = tls.chain_attn(Q, K, V, policy="tilesync", check=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(O), bits(ref))


@pytest.mark.parametrize("pol", ["serial", "rowsync", "tilesync"])
def test_trace_records_every_item_once(pol):
    """The optional per-item trace of the attention chain: one record per
    score row block (producers, then consumers) at its index, times ordered,
    a workgroup's items disjoint in time with its producer items first; O
    unchanged by tracing."""
    torch = torch_dev()
    from tile_level_sync_amd import trace
    B, heads, S = 1, 8, 512
    Q, K, V = map(to_dev, inputs.attn_inputs(B, heads, S, 128, seed=15))
    n = tls.attn_work_items(B, heads, S)
    P = n // 2
    ref, _ = _run(Q, K, V, pol, 0.125)
    buf = tls.trace_buffer(n + 3)
    note("attn trace policy=%s items=%d" % (pol, n))
    O = tls.chain_attn(Q, K, V, policy=pol, scale=0.125, trace=buf, check=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(O), bits(ref))
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
    assert 0.0 < s["busy_frac"] <= 1.0
    if pol == "serial":
        assert s["producer_consumer_gap_us"] >= 0.0


def test_trace_capacity_too_small():
    torch_dev()
    Q, K, V = map(to_dev, inputs.attn_inputs(1, 2, 256, 128, seed=1))
    with pytest.raises(tls.ChainError):
        tls.chain_attn(Q, K, V, trace=tls.trace_buffer(tls.attn_work_items(1, 2, 256) - 1))


def _bf16_dev(bits16):
    torch = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(bits16).view(np.int16)).to("cuda").view(
        torch.bfloat16)


def _bits16(t):
    torch = torch_dev()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("B,Hh,S", [(2, 3, 256), (1, 2, 384)])
def test_bf16_all_policies(B, Hh, S):
    """bf16 storage: the stored scores and O within 2e-2 of the bf16 oracle
    under every policy, O and the scores bit-equal across policies."""
    torch = torch_dev()
    scale = float(np.float32(1.0 / np.sqrt(128.0)))
    Qb, Kb, Vb = inputs.attn_inputs_bf16(B, Hh, S, 128, seed=21)
    _, Scb, _, Ob = oracle.attn_chain_bf16(Qb, Kb, Vb, scale)
    Q, K, V = map(_bf16_dev, (Qb, Kb, Vb))
    ref = None
    for pol in POLICIES:
        note("attn bf16 B=%d heads=%d S=%d policy=%s" % (B, Hh, S, pol))
        sc = torch.empty((B, Hh, S, S), dtype=torch.bfloat16, device="cuda")
        O = tls.chain_attn(Q, K, V, policy=pol, scale=scale, s_out=sc, check=True)
        torch.cuda.synchronize()
        assert O.dtype == torch.bfloat16
        assert oracle.normwise_rel_err(oracle.bf16_values(_bits16(sc)),
                                       oracle.bf16_values(Scb)) <= TOL_FP16, pol
        assert oracle.normwise_rel_err(oracle.bf16_values(_bits16(O)),
                                       oracle.bf16_values(Ob)) <= TOL_FP16, pol
        got = (_bits16(O), _bits16(sc))
        if ref is None:
            ref = got
        np.testing.assert_array_equal(got[0], ref[0], err_msg=pol)
        np.testing.assert_array_equal(got[1], ref[1], err_msg=pol)


def test_bf16_full_size_sampled_heads():
    """96 heads, S = 1024, d = 128 in bf16: policies bit-identical, sampled
    (batch, head, rows) within 2e-2 of the bf16 oracle."""
    torch = torch_dev()
    B, Hh, S = 1, 96, 1024
    Qb, Kb, Vb = inputs.attn_inputs_bf16(B, Hh, S, 128, seed=3)
    Q, K, V = map(_bf16_dev, (Qb, Kb, Vb))
    rng = np.random.default_rng(7)
    ref = None
    for pol in POLICIES:
        note("attn bf16 B=%d S=%d policy=%s" % (B, S, pol))
        O = tls.chain_attn(Q, K, V, policy=pol, scale=1.0, check=True)
        torch.cuda.synchronize()
        Ob = _bits16(O)
        if ref is None:
            ref = Ob
            for _ in range(3):
                h = int(rng.integers(Hh))
                rows = sorted(set([0, S - 1, 127, 128] + rng.integers(0, S, 6).tolist()))
                Orow = oracle.attn_chain_bf16_rows(Qb, Kb, Vb, 0, h, rows, 1.0)[3]
                assert oracle.normwise_rel_err(oracle.bf16_values(Ob[0, h, rows]),
                                               oracle.bf16_values(Orow)) <= TOL_FP16
        np.testing.assert_array_equal(Ob, ref, err_msg=pol)


def test_bf16_waiting_tilesync_and_sentinel_ring():
    """bf16 under TileSync with delayed producers and through a sentinel ring
    of two score slots: O bit-equal to the serialised launches; the ring's
    slot holds the scores, the next slot the sentinel."""
    torch = torch_dev()
    B, Hh, S = _wide_shape()
    scale = float(np.float32(1.0 / np.sqrt(128.0)))
    Qb, Kb, Vb = inputs.attn_inputs_bf16(B, Hh, S, 128, seed=4)
    Q, K, V = map(_bf16_dev, (Qb, Kb, Vb))
    note("attn bf16 wide serial B=%d heads=%d S=%d" % (B, Hh, S))
    sc = torch.empty((B, Hh, S, S), dtype=torch.bfloat16, device="cuda")
    ref = _bits16(tls.chain_attn(Q, K, V, policy="serial", scale=scale, s_out=sc, check=True))
    scref = _bits16(sc)
    note("attn bf16 wide tilesync delay=4")
    O = tls.chain_attn(Q, K, V, policy="tilesync", scale=scale, debug_delay=4, check=True)
    np.testing.assert_array_equal(_bits16(O), ref)
    ring = tls.SentinelRing(B * Hh * S, S, slots=2)
    ring.buf.fill_(0)
    for i in range(2):
        note("attn bf16 sentinel ring call %d" % i)
        O = tls.chain_attn(Q, K, V, policy="sentinel", scale=scale, ring=ring, check=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_bits16(O), ref)
        np.testing.assert_array_equal(bits(ring.slot(i)).reshape(-1), scref.reshape(-1))
        assert (bits(ring.slot(i + 1)) == 0xFFFF).all()
    rows = [0, 511, 1023]
    Orow = oracle.attn_chain_bf16_rows(Qb, Kb, Vb, B - 1, Hh - 1, rows, scale)[3]
    assert oracle.normwise_rel_err(oracle.bf16_values(ref[B - 1, Hh - 1][rows]),
                                   oracle.bf16_values(Orow)) <= TOL_FP16


@pytest.mark.parametrize("pol", POLICIES)
def test_first_items_left_to_the_sweep(pol):
    """The default order hands a launch's first producer rows out through
    eight per-XCD counters; with the test knob the odd workgroups take none,
    and the workgroup that draws the first consumer value (under serial: the
    producer launch's end) runs the rest before its own item.  O bit-equal
    to the call without the knob, every item traced exactly once."""
    torch = torch_dev()
    from tile_level_sync_amd import trace
    B, Hh, S = 1, 3, 512
    scale = float(np.float32(1.0 / np.sqrt(128.0)))
    Q, K, V = map(to_dev, inputs.attn_inputs(B, Hh, S, 128, seed=19))
    n = tls.attn_work_items(B, Hh, S)
    P = n // 2
    note("attn first items policy=%s reference" % pol)
    ref, _ = _run(Q, K, V, pol, scale)
    ref = bits(ref)
    for rep in range(2):
        note("attn first items left to the sweep policy=%s call %d" % (pol, rep))
        buf = tls.trace_buffer(n)
        O = tls.chain_attn(Q, K, V, policy=pol, scale=scale, debug_first_skip=True, trace=buf,
                           check=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(O), ref)
        r = trace.decode(buf)
        np.testing.assert_array_equal(np.sort(r["item"]), np.arange(n))
        for wg in np.unique(r["wg"]):
            w = np.sort(r[r["wg"] == wg], order="t_start")
            assert (np.diff((w["item"] >= P).astype(int)) >= 0).all(), wg

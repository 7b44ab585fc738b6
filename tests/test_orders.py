"""Work orders of the persistent scheduler (no GPU): every order the library
builds (row-major, interleaved, column-major, strided row-major, per-XCD
queues, with and without a seed) lists every work item exactly once and each
consumer item after every producer item it reads.  That is the property the
chain's freedom from deadlock rests on whatever number of workgroups is
resident (cuSync paper, "Tile Processing Order"; the wait-kernel of "Invoke
Dependent Kernels" exists for the same ordering).  The dependency sets are the
oracle's brute-force ones, not the library's closed forms."""

import functools

import pytest

import oracle
import tile_level_sync_amd as tls

ORDERS = ["xcd", "row_major", "interleaved", "col_major", "strided"]


@functools.lru_cache(maxsize=None)
def _mlp_row_deps(i, M, F, BM, BN1):
    # a consumer tile's read set depends on its rows only: one column suffices
    return frozenset(oracle.mlp_consumer_deps(i, 0, M, 1, F, BM, BN1, 1))


@functools.lru_cache(maxsize=None)
def _conv_row_deps(i, N, side, bm):
    return frozenset(r for r, _ in oracle.conv_consumer_deps(i, N, side, side, 1, bm, 1))


def _check(seq, P, C, deps_of_consumer, queues=False):
    assert sorted(seq) == list(range(P + C)), "every item exactly once"
    pos = {it: i for i, it in enumerate(seq)}
    if queues:
        # per-XCD queues: a workgroup starts consumer queues only once every
        # producer queue is empty, so producers simply precede consumers here
        assert max(pos[p] for p in range(P)) < min(pos[P + c] for c in range(C))
        return
    for c in range(C):
        need = deps_of_consumer(c)
        assert need, c
        last = max(pos[p] for p in need)
        assert pos[P + c] > last, ("consumer item %d listed before producer item %d"
                                   % (c, max(need, key=lambda p: pos[p])))


@pytest.mark.parametrize("order", ORDERS)
@pytest.mark.parametrize("seed", [0, 7])
@pytest.mark.parametrize("M,cfg,splits", [(256, 3, (1, 1)), (300, 1, (2, 1)), (64, 0, (1, 2))])
def test_mlp_orders_respect_dependencies(order, seed, M, cfg, splits):
    H, F = 512, 768
    plan = tls.chain_mlp_plan(M, H, F, tile_cfg=cfg)
    tc = tls.tile_configs()[cfg]
    seq = tls.mlp_order(M, H, F, order=order, order_seed=seed, tile_cfg=cfg, split_k=splits,
                        order_stride=3)
    ks1, ks2 = splits
    nt1, nt2 = plan["prod_col_tiles"], plan["cons_col_tiles"]
    P = plan["producer_tiles"] * ks1
    C = plan["consumer_tiles"] * ks2

    def deps(c):
        tile = c // ks2
        i, j = divmod(tile, nt2)
        ptiles = _mlp_row_deps(i, M, F, tc["bm"], tc["bn1"])
        return {(r * nt1 + cc) * ks1 + s for r, cc in ptiles for s in range(ks1)}

    queues = order == "xcd" and M > 128
    _check(seq, P, C, deps, queues=queues)


@pytest.mark.parametrize("order", ORDERS)
@pytest.mark.parametrize("seed", [0, 11])
@pytest.mark.parametrize("N,side", [(2, 56), (2, 64), (1, 112)])
def test_conv_orders_respect_halo_dependencies(order, seed, N, side):
    """Image widths where the 3x3 halo (W + 1 flattened pixels) is shorter
    than, and longer than, a 64-pixel tile."""
    C = K = 64
    plan = tls.chain_conv_plan(N, side, side, C, K)
    bm = [128, 256, 128, 64, 128, 64, 64, 128][plan["tile_cfg"]]
    ks1, ks2 = plan["split_k1"], plan["split_k2"]
    nt = plan["prod_col_tiles"]
    P = plan["producer_tiles"] * ks1
    Cn = plan["consumer_tiles"] * ks2
    seq = tls.conv_order(N, side, side, C, K, order=order, order_seed=seed)

    def deps(c):
        tile = c // ks2
        i = tile // nt
        rows = _conv_row_deps(i, N, side, bm)
        return {(r * nt + cc) * ks1 + s for r in rows for cc in range(nt) for s in range(ks1)}

    _check(seq, P, Cn, deps)


def test_conv_interleaved_lists_halo_rows_first():
    """W = 64 with 64-pixel tiles: consumer tile 0 reads producer tiles 0..2
    (halo of 65 pixels), so it follows producer tile 3 (one row of lag), not
    producer tile 1."""
    seq = tls.conv_order(2, 64, 64, 64, 64, order="interleaved")
    plan = tls.chain_conv_plan(2, 64, 64, 64, 64)
    assert plan["tile_cfg"] == 3 and plan["split_k1"] == 1
    P = plan["producer_tiles"]
    assert seq[:5] == [0, 1, 2, 3, P + 0]


@pytest.mark.parametrize("order", ORDERS)
@pytest.mark.parametrize("seed", [0, 3])
def test_attn_orders_respect_dependencies(order, seed):
    B, heads, S = 2, 3, 512
    blocks = S // 128
    P = C = B * heads * blocks
    seq = tls.attn_order(B, heads, S, order=order, order_seed=seed)

    def deps(c):
        pair, ti = divmod(c, blocks)
        return {pair * blocks + r for r, _ in oracle.attn_consumer_deps(ti, S, 128, 128)}

    _check(seq, P, C, deps)


def test_col_major_and_strided_sequences():
    """The natural (unseeded) sequences: column by column, and row by row with
    the columns of each row visited with the given stride."""
    M, H, F = 256, 512, 768  # config 3: 128 x 64 tiles, 2 rows, 12 and 8 columns
    plan = tls.chain_mlp_plan(M, H, F, tile_cfg=3)
    nt1 = plan["prod_col_tiles"]
    assert (plan["row_tiles"], nt1) == (2, 12)
    col = tls.mlp_order(M, H, F, order="col_major", tile_cfg=3, split_k=(1, 1))
    assert col[:4] == [0, nt1, 1, nt1 + 1]
    st = tls.mlp_order(M, H, F, order="strided", order_stride=4, tile_cfg=3, split_k=(1, 1))
    assert st[:6] == [0, 4, 8, 1, 5, 9]
    assert st[12:15] == [12, 16, 20]
    P = 2 * nt1
    assert st[P:P + 3] == [P + 0, P + 4, P + 1]  # consumer rows of 8 columns: 0, 4, 1, 5, ...


def test_serial_orders_keep_phases_apart():
    """The stream-serialised baseline launches producer positions [0, P) and
    then consumer positions [P, P + C): every table order keeps that split."""
    M, H, F = 256, 512, 768
    plan = tls.chain_mlp_plan(M, H, F, tile_cfg=3)
    P = plan["producer_tiles"] * plan["split_k1"]
    for order in ORDERS[1:]:
        seq = tls.mlp_order(M, H, F, policy="serial", order=order, order_seed=5, tile_cfg=3)
        assert sorted(seq[:P]) == list(range(P)), order


def test_order_argument_errors():
    with pytest.raises(tls.ChainError):
        tls.mlp_order(256, 512, 768, order=5)
    with pytest.raises(tls.ChainError):
        tls.mlp_order(256, 512, 768, order="strided", order_stride=-1)

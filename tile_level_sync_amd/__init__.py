"""Tile-level synchronised GEMM chains on MI355X (gfx950).

Thin ctypes binding of ``libtlsync.so``: every function marshals arguments
(tensor data pointers, sizes, the current HIP stream) and calls the C ABI of
``include/tlsync.h`` with the same name.  All computation runs in the
library's HIP kernels; PyTorch only provides device memory and streams.
There is no fallback: if the library is not built, the calls raise.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtlsync.so")

CHAIN_OK = 0
CHAIN_EINVAL = -1
CHAIN_EUNSUPPORTED = -2
CHAIN_EHIP = -3
CHAIN_ETIMEOUT = -4
CHAIN_ENOMEM = -5
CHAIN_ESCRATCH = -6

POLICIES = {
    "serial": 0, "stream_serial": 0, "streamsync": 0,
    "tilesync": 1, "rowsync": 2, "conv2d_tilesync": 3, "sentinel": 4, "stridedsync": 5,
}
ACTS = {"gelu_erf": 0, "gelu": 0, "gelu_tanh": 1, "none": 2, "relu": 3}
ORDERS = {"xcd": 0, "auto": 0, "row_major": 1, "producer_first": 1, "interleaved": 2,
          "col_major": 3, "strided": 4}
DTYPES = {"f16": 0, "bf16": 1}


class ChainError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        msg = _strerror(status)
        super().__init__("%s: %s (status %d)" % (what or "tlsync", msg, status))


class chain_mlp_args(ctypes.Structure):
    _fields_ = [
        ("X", ctypes.c_void_p), ("W1", ctypes.c_void_p), ("W2", ctypes.c_void_p),
        ("Y", ctypes.c_void_p),
        ("M", ctypes.c_int64), ("H", ctypes.c_int64), ("F", ctypes.c_int64),
        ("policy", ctypes.c_int32), ("dtype", ctypes.c_int32), ("act", ctypes.c_int32),
        ("tile_cfg", ctypes.c_int32),
        ("stream", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("z_out", ctypes.c_void_p), ("z_debug_f32", ctypes.c_void_p),
        ("order_seed", ctypes.c_uint64), ("order", ctypes.c_int32), ("grid", ctypes.c_int32),
        ("poll_limit", ctypes.c_uint32), ("debug_skip_producer", ctypes.c_int32),
        ("debug_delay", ctypes.c_uint32), ("split_k1", ctypes.c_int32),
        ("split_k2", ctypes.c_int32),
        ("z_ring", ctypes.c_void_p), ("ring_slots", ctypes.c_int32),
        ("ring_index", ctypes.c_uint32),
        ("trace", ctypes.c_void_p), ("trace_capacity", ctypes.c_uint32),
        ("order_stride", ctypes.c_int32),
    ]


class chain_trace_rec(ctypes.Structure):
    _fields_ = [("item", ctypes.c_uint32), ("wg", ctypes.c_uint16), ("hw", ctypes.c_uint16),
                ("t_start", ctypes.c_uint64), ("t_ready", ctypes.c_uint64),
                ("t_end", ctypes.c_uint64)]


class chain_conv_args(ctypes.Structure):
    _fields_ = [
        ("X", ctypes.c_void_p), ("Wa", ctypes.c_void_p), ("Wb", ctypes.c_void_p),
        ("Y", ctypes.c_void_p),
        ("N", ctypes.c_int32), ("Hh", ctypes.c_int32), ("Ww", ctypes.c_int32),
        ("C", ctypes.c_int32), ("K", ctypes.c_int32), ("R", ctypes.c_int32),
        ("S", ctypes.c_int32), ("pad", ctypes.c_int32), ("stride", ctypes.c_int32),
        ("policy", ctypes.c_int32), ("dtype", ctypes.c_int32), ("act", ctypes.c_int32),
        ("tile_cfg", ctypes.c_int32),
        ("stream", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t), ("z_out", ctypes.c_void_p),
        ("z_debug_f32", ctypes.c_void_p),
        ("order_seed", ctypes.c_uint64), ("order", ctypes.c_int32), ("grid", ctypes.c_int32),
        ("poll_limit", ctypes.c_uint32), ("debug_skip_producer", ctypes.c_int32),
        ("debug_delay", ctypes.c_uint32), ("split_k1", ctypes.c_int32),
        ("split_k2", ctypes.c_int32),
        ("z_ring", ctypes.c_void_p), ("ring_slots", ctypes.c_int32),
        ("ring_index", ctypes.c_uint32),
        ("trace", ctypes.c_void_p), ("trace_capacity", ctypes.c_uint32),
        ("order_stride", ctypes.c_int32), ("debug_first_skip", ctypes.c_int32),
    ]


class chain_attn_args(ctypes.Structure):
    _fields_ = [
        ("Q", ctypes.c_void_p), ("K", ctypes.c_void_p), ("V", ctypes.c_void_p),
        ("O", ctypes.c_void_p),
        ("B", ctypes.c_int32), ("heads", ctypes.c_int32), ("S", ctypes.c_int32),
        ("d", ctypes.c_int32), ("scale", ctypes.c_float),
        ("policy", ctypes.c_int32), ("dtype", ctypes.c_int32), ("tile_cfg", ctypes.c_int32),
        ("stream", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t), ("s_out", ctypes.c_void_p),
        ("order_seed", ctypes.c_uint64), ("order", ctypes.c_int32), ("grid", ctypes.c_int32),
        ("poll_limit", ctypes.c_uint32), ("debug_skip_producer", ctypes.c_int32),
        ("debug_delay", ctypes.c_uint32), ("ring_slots", ctypes.c_int32),
        ("ring_index", ctypes.c_uint32), ("s_ring", ctypes.c_void_p),
        ("trace", ctypes.c_void_p), ("trace_capacity", ctypes.c_uint32),
        ("order_stride", ctypes.c_int32), ("debug_first_skip", ctypes.c_int32),
    ]


class chain_selfattn_args(ctypes.Structure):
    _fields_ = [
        ("X", ctypes.c_void_p), ("Wqkv", ctypes.c_void_p), ("W2", ctypes.c_void_p),
        ("Y", ctypes.c_void_p),
        ("M", ctypes.c_int64), ("H", ctypes.c_int64),
        ("heads", ctypes.c_int32), ("d", ctypes.c_int32), ("scale", ctypes.c_float),
        ("policy", ctypes.c_int32), ("dtype", ctypes.c_int32), ("split_k1", ctypes.c_int32),
        ("stream", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t), ("qkv_out", ctypes.c_void_p),
        ("dot_out", ctypes.c_void_p),
        ("order_seed", ctypes.c_uint64), ("order", ctypes.c_int32), ("grid", ctypes.c_int32),
        ("poll_limit", ctypes.c_uint32), ("debug_skip_producer", ctypes.c_int32),
        ("debug_delay", ctypes.c_uint32), ("split_keys", ctypes.c_int32),
        ("trace", ctypes.c_void_p), ("trace_capacity", ctypes.c_uint32),
    ]


class chain_tile_info(ctypes.Structure):
    _fields_ = [("bm", ctypes.c_int32), ("bn1", ctypes.c_int32), ("bn2", ctypes.c_int32),
                ("bk", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32)]


class chain_plan(ctypes.Structure):
    _fields_ = [("tile_cfg", ctypes.c_int32), ("row_tiles", ctypes.c_int64),
                ("prod_col_tiles", ctypes.c_int64), ("cons_col_tiles", ctypes.c_int64),
                ("producer_tiles", ctypes.c_int64), ("consumer_tiles", ctypes.c_int64),
                ("split_k1", ctypes.c_int32), ("split_k2", ctypes.c_int32)]


class chain_selfattn_plan_info(ctypes.Structure):
    _fields_ = [("row_tile", ctypes.c_int32), ("col_tile", ctypes.c_int32),
                ("row_tiles", ctypes.c_int64), ("stage1_tiles", ctypes.c_int64),
                ("split_k1", ctypes.c_int32), ("split_keys", ctypes.c_int32),
                ("query_blocks", ctypes.c_int64), ("key_blocks", ctypes.c_int64),
                ("stage1_items", ctypes.c_int64), ("stage2_items", ctypes.c_int64),
                ("stage3_items", ctypes.c_int64), ("tail_tiles", ctypes.c_int64),
                ("split_k_tail", ctypes.c_int32), ("reserved", ctypes.c_int32)]


# Exported symbols and their C signatures (include/tlsync.h).
_I, _P, _I64, _SZ = ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "chain_mlp": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _I]),
    "chain_mlp_ex": (_I, [ctypes.POINTER(chain_mlp_args)]),
    "chain_mlp_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I, _I, _I]),
    "chain_conv": (_I, [_P, _P, _P, _P] + [_I] * 10),
    "chain_conv_ex": (_I, [ctypes.POINTER(chain_conv_args)]),
    "chain_conv_workspace_bytes": (_SZ, [_I] * 12),
    "chain_attn": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_float, _I]),
    "chain_attn_ex": (_I, [ctypes.POINTER(chain_attn_args)]),
    "chain_attn_workspace_bytes": (_SZ, [_I] * 7),
    "chain_selfattn": (_I, [_P, _P, _P, _P, _I64, _I64, _I, _I, ctypes.c_float, _I]),
    "chain_selfattn_ex": (_I, [ctypes.POINTER(chain_selfattn_args)]),
    "chain_selfattn_workspace_bytes": (_SZ, [_I64, _I64, _I, _I, _I, _I]),
    "chain_workspace_reset": (_I, [_P, _SZ, _P]),
    "chain_trace_clock_khz": (_I, [ctypes.POINTER(_I)]),
    "chain_workspace_status": (_I, [_P, _P]),
    "chain_sync": (_I, [_P]),
    "chain_release": (None, []),
    "chain_strerror": (ctypes.c_char_p, [_I]),
    "chain_last_hip_error": (_I, []),
    "chain_last_timeout": (_I, [ctypes.POINTER(_I64), ctypes.POINTER(_I)]),
    "chain_num_tile_cfgs": (_I, []),
    "chain_tile_cfg_info": (_I, [_I, ctypes.POINTER(chain_tile_info)]),
    "chain_mlp_plan": (_I, [_I64, _I64, _I64, _I, _I, ctypes.POINTER(chain_plan)]),
    "chain_conv_plan": (_I, [_I, _I, _I, _I, _I, _I, ctypes.POINTER(chain_plan)]),
    "chain_selfattn_plan": (_I, [_I64, _I64, _I, _I, _I, _I,
                                 ctypes.POINTER(chain_selfattn_plan_info)]),
    "chain_mlp_order": (_I, [ctypes.POINTER(chain_mlp_args), ctypes.POINTER(ctypes.c_uint32), _SZ,
                             ctypes.POINTER(_SZ)]),
    "chain_conv_order": (_I, [ctypes.POINTER(chain_conv_args), ctypes.POINTER(ctypes.c_uint32),
                              _SZ, ctypes.POINTER(_SZ)]),
    "chain_attn_order": (_I, [ctypes.POINTER(chain_attn_args), ctypes.POINTER(ctypes.c_uint32),
                              _SZ, ctypes.POINTER(_SZ)]),
    "chain_mlp_noalloc": (_I, [ctypes.POINTER(chain_mlp_args)]),
    "chain_calibrate_copy": (_I, [_P, _P, _SZ, _P]),
    "chain_calibrate_mfma": (_I, [_I, _I, _P, _SZ, _P, ctypes.POINTER(ctypes.c_double),
                                  ctypes.POINTER(ctypes.c_double),
                                  ctypes.POINTER(ctypes.c_double)]),
    "chain_noalloc_status": (_I, [_P]),
    "chain_wave_model": (_I, [ctypes.POINTER(_I64), _I, _I64, ctypes.POINTER(ctypes.c_double),
                              ctypes.POINTER(_I64), ctypes.POINTER(ctypes.c_double)]),
    "chain_conv_dep_range": (_I, [_I64, _I64, _I64, _I64, _I64, _I, _I, _I,
                                  ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
}

_lib = None


def load():
    """Load libtlsync.so (raises ImportError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                "libtlsync.so is not built (%s); run `python -m tile_level_sync_amd.build`"
                % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _strerror(status):
    try:
        return load().chain_strerror(status).decode()
    except ImportError:
        return "status %d" % status


def _check(status, what):
    if status != CHAIN_OK:
        raise ChainError(status, what)


# ---------------------------------------------------------------------------
# torch plumbing
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream_handle(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t, name, dtype=None, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return ctypes.c_void_p(t.data_ptr())


def _opt_ptr(t, name, dtype, shape):
    return None if t is None else _ptr(t, name, dtype, shape)


def _policy(p):
    return POLICIES[p] if isinstance(p, str) else int(p)


# ---------------------------------------------------------------------------
# MLP chain
# ---------------------------------------------------------------------------
class SentinelRing:
    """Ring of intermediate buffers for the sentinel policy (sentinel guide,
    4.6.4.5 Buffer Reuse).  The call with sequence number i consumes slot
    i % slots and, in the same launch, sets slot (i + 1) % slots back to the
    sentinel, so no fill kernel runs before the next call.  One ring serves
    one chain shape on one stream; every call through it advances ``index``.
    The intermediate is seen as [rows, cols]: [M, F] for the MLP chain,
    [N*H*W, K] for the conv pair, [B*heads*S, S] (the scores) for attention.
    ``slot(i)`` is the intermediate of call i, valid until call i + slots - 1
    is enqueued."""

    def __init__(self, rows, cols, slots=2, device="cuda"):
        if not 2 <= int(slots) <= 16:
            raise ValueError("a sentinel ring has 2..16 slots")
        torch = _torch()
        self.rows, self.cols, self.slots = int(rows), int(cols), int(slots)
        self.buf = torch.empty((self.slots, self.rows, self.cols), dtype=torch.float16,
                               device=device)
        self.index = 0

    def slot(self, i):
        return self.buf[i % self.slots]

    def _fill_args(self, a, rows, cols, field="z_ring"):
        if (rows, cols) != (self.rows, self.cols):
            raise ValueError("ring holds [%d, %d] intermediates, the call needs [%d, %d]"
                             % (self.rows, self.cols, rows, cols))
        setattr(a, field, self.buf.data_ptr())
        a.ring_slots = self.slots
        a.ring_index = self.index & 0xFFFFFFFF

    def _advance(self):
        self.index = (self.index + 1) & 0xFFFFFFFF


def chain_mlp(X, W1, W2, Y=None, policy="tilesync", *, act="gelu_erf", tile_cfg=None,
              stream=None, workspace=None, z_out=None, z_debug=None, order="xcd",
              order_seed=0, grid=0, poll_limit=0, debug_skip_producer=None, debug_delay=0,
              split_k=(0, 0), ring=None, trace=None, check=False, order_stride=0,
              noalloc=False):
    """Y = act(X W1) W2 via chain_mlp_ex.  X:[M,H], W1:[H,F], W2:[F,H], all fp16
    or all bf16 (the element type follows X).

    ``noalloc=True`` calls chain_mlp_noalloc instead: the workspace is the
    library's static device array (no ``workspace`` argument, no seeded or
    table orders), and ``check`` reads that array's status.

    ``tile_cfg`` None = automatic, else an index of ``tile_configs()``.
    ``split_k`` = (producer, consumer) K splits: 0 automatic, 1 none.
    ``workspace`` is an optional uint8 device tensor (caller-owned).
    ``ring`` is a ``SentinelRing`` of [M, F] slots (sentinel policy only).
    ``trace`` is an optional uint8 device tensor of at least 32 bytes per work
    item (``trace_buffer``) that receives one record per item.
    ``check=True`` synchronises and raises ChainError on a device timeout.
    """
    torch = _torch()
    lib = load()
    M, H = X.shape
    F = W1.shape[1]
    # fp16, or bf16 when X is bf16 (every tensor must then be bf16)
    dt = torch.bfloat16 if X.dtype == torch.bfloat16 else torch.float16
    if Y is None:
        Y = torch.empty((M, H), dtype=dt, device=X.device)
    a = chain_mlp_args()
    a.X = _ptr(X, "X", dt, (M, H))
    a.W1 = _ptr(W1, "W1", dt, (H, F))
    a.W2 = _ptr(W2, "W2", dt, (F, H))
    a.Y = _ptr(Y, "Y", dt, (M, H))
    a.M, a.H, a.F = M, H, F
    a.policy = _policy(policy)
    a.dtype = DTYPES["bf16"] if dt == torch.bfloat16 else DTYPES["f16"]
    a.act = ACTS[act] if isinstance(act, str) else int(act)
    a.tile_cfg = 0 if tile_cfg is None else int(tile_cfg) + 1
    a.stream = _stream_handle(stream)
    if workspace is not None:
        a.workspace = _ptr(workspace, "workspace", torch.uint8)
        a.workspace_bytes = workspace.numel()
    a.z_out = _opt_ptr(z_out, "z_out", dt, (M, F))
    a.z_debug_f32 = _opt_ptr(z_debug, "z_debug", torch.float32, (M, F))
    a.order_seed = int(order_seed)
    a.order = ORDERS[order] if isinstance(order, str) else int(order)
    a.order_stride = int(order_stride)
    a.grid = int(grid)
    a.poll_limit = int(poll_limit)
    a.debug_skip_producer = 0 if debug_skip_producer is None else int(debug_skip_producer) + 1
    a.debug_delay = int(debug_delay)
    a.split_k1, a.split_k2 = int(split_k[0]), int(split_k[1])
    if ring is not None:
        ring._fill_args(a, M, F)
    if trace is not None:
        a.trace = _ptr(trace, "trace", torch.uint8)
        a.trace_capacity = trace.numel() // ctypes.sizeof(chain_trace_rec)
    if noalloc:
        _check(lib.chain_mlp_noalloc(ctypes.byref(a)), "chain_mlp_noalloc")
    else:
        _check(lib.chain_mlp_ex(ctypes.byref(a)), "chain_mlp")
    if ring is not None:
        ring._advance()
    if check:
        if noalloc:
            _check(lib.chain_noalloc_status(_stream_handle(stream)), "chain_mlp_noalloc (device)")
        else:
            _check(chain_sync_status(stream, workspace), "chain_mlp (device)")
    return Y


# ---------------------------------------------------------------------------
# conv pair
# ---------------------------------------------------------------------------
def chain_conv(X, Wa, Wb, Y=None, policy="conv2d_tilesync", *, pad=1, stride=1, act="relu",
               tile_cfg=None, stream=None, workspace=None, z_out=None, z_debug=None,
               order="xcd", order_seed=0, grid=0, poll_limit=0, debug_skip_producer=None,
               debug_delay=0, split_k=(0, 0), ring=None, trace=None, check=False,
               order_stride=0, debug_first_skip=False):
    """Y = conv(act(conv(X, Wa)), Wb) via chain_conv_ex.  X:[N,H,W,C] NHWC,
    Wa:[R,S,C,K], Wb:[R,S,K,K], Y:[N,H,W,K] ("same" convolutions), all fp16
    or all bf16 (bf16 when X is).
    ``ring`` is a ``SentinelRing`` of [N*H*W, K] slots (sentinel policy only);
    ``trace`` a ``trace_buffer`` of at least ``conv_work_items`` records."""
    torch = _torch()
    lib = load()
    N, Hh, Ww, C = X.shape
    R, S, C2, K = Wa.shape
    if C2 != C or tuple(Wb.shape) != (R, S, K, K):
        raise ValueError("filter shapes do not match")
    # fp16, or bf16 when X is bf16 (every tensor must then be bf16)
    dt = torch.bfloat16 if X.dtype == torch.bfloat16 else torch.float16
    if Y is None:
        Y = torch.empty((N, Hh, Ww, K), dtype=dt, device=X.device)
    a = chain_conv_args()
    a.X = _ptr(X, "X", dt, (N, Hh, Ww, C))
    a.Wa = _ptr(Wa, "Wa", dt, (R, S, C, K))
    a.Wb = _ptr(Wb, "Wb", dt, (R, S, K, K))
    a.Y = _ptr(Y, "Y", dt, (N, Hh, Ww, K))
    a.N, a.Hh, a.Ww, a.C, a.K, a.R, a.S = N, Hh, Ww, C, K, R, S
    a.pad, a.stride = pad, stride
    a.policy = _policy(policy)
    a.dtype = DTYPES["bf16"] if dt == torch.bfloat16 else DTYPES["f16"]
    a.act = ACTS[act] if isinstance(act, str) else int(act)
    a.tile_cfg = 0 if tile_cfg is None else int(tile_cfg) + 1
    a.stream = _stream_handle(stream)
    if workspace is not None:
        a.workspace = _ptr(workspace, "workspace", torch.uint8)
        a.workspace_bytes = workspace.numel()
    a.z_out = _opt_ptr(z_out, "z_out", dt, (N, Hh, Ww, K))
    a.z_debug_f32 = _opt_ptr(z_debug, "z_debug", torch.float32, (N, Hh, Ww, K))
    a.order_seed = int(order_seed)
    a.order = ORDERS[order] if isinstance(order, str) else int(order)
    a.order_stride = int(order_stride)
    a.debug_first_skip = 1 if debug_first_skip else 0
    a.grid = int(grid)
    a.poll_limit = int(poll_limit)
    a.debug_skip_producer = 0 if debug_skip_producer is None else int(debug_skip_producer) + 1
    a.debug_delay = int(debug_delay)
    a.split_k1, a.split_k2 = int(split_k[0]), int(split_k[1])
    if ring is not None:
        ring._fill_args(a, N * Hh * Ww, K)
    if trace is not None:
        a.trace = _ptr(trace, "trace", torch.uint8)
        a.trace_capacity = trace.numel() // ctypes.sizeof(chain_trace_rec)
    _check(lib.chain_conv_ex(ctypes.byref(a)), "chain_conv")
    if ring is not None:
        ring._advance()
    if check:
        _check(chain_sync_status(stream, workspace), "chain_conv (device)")
    return Y


# ---------------------------------------------------------------------------
# attention chain
# ---------------------------------------------------------------------------
def chain_attn(Q, K, V, O=None, policy="rowsync", *, scale=1.0, stream=None, workspace=None,
               s_out=None, order="xcd", order_seed=0, grid=0, poll_limit=0,
               debug_skip_producer=None, debug_delay=0, ring=None, trace=None, check=False,
               order_stride=0, debug_first_skip=False):
    """O = softmax_rows(fp16(scale Q K^T)) V per (batch, head) via chain_attn_ex.
    Q, K, V: [B, heads, S, d] contiguous, all fp16 or all bf16 (bf16 when Q is:
    the scores and O are then bf16 too).  ``s_out`` optionally receives the
    scores [B, heads, S, S].  ``ring`` is a ``SentinelRing`` of
    [B*heads*S, S] score slots (sentinel policy only); ``trace`` a
    ``trace_buffer`` of at least ``attn_work_items`` records."""
    torch = _torch()
    lib = load()
    B, Hh, S, d = Q.shape
    # fp16, or bf16 when Q is bf16 (every tensor must then be bf16)
    dt = torch.bfloat16 if Q.dtype == torch.bfloat16 else torch.float16
    if O is None:
        O = torch.empty((B, Hh, S, d), dtype=dt, device=Q.device)
    a = chain_attn_args()
    a.Q = _ptr(Q, "Q", dt, (B, Hh, S, d))
    a.K = _ptr(K, "K", dt, (B, Hh, S, d))
    a.V = _ptr(V, "V", dt, (B, Hh, S, d))
    a.O = _ptr(O, "O", dt, (B, Hh, S, d))
    a.B, a.heads, a.S, a.d = B, Hh, S, d
    a.scale = float(scale)
    a.policy = _policy(policy)
    a.dtype = DTYPES["bf16"] if dt == torch.bfloat16 else DTYPES["f16"]
    a.stream = _stream_handle(stream)
    if workspace is not None:
        a.workspace = _ptr(workspace, "workspace", torch.uint8)
        a.workspace_bytes = workspace.numel()
    a.s_out = _opt_ptr(s_out, "s_out", dt, (B, Hh, S, S))
    a.order_seed = int(order_seed)
    a.order = ORDERS[order] if isinstance(order, str) else int(order)
    a.order_stride = int(order_stride)
    a.debug_first_skip = 1 if debug_first_skip else 0
    a.grid = int(grid)
    a.poll_limit = int(poll_limit)
    a.debug_skip_producer = 0 if debug_skip_producer is None else int(debug_skip_producer) + 1
    a.debug_delay = int(debug_delay)
    if ring is not None:
        ring._fill_args(a, B * Hh * S, S, field="s_ring")
    if trace is not None:
        a.trace = _ptr(trace, "trace", torch.uint8)
        a.trace_capacity = trace.numel() // ctypes.sizeof(chain_trace_rec)
    _check(lib.chain_attn_ex(ctypes.byref(a)), "chain_attn")
    if ring is not None:
        ring._advance()
    if check:
        _check(chain_sync_status(stream, workspace), "chain_attn (device)")
    return O


def chain_attn_workspace_bytes(B, heads, S, d, policy="rowsync"):
    return load().chain_attn_workspace_bytes(B, heads, S, d, _policy(policy), 0, -1)


# ---------------------------------------------------------------------------
# self-attention chain
# ---------------------------------------------------------------------------
def chain_selfattn(X, Wqkv, W2, Y=None, policy="stridedsync", *, heads, scale=None,
                   stream=None, workspace=None, qkv_out=None, dot_out=None, order="xcd",
                   order_seed=0, grid=0, poll_limit=0, debug_skip_producer=None, debug_delay=0,
                   split_k=0, split_keys=0, trace=None, check=False):
    """Y = XDot W2 with XDot[:, head h] = softmax(scale Q_h S2_h^T) S3_h and
    [Q | S2 | S3] = X Wqkv, via chain_selfattn_ex.  X:[M,H], Wqkv:[H,3*heads*d],
    W2:[heads*d,H], all fp16 or all bf16 (bf16 when X is).  ``scale`` defaults to 1/sqrt(d).  ``split_k`` = K splits
    of a stage-1 tile, ``split_keys`` = key splits of a stage-2 item: 0
    automatic, 1 none.  ``trace`` is a ``trace_buffer`` of at least
    ``selfattn_work_items`` records."""
    torch = _torch()
    lib = load()
    M, H = X.shape
    Hs3 = Wqkv.shape[1]
    d = Hs3 // (3 * heads)
    Hs = heads * d
    # fp16, or bf16 when X is bf16 (every tensor must then be bf16)
    dt = torch.bfloat16 if X.dtype == torch.bfloat16 else torch.float16
    if Y is None:
        Y = torch.empty((M, H), dtype=dt, device=X.device)
    a = chain_selfattn_args()
    a.X = _ptr(X, "X", dt, (M, H))
    a.Wqkv = _ptr(Wqkv, "Wqkv", dt, (H, 3 * Hs))
    a.W2 = _ptr(W2, "W2", dt, (Hs, H))
    a.Y = _ptr(Y, "Y", dt, (M, H))
    a.M, a.H, a.heads, a.d = M, H, heads, d
    a.scale = float(scale if scale is not None else 1.0 / d ** 0.5)
    a.policy = _policy(policy)
    a.dtype = DTYPES["bf16"] if dt == torch.bfloat16 else DTYPES["f16"]
    a.stream = _stream_handle(stream)
    if workspace is not None:
        a.workspace = _ptr(workspace, "workspace", torch.uint8)
        a.workspace_bytes = workspace.numel()
    a.split_k1 = int(split_k)
    a.split_keys = int(split_keys)
    a.qkv_out = _opt_ptr(qkv_out, "qkv_out", dt, (M, 3 * Hs))
    a.dot_out = _opt_ptr(dot_out, "dot_out", dt, (M, Hs))
    a.order_seed = int(order_seed)
    a.order = ORDERS[order] if isinstance(order, str) else int(order)
    a.grid = int(grid)
    a.poll_limit = int(poll_limit)
    a.debug_skip_producer = 0 if debug_skip_producer is None else int(debug_skip_producer) + 1
    a.debug_delay = int(debug_delay)
    if trace is not None:
        a.trace = _ptr(trace, "trace", torch.uint8)
        a.trace_capacity = trace.numel() // ctypes.sizeof(chain_trace_rec)
    _check(lib.chain_selfattn_ex(ctypes.byref(a)), "chain_selfattn")
    if check:
        _check(chain_sync_status(stream, workspace), "chain_selfattn (device)")
    return Y


def chain_selfattn_workspace_bytes(M, H, heads, d=128, policy="stridedsync"):
    return load().chain_selfattn_workspace_bytes(M, H, heads, d, _policy(policy), 0)


def chain_conv_workspace_bytes(N, Hh, Ww, C, K, R=3, S=3, pad=1, stride=1,
                               policy="conv2d_tilesync", tile_cfg=None):
    return load().chain_conv_workspace_bytes(N, Hh, Ww, C, K, R, S, pad, stride, _policy(policy),
                                             0, -1 if tile_cfg is None else int(tile_cfg))


def chain_mlp_workspace_bytes(M, H, F, policy="tilesync", tile_cfg=None):
    return load().chain_mlp_workspace_bytes(M, H, F, _policy(policy), 0,
                                            -1 if tile_cfg is None else int(tile_cfg))


def chain_mlp_plan(M, H, F, tile_cfg=None):
    p = chain_plan()
    _check(load().chain_mlp_plan(M, H, F, 0, -1 if tile_cfg is None else int(tile_cfg),
                                 ctypes.byref(p)), "chain_mlp_plan")
    return {k: getattr(p, k) for k, _ in chain_plan._fields_}


def chain_conv_plan(N, Hh, Ww, C, K, tile_cfg=None):
    """Tile configuration, tile counts and K splits of a conv pair call (no
    GPU needed)."""
    p = chain_plan()
    _check(load().chain_conv_plan(N, Hh, Ww, C, K, -1 if tile_cfg is None else int(tile_cfg),
                                  ctypes.byref(p)), "chain_conv_plan")
    return {k: getattr(p, k) for k, _ in chain_plan._fields_}


def chain_selfattn_plan(M, H, heads, d=128, split_k=0, split_keys=0):
    """Tiles, splits and work items of a self-attention call (no GPU needed)."""
    p = chain_selfattn_plan_info()
    _check(load().chain_selfattn_plan(M, H, heads, d, int(split_k), int(split_keys),
                                      ctypes.byref(p)), "chain_selfattn_plan")
    return {k: getattr(p, k) for k, _ in chain_selfattn_plan_info._fields_}


_DUMMY = 1 << 16  # aligned stand-in address: the order calls never touch memory


def _order_call(name, a):
    lib = load()
    n = ctypes.c_size_t(0)
    _check(getattr(lib, name)(ctypes.byref(a), None, 0, ctypes.byref(n)), name)
    buf = (ctypes.c_uint32 * max(1, n.value))()
    _check(getattr(lib, name)(ctypes.byref(a), buf, n.value, ctypes.byref(n)), name)
    return list(buf[:n.value])


def mlp_order(M, H, F, policy="tilesync", order="xcd", order_seed=0, order_stride=0,
              tile_cfg=None, split_k=(0, 0)):
    """Work items of an MLP call in the order the workgroups take them
    (chain_mlp_order; no GPU needed)."""
    a = chain_mlp_args()
    a.X = a.W1 = a.W2 = a.Y = _DUMMY
    a.M, a.H, a.F = M, H, F
    a.policy = _policy(policy)
    a.tile_cfg = 0 if tile_cfg is None else int(tile_cfg) + 1
    a.order = ORDERS[order] if isinstance(order, str) else int(order)
    a.order_seed, a.order_stride = int(order_seed), int(order_stride)
    a.split_k1, a.split_k2 = int(split_k[0]), int(split_k[1])
    return _order_call("chain_mlp_order", a)


def conv_order(N, Hh, Ww, C, K, policy="conv2d_tilesync", order="xcd", order_seed=0,
               order_stride=0, tile_cfg=None, split_k=(0, 0)):
    """Work items of a 3x3 conv pair call (pad 1, stride 1) in the order the
    workgroups take them (chain_conv_order; no GPU needed)."""
    a = chain_conv_args()
    a.X = a.Wa = a.Wb = a.Y = _DUMMY
    a.N, a.Hh, a.Ww, a.C, a.K, a.R, a.S, a.pad, a.stride = N, Hh, Ww, C, K, 3, 3, 1, 1
    a.policy = _policy(policy)
    a.tile_cfg = 0 if tile_cfg is None else int(tile_cfg) + 1
    a.order = ORDERS[order] if isinstance(order, str) else int(order)
    a.order_seed, a.order_stride = int(order_seed), int(order_stride)
    a.split_k1, a.split_k2 = int(split_k[0]), int(split_k[1])
    return _order_call("chain_conv_order", a)


def attn_order(B, heads, S, policy="rowsync", order="xcd", order_seed=0, order_stride=0):
    """Work items of an attention call in the order the workgroups take them
    (chain_attn_order; no GPU needed)."""
    a = chain_attn_args()
    a.Q = a.K = a.V = a.O = _DUMMY
    a.B, a.heads, a.S, a.d = B, heads, S, 128
    a.policy = _policy(policy)
    a.order = ORDERS[order] if isinstance(order, str) else int(order)
    a.order_seed, a.order_stride = int(order_seed), int(order_stride)
    return _order_call("chain_attn_order", a)


def calibrate_mfma(waves_per_simd=2, iters=20000, device="cuda"):
    """Sustained dense fp16 MFMA rate of the device (chain_calibrate_mfma):
    returns {"tflops", "ghz", "ms"}."""
    torch = _torch()
    cus = torch.cuda.get_device_properties(device).multi_processor_count
    buf = torch.empty(cus * waves_per_simd * 1280, dtype=torch.uint8, device=device)
    tf, gh, ms = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _check(load().chain_calibrate_mfma(int(waves_per_simd), int(iters), _ptr(buf, "scratch"),
                                       buf.numel(), _stream_handle(None), ctypes.byref(tf),
                                       ctypes.byref(gh), ctypes.byref(ms)), "chain_calibrate_mfma")
    return {"tflops": tf.value, "ghz": gh.value, "ms": ms.value}


def calibrate_copy(src, dst, stream=None):
    """Copy uint8 device tensor src to dst with the library's calibration
    kernel (16-byte buffer loads and stores; chain_calibrate_copy)."""
    torch = _torch()
    if src.numel() != dst.numel():
        raise ValueError("src and dst differ in size")
    _check(load().chain_calibrate_copy(_ptr(src, "src", torch.uint8), _ptr(dst, "dst", torch.uint8),
                                       src.numel(), _stream_handle(stream)), "chain_calibrate_copy")


def trace_clock_khz():
    """Rate of the trace clock (the GPU's constant-rate realtime counter)."""
    khz = ctypes.c_int(0)
    _check(load().chain_trace_clock_khz(ctypes.byref(khz)), "chain_trace_clock_khz")
    return khz.value


def mlp_work_items(M, H, F, tile_cfg=None):
    """Work items of one MLP call (producer tiles x splits + consumer tiles x splits)."""
    p = chain_mlp_plan(M, H, F, tile_cfg=tile_cfg)
    return p["producer_tiles"] * p["split_k1"] + p["consumer_tiles"] * p["split_k2"]


def conv_work_items(N, Hh, Ww, C, K, tile_cfg=None):
    """Work items of one conv pair call (producer tiles x splits + consumer tiles x splits)."""
    p = chain_conv_plan(N, Hh, Ww, C, K, tile_cfg=tile_cfg)
    return p["producer_tiles"] * p["split_k1"] + p["consumer_tiles"] * p["split_k2"]


def attn_work_items(B, heads, S):
    """Work items of one attention chain call: a producer and a consumer item
    per block of 128 score rows."""
    return 2 * (B * heads * S // 128)


def selfattn_work_items(M, H, heads, d=128, split_k=0, split_keys=0):
    """Work items of one self-attention call (stage 1, 2 and 3 items)."""
    p = chain_selfattn_plan(M, H, heads, d, split_k, split_keys)
    return p["stage1_items"] + p["stage2_items"] + p["stage3_items"]


def trace_buffer(items, device="cuda"):
    """A zeroed device buffer for ``items`` trace records."""
    return _torch().zeros(items * ctypes.sizeof(chain_trace_rec), dtype=_torch().uint8,
                          device=device)


def tile_configs():
    lib = load()
    out = []
    for i in range(lib.chain_num_tile_cfgs()):
        t = chain_tile_info()
        _check(lib.chain_tile_cfg_info(i, ctypes.byref(t)), "chain_tile_cfg_info")
        out.append({k: getattr(t, k) for k, _ in chain_tile_info._fields_})
    return out


# ---------------------------------------------------------------------------
# status / workspace
# ---------------------------------------------------------------------------
def chain_sync_status(stream=None, workspace=None):
    """Synchronise and return the device status code of the library-owned
    workspace, or of ``workspace`` if given."""
    lib = load()
    if workspace is not None:
        return lib.chain_workspace_status(_ptr(workspace, "workspace"), _stream_handle(stream))
    return lib.chain_sync(_stream_handle(stream))


def chain_sync(stream=None, workspace=None):
    _check(chain_sync_status(stream, workspace), "chain_sync")


def chain_workspace_reset(workspace, stream=None):
    _check(load().chain_workspace_reset(_ptr(workspace, "workspace"), workspace.numel(),
                                        _stream_handle(stream)), "chain_workspace_reset")


def chain_last_timeout():
    item = ctypes.c_int64()
    kind = ctypes.c_int()
    if load().chain_last_timeout(ctypes.byref(item), ctypes.byref(kind)) != CHAIN_OK:
        return None
    return item.value, kind.value


def chain_last_hip_error():
    return load().chain_last_hip_error()


def chain_release():
    load().chain_release()


# ---------------------------------------------------------------------------
# host planning helpers
# ---------------------------------------------------------------------------
def chain_wave_model(blocks, slots):
    """Wave model of the cuSync paper (section "Thread block Wave
    Execution"); returns (per-kernel fractional waves, serial waves, fused
    waves)."""
    n = len(blocks)
    arr = (ctypes.c_int64 * n)(*blocks)
    frac = (ctypes.c_double * n)()
    serial = ctypes.c_int64()
    fused = ctypes.c_double()
    _check(load().chain_wave_model(arr, n, slots, frac, ctypes.byref(serial),
                                   ctypes.byref(fused)), "chain_wave_model")
    return list(frac), serial.value, fused.value


def chain_conv_dep_range(tile, N, Hh, Ww, bm, R=3, S=3, pad=1):
    first = ctypes.c_int64()
    last = ctypes.c_int64()
    _check(load().chain_conv_dep_range(tile, N, Hh, Ww, bm, R, S, pad, ctypes.byref(first),
                                       ctypes.byref(last)), "chain_conv_dep_range")
    return first.value, last.value

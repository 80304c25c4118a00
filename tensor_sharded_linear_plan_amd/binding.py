"""ctypes binding of libtsl.so -- the entry points of include/tsl.h under the
same names, argument marshalling only.  Every step of the compute runs in
the library's HIP kernels; nothing here computes.

Pointer arguments take either an integer device address or any object with
a ``data_ptr()`` method (a torch tensor).  ``stream=None`` means the current
torch stream when torch has a GPU, else the null stream.  A non-OK status
raises TslError carrying the status code.

Importing this module loads libtsl.so; when it has not been built the
import fails with ImportError -- there is no fallback path.

PyTorch wheels for ROCm carry their own HIP runtime, which torch's libraries
load by a different file name than the system one.  Loading libtsl.so first
would bring in the system runtime next to torch's -- two runtimes in one
process, and launches fail.  torch is therefore imported (when installed)
before libtsl.so, whose dependency then resolves to the runtime already
loaded, so the library, torch's allocations and torch's streams share one
runtime.
"""
import ctypes
import os

try:  # see the module docstring: torch's HIP runtime must be loaded first
    import torch as _torch  # noqa: F401
except ImportError:
    _torch = None

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libtsl.so")

if not os.path.exists(LIBRARY):
    raise ImportError("libtsl.so is not built: run __graft_entry__.build() or "
                      "python tensor_sharded_linear_plan_amd/build.py")
_lib = ctypes.CDLL(LIBRARY)

# ---- enums (include/tsl.h) ----
OK = 0
ERR_INVALID_ARG, ERR_NOT_DIVISIBLE, ERR_TP_NOT_POW2, ERR_GROUP_ALIGN = -1, -2, -3, -4
ERR_BUFFER_TOO_SMALL, ERR_UNSUPPORTED, ERR_MISALIGNED, ERR_HIP = -5, -6, -7, -8

# bytes of the fixed device scratch behind shard_linear_group_noalloc
NOALLOC_SCRATCH_BYTES = 64 << 20
COLUMN, ROW, REPLICATED, EXPERT = 0, 1, 2, 3
MOE_EXPERT_PARALLEL, MOE_WITHIN_EXPERT = 0, 1
COMBINE_NONE, COMBINE_CONCAT, COMBINE_SUM = 0, 1, 2
Q, K, V, O, GATE, UP, DOWN = range(7)
NPROJ = 7
LINEAR = 7
EMBED, LM_HEAD = 8, 9
F32, BF16, Q4G64 = 0, 1, 2
ALL_REDUCE, REDUCE_SCATTER, ALL_GATHER = 0, 1, 2
MAX_PARTS = 64


class TslError(RuntimeError):
    def __init__(self, status, where=""):
        self.status = status
        msg = _lib.tsl_status_string(status).decode()
        if status == ERR_HIP:
            msg += " [%s]" % _lib.tsl_last_hip_error_string().decode()
        super().__init__("%s: %s (%d)" % (where, msg, status))


class Dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("tp_size", ctypes.c_int32),
                ("group_size", ctypes.c_int32)]


class Shard(ctypes.Structure):
    _fields_ = [("proj", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("strategy", ctypes.c_int32), ("combine", ctypes.c_int32),
                ("K", ctypes.c_int64), ("N", ctypes.c_int64),
                ("k_off", ctypes.c_int64), ("k_len", ctypes.c_int64),
                ("n_off", ctypes.c_int64), ("n_len", ctypes.c_int64),
                ("head_off", ctypes.c_int32), ("head_cnt", ctypes.c_int32)]

    FIELDS = ("proj", "rank", "strategy", "combine", "K", "N", "k_off", "k_len",
              "n_off", "n_len", "head_off", "head_cnt")

    def as_tuple(self):
        return tuple(int(getattr(self, f)) for f in self.FIELDS)

    def __repr__(self):
        return "Shard(%s)" % ", ".join("%s=%d" % (f, getattr(self, f)) for f in self.FIELDS)


class ExpertShard(ctypes.Structure):
    """The gate/up/down shards of one expert on one rank (tsl_expert_shard)."""
    _fields_ = [("expert", ctypes.c_int32), ("rank", ctypes.c_int32), ("gate", Shard),
                ("up", Shard), ("down", Shard)]


class LinearItem(ctypes.Structure):
    """One product of shard_linear_group (tsl_linear_item)."""
    _fields_ = [("shard", ctypes.POINTER(Shard)), ("packed", ctypes.c_void_p),
                ("packed_bytes", ctypes.c_size_t), ("X", ctypes.c_void_p),
                ("ldx", ctypes.c_int64), ("Y", ctypes.c_void_p), ("ldy", ctypes.c_int64),
                ("ydtype", ctypes.c_int32), ("accumulate", ctypes.c_int32),
                ("sum_next", ctypes.c_int32), ("rows", ctypes.c_int32),
                ("row_index", ctypes.c_void_p), ("x_rows", ctypes.c_int64)]


_i32, _i64, _vp, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
_P_SHARD = ctypes.POINTER(Shard)
_P_ITEM = ctypes.POINTER(LinearItem)
_lib.plan_shards.argtypes = [ctypes.POINTER(Dims), _P_SHARD, _i64]
_lib.plan_linear.argtypes = [_i64, _i64, _i32, _i32, _i32, _P_SHARD, _i64]
_lib.pack_shard_size.argtypes = [_P_SHARD, ctypes.c_int, ctypes.POINTER(_sz)]
_lib.pack_shard.argtypes = [_P_SHARD, ctypes.c_int, _vp, _i64, _i64, _vp, _vp, _i64, _i64, _vp,
                            _sz, _vp]
_lib.shard_linear_workspace_size.argtypes = [_P_SHARD, ctypes.c_int, _i64, ctypes.POINTER(_sz)]
_lib.shard_linear.argtypes = [_P_SHARD, ctypes.c_int, _vp, _sz, ctypes.c_int, _vp, _i64, _i64,
                              ctypes.c_int, _vp, _i64, ctypes.c_int, _vp, _sz, _vp]
_lib.shard_linear_group_workspace_size.argtypes = [_i32, _P_ITEM, ctypes.c_int, _i64,
                                                   ctypes.POINTER(_sz)]
_lib.shard_linear_group.argtypes = [_i32, _P_ITEM, ctypes.c_int, ctypes.c_int, _i64, _vp, _sz,
                                    _vp]
_lib.shard_linear_group_noalloc.argtypes = [_i32, _P_ITEM, ctypes.c_int, ctypes.c_int, _i64, _vp]
_lib.combine_partials.argtypes = [ctypes.c_int, _i32, ctypes.POINTER(_vp), ctypes.c_int, _i64,
                                  _i64, _i64, ctypes.c_int, _vp, _i64, _vp]
_lib.combine_to_ranks.argtypes = [ctypes.c_int, _i32, ctypes.POINTER(_vp), ctypes.c_int, _i64,
                                  _i64, _i64, ctypes.c_int, ctypes.POINTER(_vp), _i64, _vp]
_lib.plan_experts.argtypes = [_i32, _i64, _i64, _i32, _i32, _i32, ctypes.POINTER(ExpertShard),
                              _i64, ctypes.POINTER(_i64)]
_lib.moe_dispatch.argtypes = [_vp, _i64, _i32, _i32, _vp, _i32, _vp, _vp, _vp]
_lib.moe_gather.argtypes = [_vp, _i64, _i64, ctypes.c_int, _vp, _i64, _i64, _vp, _i64, _vp]
_lib.moe_combine.argtypes = [_vp, _i64, _i64, _vp, _vp, _i64, _i32, _i64, ctypes.c_int, _vp, _i64,
                             _vp]
_lib.plan_vocab.argtypes = [_i64, _i64, _i32, _i32, _P_SHARD, _i64]
_lib.embed_lookup.argtypes = [_P_SHARD, ctypes.c_int, _vp, _i64, _vp, _i64, ctypes.c_int, _vp,
                              _i64, _vp]
_lib.tsl_status_string.argtypes = [ctypes.c_int]
_lib.tsl_status_string.restype = ctypes.c_char_p
_lib.tsl_last_hip_error_string.argtypes = []
_lib.tsl_last_hip_error_string.restype = ctypes.c_char_p
for _f in ("plan_shards", "plan_linear", "pack_shard_size", "pack_shard",
           "shard_linear_workspace_size", "shard_linear", "shard_linear_group_workspace_size",
           "shard_linear_group", "shard_linear_group_noalloc", "combine_partials",
           "combine_to_ranks", "plan_vocab",
           "embed_lookup", "plan_experts", "moe_dispatch", "moe_gather", "moe_combine"):
    getattr(_lib, _f).restype = ctypes.c_int

EXPORTS = ("plan_shards", "plan_linear", "pack_shard_size", "pack_shard",
           "shard_linear_workspace_size", "shard_linear", "shard_linear_group_workspace_size",
           "shard_linear_group", "shard_linear_group_noalloc", "combine_partials",
           "combine_to_ranks", "plan_vocab",
           "embed_lookup", "plan_experts", "moe_dispatch", "moe_gather", "moe_combine",
           "tsl_status_string", "tsl_last_hip_error_string")


def _check(status, where):
    if status != OK:
        raise TslError(status, where)


def _ptr(x):
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return int(x)


def _stream(stream):
    if stream is not None:
        return getattr(stream, "cuda_stream", stream)
    if _torch is not None and _torch.cuda.is_available():
        return _torch.cuda.current_stream().cuda_stream
    return None


def tsl_status_string(status):
    return _lib.tsl_status_string(status).decode()


def tsl_last_hip_error_string():
    return _lib.tsl_last_hip_error_string().decode()


def plan_shards(hidden, n_q_heads, n_kv_heads, head_dim, ffn, tp_size, group_size=0):
    """Shards for every (rank, projection): a list indexed [rank * NPROJ + proj]."""
    d = Dims(hidden, n_q_heads, n_kv_heads, head_dim, ffn, tp_size, group_size)
    n = max(int(tp_size), 1) * NPROJ
    out = (Shard * n)()
    _check(_lib.plan_shards(ctypes.byref(d), out, n), "plan_shards")
    return list(out)


def plan_linear(K, N, tp_size, strategy, group_size=0):
    n = max(int(tp_size), 1)
    out = (Shard * n)()
    _check(_lib.plan_linear(K, N, tp_size, strategy, group_size, out, n), "plan_linear")
    return list(out)


def plan_vocab(vocab, hidden, tp_size, group_size=0):
    """[embedding shard, LM-head shard] of every rank: a list of 2*tp shards."""
    n = 2 * max(int(tp_size), 1)
    out = (Shard * n)()
    _check(_lib.plan_vocab(vocab, hidden, tp_size, group_size, out, n), "plan_vocab")
    return list(out)


def plan_experts(n_experts, hidden, expert_ffn, tp_size, mode, group_size=0):
    """Every rank's expert shards, rank-major: a list of ExpertShard."""
    n = n_experts * (max(int(tp_size), 1) if mode == MOE_WITHIN_EXPERT else 1)
    out = (ExpertShard * max(n, 1))()
    got = _i64(0)
    _check(_lib.plan_experts(n_experts, hidden, expert_ffn, tp_size, mode, group_size, out, n,
                             ctypes.byref(got)), "plan_experts")
    return list(out)[:got.value]


def moe_dispatch(topk, n_experts, experts):
    """Host routing -> (offsets int64 [n_local + 1], row_slot int32 [rows],
    slot_row int32 [T*k]); topk is an int32 array [T][k] (host)."""
    import numpy as np
    topk = np.ascontiguousarray(topk, dtype=np.int32)
    T, k = topk.shape
    ex = np.ascontiguousarray(experts, dtype=np.int32)
    offsets = np.zeros(len(ex) + 1, dtype=np.int64)
    row_slot = np.zeros(max(T * k, 1), dtype=np.int32)
    slot_row = np.zeros(max(T * k, 1), dtype=np.int32)
    _check(_lib.moe_dispatch(topk.ctypes.data, T, k, n_experts, ex.ctypes.data if len(ex) else None,
                             len(ex), offsets.ctypes.data, row_slot.ctypes.data,
                             slot_row.ctypes.data), "moe_dispatch")
    return offsets, row_slot[:offsets[-1]].copy(), slot_row[:T * k].copy()


def moe_gather(src, ld_src, n_src, dtype, idx, n, width, out, ldo, stream=None):
    _check(_lib.moe_gather(_ptr(src), ld_src, n_src, dtype, _ptr(idx), n, width, _ptr(out), ldo,
                           _stream(stream)), "moe_gather")


def moe_combine(P, ldp, n_rows, slot_row, weights, T, k, n, ydtype, Y, ldy, stream=None):
    _check(_lib.moe_combine(_ptr(P), ldp, n_rows, _ptr(slot_row), _ptr(weights), T, k, n, ydtype,
                            _ptr(Y), ldy, _stream(stream)), "moe_combine")


def embed_lookup(shard, tdtype, table, ld_table, tokens, M, ydtype, Y, ldy, stream=None):
    _check(_lib.embed_lookup(ctypes.byref(shard), tdtype, _ptr(table), ld_table, _ptr(tokens), M,
                             ydtype, _ptr(Y), ldy, _stream(stream)), "embed_lookup")


def pack_shard_size(shard, wdtype):
    b = _sz(0)
    _check(_lib.pack_shard_size(ctypes.byref(shard), wdtype, ctypes.byref(b)), "pack_shard_size")
    return b.value


def pack_shard(shard, wdtype, W, stride_k, stride_n, scales, biases, sb_stride_g, sb_stride_n,
               packed, packed_bytes, stream=None):
    _check(_lib.pack_shard(ctypes.byref(shard), wdtype, _ptr(W), stride_k, stride_n,
                           _ptr(scales), _ptr(biases), sb_stride_g, sb_stride_n, _ptr(packed),
                           packed_bytes, _stream(stream)), "pack_shard")


def shard_linear_workspace_size(shard, wdtype, M):
    b = _sz(0)
    _check(_lib.shard_linear_workspace_size(ctypes.byref(shard), wdtype, M, ctypes.byref(b)),
           "shard_linear_workspace_size")
    return b.value


def shard_linear(shard, wdtype, packed, packed_bytes, xdtype, X, ldx, M, ydtype, Y, ldy,
                 accumulate=0, workspace=None, ws_bytes=0, stream=None):
    _check(_lib.shard_linear(ctypes.byref(shard), wdtype, _ptr(packed), packed_bytes, xdtype,
                             _ptr(X), ldx, M, ydtype, _ptr(Y), ldy, accumulate, _ptr(workspace),
                             ws_bytes, _stream(stream)), "shard_linear")


def _items(items):
    """items: sequence of dicts (or LinearItem) with the tsl_linear_item
    fields (ydtype defaults to F32, accumulate, sum_next and rows to 0,
    row_index to None); shard is a Shard; a set member's Y may be None.
    Returns the ctypes array (which keeps the shard copies alive) and its
    length."""
    arr = (LinearItem * max(len(items), 1))()
    keep = []
    for i, it in enumerate(items):
        if isinstance(it, LinearItem):
            arr[i] = it
            continue
        sh = Shard(*it["shard"].as_tuple())
        keep.append(sh)
        arr[i] = LinearItem(ctypes.pointer(sh), _ptr(it["packed"]), it["packed_bytes"],
                            _ptr(it["X"]), it["ldx"], _ptr(it.get("Y")), it.get("ldy", 0),
                            it.get("ydtype", F32), it.get("accumulate", 0),
                            it.get("sum_next", 0), it.get("rows", 0),
                            _ptr(it.get("row_index")), it.get("x_rows", 0))
    arr._keep = keep
    return arr, len(items)


def shard_linear_group_workspace_size(items, wdtype, M):
    arr, n = _items(items)
    b = _sz(0)
    _check(_lib.shard_linear_group_workspace_size(n, arr, wdtype, M, ctypes.byref(b)),
           "shard_linear_group_workspace_size")
    return b.value


def shard_linear_group(items, wdtype, xdtype, M, workspace=None, ws_bytes=0, stream=None):
    arr, n = _items(items)
    _check(_lib.shard_linear_group(n, arr, wdtype, xdtype, M, _ptr(workspace), ws_bytes,
                                   _stream(stream)), "shard_linear_group")


def shard_linear_group_noalloc(items, wdtype, xdtype, M, stream=None):
    arr, n = _items(items)
    _check(_lib.shard_linear_group_noalloc(n, arr, wdtype, xdtype, M, _stream(stream)),
           "shard_linear_group_noalloc")


def combine_partials(mode, parts, pdtype, M, n_each, ld_part, ydtype, Y, ldy, stream=None):
    arr = (_vp * max(len(parts), 1))(*[_ptr(p) for p in parts])
    _check(_lib.combine_partials(mode, len(parts), arr, pdtype, M, n_each, ld_part, ydtype,
                                 _ptr(Y), ldy, _stream(stream)), "combine_partials")


def combine_to_ranks(op, parts, pdtype, M, n_each, ld_part, odtype, outs, ldo, stream=None):
    n = len(parts)
    parr = (_vp * max(n, 1))(*[_ptr(p) for p in parts])
    oarr = (_vp * max(len(outs), 1))(*[_ptr(o) for o in outs])
    if len(outs) != n:
        raise ValueError("combine_to_ranks: one output per part")
    _check(_lib.combine_to_ranks(op, n, parr, pdtype, M, n_each, ld_part, odtype, oarr, ldo,
                                 _stream(stream)), "combine_to_ranks")

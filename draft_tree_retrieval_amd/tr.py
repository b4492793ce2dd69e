"""Python binding of libtr (the C ABI in include/tr.h).

Argument marshalling only: every function takes torch tensors (device
memory), derives the sizes the C call takes from their shapes, checks that
every tensor has the shape, dtype, layout (contiguous) and device the call
assumes (ValueError before anything reaches the library: a mismatched
tensor would otherwise be read or written out of bounds on the device), and
calls the entry point of the same name.  All work runs in the HIP kernels
of libtr.so; there is no fallback.  A missing or unloadable library raises
at the first call.
"""
from __future__ import annotations

import ctypes as C
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtr.so")

TR_OK, TR_ERR_INVALID_ARGUMENT, TR_ERR_UNSUPPORTED, TR_ERR_INVALID_TREE, \
    TR_ERR_WORKSPACE_TOO_SMALL, TR_ERR_HIP = range(6)
TR_INT32, TR_INT64, TR_FLOAT32, TR_BFLOAT16 = range(4)
TR_FLAG_BAD_TOKEN, TR_FLAG_CACHE_FULL, TR_FLAG_BAD_PREFIX, TR_FLAG_BAD_PAGE = 1, 2, 4, 8
TR_FLAG_HANDOVER = 16

_DT = {torch.int32: TR_INT32, torch.int64: TR_INT64, torch.float32: TR_FLOAT32,
       torch.bfloat16: TR_BFLOAT16}

_P, _I32, _I64, _SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t

# name -> argument types (restype is tr_status = int unless noted)
_SIGS = {
    "tr_status_string": ([C.c_int], C.c_char_p),
    "tr_last_error": ([], C.c_char_p),
    "tr_tree_create": ([_I32, _P, _P, _I32, C.POINTER(_P)], C.c_int),
    "tr_tree_create_levels": ([_I32, _P, _P, _I32, C.POINTER(_P)], C.c_int),
    "tr_tree_destroy": ([_P], None),
    "tr_tree_info": ([_P, _P, _P, _P, _P, _P, _P, _P], C.c_int),
    "tr_workspace_size": ([_P, _I32, _I64, _I32, _I32, _I32, _I32, _I64], _SZ),
    "tr_workspace_init": ([_P, _SZ, _P], C.c_int),
    "tr_read_device_status": ([_P, _P, _P], C.c_int),
    "tr_retrieve": ([_P, _I32, _P, C.c_int, _I64, _I32, _P, _P, _P, _SZ, _P], C.c_int),
    "tr_tree_attn": ([_P, _I32, _I32, _I32, _I32, C.c_int, _P, _P, _P, _P, _P, _I64, _P,
                      C.c_float, _P, _P, _SZ, _P], C.c_int),
    "tr_update_topk": ([_P, _I32, _P, C.c_int, _I64, _I32, _P, _P, C.c_int, _P, _P, _SZ, _P],
                       C.c_int),
    "tr_verify": ([_P, _I32, _P, _I32, _P, _P, _P, _P, _P, _P], C.c_int),
    "tr_step": ([_P, _I32, _I64, _I32, _P, C.c_int, _P, C.c_int, _P, _P, _P, _P, _P, _I32, _I32,
                 C.c_int, _P, _P, _P, _P, _I64, _P, _P, _P, _SZ, _P], C.c_int),
    "tr_step_ex": ([_P, _I32, _I64, _I32, _P, C.c_int, _P, C.c_int, _P, _P, _P, _P, _P, _I32,
                    _I32, C.c_int, _P, _P, _P, _P, _I64, _P, _P, C.c_int, _P, _SZ, _P], C.c_int),
    "tr_step_sample": ([_P, _I32, _I64, _I32, _P, C.c_int, C.c_float, _P, _P, C.c_int, _P, _P,
                        _P, _P, _P, _I32, _I32, C.c_int, _P, _P, _P, _P, _I64, _P, _P, C.c_int,
                        _P, _SZ, _P], C.c_int),
    "tr_tree_attn_paged": ([_P, _I32, _I32, _P, _P, _I32, C.c_float, _P, _P, _SZ, _P], C.c_int),
    "tr_step_paged": ([_P, _I32, _I64, _I32, _P, C.c_int, _P, C.c_int, _P, _P, _P, _P, _P, _P, _P,
                       C.c_int, _P, _SZ, _P], C.c_int),
    "tr_lmhead_workspace_size": ([_I64, _I64, _I32], _SZ),
    "tr_lmhead_topk": ([_I32, _I32, _I64, _I32, _P, _P, C.c_int, _P, _P, _SZ, _P], C.c_int),
    "tr_step_lmhead": ([_P, _I32, _I32, _I64, _I32, _P, _P, C.c_int, _P, C.c_int, _P, _P, _P, _P,
                        _P, _I32, _I32, C.c_int, _P, _P, _P, _P, _I64, _P, _P, C.c_int, _P, _SZ,
                        _P], C.c_int),
    "tr_init_matrix": ([_I32, _I64, _I32, _P, C.c_int, C.c_int, _P, C.c_int, _I32, C.c_uint64,
                        _P], C.c_int),
    "tr_profile_enable": ([_I32], C.c_int),
    "tr_profile_read": ([_P, _I32], _I32),
    "tr_read_probe": ([_P, _SZ, _P, _P], C.c_int),
    "tr_tree_attn_noalloc": ([_P, _I32, _I32, _I32, _I32, C.c_int, _P, _P, _P, _P, _P, _I64, _P,
                              C.c_float, _P, _P, _P], C.c_int),
}

# tr_kernel_id
KERNEL_NAMES = {1: "attn_prefix", 2: "attn_combine", 3: "topk", 4: "retrieve", 5: "verify", 6: "fill",
                7: "init", 8: "lmhead", 9: "lmhead_merge", 10: "read_probe"}


class _LaunchTime(C.Structure):
    _fields_ = [("kernel", C.c_int32), ("ms", C.c_float)]

_lib = None


class TRError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"{status_string(status)}: {detail}")


def load():
    """The loaded libtr (ctypes.CDLL); raises if the library was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m draft_tree_retrieval_amd.build`")
        lib = C.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = res
        _lib = lib
    return _lib


def status_string(s):
    return load().tr_status_string(s).decode()


def _check(status):
    if status != TR_OK:
        raise TRError(status, load().tr_last_error().decode())


def _ptr(t):
    """The device address of t for the C call (None: NULL); every tensor the
    library receives passes here, after the call's shape checks."""
    if t is None:
        return None
    if t.device.type != "cuda":
        raise ValueError(f"a {list(t.shape)} {t.dtype} tensor is in {t.device} memory; "
                         "libtr takes GPU memory")
    return C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _dt(t):
    return _DT[t.dtype]


_INT = (torch.int32, torch.int64)
_FLT = (torch.float32, torch.bfloat16)
_BF16 = (torch.bfloat16,)
_I32T = (torch.int32,)


def _arg(t, name, shape, dtypes, nullable=False):
    """Checks tensor argument `name`: shape (ints; None matches any extent),
    dtype and contiguity (the device when it is marshalled, in _ptr).  None
    passes only where nullable."""
    if t is None:
        if nullable:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if len(t.shape) != len(shape) or any(w is not None and int(g) != int(w)
                                         for g, w in zip(t.shape, shape)):
        want = "[" + "][".join("*" if w is None else str(int(w)) for w in shape) + "]"
        raise ValueError(f"{name} has shape {list(t.shape)}, expected {want}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_dtype(*named):
    """All non-None tensors of (name, tensor) pairs share the first one's dtype."""
    ts = [(n, t) for n, t in named if t is not None]
    for n, t in ts[1:]:
        if t.dtype != ts[0][1].dtype:
            raise ValueError(f"{n} has dtype {t.dtype}, {ts[0][0]} has {ts[0][1].dtype}")


def _ws(ws):
    _arg(ws, "ws", [None], (torch.uint8,))


def _step_args(tree, logits, M, tree_tok, root_tok, accept_len, accept_path, emitted, topk_out,
               k_tree=None, v_tree=None, k_cache=None, v_cache=None, prefix_len=None):
    """The tensors of a tr_step-family call; returns (B, T, V)."""
    if not isinstance(logits, torch.Tensor) or logits.dim() != 3:
        raise ValueError("logits must be a [B][T][V] tensor")
    B, T, V = logits.shape
    if T != tree.n_nodes:
        raise ValueError(f"logits has {T} rows per sequence, the tree {tree.n_nodes} nodes")
    W = tree.depth + 1
    _arg(logits, "logits", [B, T, V], _FLT)
    _arg(M, "M", [B, V, tree.k], _INT)
    _arg(tree_tok, "tree_tok", [B, T], _I32T)
    _arg(root_tok, "root_tok", [B], _I32T)
    _arg(accept_len, "accept_len", [B], _I32T)
    _arg(accept_path, "accept_path", [B, W], _I32T, nullable=True)
    _arg(emitted, "emitted", [B, W], _I32T, nullable=True)
    _arg(topk_out, "topk_out", [B, T, tree.k], _I32T, nullable=True)
    if k_cache is not None:
        _arg(k_cache, "k_cache", [B, None, None, None], _FLT)
        Hkv, cap, d = k_cache.shape[1:]
        _arg(v_cache, "v_cache", [B, Hkv, cap, d], _FLT)
        _arg(k_tree, "k_tree", [B, T, Hkv, d], _FLT)
        _arg(v_tree, "v_tree", [B, T, Hkv, d], _FLT)
        _arg(prefix_len, "prefix_len", [B], _I32T)
        _same_dtype(("k_cache", k_cache), ("v_cache", v_cache), ("k_tree", k_tree), ("v_tree", v_tree))
    return B, T, V


class Tree:
    """A tr_tree template (host object)."""

    def __init__(self, handle, k):
        self._h = handle
        self.k = k
        n, d = C.c_int32(), C.c_int32()
        _check(load().tr_tree_info(self._h, C.byref(n), C.byref(d), None, None, None, None, None))
        self.n_nodes, self.depth = n.value, d.value

    @classmethod
    def from_parent_rank(cls, parent, rank, k):
        par = (C.c_int32 * len(parent))(*parent)
        rk = (C.c_int32 * len(rank))(*rank)
        h = C.c_void_p()
        _check(load().tr_tree_create(len(parent), par, rk, k, C.byref(h)))
        return cls(h, k)

    @classmethod
    def from_levels(cls, levels, k):
        lens = (C.c_int32 * max(1, len(levels)))(*[len(l) for l in levels])
        flat = [c for l in levels for c in l]
        counts = (C.c_int32 * max(1, len(flat)))(*flat)
        h = C.c_void_p()
        _check(load().tr_tree_create_levels(len(levels), lens, counts, k, C.byref(h)))
        return cls(h, k)

    def info(self):
        T = self.n_nodes
        par, rk, dp = (C.c_int32 * T)(), (C.c_int32 * T)(), (C.c_int32 * T)()
        anc = (C.c_uint64 * (2 * T))()
        _check(load().tr_tree_info(self._h, None, None, None, par, rk, dp, anc))
        return list(par), list(rk), list(dp), [(anc[2 * i], anc[2 * i + 1]) for i in range(T)]

    @property
    def handle(self):
        return self._h

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.tr_tree_destroy(self._h)
            self._h = None


def tr_workspace_size(tree, B, V=0, k=0, Hq=0, Hkv=0, d=0, cap=0):
    return int(load().tr_workspace_size(tree.handle, B, V, k, Hq, Hkv, d, cap))


def tr_workspace_init(ws, stream=None):
    _ws(ws)
    _check(load().tr_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def new_workspace(tree, B, V=0, k=0, Hq=0, Hkv=0, d=0, cap=0, device="cuda", stream=None):
    """Allocates (through torch) and zero-initialises a workspace."""
    n = tr_workspace_size(tree, B, V, k, Hq, Hkv, d, cap)
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    tr_workspace_init(ws, stream)
    return ws


def tr_read_device_status(ws, stream=None):
    _ws(ws)
    flags = C.c_uint32()
    _check(load().tr_read_device_status(_ptr(ws), C.byref(flags), _stream(stream)))
    return flags.value


def tr_retrieve(tree, M, root_tok, tree_tok, ws, stream=None):
    if not isinstance(M, torch.Tensor) or M.dim() != 3:
        raise ValueError("M must be a [B][V][k] tensor")
    B, V, k = M.shape
    _arg(M, "M", [B, V, tree.k], _INT)
    _arg(root_tok, "root_tok", [B], _I32T)
    _arg(tree_tok, "tree_tok", [B, tree.n_nodes], _I32T)
    _ws(ws)
    _check(load().tr_retrieve(tree.handle, B, _ptr(M), _dt(M), V, k, _ptr(root_tok), _ptr(tree_tok),
                              _ptr(ws), ws.numel(), _stream(stream)))


def tr_tree_attn(tree, q, k_tree, v_tree, k_cache, v_cache, prefix_len, out, ws, scale=None,
                 stream=None):
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a [B][T][Hq][d] tensor")
    if not isinstance(k_cache, torch.Tensor) or k_cache.dim() != 4:
        raise ValueError("k_cache must be a [B][Hkv][cap][d] tensor")
    B, T, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    cap = k_cache.shape[2]
    if T != tree.n_nodes:
        raise ValueError(f"q has {T} rows per sequence, the tree {tree.n_nodes} nodes")
    _arg(q, "q", [B, T, Hq, d], _FLT)
    _arg(k_tree, "k_tree", [B, T, Hkv, d], _FLT)
    _arg(v_tree, "v_tree", [B, T, Hkv, d], _FLT)
    _arg(k_cache, "k_cache", [B, Hkv, cap, d], _FLT)
    _arg(v_cache, "v_cache", [B, Hkv, cap, d], _FLT)
    _arg(prefix_len, "prefix_len", [B], _I32T)
    _arg(out, "out", [B, T, Hq, d], _FLT)
    _same_dtype(("q", q), ("k_tree", k_tree), ("v_tree", v_tree), ("k_cache", k_cache),
                ("v_cache", v_cache), ("out", out))
    _ws(ws)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(load().tr_tree_attn(tree.handle, B, Hq, Hkv, d, _dt(q), _ptr(q), _ptr(k_tree),
                               _ptr(v_tree), _ptr(k_cache), _ptr(v_cache), cap, _ptr(prefix_len),
                               float(scale), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))


def tr_tree_attn_noalloc(tree, q, k_tree, v_tree, k_cache, v_cache, prefix_len, out, flags=None,
                         scale=None, stream=None):
    """tr_tree_attn without a workspace (the library's per-GPU scratch);
    flags: an optional device int32 [1] the sticky TR_FLAG_* bits are OR-ed into."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a [B][T][Hq][d] tensor")
    if not isinstance(k_cache, torch.Tensor) or k_cache.dim() != 4:
        raise ValueError("k_cache must be a [B][Hkv][cap][d] tensor")
    B, T, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    cap = k_cache.shape[2]
    if T != tree.n_nodes:
        raise ValueError(f"q has {T} rows per sequence, the tree {tree.n_nodes} nodes")
    _arg(q, "q", [B, T, Hq, d], _FLT)
    _arg(k_tree, "k_tree", [B, T, Hkv, d], _FLT)
    _arg(v_tree, "v_tree", [B, T, Hkv, d], _FLT)
    _arg(k_cache, "k_cache", [B, Hkv, cap, d], _FLT)
    _arg(v_cache, "v_cache", [B, Hkv, cap, d], _FLT)
    _arg(prefix_len, "prefix_len", [B], _I32T)
    _arg(out, "out", [B, T, Hq, d], _FLT)
    _same_dtype(("q", q), ("k_tree", k_tree), ("v_tree", v_tree), ("k_cache", k_cache),
                ("v_cache", v_cache), ("out", out))
    _arg(flags, "flags", [None], (torch.int32, torch.uint32), nullable=True)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(load().tr_tree_attn_noalloc(tree.handle, B, Hq, Hkv, d, _dt(q), _ptr(q), _ptr(k_tree),
                                       _ptr(v_tree), _ptr(k_cache), _ptr(v_cache), cap,
                                       _ptr(prefix_len), float(scale), _ptr(out), _ptr(flags),
                                       _stream(stream)))


class _PagedKVStruct(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("Hkv", C.c_int32), ("d", C.c_int32), ("dtype", C.c_int),
                ("page_size", C.c_int32), ("num_pages", C.c_int64), ("max_pages", C.c_int32),
                ("block_table", C.c_void_p), ("k_pages", C.c_void_p), ("v_pages", C.c_void_p),
                ("k_tree", C.c_void_p), ("v_tree", C.c_void_p), ("prefix_len", C.c_void_p)]


class PagedKV:
    """A tr_paged_kv over caller tensors: pools k_pages/v_pages
    [layers][num_pages][Hkv][page_size][d], block_table [B][max_pages] int32,
    tree rows k_tree/v_tree [layers][B][T][Hkv][d], prefix_len [B] int32."""

    def __init__(self, k_pages, v_pages, block_table, k_tree, v_tree, prefix_len):
        if not isinstance(k_pages, torch.Tensor) or k_pages.dim() != 5:
            raise ValueError("k_pages must be a [layers][num_pages][Hkv][page_size][d] tensor")
        if not isinstance(k_tree, torch.Tensor) or k_tree.dim() != 5:
            raise ValueError("k_tree must be a [layers][B][T][Hkv][d] tensor")
        L, npg, Hkv, ps, d = k_pages.shape
        B, T = k_tree.shape[1], k_tree.shape[2]
        _arg(k_pages, "k_pages", [L, npg, Hkv, ps, d], _BF16)
        _arg(v_pages, "v_pages", [L, npg, Hkv, ps, d], _BF16)
        _arg(block_table, "block_table", [B, None], _I32T)
        _arg(k_tree, "k_tree", [L, B, T, Hkv, d], _BF16)
        _arg(v_tree, "v_tree", [L, B, T, Hkv, d], _BF16)
        _arg(prefix_len, "prefix_len", [B], _I32T)
        self.B, self.T, self.L = B, T, L
        self.tensors = (k_pages, v_pages, block_table, k_tree, v_tree, prefix_len)
        self.s = _PagedKVStruct(L, Hkv, d, _dt(k_pages), ps, npg, block_table.shape[1],
                                _ptr(block_table), _ptr(k_pages), _ptr(v_pages), _ptr(k_tree),
                                _ptr(v_tree), _ptr(prefix_len))

    @property
    def ref(self):
        return C.byref(self.s)


def tr_tree_attn_paged(tree, q, kv, layer, out, ws, scale=None, stream=None):
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a [B][T][Hq][d] tensor")
    B, T, Hq, d = q.shape
    if (B, T) != (kv.B, kv.T) or T != tree.n_nodes:
        raise ValueError(f"q is [{B}][{T}][..], the cache holds {kv.B} sequences of {kv.T} nodes, "
                         f"the tree {tree.n_nodes} nodes")
    _arg(q, "q", [B, T, Hq, d], _BF16)
    _arg(out, "out", [B, T, Hq, d], _BF16)
    _ws(ws)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(load().tr_tree_attn_paged(tree.handle, B, Hq, _ptr(q), kv.ref, layer, float(scale),
                                     _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))


def tr_step_paged(tree, logits, M, tree_tok, root_tok, accept_len, accept_path, emitted, ws, kv,
                  topk_out=None, update="all", stream=None):
    mode = _UPDATE_MODES[update] if isinstance(update, str) else int(update)
    B, T, V = _step_args(tree, logits, M, tree_tok, root_tok, accept_len, accept_path, emitted,
                         topk_out)
    if (B, T) != (kv.B, kv.T):
        raise ValueError(f"logits are [{B}][{T}][..], the cache holds {kv.B} sequences of {kv.T} nodes")
    _ws(ws)
    _check(load().tr_step_paged(tree.handle, B, V, tree.k, _ptr(logits), _dt(logits), _ptr(M),
                                _dt(M), _ptr(tree_tok), _ptr(root_tok), _ptr(accept_len),
                                _ptr(accept_path), _ptr(emitted), kv.ref, _ptr(topk_out), mode,
                                _ptr(ws), ws.numel(), _stream(stream)))


def tr_update_topk(tree, logits, tree_tok, M, topk_out, ws, stream=None):
    if not isinstance(logits, torch.Tensor) or logits.dim() != 3:
        raise ValueError("logits must be a [B][T][V] tensor")
    B, T, V = logits.shape
    k = tree.k
    if T != tree.n_nodes:
        raise ValueError(f"logits has {T} rows per sequence, the tree {tree.n_nodes} nodes")
    _arg(logits, "logits", [B, T, V], _FLT)
    _arg(M, "M", [B, V, k], _INT, nullable=True)
    _arg(tree_tok, "tree_tok", [B, T], _I32T, nullable=M is None)
    _arg(topk_out, "topk_out", [B, T, k], _I32T, nullable=M is not None)
    _ws(ws)
    _check(load().tr_update_topk(tree.handle, B, _ptr(logits), _dt(logits), V, k, _ptr(tree_tok),
                                 _ptr(M), _dt(M) if M is not None else TR_INT32, _ptr(topk_out),
                                 _ptr(ws), ws.numel(), _stream(stream)))


def tr_verify(tree, topk, tree_tok, accept_len, accept_path, bonus, emitted, stream=None):
    if not isinstance(topk, torch.Tensor) or topk.dim() != 3:
        raise ValueError("topk must be a [B][T][k] tensor")
    B = topk.shape[0]
    T, W = tree.n_nodes, tree.depth + 1
    _arg(topk, "topk", [B, T, tree.k], _I32T)
    _arg(tree_tok, "tree_tok", [B, T], _I32T)
    _arg(accept_len, "accept_len", [B], _I32T)
    _arg(accept_path, "accept_path", [B, W], _I32T, nullable=True)
    _arg(bonus, "bonus", [B], _I32T)
    _arg(emitted, "emitted", [B, W], _I32T, nullable=True)
    _check(load().tr_verify(tree.handle, B, _ptr(topk), topk.shape[2], _ptr(tree_tok),
                            _ptr(accept_len), _ptr(accept_path), _ptr(bonus), _ptr(emitted),
                            _stream(stream)))


def _kv_shape(k_cache):
    if k_cache is not None:
        return k_cache.shape[1], k_cache.shape[2], k_cache.shape[3], _dt(k_cache)
    return 0, 0, 0, TR_BFLOAT16


def tr_step(tree, logits, M, tree_tok, root_tok, accept_len, accept_path, emitted, ws,
            k_tree=None, v_tree=None, k_cache=None, v_cache=None, prefix_len=None, topk_out=None,
            stream=None):
    B, T, V = _step_args(tree, logits, M, tree_tok, root_tok, accept_len, accept_path, emitted,
                         topk_out, k_tree, v_tree, k_cache, v_cache, prefix_len)
    _ws(ws)
    Hkv, cap, d, kv_dt = _kv_shape(k_cache)
    _check(load().tr_step(tree.handle, B, V, tree.k, _ptr(logits), _dt(logits), _ptr(M), _dt(M),
                          _ptr(tree_tok), _ptr(root_tok), _ptr(accept_len), _ptr(accept_path),
                          _ptr(emitted), Hkv, d, kv_dt, _ptr(k_tree), _ptr(v_tree), _ptr(k_cache),
                          _ptr(v_cache), cap, _ptr(prefix_len), _ptr(topk_out), _ptr(ws),
                          ws.numel(), _stream(stream)))


# tr_update_mode
TR_UPDATE_ALL, TR_UPDATE_ACCEPTED = 0, 1
_UPDATE_MODES = {"all": TR_UPDATE_ALL, "accepted": TR_UPDATE_ACCEPTED}


def tr_step_ex(tree, logits, M, tree_tok, root_tok, accept_len, accept_path, emitted, ws,
               k_tree=None, v_tree=None, k_cache=None, v_cache=None, prefix_len=None,
               topk_out=None, update="all", stream=None):
    """tr_step with the update chosen by name: "all" or "accepted"."""
    mode = _UPDATE_MODES[update] if isinstance(update, str) else int(update)
    B, T, V = _step_args(tree, logits, M, tree_tok, root_tok, accept_len, accept_path, emitted,
                         topk_out, k_tree, v_tree, k_cache, v_cache, prefix_len)
    _ws(ws)
    Hkv, cap, d, kv_dt = _kv_shape(k_cache)
    _check(load().tr_step_ex(tree.handle, B, V, tree.k, _ptr(logits), _dt(logits), _ptr(M),
                             _dt(M), _ptr(tree_tok), _ptr(root_tok), _ptr(accept_len),
                             _ptr(accept_path), _ptr(emitted), Hkv, d, kv_dt, _ptr(k_tree),
                             _ptr(v_tree), _ptr(k_cache), _ptr(v_cache), cap, _ptr(prefix_len),
                             _ptr(topk_out), mode, _ptr(ws), ws.numel(), _stream(stream)))


def tr_step_sample(tree, logits, temperature, uniforms, M, tree_tok, root_tok, accept_len,
                   accept_path, emitted, ws, k_tree=None, v_tree=None, k_cache=None, v_cache=None,
                   prefix_len=None, topk_out=None, update="all", stream=None):
    """tr_step verifying by sampling at `temperature` with the caller's
    uniforms [B][T][2] (float32, device)."""
    mode = _UPDATE_MODES[update] if isinstance(update, str) else int(update)
    B, T, V = _step_args(tree, logits, M, tree_tok, root_tok, accept_len, accept_path, emitted,
                         topk_out, k_tree, v_tree, k_cache, v_cache, prefix_len)
    _arg(uniforms, "uniforms", [B, T, 2], (torch.float32,))
    _ws(ws)
    Hkv, cap, d, kv_dt = _kv_shape(k_cache)
    _check(load().tr_step_sample(tree.handle, B, V, tree.k, _ptr(logits), _dt(logits),
                                 float(temperature), _ptr(uniforms), _ptr(M), _dt(M),
                                 _ptr(tree_tok), _ptr(root_tok), _ptr(accept_len),
                                 _ptr(accept_path), _ptr(emitted), Hkv, d, kv_dt, _ptr(k_tree),
                                 _ptr(v_tree), _ptr(k_cache), _ptr(v_cache), cap,
                                 _ptr(prefix_len), _ptr(topk_out), mode, _ptr(ws), ws.numel(),
                                 _stream(stream)))


def tr_lmhead_workspace_size(rows, V, k):
    return int(load().tr_lmhead_workspace_size(rows, V, k))


def new_lmhead_workspace(rows, V, k, device="cuda", stream=None):
    """A zeroed workspace for tr_lmhead_topk / tr_step_lmhead."""
    n = tr_lmhead_workspace_size(rows, V, k)
    n = (n + 255) // 256 * 256
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    _check(load().tr_workspace_init(_ptr(ws), n, _stream(stream)))
    return ws


def tr_lmhead_topk(h, W, k, topk_out, ws, stream=None):
    """topk_out [rows][k] = the k best ids of h W^T per row (h [rows][H],
    W [V][H], bfloat16)."""
    if not isinstance(h, torch.Tensor) or h.dim() != 2 or not isinstance(W, torch.Tensor) or W.dim() != 2:
        raise ValueError("h must be [rows][H] and W [V][H]")
    rows, H = h.shape
    V = W.shape[0]
    _arg(h, "h", [rows, H], _BF16)
    _arg(W, "W", [V, H], _BF16)
    _arg(topk_out, "topk_out", [rows, k], _I32T)
    _ws(ws)
    _check(load().tr_lmhead_topk(rows, H, V, k, _ptr(h), _ptr(W), _dt(h), _ptr(topk_out),
                                 _ptr(ws), ws.numel(), _stream(stream)))


def tr_step_lmhead(tree, h, W, M, tree_tok, root_tok, accept_len, accept_path, emitted, ws,
                   k_tree=None, v_tree=None, k_cache=None, v_cache=None, prefix_len=None,
                   topk_out=None, update="all", stream=None):
    """tr_step_ex with the LM head fused in front: h [B][T][H], W [V][H]."""
    mode = _UPDATE_MODES[update] if isinstance(update, str) else int(update)
    if not isinstance(h, torch.Tensor) or h.dim() != 3 or not isinstance(W, torch.Tensor) or W.dim() != 2:
        raise ValueError("h must be [B][T][H] and W [V][H]")
    B, T, H = h.shape
    V = W.shape[0]
    if T != tree.n_nodes:
        raise ValueError(f"h has {T} rows per sequence, the tree {tree.n_nodes} nodes")
    _arg(h, "h", [B, T, H], _BF16)
    _arg(W, "W", [V, H], _BF16)
    Wd = tree.depth + 1
    _arg(M, "M", [B, V, tree.k], _INT)
    _arg(tree_tok, "tree_tok", [B, T], _I32T)
    _arg(root_tok, "root_tok", [B], _I32T)
    _arg(accept_len, "accept_len", [B], _I32T)
    _arg(accept_path, "accept_path", [B, Wd], _I32T, nullable=True)
    _arg(emitted, "emitted", [B, Wd], _I32T, nullable=True)
    _arg(topk_out, "topk_out", [B, T, tree.k], _I32T, nullable=True)
    if k_cache is not None:
        _arg(k_cache, "k_cache", [B, None, None, None], _FLT)
        Hk, cp, dd = k_cache.shape[1:]
        _arg(v_cache, "v_cache", [B, Hk, cp, dd], _FLT)
        _arg(k_tree, "k_tree", [B, T, Hk, dd], _FLT)
        _arg(v_tree, "v_tree", [B, T, Hk, dd], _FLT)
        _arg(prefix_len, "prefix_len", [B], _I32T)
        _same_dtype(("k_cache", k_cache), ("v_cache", v_cache), ("k_tree", k_tree), ("v_tree", v_tree))
    _ws(ws)
    Hkv, cap, d, kv_dt = _kv_shape(k_cache)
    _check(load().tr_step_lmhead(tree.handle, B, H, V, tree.k, _ptr(h), _ptr(W), _dt(h), _ptr(M),
                                 _dt(M), _ptr(tree_tok), _ptr(root_tok), _ptr(accept_len),
                                 _ptr(accept_path), _ptr(emitted), Hkv, d, kv_dt, _ptr(k_tree),
                                 _ptr(v_tree), _ptr(k_cache), _ptr(v_cache), cap,
                                 _ptr(prefix_len), _ptr(topk_out), mode, _ptr(ws), ws.numel(),
                                 _stream(stream)))


# tr_init_mode
TR_INIT_ZERO, TR_INIT_RANDOM, TR_INIT_PRIOR = 0, 1, 2
_INIT_MODES = {"zero": TR_INIT_ZERO, "random": TR_INIT_RANDOM, "prior": TR_INIT_PRIOR}


def tr_init_matrix(M, mode="zero", prior=None, seed=0, stream=None):
    """Fills M [B][V][k] on the device: "zero", "random" (SplitMix64 ids,
    seeded) or "prior" (prior [1 or B][V][k] copied into every slot)."""
    if not isinstance(M, torch.Tensor) or M.dim() != 3:
        raise ValueError("M must be a [B][V][k] tensor")
    B, V, k = M.shape
    _arg(M, "M", [B, V, k], _INT)
    if prior is not None:
        if prior.dim() != 3 or prior.shape[0] not in (1, B):
            raise ValueError(f"prior has shape {list(prior.shape)}, expected [1 or {B}][{V}][{k}]")
        _arg(prior, "prior", [prior.shape[0], V, k], _INT)
    m = _INIT_MODES[mode] if isinstance(mode, str) else int(mode)
    pb = prior.shape[0] if prior is not None else 0
    _check(load().tr_init_matrix(B, V, k, _ptr(M), _dt(M), m, _ptr(prior),
                                 _dt(prior) if prior is not None else TR_INT32, pb,
                                 int(seed) & ((1 << 64) - 1), _stream(stream)))


def tr_profile_enable(on=True):
    """Profiling aid: bracket every library launch with HIP events."""
    _check(load().tr_profile_enable(1 if on else 0))


def tr_profile_read(max_records=16384):
    """[(kernel name, ms)] of the launches recorded since the last read, in
    launch order (synchronises on their events)."""
    buf = (_LaunchTime * max_records)()
    n = load().tr_profile_read(buf, max_records)
    return [(KERNEL_NAMES.get(buf[i].kernel, str(buf[i].kernel)), float(buf[i].ms)) for i in range(n)]


def tr_read_probe(src, sink, stream=None):
    """One streaming read of every byte of src (a profiling aid)."""
    _arg(src, "src", [None] * src.dim(), None)
    _arg(sink, "sink", [None] * sink.dim(), None)
    _check(load().tr_read_probe(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                _stream(stream)))

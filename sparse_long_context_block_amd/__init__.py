"""Python binding of libsgqa.so, the MI355X sparse GQA global-attention library.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in ``include/sgqa.h``; PyTorch supplies device memory and the stream.
There is no other code path -- if the library is not built, every call raises.

Entry points (names as in the C ABI, ``sgqa_`` dropped):

* :func:`compress`      block-wise token merging into the proxy-key store
* :func:`index_topk`    indexer scores + causal top-k block selection
* :func:`sparse_attn`   sparse GQA attention over the selected original K/V
* :func:`forward`       the three in order on one stream
* :func:`workspace_size`

Tensors are CUDA (HIP) tensors, contiguous, with the dtypes and shapes the
header documents: bf16 as ``torch.bfloat16``, fp32 as ``torch.float32``,
selections as ``torch.int32``.  Calls are asynchronous on ``stream``
(default: torch's current stream).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Iterable, Optional, Sequence

import torch

__all__ = [
    "Config", "Seq", "SgqaError", "config", "seq", "lib", "workspace_size", "compress",
    "index_topk", "sparse_attn", "forward", "compress_paged", "sparse_attn_paged", "forward_paged",
    "QkConfig", "qk_config", "qk_prep", "sparse_attn_gated", "forward_gated",
    "LIB_PATH", "OP_COMPRESS", "OP_INDEX_TOPK", "OP_SPARSE_ATTN", "OP_FORWARD",
    "index_diag_offset", "forward_diag_offset", "index_diagnostics", "forward_noalloc",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsgqa.so")

OP_COMPRESS, OP_INDEX_TOPK, OP_SPARSE_ATTN, OP_FORWARD = 0, 1, 2, 3


class SgqaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)} ({status}): {message}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_groups", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("idx_heads", ctypes.c_int32),
        ("idx_dim", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32),
        ("rope_base", ctypes.c_float),
        ("block_size", ctypes.c_int32),
        ("topk_blocks", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("eps_rms", ctypes.c_float),
        ("eps_ln", ctypes.c_float),
        ("store_q8", ctypes.c_int32),
    ]


class Seq(ctypes.Structure):
    _fields_ = [
        ("q_offset", ctypes.c_int64),
        ("n_q", ctypes.c_int64),
        ("pos0", ctypes.c_int64),
        ("cache_len", ctypes.c_int64),
        ("kv_offset", ctypes.c_int64),
        ("kv_capacity", ctypes.c_int64),
        ("store_offset", ctypes.c_int64),
        ("store_capacity", ctypes.c_int64),
    ]


def config(block_size: int = 8, topk_blocks: int = 512, store_q8: int = 2, **kw) -> Config:
    """The page's layer shape (64 heads, 4 groups, head_dim 192, 4x128 indexer,
    32-dim rotary span, base 1e4, softmax scale 1/sqrt(192)); fields overridable.

    store_q8: 2 (default) E4M3 codes in a uint8 store, 1 the same values held
    in a bf16 store (twice the bytes, identical results), 0 bf16 values
    (the unrounded ablation)."""
    if int(store_q8) not in (0, 1, 2):
        raise ValueError("store_q8 must be 0, 1 or 2")
    c = Config(num_q_heads=64, num_kv_groups=4, head_dim=192, idx_heads=4, idx_dim=128,
               rope_dim=32, rope_base=10000.0, block_size=block_size, topk_blocks=topk_blocks,
               softmax_scale=1.0 / math.sqrt(192.0), eps_rms=1e-6, eps_ln=1e-6,
               store_q8=int(store_q8))
    for k, v in kw.items():
        setattr(c, k, v)
    return c


class QkConfig(ctypes.Structure):
    _fields_ = [
        ("rope_dim", ctypes.c_int32),
        ("rope_base", ctypes.c_float),
        ("eps", ctypes.c_float),
        ("reserved", ctypes.c_int32),
    ]


def qk_config(rope_dim: int = 64, rope_base: float = 10000.0, eps: float = 1e-6) -> QkConfig:
    """Main-path Q/K producer parameters (the rotary span is a parameter: the
    page names the layer's partial-rotary factor without giving it)."""
    return QkConfig(rope_dim=rope_dim, rope_base=rope_base, eps=eps, reserved=0)


def seq(n_q: int, pos0: int = 0, q_offset: int = 0, kv_offset: int = 0,
        kv_capacity: Optional[int] = None, store_offset: int = 0,
        store_capacity: Optional[int] = None, block_size: int = 8) -> Seq:
    cache_len = pos0 + n_q
    return Seq(q_offset=q_offset, n_q=n_q, pos0=pos0, cache_len=cache_len, kv_offset=kv_offset,
               kv_capacity=cache_len if kv_capacity is None else kv_capacity,
               store_offset=store_offset,
               store_capacity=(cache_len // block_size) if store_capacity is None else store_capacity)


_lib = None
_STATUS = {0: "SGQA_OK", -1: "SGQA_ERR_NULL", -2: "SGQA_ERR_CONFIG", -3: "SGQA_ERR_SHAPE",
           -4: "SGQA_ERR_CAUSAL", -5: "SGQA_ERR_CAPACITY", -6: "SGQA_ERR_WORKSPACE",
           -7: "SGQA_ERR_UNSUPPORTED", -8: "SGQA_ERR_HIP"}


def _status_name(s: int) -> str:
    return _STATUS.get(s, "SGQA_UNKNOWN_STATUS")


def lib() -> ctypes.CDLL:
    """Load libsgqa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m sparse_long_context_block_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp, seqp = ctypes.POINTER(Config), ctypes.POINTER(Seq)
    L.sgqa_workspace_size.argtypes = [cfgp, seqp, I32, I32]
    L.sgqa_workspace_size.restype = SZ
    L.sgqa_compress.argtypes = [cfgp, seqp, I32, P, P, P, P, P, P, SZ, P]
    L.sgqa_compress.restype = ctypes.c_int
    L.sgqa_index_topk.argtypes = [cfgp, seqp, I32, P, P, P, P, P, P, P, P, SZ, P]
    L.sgqa_index_topk.restype = ctypes.c_int
    L.sgqa_sparse_attn.argtypes = [cfgp, seqp, I32, P, P, P, P, P, P, P, SZ, P]
    L.sgqa_sparse_attn.restype = ctypes.c_int
    L.sgqa_forward.argtypes = [cfgp, seqp, I32, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                               P, SZ, P]
    L.sgqa_forward.restype = ctypes.c_int
    I64 = ctypes.c_int64
    L.sgqa_compress_paged.argtypes = [cfgp, seqp, I32, P, P, P, I64, I64, P, P, P, P, SZ, P]
    L.sgqa_compress_paged.restype = ctypes.c_int
    L.sgqa_sparse_attn_paged.argtypes = [cfgp, seqp, I32, P, P, P, P, I64, I64, P, P, P, P, P, SZ, P]
    L.sgqa_sparse_attn_paged.restype = ctypes.c_int
    L.sgqa_forward_paged.argtypes = [cfgp, seqp, I32, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                     I64, I64, P, P, P, P, SZ, P]
    L.sgqa_forward_paged.restype = ctypes.c_int
    L.sgqa_sparse_attn_gated.argtypes = [cfgp, seqp, I32, P, P, P, P, P, P, P, P, SZ, P]
    L.sgqa_sparse_attn_gated.restype = ctypes.c_int
    L.sgqa_forward_gated.argtypes = [cfgp, seqp, I32, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                     P, P, SZ, P]
    L.sgqa_forward_gated.restype = ctypes.c_int
    L.sgqa_qk_prep.argtypes = [cfgp, ctypes.POINTER(QkConfig), seqp, I32, P, P, P, P, P, P, P, P, P,
                               I64, I64, P]
    L.sgqa_qk_prep.restype = ctypes.c_int
    L.sgqa_status_string.argtypes = [ctypes.c_int]
    L.sgqa_status_string.restype = ctypes.c_char_p
    L.sgqa_last_error.argtypes = []
    L.sgqa_last_error.restype = ctypes.c_char_p
    L.sgqa_abi_version.argtypes = []
    L.sgqa_abi_version.restype = I32
    L.sgqa_index_diag_offset.argtypes = [cfgp, seqp, I32]
    L.sgqa_index_diag_offset.restype = I64
    L.sgqa_forward_diag_offset.argtypes = [cfgp, seqp, I32]
    L.sgqa_forward_diag_offset.restype = I64
    L.sgqa_forward_noalloc.argtypes = [cfgp, seqp, I32, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                       P, P]
    L.sgqa_forward_noalloc.restype = ctypes.c_int
    _lib = L
    return L


def _check(rc: int) -> None:
    if rc != 0:
        raise SgqaError(rc, lib().sgqa_last_error().decode())


def _seq_array(seqs: Sequence[Seq]):
    seqs = list(seqs)
    arr = (Seq * len(seqs))(*seqs)
    return arr, len(seqs)


def _ptr(t: Optional[torch.Tensor], dtype: torch.dtype, name: str, required: bool = True,
         shape: Optional[tuple] = None):
    """Device pointer of `t` after checking dtype, device, contiguity and,
    with `shape`, its extents: shape[0] is the least number of leading rows
    the call touches, the other entries are exact; a string entry names an
    extent that only has to be positive (a pool's page count)."""
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None:
        if t.dim() != len(shape):
            raise ValueError(f"{name} must have {len(shape)} dims {_fmt_shape(shape)}, got "
                             f"{tuple(t.shape)}")
        lead, rest = shape[0], tuple(shape[1:])
        if tuple(t.shape[1:]) != rest:
            raise ValueError(f"{name} must be {_fmt_shape(shape)}, got {tuple(t.shape)}")
        if isinstance(lead, str):
            if t.shape[0] < 1:
                raise ValueError(f"{name} needs at least one {lead}")
        elif t.shape[0] < lead:
            raise ValueError(f"{name} has {t.shape[0]} rows; the call touches {lead} "
                             f"{_fmt_shape(shape)}")
    return _Arg(t, name)


class _Arg:
    """A tensor argument whose dtype and extents have been checked; its
    device is checked, and its pointer taken, once every argument of the
    call has passed (_addrs)."""
    __slots__ = ("t", "name")

    def __init__(self, t, name):
        self.t, self.name = t, name


def _addrs(items):
    """Device pointers of checked arguments (None stays None)."""
    out = []
    for a in items:
        if a is None:
            out.append(None)
            continue
        if a.t.device.type != "cuda":
            raise ValueError(f"{a.name} must be a device (cuda/hip) tensor")
        out.append(a.t.data_ptr())
    return tuple(out)


def _fmt_shape(shape) -> str:
    return "[" + ", ".join(str(x) if not isinstance(x, int) or i else f">={x}"
                           for i, x in enumerate(shape)) + "]"


class _Extents:
    """Rows of each tensor family the sequences touch: query rows (Q, q_idx,
    w, sel, out, lse, gate), cache rows (K, V, proxy keys, logits of the
    contiguous layout) and store rows; plus the config's widths."""

    def __init__(self, cfg: Config, seqs: Sequence[Seq]):
        self.q_rows = max([s.q_offset + s.n_q for s in seqs if s.n_q > 0] + [0])
        self.kv_rows = max([s.kv_offset + s.kv_capacity for s in seqs] + [0])
        self.store_rows = max([s.store_offset + s.store_capacity for s in seqs] + [0])
        self.H, self.G, self.D = cfg.num_q_heads, cfg.num_kv_groups, cfg.head_dim
        self.Hi, self.Di, self.K = cfg.idx_heads, cfg.idx_dim, cfg.topk_blocks

    # per-family shapes
    def q(self):
        return (self.q_rows, self.H, self.D)

    def kv(self):
        return (self.kv_rows, self.G, self.D)

    def q_idx(self):
        return (self.q_rows, self.G, self.Hi, self.Di)

    def w(self):
        return (self.q_rows, self.G, self.Hi)

    def sel(self):
        return (self.q_rows, self.G, self.K)

    def lse(self):
        return (self.q_rows, self.H)

    def proxy(self):
        return (self.kv_rows, self.Di)

    def store(self):
        return (self.store_rows, self.Di)

    def kv_pages(self):
        return ("page", PAGE_TOKENS, self.G, self.D)

    def proxy_pages(self):
        return ("page", PAGE_TOKENS, self.Di)


PAGE_TOKENS = 16


def _vec_ptr(t, dtype, name, n):
    """An optional parameter vector of exactly n elements."""
    if t is not None and t.numel() != n:
        raise ValueError(f"{name} must have {n} elements, got {t.numel()}")
    return _ptr(t, dtype, name, False)


def _store_ptr(cfg: Config, store, ext: Optional[_Extents] = None):
    """The proxy-key store: uint8 E4M3 codes when cfg.store_q8 == 2, else bf16."""
    return _ptr(store, torch.uint8 if cfg.store_q8 == 2 else torch.bfloat16, "store",
                shape=ext.store() if ext else None)


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def workspace_size(cfg: Config, seqs: Sequence[Seq], op: int) -> int:
    arr, n = _seq_array(seqs)
    return int(lib().sgqa_workspace_size(ctypes.byref(cfg), arr, n, op))


def _workspace(cfg, seqs, op, device, ws, stream):
    """(pointer, bytes, owner) of the call's workspace; allocates through torch
    when the caller passes none.  The owner must outlive the enqueue; torch's
    stream-ordered allocator then keeps reuse after the call's work."""
    if ws is not None:
        return _addrs([_ptr(ws, torch.uint8, "ws")])[0], ws.numel(), ws
    need = workspace_size(cfg, seqs, op)
    if need == 0:
        return None, 0, None
    buf = torch.empty(need + 256, dtype=torch.uint8, device=device)
    if stream is not None:
        buf.record_stream(stream)
    off = (-buf.data_ptr()) % 256
    return buf.data_ptr() + off, need, buf


def compress(cfg: Config, seqs: Sequence[Seq], proxy_k, comp_logits, store, ln_gamma=None,
             ln_beta=None, stream=None) -> None:
    seqs = list(seqs)
    ext = _Extents(cfg, seqs)
    arr, n = _seq_array(seqs)
    ptrs = (_ptr(proxy_k, torch.bfloat16, "proxy_k", shape=ext.proxy()),
            _ptr(comp_logits, torch.float32, "comp_logits", shape=ext.proxy()),
            _vec_ptr(ln_gamma, torch.bfloat16, "ln_gamma", ext.Di),
            _vec_ptr(ln_beta, torch.bfloat16, "ln_beta", ext.Di), _store_ptr(cfg, store, ext))
    _check(lib().sgqa_compress(ctypes.byref(cfg), arr, n, *_addrs(ptrs), None, 0, _stream_ptr(stream)))


def index_topk(cfg: Config, seqs: Sequence[Seq], q_idx, w, store, sel, sel_scores=None,
               q_hat_out=None, rms_gamma=None, ws=None, stream=None) -> None:
    seqs = list(seqs)
    ext = _Extents(cfg, seqs)
    arr, n = _seq_array(seqs)
    ptrs = (_ptr(q_idx, torch.bfloat16, "q_idx", shape=ext.q_idx()),
            _ptr(w, torch.float32, "w", shape=ext.w()),
            _vec_ptr(rms_gamma, torch.bfloat16, "rms_gamma", ext.Di),
            _store_ptr(cfg, store, ext), _ptr(sel, torch.int32, "sel", shape=ext.sel()),
            _ptr(sel_scores, torch.float32, "sel_scores", False, shape=ext.sel()),
            _ptr(q_hat_out, torch.bfloat16, "q_hat_out", False, shape=ext.q_idx()))
    ptrs = _addrs(ptrs)
    wsp, wsn, _own = _workspace(cfg, seqs, OP_INDEX_TOPK, q_idx.device, ws, stream)
    _check(lib().sgqa_index_topk(ctypes.byref(cfg), arr, n, *ptrs, wsp, wsn, _stream_ptr(stream)))


def index_diag_offset(cfg: Config, seqs: Sequence[Seq]) -> Optional[int]:
    """Byte offset of the index step's diagnostics block in an OP_INDEX_TOPK
    workspace of these arguments, or None when the call keeps none
    (include/sgqa.h, sgqa_index_diag_offset)."""
    arr, n = _seq_array(seqs)
    off = int(lib().sgqa_index_diag_offset(ctypes.byref(cfg), arr, n))
    return off if off >= 0 else None


def forward_diag_offset(cfg: Config, seqs: Sequence[Seq]) -> Optional[int]:
    """The same block's byte offset in an OP_FORWARD workspace, or None
    (include/sgqa.h, sgqa_forward_diag_offset)."""
    arr, n = _seq_array(seqs)
    off = int(lib().sgqa_forward_diag_offset(ctypes.byref(cfg), arr, n))
    return off if off >= 0 else None


def index_diagnostics(ws: torch.Tensor, offset: int) -> dict:
    """Read the diagnostics block at `offset` of workspace `ws` (synchronises
    with the device): the number of rows scored again in full and the
    (query row, group) of the first 31 of them."""
    words = ws[offset:offset + 256].view(torch.int32).cpu().numpy()
    count = int(words[0])
    rows = [(int(words[2 + 2 * j]), int(words[3 + 2 * j])) for j in range(min(count, 31))]
    return {"rescored_rows": count, "rows": rows}


def sparse_attn(cfg: Config, seqs: Sequence[Seq], q, k_cache, v_cache, sel, out, lse=None,
                ws=None, stream=None) -> None:
    seqs = list(seqs)
    ext = _Extents(cfg, seqs)
    arr, n = _seq_array(seqs)
    ptrs = (_ptr(q, torch.bfloat16, "q", shape=ext.q()),
            _ptr(k_cache, torch.bfloat16, "k_cache", shape=ext.kv()),
            _ptr(v_cache, torch.bfloat16, "v_cache", shape=ext.kv()),
            _ptr(sel, torch.int32, "sel", shape=ext.sel()),
            _ptr(out, torch.bfloat16, "out", shape=ext.q()),
            _ptr(lse, torch.float32, "lse", False, shape=ext.lse()))
    ptrs = _addrs(ptrs)
    wsp, wsn, _own = _workspace(cfg, seqs, OP_SPARSE_ATTN, q.device, ws, stream)
    _check(lib().sgqa_sparse_attn(ctypes.byref(cfg), arr, n, *ptrs, wsp, wsn, _stream_ptr(stream)))


def _forward_ptrs(cfg, ext, proxy_k, comp_logits, ln_gamma, ln_beta, store, q_idx, w, rms_gamma, sel,
                  sel_scores, q, paged: bool):
    proxy_shape = ext.proxy_pages() if paged else ext.proxy()
    pname = ("proxy_pages", "logit_pages") if paged else ("proxy_k", "comp_logits")
    return (_ptr(proxy_k, torch.bfloat16, pname[0], shape=proxy_shape),
            _ptr(comp_logits, torch.float32, pname[1], shape=proxy_shape),
            _vec_ptr(ln_gamma, torch.bfloat16, "ln_gamma", ext.Di),
            _vec_ptr(ln_beta, torch.bfloat16, "ln_beta", ext.Di), _store_ptr(cfg, store, ext),
            _ptr(q_idx, torch.bfloat16, "q_idx", shape=ext.q_idx()),
            _ptr(w, torch.float32, "w", shape=ext.w()),
            _vec_ptr(rms_gamma, torch.bfloat16, "rms_gamma", ext.Di),
            _ptr(sel, torch.int32, "sel", shape=ext.sel()),
            _ptr(sel_scores, torch.float32, "sel_scores", False, shape=ext.sel()),
            _ptr(q, torch.bfloat16, "q", shape=ext.q()))


def forward(cfg: Config, seqs: Sequence[Seq], proxy_k, comp_logits, store, q_idx, w, sel, q,
            k_cache, v_cache, out, lse=None, sel_scores=None, ln_gamma=None, ln_beta=None,
            rms_gamma=None, ws=None, stream=None) -> None:
    seqs = list(seqs)
    ext = _Extents(cfg, seqs)
    arr, n = _seq_array(seqs)
    ptrs = _forward_ptrs(cfg, ext, proxy_k, comp_logits, ln_gamma, ln_beta, store, q_idx, w,
                         rms_gamma, sel, sel_scores, q, False) + (
        _ptr(k_cache, torch.bfloat16, "k_cache", shape=ext.kv()),
        _ptr(v_cache, torch.bfloat16, "v_cache", shape=ext.kv()),
        _ptr(out, torch.bfloat16, "out", shape=ext.q()),
        _ptr(lse, torch.float32, "lse", False, shape=ext.lse()))
    ptrs = _addrs(ptrs)
    wsp, wsn, _own = _workspace(cfg, seqs, OP_FORWARD, q.device, ws, stream)
    _check(lib().sgqa_forward(ctypes.byref(cfg), arr, n, *ptrs, wsp, wsn, _stream_ptr(stream)))


def forward_noalloc(cfg: Config, seqs: Sequence[Seq], proxy_k, comp_logits, store, q_idx, w, sel, q,
                    k_cache, v_cache, out, lse=None, sel_scores=None, ln_gamma=None, ln_beta=None,
                    rms_gamma=None, stream=None) -> None:
    """sgqa_forward on the library's static 64 MiB scratch: no workspace
    argument and nothing allocated (for callers that cannot allocate)."""
    seqs = list(seqs)
    ext = _Extents(cfg, seqs)
    arr, n = _seq_array(seqs)
    ptrs = _forward_ptrs(cfg, ext, proxy_k, comp_logits, ln_gamma, ln_beta, store, q_idx, w,
                         rms_gamma, sel, sel_scores, q, False) + (
        _ptr(k_cache, torch.bfloat16, "k_cache", shape=ext.kv()),
        _ptr(v_cache, torch.bfloat16, "v_cache", shape=ext.kv()),
        _ptr(out, torch.bfloat16, "out", shape=ext.q()),
        _ptr(lse, torch.float32, "lse", False, shape=ext.lse()))
    ptrs = _addrs(ptrs)
    _check(lib().sgqa_forward_noalloc(ctypes.byref(cfg), arr, n, *ptrs, _stream_ptr(stream)))


# ---------------------------------------------------------------------------
# paged caches: per-token tensors in pools of 16-position pages, a sequence's
# kv_offset indexing its first page-table entry (include/sgqa.h)
# ---------------------------------------------------------------------------

def _pages(page_table, pool, pools=()):
    """(table pointer, table length, page count); every pool in `pools` must
    have as many pages as `pool`.  Page ids are read on the device only,
    where an id outside [0, n_pages) is clamped into the pool."""
    ptp = _ptr(page_table, torch.int32, "page_table")
    if page_table.dim() != 1:
        raise ValueError("page_table must be one-dimensional")
    npg = int(pool.shape[0])
    for name, t in pools:
        if t is not None and int(t.shape[0]) != npg:
            raise ValueError(f"{name} has {int(t.shape[0])} pages, the pools have {npg}")
    return ptp, int(page_table.numel()), npg


def compress_paged(cfg: Config, seqs: Sequence[Seq], proxy_pages, logit_pages, page_table, store,
                   ln_gamma=None, ln_beta=None, stream=None) -> None:
    seqs = list(seqs)
    ext = _Extents(cfg, seqs)
    arr, n = _seq_array(seqs)
    ptrs = (_ptr(proxy_pages, torch.bfloat16, "proxy_pages", shape=ext.proxy_pages()),
            _ptr(logit_pages, torch.float32, "logit_pages", shape=ext.proxy_pages()))
    ptp, ptn, npg = _pages(page_table, proxy_pages, [("logit_pages", logit_pages)])
    rest = (_vec_ptr(ln_gamma, torch.bfloat16, "ln_gamma", ext.Di),
            _vec_ptr(ln_beta, torch.bfloat16, "ln_beta", ext.Di), _store_ptr(cfg, store, ext))
    ptrs, ptp, rest = _addrs(ptrs), _addrs([ptp])[0], _addrs(rest)
    _check(lib().sgqa_compress_paged(ctypes.byref(cfg), arr, n, *ptrs, ptp, ptn, npg, *rest, None, 0,
                                     _stream_ptr(stream)))


def sparse_attn_paged(cfg: Config, seqs: Sequence[Seq], q, k_pages, v_pages, page_table, sel, out,
                      lse=None, gate=None, ws=None, stream=None) -> None:
    seqs = list(seqs)
    ext = _Extents(cfg, seqs)
    arr, n = _seq_array(seqs)
    ptrs = (_ptr(q, torch.bfloat16, "q", shape=ext.q()),
            _ptr(k_pages, torch.bfloat16, "k_pages", shape=ext.kv_pages()),
            _ptr(v_pages, torch.bfloat16, "v_pages", shape=ext.kv_pages()))
    ptp, ptn, npg = _pages(page_table, k_pages, [("v_pages", v_pages)])
    rest = (_ptr(sel, torch.int32, "sel", shape=ext.sel()),
            _ptr(out, torch.bfloat16, "out", shape=ext.q()),
            _ptr(lse, torch.float32, "lse", False, shape=ext.lse()),
            _ptr(gate, torch.bfloat16, "gate", False, shape=ext.q()))
    ptrs, ptp, rest = _addrs(ptrs), _addrs([ptp])[0], _addrs(rest)
    wsp, wsn, _own = _workspace(cfg, seqs, OP_SPARSE_ATTN, q.device, ws, stream)
    _check(lib().sgqa_sparse_attn_paged(ctypes.byref(cfg), arr, n, *ptrs, ptp, ptn, npg, *rest,
                                        wsp, wsn, _stream_ptr(stream)))


def forward_paged(cfg: Config, seqs: Sequence[Seq], proxy_pages, logit_pages, store, q_idx, w, sel,
                  q, k_pages, v_pages, page_table, out, lse=None, sel_scores=None, ln_gamma=None,
                  ln_beta=None, rms_gamma=None, gate=None, ws=None, stream=None) -> None:
    seqs = list(seqs)
    ext = _Extents(cfg, seqs)
    arr, n = _seq_array(seqs)
    ptrs = _forward_ptrs(cfg, ext, proxy_pages, logit_pages, ln_gamma, ln_beta, store, q_idx, w,
                         rms_gamma, sel, sel_scores, q, True) + (
        _ptr(k_pages, torch.bfloat16, "k_pages", shape=ext.kv_pages()),
        _ptr(v_pages, torch.bfloat16, "v_pages", shape=ext.kv_pages()))
    ptp, ptn, npg = _pages(page_table, k_pages, [("v_pages", v_pages), ("proxy_pages", proxy_pages),
                                                 ("logit_pages", logit_pages)])
    rest = (_ptr(out, torch.bfloat16, "out", shape=ext.q()),
            _ptr(lse, torch.float32, "lse", False, shape=ext.lse()),
            _ptr(gate, torch.bfloat16, "gate", False, shape=ext.q()))
    ptrs, ptp, rest = _addrs(ptrs), _addrs([ptp])[0], _addrs(rest)
    wsp, wsn, _own = _workspace(cfg, seqs, OP_FORWARD, q.device, ws, stream)
    _check(lib().sgqa_forward_paged(ctypes.byref(cfg), arr, n, *ptrs, ptp, ptn, npg, *rest, wsp, wsn,
                                    _stream_ptr(stream)))


# ---------------------------------------------------------------------------
# the path's neighbours: main Q/K producer, sigmoid output gate
# ---------------------------------------------------------------------------

def qk_prep(cfg: Config, qk: QkConfig, seqs: Sequence[Seq], q_raw, k_raw, q_out, k_cache,
            v_raw=None, v_cache=None, q_gamma=None, k_gamma=None, page_table=None,
            stream=None) -> None:
    seqs = list(seqs)
    ext = _Extents(cfg, seqs)
    arr, n = _seq_array(seqs)
    raw_kv = (ext.q_rows, ext.G, ext.D)
    cache = ext.kv_pages() if page_table is not None else ext.kv()
    ptrs = (_ptr(q_raw, torch.bfloat16, "q_raw", shape=ext.q()),
            _ptr(k_raw, torch.bfloat16, "k_raw", shape=raw_kv),
            _ptr(v_raw, torch.bfloat16, "v_raw", False, shape=raw_kv),
            _vec_ptr(q_gamma, torch.bfloat16, "q_gamma", ext.D),
            _vec_ptr(k_gamma, torch.bfloat16, "k_gamma", ext.D),
            _ptr(q_out, torch.bfloat16, "q_out", shape=ext.q()),
            _ptr(k_cache, torch.bfloat16, "k_cache", shape=cache),
            _ptr(v_cache, torch.bfloat16, "v_cache", False, shape=cache))
    if page_table is not None:
        ptp, ptn, npg = _pages(page_table, k_cache, [("v_cache", v_cache)])
    else:
        ptp, ptn, npg = None, 0, 0
    ptrs, ptp = _addrs(ptrs), _addrs([ptp])[0]
    _check(lib().sgqa_qk_prep(ctypes.byref(cfg), ctypes.byref(qk), arr, n, *ptrs, ptp, ptn, npg,
                              _stream_ptr(stream)))


def sparse_attn_gated(cfg: Config, seqs: Sequence[Seq], q, k_cache, v_cache, sel, out, gate, lse=None,
                      ws=None, stream=None) -> None:
    seqs = list(seqs)
    ext = _Extents(cfg, seqs)
    arr, n = _seq_array(seqs)
    ptrs = (_ptr(q, torch.bfloat16, "q", shape=ext.q()),
            _ptr(k_cache, torch.bfloat16, "k_cache", shape=ext.kv()),
            _ptr(v_cache, torch.bfloat16, "v_cache", shape=ext.kv()),
            _ptr(sel, torch.int32, "sel", shape=ext.sel()),
            _ptr(out, torch.bfloat16, "out", shape=ext.q()),
            _ptr(lse, torch.float32, "lse", False, shape=ext.lse()),
            _ptr(gate, torch.bfloat16, "gate", shape=ext.q()))
    ptrs = _addrs(ptrs)
    wsp, wsn, _own = _workspace(cfg, seqs, OP_SPARSE_ATTN, q.device, ws, stream)
    _check(lib().sgqa_sparse_attn_gated(ctypes.byref(cfg), arr, n, *ptrs, wsp, wsn,
                                        _stream_ptr(stream)))


def forward_gated(cfg: Config, seqs: Sequence[Seq], proxy_k, comp_logits, store, q_idx, w, sel, q,
                  k_cache, v_cache, out, gate, lse=None, sel_scores=None, ln_gamma=None, ln_beta=None,
                  rms_gamma=None, ws=None, stream=None) -> None:
    seqs = list(seqs)
    ext = _Extents(cfg, seqs)
    arr, n = _seq_array(seqs)
    ptrs = _forward_ptrs(cfg, ext, proxy_k, comp_logits, ln_gamma, ln_beta, store, q_idx, w,
                         rms_gamma, sel, sel_scores, q, False) + (
        _ptr(k_cache, torch.bfloat16, "k_cache", shape=ext.kv()),
        _ptr(v_cache, torch.bfloat16, "v_cache", shape=ext.kv()),
        _ptr(out, torch.bfloat16, "out", shape=ext.q()),
        _ptr(lse, torch.float32, "lse", False, shape=ext.lse()),
        _ptr(gate, torch.bfloat16, "gate", shape=ext.q()))
    ptrs = _addrs(ptrs)
    wsp, wsn, _own = _workspace(cfg, seqs, OP_FORWARD, q.device, ws, stream)
    _check(lib().sgqa_forward_gated(ctypes.byref(cfg), arr, n, *ptrs, wsp, wsn, _stream_ptr(stream)))

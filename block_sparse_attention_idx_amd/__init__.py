"""MiniMax Sparse Attention (MSA) forward pass for AMD Instinct MI355X (gfx950).

A thin ctypes binding over the C ABI of ``libmsa.so`` (declared in
``include/msa.h``).  The Python layer only checks tensors, marshals pointers,
allocates the workspace through torch and passes torch's current HIP stream;
every step of the computation runs in the library's HIP kernels.  There is no
fallback: without the built library the calls raise.

Functions (same names as the C entry points):

* ``index_select(q_idx, k_idx, topk, q_offset=0)`` -> sel int32 [B, G, S_q, k]
* ``sparse_attn_fwd(q, k, v, sel, q_offset=0, scale=None, out_dtype=None,
  return_lse=False, k_scale=None, v_scale=None)`` -> out [B, S_q, Hq, d] (and
  lse fp32 [B, Hq, S_q])
* ``fwd(q, k, v, q_idx, k_idx, topk, q_offset=0, scale=None, out_dtype=None,
  return_sel=False, return_lse=False, k_scale=None, v_scale=None)``
* ``kl_teacher_fwd(q, k, q_idx, k_idx, sel, lse, q_offset=0, index_scale=1.0,
  return_idx_lse=False)`` -> KL fp32 [B, G, S_q] of the index distribution
  from the group-averaged main distribution (and the index log-sum-exp)
* ``sparse_attn_bwd(q, k, v, sel, out, lse, dout, q_offset=0)`` -> (dq, dk, dv)
  fp32, the main branch's gradients with the selection held constant (bf16)
* ``fwd_noalloc(q, k, v, q_idx, k_idx, topk, ..., out=None, sel=None, lse=None)``
  -> (out, sel, lse): ``fwd`` in the library's fixed scratch, no workspace

Layouts: q [B,S_q,Hq,d], k/v [B,Hkv,S_k,d], q_idx [B,S_q,G,D_idx],
k_idx [B,S_k,D_idx] with G = Hkv; all contiguous, on the GPU, fp32 or bf16.
The caches k, v and k_idx may instead be ``torch.float8_e4m3fn`` tensors (OCP
FP8 E4M3) next to bf16 q and q_idx; the keys and values attended to are then
``k_scale * k`` and ``v_scale * v``.

Caches of unequal length, optionally paged (``index_select_kvcache``,
``sparse_attn_fwd_kvcache``, ``fwd_kvcache``): ``seq_lens`` int32 [B] gives the
tokens of each sequence (query row i of sequence b sits at
``seq_lens[b] - S_q + i``); with ``page_table`` int32 [B, max_pages] the caches
are pools of 128-token pages, k/v [P, Hkv, 128, d] and k_idx [P, 128, D_idx].
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["index_select", "sparse_attn_fwd", "fwd", "index_select_kvcache", "sparse_attn_fwd_kvcache",
           "fwd_kvcache", "kl_teacher_fwd", "kl_teacher_fwd_kvcache", "workspace_size", "MsaShape", "MsaKvCache",
           "lib", "LIB_PATH", "MsaError", "OP_INDEX_SELECT", "OP_SPARSE_ATTN", "OP_FWD", "OP_KL_TEACHER",
           "sparse_attn_bwd", "OP_SPARSE_ATTN_BWD", "fwd_noalloc", "noalloc_scratch_bytes"]

# The in-tree build; MSA_LIBRARY may name another build of the same sources
# (the host-sanitizer build the ABI tests run under, say).
LIB_PATH = os.environ.get("MSA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsa.so")

MSA_F32, MSA_BF16 = 0, 1
CACHE_NATIVE, CACHE_FP8_E4M3 = 0, 1
OP_INDEX_SELECT, OP_SPARSE_ATTN, OP_FWD, OP_KL_TEACHER, OP_SPARSE_ATTN_BWD = 0, 1, 2, 3, 4
BLOCK_SIZE = 128


class MsaShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("kv_len", ctypes.c_int32),
        ("cache_format", ctypes.c_int32),
        ("q_offset", ctypes.c_int64),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("index_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("workspace_cap_mib", ctypes.c_int32),
    ]


class MsaKvCache(ctypes.Structure):
    _fields_ = [
        ("seq_lens", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("max_pages", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
    ]


class MsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded C library.  Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m block_sparse_attention_idx_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        shp = ctypes.POINTER(MsaShape)
        L.msa_workspace_size.argtypes = [shp, ctypes.c_int]
        L.msa_workspace_size.restype = sz
        L.msa_index_select.argtypes = [shp, vp, vp, vp, vp, sz, vp]
        L.msa_index_select.restype = ctypes.c_int
        L.msa_sparse_attn_fwd.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.msa_sparse_attn_fwd.restype = ctypes.c_int
        L.msa_fwd.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.msa_fwd.restype = ctypes.c_int
        L.msa_fwd_noalloc.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.msa_fwd_noalloc.restype = ctypes.c_int
        L.msa_noalloc_scratch_bytes.argtypes = []
        L.msa_noalloc_scratch_bytes.restype = sz
        L.msa_status_string.argtypes = [ctypes.c_int]
        L.msa_status_string.restype = ctypes.c_char_p
        L.msa_last_error.argtypes = []
        L.msa_last_error.restype = ctypes.c_char_p
        L.msa_version.argtypes = []
        L.msa_version.restype = ctypes.c_char_p
        L.msa_set_kernel_timer.argtypes = [ctypes.c_int, vp, vp]
        L.msa_set_kernel_timer.restype = ctypes.c_int
        cp = ctypes.POINTER(MsaKvCache)
        L.msa_workspace_size_kvcache.argtypes = [shp, cp, ctypes.c_int]
        L.msa_workspace_size_kvcache.restype = sz
        L.msa_index_select_kvcache.argtypes = [shp, cp, vp, vp, vp, vp, sz, vp]
        L.msa_index_select_kvcache.restype = ctypes.c_int
        L.msa_sparse_attn_fwd_kvcache.argtypes = [shp, cp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.msa_sparse_attn_fwd_kvcache.restype = ctypes.c_int
        L.msa_fwd_kvcache.argtypes = [shp, cp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.msa_fwd_kvcache.restype = ctypes.c_int
        fl = ctypes.c_float
        L.msa_kl_teacher_fwd.argtypes = [shp, vp, vp, vp, vp, vp, vp, fl, vp, vp, vp, sz, vp]
        L.msa_kl_teacher_fwd.restype = ctypes.c_int
        L.msa_kl_teacher_fwd_kvcache.argtypes = [shp, cp, vp, vp, vp, vp, vp, vp, fl, vp, vp, vp, sz, vp]
        L.msa_kl_teacher_fwd_kvcache.restype = ctypes.c_int
        L.msa_sparse_attn_bwd.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.msa_sparse_attn_bwd.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return MSA_F32
    if dt == torch.bfloat16:
        return MSA_BF16
    raise TypeError(f"unsupported dtype {dt}: fp32 or bf16")


def make_shape(B, S_q, S_k, q_offset, Hq, Hkv, d, D_idx, topk, dtype, out_dtype=None, scale=None,
               block_size=BLOCK_SIZE, cache_format=CACHE_NATIVE, k_scale=None, v_scale=None,
               workspace_cap_mib=0) -> MsaShape:
    s = MsaShape()
    s.batch, s.q_len, s.kv_len, s.cache_format = B, S_q, S_k, cache_format
    s.q_offset = q_offset
    s.num_q_heads, s.num_kv_heads = Hq, Hkv
    s.head_dim, s.index_dim = d, D_idx
    s.block_size, s.topk = block_size, topk
    s.softmax_scale = 0.0 if scale is None else float(scale)
    s.dtype = _dtype_code(dtype)
    s.out_dtype = _dtype_code(out_dtype if out_dtype is not None else dtype)
    s.k_scale = 0.0 if k_scale is None else float(k_scale)
    s.v_scale = 0.0 if v_scale is None else float(v_scale)
    s.workspace_cap_mib = int(workspace_cap_mib)
    return s


def _cache_format(q_dtype: torch.dtype, caches) -> int:
    """Cache tensors share q's dtype, or are all float8_e4m3fn next to bf16 q."""
    dts = {t.dtype for _, t in caches}
    if dts == {q_dtype}:
        return CACHE_NATIVE
    if dts == {torch.float8_e4m3fn} and q_dtype == torch.bfloat16:
        return CACHE_FP8_E4M3
    names = ", ".join(f"{n} {t.dtype}" for n, t in caches)
    raise ValueError(f"caches ({names}) must all have q's dtype {q_dtype}, or all be float8_e4m3fn with bf16 q")


def _check(st: int):
    if st != 0:
        L = lib()
        raise MsaError(st, f"{L.msa_status_string(st).decode()}: {L.msa_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, ndim: int, device=None, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def workspace_size(shape: MsaShape, op: int) -> int:
    return int(lib().msa_workspace_size(ctypes.byref(shape), op))


def _aligned(n: int, device) -> Optional[torch.Tensor]:
    """A 256-byte aligned device buffer of n bytes (None for 0)."""
    if n == 0:
        return None
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + n]


def _workspace(shape: MsaShape, op: int, device) -> Optional[torch.Tensor]:
    return _aligned(workspace_size(shape, op), device)


def index_select(q_idx: torch.Tensor, k_idx: torch.Tensor, topk: int, q_offset: int = 0,
                 sel: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-group block selection, int32 [B, G, S_q, topk] (ascending ids, -1 padded)."""
    _need(q_idx, "q_idx", 4)
    dev = q_idx.device
    _need(k_idx, "k_idx", 3, dev)
    cf = _cache_format(q_idx.dtype, [("k_idx", k_idx)])
    B, S_q, G, D = q_idx.shape
    if k_idx.shape[0] != B or k_idx.shape[2] != D:
        raise ValueError("k_idx must be [B, S_k, D_idx] matching q_idx")
    S_k = k_idx.shape[1]
    shape = make_shape(B, S_q, S_k, q_offset, G, G, 64, D, topk, q_idx.dtype, cache_format=cf)
    if sel is None:
        sel = torch.empty((B, G, S_q, topk), dtype=torch.int32, device=dev)
    else:
        _need(sel, "sel", 4, dev, torch.int32)
    ws = workspace if workspace is not None else _workspace(shape, OP_INDEX_SELECT, dev)
    L = lib()
    st = L.msa_index_select(ctypes.byref(shape), _ptr(q_idx), _ptr(k_idx), _ptr(sel), _ptr(ws),
                            0 if ws is None else ws.numel(), _stream(dev))
    _check(st)
    return sel


def sparse_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sel: torch.Tensor, q_offset: int = 0,
                    scale: Optional[float] = None, out_dtype: Optional[torch.dtype] = None,
                    return_lse: bool = False, workspace: Optional[torch.Tensor] = None,
                    k_scale: Optional[float] = None, v_scale: Optional[float] = None):
    """Exact softmax attention over the selected blocks."""
    _need(q, "q", 4)
    dev = q.device
    _need(k, "k", 4, dev)
    _need(v, "v", 4, dev)
    cf = _cache_format(q.dtype, [("k", k), ("v", v)])
    _need(sel, "sel", 4, dev, torch.int32)
    B, S_q, Hq, d = q.shape
    Hkv, S_k = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, S_k, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B, Hkv, S_k, d] matching q")
    topk = sel.shape[3]
    if tuple(sel.shape[:3]) != (B, Hkv, S_q):
        raise ValueError("sel must be [B, G, S_q, topk]")
    shape = make_shape(B, S_q, S_k, q_offset, Hq, Hkv, d, 32, topk, q.dtype, out_dtype, scale,
                       cache_format=cf, k_scale=k_scale, v_scale=v_scale)
    out = torch.empty((B, S_q, Hq, d), dtype=out_dtype or q.dtype, device=dev)
    lse = torch.empty((B, Hq, S_q), dtype=torch.float32, device=dev) if return_lse else None
    ws = workspace if workspace is not None else _workspace(shape, OP_SPARSE_ATTN, dev)
    L = lib()
    st = L.msa_sparse_attn_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(sel), _ptr(out), _ptr(lse),
                               _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev))
    _check(st)
    return (out, lse) if return_lse else out


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_idx: torch.Tensor, k_idx: torch.Tensor, topk: int,
        q_offset: int = 0, scale: Optional[float] = None, out_dtype: Optional[torch.dtype] = None,
        return_sel: bool = False, return_lse: bool = False, workspace: Optional[torch.Tensor] = None,
        k_scale: Optional[float] = None, v_scale: Optional[float] = None):
    """Index branch and main branch.  Returns out, plus sel and/or lse when asked."""
    _need(q, "q", 4)
    dev = q.device
    _need(q_idx, "q_idx", 4, dev, q.dtype)
    for name, t, nd in (("k", k, 4), ("v", v, 4), ("k_idx", k_idx, 3)):
        _need(t, name, nd, dev)
    cf = _cache_format(q.dtype, [("k", k), ("v", v), ("k_idx", k_idx)])
    B, S_q, Hq, d = q.shape
    Hkv, S_k = k.shape[1], k.shape[2]
    D = q_idx.shape[3]
    if tuple(k.shape) != (B, Hkv, S_k, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B, Hkv, S_k, d] matching q")
    if tuple(q_idx.shape) != (B, S_q, Hkv, D) or tuple(k_idx.shape) != (B, S_k, D):
        raise ValueError("q_idx must be [B, S_q, Hkv, D_idx] and k_idx [B, S_k, D_idx]")
    shape = make_shape(B, S_q, S_k, q_offset, Hq, Hkv, d, D, topk, q.dtype, out_dtype, scale,
                       cache_format=cf, k_scale=k_scale, v_scale=v_scale)
    out = torch.empty((B, S_q, Hq, d), dtype=out_dtype or q.dtype, device=dev)
    sel = torch.empty((B, Hkv, S_q, topk), dtype=torch.int32, device=dev) if return_sel else None
    lse = torch.empty((B, Hq, S_q), dtype=torch.float32, device=dev) if return_lse else None
    ws = workspace if workspace is not None else _workspace(shape, OP_FWD, dev)
    L = lib()
    st = L.msa_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(q_idx), _ptr(k_idx), _ptr(out), _ptr(sel),
                   _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev))
    _check(st)
    res = [out]
    if return_sel:
        res.append(sel)
    if return_lse:
        res.append(lse)
    return res[0] if len(res) == 1 else tuple(res)


def fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_idx: torch.Tensor, k_idx: torch.Tensor,
                topk: int, q_offset: int = 0, scale: Optional[float] = None, out_dtype: Optional[torch.dtype] = None,
                out: Optional[torch.Tensor] = None, sel: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, k_scale: Optional[float] = None, v_scale: Optional[float] = None):
    """msa_fwd_noalloc: fwd without a workspace (the library's fixed scratch).  The
    outputs may be passed in (then nothing at all is allocated); returns (out, sel, lse)."""
    _need(q, "q", 4)
    dev = q.device
    _need(q_idx, "q_idx", 4, dev, q.dtype)
    for name, t, nd in (("k", k, 4), ("v", v, 4), ("k_idx", k_idx, 3)):
        _need(t, name, nd, dev)
    cf = _cache_format(q.dtype, [("k", k), ("v", v), ("k_idx", k_idx)])
    B, S_q, Hq, d = q.shape
    Hkv, S_k = k.shape[1], k.shape[2]
    D = q_idx.shape[3]
    if tuple(k.shape) != (B, Hkv, S_k, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B, Hkv, S_k, d] matching q")
    if tuple(q_idx.shape) != (B, S_q, Hkv, D) or tuple(k_idx.shape) != (B, S_k, D):
        raise ValueError("q_idx must be [B, S_q, Hkv, D_idx] and k_idx [B, S_k, D_idx]")
    shape = make_shape(B, S_q, S_k, q_offset, Hq, Hkv, d, D, topk, q.dtype, out_dtype, scale,
                       cache_format=cf, k_scale=k_scale, v_scale=v_scale)
    if out is None:
        out = torch.empty((B, S_q, Hq, d), dtype=out_dtype or q.dtype, device=dev)
    _need(out, "out", 4, dev)
    if tuple(out.shape) != (B, S_q, Hq, d):
        raise ValueError("out must be [B, S_q, Hq, d]")
    for name, t, shp, dt in (("sel", sel, (B, Hkv, S_q, topk), torch.int32), ("lse", lse, (B, Hq, S_q), torch.float32)):
        if t is not None:
            _need(t, name, len(shp), dev, dt)
            if tuple(t.shape) != shp:
                raise ValueError(f"{name} must be {list(shp)}")
    L = lib()
    st = L.msa_fwd_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(q_idx), _ptr(k_idx), _ptr(out),
                           _ptr(sel), _ptr(lse), _stream(dev))
    _check(st)
    return out, sel, lse


def noalloc_scratch_bytes() -> int:
    """Bytes of the scratch msa_fwd_noalloc works in."""
    return int(lib().msa_noalloc_scratch_bytes())


# ---- caches of unequal length, optionally paged ----------------------------

def _kv_cache(B: int, dev, seq_lens, page_table, num_pages: int):
    """The MsaKvCache descriptor (or None) and its max_pages."""
    if seq_lens is None and page_table is None:
        return None, 0
    c = MsaKvCache()
    if seq_lens is not None:
        _need(seq_lens, "seq_lens", 1, dev, torch.int32)
        if seq_lens.shape[0] != B:
            raise ValueError(f"seq_lens must have {B} entries")
        c.seq_lens = seq_lens.data_ptr()
    max_pages = 0
    if page_table is not None:
        _need(page_table, "page_table", 2, dev, torch.int32)
        if page_table.shape[0] != B:
            raise ValueError(f"page_table must have {B} rows")
        max_pages = page_table.shape[1]
        c.page_table = page_table.data_ptr()
        c.max_pages, c.num_pages = max_pages, num_pages
    return c, max_pages


def _kv_geometry(k: torch.Tensor, k_idx: Optional[torch.Tensor], B: int, page_table, kv_len):
    """(Hkv, kv_len, num_pages) of dense [B, Hkv, S_k, d] or paged [P, Hkv, 128, d] caches."""
    if page_table is not None:
        P, Hkv, blk = k.shape[0], k.shape[1], k.shape[2]
        if blk != BLOCK_SIZE:
            raise ValueError(f"paged k/v must be [P, Hkv, {BLOCK_SIZE}, d]")
        if k_idx is not None and (k_idx.shape[0] != P or k_idx.shape[1] != BLOCK_SIZE):
            raise ValueError(f"paged k_idx must be [P, {BLOCK_SIZE}, D_idx]")
        return Hkv, (kv_len if kv_len is not None else page_table.shape[1] * BLOCK_SIZE), P
    if k.shape[0] != B:
        raise ValueError("dense k/v must be [B, Hkv, S_k, d]")
    if k_idx is not None and k_idx.shape[:2] != (B, k.shape[2]):
        raise ValueError("dense k_idx must be [B, S_k, D_idx]")
    return k.shape[1], k.shape[2], 0


def index_select_kvcache(q_idx: torch.Tensor, k_idx: torch.Tensor, topk: int, seq_lens=None, page_table=None,
                         kv_len: Optional[int] = None, q_offset: int = 0, sel: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """index_select over caches of unequal length and/or in pages."""
    _need(q_idx, "q_idx", 4)
    dev = q_idx.device
    _need(k_idx, "k_idx", 3, dev)
    cf = _cache_format(q_idx.dtype, [("k_idx", k_idx)])
    B, S_q, G, D = q_idx.shape
    if k_idx.shape[2] != D:
        raise ValueError("k_idx must end in D_idx like q_idx")
    if page_table is not None:
        P = k_idx.shape[0]
        if k_idx.shape[1] != BLOCK_SIZE:
            raise ValueError(f"paged k_idx must be [P, {BLOCK_SIZE}, D_idx]")
        S_k = kv_len if kv_len is not None else page_table.shape[1] * BLOCK_SIZE
    else:
        P = 0
        if k_idx.shape[0] != B:
            raise ValueError("dense k_idx must be [B, S_k, D_idx]")
        S_k = k_idx.shape[1]
    cache, _ = _kv_cache(B, dev, seq_lens, page_table, P)
    shape = make_shape(B, S_q, S_k, q_offset, G, G, 64, D, topk, q_idx.dtype, cache_format=cf)
    if sel is None:
        sel = torch.empty((B, G, S_q, topk), dtype=torch.int32, device=dev)
    else:
        _need(sel, "sel", 4, dev, torch.int32)
    L = lib()
    cref = ctypes.byref(cache) if cache is not None else None
    if workspace is None:
        n = int(L.msa_workspace_size_kvcache(ctypes.byref(shape), cref, OP_INDEX_SELECT))
        workspace = _aligned(n, dev)
    st = L.msa_index_select_kvcache(ctypes.byref(shape), cref, _ptr(q_idx), _ptr(k_idx), _ptr(sel),
                                    _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(dev))
    _check(st)
    return sel


def sparse_attn_fwd_kvcache(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sel: torch.Tensor, seq_lens=None,
                            page_table=None, kv_len: Optional[int] = None, q_offset: int = 0,
                            scale: Optional[float] = None, out_dtype: Optional[torch.dtype] = None,
                            return_lse: bool = False, k_scale: Optional[float] = None,
                            v_scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None):
    """sparse_attn_fwd over caches of unequal length and/or in pages."""
    _need(q, "q", 4)
    dev = q.device
    _need(k, "k", 4, dev)
    _need(v, "v", 4, dev)
    cf = _cache_format(q.dtype, [("k", k), ("v", v)])
    _need(sel, "sel", 4, dev, torch.int32)
    B, S_q, Hq, d = q.shape
    if tuple(v.shape) != tuple(k.shape) or k.shape[3] != d:
        raise ValueError("k and v must match and end in d")
    Hkv, S_k, P = _kv_geometry(k, None, B, page_table, kv_len)
    topk = sel.shape[3]
    if tuple(sel.shape[:3]) != (B, Hkv, S_q):
        raise ValueError("sel must be [B, G, S_q, topk]")
    cache, _ = _kv_cache(B, dev, seq_lens, page_table, P)
    shape = make_shape(B, S_q, S_k, q_offset, Hq, Hkv, d, 32, topk, q.dtype, out_dtype, scale,
                       cache_format=cf, k_scale=k_scale, v_scale=v_scale)
    out = torch.empty((B, S_q, Hq, d), dtype=out_dtype or q.dtype, device=dev)
    lse = torch.empty((B, Hq, S_q), dtype=torch.float32, device=dev) if return_lse else None
    L = lib()
    cref = ctypes.byref(cache) if cache is not None else None
    if workspace is None:
        n = int(L.msa_workspace_size_kvcache(ctypes.byref(shape), cref, OP_SPARSE_ATTN))
        workspace = _aligned(n, dev)
    st = L.msa_sparse_attn_fwd_kvcache(ctypes.byref(shape), cref, _ptr(q), _ptr(k), _ptr(v), _ptr(sel), _ptr(out),
                                       _ptr(lse), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                       _stream(dev))
    _check(st)
    return (out, lse) if return_lse else out


def fwd_kvcache(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_idx: torch.Tensor, k_idx: torch.Tensor,
                topk: int, seq_lens=None, page_table=None, kv_len: Optional[int] = None, q_offset: int = 0,
                scale: Optional[float] = None, out_dtype: Optional[torch.dtype] = None, return_sel: bool = False,
                return_lse: bool = False, k_scale: Optional[float] = None, v_scale: Optional[float] = None,
                workspace: Optional[torch.Tensor] = None):
    """fwd over caches of unequal length and/or in pages."""
    _need(q, "q", 4)
    dev = q.device
    _need(q_idx, "q_idx", 4, dev, q.dtype)
    for name, t, nd in (("k", k, 4), ("v", v, 4), ("k_idx", k_idx, 3)):
        _need(t, name, nd, dev)
    cf = _cache_format(q.dtype, [("k", k), ("v", v), ("k_idx", k_idx)])
    B, S_q, Hq, d = q.shape
    if tuple(v.shape) != tuple(k.shape) or k.shape[3] != d:
        raise ValueError("k and v must match and end in d")
    Hkv, S_k, P = _kv_geometry(k, k_idx, B, page_table, kv_len)
    D = q_idx.shape[3]
    if tuple(q_idx.shape) != (B, S_q, Hkv, D) or k_idx.shape[2] != D:
        raise ValueError("q_idx must be [B, S_q, Hkv, D_idx] and k_idx end in D_idx")
    cache, _ = _kv_cache(B, dev, seq_lens, page_table, P)
    shape = make_shape(B, S_q, S_k, q_offset, Hq, Hkv, d, D, topk, q.dtype, out_dtype, scale,
                       cache_format=cf, k_scale=k_scale, v_scale=v_scale)
    out = torch.empty((B, S_q, Hq, d), dtype=out_dtype or q.dtype, device=dev)
    sel = torch.empty((B, Hkv, S_q, topk), dtype=torch.int32, device=dev) if return_sel else None
    lse = torch.empty((B, Hq, S_q), dtype=torch.float32, device=dev) if return_lse else None
    L = lib()
    cref = ctypes.byref(cache) if cache is not None else None
    if workspace is None:
        n = int(L.msa_workspace_size_kvcache(ctypes.byref(shape), cref, OP_FWD))
        workspace = _aligned(n, dev)
    st = L.msa_fwd_kvcache(ctypes.byref(shape), cref, _ptr(q), _ptr(k), _ptr(v), _ptr(q_idx), _ptr(k_idx),
                           _ptr(out), _ptr(sel), _ptr(lse), _ptr(workspace),
                           0 if workspace is None else workspace.numel(), _stream(dev))
    _check(st)
    res = [out]
    if return_sel:
        res.append(sel)
    if return_lse:
        res.append(lse)
    return res[0] if len(res) == 1 else tuple(res)


# ---- KL-alignment teacher (forward only) ------------------------------------

def kl_teacher_fwd_kvcache(q: torch.Tensor, k: torch.Tensor, q_idx: torch.Tensor, k_idx: torch.Tensor,
                           sel: torch.Tensor, lse: torch.Tensor, seq_lens=None, page_table=None,
                           kv_len: Optional[int] = None, q_offset: int = 0, scale: Optional[float] = None,
                           index_scale: float = 1.0, k_scale: Optional[float] = None, return_idx_lse: bool = False,
                           workspace: Optional[torch.Tensor] = None):
    """KL(group-averaged main distribution || index distribution) per (b, g, i),
    fp32 [B, G, S_q], from the forward's selection and lse; with return_idx_lse
    also the index log-sum-exp over the same tokens."""
    _need(q, "q", 4)
    dev = q.device
    _need(q_idx, "q_idx", 4, dev, q.dtype)
    _need(k, "k", 4, dev)
    _need(k_idx, "k_idx", 3, dev)
    cf = _cache_format(q.dtype, [("k", k), ("k_idx", k_idx)])
    _need(sel, "sel", 4, dev, torch.int32)
    _need(lse, "lse", 3, dev, torch.float32)
    B, S_q, Hq, d = q.shape
    if k.shape[3] != d:
        raise ValueError("k must end in d")
    Hkv, S_k, P = _kv_geometry(k, k_idx, B, page_table, kv_len)
    D = q_idx.shape[3]
    if tuple(q_idx.shape) != (B, S_q, Hkv, D) or k_idx.shape[2] != D:
        raise ValueError("q_idx must be [B, S_q, Hkv, D_idx] and k_idx end in D_idx")
    topk = sel.shape[3]
    if tuple(sel.shape[:3]) != (B, Hkv, S_q) or tuple(lse.shape) != (B, Hq, S_q):
        raise ValueError("sel must be [B, G, S_q, topk] and lse [B, Hq, S_q]")
    cache, _ = _kv_cache(B, dev, seq_lens, page_table, P)
    shape = make_shape(B, S_q, S_k, q_offset, Hq, Hkv, d, D, topk, q.dtype, None, scale,
                       cache_format=cf, k_scale=k_scale)
    kl = torch.empty((B, Hkv, S_q), dtype=torch.float32, device=dev)
    ilse = torch.empty((B, Hkv, S_q), dtype=torch.float32, device=dev) if return_idx_lse else None
    L = lib()
    cref = ctypes.byref(cache) if cache is not None else None
    if workspace is None:
        n = int(L.msa_workspace_size_kvcache(ctypes.byref(shape), cref, OP_KL_TEACHER))
        workspace = _aligned(n, dev)
    st = L.msa_kl_teacher_fwd_kvcache(ctypes.byref(shape), cref, _ptr(q), _ptr(k), _ptr(q_idx), _ptr(k_idx),
                                      _ptr(sel), _ptr(lse), float(index_scale), _ptr(kl), _ptr(ilse),
                                      _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(dev))
    _check(st)
    return (kl, ilse) if return_idx_lse else kl


def kl_teacher_fwd(q, k, q_idx, k_idx, sel, lse, q_offset: int = 0, scale: Optional[float] = None,
                   index_scale: float = 1.0, k_scale: Optional[float] = None, return_idx_lse: bool = False,
                   workspace: Optional[torch.Tensor] = None):
    """kl_teacher_fwd_kvcache over dense caches of kv_len tokens each."""
    return kl_teacher_fwd_kvcache(q, k, q_idx, k_idx, sel, lse, q_offset=q_offset, scale=scale,
                                  index_scale=index_scale, k_scale=k_scale, return_idx_lse=return_idx_lse,
                                  workspace=workspace)


# ---- backward of the main branch ------------------------------------------------

def sparse_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sel: torch.Tensor, out: torch.Tensor,
                    lse: torch.Tensor, dout: torch.Tensor, q_offset: int = 0, scale: Optional[float] = None,
                    workspace: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv), fp32, of sparse_attn_fwd's output for the output
    gradient dout, the selection held constant; out and lse are the forward's."""
    _need(q, "q", 4, dtype=torch.bfloat16)
    dev = q.device
    for name, t in (("k", k), ("v", v), ("out", out), ("dout", dout)):
        _need(t, name, 4, dev, torch.bfloat16)
    _need(sel, "sel", 4, dev, torch.int32)
    _need(lse, "lse", 3, dev, torch.float32)
    B, S_q, Hq, d = q.shape
    Hkv, S_k = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, S_k, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B, Hkv, S_k, d] matching q")
    if tuple(out.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("out and dout must be shaped like q")
    topk = sel.shape[3]
    if tuple(sel.shape[:3]) != (B, Hkv, S_q) or tuple(lse.shape) != (B, Hq, S_q):
        raise ValueError("sel must be [B, G, S_q, topk] and lse [B, Hq, S_q]")
    shape = make_shape(B, S_q, S_k, q_offset, Hq, Hkv, d, 32, topk, torch.bfloat16, torch.bfloat16, scale)
    dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
    dk = torch.empty(k.shape, dtype=torch.float32, device=dev)
    dv = torch.empty(v.shape, dtype=torch.float32, device=dev)
    ws = workspace if workspace is not None else _workspace(shape, OP_SPARSE_ATTN_BWD, dev)
    L = lib()
    st = L.msa_sparse_attn_bwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(sel), _ptr(out), _ptr(lse),
                               _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), 0 if ws is None else ws.numel(),
                               _stream(dev))
    _check(st)
    return dq, dk, dv

"""ctypes binding of libmsa (include/msa.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  torch is used for device memory and the current stream.  The
binding raises if libmsa.so has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsa.so")

MSA_BF16, MSA_FP32, MSA_FP8_E4M3, MSA_MXFP8_E4M3 = 0, 1, 2, 3
MSA_POOL_MAX, MSA_POOL_MEAN = 0, 1
OP_INDEX, OP_PREFILL, OP_DECODE, OP_DENSE, OP_INDEX_DECODE, OP_PREFILL_BACKWARD, OP_PREFILL_BACKWARD_KL = \
    0, 1, 2, 3, 4, 5, 6
OP_INDEX_PROJECT = 7
BLOCK = 128


class MsaError(RuntimeError):
    """A libmsa call returned a non-zero msa_status."""

    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}")
        self.status = status
        self.name = name
        self.detail = detail


class Shape(ctypes.Structure):
    _fields_ = [("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32), ("d_h", ctypes.c_int32),
                ("d_idx", ctypes.c_int32), ("block_size", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("force_local", ctypes.c_int32), ("sm_scale", ctypes.c_float),
                ("idx_scale", ctypes.c_float), ("dtype", ctypes.c_int32), ("cache_dtype", ctypes.c_int32),
                ("pool", ctypes.c_int32)]


class KL(ctypes.Structure):
    _fields_ = [("q_idx", ctypes.c_void_p), ("k_idx", ctypes.c_void_p), ("kl_scale", ctypes.c_float),
                ("kl_out", ctypes.c_void_p), ("dq_idx", ctypes.c_void_p), ("dk_idx", ctypes.c_void_p)]


class KV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("k_idx", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("n_kv", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p), ("k_idx_scale", ctypes.c_void_p)]


_lib = None

EXPORTS = ["msa_index_topk", "msa_sparse_prefill", "msa_sparse_decode", "msa_dense_prefill",
           "msa_sparse_prefill_backward", "msa_index_project",
           "msa_workspace_size", "msa_status_string", "msa_last_error", "msa_abi_version",
           "msa_profile_enable", "msa_profile_read", "msa_probe_mfma", "msa_test_schedule_lds_limit",
           "msa_index_topk_decode_static"]


def lib() -> ctypes.CDLL:
    """Load libmsa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_attention_branch_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        P = ctypes.POINTER
        L.msa_index_topk.argtypes = [P(Shape), i32, i32, i32, vp, P(KV), vp, vp, vp, sz, vp]
        L.msa_index_topk_decode_static.argtypes = [P(Shape), i32, vp, P(KV), vp, vp, vp]
        L.msa_sparse_prefill.argtypes = [P(Shape), i32, i32, vp, P(KV), vp, vp, vp, vp, sz, vp]
        L.msa_sparse_decode.argtypes = [P(Shape), i32, vp, P(KV), vp, vp, vp, vp, sz, vp]
        L.msa_dense_prefill.argtypes = [P(Shape), i32, i32, vp, P(KV), vp, vp, vp, sz, vp]
        L.msa_sparse_prefill_backward.argtypes = [P(Shape), i32, i32, vp, P(KV), vp, vp, vp, vp, vp, vp, vp,
                                                  P(KL), vp, sz, vp]
        L.msa_index_project.argtypes = [P(Shape), i32, i32, vp, vp, vp, i32, ctypes.c_float, vp, vp, P(KV), vp, vp,
                                        ctypes.c_size_t, vp]
        for f in ("msa_index_topk", "msa_index_topk_decode_static", "msa_sparse_prefill", "msa_sparse_decode", "msa_dense_prefill",
                  "msa_sparse_prefill_backward", "msa_index_project"):
            getattr(L, f).restype = ctypes.c_int
        L.msa_workspace_size.argtypes = [i32, P(Shape), i32, i32, i32, i32, i32]
        L.msa_workspace_size.restype = sz
        L.msa_status_string.argtypes = [ctypes.c_int]
        L.msa_status_string.restype = ctypes.c_char_p
        L.msa_last_error.argtypes = []
        L.msa_last_error.restype = ctypes.c_char_p
        L.msa_abi_version.restype = ctypes.c_int32
        L.msa_profile_enable.argtypes = [i32]
        L.msa_profile_enable.restype = ctypes.c_int
        L.msa_profile_read.argtypes = [ctypes.c_char_p, P(ctypes.c_double), P(ctypes.c_int64)]
        L.msa_profile_read.restype = ctypes.c_int
        L.msa_probe_mfma.argtypes = [i32, i32, P(ctypes.c_float), ctypes.c_void_p]
        L.msa_probe_mfma.restype = ctypes.c_int
        L.msa_test_schedule_lds_limit.argtypes = [i32]
        L.msa_test_schedule_lds_limit.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        L = lib()
        raise MsaError(status, L.msa_status_string(status).decode(), L.msa_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MSA_BF16
    if t.dtype == torch.float32:
        return MSA_FP32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def make_shape(h_q, h_kv, d_h, d_idx, top_k, dtype_code, *, force_local=True,
               sm_scale=0.0, idx_scale=0.0, cache_dtype=None, pool=None) -> Shape:
    cd = int(dtype_code) if cache_dtype is None else int(cache_dtype)
    return Shape(int(h_q), int(h_kv), int(d_h), int(d_idx), BLOCK, int(top_k),
                 1 if force_local else 0, float(sm_scale), float(idx_scale), int(dtype_code), cd,
                 _pool_code(pool))


def _pool_code(pool) -> int:
    if pool is None or pool == "max":
        return MSA_POOL_MAX
    if pool == "mean":
        return MSA_POOL_MEAN
    return int(pool)


def _cache_code(t: torch.Tensor, compute_code: int, scale=None) -> int:
    """Cache dtype of a k/v/k_idx tensor: MXFP8 (float8_e4m3fn codes with a
    uint8 E8M0 scale tensor), e4m3 (float8_e4m3fn without one) or the call's
    dtype."""
    if t is not None and t.dtype == torch.float8_e4m3fn:
        return MSA_FP8_E4M3 if scale is None else MSA_MXFP8_E4M3
    return compute_code


def workspace_size(op: int, shape: Shape, *, batch=1, n_q=0, q_start=0, n_kv=0, max_pages=0) -> int:
    L = lib()
    n = L.msa_workspace_size(op, ctypes.byref(shape), batch, n_q, q_start, n_kv, max_pages)
    err = L.msa_last_error().decode()
    if err:
        raise MsaError(1, "MSA_ERR_INVALID_ARG", err)
    return int(n)


def _workspace(nbytes: int, device, ws):
    if nbytes == 0:
        return None
    if ws is not None and ws.numel() >= nbytes:
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- timing

def profile_enable(on: bool = True) -> None:
    """msa_profile_enable: bracket every launch of the timed kernels with HIP
    events on the launch stream (measurement only)."""
    _check(lib().msa_profile_enable(1 if on else 0))


def probe_mfma(n_wg: int, iters: int, out, stream=None) -> None:
    """msa_probe_mfma: n_wg * 4 * iters * 8 bf16 32x32x16 MFMAs (measurement only);
    ``out`` is a float32 device tensor of n_wg elements."""
    _check(lib().msa_probe_mfma(int(n_wg), int(iters), ctypes.cast(out.data_ptr(), ctypes.POINTER(ctypes.c_float)),
                                _stream(stream)))


def test_schedule_lds_limit(max_blocks: int) -> None:
    """msa_test_schedule_lds_limit (test hook): cap the block count whose
    prefill schedule counters live in LDS (0 forces global atomics, < 0
    restores the built-in limits)."""
    _check(lib().msa_test_schedule_lds_limit(int(max_blocks)))


def profile_read(kernel: str):
    """msa_profile_read: (summed GPU ms, launches) of `kernel` since the last read."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
    _check(lib().msa_profile_read(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


# ---------------------------------------------------------------- calls

def index_topk(q_idx, k_idx, *, top_k=16, q_start=0, force_local=True, idx_scale=0.0,
               page_table=None, n_kv=None, seq_lens=None, max_pages=None, h_q=None,
               with_scores=False, out=None, workspace=None, stream=None, pool="max", k_idx_scale=None):
    """msa_index_topk (``pool``: "max", the method's block max-pool, or "mean").  Prefill mode: q_idx [n_q, h_kv, d_idx], k_idx
    [n_kv, d_idx] (or pages [*, 128, d_idx] with ``page_table``).  Decode mode
    (``seq_lens`` given): q_idx [batch, h_kv, d_idx], one query per sequence.
    An MXFP8 k_idx is its float8_e4m3fn codes plus ``k_idx_scale`` (uint8,
    last dim d_idx / 32).  Returns block_idx int32 [rows, h_kv, top_k] (and
    fp32 scores)."""
    decode = seq_lens is not None
    if decode:
        batch, h_kv, d_idx = q_idx.shape
        n_q, qs = 1, 0
        rows = batch
        mp = page_table.shape[1]
        nkv = 0
    else:
        n_q, h_kv, d_idx = q_idx.shape
        batch, qs, rows = 1, int(q_start), n_q
        nkv = int(n_kv) if n_kv is not None else (k_idx.shape[0] if page_table is None else None)
        if nkv is None:
            raise ValueError("n_kv is required with a paged k_idx")
        mp = page_table.numel() if page_table is not None else 0
    if max_pages is not None:
        mp = int(max_pages)
    dt = _dtype_code(q_idx)
    shape = make_shape(h_q or h_kv, h_kv, 128, d_idx, top_k, dt, force_local=force_local,
                       idx_scale=idx_scale, cache_dtype=_cache_code(k_idx, dt, k_idx_scale), pool=pool)
    dev = q_idx.device
    bidx = out if out is not None else torch.empty((rows, h_kv, top_k), dtype=torch.int32, device=dev)
    scores = torch.empty((rows, h_kv, top_k), dtype=torch.float32, device=dev) if with_scores else None
    if decode:
        nws = workspace_size(OP_INDEX_DECODE, shape, batch=batch, n_q=1, max_pages=mp)
    else:
        nws = workspace_size(OP_INDEX, shape, n_q=n_q, q_start=qs, n_kv=nkv)
    ws = _workspace(nws, dev, workspace)
    kv = KV(None, None, _ptr(k_idx), _ptr(page_table), _ptr(seq_lens), nkv, mp, None, None, _ptr(k_idx_scale))
    _check(lib().msa_index_topk(ctypes.byref(shape), batch, n_q, qs, _ptr(q_idx), ctypes.byref(kv),
                                _ptr(bidx), _ptr(scores), _ptr(ws), nws, _stream(stream)))
    return (bidx, scores) if with_scores else bidx


def index_topk_decode_static(q_idx, k_idx_pages, page_table, seq_lens, *, top_k=16, force_local=True,
                             idx_scale=0.0, with_scores=False, out=None, out_scores=None, stream=None, pool="max",
                             k_idx_scale=None):
    """msa_index_topk_decode_static: msa_index_topk in decode mode with the
    library's own scratch instead of a workspace (nothing is allocated but the
    outputs, and those only when ``out`` / ``out_scores`` are not given).
    q_idx [batch, h_kv, d_idx]; k_idx pages [*, 128, d_idx]; page_table int32
    [batch, max_pages]; seq_lens int32 [batch]."""
    batch, h_kv, d_idx = q_idx.shape
    dt = _dtype_code(q_idx)
    shape = make_shape(h_kv, h_kv, 128, d_idx, top_k, dt, force_local=force_local, idx_scale=idx_scale,
                       cache_dtype=_cache_code(k_idx_pages, dt, k_idx_scale), pool=pool)
    dev = q_idx.device
    bidx = out if out is not None else torch.empty((batch, h_kv, top_k), dtype=torch.int32, device=dev)
    scores = None
    if with_scores:
        scores = out_scores if out_scores is not None else torch.empty((batch, h_kv, top_k), dtype=torch.float32,
                                                                       device=dev)
    kv = KV(None, None, _ptr(k_idx_pages), _ptr(page_table), _ptr(seq_lens), 0, page_table.shape[1], None, None,
            _ptr(k_idx_scale))
    _check(lib().msa_index_topk_decode_static(ctypes.byref(shape), batch, _ptr(q_idx), ctypes.byref(kv), _ptr(bidx),
                                              _ptr(scores), _stream(stream)))
    return (bidx, scores) if with_scores else bidx


def sparse_prefill(q, k, v, block_idx, *, q_start=0, sm_scale=0.0, page_table=None, n_kv=None,
                   with_lse=False, out=None, workspace=None, stream=None, k_scale=None, v_scale=None):
    """msa_sparse_prefill.  q [n_q, h_q, d_h]; k/v [n_kv, h_kv, d_h] (or pages
    [*, h_kv, 128, d_h] with ``page_table`` and ``n_kv``); block_idx int32
    [n_q, h_kv, top_k].  MXFP8 k/v: float8_e4m3fn codes plus ``k_scale`` /
    ``v_scale`` (uint8, last dim d_h / 32).  Returns o [n_q, h_q, d_h] (and
    lse fp32 [n_q, h_q])."""
    n_q, h_q, d_h = q.shape
    h_kv, top_k = block_idx.shape[1], block_idx.shape[2]
    nkv = int(n_kv) if n_kv is not None else k.shape[0]
    mp = page_table.numel() if page_table is not None else 0
    dt = _dtype_code(q)
    shape = make_shape(h_q, h_kv, d_h, 64, top_k, dt, sm_scale=sm_scale, cache_dtype=_cache_code(k, dt, k_scale))
    o = out if out is not None else torch.empty_like(q)
    lse = torch.empty((n_q, h_q), dtype=torch.float32, device=q.device) if with_lse else None
    nws = workspace_size(OP_PREFILL, shape, n_q=n_q, q_start=int(q_start), n_kv=nkv)
    ws = _workspace(nws, q.device, workspace)
    kv = KV(_ptr(k), _ptr(v), None, _ptr(page_table), None, nkv, mp, _ptr(k_scale), _ptr(v_scale), None)
    _check(lib().msa_sparse_prefill(ctypes.byref(shape), n_q, int(q_start), _ptr(q), ctypes.byref(kv),
                                    _ptr(block_idx), _ptr(o), _ptr(lse), _ptr(ws), nws, _stream(stream)))
    return (o, lse) if with_lse else o


def sparse_decode(q, k_pages, v_pages, page_table, seq_lens, block_idx, *, sm_scale=0.0,
                  with_lse=False, out=None, workspace=None, stream=None, k_scale=None, v_scale=None):
    """msa_sparse_decode.  q [batch, h_q, d_h]; pages [*, h_kv, 128, d_h];
    page_table int32 [batch, max_pages]; seq_lens int32 [batch]; block_idx
    int32 [batch, h_kv, top_k].  MXFP8 pages: float8_e4m3fn codes plus
    ``k_scale`` / ``v_scale`` [*, h_kv, 128, d_h / 32] uint8.  Returns o
    [batch, h_q, d_h] (and lse)."""
    batch, h_q, d_h = q.shape
    h_kv, top_k = block_idx.shape[1], block_idx.shape[2]
    dt = _dtype_code(q)
    shape = make_shape(h_q, h_kv, d_h, 64, top_k, dt, sm_scale=sm_scale,
                       cache_dtype=_cache_code(k_pages, dt, k_scale))
    o = out if out is not None else torch.empty_like(q)
    lse = torch.empty((batch, h_q), dtype=torch.float32, device=q.device) if with_lse else None
    nws = workspace_size(OP_DECODE, shape, batch=batch, n_q=1)
    ws = _workspace(nws, q.device, workspace)
    kv = KV(_ptr(k_pages), _ptr(v_pages), None, _ptr(page_table), _ptr(seq_lens), 0, page_table.shape[1],
            _ptr(k_scale), _ptr(v_scale), None)
    _check(lib().msa_sparse_decode(ctypes.byref(shape), batch, _ptr(q), ctypes.byref(kv), _ptr(block_idx),
                                   _ptr(o), _ptr(lse), _ptr(ws), nws, _stream(stream)))
    return (o, lse) if with_lse else o


def sparse_prefill_backward(q, k, v, block_idx, o, lse, d_o, *, q_start=0, sm_scale=0.0, top_k=None,
                            out=None, workspace=None, stream=None, q_idx=None, k_idx=None, kl_scale=1.0,
                            idx_scale=0.0, kl_out=True):
    """msa_sparse_prefill_backward: gradients (dq, dk, dv) of msa_sparse_prefill
    for one contiguous sequence, given the forward's o and lse and d_o.
    q, o, d_o [n_q, h_q, d_h]; k, v [n_kv, h_kv, d_h]; block_idx int32
    [n_q, h_kv, k]; lse fp32 [n_q, h_q].  With q_idx [n_q, h_kv, d_idx] and
    k_idx [n_kv, d_idx] also the KL-alignment term: returns (dq, dk, dv, kl,
    dq_idx, dk_idx) with kl fp32 [n_q, h_kv] (None when kl_out is False)."""
    n_q, h_q, d_h = q.shape
    n_kv, h_kv = k.shape[0], k.shape[1]
    tk = int(top_k) if top_k is not None else block_idx.shape[-1]
    with_kl = q_idx is not None
    d_idx = q_idx.shape[-1] if with_kl else 64
    shape = make_shape(h_q, h_kv, d_h, d_idx, tk, _dtype_code(q), sm_scale=sm_scale, idx_scale=idx_scale)
    dq, dk, dv = out if out is not None else (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    op = OP_PREFILL_BACKWARD_KL if with_kl else OP_PREFILL_BACKWARD
    nws = workspace_size(op, shape, n_q=n_q, q_start=int(q_start), n_kv=n_kv)
    ws = _workspace(nws, q.device, workspace)
    kv = KV(_ptr(k), _ptr(v), None, None, None, n_kv, 0)
    klp = None
    kl = dq_idx = dk_idx = None
    if with_kl:
        kl = torch.empty((n_q, h_kv), dtype=torch.float32, device=q.device) if kl_out else None
        dq_idx = torch.empty_like(q_idx)
        dk_idx = torch.empty_like(k_idx)
        klp = ctypes.byref(KL(_ptr(q_idx), _ptr(k_idx), float(kl_scale), _ptr(kl), _ptr(dq_idx), _ptr(dk_idx)))
    _check(lib().msa_sparse_prefill_backward(ctypes.byref(shape), n_q, int(q_start), _ptr(q), ctypes.byref(kv),
                                             _ptr(block_idx), _ptr(o), _ptr(lse), _ptr(d_o), _ptr(dq), _ptr(dk),
                                             _ptr(dv), klp, _ptr(ws), nws, _stream(stream)))
    if with_kl:
        return dq, dk, dv, kl, dq_idx, dk_idx
    return dq, dk, dv


def index_project(x, w_q_idx, w_k_idx, positions, k_idx_cache, *, rope_dim=64, rope_base=10000.0, page_table=None,
                  seq=None, n_kv=None, out=None, workspace=None, stream=None):
    """msa_index_project: q_idx [n_tok, h_kv, d_idx] = RoPE(W_q_idx[r] x) for every
    group, and RoPE(W_k_idx x) appended to ``k_idx_cache`` (contiguous [n_kv,
    d_idx] or pages [*, 128, d_idx] with ``page_table``) at each token's
    position.  Returns q_idx."""
    n_tok, d_model = x.shape
    h_kv, d_idx = w_q_idx.shape[0], w_q_idx.shape[1]
    shape = make_shape(h_kv, h_kv, 128, d_idx, 16, _dtype_code(x))
    q_out = out if out is not None else torch.empty((n_tok, h_kv, d_idx), dtype=x.dtype, device=x.device)
    nkv = int(n_kv) if n_kv is not None else (k_idx_cache.shape[0] if page_table is None else 0)
    mp = page_table.shape[-1] if page_table is not None else 0
    kv = KV(None, None, _ptr(k_idx_cache), _ptr(page_table), None, nkv, mp)
    nws = workspace_size(OP_INDEX_PROJECT, shape, n_q=n_tok, n_kv=d_model)
    ws = _workspace(nws, x.device, workspace)
    _check(lib().msa_index_project(ctypes.byref(shape), n_tok, d_model, _ptr(x), _ptr(w_q_idx), _ptr(w_k_idx),
                                   int(rope_dim), float(rope_base), _ptr(positions), _ptr(seq), ctypes.byref(kv),
                                   _ptr(q_out), _ptr(ws), nws, _stream(stream)))
    return q_out


def dense_prefill(q, k, v, *, q_start=0, sm_scale=0.0, with_lse=False, out=None, stream=None):
    """msa_dense_prefill (Eq. (1), the dense GQA comparison kernel)."""
    n_q, h_q, d_h = q.shape
    h_kv = k.shape[1]
    shape = make_shape(h_q, h_kv, d_h, 64, 16, _dtype_code(q), sm_scale=sm_scale)
    o = out if out is not None else torch.empty_like(q)
    lse = torch.empty((n_q, h_q), dtype=torch.float32, device=q.device) if with_lse else None
    kv = KV(_ptr(k), _ptr(v), None, None, None, k.shape[0], 0)
    _check(lib().msa_dense_prefill(ctypes.byref(shape), n_q, int(q_start), _ptr(q), ctypes.byref(kv),
                                   _ptr(o), _ptr(lse), None, 0, _stream(stream)))
    return (o, lse) if with_lse else o

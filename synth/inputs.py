"""Seeded synthetic workloads shaped like the MSA attention layer.

Shapes follow the model described on the MiniMax Sparse Attention digest
(titansim.online), §3.1: 64 query heads, 4 KV heads, head dim 128, block size
128, k = 16.  The index dimension is not given on the pages; 64 is used here
(32 for the tiny case).  All draws use torch generators with fixed seeds, on
whatever device is asked for, so both the HIP path and the oracle read the
same bits (the oracle copies the device tensors back to the host).

Nothing in this module computes scores, selections or attention.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

BLOCK = 128


@dataclass(frozen=True)
class HeadShape:
    h_q: int
    h_kv: int
    d_h: int
    d_idx: int
    top_k: int


MODEL_SHAPE = HeadShape(h_q=64, h_kv=4, d_h=128, d_idx=64, top_k=16)
TINY_SHAPE = HeadShape(h_q=4, h_kv=1, d_h=64, d_idx=32, top_k=4)


def bf16_round(x: torch.Tensor) -> torch.Tensor:
    """Values of ``x`` after one round-to-nearest-even trip through bfloat16."""
    return x.to(torch.bfloat16).to(torch.float32)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int(seed))
    return g


def _randn(shape, gen, device, dtype, scale=1.0, rows_per_chunk=None):
    """N(0, scale^2) draws in ``dtype``, generated in float32 chunks along dim 0."""
    shape = tuple(int(s) for s in shape)
    out = torch.empty(shape, dtype=dtype, device=device)
    if out.numel() == 0:
        return out
    per_row = max(1, out[0].numel()) if len(shape) > 0 else 1
    if rows_per_chunk is None:
        rows_per_chunk = max(1, (1 << 26) // per_row)
    for s in range(0, shape[0], rows_per_chunk):
        e = min(shape[0], s + rows_per_chunk)
        x = torch.randn((e - s,) + shape[1:], generator=gen, device=device,
                        dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        out[s:e].copy_(x)
    return out


MX_BLOCK = 32        # elements per shared scale of the MX formats
MXFP8 = "mxfp8"      # cache_dtype value: E4M3 codes plus one E8M0 scale per 32 elements


def mx_encode(x: torch.Tensor):
    """OCP MXFP8 (E4M3 elements) encoding of ``x`` along its last dim.

    Every run of 32 consecutive elements gets shared_exp = floor(log2(max |x|))
    - 8 (8 = the largest E4M3 exponent), clamped to [-127, 127] (an all-zero
    run gets -127); its elements x / 2^shared_exp are rounded to E4M3 (nearest
    even, saturating at +-448) and its scale byte is shared_exp + 127.
    Returns (codes as torch.float8_e4m3fn, scales uint8 [..., d / 32])."""
    d = x.shape[-1]
    assert d % MX_BLOCK == 0
    xb = x.to(torch.float32).reshape(*x.shape[:-1], d // MX_BLOCK, MX_BLOCK)
    amax = xb.abs().amax(dim=-1)
    e = torch.floor(torch.log2(amax.clamp_min(torch.finfo(torch.float32).tiny))) - 8.0
    e = torch.where(amax > 0, e, torch.full_like(e, -127.0)).clamp(-127.0, 127.0)
    q = (xb / torch.exp2(e).unsqueeze(-1)).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.reshape(x.shape), (e + 127.0).to(torch.uint8)


def _randn_mx(shape, gen, device, scale=1.0, rows_per_chunk=None):
    """MXFP8 cache tensor: N(0, scale^2) draws in which every 32-element run of
    the last dim is multiplied by 2^u, u uniform in {-4..4} (so neighbouring
    runs get different shared scales), then encoded with ``mx_encode``.
    Returns (codes float8_e4m3fn ``shape``, scales uint8 ``shape[:-1] + (d/32,)``)."""
    shape = tuple(int(s) for s in shape)
    codes = torch.empty(shape, dtype=torch.float8_e4m3fn, device=device)
    scales = torch.empty(shape[:-1] + (shape[-1] // MX_BLOCK,), dtype=torch.uint8, device=device)
    if codes.numel() == 0:
        return codes, scales
    per_row = max(1, codes[0].numel())
    if rows_per_chunk is None:
        rows_per_chunk = max(1, (1 << 25) // per_row)
    for s in range(0, shape[0], rows_per_chunk):
        e = min(shape[0], s + rows_per_chunk)
        x = torch.randn((e - s,) + shape[1:], generator=gen, device=device, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        u = torch.randint(-4, 5, (e - s,) + shape[1:-1] + (shape[-1] // MX_BLOCK, 1), generator=gen,
                          device=device, dtype=torch.int32)
        x = (x.reshape((e - s,) + shape[1:-1] + (shape[-1] // MX_BLOCK, MX_BLOCK)) * torch.exp2(u.float()))
        c, sc = mx_encode(x.reshape((e - s,) + shape[1:]))
        codes[s:e].copy_(c)
        scales[s:e].copy_(sc)
    return codes, scales


def _cache(out: dict, name: str, shape, gen, device, cdt, scale=1.0):
    """Cache tensor ``name`` in storage type ``cdt`` (a torch dtype, or MXFP8:
    E4M3 codes in ``name`` and their scales in ``name + '_scale'``)."""
    if cdt == MXFP8:
        out[name], out[name + "_scale"] = _randn_mx(shape, gen, device, scale)
    else:
        out[name] = _randn(shape, gen, device, cdt, scale)


def gen_prefill(n_kv: int, shape: HeadShape = MODEL_SHAPE, *, n_q: int | None = None,
                dtype=torch.bfloat16, seed: int = 1, device="cpu",
                scaled: bool = True, cache_dtype=None) -> dict:
    """One contiguous sequence: K/V/K_idx for ``n_kv`` tokens and queries for the
    last ``n_q`` positions (``q_start = n_kv - n_q``).

    Layouts: q [n_q, h_q, d_h], k/v [n_kv, h_kv, d_h], q_idx [n_q, h_kv, d_idx],
    k_idx [n_kv, d_idx].  With ``scaled`` every tensor is N(0,1)/sqrt(last dim),
    otherwise N(0,1).  ``cache_dtype`` (default ``dtype``) is the storage type
    of k, v and k_idx, e.g. torch.float8_e4m3fn, or MXFP8 (then ``k_scale``,
    ``v_scale`` and ``k_idx_scale`` hold the E8M0 scales, see ``_randn_mx``).
    """
    cdt = dtype if cache_dtype is None else cache_dtype
    n_q = n_kv if n_q is None else n_q
    g = _gen(seed, device)
    sh = lambda d: (1.0 / math.sqrt(d)) if scaled else 1.0  # noqa: E731
    out = {"q": _randn((n_q, shape.h_q, shape.d_h), g, device, dtype, sh(shape.d_h))}
    _cache(out, "k", (n_kv, shape.h_kv, shape.d_h), g, device, cdt, sh(shape.d_h))
    _cache(out, "v", (n_kv, shape.h_kv, shape.d_h), g, device, cdt, sh(shape.d_h))
    out["q_idx"] = _randn((n_q, shape.h_kv, shape.d_idx), g, device, dtype, sh(shape.d_idx))
    _cache(out, "k_idx", (n_kv, shape.d_idx), g, device, cdt, sh(shape.d_idx))
    out["q_start"] = n_kv - n_q
    out["n_kv"] = n_kv
    return out


def gen_decode_paged(batch: int, seq_len: int, shape: HeadShape = MODEL_SHAPE, *,
                     dtype=torch.bfloat16, seed: int = 3, device="cpu",
                     extra_tokens: int = 0, n_query_sets: int = 1,
                     seq_lens=None, cache_dtype=None) -> dict:
    """A paged KV cache of ``batch`` sequences with 128-token pages.

    Physical pages are a seeded random permutation: page_table [batch, max_pages]
    int32.  k/v pages [num_pages, h_kv, 128, d_h] (head-major inside a page),
    k_idx pages [num_pages, 128, d_idx].  ``seq_lens`` [batch] int32 counts the
    tokens held, the newest token included.  Queries: q [sets, batch, h_q, d_h],
    q_idx [sets, batch, h_kv, d_idx].  Everything N(0,1).  ``cache_dtype``
    (default ``dtype``) is the storage type of the three caches, e.g.
    torch.float8_e4m3fn (the N(0,1) draws rounded once to that format).
    """
    cdt = dtype if cache_dtype is None else cache_dtype
    if seq_lens is None:
        seq_lens = [seq_len] * batch
    max_pages = -(-(max(seq_lens) + extra_tokens) // BLOCK)
    num_pages = batch * max_pages
    g = _gen(seed, device)
    gcpu = _gen(seed + 7919, "cpu")
    perm = torch.randperm(num_pages, generator=gcpu).to(torch.int32)
    out = {
        "page_table": perm.view(batch, max_pages).contiguous().to(device),
        "seq_lens": torch.tensor(seq_lens, dtype=torch.int32).to(device),
    }
    _cache(out, "k_pages", (num_pages, shape.h_kv, BLOCK, shape.d_h), g, device, cdt)
    _cache(out, "v_pages", (num_pages, shape.h_kv, BLOCK, shape.d_h), g, device, cdt)
    _cache(out, "k_idx_pages", (num_pages, BLOCK, shape.d_idx), g, device, cdt)
    out["q"] = _randn((n_query_sets, batch, shape.h_q, shape.d_h), g, device, dtype)
    out["q_idx"] = _randn((n_query_sets, batch, shape.h_kv, shape.d_idx), g, device, dtype)
    out["max_pages"] = max_pages
    return out


def gen_planted_prefill(n: int = 131072, shape: HeadShape = MODEL_SHAPE, *,
                        dtype=torch.bfloat16, seed: int = 4, device="cpu",
                        n_designated: int = 1024, n_planted: int = 3,
                        plant_lo: int = 1, plant_hi: int = 512,
                        designated_after: int = 65536, gain: float = 8.0,
                        cos: float = 0.9) -> dict:
    """Needle-style index inputs: per KV group r, ``n_planted`` distinct past
    blocks in [plant_lo, plant_hi) each hold one token whose index key is
    ``gain * (cos * u_r + sqrt(1 - cos^2) * w)`` with w orthogonal to the group
    direction u_r; ``n_designated`` query positions after ``designated_after``
    carry index query ``gain * u_r`` in every group.  Everything else is
    N(0,1) for the index tensors and N(0,1)/sqrt(d_h) for q/k/v.
    """
    base = gen_prefill(n, shape, dtype=dtype, seed=seed, device=device, scaled=True)
    g = _gen(seed + 1, "cpu")
    d = shape.d_idx
    # unscaled index tensors for this workload
    gi = _gen(seed + 2, device)
    q_idx = _randn((n, shape.h_kv, d), gi, device, torch.float32)
    k_idx = _randn((n, d), gi, device, torch.float32)
    u = torch.randn((shape.h_kv, d), generator=g, dtype=torch.float64)
    u = u / u.norm(dim=1, keepdim=True)
    blocks = torch.empty((shape.h_kv, n_planted), dtype=torch.int64)
    tokens = torch.empty((shape.h_kv, n_planted), dtype=torch.int64)
    used = set()
    for r in range(shape.h_kv):
        cand = torch.randperm(plant_hi - plant_lo, generator=g) + plant_lo
        picked = [int(b) for b in cand.tolist() if int(b) not in used][:n_planted]
        used.update(picked)
        for t, b in enumerate(picked):
            off = int(torch.randint(0, BLOCK, (1,), generator=g))
            blocks[r, t] = b
            tokens[r, t] = b * BLOCK + off
            w = torch.randn((d,), generator=g, dtype=torch.float64)
            w = w - (w @ u[r]) * u[r]
            w = w / w.norm()
            kvec = gain * (cos * u[r] + math.sqrt(1.0 - cos * cos) * w)
            k_idx[tokens[r, t]] = kvec.to(torch.float32).to(device)
    span = n - designated_after - 1
    pos = torch.randperm(span, generator=g)[:n_designated] + designated_after + 1
    pos, _ = torch.sort(pos)
    for r in range(shape.h_kv):
        q_idx[pos.to(device), r] = (gain * u[r]).to(torch.float32).to(device)
    base["q_idx"] = q_idx.to(dtype)
    base["k_idx"] = k_idx.to(dtype)
    base["planted_blocks"] = blocks
    base["planted_tokens"] = tokens
    base["designated"] = pos
    return base


def gen_long_context(n_ctx: int = 1 << 20, n_chunk: int = 8192, n_decode: int = 256,
                     shape: HeadShape = MODEL_SHAPE, *, dtype=torch.bfloat16,
                     seed: int = 5, device="cpu") -> dict:
    """A single paged sequence of ``n_ctx`` tokens with room for ``n_decode``
    more, the queries of its last ``n_chunk`` positions (chunked prefill), and
    per decode step a new token (k, v, k_idx) plus its queries.  All N(0,1).
    """
    cache = gen_decode_paged(1, n_ctx, shape, dtype=dtype, seed=seed, device=device,
                             extra_tokens=n_decode)
    g = _gen(seed + 11, device)
    cache["chunk_q"] = _randn((n_chunk, shape.h_q, shape.d_h), g, device, dtype)
    cache["chunk_q_idx"] = _randn((n_chunk, shape.h_kv, shape.d_idx), g, device, dtype)
    cache["q_start"] = n_ctx - n_chunk
    cache["n_ctx"] = n_ctx
    cache["step_k"] = _randn((n_decode, shape.h_kv, shape.d_h), g, device, dtype)
    cache["step_v"] = _randn((n_decode, shape.h_kv, shape.d_h), g, device, dtype)
    cache["step_k_idx"] = _randn((n_decode, shape.d_idx), g, device, dtype)
    cache["step_q"] = _randn((n_decode, 1, shape.h_q, shape.d_h), g, device, dtype)
    cache["step_q_idx"] = _randn((n_decode, 1, shape.h_kv, shape.d_idx), g, device, dtype)
    return cache

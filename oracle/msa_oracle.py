"""Plain float64 CPU oracle for the MiniMax Sparse Attention (MSA) hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP library
never calls it and shares no code with it.

Sources (the pages this follows):
  [P1] MiniMax Sparse Attention digest (titansim.online blog):
       §2.2 Eq. (1) dense causal softmax attention;
       §4.2 Eq. (6) index scores and block max-pool, top-k with the local
       block always kept; §4.3 Eq. (8) attention over the gathered blocks;
       §4.4.1 exp-free selection; §5.2 Eq. (12) FLOP model; §3.1 shapes.
  [P5] 163.com commentary on MSA, "Step 1 Index Attention": one index query
       per GQA group, one shared index key (Q_idx in R^{n x h x d},
       K_idx in R^{n x 1 x d}); max-pool rather than mean-pool (the mean
       over a block's tokens is the block scoring it attributes to MoBA;
       kept here as an ablation, ``pool="mean"``).

Readings taken where the pages are silent:
  * query i of a call sits at absolute position p = q_start + i;
  * block b holds token positions [128 b, 128 b + 127]; the diagonal block of
    position p is p // 128 and its pooled score uses only keys j <= p;
  * with ``force_local`` the diagonal block always occupies one of the k slots
    and the other k - 1 slots go to the best strictly-past blocks;
  * ranking is by pooled score, descending; equal scores go to the lower
    block index;
  * the returned indices are ascending, padded with -1 to length k;
  * query head h belongs to KV group h // (h_q / h_kv);
  * paged caches map block b of sequence s to physical page page_table[s, b];
    a decode query sits at position seq_len - 1 and the cache already holds it.

Every input array is upcast to float64 before any arithmetic.

Training path (readings): the KL-alignment loss of [P1] §4.5 compares, per
query and group over the visible keys of the selected blocks, the mean over
the group's heads of the main-branch softmax (the target, detached) with the
softmax of the index scores (the prediction); KL(target || prediction),
summed over (query, group) and multiplied by a caller-given weight.
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 128


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# Index branch  ([P1] §4.2 Eq. (6); [P5] Step 1)
# --------------------------------------------------------------------------

def index_token_scores(q_idx_row, k_idx, p, idx_scale=None):
    """S_j = <q_idx, k_idx_j> * idx_scale for every key position j <= p.

    ``q_idx_row`` [h_kv, d_idx] (one index query per group), ``k_idx``
    [n_kv, d_idx] shared by all groups.  Returns [h_kv, p + 1].
    Eq. (6), left half; the default scale is 1 / sqrt(d_idx).
    """
    q = _f64(q_idx_row)
    k = _f64(k_idx)[: p + 1]
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if idx_scale is None else float(idx_scale)
    return (q @ k.T) * scale


def block_max_pool(scores, p, block=BLOCK):
    """M_b = max of S_j over the visible keys j <= p of block b, for
    b = 0 .. p // block (Eq. (6), right half).  ``scores`` [h_kv, p + 1].
    Returns [h_kv, p // block + 1]."""
    s = _f64(scores)
    nb = p // block + 1
    out = np.empty((s.shape[0], nb))
    for b in range(nb):
        lo, hi = b * block, min(b * block + block, p + 1)
        out[:, b] = s[:, lo:hi].max(axis=1)
    return out


def block_mean_pool(scores, p, block=BLOCK):
    """Ablation of Eq. (6): the mean of S_j over the visible keys j <= p of
    block b instead of their max ([P5] "Step 1 Index Attention" contrasts
    the two).  ``scores`` [h_kv, p + 1].  Returns [h_kv, p // block + 1]."""
    s = _f64(scores)
    nb = p // block + 1
    out = np.empty((s.shape[0], nb))
    for b in range(nb):
        lo, hi = b * block, min(b * block + block, p + 1)
        out[:, b] = s[:, lo:hi].sum(axis=1) / (hi - lo)
    return out


def _pool(scores, p, pool, block):
    if pool == "max":
        return block_max_pool(scores, p, block)
    if pool == "mean":
        return block_mean_pool(scores, p, block)
    raise ValueError(f"pool must be 'max' or 'mean', got {pool!r}")


def select_blocks(m_row, diag, top_k, force_local=True):
    """Exp-free causal top-k over one row of pooled scores ([P1] §4.2, §4.4.1).

    ``m_row`` holds M_b for b = 0 .. diag.  The ranking uses the raw pooled
    scores (softmax is monotone, so it cannot change the order).  With
    ``force_local`` the diagonal block is kept and the remaining k - 1 slots go
    to the best past blocks b < diag; otherwise plain top-k over b <= diag.
    Order: score descending, then block index ascending.  Returns a length-k
    int64 array, ascending, padded with -1.
    """
    m = _f64(m_row)
    if force_local:
        cand = np.arange(diag)
        n_take = top_k - 1
    else:
        cand = np.arange(diag + 1)
        n_take = top_k
    chosen = []
    if n_take > 0 and cand.size > 0:
        order = np.lexsort((cand, -m[cand]))  # primary: score desc; then b asc
        chosen = [int(b) for b in cand[order[:n_take]]]
    if force_local:
        chosen.append(int(diag))
    chosen.sort()
    out = np.full(top_k, -1, dtype=np.int64)
    out[: len(chosen)] = chosen
    return out


def index_topk(q_idx, k_idx, q_start, top_k, *, force_local=True, idx_scale=None,
               rows=None, block=BLOCK, pool="max"):
    """Index branch for one contiguous sequence.

    ``q_idx`` [n_q, h_kv, d_idx], ``k_idx`` [n_kv, d_idx].  Query i sits at
    position q_start + i.  Returns (block_idx [n_rows, h_kv, k] int64,
    block_score [n_rows, h_kv, k] float64 with -inf where the index is -1,
    pooled [list of per-row [h_kv, diag+1] arrays]) for the requested
    ``rows`` (default: all queries).
    """
    q_idx = _f64(q_idx)
    k_idx = _f64(k_idx)
    n_q, h_kv, _ = q_idx.shape
    rows = range(n_q) if rows is None else rows
    idx_out, score_out, pooled = [], [], []
    for i in rows:
        p = q_start + int(i)
        s = index_token_scores(q_idx[i], k_idx, p, idx_scale)
        m = _pool(s, p, pool, block)
        diag = p // block
        ids = np.stack([select_blocks(m[r], diag, top_k, force_local) for r in range(h_kv)])
        sc = np.where(ids >= 0, np.take_along_axis(m, np.maximum(ids, 0), axis=1), -np.inf)
        idx_out.append(ids)
        score_out.append(sc)
        pooled.append(m)
    return np.stack(idx_out), np.stack(score_out), pooled


# --------------------------------------------------------------------------
# Main branch  ([P1] §4.3 Eq. (8); dense reference §2.2 Eq. (1))
# --------------------------------------------------------------------------

def _attend(qh, keys, vals, scale):
    """softmax(qh keys^T * scale) vals for a set of visible keys.
    qh [G, d], keys/vals [T, d].  Returns (o [G, d], lse [G])."""
    s = (qh @ keys.T) * scale
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    l = w.sum(axis=1, keepdims=True)
    o = (w @ vals) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def sparse_attention(q, k, v, block_idx, q_start, *, sm_scale=None, rows=None,
                     block=BLOCK):
    """Eq. (8): each head of group r attends, with exact softmax, to the keys
    of its group's selected blocks that are causally visible (j <= p).

    ``q`` [n_q, h_q, d_h]; ``k``/``v`` [n_kv, h_kv, d_h]; ``block_idx``
    [n_q, h_kv, k] (entries -1 ignored).  Returns (o [n_rows, h_q, d_h],
    lse [n_rows, h_q]) for the requested ``rows``.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    n_q, h_q, d_h = q.shape
    h_kv = k.shape[1]
    g = h_q // h_kv
    scale = 1.0 / math.sqrt(d_h) if sm_scale is None else float(sm_scale)
    rows = range(n_q) if rows is None else rows
    o_all, lse_all = [], []
    for i in rows:
        p = q_start + int(i)
        o_i = np.empty((h_q, d_h))
        lse_i = np.empty(h_q)
        for r in range(h_kv):
            blocks = sorted(set(int(b) for b in block_idx[i, r] if b >= 0))
            toks = np.concatenate([np.arange(b * block, min(b * block + block, p + 1))
                                   for b in blocks if b * block <= p] or [np.zeros(0, int)])
            if toks.size == 0:
                o_i[r * g:(r + 1) * g] = 0.0
                lse_i[r * g:(r + 1) * g] = -np.inf
                continue
            o, lse = _attend(q[i, r * g:(r + 1) * g], k[toks, r], v[toks, r], scale)
            o_i[r * g:(r + 1) * g] = o
            lse_i[r * g:(r + 1) * g] = lse
        o_all.append(o_i)
        lse_all.append(lse_i)
    return np.stack(o_all), np.stack(lse_all)


def dense_attention(q, k, v, q_start, *, sm_scale=None, rows=None):
    """Eq. (1): causal softmax attention over every key j <= p (GQA: head h
    reads KV group h // G).  Same layouts and returns as ``sparse_attention``."""
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    n_q, h_q, d_h = q.shape
    h_kv = k.shape[1]
    g = h_q // h_kv
    scale = 1.0 / math.sqrt(d_h) if sm_scale is None else float(sm_scale)
    rows = range(n_q) if rows is None else rows
    o_all, lse_all = [], []
    for i in rows:
        p = q_start + int(i)
        o_i = np.empty((h_q, d_h))
        lse_i = np.empty(h_q)
        for r in range(h_kv):
            o, lse = _attend(q[i, r * g:(r + 1) * g], k[: p + 1, r], v[: p + 1, r], scale)
            o_i[r * g:(r + 1) * g] = o
            lse_i[r * g:(r + 1) * g] = lse
        o_all.append(o_i)
        lse_all.append(lse_i)
    return np.stack(o_all), np.stack(lse_all)


# --------------------------------------------------------------------------
# Paged caches (block b of sequence s lives in page page_table[s, b])
# --------------------------------------------------------------------------

def gather_sequence(page_table_row, seq_len, k_pages=None, v_pages=None,
                    k_idx_pages=None, block=BLOCK):
    """Rebuild one sequence's contiguous k/v [seq_len, h_kv, d_h] and k_idx
    [seq_len, d_idx] from head-major pages ([pages, h_kv, 128, d_h] and
    [pages, 128, d_idx])."""
    nb = -(-int(seq_len) // block)
    pages = [int(x) for x in np.asarray(page_table_row)[:nb]]
    out = {}
    if k_pages is not None:
        kp = np.asarray(k_pages)[pages]                      # [nb, h_kv, 128, d]
        out["k"] = _f64(np.transpose(kp, (0, 2, 1, 3)).reshape(nb * block, kp.shape[1], kp.shape[3])[:seq_len])
    if v_pages is not None:
        vp = np.asarray(v_pages)[pages]
        out["v"] = _f64(np.transpose(vp, (0, 2, 1, 3)).reshape(nb * block, vp.shape[1], vp.shape[3])[:seq_len])
    if k_idx_pages is not None:
        ip = np.asarray(k_idx_pages)[pages]                  # [nb, 128, d_idx]
        out["k_idx"] = _f64(ip.reshape(nb * block, ip.shape[2])[:seq_len])
    return out


def index_topk_decode(q_idx, k_idx_pages, page_table, seq_lens, top_k, *,
                      force_local=True, idx_scale=None, seqs=None, block=BLOCK, pool="max"):
    """Decode-time index branch: one query per sequence at position
    seq_len - 1 over its paged index keys.  ``q_idx`` [batch, h_kv, d_idx].
    Returns (block_idx [n, h_kv, k], block_score [n, h_kv, k], pooled list)."""
    seqs = range(len(seq_lens)) if seqs is None else seqs
    ids, scs, pooled = [], [], []
    for s in seqs:
        L = int(seq_lens[s])
        seq = gather_sequence(page_table[s], L, k_idx_pages=k_idx_pages, block=block)
        i_s, sc_s, m_s = index_topk(_f64(q_idx)[s:s + 1], seq["k_idx"], L - 1, top_k,
                                    force_local=force_local, idx_scale=idx_scale, block=block,
                                    pool=pool)
        ids.append(i_s[0])
        scs.append(sc_s[0])
        pooled.append(m_s[0])
    return np.stack(ids), np.stack(scs), pooled


def sparse_decode(q, k_pages, v_pages, page_table, seq_lens, block_idx, *,
                  sm_scale=None, seqs=None, block=BLOCK):
    """Decode-time main branch: Eq. (8) for the one new query of each
    sequence.  ``q`` [batch, h_q, d_h], ``block_idx`` [batch, h_kv, k].
    Returns (o [n, h_q, d_h], lse [n, h_q])."""
    seqs = range(len(seq_lens)) if seqs is None else seqs
    os_, ls_ = [], []
    for s in seqs:
        L = int(seq_lens[s])
        seq = gather_sequence(page_table[s], L, k_pages=k_pages, v_pages=v_pages, block=block)
        o, lse = sparse_attention(_f64(q)[s:s + 1], seq["k"], seq["v"],
                                  np.asarray(block_idx)[s:s + 1], L - 1, sm_scale=sm_scale)
        os_.append(o[0])
        ls_.append(lse[0])
    return np.stack(os_), np.stack(ls_)


# --------------------------------------------------------------------------
# 8-bit caches (scope table, next step: e4m3 K/V and K_idx caches; the MXFP8
# KV cache of the zhichai.net key points)
# --------------------------------------------------------------------------

# --------------------------------------------------------------------------
# Training path ([P1] §4.5): gradients of Eq. (8) over the selected blocks, and
# the KL-alignment loss between the index branch and the group-averaged main
# branch, with the main-branch side detached.
# --------------------------------------------------------------------------

def _visible_tokens(row_blocks, p, block=BLOCK):
    """Token positions j <= p of the listed blocks (entries < 0 ignored)."""
    blocks = sorted(set(int(b) for b in row_blocks if b >= 0))
    parts = [np.arange(b * block, min(b * block + block, p + 1)) for b in blocks if b * block <= p]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def sparse_attention_backward(q, k, v, block_idx, q_start, do, *, sm_scale=None, block=BLOCK, rows=None):
    """Gradients of Eq. (8) for one contiguous sequence, given dO.

    For query i (position p) and head h of group r, with T the visible keys of
    the group's selected blocks, s_j = q.k_j * scale, P = softmax_T(s),
    O = sum_j P_j v_j:
        dv_j += P_j dO
        dP_j  = dO . v_j,   ds_j = P_j (dP_j - sum_t P_t dP_t)
        dq    = scale * sum_j ds_j k_j,   dk_j += scale * ds_j q.
    Returns (dq [n_q, h_q, d_h], dk [n_kv, h_kv, d_h], dv [n_kv, h_kv, d_h]).
    With ``rows``, only those queries are taken: their dq rows, and the
    parts of dk and dv they contribute (the whole of dk/dv for any key whose
    block only those queries selected).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    n_q, h_q, d_h = q.shape
    h_kv = k.shape[1]
    g = h_q // h_kv
    scale = 1.0 / math.sqrt(d_h) if sm_scale is None else float(sm_scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for i in (range(n_q) if rows is None else rows):
        p = q_start + int(i)
        for r in range(h_kv):
            toks = _visible_tokens(block_idx[i, r], p, block)
            if toks.size == 0:
                continue
            kt, vt = k[toks, r], v[toks, r]
            for h in range(r * g, (r + 1) * g):
                s = kt @ q[i, h] * scale
                w = np.exp(s - s.max())
                pr = w / w.sum()
                dpr = vt @ do[i, h]
                ds = pr * (dpr - pr @ dpr)
                dq[i, h] = scale * (ds @ kt)
                dk[toks, r] += scale * np.outer(ds, q[i, h])
                dv[toks, r] += np.outer(pr, do[i, h])
    return dq, dk, dv


def kl_alignment(q_idx, k_idx, q, k, block_idx, q_start, *, sm_scale=None, idx_scale=None,
                 kl_scale=1.0, block=BLOCK, rows=None):
    """KL-alignment loss of the index branch ([P1] §4.5; [P4] key points).

    For query i and group r, over the visible keys T of the group's selected
    blocks:
      target    p_main(j) = mean over the group's heads h of softmax_T(q_h.k_j * sm_scale)
      predicted p_idx(j)  = softmax_T(q_idx^(r).k_idx_j * idx_scale)
      KL_{i,r}  = sum_j p_main(j) (log p_main(j) - log p_idx(j)).
    The loss is L = kl_scale * sum_{i,r} KL_{i,r}.  p_main is detached (no
    gradient reaches q or k), so dL/dS_idx(j) = kl_scale (p_idx(j) - p_main(j))
    and the gradients go to q_idx and k_idx only.
    Returns (kl [n_q, h_kv], dq_idx [n_q, h_kv, d_idx], dk_idx [n_kv, d_idx]);
    with ``rows`` only those queries are taken (as in sparse_attention_backward).
    """
    q_idx, k_idx, q, k = _f64(q_idx), _f64(k_idx), _f64(q), _f64(k)
    n_q, h_kv, d_idx = q_idx.shape
    h_q, d_h = q.shape[1], q.shape[2]
    g = h_q // h_kv
    sc = 1.0 / math.sqrt(d_h) if sm_scale is None else float(sm_scale)
    isc = 1.0 / math.sqrt(d_idx) if idx_scale is None else float(idx_scale)
    kl = np.zeros((n_q, h_kv))
    dq_idx = np.zeros_like(q_idx)
    dk_idx = np.zeros_like(k_idx)
    for i in (range(n_q) if rows is None else rows):
        p = q_start + int(i)
        for r in range(h_kv):
            toks = _visible_tokens(block_idx[i, r], p, block)
            if toks.size == 0:
                continue
            s = (q[i, r * g:(r + 1) * g] @ k[toks, r].T) * sc          # [G, T]
            w = np.exp(s - s.max(axis=1, keepdims=True))
            p_main = (w / w.sum(axis=1, keepdims=True)).mean(axis=0)   # [T]
            si = k_idx[toks] @ q_idx[i, r] * isc                       # [T]
            log_p_idx = si - (si.max() + np.log(np.exp(si - si.max()).sum()))
            p_idx = np.exp(log_p_idx)
            pos = p_main > 0
            kl[i, r] = np.sum(p_main[pos] * (np.log(p_main[pos]) - log_p_idx[pos]))
            dsi = kl_scale * (p_idx - p_main)
            dq_idx[i, r] = isc * (dsi @ k_idx[toks])
            dk_idx[toks] += isc * np.outer(dsi, q_idx[i, r])
    return kl, dq_idx, dk_idx


# --------------------------------------------------------------------------
# The steps before the index branch ([P1] §4.2: one index-query projection
# per GQA group and one shared index-key projection; §3.1: RoPE on 64 dims)
# --------------------------------------------------------------------------

def rope(v, positions, rope_dim, base=10000.0):
    """Rotary position embedding on the first ``rope_dim`` dims of the last
    axis, "rotate half" pairing: dim i < rope_dim/2 pairs with i + rope_dim/2
    and the pair turns by the angle p * base^(-2i/rope_dim).  ``v`` [n, ..., d],
    ``positions`` [n]."""
    v = _f64(v).copy()
    if rope_dim == 0:
        return v
    h = rope_dim // 2
    theta = base ** (-2.0 * np.arange(h) / rope_dim)
    ang = np.asarray(positions, np.float64).reshape((-1,) + (1,) * (v.ndim - 1)) * theta
    c, s_ = np.cos(ang), np.sin(ang)
    x1, x2 = v[..., :h].copy(), v[..., h:rope_dim].copy()
    v[..., :h] = x1 * c - x2 * s_
    v[..., h:rope_dim] = x2 * c + x1 * s_
    return v


def index_projection(x, w_q_idx, w_k_idx, positions, *, rope_dim=64, rope_base=10000.0):
    """q_idx^(r) = W_q^idx,(r) x for each group r and k_idx = W_k^idx x, then
    RoPE at each token's position.  ``x`` [n, d_model], ``w_q_idx`` [h_kv,
    d_idx, d_model], ``w_k_idx`` [d_idx, d_model].  Returns (q_idx [n, h_kv,
    d_idx], k_idx [n, d_idx])."""
    x = _f64(x)
    q = np.einsum("nm,rdm->nrd", x, _f64(w_q_idx))
    k = x @ _f64(w_k_idx).T
    return rope(q, positions, rope_dim, rope_base), rope(k, positions, rope_dim, rope_base)


def decode_e4m3(codes):
    """Values of OCP FP8 E4M3 ("fn") codes, written from the format's
    definition: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
    exponent field 0 is subnormal (m/8 * 2^-6), the code S.1111.111 is NaN
    and there are no infinities.  ``codes`` is any uint8 array; returns
    float64 of the same shape."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = sign * np.ldexp(m / 8.0, -6)
    out = np.where(e == 0, sub, normal)
    return np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, out)


def decode_e8m0(codes):
    """Values of OCP E8M0 codes, the shared scale of the MX block formats
    (the MXFP8 cache format named on the zhichai.net key points page,
    Limitations): an 8-bit biased exponent with no sign and no mantissa,
    value 2^(code - 127); the code 0xFF is NaN.  Returns float64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c == 0xFF, np.nan, np.ldexp(1.0, c - 127))


def decode_mxfp8(codes, scales, block=32):
    """Values of an MXFP8 (E4M3 elements) tensor: along the last axis, every
    run of ``block`` = 32 consecutive elements shares one E8M0 scale, and an
    element's value is its E4M3 value times that scale.  ``codes`` [..., d]
    uint8, ``scales`` [..., d / 32] uint8; returns float64 [..., d]."""
    c = np.asarray(codes, dtype=np.uint8)
    s = np.asarray(scales, dtype=np.uint8)
    d = c.shape[-1]
    assert d % block == 0 and s.shape == c.shape[:-1] + (d // block,)
    elem = decode_e4m3(c)
    scale = np.repeat(decode_e8m0(s), block, axis=-1)
    return elem * scale


# --------------------------------------------------------------------------
# FLOP model ([P1] §5.2 Eq. (12))
# --------------------------------------------------------------------------

def flops_eq12(n, h_q, h_kv, d_h, d_idx, top_k, block=BLOCK):
    """Eq. (12): F_GQA(N) = 2 H_q d_h N^2 and
    F_MSA(N) = H_kv d_idx N^2 (index branch) + 4 H_q d_h N k B_k (main branch).
    Returns (f_gqa, f_msa_index, f_msa_main)."""
    n = float(n)
    f_gqa = 2.0 * h_q * d_h * n * n
    f_index = float(h_kv) * d_idx * n * n
    f_main = 4.0 * h_q * d_h * n * top_k * block
    return f_gqa, f_index, f_main

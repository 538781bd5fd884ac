"""GPU parity of the libmsa HIP path against the float64 oracle.

Every call goes through the C ABI (ctypes binding).  Inputs come from the
seeded generators in synth/; the oracle reads back the exact bits the GPU
consumed.  Sizes span several tiles and a ragged tail while the oracle still
finishes in seconds; the full-size cases check sampled rows.
"""
import numpy as np
import pytest
import torch

from oracle import msa_oracle as orc
from synth import MODEL_SHAPE, TINY_SHAPE, gen_decode_paged, gen_long_context, gen_prefill
from synth.inputs import MXFP8, HeadShape

from _helpers import compare_grad, compare_index_rows, compare_lse, compare_out, np64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_attention_branch_amd import msa
    msa.lib()
    return msa


def _say(*a):
    print("[case]", *a, flush=True)


# ------------------------------------------------------------------ index branch

def _index_case(shape, n_kv, n_q, dtype, seed, *, force_local=True, with_scores=False, scaled=True, pool="max",
                cache_dtype=None):
    msa = _msa()
    inp = gen_prefill(n_kv, shape, n_q=n_q, dtype=dtype, seed=seed, device=DEV, scaled=scaled,
                      cache_dtype=cache_dtype)
    q_start = inp["q_start"]
    _say("index_topk", shape, n_kv, n_q, dtype, seed, force_local, pool, cache_dtype)
    out = msa.index_topk(inp["q_idx"], inp["k_idx"], top_k=shape.top_k, q_start=q_start,
                         force_local=force_local, with_scores=with_scores, pool=pool,
                         k_idx_scale=inp.get("k_idx_scale"))
    torch.cuda.synchronize()
    ids, sc = out if with_scores else (out, None)
    o_ids, o_sc, pooled = orc.index_topk(np64(inp["q_idx"]), _cache_host(inp["k_idx"], inp.get("k_idx_scale")),
                                         q_start, shape.top_k, force_local=force_local, pool=pool)
    diags = (q_start + np.arange(n_q)) // 128
    n_exact, n_exc = compare_index_rows(ids.cpu().numpy(), o_ids, pooled, diags, force_local)
    if sc is not None:
        g = ids.cpu().numpy()
        gs = sc.cpu().numpy().astype(np.float64)
        for t in range(n_q):
            for r in range(shape.h_kv):
                for j in range(shape.top_k):
                    b = g[t, r, j]
                    if b < 0:
                        assert gs[t, r, j] == -np.inf
                    else:
                        ref = pooled[t][r][b]
                        assert abs(gs[t, r, j] - ref) <= 1e-5 * max(1.0, abs(ref)), (t, r, b, gs[t, r, j], ref)
    return n_exact, n_exc


def test_index_tiny_fp32():
    n_exact, n_exc = _index_case(TINY_SHAPE, 2048, 2048, torch.float32, 0, scaled=False)
    assert n_exc <= 2


def test_index_model_shape_bf16_ragged_tail():
    _index_case(MODEL_SHAPE, 2125, 2125, torch.bfloat16, 1)


def test_index_chunked_unaligned_q_start_with_scores():
    _index_case(MODEL_SHAPE, 3000, 700, torch.bfloat16, 2, with_scores=True)


def test_index_no_forced_local_block():
    _index_case(HeadShape(8, 2, 64, 64, 5), 1500, 1500, torch.bfloat16, 3, force_local=False, with_scores=True)


def test_index_no_forced_local_block_without_scores():
    # force_local = 0 and no score output: the diagonal block is an ordinary
    # candidate and must still be scored (one chunk, several chunks, 4 groups)
    _index_case(HeadShape(8, 2, 64, 64, 5), 900, 900, torch.bfloat16, 60, force_local=False)
    _index_case(HeadShape(8, 2, 64, 64, 5), 1500, 1500, torch.bfloat16, 61, force_local=False)
    _index_case(MODEL_SHAPE, 2125, 2125, torch.bfloat16, 62, force_local=False)
    _index_case(MODEL_SHAPE, 3000, 700, torch.bfloat16, 63, force_local=False)


def _closed_form_golden():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "closed_form_selection.json")) as fh:
        g = json.load(fh)
    # d_idx 32: the golden vectors live on coordinate 0, the rest are zero
    d = 32
    k_idx = torch.zeros(g["n_kv"], d, dtype=torch.float32)
    k_idx[:, 0] = -1.0
    for b, (v, off) in enumerate(zip(g["peak_value"], g["peak_offset"])):
        k_idx[b * 128 + off, 0] = v
    q_row = torch.zeros(g["h_kv"], d, dtype=torch.float32)
    q_row[:, 0] = torch.tensor(g["group_coef"], dtype=torch.float32)
    return g, k_idx.to(torch.bfloat16), q_row.to(torch.bfloat16)


def test_index_exact_ties_closed_form_prefill_and_decode():
    # The hand-derived closed form (tests/golden/closed_form_selection.json):
    # group 1 scores every block exactly alike, so its lists are decided by the
    # tie-break alone (lower block wins); group 0 has distinct peaks (bf16
    # rounding keeps their order).  The GPU lists must equal the golden lists
    # exactly, with no near-tie excusal, in prefill mode (one query at
    # position p) and in decode mode (a paged cache, the query at seq_len - 1).
    msa = _msa()
    g, k_idx, q_row = _closed_form_golden()
    n_kv, h_kv = g["n_kv"], g["h_kv"]
    kd = k_idx.to(DEV)
    qd = q_row.to(DEV)
    n_pages = n_kv // 128
    perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(64)).to(torch.int32)
    pages = torch.empty(n_pages, 128, k_idx.shape[1], dtype=torch.bfloat16)
    pages[perm.long()] = k_idx.view(n_pages, 128, -1)
    pages = pages.to(DEV)
    pt = perm.view(1, n_pages).to(DEV)
    for case in g["cases"]:
        p, k, fl = case["p"], case["top_k"], case["force_local"]
        expect = np.asarray(case["expect"], dtype=np.int64)
        _say("exact ties, prefill", p, k, fl)
        got = msa.index_topk(qd.view(1, h_kv, -1).contiguous(), kd, top_k=k, q_start=p, force_local=fl)
        got_s, sc = msa.index_topk(qd.view(1, h_kv, -1).contiguous(), kd, top_k=k, q_start=p, force_local=fl,
                                   with_scores=True)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy()[0], expect), (case["why"], got.cpu().numpy()[0], expect)
        assert np.array_equal(got_s.cpu().numpy()[0], expect), (case["why"], got_s.cpu().numpy()[0], expect)
        _say("exact ties, decode", p, k, fl)
        sl = torch.tensor([p + 1], dtype=torch.int32, device=DEV)
        dec = msa.index_topk(qd.view(1, h_kv, -1).contiguous(), pages, top_k=k, page_table=pt, seq_lens=sl,
                             force_local=fl)
        torch.cuda.synchronize()
        assert np.array_equal(dec.cpu().numpy()[0], expect), (case["why"], dec.cpu().numpy()[0], expect)


def test_index_small_k_and_d_idx_128():
    _index_case(HeadShape(16, 4, 128, 128, 3), 1100, 1100, torch.bfloat16, 4)
    _index_case(HeadShape(16, 4, 128, 32, 1), 600, 600, torch.float32, 5)


def test_index_short_sequences():
    # fewer than k eligible blocks, a single block, a single query
    _index_case(MODEL_SHAPE, 130, 130, torch.bfloat16, 6)
    _index_case(MODEL_SHAPE, 1, 1, torch.bfloat16, 7)
    _index_case(MODEL_SHAPE, 500, 1, torch.bfloat16, 8)


def test_index_mean_pool_prefill():
    # the mean-pool ablation: ragged tail, chunked unaligned start, no forced
    # block, fp32, d_idx 32 and 128, e4m3 index keys
    _index_case(MODEL_SHAPE, 2300, 2300, torch.bfloat16, 40, pool="mean", with_scores=True)
    _index_case(MODEL_SHAPE, 3000, 700, torch.bfloat16, 41, pool="mean")
    _index_case(HeadShape(8, 2, 64, 64, 5), 1500, 1500, torch.bfloat16, 42, force_local=False, pool="mean",
                with_scores=True)
    _index_case(TINY_SHAPE, 2048, 2048, torch.float32, 43, scaled=False, pool="mean")
    _index_case(HeadShape(16, 4, 128, 128, 3), 1100, 1100, torch.bfloat16, 44, pool="mean")
    _index_case(HeadShape(16, 4, 128, 32, 16), 900, 900, torch.bfloat16, 45, pool="mean",
                cache_dtype=torch.float8_e4m3fn)


def test_index_mxfp8_keys_with_the_index_options():
    # MXFP8 index keys with every option of the index call: scores reported, no
    # forced block, mean-pool, a chunked unaligned start, d_idx 32 and 128
    _index_case(MODEL_SHAPE, 2125, 2125, torch.bfloat16, 140, with_scores=True, cache_dtype=MXFP8)
    _index_case(HeadShape(8, 2, 64, 64, 5), 1500, 1500, torch.bfloat16, 141, force_local=False, cache_dtype=MXFP8)
    _index_case(MODEL_SHAPE, 3000, 700, torch.bfloat16, 142, pool="mean", with_scores=True, cache_dtype=MXFP8)
    _index_case(HeadShape(16, 4, 128, 32, 16), 900, 900, torch.bfloat16, 143, force_local=False, pool="mean",
                cache_dtype=MXFP8)
    _index_case(HeadShape(16, 4, 128, 128, 7), 1300, 1300, torch.bfloat16, 144, cache_dtype=MXFP8)


def test_index_mean_pool_decode():
    msa = _msa()
    for shape, seq_lens, seed, cdt in ((MODEL_SHAPE, [1, 127, 128, 129, 3000, 2049, 40000], 46, None),
                                       (HeadShape(16, 2, 64, 32, 16), [5000, 700, 129], 47, torch.float8_e4m3fn),
                                       (HeadShape(16, 4, 128, 128, 8), [1500, 9000], 48, None),
                                       (HeadShape(16, 4, 128, 64, 16), [4000, 300, 128], 49, MXFP8)):
        inp = gen_decode_paged(len(seq_lens), max(seq_lens), shape, seed=seed, device=DEV, seq_lens=seq_lens,
                               cache_dtype=cdt)
        _say("decode index mean-pool", shape, seq_lens, seed, cdt)
        q_idx = inp["q_idx"][0].contiguous()
        kis = inp.get("k_idx_pages_scale")
        bidx, bsc = msa.index_topk(q_idx, inp["k_idx_pages"], top_k=shape.top_k, page_table=inp["page_table"],
                                   seq_lens=inp["seq_lens"], pool="mean", with_scores=True, k_idx_scale=kis)
        torch.cuda.synchronize()
        pt = inp["page_table"].cpu().numpy()
        o_ids, _, pooled = orc.index_topk_decode(np64(q_idx), _cache_host(inp["k_idx_pages"], kis), pt, seq_lens,
                                                 shape.top_k, pool="mean")
        diags = (np.asarray(seq_lens) - 1) // 128
        compare_index_rows(bidx.cpu().numpy(), o_ids, pooled, diags)
        g, gs = bidx.cpu().numpy(), bsc.cpu().numpy().astype(np.float64)
        for t in range(len(seq_lens)):
            for r in range(shape.h_kv):
                for j in range(shape.top_k):
                    b = g[t, r, j]
                    if b >= 0:
                        ref = pooled[t][r][b]
                        assert abs(gs[t, r, j] - ref) <= 1e-5 * max(1.0, abs(ref)), (t, r, b)


# ------------------------------------------------------------------ main branch

def _prefill_case(shape, n_kv, n_q, dtype, seed, *, use_gpu_index=False, scaled=True):
    msa = _msa()
    inp = gen_prefill(n_kv, shape, n_q=n_q, dtype=dtype, seed=seed, device=DEV, scaled=scaled)
    q_start = inp["q_start"]
    _say("sparse_prefill", shape, n_kv, n_q, dtype, seed, "gpu-index" if use_gpu_index else "oracle-index")
    if use_gpu_index:
        bidx = msa.index_topk(inp["q_idx"], inp["k_idx"], top_k=shape.top_k, q_start=q_start)
        ids = bidx.cpu().numpy()
    else:
        ids, _, _ = orc.index_topk(np64(inp["q_idx"]), np64(inp["k_idx"]), q_start, shape.top_k)
        bidx = torch.from_numpy(ids.astype(np.int32)).to(DEV)
    o, lse = msa.sparse_prefill(inp["q"], inp["k"], inp["v"], bidx, q_start=q_start, with_lse=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.sparse_attention(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]), ids, q_start)
    compare_out(o, o_ref, dtype)
    compare_lse(lse, lse_ref, dtype)
    return inp, bidx, o


def test_prefill_tiny_fp32():
    _prefill_case(TINY_SHAPE, 2048, 2048, torch.float32, 0, scaled=False)


def test_prefill_model_shape_bf16_ragged():
    _prefill_case(MODEL_SHAPE, 2125, 2125, torch.bfloat16, 1)


def test_prefill_chunked_q_start_fp32():
    _prefill_case(HeadShape(16, 2, 128, 64, 6), 2600, 900, torch.float32, 9)


def test_prefill_end_to_end_with_gpu_indices():
    _prefill_case(MODEL_SHAPE, 1800, 1800, torch.bfloat16, 10, use_gpu_index=True)


def test_prefill_d64_group4_bf16():
    _prefill_case(HeadShape(8, 2, 64, 32, 4), 1300, 1300, torch.bfloat16, 11)


def test_prefill_groups_of_1_2_and_8():
    # every supported head-to-group ratio besides 4 and 16, both dtypes
    _prefill_case(HeadShape(4, 4, 128, 64, 5), 1700, 1700, torch.bfloat16, 15)
    _prefill_case(HeadShape(4, 2, 64, 32, 3), 900, 600, torch.float32, 16)
    _prefill_case(HeadShape(16, 2, 128, 64, 16), 1400, 1400, torch.bfloat16, 17, use_gpu_index=True)


def _e4m3_prefill_case(shape, n_kv, n_q, seed, paged):
    msa = _msa()
    f8 = torch.float8_e4m3fn
    inp = gen_prefill(n_kv, shape, n_q=n_q, dtype=torch.bfloat16, seed=seed, device=DEV, cache_dtype=f8)
    q_start = inp["q_start"]
    _say("e4m3 prefill", shape, n_kv, n_q, seed, "paged" if paged else "contiguous")
    k, v, ki = inp["k"], inp["v"], inp["k_idx"]
    kw = {}
    if paged:
        # the same tokens in head-major 128-token pages placed by a random permutation
        nb = -(-n_kv // 128)
        pad = nb * 128 - n_kv
        perm = torch.randperm(nb, generator=torch.Generator().manual_seed(seed)).to(torch.int32)
        def pages(t):
            u8 = t.view(torch.uint8)
            u8 = torch.cat([u8, torch.zeros((pad,) + u8.shape[1:], dtype=torch.uint8, device=DEV)])
            u8 = u8.view((nb, 128) + u8.shape[1:])
            if u8.dim() == 4:
                u8 = u8.permute(0, 2, 1, 3)
            out = torch.empty_like(u8.contiguous())
            out[perm.long().to(DEV)] = u8.contiguous()
            return out.view(f8)
        k, v, ki = pages(k), pages(v), pages(ki)
        kw = dict(page_table=perm.to(DEV), n_kv=n_kv)
    bidx = msa.index_topk(inp["q_idx"], ki, top_k=shape.top_k, q_start=q_start, **kw)
    o, lse = msa.sparse_prefill(inp["q"], k, v, bidx, q_start=q_start, with_lse=True, **kw)
    torch.cuda.synchronize()
    k64 = orc.decode_e4m3(inp["k"].view(torch.uint8).cpu().numpy())
    v64 = orc.decode_e4m3(inp["v"].view(torch.uint8).cpu().numpy())
    ki64 = orc.decode_e4m3(inp["k_idx"].view(torch.uint8).cpu().numpy())
    o_ids, _, pooled = orc.index_topk(np64(inp["q_idx"]), ki64, q_start, shape.top_k)
    compare_index_rows(bidx.cpu().numpy(), o_ids, pooled, (q_start + np.arange(n_q)) // 128)
    o_ref, lse_ref = orc.sparse_attention(np64(inp["q"]), k64, v64, bidx.cpu().numpy(), q_start)
    compare_out(o, o_ref, torch.bfloat16)
    compare_lse(lse, lse_ref, torch.bfloat16)


def test_prefill_e4m3_caches_contiguous_and_paged():
    _e4m3_prefill_case(MODEL_SHAPE, 2300, 2300, 29, paged=False)
    _e4m3_prefill_case(HeadShape(16, 2, 64, 32, 6), 1700, 900, 30, paged=True)
    _e4m3_prefill_case(HeadShape(16, 4, 128, 128, 16), 1300, 1300, 31, paged=True)


def _mx_prefill_case(shape, n_kv, n_q, seed, paged):
    msa = _msa()
    inp = gen_prefill(n_kv, shape, n_q=n_q, dtype=torch.bfloat16, seed=seed, device=DEV, cache_dtype=MXFP8)
    q_start = inp["q_start"]
    _say("MXFP8 prefill", shape, n_kv, n_q, seed, "paged" if paged else "contiguous")
    names = ("k", "v", "k_idx", "k_scale", "v_scale", "k_idx_scale")
    t = {n: inp[n] for n in names}
    kw = {}
    if paged:
        # the same tokens (and their scale rows) in head-major 128-token pages
        # placed by a random permutation
        nb = -(-n_kv // 128)
        pad = nb * 128 - n_kv
        perm = torch.randperm(nb, generator=torch.Generator().manual_seed(seed)).to(torch.int32)
        def pages(x):
            u8 = x.view(torch.uint8)
            u8 = torch.cat([u8, torch.zeros((pad,) + u8.shape[1:], dtype=torch.uint8, device=DEV)])
            u8 = u8.view((nb, 128) + u8.shape[1:])
            if u8.dim() == 4:
                u8 = u8.permute(0, 2, 1, 3)
            out = torch.empty_like(u8.contiguous())
            out[perm.long().to(DEV)] = u8.contiguous()
            return out.view(x.dtype)
        t = {n: pages(x) for n, x in t.items()}
        kw = dict(page_table=perm.to(DEV), n_kv=n_kv)
    bidx = msa.index_topk(inp["q_idx"], t["k_idx"], top_k=shape.top_k, q_start=q_start, k_idx_scale=t["k_idx_scale"],
                          **kw)
    o, lse = msa.sparse_prefill(inp["q"], t["k"], t["v"], bidx, q_start=q_start, with_lse=True, k_scale=t["k_scale"],
                                v_scale=t["v_scale"], **kw)
    torch.cuda.synchronize()
    k64 = _cache_host(inp["k"], inp["k_scale"])
    v64 = _cache_host(inp["v"], inp["v_scale"])
    ki64 = _cache_host(inp["k_idx"], inp["k_idx_scale"])
    o_ids, _, pooled = orc.index_topk(np64(inp["q_idx"]), ki64, q_start, shape.top_k)
    compare_index_rows(bidx.cpu().numpy(), o_ids, pooled, (q_start + np.arange(n_q)) // 128)
    o_ref, lse_ref = orc.sparse_attention(np64(inp["q"]), k64, v64, bidx.cpu().numpy(), q_start)
    compare_out(o, o_ref, torch.bfloat16, rel_elem=MX_REL)
    compare_lse(lse, lse_ref, torch.bfloat16)


# MXFP8 test data reach |v| ~ 7 (block scales up to 2^4), so the bf16 output
# rounding (2^-9 relative) exceeds the fixed 1e-2 bound near the largest
# outputs: those tests add 2^-7 of each reference value to it (4x the rounding).
MX_REL = 2.0 ** -7


def test_prefill_mxfp8_caches_contiguous_and_paged():
    _mx_prefill_case(MODEL_SHAPE, 2300, 2300, 129, paged=False)
    _mx_prefill_case(HeadShape(16, 2, 64, 32, 6), 1700, 900, 130, paged=True)
    _mx_prefill_case(HeadShape(16, 4, 128, 128, 16), 1300, 1300, 131, paged=True)


def test_prefill_full_coverage_equals_dense():
    msa = _msa()
    shape = HeadShape(16, 2, 128, 64, 16)
    n = 1900                                   # 15 blocks <= k: every block selected
    inp = gen_prefill(n, shape, dtype=torch.bfloat16, seed=12, device=DEV)
    _say("full coverage", n)
    bidx = msa.index_topk(inp["q_idx"], inp["k_idx"], top_k=16)
    o_s = msa.sparse_prefill(inp["q"], inp["k"], inp["v"], bidx)
    o_d, lse_d = msa.dense_prefill(inp["q"], inp["k"], inp["v"], with_lse=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.dense_attention(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]), 0)
    compare_out(o_s, o_ref, torch.bfloat16, "sparse")
    compare_out(o_d, o_ref, torch.bfloat16, "dense")
    compare_lse(lse_d, lse_ref, torch.bfloat16)


def test_dense_fp32_chunked():
    msa = _msa()
    shape = HeadShape(8, 2, 64, 32, 4)
    inp = gen_prefill(1000, shape, n_q=333, dtype=torch.float32, seed=13, device=DEV)
    _say("dense fp32 chunked")
    o, lse = msa.dense_prefill(inp["q"], inp["k"], inp["v"], q_start=inp["q_start"], with_lse=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.dense_attention(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]), inp["q_start"])
    compare_out(o, o_ref, torch.float32)
    compare_lse(lse, lse_ref, torch.float32)


def test_prefill_deterministic_and_chunked_equals_one_shot():
    msa = _msa()
    shape = MODEL_SHAPE
    n = 1500
    inp = gen_prefill(n, shape, dtype=torch.bfloat16, seed=14, device=DEV)
    _say("determinism + chunked == one-shot")
    b1 = msa.index_topk(inp["q_idx"], inp["k_idx"], top_k=16)
    o1 = msa.sparse_prefill(inp["q"], inp["k"], inp["v"], b1)
    b2 = msa.index_topk(inp["q_idx"], inp["k_idx"], top_k=16)
    o2 = msa.sparse_prefill(inp["q"], inp["k"], inp["v"], b2)
    torch.cuda.synchronize()
    assert torch.equal(b1, b2) and torch.equal(o1, o2)
    cut = 650
    parts_b, parts_o = [], []
    for lo, hi in ((0, cut), (cut, n)):
        kv = {k: inp[k][:hi].contiguous() for k in ("k", "v", "k_idx")}
        bb = msa.index_topk(inp["q_idx"][lo:hi].contiguous(), kv["k_idx"], top_k=16, q_start=lo)
        oo = msa.sparse_prefill(inp["q"][lo:hi].contiguous(), kv["k"], kv["v"], bb, q_start=lo)
        parts_b.append(bb)
        parts_o.append(oo)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(parts_b), b1)
    assert torch.equal(torch.cat(parts_o), o1)


# ------------------------------------------------- more prefill shapes
# Group counts with 16 heads each (1, 3 and 8 groups), paged bf16 and e4m3
# caches, single-token and 17-token query counts, scores tens of nats
# apart, and bitwise repeatability.

def _pages(t, perm, n_kv):
    """[n_kv, h_kv, ...] cache -> head-major 128-token pages [nb, h_kv, 128, ...] placed by perm."""
    nb = perm.numel()
    u8 = t.contiguous().view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t.contiguous()
    pad = nb * 128 - n_kv
    u8 = torch.cat([u8, torch.zeros((pad,) + tuple(u8.shape[1:]), dtype=u8.dtype, device=u8.device)])
    u8 = u8.view((nb, 128) + tuple(u8.shape[1:])).permute(0, 2, 1, 3).contiguous()
    out = torch.empty_like(u8)
    out[perm.long().to(u8.device)] = u8
    return out.view(torch.float8_e4m3fn) if t.dtype == torch.float8_e4m3fn else out


def _shape_case(shape, n_kv, n_q, seed, *, paged=False, cache_dtype=None, boost=None, repeats=1):
    msa = _msa()
    inp = gen_prefill(n_kv, shape, n_q=n_q, dtype=torch.bfloat16, seed=seed, device=DEV, cache_dtype=cache_dtype)
    q_start = inp["q_start"]
    k, v = inp["k"], inp["v"]
    if boost is not None:
        # one block's keys scaled up: its scores lie tens of nats above the
        # rest of each row
        blk, f = boost
        k = k.clone()
        k[blk * 128:(blk + 1) * 128] *= f
    if cache_dtype == torch.float8_e4m3fn:
        k64 = orc.decode_e4m3(k.view(torch.uint8).cpu().numpy())
        v64 = orc.decode_e4m3(v.view(torch.uint8).cpu().numpy())
        ki64 = orc.decode_e4m3(inp["k_idx"].view(torch.uint8).cpu().numpy())
    else:
        k64, v64, ki64 = np64(k), np64(v), np64(inp["k_idx"])
    ids, _, _ = orc.index_topk(np64(inp["q_idx"]), ki64, q_start, shape.top_k)
    bidx = torch.from_numpy(ids.astype(np.int32)).to(DEV)
    kw = {}
    if paged:
        nb = -(-n_kv // 128)
        perm = torch.randperm(nb, generator=torch.Generator().manual_seed(seed)).to(torch.int32)
        k, v = _pages(k, perm, n_kv), _pages(v, perm, n_kv)
        kw = dict(page_table=perm.to(DEV), n_kv=n_kv)
    o_ref, lse_ref = orc.sparse_attention(np64(inp["q"]), k64, v64, ids, q_start)
    outs = []
    for _ in range(repeats):
        _say("prefill shape", shape, n_kv, n_q, seed, "paged" if paged else "contiguous", cache_dtype, boost)
        o, lse = msa.sparse_prefill(inp["q"], k, v, bidx, q_start=q_start, with_lse=True, **kw)
        torch.cuda.synchronize()
        compare_out(o, o_ref, torch.bfloat16)
        compare_lse(lse, lse_ref, torch.bfloat16)
        outs.append(o)
    return outs


def test_prefill_model_shape_query_counts():
    _shape_case(MODEL_SHAPE, 2125, 2125, 41)          # ragged last block
    _shape_case(MODEL_SHAPE, 3001, 1013, 42)          # q_start 1988, unaligned
    _shape_case(MODEL_SHAPE, 777, 1, 43)              # one query
    _shape_case(MODEL_SHAPE, 300, 17, 44)             # 17 queries, q_start 283


def test_prefill_sixteen_head_groups():
    # 16 heads per group with 1, 3 and 8 groups, and small k
    _shape_case(HeadShape(16, 1, 128, 64, 16), 1500, 1500, 45)
    _shape_case(HeadShape(48, 3, 128, 64, 16), 900, 900, 46)
    _shape_case(HeadShape(128, 8, 128, 64, 8), 1100, 700, 47)
    _shape_case(HeadShape(32, 2, 128, 64, 2), 800, 800, 48)


def test_prefill_paged_bf16_and_e4m3_model_shape():
    _shape_case(MODEL_SHAPE, 1700, 1700, 49, paged=True)
    _shape_case(MODEL_SHAPE, 1300, 1100, 50, paged=True, cache_dtype=torch.float8_e4m3fn)
    _shape_case(MODEL_SHAPE, 1500, 1500, 51, cache_dtype=torch.float8_e4m3fn)


def test_prefill_far_apart_scores_and_determinism():
    # block 2 scores tens of nats above the rest of the rows that select it
    _shape_case(MODEL_SHAPE, 1200, 1200, 52, boost=(2, 3000.0))
    a, b = _shape_case(MODEL_SHAPE, 1400, 1400, 53, repeats=2)
    assert torch.equal(a, b)


def test_prefill_schedule_lds_and_global_counters_agree():
    # The schedule counts and scatters each (window, group) in LDS while its
    # blocks fit there, else with global atomics; the test hook with limit 0
    # forces the latter.  Each (token, block) partial is computed the same way whatever
    # item holds it, so the outputs are bitwise equal.
    msa = _msa()
    for shape, n_kv, n_q, seed in ((MODEL_SHAPE, 1800, 1800, 54), (HeadShape(32, 2, 128, 64, 8), 2500, 700, 55)):
        inp = gen_prefill(n_kv, shape, n_q=n_q, dtype=torch.bfloat16, seed=seed, device=DEV)
        q_start = inp["q_start"]
        ids, _, _ = orc.index_topk(np64(inp["q_idx"]), np64(inp["k_idx"]), q_start, shape.top_k)
        bidx = torch.from_numpy(ids.astype(np.int32)).to(DEV)
        outs = []
        try:
            for thr in (-1, 0):
                msa.test_schedule_lds_limit(thr)
                _say("prefill schedule", "lds" if thr < 0 else "global atomics", shape, n_kv, n_q, seed)
                o, lse = msa.sparse_prefill(inp["q"], inp["k"], inp["v"], bidx, q_start=q_start, with_lse=True)
                torch.cuda.synchronize()
                outs.append((o, lse))
        finally:
            msa.test_schedule_lds_limit(-1)
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
        o_ref, lse_ref = orc.sparse_attention(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]), ids, q_start)
        compare_out(outs[1][0], o_ref, torch.bfloat16)
        compare_lse(outs[1][1], lse_ref, torch.bfloat16)


def test_backward_bitmap_lds_and_global_agree():
    # The ordered schedule of the dK/dV pass builds its per-cell token bitmaps
    # in LDS (256 tokens per workgroup) while a window's blocks fit there, else
    # with global atomics; both give the same bits, so the gradients are
    # bitwise equal (and match the oracle).
    msa = _msa()
    shape = MODEL_SHAPE
    inp = gen_prefill(1700, shape, dtype=torch.bfloat16, seed=56, device=DEV)
    ids, _, _ = orc.index_topk(np64(inp["q_idx"]), np64(inp["k_idx"]), 0, shape.top_k)
    bidx = torch.from_numpy(ids.astype(np.int32)).to(DEV)
    o, lse = msa.sparse_prefill(inp["q"], inp["k"], inp["v"], bidx, with_lse=True)
    d_o = torch.randn(o.shape, generator=torch.Generator(device="cpu").manual_seed(57)).to(torch.bfloat16).to(DEV)
    grads = []
    try:
        for thr in (-1, 0):
            msa.test_schedule_lds_limit(thr)
            _say("backward bitmaps", "lds" if thr < 0 else "global atomics")
            grads.append(msa.sparse_prefill_backward(inp["q"], inp["k"], inp["v"], bidx, o, lse, d_o))
            torch.cuda.synchronize()
    finally:
        msa.test_schedule_lds_limit(-1)
    for a, b in zip(grads[0], grads[1]):
        assert torch.equal(a, b)
    dq_ref, dk_ref, dv_ref = orc.sparse_attention_backward(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]), ids, 0,
                                                           np64(d_o))
    compare_grad(grads[0][0], dq_ref, "dq")
    compare_grad(grads[0][1], dk_ref, "dk")
    compare_grad(grads[0][2], dv_ref, "dv")


def _irregular_lists(n_rows, h_kv, top_k, diags, seed):
    """Ascending block lists within the ABI's contract but unlike the index
    branch's output: repeated entries, -1 between entries, blocks past the
    row's own block at the end, short lists, and some empty rows."""
    rng = np.random.default_rng(seed)
    out = np.full((n_rows, h_kv, top_k), -1, dtype=np.int32)
    for t in range(n_rows):
        d = int(diags[t])
        for r in range(h_kv):
            kind = rng.integers(0, 6)
            if kind == 0:
                continue                                  # empty row: o = 0, lse = -inf
            m = int(rng.integers(1, top_k + 1))
            picks = np.sort(rng.integers(0, d + 3, size=m))  # may repeat, may pass d
            row = []
            for b in picks:
                row.append(int(b))
                if rng.random() < 0.2 and len(row) < top_k:
                    row.append(-1 if rng.random() < 0.5 else int(b))   # a gap or a repeat
            out[t, r, :min(top_k, len(row))] = row[:top_k]
    return out


def test_prefill_and_decode_irregular_block_lists():
    msa = _msa()
    shape = MODEL_SHAPE
    inp = gen_prefill(1500, shape, n_q=1100, dtype=torch.bfloat16, seed=58, device=DEV)
    q_start = inp["q_start"]
    ids = _irregular_lists(1100, shape.h_kv, shape.top_k, (q_start + np.arange(1100)) // 128, 59)
    _say("irregular block lists: prefill")
    o, lse = msa.sparse_prefill(inp["q"], inp["k"], inp["v"], torch.from_numpy(ids).to(DEV), q_start=q_start,
                                with_lse=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.sparse_attention(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]), ids, q_start)
    compare_out(o, o_ref, torch.bfloat16)
    compare_lse(lse, lse_ref, torch.bfloat16)
    assert np.all(np.isneginf(lse.cpu().numpy()[np.repeat(np.all(ids < 0, axis=2), shape.h_q // shape.h_kv, 1)]))
    # the training path on the same lists (empty rows get dq = 0)
    d_o = torch.randn(o.shape, generator=torch.Generator(device="cpu").manual_seed(62)).to(torch.bfloat16).to(DEV)
    _say("irregular block lists: backward")
    dq, dk, dv = msa.sparse_prefill_backward(inp["q"], inp["k"], inp["v"], torch.from_numpy(ids).to(DEV), o, lse, d_o,
                                             q_start=q_start)
    torch.cuda.synchronize()
    rq, rk, rv = orc.sparse_attention_backward(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]), ids, q_start,
                                               np64(d_o))
    compare_grad(dq, rq, "dq")
    compare_grad(dk, rk, "dk")
    compare_grad(dv, rv, "dv")

    seq_lens = [3000, 129, 777, 4096, 1, 2500]
    dec = gen_decode_paged(len(seq_lens), max(seq_lens), shape, seed=60, device=DEV, seq_lens=seq_lens)
    dids = _irregular_lists(len(seq_lens), shape.h_kv, shape.top_k, (np.asarray(seq_lens) - 1) // 128, 61)
    _say("irregular block lists: decode")
    q = dec["q"][0].contiguous()
    od, ld = msa.sparse_decode(q, dec["k_pages"], dec["v_pages"], dec["page_table"], dec["seq_lens"],
                               torch.from_numpy(dids).to(DEV), with_lse=True)
    torch.cuda.synchronize()
    od_ref, ld_ref = orc.sparse_decode(np64(q), _cache_host(dec["k_pages"]), _cache_host(dec["v_pages"]),
                                       dec["page_table"].cpu().numpy(), seq_lens, dids)
    compare_out(od, od_ref, torch.bfloat16)
    compare_lse(ld, ld_ref, torch.bfloat16)


# ------------------------------------------------------------------ decode

def _cache_host(t, scale=None):
    """Host float64 copy of a cache tensor; e4m3 codes (with their E8M0 block
    scales for MXFP8) go through the oracle's decoders."""
    if t.dtype == torch.float8_e4m3fn:
        if scale is not None:
            return orc.decode_mxfp8(t.view(torch.uint8).cpu().numpy(), scale.cpu().numpy())
        return orc.decode_e4m3(t.view(torch.uint8).cpu().numpy())
    return t.cpu().double().numpy()


def _decode_case(shape, seq_lens, seed, n_sets=1, cache_dtype=None):
    msa = _msa()
    batch = len(seq_lens)
    inp = gen_decode_paged(batch, max(seq_lens), shape, seed=seed, device=DEV, seq_lens=seq_lens,
                           cache_dtype=cache_dtype)
    _say("decode", shape, seq_lens, seed, cache_dtype)
    q_idx = inp["q_idx"][0].contiguous()
    q = inp["q"][0].contiguous()
    ks, vs, kis = inp.get("k_pages_scale"), inp.get("v_pages_scale"), inp.get("k_idx_pages_scale")
    bidx = msa.index_topk(q_idx, inp["k_idx_pages"], top_k=shape.top_k, page_table=inp["page_table"],
                          seq_lens=inp["seq_lens"], k_idx_scale=kis)
    o, lse = msa.sparse_decode(q, inp["k_pages"], inp["v_pages"], inp["page_table"], inp["seq_lens"], bidx,
                               with_lse=True, k_scale=ks, v_scale=vs)
    if kis is not None:
        # the allocation-free entry point reads the same scales
        b2 = msa.index_topk_decode_static(q_idx, inp["k_idx_pages"], inp["page_table"], inp["seq_lens"],
                                          top_k=shape.top_k, k_idx_scale=kis)
        assert torch.equal(b2, bidx)
    torch.cuda.synchronize()
    pt = inp["page_table"].cpu().numpy()
    kp = _cache_host(inp["k_pages"], ks)
    vp = _cache_host(inp["v_pages"], vs)
    ip = _cache_host(inp["k_idx_pages"], kis)
    o_ids, _, pooled = orc.index_topk_decode(np64(q_idx), ip, pt, seq_lens, shape.top_k)
    diags = (np.asarray(seq_lens) - 1) // 128
    compare_index_rows(bidx.cpu().numpy(), o_ids, pooled, diags)
    o_ref, lse_ref = orc.sparse_decode(np64(q), kp, vp, pt, seq_lens, bidx.cpu().numpy())
    compare_out(o, o_ref, torch.bfloat16, rel_elem=MX_REL if ks is not None else 0.0)
    compare_lse(lse, lse_ref, torch.bfloat16)


def test_decode_index_at_maximum_page_counts():
    # The decode select's largest candidate counts per thread: 16384 pages (a
    # 2M-token sequence, the most the library accepts: 64 per thread) and
    # 12000 pages (48 per thread).  Only the index-key pages are made (N(0,1)
    # keys and queries); the oracle scores every key of each sequence.
    msa = _msa()
    shape = MODEL_SHAPE
    g = torch.Generator(device=DEV).manual_seed(88)
    for seq_lens in ([2097152], [1536000, 700]):
        B = len(seq_lens)
        mp = -(-max(seq_lens) // 128)
        npg = B * mp
        pt = torch.randperm(npg, generator=torch.Generator().manual_seed(89)).to(torch.int32).view(B, mp).to(DEV)
        kp = torch.randn((npg, 128, shape.d_idx), generator=g, device=DEV).to(torch.bfloat16)
        qi = torch.randn((B, shape.h_kv, shape.d_idx), generator=g, device=DEV).to(torch.bfloat16)
        sl = torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
        _say("decode index at maximum page counts", seq_lens, mp)
        bidx = msa.index_topk(qi, kp, top_k=shape.top_k, page_table=pt, seq_lens=sl)
        torch.cuda.synchronize()
        o_ids, _, pooled = orc.index_topk_decode(np64(qi), kp.cpu().double().numpy(), pt.cpu().numpy(), seq_lens,
                                                 shape.top_k)
        compare_index_rows(bidx.cpu().numpy(), o_ids, pooled, (np.asarray(seq_lens) - 1) // 128)
        del kp


def test_decode_step_graph_replays_match_eager():
    # The decode step (index top-k, then the sparse gather) captured once in a
    # HIP graph and replayed with new queries and longer sequences written
    # into the captured buffers between replays (eager work and syncs in
    # between); every replay must equal the eager calls bitwise.
    msa = _msa()
    shape = MODEL_SHAPE
    seq_lens = [3000, 700, 5000, 129]
    dec = gen_decode_paged(len(seq_lens), max(seq_lens), shape, seed=63, device=DEV, seq_lens=seq_lens,
                           extra_tokens=300, n_query_sets=4)
    B = len(seq_lens)
    sl = torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
    qb = dec["q"][0].clone()
    qib = dec["q_idx"][0].clone()
    s_idx = msa.make_shape(shape.h_q, shape.h_kv, shape.d_h, shape.d_idx, shape.top_k, msa.MSA_BF16)
    mp = dec["page_table"].shape[1]
    ws_i = torch.empty(msa.workspace_size(msa.OP_INDEX_DECODE, s_idx, batch=B, n_q=1, max_pages=mp),
                       dtype=torch.uint8, device=DEV)
    ws_d = torch.empty(max(1, msa.workspace_size(msa.OP_DECODE, s_idx, batch=B, n_q=1)), dtype=torch.uint8,
                       device=DEV)
    bidx = torch.empty((B, shape.h_kv, shape.top_k), dtype=torch.int32, device=DEV)
    o = torch.empty((B, shape.h_q, shape.d_h), dtype=torch.bfloat16, device=DEV)

    def step(q, qi, out_b, out_o):
        msa.index_topk(qi, dec["k_idx_pages"], top_k=shape.top_k, page_table=dec["page_table"], seq_lens=sl,
                       out=out_b, workspace=ws_i)
        msa.sparse_decode(q, dec["k_pages"], dec["v_pages"], dec["page_table"], sl, out_b, out=out_o, workspace=ws_d)

    step(qb, qib, bidx, o)       # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(qb, qib, bidx, o)
    torch.cuda.synchronize()
    for rep in range(4):
        qb.copy_(dec["q"][rep])
        qib.copy_(dec["q_idx"][rep])
        sl.add_(37 * rep)                       # the sequences grow between steps
        torch.cuda.synchronize()
        _say("decode graph replay", rep, sl.tolist())
        g.replay()
        torch.cuda.synchronize()
        eb = torch.empty_like(bidx)
        eo = torch.empty_like(o)
        step(dec["q"][rep].contiguous(), dec["q_idx"][rep].contiguous(), eb, eo)
        torch.cuda.synchronize()
        assert torch.equal(bidx, eb) and torch.equal(o, eo), rep


def test_decode_mixed_lengths():
    _decode_case(MODEL_SHAPE, [1, 127, 128, 129, 3000, 2049], 20)


def test_decode_batch_many_short():
    _decode_case(HeadShape(32, 4, 128, 64, 16), [700 + 37 * i for i in range(40)], 21)


def test_decode_groups_of_1_and_8_d64():
    _decode_case(HeadShape(4, 4, 128, 64, 7), [900, 129, 1], 23)
    _decode_case(HeadShape(16, 2, 64, 32, 16), [5000, 2500], 24)


def test_decode_e4m3_caches():
    # e4m3 K, V and K_idx pages, bf16 queries: mixed lengths, d_h 128 and 64
    f8 = torch.float8_e4m3fn
    _decode_case(MODEL_SHAPE, [1, 127, 128, 129, 3000, 2049], 25, cache_dtype=f8)
    _decode_case(HeadShape(16, 2, 64, 32, 16), [5000, 2500, 700], 26, cache_dtype=f8)
    _decode_case(HeadShape(16, 4, 128, 128, 8), [1500, 9000], 27, cache_dtype=f8)


def test_decode_mxfp8_caches():
    # MXFP8 K, V and K_idx pages (E4M3 codes, one E8M0 scale per 32 elements,
    # neighbouring blocks scaled differently), bf16 queries
    _decode_case(MODEL_SHAPE, [1, 127, 128, 129, 3000, 2049], 125, cache_dtype=MXFP8)
    _decode_case(HeadShape(16, 2, 64, 32, 16), [5000, 2500, 700], 126, cache_dtype=MXFP8)
    _decode_case(HeadShape(16, 4, 128, 128, 8), [1500, 9000], 127, cache_dtype=MXFP8)
    # 64 sequences: no key split in the gather (8-wave workgroups)
    _decode_case(HeadShape(16, 4, 64, 64, 16), [600 + 37 * i for i in range(64)], 128, cache_dtype=MXFP8)


def test_decode_single_long_sequence():
    _decode_case(MODEL_SHAPE, [40000], 22)


# ------------------------------------------------------------------ full size (sampled)

def test_full_size_prefill_32k_sampled_rows():
    msa = _msa()
    shape = MODEL_SHAPE
    n = 32768
    inp = gen_prefill(n, shape, dtype=torch.bfloat16, seed=1, device=DEV)
    _say("32K prefill full size")
    bidx = msa.index_topk(inp["q_idx"], inp["k_idx"], top_k=16)
    o = msa.sparse_prefill(inp["q"], inp["k"], inp["v"], bidx)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = np.sort(np.concatenate([rng.choice(n, 40, replace=False), [0, 127, 128, n - 129, n - 1]]))
    o_ids, _, pooled = orc.index_topk(np64(inp["q_idx"]), np64(inp["k_idx"]), 0, 16, rows=rows)
    g_ids = bidx.cpu().numpy()[rows]
    compare_index_rows(g_ids, o_ids, pooled, rows // 128)
    k64, v64 = np64(inp["k"]), np64(inp["v"])
    q_rows = np64(inp["q"][torch.from_numpy(rows).to(DEV)])
    o_ref = np.stack([orc.sparse_attention(q_rows[t:t + 1], k64, v64, g_ids[t:t + 1], int(i))[0][0]
                      for t, i in enumerate(rows)])
    compare_out(o[torch.from_numpy(rows).to(DEV)], o_ref, torch.bfloat16)


def test_prefill_merge_span_of_several_windows_sampled():
    """16384 queries at 64K context: windows of 1408 tokens whose partials
    (380 MB each) are merged 8 windows per launch, so the second merge covers
    the last 4 windows, the last one ragged (896 tokens).  Rows on both sides
    of every window edge and of the span edge are checked against the oracle."""
    msa = _msa()
    shape = MODEL_SHAPE
    n_kv, n_q, win = 65536, 16384, 1408
    inp = gen_prefill(n_kv, shape, n_q=n_q, dtype=torch.bfloat16, seed=6, device=DEV)
    q0 = inp["q_start"]
    _say("64K context, 16384 queries: merge spans of 8 windows")
    bidx = msa.index_topk(inp["q_idx"], inp["k_idx"], top_k=16, q_start=q0)
    o, lse = msa.sparse_prefill(inp["q"], inp["k"], inp["v"], bidx, q_start=q0, with_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    edges = [e + d for e in range(win, n_q, win) for d in (-1, 0)]
    rows = np.unique(np.concatenate([edges, rng.choice(n_q, 16, replace=False), [0, n_q - 1]]))
    g_ids = bidx.cpu().numpy()[rows]
    o_ids, _, pooled = orc.index_topk(np64(inp["q_idx"]), np64(inp["k_idx"]), q0, 16, rows=rows)
    compare_index_rows(g_ids, o_ids, pooled, (q0 + rows) // 128)
    k64, v64 = np64(inp["k"]), np64(inp["v"])
    rows_t = torch.from_numpy(rows).to(DEV)
    q_rows = np64(inp["q"][rows_t])
    ref = [orc.sparse_attention(q_rows[t:t + 1], k64, v64, g_ids[t:t + 1], q0 + int(i))
           for t, i in enumerate(rows)]
    compare_out(o[rows_t], np.stack([r[0][0] for r in ref]), torch.bfloat16)
    compare_lse(lse[rows_t], np.stack([r[1][0] for r in ref]), torch.bfloat16)


def test_full_size_decode_64x128k_sampled_sequences():
    """Decode step at the benchmark shape (64 x 131072 paged, random page
    table), in the benchmark's launch configuration; 3 sequences checked."""
    msa = _msa()
    shape = MODEL_SHAPE
    inp = gen_decode_paged(64, 131072, shape, seed=3, device=DEV)
    _say("decode 64 x 128K full size")
    q_idx = inp["q_idx"][0].contiguous()
    q = inp["q"][0].contiguous()
    bidx = msa.index_topk(q_idx, inp["k_idx_pages"], top_k=16, page_table=inp["page_table"],
                          seq_lens=inp["seq_lens"])
    o, lse = msa.sparse_decode(q, inp["k_pages"], inp["v_pages"], inp["page_table"], inp["seq_lens"], bidx,
                               with_lse=True)
    torch.cuda.synchronize()
    g_ids = bidx.cpu().numpy()
    L = 131072
    local_pt = np.arange(L // 128)[None, :]
    for s in (0, 21, 63):
        pages = inp["page_table"][s].long()
        kp = np64(inp["k_pages"][pages])
        vp = np64(inp["v_pages"][pages])
        ip = np64(inp["k_idx_pages"][pages])
        o_ids, _, pooled = orc.index_topk_decode(np64(q_idx[s:s + 1]), ip, local_pt, [L], 16)
        compare_index_rows(g_ids[s:s + 1], o_ids, pooled, [(L - 1) // 128])
        o_ref, lse_ref = orc.sparse_decode(np64(q[s:s + 1]), kp, vp, local_pt, [L], g_ids[s:s + 1])
        compare_out(o[s:s + 1], o_ref, torch.bfloat16)
        compare_lse(lse[s:s + 1], lse_ref, torch.bfloat16)


def test_full_size_decode_64x128k_e4m3_sampled_sequences():
    """The 64 x 131072 decode step with e4m3 caches; 2 sequences checked."""
    msa = _msa()
    shape = MODEL_SHAPE
    inp = gen_decode_paged(64, 131072, shape, seed=3, device=DEV, cache_dtype=torch.float8_e4m3fn)
    _say("decode 64 x 128K e4m3 full size")
    q_idx = inp["q_idx"][0].contiguous()
    q = inp["q"][0].contiguous()
    bidx = msa.index_topk(q_idx, inp["k_idx_pages"], top_k=16, page_table=inp["page_table"],
                          seq_lens=inp["seq_lens"])
    o, lse = msa.sparse_decode(q, inp["k_pages"], inp["v_pages"], inp["page_table"], inp["seq_lens"], bidx,
                               with_lse=True)
    torch.cuda.synchronize()
    g_ids = bidx.cpu().numpy()
    L = 131072
    local_pt = np.arange(L // 128)[None, :]
    for s in (5, 60):
        pages = inp["page_table"][s].long()
        kp = _cache_host(inp["k_pages"][pages])
        vp = _cache_host(inp["v_pages"][pages])
        ip = _cache_host(inp["k_idx_pages"][pages])
        o_ids, _, pooled = orc.index_topk_decode(np64(q_idx[s:s + 1]), ip, local_pt, [L], 16)
        compare_index_rows(g_ids[s:s + 1], o_ids, pooled, [(L - 1) // 128])
        o_ref, lse_ref = orc.sparse_decode(np64(q[s:s + 1]), kp, vp, local_pt, [L], g_ids[s:s + 1])
        compare_out(o[s:s + 1], o_ref, torch.bfloat16)
        compare_lse(lse[s:s + 1], lse_ref, torch.bfloat16)


def test_full_size_decode_64x128k_mxfp8_sampled_sequences():
    """The 64 x 131072 decode step with MXFP8 caches; 2 sequences checked."""
    msa = _msa()
    shape = MODEL_SHAPE
    inp = gen_decode_paged(64, 131072, shape, seed=3, device=DEV, cache_dtype=MXFP8)
    _say("decode 64 x 128K MXFP8 full size")
    q_idx = inp["q_idx"][0].contiguous()
    q = inp["q"][0].contiguous()
    ks, vs, kis = inp["k_pages_scale"], inp["v_pages_scale"], inp["k_idx_pages_scale"]
    bidx = msa.index_topk(q_idx, inp["k_idx_pages"], top_k=16, page_table=inp["page_table"],
                          seq_lens=inp["seq_lens"], k_idx_scale=kis)
    o, lse = msa.sparse_decode(q, inp["k_pages"], inp["v_pages"], inp["page_table"], inp["seq_lens"], bidx,
                               with_lse=True, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    g_ids = bidx.cpu().numpy()
    L = 131072
    local_pt = np.arange(L // 128)[None, :]
    for s in (7, 44):
        pages = inp["page_table"][s].long()
        kp = _cache_host(inp["k_pages"][pages], ks[pages])
        vp = _cache_host(inp["v_pages"][pages], vs[pages])
        ip = _cache_host(inp["k_idx_pages"][pages], kis[pages])
        o_ids, _, pooled = orc.index_topk_decode(np64(q_idx[s:s + 1]), ip, local_pt, [L], 16)
        compare_index_rows(g_ids[s:s + 1], o_ids, pooled, [(L - 1) // 128])
        o_ref, lse_ref = orc.sparse_decode(np64(q[s:s + 1]), kp, vp, local_pt, [L], g_ids[s:s + 1])
        compare_out(o[s:s + 1], o_ref, torch.bfloat16, rel_elem=MX_REL)
        compare_lse(lse[s:s + 1], lse_ref, torch.bfloat16)


def test_full_size_prefill_128k_planted():
    """131072-token prefill with planted index keys: every designated query
    of every group retrieves its 3 planted blocks; sampled rows match the
    oracle (index lists and outputs)."""
    from synth import gen_planted_prefill
    msa = _msa()
    shape = MODEL_SHAPE
    n = 131072
    inp = gen_planted_prefill(n, shape, device=DEV)
    _say("128K planted prefill full size")
    bidx = msa.index_topk(inp["q_idx"], inp["k_idx"], top_k=16)
    o = msa.sparse_prefill(inp["q"], inp["k"], inp["v"], bidx)
    torch.cuda.synchronize()
    g_ids = bidx.cpu().numpy()
    des = inp["designated"].numpy()
    for r in range(shape.h_kv):
        planted = set(inp["planted_blocks"][r].tolist())
        for i in des:
            assert planted <= set(g_ids[i, r].tolist()), (r, int(i), g_ids[i, r], planted)
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([des[:6], rng.choice(n, 12, replace=False), [0, 129, n - 1]]))
    o_ids, _, pooled = orc.index_topk(np64(inp["q_idx"]), np64(inp["k_idx"]), 0, 16, rows=rows)
    compare_index_rows(g_ids[rows], o_ids, pooled, rows // 128)
    rows_t = torch.from_numpy(rows).to(DEV)
    k64, v64 = np64(inp["k"]), np64(inp["v"])
    q_rows = np64(inp["q"][rows_t])
    o_ref = np.stack([orc.sparse_attention(q_rows[t:t + 1], k64, v64, g_ids[rows][t:t + 1], int(i))[0][0]
                      for t, i in enumerate(rows)])
    compare_out(o[rows_t], o_ref, torch.bfloat16)


def _selected_tokens(k_pages, v_pages, page_row, ids_row, p, r):
    """Keys/values of group r over the listed blocks (ascending), visible up
    to position p, gathered from a paged cache, and the query position
    inside that gathered run.  Eq. (8) reads nothing else, so attending over
    this run equals attending over the whole sequence with the same list."""
    blocks = sorted(int(b) for b in set(ids_row.tolist()) if b >= 0 and b * 128 <= p)
    pages = torch.tensor([int(page_row[b]) for b in blocks], dtype=torch.long, device=k_pages.device)
    kb = np64(k_pages[pages, r].reshape(-1, k_pages.shape[-1]))   # [nb * 128, d]
    vb = np64(v_pages[pages, r].reshape(-1, v_pages.shape[-1]))
    n_vis = 128 * (len(blocks) - 1) + (p - 128 * blocks[-1]) + 1
    return kb[:n_vis], vb[:n_vis], len(blocks)


def _oracle_rows_paged(q_rows, k_pages, v_pages, page_row, ids_rows, positions, h_kv):
    """orc.sparse_attention per (row, group) on the gathered selected run."""
    h_q = q_rows.shape[1]
    G = h_q // h_kv
    o_all = np.empty(q_rows.shape)
    lse_all = np.empty(q_rows.shape[:2])
    for t, p in enumerate(positions):
        for r in range(h_kv):
            kb, vb, nb = _selected_tokens(k_pages, v_pages, page_row, ids_rows[t, r], int(p), r)
            local = np.arange(nb, dtype=np.int64)[None, None, :]
            qg = q_rows[t:t + 1, r * G:(r + 1) * G]
            o, lse = orc.sparse_attention(qg, kb[:, None, :], vb[:, None, :], local, kb.shape[0] - 1)
            o_all[t, r * G:(r + 1) * G] = o[0]
            lse_all[t, r * G:(r + 1) * G] = lse[0]
    return o_all, lse_all


def test_long_context_1m_chunked_prefill_and_decode_sampled():
    """1,048,576-token paged cache: chunked prefill of the last 8192 queries
    (sampled rows checked) and the first two decode steps, each appending
    its token first (both checked)."""
    msa = _msa()
    shape = MODEL_SHAPE
    lc = gen_long_context(device=DEV)
    n_ctx, q_start = lc["n_ctx"], lc["q_start"]
    pt = lc["page_table"]
    _say("1M chunked prefill + decode")
    bidx = msa.index_topk(lc["chunk_q_idx"], lc["k_idx_pages"], top_k=16, q_start=q_start, page_table=pt[0],
                          n_kv=n_ctx)
    o = msa.sparse_prefill(lc["chunk_q"], lc["k_pages"], lc["v_pages"], bidx, q_start=q_start, page_table=pt[0],
                           n_kv=n_ctx)
    torch.cuda.synchronize()
    g_ids = bidx.cpu().numpy()
    pt_row = pt[0].cpu().numpy()
    seq = orc.gather_sequence(pt_row, n_ctx, k_idx_pages=lc["k_idx_pages"].float().cpu().numpy())
    rng = np.random.default_rng(5)
    nq = lc["chunk_q"].shape[0]
    rows = np.unique(np.concatenate([rng.choice(nq, 10, replace=False), [0, 1, 127, nq - 1]]))
    o_ids, _, pooled = orc.index_topk(np64(lc["chunk_q_idx"]), seq["k_idx"], q_start, 16, rows=rows)
    compare_index_rows(g_ids[rows], o_ids, pooled, (q_start + rows) // 128)
    rows_t = torch.from_numpy(rows).to(DEV)
    o_ref, _ = _oracle_rows_paged(np64(lc["chunk_q"][rows_t]), lc["k_pages"], lc["v_pages"], pt_row,
                                  g_ids[rows], q_start + rows, shape.h_kv)
    compare_out(o[rows_t], o_ref, torch.bfloat16)
    # two decode steps
    seq_lens = torch.tensor([n_ctx], dtype=torch.int32, device=DEV)
    k_idx_host = seq["k_idx"]
    for t in range(2):
        pos = n_ctx + t
        page = pt[0, pos // 128].long()
        lc["k_pages"][page, :, pos % 128] = lc["step_k"][t]
        lc["v_pages"][page, :, pos % 128] = lc["step_v"][t]
        lc["k_idx_pages"][page, pos % 128] = lc["step_k_idx"][t]
        seq_lens.fill_(pos + 1)
        db = msa.index_topk(lc["step_q_idx"][t], lc["k_idx_pages"], top_k=16, page_table=pt, seq_lens=seq_lens)
        do, dl = msa.sparse_decode(lc["step_q"][t], lc["k_pages"], lc["v_pages"], pt, seq_lens, db,
                                   with_lse=True)
        torch.cuda.synchronize()
        k_idx_host = np.concatenate([k_idx_host, np64(lc["step_k_idx"][t:t + 1])])
        d_ids = db.cpu().numpy()
        oi, _, dp = orc.index_topk(np64(lc["step_q_idx"][t][0:1]), k_idx_host, pos, 16)
        compare_index_rows(d_ids, oi, dp, [pos // 128])
        d_ref, l_ref = _oracle_rows_paged(np64(lc["step_q"][t]), lc["k_pages"], lc["v_pages"], pt_row,
                                          d_ids, [pos], shape.h_kv)
        compare_out(do, d_ref, torch.bfloat16)
        compare_lse(dl, l_ref, torch.bfloat16)


# ------------------------------------------------------------- training path

def _backward_case(shape, n_kv, n_q, seed, *, all_blocks=False):
    msa = _msa()
    inp = gen_prefill(n_kv, shape, n_q=n_q, dtype=torch.bfloat16, seed=seed, device=DEV)
    q_start = inp["q_start"]
    _say("backward", shape, n_kv, n_q, seed, "all blocks" if all_blocks else "")
    top_k = shape.top_k
    if all_blocks:
        # every query keeps the first k - 1 blocks ("sink" blocks) and its own
        bidx = torch.full((n_q, shape.h_kv, top_k), -1, dtype=torch.int32)
        for i in range(n_q):
            d = (q_start + i) // 128
            ids = sorted(set(range(min(top_k - 1, d))) | {d})
            bidx[i, :, :len(ids)] = torch.tensor(ids, dtype=torch.int32)
        bidx = bidx.to(DEV)
    else:
        bidx = msa.index_topk(inp["q_idx"], inp["k_idx"], top_k=top_k, q_start=q_start)
    o, lse = msa.sparse_prefill(inp["q"], inp["k"], inp["v"], bidx, q_start=q_start, with_lse=True)
    g = torch.Generator(device="cpu").manual_seed(seed + 1000)
    d_o = torch.randn(inp["q"].shape, generator=g).to(torch.bfloat16).to(DEV)
    dq, dk, dv = msa.sparse_prefill_backward(inp["q"], inp["k"], inp["v"], bidx, o, lse, d_o, q_start=q_start)
    torch.cuda.synchronize()
    ids = bidx.cpu().numpy()
    rq, rk, rv = orc.sparse_attention_backward(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]), ids, q_start,
                                               np64(d_o))
    compare_grad(dq, rq, "dq")
    compare_grad(dk, rk, "dk")
    compare_grad(dv, rv, "dv")
    return dq, dk, dv


def test_backward_model_shape_ragged():
    _backward_case(MODEL_SHAPE, 2300, 2300, 50)


def test_backward_chunked_q_start_and_untouched_keys():
    # queries over the last 700 of 3000 keys: keys no query selected get 0
    dq, dk, dv = _backward_case(MODEL_SHAPE, 3000, 700, 51)
    assert torch.isfinite(dk.float()).all() and torch.isfinite(dv.float()).all()


def test_backward_head_ratios_and_d64():
    _backward_case(HeadShape(16, 2, 64, 32, 6), 1700, 1700, 52)
    _backward_case(HeadShape(16, 16, 128, 64, 8), 900, 900, 53)
    _backward_case(HeadShape(64, 8, 128, 64, 16), 1300, 1300, 54)


def test_backward_hot_block_split_over_items():
    # every query selects the same 15 sink blocks: those cells hold 4500
    # tokens, more than one item takes, so their dK/dV go through the
    # split-cell reduction
    _backward_case(HeadShape(16, 1, 128, 64, 16), 4500, 4500, 55, all_blocks=True)


def test_backward_deterministic():
    msa = _msa()
    inp = gen_prefill(1500, MODEL_SHAPE, dtype=torch.bfloat16, seed=56, device=DEV)
    bidx = msa.index_topk(inp["q_idx"], inp["k_idx"], top_k=16)
    o, lse = msa.sparse_prefill(inp["q"], inp["k"], inp["v"], bidx, with_lse=True)
    d_o = torch.randn(inp["q"].shape, generator=torch.Generator().manual_seed(9)).to(torch.bfloat16).to(DEV)
    a = msa.sparse_prefill_backward(inp["q"], inp["k"], inp["v"], bidx, o, lse, d_o)
    b = msa.sparse_prefill_backward(inp["q"], inp["k"], inp["v"], bidx, o, lse, d_o)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_no_queries_zero_fills():
    msa = _msa()
    inp = gen_prefill(600, MODEL_SHAPE, n_q=1, dtype=torch.bfloat16, seed=57, device=DEV)
    q0 = inp["q"][:0]
    bidx = torch.empty((0, 4, 16), dtype=torch.int32, device=DEV)
    dk = torch.full_like(inp["k"], 3.0)
    dv = torch.full_like(inp["v"], 3.0)
    msa.sparse_prefill_backward(q0, inp["k"], inp["v"], bidx, q0, torch.empty((0, 64), device=DEV), q0,
                                q_start=600, out=(q0, dk, dv))
    torch.cuda.synchronize()
    assert not dk.any() and not dv.any()


def _kl_case(shape, n_kv, n_q, seed, *, kl_scale=1.0, sinks=False):
    msa = _msa()
    inp = gen_prefill(n_kv, shape, n_q=n_q, dtype=torch.bfloat16, seed=seed, device=DEV)
    q_start = inp["q_start"]
    _say("kl alignment", shape, n_kv, n_q, seed, kl_scale, "sinks" if sinks else "")
    if sinks:
        bidx = torch.full((n_q, shape.h_kv, shape.top_k), -1, dtype=torch.int32)
        for i in range(n_q):
            d = (q_start + i) // 128
            ids = sorted(set(range(min(shape.top_k - 1, d))) | {d})
            bidx[i, :, :len(ids)] = torch.tensor(ids, dtype=torch.int32)
        bidx = bidx.to(DEV)
    else:
        bidx = msa.index_topk(inp["q_idx"], inp["k_idx"], top_k=shape.top_k, q_start=q_start)
    o, lse = msa.sparse_prefill(inp["q"], inp["k"], inp["v"], bidx, q_start=q_start, with_lse=True)
    d_o = torch.randn(inp["q"].shape, generator=torch.Generator().manual_seed(seed + 7)).to(torch.bfloat16).to(DEV)
    dq, dk, dv, kl, dqi, dki = msa.sparse_prefill_backward(inp["q"], inp["k"], inp["v"], bidx, o, lse, d_o,
                                                           q_start=q_start, q_idx=inp["q_idx"], k_idx=inp["k_idx"],
                                                           kl_scale=kl_scale)
    torch.cuda.synchronize()
    ids = bidx.cpu().numpy()
    r_kl, r_dqi, r_dki = orc.kl_alignment(np64(inp["q_idx"]), np64(inp["k_idx"]), np64(inp["q"]), np64(inp["k"]),
                                          ids, q_start, kl_scale=kl_scale)
    g_kl = kl.cpu().double().numpy()
    err = np.abs(g_kl - r_kl)
    assert err.max() <= 2e-2 * max(1.0, float(np.abs(r_kl).max())), ("kl", float(err.max()))
    assert np.linalg.norm(g_kl - r_kl) <= 1e-2 * max(np.linalg.norm(r_kl), 1e-30), "kl relative L2"
    compare_grad(dqi, r_dqi, "dq_idx")
    compare_grad(dki, r_dki, "dk_idx")
    # the attention gradients are unchanged by asking for the KL term
    rq, rk, rv = orc.sparse_attention_backward(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]), ids, q_start,
                                               np64(d_o))
    compare_grad(dq, rq, "dq")
    compare_grad(dk, rk, "dk")
    compare_grad(dv, rv, "dv")


def test_kl_alignment_model_shape_ragged():
    _kl_case(MODEL_SHAPE, 2300, 2300, 60, kl_scale=0.5)


def test_kl_alignment_head_ratios_d_idx_and_chunked_start():
    _kl_case(HeadShape(16, 2, 64, 32, 6), 1700, 1700, 61)
    _kl_case(HeadShape(8, 8, 128, 128, 8), 900, 900, 62, kl_scale=2.0)
    _kl_case(MODEL_SHAPE, 3000, 700, 63)


def test_kl_alignment_hot_blocks():
    _kl_case(HeadShape(16, 1, 128, 64, 16), 4500, 4500, 64, sinks=True)


def test_kl_alignment_vanishes_when_branches_agree():
    # one KV group with one head, d_idx = d_h, q_idx = q, k_idx = k and equal
    # scales: the two distributions coincide, so KL and its gradients are ~0
    msa = _msa()
    shape = HeadShape(1, 1, 64, 64, 4)
    inp = gen_prefill(900, shape, dtype=torch.bfloat16, seed=65, device=DEV)
    q, k = inp["q"], inp["k"]
    k_idx = k[:, 0].contiguous()
    bidx = msa.index_topk(q, k_idx, top_k=4)
    o, lse = msa.sparse_prefill(q, k, inp["v"], bidx, with_lse=True)
    out = msa.sparse_prefill_backward(q, k, inp["v"], bidx, o, lse, torch.zeros_like(q), q_idx=q, k_idx=k_idx)
    torch.cuda.synchronize()
    kl, dqi, dki = out[3].cpu(), out[4].cpu().float(), out[5].cpu().float()
    assert kl.abs().max().item() < 5e-3
    # the gradients are small next to those of an unrelated index branch
    ref = msa.sparse_prefill_backward(q, k, inp["v"], bidx, o, lse, torch.zeros_like(q), q_idx=inp["q_idx"],
                                      k_idx=k_idx)
    torch.cuda.synchronize()
    assert dqi.abs().max().item() < 0.05 * max(ref[4].cpu().float().abs().max().item(), 1e-6)


# ------------------------------------------ index projections, RoPE, append

def _project_case(n_tok, d_model, h_kv, d_idx, rope_dim, seed, *, paged, positions=None):
    msa = _msa()
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(n_tok, d_model, generator=g).to(torch.bfloat16)
    wq = (torch.randn(h_kv, d_idx, d_model, generator=g) * (0.5 / d_model ** 0.5)).to(torch.bfloat16)
    wk = (torch.randn(d_idx, d_model, generator=g) * (0.5 / d_model ** 0.5)).to(torch.bfloat16)
    _say("index_project", n_tok, d_model, h_kv, d_idx, rope_dim, "paged" if paged else "contiguous")
    if paged:
        # decode-like: token t is the new token of sequence t
        pos = positions if positions is not None else torch.randint(0, 1 << 20, (n_tok,), generator=g)
        max_pages = int(pos.max().item()) // 128 + 1
        # every logical page of sequence t maps to physical page perm[t] (only
        # the page holding the new token is written)
        perm = torch.randperm(n_tok + 3, generator=g)[:n_tok].to(torch.int32)
        pt = perm[:, None].expand(n_tok, max_pages).contiguous()
        cache = torch.randn(n_tok + 3, 128, d_idx, generator=g).to(torch.bfloat16)
        before = cache.clone()
        q = msa.index_project(x.to(DEV), wq.to(DEV), wk.to(DEV), pos.to(torch.int32).to(DEV), c := cache.to(DEV),
                              rope_dim=rope_dim, page_table=pt.to(DEV), seq=torch.arange(n_tok, dtype=torch.int32).to(DEV))
    else:
        q_start = 5000
        pos = torch.arange(q_start, q_start + n_tok)
        cache = torch.randn(q_start + n_tok + 7, d_idx, generator=g).to(torch.bfloat16)
        before = cache.clone()
        q = msa.index_project(x.to(DEV), wq.to(DEV), wk.to(DEV), pos.to(torch.int32).to(DEV), c := cache.to(DEV),
                              rope_dim=rope_dim)
    torch.cuda.synchronize()
    rq, rk = orc.index_projection(np64(x), np64(wq), np64(wk), pos.numpy(), rope_dim=rope_dim)
    compare_out(q, rq, torch.bfloat16, "q_idx")
    got = c.cpu()
    expect = before.clone()
    if paged:
        for t in range(n_tok):
            p = int(pos[t])
            expect[pt[t, p // 128], p % 128] = torch.from_numpy(rk[t]).to(torch.bfloat16)
            compare_out(got[pt[t, p // 128], p % 128][None], rk[t][None], torch.bfloat16, "k_idx row")
        written = torch.zeros(got.shape[:2], dtype=torch.bool)
        for t in range(n_tok):
            p = int(pos[t])
            written[pt[t, p // 128], p % 128] = True
        assert torch.equal(got[~written], before[~written]), "rows other than the appended ones changed"
    else:
        compare_out(got[pos], rk, torch.bfloat16, "k_idx rows")
        keep = torch.ones(got.shape[0], dtype=torch.bool)
        keep[pos] = False
        assert torch.equal(got[keep], before[keep]), "rows other than the appended ones changed"


def test_index_project_decode_paged_rope64():
    _project_case(64, 1024, 4, 64, 64, 70, paged=True)


def test_index_project_prefill_contiguous_variants():
    _project_case(1000, 512, 4, 64, 64, 71, paged=False)
    _project_case(300, 256, 2, 32, 32, 72, paged=False)
    _project_case(200, 768, 8, 128, 64, 73, paged=False)
    _project_case(150, 256, 1, 128, 128, 74, paged=False)
    _project_case(97, 256, 4, 64, 0, 75, paged=False)


def test_index_project_long_call_tiles():
    # calls of 256 tokens and more take the tiled kernel: d_idx 32 / 64 / 128,
    # d_model with a 16-wide tail past the last 64-wide chunk, token counts
    # that end inside a tile, projections split over several workgroups with
    # an idle wave in the last (h_kv 16: 17 projections as 6 + 6 + 5), and a
    # paged cache
    _project_case(1000, 784, 8, 128, 64, 78, paged=False)
    _project_case(600, 528, 1, 128, 128, 79, paged=False)
    _project_case(513, 1040, 4, 32, 32, 80, paged=False)
    _project_case(700, 256, 16, 64, 64, 81, paged=False)
    _project_case(256, 272, 4, 64, 0, 82, paged=False)
    _project_case(300, 512, 4, 64, 64, 83, paged=True)


def test_index_project_short_call_splits():
    # calls under 256 tokens split d_model over workgroups and add the fp32
    # slices in a second kernel: RoPE pairs only (rope_dim = d_idx), pairs and
    # plain dims (d_idx 128, RoPE 64), no RoPE, d_idx 32, paged and contiguous
    _project_case(40, 1024, 2, 32, 0, 84, paged=False)      # 4 slices, no RoPE
    _project_case(100, 2048, 4, 32, 32, 85, paged=True)     # 8 slices
    _project_case(33, 4096, 4, 128, 64, 86, paged=False)    # 16 slices, 64 rotated + 64 plain dims
    _project_case(255, 784, 4, 64, 64, 87, paged=False)     # 3 slices of 272


def test_index_project_large_positions_paged():
    # positions near 2^20 + 255: the angle must be formed without fp32 rounding
    pos = torch.tensor([1048575, 1048831, 1048576, 0, 127, 128, 999999, 524288], dtype=torch.int64)
    _project_case(8, 256, 4, 64, 64, 76, paged=True, positions=pos)


# ------------------------------------------------ full sizes, sampled outputs

def test_full_size_backward_and_kl_32k_sampled():
    """The 32K prefill shape as bench.py times it (backward with the KL term):
    dq, KL and dq_idx on sampled query rows (a row's values depend on that row
    only); dk, dv on sampled (group, block) cells and dk_idx on sampled blocks,
    from the oracle run on exactly the queries that selected them."""
    msa = _msa()
    n = 32768
    inp = gen_prefill(n, MODEL_SHAPE, dtype=torch.bfloat16, seed=1, device=DEV)
    _say("backward + KL 32K full size")
    bidx = msa.index_topk(inp["q_idx"], inp["k_idx"], top_k=16)
    o, lse = msa.sparse_prefill(inp["q"], inp["k"], inp["v"], bidx, with_lse=True)
    d_o = torch.randn(inp["q"].shape, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16).to(DEV)
    kl_scale = 1.0 / (n * 4)
    dq, dk, dv, kl, dqi, dki = msa.sparse_prefill_backward(inp["q"], inp["k"], inp["v"], bidx, o, lse, d_o,
                                                           q_idx=inp["q_idx"], k_idx=inp["k_idx"], kl_scale=kl_scale)
    torch.cuda.synchronize()
    ids = bidx.cpu().numpy()
    q64, k64, v64, do64 = np64(inp["q"]), np64(inp["k"]), np64(inp["v"]), np64(d_o)
    qi64, ki64 = np64(inp["q_idx"]), np64(inp["k_idx"])
    rng = np.random.default_rng(7)
    rows = sorted(set([0, 127, 128, 4095, n - 1] + rng.integers(0, n, 27).tolist()))
    rq, _, _ = orc.sparse_attention_backward(q64, k64, v64, ids, 0, do64, rows=rows)
    compare_grad(np64(dq)[rows], rq[rows], "dq rows")
    r_kl, r_dqi, _ = orc.kl_alignment(qi64, ki64, q64, k64, ids, 0, kl_scale=kl_scale, rows=rows)
    g_kl = kl.cpu().double().numpy()[rows]
    assert np.abs(g_kl - r_kl[rows]).max() <= 2e-2 * max(1.0, float(np.abs(r_kl[rows]).max())), "kl rows"
    compare_grad(np64(dqi)[rows], r_dqi[rows], "dq_idx rows")
    for r, b in ((1, 200), (3, 255), (0, 180)):
        sel = np.nonzero((ids[:, r, :] == b).any(axis=1))[0]
        sub = np.full_like(ids, -1)
        sub[sel, r] = ids[sel, r]
        _, rk, rv = orc.sparse_attention_backward(q64, k64, v64, sub, 0, do64, rows=sel)
        keys = slice(b * 128, min(b * 128 + 128, n))
        compare_grad(np64(dk)[keys, r], rk[keys, r], f"dk block {b} group {r}")
        compare_grad(np64(dv)[keys, r], rv[keys, r], f"dv block {b} group {r}")
    for b in (240, 255):
        sel = np.nonzero((ids == b).any(axis=(1, 2)))[0]
        _, _, rki = orc.kl_alignment(qi64, ki64, q64, k64, ids, 0, kl_scale=kl_scale, rows=sel)
        keys = slice(b * 128, min(b * 128 + 128, n))
        compare_grad(np64(dki)[keys], rki[keys], f"dk_idx block {b}")


def test_full_size_index_project_32k_and_decode64_sampled():
    """bench.py's projection shapes: 32768 tokens at d_model 6144 (sampled rows)
    and a 64-sequence paged decode step (all rows)."""
    msa = _msa()
    dm, h_kv, di = 6144, 4, 64
    g = torch.Generator().manual_seed(5)
    wq = (torch.randn(h_kv, di, dm, generator=g) / dm ** 0.5).to(torch.bfloat16)
    wk = (torch.randn(di, dm, generator=g) / dm ** 0.5).to(torch.bfloat16)
    n = 32768
    _say("index_project 32K x 6144")
    x = torch.randn(n, dm, generator=g).to(torch.bfloat16)
    pos = torch.arange(n, dtype=torch.int32)
    cache = torch.zeros(n, di, dtype=torch.bfloat16, device=DEV)
    q = msa.index_project(x.to(DEV), wq.to(DEV), wk.to(DEV), pos.to(DEV), cache)
    torch.cuda.synchronize()
    rows = [0, 1, 127, 4096, 20000, n - 1]
    rq, rk = orc.index_projection(np64(x[rows]), np64(wq), np64(wk), pos[rows].numpy())
    compare_out(q.cpu()[rows], rq, torch.bfloat16, "q_idx rows")
    compare_out(cache.cpu()[rows], rk, torch.bfloat16, "k_idx rows")
    _project_case(64, dm, h_kv, di, 64, 77, paged=True, positions=torch.full((64,), 131071, dtype=torch.int64))

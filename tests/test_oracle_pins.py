"""Pins for the float64 oracle, each against something other than the oracle
itself: printed numbers on the pages, hand-derived closed forms, brute force
over subsets, an independent library (torch's SDPA in float64 on the CPU),
special cases and invariants.  CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import msa_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- Eq. (12)

def test_eq12_ratio_matches_printed_28_4():
    g = _golden("eq12_flop_ratio.json")
    f_gqa, f_idx, f_main = orc.flops_eq12(g["n"], g["h_q"], g["h_kv"], g["d_h"], 128,
                                          g["top_k"], g["block"])
    ratio = f_gqa / (f_idx + f_main)
    assert abs(ratio - g["ratio_printed"]) < g["printed_precision"]
    # the index term is quadratic, the main term linear in N
    f2 = orc.flops_eq12(2 * g["n"], g["h_q"], g["h_kv"], g["d_h"], 128, g["top_k"])
    assert f2[1] == pytest.approx(4 * f_idx)
    assert f2[2] == pytest.approx(2 * f_main)


# ------------------------------------------------- index branch: closed form

def _closed_form_inputs(g):
    n_kv, d = g["n_kv"], g["d_idx"]
    k_idx = np.zeros((n_kv, d))
    k_idx[:, 0] = -1.0
    for b, (v, o) in enumerate(zip(g["peak_value"], g["peak_offset"])):
        k_idx[b * 128 + o, 0] = v
    q_row = np.zeros((g["h_kv"], d))
    q_row[:, 0] = g["group_coef"]
    return q_row, k_idx


def test_closed_form_selection_and_scores():
    g = _golden("closed_form_selection.json")
    q_row, k_idx = _closed_form_inputs(g)
    for case in g["cases"]:
        p = case["p"]
        ids, sc, pooled = orc.index_topk(q_row[None], k_idx, p, case["top_k"],
                                         force_local=case["force_local"])
        assert ids[0].tolist() == case["expect"], case["why"]
        if "expect_score_group0" in case:
            np.testing.assert_allclose(sc[0, 0], case["expect_score_group0"], rtol=1e-12)
        if "expect_diag_score_group0" in case:
            assert pooled[0][0, p // 128] == pytest.approx(case["expect_diag_score_group0"], rel=1e-12)


def test_token_scores_closed_form_scale():
    # S_j = <q, k_j> / sqrt(d): orthogonal unit vectors give 0, parallel give |q||k|/sqrt(d)
    d = 16
    q = np.zeros((1, d))
    q[0, 3] = 5.0
    k = np.zeros((4, d))
    k[0, 3] = 2.0
    k[1, 4] = 7.0
    k[2, 3] = -1.5
    k[3, :] = 1.0
    s = orc.index_token_scores(q, k, 3)
    np.testing.assert_allclose(s[0], [10.0 / 4.0, 0.0, -7.5 / 4.0, 5.0 / 4.0], rtol=1e-15)
    s2 = orc.index_token_scores(q, k, 1, idx_scale=1.0)
    np.testing.assert_allclose(s2[0], [10.0, 0.0])


# ---------------------------------------------- index branch: brute force

def _brute_force_topk(m, diag, k, force_local):
    """Enumerate every subset of the eligible blocks of the right size and keep
    the one(s) where every chosen block beats every left-out block under
    (score desc, index asc)."""
    cand = list(range(diag)) if force_local else list(range(diag + 1))
    take = min(len(cand), k - 1 if force_local else k)
    winners = []
    for sub in itertools.combinations(cand, take):
        rest = [b for b in cand if b not in sub]
        ok = all((m[s] > m[u]) or (m[s] == m[u] and s < u) for s in sub for u in rest)
        if ok:
            winners.append(sorted(list(sub) + ([diag] if force_local else [])))
    assert len(winners) == 1
    w = winners[0]
    return w + [-1] * (k - len(w))


@pytest.mark.parametrize("seed", range(40))
def test_selection_matches_subset_brute_force(seed):
    rng = np.random.default_rng(seed)
    diag = int(rng.integers(0, 9))
    k = int(rng.integers(1, 6))
    # few distinct values so ties are common
    m = rng.integers(-3, 4, size=diag + 1).astype(np.float64) * 0.5
    for force in (True, False):
        if not force and k < 1:
            continue
        got = orc.select_blocks(m, diag, k, force_local=force).tolist()
        assert got == _brute_force_topk(m, diag, k, force)


def test_exp_free_selection_invariance():
    # selection on raw pooled scores equals selection on exp(scores) and on a
    # row softmax of the token scores (monotone maps keep the order)
    rng = np.random.default_rng(7)
    n, d = 1500, 16
    q = rng.standard_normal((6, 2, d))
    k = rng.standard_normal((n, d))
    for i in range(q.shape[0]):
        p = int(rng.integers(0, n))
        s = orc.index_token_scores(q[i], k, p)
        m_raw = orc.block_max_pool(s, p)
        m_exp = orc.block_max_pool(np.exp(s), p)
        soft = np.exp(s - s.max(axis=1, keepdims=True))
        soft /= soft.sum(axis=1, keepdims=True)
        m_soft = orc.block_max_pool(soft, p)
        for r in range(2):
            a = orc.select_blocks(m_raw[r], p // 128, 5)
            assert (a == orc.select_blocks(m_exp[r], p // 128, 5)).all()
            assert (a == orc.select_blocks(m_soft[r], p // 128, 5)).all()


def test_selection_invariants_random():
    rng = np.random.default_rng(11)
    n, d, h_kv, k = 3000, 32, 3, 6
    q = rng.standard_normal((n, h_kv, d))
    kk = rng.standard_normal((n, d))
    rows = rng.choice(n, 60, replace=False)
    ids, sc, _ = orc.index_topk(q, kk, 0, k, rows=rows)
    for t, i in enumerate(rows):
        diag = i // 128
        for r in range(h_kv):
            row = ids[t, r]
            valid = row[row >= 0]
            assert len(valid) == min(k, diag + 1)
            assert (row[len(valid):] == -1).all()
            assert (np.diff(valid) > 0).all()
            assert valid.max() == diag and diag in valid
            assert (sc[t, r][row < 0] == -np.inf).all()
    # scaling either index tensor by c > 0 changes nothing
    ids2, _, _ = orc.index_topk(q * 3.5, kk, 0, k, rows=rows)
    ids3, _, _ = orc.index_topk(q, kk * 0.25, 0, k, rows=rows)
    assert (ids2 == ids).all() and (ids3 == ids).all()


def test_block_pool_is_order_free_inside_past_blocks():
    rng = np.random.default_rng(5)
    n, d = 1024, 8
    q = rng.standard_normal((2, d))
    k = rng.standard_normal((n, d))
    p = 1000
    m0 = orc.block_max_pool(orc.index_token_scores(q, k, p), p)
    k2 = k.copy()
    perm = rng.permutation(128) + 256          # shuffle tokens of block 2
    k2[256:384] = k[perm]
    m1 = orc.block_max_pool(orc.index_token_scores(q, k2, p), p)
    np.testing.assert_array_equal(m0, m1)
    # moving the block's best token into the next block moves the block max
    s = orc.index_token_scores(q, k, p)
    j = 256 + int(np.argmax(s[0, 256:384]))
    k3 = k.copy()
    k3[[j, 384]] = k3[[384, j]]
    m3 = orc.block_max_pool(orc.index_token_scores(q, k3, p), p)
    assert m3[0, 3] >= m0[0, 2]


def test_planted_blocks_are_retrieved():
    # scaled-down version of the planted long-context workload
    from synth import gen_planted_prefill
    from synth.inputs import HeadShape as HS
    shape = HS(h_q=8, h_kv=4, d_h=32, d_idx=64, top_k=16)
    inp = gen_planted_prefill(16384, shape, dtype=torch.float32, n_designated=12,
                              plant_hi=64, designated_after=8192, seed=21)
    q_idx = inp["q_idx"].double().numpy()
    k_idx = inp["k_idx"].double().numpy()
    rows = inp["designated"].tolist()
    ids, _, _ = orc.index_topk(q_idx, k_idx, 0, 16, rows=rows)
    for t in range(len(rows)):
        for r in range(4):
            assert set(inp["planted_blocks"][r].tolist()) <= set(ids[t, r].tolist())


# ------------------------------------------------- main branch pins

def _sdpa_masked(q, k, v, mask, scale=None):
    """torch SDPA in float64 on the CPU with an explicit boolean mask
    [n_q, n_kv] per KV group.  q [n_q, h_q, d]; k/v [n_kv, h_kv, d]."""
    n_q, h_q, d = q.shape
    h_kv = k.shape[1]
    g = h_q // h_kv
    qt = torch.from_numpy(np.ascontiguousarray(q)).permute(1, 0, 2)              # [h_q, n_q, d]
    kt = torch.from_numpy(np.ascontiguousarray(k)).permute(1, 0, 2).repeat_interleave(g, 0)
    vt = torch.from_numpy(np.ascontiguousarray(v)).permute(1, 0, 2).repeat_interleave(g, 0)
    m = torch.from_numpy(mask).repeat_interleave(g, 0)                          # [h_q, n_q, n_kv]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return o.permute(1, 0, 2).numpy()


def _rand_qkv(rng, n_q, n_kv, h_q, h_kv, d):
    return (rng.standard_normal((n_q, h_q, d)), rng.standard_normal((n_kv, h_kv, d)),
            rng.standard_normal((n_kv, h_kv, d)))


def test_dense_matches_torch_sdpa():
    rng = np.random.default_rng(3)
    n_kv, n_q, h_q, h_kv, d = 300, 50, 8, 2, 16
    q, k, v = _rand_qkv(rng, n_q, n_kv, h_q, h_kv, d)
    q_start = n_kv - n_q
    o, lse = orc.dense_attention(q, k, v, q_start)
    pos = q_start + np.arange(n_q)
    mask = (np.arange(n_kv)[None, :] <= pos[:, None])
    ref = _sdpa_masked(q, k, v, np.broadcast_to(mask, (h_kv, n_q, n_kv)).copy())
    np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-12)
    # lse against torch.logsumexp of the masked scores
    s = np.einsum("ihd,jhd->hij", q[:, :1], k[:, :1]) / math.sqrt(d)
    s = np.where(mask[None], s, -np.inf)
    ref_lse = torch.logsumexp(torch.from_numpy(s), dim=-1).numpy()[0]
    np.testing.assert_allclose(lse[:, 0], ref_lse, rtol=1e-12)


def test_sparse_matches_masked_sdpa_for_arbitrary_selections():
    rng = np.random.default_rng(4)
    n, h_q, h_kv, d, k = 900, 8, 2, 16, 3
    q, kk, v = _rand_qkv(rng, n, n, h_q, h_kv, d)
    bidx = np.full((n, h_kv, k), -1, dtype=np.int64)
    mask = np.zeros((h_kv, n, n), dtype=bool)
    for i in range(n):
        diag = i // 128
        for r in range(h_kv):
            chosen = sorted(set(rng.choice(diag + 1, size=min(k, diag + 1), replace=False).tolist()))
            bidx[i, r, :len(chosen)] = chosen
            for b in chosen:
                mask[r, i, b * 128:min(b * 128 + 128, i + 1)] = True
    rows = list(range(0, n, 7))
    o, _ = orc.sparse_attention(q, kk, v, bidx, 0, rows=rows)
    ref = _sdpa_masked(q, kk, v, mask)
    np.testing.assert_allclose(o, ref[rows], rtol=1e-10, atol=1e-12)
    # a scale argument reaches the softmax
    o2, _ = orc.sparse_attention(q, kk, v, bidx, 0, rows=rows, sm_scale=0.3)
    ref2 = _sdpa_masked(q, kk, v, mask, scale=0.3)
    np.testing.assert_allclose(o2, ref2[rows], rtol=1e-10, atol=1e-12)


def test_full_coverage_and_short_sequences_reduce_to_dense():
    rng = np.random.default_rng(6)
    n, h_q, h_kv, d = 700, 4, 1, 8
    q, k, v = _rand_qkv(rng, n, n, h_q, h_kv, d)
    qi = rng.standard_normal((n, h_kv, 4))
    ki = rng.standard_normal((n, 4))
    nb = -(-n // 128)
    ids, _, _ = orc.index_topk(qi, ki, 0, nb)
    o_s, l_s = orc.sparse_attention(q, k, v, ids, 0)
    o_d, l_d = orc.dense_attention(q, k, v, 0)
    np.testing.assert_allclose(o_s, o_d, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l_s, l_d, rtol=1e-12)
    # N <= 128: one block, any k gives dense attention
    ids1, _, _ = orc.index_topk(qi[:100], ki[:100], 0, 1)
    o1, _ = orc.sparse_attention(q[:100], k[:100], v[:100], ids1, 0)
    np.testing.assert_allclose(o1, orc.dense_attention(q[:100], k[:100], v[:100], 0)[0], rtol=1e-12)


def test_k_equal_one_is_block_local_attention():
    rng = np.random.default_rng(8)
    n, h_q, h_kv, d = 400, 4, 2, 8
    q, k, v = _rand_qkv(rng, n, n, h_q, h_kv, d)
    qi = rng.standard_normal((n, h_kv, 4))
    ki = rng.standard_normal((n, 4))
    ids, _, _ = orc.index_topk(qi, ki, 0, 1)
    assert (ids[:, :, 0] == (np.arange(n) // 128)[:, None]).all()
    o, _ = orc.sparse_attention(q, k, v, ids, 0)
    blk = np.arange(n) // 128
    mask = (blk[None, :] == blk[:, None]) & (np.arange(n)[None, :] <= np.arange(n)[:, None])
    ref = _sdpa_masked(q, k, v, np.broadcast_to(mask, (h_kv, n, n)).copy())
    np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-12)


def test_uniform_values_and_two_key_closed_form():
    rng = np.random.default_rng(9)
    n, h_q, h_kv, d = 260, 4, 1, 8
    q, k, _ = _rand_qkv(rng, n, n, h_q, h_kv, d)
    vrow = rng.standard_normal(d)
    v = np.broadcast_to(vrow, (n, h_kv, d)).copy()
    ids = np.tile(np.array([0, 1, 2, -1]), (n, h_kv, 1))
    o, _ = orc.sparse_attention(q, k, v, ids, 0)
    np.testing.assert_allclose(o, np.broadcast_to(vrow, o.shape), rtol=1e-13)
    # two visible keys with scores 0 and ln 3 -> weights 1/4 and 3/4
    d = 4
    q2 = np.zeros((2, 1, d))
    q2[1, 0, 0] = 2.0
    k2 = np.zeros((2, 1, d))
    k2[1, 0, 0] = math.log(3.0)            # (2 * ln3) / sqrt(4) = ln 3
    v2 = np.array([[[1.0, 0, 0, 0]], [[0, 1.0, 0, 0]]])
    o2, lse2 = orc.sparse_attention(q2, k2, v2, np.array([[[0]], [[0]]]), 0)
    np.testing.assert_allclose(o2[1, 0], [0.25, 0.75, 0, 0], rtol=1e-14)
    assert lse2[1, 0] == pytest.approx(math.log(4.0))
    np.testing.assert_allclose(o2[0, 0], v2[0, 0])


def test_lse_merge_of_per_block_results_equals_whole():
    rng = np.random.default_rng(10)
    n, h_q, h_kv, d = 800, 8, 2, 16
    q, k, v = _rand_qkv(rng, n, n, h_q, h_kv, d)
    i = 777
    ids = np.array([[[0, 2, 5, 6], [1, 3, 4, 6]]])
    o, lse = orc.sparse_attention(q[i:i + 1], k, v, ids, i)
    parts = []
    for j in range(4):
        one = ids[:, :, j:j + 1]
        parts.append(orc.sparse_attention(q[i:i + 1], k, v, one, i))
    lses = np.stack([pl for _, pl in parts])            # [4, 1, h_q]
    outs = np.stack([po for po, _ in parts])            # [4, 1, h_q, d]
    top = lses.max(axis=0)
    w = np.exp(lses - top)
    merged = (w[..., None] * outs).sum(axis=0) / w.sum(axis=0)[..., None]
    np.testing.assert_allclose(merged, o, rtol=1e-12)
    np.testing.assert_allclose(top + np.log(w.sum(axis=0)), lse, rtol=1e-12)


# ------------------------------------------------------------ paged caches

def test_paged_oracles_equal_contiguous():
    rng = np.random.default_rng(12)
    h_q, h_kv, d, di, k = 8, 2, 16, 8, 4
    lens = [700, 129, 1024]
    max_pages = 8
    n_pages = len(lens) * max_pages
    pt = rng.permutation(n_pages).reshape(len(lens), max_pages)
    kp = rng.standard_normal((n_pages, h_kv, 128, d))
    vp = rng.standard_normal((n_pages, h_kv, 128, d))
    ip = rng.standard_normal((n_pages, 128, di))
    q = rng.standard_normal((len(lens), h_q, d))
    qi = rng.standard_normal((len(lens), h_kv, di))
    ids, _, _ = orc.index_topk_decode(qi, ip, pt, lens, k)
    o, lse = orc.sparse_decode(q, kp, vp, pt, lens, ids)
    for s, L in enumerate(lens):
        # contiguous copies built here by scattering page rows token by token
        kc = np.empty((L, h_kv, d))
        vc = np.empty((L, h_kv, d))
        ic = np.empty((L, di))
        for j in range(L):
            page, row = pt[s, j // 128], j % 128
            kc[j] = kp[page, :, row, :]
            vc[j] = vp[page, :, row, :]
            ic[j] = ip[page, row, :]
        ids_c, _, _ = orc.index_topk(qi[s:s + 1], ic, L - 1, k)
        assert (ids_c[0] == ids[s]).all()
        o_c, l_c = orc.sparse_attention(q[s:s + 1], kc, vc, ids_c, L - 1)
        np.testing.assert_allclose(o[s], o_c[0], rtol=1e-13)
        np.testing.assert_allclose(lse[s], l_c[0], rtol=1e-13)


# ------------------------------------------------------------------ e4m3 decoder

def test_e4m3_decoder_closed_forms():
    # values fixed by the format's definition (sign, 4-bit exponent bias 7,
    # 3-bit mantissa, subnormals at exponent 0, S.1111.111 = NaN)
    cases = {0x00: 0.0, 0x38: 1.0, 0xB8: -1.0, 0x3C: 1.5, 0x40: 2.0, 0x7E: 448.0, 0xFE: -448.0,
             0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x0F: 1.875 * 2.0 ** -6, 0x77: 240.0}
    got = orc.decode_e4m3(np.array(list(cases), dtype=np.uint8))
    assert np.array_equal(got, np.array(list(cases.values())))
    nan = orc.decode_e4m3(np.array([0x7F, 0xFF], dtype=np.uint8))
    assert np.all(np.isnan(nan))
    assert np.signbit(orc.decode_e4m3(np.array([0x80], dtype=np.uint8)))[0]


def test_e4m3_decoder_is_monotone_and_symmetric():
    pos = orc.decode_e4m3(np.arange(0, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    neg = orc.decode_e4m3(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -pos)


def test_e4m3_decoder_matches_torch_float8_e4m3fn():
    # an independent implementation of the same format
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.decode_e4m3(codes.numpy())
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))


# ------------------------------------------------------- MXFP8 (E8M0 scales)

def test_e8m0_decoder_closed_forms_and_torch():
    # the scale format's definition: 2^(code - 127), 0xFF = NaN, no sign
    cases = {127: 1.0, 128: 2.0, 126: 0.5, 0: 2.0 ** -127, 1: 2.0 ** -126, 254: 2.0 ** 127, 137: 1024.0}
    got = orc.decode_e8m0(np.array(list(cases), dtype=np.uint8))
    assert np.array_equal(got, np.array(list(cases.values())))
    assert np.isnan(orc.decode_e8m0(np.array([255], dtype=np.uint8)))[0]
    # an independent implementation of the same format, every code
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = orc.decode_e8m0(codes.numpy())
    assert np.all((np.isnan(ref) & np.isnan(got)) | (ref == got))


def test_mxfp8_decoder_unit_scale_and_block_mapping():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, size=(3, 2, 128), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38  # no NaN codes
    unit = np.full((3, 2, 4), 127, dtype=np.uint8)
    # unit scales reduce to the element format
    assert np.array_equal(orc.decode_mxfp8(codes, unit), orc.decode_e4m3(codes))
    # one scale byte moves exactly its own 32 elements, by its power of two
    base = orc.decode_mxfp8(codes, unit)
    for (i, j, q, de) in ((0, 0, 0, 1), (2, 1, 3, -3), (1, 0, 2, 10)):
        sc = unit.copy()
        sc[i, j, q] = 127 + de
        got = orc.decode_mxfp8(codes, sc)
        want = base.copy()
        want[i, j, 32 * q:32 * q + 32] *= 2.0 ** de
        assert np.array_equal(got, want)
    # closed forms: 1.0 at scale 2^3, 448 at 2^10, -2^-9 at 2^-5
    c = np.zeros((1, 96), dtype=np.uint8)
    c[0, 5], c[0, 40], c[0, 70] = 0x38, 0x7E, 0x81
    v = orc.decode_mxfp8(c, np.array([[130, 137, 122]], dtype=np.uint8))
    assert v[0, 5] == 8.0 and v[0, 40] == 448.0 * 1024 and v[0, 70] == -(2.0 ** -14)


def test_mx_encoder_round_trip_through_the_oracle_decoder():
    # values an MXFP8 block holds exactly (E4M3 values whose block maximum
    # lies in [256, 448], times a power of two per block) come back exactly;
    # arbitrary values come back within half an E4M3 step of their block
    from synth.inputs import mx_encode
    g = torch.Generator().manual_seed(3)
    e4 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32)
    e4 = e4[torch.isfinite(e4)]
    x = e4[torch.randint(0, e4.numel(), (6, 4, 32), generator=g)]
    x[..., 0] = 256.0 + 32.0 * torch.randint(0, 6, (6, 4), generator=g).float()  # block max in [256, 416]
    x = x * torch.exp2(torch.randint(-20, 20, (6, 4, 1), generator=g).float())
    codes, scales = mx_encode(x.reshape(6, 128))
    back = orc.decode_mxfp8(codes.view(torch.uint8).numpy(), scales.numpy())
    assert np.array_equal(back, x.reshape(6, 128).double().numpy())
    y = torch.randn(64, 256, generator=g) * torch.exp2(torch.randint(-8, 8, (64, 8), generator=g).float()).repeat_interleave(32, 1)
    codes, scales = mx_encode(y)
    back = orc.decode_mxfp8(codes.view(torch.uint8).numpy(), scales.numpy())
    yd = y.double().numpy()
    X = np.repeat(orc.decode_e8m0(scales.numpy()), 32, axis=1)
    # the block maximum scales into [256, 512): elements past the largest E4M3
    # value, 448, saturate to it; the others keep 3 mantissa bits (relative
    # error <= 2^-4), down to the subnormal step 2^-9 (absolute error <= 2^-10)
    assert np.all((np.abs(yd).reshape(64, 8, 32).max(-1) / X[:, ::32] >= 256.0))
    sat = np.abs(yd) > 448.0 * X
    assert np.array_equal(back[sat], np.sign(yd[sat]) * 448.0 * X[sat])
    err = np.abs(back - yd)[~sat]
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(yd[~sat]), 2.0 ** -10 * X[~sat]))
    assert scales.dtype == torch.uint8 and codes.dtype == torch.float8_e4m3fn


# ------------------------------------------------- mean-pool ablation ([P5])

def test_mean_pool_equals_score_of_mean_key():
    # linearity: the mean of q.k_j over a block's visible keys is q . (mean of
    # those keys), computed here without forming any token score
    rng = np.random.default_rng(11)
    d, h_kv, n_kv = 32, 3, 700
    q = rng.standard_normal((h_kv, d))
    k = rng.standard_normal((n_kv, d))
    for p in (0, 5, 127, 128, 300, 699):
        m = orc.block_mean_pool(orc.index_token_scores(q, k, p), p)
        for b in range(p // 128 + 1):
            lo, hi = 128 * b, min(128 * b + 128, p + 1)
            kbar = k[lo:hi].mean(axis=0)
            np.testing.assert_allclose(m[:, b], q @ kbar / math.sqrt(d), rtol=1e-12, atol=1e-13)


def test_mean_pool_brute_force_and_constant_block():
    rng = np.random.default_rng(12)
    s = rng.standard_normal((2, 400))
    p = 399
    m = orc.block_mean_pool(s, p)
    for r in range(2):
        for b in range(p // 128 + 1):
            vals = [s[r, j] for j in range(128 * b, min(128 * b + 128, p + 1))]
            tot = 0.0
            for v in vals:
                tot += v
            assert m[r, b] == pytest.approx(tot / len(vals), rel=1e-13)
    # a block whose visible scores are all equal has mean = max = that score
    c = np.full((1, 300), 0.75)
    np.testing.assert_array_equal(orc.block_mean_pool(c, 299), orc.block_max_pool(c, 299))


def test_mean_and_max_pool_select_differently_by_construction():
    # block 1: one spike of 5 and 127 keys at -1 (max 5, mean (5-127)/128);
    # block 2: every key at 0.5 (max 0.5, mean 0.5); block 0 and 3: -2.
    # With one free slot (k = 2 with the diagonal block 3 forced) max-pool
    # takes block 1 and mean-pool takes block 2.
    d = 4
    k = np.zeros((4 * 128, d))
    k[:, 0] = -2.0
    k[128:256, 0] = -1.0
    k[128 + 17, 0] = 5.0
    k[256:384, 0] = 0.5
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = math.sqrt(d)  # makes S_j = k_j[0]
    p = 4 * 128 - 1
    ids_max, sc_max, _ = orc.index_topk(q, k, p, 2)
    ids_mean, sc_mean, _ = orc.index_topk(q, k, p, 2, pool="mean")
    assert ids_max[0, 0].tolist() == [1, 3]
    assert ids_mean[0, 0].tolist() == [2, 3]
    assert sc_max[0, 0, 0] == pytest.approx(5.0, rel=1e-14)
    assert sc_mean[0, 0, 0] == pytest.approx(0.5, rel=1e-14)
    # the diagonal block's mean uses only the keys j <= p
    _, _, pooled = orc.index_topk(q, k, 3 * 128 + 9, 2, pool="mean")
    assert pooled[0][0, 3] == pytest.approx(-2.0, rel=1e-14)


def test_mean_pool_rejects_unknown_mode():
    with pytest.raises(ValueError):
        orc.index_topk(np.zeros((1, 1, 4)), np.zeros((10, 4)), 9, 2, pool="median")


# ---------------------------------------------- training path ([P1] §4.5)

def _rand_training_case(seed, n=300, h_q=4, h_kv=2, d_h=16, d_idx=8, top_k=2):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, h_q, d_h))
    k = rng.standard_normal((n, h_kv, d_h))
    v = rng.standard_normal((n, h_kv, d_h))
    do = rng.standard_normal((n, h_q, d_h))
    q_idx = rng.standard_normal((n, h_kv, d_idx))
    k_idx = rng.standard_normal((n, d_idx))
    ids, _, _ = orc.index_topk(q_idx, k_idx, 0, top_k)
    return q, k, v, do, q_idx, k_idx, ids


def _visible_mask(ids, n, h_q, h_kv, q_start=0, n_kv=None):
    n_kv = n if n_kv is None else n_kv
    g = h_q // h_kv
    m = np.zeros((n, h_q, n_kv), dtype=bool)
    for i in range(n):
        p = q_start + i
        for r in range(h_kv):
            for b in ids[i, r]:
                if b >= 0:
                    lo, hi = 128 * b, min(128 * b + 128, p + 1)
                    m[i, r * g:(r + 1) * g, lo:hi] = True
    return m


def test_backward_matches_torch_autograd_of_masked_attention():
    # autograd differentiates the masked softmax attention; the oracle's
    # gradient formulas are hand-derived
    q, k, v, do, _, _, ids = _rand_training_case(20)
    n, h_q, d = q.shape
    h_kv = k.shape[1]
    g = h_q // h_kv
    mask = torch.from_numpy(_visible_mask(ids, n, h_q, h_kv))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    ke = tk.repeat_interleave(g, dim=1)
    ve = tv.repeat_interleave(g, dim=1)
    s = torch.einsum("ihd,jhd->ihj", tq, ke) / math.sqrt(d)
    s = s.masked_fill(~mask, float("-inf"))
    o = torch.einsum("ihj,jhd->ihd", torch.softmax(s, dim=-1), ve)
    (o * torch.from_numpy(do)).sum().backward()
    dq, dk, dv = orc.sparse_attention_backward(q, k, v, ids, 0, do)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-9, atol=1e-11)


def test_backward_full_coverage_equals_sdpa_backward():
    # k covering every block: the gradient of dense causal attention (torch SDPA)
    rng = np.random.default_rng(21)
    n, h_q, h_kv, d = 260, 4, 1, 16
    q = rng.standard_normal((n, h_q, d))
    k = rng.standard_normal((n, h_kv, d))
    v = rng.standard_normal((n, h_kv, d))
    do = rng.standard_normal((n, h_q, d))
    ids, _, _ = orc.index_topk(rng.standard_normal((n, h_kv, 8)), rng.standard_normal((n, 8)), 0, 4)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq.transpose(0, 1), tk.expand(n, h_q, d).transpose(0, 1), tv.expand(n, h_q, d).transpose(0, 1),
        is_causal=True)
    (o.transpose(0, 1) * torch.from_numpy(do)).sum().backward()
    dq, dk, dv = orc.sparse_attention_backward(q, k, v, ids, 0, do)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-9, atol=1e-11)


def test_backward_finite_differences():
    q, k, v, do, _, _, ids = _rand_training_case(22, n=200)

    def loss(q_, k_, v_):
        o, _ = orc.sparse_attention(q_, k_, v_, ids, 0)
        return float(np.sum(o * do))

    dq, dk, dv = orc.sparse_attention_backward(q, k, v, ids, 0, do)
    rng = np.random.default_rng(0)
    eps = 1e-6
    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        for _ in range(5):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            plus, minus = [x.copy() for x in (q, k, v)], [x.copy() for x in (q, k, v)]
            plus[which][idx] += eps
            minus[which][idx] -= eps
            fd = (loss(*plus) - loss(*minus)) / (2 * eps)
            assert fd == pytest.approx(grad[idx], rel=1e-5, abs=1e-7), (which, idx)


def _torch_kl(q_idx, k_idx, q, k, ids, kl_scale):
    n, h_kv, d_idx = q_idx.shape
    h_q, d = q.shape[1], q.shape[2]
    g = h_q // h_kv
    mask = torch.from_numpy(_visible_mask(ids, n, h_q, h_kv))
    with torch.no_grad():
        s = torch.einsum("ihd,jhd->ihj", torch.from_numpy(q), torch.from_numpy(k).repeat_interleave(g, dim=1))
        s = (s / math.sqrt(d)).masked_fill(~mask, float("-inf"))
        p_main = torch.softmax(s, dim=-1).view(n, h_kv, g, n).mean(dim=2)   # [n, h_kv, n]
    tqi = torch.tensor(q_idx, requires_grad=True)
    tki = torch.tensor(k_idx, requires_grad=True)
    si = torch.einsum("ird,jd->irj", tqi, tki) / math.sqrt(d_idx)
    gmask = mask.view(n, h_kv, g, n)[:, :, 0]
    log_p_idx = torch.log_softmax(si.masked_fill(~gmask, float("-inf")), dim=-1)
    # library KL per row: sum p_main (log p_main - log p_idx) over visible keys
    kl_rows = torch.nn.functional.kl_div(log_p_idx.masked_fill(~gmask, 0.0), p_main, reduction="none").sum(-1)
    (kl_scale * kl_rows.sum()).backward()
    return kl_rows.detach().numpy(), tqi.grad.numpy(), tki.grad.numpy()


def test_kl_alignment_matches_torch_kl_div_and_autograd():
    q, k, _, _, q_idx, k_idx, ids = _rand_training_case(23)
    kl, dqi, dki = orc.kl_alignment(q_idx, k_idx, q, k, ids, 0, kl_scale=0.37)
    t_kl, t_dqi, t_dki = _torch_kl(q_idx, k_idx, q, k, ids, 0.37)
    np.testing.assert_allclose(kl, t_kl, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dqi, t_dqi, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dki, t_dki, rtol=1e-9, atol=1e-12)
    assert np.all(kl >= -1e-15)


def test_kl_alignment_zero_when_index_branch_equals_main_branch():
    # one head per group, q_idx = q, k_idx = k, equal scales: the two
    # distributions coincide, so the loss and its gradients vanish
    rng = np.random.default_rng(24)
    n, d = 300, 16
    q = rng.standard_normal((n, 1, d))
    k = rng.standard_normal((n, 1, d))
    ids, _, _ = orc.index_topk(rng.standard_normal((n, 1, 8)), rng.standard_normal((n, 8)), 0, 2)
    kl, dqi, dki = orc.kl_alignment(q, k[:, 0], q, k, ids, 0)
    assert np.max(np.abs(kl)) < 1e-13
    assert np.max(np.abs(dqi)) < 1e-12 and np.max(np.abs(dki)) < 1e-12
    # scaling the loss weight scales the gradients only
    q2, k2, _, _, qi2, ki2, ids2 = _rand_training_case(25)
    a = orc.kl_alignment(qi2, ki2, q2, k2, ids2, 0, kl_scale=1.0)
    b = orc.kl_alignment(qi2, ki2, q2, k2, ids2, 0, kl_scale=2.5)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_allclose(b[1], 2.5 * a[1], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(b[2], 2.5 * a[2], rtol=1e-12, atol=1e-15)


# ------------------------------------- index projections and RoPE ([P1] §3.1, §4.2)

def test_rope_closed_form_angles():
    # a unit vector on dim i turns into (cos a, sin a) on dims (i, i + 32) with
    # a = p * 10000^(-2i/64)
    d = 64
    for i, p in ((0, 1), (0, 5), (16, 1), (31, 1000), (7, 123456)):
        v = np.zeros((1, d))
        v[0, i] = 1.0
        out = orc.rope(v, [p], 64)
        a = p * 10000.0 ** (-2.0 * i / 64)
        expect = np.zeros(d)
        expect[i] = math.cos(a)
        expect[i + 32] = math.sin(a)
        np.testing.assert_allclose(out[0], expect, atol=1e-12)
    # position 0 is the identity; dims past rope_dim are untouched
    rng = np.random.default_rng(30)
    v = rng.standard_normal((3, 128))
    np.testing.assert_array_equal(orc.rope(v, [0, 0, 0], 64), v)
    np.testing.assert_array_equal(orc.rope(v, [5, 9, 77], 64)[:, 64:], v[:, 64:])


def test_rope_is_a_rotation_with_relative_positions():
    rng = np.random.default_rng(31)
    q = rng.standard_normal((1, 64))
    k = rng.standard_normal((1, 64))
    np.testing.assert_allclose(np.linalg.norm(orc.rope(q, [987654], 64)), np.linalg.norm(q), rtol=1e-12)
    # the score of a rotated pair depends only on the position difference
    for p1, p2, sft in ((10, 3, 100), (5000, 4990, 1 << 20), (0, 0, 77)):
        a = orc.rope(q, [p1], 64) @ orc.rope(k, [p2], 64).T
        b = orc.rope(q, [p1 + sft], 64) @ orc.rope(k, [p2 + sft], 64).T
        assert a[0, 0] == pytest.approx(b[0, 0], rel=1e-9, abs=1e-9)


def test_index_projection_groups_and_shared_key():
    rng = np.random.default_rng(32)
    n, dm, h_kv, di = 5, 48, 3, 32
    x = rng.standard_normal((n, dm))
    wq = rng.standard_normal((h_kv, di, dm))
    wk = rng.standard_normal((di, dm))
    pos = np.array([0, 1, 2, 300, 70000])
    q, k = orc.index_projection(x, wq, wk, pos, rope_dim=0)
    for r in range(h_kv):
        np.testing.assert_allclose(q[:, r], x @ wq[r].T, rtol=1e-12)
    np.testing.assert_allclose(k, x @ wk.T, rtol=1e-12)
    # group r's query depends on W_q[r] only
    wq2 = wq.copy()
    wq2[1] += 1.0
    q2, _ = orc.index_projection(x, wq2, wk, pos, rope_dim=32)
    q1, _ = orc.index_projection(x, wq, wk, pos, rope_dim=32)
    np.testing.assert_array_equal(q2[:, 0], q1[:, 0])
    np.testing.assert_array_equal(q2[:, 2], q1[:, 2])
    assert not np.allclose(q2[:, 1], q1[:, 1])


def test_training_oracle_rows_subset_is_the_restriction():
    # taking a subset of queries equals the full computation for their rows,
    # and for a block that only those queries selected
    q, k, v, do, q_idx, k_idx, ids = _rand_training_case(26)
    rows = [5, 131, 200, 299]
    dq_a, dk_a, dv_a = orc.sparse_attention_backward(q, k, v, ids, 0, do)
    dq_s, dk_s, dv_s = orc.sparse_attention_backward(q, k, v, ids, 0, do, rows=rows)
    np.testing.assert_allclose(dq_s[rows], dq_a[rows], rtol=1e-12)
    assert not dq_s[[0, 1, 2]].any()
    sub = np.zeros_like(ids) - 1
    sub[rows] = ids[rows]
    dq_b, dk_b, dv_b = orc.sparse_attention_backward(q, k, v, sub, 0, do)
    np.testing.assert_allclose(dk_s, dk_b, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dv_s, dv_b, rtol=1e-12, atol=1e-14)
    kl_a, dqi_a, _ = orc.kl_alignment(q_idx, k_idx, q, k, ids, 0)
    kl_s, dqi_s, dki_s = orc.kl_alignment(q_idx, k_idx, q, k, ids, 0, rows=rows)
    np.testing.assert_allclose(kl_s[rows], kl_a[rows], rtol=1e-12)
    np.testing.assert_allclose(dqi_s[rows], dqi_a[rows], rtol=1e-12)
    _, _, dki_b = orc.kl_alignment(q_idx, k_idx, q, k, sub, 0)
    np.testing.assert_allclose(dki_s, dki_b, rtol=1e-12, atol=1e-14)

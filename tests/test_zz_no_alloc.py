"""msa_index_topk_decode_static (the decode index call with the library's own
scratch, for callers that cannot allocate) against msa_index_topk with a
caller workspace: identical block lists and scores, on consecutive calls of
decreasing size (the scratch keeps the earlier call's contents)."""
import pytest
import torch

from synth import MODEL_SHAPE, gen_decode_paged
from synth.inputs import HeadShape

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_attention_branch_amd import msa
    msa.lib()
    return msa


def _case(msa, shape, seq_lens, seed, **kw):
    inp = gen_decode_paged(len(seq_lens), max(seq_lens), shape, seed=seed, device=DEV, seq_lens=seq_lens)
    q_idx = inp["q_idx"][0].contiguous()
    print("[case] decode static", shape, len(seq_lens), max(seq_lens), seed, kw, flush=True)
    ref, ref_sc = msa.index_topk(q_idx, inp["k_idx_pages"], top_k=shape.top_k, page_table=inp["page_table"],
                                 seq_lens=inp["seq_lens"], with_scores=True, **kw)
    got, got_sc = msa.index_topk_decode_static(q_idx, inp["k_idx_pages"], inp["page_table"], inp["seq_lens"],
                                               top_k=shape.top_k, with_scores=True, **kw)
    got2 = msa.index_topk_decode_static(q_idx, inp["k_idx_pages"], inp["page_table"], inp["seq_lens"],
                                        top_k=shape.top_k, **kw)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert torch.equal(got2, ref)
    assert torch.equal(got_sc, ref_sc)
    return ref


def test_decode_static_matches_workspace_call_on_shrinking_inputs():
    msa = _msa()
    # a large call, then a smaller one (fewer sequences, fewer pages): every
    # score the second call reads must be its own, not the first call's
    big = _case(msa, MODEL_SHAPE, [131072, 70000, 129, 5000, 98304, 1, 128, 131071], 90)
    small = _case(msa, MODEL_SHAPE, [3000, 2049, 640], 91)
    assert big.shape[0] == 8 and small.shape[0] == 3
    # no forced block, then a smaller call with the forced block and other head shapes
    _case(msa, MODEL_SHAPE, [40000, 7000, 300], 92, force_local=False)
    _case(msa, HeadShape(16, 2, 64, 32, 8), [900, 1200], 93)


def test_decode_static_at_the_scratch_limit():
    msa = _msa()
    # 64 sequences x 4 groups x 16384 pages = 2^22 page scores, the whole scratch
    shape = MODEL_SHAPE
    lens = [16384 * 128 if s % 16 == 0 else 3000 + 97 * s for s in range(4)]
    inp = gen_decode_paged(4, max(lens), shape, seed=94, device=DEV, seq_lens=lens)
    pt = torch.zeros((64, 16384), dtype=torch.int32, device=DEV)
    pt[:4, :inp["page_table"].shape[1]] = inp["page_table"]
    sl = torch.ones(64, dtype=torch.int32, device=DEV)
    sl[:4] = inp["seq_lens"]
    q_idx = torch.zeros((64, shape.h_kv, shape.d_idx), dtype=torch.bfloat16, device=DEV)
    q_idx[:4] = inp["q_idx"][0]
    print("[case] decode static at the limit", flush=True)
    ref = msa.index_topk(q_idx, inp["k_idx_pages"], top_k=16, page_table=pt, seq_lens=sl)
    got = msa.index_topk_decode_static(q_idx, inp["k_idx_pages"], pt, sl, top_k=16)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    with pytest.raises(msa.MsaError, match="scratch"):
        msa.index_topk_decode_static(torch.zeros((65, shape.h_kv, shape.d_idx), dtype=torch.bfloat16, device=DEV),
                                     inp["k_idx_pages"], torch.zeros((65, 16384), dtype=torch.int32, device=DEV),
                                     torch.ones(65, dtype=torch.int32, device=DEV), top_k=16)

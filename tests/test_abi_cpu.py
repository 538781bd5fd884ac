"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before launching
anything (outputs untouched)."""
import ctypes
import os
import re

import pytest

from block_sparse_attention_branch_amd import msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "msa.h")).read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(msa_\w+)\s*\(", src, flags=re.M)))


def test_header_symbols_exported():
    names = _declared()
    assert set(names) == set(msa.EXPORTS), names
    L = msa.lib()
    for n in names:
        assert hasattr(L, n), n
    assert L.msa_abi_version() == 6
    for st in range(5):
        assert L.msa_status_string(st).decode().startswith("MSA_")


def _shape(**kw):
    base = dict(h_q=64, h_kv=4, d_h=128, d_idx=64, top_k=16, dtype_code=0)
    base.update(kw)
    return msa.make_shape(base["h_q"], base["h_kv"], base["d_h"], base["d_idx"], base["top_k"],
                          base["dtype_code"])


FAKE = 1 << 20  # 16-byte aligned non-null "device" address, never dereferenced


def _idx_call(shape, *, batch=1, n_q=8, q_start=0, q_idx=FAKE, k_idx=FAKE, n_kv=64, page_table=None,
              seq_lens=None, max_pages=0, out=FAKE, ws=None, ws_bytes=0):
    kv = msa.KV(None, None, k_idx, page_table, seq_lens, n_kv, max_pages)
    return msa.lib().msa_index_topk(ctypes.byref(shape) if shape is not None else None, batch, n_q, q_start,
                                    q_idx, ctypes.byref(kv), out, None, ws, ws_bytes, None)


def _err():
    return msa.lib().msa_last_error().decode()


@pytest.mark.parametrize("bad,status,msg", [
    (dict(h_kv=3), 1, "multiple"),
    (dict(h_q=96, h_kv=2), 2, "heads per group"),
    (dict(d_idx=48), 2, "d_idx"),
    (dict(top_k=17), 2, "top_k"),
    (dict(top_k=0), 2, "top_k"),
    (dict(dtype_code=7), 1, "dtype"),
])
def test_index_shape_validation(bad, status, msg):
    assert _idx_call(_shape(**bad)) == status
    assert msg in _err()


def test_index_argument_validation():
    s = _shape()
    assert _idx_call(None) == 1 and "shape" in _err()
    assert _idx_call(s, batch=2) == 1 and "batch" in _err()
    assert _idx_call(s, n_q=60, q_start=10, n_kv=64) == 1 and "exceeds" in _err()
    assert _idx_call(s, k_idx=None) == 1 and "k_idx" in _err()
    assert _idx_call(s, q_idx=FAKE + 4) == 1 and "aligned" in _err()
    assert _idx_call(s, out=None) == 1 and "NULL" in _err()
    # decode mode
    assert _idx_call(s, n_q=2, seq_lens=FAKE, page_table=FAKE, max_pages=4) == 1 and "n_q == 1" in _err()
    assert _idx_call(s, n_q=1, seq_lens=FAKE, max_pages=4) == 1 and "page_table" in _err()
    assert _idx_call(s, n_q=1, seq_lens=FAKE, page_table=FAKE, max_pages=20000) == 2
    # workspace: a long prefill needs one
    need = msa.workspace_size(msa.OP_INDEX, s, n_q=20000, n_kv=20000)
    assert need > 0
    assert _idx_call(s, n_q=20000, n_kv=20000) == 3 and "workspace" in _err()
    assert _idx_call(s, n_q=20000, n_kv=20000, ws=FAKE, ws_bytes=need - 1) == 3
    assert _idx_call(s, n_q=20000, n_kv=20000, ws=FAKE + 16, ws_bytes=need) == 3 and "aligned" in _err()
    # empty inputs are a no-op
    assert _idx_call(s, n_q=0) == 0 and _err() == ""


def test_prefill_decode_dense_validation():
    L = msa.lib()
    s = _shape()
    kv = msa.KV(FAKE, FAKE, None, None, None, 256, 0)
    assert L.msa_sparse_prefill(ctypes.byref(s), 300, 0, FAKE, ctypes.byref(kv), FAKE, FAKE, None, None, 0, None) == 1
    assert "exceeds" in _err()
    assert L.msa_sparse_prefill(ctypes.byref(_shape(d_h=96)), 8, 0, FAKE, ctypes.byref(kv), FAKE, FAKE, None,
                                None, 0, None) == 2
    assert L.msa_sparse_prefill(ctypes.byref(s), 8, 0, FAKE, ctypes.byref(kv), None, FAKE, None, None, 0, None) == 1
    need = msa.workspace_size(msa.OP_PREFILL, s, n_q=8, n_kv=256)
    assert need > 0
    assert L.msa_sparse_prefill(ctypes.byref(s), 8, 0, FAKE, ctypes.byref(kv), FAKE, FAKE, None, None, 0, None) == 3
    # decode needs paging, and is bf16-only
    assert L.msa_sparse_decode(ctypes.byref(s), 2, FAKE, ctypes.byref(kv), FAKE, FAKE, None, None, 0, None) == 1
    kvp = msa.KV(FAKE, FAKE, None, FAKE, FAKE, 0, 8)
    assert L.msa_sparse_decode(ctypes.byref(_shape(dtype_code=1)), 2, FAKE, ctypes.byref(kvp), FAKE, FAKE, None,
                               None, 0, None) == 2
    assert L.msa_sparse_decode(ctypes.byref(s), 0, FAKE, ctypes.byref(kvp), FAKE, FAKE, None, None, 0, None) == 0
    # dense takes a contiguous cache only
    assert L.msa_dense_prefill(ctypes.byref(s), 8, 0, FAKE, ctypes.byref(kvp), FAKE, None, None, 0, None) == 2
    assert L.msa_dense_prefill(ctypes.byref(s), 8, 250, FAKE, ctypes.byref(kv), FAKE, None, None, 0, None) == 1


def test_workspace_size_queries():
    s = _shape()
    assert msa.workspace_size(msa.OP_INDEX, s, n_q=1000, n_kv=1000) >= 0
    p = msa.workspace_size(msa.OP_PREFILL, s, n_q=32768, n_kv=32768)
    assert p > 0
    assert msa.workspace_size(msa.OP_INDEX_DECODE, s, batch=64, n_q=1, max_pages=1024) == 64 * 4 * 1024 * 4
    assert msa.workspace_size(msa.OP_DENSE, s, n_q=100, n_kv=100) == 0
    with pytest.raises(msa.MsaError):
        msa.workspace_size(9, s)


def test_prefill_workspace_holds_the_merge_span():
    """Partial buffers of the sparse prefill (model shape, bf16: 270336 bytes
    per query token): a window whose partials fit the 256 MiB merge-alone
    bound gets one buffer; past it the buffers of up to 12288 tokens of
    windows are kept for one merge launch."""
    s = _shape()
    per_token = 4 * 16 * 16 * (128 * 2 + 8)
    # 32K: window 704 tokens (40 per (group, block) cell), 190 MB: alone
    p32 = msa.workspace_size(msa.OP_PREFILL, s, n_q=32768, n_kv=32768)
    assert 704 * per_token <= p32 < 2 * 704 * per_token
    # 16384 queries at 64K: window 1408 tokens (380 MB), 8 windows per merge
    p64 = msa.workspace_size(msa.OP_PREFILL, s, n_q=16384, q_start=49152, n_kv=65536)
    assert 8 * 1408 * per_token <= p64 < 9 * 1408 * per_token
    # 128K: window 2752 tokens, 4 windows per merge
    p128 = msa.workspace_size(msa.OP_PREFILL, s, n_q=131072, n_kv=131072)
    assert 4 * 2752 * per_token <= p128 < 5 * 2752 * per_token


def test_profile_api_host_side():
    msa.profile_enable(True)
    msa.profile_enable(False)
    ms, n = msa.profile_read("kp_kernel")          # nothing recorded: no HIP call needed
    assert ms == 0.0 and n == 0
    with pytest.raises(msa.MsaError) as e:
        msa.profile_read("no_such_kernel")
    assert e.value.status == 1


def test_e4m3_cache_validation():
    """e4m3 caches are accepted with bf16 compute by every call but the dense one."""
    L = msa.lib()
    f8 = msa.make_shape(64, 4, 128, 64, 16, msa.MSA_BF16, cache_dtype=msa.MSA_FP8_E4M3)
    f8_32 = msa.make_shape(64, 4, 128, 64, 16, msa.MSA_FP32, cache_dtype=msa.MSA_FP8_E4M3)
    kv = msa.KV(FAKE, FAKE, None, None, None, 256, 0)
    assert L.msa_dense_prefill(ctypes.byref(f8), 8, 0, FAKE, ctypes.byref(kv), FAKE, None, None, 0, None) == 2
    assert "dense" in _err()
    assert L.msa_sparse_prefill(ctypes.byref(f8_32), 8, 0, FAKE, ctypes.byref(kv), FAKE, FAKE, None, None, 0,
                                None) == 2
    assert "MSA_BF16" in _err()
    assert _idx_call(f8_32) == 2 and "MSA_BF16" in _err()
    # accepted: the call gets as far as the workspace check
    assert _idx_call(f8, n_q=20000, n_kv=20000) == 3
    assert msa.workspace_size(msa.OP_PREFILL, f8, n_q=8, n_kv=256) > 0
    assert msa.lib().msa_workspace_size(msa.OP_DENSE, ctypes.byref(f8), 1, 8, 0, 8, 0) == 0
    assert "dense" in _err()


def test_mxfp8_cache_validation():
    """MXFP8 caches: the calls that take 8-bit caches accept them when the scale
    arrays they read are given, and refuse them without (or elsewhere)."""
    L = msa.lib()
    mx = msa.make_shape(64, 4, 128, 64, 16, msa.MSA_BF16, cache_dtype=msa.MSA_MXFP8_E4M3)
    mx32 = msa.make_shape(64, 4, 128, 64, 16, msa.MSA_FP32, cache_dtype=msa.MSA_MXFP8_E4M3)
    no_sc = msa.KV(FAKE, FAKE, FAKE, None, None, 256, 0)
    only_idx = msa.KV(FAKE, FAKE, FAKE, None, None, 256, 0, None, None, FAKE)
    full = msa.KV(FAKE, FAKE, FAKE, None, None, 256, 0, FAKE, FAKE, FAKE)
    pre = lambda shp, kv: L.msa_sparse_prefill(ctypes.byref(shp), 8, 0, FAKE, ctypes.byref(kv), FAKE, FAKE, None,
                                               None, 0, None)
    assert pre(mx, no_sc) == 1 and "k_scale" in _err()
    assert pre(mx, only_idx) == 1 and "k_scale" in _err()
    assert pre(mx, full) == 3 and "workspace" in _err()  # accepted up to the workspace check
    assert pre(mx32, full) == 2 and "MSA_BF16" in _err()
    idx = lambda shp, kv: L.msa_index_topk(ctypes.byref(shp), 1, 20000, 0, FAKE, ctypes.byref(kv), FAKE, None, None,
                                           0, None)
    kv_i = msa.KV(None, None, FAKE, None, None, 20000, 0)
    assert idx(mx, kv_i) == 1 and "k_idx_scale" in _err()
    kv_i = msa.KV(None, None, FAKE, None, None, 20000, 0, None, None, FAKE)
    assert idx(mx, kv_i) == 3
    dec = lambda kv: L.msa_sparse_decode(ctypes.byref(mx), 2, FAKE, ctypes.byref(kv), FAKE, FAKE, None, None, 0, None)
    assert dec(msa.KV(FAKE, FAKE, None, FAKE, FAKE, 0, 8)) == 1 and "k_scale" in _err()
    assert dec(msa.KV(FAKE, FAKE, None, FAKE, FAKE, 0, 8, FAKE, FAKE, None)) == 3
    st = lambda kv: L.msa_index_topk_decode_static(ctypes.byref(mx), 2, FAKE, ctypes.byref(kv), FAKE, None, None)
    assert st(msa.KV(None, None, FAKE, FAKE, FAKE, 0, 8)) == 1 and "k_idx_scale" in _err()
    # not built for MXFP8: the dense comparison and the backward
    assert L.msa_dense_prefill(ctypes.byref(mx), 8, 0, FAKE, ctypes.byref(full), FAKE, None, None, 0, None) == 2
    assert msa.lib().msa_workspace_size(msa.OP_DENSE, ctypes.byref(mx), 1, 8, 0, 8, 0) == 0
    # the binding picks MXFP8 when a scale tensor comes with e4m3 codes
    import torch
    t = torch.empty(4, dtype=torch.float8_e4m3fn)
    assert msa._cache_code(t, msa.MSA_BF16) == msa.MSA_FP8_E4M3
    assert msa._cache_code(t, msa.MSA_BF16, torch.empty(1, dtype=torch.uint8)) == msa.MSA_MXFP8_E4M3


def test_pool_mode_validation():
    s = msa.make_shape(64, 4, 128, 64, 16, msa.MSA_BF16, pool=7)
    assert _idx_call(s) == 1 and "pool" in _err()
    s = msa.make_shape(64, 4, 128, 64, 16, msa.MSA_BF16, pool="mean")
    assert s.pool == msa.MSA_POOL_MEAN
    assert _idx_call(s, n_q=0) == 0
    # the attention calls ignore the index branch's pool mode
    kv = msa.KV(FAKE, FAKE, None, None, None, 256, 0)
    bad = msa.make_shape(64, 4, 128, 64, 16, msa.MSA_BF16, pool=7)
    assert msa.lib().msa_sparse_prefill(ctypes.byref(bad), 0, 0, FAKE, ctypes.byref(kv), FAKE, FAKE, None, None, 0,
                                        None) == 0


def test_backward_validation():
    L = msa.lib()
    s = _shape()
    kv = msa.KV(FAKE, FAKE, None, None, None, 256, 0)
    args = lambda shp, n_q=8, q_start=0, kv_=kv, dq=FAKE, kl=None: (
        ctypes.byref(shp), n_q, q_start, FAKE, ctypes.byref(kv_), FAKE, FAKE, FAKE, FAKE, dq, FAKE, FAKE, kl, None, 0,
        None)
    assert L.msa_sparse_prefill_backward(*args(_shape(dtype_code=1))) == 2 and "MSA_BF16" in _err()
    assert L.msa_sparse_prefill_backward(*args(_shape(d_h=96))) == 2
    paged = msa.KV(FAKE, FAKE, None, FAKE, None, 256, 2)
    assert L.msa_sparse_prefill_backward(*args(s, kv_=paged)) == 2 and "contiguous" in _err()
    assert L.msa_sparse_prefill_backward(*args(s, n_q=300)) == 1 and "exceeds" in _err()
    assert L.msa_sparse_prefill_backward(*args(s, dq=None)) == 1 and "NULL" in _err()
    assert L.msa_sparse_prefill_backward(*args(s)) == 3 and "workspace" in _err()
    f8 = msa.make_shape(64, 4, 128, 64, 16, msa.MSA_BF16, cache_dtype=msa.MSA_FP8_E4M3)
    assert L.msa_sparse_prefill_backward(*args(f8)) == 2 and "e4m3" in _err()
    need = msa.workspace_size(msa.OP_PREFILL_BACKWARD, s, n_q=8, n_kv=256)
    assert need > msa.workspace_size(msa.OP_PREFILL, s, n_q=8, n_kv=256)
    assert msa.workspace_size(msa.OP_PREFILL_BACKWARD, s, n_q=0, n_kv=256) == 0
    # with the KL-alignment term
    assert msa.workspace_size(msa.OP_PREFILL_BACKWARD_KL, s, n_q=8, n_kv=256) > need
    bad_kl = msa.KL(FAKE, None, 1.0, None, FAKE, FAKE)
    assert L.msa_sparse_prefill_backward(*args(s, kl=ctypes.byref(bad_kl))) == 1 and "kl" in _err()
    good_kl = msa.KL(FAKE, FAKE, 1.0, None, FAKE, FAKE)
    assert L.msa_sparse_prefill_backward(*args(s, kl=ctypes.byref(good_kl))) == 3
    assert L.msa_sparse_prefill_backward(*args(_shape(d_idx=48), kl=ctypes.byref(good_kl))) == 2


def test_index_project_validation():
    L = msa.lib()
    s = msa.make_shape(4, 4, 128, 64, 16, msa.MSA_BF16)
    kv = msa.KV(None, None, FAKE, None, None, 1000, 0)
    call = lambda shp=s, n=8, dm=256, rope=64, base=10000.0, kv_=kv, x=FAKE, ws=None, wsb=0: L.msa_index_project(
        ctypes.byref(shp), n, dm, x, FAKE, FAKE, rope, base, FAKE, None, ctypes.byref(kv_), FAKE, ws, wsb, None)
    assert call(dm=100) == 1 and "d_model" in _err()
    assert call(rope=48) == 2 and "rope_dim" in _err()
    assert call(rope=128) == 1 and "exceeds" in _err()
    assert call(base=1.0) == 1 and "rope_base" in _err()
    assert call(x=None) == 1 and "NULL" in _err()
    assert call(shp=msa.make_shape(4, 4, 128, 64, 16, msa.MSA_FP32)) == 2
    assert call(n=0) == 0 and _err() == ""
    # short calls split d_model and need a workspace (none at d_model 256 with 8 tokens: too short to split)
    need = L.msa_workspace_size(7, ctypes.byref(s), 0, 64, 0, 6144, 0)
    assert need == 24 * 64 * 5 * 64 * 4  # 24 slices of 256 dims, fp32 sums per (token, projection, dim)
    assert L.msa_workspace_size(7, ctypes.byref(s), 0, 8, 0, 256, 0) == 0
    assert L.msa_workspace_size(7, ctypes.byref(s), 0, 4096, 0, 6144, 0) == 0  # long calls: tiled, no split
    assert call(n=64, dm=6144) == 3 and "workspace" in _err()
    assert call(n=64, dm=6144, ws=FAKE, wsb=need - 1) == 3


def test_mfma_probe_validation():
    # argument checks of the measurement probe run on the host, before any launch
    L = msa.lib()
    fp = ctypes.cast(FAKE, ctypes.POINTER(ctypes.c_float))
    assert L.msa_probe_mfma(0, 10, fp, None) == 1 and "n_wg" in _err()
    assert L.msa_probe_mfma(4, 0, fp, None) == 1 and "iters" in _err()
    assert L.msa_probe_mfma(4, 10, None, None) == 1 and "NULL" in _err()


def test_decode_static_argument_validation():
    # the allocation-free decode index call checks everything on the host,
    # its scratch limit included, before it looks at the device
    L = msa.lib()
    s = _shape()

    def call(batch=2, max_pages=1024, seq_lens=FAKE, page_table=FAKE, q_idx=FAKE, out=FAKE, shape=s):
        kv = msa.KV(None, None, FAKE, page_table, seq_lens, 0, max_pages)
        return L.msa_index_topk_decode_static(ctypes.byref(shape), batch, q_idx, ctypes.byref(kv), out, None, None)

    assert call(seq_lens=None) == 1 and "seq_lens" in _err()
    assert call(page_table=None) == 1 and "page_table" in _err()
    assert call(max_pages=0) == 2 and "max_pages" in _err()
    assert call(batch=-1) == 1 and "batch" in _err()
    # 2^22 page scores: 64 sequences x 4 groups x 16384 pages fit, one more sequence does not
    assert call(batch=65, max_pages=16384) == 2 and "scratch" in _err()
    assert call(batch=4097, max_pages=1024) == 2 and "scratch" in _err()
    assert call(batch=0) == 0
    assert call(out=None) == 1 and "NULL" in _err()
    assert call(shape=_shape(d_idx=48)) == 2 and "d_idx" in _err()


def test_bench_refuses_several_gpus():
    # bench.py measures one GPU; a request for more exits with status 2 and says why
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_bench_summarizes_traffic_without_gpu(tmp_path, monkeypatch):
    # The counter summary is host logic: per-dispatch FETCH_SIZE / WRITE_SIZE
    # rows of rocprofv3 CSVs (several rows of one dispatch add up), scaled by
    # the ratio of the calibration copy's known bytes to what the same counter
    # read for it, divided by the calls in the run.  Checked on made-up CSVs.
    import csv
    import importlib.util
    import json
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tmp_path / "traffic.json"))

    def write(path, counter, rows):
        with open(path, "w", newline="") as fh:
            w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writeheader()
            for did, name, val in rows:
                w.writerow({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": val})

    copy_kib = bench.COPY_BYTES / 1024.0
    # the copy reads half its bytes on FETCH_SIZE (factor 2) and all of them on WRITE_SIZE (factor 1),
    # each dispatch reported as two rows
    write(tmp_path / "cf.csv", "FETCH_SIZE", [(1, "copyBuffer", copy_kib / 4), (1, "copyBuffer", copy_kib / 4)])
    write(tmp_path / "cw.csv", "WRITE_SIZE", [(1, "copyBuffer", copy_kib / 2), (1, "copyBuffer", copy_kib / 2)])
    # a one-leg workload: two sparse-decode calls, kd_kernel 100 KiB fetched / 4 written, kd_merge_kernel 10 / 1
    fetch = [(10, "msa::kd_kernel<128>", 100), (11, "msa::kd_merge_kernel<128>", 10),
             (12, "msa::kd_kernel<128>", 100), (13, "msa::kd_merge_kernel<128>", 10)]
    wr = [(10, "msa::kd_kernel<128>", 4), (11, "msa::kd_merge_kernel<128>", 1),
          (12, "msa::kd_kernel<128>", 4), (13, "msa::kd_merge_kernel<128>", 1)]
    write(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    write(tmp_path / "w.csv", "WRITE_SIZE", wr)
    bench.summarize_traffic("decode_fp8", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                            str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"))
    t = json.load(open(tmp_path / "traffic.json"))
    assert t["source_hash"] == bench.source_hash()
    call = t["workloads"]["decode_fp8"]["sparse_decode"]
    assert call["fetch_bytes"] == round(110 * 1024 * 2.0) and call["write_bytes"] == round(5 * 1024 * 1.0)
    kd = t["kernels"]["decode_fp8"]["kd_kernel"]  # per launch, the merge kernel excluded
    assert kd["fetch_bytes_per_launch"] == 100 * 1024 * 2 and kd["write_bytes_per_launch"] == 4 * 1024
    assert "index_prefill" not in t["workloads"]["decode_fp8"]  # no dispatch of that call in the run

    # the default step: its legs are told apart by launch order (prefill 128K, prefill 1M, the
    # 64 x 128K decode step, then 1M decode steps); a cache-append kernel belongs to no call
    def step(did0, kp128, kp1m, kd1m):
        return [(did0, "ki_prefill_kernel", 7), (did0 + 1, "ks_count_lds_kernel", 1),
                (did0 + 2, "kp_kernel", kp128), (did0 + 3, "km_kernel", 3), (did0 + 4, "kp_kernel", kp128),
                (did0 + 5, "km_kernel", 3), (did0 + 6, "ki_prefill_kernel", 9), (did0 + 7, "ks_count_lds_kernel", 2),
                (did0 + 8, "kp_kernel", kp1m), (did0 + 9, "km_kernel", 5), (did0 + 10, "ki_decode_scan_kernel", 50),
                (did0 + 11, "kd_kernel", 20), (did0 + 12, "index_put_kernel", 99),
                (did0 + 13, "ki_decode_scan_kernel", 30), (did0 + 14, "kd_kernel", kd1m),
                (did0 + 15, "index_put_kernel", 99), (did0 + 16, "ki_decode_scan_kernel", 30),
                (did0 + 17, "kd_kernel", kd1m)]
    fetch = step(100, 40, 60, 2) + step(200, 40, 60, 2)
    wr = [(d, n, 1) for d, n, _ in fetch]
    write(tmp_path / "f2.csv", "FETCH_SIZE", fetch)
    write(tmp_path / "w2.csv", "WRITE_SIZE", wr)
    assert bench.step_legs([n for _, n, _ in step(0, 1, 1, 1)]) == (
        ["prefill128k"] * 6 + ["prefill1m"] * 4 + ["decode64x128k"] * 2 + [None] + ["decode1m"] * 2 + [None]
        + ["decode1m"] * 2)
    bench.summarize_traffic("step", str(tmp_path / "f2.csv"), str(tmp_path / "w2.csv"), str(tmp_path / "cf.csv"),
                            str(tmp_path / "cw.csv"))
    t = json.load(open(tmp_path / "traffic.json"))
    w = t["workloads"]
    assert w["prefill128k"]["index_prefill"]["fetch_bytes"] == 7 * 1024 * 2
    assert w["prefill128k"]["sparse_prefill"]["fetch_bytes"] == (1 + 2 * 40 + 2 * 3) * 1024 * 2
    assert w["prefill1m"]["sparse_prefill"]["fetch_bytes"] == (2 + 60 + 5) * 1024 * 2
    assert w["decode64x128k"]["sparse_decode"]["fetch_bytes"] == 20 * 1024 * 2
    assert w["decode1m"]["index_decode"]["fetch_bytes"] == 30 * 1024 * 2
    assert w["decode1m"]["sparse_decode"]["fetch_bytes"] == 2 * 1024 * 2
    assert w["decode1m"]["sparse_decode"]["write_bytes"] == 1 * 1024
    # per launch of a kernel over the whole step (3 kp launches per step)
    assert t["kernels"]["step"]["kp_kernel"]["fetch_bytes_per_launch"] == round((40 + 40 + 60) / 3 * 1024 * 2)
    assert "decode_fp8" in w  # measurements of other workloads for the same sources are kept


def test_header_is_plain_c_and_links(tmp_path):
    # the boundary is usable from C: the header compiles as C99 (-pedantic) and a C
    # program links against libmsa.so and calls its host-only entry points
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    msa.lib()  # the library must be built
    src = tmp_path / "abi.c"
    src.write_text(
        '#include <stdio.h>\n#include <string.h>\n#include "msa.h"\n'
        "int main(void) {\n"
        "  if (msa_abi_version() != MSA_ABI_VERSION) return 1;\n"
        '  if (strcmp(msa_status_string(MSA_ERR_WORKSPACE), "") == 0) return 2;\n'
        "  if (msa_probe_mfma(0, 1, NULL, NULL) != MSA_ERR_INVALID_ARG) return 3;\n"
        '  if (strstr(msa_last_error(), "n_wg") == NULL) return 4;\n'
        '  printf("ok %d\\n", msa_abi_version());\n  return 0;\n}\n')
    libdir = os.path.join(ROOT, "block_sparse_attention_branch_amd")
    exe = tmp_path / "abi"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe), "-L", libdir, "-l:libmsa.so", f"-Wl,-rpath,{libdir}"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert r.stdout.strip() == "ok 6"


def test_bench_summarizes_stats_and_counters_without_gpu(tmp_path, capsys):
    # The profile tables are host logic over rocprofv3 CSVs: the kernel table
    # with the KV-outer kernel's launch-weighted mean over its instances, and
    # per-kernel counter averages (matrix-core share of GRBM cycles over 8 XCDs
    # and 1024 SIMDs, VALU per MFMA instruction, L2 hit rate, several rows of one
    # dispatch adding up).  Checked on made-up CSVs with hand-computed values.
    import csv
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod2", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    stats = tmp_path / "stats.csv"
    with open(stats, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                                           "MaxNs", "StdDev"])
        w.writeheader()
        w.writerow({"Name": "msa::kp_kernel<true>", "Calls": 3, "TotalDurationNs": 900000, "AverageNs": 300000,
                    "Percentage": 60.0, "MinNs": 1, "MaxNs": 2, "StdDev": 0})
        w.writerow({"Name": "msa::kp_kernel<false>", "Calls": 1, "TotalDurationNs": 1100000, "AverageNs": 1100000,
                    "Percentage": 40.0, "MinNs": 1, "MaxNs": 2, "StdDev": 0})
    bench.summarize_stats(str(stats))
    out = capsys.readouterr().out
    assert "(3 x 300.00 + 1 x 1100.00) / 4 = 500.0 us" in out  # (900 + 1100) / 4

    def write(path, rows):
        with open(path, "w", newline="") as fh:
            w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writeheader()
            for did, name, c, v in rows:
                w.writerow({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": c, "Counter_Value": v})

    k = "_ZN3msa17ki_prefill_kernelIDF16bLi64EEEv"
    # two dispatches: GRBM 8192 cycles (1024 per XCD), MFMA busy 1024 * 1024 * 0.5 cycles, 6 VALU per MFMA
    sq = []
    for did in (1, 2):
        sq += [(did, k, "GRBM_GUI_ACTIVE", 8192), (did, k, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 1024 * 0.5),
               (did, k, "SQ_INSTS_VALU", 600), (did, k, "SQ_INSTS_MFMA", 100), (did, k, "SQ_INSTS_LDS", 7),
               (did, k, "SQ_WAVES", 64), (did, k, "SQ_BUSY_CYCLES", 1)]
    # TCC rows per dispatch split in two (they add up): 3 hits, 1 miss
    tcc = [(1, k, "TCC_HIT_sum", 1), (1, k, "TCC_HIT_sum", 2), (1, k, "TCC_MISS_sum", 1),
           (2, k, "TCC_HIT_sum", 3), (2, k, "TCC_MISS_sum", 1)]
    write(tmp_path / "sq.csv", sq)
    write(tmp_path / "tcc.csv", tcc)
    bench.summarize_counters(str(tmp_path / "sq.csv"), str(tmp_path / "tcc.csv"))
    row = [l for l in capsys.readouterr().out.splitlines() if l.startswith("ki_prefill_kernel")][0].split()
    assert row[1] == "2" and row[2] == "0.500" and row[3] == "6.00" and row[-1] == "0.750"

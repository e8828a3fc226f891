"""Host logic of bench.py, on the CPU: the algorithmic byte counts behind the
roofline figures, the one-GPU refusal, kernel-name handling and the rocprofv3
counter summary (scaling by the calibration copy, the source digest check)."""
import csv
import json
import os
import subprocess
import sys
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _meta(lengths, tokens, fmt="bf16", k=2048):
    """The metadata the byte model reads, without any tensor data."""
    return types.SimpleNamespace(
        token_seq=np.array([b for b, _ in tokens], dtype=np.int32),
        token_pos=np.array([p for _, p in tokens], dtype=np.int32),
        num_seqs=len(lengths), num_tokens=len(tokens), cache_fmt=fmt, k=k)


PER_TOKEN_INDEXER = 64 * 128 * 2 + 64 * 4            # bf16 query, fp32 head weights
PER_TOKEN_STEP = 64 * 576 * 2 + 64 * 4 + 64 * 512 * 4 + 64 * 4   # q_A, gate, out, lse


def test_long_decode_bytes():
    # 16 sequences of 131,072 positions, one decode token at the last position
    wl = _meta([131072] * 16, [(b, 131071) for b in range(16)])
    assert bench.indexer_bytes(wl) == 16 * 131072 * 256 + 16 * PER_TOKEN_INDEXER == 537_137_152
    assert bench.step_bytes(wl) == 537_137_152 + 16 * 2048 * 1152 + 16 * PER_TOKEN_STEP == 578_170_880
    assert bench.indexer_flops(wl) == 16 * 131072 * 2 * 64 * 128


def test_fp8_and_mx_row_sizes():
    tokens = [(b, 262143) for b in range(8)]
    for fmt, key, row in (("e4m3fn", 132, 580), ("mxfp8", 132, 594), ("mxfp4", 68, 306)):
        wl = _meta([262144] * 8, tokens, fmt=fmt)
        assert bench.indexer_bytes(wl) == 8 * 262144 * key + 8 * PER_TOKEN_INDEXER
        assert bench.step_bytes(wl) == bench.indexer_bytes(wl) + 8 * 2048 * row + 8 * PER_TOKEN_STEP


def test_shared_rows_count_once_and_short_contexts_keep_all():
    # eight tokens of one sequence at positions 100..107 read the sequence's
    # first 108 keys once; a second sequence's token sees 5 positions, fewer than k
    wl = _meta([108, 5], [(0, p) for p in range(100, 108)] + [(1, 4)])
    assert bench.indexer_bytes(wl) == (108 + 5) * 256 + 9 * PER_TOKEN_INDEXER
    sel = sum(min(p + 1, 2048) for p in range(100, 108)) + 5
    assert bench.step_bytes(wl) == bench.indexer_bytes(wl) + sel * 1152 + 9 * PER_TOKEN_STEP


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_kernel_names():
    name = "void sga::(anonymous namespace)::attn_kernel<0, false, true>(sga::AttnArgs, sga::TopkArgs)"
    assert bench.kernel_key(name) == "attn_kernel<0, false, true>"
    assert bench.kernel_key("sga::(anonymous namespace)::combine_kernel(sga::AttnArgs)") == "combine_kernel"
    assert bench.in_step("attn_kernel<0, false, true>") and bench.in_step("attn_kernel<1, false, false>")
    assert not bench.in_step("attn_kernel<0, true, false>")        # the probabilities variant
    assert bench.in_step("indexer_kernel<0, true>") and not bench.in_step("indexer_kernel<0, false>")
    assert bench.in_step("indexer_prefill_kernel<0, true>")
    for k in ("clear_kernel", "topk_select_kernel", "topk_finalize_kernel", "combine_kernel"):
        assert bench.in_step(k)
    for k in ("proj_vec_kernel", "proj_kernel<1, 1>", "cache_append_kernel", "hbm_read_kernel"):
        assert not bench.in_step(k)
    lib = bench.library_kernels()
    assert {"indexer_kernel", "indexer_prefill_kernel", "topk_select_kernel", "attn_kernel",
            "combine_kernel", "proj_vec_kernel", "hbm_read_kernel"} <= lib


def _write_pass(root, pas, rows):
    d = os.path.join(root, pas)
    os.makedirs(d)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_counter_summary_scaling_and_digest(tmp_path, monkeypatch):
    out = tmp_path / "pmc.json"
    monkeypatch.setattr(bench, "pmc_file", lambda workload: str(out))
    idx = "void sga::(anonymous namespace)::indexer_kernel<0, true>(sga::IndexerArgs)"
    copy = "__amd_rocclr_copyBuffer"
    kib = bench.COPY_BYTES / 1024
    root = str(tmp_path / "runs")
    # the calibration copy: FETCH_SIZE reads half its bytes, WRITE_SIZE all of them
    _write_pass(root, "copy_fetch", [(copy, "FETCH_SIZE", kib / 2)] * 5)
    _write_pass(root, "copy_write", [(copy, "WRITE_SIZE", kib)] * 5)
    _write_pass(root, "fetch", [(idx, "FETCH_SIZE", 1000.0), (idx, "FETCH_SIZE", 1200.0),
                                ("at::native::other_kernel", "FETCH_SIZE", 7.0)])
    _write_pass(root, "write", [(idx, "WRITE_SIZE", 8.0), (idx, "WRITE_SIZE", 8.0)])
    _write_pass(root, "mfma", [(idx, "MfmaUtil", 15.0), (idx, "MfmaUtil", 16.0),
                               (idx, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 100.0),
                               (idx, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 100.0)])
    s = bench.summarize_pmc(root, "long_decode_128k")
    assert s["fetch_scale"] == pytest.approx(2.0) and s["write_scale"] == pytest.approx(1.0)
    e = s["kernels"]["indexer_kernel<0, true>"]
    assert e["fetch_bytes_per_launch"] == 1100 * 1024 * 2
    assert e["write_bytes_per_launch"] == 8 * 1024
    assert e["traffic_bytes_per_launch"] == 1100 * 1024 * 2 + 8 * 1024
    assert e["mfma_util_pct"] == pytest.approx(15.5)
    assert e["bf16_mfma_flops_per_launch"] == 100 * 512
    assert e["in_forward_step"] and e["dispatches"] == 2
    assert set(s["kernels"]) == {"indexer_kernel<0, true>"}   # torch's kernels are left out
    # the summary is used only while the kernel sources are the ones it was taken on
    assert bench.counter_summary("long_decode_128k") == json.loads(out.read_text())
    d = json.loads(out.read_text())
    d["csrc_sha256_16"] = "0" * 16
    out.write_text(json.dumps(d))
    assert bench.counter_summary("long_decode_128k") is None


def test_summary_without_calibration_copy_is_an_error(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "pmc_file", lambda workload: str(tmp_path / "pmc.json"))
    root = str(tmp_path / "runs")
    _write_pass(root, "fetch", [("indexer_kernel<0, true>", "FETCH_SIZE", 1.0)])
    with pytest.raises(SystemExit):
        bench.summarize_pmc(root, "long_decode_128k")
    assert not (tmp_path / "pmc.json").exists()


def test_timeline_summary_reads_the_stamp_layout():
    # two indexer workgroups, one select, one attention and one combine
    # workgroup, stamped at known device-clock ticks (100 per microsecond)
    ix = np.zeros((8192, 8), np.uint64)
    tk = np.zeros((8192, 8), np.uint64)
    at = np.zeros((8192, 8), np.uint64)
    t0 = 10_000_000
    ix[0, [0, 1, 2, 3, 4]] = [t0, t0 + 200, t0 + 400, t0 + 2900, t0 + 3000]
    ix[0, 7] = (3 << 32) | 0x123
    ix[1, [0, 1, 2, 3, 4]] = [t0 + 10, t0 + 500, t0 + 1300, t0 + 4300, t0 + 4400]
    ix[1, 7] = (5 << 32) | 0x456
    tk[0, [0, 2, 3, 4, 5, 1]] = [t0 + 4600, t0 + 4740, t0 + 4820, t0 + 4920, t0 + 5180, t0 + 5190]
    at[0, [0, 1, 2, 3, 4]] = [t0 + 5400, t0 + 6200, t0 + 6540, t0 + 7360, t0 + 7460]
    at[4096, [0, 1]] = [t0 + 7650, t0 + 8090]
    lines = bench.timeline_summary(ix.reshape(-1), tk.reshape(-1), at.reshape(-1), cus=1)
    text = "\n".join(lines)
    assert "indexer: 2 workgroups, last end   44.00" in text
    rows = {ln.split("(")[0].strip(): ln.split(")")[1].split() for ln in lines if "per CU (" in ln}
    assert rows["first per CU"] == ["1", "0.00", "2.00", "4.00", "30.00", "30.00"]
    assert rows["second per CU"] == ["1", "0.10", "5.00", "13.00", "44.00", "44.00"]
    assert "3:30.00" in text and "5:44.00" in text
    assert "select: 1 workgroups, start   46.00, end   51.90" in text
    assert "inputs in    1.40, list slots summed    0.80, cut    1.00, candidates written    2.60, whole    5.90" in text
    assert "start   54.00, final stage done   62.00, first tile   65.40, tiles done   73.60, end   74.60" in text
    assert "combine: 1 workgroups, start   76.50, end   80.90" in text

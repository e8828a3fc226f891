"""Benchmark of the SGA decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long_decode_128k]

One step is one sga_forward call (indexer -> top-k -> sparse MLA attention ->
gate) over the whole batch. The default workload is 16 sequences at 128K
context, one query token each, top-2048. The inputs are seeded synthetic
caches (sga_inputs) and are resident in HBM before the timed region starts.
Two copies of the inputs alternate between steps, so no step finds the
previous step's data in the 256 MB Infinity Cache.

Prints one JSON line with:
- query-tokens/s;
- roofline: the indexer kernel, timed with HIP events on the library's stream
  inside the timed steps (one step in EVENT_EVERY records them; they are the
  only events the timed steps record), against the 8 TB/s HBM peak. The
  algorithmic bytes
  are the indexer keys it must read plus its query inputs. For a chunked
  prefill, where thousands of tokens share one sequence's keys, the roof is
  the 2.5 PFLOP/s dense bf16 MFMA peak instead;
- cpu_baseline: the float64 CPU oracle, timed on this host over whole batches
  of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import sga_inputs as si  # noqa: E402
import sparse_gated_mla_amd as sga  # noqa: E402

METRIC = "SGA decode query-tokens/sec at 128K ctx, k=2048; achieved HBM GB/s vs peak"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
COPY_BYTES = 1 << 30                # calibration copy size
WORKLOADS = {"tiny_decode_4k": 0, "batched_decode_ragged_16k_32k": 1, "long_decode_128k": 2,
             "chunked_prefill_128k": 3,
             "extended_decode_256k_fp8": 4, "extended_decode_256k_mxfp8": 5,
             "extended_decode_256k_mxfp4": 6}
PMC_WORKLOAD = "long_decode_128k"
EVENT_EVERY = 4                     # timed steps per step that times the indexer
PMC_FILE = os.path.join(ROOT, "profiles", "indexer_long_decode_128k_pmc.json")
# the sources the indexer kernel is built from
INDEXER_SRC = [os.path.join(ROOT, "sparse_gated_mla_amd", "csrc", f)
               for f in ("indexer.hip", "sga_kernels.h", "sga_device.h", "sga_block.h")]


# ---------------------------------------------------------------- HIP events
class HipEvents:
    """Timing-only HIP events through libamdhip64 (raw handles for sga_trace).

    They are created with hipEventDisableSystemFence, so recording one between
    two kernels adds no system-scope cache writeback: the timed kernels run as
    they would untraced."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.events = []

    def create(self) -> ctypes.c_void_p:
        e = ctypes.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
        self.events.append(e)
        return e

    def record(self, e, stream: int):
        rc = self.hip.hipEventRecord(e, ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(ms.value)

    def close(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


# ---------------------------------------------------------------- byte model
def visible(wl) -> np.ndarray:
    return wl.token_pos.astype(np.int64) + 1


# bytes per cached row, scales included: the indexer key (128 elements) and the
# latent row (576): bf16; E4M3FN + an fp32 row scale; MX E4M3FN or E2M1 + one
# E8M0 byte per 32 elements
KEY_ROW_BYTES = {"bf16": 256, "e4m3fn": 128 + 4, "mxfp8": 128 + 4, "mxfp4": 64 + 4}
KV_ROW_BYTES = {"bf16": 1152, "e4m3fn": 576 + 4, "mxfp8": 576 + 18, "mxfp4": 288 + 18}


def indexer_bytes(wl) -> int:
    """Algorithmic bytes of one indexer launch: every visible indexer key once
    (KEY_ROW_BYTES for the cache format) and each token's 64x128 bf16
    query and 64 fp32 head weights. Keys shared by several tokens of one
    sequence count once."""
    per_row = KEY_ROW_BYTES[wl.cache_fmt]
    rows = 0
    for b in range(wl.num_seqs):
        sel = wl.token_seq == b
        if sel.any():
            rows += int(visible(wl)[sel].max())
    return rows * per_row + wl.num_tokens * (64 * 128 * 2 + 64 * 4)


def indexer_flops(wl) -> int:
    """Multiply-add work of one indexer launch: 2*64*128 flops per (token,
    visible position) for the logits; the ReLU and head weighting are not
    counted."""
    return int(visible(wl).astype(np.int64).sum()) * 2 * 64 * 128


def step_bytes(wl) -> int:
    """Algorithmic bytes of one whole step: the indexer's bytes plus, per token,
    its min(k, visible) selected latent rows (KV_ROW_BYTES for the format),
    its 64x576 bf16 absorbed query, 64 gate logits, and its fp32 output
    (64x512) and lse (64)."""
    per_row = KV_ROW_BYTES[wl.cache_fmt]
    sel_rows = int(np.minimum(visible(wl), wl.k).sum())
    per_tok = 64 * 576 * 2 + 64 * 4 + 64 * 512 * 4 + 64 * 4
    return indexer_bytes(wl) + sel_rows * per_row + wl.num_tokens * per_tok


def append_bytes(wl) -> int:
    """Algorithmic bytes of one cache append of every token's new rows: the
    bf16 latent (576) and indexer key (128) read, the token's metadata
    (sequence, position, start, length: 20 bytes) read, and the rows written
    in the cache format, scales included (KV_ROW_BYTES + KEY_ROW_BYTES)."""
    out = KV_ROW_BYTES[wl.cache_fmt] + KEY_ROW_BYTES[wl.cache_fmt]
    return wl.num_tokens * ((576 + 128) * 2 + 20 + out)


def time_cache_append(wl, s, ev, reps: int) -> dict:
    """Times sga_cache_append of one new row per token into the step's caches
    (the write that precedes a decode step), one event pair per launch."""
    dev = s["kv"].device
    lat, key = si.append_rows(wl.num_tokens, seed=99)
    lat, key = lat.to(dev), key.to(dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    pairs = [(ev.create(), ev.create()) for _ in range(reps)]
    append = lambda: sga.sga_cache_append(s["batch"], lat, key, s["kv"], s["kv_scale"], s["k_idx"],
                                          s["k_idx_scale"])
    for _ in range(3):
        append()
    torch.cuda.synchronize()
    # a spin kernel keeps the GPU busy while the host queues the timed launches,
    # so each event pair brackets one kernel and not the host's call overhead
    s0, s1 = ev.create(), ev.create()
    ev.record(s0, stream)
    torch.cuda._sleep(5_000_000)
    ev.record(s1, stream)
    t0 = time.perf_counter()
    for a, b in pairs:
        ev.record(a, stream)
        append()
        ev.record(b, stream)
    host_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    us = float(np.mean([ev.elapsed_ms(a, b) for a, b in pairs])) * 1e3
    nb = append_bytes(wl)
    return {"us": round(us, 2), "algorithmic_bytes": nb, "gbps": round(nb / (us * 1e-6) / 1e9, 1),
            "tokens": wl.num_tokens, "spin_ms": round(ev.elapsed_ms(s0, s1), 3),
            "host_enqueue_ms": round(host_ms, 3)}


def time_output_proj(wl, out, ev, reps: int) -> dict:
    """Times sga_output_proj of the step's gated output (the output epilogue
    after the gate), with synthetic bf16 weights for a 7,168-wide hidden state,
    the same way as the cache append."""
    dev = out.device
    w_uv, w_o = si.proj_weights(seed=98)
    w_uv, w_o = w_uv.to(dev), w_o.to(dev)
    T, d_model = wl.num_tokens, w_o.shape[0]
    y = torch.empty((T, d_model), dtype=torch.float32, device=dev)
    ws = sga.workspace(sga.sga_output_proj_workspace_size(T, d_model), dev)
    run = lambda: sga.sga_output_proj(out, w_uv, w_o, y, ws=ws)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev).cuda_stream
    pairs = [(ev.create(), ev.create()) for _ in range(reps)]
    torch.cuda._sleep(5_000_000)
    for a, b in pairs:
        ev.record(a, stream)
        run()
        ev.record(b, stream)
    torch.cuda.synchronize()
    us = float(np.mean([ev.elapsed_ms(a, b) for a, b in pairs])) * 1e3
    nbytes = (w_uv.numel() + w_o.numel()) * 2 + out.numel() * 4 + y.numel() * 4
    flops = 2 * T * (64 * 128 * 512 + d_model * 64 * 128)
    return {"us": round(us, 2), "d_model": int(d_model), "algorithmic_bytes": int(nbytes),
            "gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "tflops": round(flops / (us * 1e-6) / 1e12, 2)}


def time_indexer_loss(wl, s, idx, lse, ev, reps: int) -> dict:
    """Times sga_indexer_loss over the step's selection (indices and lse of the
    last step, the scores from sga_index_scores), the same way as the cache append."""
    dev = idx.device
    T = wl.num_tokens
    scores = torch.empty((T, wl.max_len), dtype=torch.float32, device=dev)
    sga.sga_index_scores(s["batch"], s["q_idx"], s["w"], s["k_idx"], s["k_idx_scale"], scores)
    loss = torch.empty((T,), dtype=torch.float32, device=dev)
    ws = sga.workspace(sga.sga_indexer_loss_workspace_size(T, wl.k), dev)
    run = lambda: sga.sga_indexer_loss(s["batch"], s["q_abs"], s["kv"], s["kv_scale"], idx, wl.k,
                                       wl.sm_scale, lse, scores, loss, ws=ws)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev).cuda_stream
    pairs = [(ev.create(), ev.create()) for _ in range(reps)]
    torch.cuda._sleep(5_000_000)
    for a, b in pairs:
        ev.record(a, stream)
        run()
        ev.record(b, stream)
    torch.cuda.synchronize()
    us = float(np.mean([ev.elapsed_ms(a, b) for a, b in pairs])) * 1e3
    return {"us": round(us, 2), "mean_loss": round(float(loss.mean().item()), 6)}


# ---------------------------------------------------------------- traffic
def src_digest() -> str:
    h = hashlib.sha256()
    for p in INDEXER_SRC:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per indexer launch from the committed rocprofv3 counter summary,
    or None when it is missing or was taken on a different indexer source."""
    try:
        with open(PMC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("indexer_source_sha256_16") != src_digest():
        return None
    return d.get("traffic_bytes_per_launch")


def summarize_pmc(root: str) -> dict:
    """Writes the indexer's HBM traffic summary from rocprofv3 counter runs.

    `root` holds one rocprofv3 output folder per pass: a FETCH_SIZE pass and a
    WRITE_SIZE pass over a short bench run, and the same two counters over
    `--copy-calibration` (five copies of 1 GiB). Both counters read KiB per
    dispatch; each is scaled by the bytes a known copy moves over what the
    counter reads for that copy."""
    import csv
    import glob
    per = {}                        # (run, kernel, counter) -> values per dispatch
    for f in glob.glob(os.path.join(root, "*", "*counter_collection.csv")):
        for row in csv.DictReader(open(f)):
            per.setdefault((f, row["Kernel_Name"], row["Counter_Name"]), []).append(
                float(row["Counter_Value"]))
    mean = lambda v: sum(v) / len(v)
    copy_kib = COPY_BYTES / 1024.0
    out = {"indexer_source_sha256_16": src_digest(), "workload": PMC_WORKLOAD,
           "copy_bytes": COPY_BYTES,
           "commands": [
               "rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d <dir>/fetch -o run "
               "-- python3 bench.py --steps 3 --warmup 1 --copies 1 --no-cpu-baseline",
               "rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d <dir>/write -o run "
               "-- python3 bench.py --steps 3 --warmup 1 --copies 1 --no-cpu-baseline",
               "rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d <dir>/copy_fetch "
               "-o run -- python3 bench.py --copy-calibration",
               "rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d <dir>/copy_write "
               "-o run -- python3 bench.py --copy-calibration",
               "python3 bench.py --summarize-pmc <dir>"]}
    total = 0.0
    for ctr, name in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        copies = [mean(v) for (_, k, c), v in per.items() if c == ctr and "copyBuffer" in k]
        idx = [v for (_, k, c), v in per.items() if c == ctr and "indexer_kernel" in k]
        if not copies or not idx:
            raise SystemExit(f"no {ctr} rows for the copy or the indexer under {root}")
        # the calibration copy moves the largest amount of any copy in the runs
        factor = copy_kib / max(copies)
        kib = mean(idx[0])
        out[f"{name}_kib_per_dispatch"] = kib
        out[f"{name}_copy_kib_per_dispatch"] = max(copies)
        out[f"{name}_scale"] = factor
        out[f"{name}_bytes_per_launch"] = kib * 1024.0 * factor
        total += kib * 1024.0 * factor
    out["traffic_bytes_per_launch"] = total
    os.makedirs(os.path.dirname(PMC_FILE), exist_ok=True)
    with open(PMC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    return out


# ---------------------------------------------------------------- CPU oracle
def cpu_baseline(wl, min_seconds: float):
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the affinity size
        threads = len(os.sched_getaffinity(0))
    ks = (oracle.Store(wl.k_idx.view(torch.uint8).numpy(), wl.cache_fmt, wl.k_idx_scale.numpy()) if wl.fp8
          else oracle.Store(wl.k_idx.view(torch.int16).numpy().view(np.uint16), "bf16"))
    vs = (oracle.Store(wl.kv.view(torch.uint8).numpy(), wl.cache_fmt, wl.kv_scale.numpy()) if wl.fp8
          else oracle.Store(wl.kv.view(torch.int16).numpy().view(np.uint16), "bf16"))
    args = (wl.token_seq, wl.token_pos, wl.seq_start, wl.seq_len, wl.q_idx.double().numpy(),
            wl.w.double().numpy(), ks, wl.q_abs.double().numpy(), vs, wl.gate.double().numpy(),
            wl.k, wl.sm_scale)
    done, t0 = 0, time.perf_counter()
    passes = 0
    while True:
        oracle.forward(*args)
        done += wl.num_tokens
        passes += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return {"value": done / el, "unit": "query-tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{passes} full pass(es) over the {wl.num_tokens}-token {wl.name} batch "
                      f"({done} query tokens, {el:.1f} s, float64 numpy)"}


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first (the clocks settle over the first few dozen)")
    ap.add_argument("--workload", default="long_decode_128k", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copies", type=int, default=2, help="input sets alternated between steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of known size (for counter calibration)")
    ap.add_argument("--summarize-pmc", metavar="DIR",
                    help="write the indexer traffic summary from rocprofv3 counter runs under DIR")
    args = ap.parse_args()
    if args.summarize_pmc:
        print(json.dumps(summarize_pmc(args.summarize_pmc)))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path runs on one GPU with no collectives)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = COPY_BYTES
        a = torch.ones(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 5}))
        return

    wl = si.config(WORKLOADS[args.workload])
    T = wl.num_tokens
    sets = []
    for c in range(max(1, args.copies)):
        d = lambda x: None if x is None else x.to(dev)
        batch = sga.batch_to_device(wl.token_seq, wl.token_pos, wl.seq_start, wl.seq_len,
                                    wl.cache_rows, device=dev, max_len=wl.max_len)
        sets.append(dict(batch=batch, q_idx=d(wl.q_idx), w=d(wl.w), k_idx=d(wl.k_idx),
                         k_idx_scale=d(wl.k_idx_scale), q_abs=d(wl.q_abs), kv=d(wl.kv),
                         kv_scale=d(wl.kv_scale), gate=d(wl.gate)))
    out = torch.empty((T, 64, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((T, 64), dtype=torch.float32, device=dev)
    idx = torch.empty((T, wl.k), dtype=torch.int32, device=dev)
    ws = sga.workspace(sga.sga_forward_workspace_size(T, wl.max_len, wl.k), dev)

    ev = HipEvents()
    K, W = args.steps, args.warmup
    # one timed step in EVENT_EVERY records the two events around the indexer
    # (the roofline's kernel): every event recorded between two kernels costs
    # its step about a microsecond and a half
    tr = [sga.SgaTrace(ev.create().value, ev.create().value, None, None)
          if i % EVENT_EVERY == 0 else None for i in range(K)]
    # the top-k and attention split comes from separate, untimed steps
    KB = min(K, 10)
    tb = [sga.SgaTrace(ev.create().value, ev.create().value, ev.create().value, ev.create().value)
          for _ in range(KB)]

    def step(i, trace=None):
        s = sets[i % len(sets)]
        sga.sga_forward(s["batch"], s["q_idx"], s["w"], s["k_idx"], s["k_idx_scale"], s["q_abs"],
                        s["kv"], s["kv_scale"], wl.k, wl.sm_scale, s["gate"], out, lse, idx,
                        ws=ws, trace=trace)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i, tr[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    for i in range(KB):
        step(K + i, tb[i])
    torch.cuda.synchronize()

    # around the step, after it: the indexer loss over the last step's selection
    # (input set (K - 1) % copies), the output epilogue of its output, then the
    # cache append (which writes into the caches, so it comes last)
    loss = time_indexer_loss(wl, sets[(K + KB - 1) % len(sets)], idx, lse, ev, reps=10)
    proj = time_output_proj(wl, out, ev, reps=10)
    append = time_cache_append(wl, sets[0], ev, reps=20)
    idx_ms = [ev.elapsed_ms(t.indexer_begin, t.indexer_end) for t in tr if t is not None]
    topk_ms = [ev.elapsed_ms(tb[i].indexer_end, tb[i].topk_end) for i in range(KB)]
    attn_ms = [ev.elapsed_ms(tb[i].topk_end, tb[i].attn_end) for i in range(KB)]
    ev.close()
    ms_per_step = 1e3 * wall / K
    value = T * K / wall
    ib = indexer_bytes(wl)
    idx_avg_s = float(np.mean(idx_ms)) / 1e3
    sb = step_bytes(wl)
    # the indexer's roof: HBM for decode; the MFMA when many tokens share one
    # sequence's keys (chunked prefill), whichever takes longer at peak
    flops = indexer_flops(wl)
    if flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > ib / (HBM_PEAK_GBPS * 1e9):
        roof = {"bound": "mfma", "kernel": "indexer_kernel",
                "achieved": round(flops / idx_avg_s / 1e12, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(flops / idx_avg_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": None, "algorithmic_flops_per_launch": flops}
    else:
        achieved = ib / idx_avg_s / 1e9
        roof = {"bound": "hbm", "kernel": "indexer_kernel", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic() if wl.name == PMC_WORKLOAD else None,
                "algorithmic_bytes_per_launch": ib}
    roof["avg_launch_us"] = round(idx_avg_s * 1e6, 2)
    roof["timed_launches"] = len(idx_ms)
    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "query-tokens/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": dict(si.describe(wl), parallelism="single GPU"),
        "roofline": roof,
        "extra": {"step_algorithmic_bytes": sb,
                  "step_gbps": round(sb / (ms_per_step / 1e3) / 1e9, 1),
                  "step_frac_of_hbm_peak": round(sb / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
                  "indexer_us": round(float(np.mean(idx_ms)) * 1e3, 2),
                  "topk_us": round(float(np.mean(topk_ms)) * 1e3, 2),
                  "attention_us": round(float(np.mean(attn_ms)) * 1e3, 2),
                  "input_copies": len(sets),
                  "cache_append": append,
                  "output_proj": proj,
                  "indexer_loss": loss},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

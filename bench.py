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
- roofline: the dominant kernel, the indexer, timed with HIP events on the
  library's stream inside the timed steps (one step in EVENT_EVERY records
  them; they are the only events the timed steps record), against the 8 TB/s
  HBM peak. The algorithmic bytes are the indexer keys it must read plus its
  query inputs. For a chunked prefill, where thousands of tokens share one
  sequence's keys, the roof is the 2.5 PFLOP/s dense bf16 MFMA peak instead.
  Beside it: the whole step against the same peak (roofline.step), the
  bandwidth a plain 1 GiB device copy and sum reach here, and, when the
  committed rocprofv3 counter summary matches the kernel sources, the HBM
  traffic and the MFMA utilisation per kernel;
- cpu_baseline: the float64 CPU oracle, timed on this host over whole batches
  of the same workload.

The timed steps start after W warm-up steps and at least --settle-seconds of
untimed steps, so a short warm-up still times settled clocks.
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
EVENT_EVERY = 4                     # timed steps per step that times the indexer
SIMD_NUM = 1024                     # 256 compute units x 4 SIMDs
CSRC = os.path.join(ROOT, "sparse_gated_mla_amd", "csrc")


def pmc_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"pmc_{workload}.json")


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
    the same way as the cache append: with one weight set reused ("us"; the
    256 MB MALL can hold part of it between calls) and with three sets
    alternating ("us_three_weight_sets"; as in a model whose layers each have
    their own weights)."""
    dev = out.device
    sets = [tuple(x.to(dev) for x in si.proj_weights(seed=98 + i)) for i in range(3)]
    w_uv, w_o = sets[0]
    T, d_model = wl.num_tokens, w_o.shape[0]
    y = torch.empty((T, d_model), dtype=torch.float32, device=dev)
    ws = sga.workspace(sga.sga_output_proj_workspace_size(T, d_model), dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    res = {}
    for key, pick in (("us", lambda i: sets[0]), ("us_three_weight_sets", lambda i: sets[i % 3])):
        run = lambda i: sga.sga_output_proj(out, *pick(i), y, ws=ws)
        for i in range(3):
            run(i)
        torch.cuda.synchronize()
        pairs = [(ev.create(), ev.create()) for _ in range(reps)]
        torch.cuda._sleep(5_000_000)
        for i, (a, b) in enumerate(pairs):
            ev.record(a, stream)
            run(i)
            ev.record(b, stream)
        torch.cuda.synchronize()
        res[key] = round(float(np.mean([ev.elapsed_ms(a, b) for a, b in pairs])) * 1e3, 2)
    nbytes = (w_uv.numel() + w_o.numel()) * 2 + out.numel() * 4 + y.numel() * 4
    flops = 2 * T * (64 * 128 * 512 + d_model * 64 * 128)
    us = res["us"]
    return {"us": us, "us_three_weight_sets": res["us_three_weight_sets"], "d_model": int(d_model),
            "algorithmic_bytes": int(nbytes), "gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "gbps_three_weight_sets": round(nbytes / (res["us_three_weight_sets"] * 1e-6) / 1e9, 1),
            "tflops": round(flops / (us * 1e-6) / 1e12, 2)}


def time_two_streams(wl, sets, dev, steps: int) -> dict:
    """The same steps with two batches in flight: the two input sets alternate
    over two streams (default priority), each with its own workspace and
    outputs, so one batch's latency-bound tail overlaps the next one's
    bandwidth-bound indexer. Reported beside the single-stream value, as a
    serving configuration, not as the step time."""
    T = wl.num_tokens
    own = []
    for s in sets[:2]:
        own.append(dict(s, out=torch.empty((T, 64, 512), dtype=torch.float32, device=dev),
                        lse=torch.empty((T, 64), dtype=torch.float32, device=dev),
                        idx=torch.empty((T, wl.k), dtype=torch.int32, device=dev),
                        ws=sga.workspace(sga.sga_forward_workspace_size(T, wl.max_len, wl.k), dev),
                        stream=torch.cuda.Stream(device=dev)))
    if len(own) < 2:
        return None

    def step(i):
        s = own[i % 2]
        with torch.cuda.stream(s["stream"]):
            sga.sga_forward(s["batch"], s["q_idx"], s["w"], s["k_idx"], s["k_idx_scale"], s["q_abs"],
                            s["kv"], s["kv_scale"], wl.k, wl.sm_scale, s["gate"], s["out"], s["lse"],
                            s["idx"], ws=s["ws"])
    for i in range(100):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return {"us_per_step": round(wall * 1e6 / steps, 2), "query_tokens_per_s": round(T * steps / wall, 1),
            "steps": steps}


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
    """Digest of every kernel source: counter figures taken on other sources are stale."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def counter_summary(workload: str):
    """The committed rocprofv3 counter summary of a workload, or None when it is
    missing or was taken on different kernel sources."""
    try:
        with open(pmc_file(workload)) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    return d if d.get("csrc_sha256_16") == src_digest() else None


def library_kernels() -> set:
    """The names of the library's kernels, from its sources."""
    import re
    names = set()
    for f in os.listdir(CSRC):
        if f.endswith(".hip"):
            names |= set(re.findall(r"\bvoid\s+(\w+_kernel)\s*\(", open(os.path.join(CSRC, f)).read()))
    return names


def in_step(key: str) -> bool:
    """Whether a kernel (short name with template arguments) runs in sga_forward:
    the indexer variant that counts the histogram, the top-k kernels, the
    attention variant without probabilities and the merge."""
    base, _, targs = key.partition("<")
    args = [x.strip() for x in targs.rstrip(">").split(",")] if targs else []
    if base in ("indexer_kernel", "indexer_prefill_kernel"):
        return args[-1:] == ["true"]
    if base == "attn_kernel":
        return len(args) > 1 and args[1] == "false"
    return base in ("clear_kernel", "topk_select_kernel", "topk_finalize_kernel", "topk_token_kernel",
                    "combine_kernel")


def kernel_key(name: str) -> str:
    """A kernel's short name, with its template arguments: 'attn_kernel<0, false, true>'."""
    import re
    m = re.search(r"(\w+_kernel|copyBuffer)(<[^>]*>)?", name)
    return m.group(0) if m else name[:40]


def summarize_pmc(root: str, workload: str) -> dict:
    """Writes a workload's per-kernel counter summary from rocprofv3 runs.

    `root` holds one rocprofv3 output folder per pass (each `-o run`):
    fetch/ and write/ (FETCH_SIZE, WRITE_SIZE over a short bench run),
    copy_fetch/ and copy_write/ (the same counters over `--copy-calibration`,
    five copies of 1 GiB) and mfma/ (MfmaUtil with its inputs and the bf16
    MFMA op count). FETCH_SIZE and WRITE_SIZE read KiB per dispatch; each is
    scaled by the bytes the known copy moves over what the counter reads for
    it. MfmaUtil is rocprofv3's derived counter: the summed MFMA-busy cycles of
    all SIMDs over the busiest XCD's active cycles times the SIMD count."""
    import csv
    per = {}                        # (pass, kernel, counter) -> values per dispatch
    for pas in ("fetch", "write", "copy_fetch", "copy_write", "mfma"):
        f = os.path.join(root, pas, "run_counter_collection.csv")
        if not os.path.exists(f):
            continue
        for row in csv.DictReader(open(f)):
            per.setdefault((pas, kernel_key(row["Kernel_Name"]), row["Counter_Name"]), []).append(
                float(row["Counter_Value"]))
    mean = lambda v: sum(v) / len(v)
    cmd = ("rocprofv3 --pmc {c} --kernel-trace --output-format csv -d <dir>/{d} -o run -- python3 "
           "bench.py {a}")
    run = f"--workload {workload} --steps 3 --warmup 1 --settle-seconds 0 --copies 1 --no-cpu-baseline"
    out = {"csrc_sha256_16": src_digest(), "workload": workload, "copy_bytes": COPY_BYTES,
           "commands": [cmd.format(c="FETCH_SIZE", d="fetch", a=run),
                        cmd.format(c="WRITE_SIZE", d="write", a=run),
                        cmd.format(c="FETCH_SIZE", d="copy_fetch", a="--copy-calibration"),
                        cmd.format(c="WRITE_SIZE", d="copy_write", a="--copy-calibration"),
                        cmd.format(c="MfmaUtil SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE "
                                     "SQ_INSTS_VALU_MFMA_MOPS_BF16", d="mfma", a=run),
                        f"python3 bench.py --workload {workload} --summarize-pmc <dir>"],
           "kernels": {}}
    scale = {}
    for ctr, pas in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        copies = [mean(v) for (p, k, c), v in per.items() if p == "copy_" + pas and "copyBuffer" in k]
        if not copies:
            raise SystemExit(f"no {ctr} rows for the calibration copy under {root}")
        # the calibration copy moves the largest amount of any copy in the run
        scale[pas] = (COPY_BYTES / 1024.0) / max(copies)
        out[f"{pas}_scale"] = scale[pas]
    ours = library_kernels()
    for (pas, k, c), v in sorted(per.items()):
        if pas.startswith("copy") or k.partition("<")[0] not in ours:
            continue
        e = out["kernels"].setdefault(k, {})
        e["dispatches"] = max(e.get("dispatches", 0), len(v))
        if pas in ("fetch", "write"):
            e[f"{pas}_bytes_per_launch"] = round(mean(v) * 1024.0 * scale[pas])
        elif c == "MfmaUtil":
            e["mfma_util_pct"] = round(mean(v), 2)
        elif c == "SQ_INSTS_VALU_MFMA_MOPS_BF16":
            e["bf16_mfma_flops_per_launch"] = round(mean(v) * 512)
    for k, e in out["kernels"].items():
        e["in_forward_step"] = in_step(k)
        if "fetch_bytes_per_launch" in e and "write_bytes_per_launch" in e:
            e["traffic_bytes_per_launch"] = e["fetch_bytes_per_launch"] + e["write_bytes_per_launch"]
    os.makedirs(os.path.dirname(pmc_file(workload)), exist_ok=True)
    with open(pmc_file(workload), "w") as f:
        json.dump(out, f, indent=1)
    return out


def measure_bandwidth(dev, n: int = 512 << 20, reps: int = 20) -> dict:
    """HBM bandwidth this GPU reaches, timed with events on torch's stream:
    the library's streaming read probe over two alternating 512 MiB buffers
    (the indexer's access pattern; more than the 256 MB MALL holds), and a
    torch device copy of 512 MiB (read plus write)."""
    bufs = [torch.full((n,), i + 1, dtype=torch.uint8, device=dev) for i in range(2)]
    sink = torch.zeros(262144, dtype=torch.int32, device=dev)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    res = {}
    for name, fn, moved in (("stream_read", lambda i: sga.sga_hbm_read_probe(bufs[i & 1], sink), n),
                            ("device_copy", lambda i: dst.copy_(bufs[i & 1]), 2 * n)):
        for i in range(4):
            fn(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        res[f"{name}_gbps"] = round(moved * reps / (e0.elapsed_time(e1) / 1e3) / 1e9, 1)
    del bufs, dst
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


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
    T = wl.num_tokens
    # whole passes over the batch when one fits the time budget; otherwise an
    # evenly spaced sample of its tokens, sized from the time of one token
    t0 = time.perf_counter()
    oracle.forward(*args, tokens=[T - 1])
    per_token = time.perf_counter() - t0
    n = T if per_token * T <= min_seconds else max(1, int(min_seconds / per_token))
    sample = None if n == T else sorted({int(i) for i in np.linspace(0, T - 1, n)})
    done, passes, t0 = 0, 0, time.perf_counter()
    while True:
        oracle.forward(*args, tokens=sample)
        done += T if sample is None else len(sample)
        passes += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    what = (f"the {T}-token {wl.name} batch" if sample is None else
            f"{len(sample)} evenly spaced tokens of the {T}-token {wl.name} batch")
    return {"value": done / el, "unit": "query-tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{passes} pass(es) over {what} ({done} query tokens, {el:.1f} s, float64 numpy)"}


# ---------------------------------------------------------------- main
# ---------------------------------------------------------------- device timeline
TIMELINE_LIB = os.path.join(ROOT, "sparse_gated_mla_amd", "libsga_timeline.so")
TL_WORDS = 1 << 16                   # 64-bit words per stamp record (slot s, point k: 8s + k)
TL_RECORDS = ("indexer", "topk", "attn")


def timeline_summary(ix: np.ndarray, tk: np.ndarray, at: np.ndarray, cus: int) -> list:
    """Text lines for one forward step from the timeline build's three stamp
    records (uint64 words; point k of slot s at 8s + k, point 7 the ids XCC_ID
    << 32 | HW_ID; slots and points the step did not reach read 0). Times are
    microseconds of the 100 MHz device clock from the first indexer
    workgroup's start. Indexer slots (decode indexer of the forward pass): 0
    start, 1 keys set up (batch metadata known), 2 first key tile in LDS, 3
    last tile scored, 4 end. Select slots: 0 start, 2 inputs in, 3 list slots
    summed, 4 cut taken, 5 candidates written, 1 end. Attention slots below
    4,096: 0 start, 1 the top-k's final stage done (selecting variant), 2 first
    row tile in LDS, 3 tiles done, 4 partials written; combine slots from
    4,096: 0 start, 1 end."""
    ix, tk, at = (r.reshape(-1, 8).astype(np.int64) for r in (ix, tk, at))
    wi = ix[ix[:, 0] > 0]
    if len(wi) == 0:
        return ["no indexer stamps (the decode indexer of the forward pass did not run)"]
    base = wi[:, 0].min()

    def t(col):   # microseconds from base; unstamped points become NaN
        return np.where(col > 0, (col - base) / 100.0, np.nan)

    def med(x):
        x = x[~np.isnan(x)]
        return f"{np.median(x):7.2f}" if len(x) else "      -"

    def lo(x):
        x = x[~np.isnan(x)]
        return f"{x.min():7.2f}" if len(x) else "      -"

    def hi(x):
        x = x[~np.isnan(x)]
        return f"{x.max():7.2f}" if len(x) else "      -"

    slots = np.nonzero(ix[:, 0] > 0)[0]
    lines = [f"indexer: {len(wi)} workgroups, last end {hi(t(wi[:, 4]))}",
             "  dispatch group (slots)        n   start  keys set up  first tile      end   last end"]
    groups = ((f"first per CU (0-{cus - 1})", slots < cus),
              (f"second per CU ({cus}-{2 * cus - 1})", (slots >= cus) & (slots < 2 * cus)),
              (f"later ({2 * cus}-)", slots >= 2 * cus))
    for name, m in groups:
        if not m.any():
            continue
        g = wi[m]
        lines.append(f"  {name:<27}{m.sum():>5} {med(t(g[:, 0]))}      {med(t(g[:, 1]))}    {med(t(g[:, 2]))}  "
                     f"{med(t(g[:, 4]))}    {hi(t(g[:, 4]))}")
    xcc = (wi[:, 7] >> 32) & 0xF
    lines.append("  last end per XCD: " + " ".join(f"{x}:{hi(t(wi[xcc == x, 4])).strip()}"
                                                for x in range(8) if (xcc == x).any()))
    ws = tk[tk[:, 0] > 0]
    if len(ws):
        full = ws[(ws[:, 1:6] > 0).all(axis=1)]   # workgroups that ran every phase
        lines.append(f"select: {len(ws)} workgroups, start {lo(t(ws[:, 0]))}, end {hi(t(ws[:, 1]))}")
        if len(full):
            d = lambda a, b: (full[:, a] - full[:, b]) / 100.0
            lines.append(f"  per workgroup (medians): inputs in {med(d(2, 0))}, list slots summed {med(d(3, 2))}, "
                         f"cut {med(d(4, 3))}, candidates written {med(d(5, 4))}, whole {med(d(1, 0))}")
    wa = at[:4096][at[:4096, 0] > 0]
    if len(wa):
        lines.append(f"attention: {len(wa)} workgroups, start {lo(t(wa[:, 0]))}, final stage done {med(t(wa[:, 1]))}, "
                     f"first tile {med(t(wa[:, 2]))}, tiles done {med(t(wa[:, 3]))}, end {hi(t(wa[:, 4]))}")
    wc = at[4096:][at[4096:, 0] > 0]
    if len(wc):
        lines.append(f"combine: {len(wc)} workgroups, start {lo(t(wc[:, 0]))}, end {hi(t(wc[:, 1]))}")
    return lines


def run_timeline(workload: str, steps: int, reps: int = 3) -> None:
    """Prints the device-clock timeline of the last of `steps` back-to-back
    forward steps, `reps` times, from libsga_timeline.so (the same kernels
    with per-workgroup stamps; see sga_device.h)."""
    if not os.path.exists(TIMELINE_LIB):
        raise SystemExit(f"{TIMELINE_LIB} is missing: build it with "
                         "`python -m sparse_gated_mla_amd.build --timeline`")
    from sparse_gated_mla_amd import _lib as L
    lib = L.load(TIMELINE_LIB)
    L._lib = lib
    for r in TL_RECORDS:
        for fn in (f"sga_tl_read_{r}", f"sga_tl_clear_{r}"):
            getattr(lib, fn).argtypes = [ctypes.c_void_p]
            getattr(lib, fn).restype = ctypes.c_int
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = si.config(WORKLOADS[workload])
    T = wl.num_tokens
    sets = []
    for _ in range(2):
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

    def step(i):
        s = sets[i % 2]
        sga.sga_forward(s["batch"], s["q_idx"], s["w"], s["k_idx"], s["k_idx_scale"], s["q_abs"],
                        s["kv"], s["kv_scale"], wl.k, wl.sm_scale, s["gate"], out, lse, idx, ws=ws)

    for i in range(200):
        step(i)
    torch.cuda.synchronize()
    zeros = np.zeros(TL_WORDS, dtype=np.uint64)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    print(f"device timeline: {workload}; the last of {steps} back-to-back forward steps, "
          f"microseconds from the first indexer workgroup's start", flush=True)
    for rep in range(reps):
        for r in TL_RECORDS:
            if getattr(lib, f"sga_tl_clear_{r}")(zeros.ctypes.data) != 0:
                raise SystemExit(f"sga_tl_clear_{r} failed")
        # every step stamps the same slots and points, so the records hold the last step's
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        recs = []
        for r in TL_RECORDS:
            buf = np.zeros(TL_WORDS, dtype=np.uint64)
            if getattr(lib, f"sga_tl_read_{r}")(buf.ctypes.data) != 0:
                raise SystemExit(f"sga_tl_read_{r} failed")
            recs.append(buf)
        print(f"run {rep + 1}:", flush=True)
        for line in timeline_summary(*recs, cus):
            print("  " + line, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200, help="untimed steps first")
    ap.add_argument("--settle-seconds", type=float, default=1.0,
                    help="after the warm-up steps, untimed steps until this much time has "
                         "passed since the first, so the timed steps start at settled clocks")
    ap.add_argument("--workload", default="long_decode_128k", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-two-streams", action="store_true",
                    help="skip the phase with two batches in flight (profiles of single kernels)")
    ap.add_argument("--copies", type=int, default=2, help="input sets alternated between steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of known size (for counter calibration)")
    ap.add_argument("--timeline", action="store_true",
                    help="print the device-clock timeline of a forward step from libsga_timeline.so "
                         "(python -m sparse_gated_mla_amd.build --timeline) instead of the benchmark")
    ap.add_argument("--summarize-pmc", metavar="DIR",
                    help="write the workload's per-kernel counter summary from rocprofv3 runs under DIR")
    args = ap.parse_args()
    if args.summarize_pmc:
        print(json.dumps(summarize_pmc(args.summarize_pmc, args.workload)))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path runs on one GPU with no collectives)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.timeline:
        run_timeline(args.workload, steps=20)
        return
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

    t_settle = time.perf_counter()
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    # time-based settle: the clocks and caches reach their steady state over
    # the first tenths of a second of back-to-back steps, whatever W is
    settle = 0
    while time.perf_counter() - t_settle < args.settle_seconds:
        for _ in range(32):
            step(W + settle)
            settle += 1
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i, tr[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    for i in range(KB):
        step(K + i, tb[i])
    torch.cuda.synchronize()

    two = None if args.no_two_streams else time_two_streams(wl, sets, dev, steps=max(K, 50))
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
    bw = measure_bandwidth(dev)
    ms_per_step = 1e3 * wall / K
    value = T * K / wall
    ib = indexer_bytes(wl)
    idx_avg_s = float(np.mean(idx_ms)) / 1e3
    sb = step_bytes(wl)
    counters = counter_summary(wl.name)
    kc = (counters or {}).get("kernels", {})
    # the forward step's kernels: HBM traffic and MFMA utilisation per launch
    step_counters = {k: {f: e[f] for f in ("traffic_bytes_per_launch", "mfma_util_pct") if f in e}
                     for k, e in kc.items() if in_step(k)}
    mfma_util = {k: e["mfma_util_pct"] for k, e in step_counters.items()
                 if "mfma_util_pct" in e and (k.startswith("indexer") or k.startswith("attn"))}
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
        traffic = [e["traffic_bytes_per_launch"] for k, e in step_counters.items()
                   if k.startswith("indexer_kernel") and "traffic_bytes_per_launch" in e]
        roof = {"bound": "hbm", "kernel": "indexer_kernel", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic[0] if len(traffic) == 1 else None,
                "algorithmic_bytes_per_launch": ib,
                "frac_of_measured_read": round(achieved / bw["stream_read_gbps"], 4)}
    roof["avg_launch_us"] = round(idx_avg_s * 1e6, 2)
    roof["timed_launches"] = len(idx_ms)
    # the whole step against the same peak: every byte the step must move
    roof["step"] = {"achieved": round(sb / (ms_per_step / 1e3) / 1e9, 1), "unit": "GB/s",
                    "frac": round(sb / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
                    "algorithmic_bytes": sb, "us": round(ms_per_step * 1e3, 2)}
    roof["measured_hbm_gbps"] = bw
    roof["mfma_util_pct"] = mfma_util or None
    roof["step_kernel_counters"] = step_counters or None
    roof["counters"] = os.path.relpath(pmc_file(wl.name), ROOT) if counters else None
    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "query-tokens/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": dict(si.describe(wl), parallelism="single GPU"),
        "roofline": roof,
        "extra": {"settle_steps": settle,
                  "step_algorithmic_bytes": sb,
                  "step_gbps": round(sb / (ms_per_step / 1e3) / 1e9, 1),
                  "step_frac_of_hbm_peak": round(sb / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
                  "indexer_us": round(float(np.mean(idx_ms)) * 1e3, 2),
                  "topk_us": round(float(np.mean(topk_ms)) * 1e3, 2),
                  "attention_us": round(float(np.mean(attn_ms)) * 1e3, 2),
                  "input_copies": len(sets),
                  "two_batches_in_flight": two,
                  "cache_append": append,
                  "output_proj": proj,
                  "indexer_loss": loss},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the attention hot path on one MI355X.

A step is one pass of the whole path over resident inputs: the causal GQA
prefill of the headline workload (bf16, B=4, Hq=32, Hkv=8, N=4096, d=128,
[B,N,H,d]) followed by one paged decode step of the long-context workload
(bf16, B=4, Hq=64, Hkv=8, d=128, seq_lens ~ U[98304, 131072], 16-token pages,
permuted block table, split-K + LSE merge).

Prints ONE JSON line. `value` is the prefill throughput in TFLOP/s under the
causal-FLOP count (4 * B * Hq * d * N(N+1)/2 per launch, visible pairs only);
the decode throughput (KV bytes read / time, K+V of every visible token once)
is reported under "decode". Both are timed with HIP events recorded on the
stream the kernels run on. The CPU baseline is the float64 oracle timed on a
bounded sample of the same workloads on the host cores.

Outside the timed step, "chunked_prefill" reports the chunked-prefill pair
on its own workload (bf16, B=4, Hq=32, Hkv=8, d=128, a 2048-token chunk after
a cached prefix of U[6144, 14336] tokens, permuted 16-token pages): the KV
append in GB/s (new K/V rows read once and written once) and the paged
prefill in TFLOP/s (visible (query, key) pairs, 4 d flops each). "variants"
reports the headline prefill with a 1024-token window, 4 initial tokens and
per-head sink logits (TFLOP/s over the visible pairs), and the long-context
decode with an 8192-token window, 4 initial tokens and sink logits (GB/s over
the K/V bytes of the visible tokens). "backward" reports dq, dk, dv of the
headline prefill given an output gradient (TFLOP/s over 5 products of 2 d
flops per visible pair, 2.5 times the forward count). "mla_decode" reports
the absorbed multi-head latent attention decode (B=16, Hq=128, 576-wide latent
rows, L ~ U[8192, 16384]) in GB/s over the latent rows read once.
"configs" times the remaining single-GPU configurations on their own: the
d=64 causal prefill (B=8, Hq=16, N=2048) at Hkv=16 and at Hkv=1 in TFLOP/s,
and the batched decode (B=64, Hq=32, Hkv=8, d=128, 8192 tokens each) in
GB/s, each with its roofline fraction.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]

Before the W warm-up steps the step runs untimed for --settle-ms (default
50 ms; reported in the JSON line as "settle"): under sustained MFMA load the
part's power management needs about 30 ms to settle (in a kernel trace of
this loop after 5 warm-up steps the prefill ran 570-580 us for the first two
launches, 660-710 us for the next few and then fell steadily to 520-523 us
after about 30 ms, while the decode stayed at 281-298 us throughout), so
without it a short warm-up times that transient rather than the steady
state. Every other timed call follows at least 40 ms of untimed calls.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "prefill TFLOP/s (causal GQA fwd) + decode KV-read GB/s, % of MI355X roofline"
CSRC = os.path.join(ROOT, "exact_attention_flashattention_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def causal_flops(B, Hq, N, d) -> int:
    return 4 * B * Hq * d * N * (N + 1) // 2


def kv_bytes(seq_lens, Hkv, d, elem=2) -> int:
    return int(sum(int(L) for L in seq_lens)) * Hkv * d * elem * 2


def chunk_flops(x) -> int:
    """Visible (query, key) pairs of a chunked prefill, 4 * d flops each:
    row i of a chunk of c rows after P cached tokens sees P + i + 1 keys."""
    pairs = 0
    for P, L in zip(x.prefix_lens.tolist(), x.seq_lens.tolist()):
        c = L - P
        pairs += c * P + c * (c + 1) // 2
    return 4 * x.Hq * x.d * pairs


def append_bytes(x) -> int:
    """K and V rows of the new tokens, read once and written once."""
    return x.total_q * x.Hkv * x.d * 2 * 2 * 2


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str, sources) -> float | None:
    """HBM bytes per launch from the committed counter summary, or None when
    the kernel source has changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != source_hash(*sources):
        return None
    return float(rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"])


def cpu_baseline(x2, x5, batches: int):
    """Time the oracle (unchanged) on a bounded sample of both workloads."""
    import numpy as np
    from oracle import attention_oracle as ao
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    nb = max(1, min(x2.B, batches))
    q = ao.to_bhnd(x2.q[:nb], "BNHD")
    k = ao.to_bhnd(x2.k[:nb], "BNHD")
    v = ao.to_bhnd(x2.v[:nb], "BNHD")
    t0 = time.perf_counter()
    ao.sdpa_ref(q, k, v, x2.scale, causal=True)
    tp = time.perf_counter() - t0
    pflops = causal_flops(nb, x2.Hq, x2.N, x2.d)
    pf = pflops / tp / 1e12
    t0 = time.perf_counter()
    ao.decode_ref(x5.q, x5.k_pages, x5.v_pages, x5.block_table, x5.seq_lens, x5.scale)
    td = time.perf_counter() - t0
    dg = kv_bytes(x5.seq_lens.tolist(), x5.Hkv, x5.d) / td / 1e9
    return {
        "value": round(pf, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "sample": f"prefill: batch entries 0..{nb - 1} (all {x2.Hq} query heads, full N={x2.N}) of the "
                  f"headline prefill, causal-FLOP count {pflops}, in {tp:.2f} s; decode: all {x5.B} "
                  f"sequences of the paged decode ({kv_bytes(x5.seq_lens.tolist(), x5.Hkv, x5.d)} KV bytes) "
                  f"in {td:.2f} s",
        "decode_value": round(dg, 4), "decode_unit": "GB/s",
        "blas": "OpenBLAS (numpy)",
    }


def time_calls(fn, stream, warmup: int, steps: int, settle_ms: float = 40.0) -> float:
    """Average microseconds per call from HIP events on ``stream``, after at
    least ``warmup`` untimed calls and at least ``settle_ms`` of them (the
    clocks settle over the first tens of milliseconds of sustained load)."""
    import torch
    n, t0 = 0, time.perf_counter()
    while n < warmup or (time.perf_counter() - t0) * 1e3 < settle_ms:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / steps


def chunked_setup(dev, stream):
    """Resident inputs of the chunked-prefill workload and its two calls."""
    import torch
    import exact_attention_flashattention_amd as pkg
    from exact_attention_flashattention_amd import workloads as wl
    x = wl.workload_6()
    q, kn, vn = x.q.to(dev), x.k_new.to(dev), x.v_new.to(dev)
    kp, vp = x.k_pages.to(dev), x.v_pages.to(dev)
    bt, cu, start, lens = (t.to(dev) for t in (x.block_table, x.cu_q, x.prefix_lens, x.seq_lens))
    o = torch.empty_like(q)
    append = lambda: pkg.attn_kv_append(kn, vn, kp, vp, bt, cu, start, max_new=x.max_q_len, stream=stream)
    attend = lambda: pkg.attn_prefill_paged(q, kp, vp, bt, cu, lens, o, max_q_len=x.max_q_len,
                                            scale=x.scale, stream=stream)
    append()
    torch.cuda.synchronize()
    return x, append, attend


def chunked_report(dev, stream, steps: int) -> dict:
    """The chunked-prefill pair (KV append, then paged prefill), timed apart
    from the step: it widens the path and is not part of `value`."""
    x, append, attend = chunked_setup(dev, stream)
    t_app = time_calls(append, stream, 3, steps)
    t_att = time_calls(attend, stream, 3, steps)
    fl = chunk_flops(x)
    tf = fl / (t_att * 1e-6) / 1e12
    by = append_bytes(x)
    gb = by / (t_app * 1e-6) / 1e9
    log(f"chunked: append {t_app:.1f} us ({gb:.0f} GB/s), paged prefill {t_att:.1f} us ({tf:.1f} TFLOP/s)")
    return {
        "workload": x.name, "seq_lens": x.seq_lens.tolist(), "prefix_lens": x.prefix_lens.tolist(),
        "paged_prefill": {"value": round(tf, 3), "unit": "TFLOP/s", "avg_launch_us": round(t_att, 2),
                          "flops_per_launch": fl,
                          "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": BF16_PEAK_TFLOPS,
                                       "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                                       "traffic": measured_traffic("prefill_paged", PREFILL_SOURCES),
                                       "kernel": "prefill_bf16_kernel<128,8,64,paged>"}},
        "kv_append": {"value": round(gb, 2), "unit": "GB/s", "avg_launch_us": round(t_app, 2),
                      "bytes_per_launch": by,
                      "roofline": {"bound": "hbm", "achieved": round(gb, 2), "peak": HBM_PEAK_GBS,
                                   "unit": "GB/s", "frac": round(gb / HBM_PEAK_GBS, 4),
                                   "traffic": measured_traffic("kv_append", APPEND_SOURCES),
                                   "kernel": "kv_append_kernel"}},
    }


def c3_setup(dev, stream, hkv: int):
    """The d=64 causal prefill (B=8, Hq=16, N=2048) with Hkv=16 (MHA) or 1 (MQA)."""
    import torch
    import exact_attention_flashattention_amd as pkg
    from exact_attention_flashattention_amd import workloads as wl
    x = wl.workload_3(hkv)
    q, k, v = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    o = torch.empty_like(q)
    fn = lambda: pkg.attn_prefill(q, k, v, o, scale=x.scale, stream=stream)
    torch.cuda.synchronize()
    return x, fn


def c4_setup(dev, stream):
    """The batched decode (B=64, Hq=32, Hkv=8, d=128, 8192 tokens each)."""
    import torch
    import exact_attention_flashattention_amd as pkg
    from exact_attention_flashattention_amd import workloads as wl
    x = wl.workload_4()
    t = [a.to(dev) for a in (x.q, x.k_pages, x.v_pages, x.block_table, x.seq_lens)]
    o = torch.empty_like(t[0])
    splits = pkg.attn_decode_num_splits(x.B, x.Hkv, x.max_pages_per_seq, 0)
    ws = torch.empty(pkg.attn_decode_workspace_size(x.B, x.Hq, x.Hkv, x.d, x.max_pages_per_seq, 0) // 4 + 4,
                     dtype=torch.float32, device=dev)
    fn = lambda: pkg.attn_decode(*t, o, scale=x.scale, num_splits=splits, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    return x, fn, splits


def configs_report(dev, stream, steps: int) -> dict:
    """The other single-GPU configurations, each timed on its own with HIP
    events: the d=64 prefill at Hkv=16 and Hkv=1, and the batched decode."""
    out = {}
    for hkv in (16, 1):
        x, fn = c3_setup(dev, stream, hkv)
        t = time_calls(fn, stream, 3, steps)
        fl = causal_flops(x.B, x.Hq, x.N, x.d)
        tf = fl / (t * 1e-6) / 1e12
        log(f"config 3 (Hkv={hkv}): prefill {t:.1f} us ({tf:.1f} TFLOP/s)")
        out[f"prefill_d64_hkv{hkv}"] = {
            "workload": x.name, "value": round(tf, 3), "unit": "TFLOP/s", "avg_launch_us": round(t, 2),
            "flops_per_launch": fl,
            "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic(f"prefill_d64_hkv{hkv}", PREFILL_SOURCES),
                         "kernel": "prefill_bf16_kernel<64,8,32>"}}
        del fn
    x, fn, splits = c4_setup(dev, stream)
    t = time_calls(fn, stream, 3, steps)
    by = kv_bytes(x.seq_lens.tolist(), x.Hkv, x.d)
    gb = by / (t * 1e-6) / 1e9
    log(f"config 4: batched decode {t:.1f} us ({gb:.0f} GB/s)")
    out["decode_batched"] = {
        "workload": x.name, "value": round(gb, 2), "unit": "GB/s", "avg_call_us": round(t, 2),
        "kv_bytes_per_call": by, "num_splits": splits,
        "roofline": {"bound": "hbm", "achieved": round(gb, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gb / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("decode_batched", DECODE_SOURCES),
                     "kernel": "decode_split_kernel<128> + decode_merge_kernel<128>"}}
    return out


def window_pairs(N: int, W: int, n_sink: int = 0) -> int:
    """Visible (query, key) pairs of causal self-attention with a window W
    and n_sink initial positions kept: row i sees min(i+1, W) window keys
    plus the anchors before its window."""
    pairs = 0
    for i in range(N):
        lo = max(i - W + 1, 0)
        pairs += (i + 1 - lo) + min(n_sink, lo)
    return pairs


def variants_report(dev, stream, steps: int) -> dict:
    """Sliding window + initial tokens + learned sink logits on the headline
    prefill shape and the long-context decode, timed apart from the step."""
    import torch
    import exact_attention_flashattention_amd as pkg
    from exact_attention_flashattention_amd import workloads as wl
    W, S = 1024, 4
    x2 = wl.workload_2()
    q, k, v = x2.q.to(dev), x2.k.to(dev), x2.v.to(dev)
    o = torch.empty_like(q)
    sinks = torch.linspace(-1.0, 3.0, x2.Hq, device=dev, dtype=torch.float32)
    pre = lambda: pkg.attn_prefill_ex(q, k, v, o, scale=x2.scale, window=W, n_sink=S, sinks=sinks,
                                      stream=stream)
    t_pre = time_calls(pre, stream, 3, steps)
    fl = 4 * x2.B * x2.Hq * x2.d * window_pairs(x2.N, W, S)
    tf = fl / (t_pre * 1e-6) / 1e12
    del q, k, v, o
    x5 = wl.workload_5()
    Wd = 8192
    t = [a.to(dev) for a in (x5.q, x5.k_pages, x5.v_pages, x5.block_table, x5.seq_lens)]
    do = torch.empty_like(t[0])
    dsinks = torch.linspace(-1.0, 3.0, x5.Hq, device=dev, dtype=torch.float32)
    ws = torch.empty(pkg.attn_decode_workspace_size(x5.B, x5.Hq, x5.Hkv, x5.d, x5.max_pages_per_seq, 0) // 4 + 4,
                     dtype=torch.float32, device=dev)
    dec = lambda: pkg.attn_decode_ex(*t, do, scale=x5.scale, window=Wd, n_sink=S, sinks=dsinks, workspace=ws,
                                     stream=stream)
    t_dec = time_calls(dec, stream, 3, steps)
    # K+V bytes of the visible tokens (window + anchors) once
    vis = sum(min(int(L), Wd) + min(S, max(int(L) - Wd, 0)) for L in x5.seq_lens.tolist())
    by = vis * x5.Hkv * x5.d * 2 * 2
    gb = by / (t_dec * 1e-6) / 1e9
    log(f"variants: windowed prefill {t_pre:.1f} us ({tf:.1f} TFLOP/s), windowed decode {t_dec:.1f} us "
        f"({gb:.0f} GB/s)")
    return {
        "prefill": {"workload": f"{x2.name} window={W} n_sink={S} sinks=per-head", "value": round(tf, 3),
                    "unit": "TFLOP/s", "avg_launch_us": round(t_pre, 2), "flops_per_launch": fl,
                    "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": BF16_PEAK_TFLOPS,
                                 "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4)}},
        "decode": {"workload": f"{x5.name} window={Wd} n_sink={S} sinks=per-head", "value": round(gb, 2),
                   "unit": "GB/s", "avg_call_us": round(t_dec, 2), "kv_bytes_per_call": by,
                   "roofline": {"bound": "hbm", "achieved": round(gb, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(gb / HBM_PEAK_GBS, 4)}},
    }


def backward_setup(dev, stream):
    """The headline prefill's inputs, its forward output and LSE, an output
    gradient, and the backward call."""
    import torch
    import exact_attention_flashattention_amd as pkg
    from exact_attention_flashattention_amd import workloads as wl
    x = wl.workload_2()
    q, k, v = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    do = wl.output_gradient(x, seed=144).to(dev)
    lse = torch.empty((x.B, x.Hq, x.N), dtype=torch.float32, device=dev)
    o = pkg.attn_prefill_ex(q, k, v, scale=x.scale, lse=lse, stream=stream)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(pkg.attn_backward_workspace_size(x.B, x.N, x.Hq) // 4 + 4, dtype=torch.float32, device=dev)
    fn = lambda: pkg.attn_backward(q, k, v, o, do, lse, dq, dk, dv, scale=x.scale, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    return x, fn


def backward_report(dev, stream, steps: int) -> dict:
    """dq, dk, dv of the headline prefill, timed apart from the step."""
    x, fn = backward_setup(dev, stream)
    t = time_calls(fn, stream, 3, steps)
    fl = 5 * causal_flops(x.B, x.Hq, x.N, x.d) // 2   # 5 products of 2 d flops per visible pair
    tf = fl / (t * 1e-6) / 1e12
    log(f"backward: {t:.1f} us ({tf:.1f} TFLOP/s)")
    return {"workload": f"{x.name}, dq/dk/dv given dO", "value": round(tf, 3), "unit": "TFLOP/s",
            "avg_call_us": round(t, 2), "flops_per_call": fl,
            "kernels": "bwd_dq_kernel<128,8,64> + bwd_dkdv_kernel<128,4,64>",
            "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic("backward", BACKWARD_SOURCES)}}


def mla_setup(dev, stream):
    import torch
    import exact_attention_flashattention_amd as pkg
    from exact_attention_flashattention_amd import workloads as wl
    x = wl.workload_7()
    q, kv, bt, sl = (t.to(dev) for t in (x.q, x.kv_pages, x.block_table, x.seq_lens))
    o = torch.empty((x.B, x.Hq, x.d_c), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(pkg.attn_decode_mla_workspace_size(x.B, x.Hq, x.max_pages_per_seq, 0) // 4 + 4,
                     dtype=torch.float32, device=dev)
    fn = lambda: pkg.attn_decode_mla(q, kv, bt, sl, o, scale=x.scale, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    return x, fn


def mla_report(dev, stream, steps: int) -> dict:
    """Absorbed-MLA decode: latent rows read once (K and V share them)."""
    import exact_attention_flashattention_amd as pkg
    x, fn = mla_setup(dev, stream)
    t = time_calls(fn, stream, 3, steps)
    by = int(x.seq_lens.sum()) * (x.d_c + x.d_r) * 2
    gb = by / (t * 1e-6) / 1e9
    fl = int(x.seq_lens.sum()) * x.Hq * 2 * (2 * x.d_c + x.d_r)
    log(f"mla decode: {t:.1f} us ({gb:.0f} GB/s, {fl / (t * 1e-6) / 1e12:.1f} TFLOP/s)")
    return {"workload": x.name, "seq_lens": x.seq_lens.tolist(),
            "splits": pkg.attn_decode_mla_num_splits(x.B, x.Hq, x.max_pages_per_seq, 0),
            "value": round(gb, 2), "unit": "GB/s", "avg_call_us": round(t, 2), "kv_bytes_per_call": by,
            "tflops": round(fl / (t * 1e-6) / 1e12, 3),
            "kernels": "mla_split_kernel + mla_merge_kernel",
            "roofline": {"bound": "hbm", "achieved": round(gb, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gb / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("decode_mla", MLA_SOURCES)}}


PREFILL_SOURCES = ["prefill_bf16.hip", "attn_internal.h", "cdna4.h"]
DECODE_SOURCES = ["decode.hip", "attn_internal.h"]
APPEND_SOURCES = ["kv_append.hip", "attn_internal.h"]
BACKWARD_SOURCES = ["backward_bf16.hip", "attn_internal.h", "cdna4.h"]
MLA_SOURCES = ["decode_mla.hip", "attn_internal.h", "cdna4.h"]


def write_traffic(root: str) -> int:
    """Turn rocprofv3 --pmc CSVs into profiles/traffic.json (no GPU needed).

    Expects <root>/<COUNTER>_<kind>/**/*counter_collection.csv for COUNTER in
    FETCH_SIZE, WRITE_SIZE and kind in prefill, decode, chunked, append,
    backward, mla, c3_16, c3_1, c4, copy,
    as written by
        rocprofv3 --pmc <COUNTER> -d <root>/<COUNTER>_<kind> -o run --output-format csv \
            -- python bench.py --only <kind> --steps 3 --warmup 1 > <root>/<COUNTER>_<kind>.log
    Each counter (KiB per dispatch) is scaled by the ratio between the bytes a
    plain 1 GiB device copy moves and what the same counter reports for it.
    The kernel source hash each run printed into its .log must match the
    current source, else nothing is written.
    """
    import csv
    import glob

    def per_dispatch(counter, kind, name_part):
        vals = []
        for f in glob.glob(os.path.join(root, f"{counter}_{kind}", "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
                    vals.append(float(r["Counter_Value"]) * 1024.0)
        if not vals:
            raise SystemExit(f"no {counter} rows for {name_part} under {root}")
        return sum(vals) / len(vals)

    copy_bytes = float(1 << 30)
    fetch_factor = copy_bytes / per_dispatch("FETCH_SIZE", "copy", "copyBuffer")
    write_factor = copy_bytes / per_dispatch("WRITE_SIZE", "copy", "copyBuffer")
    out = {"calibration": {"copy_bytes_each_way": copy_bytes, "fetch_factor": round(fetch_factor, 4),
                           "write_factor": round(write_factor, 4)}}
    for key, kind, parts, srcs in [("prefill_bf16", "prefill", ["prefill_bf16_kernel"], PREFILL_SOURCES),
                                   ("decode", "decode", ["decode_split_kernel", "decode_merge_kernel"],
                                    DECODE_SOURCES),
                                   ("prefill_paged", "chunked", ["prefill_bf16_kernel"], PREFILL_SOURCES),
                                   ("kv_append", "append", ["kv_append_kernel"], APPEND_SOURCES),
                                   ("backward", "backward", ["bwd_dq_kernel", "bwd_dkdv_kernel"],
                                    BACKWARD_SOURCES),
                                   ("decode_mla", "mla", ["mla_split_kernel", "mla_merge_kernel"], MLA_SOURCES),
                                   ("prefill_d64_hkv16", "c3_16", ["prefill_bf16_kernel"], PREFILL_SOURCES),
                                   ("prefill_d64_hkv1", "c3_1", ["prefill_bf16_kernel"], PREFILL_SOURCES),
                                   ("decode_batched", "c4", ["decode_split_kernel", "decode_merge_kernel"],
                                    DECODE_SOURCES)]:
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            ran = None
            with open(os.path.join(root, f"{counter}_{kind}.log")) as f:
                for line in f:
                    if line.startswith('{"only"'):
                        ran = json.loads(line).get("source_sha256")
            if ran != source_hash(*srcs):
                raise SystemExit(f"{counter}_{kind}: counters were taken from another kernel source")
        fetch = sum(per_dispatch("FETCH_SIZE", kind, n) for n in parts) * fetch_factor
        write = sum(per_dispatch("WRITE_SIZE", kind, n) for n in parts) * write_factor
        out[key] = {"source_sha256": source_hash(*srcs), "kernels": parts,
                    "fetch_bytes_per_launch": round(fetch), "write_bytes_per_launch": round(write)}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))
    return 0


def only(args, dev) -> int:
    """Launch one kernel kind warmup + steps times and report its event time."""
    import torch
    import exact_attention_flashattention_amd as pkg
    from exact_attention_flashattention_amd import workloads as wl
    stream = torch.cuda.current_stream()
    if args.only == "prefill":
        x = wl.workload_2()
        q, k, v = x.q.to(dev), x.k.to(dev), x.v.to(dev)
        o = torch.empty_like(q)
        fn = lambda: pkg.attn_prefill(q, k, v, o, scale=x.scale, stream=stream)
        work = {"flops_per_launch": causal_flops(x.B, x.Hq, x.N, x.d)}
    elif args.only in ("c3_16", "c3_1"):
        x, fn = c3_setup(dev, stream, 16 if args.only == "c3_16" else 1)
        work = {"flops_per_launch": causal_flops(x.B, x.Hq, x.N, x.d)}
    elif args.only == "c4":
        x, fn, _ = c4_setup(dev, stream)
        work = {"kv_bytes_per_call": kv_bytes(x.seq_lens.tolist(), x.Hkv, x.d)}
    elif args.only == "mla":
        x, fn = mla_setup(dev, stream)
        work = {"kv_bytes_per_call": int(x.seq_lens.sum()) * (x.d_c + x.d_r) * 2}
    elif args.only == "backward":
        x, fn = backward_setup(dev, stream)
        work = {"flops_per_call": 5 * causal_flops(x.B, x.Hq, x.N, x.d) // 2}
    elif args.only in ("chunked", "append"):
        x, append, attend = chunked_setup(dev, stream)
        fn = attend if args.only == "chunked" else append
        work = ({"flops_per_launch": chunk_flops(x)} if args.only == "chunked"
                else {"bytes_per_launch": append_bytes(x)})
    elif args.only == "decode":
        x = wl.workload_5()
        t = [a.to(dev) for a in (x.q, x.k_pages, x.v_pages, x.block_table, x.seq_lens)]
        o = torch.empty_like(t[0])
        splits = pkg.attn_decode_num_splits(x.B, x.Hkv, x.max_pages_per_seq, 0)
        ws = torch.empty(pkg.attn_decode_workspace_size(x.B, x.Hq, x.Hkv, x.d, x.max_pages_per_seq, 0) // 4 + 4,
                         dtype=torch.float32, device=dev)
        fn = lambda: pkg.attn_decode(*t, o, scale=x.scale, num_splits=splits, workspace=ws, stream=stream)
        work = {"kv_bytes_per_call": kv_bytes(x.seq_lens.tolist(), x.Hkv, x.d)}
    else:
        n = 1 << 29  # 2**29 bf16 = 1 GiB read + 1 GiB written per launch
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        fn = lambda: dst.copy_(src)
        work = {"bytes_read_per_launch": 2 * n, "bytes_written_per_launch": 2 * n}
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(args.steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    srcs = {"prefill": PREFILL_SOURCES, "decode": DECODE_SOURCES, "chunked": PREFILL_SOURCES,
            "append": APPEND_SOURCES, "backward": BACKWARD_SOURCES, "mla": MLA_SOURCES,
            "c3_16": PREFILL_SOURCES, "c3_1": PREFILL_SOURCES, "c4": DECODE_SOURCES}.get(args.only)
    print(json.dumps({"only": args.only, "steps": args.steps,
                      "avg_us": round(a.elapsed_time(b) * 1e3 / args.steps, 2),
                      "source_sha256": source_hash(*srcs) if srcs else None, **work}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=50.0,
                    help="untimed steps for this long before the warm-up steps (clocks settle)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-chunked", action="store_true",
                    help="skip the chunked-prefill (KV append + paged prefill) and variant reports")
    ap.add_argument("--cpu-batches", type=int, default=2,
                    help="batch entries of the headline prefill the CPU oracle is timed on")
    ap.add_argument("--only", choices=["prefill", "decode", "copy", "chunked", "append", "backward", "mla",
                                       "c3_16", "c3_1", "c4"],
                    default=None,
                    help="launch only this kernel (for counter runs under rocprofv3); "
                         "'copy' is a plain 1 GiB device copy used to calibrate byte counters")
    ap.add_argument("--write-traffic", metavar="DIR", default=None,
                    help="parse rocprofv3 FETCH_SIZE/WRITE_SIZE runs under DIR into profiles/traffic.json")
    args = ap.parse_args()
    if args.write_traffic:
        return write_traffic(args.write_traffic)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the kernels would shard over (batch, KV head) with no exchange)",
              file=sys.stderr)
        return 2

    import torch
    import exact_attention_flashattention_amd as pkg
    from exact_attention_flashattention_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    pkg.lib()
    dev = torch.device("cuda:0")
    if args.only:
        return only(args, dev)

    log("generating inputs ...")
    x2 = wl.workload_2()
    x5 = wl.workload_5()
    q, k, v = x2.q.to(dev), x2.k.to(dev), x2.v.to(dev)
    o = torch.empty_like(q)
    dq, dk, dv = x5.q.to(dev), x5.k_pages.to(dev), x5.v_pages.to(dev)
    dbt, dsl = x5.block_table.to(dev), x5.seq_lens.to(dev)
    do = torch.empty_like(dq)
    ws_bytes = pkg.attn_decode_workspace_size(x5.B, x5.Hq, x5.Hkv, x5.d, x5.max_pages_per_seq, 0)
    ws = torch.empty(ws_bytes // 4 + 4, dtype=torch.float32, device=dev)
    splits = pkg.attn_decode_num_splits(x5.B, x5.Hkv, x5.max_pages_per_seq, 0)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def step(evs=None):
        if evs is not None:
            evs[0].record(stream)
        pkg.attn_prefill(q, k, v, o, scale=x2.scale, stream=stream)
        if evs is not None:
            evs[1].record(stream)
        pkg.attn_decode(dq, dk, dv, dbt, dsl, do, scale=x5.scale, num_splits=splits, workspace=ws,
                        stream=stream)
        if evs is not None:
            evs[2].record(stream)

    n_settle, t_settle = 0, time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        step()
        n_settle += 1
        if n_settle % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    log(f"settle {n_settle} untimed steps ({settle_ms:.0f} ms), warmup {args.warmup} ...")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(end)
    pre_ms = [e[0].elapsed_time(e[1]) for e in evs]
    dec_ms = [e[1].elapsed_time(e[2]) for e in evs]
    pre_avg = sum(pre_ms) / len(pre_ms)
    dec_avg = sum(dec_ms) / len(dec_ms)

    flops = causal_flops(x2.B, x2.Hq, x2.N, x2.d)
    tflops = flops / (pre_avg * 1e-3) / 1e12
    kvb = kv_bytes(x5.seq_lens.tolist(), x5.Hkv, x5.d)
    gbs = kvb / (dec_avg * 1e-3) / 1e9
    log(f"prefill avg {pre_avg * 1e3:.1f} us ({tflops:.1f} TFLOP/s, min {min(pre_ms) * 1e3:.1f} us); "
        f"decode avg {dec_avg * 1e3:.1f} us ({gbs} GB/s); wall {t_wall:.3f} s")

    traffic = measured_traffic("prefill_bf16", PREFILL_SOURCES)
    dtraffic = measured_traffic("decode", DECODE_SOURCES)
    result = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"untimed_steps": n_settle, "ms": round(settle_ms, 1),
                   "why": "steps run untimed before the warm-up until the clocks settle under sustained load"},
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": x2.name,
            "B": x2.B, "N": x2.N, "Hq": x2.Hq, "Hkv": x2.Hkv, "d": x2.d, "causal": True,
            "layout": "BNHD", "flops_per_launch": flops,
            "decode_workload": x5.name,
            "decode_seq_lens": x5.seq_lens.tolist(), "decode_num_splits": splits,
            "step": "one prefill launch + one decode call (split kernel + merge kernel)",
        },
        "roofline": {
            "bound": "mfma", "achieved": round(tflops, 3), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "kernel": "prefill_bf16_kernel<128,8,64>", "avg_launch_us": round(pre_avg * 1e3, 2),
        },
        "decode": {
            "value": round(gbs, 2), "unit": "GB/s", "avg_call_us": round(dec_avg * 1e3, 2),
            "kv_bytes_per_call": kvb,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": dtraffic,
                         "kernel": "decode_split_kernel<128> + decode_merge_kernel<128>"},
        },
        "chunked_prefill": None,
        "variants": None,
        "backward": None,
        "mla_decode": None,
        "configs": None,
        "cpu_baseline": None,
    }
    if not args.no_chunked:
        result["chunked_prefill"] = chunked_report(dev, stream, max(10, args.steps // 2))
        result["variants"] = variants_report(dev, stream, max(10, args.steps // 2))
        result["backward"] = backward_report(dev, stream, max(10, args.steps // 5))
        result["mla_decode"] = mla_report(dev, stream, max(10, args.steps // 2))
    result["configs"] = configs_report(dev, stream, max(10, args.steps // 2))
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(x2, x5, args.cpu_batches)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

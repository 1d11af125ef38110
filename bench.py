"""Benchmark of the Ulysses per-rank hot path on one MI355X.

A step is one pass of the whole path over one rank's share of a layer:
pack Q, K, V (seq->head send side), head-sharded attention over the whole
sequence, and the output's head->seq exchange.  The first all-to-all itself
is not part of a one-GPU step: the rank's own send buffer stands in for its
receive buffer (same shape, [s, b, h/P, d]), so the attention consumes the
pack's output.  For bf16 the attention writes its output rows straight into
the P destination shards (ulys_attn_fwd_push: the O exchange and unpack in
its epilogue; the destinations are P buffers on this GPU); fp32 runs the
attention and then the unpack.  The pack and unpack kernels are also timed
alone, streaming from HBM (layout_hbm).

Before any timed step the GPU runs untimed steps until its clock has
settled (a minimum wall time, then two consecutive runs of steps agreeing
to 1%), whatever --warmup says: the board lowers its clock under sustained
matrix-core load within the first seconds, so a few warm-up steps would time
a clock that is still falling.

The headline workload is the 128K MHA share (the largest share the
throughput targets bind); the 32K GPT share and the 64K GQA share are timed
the same way and reported as sub-records under "configs".

Prints ONE JSON line.  ``value`` is attention FLOPs per step over the whole
step time (TFLOP/s); per-kernel durations come from HIP events recorded on
the stream the kernels run on, inside the timed region (mean, median and min
over the timed steps).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn TFLOP/s (% bf16 MFMA peak) + pack/unpack GB/s (% HBM peak), 1 GPU"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3    # MI355X fp32 vector
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
PROFILE_DIR = os.path.join(ROOT, "profiles")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mha-128k")
    ap.add_argument("--also", default="gpt1.2b-32k,gqa-64k",
                    help="comma-separated workloads timed after the headline one and reported "
                         "under 'configs' ('' for none)")
    ap.add_argument("--settle-seconds", type=float, default=2.0,
                    help="minimum wall time of untimed steps before any timed ones")
    ap.add_argument("--settle-max-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-time budget of the oracle's cpu_baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--merge-steps", type=int, default=50,
                    help="timed ulys_attn_merge calls on the share (one ring step's merge of "
                         "two partial results), reported under 'merge'; 0 skips them")
    ap.add_argument("--push-steps", type=int, default=20,
                    help="timed pushes of the Q shard into P share buffers on this GPU "
                         "(ulys_seq2head_push), reported under 'exchange_push'; 0 skips them")
    ap.add_argument("--layout-calls", type=int, default=64,
                    help="pack and unpack calls over rotating buffer sets of >= 2 GiB, "
                         "reported under 'layout_hbm'; 0 skips them")
    ap.add_argument("--push-attn-calls", type=int, default=50,
                    help="timed calls of the attention with the O exchange in its epilogue "
                         "(ulys_attn_fwd_push) and of attention + unpack, reported under "
                         "'attn_push'; 0 skips them")
    ap.add_argument("--bwd-steps", type=int, default=100,
                    help="timed backward steps (pack dO, attention backward, unpack dQ, dK, "
                         "dV) reported under 'backward'; 0 skips them")
    ap.add_argument("--inputs", choices=("normal", "constant"), default="normal",
                    help="normal: the seeded N(0,1) tensors (the workload); constant: the "
                         "same work on constant tensors, a diagnostic of how much the GPU "
                         "clock depends on the data the matrix cores see (not a result)")
    ap.add_argument("--layout-sweep", action="store_true",
                    help="only time the fused Q/K/V pack and the O unpack from HBM over shard "
                         "sizes of the 32K share's head layout (s from 8192 to 262144) and fit "
                         "time = fixed + bytes / bandwidth; prints one JSON line and exits")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device-to-device copy of known size (for scaling "
                         "rocprofv3 FETCH_SIZE/WRITE_SIZE to bytes) and exit")
    return ap.parse_args()


def copy_calibration():
    """Three plain copies of a 1 GiB buffer; the copy kernel reads and writes
    exactly 1 GiB per dispatch, the yardstick for the HBM byte counters."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(7)
    dst = torch.empty_like(src)
    evict = torch.empty_like(src)
    for _ in range(3):
        evict.fill_(1)  # 1 GiB of other writes push src out of L2 and the 256 MiB MALL
        torch.cuda.synchronize()
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_dispatch": n}), flush=True)


def layout_sweep(args):
    """The layout kernels' time against their size: the fused Q/K/V pack and
    the O unpack of the 32K share's head layout (h = 16, P = 8, d = 128, bf16)
    at s = 8192 .. 262144, each streaming from HBM (rotating buffer sets of at
    least 2 GiB), and a least-squares fit time = fixed + bytes / bandwidth.
    A fixed cost that is large against the 32K share's time shows that kernel
    is bound by its launch and drain rather than by HBM bandwidth."""
    import numpy as np
    import torch

    from ulysses_head_sharded_amd import binding
    from ulysses_head_sharded_amd.workloads import Workload

    binding.load()
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream()
    sh = st.cuda_stream
    rows = []
    for s in (8192, 16384, 32768, 65536, 131072, 262144):
        w = Workload("sweep", 2, 8, s, 1, 16, 16, 128, "bf16", True, "")
        args.layout_calls = 64
        r = bench_layout_hbm(args, w, binding, torch, torch.bfloat16, binding.ULYS_BF16, st)
        pack_b = 2 * w.shard_bytes() + 2 * (w.shard_bytes(kv=True) + w.kv_blocks_bytes())
        rows.append({"s": s, "pack_qkv_bytes": pack_b, "pack_qkv_us": r["pack_qkv_us"],
                     "pack_gbps": r["pack_gbps"], "unpack_o_bytes": 2 * w.shard_bytes(),
                     "unpack_o_us": r["unpack_o_us"], "unpack_gbps": r["unpack_gbps"]})
        torch.cuda.empty_cache()
    fit = {}
    for kind in ("pack_qkv", "unpack_o"):
        x = np.array([r[f"{kind}_bytes"] for r in rows], dtype=np.float64)
        y = np.array([r[f"{kind}_us"] for r in rows], dtype=np.float64)
        slope, fixed = np.polyfit(x, y, 1)
        fit[kind] = {"fixed_us": round(float(fixed), 2),
                     "steady_gbps": round(float(1e-3 / slope), 1),
                     "steady_frac_hbm_peak": round(float(1e-3 / slope) / PEAK_HBM_GBPS, 4)}
    print(json.dumps({"layout_sweep": rows, "fit": fit,
                      "shape": "h=16, P=8, d_h=128, b=1, bf16 (the 32K share's layout)"}), flush=True)


def source_digest(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def counter_traffic(kernel_src: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, or None
    when none exist or the kernel source changed since they were taken."""
    path = os.path.join(PROFILE_DIR, f"attn_bf16_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path, encoding="utf-8") as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                key = key.strip()
                if key == "kernel" and "kernel" in fields:
                    break  # only the first section describes the attention call
                fields[key] = val.strip()
    if fields.get("source_sha256") != source_digest(kernel_src):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, q, k, v, budget_s: float):
    """The oracle, as it stands, on a bounded sample of the same share: random
    query rows in batches until the wall-time budget is spent."""
    import numpy as np

    import oracle
    from ulysses_head_sharded_amd import synth

    threads = oracle.default_threads()
    u = synth.uniform01(100 * w.c + 7, 1 << 16)
    flops, rows_done, t_used, idx = 0.0, 0, 0.0, 0
    batch = max(threads, 16)
    while t_used < budget_s and idx + batch <= u.size:
        sel = u[idx:idx + batch]
        idx += batch
        t = np.minimum((sel * w.s).astype(np.int64), w.s - 1)
        rows = np.stack([np.zeros_like(t), (np.arange(t.size) % w.hp), t], axis=1)
        keys = (t + 1) if w.causal else np.full_like(t, w.s)
        t0 = time.perf_counter()
        oracle.attn_rows(q, k, v, rows, w.s, w.b, w.h, w.h_kv, w.d, w.P, w.causal,
                         nthreads=threads)
        t_used += time.perf_counter() - t0
        flops += float(4 * w.d * keys.sum())
        rows_done += t.size
    # the layout oracle (orc_pack, one thread) on one rank-local shard of the
    # workload's Q ([s/P, b, h, d]: as many elements as the share; the share's
    # bits serve as its contents, the pack only moves them)
    x = np.ascontiguousarray(q).reshape(w.s // w.P, w.b, w.h, w.d)
    nbytes = x.nbytes
    reps, t_lay = 0, 0.0
    while t_lay < min(2.0, budget_s) and reps < 50:
        t0 = time.perf_counter()
        oracle.pack(x, w.s, w.b, w.h, w.d, w.P)
        t_lay += time.perf_counter() - t0
        reps += 1
    return {
        "value": flops / t_used / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": f"{rows_done} uniformly drawn query rows of the {w.name} share the GPU "
                  f"attends over (fp64 oracle, {t_used:.1f} s wall, algorithmic flops of the "
                  f"sample)",
        "layout": {"value": 2.0 * nbytes * reps / t_lay / 1e9, "unit": "GB/s", "cores": 1,
                   "kind": "oracle",
                   "sample": f"orc_pack of one {size_text(nbytes)} rank-local Q shard of "
                             f"{w.name}, {reps} calls in {t_lay:.2f} s (bytes read + written)"},
    }


def size_text(nbytes: int) -> str:
    """A byte count in MiB, or KiB below one MiB."""
    return f"{nbytes / 2**20:.0f} MiB" if nbytes >= 2**20 else f"{nbytes / 2**10:.0f} KiB"


def cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def settle(torch, run, min_s: float, max_s: float, tol: float = 0.01):
    """Untimed steps until the GPU clock has settled: runs of steps lasting
    about a quarter of a second each, for at least min_s seconds and until two
    consecutive runs agree on the time per step to within tol (at most max_s
    seconds).  run(n) enqueues n steps.  Returns (seconds spent, steps run,
    ms per step of the last run)."""
    t_start = time.perf_counter()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(1)
    torch.cuda.synchronize()
    per = max(time.perf_counter() - t0, 1e-5)
    steps, prev = 1, None
    while True:
        n = max(1, int(0.25 / per))
        t0 = time.perf_counter()
        run(n)
        torch.cuda.synchronize()
        per = (time.perf_counter() - t0) / n
        steps += n
        spent = time.perf_counter() - t_start
        if spent >= max_s:
            break
        if prev is not None and spent >= min_s and abs(per - prev) <= tol * prev:
            break
        prev = per
    return spent, steps, per * 1e3


def stats_ms(xs):
    """mean, median and min of per-step event windows (ms)."""
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"mean": float(a.mean()), "median": float(np.median(a)), "min": float(a.min())}


def bench_merge(args, w, binding, torch, np, o, code, stream):
    """ulys_attn_merge of two partial results of the share (O [s, b, hp, d] in the
    workload's dtype, lse [b, hp, s] fp32), accumulating in place as a ring step
    does.  HBM-bound: 3 O tensors and 3 lse tensors move per call."""
    s, b, hp, d = w.s, w.b, w.hp, w.d
    o_a = o.clone()
    o_b = o.flip(0).contiguous()
    lse_a = torch.zeros((b, hp, s), dtype=torch.float32, device=o.device)
    lse_b = torch.full((b, hp, s), -0.5, dtype=torch.float32, device=o.device)
    sh = stream.cuda_stream

    def call():
        rc = binding.ulys_attn_merge(o_a.data_ptr(), lse_a.data_ptr(), o_b.data_ptr(),
                                     lse_b.data_ptr(), o_a.data_ptr(), lse_a.data_ptr(), s, b,
                                     hp, d, code, sh)
        if rc != 0:
            raise RuntimeError(f"merge: {binding.ulys_status_string(rc)}")

    for _ in range(5):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.merge_steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.merge_steps
    nbytes = 3 * (s * b * hp * d * w.elt + s * b * hp * 4)
    return {"calls": args.merge_steps, "us": round(us, 2), "bytes": nbytes,
            "gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}


def bench_push(args, w, binding, torch, np, xq, tdt, code, stream):
    """One rank's seq->head push of its Q shard into the P ranks' share buffers,
    all on this GPU (on a node the destinations are peers' buffers and the
    writes cross xGMI).  Moves the shard's bytes once: read + write."""
    shares = [torch.empty((w.s, w.b, w.hp, w.d), dtype=tdt, device=xq.device)
              for _ in range(w.P)]
    ptrs = [t.data_ptr() for t in shares]
    sh = stream.cuda_stream

    def call():
        rc = binding.ulys_seq2head_push(xq.data_ptr(), ptrs, 0, w.s, w.b, w.h, w.d, w.P, code, sh)
        if rc != 0:
            raise RuntimeError(f"push: {binding.ulys_status_string(rc)}")

    for _ in range(3):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.push_steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.push_steps
    nbytes = 2 * w.shard_bytes()
    return {"calls": args.push_steps, "us": round(us, 2), "bytes": nbytes,
            "gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}


def bench_layout_hbm(args, w, binding, torch, tdt, code, stream):
    """The step's layout kernels streaming from HBM: the fused Q/K/V pack and
    the O unpack, called back to back over rotating buffer sets whose total is
    at least 2 GiB (8x the 256 MiB last-level cache), so no call finds its
    inputs cached; one event pair around each run of calls."""
    sl, hp, hkvp = w.s // w.P, w.hp, w.hkvp
    dev = stream.device

    def new_set():
        return {"xq": torch.empty((sl, w.b, w.h, w.d), dtype=tdt, device=dev),
                "xk": torch.empty((sl, w.b, w.h_kv, w.d), dtype=tdt, device=dev),
                "xv": torch.empty((sl, w.b, w.h_kv, w.d), dtype=tdt, device=dev),
                "yq": torch.empty((w.P, sl, w.b, hp, w.d), dtype=tdt, device=dev),
                "yk": torch.empty((w.P, sl, w.b, hkvp, w.d), dtype=tdt, device=dev),
                "yv": torch.empty((w.P, sl, w.b, hkvp, w.d), dtype=tdt, device=dev),
                "o": torch.empty((w.s, w.b, hp, w.d), dtype=tdt, device=dev),
                "xo": torch.empty((sl, w.b, w.h, w.d), dtype=tdt, device=dev)}

    pack_bytes = 2 * w.shard_bytes() + 2 * (w.shard_bytes(kv=True) + w.kv_blocks_bytes())
    unpack_bytes = 2 * w.shard_bytes()
    n_sets = max(2, -(-(2 << 30) // (pack_bytes + unpack_bytes)))
    sets = [new_set() for _ in range(n_sets)]
    sh = stream.cuda_stream

    def pack(t):
        rc = binding.ulys_pack_seq2head_qkv(t["xq"].data_ptr(), t["xk"].data_ptr(),
                                            t["xv"].data_ptr(), t["yq"].data_ptr(),
                                            t["yk"].data_ptr(), t["yv"].data_ptr(), w.s, w.b,
                                            w.h, w.h_kv, w.d, w.P, code, sh)
        if rc != 0:
            raise RuntimeError(f"pack qkv: {binding.ulys_status_string(rc)}")

    def unpack(t):
        rc = binding.ulys_unpack_head2seq(t["o"].data_ptr(), t["xo"].data_ptr(), w.s, w.b, w.h,
                                          w.d, w.P, code, sh)
        if rc != 0:
            raise RuntimeError(f"unpack o: {binding.ulys_status_string(rc)}")

    def timed(fn, passes):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(passes):
            for t in sets:
                fn(t)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (passes * n_sets)  # us per call

    for t in sets:
        pack(t)
        unpack(t)
    passes = max(1, args.layout_calls // n_sets)
    pack_us, unpack_us = timed(pack, passes), timed(unpack, passes)
    del sets
    gbps = (pack_bytes + unpack_bytes) / ((pack_us + unpack_us) * 1e-6) / 1e9
    return {"sets": n_sets, "set_bytes": pack_bytes + unpack_bytes, "calls": passes * n_sets,
            "pack_qkv_us": round(pack_us, 2),
            "pack_gbps": round(pack_bytes / (pack_us * 1e-6) / 1e9, 1),
            "unpack_o_us": round(unpack_us, 2),
            "unpack_gbps": round(unpack_bytes / (unpack_us * 1e-6) / 1e9, 1),
            "gbps": round(gbps, 1), "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4)}


def bench_attn_push(args, w, binding, torch, yq, yk, yv, o, xo, tdt, code, ws, ws_bytes, stream):
    """The attention with the head->seq exchange in its epilogue
    (ulys_attn_fwd_push, rank 0 writing its head columns into P destination
    shards on this GPU) against the step's attention followed by the O unpack,
    each timed back to back over the same number of calls."""
    sl = w.s // w.P
    dst = [torch.empty((sl, w.b, w.h, w.d), dtype=tdt, device=o.device) for _ in range(w.P)]
    ptrs = [t.data_ptr() for t in dst]
    sh = stream.cuda_stream

    def fused():
        rc = binding.ulys_attn_fwd_push(yq.data_ptr(), yk.data_ptr(), yv.data_ptr(), ptrs, 0, None,
                                        w.s, w.b, w.h, w.h_kv, w.d, w.P, int(w.causal), code,
                                        ws.data_ptr(), ws_bytes, sh)
        if rc != 0:
            raise RuntimeError(f"attn push: {binding.ulys_status_string(rc)}")

    def separate():
        rc = binding.ulys_attn_fwd_ws(yq.data_ptr(), yk.data_ptr(), yv.data_ptr(), o.data_ptr(),
                                      None, w.s, w.b, w.h, w.h_kv, w.d, w.P, int(w.causal), code,
                                      ws.data_ptr(), ws_bytes, sh)
        if rc == 0:
            rc = binding.ulys_unpack_head2seq(o.data_ptr(), xo.data_ptr(), w.s, w.b, w.h, w.d,
                                              w.P, code, sh)
        if rc != 0:
            raise RuntimeError(f"attn + unpack: {binding.ulys_status_string(rc)}")

    def timed(fn):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.push_attn_calls):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.push_attn_calls

    sep_us, fused_us = timed(separate), timed(fused)
    return {"calls": args.push_attn_calls, "attn_then_unpack_us": round(sep_us, 2),
            "attn_push_us": round(fused_us, 2),
            "tflops": round(w.attn_flops() / (fused_us * 1e-6) / 1e12, 2)}


def bench_backward(args, w, binding, torch, np, q, k, v, code, stream):
    """The backward of the same step: the output gradient's pack (seq->head),
    the attention backward on the share, and the head->seq exchange of dQ, dK
    and dV -- in the backward's epilogues (ulys_attn_bwd_push into P
    destination shards of each on this GPU), or, with replicated KV heads
    (whose gradient copies are summed after the exchange), by the unpack
    kernels.  q, k, v are the forward's packed shares."""
    from ulysses_head_sharded_amd import synth

    dev = q.device
    sl, hp, hkvp = w.s // w.P, w.hp, w.hkvp
    sh = stream.cuda_stream
    qs = q.view(w.s, w.b, hp, w.d)
    ks = k.view(w.s, w.b, hkvp, w.d)
    vs = v.view(w.s, w.b, hkvp, w.d)
    o, lse = binding.attn_fwd(qs, ks, vs, P=w.P, causal=w.causal, lse=True)
    gx = torch.from_numpy(synth.tensor(100 * w.c + 4, (sl, w.b, w.h, w.d), w.dtype)
                          .view(np.int16)).to(dev).view(torch.bfloat16)
    gy = torch.empty((w.s, w.b, hp, w.d), dtype=q.dtype, device=dev)
    dq, dk, dv = torch.empty_like(qs), torch.empty_like(ks), torch.empty_like(vs)
    xdq = torch.empty((sl, w.b, w.h, w.d), dtype=q.dtype, device=dev)
    xdk = torch.empty((sl, w.b, w.h_kv, w.d), dtype=q.dtype, device=dev)
    xdv = torch.empty_like(xdk)
    fused = w.h_kv % w.P == 0
    if fused:
        dst = {n: [torch.empty((sl, w.b, heads, w.d), dtype=q.dtype, device=dev)
                   for _ in range(w.P)] for n, heads in (("dq", w.h), ("dk", w.h_kv), ("dv", w.h_kv))}
        dst_ptrs = {n: [t.data_ptr() for t in ts] for n, ts in dst.items()}
    nbytes = binding.ulys_attn_bwd_workspace_size(w.s, w.b, w.h, w.h_kv, w.d, w.P,
                                                  int(w.causal), code)
    if nbytes < 0:
        raise RuntimeError(f"backward workspace: {binding.ulys_status_string(int(nbytes))}")
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)

    def call(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: {binding.ulys_status_string(rc)}")

    marks = []

    def step(record):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)] if record else None
        if record:
            e[0].record(stream)
        call(binding.ulys_pack_seq2head(gx.data_ptr(), gy.data_ptr(), w.s, w.b, w.h, w.d, w.P,
                                        code, sh), "pack dO")
        if record:
            e[1].record(stream)
        if fused:
            call(binding.ulys_attn_bwd_push(qs.data_ptr(), ks.data_ptr(), vs.data_ptr(),
                                            o.data_ptr(), gy.data_ptr(), lse.data_ptr(),
                                            dst_ptrs["dq"], dst_ptrs["dk"], dst_ptrs["dv"], 0,
                                            w.s, w.b, w.h, w.h_kv, w.d, w.P, int(w.causal), code,
                                            ws.data_ptr(), nbytes, sh), "attn bwd push")
        else:
            call(binding.ulys_attn_bwd(qs.data_ptr(), ks.data_ptr(), vs.data_ptr(), o.data_ptr(),
                                       gy.data_ptr(), lse.data_ptr(), dq.data_ptr(),
                                       dk.data_ptr(), dv.data_ptr(), w.s, w.b, w.h, w.h_kv, w.d,
                                       w.P, int(w.causal), code, ws.data_ptr(), nbytes, sh),
                 "attn bwd")
        if record:
            e[2].record(stream)
        if not fused:
            call(binding.ulys_unpack_head2seq(dq.data_ptr(), xdq.data_ptr(), w.s, w.b, w.h, w.d,
                                              w.P, code, sh), "unpack dq")
            # dK, dV: the replicated KV heads' gradient copies are summed
            for src, dst_t in ((dk, xdk), (dv, xdv)):
                call(binding.ulys_unpack_head2seq_kv(src.data_ptr(), dst_t.data_ptr(), w.s, w.b,
                                                     w.h_kv, w.d, w.P, code, sh), "unpack dkv")
        if record:
            e.append(torch.cuda.Event(enable_timing=True))
            e[3].record(stream)
            marks.append(e)

    settle_s, _, _ = settle(torch, lambda n: [step(False) for _ in range(n)],
                            args.settle_seconds, args.settle_max_seconds)
    # the timed steps: at most about two seconds of them
    per_ms = max(1e-3, settle_probe_ms(torch, step))
    n_steps = max(5, min(args.bwd_steps, int(2000.0 / per_ms)))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_steps):
        step(True)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / n_steps
    attn = stats_ms([e[1].elapsed_time(e[2]) for e in marks])
    layout_ms = float(np.mean([e[0].elapsed_time(e[1]) + e[2].elapsed_time(e[3]) for e in marks]))
    flops = w.attn_bwd_flops()
    if fused:  # the pack of dO only; the gradients' exchange is in the backward's epilogues
        layout_bytes = 2 * w.shard_bytes()
        layout = {"pack_do_us": round(layout_ms * 1e3, 2),
                  "gbps": round(layout_bytes / (layout_ms * 1e-3) / 1e9, 1), "bytes": layout_bytes,
                  "dqkv_exchange": "in the backward's epilogues (ulys_attn_bwd_push)"}
    else:
        layout_bytes = w.layout_bytes()  # pack dO + unpack dQ as pack Q + unpack O; dK, dV as K, V
        layout = {"pack_do_unpack_dqkv_us": round(layout_ms * 1e3, 2),
                  "gbps": round(layout_bytes / (layout_ms * 1e-3) / 1e9, 1), "bytes": layout_bytes}
    tfl = flops / (attn["mean"] * 1e-3) / 1e12
    return {
        "steps": n_steps, "settle_s": round(settle_s, 2), "ms_per_step": round(ms_step, 4),
        "tflops_step": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "attn_bwd": {"ms": round(attn["mean"], 4), "ms_median": round(attn["median"], 4),
                     "ms_min": round(attn["min"], 4), "tflops": round(tfl, 2),
                     "frac_peak": round(tfl / PEAK_BF16_TFLOPS, 4),
                     "flops": flops, "flops_rule": "10 d b hp pairs (five products)",
                     "workspace_bytes": int(nbytes)},
        "layout": layout,
    }


def settle_probe_ms(torch, step) -> float:
    """Wall time of one more untimed step (ms), to size the timed run."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step(False)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3


def run_workload(args, w, headline: bool):
    """Times the forward step (and, for bf16, the backward step) of one share.
    Returns the record (the headline's carries the extra measurements) and the
    device tensors of the share the attention consumed."""
    import numpy as np
    import torch

    from ulysses_head_sharded_amd import binding, synth

    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    sl, hp, hkvp = w.s // w.P, w.hp, w.hkvp

    def upload(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    # rank-local shards [s/P, b, heads, d] of Q, K, V (seeded, synthetic)
    xq_h = synth.tensor(100 * w.c + 1, (sl, w.b, w.h, w.d), w.dtype)
    xk_h = synth.tensor(100 * w.c + 2, (sl, w.b, w.h_kv, w.d), w.dtype)
    xv_h = synth.tensor(100 * w.c + 3, (sl, w.b, w.h_kv, w.d), w.dtype)
    if args.inputs == "constant":
        for a, val in ((xq_h, 0.5), (xk_h, 0.25), (xv_h, 1.0)):
            if a.dtype == np.uint16:
                a[...] = synth.f32_to_bf16_bits(np.full(1, val, dtype=np.float32))[0]
            else:
                a[...] = val
    xq, xk, xv = upload(xq_h), upload(xk_h), upload(xv_h)
    del xq_h, xk_h, xv_h
    yq = torch.empty((w.P, sl, w.b, hp, w.d), dtype=tdt, device=dev)
    yk = torch.empty((w.P, sl, w.b, hkvp, w.d), dtype=tdt, device=dev)
    yv = torch.empty((w.P, sl, w.b, hkvp, w.d), dtype=tdt, device=dev)
    o = torch.empty((w.s, w.b, hp, w.d), dtype=tdt, device=dev)
    xo = torch.empty((sl, w.b, w.h, w.d), dtype=tdt, device=dev)
    code = binding.ULYS_BF16 if w.dtype == "bf16" else binding.ULYS_F32
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    # workspace for the attention's causal load balancing, allocated once
    ws_bytes = binding.ulys_attn_fwd_workspace_size(w.s, w.b, w.h, w.h_kv, w.d, w.P,
                                                    int(w.causal), code)
    if ws_bytes < 0:
        raise RuntimeError(f"workspace size: {binding.ulys_status_string(int(ws_bytes))}")
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    def call(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: {binding.ulys_status_string(rc)}")

    ev = {n: [] for n in ("pack0", "pack1", "attn1", "unpack1")}
    # bf16: the attention pushes its rows into rank 0's P destination shards
    fused = w.dtype == "bf16"
    dst = [torch.empty((sl, w.b, w.h, w.d), dtype=tdt, device=dev) for _ in range(w.P)] \
        if fused else []
    dst_ptrs = [t.data_ptr() for t in dst]

    def step(record: bool):
        if record:  # the fused step has no unpack call to bracket
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3 if fused else 4)]
            e[0].record(stream)
        # Q, K and V packed by one call (K and V replicated when h_kv < P)
        call(binding.ulys_pack_seq2head_qkv(xq.data_ptr(), xk.data_ptr(), xv.data_ptr(),
                                            yq.data_ptr(), yk.data_ptr(), yv.data_ptr(), w.s,
                                            w.b, w.h, w.h_kv, w.d, w.P, code, sh), "pack qkv")
        if record:
            e[1].record(stream)
        # the send buffers stand in for the receive buffers: [P, s/P, b, hp, d] == [s, b, hp, d]
        if fused:
            call(binding.ulys_attn_fwd_push(yq.data_ptr(), yk.data_ptr(), yv.data_ptr(), dst_ptrs,
                                            0, None, w.s, w.b, w.h, w.h_kv, w.d, w.P,
                                            int(w.causal), code, ws.data_ptr(), ws_bytes, sh),
                 "attn push")
        else:
            call(binding.ulys_attn_fwd_ws(yq.data_ptr(), yk.data_ptr(), yv.data_ptr(),
                                          o.data_ptr(), None, w.s, w.b, w.h, w.h_kv, w.d, w.P,
                                          int(w.causal), code, ws.data_ptr(), ws_bytes, sh), "attn")
        if record:
            e[2].record(stream)
        if not fused:
            call(binding.ulys_unpack_head2seq(o.data_ptr(), xo.data_ptr(), w.s, w.b, w.h, w.d,
                                              w.P, code, sh), "unpack o")
        if record:
            if not fused:
                e[3].record(stream)
                ev["unpack1"].append(e[3])
            ev["pack0"].append(e[0])
            ev["pack1"].append(e[1])
            ev["attn1"].append(e[2])

    for _ in range(args.warmup):
        step(False)
    settle_s, settle_steps, settle_ms = settle(torch, lambda n: [step(False) for _ in range(n)],
                                               args.settle_seconds, args.settle_max_seconds)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps

    pack = stats_ms([a.elapsed_time(b) for a, b in zip(ev["pack0"], ev["pack1"])])
    attn = stats_ms([a.elapsed_time(b) for a, b in zip(ev["pack1"], ev["attn1"])])
    unpack_ms = (0.0 if fused else
                 float(np.mean([a.elapsed_time(b) for a, b in zip(ev["attn1"], ev["unpack1"])])))
    pack_ms, attn_ms = pack["mean"], attn["mean"]

    flops = w.attn_flops()
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    pack_bytes = 2 * w.shard_bytes() + 2 * (w.shard_bytes(kv=True) + w.kv_blocks_bytes())
    unpack_bytes = 2 * w.shard_bytes()
    pack_gbps = pack_bytes / (pack_ms * 1e-3) / 1e9
    if fused:  # the O exchange is inside the attention call
        layout = {"pack_qkv_us": round(pack_ms * 1e3, 2),
                  "pack_qkv_us_median": round(pack["median"] * 1e3, 2),
                  "pack_qkv_us_min": round(pack["min"] * 1e3, 2), "pack_gbps": round(pack_gbps, 1),
                  "frac_hbm_peak": round(pack_gbps / PEAK_HBM_GBPS, 4), "bytes": pack_bytes,
                  "o_exchange": "in the attention epilogue (ulys_attn_fwd_push)"}
    else:
        unpack_gbps = unpack_bytes / (unpack_ms * 1e-3) / 1e9
        layout_gbps = (pack_bytes + unpack_bytes) / ((pack_ms + unpack_ms) * 1e-3) / 1e9
        layout = {"pack_qkv_us": round(pack_ms * 1e3, 2), "unpack_o_us": round(unpack_ms * 1e3, 2),
                  "pack_gbps": round(pack_gbps, 1), "unpack_gbps": round(unpack_gbps, 1),
                  "gbps": round(layout_gbps, 1),
                  "frac_hbm_peak": round(layout_gbps / PEAK_HBM_GBPS, 4),
                  "bytes": pack_bytes + unpack_bytes}
    kernel_src = os.path.join(ROOT, "ulysses_head_sharded_amd", "csrc",
                              "attn_bf16.hip" if w.dtype == "bf16" else "attn_f32.hip")
    rec = {
        "ms_per_step": round(ms_step, 4),
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "settle": {"seconds": round(settle_s, 2), "steps": settle_steps,
                   "last_ms_per_step": round(settle_ms, 4)},
        "config": {"workload": w.name, "P": w.P, "s": w.s, "b": w.b, "h": w.h, "h_kv": w.h_kv,
                   "d_h": w.d, "causal": w.causal, "share": f"[{w.s},{w.b},{hp},{w.d}]"},
        "attn": {"ms": round(attn_ms, 4), "ms_median": round(attn["median"], 4),
                 "ms_min": round(attn["min"], 4), "tflops": round(attn_tflops, 2),
                 "tflops_at_median": round(flops / (attn["median"] * 1e-3) / 1e12, 2),
                 "frac_peak": round(attn_tflops / peak, 4), "flops": flops,
                 "workspace_bytes": int(ws_bytes)},
        "layout": layout,
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / peak, 4),
                     "traffic": counter_traffic(kernel_src, w.name)},
    }
    if args.layout_calls > 0:
        rec["layout_hbm"] = bench_layout_hbm(args, w, binding, torch, tdt, code, stream)
    if headline:
        if fused:  # o itself, the merge's input, is filled by a plain call
            call(binding.ulys_attn_fwd_ws(yq.data_ptr(), yk.data_ptr(), yv.data_ptr(),
                                          o.data_ptr(), None, w.s, w.b, w.h, w.h_kv, w.d, w.P,
                                          int(w.causal), code, ws.data_ptr(), ws_bytes, sh),
                 "attn")
        if args.merge_steps > 0:
            rec["merge"] = bench_merge(args, w, binding, torch, np, o, code, stream)
        if args.push_steps > 0:
            rec["exchange_push"] = bench_push(args, w, binding, torch, np, xq, tdt, code, stream)
        if args.push_attn_calls > 0 and w.dtype == "bf16":
            rec["attn_push"] = bench_attn_push(args, w, binding, torch, yq, yk, yv, o, xo, tdt,
                                               code, ws, ws_bytes, stream)
    if args.bwd_steps > 0 and w.dtype == "bf16":
        rec["backward"] = bench_backward(args, w, binding, torch, np, yq, yk, yv, code, stream)
    torch.cuda.synchronize()
    return rec, (yq, yk, yv)


def main():
    args = parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.layout_sweep:
        layout_sweep(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one rank's share on ONE GPU; --gpus {args.gpus} is not "
              "supported (the all-to-all across GPUs is not implemented here)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from ulysses_head_sharded_amd import binding
    from ulysses_head_sharded_amd.workloads import WORKLOADS

    binding.load()
    w = WORKLOADS[args.workload]
    others = [WORKLOADS[n] for n in args.also.split(",") if n and n != w.name]
    head, share = run_workload(args, w, headline=True)
    rec = {
        "metric": METRIC,
        "value": head.pop("value"),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": ("synthetic (seeded N(0,1), SplitMix64 + Box-Muller)" if args.inputs == "normal"
                 else "constant tensors (diagnostic, not the workload)"),
    }
    rec.update(head)
    if not args.no_cpu_baseline:
        # the oracle on the very share the GPU attended over (the packed send
        # buffers [P, s/P, b, hp, d] are the share [s, b, hp, d])
        def host(t):
            t = t.contiguous().view(w.s, w.b, -1, w.d)
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).cpu().numpy().view(np.uint16)
            return t.cpu().numpy()
        q_h, k_h, v_h = (host(t) for t in share)
    del share
    torch.cuda.empty_cache()
    if others:
        rec["configs"] = {}
        for o_w in others:
            sub, sub_share = run_workload(args, o_w, headline=False)
            del sub_share
            torch.cuda.empty_cache()
            rec["configs"][o_w.name] = sub
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, q_h, k_h, v_h, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

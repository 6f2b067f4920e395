"""Benchmark of the Parallax forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads all|main|prefill]
    python bench.py --only NAME        # one workload alone (for profiling)

A step is one pass of the decode hot path (one launch of the split-KV decode
kernel, whose last workgroup per stream merges the partial states) over one
batch of the GQA decode workload (B=8, H_q=16, H_kv=8, d=128, 4096 keys per
sequence, bf16). The KV cache is held in 8 copies in HBM (1.07 GB) and step i
reads copy i mod 8, so no step finds its 134 MB stream in the 256 MB Infinity
Cache left there by the previous one. K timed steps are bracketed by device
synchronisations; `value` is the KV stream (algorithmic bytes: every valid K
and V row once) divided by the mean step time. A step is a single kernel
launch, so a pair of HIP events on the launch stream around the timed region,
divided by K, gives the kernel's average launch duration for the `roofline`
object.

Every workload (the main one included) also reports the distribution of 100
single launches, each inside its own pair of HIP events on the launch stream
(median, p10, p90). Workloads that read their inputs from one copy (no
rotation) write a 512 MB scratch buffer before each of those launches, outside
the event pair, so that no launch finds its inputs in the L2 or the Infinity
Cache. `traffic` per workload comes from the committed rocprofv3 counter
summaries (FETCH_SIZE and WRITE_SIZE, calibrated) while the kernel sources
they were taken on are unchanged.

Workloads: the GQA decode line (also at head dim 64), single-head fp32,
ragged batch, 128K-context split-KV decode, 64 query heads on 8 KV heads,
multi-token decode (2, 3 and 4 new tokens), causal prefill, chunked prefill
(1024 new rows after 3072 cached tokens, and 32, 64, 128 or 256 new rows
after the rest of a 4096-key cache at the GQA decode shape), the prefill backward and
the fused q/k/v/rho projection. The `cpu_baseline` leg times the fp64 oracle on a
bounded sample of the GQA decode workload on the host cores.

One JSON line is printed at the end.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode KV-stream HBM GB/s (% of peak) + us/step; prefill MFMA util"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


KERNEL_SOURCES = {
    # profile file prefix -> the sources its kernel is built from
    "decode_partial": ("decode.hip", "device_common.h"),
    "prefill": ("prefill.hip", "device_common.h"),
}


def kernel_source_digest(prefix: str = "decode_partial") -> str:
    """Digest of a kernel's sources (ties counter figures to a build)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[prefix]:
        with open(os.path.join(ROOT, "local_linear_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str, prefix: str = "decode_partial"):
    """HBM bytes per kernel launch from the committed counter summary
    profiles/<prefix>_<workload>_pmc.md.

    Returns None when there is no summary or the kernel source changed since
    the counters were taken.
    """
    path = os.path.join(PROFILE_DIR, f"{prefix}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_digest:\s*([0-9a-f]+)", text)
    if not m or m.group(1) != kernel_source_digest(prefix):
        return None
    vals = {}
    for key in ("fetch_bytes_per_launch", "write_bytes_per_launch"):
        mm = re.search(key + r":\s*([0-9.eE+]+)", text)
        if not mm:
            return None
        vals[key] = float(mm.group(1))
    return vals


def traffic_entry(workload: str, algorithmic_read_bytes: float, prefix: str = "decode_partial"):
    """The `traffic` fields of a workload entry (None when not measured on
    these sources); reads are compared with the algorithmic read bytes."""
    t = read_traffic(workload, prefix)
    if t is None:
        return {"traffic": None}
    tot = t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"]
    return {"traffic": int(tot), "traffic_fetch_bytes": int(t["fetch_bytes_per_launch"]),
            "traffic_write_bytes": int(t["write_bytes_per_launch"]),
            "fetch_over_algorithmic": round(t["fetch_bytes_per_launch"] / algorithmic_read_bytes, 4)}


class Flusher:
    """Writes a 512 MB scratch buffer (more than the 256 MB Infinity Cache and
    every L2), so that the launch after it reads its inputs from HBM."""

    def __init__(self):
        import torch

        self.buf = torch.empty(128 << 20, dtype=torch.float32, device="cuda")
        self.i = 0

    def __call__(self):
        self.i += 1
        self.buf.fill_(float(self.i & 7))


def launch_stats(launch, n=100, warmup=3, flush=None):
    """Per-launch durations: n single launches, each inside its own pair of HIP
    events on the current stream (the one every launch here uses), with an
    optional cache flush before each, outside the pair. Returns median, p10,
    p90 and mean in microseconds."""
    import numpy as np
    import torch

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for i, (e0, e1) in enumerate(ev):
        if flush is not None:
            flush()
        e0.record()
        launch(i)
        e1.record()
    torch.cuda.synchronize()
    t = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev])
    return {"n": n, "median_us": float(np.median(t)), "p10_us": float(np.percentile(t, 10)),
            "p90_us": float(np.percentile(t, 90)), "mean_us": float(t.mean()),
            "flushed": flush is not None}


class DecodeRunner:
    """Holds device buffers and pre-marshalled C-ABI arguments for one workload."""

    def __init__(self, w, nbuf, seed=None, num_splits=0):
        import torch

        import local_linear_attention_amd as pa
        from workloads import make_decode_inputs

        self.torch = torch
        self.w = w
        dev = torch.device("cuda:0")
        inp = make_decode_inputs(w, seed=seed, device=dev)
        self.inp = inp
        self.lens = inp["seq_lens"].cpu().tolist()
        self.kv_bytes = w.kv_bytes(self.lens)
        ks, vs = [inp["k_cache"]], [inp["v_cache"]]
        for _ in range(nbuf - 1):
            ks.append(inp["k_cache"].clone())
            vs.append(inp["v_cache"].clone())
        self.ks, self.vs = ks, vs
        self.ns, self.chunk = pa.decode_plan(w.B, w.H_q, w.H_kv, w.d, w.S_max, num_splits)
        ws_bytes = max(pa.decode_workspace_size(w.B, w.H_q, w.d, self.ns), 16)
        self.ws = torch.zeros(ws_bytes // 4, dtype=torch.float32, device=dev)
        self.out = torch.empty((w.B, w.H_q, w.d), dtype=torch.float32, device=dev)
        self.stream = torch.cuda.current_stream(dev).cuda_stream
        self.L = pa.lib()
        dcode = 0 if w.dtype == torch.bfloat16 else 1
        self.pargs = [
            (inp["q"].data_ptr(), inp["rho"].data_ptr(), k.data_ptr(), v.data_ptr(),
             inp["seq_lens"].data_ptr(), self.out.data_ptr(), w.B, w.H_q, w.H_kv, w.d, w.S_max,
             float(inp["scale"]), dcode, self.ns, self.ws.data_ptr(), ws_bytes, self.stream)
            for k, v in zip(ks, vs)]

    def read_probe(self, steps, warmup):
        """Event-timed seconds per launch of the plain streaming read over the
        same rotated K and V buffers (the whole caches; used only where every
        cache row is valid, so it reads exactly the decode's KV bytes)."""
        torch = self.torch
        sink = torch.zeros(4096, dtype=torch.int32, device=self.ks[0].device)
        nbytes = self.ks[0].numel() * self.ks[0].element_size()
        args = [(k.data_ptr(), v.data_ptr(), nbytes, sink.data_ptr(), sink.numel(), self.stream)
                for k, v in zip(self.ks, self.vs)]

        def one(i):
            st = self.L.parallax_read_probe(*args[i % len(args)])
            if st != 0:
                raise RuntimeError(f"read probe failed with status {st}")

        for i in range(warmup):
            one(i)
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record()
        for i in range(steps):
            one(i)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps / 1e3

    def step(self, i):
        st = self.L.parallax_decode(*self.pargs[i % len(self.pargs)])
        if st != 0:
            raise RuntimeError(f"decode failed with status {st}")

    def run(self, steps, warmup):
        """(wall seconds per step, event-timed seconds per decode launch).

        A step is one decode launch, so the event pair recorded on the launch
        stream around the whole timed region, divided by the step count, is
        the kernel's average launch duration (back-to-back launches).
        """
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record()
        for i in range(steps):
            self.step(i)
        ev1.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return (t1 - t0) / steps, ev0.elapsed_time(ev1) / steps / 1e3

    def launches(self, flush=None):
        """Per-launch statistics (rotating over the cache copies)."""
        return launch_stats(self.step, flush=flush)


def bench_decode(w, nbuf, steps, warmup, flush=None, read_ref=False, shape=None):
    """A decode workload: back-to-back launches (wall and event span per
    step) and the per-launch distribution; with `read_ref`, the plain read of
    the same bytes."""
    import torch

    r = DecodeRunner(w, nbuf=nbuf)
    s, p = r.run(steps, warmup)
    res = {"us_per_step": s * 1e6, "kernel_us": p * 1e6, "kv_bytes": r.kv_bytes,
           "GB_per_s": r.kv_bytes / p / 1e9,
           "pct_of_hbm_peak": 100 * r.kv_bytes / p / 1e9 / HBM_PEAK_GBS,
           "num_splits": r.ns, "chunk": r.chunk, "steps": steps,
           "dtype": "f32" if w.dtype == torch.float32 else "bf16",
           "launches": r.launches(flush=flush)}
    res["pct_of_hbm_peak_median"] = 100 * r.kv_bytes / (res["launches"]["median_us"] * 1e-6) \
        / 1e9 / HBM_PEAK_GBS
    if shape is not None:
        res["shape"] = shape
    if read_ref and all(n == w.S_max for n in r.lens):
        rs = r.read_probe(steps, warmup)
        res["read_reference_us"] = rs * 1e6
        res["decode_over_read"] = round(rs / p, 4)
    res.update(traffic_entry(w.name, r.kv_bytes))
    del r
    torch.cuda.empty_cache()
    return res


def bench_prefill(w, steps, warmup, seed=None, keep=None, flush=None):
    """Causal prefill per step. With `keep` (a dict), the inputs and the last
    output stay there for the oracle's timing leg."""
    import torch

    import local_linear_attention_amd as pa
    from workloads import make_prefill_inputs

    dev = torch.device("cuda:0")
    inp = make_prefill_inputs(w, seed=seed, device=dev)
    out = torch.empty((w.B, w.H_q, w.T, w.d), dtype=torch.float32, device=dev)
    L = pa.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (inp["q"].data_ptr(), inp["rho"].data_ptr(), inp["k"].data_ptr(), inp["v"].data_ptr(),
            inp["seq_lens"].data_ptr(), out.data_ptr(), w.B, w.H_q, w.H_kv, w.d, w.T,
            inp["k"].shape[2], float(inp["scale"]), 0, stream)

    def one(_i=0):
        if L.parallax_prefill(*args) != 0:
            raise RuntimeError("prefill failed")

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        one()
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern = ev0.elapsed_time(ev1) / steps / 1e3
    lst = launch_stats(one, flush=flush)
    if keep is not None:
        keep.update(inp=inp, out=out)
    # algorithmic work: q.k, rho.k, e.v and (e r).v over the causal half, 2 d flops each
    flops = 8.0 * w.d * (w.T * (w.T + 1) / 2) * w.B * w.H_q
    # algorithmic bytes: q, rho, K, V read once (bf16), out written once (fp32)
    reads = (2 * w.B * w.H_q * w.T * w.d + 2 * w.B * w.H_kv * w.T * w.d) * 2
    writes = w.B * w.H_q * w.T * w.d * 4
    res = {"us_per_step": (t1 - t0) / steps * 1e6, "kernel_us": kern * 1e6,
           "algorithmic_tflop": flops / 1e12, "tflops": flops / kern / 1e12,
           "mfma_util": flops / kern / 1e12 / MFMA_BF16_PEAK_TFLOPS,
           "launches": lst,
           "mfma_util_median": flops / (lst["median_us"] * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
           "algorithmic_read_bytes": reads, "algorithmic_write_bytes": writes,
           "shape": dict(B=w.B, T=w.T, H_q=w.H_q, H_kv=w.H_kv, d=w.d)}
    res.update(traffic_entry(w.name, reads, prefix="prefill"))
    return res


def bench_backward(w, steps, warmup, seed=None, flush=None):
    """Causal-prefill backward (dq/drho and dk/dv launches) per step, and
    the training forward that saves mu_v and the row statistics."""
    import torch

    import local_linear_attention_amd as pa
    from workloads import make_prefill_inputs

    dev = torch.device("cuda:0")
    inp = make_prefill_inputs(w, seed=seed, device=dev)
    g = torch.Generator(device=dev).manual_seed(int(w.seed) + 99)
    dout = torch.randn((w.B, w.H_q, w.T, w.d), generator=g, device=dev, dtype=torch.float32)
    args = (inp["q"], inp["rho"], inp["k"], inp["v"], inp["seq_lens"])
    out, mu, stats = pa.prefill_train(*args, inp["scale"])
    ws = torch.empty(pa.prefill_backward_workspace_size(w.B, w.H_q, w.T, w.d), dtype=torch.uint8,
                     device=dev)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(steps):
            fn()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps / 1e3

    fwd = lambda _i=0: pa.prefill_train(*args, inp["scale"])
    bwd = lambda _i=0: pa.prefill_backward(*args, out, mu, stats, dout, inp["scale"], workspace=ws)
    t_fwd = timed(fwd)
    t_bwd = timed(bwd)
    lst = launch_stats(bwd, n=30, flush=flush)
    pairs = w.T * (w.T + 1) / 2 * w.B * w.H_q
    # algorithmic backward work: the six gradient products (g = dO V^T, dV,
    # dQ, drho, and dK from q and from rho) plus recomputing s and r: 8
    # contractions of 2d flops per causal pair (twice the forward's 4)
    flops = 16.0 * w.d * pairs
    return {"train_forward_us": t_fwd * 1e6, "backward_us": t_bwd * 1e6,
            "algorithmic_tflop": flops / 1e12, "tflops": flops / t_bwd / 1e12,
            "mfma_util": flops / t_bwd / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "launches": lst,
            "shape": dict(B=w.B, T=w.T, H_q=w.H_q, H_kv=w.H_kv, d=w.d)}


def bench_projection(w, steps, warmup, d_model=None, flush=None):
    """Fused q, k, v, rho projection for the causal-prefill shapes: x
    [B, T, d_model] by the packed weight [(2 H_q + 2 H_kv) d, d_model]
    (d_model = H_q d unless given), bf16 in, bf16 out."""
    import torch

    import local_linear_attention_amd as pa

    dev = torch.device("cuda:0")
    C = w.H_q * w.d if d_model is None else d_model
    g = torch.Generator(device=dev).manual_seed(int(w.seed) + 123)
    x = torch.randn((w.B, w.T, C), generator=g, device=dev).to(torch.bfloat16)
    N = (2 * w.H_q + 2 * w.H_kv) * w.d
    wt = (torch.randn((N, C), generator=g, device=dev) * C ** -0.5).to(torch.bfloat16)
    kc = torch.zeros((w.B, w.H_kv, w.T, w.d), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    run = lambda _i=0: pa.qkvr_projection(x, wt, w.H_q, w.H_kv, w.d, k_cache=kc, v_cache=vc)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        run()
    ev1.record()
    torch.cuda.synchronize()
    kern = ev0.elapsed_time(ev1) / steps / 1e3
    lst = launch_stats(run, flush=flush)
    flops = 2.0 * w.B * w.T * N * C
    return {"kernel_us": kern * 1e6, "algorithmic_tflop": flops / 1e12,
            "tflops": flops / kern / 1e12,
            "mfma_util": flops / kern / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "launches": lst,
            "shape": dict(tokens=w.B * w.T, d_model=C, out_features=N)}


def bench_chunked(w, steps, warmup, seed=None, flush=None):
    """Chunked prefill: w.T new rows after w.past cached tokens per sequence."""
    import torch

    import local_linear_attention_amd as pa
    from workloads import make_chunk_inputs

    dev = torch.device("cuda:0")
    inp = make_chunk_inputs(w, seed=seed, device=dev)
    out = torch.empty((w.B, w.H_q, w.T, w.d), dtype=torch.float32, device=dev)
    L = pa.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (inp["q"].data_ptr(), inp["rho"].data_ptr(), inp["k_cache"].data_ptr(),
            inp["v_cache"].data_ptr(), inp["past_lens"].data_ptr(), inp["chunk_lens"].data_ptr(),
            out.data_ptr(), w.B, w.H_q, w.H_kv, w.d, w.T, inp["k_cache"].shape[2],
            float(inp["scale"]), 0, stream)

    def one(_i=0):
        if L.parallax_prefill_chunked(*args) != 0:
            raise RuntimeError("chunked prefill failed")

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        one()
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern = ev0.elapsed_time(ev1) / steps / 1e3
    lst = launch_stats(one, flush=flush)
    # row t sees past + t + 1 keys: 4 contractions of 2 d flops per (row, key)
    pairs = w.T * w.past + w.T * (w.T + 1) / 2
    flops = 8.0 * w.d * pairs * w.B * w.H_q
    return {"us_per_step": (t1 - t0) / steps * 1e6, "kernel_us": kern * 1e6,
            "algorithmic_tflop": flops / 1e12, "tflops": flops / kern / 1e12,
            "mfma_util": flops / kern / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "launches": lst,
            "mfma_util_median": flops / (lst["median_us"] * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "shape": dict(B=w.B, T=w.T, past=w.past, H_q=w.H_q, H_kv=w.H_kv, d=w.d)}


def bench_tokens(T, steps, warmup, seed=None):
    """Multi-token decode (parallax_decode_tokens) at the GQA decode shape: T new
    tokens per sequence after 4096 - T cached ones, 8 rotated cache copies. The
    algorithmic bytes are the KV stream read once, as for the decode."""
    import torch

    import local_linear_attention_amd as pa
    from workloads import CHUNK_WORKLOAD, make_chunk_inputs, replace_shape

    w = replace_shape(CHUNK_WORKLOAD, name=f"multi-token-decode-T{T}", B=8, T=T, past=4096 - T,
                      H_q=16, H_kv=8, d=128)
    dev = torch.device("cuda:0")
    inp = make_chunk_inputs(w, seed=seed, device=dev)
    S_max = inp["k_cache"].shape[2]
    caches = [(inp["k_cache"], inp["v_cache"])]
    for _ in range(7):
        caches.append((inp["k_cache"].clone(), inp["v_cache"].clone()))
    ns, chunk = pa.decode_plan(w.B, w.H_q * T, w.H_kv, w.d, S_max, 0)
    ws_bytes = max(pa.decode_workspace_size(w.B, w.H_q * T, w.d, ns), 16)
    ws = torch.zeros(ws_bytes // 4, dtype=torch.float32, device=dev)
    out = torch.empty((w.B, w.H_q, T, w.d), dtype=torch.float32, device=dev)
    L = pa.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = [(inp["q"].data_ptr(), inp["rho"].data_ptr(), k.data_ptr(), v.data_ptr(),
             inp["past_lens"].data_ptr(), inp["chunk_lens"].data_ptr(), out.data_ptr(), w.B,
             w.H_q, w.H_kv, w.d, T, S_max, float(inp["scale"]), 0, ns, ws.data_ptr(), ws_bytes,
             stream) for k, v in caches]

    def one(i):
        if L.parallax_decode_tokens(*args[i % len(args)]) != 0:
            raise RuntimeError("multi-token decode failed")

    for i in range(warmup):
        one(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(steps):
        one(i)
    ev1.record()
    torch.cuda.synchronize()
    kern = ev0.elapsed_time(ev1) / steps / 1e3
    lst = launch_stats(one)
    kv_bytes = w.B * w.H_kv * S_max * w.d * 2 * 2
    return {"kernel_us": kern * 1e6, "kv_bytes": kv_bytes, "GB_per_s": kv_bytes / kern / 1e9,
            "pct_of_hbm_peak": 100 * kv_bytes / kern / 1e9 / HBM_PEAK_GBS,
            "num_splits": ns, "chunk": chunk, "launches": lst,
            "shape": dict(B=w.B, H_q=w.H_q, H_kv=w.H_kv, d=w.d, new_tokens=T, cached=w.past)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def prefill_oracle_sample(w, keep, min_s=5.0, n_rows=16):
    """Times the fp64 prefill oracle on the causal-prefill workload.

    Two legs: every row of (b, h) pairs, taken in order until at least `min_s`
    seconds have accumulated, through the dense masked-matrix form; and
    `n_rows` single rows spread over the positions through the explicit
    d x d Sigma_KV form. Both are compared with the GPU output of the same
    inputs.
    """
    import numpy as np

    import oracle

    inp, got = keep["inp"], keep["out"]
    G = w.H_q // w.H_kv
    t_full = 0.0
    err = 0.0
    pairs = []
    for b in range(w.B):
        for h in range(w.H_q):
            if t_full >= min_s:
                break
            args = [inp["q"][b:b + 1, h:h + 1], inp["rho"][b:b + 1, h:h + 1],
                    inp["k"][b:b + 1, h // G:h // G + 1], inp["v"][b:b + 1, h // G:h // G + 1],
                    inp["seq_lens"][b:b + 1]]
            args = [a.cpu() for a in args]
            t0 = time.perf_counter()
            full = oracle.oracle_prefill_full(*args, inp["scale"])[(0, 0)]
            t_full += time.perf_counter() - t0
            g = got[b, h].cpu().numpy()
            err = max(err, float(np.max(np.abs(g - full).max(axis=1) / np.abs(full).max(axis=1))))
            pairs.append((b, h))
    rows = [((i + 1) % w.B, (7 * i + 1) % w.H_q, (w.T - 1) * (i + 1) // n_rows)
            for i in range(n_rows)]
    t0 = time.perf_counter()
    ref = oracle.oracle_prefill_rows(inp["q"].cpu(), inp["rho"].cpu(), inp["k"].cpu(),
                                     inp["v"].cpu(), inp["seq_lens"].cpu(), inp["scale"], rows)
    t_rows = time.perf_counter() - t0
    for (b, h, t), o in ref.items():
        err = max(err, float(np.abs(got[b, h, t].cpu().numpy() - o).max() / np.abs(o).max()))
    pair_flops = 8.0 * w.d * w.T * (w.T + 1) / 2
    return {"seconds_per_pair": t_full / len(pairs),
            "gflops": pair_flops * len(pairs) / t_full / 1e9,
            "pairs_sample": f"all {w.T} rows of {len(pairs)} (b, h) pairs, dense masked T x T "
                            f"fp64 NumPy, {t_full:.1f} s",
            "rows_seconds": t_rows,
            "rows_sample": f"{len(rows)} explicit rows (d x d Sigma_KV each) at positions "
                           f"spread over 0..{w.T - 1}",
            "gpu_vs_oracle_max_rel_err": err}


def cpu_baseline(runner, min_s=10.0, budget_s=30.0, prefill=None):
    """Times the fp64 oracle on a bounded sample of the GQA decode workload.

    Query heads are taken in order, cycling over the workload, until at least
    `min_s` seconds of oracle time (or `budget_s` at most) have accumulated.
    With `prefill` = (workload, kept inputs and output), the prefill oracle is
    timed as well (``prefill_oracle_sample``).
    """
    import numpy as np

    import oracle
    from oracle.parallax_oracle import _f64

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    w = runner.w
    inp = runner.inp
    G = w.H_q // w.H_kv
    got = runner.out.cpu().numpy()
    q = inp["q"].cpu()
    rho = inp["rho"].cpu()
    done = 0
    t_total = 0.0
    err = 0.0
    pairs = [(b, h) for b in range(w.B) for h in range(w.H_q)]
    while t_total < min_s:
        b, h = pairs[done % len(pairs)]
        n = runner.lens[b]
        K = _f64(inp["k_cache"][b, h // G, :n].cpu())
        V = _f64(inp["v_cache"][b, h // G, :n].cpu())
        qq, rr = _f64(q[b, h]), _f64(rho[b, h])
        t0 = time.perf_counter()
        o = oracle.parallax_attend(qq, rr, K, V, inp["scale"])
        t_total += time.perf_counter() - t0
        done += 1
        err = max(err, float(np.abs(got[b, h] - o).max() / np.abs(o).max()))
        if t_total > budget_s:
            break
    frac = done / len(pairs)
    gbs = runner.kv_bytes * frac / t_total / 1e9
    res = {"value": gbs, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{done} query-head evaluations ({frac:.2f} passes over the {len(pairs)} "
                     f"query heads of the gqa-decode workload; fp64 NumPy, explicit d x d "
                     f"Sigma_KV), {t_total:.1f} s of oracle time; GB/s is the workload's KV "
                     f"stream times the passes completed, over that time",
           "seconds": t_total, "gpu_vs_oracle_max_rel_err": err,
           "host_cpus": os.cpu_count(),
           "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
           "blas_threads": int(threads), "cpu_model": cpu_model()}
    if prefill is not None:
        res["causal_prefill"] = prefill_oracle_sample(*prefill)
    return res


def workload_registry(steps, warmup, flush, prefill_keep=None):
    """name -> zero-argument function measuring that workload."""
    from workloads import CHUNK_WORKLOAD, WORKLOADS, replace_shape

    w2 = WORKLOADS[2]
    w64 = replace_shape(w2, name="gqa-decode-d64", d=64, q_std=64 ** -0.25, k_std=64 ** -0.25)
    w8 = replace_shape(w2, name="gqa8-decode", H_q=64)
    reg = {
        "gqa-decode-d64": lambda: bench_decode(
            w64, 8, steps, max(3, warmup // 4), read_ref=True,
            shape=dict(B=8, H_q=16, H_kv=8, d=64, kv_len=4096)),
        "single-head-decode": lambda: bench_decode(
            WORKLOADS[1], 1, max(10, steps // 2), max(3, warmup // 4), flush=flush),
        "ragged-batch-decode": lambda: bench_decode(
            WORKLOADS[3], 1, max(10, steps // 10), max(3, warmup // 4)),
        "long-context-splitkv-decode": lambda: bench_decode(
            WORKLOADS[4], 2, max(10, steps // 2), max(3, warmup // 4)),
        "gqa8-decode": lambda: bench_decode(
            w8, 8, steps, max(3, warmup // 4), shape=dict(B=8, H_q=64, H_kv=8, d=128, kv_len=4096)),
    }
    for T in (2, 3, 4):
        reg[f"multi-token-decode-T{T}"] = (lambda T=T: bench_tokens(T, steps, max(3, warmup // 4)))
    reg["causal-prefill"] = lambda: bench_prefill(WORKLOADS[5], max(5, steps // 20), 10,
                                                  keep=prefill_keep, flush=flush)
    reg["chunked-prefill"] = lambda: bench_chunked(CHUNK_WORKLOAD, max(5, steps // 10), 10,
                                                   flush=flush)
    for T in (32, 64, 128, 256):
        wc = replace_shape(CHUNK_WORKLOAD, name=f"short-chunk-prefill-T{T}", B=8, T=T,
                           past=4096 - T, H_q=16, H_kv=8, d=128)
        reg[f"short-chunk-prefill-T{T}"] = (lambda wc=wc: bench_chunked(
            wc, max(10, steps // 2), 10, flush=flush))
    reg["causal-prefill-backward"] = lambda: bench_backward(WORKLOADS[5], max(5, steps // 40), 5,
                                                            flush=flush)
    reg["qkvr-projection"] = lambda: bench_projection(WORKLOADS[5], max(20, steps // 4), 10,
                                                      flush=flush)
    return reg


PREFILL_NAMES = ("causal-prefill", "chunked-prefill", "causal-prefill-backward", "qkvr-projection")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workloads", choices=["all", "main", "prefill"], default="all",
                    help="all: every workload; main: the GQA decode line only; "
                         "prefill: the causal and chunked prefill, the prefill backward and "
                         "the q/k/v/rho projection only (for profiling)")
    ap.add_argument("--only", default=None,
                    help="measure this one workload alone and print {\"workloads\": {...}} "
                         "(for profiling); gqa-decode is the main line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the decode "
              f"path shards by (batch, KV head) with no exchange, so N GPUs run N "
              f"independent copies of this measurement.", file=sys.stderr)
        sys.exit(2)

    import torch

    from workloads import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        b = torch.empty_like(a)
        a.fill_(1.0)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    flush = Flusher()
    prefill_keep = None if (args.no_cpu_baseline or args.only) else {}
    reg = workload_registry(args.steps, args.warmup, flush, prefill_keep)

    if args.only and args.only != WORKLOADS[2].name:
        if args.only not in reg:
            print(f"unknown workload {args.only}; choose from {sorted(reg)} or "
                  f"{WORKLOADS[2].name}", file=sys.stderr)
            sys.exit(2)
        log(f"workload {args.only}")
        print(json.dumps({"workloads": {args.only: reg[args.only]()}}), flush=True)
        return
    if args.workloads == "prefill":
        res = {}
        for name in PREFILL_NAMES:
            log(f"workload {name}")
            res[name] = reg[name]()
        print(json.dumps({"workloads": res}), flush=True)
        return

    w = WORKLOADS[2]
    log(f"main workload {w.name}")
    main_r = DecodeRunner(w, nbuf=8)
    step_s, part_s = main_r.run(args.steps, args.warmup)
    gbs = main_r.kv_bytes / step_s / 1e9
    part_gbs = main_r.kv_bytes / part_s / 1e9
    traffic = read_traffic(w.name)
    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k~N(0,1)/d^0.25, v~N(0,1), rho~N(0,0.05^2), bf16)",
        "config": {"workload": w.name, "B": w.B, "H_q": w.H_q, "H_kv": w.H_kv, "d": w.d,
                   "kv_len": w.S_max, "num_splits": main_r.ns, "chunk": main_r.chunk,
                   "kv_bytes": main_r.kv_bytes, "kv_copies_rotated": 8},
        "us_per_step": step_s * 1e6,
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {
            "bound": "hbm", "kernel": "decode_partial_kernel<bf16,128> (fused merge)",
            "achieved": round(part_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(part_gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_per_launch": main_r.kv_bytes,
            "kernel_us": part_s * 1e6,
            "traffic": None if traffic is None else
            int(traffic["fetch_bytes_per_launch"] + traffic["write_bytes_per_launch"]),
            "traffic_fetch_bytes": None if traffic is None else int(traffic["fetch_bytes_per_launch"]),
            "traffic_write_bytes": None if traffic is None else int(traffic["write_bytes_per_launch"]),
        },
    }
    log(f"{w.name}: {gbs:.0f} GB/s per step, decode kernel {part_gbs:.0f} GB/s")
    launches = main_r.launches()
    result["launches"] = launches
    if all(n == w.S_max for n in main_r.lens):
        read_s = main_r.read_probe(args.steps, args.warmup)
        read_gbs = main_r.kv_bytes / read_s / 1e9
        result["read_reference"] = {
            "kernel": "parallax_read_probe: plain streaming read of the same K and V buffers",
            "kernel_us": read_s * 1e6, "GB_per_s": round(read_gbs, 1),
            "pct_of_hbm_peak": round(100 * read_gbs / HBM_PEAK_GBS, 2),
            "decode_over_read": round(part_gbs / read_gbs, 4)}
        log(f"plain read of the same bytes: {read_gbs:.0f} GB/s")
    if args.only:
        print(json.dumps({"workloads": {w.name: {
            "kernel_us": part_s * 1e6, "launches": launches, "num_splits": main_r.ns,
            "kv_bytes": main_r.kv_bytes}}}), flush=True)
        return

    workloads = {}
    if args.workloads == "all":
        for name, fn in reg.items():
            log(f"workload {name}")
            workloads[name] = fn()
            torch.cuda.empty_cache()
    result["workloads"] = workloads

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(
            main_r, prefill=(WORKLOADS[5], prefill_keep) if prefill_keep else None)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

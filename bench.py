"""Benchmark of the tensor-parallel shard hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-rows] [--no-cpu]
    python bench.py --op NAME [--iters N]      # one kernel family, for rocprofv3

Headline workload (one "step"): the GPT-2-medium-shaped TP MLP layer,
tokens b*s = 8*1024, h = 1024, ffn = 4096 split into N = 4 shards, all four
shards run in sequence on the one GPU:
    for i in 0..3:  H_i = GELU(X W1_i)   (column GEMM + fused GELU epilogue)
                    P_i = H_i W2_i       (row GEMM, fp32 partial)
    Y = sum_i P_i                        (shard sum, stands in for the all-reduce)
bf16 storage, fp32 accumulation, seeded synthetic N(0,1) activations and
N(0, 0.02^2) weights.  value = algorithmic TFLOP/s of the whole step
(8 GEMMs x 2*T*h*ffn/N flops) with inputs resident in HBM.

The step's nine launches are enqueued directly (the host stays ahead of the
GPU; a HIP-graph replay of the same step measured 2% slower); the default
50 warm-up steps bring the clocks to their steady state first (10 left the
first timed pass ~10% slow).  The JSON line also carries: the roofline of
the dominant kernel (the column GEMM + GELU, timed with HIP events over
back-to-back launches on the launch stream), per-call medians and minima,
a measured HBM copy rate, the fp64 CPU oracle timed on this host as a
baseline, and per-row figures for the other workloads (SwiGLU forward /
backward, head-sharded and grouped-query attention and their backward,
sequence-parallel reduce-scatter + LayerNorm, vocabulary-parallel
cross-entropy, decode GEMV) unless --no-rows.
"""
import argparse
import contextlib
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "shard GEMM TFLOP/s (% bf16 MFMA peak); decode GEMV GB/s (% HBM peak)"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-rows", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--op", default=None, help="run one op repeatedly (profiling)")
    ap.add_argument("--iters", type=int, default=100)
    return ap.parse_args()


def dev(t, torch):
    import numpy as np
    if t.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).to("cuda:0").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(t.f32)).to("cuda:0")


@contextlib.contextmanager
def no_gc():
    """Python's cyclic garbage collector paused (as timeit does): a collection
    inside a timed region stalls the host thread that enqueues the launches,
    and the GPU idles meanwhile.  No collection is forced on entry either:
    the GPU would idle through it and its clock drop before the region."""
    was = gc.isenabled()
    gc.disable()
    try:
        yield
    finally:
        if was:
            gc.enable()


def timed(torch, step, steps, warmup):
    """`warmup` untimed calls of step(), then the mean GPU time of `steps`
    back-to-back calls between two HIP events on torch's current stream
    (the launch stream), synchronised on both sides."""
    with no_gc():
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            step()
        t1.record()
        torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


# --------------------------------------------------------------------------- headline
class Headline:
    """gpt2m_mlp_bf16 inputs (numpy PCG64 seed 0, the same draws as the parity tests)."""

    def __init__(self, torch, tp, synth):
        W = synth.WORKLOADS["gpt2m_mlp_bf16"]
        d = synth.make_mlp_inputs(W.tokens, W.h, W.ffn, "bf16", seed=W.seed)
        self.W = W
        n, T, h, f = W.n_shards, W.tokens, W.h, W.ffn_shard
        self.n, self.T, self.h, self.f = n, T, h, f
        self.X = dev(d["X"], torch)
        self.W1 = [dev(synth.column_shard(d["W1"], i, n), torch) for i in range(n)]
        self.W2 = [dev(synth.row_shard(d["W2"], i, n), torch) for i in range(n)]
        self.H = [torch.empty((T, f), dtype=torch.bfloat16, device="cuda:0") for _ in range(n)]
        self.P = [torch.empty((T, h), dtype=torch.float32, device="cuda:0") for _ in range(n)]
        self.Y = torch.empty((T, h), dtype=torch.float32, device="cuda:0")
        self.tp = tp
        self.gemm_flops = 2.0 * T * h * f

    def col(self, i):
        self.tp.tp_col_linear_gelu(self.X, self.W1[i], self.H[i])

    def row(self, i):
        self.tp.tp_row_linear_partial(self.H[i], self.W2[i], self.P[i])

    def total(self):
        self.tp.tp_shard_sum(self.P, self.Y)

    def step(self):
        for i in range(self.n):
            self.col(i)
            self.row(i)
        self.total()


def per_call_ms(torch, fn, iters):
    """Median and minimum GPU time of fn over iters calls, each bracketed by
    its own HIP events (outside the contract's timed region)."""
    pairs = []
    with no_gc():
        for _ in range(iters):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            pairs.append((a, b))
        torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in pairs)
    return t[len(t) // 2], t[0]


def device_peaks():
    """The denominators measured on this machine: compute units and maximum engine
    clock of the GPU agent (rocminfo), and the dense bf16 MFMA peak they give
    (4096 flop per clock per CU: 4 SIMDs x 1024), beside the published figures
    the fractions use."""
    import subprocess
    cus = mhz = None
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
        for block in txt.split("*******"):
            if "gfx950" in block and "Compute Unit:" in block:
                for line in block.splitlines():
                    if line.strip().startswith("Compute Unit:"):
                        cus = int(line.split(":")[1])
                    if line.strip().startswith("Max Clock Freq. (MHz):"):
                        mhz = int(line.split(":")[1])
                break
    except Exception:
        pass
    out = {"source": "rocminfo", "compute_units": cus, "max_sclk_mhz": mhz,
           "spec_bf16_tflops": PEAK_BF16_TFLOPS, "spec_hbm_gbs": PEAK_HBM_GBS}
    if cus and mhz:
        out["derived_bf16_tflops"] = round(cus * 4096 * mhz * 1e6 / 1e12, 1)
    return out


def copy_gbs(torch):
    """Measured HBM reference: a 1 GiB device-to-device copy (reads 1 GiB,
    writes 1 GiB; 4x the 256 MiB last-level cache), bytes moved / time."""
    src = torch.empty(256 << 20, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    med, _ = per_call_ms(torch, lambda: dst.copy_(src), 10)
    del src, dst
    return 2.0 * (1 << 30) / (med * 1e-3) / 1e9


def graph_of(torch, fn):
    """Capture one call of fn (library launches on the current stream) in a HIP graph."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def warm(torch, fn, ms=40.0):
    """Enqueue fn back to back for about `ms` of GPU time and return without
    waiting for it: from idle the engine clock needs ~20 ms of load to ramp,
    and a timed region enqueued behind this backlog starts with the GPU busy,
    so host-side stalls at its start (runtime housekeeping after a burst of
    launches) do not show as idle time inside it."""
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    fn()
    b.record()
    torch.cuda.synchronize()
    for _ in range(min(int(ms / max(a.elapsed_time(b), 1e-3)) + 1, 4000)):
        fn()


def back_to_back_ms(torch, fn, iters):
    """Average GPU time per call of fn over iters back-to-back calls (HIP
    events on torch's current stream, which is the launch stream), enqueued
    behind warm()'s backlog: the steady-state rate of a loop of such calls."""
    with no_gc():
        warm(torch, fn)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        torch.cuda.synchronize()
    return a.elapsed_time(b) / iters


def timed_row(torch, fn, steps, warmup):
    """Mean GPU time of `steps` calls of fn, for a row other than the
    headline: back_to_back_ms after `warmup` further untimed calls."""
    for _ in range(warmup):
        fn()
    return back_to_back_ms(torch, fn, steps)


def headline(torch, hl, steps, warmup):
    """One step = the 9 launches of the 4-shard MLP layer + shard sum,
    enqueued back to back on the current stream (hl: a Headline)."""
    ms = timed(torch, lambda: hl.step(), steps, warmup)
    step_flops = 2 * hl.n * hl.gemm_flops
    col_ms = back_to_back_ms(torch, lambda: hl.col(0), max(steps, 50))
    step_med, step_min = per_call_ms(torch, lambda: hl.step(), steps)
    col_med, col_min = per_call_ms(torch, lambda: hl.col(0), max(steps, 50))
    return {
        "ms": ms, "tflops": step_flops / (ms * 1e-3) / 1e12, "step_flops": step_flops,
        "step_med": step_med, "step_min": step_min, "col_med": col_med, "col_min": col_min,
        "col_ms": col_ms, "col_tflops": hl.gemm_flops / (col_ms * 1e-3) / 1e12,
        "gemm_flops": hl.gemm_flops, "col_bytes": 2.0 * (hl.T * hl.h + hl.h * hl.f + hl.T * hl.f),
        "config": {"workload": "gpt2m_mlp_bf16: TP MLP layer, tokens 8x1024, h 1024, ffn 4096, "
                               "4 shards in sequence + shard sum",
                   "tokens": hl.T, "h": hl.h, "ffn": hl.W.ffn, "n_shards": hl.n,
                   "activation": "gelu_erf", "timing": "9 launches per step, enqueued back to back"},
    }


def other_rooflines(torch, tp):
    """Roofline blocks of the largest workload's dominant kernel (the Llama
    SwiGLU column dual GEMM, 481 GFLOP per launch) and of the decode GEMV
    (one column GEMV of the 8-shard decode MLP: 58.7 MB of weights per call,
    the 8 shards' weights rotated so that none is cache-resident), each timed
    with HIP events over back-to-back launches on the launch stream."""
    R = Rows(torch, tp)
    out = {}
    s = R.swiglu()
    ms = back_to_back_ms(torch, lambda: R.swiglu_col(s), 10)
    fl = 2 * s["flop_gemm"]
    out["llama_swiglu_dual_gemm"] = {
        "bound": "mfma", "kernel": "column dual GEMM + SwiGLU epilogue (8192 x 4096 x 2 x 3584)",
        "achieved": round(fl / ms / 1e9, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
        "frac": round(fl / ms / 1e9 / PEAK_BF16_TFLOPS, 4), "avg_launch_us": round(ms * 1e3, 2),
        "flops_per_launch": fl, "traffic": traffic_record(DUAL_TRAFFIC_PROFILE, TRAFFIC_SOURCES),
        "traffic_unit": "HBM bytes per call (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"}
    del s
    s = R.decode()
    it = [0]

    def col(noalloc=False):
        i = it[0] % s["n"]
        it[0] += 1
        f = tp.tp_col_linear_gelu_noalloc if noalloc else tp.tp_col_linear_gelu
        f(s["x"], s["W1"][i], s["H"][i])
    ms = back_to_back_ms(torch, col, 64)
    ms_na = back_to_back_ms(torch, lambda: col(True), 64)
    wb = s["w_bytes"]
    out["decode_gemv"] = {
        "bound": "hbm", "kernel": "decode column GEMV (split-K pass + finalize, 16 x 8192 x 3584, GELU)",
        "achieved": round(wb / ms / 1e6, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
        "frac": round(wb / ms / 1e6 / PEAK_HBM_GBS, 4), "avg_call_us": round(ms * 1e3, 2),
        "weight_bytes_per_call": wb, "noalloc_avg_call_us": round(ms_na * 1e3, 2),
        "traffic": traffic_record(GEMV_TRAFFIC_PROFILE, GEMV_TRAFFIC_SOURCES, "(column GEMV)"),
        "traffic_unit": "HBM bytes per call, split-K pass + finalize (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                        "copy-calibrated)"}
    R.decode_pack(s)

    def col_packed():
        i = it[0] % s["n"]
        it[0] += 1
        tp.tp_decode_linear_packed(s["x"], s["W1p"][i], s["H"][i], act="gelu")
    ms_p = back_to_back_ms(torch, col_packed, 64)
    out["decode_gemv_packed"] = {
        "bound": "hbm", "kernel": "decode column GEMV on 64-column weight panels (tp_decode_linear_packed: "
                                  "split-K pass + finalize, 16 x 8192 x 3584, GELU)",
        "achieved": round(wb / ms_p / 1e6, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
        "frac": round(wb / ms_p / 1e6 / PEAK_HBM_GBS, 4), "avg_call_us": round(ms_p * 1e3, 2),
        "weight_bytes_per_call": wb,
        "traffic": traffic_record(GEMV_TRAFFIC_PROFILE, GEMV_TRAFFIC_SOURCES, "(packed column GEMV)"),
        "traffic_unit": "HBM bytes per call, split-K pass + finalize (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                        "copy-calibrated)"}
    return out


# --------------------------------------------------------------------------- other workloads
class Rows:
    """The other workloads, at their full per-shard sizes.  Inputs come from a
    seeded device generator (torch.Generator on cuda:0, seed 0) with the same
    distributions as the parity tests: activations N(0,1), weights N(0,0.02^2),
    rounded to bf16."""

    def __init__(self, torch, tp):
        self.torch, self.tp = torch, tp
        self.g = torch.Generator(device="cuda:0")
        self.g.manual_seed(0)

    def randn(self, shape, std):
        t = self.torch
        return (t.randn(shape, generator=self.g, device="cuda:0", dtype=t.float32) * std).to(t.bfloat16)

    def empty(self, shape, dtype):
        return self.torch.empty(shape, dtype=dtype, device="cuda:0")

    # ---- Llama-style SwiGLU shard: T 8192, h 4096, ffn 14336 / 4
    def swiglu(self):
        t = self.torch
        T, h, f = 8192, 4096, 3584
        s = {"X": self.randn((T, h), 1.0), "dY": self.randn((T, h), 1.0),
             "Wg": self.randn((h, f), 0.02), "Wu": self.randn((h, f), 0.02),
             "Wd": self.randn((f, h), 0.02)}
        s["H"] = self.empty((T, f), t.bfloat16)
        s["P"] = self.empty((T, h), t.float32)
        s["dWg"] = self.empty((h, f), t.float32)
        s["dWu"] = self.empty((h, f), t.float32)
        s["dWd"] = self.empty((f, h), t.float32)
        s["dXi"] = self.empty((T, h), t.float32)
        s["flop_gemm"] = 2.0 * T * h * f
        return s

    def swiglu_col(self, s):
        self.tp.tp_col_linear_gelu(s["X"], s["Wg"], s["H"], act="swiglu", Wup=s["Wu"])

    def swiglu_down(self, s):
        self.tp.tp_row_linear_partial(s["H"], s["Wd"], s["P"])

    def swiglu_bwd(self, s):
        self.tp.tp_mlp_shard_backward(s["X"], s["Wg"], s["Wd"], s["dY"], s["dWg"], s["dWd"], s["dXi"],
                                      act="swiglu", Wup=s["Wu"], dWup=s["dWu"])

    # ---- GPT-2-medium GELU MLP shard backward: T 8192, h 1024, ffn 4096 / 4
    def gelu_mlp(self):
        t = self.torch
        T, h, f = 8192, 1024, 1024
        s = {"X": self.randn((T, h), 1.0), "dY": self.randn((T, h), 1.0),
             "W1": self.randn((h, f), 0.02), "W2": self.randn((f, h), 0.02), "b1": self.randn((f,), 0.02)}
        s["dW1"] = self.empty((h, f), t.float32)
        s["dW2"] = self.empty((f, h), t.float32)
        s["db1"] = self.empty((f,), t.float32)
        s["dXi"] = self.empty((T, h), t.float32)
        s["flop_gemm"] = 2.0 * T * h * f
        return s

    def gelu_mlp_bwd(self, s):
        self.tp.tp_mlp_shard_backward(s["X"], s["W1"], s["W2"], s["dY"], s["dW1"], s["dW2"], s["dXi"],
                                      act="gelu", b1=s["b1"], db1=s["db1"])

    # ---- head-sharded MHA: b 4, s 2048, h 4096, 8 local heads of 128
    def mha(self):
        t = self.torch
        b, sq, h, hl, dh = 4, 2048, 4096, 8, 128
        T = b * sq
        s = {"X": self.randn((T, h), 1.0), "Wqkv": self.randn((h, 3 * hl * dh), 0.02),
             "Wo": self.randn((hl * dh, h), 0.02), "P": self.empty((T, h), t.float32),
             "dims": (b, sq, hl, dh)}
        s["ws"] = self.empty((self.tp.tp_attn_heads_shard_workspace(1, b, sq, hl, dh),), t.uint8)
        s["flop_qkv"] = 2.0 * T * h * 3 * hl * dh
        s["flop_att"] = 4.0 * dh * (sq * (sq + 1) / 2) * b * hl
        s["flop_o"] = 2.0 * T * hl * dh * h
        return s

    def attn(self, s):
        b, sq, hl, dh = s["dims"]
        self.tp.tp_attn_heads_shard(s["X"], s["Wqkv"], s["Wo"], s["P"], b, sq, hl, dh, causal=True,
                                    ws=s["ws"])

    # ---- head-sharded MHA backward (same shard): the forward once to fill
    #      its workspace, then dY -> dWqkv, dWo, dX_i per timed call
    def mha_bwd(self, kvl=None):
        t = self.torch
        s = self.mha() if kvl is None else self.gqa()
        if kvl is None:
            b, sq, hl, dh = s["dims"]
            kv = hl
            self.attn(s)
        else:
            b, sq, hl, kv, dh = s["dims"]
            self.gqa_attn(s)
        T, h = b * sq, s["X"].shape[1]
        s["bdims"] = (b, sq, hl, kv, dh)
        s["dY"] = self.randn((T, h), 1.0)
        s["dWqkv"] = self.empty(tuple(s["Wqkv"].shape), t.float32)
        s["dWo"] = self.empty(tuple(s["Wo"].shape), t.float32)
        s["dX"] = self.empty((T, h), t.float32)
        s["bws"] = self.empty((self.tp.tp_attn_shard_backward_workspace(1, b, sq, hl, kv, dh),), t.uint8)
        n3 = (hl + 2 * kv) * dh
        s["flop_bwd_gemm"] = 2.0 * T * h * hl * dh * 2 + 2.0 * T * h * n3 * 2
        s["flop_bwd_att"] = 2.5 * 4.0 * dh * (sq * (sq + 1) / 2) * b * hl
        return s

    def attn_bwd(self, s):
        b, sq, hl, kv, dh = s["bdims"]
        self.tp.tp_attn_shard_backward(s["X"], s["Wqkv"], s["Wo"], s["dY"], s["ws"], s["dWqkv"], s["dWo"], s["dX"],
                                       b, sq, hl, kv, dh, causal=True, ws=s["bws"])

    # ---- grouped-query attention shard: b 4, s 2048, h 4096, 32 query / 8
    #      kv heads of 128 over 4 shards -> 8 query + 2 kv heads per shard
    def gqa(self):
        t = self.torch
        b, sq, h, hl, kvl, dh = 4, 2048, 4096, 8, 2, 128
        T = b * sq
        s = {"X": self.randn((T, h), 1.0), "Wqkv": self.randn((h, (hl + 2 * kvl) * dh), 0.02),
             "Wo": self.randn((hl * dh, h), 0.02), "P": self.empty((T, h), t.float32),
             "dims": (b, sq, hl, kvl, dh)}
        s["ws"] = self.empty((self.tp.tp_attn_gqa_shard_workspace(1, b, sq, hl, kvl, dh),), t.uint8)
        s["flop_qkv"] = 2.0 * T * h * (hl + 2 * kvl) * dh
        s["flop_att"] = 4.0 * dh * (sq * (sq + 1) / 2) * b * hl
        s["flop_o"] = 2.0 * T * hl * dh * h
        return s

    def gqa_attn(self, s):
        b, sq, hl, kvl, dh = s["dims"]
        self.tp.tp_attn_gqa_shard(s["X"], s["Wqkv"], s["Wo"], s["P"], b, sq, hl, kvl, dh, causal=True,
                                  ws=s["ws"])

    # ---- sequence-parallel reduce-scatter + LayerNorm, GPT-2-medium block end:
    #      4 fp32 partials [8192 x 1024], bias, residual; 4 ranks x 2048 rows
    def sp_ln(self):
        t = self.torch
        T, N, n = 8192, 1024, 4
        f32 = lambda shape, std: t.randn(shape, generator=self.g, device="cuda:0", dtype=t.float32) * std
        s = {"P": [f32((T, N), 1.0) for _ in range(n)], "bias": f32((N,), 0.1), "res": f32((T, N), 1.0),
             "gamma": 1.0 + f32((N,), 0.1), "beta": f32((N,), 0.1), "n": n, "T": T,
             "Ysum": self.empty((T, N), t.float32), "Y": self.empty((T, N), t.bfloat16)}
        s["bytes"] = float(T) * N * (4 * n + 4 + 4 + 2)
        return s

    def cold_sets(self, make, nsets):
        """nsets independent input sets (rotated per call so that each call's
        inputs were last touched nsets - 1 calls earlier: with nsets x the set
        size above the 256 MiB last-level cache, every call reads HBM)."""
        return [make() for _ in range(nsets)]

    def sp_ln_step(self, s):
        rows = s["T"] // s["n"]
        for r in range(s["n"]):
            sl = slice(r * rows, (r + 1) * rows)
            self.tp.tp_shard_reduce_scatter_layernorm([p[sl] for p in s["P"]], s["gamma"], s["beta"], s["Y"][sl],
                                                      eps=1e-5, bias=s["bias"], residual=s["res"][sl],
                                                      Ysum=s["Ysum"][sl])

    # ---- vocabulary-parallel cross-entropy, Llama-3 vocabulary 128256 over
    #      4 shards of 32064 columns, b 4 x s 2048 token rows; all 4 shards'
    #      stats, the log-sum-exp combination, 4 shard losses and the total
    def vocab_ce(self):
        t = self.torch
        T, V, n = 8192, 128256, 4
        w = V // n
        s = {"Z": [self.randn((T, w), 2.0) for _ in range(n)], "n": n, "T": T, "w": w,
             "tg": t.randint(0, V, (T,), generator=self.g, device="cuda:0", dtype=t.int32)}
        s["stats"] = [self.empty((T, 2), t.float32) for _ in range(n)]
        s["lse"] = self.empty((T,), t.float32)
        s["loss"] = [self.empty((1,), t.float32) for _ in range(n)]
        s["total"] = self.empty((1,), t.float32)
        s["bytes"] = 2.0 * T * V
        return s

    def vocab_ce_step(self, s):
        tp = self.tp
        for i in range(s["n"]):
            tp.tp_vocab_ce_shard_stats(s["Z"][i], s["stats"][i])
        tp.tp_vocab_ce_lse(s["stats"], s["lse"])
        for i in range(s["n"]):
            tp.tp_vocab_ce_shard_loss(s["Z"][i], i * s["w"], s["tg"], s["lse"], s["loss"][i])
        tp.tp_vocab_ce_total(s["loss"], s["total"])

    # ---- decode GEMV: 16 tokens, h 8192, ffn 28672 / 8, all 8 shards
    #      (940 MB of weights > the 256 MB Infinity Cache: every GEMV streams from HBM)
    def decode(self):
        t = self.torch
        M, h, f, n = 16, 8192, 3584, 8
        s = {"x": self.randn((M, h), 1.0), "n": n, "M": M, "h": h, "f": f}
        s["W1"] = [self.randn((h, f), 0.02) for _ in range(n)]
        s["W2"] = [self.randn((f, h), 0.02) for _ in range(n)]
        s["H"] = [self.empty((M, f), t.bfloat16) for _ in range(n)]
        s["P"] = [self.empty((M, h), t.float32) for _ in range(n)]
        s["Y"] = self.empty((M, h), t.float32)
        s["w_bytes"] = 2.0 * h * f
        return s

    def decode_pack(self, s):
        """Panel copies of the decode weights (packed once, as a server does
        when it loads them; outside every timed region)."""
        s["W1p"] = [self.tp.tp_decode_pack_weight(w) for w in s["W1"]]
        s["W2p"] = [self.tp.tp_decode_pack_weight(w) for w in s["W2"]]
        self.torch.cuda.synchronize()
        return s

    def decode_step_packed(self, s):
        for i in range(s["n"]):
            self.tp.tp_decode_linear_packed(s["x"], s["W1p"][i], s["H"][i], act="gelu")
            self.tp.tp_decode_linear_packed(s["H"][i], s["W2p"][i], s["P"][i], act="none")
        self.tp.tp_shard_sum(s["P"], s["Y"])

    def decode_step(self, s):
        for i in range(s["n"]):
            self.tp.tp_col_linear_gelu(s["x"], s["W1"][i], s["H"][i])
            self.tp.tp_row_linear_partial(s["H"][i], s["W2"][i], s["P"][i])
        self.tp.tp_shard_sum(s["P"], s["Y"])


ROW_ORDER = ["llama_swiglu_fwd", "llama_swiglu_bwd", "gpt2m_gelu_mlp_bwd", "mha_heads_shard", "gqa_heads_shard", "mha_heads_shard_backward", "gqa_heads_shard_backward", "sp_reduce_scatter_layernorm", "shard_sum_cold", "sp_reduce_scatter_layernorm_cold", "vocab_parallel_cross_entropy", "decode_gemv", "decode_gemv_packed"]


def rows(torch, tp, steps, warmup):
    R = Rows(torch, tp)
    out = {}
    s_ms = min(steps, 20)
    w_ms = min(warmup, 10)
    # the HBM-bound rows first and the matrix-core ones last, so that the
    # headline, timed next, starts with the engine clock at its loaded
    # steady state rather than where the memory-bound rows left it
    s = R.sp_ln()
    gl = graph_of(torch, lambda: R.sp_ln_step(s))
    ms_l = timed_row(torch, lambda: gl.replay(), s_ms, w_ms)
    out["sp_reduce_scatter_layernorm"] = {"ms": ms_l, "bytes": s["bytes"], "gbs": s["bytes"] / ms_l / 1e6,
                                          "frac_hbm_peak": s["bytes"] / ms_l / 1e6 / PEAK_HBM_GBS,
                                          "note": "4 ranks x (sum of 4 fp32 partials + bias + residual, "
                                                  "LayerNorm) per graph replay; bytes = partials + residual "
                                                  "read, fp32 sum + bf16 output written"}
    del s
    # shard sum and sequence-parallel LayerNorm with their inputs out of the
    # last-level cache: 3 input sets (3 x 160 MiB / 3 x 208 MiB) rotated
    sets = R.cold_sets(lambda: {"P": [R.empty((8192, 1024), torch.float32).normal_() for _ in range(4)],
                                "Y": R.empty((8192, 1024), torch.float32)}, 3)
    it = [0]

    def sum_cold():
        c = sets[it[0] % 3]
        it[0] += 1
        tp.tp_shard_sum(c["P"], c["Y"])
    ms_s = back_to_back_ms(torch, sum_cold, 30)
    bsum = 5.0 * 8192 * 1024 * 4
    out["shard_sum_cold"] = {"ms": ms_s, "bytes": bsum, "gbs": bsum / ms_s / 1e6,
                             "frac_hbm_peak": bsum / ms_s / 1e6 / PEAK_HBM_GBS,
                             "note": "Y = sum of 4 fp32 partials [8192 x 1024], 3 input sets rotated (480 MiB > "
                                     "the 256 MiB last-level cache): reads and writes reach HBM"}
    del sets
    # four launches per step: one HIP graph per input set, replayed in
    # rotation, so that host-side call overhead stays out of the timing
    sl = [R.sp_ln() for _ in range(3)]
    gs = [graph_of(torch, lambda c=c: R.sp_ln_step(c)) for c in sl]
    it = [0]

    def spln_cold():
        gs[it[0] % 3].replay()
        it[0] += 1
    ms_l2 = back_to_back_ms(torch, spln_cold, 30)
    out["sp_reduce_scatter_layernorm_cold"] = {
        "ms": ms_l2, "bytes": sl[0]["bytes"], "gbs": sl[0]["bytes"] / ms_l2 / 1e6,
        "frac_hbm_peak": sl[0]["bytes"] / ms_l2 / 1e6 / PEAK_HBM_GBS,
        "note": "as sp_reduce_scatter_layernorm, 3 input sets rotated (~650 MiB, one HIP graph per set): "
                "HBM-resident inputs"}
    del gs, sl
    s = R.vocab_ce()
    gv = graph_of(torch, lambda: R.vocab_ce_step(s))
    ms_c = timed_row(torch, lambda: gv.replay(), s_ms, w_ms)
    out["vocab_parallel_cross_entropy"] = {"ms": ms_c, "bytes": s["bytes"], "gbs": s["bytes"] / ms_c / 1e6,
                                           "frac_hbm_peak": s["bytes"] / ms_c / 1e6 / PEAK_HBM_GBS,
                                           "note": "4 shards x [8192 x 32064] bf16 logits: row stats, "
                                                   "log-sum-exp, shard losses, total per graph replay; "
                                                   "bytes = the logits read once"}
    del s
    s = R.decode()
    gd = graph_of(torch, lambda: R.decode_step(s))
    ms_d = timed_row(torch, lambda: gd.replay(), s_ms, 3)
    w_bytes = s["n"] * 2 * s["w_bytes"]
    out["decode_gemv"] = {"ms_step": ms_d, "weight_bytes": w_bytes,
                          "gbs": w_bytes / ms_d / 1e6, "frac_hbm_peak": w_bytes / ms_d / 1e6 / PEAK_HBM_GBS,
                          "note": "16 GEMVs (8 shards x col + row) + shard sum per HIP-graph replay; "
                                  "GB/s counts weight bytes only"}
    R.decode_pack(s)
    gp = graph_of(torch, lambda: R.decode_step_packed(s))
    ms_p = timed_row(torch, lambda: gp.replay(), s_ms, 3)
    out["decode_gemv_packed"] = {"ms_step": ms_p, "weight_bytes": w_bytes,
                                 "gbs": w_bytes / ms_p / 1e6, "frac_hbm_peak": w_bytes / ms_p / 1e6 / PEAK_HBM_GBS,
                                 "note": "as decode_gemv, on the weights packed once into 64-column panels "
                                         "(tp_decode_pack_weight, outside the timed region)"}
    del s
    s = R.gelu_mlp()
    gg = graph_of(torch, lambda: R.gelu_mlp_bwd(s))
    ms_g = timed_row(torch, lambda: gg.replay(), s_ms, w_ms)
    out["gpt2m_gelu_mlp_bwd"] = {"ms": ms_g, "tflops": 4 * s["flop_gemm"] / ms_g / 1e9,
                                 "frac_peak": 4 * s["flop_gemm"] / ms_g / 1e9 / PEAK_BF16_TFLOPS,
                                 "note": "one GPT-2-medium shard (T 8192, h 1024, ffn 1024 per shard): "
                                         "algorithmic flops of dH, dW2, dW1, dX; the Z recompute and db1 "
                                         "are not counted"}
    del s
    s = R.mha()
    ga = graph_of(torch, lambda: R.attn(s))
    ms_a = timed_row(torch, lambda: ga.replay(), s_ms, w_ms)
    fa = s["flop_qkv"] + s["flop_att"] + s["flop_o"]
    out["mha_heads_shard"] = {"ms": ms_a, "tflops": fa / ms_a / 1e9,
                              "frac_peak": fa / ms_a / 1e9 / PEAK_BF16_TFLOPS,
                              "note": "QKV GEMM + causal attention (4*d*s(s+1)/2 per head) + W_o GEMM"}
    del s
    s = R.gqa()
    gq = graph_of(torch, lambda: R.gqa_attn(s))
    ms_q = timed_row(torch, lambda: gq.replay(), s_ms, w_ms)
    fq = s["flop_qkv"] + s["flop_att"] + s["flop_o"]
    out["gqa_heads_shard"] = {"ms": ms_q, "tflops": fq / ms_q / 1e9,
                              "frac_peak": fq / ms_q / 1e9 / PEAK_BF16_TFLOPS,
                              "note": "8 query + 2 kv heads: QKV GEMM + causal attention + W_o GEMM"}
    del s
    for key, kvl in (("mha_heads_shard_backward", None), ("gqa_heads_shard_backward", 2)):
        s = R.mha_bwd(kvl)
        gbw = graph_of(torch, lambda: R.attn_bwd(s))
        ms_bw = timed_row(torch, lambda: gbw.replay(), s_ms, w_ms)
        fb = s["flop_bwd_gemm"] + s["flop_bwd_att"]
        out[key] = {"ms": ms_bw, "tflops": fb / ms_bw / 1e9, "frac_peak": fb / ms_bw / 1e9 / PEAK_BF16_TFLOPS,
                    "note": "dO, dWo, dWqkv, dX GEMMs + attention backward counted as 2.5x the causal "
                            "forward (S recompute, dP, dV, dK, dQ); the kernels recompute S and dP twice"}
        del s
    s = R.swiglu()
    gf = graph_of(torch, lambda: (R.swiglu_col(s), R.swiglu_down(s)))
    gb = graph_of(torch, lambda: R.swiglu_bwd(s))
    ms_f = timed_row(torch, lambda: gf.replay(), s_ms, w_ms)
    ms_b = timed_row(torch, lambda: gb.replay(), s_ms, w_ms)
    flop_f, flop_b = 3 * s["flop_gemm"], 6 * s["flop_gemm"]
    out["llama_swiglu_fwd"] = {"ms": ms_f, "tflops": flop_f / ms_f / 1e9,
                               "frac_peak": flop_f / ms_f / 1e9 / PEAK_BF16_TFLOPS}
    out["llama_swiglu_bwd"] = {"ms": ms_b, "tflops": flop_b / ms_b / 1e9,
                               "frac_peak": flop_b / ms_b / 1e9 / PEAK_BF16_TFLOPS,
                               "note": "algorithmic flops (dgrad x3 + wgrad x3); the Z recompute "
                                       "(+2 GEMMs) is not counted"}
    del s
    return {k: out[k] for k in ROW_ORDER}


# --------------------------------------------------------------------------- single ops
def run_op(torch, tp, synth, name, iters):
    """Run one op `iters` times after a warm-up and print its mean time."""
    if name == "copy":
        # plain device copy of a known size (1 GiB, four times the 256 MiB
        # last-level cache), to calibrate the HBM byte counters:
        # FETCH_SIZE / WRITE_SIZE should each read 1 GiB per copy
        src = torch.empty(256 << 20, dtype=torch.float32, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        fn = lambda: dst.copy_(src)
    elif name in ("gpt2m_col", "gpt2m_row", "gpt2m_sum", "gpt2m_step"):
        hl = Headline(torch, tp, synth)
        fn = {"gpt2m_col": lambda: hl.col(0), "gpt2m_row": lambda: hl.row(0), "gpt2m_sum": hl.total,
              "gpt2m_step": lambda: hl.step()}[name]
    else:
        R = Rows(torch, tp)
        if name in ("llama_swiglu_col", "llama_down", "llama_swiglu_bwd"):
            s = R.swiglu()
            fn = {"llama_swiglu_col": lambda: R.swiglu_col(s), "llama_down": lambda: R.swiglu_down(s),
                  "llama_swiglu_bwd": lambda: R.swiglu_bwd(s)}[name]
        elif name == "gpt2m_mlp_bwd":
            s = R.gelu_mlp()
            fn = lambda: R.gelu_mlp_bwd(s)
        elif name == "mha_shard":
            s = R.mha()
            fn = lambda: R.attn(s)
        elif name == "gqa_shard":
            s = R.gqa()
            fn = lambda: R.gqa_attn(s)
        elif name in ("mha_shard_bwd", "gqa_shard_bwd"):
            s = R.mha_bwd(None if name == "mha_shard_bwd" else 2)
            fn = lambda: R.attn_bwd(s)
        elif name == "sp_layernorm":
            s = R.sp_ln()
            fn = lambda: R.sp_ln_step(s)
        elif name == "sp_layernorm_cold":
            sl = [R.sp_ln() for _ in range(3)]
            it = [0]

            def fn():
                R.sp_ln_step(sl[it[0] % 3])
                it[0] += 1
        elif name == "gpt2m_sum_cold":
            sets = [{"P": [R.empty((8192, 1024), torch.float32).normal_() for _ in range(4)],
                     "Y": R.empty((8192, 1024), torch.float32)} for _ in range(3)]
            it = [0]

            def fn():
                c = sets[it[0] % 3]
                it[0] += 1
                tp.tp_shard_sum(c["P"], c["Y"])
        elif name == "vocab_ce":
            s = R.vocab_ce()
            fn = lambda: R.vocab_ce_step(s)
        elif name in ("decode_col", "decode_row", "decode_col_noalloc", "decode_col_packed", "decode_row_packed"):
            s = R.decode()
            k = {"decode_col": 0, "decode_row": 1, "decode_col_noalloc": 2, "decode_col_packed": 3,
                 "decode_row_packed": 4}[name]
            if k >= 3:
                R.decode_pack(s)
            it = [0]

            def fn():
                i = it[0] % s["n"]
                it[0] += 1
                if k == 0:
                    tp.tp_col_linear_gelu(s["x"], s["W1"][i], s["H"][i])
                elif k == 2:
                    tp.tp_col_linear_gelu_noalloc(s["x"], s["W1"][i], s["H"][i])
                elif k == 3:
                    tp.tp_decode_linear_packed(s["x"], s["W1p"][i], s["H"][i], act="gelu")
                elif k == 4:
                    tp.tp_decode_linear_packed(s["H"][i], s["W2p"][i], s["P"][i], act="none")
                else:
                    tp.tp_row_linear_partial(s["H"][i], s["W2"][i], s["P"][i])
        else:
            raise SystemExit(f"unknown op {name}")
    for _ in range(50):  # the clocks reach their steady state (as the bench's warm-up)
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        fn()
    b.record()
    torch.cuda.synchronize()
    print(json.dumps({"op": name, "iters": iters, "ms_per_iter": a.elapsed_time(b) / iters,
                      "wall_s": time.perf_counter() - t0}), flush=True)


# --------------------------------------------------------------------------- HBM traffic
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemm_col_gelu_gpt2m_shard.md")
TRAFFIC_SOURCES = ["gemm_k64.hip", "gemm_common.hpp", "device_common.hpp", "lds_dma.hpp"]
DUAL_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemm_swiglu_llama_shard.md")
GEMV_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemv_decode_mlp_shard.md")
GEMV_TRAFFIC_SOURCES = ["gemv.hip", "device_common.hpp", "lds_dma.hpp"]


def col_gemm_traffic():
    """HBM bytes per launch of the column GEMM from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE record, or None (see traffic_record)."""
    return traffic_record(TRAFFIC_PROFILE, TRAFFIC_SOURCES)


def traffic_record(profile, sources, kernel=None):
    """HBM bytes per call from a committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    record (KiB per call, summed over the call's dispatches, scaled by the
    factors a 1 GiB copy gave), or None when the record is missing or the
    kernel's sources changed since the counters were taken.  ``kernel``
    picks the record whose kernel name contains it (default: the first)."""
    import hashlib
    try:
        line = next(l for l in open(profile) if l.startswith("traffic-record:")
                    and (kernel is None or kernel in json.loads(l.split(":", 1)[1]).get("kernel", "")))
        rec = json.loads(line.split(":", 1)[1])
        h = hashlib.sha256()
        for f in sources:
            with open(os.path.join(ROOT, "megatron_tensor_transformer_col_amd", "csrc", f), "rb") as fh:
                h.update(fh.read())
    except (OSError, StopIteration, ValueError):
        return None
    if h.hexdigest() != rec.get("sources_sha256"):
        return None
    return 1024.0 * (rec["fetch_kib"] * rec["fetch_factor"] + rec["write_kib"] * rec["write_factor"])


# --------------------------------------------------------------------------- CPU baseline
def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def _time(fn, min_s):
    """Wall seconds per call of fn, repeated until min_s have passed."""
    t0 = time.perf_counter()
    n = 0
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= min_s:
            return el / n, n


def cpu_baseline(synth, seconds):
    """The fp64 oracle (NumPy BLAS, as it stands) timed on this host's cores on
    bounded samples of every workload, the unsharded computation each time.
    `value` is the headline workload's (GPT-2-medium MLP, forward); `configs`
    carries every workload, scaled from its sample to the full unsharded
    algorithmic flops (rows are independent, and weight gradients are sums
    over rows, so the work is linear in the sampled rows / batch elements /
    column blocks).  Inputs are seeded float32 draws of each workload's
    distributions; the oracle's cost does not depend on the values."""
    import numpy as np
    import oracle
    from oracle import brute
    rng = np.random.default_rng(0)
    nrm = lambda shape, std: rng.standard_normal(shape, dtype=np.float32).astype(np.float64) * std
    share = max(seconds / 6.0, 0.5)
    out = {}

    def rec(name, sec, flops_sample, flops_full, sample, calls):
        out[name] = {"sec_per_call": round(sec, 4), "gflops": round(flops_sample / sec / 1e9, 2),
                     "full_unsharded_gflop": round(flops_full / 1e9, 3),
                     "est_full_sec": round(sec * flops_full / flops_sample, 3), "sample": sample, "calls": calls}

    # tiny fp32 MLP, T 32, h 128, ffn 512: whole forward and backward, and the loop version
    w = synth.WORKLOADS["tiny_mlp_f32"]
    d = synth.make_mlp_inputs(w.tokens, w.h, w.ffn, "f32", seed=w.seed, with_dy=True)
    X, W1, W2, dY = d["X"].f64(), d["W1"].f64(), d["W2"].f64(), d["dY"].f64()
    f1 = 2.0 * 2 * w.tokens * w.h * w.ffn
    sec, n = _time(lambda: oracle.mlp_gelu(X, W1, W2), 0.2)
    rec("tiny_mlp_f32_fwd", sec, f1, f1, "whole workload", n)
    sec, n = _time(lambda: oracle.mlp_gelu_backward(X, W1, W2, dY), 0.2)
    rec("tiny_mlp_f32_bwd", sec, 2 * f1, 2 * f1, "whole workload (dH, dW2, dW1, dX)", n)
    Xl, W1l, W2l = X.tolist(), W1.tolist(), W2.tolist()
    sec, n = _time(lambda: brute.mlp_gelu(Xl, W1l, W2l), 0.5)
    rec("tiny_mlp_f32_fwd_brute", sec, f1, f1, "whole workload, pure-Python loops, one core", n)

    # GPT-2-medium MLP forward on 1024-row blocks (the headline)
    W = synth.WORKLOADS["gpt2m_mlp_bf16"]
    d = synth.make_mlp_inputs(W.tokens, W.h, W.ffn, "bf16", seed=W.seed)
    X, W1, W2 = d["X"].f64(), d["W1"].f64(), d["W2"].f64()
    rows = 1024
    it = [0]

    def gpt2m_fwd():
        r0 = (it[0] * rows) % W.tokens
        it[0] += 1
        oracle.mlp_gelu(X[r0:r0 + rows], W1, W2)
    sec, n = _time(gpt2m_fwd, max(2 * share, 2.0))
    f2s, f2 = 2.0 * 2 * rows * W.h * W.ffn, 2.0 * 2 * W.tokens * W.h * W.ffn
    rec("gpt2m_mlp_bf16_fwd", sec, f2s, f2, f"{rows} of {W.tokens} token rows per call", n)
    head = out["gpt2m_mlp_bf16_fwd"]
    del d, X, W1, W2

    # Llama SwiGLU MLP, forward and backward on 256 token rows, full weights
    T3, h3, f3, r3 = 8192, 4096, 14336, 256
    X, Wg, Wu, Wd, dY = nrm((r3, h3), 1.0), nrm((h3, f3), 0.02), nrm((h3, f3), 0.02), nrm((f3, h3), 0.02), nrm((r3, h3), 1.0)
    g3 = 2.0 * h3 * f3
    sec, n = _time(lambda: oracle.mlp_swiglu(X, Wg, Wu, Wd), share)
    rec("llama_swiglu_bf16_fwd", sec, 3 * g3 * r3, 3 * g3 * T3, f"{r3} of {T3} token rows per call", n)
    rb = r3 // 2
    sec, n = _time(lambda: oracle.mlp_swiglu_backward(X[:rb], Wg, Wu, Wd, dY[:rb]), share)
    rec("llama_swiglu_bf16_bwd", sec, 6 * g3 * rb, 6 * g3 * T3,
        f"{rb} of {T3} token rows per call (dWg, dWu, dWd summed over those rows)", n)
    del X, Wg, Wu, Wd, dY

    # MHA, b 4 x s 2048, h 4096, 32 heads of 128, causal: one batch element
    s4, h4, H4, b4 = 2048, 4096, 32, 4
    X = nrm((s4, h4), 1.0)
    Wq, Wk, Wv, Wo = (nrm((h4, h4), 0.02) for _ in range(4))
    f4 = 2.0 * s4 * h4 * 3 * h4 + 4.0 * 128 * s4 * (s4 + 1) / 2 * H4 + 2.0 * s4 * h4 * h4
    sec, n = _time(lambda: oracle.mha(X, Wq, Wk, Wv, Wo, heads=H4, b=1, s=s4, causal=True), share)
    rec("mha_heads_bf16_fwd", sec, f4, b4 * f4, f"batch element 1 of {b4} (the oracle forms the full score matrix)", n)
    del X, Wq, Wk, Wv, Wo

    # decode MLP, 16 tokens, h 8192, ffn 28672: one shard's column block (3584) of W1 / row block of W2
    h5, f5, n5 = 8192, 28672, 8
    x, W1, W2 = nrm((16, h5), 1.0), nrm((h5, f5 // n5), 0.02), nrm((f5 // n5, h5), 0.02)
    f5s = 2.0 * 2 * 16 * h5 * (f5 // n5)
    sec, n = _time(lambda: oracle.mlp_gelu(x, W1, W2), share)
    rec("decode_mlp_bf16_fwd", sec, f5s, n5 * f5s, f"column block 1 of {n5} of the ffn (GELU is column-separable)", n)
    return {"value": round(head["gflops"] / 1e3, 4), "unit": "TFLOP/s", "cores": int(_blas_threads()),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"fp64 oracle (NumPy BLAS), unsharded GELU MLP of the headline workload (h 1024, ffn 4096) "
                      f"on {head['sample']}; per-workload samples in configs",
            "configs": out}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library computes one "
              "GPU's shard and has no cross-GPU exchange", file=sys.stderr)
        sys.exit(2)
    import torch
    import megatron_tensor_transformer_col_amd as tp
    import synth
    tp.lib()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.op:
        run_op(torch, tp, synth, args.op, args.iters)
        return

    # The other GPU measurements run first and the headline after them: a GPU
    # that has been idle (while the inputs are drawn on the host) needs ~20 ms
    # of load before its engine clock settles, and a short warm-up (the 5
    # steps of a 20-step run are ~1 ms) would otherwise time that ramp.  The
    # headline itself still runs exactly `warmup` untimed and `steps` timed
    # steps.
    # Its inputs are drawn before the rows, so that no host-side work
    # separates the rows from the timed steps.
    hl_inputs = Headline(torch, tp, synth)
    others = rows_out = None
    if not args.no_rows:
        others = other_rooflines(torch, tp)
        rows_out = {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in rows(torch, tp, args.steps, args.warmup).items()}
    hl = headline(torch, hl_inputs, args.steps, args.warmup)
    hl["config"]["order"] = ("timed after the other rows' GPU work" if not args.no_rows
                             else "timed first (--no-rows), from an idle GPU")
    result = {
        "metric": METRIC, "value": round(hl["tflops"], 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(hl["ms"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "config": hl["config"],
        "roofline": {"bound": "mfma", "kernel": "column GEMM + GELU epilogue (gemm_k64_kernel NN, 128x128 tiles, two workgroups per CU)",
                     "achieved": round(hl["col_tflops"], 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(hl["col_tflops"] / PEAK_BF16_TFLOPS, 4),
                     "traffic": col_gemm_traffic(), "traffic_unit": "HBM bytes per launch (rocprofv3 "
                     "FETCH_SIZE + WRITE_SIZE, copy-calibrated)", "avg_launch_us": round(hl["col_ms"] * 1e3, 3),
                     "flops_per_launch": hl["gemm_flops"], "algorithmic_bytes_per_launch": hl["col_bytes"]},
        "frac_peak": round(hl["tflops"] / PEAK_BF16_TFLOPS, 4),
        "per_call": {"step_ms_median": round(hl["step_med"], 5), "step_ms_min": round(hl["step_min"], 5),
                     "col_gemm_us_median": round(hl["col_med"] * 1e3, 3),
                     "col_gemm_us_min": round(hl["col_min"] * 1e3, 3),
                     "note": "each call bracketed by its own HIP events, after the timed region"},
        "hbm_copy_gbs": round(copy_gbs(torch), 1),
        "peaks": device_peaks(),
    }
    if others is not None:
        result["rooflines_other"] = others
        result["rows"] = rows_out
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(synth, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

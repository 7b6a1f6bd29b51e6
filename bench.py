"""Benchmark of the tensor-parallel shard hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-rows] [--no-cpu]

Headline workload (one "step"): the GPT-2-medium-shaped TP MLP layer,
tokens b*s = 8*1024, h = 1024, ffn = 4096 split into N = 4 shards, all four
shards run in sequence on the one GPU:
    for i in 0..3:  H_i = GELU(X W1_i)   (column GEMM + fused GELU epilogue)
                    P_i = H_i W2_i       (row GEMM, fp32 partial)
    Y = sum_i P_i                        (shard sum, stands in for the all-reduce)
bf16 storage, fp32 accumulation, seeded synthetic N(0,1) activations and
N(0, 0.02^2) weights.  value = algorithmic TFLOP/s of the whole step
(8 GEMMs x 2*T*h*ffn/N flops) with inputs resident in HBM.

The JSON line also carries: the roofline of the dominant kernel (the column
GEMM, timed with HIP events around each launch on the launch stream), the
fp64 CPU oracle timed on this host as a baseline, and per-row figures for the
other workloads (SwiGLU forward/backward, head-sharded attention, decode
GEMV) unless --no-rows.
"""
import argparse
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
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-rows", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    return ap.parse_args()


def dev(t, torch):
    import numpy as np
    if t.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).to("cuda:0").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(t.f32)).to("cuda:0")


class Timer:
    """HIP events on the stream the library launches on (torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def mark(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def region(self, fn):
        a = self.mark()
        fn()
        b = self.mark()
        self.pairs.append((a, b))

    def mean_ms(self):
        self.torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in self.pairs) / max(1, len(self.pairs))


def timed(torch, step, steps, warmup):
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    kt = Timer(torch)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        step(kt)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps, kt


# --------------------------------------------------------------------------- headline
def headline(torch, tp, synth, steps, warmup):
    W = synth.WORKLOADS["gpt2m_mlp_bf16"]
    d = synth.make_mlp_inputs(W.tokens, W.h, W.ffn, "bf16", seed=W.seed)
    n, T, h, f = W.n_shards, W.tokens, W.h, W.ffn_shard
    X = dev(d["X"], torch)
    W1 = [dev(synth.column_shard(d["W1"], i, n), torch) for i in range(n)]
    W2 = [dev(synth.row_shard(d["W2"], i, n), torch) for i in range(n)]
    H = [torch.empty((T, f), dtype=torch.bfloat16, device="cuda:0") for _ in range(n)]
    P = [torch.empty((T, h), dtype=torch.float32, device="cuda:0") for _ in range(n)]
    Y = torch.empty((T, h), dtype=torch.float32, device="cuda:0")

    def step(kt):
        for i in range(n):
            if kt is None:
                tp.tp_col_linear_gelu(X, W1[i], H[i])
            else:
                kt.region(lambda i=i: tp.tp_col_linear_gelu(X, W1[i], H[i]))
            tp.tp_row_linear_partial(H[i], W2[i], P[i])
        tp.tp_shard_sum(P, Y)

    ms, kt = timed(torch, step, steps, warmup)
    gemm_flops = 2.0 * T * h * f
    step_flops = 2 * n * gemm_flops
    col_ms = kt.mean_ms()
    col_tflops = gemm_flops / (col_ms * 1e-3) / 1e12
    return {
        "ms": ms, "tflops": step_flops / (ms * 1e-3) / 1e12, "step_flops": step_flops,
        "col_ms": col_ms, "col_tflops": col_tflops, "gemm_flops": gemm_flops,
        "config": {"workload": "gpt2m_mlp_bf16: TP MLP layer, tokens 8x1024, h 1024, ffn 4096, "
                               "4 shards in sequence + shard sum",
                   "tokens": T, "h": h, "ffn": W.ffn, "n_shards": n, "activation": "gelu_erf"},
    }


# --------------------------------------------------------------------------- other rows
def rows(torch, tp, steps, warmup):
    g = torch.Generator(device="cuda:0")
    g.manual_seed(0)

    def randn(shape, std):
        return (torch.randn(shape, generator=g, device="cuda:0", dtype=torch.float32) * std).to(torch.bfloat16)

    out = {}
    # ---- Llama-style SwiGLU shard: T 8192, h 4096, ffn 14336 / 4
    T, h, f = 8192, 4096, 3584
    X, dY = randn((T, h), 1.0), randn((T, h), 1.0)
    Wg, Wu, Wd = randn((h, f), 0.02), randn((h, f), 0.02), randn((f, h), 0.02)
    H = torch.empty((T, f), dtype=torch.bfloat16, device="cuda:0")
    P = torch.empty((T, h), dtype=torch.float32, device="cuda:0")
    dWg = torch.empty((h, f), dtype=torch.float32, device="cuda:0")
    dWu = torch.empty_like(dWg)
    dWd = torch.empty((f, h), dtype=torch.float32, device="cuda:0")
    dXi = torch.empty((T, h), dtype=torch.float32, device="cuda:0")

    def fwd(kt):
        tp.tp_col_linear_gelu(X, Wg, H, act="swiglu", Wup=Wu)
        tp.tp_row_linear_partial(H, Wd, P)

    def bwd(kt):
        tp.tp_mlp_shard_backward(X, Wg, Wd, dY, dWg, dWd, dXi, act="swiglu", Wup=Wu, dWup=dWu)

    s_ms = min(steps, 20)
    ms_f, _ = timed(torch, fwd, s_ms, min(warmup, 3))
    ms_b, _ = timed(torch, bwd, s_ms, min(warmup, 3))
    flop_f = 2.0 * T * h * f * 3
    flop_b = 2.0 * T * h * f * 6            # algorithmic: dgrad x3 + wgrad x3
    out["llama_swiglu_fwd"] = {"ms": ms_f, "tflops": flop_f / ms_f / 1e9,
                               "frac_peak": flop_f / ms_f / 1e9 / PEAK_BF16_TFLOPS}
    out["llama_swiglu_bwd"] = {"ms": ms_b, "tflops": flop_b / ms_b / 1e9,
                               "frac_peak": flop_b / ms_b / 1e9 / PEAK_BF16_TFLOPS,
                               "note": "algorithmic flops; the Z recompute (+2*T*h*f*2) is not counted"}
    del X, dY, Wg, Wu, Wd, H, P, dWg, dWu, dWd, dXi

    # ---- head-sharded MHA: b 4, s 2048, h 4096, 8 local heads of 128
    b, s, h, hl, dh = 4, 2048, 4096, 8, 128
    T = b * s
    X = randn((T, h), 1.0)
    Wqkv, Wo = randn((h, 3 * hl * dh), 0.02), randn((hl * dh, h), 0.02)
    P = torch.empty((T, h), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(tp.tp_attn_heads_shard_workspace(1, b, s, hl, dh), dtype=torch.uint8, device="cuda:0")

    def attn(kt):
        tp.tp_attn_heads_shard(X, Wqkv, Wo, P, b, s, hl, dh, causal=True, ws=ws)

    ms_a, _ = timed(torch, attn, s_ms, min(warmup, 3))
    flop_qkv = 2.0 * T * h * 3 * hl * dh
    flop_att = 4.0 * dh * (s * (s + 1) / 2) * b * hl
    flop_o = 2.0 * T * hl * dh * h
    fa = flop_qkv + flop_att + flop_o
    out["mha_heads_shard"] = {"ms": ms_a, "tflops": fa / ms_a / 1e9,
                              "frac_peak": fa / ms_a / 1e9 / PEAK_BF16_TFLOPS,
                              "note": "causal attention counted as 4*d*s(s+1)/2 per head"}
    del X, Wqkv, Wo, P, ws

    # ---- decode GEMV: 16 tokens, h 8192, ffn 28672 / 8; all 8 shards per step
    #      (940 MB of weights > the 256 MB Infinity Cache, so each GEMV streams from HBM)
    M, h, f, n = 16, 8192, 3584, 8
    x = randn((M, h), 1.0)
    W1 = [randn((h, f), 0.02) for _ in range(n)]
    W2 = [randn((f, h), 0.02) for _ in range(n)]
    Hd = [torch.empty((M, f), dtype=torch.bfloat16, device="cuda:0") for _ in range(n)]
    Pd = [torch.empty((M, h), dtype=torch.float32, device="cuda:0") for _ in range(n)]
    Yd = torch.empty((M, h), dtype=torch.float32, device="cuda:0")

    def dec(kt):
        for i in range(n):
            tp.tp_col_linear_gelu(x, W1[i], Hd[i])
            tp.tp_row_linear_partial(Hd[i], W2[i], Pd[i])
        tp.tp_shard_sum(Pd, Yd)

    # capture the 17 launches in a graph so the GPU never waits on the host
    for _ in range(3):
        dec(None)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dec(None)
    ms_d, _ = timed(torch, lambda kt: graph.replay(), s_ms, 3)
    w_bytes = n * 2 * (2.0 * h * f)
    out["decode_gemv"] = {"ms_step": ms_d, "weight_bytes": w_bytes,
                          "gbs": w_bytes / ms_d / 1e6, "frac_hbm_peak": w_bytes / ms_d / 1e6 / PEAK_HBM_GBS,
                          "note": "weights of 16 GEMVs (8 shards x 2) + shard sum per graph replay; "
                                  "GB/s counts weight bytes only"}
    return out


# --------------------------------------------------------------------------- CPU baseline
def cpu_baseline(synth, seconds):
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    W = synth.WORKLOADS["gpt2m_mlp_bf16"]
    d = synth.make_mlp_inputs(W.tokens, W.h, W.ffn, "bf16", seed=W.seed)
    X, W1, W2 = d["X"].f64(), d["W1"].f64(), d["W2"].f64()
    rows = 1024                       # token rows per oracle call (rows are independent)
    flops = 2 * 2.0 * rows * W.h * W.ffn
    t0 = time.perf_counter()
    done, calls = 0.0, 0
    while True:
        r0 = (calls * rows) % W.tokens
        oracle.mlp_gelu(X[r0:r0 + rows], W1, W2)
        calls += 1
        done += flops
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    return {"value": done / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 oracle, unsharded GELU MLP (h 1024, ffn 4096) on {calls} x {rows} "
                      f"token rows of the headline workload, {el:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU "
              "exchange is not part of this build", file=sys.stderr)
        sys.exit(2)
    import torch
    import megatron_tensor_transformer_col_amd as tp
    import synth
    tp.lib()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    hl = headline(torch, tp, synth, args.steps, args.warmup)
    result = {
        "metric": METRIC, "value": round(hl["tflops"], 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(hl["ms"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "config": hl["config"],
        "roofline": {"bound": "mfma", "kernel": "column GEMM + GELU (gemm_kernel NN, EPI_GELU)",
                     "achieved": round(hl["col_tflops"], 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(hl["col_tflops"] / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "avg_launch_us": round(hl["col_ms"] * 1e3, 3),
                     "flops_per_launch": hl["gemm_flops"]},
        "frac_peak": round(hl["tflops"] / PEAK_BF16_TFLOPS, 4),
    }
    if not args.no_rows:
        result["rows"] = {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                          for k, v in rows(torch, tp, args.steps, args.warmup).items()}
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(synth, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

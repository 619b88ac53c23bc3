#!/usr/bin/env python3
"""Benchmark of the large-chunk TTT-KVB layer on one MI355X.

A step is one ttt_forward call over the LaCT language-model layer workload: B=8 sequences of
N=32768 tokens, H=4 heads of d_h=384 with SwiGLU hidden m_h=768, chunks of 2048 tokens,
apply-then-update, L2-Normalize(W - g), bf16 q/k/v with fp32 fast weights.  Every chunk step
(SwiGLU forward/backward, outputs, gradients, weight update) runs inside the timed call.
Inputs are seeded synthetic tensors already resident in HBM.

Prints one JSON line.  Besides the headline figure it reports the dominant kernel against its
roofline (timed with HIP events on the launching stream), the fp64 oracle timed on host cores on a
bounded sample, parity of sampled slices against that oracle, and the other workloads (Muon with
momentum, the strided view-synthesis mask, chunked linear attention) as extra measurements.
"""
import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TTT-layer fwd tokens/sec at chunk 2048 + % of bf16 MFMA peak on 1 MI355X"
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E


def lact_flops(B, H, N, d, m, upd_tokens=None, ns_iters=0, n_updates=0):
    """Algorithmic FLOPs of a ttt_forward call: 6dm per applied token-head (SwiGLU apply), 12dm per
    updated token-head (key forward 4dm, value back-projection 2dm, three gradient sums 6dm), and
    4 p^2 q per Newton-Schulz step per matrix (p = min(d, m), q = max(d, m))."""
    upd_tokens = N if upd_tokens is None else upd_tokens
    p, q = min(d, m), max(d, m)
    return B * H * (6 * d * m * N + 12 * d * m * upd_tokens + n_updates * 3 * ns_iters * 4 * p * p * q)


def lact_bytes(B, H, N, d, m, es=2, n_updates=0, muon=False, momentum=False):
    """Algorithmic HBM bytes: q, k, v, o once, eta once, and the fp32 fast weights (and momentum)
    read and written once per update."""
    io = B * H * N * (4 * d * es + 4)
    w = B * H * 3 * d * m * 4 * 2 * n_updates * (2 if momentum else 1)
    return io + w


def gpu_inputs(torch, B, H, N, d, m, seed, eta_kind="softplus", eta_scale=0.01):
    """Seeded synthetic device inputs (torch's generator on the device) with the workload's
    distributions: q, k, v ~ N(0, 1)/sqrt(d) in bf16, eta = 0.01 softplus(N(0, 1)) (or
    0.05 sigmoid), W0 per head N(0, 1/d) fp32."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    s = 1.0 / d ** 0.5
    q = (torch.randn((B, H, N, d), generator=g, device="cuda") * s).to(torch.bfloat16)
    k = (torch.randn((B, H, N, d), generator=g, device="cuda") * s).to(torch.bfloat16)
    v = (torch.randn((B, H, N, d), generator=g, device="cuda") * s).to(torch.bfloat16)
    raw = torch.randn((B, H, N), generator=g, device="cuda")
    eta = (eta_scale * (torch.nn.functional.softplus(raw) if eta_kind == "softplus" else torch.sigmoid(raw)))
    W0 = None
    if m:
        W0 = torch.randn((H, 3 * d * m), generator=g, device="cuda") * s
    return q, k, v, eta.float().contiguous(), W0


def time_calls(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--oracle-seconds", type=float, default=12.0, help="stop sampling oracle slices after this")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures a single GPU: this build runs each (batch, head) scan on one device and "
              "has no multi-GPU path; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import linear_attention_chunk_amd as T
    from linear_attention_chunk_amd import _lib as C
    import synth

    C.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    # ---------------- headline workload: LaCT LM layer, GD + L2 ----------------
    B, H, N, d, m, chunk = 8, 4, 32768, 384, 768, 2048
    print(f"[bench] generating inputs B{B} H{H} N{N} d{d} m{m}", file=sys.stderr, flush=True)
    q, k, v, eta, _ = gpu_inputs(torch, B, H, N, d, m, 1000 + args.seed)
    sample = [(0, 0), (B - 1, H - 1), (3, 1), (5, 2)]
    exact = {}
    for (b, h) in sample:
        qs, ks, vs, es = synth.slice_inputs(args.seed, b, h, N, d, d, "softplus", 0.01, True)
        exact[(b, h)] = (qs, ks, vs, es)
        for t, x in ((q, qs), (k, ks), (v, vs)):
            t[b, h] = torch.from_numpy(x).to("cuda").to(torch.bfloat16)
        eta[b, h] = torch.from_numpy(es).to("cuda")
    Wh = [synth.head_weights(args.seed, h, d, m) for h in range(H)]
    W0 = torch.from_numpy(np.stack([np.concatenate([w[0].ravel(), w[1].ravel(), w[2].ravel()]) for w in Wh])).cuda()
    D, keep = T.ttt_desc(B, H, N, d, m, chunk, C.TTT_BF16, C.MASK_APPLY_THEN_UPDATE, C.UPD_GD_L2)
    ws = torch.empty(T.ttt_workspace_bytes(D), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)

    def call():
        return T.ttt_forward(q, k, v, eta, W0, chunk, C.MASK_APPLY_THEN_UPDATE, C.UPD_GD_L2, m_h=m, out=o,
                             workspace=ws)

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    C.profile_enable(True)
    C.profile_read()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        _, W_out = call()
    ev1.record()
    torch.cuda.synchronize()
    prof = C.profile_read()
    C.profile_enable(False)
    ms = ev0.elapsed_time(ev1) / args.steps
    tokens = B * N
    value = tokens / (ms * 1e-3)
    nchunks = N // chunk
    flops = lact_flops(B, H, N, d, m, n_updates=nchunks)
    layer_tflops = flops / (ms * 1e-3) / 1e12

    # dominant kernel against its roofline: per-launch algorithmic FLOPs / average launch time
    per_launch = {  # FLOP per launch = per-token-head FLOP x token-heads in one launch
        "k_up": 10 * d * m * B * H * chunk,    # [Q; K] x [W1; W3]^T (4dm + 4dm) and V x W2 (2dm)
        "k_down": 8 * d * m * B * H * chunk,   # O = Hq W2^T (2dm), G1, G3, G2 (6dm)
    }
    dom = max(prof.items(), key=lambda kv: kv[1][0])[0]
    dom_ms, dom_n = prof[dom]
    avg = dom_ms / max(dom_n, 1)
    if dom in per_launch:
        ach = per_launch[dom] / (avg * 1e-3) / 1e12
        roofline = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": None,
                    "avg_launch_us": round(avg * 1e3, 2), "launches": dom_n,
                    "flop_per_launch": per_launch[dom]}
    else:
        roofline = {"kernel": dom, "bound": "hbm", "achieved": None, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": None, "traffic": None, "avg_launch_us": round(avg * 1e3, 2), "launches": dom_n}
    kernels = {kname: {"ms_per_step": round(t / args.steps, 4), "launches_per_step": n / args.steps}
               for kname, (t, n) in prof.items() if n}

    # ---------------- parity of sampled slices + CPU baseline (fp64 oracle) ----------------
    out = {}
    parity = None
    cpu = None
    o_host = {s: o[s[0], s[1]].float().cpu().numpy() for s in sample}
    W_host = {s: W_out[s[0], s[1]].cpu().numpy() for s in sample}
    if not args.no_cpu_baseline:
        import oracle as O
        print("[bench] oracle on sampled slices", file=sys.stderr, flush=True)
        errs_o, errs_w, done = [], [], []
        t0 = time.perf_counter()
        for (b, h) in sample:
            qs, ks, vs, es = exact[(b, h)]
            o_ref, W_ref, _ = O.ttt_scan_ref(qs, ks, vs, es, *Wh[h], chunk, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2)
            done.append((b, h))
            og = o_host[(b, h)].astype(np.float64)
            errs_o.append(float(np.linalg.norm(og - o_ref) / np.linalg.norm(o_ref)))
            Wg = W_host[(b, h)].astype(np.float64)
            dm = d * m
            parts = (Wg[:dm].reshape(m, d), Wg[dm:2 * dm].reshape(m, d), Wg[2 * dm:].reshape(d, m))
            errs_w.append(max(float(np.linalg.norm(a - r) / np.linalg.norm(r)) for a, r in zip(parts, W_ref)))
            if time.perf_counter() - t0 > args.oracle_seconds:
                break
        t_cpu = time.perf_counter() - t0
        per_scan = t_cpu / len(done)
        cpu = {"value": round(N / (H * per_scan), 1), "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
               "sample": f"{len(done)} of {B * H} (batch, head) scans, each the full {N}-token sequence "
                         f"({nchunks} chunks), numpy fp64; scaled to the whole workload",
               "seconds": round(t_cpu, 2), "cpu": cpu_model()}
        parity = {"slices": [list(s) for s in done], "max_rel_l2_o": max(errs_o), "max_rel_l2_W": max(errs_w),
                  "tol": 2e-2, "ok": max(errs_o) <= 2e-2 and max(errs_w) <= 2e-2}

    # ---------------- other workloads (extra measurements, not the headline) ----------------
    extras = {}
    if not args.no_extras:
        st = max(3, args.steps // 4)
        print("[bench] extras: Muon + momentum", file=sys.stderr, flush=True)
        M = torch.zeros((B, H, 3 * d * m), dtype=torch.float32, device="cuda")
        D4, _ = T.ttt_desc(B, H, N, d, m, chunk, C.TTT_BF16, C.MASK_APPLY_THEN_UPDATE, C.UPD_MUON_L2, 5, 0.9)
        ws4 = torch.empty(T.ttt_workspace_bytes(D4), dtype=torch.uint8, device="cuda")
        ms4 = time_calls(torch, lambda: T.ttt_forward(q, k, v, eta, W0, chunk, C.MASK_APPLY_THEN_UPDATE,
                                                      C.UPD_MUON_L2, m_h=m, momentum=0.9, M=M, out=o,
                                                      workspace=ws4), st, 1)
        f4 = lact_flops(B, H, N, d, m, ns_iters=5, n_updates=nchunks)
        extras["lact_lm_muon_momentum"] = {"tokens_per_s": round(tokens / (ms4 * 1e-3)), "ms_per_call": round(ms4, 3),
                                           "mfma_frac": round(f4 / (ms4 * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                                           "algorithmic_tflop": round(f4 / 1e12, 3)}
        del ws4, M
        print("[bench] extras: strided NVS mask", file=sys.stderr, flush=True)
        B5, H5, N5, d5, m5, c5 = 2, 4, 65536, 256, 512, 4096
        q5, k5, v5, e5, W05 = gpu_inputs(torch, B5, H5, N5, d5, m5, 2000 + args.seed)
        flags = [1] * 12 + [0] * 4
        D5, _ = T.ttt_desc(B5, H5, N5, d5, m5, c5, C.TTT_BF16, C.MASK_STRIDED, C.UPD_MUON_L2, 5, 0.0,
                           update_chunks=flags)
        ws5 = torch.empty(T.ttt_workspace_bytes(D5), dtype=torch.uint8, device="cuda")
        o5 = torch.empty_like(q5)
        ms5 = time_calls(torch, lambda: T.ttt_forward(q5, k5, v5, e5, W05, c5, C.MASK_STRIDED, C.UPD_MUON_L2, m_h=m5,
                                                      update_chunks=flags, out=o5, workspace=ws5), st, 1)
        f5 = lact_flops(B5, H5, N5, d5, m5, upd_tokens=12 * c5, ns_iters=5, n_updates=12)
        extras["nvs_strided_muon"] = {"tokens_per_s": round(B5 * N5 / (ms5 * 1e-3)), "ms_per_call": round(ms5, 3),
                                      "mfma_frac": round(f5 / (ms5 * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
        del q5, k5, v5, e5, W05, ws5, o5
        print("[bench] extras: linear attention", file=sys.stderr, flush=True)
        B2, H2, N2, d2, c2 = 4, 16, 8192, 128, 256
        q2, k2, v2, e2, _ = gpu_inputs(torch, B2, H2, N2, d2, 0, 3000 + args.seed, "sigmoid", 0.05)
        o2 = torch.empty_like(q2)
        lin_bytes = B2 * H2 * N2 * (4 * d2 * 2 + 4)
        for name, mask in (("linattn_chunked", C.MASK_APPLY_THEN_UPDATE), ("linattn_token_causal", C.MASK_TOKEN_CAUSAL)):
            msl = time_calls(torch, lambda: T.linattn_forward(q2, k2, v2, e2, c2, mask, out=o2, want_S=False),
                             max(st, 10), 2)
            extras[name] = {"tokens_per_s": round(B2 * N2 / (msl * 1e-3)), "ms_per_call": round(msl, 4),
                            "hbm_GBps": round(lin_bytes / (msl * 1e-3) / 1e9, 1),
                            "hbm_frac": round(lin_bytes / (msl * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "workload": f"B{B2} H{H2} N{N2} d_k=d_v={d2} chunk {c2} bf16"}
        # the SwiGLU layer at the same shape (m = 2d), for the linear-vs-SwiGLU comparison
        m2 = 2 * d2
        W02 = torch.randn((H2, 3 * d2 * m2), device="cuda") / d2 ** 0.5
        Ds, _ = T.ttt_desc(B2, H2, N2, d2, m2, c2, C.TTT_BF16, C.MASK_APPLY_THEN_UPDATE, C.UPD_GD_L2)
        wss = torch.empty(T.ttt_workspace_bytes(Ds), dtype=torch.uint8, device="cuda")
        mss = time_calls(torch, lambda: T.ttt_forward(q2, k2, v2, e2, W02, c2, C.MASK_APPLY_THEN_UPDATE, C.UPD_GD_L2,
                                                      m_h=m2, out=o2, workspace=wss), st, 1)
        extras["swiglu_at_linattn_shape"] = {"tokens_per_s": round(B2 * N2 / (mss * 1e-3)), "ms_per_call": round(mss, 3),
                                             "m_h": m2, "linattn_speedup": round(mss / extras["linattn_chunked"]["ms_per_call"], 2)}

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1)/sqrt(d) q,k,v in bf16, eta = 0.01 softplus(N(0,1)), W0 ~ N(0,1/d) per head",
        "config": {"workload": "lact_lm_layer_b8_h4_n32768_d384_m768_chunk2048_gd_l2", "B": B, "H": H, "seq_len": N,
                   "d_h": d, "m_h": m, "chunk": chunk, "mask": "apply_then_update", "update": "L2-Normalize(W - g)",
                   "parallelism": "none (one GPU)"},
        "mfma_frac_layer": round(layer_tflops / BF16_PEAK_TFLOPS, 4),
        "layer_tflops": round(layer_tflops, 2),
        "algorithmic_tflop_per_step": round(flops / 1e12, 4),
        "algorithmic_gb_per_step": round(lact_bytes(B, H, N, d, m, 2, nchunks) / 1e9, 3),
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "parity": parity,
        "extras": extras,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the large-chunk TTT-KVB layer on one MI355X.

A step is one ttt_forward call over the LaCT language-model layer workload: B=8 sequences of
N=32768 tokens, H=4 heads of d_h=384 with SwiGLU hidden m_h=768, chunks of 2048 tokens,
apply-then-update, L2-Normalize(W - g), bf16 q/k/v with fp32 fast weights.  Every chunk step
(SwiGLU forward/backward, outputs, gradients, weight update) runs inside the timed call.
Inputs are seeded synthetic tensors already resident in HBM.

Prints one JSON line.  Besides the headline figure it reports the dominant kernel against its
roofline (timed with HIP events on the launching stream), the fp64 oracle timed on host cores on a
bounded sample of scans, parity of those scans against that oracle, and the other workloads (Muon with
momentum, the strided view-synthesis mask, chunked linear attention) as extra measurements.
"""
import argparse
import ctypes
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


# HBM bytes per launch at the headline workload from rocprofv3 FETCH_SIZE and WRITE_SIZE, each scaled
# by what the counter reads for a 1 GiB device copy, with the hash of the kernel sources they were
# taken on.  They are reported only while those sources are unchanged.
TRAFFIC_SOURCES = ("linear_attention_chunk_amd/csrc/ttt_layer.hip", "linear_attention_chunk_amd/csrc/tile.hpp")
MEASURED_TRAFFIC = {
    "source_sha": "d17b1313d14fec8b",
    "k_up": {"read": 339.3e6, "write": 497.7e6},
    "k_down": {"read": 569.3e6, "write": 163.9e6},
    "k_update": {"read": 214.4e6, "write": 177.7e6},
}


def sources_sha():
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    t = MEASURED_TRAFFIC.get(kernel)
    if t is None or sources_sha() != MEASURED_TRAFFIC["source_sha"]:
        return None
    return round(t["read"] + t["write"])


def lact_flops(B, H, N, d, m, upd_tokens=None, ns_iters=0, n_updates=0, last_only=False):
    """Algorithmic FLOPs of a ttt_forward call: 6dm per applied token-head (SwiGLU apply), 12dm per
    updated token-head (key forward 4dm, value back-projection 2dm, three gradient sums 6dm; with
    only W2 learning, key forward 4dm and the W2 gradient 2dm), and 4 p^2 q per Newton-Schulz step
    per matrix (p = min(d, m), q = max(d, m))."""
    upd_tokens = N if upd_tokens is None else upd_tokens
    p, q = min(d, m), max(d, m)
    per_upd = 6 if last_only else 12
    return B * H * (6 * d * m * N + per_upd * d * m * upd_tokens + n_updates * 3 * ns_iters * 4 * p * p * q)


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


def graph_replay_ms(torch, fn, steps):
    """The call captured once into a HIP graph (after an eager call), then timed as graph replays."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        fn()
    torch.cuda.synchronize()
    ms = time_calls(torch, g.replay, steps, 2)
    del g
    return ms


def measured_peaks(torch, C):
    """Rates this device sustains, timed outside the timed region: the library's MFMA-loop probe
    (bf16 32x32x16 MFMAs on register operands, 1024 workgroups x 512 rounds) and a 1 GiB
    device-to-device copy (2^30 bytes read and 2^30 written).  Best of three each."""
    out = torch.empty(1024, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    blocks, iters = 1024, 512
    flop = blocks * 4 * iters * 4 * 32 * 32 * 16 * 2

    def probe():
        C.check(C.lib().ttt_probe_mfma_bf16(blocks, iters, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream)))

    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    best = {}
    for name, fn in (("mfma", probe), ("copy", lambda: dst.copy_(src))):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        best[name] = min(ts)
    del src, dst
    return {"bf16_mfma_TFLOPs": round(flop / (best["mfma"] * 1e-3) / 1e12, 1),
            "copy_GBps": round(2 * (1 << 30) / (best["copy"] * 1e-3) / 1e9, 1),
            "how": "MFMA-loop probe (register operands, 4 independent accumulators per wave) and a 1 GiB "
                   "device copy, best of 3, outside the timed region"}


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
    ap.add_argument("--oracle-seconds", type=float, default=25.0,
                    help="stop the oracle after the scan that passes this many seconds")
    ap.add_argument("--update", choices=["gd_l2", "muon_momentum", "last_layer_gd_parallel"], default="gd_l2",
                    help="update rule of the timed layer (the headline metric uses gd_l2); last_layer_gd_parallel: "
                         "only W2 learns, W - g, in the parallel static-kernel form")
    ap.add_argument("--profile-backward", choices=["gd_l2", "muon_momentum"], default=None,
                    help="time only the layer's backward with all weights learning (for kernel traces) and print "
                         "its own JSON line instead of the headline's")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first copy a 1 GiB device buffer three times (a known-size kernel that scales "
                         "hardware byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures a single GPU: the library runs each (batch, head) scan on one device and "
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

    if args.copy_probe:
        src = torch.empty(1 << 29, dtype=torch.float16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print("[bench] copy probe: 3 x 1 GiB device copies done", file=sys.stderr, flush=True)

    # ---------------- headline workload: LaCT LM layer, GD + L2 ----------------
    B, H, N, d, m, chunk = 8, 4, 32768, 384, 768, 2048
    print(f"[bench] generating inputs B{B} H{H} N{N} d{d} m{m}", file=sys.stderr, flush=True)
    exact = {}
    if args.no_cpu_baseline:  # same distributions, drawn on the device (nothing to check them against)
        q, k, v, eta, _ = gpu_inputs(torch, B, H, N, d, 0, 1000 + args.seed)
    else:  # every (batch, head) scan from the seeded per-slice recipe, so the oracle can check any of them
        q = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
        k = torch.empty_like(q)
        v = torch.empty_like(q)
        eta = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        for b in range(B):
            for h in range(H):
                qs, ks, vs, es = synth.slice_inputs(args.seed, b, h, N, d, d, "softplus", 0.01, True)
                exact[(b, h)] = (qs, ks, vs, es)
                for t, x in ((q, qs), (k, ks), (v, vs)):
                    t[b, h] = torch.from_numpy(x).to("cuda").to(torch.bfloat16)
                eta[b, h] = torch.from_numpy(es).to("cuda")
            print(f"[bench] inputs of batch {b} ready", file=sys.stderr, flush=True)
    Wh = [synth.head_weights(args.seed, h, d, m) for h in range(H)]
    W0 = torch.from_numpy(np.stack([np.concatenate([w[0].ravel(), w[1].ravel(), w[2].ravel()]) for w in Wh])).cuda()
    if args.profile_backward:  # the backward alone, on the headline's inputs
        rb, bb = {"gd_l2": (C.UPD_GD_L2, 0.0), "muon_momentum": (C.UPD_MUON_L2, 0.9)}[args.profile_backward]
        gb = torch.Generator(device="cuda")
        gb.manual_seed(3600 + args.seed)
        dOb = (torch.randn((B, H, N, d), generator=gb, device="cuda") / d ** 0.5).to(torch.bfloat16)
        Db, _ = T.ttt_desc(B, H, N, d, m, chunk, C.TTT_BF16, C.MASK_APPLY_THEN_UPDATE, rb, 5, bb)
        wsb = torch.empty(T.ttt_backward_workspace_bytes(Db), dtype=torch.uint8, device="cuda")
        msb = time_calls(torch, lambda: T.ttt_backward(q, k, v, eta, W0, dOb, chunk, C.MASK_APPLY_THEN_UPDATE, m_h=m,
                                                       update_rule=rb, momentum=bb, last_layer_only=False,
                                                       workspace=wsb), args.steps, args.warmup)
        print(json.dumps({"profile_backward": args.profile_backward, "ms_per_call": round(msb, 3),
                          "calls": args.steps + args.warmup,
                          "workload": f"B{B} H{H} N{N} d{d} m{m} chunk {chunk} bf16, apply-then-update, all weights "
                                      "learning"}))
        return
    rule, beta = {"gd_l2": (C.UPD_GD_L2, 0.0), "muon_momentum": (C.UPD_MUON_L2, 0.9),
                  "last_layer_gd_parallel": (C.UPD_GD, 0.0)}[args.update]
    par = args.update == "last_layer_gd_parallel"
    D, keep = T.ttt_desc(B, H, N, d, m, chunk, C.TTT_BF16, C.MASK_APPLY_THEN_UPDATE, rule, 5, beta, last_layer_only=par,
                         parallel_form=par)
    ws = torch.empty(T.ttt_workspace_bytes(D), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    Mom = torch.zeros((B, H, 3 * d * m), dtype=torch.float32, device="cuda") if beta else None

    def call():
        if Mom is not None:
            Mom.zero_()
        return T.ttt_forward(q, k, v, eta, W0, chunk, C.MASK_APPLY_THEN_UPDATE, rule, m_h=m, momentum=beta, M=Mom,
                             out=o, workspace=ws, last_layer_only=par, parallel_form=par)

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    # the dominant kernel class: most time in one untimed call with every launch bracketed
    C.profile_select(None)
    C.profile_enable(True)
    C.profile_read()
    call()
    torch.cuda.synchronize()
    dom = max(C.profile_read().items(), key=lambda kv: kv[1][0])[0]
    # in the timed region only the dominant kernel's launches are bracketed by events: each bracket
    # costs the stream a few microseconds (all 49 launches of a call: about 3%)
    C.profile_select([dom])
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
    flops = lact_flops(B, H, N, d, m, ns_iters=5 if beta else 0, n_updates=nchunks, last_only=par)
    layer_tflops = flops / (ms * 1e-3) / 1e12

    # dominant kernel against its roofline: algorithmic work per launch / average launch time
    S, dm, p_ns, q_ns, es = B * H, d * m, min(d, m), max(d, m), 2
    work = {  # kernel: (bound, FLOP or HBM bytes per launch)
        # [Q; K] x [W1; W3]^T (4dm + 4dm) and V x W2 (2dm) per token-head, one chunk of every scan
        "k_up": ("mfma", 10 * dm * S * chunk),
        # O = Hq W2^T (2dm), gradient sums G1, G3, G2 (6dm) per token-head
        "k_down": ("mfma", 8 * dm * S * chunk),
        # read W and G in fp32, write W in fp32 and the bf16 copies of W1, W3, W2, W2^T; averaged
        # over a call's launches: the initial bf16 copies of W0 (read per head), the chunk updates
        # (the first reads W0), and the last one, which writes W_out and no copies
        "k_update": ("hbm", (4 * 3 * dm * H + es * 4 * dm * S
                             + (nchunks - 1) * ((4 + 4 + 4) * 3 * dm * S + es * 4 * dm * S)
                             + (4 + 4 + 4) * 3 * dm * S) / (nchunks + 1)),
        # read G (and read/write M) in fp32, write U as the bf16 hi + lo pair that starts Newton-Schulz
        "k_muon_prep": ("hbm", ((12 if beta else 4) + 2 * es) * 3 * dm * S),
        # zero Newton-Schulz steps only: read U, write U / ||U||_F in fp32
        "k_ns_init": ("hbm", (4 + 4) * 3 * dm * S),
        # Gram p x p from the bf16 hi plane: 2 p^2 q per matrix
        "k_ns_gram": ("mfma", 2 * p_ns * p_ns * q_ns * 3 * S),
        # read the iterate's hi + lo planes and the bf16 Gram; write hi + lo (the last step: fp32)
        "k_ns_step": ("hbm", ((2 * es + 2 * es) * dm + es * p_ns * p_ns) * 3 * S),
        # parallel form, one launch each per call: phi(q) and phi(k) (2 x 4dm per token-head),
        # dS = (eta V)^T phi(K) and o = phi(Q) S^T (2dm each per token-head), and the state scan
        # (dS read, S_c written as hi + lo: 8 bytes per state element per chunk)
        "k_phi": ("mfma", 8 * dm * S * N),
        "k_lin_delta": ("mfma", 2 * dm * S * N),
        "k_lin_apply": ("mfma", 2 * dm * S * N),
        "k_lin_scan": ("hbm", 8 * dm * S * nchunks),
        # W1 | W3 of the H weight blocks read in fp32 and written in bf16
        "k_w13_cvt": ("hbm", (4 + es) * 2 * dm * H),
        # sliding-window attention: 4d FLOP per (query, key) pair inside the windows (algorithmic)
        "k_swa": ("mfma", 4 * d * B * H * (chunk * (chunk + 1) // 2 + (N - chunk) * chunk)),
        "k_swa_qprep": ("hbm", 2 * 2 * B * H * N * d),
        "k_swa_vprep": ("hbm", 2 * 2 * B * H * N * d),
        # parallel form with Muon: every chunk's W2 update read and its momentum written (fp32)
        "k_par_momentum": ("hbm", 8 * dm * S * nchunks),
    }
    dom_ms, dom_n = prof[dom]
    avg = dom_ms / max(dom_n, 1)
    bound, amount = work[dom]
    if bound == "mfma":
        ach = amount / (avg * 1e-3) / 1e12
        peak, unit, key = BF16_PEAK_TFLOPS, "TFLOP/s", "flop_per_launch"
    else:
        ach = amount / (avg * 1e-3) / 1e9
        peak, unit, key = HBM_PEAK_GBS, "GB/s", "bytes_per_launch"
    roofline = {"kernel": dom, "bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
                "frac": round(ach / peak, 4), "traffic": measured_traffic(dom), "traffic_unit": "bytes/launch", "avg_launch_us": round(avg * 1e3, 2),
                "launches": dom_n, key: amount}
    # the same against the rates this device sustains (vendor peaks above remain the roofline)
    peaks = measured_peaks(torch, C)
    mpeak = peaks["bf16_mfma_TFLOPs"] if bound == "mfma" else peaks["copy_GBps"]
    roofline.update({"measured_peak": mpeak, "frac_of_measured": round(ach / mpeak, 4)})
    # per-kernel breakdown: a short pass after the timed region with every launch bracketed
    nb = min(args.steps, 3)
    C.profile_select(None)
    C.profile_enable(True)
    C.profile_read()
    for _ in range(nb):
        call()
    torch.cuda.synchronize()
    brk = C.profile_read()
    C.profile_enable(False)
    kernels = {}
    for kname, (t, n) in brk.items():
        if not n:
            continue
        kb, kw = work.get(kname, (None, None))
        kernels[kname] = {"ms_per_step": round(t / nb, 4), "launches_per_step": n / nb}
        if kb is not None:
            rate = kw / (t / n * 1e-3) / (1e12 if kb == "mfma" else 1e9)
            kernels[kname]["frac_of_" + ("bf16_mfma" if kb == "mfma" else "hbm")] = round(
                rate / (BF16_PEAK_TFLOPS if kb == "mfma" else HBM_PEAK_GBS), 4)

    # ---------------- parity of sampled slices + CPU baseline (fp64 oracle) ----------------
    out = {}
    parity = None
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        # scans in an order that visits every batch and head early; the oracle stops at the time cap
        order = [(i % B, (i + i // B) % H) for i in range(B * H)]
        print(f"[bench] fp64 oracle on up to {len(order)} scans ({args.oracle_seconds:.0f} s cap)",
              file=sys.stderr, flush=True)
        o_host = o.float().cpu().numpy()
        W_host = W_out.cpu().numpy()
        errs_o, errs_w, done = [], [], []
        t0 = time.perf_counter()
        for (b, h) in order:
            qs, ks, vs, es = exact[(b, h)]
            o_ref, W_ref, _ = O.ttt_scan_ref(qs, ks, vs, es, *Wh[h], chunk, O.MASK_APPLY_THEN_UPDATE, rule, 5, beta,
                                             par)
            done.append((b, h))
            og = o_host[b, h].astype(np.float64)
            errs_o.append(float(np.linalg.norm(og - o_ref) / np.linalg.norm(o_ref)))
            Wg = W_host[b, h].astype(np.float64)
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
        parity = {"scans": len(done), "max_rel_l2_o": max(errs_o), "max_rel_l2_W": max(errs_w),
                  "tol": 2e-2, "ok": max(errs_o) <= 2e-2 and max(errs_w) <= 2e-2}
        del exact, o_host, W_host

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
        # the same two launch-bound calls captured once into a HIP graph and replayed: the tiny layer
        # (4 chunks, a few microseconds of work per launch) and the strided mask (12 Muon updates,
        # about 140 launches)
        print("[bench] extras: graph replay", file=sys.stderr, flush=True)
        q1, k1, v1, e1, W01 = gpu_inputs(torch, 1, 1, 256, 32, 32, 2500 + args.seed)
        q1, k1, v1 = q1.float(), k1.float(), v1.float()
        D1, _ = T.ttt_desc(1, 1, 256, 32, 32, 64, C.TTT_F32, C.MASK_APPLY_THEN_UPDATE, C.UPD_GD_L2)
        ws1 = torch.empty(max(1, T.ttt_workspace_bytes(D1)), dtype=torch.uint8, device="cuda")
        o1 = torch.empty_like(q1)
        tiny = lambda: T.ttt_forward(q1, k1, v1, e1, W01, 64, C.MASK_APPLY_THEN_UPDATE, C.UPD_GD_L2,  # noqa: E731
                                     m_h=32, out=o1, want_W=False, workspace=ws1)
        st_g = max(20, args.steps)
        ms1e, ms1g = time_calls(torch, tiny, st_g, 3), graph_replay_ms(torch, tiny, st_g)
        q5, k5, v5, e5, W05 = gpu_inputs(torch, B5, H5, N5, d5, m5, 2000 + args.seed)
        ws5 = torch.empty(T.ttt_workspace_bytes(D5), dtype=torch.uint8, device="cuda")
        o5 = torch.empty_like(q5)
        nvs = lambda: T.ttt_forward(q5, k5, v5, e5, W05, c5, C.MASK_STRIDED, C.UPD_MUON_L2, m_h=m5,  # noqa: E731
                                    update_chunks=flags, out=o5, want_W=False, workspace=ws5)
        ms5e, ms5g = time_calls(torch, nvs, st, 1), graph_replay_ms(torch, nvs, st)
        extras["graph_replay"] = {
            "tiny_layer": {"workload": "B1 H1 N256 d32 m32 chunk 64 fp32, L2-Normalize(W - g)",
                           "eager_ms_per_call": round(ms1e, 4), "graph_ms_per_call": round(ms1g, 4)},
            "nvs_strided_muon": {"eager_ms_per_call": round(ms5e, 3), "graph_ms_per_call": round(ms5g, 3)}}
        del q1, k1, v1, e1, W01, ws1, o1, q5, k5, v5, e5, W05, ws5, o5
        print("[bench] extras: linear attention", file=sys.stderr, flush=True)
        B2, H2, N2, d2, c2 = 4, 16, 8192, 128, 256
        q2, k2, v2, e2, _ = gpu_inputs(torch, B2, H2, N2, d2, 0, 3000 + args.seed, "sigmoid", 0.05)
        o2 = torch.empty_like(q2)
        lin_bytes = B2 * H2 * N2 * (4 * d2 * 2 + 4)
        for name, mask in (("linattn_chunked", C.MASK_APPLY_THEN_UPDATE), ("linattn_token_causal", C.MASK_TOKEN_CAUSAL)):
            Dl, _ = T.linattn_desc(B2, H2, N2, d2, d2, c2, C.TTT_BF16, mask)
            wsl = torch.empty(max(1, T.linattn_workspace_bytes(Dl)), dtype=torch.uint8, device="cuda")
            msl = time_calls(torch, lambda: T.linattn_forward(q2, k2, v2, e2, c2, mask, out=o2, want_S=False,
                                                              workspace=wsl), max(st, 10), 2)
            del wsl
            extras[name] = {"tokens_per_s": round(B2 * N2 / (msl * 1e-3)), "ms_per_call": round(msl, 4),
                            "hbm_GBps": round(lin_bytes / (msl * 1e-3) / 1e9, 1),
                            "hbm_frac": round(lin_bytes / (msl * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "workload": f"B{B2} H{H2} N{N2} d_k=d_v={d2} chunk {c2} bf16"}
        # the backward of the chunked mask at the same shape (the gradients that training through the
        # parallel form needs), with its kernels' times from one bracketed pass after the timed calls
        print("[bench] extras: linear-attention backward", file=sys.stderr, flush=True)
        gb = torch.Generator(device="cuda")
        gb.manual_seed(3500 + args.seed)
        dO2 = (torch.randn((B2, H2, N2, d2), generator=gb, device="cuda") / d2 ** 0.5).to(torch.bfloat16)
        Db, _ = T.linattn_desc(B2, H2, N2, d2, d2, c2, C.TTT_BF16, C.MASK_APPLY_THEN_UPDATE)
        wsb = torch.empty(max(1, T.linattn_backward_workspace_bytes(Db)), dtype=torch.uint8, device="cuda")
        bwd = lambda: T.linattn_backward(q2, k2, v2, e2, dO2, c2, C.MASK_APPLY_THEN_UPDATE, want_dS0=False,  # noqa: E731
                                         workspace=wsb)
        msb = time_calls(torch, bwd, max(st, 10), 2)
        C.profile_select(None)
        C.profile_enable(True)
        C.profile_read()
        for _ in range(3):
            bwd()
        torch.cuda.synchronize()
        bk = {kn: round(t / 3, 4) for kn, (t, n) in C.profile_read().items() if n}
        C.profile_enable(False)
        # algorithmic bytes: q, k, v, dO and eta in, dq, dk, dv and deta out; algorithmic flops: the two
        # chunk-update sums (eta v k^T, dO q^T) and the three gradient products, 2 d_k d_v each per token
        bwd_bytes = B2 * H2 * N2 * (7 * d2 * 2 + 8)
        bwd_flops = B2 * H2 * N2 * 10 * d2 * d2
        extras["linattn_backward"] = {
            "tokens_per_s": round(B2 * N2 / (msb * 1e-3)), "ms_per_call": round(msb, 4),
            "hbm_GBps": round(bwd_bytes / (msb * 1e-3) / 1e9, 1),
            "hbm_frac": round(bwd_bytes / (msb * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_frac": round(bwd_flops / (msb * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "over_forward": round(msb / extras["linattn_chunked"]["ms_per_call"], 2),
            "kernels_ms": bk,
            "workload": f"B{B2} H{H2} N{N2} d_k=d_v={d2} chunk {c2} bf16, apply-then-update, dO given"}
        del dO2, wsb
        # the SwiGLU layer at the same shape (m = 2d), for the linear-vs-SwiGLU comparison
        m2 = 2 * d2
        W02 = torch.randn((H2, 3 * d2 * m2), device="cuda") / d2 ** 0.5
        Ds, _ = T.ttt_desc(B2, H2, N2, d2, m2, c2, C.TTT_BF16, C.MASK_APPLY_THEN_UPDATE, C.UPD_GD_L2)
        wss = torch.empty(T.ttt_workspace_bytes(Ds), dtype=torch.uint8, device="cuda")
        mss = time_calls(torch, lambda: T.ttt_forward(q2, k2, v2, e2, W02, c2, C.MASK_APPLY_THEN_UPDATE, C.UPD_GD_L2,
                                                      m_h=m2, out=o2, workspace=wss), st, 1)
        extras["swiglu_at_linattn_shape"] = {"tokens_per_s": round(B2 * N2 / (mss * 1e-3)), "ms_per_call": round(mss, 3),
                                             "m_h": m2, "linattn_speedup": round(mss / extras["linattn_chunked"]["ms_per_call"], 2)}
        del q2, k2, v2, e2, o2, W02, wss
        # and the reverse: linear attention at the LaCT LM layer's shape (d_k = d_v = d_h, chunk 2048),
        # on the headline inputs, against the SwiGLU layer's time measured above
        print("[bench] extras: linear attention at the LaCT LM shape", file=sys.stderr, flush=True)
        Dll, _ = T.linattn_desc(B, H, N, d, d, chunk, C.TTT_BF16, C.MASK_APPLY_THEN_UPDATE)
        wsll = torch.empty(max(1, T.linattn_workspace_bytes(Dll)), dtype=torch.uint8, device="cuda")
        oll = torch.empty_like(q)
        msll = time_calls(torch, lambda: T.linattn_forward(q, k, v, eta, chunk, C.MASK_APPLY_THEN_UPDATE, out=oll,
                                                           want_S=False, workspace=wsll), max(st, 10), 2)
        ll_bytes = B * H * N * (4 * d * 2 + 4)
        extras["linattn_at_lact_lm_shape"] = {
            "tokens_per_s": round(tokens / (msll * 1e-3)), "ms_per_call": round(msll, 4),
            "hbm_GBps": round(ll_bytes / (msll * 1e-3) / 1e9, 1),
            "hbm_frac": round(ll_bytes / (msll * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "workload": f"B{B} H{H} N{N} d_k=d_v={d} chunk {chunk} bf16, apply-then-update",
            "swiglu_layer_ms_per_call": round(ms, 3), "linattn_speedup": round(ms / msll, 2)}
        del wsll, oll
        # last-layer-only plain GD on the headline inputs: the chunk recurrence against the parallel
        # static-kernel form (features, then chunked linear attention with W2 as the state)
        print("[bench] extras: last-layer GD, recurrence and parallel form", file=sys.stderr, flush=True)
        msp = {}
        for pf in (False, True):
            Dp, _ = T.ttt_desc(B, H, N, d, m, chunk, C.TTT_BF16, C.MASK_APPLY_THEN_UPDATE, C.UPD_GD, 5, 0.0,
                               last_layer_only=True, parallel_form=pf)
            wsp = torch.empty(max(1, T.ttt_workspace_bytes(Dp)), dtype=torch.uint8, device="cuda")
            msp[pf] = time_calls(torch, lambda: T.ttt_forward(q, k, v, eta, W0, chunk, C.MASK_APPLY_THEN_UPDATE,
                                                              C.UPD_GD, m_h=m, last_layer_only=True, parallel_form=pf,
                                                              out=o, workspace=wsp), st, 1)
            del wsp
        extras["lact_lm_last_layer_gd"] = {
            "workload": f"B{B} H{H} N{N} d{d} m{m} chunk {chunk} bf16, apply-then-update, only W2 learns, W - g "
                        "(plain GD: no momentum, no Muon, no weight norm)",
            "recurrence_ms_per_call": round(msp[False], 3), "parallel_form_ms_per_call": round(msp[True], 3),
            "parallel_form_tokens_per_s": round(tokens / (msp[True] * 1e-3)),
            "parallel_form_speedup": round(msp[False] / msp[True], 2)}
        # its backward (the outer-loop gradients of q, k, v, eta and W0 from dO), the training-side twin
        print("[bench] extras: last-layer GD backward", file=sys.stderr, flush=True)
        gb = torch.Generator(device="cuda")
        gb.manual_seed(3600 + args.seed)
        dOl = (torch.randn((B, H, N, d), generator=gb, device="cuda") / d ** 0.5).to(torch.bfloat16)
        Dg, _ = T.ttt_desc(B, H, N, d, m, chunk, C.TTT_BF16, C.MASK_APPLY_THEN_UPDATE, C.UPD_GD, 0, 0.0,
                           last_layer_only=True)
        wsg = torch.empty(T.ttt_backward_workspace_bytes(Dg), dtype=torch.uint8, device="cuda")
        lbwd = lambda: T.ttt_backward(q, k, v, eta, W0, dOl, chunk, C.MASK_APPLY_THEN_UPDATE, m_h=m,  # noqa: E731
                                      workspace=wsg)
        msg = time_calls(torch, lbwd, st, 1)
        C.profile_select(None)
        C.profile_enable(True)
        C.profile_read()
        for _ in range(3):
            lbwd()
        torch.cuda.synchronize()
        gk = {kn: round(t / 3, 4) for kn, (t, n) in C.profile_read().items() if n}
        C.profile_enable(False)
        # algorithmic flops per token and scan: the features again (a and c of q and k, 8 d m), the
        # linear-attention backward over d_k = m, d_v = d (the chunk states again, the query-gradient
        # sums, dphi(q), dphi(k), dv: 10 d m), dq and dk (8 d m), dW1 and dW3 (8 d m)
        gflops = tokens * H * 34 * d * m
        # the same layer trained through its recurrence: the forward keeping its record, then the
        # recurrence walked back (W1, W3 frozen), against the parallel forward and its backward
        rb_, rw_ = T.ttt_record_bytes(Dg)
        recg = torch.empty(rb_, dtype=torch.uint8, device="cuda")
        wsr_ = torch.empty(max(1, rw_), dtype=torch.uint8, device="cuda")

        def rec_step():
            T.ttt_forward_record(q, k, v, eta, W0, chunk, C.MASK_APPLY_THEN_UPDATE, C.UPD_GD, m_h=m,
                                 last_layer_only=True, out=o, record=recg, workspace=wsr_)
            T.ttt_backward(q, k, v, eta, W0, dOl, chunk, C.MASK_APPLY_THEN_UPDATE, m_h=m, record=recg)

        msr = time_calls(torch, rec_step, 1, 1)
        del recg, wsr_
        extras["lact_lm_last_layer_gd_backward"] = {
            "workload": f"B{B} H{H} N{N} d{d} m{m} chunk {chunk} bf16, apply-then-update, only W2 learns (plain "
                        "GD): gradients of q, k, v, eta and the per-head W0 from dO",
            "ms_per_call": round(msg, 3), "tokens_per_s": round(tokens / (msg * 1e-3)),
            "algorithmic_tflop": round(gflops / 1e12, 3),
            "mfma_frac": round(gflops / (msg * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "over_parallel_forward": round(msg / msp[True], 2),
            "training_step_ms": round(msg + msp[True], 3),
            "recurrence_training_step_ms": round(msr, 3),
            "parallel_form_training_speedup": round(msr / (msg + msp[True]), 2), "kernels_ms": gk}
        # the headline layer's backward (all three weights learning, GD + L2): the forward again for its
        # record, then the reverse of the chunk recurrence
        print("[bench] extras: GD + L2 backward, all weights learning", file=sys.stderr, flush=True)
        Df, _ = T.ttt_desc(B, H, N, d, m, chunk, C.TTT_BF16, C.MASK_APPLY_THEN_UPDATE, C.UPD_GD_L2, 0, 0.0)
        wsf = torch.empty(T.ttt_backward_workspace_bytes(Df), dtype=torch.uint8, device="cuda")
        fbwd = lambda: T.ttt_backward(q, k, v, eta, W0, dOl, chunk, C.MASK_APPLY_THEN_UPDATE, m_h=m,  # noqa: E731
                                      update_rule=C.UPD_GD_L2, last_layer_only=False, workspace=wsf)
        msf = time_calls(torch, fbwd, st, 1)
        C.profile_select(None)
        C.profile_enable(True)
        C.profile_read()
        for _ in range(3):
            fbwd()
        torch.cuda.synchronize()
        fk = {kn: round(t / 3, 4) for kn, (t, n) in C.profile_read().items() if n}
        C.profile_enable(False)
        # algorithmic flops per token and scan: the forward again without outputs (a, c and v W2 of the
        # keys, the three chunk gradients: 12 d m), then the key tiles' two passes (12 d m), the query
        # tiles (6 d m), dk (8 d m), dv (4 d m), dq (4 d m) and the weight gradients over keys and
        # queries (12 d m)
        fflops = tokens * H * 58 * d * m
        # the training pair: the forward keeps a record, the backward reads it instead of running the
        # forward again
        rbytes, rws = T.ttt_record_bytes(Df)
        rec = torch.empty(rbytes, dtype=torch.uint8, device="cuda")
        wsr = torch.empty(max(1, rws), dtype=torch.uint8, device="cuda")
        nbr = ctypes.c_size_t(0)
        C.check(C.lib().ttt_backward_record_workspace_bytes(ctypes.byref(Df), ctypes.byref(nbr)))
        wsb = torch.empty(nbr.value, dtype=torch.uint8, device="cuda")

        def train_step():
            T.ttt_forward_record(q, k, v, eta, W0, chunk, C.MASK_APPLY_THEN_UPDATE, C.UPD_GD_L2, m_h=m, out=o,
                                 record=rec, workspace=wsr)
            T.ttt_backward(q, k, v, eta, W0, dOl, chunk, C.MASK_APPLY_THEN_UPDATE, m_h=m, update_rule=C.UPD_GD_L2,
                           last_layer_only=False, record=rec, workspace=wsb)

        mst = time_calls(torch, train_step, st, 1)
        del rec, wsr, wsb
        extras["lact_lm_gd_l2_backward"] = {
            "workload": f"B{B} H{H} N{N} d{d} m{m} chunk {chunk} bf16, apply-then-update, GD + L2 with all three "
                        "weights learning: gradients of q, k, v, eta and the per-head W0 from dO",
            "ms_per_call": round(msf, 3), "tokens_per_s": round(tokens / (msf * 1e-3)),
            "algorithmic_tflop": round(fflops / 1e12, 3),
            "mfma_frac": round(fflops / (msf * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "over_forward": round(msf / ms, 2), "training_step_ms": round(msf + ms, 3),
            "training_step_with_record_ms": round(mst, 3),
            "workspace_GB": round(wsf.numel() / 1e9, 2), "kernels_ms": fk}
        del wsf
        # the Muon + momentum layer's backward (Newton-Schulz walked back in fp32 on every update)
        print("[bench] extras: Muon + momentum backward, all weights learning", file=sys.stderr, flush=True)
        Dm_, _ = T.ttt_desc(B, H, N, d, m, chunk, C.TTT_BF16, C.MASK_APPLY_THEN_UPDATE, C.UPD_MUON_L2, 5, 0.9)
        wsm = torch.empty(T.ttt_backward_workspace_bytes(Dm_), dtype=torch.uint8, device="cuda")
        mbwd = lambda: T.ttt_backward(q, k, v, eta, W0, dOl, chunk, C.MASK_APPLY_THEN_UPDATE, m_h=m,  # noqa: E731
                                      update_rule=C.UPD_MUON_L2, momentum=0.9, last_layer_only=False, workspace=wsm)
        msm = time_calls(torch, mbwd, 1, 1)
        C.profile_select(None)
        C.profile_enable(True)
        C.profile_read()
        mbwd()
        torch.cuda.synchronize()
        mk = {kn: round(t, 3) for kn, (t, n) in C.profile_read().items() if n}
        C.profile_enable(False)
        extras["lact_lm_muon_momentum_backward"] = {
            "workload": f"B{B} H{H} N{N} d{d} m{m} chunk {chunk} bf16, apply-then-update, L2-Normalize(W - Muon(M)), "
                        "M <- 0.9 M + g, 5 NS steps, all three weights learning: gradients of q, k, v, eta and W0",
            "ms_per_call": round(msm, 3), "tokens_per_s": round(tokens / (msm * 1e-3)),
            "workspace_GB": round(wsm.numel() / 1e9, 2), "kernels_ms": mk}
        del dOl, wsg, wsm
        # Variant 2 of the paper's ablation: only W2 learns, momentum 0.9, per-token eta and Muon (5
        # Newton-Schulz steps) kept, no weight norm; chunk recurrence against the parallel form
        print("[bench] extras: Variant 2 (last layer, Muon + momentum), recurrence and parallel form",
              file=sys.stderr, flush=True)
        msv = {}
        for pf in (False, True):
            Dv, _ = T.ttt_desc(B, H, N, d, m, chunk, C.TTT_BF16, C.MASK_APPLY_THEN_UPDATE, C.UPD_MUON, 5, 0.9,
                               last_layer_only=True, parallel_form=pf)
            wsv = torch.empty(max(1, T.ttt_workspace_bytes(Dv)), dtype=torch.uint8, device="cuda")
            Mv = torch.zeros((B, H, 3 * d * m), dtype=torch.float32, device="cuda")
            msv[pf] = time_calls(torch, lambda: T.ttt_forward(q, k, v, eta, W0, chunk, C.MASK_APPLY_THEN_UPDATE,
                                                              C.UPD_MUON, m_h=m, momentum=0.9, M=Mv,
                                                              last_layer_only=True, parallel_form=pf, out=o,
                                                              workspace=wsv), st, 1)
            del wsv, Mv
        # LaCT's sliding-window attention beside the layer: window = chunk, on the headline q, k, v
        print("[bench] extras: sliding-window attention", file=sys.stderr, flush=True)
        Dw = C.SwaDesc(B, H, N, d, chunk, C.TTT_BF16)
        wsw = torch.empty(T.swa_workspace_bytes(Dw), dtype=torch.uint8, device="cuda")
        gen = torch.Generator(device="cuda")
        gen.manual_seed(4000 + args.seed)
        qs_ = 0.5 + torch.rand((H, d), generator=gen, device="cuda")
        qb_ = 0.3 * torch.randn((H, d), generator=gen, device="cuda")
        ks_ = 0.5 + torch.rand((H, d), generator=gen, device="cuda")
        msw = time_calls(torch, lambda: T.swa_forward(q, k, v, chunk, q_scale=qs_, q_shift=qb_, k_scale=ks_, out=o,
                                                      workspace=wsw), st, 1)
        pairs = B * H * (chunk * (chunk + 1) // 2 + (N - chunk) * chunk)  # (query, key) pairs in windows
        fsw = 4 * d * pairs  # q'' . k and p v: 2d each per pair
        extras["sliding_window_attention"] = {
            "workload": f"B{B} H{H} N{N} d{d}, causal window {chunk} (= the chunk), bf16, per-channel scale/shift",
            "ms_per_call": round(msw, 3), "tokens_per_s": round(tokens / (msw * 1e-3)),
            "algorithmic_tflop": round(fsw / 1e12, 3),
            "mfma_frac": round(fsw / (msw * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "note": "query-resident walk (one workgroup of 128 queries per CU, keys in blocks of 32) after "
                    "a pass that rearranges v; the executed FLOPs are the algorithmic ones"}
        del wsw
        extras["lact_lm_variant2_muon"] = {
            "workload": f"B{B} H{H} N{N} d{d} m{m} chunk {chunk} bf16, apply-then-update, only W2 learns, "
                        "momentum 0.9 + Muon (5 steps), no weight norm",
            "recurrence_ms_per_call": round(msv[False], 3), "parallel_form_ms_per_call": round(msv[True], 3),
            "recurrence_tokens_per_s": round(tokens / (msv[False] * 1e-3)),
            "parallel_form_tokens_per_s": round(tokens / (msv[True] * 1e-3)),
            "parallel_form_speedup": round(msv[False] / msv[True], 2),
            "pages_context": "Table 2 Variant 2 on the pages' (unstated) hardware: 11.02 M tokens/s recurrent, "
                             "30.18 M parallel"}

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1)/sqrt(d) q,k,v in bf16, eta = 0.01 softplus(N(0,1)), W0 ~ N(0,1/d) per head",
        "config": {"workload": "lact_lm_layer_b8_h4_n32768_d384_m768_chunk2048_" + args.update, "B": B, "H": H,
                   "seq_len": N, "d_h": d, "m_h": m, "chunk": chunk, "mask": "apply_then_update",
                   "update": {"gd_l2": "L2-Normalize(W - g)",
                              "muon_momentum": "L2-Normalize(W - Muon(M)), M <- 0.9 M + g, 5 NS steps",
                              "last_layer_gd_parallel": "only W2 learns, W - g, parallel static-kernel form"}[args.update],
                   "parallelism": "none (one GPU)"},
        "mfma_frac_layer": round(layer_tflops / BF16_PEAK_TFLOPS, 4),
        "layer_tflops": round(layer_tflops, 2),
        "algorithmic_tflop_per_step": round(flops / 1e12, 4),
        "algorithmic_gb_per_step": round(lact_bytes(B, H, N, d, m, 2, nchunks) / 1e9, 3),
        "roofline": roofline,
        "measured_peaks": peaks,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "parity": parity,
        "extras": extras,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""GPU parity of swa_forward (LaCT's sliding-window attention, through the C ABI) against the fp64
oracle: relative L2 <= 1e-5 with fp32 inputs and <= 2e-2 with bf16 inputs, over the whole tensor,
per (batch, head), per window-sized block of rows and (times 5) per row."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O
import synth
import linear_attention_chunk_amd as T
from gpu_util import assert_close, dev, host, say

pytestmark = pytest.mark.gpu

TOL = {False: 1e-5, True: 2e-2}


def params(seed, H, d):
    rng = np.random.default_rng(seed)
    return [(0.5 + rng.random((H, d))).astype(np.float32), (0.3 * rng.standard_normal((H, d))).astype(np.float32),
            (0.5 + rng.random((H, d))).astype(np.float32), (0.3 * rng.standard_normal((H, d))).astype(np.float32)]


def run(seed, B, H, N, d, window, bf16, affine=True):
    say(f"swa case B{B} H{H} N{N} d{d} window{window} bf16={bf16} affine={affine}")
    q, k, v, _ = synth.make_linattn_inputs(seed, B, H, N, d, d, bf16)
    dt = torch.bfloat16 if bf16 else torch.float32
    ps = params(seed + 7, H, d) if affine else [None] * 4
    o = T.swa_forward(dev(q, dt), dev(k, dt), dev(v, dt), window, q_scale=None if ps[0] is None else dev(ps[0]),
                      q_shift=None if ps[1] is None else dev(ps[1]), k_scale=None if ps[2] is None else dev(ps[2]),
                      k_shift=None if ps[3] is None else dev(ps[3]))
    torch.cuda.synchronize()
    o_ref = O.swa_forward_ref(q, k, v, window, *ps)
    assert_close(host(o), o_ref, TOL[bf16], "o", min(window, 256))
    return o, (q, k, v)


@pytest.mark.parametrize("bf16", [False, True])
def test_ragged_and_window_edges(bf16):
    # 300 tokens: two 128-query blocks and a tail of 44; a window of 100 starts mid key block
    run(1, 1, 2, 300, 64, 100, bf16)
    # several key blocks per query block, the window not a multiple of 64
    run(2, 2, 2, 700, 128, 257, bf16)


@pytest.mark.parametrize("bf16", [False, True])
def test_window_covering_the_sequence_and_one_token_window(bf16):
    run(3, 1, 1, 333, 96, 5000, bf16)          # full causal attention
    o, (q, k, v) = run(4, 1, 2, 200, 32, 1, bf16, affine=False)
    assert np.array_equal(host(o), np.asarray(v, np.float64))   # each token sees itself only: o = v


@pytest.mark.parametrize("d", [256, 320, 384])
def test_wide_heads_bf16(d):
    # 256: one workgroup per query block; 320 and 384: two column blocks of 192 (the second partial at 320)
    run(5, 1, 2, 400, d, 150, True)


@pytest.mark.parametrize("d", [192, 384])
def test_wide_heads_fp32(d):
    run(6, 1, 1, 260, d, 130, False)


@pytest.mark.parametrize("d", [64, 128, 192])
def test_mid_widths_bf16(d):
    # several 128-query blocks (the last ragged) and windows over many 32-key blocks
    run(10, 1, 2, 500, d, 300, True)


@pytest.mark.parametrize("d", [128, 384])
def test_growing_scores_bf16(d):
    """Scores that rise along the sequence (keys along one direction with a growing length), so a
    query's running maximum keeps jumping by several units from one key block to the next: the
    kernel's rescale of the output rows runs many times."""
    N, w = 600, 400
    say(f"swa growing scores N{N} d{d} window {w}")
    rng = np.random.default_rng(11 + d)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = np.sqrt(d) * u[None, :] + 0.1 * rng.standard_normal((N, d))
    k = (np.arange(N) / 8.0)[:, None] * u[None, :] + 0.1 * rng.standard_normal((N, d))
    v = rng.standard_normal((N, d)) / np.sqrt(d)
    q, k, v = (synth.round_to_bf16(x.astype(np.float32))[None, None] for x in (q, k, v))
    o = T.swa_forward(dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16), w)
    torch.cuda.synchronize()
    o_ref = O.swa_forward_ref(q, k, v, w)
    assert_close(host(o), o_ref, TOL[True], "o", 256)


def test_lact_lm_shape_sampled():
    """B8 H4 N32768 d384, window = chunk = 2048 (the LaCT language-model layer's local branch); two
    (batch, head) slices from the seeded generator, the rest from torch's seeded device generator."""
    B, H, N, d, w = 8, 4, 32768, 384, 2048
    sample = [(0, 0), (7, 3)]
    say(f"swa full size B{B} H{H} N{N} d{d} window {w}")
    g = torch.Generator(device="cuda")
    g.manual_seed(88)
    s = 1.0 / np.sqrt(d)
    q = (torch.randn((B, H, N, d), generator=g, device="cuda") * s).to(torch.bfloat16)
    k = (torch.randn((B, H, N, d), generator=g, device="cuda") * s).to(torch.bfloat16)
    v = (torch.randn((B, H, N, d), generator=g, device="cuda") * s).to(torch.bfloat16)
    ex = {}
    for b, h in sample:
        qs, ks, vs, _ = synth.slice_inputs(0, b, h, N, d, d, "sigmoid", 0.05, True)
        q[b, h], k[b, h], v[b, h] = dev(qs, torch.bfloat16), dev(ks, torch.bfloat16), dev(vs, torch.bfloat16)
        ex[(b, h)] = (qs, ks, vs)
    ps = params(9, H, d)
    o = T.swa_forward(q, k, v, w, q_scale=dev(ps[0]), q_shift=dev(ps[1]), k_scale=dev(ps[2]), k_shift=dev(ps[3]))
    torch.cuda.synchronize()
    for b, h in sample:
        qs, ks, vs = ex[(b, h)]
        o_ref = O.swa_scan_ref(qs, ks, vs, w, ps[0][h], ps[1][h], ps[2][h], ps[3][h])
        say(f"  slice ({b},{h})")
        assert_close(host(o[b, h]), o_ref, 2e-2, "o", w)

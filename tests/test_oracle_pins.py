"""Pins of the CPU oracle to facts other than itself (no GPU needed).

Each test ties one step of the oracle to something the pages, the number
formats or plain mathematics fix: a library decoder of the same format, a
closed form, an invariant, brute force on tiny inputs, or a hand-derived
example.  A plausible slip in the oracle (a dropped term, a wrong sign, a
transposed block index, gate and up swapped, a weight from the biased score)
fails at least one of them.
"""

import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import moe_oracle as mo
from synth import LayerShape, make_layer, make_layer_from_arrays, quantize_blocks, WORKLOADS
from synth import f32_to_bf16_bits


# --------------------------------------------------------------- encodings

def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_codes_to_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.nanmax(got) == 448.0 and got[1] == 2.0 ** -9


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 16, 4096, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # drop inf / nan patterns
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), ref)


def test_e8m0_decode_matches_torch():
    b = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(oracle.e8m0_bytes_to_f64(b), ref)
    assert np.isnan(oracle.e8m0_bytes_to_f64(np.array([255], np.uint8)))[0]


@pytest.mark.parametrize("fmt", ["fp32", "e8m0"])
def test_block_dequant_recovers_weights(fmt):
    """Dequantised blocks equal the original weights to the e4m3 rounding
    bound: |w - q*s| <= s*2^-4 relative to the code (3 mantissa bits) and
    <= s*2^-10 in the subnormal range.  A transposed or shifted block index
    breaks this by orders of magnitude (the blocks are scaled very
    differently below)."""
    rng = np.random.default_rng(2)
    R, C = 256, 384
    w = rng.standard_normal((R, C)).astype(np.float32)
    w *= np.repeat(np.repeat(np.exp2(rng.integers(-6, 6, (R // 128, C // 128))), 128, 0),
                   128, 1).astype(np.float32)
    codes, scales = quantize_blocks(w, fmt)
    deq = oracle.dequantize(codes, scales)
    s = np.repeat(np.repeat(mo.scales_to_f64(scales), 128, 0), 128, 1)
    err = np.abs(deq - w.astype(np.float64))
    bound = np.maximum(np.abs(w) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 1e-12)
    assert np.all(err <= bound)
    if fmt == "e8m0":
        sv = mo.scales_to_f64(scales)
        amax = np.abs(w.reshape(R // 128, 128, C // 128, 128)).max(axis=(1, 3))
        assert np.all(sv >= amax / 448) and np.all(sv < 2 * amax / 448)
        assert np.all(np.log2(sv) == np.round(np.log2(sv)))


def test_quantiser_rounding_cases():
    """Round to nearest even inside a block whose fp32 scale is exactly 1
    (amax = 448), and no NaN code from blocks with large amax."""
    w = np.zeros((128, 128), np.float32)
    w[0, :7] = [448.0, 2.0 ** -10, 1.5 * 2.0 ** -10, 3 * 2.0 ** -10, 1 + 1 / 16, 1 + 3 / 16, -300.0]
    codes, scales = quantize_blocks(w, "fp32")
    assert scales[0, 0] == 1.0
    vals = oracle.e4m3_codes_to_f64(codes[0, :7])
    assert vals.tolist() == [448.0, 0.0, 2.0 ** -9, 2.0 ** -8, 1.0, 1.25, -288.0]
    rng = np.random.default_rng(7)
    big = (rng.standard_normal((256, 256)) * 1e4).astype(np.float32)
    for fmt in ("fp32", "e8m0"):
        c, _ = quantize_blocks(big, fmt)
        v = oracle.e4m3_codes_to_f64(c)
        assert not np.isnan(v).any() and np.abs(v).max() <= 448.0


# ----------------------------------------------------------------- routing

def _brute_topk(key, k):
    """The k-subset with the largest key sum; among equal sums the one whose
    ascending id list is smallest (ties go to lower ids)."""
    best, best_ids = None, None
    for sub in itertools.combinations(range(len(key)), k):
        s = sum(key[i] for i in sub)
        if best is None or s > best + 1e-15:
            best, best_ids = s, sub
    return sorted(best_ids)


@pytest.mark.parametrize("E,k", [(8, 2), (16, 4), (12, 1), (6, 6)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_topk_brute_force(E, k, with_bias):
    rng = np.random.default_rng(E * 10 + k)
    for _ in range(20):
        scores = mo.sigmoid(rng.standard_normal((1, E)))
        bias = rng.normal(0, 0.1, E) if with_bias else None
        ids = oracle.select_experts(scores, bias, k)
        key = scores[0] + (bias if with_bias else 0)
        assert sorted(ids[0].tolist()) == _brute_topk(key, k)
        # descending order of the keys
        assert np.all(np.diff(key[ids[0]]) <= 0)


def test_topk_ties_go_to_lower_id():
    scores = np.full((1, 10), 0.5)
    scores[0, 7] = 0.9
    assert oracle.select_experts(scores, None, 3)[0].tolist() == [7, 0, 1]


def test_weights_use_unbiased_scores_and_sum_to_rsf():
    rng = np.random.default_rng(3)
    scores = mo.sigmoid(rng.standard_normal((50, 32)))
    bias = rng.normal(0, 0.3, 32)
    ids = oracle.select_experts(scores, bias, 6)
    w = oracle.route_weights(scores, ids, 2.5)
    assert np.allclose(w.sum(1), 2.5, rtol=0, atol=1e-12)
    sel = np.take_along_axis(scores, ids.astype(np.int64), 1)
    # weights are proportional to the scores themselves, not score + bias
    assert np.allclose(w / sel, (w / sel)[:, :1], rtol=1e-12)
    w1 = oracle.route_weights(scores, oracle.select_experts(scores, None, 1), 2.5)
    assert np.allclose(w1, 2.5, rtol=4e-16, atol=0)


def test_score_gap():
    scores = np.array([[0.1, 0.9, 0.5, 0.50001, 0.3]])
    assert np.isclose(oracle.score_gaps(scores, None, 2)[0], 0.00001)
    assert oracle.score_gaps(scores, None, 5)[0] == np.inf


def test_route_table_brute_force():
    rng = np.random.default_rng(4)
    for T, E, k in [(1, 8, 2), (5, 7, 3), (16, 32, 8), (3, 4, 4)]:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        counts, offsets, perm, inv = oracle.route_table(ids, E)
        exp_perm = [t * k + j for e in range(E) for t in range(T) for j in range(k)
                    if ids[t, j] == e]
        assert perm.tolist() == exp_perm
        assert counts.tolist() == [int((ids == e).sum()) for e in range(E)]
        assert offsets[0] == 0 and offsets[-1] == T * k
        for t in range(T):
            for j in range(k):
                assert perm[inv[t, j]] == t * k + j
                assert offsets[ids[t, j]] <= inv[t, j] < offsets[ids[t, j] + 1]


# ------------------------------------------------------------ expert math

def test_clamped_swiglu_closed_forms():
    L = 7.0
    g = np.array([2.0, -2.0, 8.0, 100.0, -50.0])
    u = np.array([2.0, 8.0, -9.0, 3.0, 1.0])
    got = oracle.clamped_swiglu(g, u, L)
    silu = lambda z: z / (1 + math.exp(-z))
    exp = [silu(2) * 2, silu(-2) * 7, silu(7) * -7, silu(7) * 3, silu(-50) * 1]
    assert np.allclose(got, exp, rtol=1e-15, atol=0)


def test_expert_mlp_tracks_unquantised_weights():
    """An expert on dequantised weights stays within the fp8 rounding error of
    the same expert on the fp32 weights it was quantised from (gate, up and
    down each use their own rows; swapping gate and up or transposing a block
    index moves the result far outside this bound)."""
    rng = np.random.default_rng(5)
    H, I, n = 256, 128, 3
    w13 = (rng.standard_normal((2 * I, H)) / 16).astype(np.float32)
    w2 = (rng.standard_normal((H, I)) / 11).astype(np.float32)
    x = rng.standard_normal((n, H))
    c13, s13 = quantize_blocks(w13, "fp32")
    c2, s2 = quantize_blocks(w2, "fp32")
    got = oracle.expert_mlp(oracle.dequantize(c13, s13), oracle.dequantize(c2, s2), x, 7.0)
    # the unquantised expert, written out per element with Python math
    ref = np.zeros((n, H))
    for t in range(n):
        gu = [sum(float(w13[r, c]) * x[t, c] for c in range(H)) for r in range(2 * I)]
        a = []
        for i in range(I):
            gg = min(gu[i], 7.0)
            uu = max(-7.0, min(7.0, gu[I + i]))
            a.append(gg / (1 + math.exp(-gg)) * uu)
        ref[t] = [sum(float(w2[r, i]) * a[i] for i in range(I)) for r in range(H)]
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    # e4m3 rounds each weight by up to 2^-4 relative (rms ~3.6%); two
    # projections in a row give ~5%
    assert rel < 0.08
    # and the element-wise agreement is far better than a swapped layout
    swapped = oracle.expert_mlp(np.concatenate([oracle.dequantize(c13, s13)[I:],
                                                oracle.dequantize(c13, s13)[:I]]),
                                oracle.dequantize(c2, s2), x, 7.0)
    assert np.linalg.norm(swapped - ref) / np.linalg.norm(ref) > 0.5


def test_rms_norm_closed_form():
    rng = np.random.default_rng(6)
    h = rng.standard_normal((4, 512)) * 3
    eps = 1e-5
    y = oracle.rms_norm(h, np.ones(512), eps)
    m = np.mean(h * h, axis=1)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), np.sqrt(m / (m + eps)), rtol=1e-13)
    g = rng.standard_normal(512)
    assert np.allclose(oracle.rms_norm(h, g, eps), y * g, rtol=1e-13)


# ------------------------------------------------------- hand-built layer

def _hand_layer(k=2):
    """Two experts, H = I = Is = 128, one token, every scale 1, gamma 1.

    x = 2 e0; router rows give logits (2, -2); expert 0: gate = up = 1 on
    column 0, down = 1 at [0, 0]; expert 1: gate = -1, up = 4 on column 0,
    down = 1 at [1, 0]; shared: gate = up = 4 on column 0, down = 1 at [2, 0];
    residual = e3.  Every value is exact in bf16 and e4m3.
    """
    H = I = 128
    sh = LayerShape(T=1, H=H, E=2, k=k, I=I, Is=I, scale_fmt="fp32", limit=7.0, rsf=2.5,
                    eps=1e-5, tag=999)
    e4 = lambda a: torch.from_numpy(np.asarray(a, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()
    x = np.zeros((1, H), np.float32); x[0, 0] = 2
    res = np.zeros((1, H), np.float32); res[0, 3] = 1
    wr = np.zeros((2, H), np.float32); wr[0, 0] = 1; wr[1, 0] = -1
    w13 = np.zeros((2, 2 * I, H), np.float32)
    w13[0, 0, 0] = 1; w13[0, I, 0] = 1
    w13[1, 0, 0] = -1; w13[1, I, 0] = 4
    w2 = np.zeros((2, H, I), np.float32); w2[0, 0, 0] = 1; w2[1, 1, 0] = 1
    sw13 = np.zeros((2 * I, H), np.float32); sw13[0, 0] = 4; sw13[I, 0] = 4
    sw2 = np.zeros((H, I), np.float32); sw2[2, 0] = 1
    one = lambda *s: np.ones(s, np.float32)
    return make_layer_from_arrays(
        sh, hidden=f32_to_bf16_bits(x), residual=f32_to_bf16_bits(res),
        router_w=f32_to_bf16_bits(wr), w13=e4(w13), w13_scale=one(2, 2, 1), w2=e4(w2),
        w2_scale=one(2, 1, 1), sw13=e4(sw13), sw13_scale=one(2, 1), sw2=e4(sw2),
        sw2_scale=one(1, 1), gamma=f32_to_bf16_bits(np.ones(H, np.float32)))


def _hand_expected(k):
    sig = lambda z: 1 / (1 + math.exp(-z))
    silu = lambda z: z * sig(z)
    a0, a1, a_s = silu(2) * 2, silu(-2) * 7, silu(7) * 7
    if k == 2:
        w = [2.5 * sig(2) / (sig(2) + sig(-2)), 2.5 * sig(-2) / (sig(2) + sig(-2))]
        h4 = [w[0] * a0, w[1] * a1, a_s, 1.0]
    else:
        w = [2.5]
        h4 = [w[0] * a0, 0.0, a_s, 1.0]
    ms = sum(v * v for v in h4) / 128
    out4 = [v / math.sqrt(ms + 1e-5) for v in h4]
    return w, h4, out4


@pytest.mark.parametrize("k", [2, 1])
@pytest.mark.parametrize("which", ["numpy", "c"])
def test_hand_two_expert_example(k, which, c_oracle):
    inp = _hand_layer(k)
    r = oracle.moe_layer(inp) if which == "numpy" else c_oracle.moe_layer(inp)
    w, h4, out4 = _hand_expected(k)
    assert r["ids"][0].tolist() == ([0, 1] if k == 2 else [0])
    assert np.allclose(r["weights"][0], w, rtol=1e-14)
    assert np.allclose(r["h"][0, :4], h4, rtol=1e-14)
    assert np.all(r["h"][0, 4:] == 0)
    # the finalized MoE output: h without the residual (e3)
    assert np.allclose(r["moe"][0, :4], h4[:3] + [0.0], rtol=1e-14, atol=1e-15)
    assert np.all(r["moe"][0, 4:] == 0)
    assert np.allclose(r["out"][0, :4], out4, rtol=1e-13)
    # the numbers themselves (k = 2): 2.2019926949447, 0.2980073050553, ...
    if k == 2:
        assert abs(w[0] - 2.201992694944706) < 1e-14
        assert abs(out4[2] - 11.17142897897562) < 1e-12


def test_hand_dense_layer():
    """A dense layer (no routed experts): the shared-expert weights of the
    hand-built layer above as the layer's MLP.  x = 2 e0, gate = up = 4 on
    column 0 give g = u = 8, clamped to 7; down = 1 at [2, 0]; residual e3:
    h = (0, 0, silu(7) * 7, 1, 0, ...)."""
    base = _hand_layer(2)
    sh = base.shape.replace(E=0, k=0, I=0)
    inp = make_layer_from_arrays(
        sh, hidden=base.hidden, residual=base.residual, sw13=base.sw13,
        sw13_scale=base.sw13_scale, sw2=base.sw2, sw2_scale=base.sw2_scale, gamma=base.gamma)
    r = oracle.moe_layer(inp)
    sig = lambda z: 1 / (1 + math.exp(-z))
    a_s = 7 * sig(7) * 7
    h4 = [0.0, 0.0, a_s, 1.0]
    assert r["ids"].shape == (1, 0)
    assert np.allclose(r["h"][0, :4], h4, rtol=1e-14, atol=0)
    assert np.all(r["h"][0, 4:] == 0)
    assert np.allclose(r["moe"][0, :4], [0.0, 0.0, a_s, 0.0], rtol=1e-14, atol=0)
    ms = sum(v * v for v in h4) / 128
    assert np.allclose(r["out"][0, :4], [v / math.sqrt(ms + 1e-5) for v in h4], rtol=1e-13)
    # the same numbers as the shared part of the two-expert example
    full = oracle.moe_layer(base)
    assert np.allclose(r["h"][0, 2], full["h"][0, 2], rtol=1e-15)


# ---------------------------------------------- the two oracles agree

@pytest.mark.parametrize("fmt", ["fp32", "e8m0"])
@pytest.mark.parametrize("with_bias", [False, True])
def test_c_and_numpy_oracles_agree(fmt, with_bias, c_oracle):
    sh = LayerShape(T=5, H=256, E=16, k=4, I=256, Is=128, scale_fmt=fmt, tag=500)
    inp = make_layer(sh, with_bias=with_bias, bias_std=0.1)
    a = oracle.moe_layer(inp)
    b = c_oracle.moe_layer(inp)
    assert np.array_equal(a["ids"], b["ids"])
    assert np.allclose(a["weights"], b["weights"], rtol=1e-13)
    assert np.allclose(a["gaps"], b["gaps"], rtol=1e-10, atol=1e-15)
    assert np.abs(a["out"] - b["out"]).max() <= 1e-12 * np.abs(a["out"]).max()
    rows = [3, 0]
    c = c_oracle.moe_layer(inp, rows=rows)
    assert np.allclose(c["out"], a["out"][rows], rtol=1e-12, atol=1e-12)
    forced = np.roll(a["ids"], 1, axis=1)
    d = oracle.moe_layer(inp, forced_ids=forced)
    e = c_oracle.moe_layer(inp, forced_ids=forced)
    assert np.abs(d["out"] - e["out"]).max() <= 1e-12 * np.abs(d["out"]).max()
    # forcing a permutation of the same experts leaves the output unchanged
    assert np.abs(d["out"] - a["out"]).max() <= 1e-12 * np.abs(a["out"]).max()


@pytest.mark.parametrize("name", ["tiny_t1", "decode_t1"])
def test_c_and_numpy_oracles_agree_on_workloads(name, c_oracle):
    """The two independent oracles on the tiny layer and the one-token decode
    layer (H = 4096, 128 experts, top-8, I = 1536) at their real sizes: the
    same experts and weights, and every output element within float64
    rounding of each other."""
    inp = make_layer(WORKLOADS[name])
    a = oracle.moe_layer(inp)
    b = c_oracle.moe_layer(inp)
    assert np.array_equal(a["ids"], b["ids"])
    assert np.allclose(a["weights"], b["weights"], rtol=1e-13)
    assert np.allclose(a["logits"], b["logits"], rtol=1e-12, atol=1e-14)
    for key in ("out", "h", "moe"):
        assert np.abs(a[key] - b[key]).max() <= 1e-12 * np.abs(a[key]).max(), key


def test_no_shared_expert(c_oracle):
    sh = LayerShape(T=2, H=128, E=4, k=2, I=128, Is=0, tag=501)
    inp = make_layer(sh)
    a = oracle.moe_layer(inp)
    b = c_oracle.moe_layer(inp)
    assert np.all(a["y_shared"] == 0)
    assert np.abs(a["out"] - b["out"]).max() <= 1e-12 * np.abs(a["out"]).max()


def test_tiny_workload_shape_and_invariants():
    inp = make_layer(WORKLOADS["tiny_t1"])
    r = oracle.moe_layer(inp)
    assert r["ids"].shape == (1, 2) and r["out"].shape == (1, 256)
    assert np.isclose(r["weights"].sum(), 2.5, rtol=0, atol=1e-12)
    assert r["gaps"][0] > 1e-4

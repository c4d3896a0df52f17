"""Float64 NumPy oracle of one decode-step MoE layer with a sigmoid router.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg; never by the product path.

What the layer computes, step by step, from the vLLM API pages:

* ``vllm.models.glm5next.nvidia.specialized_decode.runtime.decode``,
  ``LayerStages._build_mega``: the fused MoE stage exists only for
  ``scoring_func == "sigmoid"``, ``n_group == 1`` and ``norm_topk_prob``; it is
  built from ``w13_weight``, ``w13_weight_scale_inv``, ``w2_weight``,
  ``w2_weight_scale_inv``, ``num_experts_per_tok``, ``swiglu_limit``,
  ``routed_scaling_factor`` and the e8m0 (power-of-two scale) flag.
* same page, ``LayerStages._mega_moe``: the shared expert runs beside the
  routed experts and comes back as a separate, unweighted output; the routed
  rows stay unfinalized together with their expert weights; the router bias
  ``e_score_correction_bias`` is passed along with the logits.
* ``vllm.models.glm5next.nvidia.specialized_decode.runtime.draft``,
  ``SpecializedDraft.reduced_norm`` / ``_build_ar_norm``: the boundary after
  the MoE returns norm(x + residual) and the new residual, and it is built
  with ``top_k`` because it finalizes (weights and sums) the routed rows.

Readings where the pages are silent (each one is listed with its reason in
the design notes):
  * scores s = sigmoid(logit); experts ranked by s (+ bias when one is given),
    ties to the lower expert id; weights w_j = R * s_j / sum_i s_i from the
    unbiased scores.
  * a weight block is dequantised as code value * block scale (the
    ``*_scale_inv`` tensors are multiplied in).
  * w13 rows [0, I) are the gate projection, rows [I, 2I) the up projection.
  * clamped SwiGLU: silu(min(g, L)) * clamp(u, -L, L).
  * RMSNorm: h / sqrt(mean(h^2) + eps) * gamma, on the unrounded sum h.

Everything is float64.  Activations are not quantised.
"""

from __future__ import annotations

import numpy as np

BLOCK = 128


# ---------------------------------------------------------------- encodings

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Value of bf16 bit patterns: the top 16 bits of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _e4m3_value(code: int) -> float:
    """OCP FP8 E4M3 (e4m3fn): 1 sign, 4 exponent (bias 7), 3 mantissa bits;
    no infinities; S.1111.111 is NaN; exponent field 0 is subnormal."""
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * man * 2.0 ** -9  # 2^(1-7) * man/8
    return sign * 2.0 ** (exp - 7) * (1.0 + man / 8.0)


_E4M3 = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_codes_to_f64(codes: np.ndarray) -> np.ndarray:
    """Values of e4m3fn codes (uint8)."""
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def e8m0_bytes_to_f64(b: np.ndarray) -> np.ndarray:
    """Values of e8m0 scale bytes: 2^(b - 127); 255 is NaN."""
    b = np.asarray(b, dtype=np.uint8)
    v = np.ldexp(1.0, b.astype(np.int64) - 127)
    return np.where(b == 255, np.nan, v)


def scales_to_f64(scales: np.ndarray) -> np.ndarray:
    """Block scales as float64: float32 scales as they are, uint8 as e8m0."""
    if scales.dtype == np.uint8:
        return e8m0_bytes_to_f64(scales)
    return np.asarray(scales, dtype=np.float64)


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """A weight matrix [R, C] from its e4m3fn codes and its [R/128, C/128]
    block scales: every element is its code's value times its block's scale."""
    R, C = codes.shape
    s = scales_to_f64(scales)
    assert s.shape == (R // BLOCK, C // BLOCK), (s.shape, R, C)
    full = np.repeat(np.repeat(s, BLOCK, axis=0), BLOCK, axis=1)
    return e4m3_codes_to_f64(codes) * full


# ------------------------------------------------------------------ routing

def router_logits(x: np.ndarray, router_w: np.ndarray) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] * W_r[e, h]  (the router GEMM, fp32 out
    on the pages; exact here)."""
    return x @ router_w.T


def sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def select_experts(scores: np.ndarray, bias, k: int) -> np.ndarray:
    """The k experts of each token with the largest score (+ bias), in
    descending order; equal keys go to the lower expert id."""
    key = scores if bias is None else scores + np.asarray(bias, np.float64)[None, :]
    # A stable sort of the negated keys keeps equal keys in id order.
    order = np.argsort(-key, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def route_weights(scores: np.ndarray, ids: np.ndarray, rsf: float) -> np.ndarray:
    """Renormalised top-k weights times routed_scaling_factor, from the
    unbiased scores of the selected experts."""
    sel = np.take_along_axis(scores, ids.astype(np.int64), axis=1)
    return rsf * sel / sel.sum(axis=1, keepdims=True)


def score_gaps(scores: np.ndarray, bias, k: int) -> np.ndarray:
    """Per token, the gap between the k-th and (k+1)-th largest ranking key
    (inf when k equals the expert count)."""
    key = scores if bias is None else scores + np.asarray(bias, np.float64)[None, :]
    srt = -np.sort(-key, axis=1)
    if k >= key.shape[1]:
        return np.full(key.shape[0], np.inf)
    return srt[:, k - 1] - srt[:, k]


def route_table(ids: np.ndarray, E: int):
    """The token -> expert permutation of one step.

    Routes are numbered r = t * k + j.  Returns
      counts [E]     routes per expert
      offsets [E+1]  exclusive prefix sum of counts
      perm [T*k]     routes sorted by expert, in route order within an expert
      inv [T, k]     position of route (t, j) in perm
    """
    T, k = ids.shape
    flat = ids.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    inv = np.empty(T * k, np.int32)
    inv[perm] = np.arange(T * k, dtype=np.int32)
    return counts, offsets, perm, inv.reshape(T, k)


# ------------------------------------------------------------------ experts

def clamped_swiglu(g: np.ndarray, u: np.ndarray, limit: float) -> np.ndarray:
    """silu(min(g, L)) * clamp(u, -L, L), silu(z) = z * sigmoid(z)."""
    gc = np.minimum(g, limit)
    return gc * sigmoid(gc) * np.clip(u, -limit, limit)


def expert_mlp(w13: np.ndarray, w2: np.ndarray, x: np.ndarray, limit: float) -> np.ndarray:
    """One expert on the rows of x [n, H]: dequantised w13 [2I, H] gives the
    gate (rows [0, I)) and up (rows [I, 2I)) projections, then the clamped
    SwiGLU, then the dequantised down projection w2 [H, I]."""
    I = w13.shape[0] // 2
    gu = x @ w13.T
    a = clamped_swiglu(gu[:, :I], gu[:, I:], limit)
    return a @ w2.T


def rms_norm(h: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """h / sqrt(mean over the hidden dim of h^2 + eps) * gamma."""
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + eps) * gamma


# -------------------------------------------------------------------- layer

def dense_layer(inp, rows=None) -> dict:
    """A dense layer step in float64: no router and no routed experts (E = 0);
    the layer's MLP is held in the shared-expert weights (sw13, sw2).

    The decode page's LayerStages._build_dense builds a DenseMlp from a dense
    layer's fp8 gate_up / down weights with their weight_scale_inv, the
    swiglu_limit and the e8m0 flag, and LayerStages.mlp returns dense(x) as
    the layer's FFN output, which goes through the same boundary as the MoE
    output (the draft page's reduced_norm).  So y = W2 a with a =
    silu(min(g, L)) clamp(u, -L, L), [g; u] = W13 x; h = y + residual; out =
    RMSNorm(h) * gamma.  Returns moe (= y), h and out (ids and weights empty).
    """
    sh = inp.shape
    rows = np.arange(sh.T) if rows is None else np.asarray(rows)
    x = bf16_bits_to_f64(inp.hidden[rows])
    res = bf16_bits_to_f64(inp.residual[rows])
    gamma = bf16_bits_to_f64(inp.gamma)
    y = expert_mlp(dequantize(inp.sw13, inp.sw13_scale), dequantize(inp.sw2, inp.sw2_scale), x,
                   sh.limit)
    h = y + res
    n = len(rows)
    return dict(ids=np.zeros((n, 0), np.int32), weights=np.zeros((n, 0)), y_shared=y, moe=y, h=h,
                out=rms_norm(h, gamma, sh.eps))


def moe_layer(inp, forced_ids=None, rows=None) -> dict:
    """The whole layer step in float64 (a dense layer when the shape has no
    routed experts: dense_layer).

    inp         synth.LayerInputs (device bytes of every input)
    forced_ids  optional [T, k] expert ids (indexed by token) to use instead
                of the oracle's own selection; weights still follow from the
                scores
    rows        optional token rows to compute (all when None); the outputs
                then hold only those rows, in that order

    Returns a dict with logits, scores, ids, weights, gaps, y_shared, moe
    (the finalized MoE output: the weighted routed rows plus the shared
    expert, before the residual; what the decode page's LayerStages.
    _grouped_moe gets from the grouped kernel with finalize=True), h (= moe +
    residual, the new residual before rounding) and out (the normalised
    output).
    """
    sh = inp.shape
    if sh.E == 0:
        return dense_layer(inp, rows)
    rows = np.arange(sh.T) if rows is None else np.asarray(rows)
    x = bf16_bits_to_f64(inp.hidden[rows])
    res = bf16_bits_to_f64(inp.residual[rows])
    gamma = bf16_bits_to_f64(inp.gamma)
    bias = None if inp.router_bias is None else inp.router_bias.astype(np.float64)

    logits = router_logits(x, bf16_bits_to_f64(inp.router_w))
    scores = sigmoid(logits)
    if forced_ids is None:
        ids = select_experts(scores, bias, sh.k)
    else:
        ids = np.asarray(forced_ids, np.int32).reshape(sh.T, sh.k)[rows]
    weights = route_weights(scores, ids, sh.rsf)

    n = len(rows)
    routed = np.zeros((n, sh.H))
    for e in np.unique(ids):
        tok, slot = np.nonzero(ids == e)
        w13 = dequantize(inp.w13[e], inp.w13_scale[e])
        w2 = dequantize(inp.w2[e], inp.w2_scale[e])
        y = expert_mlp(w13, w2, x[tok], sh.limit)
        np.add.at(routed, tok, weights[tok, slot][:, None] * y)

    if sh.Is:
        y_shared = expert_mlp(dequantize(inp.sw13, inp.sw13_scale),
                              dequantize(inp.sw2, inp.sw2_scale), x, sh.limit)
    else:
        y_shared = np.zeros((n, sh.H))

    moe = routed + y_shared
    h = moe + res
    out = rms_norm(h, gamma, sh.eps)
    return dict(logits=logits, scores=scores, ids=ids, weights=weights,
                gaps=score_gaps(scores, bias, sh.k), y_shared=y_shared, moe=moe, h=h, out=out)

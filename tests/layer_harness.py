"""Shared helpers of the parity tests: move seeded inputs to the GPU, run the
layer through the C ABI, and compare against the CPU oracle.

Tolerances (floating point), applied per output tensor over all compared
elements:
  relative L2 error            <= 5e-3
  max |gpu - oracle|           <= 3e-2 * RMS(oracle)
  top-k weights                 relative error <= 1e-5
Expert ids must equal the oracle's selection (as sets) for every token whose
k-th / (k+1)-th ranking-key gap exceeds 1e-4; for the other tokens any
selection whose keys are all within 1e-4 of the oracle's k-th key is valid.
Outputs are always compared with the oracle run on the GPU's own ids (forced
routing), so a valid near-tie choice is checked on its own arithmetic.
"""

from __future__ import annotations

import numpy as np
import torch

import moe_decode_layer_sigmoid_amd as md
import oracle
from oracle import moe_oracle as mo

REL_L2 = 5e-3
MAX_ABS_FRAC = 3e-2
GAP = 1e-4
W_RTOL = 1e-5


def _dev(a, device):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def to_device(inp, device="cuda"):
    names = ["hidden", "residual", "router_w", "router_bias", "w13", "w13_scale", "w2",
             "w2_scale", "sw13", "sw13_scale", "sw2", "sw2_scale", "gamma"]
    return {n: _dev(getattr(inp, n), device) for n in names}


def make_plan(shape, max_tokens=None, path=md.PATH_AUTO, device=0):
    d = md.make_desc(shape.H, shape.E, shape.k, shape.I, shape.Is, max_tokens or shape.T,
                     shape.scale_fmt, path, shape.limit, shape.rsf, shape.eps)
    return md.Plan(d, device)


def bf16_to_np(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_bits_to_f64(t.cpu().numpy().view(np.uint16))


def run_layer(plan, dev, T, alias_residual=False, stream=None, keep_device=False):
    """One moe_decode_run; returns host copies (and the device outputs)."""
    H, k = plan.desc.hidden, plan.desc.top_k
    device = dev["hidden"].device
    out = torch.empty((T, H), dtype=torch.int16, device=device)
    if alias_residual:
        res_out = dev["residual"][:T].clone()
        residual = res_out
    else:
        res_out = torch.empty((T, H), dtype=torch.int16, device=device)
        residual = dev["residual"]
    moe = torch.empty((T, H), dtype=torch.int16, device=device)
    ids = torch.full((T, k), -1, dtype=torch.int32, device=device)
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device=device)
    plan.run(T, stream=stream, hidden=dev["hidden"], residual=residual, router_w=dev["router_w"],
             router_bias=dev["router_bias"], w13=dev["w13"], w13_scale=dev["w13_scale"],
             w2=dev["w2"], w2_scale=dev["w2_scale"], sw13=dev["sw13"],
             sw13_scale=dev["sw13_scale"], sw2=dev["sw2"], sw2_scale=dev["sw2_scale"],
             gamma=dev["gamma"], out=out, residual_out=res_out, topk_ids=ids, topk_weights=w,
             moe_out=moe)
    torch.cuda.synchronize()
    # the single-launch step, the expert chain and the grouped merged launch
    # hand work between workgroups through bounded waits
    assert not plan.check_waits(), "a bounded wait gave up"
    got = dict(out=bf16_to_np(out), residual_out=bf16_to_np(res_out), moe=bf16_to_np(moe),
               ids=ids.cpu().numpy(),
               weights=w.cpu().numpy().astype(np.float64))
    if keep_device:
        got["dev"] = dict(out=out, residual_out=res_out, ids=ids, weights=w)
    return got


def tensor_errors(got: np.ndarray, ref: np.ndarray):
    diff = got - ref
    rel_l2 = np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300)
    rms = np.sqrt(np.mean(ref * ref))
    max_frac = np.abs(diff).max() / max(rms, 1e-300)
    return rel_l2, max_frac


def assert_close(got, ref, what):
    rel_l2, max_frac = tensor_errors(got, ref)
    assert rel_l2 <= REL_L2, "%s: relative L2 %.3g > %.3g" % (what, rel_l2, REL_L2)
    assert max_frac <= MAX_ABS_FRAC, "%s: max-abs/RMS %.3g > %.3g" % (what, max_frac, MAX_ABS_FRAC)
    return rel_l2, max_frac


def check_ids(inp, got_ids, rows=None):
    """GPU ids against the oracle's selection (router only: cheap at any size)."""
    sh = inp.shape
    rows = np.arange(sh.T) if rows is None else np.asarray(rows)
    x = oracle.bf16_bits_to_f64(inp.hidden[rows])
    scores = oracle.sigmoid(oracle.router_logits(x, oracle.bf16_bits_to_f64(inp.router_w)))
    bias = None if inp.router_bias is None else inp.router_bias.astype(np.float64)
    ref = oracle.select_experts(scores, bias, sh.k)
    gaps = oracle.score_gaps(scores, bias, sh.k)
    key = scores if bias is None else scores + bias[None, :]
    g = got_ids[rows]
    n_tie = 0
    for i in range(len(rows)):
        assert len(set(g[i].tolist())) == sh.k and g[i].min() >= 0 and g[i].max() < sh.E, \
            "token %d: ids %s are not k distinct experts" % (rows[i], g[i])
        if gaps[i] > GAP:
            assert set(g[i].tolist()) == set(ref[i].tolist()), \
                "token %d: ids %s != oracle %s (gap %.3g)" % (rows[i], g[i], ref[i], gaps[i])
        else:
            n_tie += 1
            kth = np.sort(key[i])[::-1][sh.k - 1]
            assert np.all(key[i][g[i]] >= kth - GAP), "token %d: invalid near-tie pick" % rows[i]
        # rank order: descending keys (within the tie slack)
        assert np.all(np.diff(key[i][g[i]]) <= GAP)
    return n_tie


def check_layer(inp, got, rows=None, use_c=None, c_oracle=None):
    """Full comparison of one run; rows = token rows to compute with the
    oracle (all when None).  Returns a dict of the measured errors."""
    sh = inp.shape
    rows_list = np.arange(sh.T) if rows is None else np.asarray(rows)
    if sh.E == 0:
        # a dense layer: no routing to check; the NumPy oracle computes it
        ref = mo.moe_layer(inp, rows=rows_list)
        e_out = assert_close(got["out"][rows_list], ref["out"], "out")
        e_res = assert_close(got["residual_out"][rows_list], ref["h"], "residual_out")
        assert_close(got["moe"][rows_list], ref["moe"], "moe_out")
        return dict(n_tie=0, out_rel_l2=e_out[0], out_max=e_out[1], res_rel_l2=e_res[0])
    n_tie = check_ids(inp, got["ids"])
    if use_c is None:
        use_c = sh.H * sh.I * len(rows_list) > 2 ** 24
    if use_c:
        ref = c_oracle.moe_layer(inp, forced_ids=got["ids"], rows=rows_list)
    else:
        ref = mo.moe_layer(inp, forced_ids=got["ids"], rows=rows_list)
    w_rel = np.abs(got["weights"][rows_list] - ref["weights"]) / np.abs(ref["weights"])
    assert w_rel.max() <= W_RTOL, "weights rel err %.3g" % w_rel.max()
    assert np.allclose(got["weights"].sum(1), sh.rsf, rtol=1e-5)
    e_out = assert_close(got["out"][rows_list], ref["out"], "out")
    e_res = assert_close(got["residual_out"][rows_list], ref["h"], "residual_out")
    if "moe" in got:
        assert_close(got["moe"][rows_list], ref["moe"], "moe_out")
    return dict(n_tie=n_tie, out_rel_l2=e_out[0], out_max=e_out[1], res_rel_l2=e_res[0],
                res_max=e_res[1], w_rel=float(w_rel.max()))

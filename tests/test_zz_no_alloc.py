"""moe_decode_run_static, the entry point that allocates nothing, through the
C ABI: its outputs against moe_decode_run's on the same inputs (bit for bit:
the same kernels run, the shared passes above 64 tokens on the caller's
stream instead of a side stream) and against the oracle, on calls in a row
whose later inputs are smaller than the first (the static scratch array
keeps the previous call's contents); and its rejection of a size whose
workspace exceeds the array."""

import numpy as np
import pytest
import torch

import moe_decode_layer_sigmoid_amd as md
from synth import LayerShape, make_layer
from layer_harness import bf16_to_np, check_layer, make_plan, run_layer, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert md.lib() is not None


def _outputs(T, H, k, device="cuda"):
    return dict(out=torch.empty((T, H), dtype=torch.int16, device=device),
                residual_out=torch.empty((T, H), dtype=torch.int16, device=device),
                moe_out=torch.empty((T, H), dtype=torch.int16, device=device),
                topk_ids=torch.full((T, k), -1, dtype=torch.int32, device=device),
                topk_weights=torch.full((T, k), float("nan"), dtype=torch.float32,
                                        device=device))


def _run_static(sh, dev, path):
    T = sh.T
    o = _outputs(T, sh.H, sh.k)
    desc = md.make_desc(sh.H, sh.E, sh.k, sh.I, sh.Is, T, sh.scale_fmt, path, sh.limit,
                        sh.rsf, sh.eps)
    md.run_static(desc, T, hidden=dev["hidden"], residual=dev["residual"],
                  router_w=dev["router_w"], router_bias=dev["router_bias"], w13=dev["w13"],
                  w13_scale=dev["w13_scale"], w2=dev["w2"], w2_scale=dev["w2_scale"],
                  sw13=dev["sw13"], sw13_scale=dev["sw13_scale"], sw2=dev["sw2"],
                  sw2_scale=dev["sw2_scale"], gamma=dev["gamma"], **o)
    torch.cuda.synchronize()
    return dict(out=bf16_to_np(o["out"]), residual_out=bf16_to_np(o["residual_out"]),
                moe=bf16_to_np(o["moe_out"]), ids=o["topk_ids"].cpu().numpy(),
                weights=o["topk_weights"].cpu().numpy().astype(np.float64))


# Calls in a row, each smaller than the one before: 80 tokens (MFMA path,
# shared passes queued on the caller's stream), 40 (MFMA merged launch), 3
# (router + expert chain), 1.
SEQUENCE = [80, 40, 3, 1]


@pytest.mark.parametrize("path", [md.PATH_AUTO, md.PATH_GEMV_SPLIT], ids=["auto", "split"])
def test_static_matches_plan_run(path, c_oracle):
    base = LayerShape(T=SEQUENCE[0], H=1024, E=32, k=4, I=256, Is=256, scale_fmt="fp32",
                      tag=330)
    for i, T in enumerate(SEQUENCE):
        sh = base.replace(T=T, tag=330 + T)
        inp = make_layer(sh, with_bias=(i % 2 == 1), bias_std=0.1)
        dev = to_device(inp)
        plan = make_plan(sh, path=path)
        ref = run_layer(plan, dev, T)
        plan.close()
        got = _run_static(sh, dev, path)
        print("static call", i, "T", T, "path", path, flush=True)
        for key in ("ids", "weights", "out", "residual_out", "moe"):
            assert np.array_equal(got[key], ref[key]), (T, key)
        assert not np.isnan(got["out"]).any()
        check_layer(inp, got, c_oracle=c_oracle)


def test_static_dense_matches_plan_run():
    """A dense layer (no routed experts) through the static entry point:
    calls of 40, 16 and 1 tokens in a row (the matrix-core kernels' partial
    planes and the GEMV kernels), each equal to moe_decode_run's output and
    within the oracle's tolerance."""
    base = LayerShape(T=40, H=1024, E=0, k=0, I=0, Is=2048, scale_fmt="fp32", tag=332)
    for i, (T, path) in enumerate([(40, md.PATH_AUTO), (16, md.PATH_AUTO),
                                   (1, md.PATH_GEMV_SPLIT)]):
        sh = base.replace(T=T, tag=332 + T)
        inp = make_layer(sh)
        dev = to_device(inp)
        plan = make_plan(sh, path=path)
        ref = run_layer(plan, dev, T)
        plan.close()
        got = _run_static(sh, dev, path)
        print("static dense call", i, "T", T, "path", path, flush=True)
        for key in ("out", "residual_out", "moe"):
            assert np.array_equal(got[key], ref[key]), (T, key)
        check_layer(inp, got)


def test_static_rejects_oversized_workspace():
    # 256 tokens x k = 16 x H = 8192 f32 down rows alone need 128 MiB
    sh = LayerShape(T=256, H=8192, E=64, k=16, I=128, Is=0, tag=331)
    desc = md.make_desc(sh.H, sh.E, sh.k, sh.I, sh.Is, sh.T)
    x = torch.zeros((sh.T, sh.H), dtype=torch.int16, device="cuda")
    w = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(md.MoeDecodeError) as e:
        md.run_static(desc, sh.T, hidden=x, residual=x, router_w=x, w13=w, w13_scale=w, w2=w,
                      w2_scale=w, gamma=x, out=torch.empty_like(x),
                      residual_out=torch.empty_like(x))
    assert e.value.code == md.ERR_SCRATCH

"""GPU parity: the HIP layer (through the C ABI) against the CPU oracle.

Needs an MI355X; every test is marked `gpu`.  Every layer here is compared
in full: every token's expert ids, and every element of out, residual_out
and moe_out (all T x H) against the oracle run on the GPU's own ids (the C
oracle at full size).
"""

import numpy as np
import pytest
import torch

import moe_decode_layer_sigmoid_amd as md
import oracle
from synth import LayerShape, WORKLOADS, make_layer
from layer_harness import (check_ids, check_layer, make_plan, run_layer, to_device,
                           assert_close)

pytestmark = pytest.mark.gpu


def _log(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert md.lib() is not None


def _case(shape, c_oracle, rows=None, max_tokens=None, path=md.PATH_AUTO, with_bias=False,
          alias=False, seed=0):
    _log("case", shape, "rows", rows, "bias", with_bias, "alias", alias)
    inp = make_layer(shape, seed=seed, with_bias=with_bias, bias_std=0.1)
    dev = to_device(inp)
    plan = make_plan(shape, max_tokens=max_tokens, path=path)
    got = run_layer(plan, dev, shape.T, alias_residual=alias)
    err = check_layer(inp, got, rows=rows, c_oracle=c_oracle)
    _log("  errors", err)
    plan.close()
    return inp, got, err


def test_tiny_layer(c_oracle):
    _case(WORKLOADS["tiny_t1"], c_oracle)


@pytest.mark.parametrize("name", ["decode_t1", "decode_t16"])
@pytest.mark.parametrize("path", [md.PATH_GEMV, md.PATH_GEMV_SPLIT, md.PATH_GROUPED],
                         ids=["step", "split", "grouped"])
def test_decode_layers_full(name, path, c_oracle):
    inp, got, err = _case(WORKLOADS[name], c_oracle, path=path)
    if name == "decode_t16":
        d = len(np.unique(got["ids"]))
        _log("  distinct experts", d)
        assert 60 <= d <= 100


@pytest.mark.parametrize("name", ["wide_t64_e8m0", "verify_t128"])
@pytest.mark.parametrize("path", [md.PATH_AUTO, md.PATH_GEMV_SPLIT], ids=["auto", "split"])
def test_wide_layers_full(name, path, c_oracle):
    """The 64-token e8m0 layer and the 128-token verify batch at full size
    (H = 6144, E = 256, I = 2048), every token row compared."""
    _case(WORKLOADS[name], c_oracle, path=path)


@pytest.mark.parametrize("T", [48, 128, 192, 256])
def test_decode_shape_many_tokens_full(T, c_oracle):
    """The decode shape (H = 4096, E = 128) with more tokens, at full size:
    the rotated block walk past 32 tokens (H is a power of two), the shared
    expert on its own stream past 64 tokens, from 128 tokens (8 or more
    tokens per expert on average) the routed launches' activation tiles
    shared per workgroup, and from 160 tokens (10 or more) their two 16-token
    groups per pass over the weights."""
    sh = WORKLOADS["decode_t16"].replace(T=T)
    _, got, _ = _case(sh, c_oracle)
    counts = np.bincount(got["ids"].ravel(), minlength=sh.E)
    _log("  most tokens on one expert", counts.max())
    if T >= 192:
        assert counts.max() > 16  # some pass carries two 16-token groups


def test_wide_shape_max_tokens_full(c_oracle):
    """H = 6144, E = 256, e8m0 scales at the plan's 256-token maximum, full
    size: sixteen shared-expert passes on the side stream beside the routed
    launches, and one 16-token group per pass (8 tokens per expert on
    average) with the activation tiles shared per workgroup."""
    sh = WORKLOADS["wide_t64_e8m0"].replace(T=256)
    _case(sh, c_oracle)


SMALL = [
    # T, H, E, k, I, Is, fmt
    (1, 128, 4, 1, 128, 0, "fp32"),
    (3, 256, 16, 4, 256, 128, "e8m0"),
    (7, 384, 33, 5, 128, 256, "fp32"),
    (20, 256, 64, 8, 384, 128, "fp32"),
    (5, 1152, 70, 16, 256, 128, "e8m0"),
    (2, 640, 8, 8, 128, 128, "fp32"),  # k == E: every expert taken
    (64, 256, 128, 8, 128, 128, "e8m0"),
    (130, 128, 200, 6, 128, 0, "fp32"),  # more than two 64-token mask words
    (1, 8192, 16, 2, 128, 128, "fp32"),  # widest hidden
    (3, 256, 1024, 8, 128, 0, "fp32"),  # most experts: top-k by rounds of wave arg-max
    (40, 256, 1024, 16, 128, 128, "e8m0"),  # most experts with the largest k
    (256, 256, 64, 8, 128, 128, "fp32"),  # most tokens (four 64-token mask words)
    # every limit at once: 256 tokens, 1024 experts, k = 16 (4096 routes, the
    # routing step's largest LDS carve-up and packed route scan)
    (256, 256, 1024, 16, 128, 128, "fp32"),
    # the single-launch step's widest router (four keys per lane) at one and
    # two tokens
    (1, 512, 256, 8, 256, 256, "e8m0"),
    (2, 384, 150, 6, 128, 0, "fp32"),
    # the router's two-token blocks with a last block of one token
    (13, 512, 48, 6, 256, 128, "fp32"),
]


@pytest.mark.parametrize("case", SMALL, ids=[str(c) for c in SMALL])
@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("path", [md.PATH_GEMV, md.PATH_GEMV_SPLIT, md.PATH_GROUPED],
                         ids=["step", "split", "grouped"])
def test_small_layers(case, with_bias, path, c_oracle):
    T, H, E, k, I, Is, fmt = case
    sh = LayerShape(T=T, H=H, E=E, k=k, I=I, Is=Is, scale_fmt=fmt, tag=300 + sum(case[:6]))
    _case(sh, c_oracle, with_bias=with_bias, path=path)


@pytest.mark.parametrize("T", [1, 3, 16, 40])
def test_paths_agree(T, c_oracle):
    """The single-launch step, the separate GEMV kernels and the MFMA
    kernels compute the same layer (same ids, outputs within the oracle
    tolerance of each other)."""
    sh = WORKLOADS["decode_t16"].replace(T=T, H=2048, I=768, Is=512, tag=310 + T)
    inp = make_layer(sh)
    dev = to_device(inp)
    paths = [md.PATH_GEMV_SPLIT, md.PATH_GROUPED] + ([md.PATH_GEMV] if T <= 16 else [])
    res = []
    for path in paths:
        plan = make_plan(sh, path=path)
        assert plan.path_for(T) == path
        res.append(run_layer(plan, dev, T))
        plan.close()
    for r in res[1:]:
        assert np.array_equal(res[0]["ids"], r["ids"])
        assert_close(r["out"], res[0]["out"], "paths agree: out")
    for r in res:
        check_layer(inp, r, c_oracle=c_oracle)


@pytest.mark.parametrize("T,E,k", [(1, 128, 8), (16, 128, 8), (256, 1024, 16)])
def test_route_tables_match_oracle(T, E, k, c_oracle):
    H = 1024 if T <= 16 else 256
    sh = WORKLOADS["decode_t16"].replace(T=T, H=H, E=E, k=k, I=256, Is=256, tag=301)
    inp = make_layer(sh)
    dev = to_device(inp)
    plan = make_plan(sh)
    got = run_layer(plan, dev, sh.T)
    E, R = sh.E, sh.T * sh.k
    cnt = torch.empty(E, dtype=torch.int32, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(R, dtype=torch.int32, device="cuda")
    tch = torch.empty(E, dtype=torch.int32, device="cuda")
    nt = torch.empty(1, dtype=torch.int32, device="cuda")
    plan.last_routes(sh.T, cnt, off, perm, tch, nt)
    torch.cuda.synchronize()
    counts, offsets, operm, _ = oracle.route_table(got["ids"], E)
    assert np.array_equal(cnt.cpu().numpy(), counts)
    assert np.array_equal(off.cpu().numpy(), offsets)
    assert np.array_equal(perm.cpu().numpy(), operm)
    touched = np.nonzero(counts)[0]
    assert nt.item() == len(touched)
    assert np.array_equal(tch.cpu().numpy()[: len(touched)], touched)
    plan.close()


@pytest.mark.parametrize("T,H,I", [(37, 256, 128), (150, 256, 128), (150, 1152, 640)],
                         ids=["T37", "T150", "T150-wide"])
@pytest.mark.parametrize("path", [md.PATH_GEMV_SPLIT, md.PATH_GROUPED], ids=["split", "grouped"])
def test_same_expert_for_every_token(T, H, I, path, c_oracle):
    """All tokens pick the same experts: one expert carries T tokens (the
    GEMV token loop runs several register passes; the MFMA kernels run
    several 16-token passes per workgroup, each over the whole contraction)."""
    sh = LayerShape(T=T, H=H, E=16, k=2, I=I, Is=128, tag=302)
    inp = make_layer(sh)
    # Every token carries token 0's vector x0; router rows 3 and 9 point along
    # x0 (logits |x0| and |x0|/2), every other row is zero (logit 0).
    from synth import f32_to_bf16_bits
    inp.hidden = np.ascontiguousarray(np.tile(inp.hidden[:1], (T, 1)))
    x0 = oracle.bf16_bits_to_f64(inp.hidden[0])
    wr = np.zeros((16, H), np.float32)
    wr[3] = (x0 / np.linalg.norm(x0)).astype(np.float32)
    wr[9] = 0.5 * wr[3]
    inp.router_w = f32_to_bf16_bits(wr)
    dev = to_device(inp)
    plan = make_plan(sh, path=path)
    got = run_layer(plan, dev, sh.T)
    assert np.all(np.sort(got["ids"], 1) == [3, 9])
    check_layer(inp, got, c_oracle=c_oracle)
    plan.close()


@pytest.mark.parametrize("T", [1, 3, 7, 8, 16, 70])
@pytest.mark.parametrize("fmt", ["fp32", "e8m0"])
def test_dense_layer(T, fmt, c_oracle):
    """No routed experts: the layer's fp8 clamped-SwiGLU MLP (in the shared-
    expert slot) and the boundary, on the MFMA kernels (AUTO at every token
    count) and the GEMV kernels, against the dense oracle; each path forced
    at T = 3 and 16 as well."""
    sh = LayerShape(T=T, H=2048, E=0, k=0, I=0, Is=3072, scale_fmt=fmt, tag=320 + T)
    inp = make_layer(sh)
    dev = to_device(inp)
    paths = [md.PATH_AUTO] + ([md.PATH_GEMV_SPLIT, md.PATH_GROUPED] if T in (3, 16) else [])
    for path in paths:
        _log("dense", sh, "path", path)
        plan = make_plan(sh, path=path)
        want = md.PATH_GROUPED if path == md.PATH_AUTO else path
        assert plan.path_for(T) == want
        got = run_layer(plan, dev, T)
        err = check_layer(inp, got)
        _log("  errors", err)
        plan.close()


@pytest.mark.parametrize("T,H,Is,fmt", [(16, 4096, 8192, "fp32"), (64, 4096, 8192, "e8m0"),
                                         (20, 1024, 6144, "fp32"), (33, 384, 512, "e8m0"),
                                         (5, 4096, 4096, "fp32"), (40, 1408, 640, "fp32"),
                                         (75, 2048, 1024, "e8m0"), (128, 4096, 8192, "fp32"),
                                         (256, 2048, 3072, "e8m0"), (1, 128, 128, "fp32"),
                                         (40, 128, 128, "e8m0")])
def test_dense_layer_mfma_splits(T, H, Is, fmt):
    """The dense MFMA kernels at the shapes that set their contraction
    ranges and token groups: 4 and 1 gate_up ranges, 8 and 2 down ranges,
    ranges of unequal length (H = 1408 and I_s = 640: 11 and 5 blocks), one
    range per launch (H = 384, I_s = 512: no hand-over of sums), the
    one-group gate_up kernel (whose waves split the contraction), two and
    four 16-token groups per gate_up workgroup, two passes of the down
    launch, a second pass with one group (33 tokens), a second pass whose
    one group is partial (75 tokens), and many passes at the full size and
    at the plan's 256-token limit, and the smallest layer (H = I_s = 128:
    one contraction block, so three of the one-group kernel's waves have
    no range, and one down tile); every output row against the dense
    oracle."""
    sh = LayerShape(T=T, H=H, E=0, k=0, I=0, Is=Is, scale_fmt=fmt, tag=340 + T)
    inp = make_layer(sh)
    dev = to_device(inp)
    _log("dense mfma", sh)
    plan = make_plan(sh, path=md.PATH_GROUPED)
    got = run_layer(plan, dev, T)
    err = check_layer(inp, got)
    _log("  errors", err)
    plan.close()


def test_dense_token_counts_in_turn():
    """The dense MFMA launches leave their arrival counters at zero and
    nothing else behind: dense layers in turn on one plan (another layer's
    weights and tokens each run), at token counts that change the grid
    between runs (64: four gate_up ranges of four groups; 20 and 33: two
    groups; 16 and 1: the one-group kernel; 80: two passes), each match
    their own oracle; the first layer run again at the end is bitwise equal
    to its first run (the last workgroup adds the ranges in range order)."""
    base = LayerShape(T=80, H=1024, E=0, k=0, I=0, Is=2048, tag=360)
    plan = make_plan(base, path=md.PATH_GROUPED)
    first = None
    for i, T in enumerate([64, 20, 16, 80, 1, 33, 64]):
        sh = base.replace(T=T, tag=360 if i in (0, 6) else 361 + i)
        inp = make_layer(sh)
        _log("dense in turn", sh)
        got = run_layer(plan, to_device(inp), T)
        check_layer(inp, got)
        if i == 0:
            first = got
        if i == 6:
            for key in ("out", "residual_out", "moe"):
                assert np.array_equal(first[key], got[key]), key
    plan.close()


@pytest.mark.parametrize("T", [1, 5, 16])
@pytest.mark.parametrize("path", [md.PATH_GEMV, md.PATH_GEMV_SPLIT, md.PATH_GROUPED],
                         ids=["step", "split", "grouped"])
def test_alternating_inputs_on_one_plan(path, T, c_oracle):
    """Two different layers (other weights, other tokens) run in turn on one
    plan: every run matches its own oracle, so nothing a run leaves in the
    workspace or in the caches (SwiGLU rows, down rows, route tables,
    counters) leaks into the next one."""
    sh = WORKLOADS["decode_t16"].replace(T=T, H=2048, I=768, Is=512, E=32, tag=306)
    inps = [make_layer(sh, seed=s) for s in (0, 1)]
    devs = [to_device(i) for i in inps]
    plan = make_plan(sh, path=path)
    for r in range(4):
        got = run_layer(plan, devs[r % 2], T)
        check_layer(inps[r % 2], got, c_oracle=c_oracle)
    plan.close()


def test_step_token_counts_in_turn(c_oracle):
    """The single-launch step leaves its counters, flags, logits and
    boundary slots zeroed for the next launch; runs of 1, 3, 16, 1, 2 and 1
    tokens in turn on one plan (other layers' inputs each time) each match
    their own oracle, with the route tables of the multi-token runs and the
    self-routed one-token runs agreeing with the oracle's selection."""
    base = WORKLOADS["decode_t16"].replace(H=1024, I=256, Is=256, E=64, tag=307)
    plan = make_plan(base.replace(T=16), path=md.PATH_GEMV)
    for i, T in enumerate([1, 3, 16, 1, 2, 1]):
        sh = base.replace(T=T, tag=307 + i)
        inp = make_layer(sh, with_bias=(i % 2 == 0), bias_std=0.1)
        assert plan.path_for(T) == md.PATH_GEMV
        got = run_layer(plan, to_device(inp), T)
        check_layer(inp, got, c_oracle=c_oracle)
    plan.close()


@pytest.mark.parametrize("path", [md.PATH_GEMV, md.PATH_GEMV_SPLIT, md.PATH_GROUPED],
                         ids=["step", "split", "grouped"])
def test_residual_alias_and_determinism(path, c_oracle):
    sh = WORKLOADS["decode_t16"].replace(H=2048, I=512, Is=512, tag=303)
    inp = make_layer(sh)
    dev = to_device(inp)
    plan = make_plan(sh, path=path)
    a = run_layer(plan, dev, sh.T)
    b = run_layer(plan, dev, sh.T)
    c = run_layer(plan, dev, sh.T, alias_residual=True)
    for key in ("out", "residual_out", "ids", "weights"):
        assert np.array_equal(a[key], b[key]), key
        assert np.array_equal(a[key], c[key]), key
    check_layer(inp, a, c_oracle=c_oracle)
    plan.close()


def test_smaller_T_than_plan_and_zero(c_oracle):
    sh = LayerShape(T=9, H=512, E=32, k=4, I=256, Is=128, tag=304)
    inp = make_layer(sh)
    dev = to_device(inp)
    plan = make_plan(sh, max_tokens=64)
    got = run_layer(plan, dev, sh.T)
    check_layer(inp, got, c_oracle=c_oracle)
    # T = 0 launches nothing and succeeds
    plan.run(0, hidden=dev["hidden"], residual=dev["residual"], router_w=dev["router_w"],
             w13=dev["w13"], w13_scale=dev["w13_scale"], w2=dev["w2"], w2_scale=dev["w2_scale"],
             sw13=dev["sw13"], sw13_scale=dev["sw13_scale"], sw2=dev["sw2"],
             sw2_scale=dev["sw2_scale"], gamma=dev["gamma"],
             out=torch.empty(1, 512, dtype=torch.int16, device="cuda"),
             residual_out=torch.empty(1, 512, dtype=torch.int16, device="cuda"))
    with pytest.raises(md.MoeDecodeError):
        run_layer(plan, dev, 65)
    plan.close()


def test_dense_smaller_T_than_plan_and_zero():
    """A dense plan runs fewer tokens than it was made for, T = 0 launches
    nothing and succeeds, and more tokens than the plan holds is refused."""
    sh = LayerShape(T=5, H=1024, E=0, k=0, I=0, Is=1024, tag=370)
    inp = make_layer(sh)
    dev = to_device(inp)
    plan = make_plan(sh, max_tokens=40, path=md.PATH_GROUPED)
    check_layer(inp, run_layer(plan, dev, sh.T))
    # (no router or routed weights: the layer has no routed experts)
    plan.run(0, hidden=dev["hidden"], residual=dev["residual"], router_w=None, w13=None,
             w13_scale=None, w2=None, w2_scale=None, sw13=dev["sw13"],
             sw13_scale=dev["sw13_scale"], sw2=dev["sw2"], sw2_scale=dev["sw2_scale"],
             gamma=dev["gamma"], out=torch.empty(1, 1024, dtype=torch.int16, device="cuda"),
             residual_out=torch.empty(1, 1024, dtype=torch.int16, device="cuda"))
    with pytest.raises(md.MoeDecodeError):
        run_layer(plan, dev, 41)
    plan.close()


def _graph_vs_eager(sh, path):
    """One run captured into a HIP graph, replayed four times with eager runs
    in between; every replay equals the eager result bit for bit."""
    inp = make_layer(sh)
    dev = to_device(inp)
    plan = make_plan(sh, path=path)
    eager = run_layer(plan, dev, sh.T, keep_device=True)
    T, H, k = sh.T, sh.H, sh.k
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    res = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    args = plan.make_args(hidden=dev["hidden"], residual=dev["residual"],
                          router_w=dev["router_w"], w13=dev["w13"], w13_scale=dev["w13_scale"],
                          w2=dev["w2"], w2_scale=dev["w2_scale"], sw13=dev["sw13"],
                          sw13_scale=dev["sw13_scale"], sw2=dev["sw2"],
                          sw2_scale=dev["sw2_scale"], gamma=dev["gamma"], out=out,
                          residual_out=res, topk_ids=ids, topk_weights=w)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        plan.run_args(args, T)  # warm up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            plan.run_args(args, T)
    torch.cuda.synchronize()
    for i in range(4):
        out.zero_()
        res.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager["dev"]["out"]), i
        assert torch.equal(res, eager["dev"]["residual_out"]), i
        assert torch.equal(ids, eager["dev"]["ids"]), i
        # eager work between replays
        run_layer(plan, dev, T)
    plan.close()


@pytest.mark.parametrize("path,T,H,I", [(md.PATH_GEMV, 16, 1024, 512),
                                        (md.PATH_GEMV_SPLIT, 16, 1024, 512),
                                        (md.PATH_GROUPED, 16, 1024, 512),
                                        (md.PATH_GROUPED, 80, 1024, 512),
                                        (md.PATH_GROUPED, 24, 2304, 640),
                                        (md.PATH_GROUPED, 80, 2304, 640)],
                         ids=["step", "split", "grouped", "grouped-side-stream",
                              "grouped-wide", "grouped-wide-side-stream"])
def test_graph_replay_matches_eager(path, T, H, I, c_oracle):
    """One run captured into a HIP graph, replayed several times with eager
    work in between; every replay equals the eager result bit for bit.  At
    80 tokens the MFMA path puts the shared expert on the side stream.  The
    H = 2304, I = 640 cases give the MFMA kernels contractions of 18 and 5
    blocks (so at 24 tokens the rotated block walks wrap at odd points) and a
    shared expert narrower than the routed ones."""
    _graph_vs_eager(WORKLOADS["decode_t16"].replace(T=T, H=H, I=I, Is=256, tag=305), path)


@pytest.mark.parametrize("path,T,H,Is", [(md.PATH_AUTO, 16, 2048, 3072),
                                         (md.PATH_AUTO, 70, 1024, 2048),
                                         (md.PATH_GEMV_SPLIT, 3, 1024, 2048)],
                         ids=["dense-mfma-16", "dense-mfma-70", "dense-gemv-3"])
def test_dense_graph_replay_matches_eager(path, T, H, Is):
    """A dense layer's launches (the matrix-core kernels, whose workgroups
    hand partial sums to the last of each tile through counters that they
    reset, or the GEMV kernels) captured and replayed: every replay equals
    the eager run."""
    _graph_vs_eager(LayerShape(T=T, H=H, E=0, k=0, I=0, Is=Is, scale_fmt="fp32", tag=350 + T),
                    path)


@pytest.mark.parametrize("name", ["decode_t1", "decode_t16"])
def test_workload_graph_replay(name, c_oracle):
    """The decode workloads at full size on the AUTO path (the launches the
    benchmark times: the expert chain at one token, the grouped merged launch
    at 16), captured and replayed: every replay equals the eager run, which
    the oracle checks (test_decode_layers_full)."""
    _graph_vs_eager(WORKLOADS[name], md.PATH_AUTO)

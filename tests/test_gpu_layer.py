"""Whole-layer parity through moe_layer_fwd / moe_layer_bwd at sizes the oracle
finishes in seconds (the workloads' structure at reduced N, D, E, H), plus
bitwise run-to-run determinism.

Routing is decided on fp32 logits.  The GPU sums them in another order than
the float64 oracle, so a token whose K-th and (K+1)-th logits are closer than
that rounding could pick another expert: such a token is a near-tie, both
choices are correct, and it is excluded from the row comparison after its tie
is checked.  Every other token must route identically (bit-exact route map
when no near-tie exists).
"""
import numpy as np
import pytest
import torch

import mixture_experts_expert_router_amd as M
import moe_synth as S
import oracle as O
from gpu_util import assert_bf16_close, bits, dev, dev_bf16, host, rel_frobenius, vals

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.load()


def _weights(inp, mxfp8=False):
    w = M.LayerWeights(w_r=dev_bf16(inp.w_r), bias=dev(inp.bias) if inp.bias is not None else None)
    if mxfp8:
        q = O.quantize_weights_mxfp8(inp.w_gate, inp.w_up, inp.w_down)
        w.wq = {k: dev(v) for k, v in q.items()}
        return w, q
    w.w_gate, w.w_up, w.w_down = dev_bf16(inp.w_gate), dev_bf16(inp.w_up), dev_bf16(inp.w_down)
    return w, None


def check_routing(saved, ref, K):
    """Compare logits (tolerance) and the per-token expert sets; return the
    mask of tokens that route identically."""
    Lg = host(saved["logits"]).astype(np.float64)
    Lr = ref["logits"].astype(np.float64)
    scale = np.max(np.abs(Lr))
    assert np.max(np.abs(Lg - Lr)) <= 1e-4 * scale + 1e-6
    same = np.all(host(saved["topk_idx"]) == ref["topk_idx"], axis=1)
    if not np.all(same):
        srt = -np.sort(-Lr, axis=1)
        gap = srt[:, K - 1] - srt[:, K] if Lr.shape[1] > K else np.full(len(Lr), np.inf)
        # every differing token must be a near-tie at the top-K boundary
        # (or a tie inside the top-K changing only the order)
        inner = np.min(np.abs(np.diff(srt[:, :K + 1], axis=1)), axis=1)
        assert np.all(np.minimum(gap, inner)[~same] <= 2e-4 * scale), "routing differs beyond a near-tie"
    return same


def logits_checked(saved, inp):
    """The GPU's router logits after their parity check against the oracle's
    (tolerance).  The whole-layer references below run the oracle's route
    and everything after it on these same fp32 logits, so the route map is
    the GPU's by construction at a near-tie and no token is excluded."""
    Lg = host(saved["logits"])
    Lr = O.router_logits(inp.x, inp.w_r, inp.bias)
    scale = float(np.max(np.abs(Lr)))
    assert np.max(np.abs(Lg.astype(np.float64) - Lr)) <= 1e-4 * scale + 1e-6, "router logits"
    return Lg


def assert_same_route(saved, ref):
    for k in ("topk_idx", "counts", "offsets", "dst_rows", "row_route"):
        assert np.array_equal(host(saved[k]), ref[k]), k
    assert np.max(np.abs(host(saved["topk_prob"]).astype(np.float64) - ref["topk_prob"]), initial=0) <= 1e-6


LAYER_CASES = {
    "tiny_bf16": S.WORKLOADS["tiny_bf16"],
    "dsv3_shape_small": S.scaled(S.WORKLOADS["dsv3_bf16"], "dsv3_shape_small", N=512, D=256, E=32, K=8, H=128),
    "mixtral_shape_small": S.scaled(S.WORKLOADS["mixtral_bf16"], "mixtral_shape_small", N=600, D=256, E=8, K=2, H=448),
    "qwen3_shape_small": S.scaled(S.WORKLOADS["qwen3_235b_bf16_fwdbwd"], "qwen3_shape_small", N=700, D=256,
                                  E=16, K=4, H=192),
}


@pytest.mark.parametrize("sched", [M.MOE_SCHED_STAGED, M.MOE_SCHED_READY])
@pytest.mark.parametrize("name", list(LAYER_CASES))
def test_layer_fwd_bf16(name, sched):
    wl = LAYER_CASES[name]
    print(f"layer fwd {name} sched={sched}", flush=True)
    inp = S.make_inputs(wl, 1)
    w, _ = _weights(inp)
    drop = dev(inp.drop) if inp.drop is not None else None
    layer = M.MoeLayer(w, wl.N, wl.K, drop=drop, sched=sched)
    out = layer.forward(dev_bf16(inp.x))
    torch.cuda.synchronize()
    ref = O.layer_fwd(inp.x, inp.w_r, inp.bias, inp.w_gate, inp.w_up, inp.w_down, wl.K, drop=inp.drop)
    sv = layer.saved
    assert int(host(sv["status"])[0]) == 0
    same = check_routing(sv, ref, wl.K)
    assert np.max(np.abs(host(sv["topk_prob"])[same] - ref["topk_prob"][same]), initial=0) <= 1e-6
    if np.all(same):
        for k in ("counts", "offsets", "dst_rows", "row_route"):
            assert np.array_equal(host(sv[k]), ref[k]), k
        n = int(ref["offsets"][-1])
        assert np.array_equal(bits(sv["xd"])[:n], O.bf16_bits(ref["xd"][:n]))
        for k in ("g", "u", "h", "y"):
            assert_bf16_close(vals(sv[k])[:n], ref[k][:n], k)
    assert_bf16_close(vals(out)[same], ref["out"][same], "out")


SINGLE_CASES = {
    "dsv3_shape_small": LAYER_CASES["dsv3_shape_small"],
    "qwen3_shape_small": LAYER_CASES["qwen3_shape_small"],
    # ragged: tokens not a multiple of a route chunk (16) or router block, few experts empty
    "ragged_e24": S.scaled(S.WORKLOADS["dsv3_bf16"], "ragged_e24", N=333, D=192, E=24, K=3, H=320),
    # 2048+ tokens: the staged router takes 128-row blocks (and another split)
    "router_bm128": S.scaled(S.WORKLOADS["qwen3_235b_bf16_fwdbwd"], "router_bm128", N=2100, D=128, E=64, K=6,
                             H=192),
    # rows of three fold segments, the last one short, and dispatch rows wider
    # than one pass of its two-row loop
    "wide_rows": S.scaled(S.WORKLOADS["dsv3_bf16"], "wide_rows", N=96, D=8256, E=16, K=2, H=128),
}
SINGLE_KEYS = ("logits", "topk_idx", "topk_prob", "counts", "offsets", "dst_rows", "row_route", "xd", "g", "u",
               "h", "y")


@pytest.mark.parametrize("name", list(SINGLE_CASES))
def test_layer_fwd_single_launch_equals_staged(name):
    """The single-launch forward (router, route, dispatch, GEMM1, GEMM2 and
    the fold in one persistent launch) computes each step as its separate
    launch does: every saved tensor and the output are bitwise the staged
    forward's, whose parity with the oracle the tests above establish.  The
    single-launch outputs are poisoned first, so an element it fails to write
    cannot pass."""
    wl = SINGLE_CASES[name]
    print(f"single-launch fwd {name}", flush=True)
    inp = S.make_inputs(wl, 3)
    w, _ = _weights(inp)
    drop = dev(inp.drop) if inp.drop is not None else None
    x = dev_bf16(inp.x)
    staged = M.MoeLayer(w, wl.N, wl.K, drop=drop)
    want = staged.forward(x)
    one = M.MoeLayer(w, wl.N, wl.K, drop=drop, sched=M.MOE_SCHED_SINGLE)
    for t in list(one.saved.values()) + [one.out]:
        t.view(torch.uint8).fill_(0xA5)
    got = one.forward(x)
    torch.cuda.synchronize()
    assert int(host(one.saved["status"])[0]) == 0
    n = int(host(staged.saved["offsets"])[-1])
    for k in SINGLE_KEYS:
        a, b = staged.saved[k], one.saved[k]
        if k in ("xd", "g", "u", "h", "y"):
            a, b = a[:n], b[:n]
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), k
    assert torch.equal(got.view(torch.int16), want.view(torch.int16)), "out"
    # and the oracle on the same logits, for the output
    ref = O.layer_fwd(inp.x, inp.w_r, inp.bias, inp.w_gate, inp.w_up, inp.w_down, wl.K, drop=inp.drop,
                      logits=logits_checked(one.saved, inp))
    assert_same_route(one.saved, ref)
    assert_bf16_close(vals(got), ref["out"], "out")


READY_CASES = {
    # rows wider than one pass of the dispatch's two-row loop (D > 8192)
    "wide_rows": S.scaled(S.WORKLOADS["dsv3_bf16"], "wide_rows", N=96, D=8256, E=16, K=2, H=128),
    # fewer tokens than workgroups: most dispatch shares are empty
    "five_tokens": S.scaled(S.WORKLOADS["dsv3_bf16"], "five_tokens", N=5, D=256, E=16, K=4, H=128),
    # enough GEMM1 tiles (about 6000) that workgroups publish full batches
    # of stored tiles before the queue's last window
    "many_tiles": S.scaled(S.WORKLOADS["qwen3_235b_bf16_fwdbwd"], "many_tiles", N=9216, D=256, E=64, K=8,
                           H=2048),
}


@pytest.mark.parametrize("name", list(READY_CASES))
def test_ready_queue_equals_staged(name):
    """The readiness-gated launch (dispatch shares, GEMM1 tiles after the
    dispatch, GEMM2 tiles per GEMM1 row block) stores every row of X_d, G,
    U, H and Y bitwise as the staged launches do, outputs poisoned first."""
    wl = READY_CASES[name]
    print(f"READY fwd {name}", flush=True)
    inp = S.make_inputs(wl, 5)
    w, _ = _weights(inp)
    drop = dev(inp.drop) if inp.drop is not None else None
    x = dev_bf16(inp.x)
    staged = M.MoeLayer(w, wl.N, wl.K, drop=drop)
    want = staged.forward(x)
    ready = M.MoeLayer(w, wl.N, wl.K, drop=drop, sched=M.MOE_SCHED_READY)
    for t in list(ready.saved.values()) + [ready.out]:
        t.view(torch.uint8).fill_(0xA5)
    got = ready.forward(x)
    torch.cuda.synchronize()
    assert int(host(ready.saved["status"])[0]) == 0
    n = int(host(staged.saved["offsets"])[-1])
    for k in ("counts", "offsets", "dst_rows", "xd", "g", "u", "h", "y"):
        a, b = staged.saved[k], ready.saved[k]
        if k in ("xd", "g", "u", "h", "y"):
            a, b = a[:n], b[:n]
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), k
    assert torch.equal(got.view(torch.int16), want.view(torch.int16)), "out"


def test_single_launch_barrier_expiry_is_reported_and_the_next_call_recovers():
    """Barrier arrivals and readiness withheld from the host, every wait
    bounded to a few polls: each barrier wait expires, the workgroups stop,
    the launch ends and the status word reports MOE_STATUS_WAIT_EXPIRED.  The
    next call reports 0 and equals the staged forward bit for bit."""
    wl = SINGLE_CASES["ragged_e24"]
    print("single-launch fwd: forced barrier expiry", flush=True)
    inp = S.make_inputs(wl, 4)
    w, _ = _weights(inp)
    x = dev_bf16(inp.x)
    want = M.MoeLayer(w, wl.N, wl.K).forward(x).clone()
    layer = M.MoeLayer(w, wl.N, wl.K, sched=M.MOE_SCHED_SINGLE)
    layer.ready_test_polls = 4
    layer.forward(x)
    torch.cuda.synchronize()
    assert int(host(layer.saved["status"])[0]) == M.MOE_STATUS_WAIT_EXPIRED
    layer.ready_test_polls = 0
    out = layer.forward(x)
    torch.cuda.synchronize()
    assert int(host(layer.saved["status"])[0]) == 0
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))


# the router's dX_r product contracts over E in whole 64-column steps, so the
# single launch takes the router backward for E % 64 == 0
SINGLE_CASES["router_e64"] = S.scaled(S.WORKLOADS["qwen3_235b_bf16_fwdbwd"], "router_e64", N=700, D=256, E=64,
                                      K=4, H=192)
BWD_SINGLE_CASES = [("tiny_bf16", False), ("qwen3_shape_small", False), ("dsv3_shape_small", False),
                    ("ragged_e24", False), ("router_e64", True), ("router_bm128", True)]


@pytest.mark.parametrize("name,router", BWD_SINGLE_CASES)
def test_layer_bwd_single_launch_equals_staged(name, router):
    """The single-launch backward (combine backward, both dgrads and all
    weight gradients, the router backward and the fold in one persistent
    launch) gives every gradient bitwise equal to the staged backward's,
    whose parity with the oracle the tests below establish.  The gradients
    are poisoned first.  Its forward is the staged one (any E)."""
    wl = {**LAYER_CASES, **SINGLE_CASES}[name]
    print(f"single-launch bwd {name} router={router}", flush=True)
    inp = S.make_inputs(wl, 6)
    dout = dev_bf16(inp.dout if inp.dout is not None else S.random_bf16((wl.N, wl.D), 6, 9))
    w, _ = _weights(inp)
    drop = dev(inp.drop) if inp.drop is not None else None
    x = dev_bf16(inp.x)
    want = M.MoeLayer(w, wl.N, wl.K, drop=drop, with_bwd=True, router_bwd=router)
    want.forward(x)
    gs = {k: v.clone() for k, v in want.backward(x, dout).items()}
    one = M.MoeLayer(w, wl.N, wl.K, drop=drop, with_bwd=True, router_bwd=router)
    one.forward(x)
    one.sched = M.MOE_SCHED_SINGLE
    for t in one.grads.values():
        t.view(torch.uint8).fill_(0xA5)
    g1 = one.backward(x, dout)
    torch.cuda.synchronize()
    assert int(host(one.saved["status"])[0]) == 0
    assert set(gs) == set(g1)
    for k in gs:
        assert torch.equal(gs[k].view(torch.uint8), g1[k].view(torch.uint8)), k


def test_single_launch_backward_with_aux_loss_and_barrier_expiry():
    """The aux loss's gradient joins the router backward in the single launch
    too (bitwise the staged result); and with barrier arrivals withheld every
    barrier wait of the backward expires and is reported, after which the
    next call is exact again."""
    wl = SINGLE_CASES["router_e64"]
    inp = S.make_inputs(wl, 7)
    dout = dev_bf16(S.random_bf16((wl.N, wl.D), 7, 9))
    w, _ = _weights(inp)
    x = dev_bf16(inp.x)
    want = M.MoeLayer(w, wl.N, wl.K, with_bwd=True, router_bwd=True, aux_alpha=0.01)
    want.forward(x)
    gs = {k: v.clone() for k, v in want.backward(x, dout, d_aux=1.5).items()}
    one = M.MoeLayer(w, wl.N, wl.K, with_bwd=True, router_bwd=True, aux_alpha=0.01)
    one.forward(x)
    one.sched = M.MOE_SCHED_SINGLE
    g1 = one.backward(x, dout, d_aux=1.5)
    torch.cuda.synchronize()
    for k in gs:
        assert torch.equal(gs[k].view(torch.uint8), g1[k].view(torch.uint8)), k
    print("single-launch bwd: forced barrier expiry", flush=True)
    one.saved["status"].zero_()
    one.ready_test_polls = 4
    one.backward(x, dout, d_aux=1.5)
    torch.cuda.synchronize()
    assert int(host(one.saved["status"])[0]) == M.MOE_STATUS_WAIT_EXPIRED
    one.ready_test_polls = 0
    one.saved["status"].zero_()
    g1 = one.backward(x, dout, d_aux=1.5)
    torch.cuda.synchronize()
    assert int(host(one.saved["status"])[0]) == 0
    for k in gs:
        assert torch.equal(gs[k].view(torch.uint8), g1[k].view(torch.uint8)), k


@pytest.mark.parametrize("name", ["tiny_bf16", "qwen3_shape_small", "dsv3_shape_small"])
def test_layer_bwd_bf16(name):
    wl = LAYER_CASES[name]
    print(f"layer bwd {name}", flush=True)
    inp = S.make_inputs(wl, 2)
    dout = inp.dout if inp.dout is not None else S.random_bf16((wl.N, wl.D), 2, 9)
    w, _ = _weights(inp)
    drop = dev(inp.drop) if inp.drop is not None else None
    layer = M.MoeLayer(w, wl.N, wl.K, drop=drop, with_bwd=True)
    x = dev_bf16(inp.x)
    layer.forward(x)
    g = layer.backward(x, dev_bf16(dout))
    torch.cuda.synchronize()
    ref = O.layer_fwd(inp.x, inp.w_r, inp.bias, inp.w_gate, inp.w_up, inp.w_down, wl.K, drop=inp.drop,
                      logits=logits_checked(layer.saved, inp))
    assert_same_route(layer.saved, ref)
    rb = O.layer_bwd(ref, dout, inp.w_gate, inp.w_up, inp.w_down)
    assert_bf16_close(vals(g["dx"]), rb["dx"], "dx")
    assert_bf16_close(host(g["dprob"]), rb["dprob"], "dprob")
    assert np.all(host(g["dprob"])[ref["dst_rows"] < 0] == 0)
    assert_bf16_close(vals(g["dw_down"]), rb["dw_down"], "dw_down")
    assert_bf16_close(vals(g["dw_gate"]), rb["dw_gate"], "dw_gate")
    assert_bf16_close(vals(g["dw_up"]), rb["dw_up"], "dw_up")
    for e in np.nonzero(ref["counts"] == 0)[0]:
        assert np.all(bits(g["dw_gate"])[e] == 0)


ROUTER_BWD_CASES = dict(LAYER_CASES)
ROUTER_BWD_CASES.update({
    "router_e128": S.scaled(S.WORKLOADS["qwen3_235b_bf16_fwdbwd"], "router_e128", N=2100, D=512, E=128, K=8,
                            H=128),
    "router_e256": S.scaled(S.WORKLOADS["dsv3_bf16"], "router_e256", N=1000, D=384, E=256, K=8, H=64),
})


@pytest.mark.parametrize("renorm", [0, 1])
@pytest.mark.parametrize("name", ["tiny_bf16", "qwen3_shape_small", "dsv3_shape_small", "router_e128",
                                  "router_e256"])
def test_layer_bwd_router(name, renorm):
    """Router gradients through the layer backward (KOSMOS section 3.3.2 step 2):
    dlogits, dW_r, db_r, and dx including dlogits . W_r."""
    wl = ROUTER_BWD_CASES[name]
    print(f"layer bwd with router {name} renorm={renorm}", flush=True)
    inp = S.make_inputs(wl, 3)
    dout = inp.dout if inp.dout is not None else S.random_bf16((wl.N, wl.D), 3, 9)
    w, _ = _weights(inp)
    drop = dev(inp.drop) if inp.drop is not None else None
    layer = M.MoeLayer(w, wl.N, wl.K, drop=drop, renorm=renorm, with_bwd=True, router_bwd=True)
    x = dev_bf16(inp.x)
    layer.forward(x)
    g = layer.backward(x, dev_bf16(dout))
    torch.cuda.synchronize()
    ref = O.layer_fwd(inp.x, inp.w_r, inp.bias, inp.w_gate, inp.w_up, inp.w_down, wl.K, drop=inp.drop,
                      renorm=renorm, logits=logits_checked(layer.saved, inp))
    assert_same_route(layer.saved, ref)
    rb = O.layer_bwd(ref, dout, inp.w_gate, inp.w_up, inp.w_down)
    rr = O.router_bwd(ref["logits"], ref["topk_idx"], rb["dprob"], inp.x, inp.w_r, renorm)
    dl = host(g["dlogits"]).astype(np.float64)
    assert np.max(np.abs(dl - rr["dlogits"])) <= 1e-3 * np.max(np.abs(rr["dlogits"])) + 1e-7, "dlogits"
    assert_bf16_close(vals(g["dw_r"]), rr["dw_r"], "dw_r")
    # db_r is the column sum of dlogits, in fp32: against the GPU's own dlogits
    # to summation accuracy, and against the oracle within what dprob's bf16
    # tolerance (the forward Y it is taken from) allows per term, since the
    # columns cancel
    db = host(g["db_r"]).astype(np.float64)
    assert np.all(np.abs(db - dl.sum(axis=0)) <= 1e-5 * np.abs(dl).sum(axis=0) + 1e-7), "db_r vs its dlogits"
    assert np.all(np.abs(db - rr["db_r"]) <= 1e-2 * np.abs(rr["dlogits"]).sum(axis=0) + 1e-6), "db_r"
    assert_bf16_close(vals(g["dx"]), O.values(rb["dx"]) + rr["dx_r"], "dx with dX_r")
    assert_bf16_close(vals(g["dw_down"]), rb["dw_down"], "dw_down")


@pytest.mark.parametrize("name", ["qwen3_shape_small", "mixtral_shape_small"])
def test_layer_bwd_recompute_h_is_bitwise_equal(name):
    """SwiGLU-recompute mode: the backward without the saved H (recomputed from
    G and U) gives every gradient bit for bit as with it."""
    wl = LAYER_CASES[name]
    print(f"layer bwd recompute H {name}", flush=True)
    inp = S.make_inputs(wl, 4)
    dout = dev_bf16(inp.dout if inp.dout is not None else S.random_bf16((wl.N, wl.D), 4, 9))
    w, _ = _weights(inp)
    drop = dev(inp.drop) if inp.drop is not None else None
    layer = M.MoeLayer(w, wl.N, wl.K, drop=drop, with_bwd=True, router_bwd=True)
    x = dev_bf16(inp.x)
    layer.forward(x)
    g1 = {k: v.clone() for k, v in layer.backward(x, dout).items()}
    layer.saved["h"].fill_(float("nan"))        # the saved H must not be read
    g2 = layer.backward(x, dout, recompute_h=True)
    torch.cuda.synchronize()
    for k in g1:
        assert torch.equal(g1[k].view(torch.uint8), g2[k].view(torch.uint8)), k


@pytest.mark.parametrize("grouped", [False, True])
def test_layer_aux_loss_and_grouped_routing(grouped):
    """The aux loss from the route step, its gradient in the router backward,
    and group-limited routing through the whole layer (KOSMOS section 3.3.1
    step 1)."""
    wl = S.scaled(S.WORKLOADS["dsv3_bf16"], "aux_case", N=512, D=256, E=32, K=8, H=128)
    G, M_ = (4, 2) if grouped else (0, 0)
    alpha, d_aux = 0.01, 3.0
    print(f"layer aux loss grouped={grouped}", flush=True)
    inp = S.make_inputs(wl, 6)
    dout = S.random_bf16((wl.N, wl.D), 6, 9)
    w, _ = _weights(inp)
    layer = M.MoeLayer(w, wl.N, wl.K, with_bwd=True, router_bwd=True, n_group=G, topk_group=M_,
                       aux_alpha=alpha)
    x = dev_bf16(inp.x)
    out = layer.forward(x)
    g = layer.backward(x, dev_bf16(dout), d_aux=d_aux)
    torch.cuda.synchronize()
    Lg = logits_checked(layer.saved, inp)
    ref = O.layer_fwd(inp.x, inp.w_r, inp.bias, inp.w_gate, inp.w_up, inp.w_down, wl.K, logits=Lg)
    idx_ref = O.topk_select_grouped(Lg, wl.K, G, M_) if grouped else ref["topk_idx"]
    idx_gpu = host(layer.saved["topk_idx"])
    diff = np.nonzero(np.any(idx_gpu != idx_ref, axis=1))[0]
    if len(diff):
        # the group decision is taken on fp32 probabilities on the GPU and in
        # float64 here: a token may differ only at a near-tie of its kept/dropped
        # group scores, and the GPU's choice must be a valid grouped selection;
        # the reference then follows the GPU's choice for those tokens
        assert grouped, "plain top-K on identical logits must agree"
        gsc = np.sort(O.group_scores(Lg[diff], G), axis=1)[:, ::-1]
        assert np.all(gsc[:, M_ - 1] - gsc[:, M_] <= 1e-5), "grouped routing differs beyond a near-tie"
        for t in diff:
            kept = set(int(e) // (wl.E // G) for e in idx_gpu[t])
            assert len(kept) <= M_ and len(set(idx_gpu[t])) == wl.K
        idx_ref = idx_ref.copy()
        idx_ref[diff] = idx_gpu[diff]
    assert np.array_equal(idx_gpu, idx_ref)
    counts = host(layer.saved["counts"])
    aux_ref, _ = O.aux_loss(Lg, counts, wl.K, alpha)
    assert abs(float(host(layer.saved["aux"])[0]) - aux_ref) <= 1e-5 * abs(aux_ref), "aux"
    if grouped:
        fr = O.layer_fwd(inp.x, inp.w_r, inp.bias, inp.w_gate, inp.w_up, inp.w_down, wl.K)
        assert not np.array_equal(idx_ref, fr["topk_idx"]), "grouping should change some selections"
    # the routed layer with the grouped selection, then the backward with the aux term
    prob = O.route_probs(Lg, idx_ref, 0)
    c, o, d, r = O.route_map(idx_ref, None, wl.E, 1, wl.N * wl.K)
    xd = O.dispatch(inp.x, r, wl.K)
    G_, U_, H_, Y_ = O.experts_fwd(xd, o, inp.w_gate, inp.w_up, inp.w_down)
    assert_bf16_close(vals(out), O.combine(Y_, d, prob), "out")
    fwd = dict(xd=xd, g=G_, u=U_, h=H_, y=Y_, dst_rows=d, topk_prob=prob, offsets=o)
    rb = O.layer_bwd(fwd, dout, inp.w_gate, inp.w_up, inp.w_down)
    rr = O.router_bwd(Lg, idx_ref, rb["dprob"], inp.x, inp.w_r, 0,
                      aux_dl=O.aux_dlogits(Lg, counts, wl.K, alpha, d_aux))
    dl = host(g["dlogits"]).astype(np.float64)
    assert np.max(np.abs(dl - rr["dlogits"])) <= 1e-3 * np.max(np.abs(rr["dlogits"])) + 1e-7, "dlogits"
    assert_bf16_close(vals(g["dw_r"]), rr["dw_r"], "dw_r")


def _with_shared(inp, seed):
    """The test weights plus one shared expert (the last), N(0, 1/D) and N(0, 1/H)."""
    rng = np.random.default_rng(seed)
    D, H = inp.w_gate.shape[2], inp.w_gate.shape[1]
    add = lambda a, std: np.concatenate([a, S.f32_to_bf16_bits((rng.standard_normal((1,) + a.shape[1:]) * std)
                                                             .astype(np.float32))])
    return add(inp.w_gate, D ** -0.5), add(inp.w_up, D ** -0.5), add(inp.w_down, H ** -0.5)


@pytest.mark.parametrize("name", ["qwen3_shape_small", "dsv3_shape_small"])
def test_layer_shared_expert_bf16(name):
    """A shared expert in the same grouped-GEMM launches as the routed ones
    (KOSMOS Appendix A, Table A.1): forward and backward against the oracle."""
    wl = LAYER_CASES[name]
    print(f"layer shared expert {name}", flush=True)
    inp = S.make_inputs(wl, 7)
    dout = S.random_bf16((wl.N, wl.D), 7, 9)
    wg, wu, wd = _with_shared(inp, 7)
    w = M.LayerWeights(w_r=dev_bf16(inp.w_r), bias=dev(inp.bias) if inp.bias is not None else None)
    w.w_gate, w.w_up, w.w_down = dev_bf16(wg), dev_bf16(wu), dev_bf16(wd)
    drop = dev(inp.drop) if inp.drop is not None else None
    layer = M.MoeLayer(w, wl.N, wl.K, drop=drop, with_bwd=True)
    x = dev_bf16(inp.x)
    out = layer.forward(x)
    g = layer.backward(x, dev_bf16(dout))
    torch.cuda.synchronize()
    ref = O.layer_fwd(inp.x, inp.w_r, inp.bias, wg, wu, wd, wl.K, drop=inp.drop, n_shared=1,
                      logits=logits_checked(layer.saved, inp))
    sv = layer.saved
    assert_same_route(sv, ref)
    n = int(ref["offsets"][-1])
    assert np.array_equal(bits(sv["xd"])[:n], O.bf16_bits(ref["xd"][:n]))
    assert_bf16_close(vals(sv["y"])[:n], ref["y"][:n], "y")
    assert_bf16_close(vals(out), ref["out"], "out")
    rb = O.layer_bwd(ref, dout, wg, wu, wd)
    assert_bf16_close(vals(g["dx"]), rb["dx"], "dx")
    assert_bf16_close(host(g["dprob"]), rb["dprob"], "dprob")
    for k in ("dw_gate", "dw_up", "dw_down"):
        assert_bf16_close(vals(g[k]), rb[k], k)
        assert_bf16_close(vals(g[k])[-1], rb[k][-1], k + " (shared)")


def test_layer_shared_expert_mxfp8():
    wl = S.scaled(S.WORKLOADS["dsv3_mxfp8"], "mx_shared", N=300, D=256, E=16, K=4, H=128)
    print("layer mxfp8 shared expert", flush=True)
    inp = S.make_inputs(wl, 8)
    wg, wu, wd = _with_shared(inp, 8)
    q = O.quantize_weights_mxfp8(wg, wu, wd)
    w = M.LayerWeights(w_r=dev_bf16(inp.w_r), bias=dev(inp.bias) if inp.bias is not None else None)
    w.wq = {k: dev(v) for k, v in q.items()}
    layer = M.MoeLayer(w, wl.N, wl.K, mxfp8=True)
    out = layer.forward(dev_bf16(inp.x))
    torch.cuda.synchronize()
    sv = layer.saved
    ref = O.layer_fwd_mxfp8(inp.x, inp.w_r, inp.bias, q, wl.K, n_shared=1, logits=logits_checked(sv, inp))
    assert_same_route(sv, ref)
    n = int(ref["offsets"][-1])
    assert np.array_equal(host(sv["xd_q"])[:n], ref["xq"][:n])
    assert np.array_equal(host(sv["xd_s"])[:n], ref["xs"][:n])
    assert rel_frobenius(vals(out), ref["out"]) <= 3e-2


MX_BWD_CASES = {
    "mx_16e": dict(N=256, D=256, E=16, K=4, H=128),
    "mx_32e": dict(N=300, D=512, E=32, K=8, H=256),
    "mx_8e_ragged": dict(N=333, D=384, E=8, K=2, H=192),
}


@pytest.mark.parametrize("shared,router", [(False, False), (True, False), (False, True)])
@pytest.mark.parametrize("name", list(MX_BWD_CASES))
def test_layer_bwd_mxfp8(name, shared, router):
    """MXFP8 backward through moe_layer_bwd against the oracle's: block-scaled
    dgrads, bf16 wgrads on dequantized activations.

    Tolerances (relative Frobenius): the quantized operands of the down dgrad
    (dY_d from the same bf16 values, the weight copies) are identical on both
    sides, so dG and dU differ only by fp32-vs-float64 accumulation and their
    bf16 rounding (2^-9 relative), and with them the gate/up weight gradients:
    5e-3.  dX_d re-quantizes [dG | dU] and dW_down reads the forward's
    quantized H: where the two sides' bf16 inputs differ in the last bit, an
    E4M3 code can move by one step (2^-4 of that element) on a small fraction
    of elements, so dx, dw_down and dprob (from the forward's Y) get 1e-2;
    the router's gradients follow dprob."""
    cfg = MX_BWD_CASES[name]
    wl = S.scaled(S.WORKLOADS["dsv3_mxfp8"], name, bwd=True, **cfg)
    print(f"layer bwd mxfp8 {name} shared={shared} router={router}", flush=True)
    inp = S.make_inputs(wl, 31)
    wg, wu, wd = _with_shared(inp, 31) if shared else (inp.w_gate, inp.w_up, inp.w_down)
    q = O.quantize_weights_mxfp8(wg, wu, wd)
    qt = O.quantize_weights_mxfp8_dgrad(wg, wu, wd)
    w = M.LayerWeights(w_r=dev_bf16(inp.w_r), bias=dev(inp.bias) if inp.bias is not None else None)
    w.wq = {k: dev(v) for k, v in q.items()}
    w.wq.update(M.quantize_weights_mxfp8_dgrad(dev_bf16(wg), dev_bf16(wu), dev_bf16(wd)))
    layer = M.MoeLayer(w, wl.N, wl.K, mxfp8=True, with_bwd=True, router_bwd=router)
    x = dev_bf16(inp.x)
    layer.forward(x)
    g = layer.backward(x, dev_bf16(inp.dout))
    torch.cuda.synchronize()
    for k in qt:
        assert np.array_equal(host(w.wq[k]), qt[k]), k
    ref = O.layer_fwd_mxfp8(inp.x, inp.w_r, inp.bias, q, wl.K, n_shared=1 if shared else 0,
                            logits=logits_checked(layer.saved, inp))
    assert_same_route(layer.saved, ref)
    rb = O.layer_bwd_mxfp8(ref, inp.dout, qt)
    for k, tol in (("dw_gate", 5e-3), ("dw_up", 5e-3), ("dw_down", 1e-2), ("dprob", 1e-2)):
        got = vals(g[k]) if k != "dprob" else host(g[k])
        assert np.all(np.isfinite(got)), k
        err = rel_frobenius(got, rb[k])
        print(f"  {k} rel {err:.2e}", flush=True)
        assert err <= tol, (k, err)
    for e in np.nonzero(ref["counts"] == 0)[0]:
        assert np.all(bits(g["dw_gate"])[e] == 0)
    dx_ref = rb["dx"]
    if router:
        rr = O.router_bwd(ref["logits"], ref["topk_idx"], rb["dprob"], inp.x, inp.w_r, 0)
        dx_ref = O.values(rb["dx"]) + rr["dx_r"]
        err = rel_frobenius(host(g["dlogits"]), rr["dlogits"])
        err_w = rel_frobenius(vals(g["dw_r"]), rr["dw_r"])
        print(f"  dlogits rel {err:.2e}  dw_r rel {err_w:.2e}", flush=True)
        assert err <= 1e-2, ("dlogits", err)
        assert err_w <= 1e-2, ("dw_r", err_w)
    err = rel_frobenius(vals(g["dx"]), dx_ref)
    print(f"  dx rel {err:.2e}", flush=True)
    assert err <= 1e-2, ("dx", err)


def test_layer_bwd_mxfp8_deterministic():
    """Two MXFP8 backward calls give the same bits (the persistent GEMMs'
    results do not depend on which workgroup claims a tile)."""
    wl = S.scaled(S.WORKLOADS["dsv3_mxfp8"], "mx_det", N=400, D=256, E=16, K=4, H=128, bwd=True)
    print("layer bwd mxfp8 determinism", flush=True)
    inp = S.make_inputs(wl, 32)
    w = M.LayerWeights(w_r=dev_bf16(inp.w_r), bias=dev(inp.bias) if inp.bias is not None else None)
    wg, wu, wd = dev_bf16(inp.w_gate), dev_bf16(inp.w_up), dev_bf16(inp.w_down)
    w.wq = M.quantize_weights_mxfp8(wg, wu, wd)
    w.wq.update(M.quantize_weights_mxfp8_dgrad(wg, wu, wd))
    layer = M.MoeLayer(w, wl.N, wl.K, mxfp8=True, with_bwd=True)
    x, dout = dev_bf16(inp.x), dev_bf16(inp.dout)
    layer.forward(x)
    g1 = {k: v.clone() for k, v in layer.backward(x, dout).items()}
    g2 = layer.backward(x, dout)
    torch.cuda.synchronize()
    for k in g1:
        assert torch.equal(g1[k].view(torch.uint8), g2[k].view(torch.uint8)), k


@pytest.mark.parametrize("N,D,E,K,H", [(256, 256, 16, 4, 128), (300, 512, 32, 8, 256)])
def test_layer_fwd_mxfp8(N, D, E, K, H):
    wl = S.scaled(S.WORKLOADS["dsv3_mxfp8"], "mx_small", N=N, D=D, E=E, K=K, H=H)
    print(f"layer mxfp8 {wl}", flush=True)
    inp = S.make_inputs(wl, 3)
    w, q = _weights(inp, mxfp8=True)
    layer = M.MoeLayer(w, wl.N, wl.K, mxfp8=True)
    out = layer.forward(dev_bf16(inp.x))
    torch.cuda.synchronize()
    ref = O.layer_fwd_mxfp8(inp.x, inp.w_r, inp.bias, q, wl.K)
    sv = layer.saved
    same = check_routing(sv, ref, wl.K)
    if np.all(same):
        for k in ("counts", "offsets", "dst_rows", "row_route"):
            assert np.array_equal(host(sv[k]), ref[k]), k
        n = int(ref["offsets"][-1])
        assert np.array_equal(host(sv["xd_q"])[:n], ref["xq"][:n])
        assert np.array_equal(host(sv["xd_s"])[:n], ref["xs"][:n])
        assert_bf16_close(vals(sv["g"])[:n], ref["g"][:n], "G")
        assert rel_frobenius(vals(sv["y"])[:n], ref["y"][:n]) <= 3e-2
    assert rel_frobenius(vals(out)[same], ref["out"][same]) <= 3e-2


def test_weight_prequantization_bit_exact():
    wl = S.scaled(S.WORKLOADS["dsv3_mxfp8"], "mx_w", N=8, D=256, E=3, K=2, H=96)
    inp = S.make_inputs(wl, 4)
    q = M.quantize_weights_mxfp8(dev_bf16(inp.w_gate), dev_bf16(inp.w_up), dev_bf16(inp.w_down))
    torch.cuda.synchronize()
    ref = O.quantize_weights_mxfp8(inp.w_gate, inp.w_up, inp.w_down)
    for k in ref:
        assert np.array_equal(host(q[k]), ref[k]), k


@pytest.mark.parametrize("sched", [M.MOE_SCHED_STAGED, M.MOE_SCHED_READY, M.MOE_SCHED_SINGLE])
def test_layer_deterministic_and_overwrites_outputs(sched):
    """Bitwise identical results run to run, with every output poisoned in
    between (catches unwritten elements and races)."""
    wl = LAYER_CASES["qwen3_shape_small"]
    inp = S.make_inputs(wl, 5)
    w, _ = _weights(inp)
    layer = M.MoeLayer(w, wl.N, wl.K, drop=dev(inp.drop), with_bwd=True, sched=sched)
    x = dev_bf16(inp.x)
    dout = dev_bf16(inp.dout)
    runs = []
    for it in range(2):
        for t in list(layer.saved.values()) + list(layer.grads.values()) + [layer.out]:
            t.view(torch.uint8).fill_(0xFF if it else 0x7F)
        layer.forward(x)
        layer.backward(x, dout)
        torch.cuda.synchronize()
        runs.append({k: host(v.view(torch.uint8)).copy() for k, v in
                     dict(out=layer.out, **layer.grads).items()})
    for k in runs[0]:
        assert np.array_equal(runs[0][k], runs[1][k]), k


READY_MX_CASES = {
    # padding rows in every expert, GEMM2's last n-tile ragged (D = 640)
    "mx_small": S.scaled(S.WORKLOADS["dsv3_mxfp8"], "mx_small", N=300, D=640, E=32, K=8, H=384),
    # most experts empty, most dispatch shares empty
    "mx_five_tokens": S.scaled(S.WORKLOADS["dsv3_mxfp8"], "mx_five_tokens", N=5, D=256, E=16, K=4, H=128),
    # thousands of GEMM1 tiles: full publication batches, Big and Small tiles
    "mx_many_tiles": S.scaled(S.WORKLOADS["dsv3_mxfp8"], "mx_many_tiles", N=6144, D=512, E=64, K=8, H=2048),
}


@pytest.mark.parametrize("name", list(READY_MX_CASES))
def test_ready_queue_mxfp8_equals_staged(name):
    """The readiness-gated MXFP8 launch (quantize-on-dispatch shares with the
    padding rows zeroed, block-scaled GEMM1 storing G, U and the quantized H,
    GEMM2 gated per GEMM1 row block) stores every row of X_d, its scales, G,
    U, H, H's scales and Y bitwise as the staged MXFP8 launches do, outputs
    poisoned first."""
    wl = READY_MX_CASES[name]
    print(f"READY fwd mxfp8 {name}", flush=True)
    inp = S.make_inputs(wl, 6)
    w, _ = _weights(inp, mxfp8=True)
    x = dev_bf16(inp.x)
    staged = M.MoeLayer(w, wl.N, wl.K, mxfp8=True)
    want = staged.forward(x)
    ready = M.MoeLayer(w, wl.N, wl.K, mxfp8=True, sched=M.MOE_SCHED_READY)
    for t in list(ready.saved.values()) + [ready.out]:
        t.view(torch.uint8).fill_(0xA5)
    got = ready.forward(x)
    torch.cuda.synchronize()
    assert int(host(ready.saved["status"])[0]) == 0
    n = int(host(staged.saved["offsets"])[-1])
    for k in ("counts", "offsets", "dst_rows", "xd_q", "xd_s", "g", "u", "h_q", "h_s", "y"):
        a, b = staged.saved[k], ready.saved[k]
        if k not in ("counts", "offsets", "dst_rows"):
            a, b = a[:n], b[:n]
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), k
    assert torch.equal(got.view(torch.int16), want.view(torch.int16)), "out"


def test_ready_mxfp8_wait_expiry_is_reported_and_the_next_call_recovers():
    """The MXFP8 form of the forced give-up: every bounded wait expires and
    is reported, all kernels exit, and the next call equals the staged
    MXFP8 forward bit for bit."""
    wl = READY_MX_CASES["mx_small"]
    print("READY schedule mxfp8: forced wait expiry", flush=True)
    inp = S.make_inputs(wl, 9)
    w, _ = _weights(inp, mxfp8=True)
    x = dev_bf16(inp.x)
    want = M.MoeLayer(w, wl.N, wl.K, mxfp8=True).forward(x).clone()
    layer = M.MoeLayer(w, wl.N, wl.K, mxfp8=True, sched=M.MOE_SCHED_READY)
    layer.ready_test_polls = 4
    layer.forward(x)
    torch.cuda.synchronize()
    assert int(host(layer.saved["status"])[0]) == M.MOE_STATUS_WAIT_EXPIRED
    layer.ready_test_polls = 0
    out = layer.forward(x)
    torch.cuda.synchronize()
    assert int(host(layer.saved["status"])[0]) == 0
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))


def test_ready_wait_expiry_is_reported_and_the_next_call_recovers():
    """A forced give-up from the host (readiness withheld, every wait bounded
    to a few polls): each wait expires, the waiting items are skipped, all
    kernels exit, and the status word reports MOE_STATUS_WAIT_EXPIRED.  The
    next call, with readiness published, reports 0 and equals the staged
    schedule bit for bit."""
    wl = LAYER_CASES["dsv3_shape_small"]
    print("READY schedule: forced wait expiry", flush=True)
    inp = S.make_inputs(wl, 9)
    w, _ = _weights(inp)
    x = dev_bf16(inp.x)
    staged = M.MoeLayer(w, wl.N, wl.K)
    want = staged.forward(x).clone()
    layer = M.MoeLayer(w, wl.N, wl.K, sched=M.MOE_SCHED_READY)
    layer.ready_test_polls = 4
    layer.forward(x)
    torch.cuda.synchronize()
    assert int(host(layer.saved["status"])[0]) == M.MOE_STATUS_WAIT_EXPIRED
    layer.ready_test_polls = 0
    out = layer.forward(x)
    torch.cuda.synchronize()
    assert int(host(layer.saved["status"])[0]) == 0
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))


@pytest.mark.parametrize("mxfp8,sched", [(False, M.MOE_SCHED_STAGED), (False, M.MOE_SCHED_READY),
                                         (False, M.MOE_SCHED_SINGLE), (True, M.MOE_SCHED_STAGED),
                                         (True, M.MOE_SCHED_READY)])
def test_empty_batch(mxfp8, sched):
    """N = 0 under every schedule: the forward writes counts and offsets of 0
    and marks every row unused, the backward writes every weight gradient
    (and the router's) as 0; outputs poisoned first."""
    wl = S.scaled(S.WORKLOADS["dsv3_mxfp8" if mxfp8 else "dsv3_bf16"], "empty", N=8, D=256, E=16, K=4, H=128)
    print(f"empty batch mxfp8={mxfp8} sched={sched}", flush=True)
    inp = S.make_inputs(wl, 4)
    w, _ = _weights(inp, mxfp8=mxfp8)
    if mxfp8:
        wg, wu, wd = dev_bf16(inp.w_gate), dev_bf16(inp.w_up), dev_bf16(inp.w_down)
        w.wq.update(M.quantize_weights_mxfp8_dgrad(wg, wu, wd))
    layer = M.MoeLayer(w, 0, wl.K, mxfp8=mxfp8, with_bwd=True, router_bwd=not mxfp8, sched=sched)
    for t in list(layer.saved.values()) + list(layer.grads.values()):
        t.view(torch.uint8).fill_(0xA5)
    x = torch.empty((0, wl.D), dtype=torch.bfloat16, device="cuda")
    out = layer.forward(x)
    torch.cuda.synchronize()
    assert out.shape == (0, wl.D)
    sv = layer.saved
    assert int(host(sv["status"])[0]) == 0
    assert not host(sv["counts"]).any() and not host(sv["offsets"]).any()
    assert np.all(host(sv["row_route"]) == -1)
    g = layer.backward(x, torch.empty((0, wl.D), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    names = ["dw_gate", "dw_up", "dw_down"] + ([] if mxfp8 else ["dw_r", "db_r"])
    for k in names:
        assert not host(g[k].view(torch.uint8)).any(), k


DEGENERATE_CASES = {
    # every route dropped: every expert segment is empty
    "all_dropped": S.scaled(S.WORKLOADS["dsv3_bf16"], "all_dropped", N=100, D=256, E=16, K=4, H=128),
    # K = E: every expert takes every token
    "k_equals_e": S.scaled(S.WORKLOADS["dsv3_bf16"], "k_equals_e", N=96, D=256, E=16, K=16, H=128),
}


@pytest.mark.parametrize("mxfp8,sched", [(False, M.MOE_SCHED_STAGED), (False, M.MOE_SCHED_READY),
                                         (False, M.MOE_SCHED_SINGLE), (True, M.MOE_SCHED_STAGED),
                                         (True, M.MOE_SCHED_READY)])
@pytest.mark.parametrize("name", list(DEGENERATE_CASES))
def test_degenerate_routing(name, mxfp8, sched):
    """Routing's degenerate cases through the whole layer under every
    schedule, against the oracle: with every route dropped no expert has a
    row, the output is exactly 0 and every weight gradient is 0; with K = E
    every expert holds every token."""
    wl = DEGENERATE_CASES[name]
    print(f"degenerate routing {name} mxfp8={mxfp8} sched={sched}", flush=True)
    inp = S.make_inputs(wl, 7)
    drop = np.ones((wl.N, wl.K), np.uint8) if name == "all_dropped" else None
    w, q = _weights(inp, mxfp8=mxfp8)
    if mxfp8:
        w.wq.update(M.quantize_weights_mxfp8_dgrad(dev_bf16(inp.w_gate), dev_bf16(inp.w_up), dev_bf16(inp.w_down)))
    layer = M.MoeLayer(w, wl.N, wl.K, mxfp8=mxfp8, drop=dev(drop) if drop is not None else None, with_bwd=True,
                       sched=sched)
    for t in list(layer.saved.values()) + [layer.out] + list(layer.grads.values()):
        t.view(torch.uint8).fill_(0xA5)
    x = dev_bf16(inp.x)
    out = layer.forward(x)
    torch.cuda.synchronize()
    sv = layer.saved
    assert int(host(sv["status"])[0]) == 0
    logits = logits_checked(sv, inp)
    if mxfp8:
        ref = O.layer_fwd_mxfp8(inp.x, inp.w_r, inp.bias, q, wl.K, drop=drop, logits=logits)
    else:
        ref = O.layer_fwd(inp.x, inp.w_r, inp.bias, inp.w_gate, inp.w_up, inp.w_down, wl.K, drop=drop,
                          logits=logits)
    assert_same_route(sv, ref)
    if name == "all_dropped":
        assert not host(sv["counts"]).any() and not host(sv["offsets"]).any()
        assert not bits(out).any()
    else:
        assert np.all(host(sv["counts"]) == wl.N)
        if mxfp8:
            assert rel_frobenius(vals(out), ref["out"]) <= 3e-2
        else:
            assert_bf16_close(vals(out), ref["out"], "out")
    dout = dev_bf16(S.random_bf16((wl.N, wl.D), 7, 9))
    g = layer.backward(x, dout)
    torch.cuda.synchronize()
    if name == "all_dropped":
        for k in ("dw_gate", "dw_up", "dw_down", "dx", "dprob"):
            assert not host(g[k].view(torch.uint8)).any(), k
    else:
        for k in ("dw_gate", "dw_up", "dw_down", "dx"):
            assert np.all(np.isfinite(vals(g[k]))), k


def test_nan_logits_leave_slots_invalid_and_set_the_status():
    """Logits that are NaN never win a slot; a slot with no candidate left is
    an invalid route (expert -1, probability 0, no row).  Through moe_route on
    chosen logits, then through the layer on a token row of NaN, whose status
    word reports MOE_STATUS_NO_FINITE_LOGIT while every other token routes
    and combines as usual."""
    N, E, K = 64, 8, 3
    rng = np.random.default_rng(5)
    L = rng.standard_normal((N, E)).astype(np.float32)
    L[3, :] = np.nan                       # no finite logit: all K slots invalid
    L[7, 2:] = np.nan                      # two finite logits: slot 2 invalid
    L[9, 0] = np.nan                       # one NaN: routes as usual among the rest
    o = M.route(dev(L), K)
    torch.cuda.synchronize()
    idx, dst = host(o["topk_idx"]), host(o["dst_rows"])
    assert np.all(idx[3] == -1) and np.all(dst[3] == -1)
    assert np.all(idx[7, :2] >= 0) and idx[7, 2] == -1 and dst[7, 2] == -1 and np.all(dst[7, :2] >= 0)
    assert host(o["topk_prob"])[7, 2] == 0
    ok = np.ones(N, bool)
    ok[[3, 7, 9]] = False
    assert np.array_equal(idx[ok], O.topk_select(L[ok], K))
    assert np.array_equal(idx[9], O.topk_select(np.where(np.isnan(L[9:10]), -np.inf, L[9:10]), K)[0])
    valid = idx >= 0
    c, of, d, r = O.route_map(np.where(valid, idx, -1), None, E, 1, N * K)
    for name, ref in (("counts", c), ("offsets", of), ("dst_rows", d), ("row_route", r)):
        assert np.array_equal(host(o[name]), ref), name
    # through the layer: one token row of NaN
    wl = LAYER_CASES["qwen3_shape_small"]
    inp = S.make_inputs(wl, 10)
    w, _ = _weights(inp)
    xb = inp.x.copy()
    xb[5] = 0x7FC0                         # bf16 NaN
    layer = M.MoeLayer(w, wl.N, wl.K)
    out = layer.forward(dev_bf16(xb))
    torch.cuda.synchronize()
    sv = layer.saved
    assert int(host(sv["status"])[0]) == M.MOE_STATUS_NO_FINITE_LOGIT
    assert np.all(host(sv["topk_idx"])[5] == -1) and np.all(host(sv["dst_rows"])[5] == -1)
    assert not bits(out)[5].any()          # a token without a route folds to zero
    keep = np.arange(wl.N) != 5
    Lg = host(sv["logits"])
    ref = O.layer_fwd(xb[keep], inp.w_r, inp.bias, inp.w_gate, inp.w_up, inp.w_down, wl.K, logits=Lg[keep])
    assert_bf16_close(vals(out)[keep], ref["out"], "out")


def test_layer_bwd_mxfp8_recompute_mode():
    """MXFP8 SwiGLU-recompute (OLMo-core Appendix A, A.14): the backward does
    not read the saved H codes (they are overwritten with NaN codes first) and
    takes the down weight gradient on H = bf16(silu(G) U) rebuilt from the
    saved G and U, against the oracle's recompute mode; the other gradients
    are bitwise those of the saved-codes backward."""
    cfg = MX_BWD_CASES["mx_32e"]
    wl = S.scaled(S.WORKLOADS["dsv3_mxfp8"], "mx_rc", bwd=True, **cfg)
    print("layer bwd mxfp8 recompute", flush=True)
    inp = S.make_inputs(wl, 33)
    q = O.quantize_weights_mxfp8(inp.w_gate, inp.w_up, inp.w_down)
    qt = O.quantize_weights_mxfp8_dgrad(inp.w_gate, inp.w_up, inp.w_down)
    w = M.LayerWeights(w_r=dev_bf16(inp.w_r), bias=dev(inp.bias) if inp.bias is not None else None)
    w.wq = {k: dev(v) for k, v in q.items()}
    w.wq.update({k: dev(v) for k, v in qt.items()})
    layer = M.MoeLayer(w, wl.N, wl.K, mxfp8=True, with_bwd=True)
    assert "h" not in layer.saved                  # the MXFP8 forward keeps H quantized only
    x, dout = dev_bf16(inp.x), dev_bf16(inp.dout)
    layer.forward(x)
    g1 = {k: v.clone() for k, v in layer.backward(x, dout).items()}
    layer.saved["h_q"].fill_(0x7F)                 # E4M3 NaN: must not be read
    g2 = layer.backward(x, dout, recompute_h=True)
    torch.cuda.synchronize()
    for k in ("dx", "dprob", "dw_gate", "dw_up"):
        assert torch.equal(g1[k].view(torch.uint8), g2[k].view(torch.uint8)), k
    ref = O.layer_fwd_mxfp8(inp.x, inp.w_r, inp.bias, q, wl.K, logits=logits_checked(layer.saved, inp))
    assert_same_route(layer.saved, ref)
    rb = O.layer_bwd_mxfp8(ref, inp.dout, qt, recompute=True)
    got = vals(g2["dw_down"])
    assert np.all(np.isfinite(got))
    err = rel_frobenius(got, rb["dw_down"])
    print(f"  dw_down rel {err:.2e}", flush=True)
    assert err <= 5e-3, err
    assert not torch.equal(g1["dw_down"].view(torch.uint8), g2["dw_down"].view(torch.uint8))


@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("name", list(MX_BWD_CASES))
def test_layer_bwd_mxfp8_native_wgrad(name, shared):
    """Native MXFP8 weight gradients (OLMo-core Appendix A, A.15) through
    moe_layer_bwd with mx_wgrad = 1, against the oracle's mx_wgrad: block-
    scaled products on column-wise copies of dY_d, H, dG, dU and X_d, each
    quantized from its bf16 values.  The copies of X_d are exact on both
    sides (gathered from the same token rows); dY_d, dG, dU and H can differ
    in a last bf16 bit between fp32 and float64 accumulation, which moves an
    E4M3 code by one step on a small fraction of elements: relative Frobenius
    1e-2.  The other gradients are bitwise those of the default mode."""
    cfg = MX_BWD_CASES[name]
    wl = S.scaled(S.WORKLOADS["dsv3_mxfp8"], name + "_nat", bwd=True, **cfg)
    print(f"layer bwd mxfp8 native wgrad {name} shared={shared}", flush=True)
    inp = S.make_inputs(wl, 35)
    wg, wu, wd = _with_shared(inp, 35) if shared else (inp.w_gate, inp.w_up, inp.w_down)
    q = O.quantize_weights_mxfp8(wg, wu, wd)
    qt = O.quantize_weights_mxfp8_dgrad(wg, wu, wd)
    w = M.LayerWeights(w_r=dev_bf16(inp.w_r), bias=dev(inp.bias) if inp.bias is not None else None)
    w.wq = {k: dev(v) for k, v in q.items()}
    w.wq.update({k: dev(v) for k, v in qt.items()})
    x, dout = dev_bf16(inp.x), dev_bf16(inp.dout)
    base = M.MoeLayer(w, wl.N, wl.K, mxfp8=True, with_bwd=True)
    base.forward(x)
    gb = {k: v.clone() for k, v in base.backward(x, dout).items()}
    layer = M.MoeLayer(w, wl.N, wl.K, mxfp8=True, with_bwd=True, mx_wgrad=True)
    layer.forward(x)
    for t in layer.grads.values():
        t.view(torch.uint8).fill_(0xFF)
    g = layer.backward(x, dout)
    torch.cuda.synchronize()
    for k in ("dx", "dprob"):
        assert torch.equal(g[k].view(torch.uint8), gb[k].view(torch.uint8)), k
    ref = O.layer_fwd_mxfp8(inp.x, inp.w_r, inp.bias, q, wl.K, n_shared=1 if shared else 0,
                            logits=logits_checked(layer.saved, inp))
    assert_same_route(layer.saved, ref)
    rb = O.layer_bwd_mxfp8(ref, inp.dout, qt, wgrad="mx")
    for k in ("dw_gate", "dw_up", "dw_down"):
        got = vals(g[k])
        assert np.all(np.isfinite(got)), k
        err = rel_frobenius(got, rb[k])
        print(f"  {k} rel {err:.2e}", flush=True)
        assert err <= 1e-2, (k, err)
    for e in np.nonzero(ref["counts"] == 0)[0]:
        for k in ("dw_gate", "dw_up", "dw_down"):
            assert not bits(g[k])[e].any(), (k, e)


@pytest.mark.parametrize("mxfp8,sched", [(False, M.MOE_SCHED_STAGED), (False, M.MOE_SCHED_READY),
                                         (False, M.MOE_SCHED_SINGLE), (True, M.MOE_SCHED_STAGED),
                                         (True, M.MOE_SCHED_READY)])
def test_layer_calls_replay_from_a_captured_graph(mxfp8, sched):
    """The layer forward and backward captured in one HIP graph (every step is
    a kernel: queue heads, plans, barrier words and the status word are reset
    by kernels of the call, no memset node) and replayed three times, with
    eager calls and synchronizations between the replays: every replay
    reproduces the eager results bit for bit, outputs poisoned before each."""
    wl = S.scaled(S.WORKLOADS["dsv3_mxfp8" if mxfp8 else "dsv3_bf16"], "graph", N=300, D=256, E=64, K=4, H=128)
    print(f"graph capture mxfp8={mxfp8} sched={sched}", flush=True)
    inp = S.make_inputs(wl, 11)
    w, _ = _weights(inp, mxfp8=mxfp8)
    if mxfp8:
        w.wq.update(M.quantize_weights_mxfp8_dgrad(dev_bf16(inp.w_gate), dev_bf16(inp.w_up), dev_bf16(inp.w_down)))
    x = dev_bf16(inp.x)
    dout = dev_bf16(S.random_bf16((wl.N, wl.D), 11, 9))
    eager = M.MoeLayer(w, wl.N, wl.K, mxfp8=mxfp8, with_bwd=True, router_bwd=not mxfp8, sched=sched)
    want_out = eager.forward(x).clone()
    want_g = {k: v.clone() for k, v in eager.backward(x, dout).items()}
    torch.cuda.synchronize()
    layer = M.MoeLayer(w, wl.N, wl.K, mxfp8=mxfp8, with_bwd=True, router_bwd=not mxfp8, sched=sched)
    layer.forward(x)   # warm-up outside the capture (the binding resolves its symbols once)
    layer.backward(x, dout)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x)
        layer.backward(x, dout)
    for rep in range(3):
        layer.out.view(torch.int16).fill_(0x7FA0)
        for t in layer.grads.values():
            t.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(host(layer.saved["status"])[0]) == 0, rep
        assert torch.equal(layer.out.view(torch.int16), want_out.view(torch.int16)), rep
        for k, v in want_g.items():
            assert torch.equal(layer.grads[k].view(torch.uint8), v.view(torch.uint8)), (rep, k)
        eager.forward(x)   # eager work on the same stream between replays
        torch.cuda.synchronize()

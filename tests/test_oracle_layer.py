"""Pins for the oracle's dispatch, experts, combine and backward.

Dispatch and combine are each other's adjoints (OLMo-core Appendix A, A.1:
dispatch forward / combine backward and combine forward / dispatch backward),
the fold sums each token's K rows weighted by its router weights (KOSMOS,
section 3.3.1 step 5), invalid routes contribute nothing (A.2), and the
backward is the adjoint sequence of the fused routed-expert node (A.1; KOSMOS
section 3.3.2).  These are checked here with identities, dot-product tests, a
dense special case computed by torch, and finite differences.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import moe_synth as S
import oracle as O


def _small(name="tiny_bf16", **kw):
    base = dict(N=16, D=32, E=4, K=2, H=32)
    base.update(kw)
    return S.scaled(S.WORKLOADS[name], **base)


def _route(inp, wl):
    L = O.router_logits(inp.x, inp.w_r, inp.bias)
    idx = O.topk_select(L, wl.K)
    p = O.route_probs(L, idx, wl.renorm)
    c, o, d, r = O.route_map(idx, inp.drop, wl.E, wl.align, wl.rows_cap)
    return L, idx, p, c, o, d, r


@pytest.mark.parametrize("K,w", [(2, (0.75, 0.25)), (8, (0.125,) * 8), (4, (0.5, 0.25, 0.125, 0.125))])
def test_identity_round_trip_is_exact(K, w):
    """Identity experts (Y_d = X_d) and dyadic weights summing to 1 give x back."""
    wl = _small(E=8, K=K, N=40)
    inp = S.make_inputs(wl, 1, weights=False)
    _, idx, _, c, o, d, r = _route(inp, wl)
    xd = O.dispatch(inp.x, r, K)
    prob = np.tile(np.array(w, np.float32), (wl.N, 1))
    out = O.combine(xd, d, prob)
    assert np.array_equal(out, O.bits_to_f64(inp.x))


def test_identity_round_trip_with_renormalised_weights_within_one_ulp():
    wl = _small(E=8, K=3, N=64, renorm=1)
    inp = S.make_inputs(wl, 2, weights=False)
    _, idx, p, c, o, d, r = _route(inp, wl)
    out = O.combine(O.dispatch(inp.x, r, 3), d, p)
    x = O.bits_to_f64(inp.x)
    ulp = np.ldexp(1.0, np.frexp(np.abs(x))[1] - 8)
    assert np.all(np.abs(out - x) <= ulp)


def test_all_invalid_routes_give_zero():
    wl = _small()
    inp = S.make_inputs(wl, 3)
    L, idx, p, *_ = _route(inp, wl)
    drop = np.ones((wl.N, wl.K), np.uint8)
    f = O.layer_fwd(inp.x, inp.w_r, inp.bias, inp.w_gate, inp.w_up, inp.w_down, wl.K, drop=drop)
    assert np.all(f["counts"] == 0) and np.all(f["out"] == 0) and np.all(f["dst_rows"] == -1)
    dout = S.random_bf16((wl.N, wl.D), 3, 0)
    b = O.layer_bwd(f, dout, inp.w_gate, inp.w_up, inp.w_down)
    assert np.all(b["dx"] == 0) and np.all(b["dprob"] == 0) and np.all(b["dw_gate"] == 0)


def test_invalid_route_contributes_nothing():
    wl = _small(N=24)
    inp = S.make_inputs(wl, 4)
    drop = np.zeros((wl.N, wl.K), np.uint8)
    drop[5, 1] = 1
    f0 = O.layer_fwd(inp.x, inp.w_r, inp.bias, inp.w_gate, inp.w_up, inp.w_down, wl.K)
    f1 = O.layer_fwd(inp.x, inp.w_r, inp.bias, inp.w_gate, inp.w_up, inp.w_down, wl.K, drop=drop)
    e = f0["topk_idx"][5, 1]
    y = f0["y"][f0["dst_rows"][5, 1]]
    manual = O.round_bf16(f0["topk_prob"][5, 0].astype(np.float64) * f0["y"][f0["dst_rows"][5, 0]])
    assert np.array_equal(f1["out"][5], manual)
    others = np.arange(wl.N) != 5
    assert np.array_equal(f1["out"][others], f0["out"][others])
    assert f1["counts"][e] == f0["counts"][e] - 1 and np.any(y != 0)


def test_adjointness_dot_products():
    wl = _small(N=30, E=6, K=3, D=24)
    inp = S.make_inputs(wl, 5, weights=False)
    _, idx, p, c, o, d, r = _route(inp, wl)
    rng = np.random.default_rng(0)
    Y = rng.standard_normal((wl.rows_cap, wl.D))
    G = rng.standard_normal((wl.N, wl.D))
    lhs = np.sum(O.combine(Y, d, p, exact=True) * G)
    rhs = np.sum(Y * O.combine_bwd(G, d, p, wl.rows_cap, exact=True))
    assert np.isclose(lhs, rhs, rtol=1e-12)
    x = rng.standard_normal((wl.N, wl.D))
    Z = rng.standard_normal((wl.rows_cap, wl.D))
    lhs = np.sum(O.dispatch(x, r, wl.K) * Z)
    rhs = np.sum(x * O.dispatch_bwd(Z, d, exact=True))
    assert np.isclose(lhs, rhs, rtol=1e-12)


def test_dense_special_case_against_torch():
    """E = 1, K = 1: the layer is the dense SwiGLU MLP times the (unit) weight.
    torch computes it in fp64 with its own fp32 -> bf16 cast at each stored
    tensor (every value there is an fp32 value rounded once)."""
    wl = _small(E=1, K=1, N=20, D=64, H=96)
    inp = S.make_inputs(wl, 6)
    f = O.layer_fwd(inp.x, inp.w_r, inp.bias, inp.w_gate, inp.w_up, inp.w_down, 1)
    assert np.all(f["topk_prob"] == 1.0)
    t = lambda a: torch.from_numpy(S.bf16_bits_to_f32(a)).double()
    bf = lambda z: z.float().to(torch.bfloat16).double()
    x, wg, wu, wd = t(inp.x), t(inp.w_gate[0]), t(inp.w_up[0]), t(inp.w_down[0])
    G, U = x @ wg.T, x @ wu.T
    # torch's cast rounds through fp32 first; that differs from one rounding
    # only when the fp32 value lands exactly on a bf16 midpoint, which these
    # seeded inputs never hit, so the comparison is exact
    Gb, Ub = bf(G), bf(U)
    H = bf(F.silu(Gb) * Ub)
    Y = bf(H @ wd.T)
    assert np.array_equal(f["g"][:20], Gb.numpy()) and np.array_equal(f["u"][:20], Ub.numpy())
    assert np.array_equal(f["h"][:20], H.numpy())
    assert np.array_equal(f["out"], Y.numpy())


def test_empty_expert_weights_are_never_read():
    wl = _small(E=8, K=1, N=8)
    inp = S.make_inputs(wl, 7)
    L = np.full((8, 8), -1.0, np.float32)
    L[:, 2] = 1.0                                        # every token picks expert 2
    wg = S.bf16_bits_to_f32(inp.w_gate).astype(np.float64)
    for e in range(8):
        if e != 2:
            wg[e] = np.nan
    f = O.layer_fwd(inp.x, inp.w_r, None, wg, inp.w_up, inp.w_down, 1, logits=L)
    assert np.all(np.isfinite(f["out"])) and f["counts"][2] == 8


@pytest.mark.parametrize("pdrop", [0.0, 0.25])
def test_backward_matches_finite_differences(pdrop):
    """fp64 central differences of the exact (unrounded) forward, route fixed."""
    wl = _small(N=16, D=32, E=4, K=2, H=32, p_drop=pdrop, bwd=True)
    inp = S.make_inputs(wl, 8)
    L, idx, p, c, o, d, r = _route(inp, wl)
    x = O.bits_to_f64(inp.x)
    wg, wu, wd = (O.bits_to_f64(a) for a in (inp.w_gate, inp.w_up, inp.w_down))
    p64 = p.astype(np.float64)
    dout = O.bits_to_f64(inp.dout)

    def fwd(x, wg, wu, wd, p64):
        xd = O.dispatch(x, r, wl.K)
        G, U, Hh, Y = O.experts_fwd(xd, o, wg, wu, wd, exact=True)
        return dict(xd=xd, g=G, u=U, h=Hh, y=Y, dst_rows=d, topk_prob=p64, offsets=o,
                    out=O.combine(Y, d, p64, exact=True))

    def loss(*a):
        return float(np.sum(fwd(*a)["out"] * dout))

    base = (x, wg, wu, wd, p64)
    f = fwd(*base)
    g = O.layer_bwd(f, dout, wg, wu, wd, exact=True)
    # dprob is stored in fp32; take the exact value for the check
    dprob_exact = np.zeros_like(p64)
    for k in range(wl.K):
        ok = d[:, k] >= 0
        dprob_exact[ok, k] = np.sum(dout[ok] * f["y"][d[ok, k]], axis=1)
    grads = (g["dx"], g["dw_gate"], g["dw_up"], g["dw_down"], dprob_exact)
    rng = np.random.default_rng(1)
    eps = 1e-6
    for i, (theta, gr) in enumerate(zip(base, grads)):
        v = rng.standard_normal(theta.shape)
        plus = list(base)
        minus = list(base)
        plus[i] = theta + eps * v
        minus[i] = theta - eps * v
        fd = (loss(*plus) - loss(*minus)) / (2 * eps)
        an = float(np.sum(gr * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (i, fd, an)
    assert np.allclose(g["dprob"], dprob_exact, rtol=1e-6, atol=1e-7)
    if pdrop:
        assert np.all(g["dprob"][d < 0] == 0)


def test_swiglu_backward_closed_form():
    """d/dg [silu(g) u] and d/du, checked against torch autograd in fp64."""
    rng = np.random.default_rng(2)
    g = torch.tensor(rng.standard_normal(1000) * 4, requires_grad=True)
    u = torch.tensor(rng.standard_normal(1000), requires_grad=True)
    dh = torch.tensor(rng.standard_normal(1000))
    (F.silu(g) * u * dh).sum().backward()
    wl = _small(N=4, D=8, E=1, K=1, H=8)
    # single expert, identity-shaped down projection isolates the SwiGLU backward
    G = g.detach().numpy().reshape(125, 8)
    U = u.detach().numpy().reshape(125, 8)
    dH = dh.numpy().reshape(125, 8)
    eye = np.eye(8)[None]
    res = O.experts_bwd(dH, np.zeros((125, 8)), G, U, np.zeros((125, 8)), np.array([0, 125]),
                        np.zeros((1, 8, 8)), np.zeros((1, 8, 8)), eye, exact=True)
    assert np.allclose(res["dg"].reshape(-1), g.grad.numpy(), rtol=1e-12, atol=1e-14)
    assert np.allclose(res["du"].reshape(-1), u.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_grouped_products_are_the_layer_parts():
    """The stand-alone grouped products equal the corresponding pieces of the
    expert forward and backward."""
    wl = _small(N=24, D=32, E=4, K=2, H=48, bwd=True)
    inp = S.make_inputs(wl, 9)
    f = O.layer_fwd(inp.x, inp.w_r, inp.bias, inp.w_gate, inp.w_up, inp.w_down, wl.K)
    o = f["offsets"]
    assert np.array_equal(O.grouped_gemm(f["xd"], inp.w_gate, o), f["g"])
    assert np.array_equal(O.grouped_gemm(f["h"], inp.w_down, o), f["y"])
    b = O.layer_bwd(f, inp.dout, inp.w_gate, inp.w_up, inp.w_down)
    assert np.array_equal(O.grouped_dgrad(b["dg"], inp.w_gate, o, b["du"], inp.w_up), b["dxd"])
    assert np.array_equal(O.grouped_wgrad(b["dyd"], f["h"], o), b["dw_down"])
    assert np.array_equal(O.grouped_wgrad(b["dg"], f["xd"], o), b["dw_gate"])
    # dgrad/wgrad are the adjoints of the forward product (dot-product test)
    rng = np.random.default_rng(3)
    A = rng.standard_normal((f["xd"].shape[0], 32))
    W = rng.standard_normal((4, 48, 32))
    Z = rng.standard_normal((A.shape[0], 48))
    lhs = np.sum(O.grouped_gemm(A, W, o, exact=True) * Z)
    assert np.isclose(lhs, np.sum(A * O.grouped_dgrad(Z, W, o, exact=True)), rtol=1e-12)
    assert np.isclose(lhs, np.sum(W * O.grouped_wgrad(Z, A, o, exact=True)), rtol=1e-12)


# ------------------------------------------------------------ shared expert ----
def _shared_case(seed=12):
    wl = _small(N=24, D=32, E=4, K=2, H=32, bwd=True)
    inp = S.make_inputs(wl, seed)
    rng = np.random.default_rng(seed)
    extra = lambda a: np.concatenate([O.bits_to_f64(a), rng.standard_normal((1,) + a.shape[1:]) * 0.1])
    return wl, inp, extra(inp.w_gate), extra(inp.w_up), extra(inp.w_down)


def test_shared_expert_with_zero_down_weights_changes_nothing():
    wl, inp, wg, wu, wd = _shared_case()
    wd[-1] = 0.0
    a = O.layer_fwd(inp.x, inp.w_r, inp.bias, wg[:-1], wu[:-1], wd[:-1], wl.K)
    b = O.layer_fwd(inp.x, inp.w_r, inp.bias, wg, wu, wd, wl.K, n_shared=1)
    assert np.array_equal(a["out"], b["out"])
    assert int(b["counts"][-1]) == wl.N and int(b["offsets"][-1] - b["offsets"][-2]) == wl.N


def test_shared_expert_adds_a_dense_swiglu_mlp():
    """Exact mode: the layer with a shared expert minus the layer without it is
    the dense SwiGLU MLP of the shared weights on every token (torch)."""
    wl, inp, wg, wu, wd = _shared_case(13)
    a = O.layer_fwd(inp.x, inp.w_r, inp.bias, wg[:-1], wu[:-1], wd[:-1], wl.K, exact=True)
    b = O.layer_fwd(inp.x, inp.w_r, inp.bias, wg, wu, wd, wl.K, exact=True, n_shared=1)
    x = torch.tensor(O.bits_to_f64(inp.x))
    mlp = (F.silu(x @ torch.tensor(wg[-1]).T) * (x @ torch.tensor(wu[-1]).T)) @ torch.tensor(wd[-1]).T
    assert np.allclose(b["out"] - a["out"], mlp.numpy(), rtol=1e-10, atol=1e-12)


def test_backward_with_shared_expert_matches_finite_differences():
    wl, inp, wg, wu, wd = _shared_case(14)
    x = O.bits_to_f64(inp.x)
    L = O.router_logits(inp.x, inp.w_r, inp.bias)     # routing fixed
    dout = O.bits_to_f64(inp.dout)

    def fwd(x, wg, wu, wd):
        return O.layer_fwd(x, inp.w_r, None, wg, wu, wd, wl.K, logits=L, exact=True, n_shared=1)

    def loss(*a):
        return float(np.sum(fwd(*a)["out"] * dout))

    base = (x, wg, wu, wd)
    g = O.layer_bwd(fwd(*base), dout, wg, wu, wd, exact=True)
    rng = np.random.default_rng(3)
    eps = 1e-6
    for i, gr in enumerate((g["dx"], g["dw_gate"], g["dw_up"], g["dw_down"])):
        v = rng.standard_normal(base[i].shape)
        plus, minus = list(base), list(base)
        plus[i] = base[i] + eps * v
        minus[i] = base[i] - eps * v
        fd = (loss(*plus) - loss(*minus)) / (2 * eps)
        an = float(np.sum(gr * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (i, fd, an)

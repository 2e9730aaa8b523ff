"""Pins for the oracle's route: logits, softmax, top-K and the route map.

The route map is the one the OLMo-core Appendix A describes in A.2/A.3
(dst_rows[N,K], route id = token_row*top_k + k, negative = invalid) built by
the stable counting sort of the KOSMOS forward pass ("Plan", section 3.3.1
step 2).  The oracle builds it with a library stable sort; here it is checked
against a plain per-route loop with per-expert cursors and against invariants.
"""
import numpy as np
import pytest
import torch

import moe_synth as S
import oracle as O


def _brute_route_map(idx, drop, E, align, rows_cap):
    N, K = idx.shape
    counts = [0] * E
    for t in range(N):
        for k in range(K):
            e = int(idx[t, k])
            if 0 <= e < E and (drop is None or drop[t, k] == 0):
                counts[e] += 1
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + -(-counts[e] // align) * align)
    cursor = list(offsets[:E])
    dst = np.full((N, K), -1, np.int64)
    rr = np.full(rows_cap, -1, np.int64)
    for t in range(N):
        for k in range(K):
            e = int(idx[t, k])
            if 0 <= e < E and (drop is None or drop[t, k] == 0):
                dst[t, k] = cursor[e]
                rr[cursor[e]] = t * K + k
                cursor[e] += 1
    return np.array(counts), np.array(offsets), dst, rr


@pytest.mark.parametrize("N,E,K,align,pdrop", [(37, 8, 2, 1, 0.0), (64, 16, 4, 32, 0.1),
                                               (50, 5, 5, 1, 0.3), (1, 4, 1, 1, 0.0),
                                               (30, 12, 3, 8, 0.0)])
def test_route_map_vs_brute_force(N, E, K, align, pdrop):
    rng = np.random.default_rng(N * 7 + E)
    L = rng.integers(-3, 4, size=(N, E)).astype(np.float32)     # many exact ties
    idx = O.topk_select(L, K)
    drop = (rng.random((N, K)) < pdrop).astype(np.uint8) if pdrop else None
    cap = N * K + E * (align - 1)
    c, o, d, r = O.route_map(idx, drop, E, align, cap)
    bc, bo, bd, br = _brute_route_map(idx, drop, E, align, cap)
    assert np.array_equal(c, bc) and np.array_equal(o, bo)
    assert np.array_equal(d, bd) and np.array_equal(r, br)


def test_topk_vs_stable_argsort_and_sorted():
    rng = np.random.default_rng(7)
    for E, K in ((8, 2), (256, 8), (128, 8), (5, 5), (1024, 3)):
        L = rng.integers(-4, 5, size=(200, E)).astype(np.float32)   # heavy ties
        want = np.argsort(-L, axis=1, kind="stable")[:, :K]
        got = O.topk_select(L, K)
        assert np.array_equal(got, want)
        for t in range(5):
            order = sorted(range(E), key=lambda e: (-float(L[t, e]), e))[:K]
            assert list(got[t]) == order


def test_all_ties_closed_form():
    """W_r = 0 and no bias: every logit is 0, so the top-K are experts 0..K-1,
    every probability is 1/E, and 1/K after renormalisation."""
    wl = S.scaled(S.WORKLOADS["tiny_bf16"], N=32, D=64, E=8, K=3, H=32)
    inp = S.make_inputs(wl, 0, weights=False)
    L = O.router_logits(inp.x, np.zeros_like(inp.w_r), None)
    assert np.all(L == 0)
    idx = O.topk_select(L, 3)
    assert np.array_equal(idx, np.tile(np.arange(3), (32, 1)))
    assert np.all(O.route_probs(L, idx, 0) == np.float32(1 / 8))
    assert np.allclose(O.route_probs(L, idx, 1), 1 / 3, rtol=0, atol=1e-7)


def test_logits_vs_brute_force_loop():
    wl = S.scaled(S.WORKLOADS["dsv3_bf16"], N=6, D=40, E=5, K=2, H=32)
    inp = S.make_inputs(wl, 3, weights=False)
    L = O.router_logits(inp.x, inp.w_r, inp.bias)
    x = S.bf16_bits_to_f32(inp.x).astype(np.float64)
    w = S.bf16_bits_to_f32(inp.w_r).astype(np.float64)
    for t in range(6):
        for e in range(5):
            acc = 0.0
            for d in range(40):
                acc += x[t, d] * w[e, d]
            assert L[t, e] == np.float32(np.float32(acc) + inp.bias[e])


def test_softmax_vs_torch():
    rng = np.random.default_rng(9)
    L = (rng.standard_normal((100, 64)) * 5).astype(np.float32)
    want = torch.softmax(torch.from_numpy(L).double(), dim=1).numpy()
    assert np.allclose(O.softmax(L), want, rtol=1e-13, atol=0)
    idx = O.topk_select(L, 4)
    p = O.route_probs(L, idx, 1)
    assert np.allclose(p.astype(np.float64).sum(1), 1.0, atol=1e-6)


@pytest.mark.parametrize("name,seed", [("tiny_bf16", 0), ("dsv3_bf16", 1), ("qwen3_235b_bf16_fwdbwd", 2),
                                       ("dsv3_mxfp8", 0)])
def test_route_map_invariants(name, seed):
    wl = S.WORKLOADS[name]
    if wl.N > 4096:
        wl = S.scaled(wl, N=4096)
    inp = S.make_inputs(wl, seed, weights=False)
    L = S.random_logits(wl.N, wl.E, seed) + (inp.bias if inp.bias is not None else 0)
    L = L.astype(np.float32)
    idx = O.topk_select(L, wl.K)
    c, o, d, r = O.route_map(idx, inp.drop, wl.E, wl.align, wl.rows_cap)
    N, K, E = wl.N, wl.K, wl.E
    # every token has K distinct experts
    assert all(len(set(row)) == K for row in idx.tolist())
    valid = O.route_valid(idx, inp.drop, E)
    assert c.sum() == N * K - (~valid).sum()
    assert np.all(d[~valid] == -1) and np.all(d[valid] >= 0)
    # offsets: start 0, non-decreasing, multiples of align, last within rows_cap
    assert o[0] == 0 and np.all(np.diff(o) >= 0) and np.all(o % wl.align == 0)
    assert o[-1] <= wl.rows_cap and np.all(np.diff(o) >= c)
    # dst_rows is a bijection from valid routes onto the non-padding rows
    rid = np.arange(N * K).reshape(N, K)
    assert np.array_equal(r[d[valid]], rid[valid])
    assert (r >= 0).sum() == valid.sum()
    for e in range(E):
        seg = r[o[e]:o[e] + c[e]]
        assert np.all(seg >= 0) and np.all(np.diff(seg) > 0)        # ascending route id
        assert np.all(idx.reshape(-1)[seg] == e)
        assert np.all(r[o[e] + c[e]:o[e + 1]] == -1)                # padding


# ------------------------------------------------------ router backward ----
def _router_case(N, D, E, K, seed, pdrop=0.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, D))
    w = rng.standard_normal((E, D)) * 0.3
    b = rng.standard_normal(E) * 0.1
    L = x @ w.T + b
    idx = O.topk_select(L, K)
    dprob = rng.standard_normal((N, K))
    dprob[rng.random((N, K)) < pdrop] = 0.0      # dropped routes carry no gradient
    return x, w, b, L, idx, dprob


@pytest.mark.parametrize("renorm", [0, 1])
@pytest.mark.parametrize("pdrop", [0.0, 0.3])
def test_router_bwd_matches_finite_differences(renorm, pdrop):
    """fp64 central differences of sum(dprob * route_weights(x W^T + b)), with
    the selection fixed (it is piecewise constant in the logits)."""
    N, D, E, K = 12, 16, 8, 3
    x, w, b, L, idx, dprob = _router_case(N, D, E, K, 5 + renorm, pdrop)

    def loss_L(Lm):
        return float(np.sum(dprob * O.route_weights(Lm, idx, renorm)))

    def loss(xm, wm, bm):
        return loss_L(xm @ wm.T + bm)

    g = O.router_bwd(L, idx, dprob, x, w, renorm)
    rng = np.random.default_rng(2)
    eps = 1e-6
    base = (x, w, b)
    for i, gr in enumerate((g["dx_r"], g["dw_r"], g["db_r"])):
        v = rng.standard_normal(base[i].shape)
        plus, minus = list(base), list(base)
        plus[i] = base[i] + eps * v
        minus[i] = base[i] - eps * v
        fd = (loss(*plus) - loss(*minus)) / (2 * eps)
        an = float(np.sum(gr * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (i, fd, an)
    v = rng.standard_normal(L.shape)
    fd = (loss_L(L + eps * v) - loss_L(L - eps * v)) / (2 * eps)
    assert abs(fd - float(np.sum(g["dlogits"] * v))) <= 1e-7 * max(1.0, abs(fd))


@pytest.mark.parametrize("renorm", [0, 1])
def test_router_bwd_dlogits_vs_torch_autograd(renorm):
    N, E, K = 20, 32, 6
    x, w, b, L, idx, dprob = _router_case(N, 8, E, K, 11)
    Lt = torch.tensor(L, dtype=torch.float64, requires_grad=True)
    p = torch.softmax(Lt, dim=1)
    sel = torch.gather(p, 1, torch.tensor(idx, dtype=torch.int64))
    if renorm:
        sel = sel / sel.sum(dim=1, keepdim=True)
    (sel * torch.tensor(dprob)).sum().backward()
    got = O.router_bwd(L, idx, dprob, x, w, renorm)["dlogits"]
    assert np.allclose(got, Lt.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_router_bwd_closed_forms():
    # one expert per token, renormalised: the weight is 1 whatever the logits
    x, w, b, L, idx, dprob = _router_case(10, 8, 6, 1, 3)
    g = O.router_bwd(L, idx, dprob, x, w, renorm=1)
    assert np.all(g["dlogits"] == 0.0)
    # every expert selected with the same upstream gradient: the weights sum to 1
    x, w, b, L, idx, _ = _router_case(10, 8, 6, 6, 4)
    g = O.router_bwd(L, idx, np.full((10, 6), 0.7), x, w, renorm=0)
    assert np.max(np.abs(g["dlogits"])) <= 1e-15
    # no upstream gradient, no router gradient
    g = O.router_bwd(L, idx, np.zeros((10, 6)), x, w, renorm=1)
    assert not np.any(g["dlogits"]) and not np.any(g["dw_r"]) and not np.any(g["db_r"])


# -------------------------------------------- group-limited top-K, aux loss ----
def test_grouped_topk_worked_example():
    """Eight experts in four pairs, keep two groups, top-2.  Probabilities are
    proportional to exp(logit): group sums e^5 = 148.4 (pair 0), e^4.9 + e^4.8 =
    255.8 (pair 1), e^4.95 = 141.2 (pair 2), ~0 (pair 3).  Pairs 1 and 0 are
    kept, so expert 4 (logit 4.95, second best overall) is excluded and the
    selection is experts 0 and 2 instead of the plain 0 and 4."""
    L = np.array([[5.0, -9.0, 4.9, 4.8, 4.95, -9.0, -9.0, -9.0]])
    assert O.topk_select(L, 2).tolist() == [[0, 4]]
    assert O.topk_select_grouped(L, 2, n_group=4, topk_group=2).tolist() == [[0, 2]]
    g = O.group_scores(L, 4)
    assert np.argsort(-g[0]).tolist()[:2] == [1, 0]


def test_grouped_topk_reduces_to_plain():
    rng = np.random.default_rng(7)
    L = rng.standard_normal((50, 32))
    assert np.array_equal(O.topk_select_grouped(L, 4, 1, 1), O.topk_select(L, 4))
    assert np.array_equal(O.topk_select_grouped(L, 4, 8, 8), O.topk_select(L, 4))


def test_grouped_topk_keeps_whole_groups_and_ties():
    rng = np.random.default_rng(8)
    L = rng.standard_normal((40, 24))
    # K = topk_group * group size: exactly the kept groups' experts, best first
    sel = O.topk_select_grouped(L, 12, n_group=6, topk_group=3)
    gsc = O.group_scores(L, 6)
    for t in range(40):
        groups = set((sel[t] // 4).tolist())
        assert len(groups) == 3 and all(len([e for e in sel[t] if e // 4 == g]) == 4 for g in groups)
        assert min(gsc[t, list(groups)]) >= max(np.delete(gsc[t], list(groups)))
        assert np.all(np.diff(L[t, sel[t]]) <= 0)
    # two groups with equal scores: the lower group is kept
    L = np.zeros((1, 8))
    L[0, [2, 3, 6, 7]] = 1.0
    assert O.topk_select_grouped(L, 2, n_group=4, topk_group=1).tolist() == [[2, 3]]


def test_aux_loss_closed_form_and_gradient():
    # uniform probabilities and loads: f = P = 1/E, so aux = alpha exactly
    N, E, K = 64, 16, 4
    aux, P = O.aux_loss(np.zeros((N, E)), np.full(E, N * K // E), K, 0.01)
    assert abs(aux - 0.01) <= 1e-15 and np.allclose(P, 1 / E)
    rng = np.random.default_rng(9)
    L = rng.standard_normal((N, E))
    counts = rng.integers(0, 3 * N * K // E, E)
    alpha, d_aux = 0.003, 1.7
    g = O.aux_dlogits(L, counts, K, alpha, d_aux)
    v = rng.standard_normal(L.shape)
    eps = 1e-6
    fd = d_aux * (O.aux_loss(L + eps * v, counts, K, alpha)[0] - O.aux_loss(L - eps * v, counts, K, alpha)[0]) / (2 * eps)
    assert abs(fd - float(np.sum(g * v))) <= 1e-8 * max(1.0, abs(fd))
    Lt = torch.tensor(L, requires_grad=True)
    f = torch.tensor(counts, dtype=torch.float64) / (N * K)
    (d_aux * alpha * E * (f * torch.softmax(Lt, dim=1).mean(dim=0)).sum()).backward()
    assert np.allclose(g, Lt.grad.numpy(), rtol=1e-12, atol=1e-16)

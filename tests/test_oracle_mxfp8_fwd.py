"""Pins for the oracle's MXFP8 forward composition.

The MXFP8 forward (KOSMOS section 3.3.1 step 3: quantize on dispatch, pad each
group to 32 rows, block-scaled GEMM1, bf16 SwiGLU, H quantized row-wise for
GEMM2; OLMo-core Appendix A, A.5 eq. 87: the block-scaled product with an fp32
accumulator) differs from the bf16 forward only where a tensor is quantized.
So when every quantized tensor is exactly representable at its block scale the
two must agree bit for bit, and on random inputs each stored tensor must be the
documented function of the previous one, checked here through torch's own
float8 decoder and silu.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import moe_synth as S
import oracle as O


def _lossless_inputs(seed, E=4, N=48, K=2, D=64, H=64, n_shared=0):
    """x rows in {0, 2^j_t} (j_t per token, so block scales differ between
    tokens); W_gate one-hot per output column with 64, so G = 64 x[t, d_h] in
    {0, 64 * 2^j} and silu(G) = G exactly in float64 (exp(-64) vanishes next
    to 1); W_up with two +-1 per output column, so U = 2^j {-2..2}; then
    H = G U has a power-of-two block maximum and is exact in E4M3 at its
    block scale.  W_down entries are in {0, +-1/2, +-1}.  The router weight is
    a plain bf16 normal matrix, so routing is the usual one."""
    rng = np.random.default_rng(seed)
    Et = E + n_shared
    j = rng.integers(0, 4, size=N)
    x = (rng.random((N, D)) < 0.5) * np.ldexp(1.0, j)[:, None]
    x[np.arange(N), rng.integers(0, D, size=N)] = np.ldexp(1.0, j)     # no all-zero row
    wg = np.zeros((Et, H, D))
    wu = np.zeros((Et, H, D))
    for e in range(Et):
        wg[e, np.arange(H), rng.integers(0, D, size=H)] = 64.0
        for _ in range(2):
            wu[e, np.arange(H), rng.integers(0, D, size=H)] += rng.choice([-1.0, 1.0], size=H)
    wd = rng.choice([0.0, 0.5, -0.5, 1.0, -1.0], size=(Et, D, H))
    w_r = O.round_bf16(rng.standard_normal((E, D)) / 8.0)
    return x, w_r, wg, wu, wd


@pytest.mark.parametrize("n_shared", [0, 1])
def test_lossless_inputs_give_the_bf16_forward_bit_for_bit(n_shared):
    """With every quantized operand exact, layer_fwd_mxfp8 equals layer_fwd with
    32-row groups in the route map, G, U, H, Y and the output, and its X_d and
    H codes decode to the bf16 path's X_d and H.  The case keeps G, U, H, Y and
    the output mostly nonzero and the token scales varied, so a wrong scale
    row, a swapped gate/up, a transposed weight or a wrong dispatch row fails."""
    K = 2
    x, w_r, wg, wu, wd = _lossless_inputs(11 + n_shared, K=K, n_shared=n_shared)
    wq = O.quantize_weights_mxfp8(wg, wu, wd)
    for name, w in (("wg", wg), ("wu", wu), ("wd", wd)):
        for e in range(w.shape[0]):
            assert np.array_equal(O.dequantize_mxfp8(wq[name + "_q"][e], wq[name + "_s"][e]), w[e]), name
    mx = O.layer_fwd_mxfp8(x, w_r, None, wq, K, n_shared=n_shared)
    ref = O.layer_fwd(x, w_r, None, wg, wu, wd, K, align=32, n_shared=n_shared)
    for k in ("topk_idx", "counts", "offsets", "dst_rows", "row_route", "g", "u", "h", "y", "out"):
        assert np.array_equal(mx[k], ref[k]), (n_shared, k)
    assert np.array_equal(O.dequantize_mxfp8(mx["xq"], mx["xs"]), ref["xd"])
    assert np.array_equal(O.dequantize_mxfp8(mx["hq"], mx["hs"]), ref["h"])
    live = ref["row_route"] >= 0
    for k in ("g", "u", "h", "y"):
        assert np.count_nonzero(ref[k][live]) > ref[k][live].size // 8, (n_shared, k)
    assert np.count_nonzero(ref["out"]) > ref["out"].size // 2
    assert len(np.unique(mx["xs"][live])) >= 3            # several block scales in play
    assert len(np.unique(mx["hs"][live])) >= 3


def _tdeq(q, s):
    """Dequantize through torch's float8_e4m3fn decoder (independent of the
    oracle's e4m3_decode)."""
    v = torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64)
    sc = torch.pow(2.0, torch.from_numpy(np.asarray(s, np.int64) - 127).to(torch.float64))
    return (v.reshape(q.shape[0], -1, 32) * sc[..., None]).reshape(q.shape)


def test_random_forward_each_stored_tensor_follows_from_the_previous():
    """Workload-shaped random inputs: X_d codes are the token rows' codes;
    G and U are the eq. 87 products of the decoded operands rounded once to
    bf16; H is bf16(silu(G) U) from those bf16 values (a torch silu); the H
    codes are H's own row-wise quantization; Y is the eq. 87 product of the
    decoded H and W_down codes; the output is the fp32-weighted fold of Y."""
    wl = S.scaled(S.WORKLOADS["dsv3_mxfp8"], "mx_fwd_pin", N=64, D=128, E=8, K=3, H=96)
    inp = S.make_inputs(wl, 3)
    wq = O.quantize_weights_mxfp8(inp.w_gate, inp.w_up, inp.w_down)
    f = O.layer_fwd_mxfp8(inp.x, inp.w_r, inp.bias, wq, wl.K)
    tq, ts = O.quantize_mxfp8(inp.x)
    rr = f["row_route"]
    live = rr >= 0
    assert np.array_equal(f["xq"][live], tq[rr[live] // wl.K])
    assert np.array_equal(f["xs"][live], ts[rr[live] // wl.K])
    assert not f["xq"][~live].any() and not f["xs"][~live].any()
    o = f["offsets"]
    for e in range(wl.E):
        a, b = int(o[e]), int(o[e + 1])
        if b == a:
            continue
        xe = _tdeq(f["xq"][a:b], f["xs"][a:b])
        G = O.round_bf16((xe @ _tdeq(wq["wg_q"][e], wq["wg_s"][e]).T).numpy())
        U = O.round_bf16((xe @ _tdeq(wq["wu_q"][e], wq["wu_s"][e]).T).numpy())
        assert np.array_equal(f["g"][a:b], G) and np.array_equal(f["u"][a:b], U), e
        h = O.round_bf16((F.silu(torch.from_numpy(G)) * torch.from_numpy(U)).numpy())
        assert np.array_equal(f["h"][a:b], h), e
        hq, hs = O.quantize_mxfp8(h)
        assert np.array_equal(f["hq"][a:b], hq) and np.array_equal(f["hs"][a:b], hs), e
        Y = O.round_bf16((_tdeq(hq, hs) @ _tdeq(wq["wd_q"][e], wq["wd_s"][e]).T).numpy())
        assert np.array_equal(f["y"][a:b], Y), e
    # the fold: each token's valid rows, fp32 weights, one rounding
    want = np.zeros((wl.N, wl.D))
    for t in range(wl.N):
        for k in range(wl.K):
            r = f["dst_rows"][t, k]
            if r >= 0:
                want[t] += float(f["topk_prob"][t, k]) * f["y"][r]
    assert np.array_equal(f["out"], O.round_bf16(want))
    # quantizing H before its bf16 rounding is a different tensor here
    Gall, Uall = f["g"][live], f["u"][live]
    hq_unrounded, _ = O.quantize_mxfp8(O.silu(Gall) * Uall)
    assert not np.array_equal(hq_unrounded, f["hq"][live])


def _torch_weighted_rows(x, w):
    """fp32 multiply of each row by its weight, then the fp32 -> bf16 cast."""
    xt = torch.from_numpy(np.asarray(x, np.float64).astype(np.float32))
    wt = torch.from_numpy(np.asarray(w, np.float32))
    return (wt[:, None] * xt).to(torch.bfloat16).to(torch.float64).numpy()


def test_weighted_dispatch_rounds_through_fp32_like_torch():
    """The weighted PUT (KOSMOS section 3.3.2 step 1: dY dispatched with its
    router weight, stored bf16) forms the product in fp32 and stores it as
    bf16.  torch does exactly that with a float32 multiply and a bfloat16
    cast.  The inputs include products that land on bf16 midpoints after the
    fp32 rounding but not before it, where one rounding straight to bf16
    would give the other neighbour."""
    rng = np.random.default_rng(17)
    N, K, D = 64, 4, 96
    x = O.round_bf16(rng.standard_normal((N, D)) * 10.0 ** rng.integers(-3, 3, (N, 1)))
    w = rng.random((N, K)).astype(np.float32)
    # planted cases: for a few bf16 x, fp32 weights w next to m / x for a
    # bf16 midpoint m, kept where the fp32 product is exactly m but the exact
    # product is not.  m then rounds to the even neighbour, while one rounding
    # of the exact product goes to the odd one half of the time.
    planted = []
    for xb in (1.0 + 2.0 ** -7, 1.5 - 2.0 ** -7, 3.0 + 2.0 ** -6, 0.75 + 2.0 ** -9):
        for j in range(1, 60):
            m = (1.0 + (2 * j + 1) * 2.0 ** -8) * (2.0 if xb > 2 else 1.0)
            wc = np.float32(m / xb)
            for _ in range(24):
                p = float(wc) * xb
                if float(np.float32(p)) == m and p != m and O.round_bf16(np.array([p]))[0] != \
                        O.round_bf16(np.array([m]))[0]:
                    planted.append((xb, wc))
                wc = np.nextafter(wc, np.float32(np.inf))
            if len(planted) >= 2 * K:
                break
    assert len(planted) >= K
    for k in range(K):
        x[k, :] = planted[k][0]
        w[k, :] = planted[k][1]
    idx = np.stack([rng.permutation(8)[:K] for _ in range(N)]).astype(np.int32)
    rows_cap = N * K
    _, _, dst_rows, row_route = O.route_map(idx, None, 8, 1, rows_cap)
    got = O.dispatch(x, row_route, K, weight=w)
    live = row_route >= 0
    tok = row_route[live] // K
    wr = w.reshape(-1)[row_route[live]]
    want = _torch_weighted_rows(x[tok], wr)
    assert np.array_equal(got[live], want)
    assert not got[~live].any()
    # the planted elements really separate fp32-then-bf16 from one rounding
    exact = wr[:, None].astype(np.float64) * x[tok]
    single = O.round_bf16(exact)
    differs = single != want
    assert differs.sum() >= K * D
    # the combine backward is the same weighted PUT (adjoint of the fold)
    dyd = O.combine_bwd(x, dst_rows, w, rows_cap)
    assert np.array_equal(dyd, got)

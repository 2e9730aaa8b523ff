"""Pins for the oracle's MXFP8 backward.

The MXFP8 backward quantizes dY and [dG | dU] row-wise along their contraction
dimension, uses weight copies quantized along the other dimension for the data
gradients (KOSMOS section 2.2; OLMo-core Appendix A, A.13: the right-hand
operand prequantized for dgrad) and computes the weight gradients in bf16 from
dequantized activations (A.13's wgrad policy).  When every quantized tensor is
exactly representable, quantization changes nothing and the result must equal
the bf16 backward, which is pinned by finite differences elsewhere; on random
inputs it must stay within the MXFP8 rounding error of the bf16 backward.
"""
import numpy as np

import moe_synth as S
import oracle as O


def _signs(rng, shape, p_zero=0.3):
    v = rng.choice([-1.0, 1.0], size=shape)
    return np.where(rng.random(shape) < p_zero, 0.0, v)


def _lossless_case(seed, E=3, N=40, K=2, D=64, H=64, n_shared=0):
    """Saved tensors and weights whose every quantized copy is exact: ±1 / 0
    data (dyadic multiples after the power-of-two route weights), G in {0, 64}
    so that sigmoid(G) is 1/2 or exactly 1 in float64, and a down projection
    with one ±1 per column so that dH stays in {0, ±w}."""
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(N)]).astype(np.int32)
    align = 32
    rows_cap = N * K + E * (align - 1) + n_shared * (N + align - 1)
    counts, offsets, dst_rows, row_route = O.route_map(idx, None, E, align, rows_cap, n_shared)
    x = rng.choice([-1.0, 1.0], size=(N, D))
    xd = O.dispatch(x, row_route, K)
    Et = E + n_shared
    if n_shared:
        xd[offsets[E]:offsets[E] + N] = x
    prob = np.tile(np.array([0.5, 0.25, 0.125, 0.125][:K], np.float32), (N, 1))
    G = np.where(rng.random((rows_cap, H)) < 0.5, 0.0, 64.0)
    U = rng.choice([-1.0, 1.0], size=(rows_cap, H))
    Hh = _signs(rng, (rows_cap, H)) * rng.choice([0.5, 1.0], size=(rows_cap, H))
    wg = _signs(rng, (Et, H, D))
    wu = _signs(rng, (Et, H, D))
    wd = np.zeros((Et, D, H))
    for e in range(Et):
        wd[e, rng.integers(0, D, size=H), np.arange(H)] = rng.choice([-1.0, 1.0], size=H)
    xq, xs = O.quantize_mxfp8(xd)
    hq, hs = O.quantize_mxfp8(Hh)
    fwd = dict(topk_idx=idx, topk_prob=prob, counts=counts, offsets=offsets, dst_rows=dst_rows,
               row_route=row_route, xd=xd, xq=xq, xs=xs, g=G, u=U, h=Hh, hq=hq, hs=hs,
               y=rng.standard_normal((rows_cap, D)), n_shared=n_shared)
    dout = _signs(rng, (N, D))
    return fwd, dout, wg, wu, wd


def test_dgrad_weight_copies_are_transposes_quantized_along_the_other_dim():
    rng = np.random.default_rng(0)
    wg, wu = _signs(rng, (2, 64, 96)), _signs(rng, (2, 64, 96))
    wd = _signs(rng, (2, 96, 64)) * 0.5
    q = O.quantize_weights_mxfp8_dgrad(wg, wu, wd)
    assert q["wdt_q"].shape == (2, 64, 96) and q["wdt_s"].shape == (2, 64, 3)
    assert q["wgut_q"].shape == (2, 96, 128) and q["wgut_s"].shape == (2, 96, 4)
    for e in range(2):
        assert np.array_equal(O.dequantize_mxfp8(q["wdt_q"][e], q["wdt_s"][e]), wd[e].T)
        gu = O.dequantize_mxfp8(q["wgut_q"][e], q["wgut_s"][e])
        assert np.array_equal(gu[:, :64], wg[e].T) and np.array_equal(gu[:, 64:], wu[e].T)
    # general weights: each transposed element within E4M3's relative error
    # (half spacing 2^-4 in the normal range, 2^-3 where the block top saturates
    # at 448), normal range = above 2^-14 of its block's largest magnitude
    w = rng.standard_normal((1, 64, 96))
    q = O.quantize_weights_mxfp8_dgrad(w, w, np.swapaxes(w, 1, 2).copy())
    deq = O.dequantize_mxfp8(q["wdt_q"][0], q["wdt_s"][0])          # [64, 96] = w_down^T = w
    rel = np.abs(deq - w[0]) / np.abs(w[0])
    amax = np.repeat(np.abs(w[0]).reshape(64, 3, 32).max(axis=2), 32, axis=1)
    normal = np.abs(w[0]) >= amax * 2.0 ** -14
    assert np.all(rel[normal] <= 2.0 ** -3 + 1e-12)
    assert np.median(rel[normal]) <= 2.0 ** -5
    # the other orientation would be far off
    assert np.linalg.norm(deq[:, :64] - w[0][:, :64].T) > 0.5 * np.linalg.norm(w[0][:, :64])


def test_lossless_case_equals_the_bf16_backward_exactly():
    """Every quantized copy exact -> MXFP8 backward == bf16 backward, bit for bit.
    The case is built so that dU, dX_d and every weight gradient are nonzero
    (a swapped half, a transposed copy or a wrong scale changes the result)."""
    for n_shared in (0, 1):
        fwd, dout, wg, wu, wd = _lossless_case(5 + n_shared, n_shared=n_shared)
        wqt = O.quantize_weights_mxfp8_dgrad(wg, wu, wd)
        mx = O.layer_bwd_mxfp8(fwd, dout, wqt)
        ref = O.layer_bwd(fwd, dout, wg, wu, wd)
        for k in ("dyd", "dg", "du", "dxd", "dw_gate", "dw_up", "dw_down", "dx", "dprob"):
            assert np.array_equal(mx[k], ref[k]), (n_shared, k)
        for k in ("du", "dxd", "dw_gate", "dw_up", "dw_down", "dx"):
            assert np.count_nonzero(ref[k]) > ref[k].size // 20, (n_shared, k)
        # the quantized dY and [dG | dU] copies decode to the bf16 tensors
        assert np.array_equal(O.dequantize_mxfp8(mx["dyq"], mx["dys"]), mx["dyd"])
        assert np.array_equal(O.dequantize_mxfp8(mx["guq"], mx["gus"]), np.concatenate([mx["dg"], mx["du"]], 1))


def test_random_inputs_stay_within_mxfp8_error_of_the_bf16_backward():
    """Workload-shaped random inputs: every gradient of the MXFP8 layer is
    within a few E4M3 relative spacings (2^-4) of the bf16 layer's."""
    wl = S.scaled(S.WORKLOADS["dsv3_mxfp8"], "mx_bwd_pin", N=96, D=128, E=8, K=4, H=64, bwd=True)
    inp = S.make_inputs(wl, 21)
    q = O.quantize_weights_mxfp8(inp.w_gate, inp.w_up, inp.w_down)
    wqt = O.quantize_weights_mxfp8_dgrad(inp.w_gate, inp.w_up, inp.w_down)
    f = O.layer_fwd_mxfp8(inp.x, inp.w_r, inp.bias, q, wl.K)
    mx = O.layer_bwd_mxfp8(f, inp.dout, wqt)
    fb = O.layer_fwd(inp.x, inp.w_r, inp.bias, inp.w_gate, inp.w_up, inp.w_down, wl.K, align=32)
    assert np.array_equal(fb["dst_rows"], f["dst_rows"])
    ref = O.layer_bwd(fb, inp.dout, inp.w_gate, inp.w_up, inp.w_down)
    for k in ("dx", "dw_gate", "dw_up", "dw_down", "dprob"):
        err = np.linalg.norm(mx[k] - ref[k]) / np.linalg.norm(ref[k])
        assert err <= 0.15, (k, err)


def test_recompute_mode_takes_h_from_the_saved_g_and_u():
    """SwiGLU-recompute (OLMo-core Appendix A, A.14): the down weight gradient
    uses H = bf16(silu(G) U) rebuilt from the saved bf16 G and U (a torch silu
    here) instead of the dequantized H codes; every other gradient is the
    same as with the saved codes.  On the lossless case both modes agree."""
    import torch
    import torch.nn.functional as F
    wl = S.scaled(S.WORKLOADS["dsv3_mxfp8"], "mx_bwd_rc", N=64, D=128, E=8, K=3, H=64, bwd=True)
    inp = S.make_inputs(wl, 23)
    q = O.quantize_weights_mxfp8(inp.w_gate, inp.w_up, inp.w_down)
    wqt = O.quantize_weights_mxfp8_dgrad(inp.w_gate, inp.w_up, inp.w_down)
    f = O.layer_fwd_mxfp8(inp.x, inp.w_r, inp.bias, q, wl.K)
    saved = O.layer_bwd_mxfp8(f, inp.dout, wqt)
    rc = O.layer_bwd_mxfp8(f, inp.dout, wqt, recompute=True)
    for k in ("dyd", "dg", "du", "dxd", "dw_gate", "dw_up", "dx", "dprob"):
        assert np.array_equal(rc[k], saved[k]), k
    o = f["offsets"]
    h = O.round_bf16((F.silu(torch.from_numpy(f["g"])) * torch.from_numpy(f["u"])).numpy())
    for e in range(wl.E):
        a, b = int(o[e]), int(o[e + 1])
        want = O.round_bf16(rc["dyd"][a:b].T @ h[a:b]) if b > a else np.zeros((wl.D, wl.H))
        assert np.array_equal(rc["dw_down"][e], want), e
    assert not np.array_equal(rc["dw_down"], saved["dw_down"])   # H codes are lossy here
    fwd, dout, wg, wu, wd = _lossless_case(9)
    wqt = O.quantize_weights_mxfp8_dgrad(wg, wu, wd)
    fwd["g"] = np.where(fwd["g"] > 0, 64.0, 0.0)
    fwd["h"] = O.swiglu(fwd["g"], fwd["u"])
    fwd["hq"], fwd["hs"] = O.quantize_mxfp8(fwd["h"])
    a = O.layer_bwd_mxfp8(fwd, dout, wqt)
    b = O.layer_bwd_mxfp8(fwd, dout, wqt, recompute=True)
    assert np.array_equal(a["dw_down"], b["dw_down"])


def test_native_mx_wgrad_lossless_case_equals_the_bf16_backward():
    """Native MXFP8 weight gradients (OLMo-core Appendix A, A.15; column-wise
    copies of dY, X and H quantized from their bf16 values, KOSMOS 3.3.2 step
    1): with every column-wise copy exact they equal the bf16 backward's bit
    for bit, with the shared expert too."""
    for n_shared in (0, 1):
        fwd, dout, wg, wu, wd = _lossless_case(13 + n_shared, n_shared=n_shared)
        fwd["h"] = O.swiglu(fwd["g"], fwd["u"])          # the bf16 H the native path takes
        fwd["hq"], fwd["hs"] = O.quantize_mxfp8(fwd["h"])
        wqt = O.quantize_weights_mxfp8_dgrad(wg, wu, wd)
        mx = O.layer_bwd_mxfp8(fwd, dout, wqt, wgrad="mx")
        ref = O.layer_bwd(fwd, dout, wg, wu, wd)
        for k in ("dw_gate", "dw_up", "dw_down", "dx", "dprob"):
            assert np.array_equal(mx[k], ref[k]), (n_shared, k)
            assert np.count_nonzero(ref[k]) > ref[k].size // 20, (n_shared, k)
        # the native path takes H and X from their bf16 values, never from the
        # saved row-wise codes: erasing the codes changes no weight gradient
        fwd["hq"] = np.zeros_like(fwd["hq"])
        fwd["xq"] = np.zeros_like(fwd["xq"])
        mx2 = O.layer_bwd_mxfp8(fwd, dout, wqt, wgrad="mx")
        for k in ("dw_gate", "dw_up", "dw_down"):
            assert np.array_equal(mx2[k], mx[k]), (n_shared, k)


def test_native_mx_wgrad_quantizes_along_rows():
    """The column-wise copy quantizes blocks of 32 rows of one column: with a
    gradient whose columns have very different magnitudes (2^-20 against
    2^0) but uniform magnitude down each column, every column block is exact,
    so the native wgrad equals the exact product, while row-wise blocks
    (which mix the magnitudes) would flush the small columns to zero."""
    rng = np.random.default_rng(3)
    rows, n, k = 64, 64, 32
    offsets = np.array([0, 32, 64])
    col_exp = np.where(np.arange(n) % 2 == 0, -20.0, 0.0)
    dc = rng.choice([-1.0, 1.0], size=(rows, n)) * np.ldexp(1.0, col_exp.astype(int))[None, :]
    a = rng.choice([-1.0, 0.0, 1.0], size=(rows, k))
    got = O.mx_wgrad(dc, a, offsets)
    for e in range(2):
        sl = slice(offsets[e], offsets[e + 1])
        assert np.array_equal(got[e], O.round_bf16(dc[sl].T @ a[sl]))
        assert np.count_nonzero(got[e][0::2]) > 0             # the 2^-20 columns survive
    # the row-wise reading of the same operand loses them
    rq, rs = O.quantize_mxfp8(dc)
    assert not np.any(O.dequantize_mxfp8(rq, rs)[:, 0::2])
    # shapes of the copies: [W, segment rows] codes, [W, rows/32] scales
    cq = O.quantize_mxfp8_cols(dc, offsets)
    assert cq[0][0].shape == (n, 32) and cq[0][1].shape == (n, 1)


def test_native_mx_wgrad_random_inputs_within_mxfp8_error():
    """Workload-shaped random inputs: the native MXFP8 weight gradients stay
    within a few E4M3 spacings of the bf16 backward's; the other gradients do
    not depend on the wgrad mode."""
    wl = S.scaled(S.WORKLOADS["dsv3_mxfp8"], "mx_wg", N=96, D=128, E=8, K=4, H=64, bwd=True)
    inp = S.make_inputs(wl, 25)
    q = O.quantize_weights_mxfp8(inp.w_gate, inp.w_up, inp.w_down)
    wqt = O.quantize_weights_mxfp8_dgrad(inp.w_gate, inp.w_up, inp.w_down)
    f = O.layer_fwd_mxfp8(inp.x, inp.w_r, inp.bias, q, wl.K)
    assert np.array_equal(f["xd"], O.dispatch(inp.x, f["row_route"], wl.K))
    mx = O.layer_bwd_mxfp8(f, inp.dout, wqt, wgrad="mx")
    base = O.layer_bwd_mxfp8(f, inp.dout, wqt)
    for k in ("dx", "dprob", "dg", "du"):
        assert np.array_equal(mx[k], base[k]), k
    fb = O.layer_fwd(inp.x, inp.w_r, inp.bias, inp.w_gate, inp.w_up, inp.w_down, wl.K, align=32)
    ref = O.layer_bwd(fb, inp.dout, inp.w_gate, inp.w_up, inp.w_down)
    for k in ("dw_gate", "dw_up", "dw_down"):
        err = np.linalg.norm(mx[k] - ref[k]) / np.linalg.norm(ref[k])
        assert err <= 0.15, (k, err)

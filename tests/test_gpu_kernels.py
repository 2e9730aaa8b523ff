"""Kernel-level parity: each C-ABI entry point against the oracle step it
implements, at sizes the oracle finishes in seconds that still span several
tiles and ragged tails, plus the degenerate cases of the method.

Integer and byte results (route maps, permutations, MXFP8 bytes) must be
bit-exact; bf16 results satisfy max|diff| <= 1e-2*max|ref| + 1e-3; route
probabilities |diff| <= 1e-6.
"""
import numpy as np
import pytest
import torch

import mixture_experts_expert_router_amd as M
import moe_synth as S
import oracle as O
from gpu_util import (assert_bf16_close, bits, dev, dev_bf16, host, poison_bf16, rel_frobenius,
                      vals)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.load()
    yield
    torch.cuda.synchronize()


def _sync():
    torch.cuda.synchronize()


# ---------------------------------------------------------------- router ----
@pytest.mark.parametrize("N,D,E", [(256, 128, 8), (100, 136, 24), (33, 7168, 256), (70, 4096, 128),
                                   (5, 64, 1), (130, 256, 1024), (17, 512, 40), (4096, 7168, 256),
                                   (2000, 4096, 128), (8192, 4096, 8), (300, 192, 16),
                                   (2100, 1024, 200), (3000, 640, 1000), (16384, 4096, 128), (2048, 64, 64),
                                   # E % 4 != 0 on the tiled path: scalar tile stores and split reduce
                                   (500, 256, 18), (3000, 1024, 250)])
def test_router_logits(N, D, E):
    print(f"router N={N} D={D} E={E}", flush=True)
    wl = S.scaled(S.WORKLOADS["dsv3_bf16"], N=N, D=D, E=E, K=1, H=32)
    inp = S.make_inputs(wl, N + E, weights=False)
    got = host(M.router_logits(dev_bf16(inp.x), dev_bf16(inp.w_r), dev(inp.bias)))
    _sync()
    ref = O.router_logits(inp.x, inp.w_r, inp.bias)
    err = np.max(np.abs(got.astype(np.float64) - ref))
    assert err <= 1e-4 * np.max(np.abs(ref)) + 1e-6, err


# ----------------------------------------------------------------- route ----
ROUTE_CASES = [
    # N, E, K, align, p_drop, renorm, logits mode
    (256, 8, 2, 1, 0.0, 0, "normal"),
    (1000, 256, 8, 1, 0.0, 0, "zipf"),
    (4096, 256, 8, 1, 0.0, 0, "zipf"),
    (3000, 128, 8, 1, 0.05, 0, "zipf"),
    (777, 256, 8, 32, 0.0, 0, "zipf"),
    (64, 8, 8, 1, 0.0, 1, "normal"),
    (1, 4, 1, 1, 0.0, 0, "normal"),
    (130, 16, 3, 1, 1.0, 0, "normal"),
    (500, 64, 4, 1, 0.0, 0, "ties"),
    (300, 32, 5, 32, 0.1, 1, "zeros"),
    (100, 1024, 32, 1, 0.0, 0, "normal"),
    (65, 7, 2, 1, 0.0, 0, "normal"),
    (0, 8, 2, 1, 0.0, 0, "normal"),
    # expert counts just past each logits-per-lane size of the top-K kernel
    # (64, 128, 256 per wave) and inside the 8-per-lane one
    (200, 65, 4, 1, 0.1, 0, "normal"),
    (300, 129, 6, 1, 0.0, 1, "zipf"),
    (400, 384, 8, 32, 0.0, 0, "zipf"),
    (150, 512, 16, 1, 0.0, 0, "ties"),
]


def _logits(N, E, mode, seed):
    if mode == "zeros":
        return np.zeros((N, E), np.float32)
    if mode == "ties":
        return np.random.default_rng(seed).integers(-2, 3, size=(N, E)).astype(np.float32)
    L = S.random_logits(N, E, seed)
    if mode == "zipf":
        wl = S.scaled(S.WORKLOADS["dsv3_bf16"], N=max(N, 1), E=E, K=1, D=8, H=8)
        L = (L + S.zipf_bias(wl, seed)[None, :]).astype(np.float32)
    return L


@pytest.mark.parametrize("case", ROUTE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_route_bit_exact(case):
    N, E, K, align, pdrop, renorm, mode = case
    print(f"route {case}", flush=True)
    L = _logits(N, E, mode, N + E + K)
    drop = None
    if pdrop:
        drop = (np.random.default_rng(5).random((N, K)) < pdrop).astype(np.uint8)
    rc = N * K + E * (align - 1)
    g = M.route(dev(L), K, drop=dev(drop) if drop is not None else None, renorm=renorm, align=align)
    _sync()
    idx = O.topk_select(L, K) if N else np.zeros((0, K), np.int32)
    prob = O.route_probs(L, idx, renorm) if N else np.zeros((0, K), np.float32)
    c, o, d, r = O.route_map(idx, drop, E, align, rc)
    assert np.array_equal(host(g["topk_idx"]), idx)
    assert np.max(np.abs(host(g["topk_prob"]).astype(np.float64) - prob), initial=0.0) <= 1e-6
    assert np.array_equal(host(g["counts"]), c)
    assert np.array_equal(host(g["offsets"]), o)
    assert np.array_equal(host(g["dst_rows"]), d)
    assert np.array_equal(host(g["row_route"]), r)


@pytest.mark.parametrize("N,E,K,G,M_,renorm", [(2000, 256, 8, 8, 4, 0), (700, 64, 6, 16, 3, 1),
                                               (333, 32, 8, 4, 2, 0), (129, 128, 4, 64, 8, 0),
                                               (50, 16, 4, 2, 1, 1), (300, 512, 8, 8, 4, 0)])
def test_route_grouped_bit_exact(N, E, K, G, M_, renorm):
    """Group-limited top-K through moe_route against the oracle.  Group scores
    are sums of fp32 probabilities on the GPU and fp64 ones in the oracle, so a
    token may differ only where the oracle's kept/dropped group boundary is a
    near-tie; every other token, and the whole route map of identical
    selections, is compared bit for bit."""
    print(f"route grouped N={N} E={E} K={K} G={G} M={M_}", flush=True)
    L = _logits(N, E, "zipf", N + E + G)
    g = M.route(dev(L), K, renorm=renorm, n_group=G, topk_group=M_)
    _sync()
    idx = O.topk_select_grouped(L, K, G, M_)
    got = host(g["topk_idx"])
    diff = np.any(got != idx, axis=1)
    if np.any(diff):
        sc = -np.sort(-O.group_scores(L[diff], G), axis=1)
        gap = sc[:, M_ - 1] - sc[:, M_]
        assert np.all(gap <= 1e-5 * sc[:, 0]), "selection differs away from a group-score tie"
    assert diff.mean() < 0.01
    keep = ~diff
    prob = O.route_probs(L, idx, renorm)
    assert np.max(np.abs(host(g["topk_prob"])[keep].astype(np.float64) - prob[keep]), initial=0.0) <= 1e-6
    if not np.any(diff):
        c, o, d, r = O.route_map(idx, None, E, 1, N * K)
        for k, ref in (("counts", c), ("offsets", o), ("dst_rows", d), ("row_route", r)):
            assert np.array_equal(host(g[k]), ref), k


# -------------------------------------------------------------- dispatch ----
def _routed(N, D, E, K, align, seed, pdrop=0.0):
    wl = S.scaled(S.WORKLOADS["dsv3_bf16"], N=N, D=D, E=E, K=K, H=32, p_drop=pdrop,
                  mxfp8=(align == 32))
    inp = S.make_inputs(wl, seed, weights=False)
    L = _logits(N, E, "zipf", seed)
    idx = O.topk_select(L, K)
    prob = O.route_probs(L, idx, 0)
    c, o, d, r = O.route_map(idx, inp.drop, E, align, wl.rows_cap)
    return wl, inp, idx, prob, c, o, d, r


@pytest.mark.parametrize("N,D,E,K", [(256, 128, 8, 2), (300, 7168, 64, 8), (97, 8, 4, 2),
                                     (200, 4104, 16, 4), (1, 256, 2, 2)])
def test_dispatch_bf16_and_weighted_bit_exact(N, D, E, K):
    print(f"dispatch N={N} D={D} E={E} K={K}", flush=True)
    wl, inp, idx, prob, c, o, d, r = _routed(N, D, E, K, 1, 11, pdrop=0.1)
    x = dev_bf16(inp.x)
    dst = dev(d)
    out = poison_bf16((wl.rows_cap, D))
    M.dispatch(x, dst, E, out=out)
    wout = poison_bf16((wl.rows_cap, D))
    M.dispatch(x, dst, E, weight=dev(prob), out=wout)
    _sync()
    n = int(o[-1])
    assert np.array_equal(bits(out)[:n], O.bf16_bits(O.dispatch(inp.x, r, K))[:n])
    assert np.array_equal(bits(wout)[:n], O.bf16_bits(O.dispatch(inp.x, r, K, weight=prob))[:n])


@pytest.mark.parametrize("N,D,E,K", [(256, 128, 8, 2), (300, 7168, 64, 8), (45, 32, 4, 4),
                                     (130, 4128, 16, 3), (50, 384, 16, 10)])
def test_dispatch_mxfp8_bit_exact(N, D, E, K):
    print(f"dispatch mxfp8 N={N} D={D} E={E} K={K}", flush=True)
    wl, inp, idx, prob, c, o, d, r = _routed(N, D, E, K, 32, 12)
    q = torch.full((wl.rows_cap, D), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((wl.rows_cap, D // 32), 0xCD, dtype=torch.uint8, device="cuda")
    M.dispatch(dev_bf16(inp.x), dev(d), E, counts=dev(c), offsets=dev(o), align=32, mxfp8=True,
               out=q, out_scales=s)
    _sync()
    rq, rs = O.dispatch_mxfp8(inp.x, r, K)
    n = int(o[-1])
    assert np.array_equal(host(q)[:n], rq[:n])
    assert np.array_equal(host(s)[:n], rs[:n])


# --------------------------------------------------------------- combine ----
# D = 3584 is one full row segment (7 vectors a lane), 3592 one vector more
# (two segments of 4), 4104 a ragged second segment, 8 a single lane
@pytest.mark.parametrize("N,D,E,K,pdrop", [(256, 128, 8, 2, 0.0), (300, 7168, 64, 8, 0.05),
                                           (97, 8, 4, 2, 0.3), (200, 4104, 16, 4, 1.0),
                                           (150, 3584, 16, 3, 0.1), (150, 3592, 16, 9, 0.1)])
def test_combine_and_unweighted(N, D, E, K, pdrop):
    print(f"combine N={N} D={D} E={E} K={K} drop={pdrop}", flush=True)
    wl, inp, idx, prob, c, o, d, r = _routed(N, D, E, K, 1, 13, pdrop=pdrop)
    y = S.random_bf16((wl.rows_cap, D), 13, 1)
    out = M.combine(dev_bf16(y), dev(d), dev(prob), E=E)
    out1 = M.combine(dev_bf16(y), dev(d), None, E=E)
    _sync()
    assert_bf16_close(vals(out), O.combine(y, d, prob), "combine")
    assert_bf16_close(vals(out1), O.dispatch_bwd(y, d), "combine unweighted")
    if pdrop == 1.0:
        assert np.all(bits(out) == 0) and np.all(bits(out1) == 0)


@pytest.mark.parametrize("N,D,E,K,pdrop", [(256, 128, 8, 2, 0.0), (300, 4096, 64, 8, 0.05),
                                           (61, 72, 4, 3, 0.3), (120, 1040, 16, 10, 0.1)])
def test_combine_bwd(N, D, E, K, pdrop):
    print(f"combine_bwd N={N} D={D} E={E} K={K}", flush=True)
    wl, inp, idx, prob, c, o, d, r = _routed(N, D, E, K, 1, 14, pdrop=pdrop)
    y = S.random_bf16((wl.rows_cap, D), 14, 1)
    dout = S.random_bf16((N, D), 14, 2)
    dyd, dprob = M.combine_bwd(dev_bf16(dout), dev(d), dev(prob), dev_bf16(y), wl.rows_cap, E=E)
    _sync()
    live = r >= 0
    assert np.array_equal(bits(dyd)[live], O.bf16_bits(O.combine_bwd(dout, d, prob, wl.rows_cap))[live])
    assert_bf16_close(host(dprob), O.dprob(dout, y, d), "dprob")
    assert np.all(host(dprob)[d < 0] == 0)


# -------------------------------------------------------------- quantize ----
def test_quantize_mxfp8_bit_exact():
    rng = np.random.default_rng(21)
    rows, cols = 300, 256
    v = rng.standard_normal((rows, cols)) * np.ldexp(1.0, rng.integers(-140, 120, (rows, 1)))
    v[0] = 0.0
    v[1] = -0.0
    v[2, :32] = 448.0
    v[2, 32:64] = 464.0
    v[3] = np.ldexp(1.0, -133) * rng.integers(-3, 4, cols)       # bf16 subnormals
    v[4] = np.clip(rng.standard_normal(cols), -3, 3) * 1e38       # near the top, still finite
    u = S.f32_to_bf16_bits(v.astype(np.float32))
    q, s = M.quantize_mxfp8(dev_bf16(u))
    _sync()
    rq, rs = O.quantize_mxfp8(u)
    assert np.array_equal(host(s), rs)
    assert np.array_equal(host(q), rq)


@pytest.mark.parametrize("rows,cols", [(37, 32), (50, 160), (64, 384), (21, 7168)])
def test_quantize_mxfp8_widths(rows, cols):
    """Row quantization at widths that take the one-block-per-four-lanes path
    (cols % 128 != 0) and the 16-elements-per-lane path (cols % 128 == 0, one
    partial pass at 7168 columns), against the oracle."""
    print(f"quantize rows={rows} cols={cols}", flush=True)
    rng = np.random.default_rng(rows + cols)
    v = rng.standard_normal((rows, cols)) * np.ldexp(1.0, rng.integers(-20, 20, (rows, 1)))
    v[0, : cols // 2] = 0.0                                        # all-zero blocks
    u = S.f32_to_bf16_bits(v.astype(np.float32))
    q, s = M.quantize_mxfp8(dev_bf16(u))
    _sync()
    rq, rs = O.quantize_mxfp8(u)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(s), rs)


def test_quantize_mxfp8_every_bf16_value():
    """All finite bf16 patterns, each in a block with an amax that fixes a range
    of scales: the element encoder sees every input value."""
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = O.bits_to_f64(allb)
    fin = allb[np.isfinite(v)]
    rng = np.random.default_rng(22)
    pad = (-len(fin)) % 32
    body = np.concatenate([fin, np.zeros(pad, np.uint16)])
    rng.shuffle(body)
    u = body.reshape(-1, 256 if body.size % 256 == 0 else 32)
    q, s = M.quantize_mxfp8(dev_bf16(u))
    _sync()
    rq, rs = O.quantize_mxfp8(u)
    assert np.array_equal(host(s), rs)
    assert np.array_equal(host(q), rq)


def test_quantize_mxfp8_every_value_at_every_scale():
    """Each block's amax is the top of one bf16 binade (exponent field f = 1..254,
    which spans every scale exponent a block can take); its other 31 slots run
    over all values of binade f and below, both signs.  Every finite bf16 value
    thus meets every scale that can apply to it."""
    blocks = []
    for f in range(1, 255):
        mags = np.arange(0, (f + 1) << 7, dtype=np.uint32)
        members = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        members = np.concatenate([members, np.zeros((-len(members)) % 31, np.uint16)]).reshape(-1, 31)
        amax = np.full((members.shape[0], 1), (f << 7) | 0x7F, np.uint16)
        blocks.append(np.concatenate([amax, members], axis=1))
    u = np.concatenate(blocks)
    u = np.concatenate([u, np.zeros(((-u.shape[0]) % 8, 32), np.uint16)]).reshape(-1, 256)
    print(f"quantize rows={u.shape[0]} cols=256", flush=True)
    q, s = M.quantize_mxfp8(dev_bf16(u))
    _sync()
    rq, rs = O.quantize_mxfp8(u)
    assert np.array_equal(host(s), rs)
    assert np.array_equal(host(q), rq)

def test_quantize_mxfp8_cols_every_value_at_every_scale():
    """The column-wise quantizer on the same exhaustive blocks, each block laid
    along a column (32 rows of src): bytes and scales equal the oracle's."""
    blocks = []
    for f in range(1, 255):
        mags = np.arange(0, (f + 1) << 7, dtype=np.uint32)
        members = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        members = np.concatenate([members, np.zeros((-len(members)) % 31, np.uint16)]).reshape(-1, 31)
        amax = np.full((members.shape[0], 1), (f << 7) | 0x7F, np.uint16)
        blocks.append(np.concatenate([amax, members], axis=1))
    u = np.concatenate(blocks)                              # [blocks, 32]
    u = np.concatenate([u, np.zeros(((-u.shape[0]) % 8, 32), np.uint16)])   # columns: a multiple of 8
    src = np.ascontiguousarray(u.T)[None]                   # [1, 32, blocks]: a block per column
    nb = u.shape[0]
    print(f"quantize cols blocks={nb}", flush=True)
    q = torch.empty((1, nb, 32), dtype=torch.uint8, device="cuda")
    sc = torch.empty((1, nb, 1), dtype=torch.uint8, device="cuda")
    M.quantize_mxfp8_cols(dev_bf16(src), q, sc)
    _sync()
    rq, rs = O.quantize_mxfp8(u)
    assert np.array_equal(host(sc)[0, :, 0], rs[:, 0])
    assert np.array_equal(host(q)[0], rq)


@pytest.mark.parametrize("B,R,C,ld,col0", [(3, 96, 200, 192, 96), (2, 160, 64, 160, 0), (1, 288, 328, 320, 32)])
def test_quantize_mxfp8_cols_ragged_and_offset(B, R, C, ld, col0):
    """Tails in both tile dimensions, a column offset inside a wider row:
    exactly columns col0 .. col0 + R - 1 of each q row are written."""
    print(f"quantize cols B={B} R={R} C={C} ld={ld} col0={col0}", flush=True)
    src = S.random_bf16((B, R, C), 41, 1, std=2.0)
    src[:, :32, :5] = 0                                     # all-zero blocks take scale code 0
    q = torch.full((B, C, ld), 0xAB, dtype=torch.uint8, device="cuda")
    sc = torch.full((B, C, ld // 32), 0xCD, dtype=torch.uint8, device="cuda")
    M.quantize_mxfp8_cols(dev_bf16(src), q, sc, col0)
    _sync()
    qh, sh = host(q), host(sc)
    for b in range(B):
        rq, rs = O.quantize_mxfp8(np.ascontiguousarray(src[b].T))
        assert np.array_equal(qh[b][:, col0:col0 + R], rq), b
        assert np.array_equal(sh[b][:, col0 // 32:(col0 + R) // 32], rs), b
    assert np.all(np.delete(qh, np.s_[col0:col0 + R], axis=2) == 0xAB)
    assert np.all(np.delete(sh, np.s_[col0 // 32:(col0 + R) // 32], axis=2) == 0xCD)


def test_weight_copies_for_dgrad_bit_exact():
    """W_down^T along D and [W_gate^T | W_up^T] along H, from the bf16 weights."""
    wl = S.scaled(S.WORKLOADS["dsv3_mxfp8"], "mx_wt", N=8, D=384, E=5, K=2, H=160)
    inp = S.make_inputs(wl, 42)
    print("weight copies for dgrad", flush=True)
    q = M.quantize_weights_mxfp8_dgrad(dev_bf16(inp.w_gate), dev_bf16(inp.w_up), dev_bf16(inp.w_down))
    _sync()
    ref = O.quantize_weights_mxfp8_dgrad(inp.w_gate, inp.w_up, inp.w_down)
    for k in ref:
        assert np.array_equal(host(q[k]), ref[k]), k


def test_swiglu_standalone():
    rows, n = 333, 160
    g = S.random_bf16((rows, n), 23, 1, std=3.0)
    u = S.random_bf16((rows, n), 23, 2)
    h = M.swiglu(dev_bf16(g), dev_bf16(u))
    h2, q, s = M.swiglu(dev_bf16(g), dev_bf16(u), mxfp8=True)
    _sync()
    ref = O.swiglu(O.bits_to_f64(g), O.bits_to_f64(u))
    assert_bf16_close(vals(h), ref, "swiglu")
    assert np.array_equal(bits(h), bits(h2))
    rq, rs = O.quantize_mxfp8(ref)
    assert rel_frobenius(O.dequantize_mxfp8(host(q), host(s)), O.dequantize_mxfp8(rq, rs)) <= 3e-2
    assert np.mean(host(q) == rq) > 0.99


# ---------------------------------------------------------- grouped GEMM ----
GEMM_CASES = [
    # segment sizes, k_dim, n_dim, rows_cap slack
    ((0, 1, 130, 64, 257), 200, 136, 8),
    ((300, 513), 256, 256, 0),
    ((17,), 64, 8, 3),
    ((0, 0, 5), 8, 128, 0),
    ((129, 0, 64, 1, 255, 128), 384, 264, 40),
    # shapes the persistent kernel takes (k % 64 == 0, n % 16 == 0), one per
    # row-block rule (64 / 128 / 256 rows), partial n-tiles and empty experts
    ((0, 1, 130, 64, 257), 192, 144, 8),
    ((1000, 0, 777, 1), 128, 272, 0),
    ((2000, 1700), 128, 160, 0),
    ((5000,), 64, 512, 3),
    ((3, 0, 0, 90, 0, 17, 0, 0, 200, 1, 0, 64, 0, 0, 0, 33), 320, 96, 0),
    # 32- and 64-row tile boundaries: whole experts of 32 and 33 rows, and
    # large experts whose last row block holds exactly 32 or 64 rows
    ((288, 32, 33, 320, 2), 256, 192, 0),
    # shapes the persistent backward kernels take (dgrad: n % 64 == 0 and
    # k % 16 == 0; wgrad: n, k % 16 == 0): partial 256-column tiles, ragged
    # and empty experts, experts above and below 256 rows
    ((0, 1, 130, 64, 257), 176, 320, 8),
    ((300, 0, 700, 17), 208, 192, 0),
    ((3, 0, 0, 90, 0, 17, 0, 0, 200, 1, 0, 64, 0, 0, 0, 33), 144, 64, 0),
    ((1100,), 48, 128, 5),
]


def _segments(sizes, slack):
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    return offsets, int(offsets[-1]) + slack


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: f"{len(c[0])}e-k{c[1]}-n{c[2]}")
def test_grouped_gemm_fwd_bf16(case):
    sizes, k_dim, n_dim, slack = case
    print(f"gemm fwd {case}", flush=True)
    offsets, rc = _segments(sizes, slack)
    E = len(sizes)
    a = S.random_bf16((rc, k_dim), 31, 1)
    w0 = S.random_bf16((E, n_dim, k_dim), 31, 2, std=1 / np.sqrt(k_dim))
    w1 = S.random_bf16((E, n_dim, k_dim), 31, 3, std=1 / np.sqrt(k_dim))
    da, dw0, dw1, do = dev_bf16(a), dev_bf16(w0), dev_bf16(w1), dev(offsets)
    c = poison_bf16((rc, n_dim))
    M.grouped_gemm_fwd(da, dw0, do, out=c)
    G, U, H = M.grouped_gemm_fwd(da, dw0, do, b1=dw1, swiglu=True)
    _sync()
    n = int(offsets[-1])
    ref = O.grouped_gemm(a, w0, offsets)
    assert_bf16_close(vals(c)[:n], ref[:n], "c")
    assert np.all(bits(c)[n:] == 0x7FA0)                       # rows past the segments untouched
    assert_bf16_close(vals(G)[:n], ref[:n], "G")
    refU = O.grouped_gemm(a, w1, offsets)
    assert_bf16_close(vals(U)[:n], refU[:n], "U")
    assert_bf16_close(vals(H)[:n], O.swiglu(ref, refU)[:n], "H")


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: f"{len(c[0])}e-k{c[1]}-n{c[2]}")
def test_grouped_gemm_bwd_bf16(case):
    sizes, k_dim, n_dim, slack = case
    print(f"gemm bwd {case}", flush=True)
    offsets, rc = _segments(sizes, slack)
    E = len(sizes)
    a = S.random_bf16((rc, k_dim), 32, 1)
    w0 = S.random_bf16((E, n_dim, k_dim), 32, 2, std=1 / np.sqrt(k_dim))
    w1 = S.random_bf16((E, n_dim, k_dim), 32, 3, std=1 / np.sqrt(k_dim))
    dc0 = S.random_bf16((rc, n_dim), 32, 4)
    dc1 = S.random_bf16((rc, n_dim), 32, 5)
    gg = S.random_bf16((rc, k_dim), 32, 6, std=2.0)
    uu = S.random_bf16((rc, k_dim), 32, 7)
    do = dev(offsets)
    n = int(offsets[-1])
    r1 = M.grouped_gemm_bwd(do, dev_bf16(dc0), b0=dev_bf16(w0), a=dev_bf16(a))
    r2 = M.grouped_gemm_bwd(do, dev_bf16(dc0), b0=dev_bf16(w0), a=dev_bf16(a), dc1=dev_bf16(dc1),
                            b1=dev_bf16(w1))
    r3 = M.grouped_gemm_bwd(do, dev_bf16(dc0), b0=dev_bf16(w0), swiglu_g=dev_bf16(gg),
                            swiglu_u=dev_bf16(uu), wgrad=False)
    _sync()
    assert_bf16_close(vals(r1["da"])[:n], O.grouped_dgrad(dc0, w0, offsets)[:n], "da")
    assert_bf16_close(vals(r1["db0"]), O.grouped_wgrad(dc0, a, offsets), "db0")
    assert_bf16_close(vals(r2["da"])[:n], O.grouped_dgrad(dc0, w0, offsets, dc1, w1)[:n], "da dual")
    assert_bf16_close(vals(r2["db1"]), O.grouped_wgrad(dc1, a, offsets), "db1")
    # SwiGLU backward epilogue: the oracle's expert backward with dc0 as dY
    # and w0 as the down weight ([n_dim=D][k_dim=H])
    zeros = np.zeros((E, k_dim, n_dim))
    eb = O.experts_bwd(dc0, np.zeros((rc, n_dim)), O.bits_to_f64(gg), O.bits_to_f64(uu),
                       np.zeros((rc, k_dim)), offsets, zeros, zeros, w0)
    assert_bf16_close(vals(r3["dg"])[:n], eb["dg"][:n], "dg")
    assert_bf16_close(vals(r3["du"])[:n], eb["du"][:n], "du")
    for e, sz in enumerate(sizes):
        if sz == 0:
            assert np.all(bits(r1["db0"])[e] == 0)


MX_GEMM_CASES = [
    ((0, 32, 160, 64, 288), 256, 128),
    ((320, 96), 512, 256),
    ((32,), 128, 64),
    # 256-row and 128-row tiles side by side, partial n-tiles, empty experts
    ((256, 0, 64, 600, 1, 0, 33), 384, 160),
    ((0, 0, 1000), 128, 96),
    # k % 128 != 0: the m-tile kernel
    ((96, 7), 160, 64),
]


@pytest.mark.parametrize("case", MX_GEMM_CASES, ids=lambda c: f"{len(c[0])}e-k{c[1]}-n{c[2]}")
def test_grouped_gemm_fwd_mxfp8(case):
    """Block-scaled product of quantized operands (eq. 87) against the oracle's
    dequantized float64 product, both from the same synthetic bf16 sources."""
    sizes, k_dim, n_dim = case
    print(f"gemm mxfp8 {case}", flush=True)
    offsets, rc = _segments(sizes, 32)
    E = len(sizes)
    a = S.random_bf16((rc, k_dim), 33, 1)
    w0 = S.random_bf16((E, n_dim, k_dim), 33, 2, std=1 / np.sqrt(k_dim))
    w1 = S.random_bf16((E, n_dim, k_dim), 33, 3, std=1 / np.sqrt(k_dim))
    aq, as_ = O.quantize_mxfp8(a)
    wq = O.quantize_weights_mxfp8(w0, w1, np.zeros((E, 32, n_dim), np.float64))
    do = dev(offsets)
    c = M.grouped_gemm_fwd(dev(aq), dev(wq["wg_q"]), do, a_scales=dev(as_), b0_scales=dev(wq["wg_s"]))
    G, U, H, hq, hs = M.grouped_gemm_fwd(dev(aq), dev(wq["wg_q"]), do, b1=dev(wq["wu_q"]), swiglu=True,
                                         a_scales=dev(as_), b0_scales=dev(wq["wg_s"]),
                                         b1_scales=dev(wq["wu_s"]), quantize_act=True)
    _sync()
    n = int(offsets[-1])
    refG = np.zeros((rc, n_dim))
    refU = np.zeros((rc, n_dim))
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            refG[lo:hi] = O.mxfp8_gemm(aq[lo:hi], as_[lo:hi], wq["wg_q"][e], wq["wg_s"][e])
            refU[lo:hi] = O.mxfp8_gemm(aq[lo:hi], as_[lo:hi], wq["wu_q"][e], wq["wu_s"][e])
    assert_bf16_close(vals(c)[:n], refG[:n], "mx c")
    assert_bf16_close(vals(G)[:n], refG[:n], "mx G")
    assert_bf16_close(vals(U)[:n], refU[:n], "mx U")
    refH = O.swiglu(refG, refU)
    assert_bf16_close(vals(H)[:n], refH[:n], "mx H")
    rq, rs = O.quantize_mxfp8(refH[:n])
    assert rel_frobenius(O.dequantize_mxfp8(host(hq)[:n], host(hs)[:n]), O.dequantize_mxfp8(rq, rs)) <= 3e-2
    # the epilogue's quantization of the H it stored is the block rule exactly
    oq, os_ = O.quantize_mxfp8(vals(H)[:n])
    assert np.array_equal(host(hq)[:n], oq) and np.array_equal(host(hs)[:n], os_)

"""CPU oracle for one GPU's routed MoE expert layer.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain definition that the
HIP kernels are checked against.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it; the product path
never does.  It shares no code with the GPU library and does not import it.

Everything is computed in float64 from the bf16 / fp32 values of the inputs.
A rounding to bf16 or fp32 appears exactly where the layer stores a tensor in
that format.  Passing ``exact=True`` removes every bf16 rounding, which turns
the forward into a smooth function for finite-difference checks.

Sources (the pages this follows):
  [KOSMOS]  "KOSMOS: Self-scheduling Persistent Kernels for Communication-Compute
            Overlap", section 3.3.1 (MoE forward: route, plan, dispatch with
            GEMM1 and SwiGLU, GEMM2, fold), section 3.3.2 (backward), section
            2.2 (MXFP8 training).
  [OLMo-A]  "OLMo-core MoE, Appendix A: Kernel Interfaces and Profiling
            Reference", A.1 (dispatch/combine and their adjoints, the fused
            routed-expert node), A.2 (dst_rows route tensor, invalid routes),
            A.3 (route id), A.4 (MXFP8 payload layout), A.5 (eq. 87).

Readings where the pages are silent (each listed in the design notes):
  score = softmax over all experts in fp32; top-K keyed on the fp32 logits,
  ties to the lower expert index, slot 0 = best; renormalisation optional (off
  by default); the per-expert bias is added to the logits before both; rows of
  an expert segment are in ascending route id; SwiGLU = silu(gate) * up;
  E8M0 exponent = floor(log2(amax)) - 8 (the OCP MX rule), E4M3 = OCP E4M3FN
  with round-to-nearest-even and saturation at +-448.

Parity pins: every function here is checked in tests/test_oracle_*.py against
brute force, closed forms, library routines or invariants.  The exact fp32 bits
of the softmax and of the fp32-rounded sums are not pinned beyond tolerance
(parity unpinned at the last fp32 bit; the comparison is by tolerance).
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------


def bits_to_f64(u16) -> np.ndarray:
    """bf16 bit patterns -> their exact values as float64."""
    u = np.ascontiguousarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def values(a) -> np.ndarray:
    """Accept bf16 bit patterns (uint16) or real values; return float64 values."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bits_to_f64(a)
    return a.astype(np.float64, copy=False)


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits; its smallest normal is 2^-126 and its
    subnormal spacing is 2^-133.  Written with frexp so the rounding happens
    once, straight from float64.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                 # x = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)            # below 2^-126 the spacing stays 2^-133
    return np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)


def round_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_bits(v) -> np.ndarray:
    """bf16-representable float64 values -> bit patterns (exact)."""
    f = np.ascontiguousarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _identity(x):
    return np.asarray(x, dtype=np.float64)


def _rounder(exact: bool):
    return _identity if exact else round_bf16


# --------------------------------------------------------------------------
# route: logits, score, top-K      [KOSMOS 3.3.1 step 1 "Route"]
# --------------------------------------------------------------------------


def router_logits(x, w_r, bias=None) -> np.ndarray:
    """L[t,e] = fp32(sum_d x[t,d] * W_r[e,d]) + b[e], bias added in fp32.

    x: [N,D] bf16; w_r: [E,D] bf16 (stored expert-major); bias: [E] fp32 or None.
    The dot products of bf16 values are summed in float64 and rounded once.
    """
    L = (values(x) @ values(w_r).T).astype(np.float32)
    if bias is not None:
        L = L + np.asarray(bias, dtype=np.float32)[None, :]
    return L.astype(np.float32)


def softmax(L) -> np.ndarray:
    """Softmax over all experts of each token (float64)."""
    L = np.asarray(L, dtype=np.float64)
    z = np.exp(L - L.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def topk_select(L, K: int) -> np.ndarray:
    """The K largest logits of each token, best first; ties go to the lower index.

    Done as K rounds of "take the maximum, then remove it"; argmax returns the
    first (lowest-index) maximum, which is the tie rule.
    """
    work = np.array(L, dtype=np.float64, copy=True)
    N, E = work.shape
    if K > E:
        raise ValueError("K > E")
    out = np.empty((N, K), dtype=np.int32)
    rows = np.arange(N)
    for k in range(K):
        j = np.argmax(work, axis=1)
        out[:, k] = j
        work[rows, j] = -np.inf
    return out


def group_scores(L, n_group: int) -> np.ndarray:
    """[N, n_group] score of each expert group: the sum of the two largest
    routing probabilities in the group (the one probability of a one-expert
    group).  Groups are n_group contiguous ranges of E / n_group experts."""
    p = softmax(L)
    N, E = p.shape
    gs = E // n_group
    top = -np.sort(-p.reshape(N, n_group, gs), axis=2)
    return top[:, :, :2].sum(axis=2)


def topk_select_grouped(L, K: int, n_group: int, topk_group: int) -> np.ndarray:
    """Group-limited top-K [KOSMOS 3.3.1 step 1, "(group-limited) top-k";
    the pages give no rule, see group_scores]: keep the topk_group groups with
    the largest scores (ties to the lower group), then take the K largest logits
    among the kept groups' experts (ties to the lower expert, best first)."""
    L = np.asarray(L, dtype=np.float64)
    N, E = L.shape
    if E % n_group or topk_group > n_group or topk_group * (E // n_group) < K:
        raise ValueError("bad grouping")
    gkeep = topk_select(group_scores(L, n_group), topk_group)     # same ranking rule on the groups
    gs = E // n_group
    keep = np.zeros((N, n_group), dtype=bool)
    np.put_along_axis(keep, gkeep.astype(np.int64), True, axis=1)
    masked = np.where(np.repeat(keep, gs, axis=1), L, -np.inf)
    return topk_select(masked, K)


def aux_loss(L, counts, K: int, alpha: float):
    """Load-balance loss from the route step's aux-loss inputs [KOSMOS 3.3.1
    step 1; the pages give no formula, so the Switch-style reading]:
    f_e = valid routes to e / (N K), P_e = mean over tokens of the routing
    probability of e, aux = alpha * E * sum_e f_e P_e.  Returns (aux, P)."""
    p = softmax(L)
    N, E = p.shape
    f = np.asarray(counts, dtype=np.float64) / (N * K)
    P = p.mean(axis=0)
    return float(alpha * E * np.sum(f * P)), P


def aux_dlogits(L, counts, K: int, alpha: float, d_aux: float = 1.0) -> np.ndarray:
    """Gradient of d_aux * aux_loss with respect to the logits, the counts
    (a selection) held fixed: alpha E / N * p_te (f_e - sum_j p_tj f_j)."""
    p = softmax(L)
    N, E = p.shape
    f = np.asarray(counts, dtype=np.float64) / (N * K)
    return d_aux * alpha * E / N * p * (f[None, :] - (p @ f)[:, None])


def route_weights(L, idx, renorm: int = 0) -> np.ndarray:
    """Dispatch weight of each selected slot in float64: the softmax
    probability of its expert, optionally divided by the sum over the K
    selected slots (dropped slots included: a drop happens after routing)."""
    p = softmax(L)
    sel = np.take_along_axis(p, np.asarray(idx, dtype=np.int64), axis=1)
    if renorm:
        sel = sel / sel.sum(axis=1, keepdims=True)
    return sel


def route_probs(L, idx, renorm: int = 0) -> np.ndarray:
    """The dispatch weights as the layer stores them: fp32."""
    return route_weights(L, idx, renorm).astype(np.float32)


# --------------------------------------------------------------------------
# plan: the route map     [KOSMOS 3.3.1 step 2 "Plan"; OLMo-A A.2, A.3]
# --------------------------------------------------------------------------


def route_valid(idx, drop, E: int) -> np.ndarray:
    """A route (t,k) is valid unless it is dropped or names no expert in [0,E)."""
    idx = np.asarray(idx)
    v = (idx >= 0) & (idx < E)
    if drop is not None:
        v &= np.asarray(drop) == 0
    return v


def route_map(idx, drop, E: int, align: int, rows_cap: int, n_shared: int = 0):
    """Stable counting sort of the valid routes into expert-contiguous rows.

    Route id r = t*K + k.  counts[e] = number of valid routes to e;
    each expert's segment is counts[e] rounded up to a multiple of ``align``;
    offsets is the exclusive scan of the segment sizes (E+1 entries).  Inside a
    segment the routes sit in ascending route id.  dst_rows[t,k] is the row of
    route (t,k) or -1 if invalid; row_route[i] is the route id held by row i, or
    -1 for padding and unused rows.
    Returns (counts int32 [E], offsets int32 [E+1], dst_rows int32 [N,K],
    row_route int32 [rows_cap]).
    n_shared = 1 appends the shared expert's segment: all N tokens, in token
    order, at offsets[E], padded to ``align`` like every group (counts gets N,
    offsets a last entry; its rows hold no route, row_route -1).
    """
    idx = np.asarray(idx)
    N, K = idx.shape
    valid = route_valid(idx, drop, E)
    e_of_r = np.where(valid, idx, E).reshape(-1).astype(np.int64)   # E = "no expert"
    counts = np.bincount(e_of_r, minlength=E + 1)[:E]
    seg = ((counts + align - 1) // align) * align
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(seg)
    if offsets[E] > rows_cap:
        raise ValueError("rows_cap too small")
    order = np.argsort(e_of_r, kind="stable")      # grouped by expert, route id ascending
    nvalid = int(counts.sum())
    order = order[:nvalid]
    first_in_order = np.concatenate([[0], np.cumsum(counts)[:-1]])
    e_sorted = e_of_r[order]
    dst = offsets[e_sorted] + (np.arange(nvalid) - first_in_order[e_sorted])
    dst_rows = np.full(N * K, -1, dtype=np.int64)
    dst_rows[order] = dst
    row_route = np.full(rows_cap, -1, dtype=np.int64)
    row_route[dst] = order
    if n_shared:
        counts = np.append(counts, N)
        offsets = np.append(offsets, offsets[E] + ((N + align - 1) // align) * align)
        if offsets[-1] > rows_cap:
            raise ValueError("rows_cap too small")
    return (counts.astype(np.int32), offsets.astype(np.int32),
            dst_rows.reshape(N, K).astype(np.int32), row_route.astype(np.int32))


# --------------------------------------------------------------------------
# dispatch / combine and their adjoints   [OLMo-A A.1-A.3; KOSMOS 3.3.1 steps 3, 5]
# --------------------------------------------------------------------------


def dispatch(x, row_route, K: int, weight=None, exact: bool = False) -> np.ndarray:
    """X_d[i] = x[row_route[i] // K] for every row that holds a route; other
    rows (padding, unused tail) are 0.

    With ``weight`` ([N,K] fp32) each copy is scaled by its route's weight:
    the product is formed in fp32 and stored as bf16 (the weighted PUT).
    """
    xv = values(x)
    rr = np.asarray(row_route, dtype=np.int64)
    out = np.zeros((rr.shape[0], xv.shape[1]), dtype=np.float64)
    live = rr >= 0
    tok = rr[live] // K
    if weight is None:
        out[live] = xv[tok]
    else:
        w = np.asarray(weight, dtype=np.float64).reshape(-1)[rr[live]]
        prod = w[:, None] * xv[tok]                 # exact in float64 for fp32 weights
        out[live] = prod if exact else round_bf16(round_f32(prod))
    return out


def combine(y, dst_rows, weight=None, exact: bool = False, addend=None) -> np.ndarray:
    """out[t] = sum over valid k of w[t,k] * Y[dst_rows[t,k]], stored once as bf16.

    Invalid routes (dst_rows < 0) contribute nothing; ``weight`` None means 1.
    ``addend`` [N, D] (a shared expert's rows, say) joins the sum.  The sum is
    exact (float64) and rounded once.
    """
    yv = values(y)
    dst = np.asarray(dst_rows, dtype=np.int64)
    N, K = dst.shape
    acc = np.zeros((N, yv.shape[1]), dtype=np.float64) if addend is None else np.array(values(addend), np.float64)
    for k in range(K):
        ok = dst[:, k] >= 0
        w = np.ones(N) if weight is None else np.asarray(weight, np.float64)[:, k]
        acc[ok] += w[ok, None] * yv[dst[ok, k]]
    return _rounder(exact)(acc)


def combine_bwd(dout, dst_rows, weight, rows_cap: int, exact: bool = False) -> np.ndarray:
    """Adjoint of the weighted combine: dY_d[dst_rows[t,k]] = w[t,k] * dOut[t]
    (the router-weighted dY dispatch of the backward)."""
    dst = np.asarray(dst_rows, dtype=np.int64)
    N, K = dst.shape
    rr = np.full(rows_cap, -1, dtype=np.int64)
    ok = dst.reshape(-1) >= 0
    rr[dst.reshape(-1)[ok]] = np.arange(N * K)[ok]
    return dispatch(dout, rr, K, weight=weight, exact=exact)


def dprob(dout, y, dst_rows) -> np.ndarray:
    """Gradient w.r.t. each route's weight: <dOut[t], Y[dst_rows[t,k]]>, 0 if
    invalid, fp32.  [KOSMOS 3.3.2: routing-weight gradients]"""
    dv = values(dout)
    yv = values(y)
    dst = np.asarray(dst_rows, dtype=np.int64)
    N, K = dst.shape
    g = np.zeros((N, K), dtype=np.float64)
    for k in range(K):
        ok = dst[:, k] >= 0
        g[ok, k] = np.einsum("nd,nd->n", dv[ok], yv[dst[ok, k]])
    return g.astype(np.float32)


def dispatch_bwd(dxd, dst_rows, exact: bool = False, addend=None) -> np.ndarray:
    """Adjoint of dispatch: dx[t] = sum over valid k of dX_d[dst_rows[t,k]]
    (plus ``addend``, e.g. the shared expert's dX_d rows, in the same sum)."""
    return combine(dxd, dst_rows, None, exact=exact, addend=addend)


# --------------------------------------------------------------------------
# experts: GEMM1 + SwiGLU, GEMM2       [KOSMOS 3.3.1 steps 3-4; OLMo-A A.1]
# --------------------------------------------------------------------------


def silu(g):
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def sigmoid(g):
    return 1.0 / (1.0 + np.exp(-np.asarray(g, dtype=np.float64)))


def swiglu(g, u, exact: bool = False):
    """H = silu(gate) * up, from the stored (bf16) gate and up values."""
    return _rounder(exact)(silu(g) * np.asarray(u, np.float64))


def expert_mlp(xrows, wg, wu, wd, exact: bool = False):
    """One expert on its rows.  wg, wu: [H,D]; wd: [D,H] (output-major storage).

    G = X Wg^T, U = X Wu^T (each stored bf16), H = silu(G)*U (bf16),
    Y = H Wd^T (bf16).  Returns (G, U, H, Y).
    """
    r = _rounder(exact)
    X = values(xrows)
    G = r(X @ values(wg).T)
    U = r(X @ values(wu).T)
    Hh = swiglu(G, U, exact)
    Y = r(Hh @ values(wd).T)
    return G, U, Hh, Y


def experts_fwd(xd, offsets, w_gate, w_up, w_down, exact: bool = False):
    """Apply expert e to rows offsets[e]..offsets[e+1] of X_d.  Rows outside
    every segment stay 0.  Returns (G, U, H, Y) over all rows."""
    xv = values(xd)
    rows = xv.shape[0]
    E = len(offsets) - 1
    Hd = np.asarray(w_gate).shape[1]
    D = xv.shape[1]
    G = np.zeros((rows, Hd))
    U = np.zeros((rows, Hd))
    Hh = np.zeros((rows, Hd))
    Y = np.zeros((rows, D))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b == a:
            continue          # an expert with no rows is never read
        G[a:b], U[a:b], Hh[a:b], Y[a:b] = expert_mlp(xv[a:b], w_gate[e], w_up[e], w_down[e], exact)
    return G, U, Hh, Y


# --------------------------------------------------------------------------
# grouped products on their own (the building blocks of the expert GEMMs)
# --------------------------------------------------------------------------


def grouped_gemm(a, w, offsets, exact: bool = False):
    """c[i] = a[i] . w[e]^T for the rows i of expert e's segment; w: [E, n, k]
    (output-major).  Rows outside every segment are 0."""
    av = values(a)
    E = len(offsets) - 1
    n = np.asarray(w).shape[1]
    c = np.zeros((av.shape[0], n))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            c[lo:hi] = av[lo:hi] @ values(w[e]).T
    return _rounder(exact)(c)


def grouped_dgrad(dc, w, offsets, dc1=None, w1=None, exact: bool = False):
    """da[i] = dc[i] . w[e] (+ dc1[i] . w1[e], one sum): the gradient of
    grouped_gemm with respect to a."""
    dv = values(dc)
    E = len(offsets) - 1
    k = np.asarray(w).shape[2]
    out = np.zeros((dv.shape[0], k))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            acc = dv[lo:hi] @ values(w[e])
            if dc1 is not None:
                acc = acc + values(dc1)[lo:hi] @ values(w1[e])
            out[lo:hi] = acc
    return _rounder(exact)(out)


def grouped_wgrad(dc, a, offsets, exact: bool = False):
    """dw[e] = sum over rows i of e of dc[i]^T a[i]: the gradient of grouped_gemm
    with respect to w, shape [E, n, k]; experts without rows get 0."""
    dv = values(dc)
    av = values(a)
    E = len(offsets) - 1
    out = np.zeros((E, dv.shape[1], av.shape[1]))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            out[e] = dv[lo:hi].T @ av[lo:hi]
    return _rounder(exact)(out)


# --------------------------------------------------------------------------
# whole layer, forward       [KOSMOS 3.3.1; OLMo-A A.1 fused node, A.14 saved set]
# --------------------------------------------------------------------------


def layer_fwd(x, w_r, bias, w_gate, w_up, w_down, K: int, drop=None, renorm: int = 0,
              align: int = 1, rows_cap: int = None, logits=None, exact: bool = False, n_shared: int = 0):
    """Router -> top-K -> route map -> dispatch -> experts -> weighted combine.

    ``logits`` may be given to skip the router product (route-map tests).
    n_shared = 1: a shared expert (the last of the expert weights, after the E
    routed ones) sees every token and adds its output with weight 1 [KOSMOS
    Appendix A, Table A.1: the shared expert in the MoE launch]; it is expert
    E over a segment that holds x itself.
    Returns a dict with every saved tensor and ``out``.
    """
    xv = values(x)
    N = xv.shape[0]
    E = np.asarray(w_r).shape[0]
    if rows_cap is None:
        rows_cap = N * K + E * (align - 1) + n_shared * (N + align - 1)
    L = router_logits(x, w_r, bias) if logits is None else np.asarray(logits, np.float32)
    idx = topk_select(L, K)
    prob = route_probs(L, idx, renorm)
    counts, offsets, dst_rows, row_route = route_map(idx, drop, E, align, rows_cap, n_shared)
    xd = dispatch(xv, row_route, K)
    if n_shared:
        xd[offsets[E]:offsets[E] + N] = xv
    G, U, Hh, Y = experts_fwd(xd, offsets, w_gate, w_up, w_down, exact)
    out = combine(Y, dst_rows, prob, exact, addend=Y[offsets[E]:offsets[E] + N] if n_shared else None)
    return dict(logits=L, topk_idx=idx, topk_prob=prob, counts=counts, offsets=offsets,
                dst_rows=dst_rows, row_route=row_route, xd=xd, g=G, u=U, h=Hh, y=Y, out=out,
                n_shared=n_shared)


# --------------------------------------------------------------------------
# whole layer, backward                   [KOSMOS 3.3.2; OLMo-A A.1 adjoint sequence]
# --------------------------------------------------------------------------


def swiglu_bwd(dH, G, U):
    """Adjoint of H = silu(G) U at the stored G, U, in float64:
    dG = dH U s (1 + G (1 - s)), dU = dH G s, with s = sigmoid(G)."""
    s = sigmoid(G)
    return dH * U * s * (1.0 + G * (1.0 - s)), dH * G * s


def experts_bwd(dyd, xd, g, u, h, offsets, w_gate, w_up, w_down, exact: bool = False):
    """Down dgrad with the SwiGLU backward, down wgrad, gate/up dgrad and wgrad.

    dH = dY W_down (kept at full precision; it only feeds the SwiGLU backward)
    dG = dH * U * s * (1 + G (1 - s)), s = sigmoid(G);  dU = dH * silu(G)
    dW_down[e] = dY_e^T H_e;  dX_d = dG W_gate + dU W_up (one sum);
    dW_gate[e] = dG_e^T X_e;  dW_up[e] = dU_e^T X_e.   Every stored tensor is bf16.
    """
    r = _rounder(exact)
    dy = values(dyd)
    xv = values(xd)
    rows, D = dy.shape
    E = len(offsets) - 1
    Hd = np.asarray(w_gate).shape[1]
    dG = np.zeros((rows, Hd))
    dU = np.zeros((rows, Hd))
    dXd = np.zeros((rows, D))
    dWg = np.zeros((E, Hd, D))
    dWu = np.zeros((E, Hd, D))
    dWd = np.zeros((E, D, Hd))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b == a:
            continue
        Wg, Wu, Wd = values(w_gate[e]), values(w_up[e]), values(w_down[e])
        G, U = np.asarray(g[a:b], np.float64), np.asarray(u[a:b], np.float64)
        dg_e, du_e = swiglu_bwd(dy[a:b] @ Wd, G, U)
        dG[a:b] = r(dg_e)
        dU[a:b] = r(du_e)
        dWd[e] = r(dy[a:b].T @ np.asarray(h[a:b], np.float64))
        dXd[a:b] = r(dG[a:b] @ Wg + dU[a:b] @ Wu)
        dWg[e] = r(dG[a:b].T @ xv[a:b])
        dWu[e] = r(dU[a:b].T @ xv[a:b])
    return dict(dg=dG, du=dU, dxd=dXd, dw_gate=dWg, dw_up=dWu, dw_down=dWd)


def _layer_bwd_around(fwd: dict, dout, experts, exact: bool = False):
    """The layer's adjoint sequence around an expert backward ``experts(dyd)``:
    combine-bwd (weighted dY dispatch) and the route-weight gradient before it,
    dispatch-bwd (sum of each token's K rows) after it."""
    rows_cap = fwd["y"].shape[0]
    dyd = combine_bwd(dout, fwd["dst_rows"], fwd["topk_prob"], rows_cap, exact)
    shared = None
    if fwd.get("n_shared"):
        o = fwd["offsets"]
        n = values(dout).shape[0]
        shared = slice(int(o[-2]), int(o[-2]) + n)   # its first N rows; the rest pads to the alignment
        dyd[shared] = values(dout)           # the shared expert's weight is 1
    dp = dprob(dout, fwd["y"], fwd["dst_rows"])
    eb = experts(dyd)
    dx = dispatch_bwd(eb["dxd"], fwd["dst_rows"], exact, addend=eb["dxd"][shared] if shared else None)
    eb.update(dyd=dyd, dprob=dp, dx=dx)
    return eb


def layer_bwd(fwd: dict, dout, w_gate, w_up, w_down, exact: bool = False):
    """Adjoint sequence of the layer: combine-bwd (weighted dY dispatch) and the
    route-weight gradient, expert backward, dispatch-bwd (sum of the K rows)."""
    return _layer_bwd_around(
        fwd, dout, lambda dyd: experts_bwd(dyd, fwd["xd"], fwd["g"], fwd["u"], fwd["h"], fwd["offsets"],
                                           w_gate, w_up, w_down, exact), exact)


def router_bwd(logits, idx, dprob, x, w_r, renorm: int = 0, aux_dl=None) -> dict:
    """Gradients of the router from the route-weight gradient dprob [N,K]
    (0 for invalid routes), in float64.  [KOSMOS 3.3.2 step 2: the router's
    dX_r and dW_r; the adjoint of router_logits and route_weights]

    The chain, token by token, with p = softmax(L) and s_k = p[idx_k]:
      renorm: w_k = s_k / S, S = sum_j s_j, so ds_k = (dprob_k - sum_j w_j dprob_j) / S;
      else ds_k = dprob_k;
      g_e = ds_k where e = idx_k (the K experts are distinct), else 0;
      dL_e = p_e (g_e - sum_j p_j g_j)          (softmax backward);
    then dX_r = dL W_r, dW_r = dL^T x, db_r = sum over tokens of dL.
    aux_dl, when given, is added to dL first (the aux loss's gradient).
    """
    L = np.asarray(logits, dtype=np.float64)
    N, E = L.shape
    ix = np.asarray(idx, dtype=np.int64)
    gw = np.asarray(dprob, dtype=np.float64)
    p = softmax(L)
    s = np.take_along_axis(p, ix, axis=1)
    if renorm:
        tot = s.sum(axis=1, keepdims=True)
        w = s / tot
        ds = (gw - np.sum(w * gw, axis=1, keepdims=True)) / tot
    else:
        ds = gw
    g = np.zeros((N, E))
    np.put_along_axis(g, ix, ds, axis=1)
    dL = p * (g - np.sum(p * g, axis=1, keepdims=True))
    if aux_dl is not None:          # the aux loss's own gradient (aux_dlogits)
        dL = dL + aux_dl
    xv = values(x)
    wv = values(w_r)
    return dict(dlogits=dL, dx_r=dL @ wv, dw_r=dL.T @ xv, db_r=dL.sum(axis=0))


# --------------------------------------------------------------------------
# MXFP8: E4M3 elements with one E8M0 scale per 32    [KOSMOS 2.2; OLMo-A A.4, A.5]
# --------------------------------------------------------------------------

E4M3_MAX = 448.0


def floor_log2_f32(a) -> np.ndarray:
    """floor(log2 a) for positive finite fp32 values, read from the bit fields."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    ef = ((bits >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int64)
    man = (bits & np.uint32(0x7FFFFF)).astype(np.int64)
    E = ef - 127
    sub = (ef == 0) & (man > 0)
    if np.any(sub):
        # subnormal: a = man * 2^-149; floor(log2 man) = bit length - 1
        _, bl = np.frexp(man[sub].astype(np.float64))
        E[sub] = -149 + (bl - 1)
    return E


def e4m3_encode(y) -> np.ndarray:
    """float64 -> OCP E4M3FN code: nearest-even on the 3-bit mantissa (subnormal
    spacing 2^-9), magnitudes above 448 saturate to 448, sign kept (-0 -> 0x80)."""
    y = np.asarray(y, dtype=np.float64)
    neg = np.signbit(y)
    a = np.abs(y)
    _, ex = np.frexp(a)
    E = np.maximum(ex - 1, -6)                  # binade; below 2^-6 spacing is 2^-9
    q = np.ldexp(1.0, E - 3)
    r = np.minimum(np.rint(a / q) * q, E4M3_MAX)
    _, ex2 = np.frexp(r)
    E2 = ex2 - 1
    normal = r >= 2.0 ** -6
    man_n = np.where(normal, r / np.ldexp(1.0, np.where(normal, E2, 0)) * 8 - 8, 0)
    code_n = ((E2 + 7) << 3).astype(np.int64) + man_n.astype(np.int64)
    code_s = np.rint(r / 2.0 ** -9).astype(np.int64)
    code = np.where(normal, code_n, code_s)
    code = code | (neg.astype(np.int64) << 7)
    return code.astype(np.uint8)


def e4m3_decode(code) -> np.ndarray:
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = c & 0x7
    v = np.where(ef == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, ef - 7))
    v = np.where((ef == 15) & (m == 7), np.nan, v)
    return s * v


def quantize_mxfp8(v, block: int = 32):
    """Quantize along the last axis in blocks of 32 consecutive elements.

    scale exponent e = clamp(floor(log2 amax) - 8, -127, 127), code e + 127
    (amax = 0 gives code 0); q = E4M3(v * 2^-e).  Returns (q u8 [..., n],
    scale u8 [..., n/32]).
    """
    v = values(v)
    n = v.shape[-1]
    if n % block:
        raise ValueError("length not a multiple of the block")
    blk = v.reshape(v.shape[:-1] + (n // block, block))
    amax = np.abs(blk).max(axis=-1)
    E = floor_log2_f32(np.where(amax > 0, amax, 1.0).astype(np.float32))
    e = np.clip(E - 8, -127, 127)
    e = np.where(amax > 0, e, -127)
    q = e4m3_encode(blk * np.ldexp(1.0, -e)[..., None])
    return q.reshape(v.shape), (e + 127).astype(np.uint8)


def dequantize_mxfp8(q, s, block: int = 32) -> np.ndarray:
    q = np.asarray(q)
    vals = e4m3_decode(q)
    sc = np.ldexp(1.0, np.asarray(s, np.int64) - 127)
    n = q.shape[-1]
    return (vals.reshape(q.shape[:-1] + (n // block, block)) * sc[..., None]).reshape(q.shape)


def mxfp8_gemm(aq, as_, bq, bs) -> np.ndarray:
    """eq. 87 with C = 0: sum over k of (S_A a)(S_B b) in float64 -> bf16.
    a: [M,K] row-quantized along K; b: [N,K] (output-major) quantized along K."""
    return round_bf16(dequantize_mxfp8(aq, as_) @ dequantize_mxfp8(bq, bs).T)


def dispatch_mxfp8(x, row_route, K: int):
    """Quantize-on-dispatch: each token row quantized along D once, its bytes
    and scales written to every row of its routes; other rows q = 0, s = 0."""
    xq, xs = quantize_mxfp8(x)
    rr = np.asarray(row_route, dtype=np.int64)
    q = np.zeros((rr.shape[0], xq.shape[1]), np.uint8)
    s = np.zeros((rr.shape[0], xs.shape[1]), np.uint8)
    live = rr >= 0
    q[live] = xq[rr[live] // K]
    s[live] = xs[rr[live] // K]
    return q, s


def expert_mlp_mxfp8(xq, xs, wgq, wgs, wuq, wus, wdq, wds):
    """GEMM1 on MXFP8 operands, bf16 G/U, H = bf16(silu(G)U) quantized along H,
    GEMM2 on MXFP8 operands -> bf16 Y.  Returns (G, U, H, Hq, Hs, Y)."""
    G = mxfp8_gemm(xq, xs, wgq, wgs)
    U = mxfp8_gemm(xq, xs, wuq, wus)
    Hh = swiglu(G, U)
    hq, hs = quantize_mxfp8(Hh)
    Y = mxfp8_gemm(hq, hs, wdq, wds)
    return G, U, Hh, hq, hs, Y


def layer_fwd_mxfp8(x, w_r, bias, wq, K: int, drop=None, renorm=0, align=32, rows_cap=None, n_shared: int = 0,
                    logits=None):
    """MXFP8 forward: same route as bf16, groups padded to ``align`` rows,
    quantize-on-dispatch, block-scaled expert GEMMs, bf16 weighted combine.

    wq: dict with pre-quantized weights wg_q [E,H,D], wg_s [E,H,D/32], wu_q,
    wu_s, wd_q [E,D,H], wd_s [E,D,H/32] (one more expert, the shared one, with
    n_shared = 1, whose segment holds every token's quantized row).
    ``logits`` may be given to skip the router product, as in layer_fwd.
    """
    xv = values(x)
    N, D = xv.shape
    E = np.asarray(w_r).shape[0]
    if rows_cap is None:
        rows_cap = N * K + E * (align - 1) + n_shared * (N + align - 1)
    L = router_logits(x, w_r, bias) if logits is None else np.asarray(logits, np.float32)
    idx = topk_select(L, K)
    prob = route_probs(L, idx, renorm)
    counts, offsets, dst_rows, row_route = route_map(idx, drop, E, align, rows_cap, n_shared)
    xq, xs = dispatch_mxfp8(xv, row_route, K)
    xd = dispatch(xv, row_route, K)            # the bf16 rows the codes were made from
    if n_shared:
        xq[offsets[E]:offsets[E] + N], xs[offsets[E]:offsets[E] + N] = quantize_mxfp8(xv)
        xd[offsets[E]:offsets[E] + N] = xv
    Hd = wq["wg_q"].shape[1]
    G = np.zeros((rows_cap, Hd))
    U = np.zeros((rows_cap, Hd))
    Hh = np.zeros((rows_cap, Hd))
    hq = np.zeros((rows_cap, Hd), np.uint8)
    hs = np.zeros((rows_cap, Hd // 32), np.uint8)
    Y = np.zeros((rows_cap, D))
    for e in range(E + n_shared):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b == a:
            continue
        G[a:b], U[a:b], Hh[a:b], hq[a:b], hs[a:b], Y[a:b] = expert_mlp_mxfp8(
            xq[a:b], xs[a:b], wq["wg_q"][e], wq["wg_s"][e], wq["wu_q"][e], wq["wu_s"][e],
            wq["wd_q"][e], wq["wd_s"][e])
    out = combine(Y, dst_rows, prob, addend=Y[offsets[E]:offsets[E] + N] if n_shared else None)
    return dict(logits=L, topk_idx=idx, topk_prob=prob, counts=counts, offsets=offsets,
                dst_rows=dst_rows, row_route=row_route, xq=xq, xs=xs, xd=xd, g=G, u=U, h=Hh,
                hq=hq, hs=hs, y=Y, out=out, n_shared=n_shared)


def quantize_weights_mxfp8(w_gate, w_up, w_down):
    """Pre-quantize the expert weights along their contraction dimension
    (D for gate/up stored [E,H,D], H for down stored [E,D,H])."""
    out = {}
    for name, w in (("wg", w_gate), ("wu", w_up), ("wd", w_down)):
        q = np.empty(np.asarray(w).shape, np.uint8)
        s = np.empty(np.asarray(w).shape[:-1] + (np.asarray(w).shape[-1] // 32,), np.uint8)
        for e in range(q.shape[0]):
            q[e], s[e] = quantize_mxfp8(w[e])
        out[name + "_q"], out[name + "_s"] = q, s
    return out


# --------------------------------------------------------------------------
# MXFP8 backward            [KOSMOS 2.2 and 3.3.2; OLMo-A A.13 wgrad policy]
# --------------------------------------------------------------------------


def quantize_weights_mxfp8_dgrad(w_gate, w_up, w_down):
    """The expert weights quantized for the data-gradient GEMMs, whose
    contraction runs over the other dimension of each matrix: each copy is
    quantized from the bf16 weights, never from the forward's copy [KOSMOS 2.2:
    a matrix and its transpose are both quantized from the high-precision
    source; OLMo-A A.13: the right-hand operand prequantized for dgrad].

    wdt_q [E,H,D], wdt_s [E,H,D/32]: W_down[e]^T quantized along D;
    wgut_q [E,D,2H], wgut_s [E,D,2H/32]: [W_gate[e]^T | W_up[e]^T] quantized
    along H (H % 32 == 0, so no block straddles the two halves).
    """
    wg, wu, wd = values(w_gate), values(w_up), values(w_down)
    out = {"wdt_q": [], "wdt_s": [], "wgut_q": [], "wgut_s": []}
    for e in range(wg.shape[0]):
        q, s = quantize_mxfp8(wd[e].T)
        out["wdt_q"].append(q)
        out["wdt_s"].append(s)
        q, s = quantize_mxfp8(np.concatenate([wg[e].T, wu[e].T], axis=1))
        out["wgut_q"].append(q)
        out["wgut_s"].append(s)
    return {k: np.stack(v) for k, v in out.items()}


def quantize_mxfp8_cols(v, offsets):
    """Column-wise MXFP8 copy of a row-segmented matrix v [rows, W]: for each
    expert segment [offsets[e], offsets[e+1]) (lengths multiples of 32), the
    transposed block v[seg].T [W, len] quantized along its rows, i.e. blocks
    of 32 consecutive rows of one column [KOSMOS 2.2: the copy for the product
    that contracts over rows is quantized along rows, from the bf16 source;
    OLMo-A A.15: native MXFP8 grouped wgrad].  Returns {e: (q [W, len],
    s [W, len/32])} for the experts with rows."""
    vv = values(v)
    out = {}
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            if (b - a) % 32:
                raise ValueError("segments must be multiples of 32 rows")
            out[e] = quantize_mxfp8(vv[a:b].T)
    return out


def mx_wgrad(dc, a, offsets):
    """Native MXFP8 weight gradient: dw[e] = bf16(deq(colq(dc_e)) .
    deq(colq(a_e))^T), eq. 87 over the expert's rows with both operands
    quantized column-wise (quantize_mxfp8_cols) from their bf16 values;
    experts without rows get 0.  dc [rows, n], a [rows, k] -> dw [E, n, k]."""
    E = len(offsets) - 1
    qc = quantize_mxfp8_cols(dc, offsets)
    qa = quantize_mxfp8_cols(a, offsets)
    out = np.zeros((E, values(dc).shape[1], values(a).shape[1]))
    for e, (q, s) in qc.items():
        out[e] = round_bf16(dequantize_mxfp8(q, s) @ dequantize_mxfp8(*qa[e]).T)
    return out


def experts_bwd_mxfp8(dyd, xq, xs, g, u, hq, hs, offsets, wqt, wgrad: str = "bf16", xd=None):
    """Expert backward with block-scaled data gradients and bf16 weight
    gradients on dequantized activations.

    dY_d is quantized row-wise along D from its bf16 values [KOSMOS 3.3.2
    step 1: dY arrives in bf16 and is quantized where it lands];
    dH = deq(dY_q) deq(W_down^T q)^T in float64 (it only feeds the SwiGLU
    backward); dG, dU from the SwiGLU backward, stored bf16;
    [dG | dU] quantized row-wise along 2H from those bf16 values;
    dX_d = bf16(deq([dG|dU]_q) deq([W_gate^T|W_up^T]_q)^T), one sum over 2H
    [KOSMOS 3.3.2 steps 2-3; OLMo-A A.13: forward and dgrad on the scaled
    grouped GEMM];
    dW_down = bf16(dY_d^T deq(H_q)), dW_gate = bf16(dG^T deq(X_q)),
    dW_up = bf16(dU^T deq(X_q)) [OLMo-A A.13: wgrad dequantizes its operands
    and runs a bf16 grouped GEMM].
    hq = None is the SwiGLU-recompute mode [OLMo-A A.14: H rebuilt in the
    backward instead of saved]: dW_down takes H = bf16(silu(G) U) from the
    saved bf16 G and U in place of deq(H_q).
    wgrad = "mx": the native MXFP8 weight gradients instead [OLMo-A A.15;
    KOSMOS 3.3.1 step 3 and 3.3.2 step 1: column-wise copies quantized from
    the bf16 sources]: dW_down = mx_wgrad(dY_d, H), dW_gate = mx_wgrad(dG,
    X_d), dW_up = mx_wgrad(dU, X_d), with H = bf16(silu(G) U) and X_d the
    bf16 dispatched rows (``xd``), not the dequantized codes.
    """
    dy = values(dyd)
    rows, D = dy.shape
    E = len(offsets) - 1
    Hd = np.asarray(g).shape[1]
    dyq, dys = quantize_mxfp8(dy)
    dy_deq = dequantize_mxfp8(dyq, dys)
    x_deq = dequantize_mxfp8(xq, xs)
    h_deq = swiglu(g, u) if hq is None else dequantize_mxfp8(hq, hs)
    dG = np.zeros((rows, Hd))
    dU = np.zeros((rows, Hd))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b == a:
            continue
        wdt = dequantize_mxfp8(wqt["wdt_q"][e], wqt["wdt_s"][e])          # [H, D]
        dg_e, du_e = swiglu_bwd(dy_deq[a:b] @ wdt.T, np.asarray(g[a:b], np.float64),
                                np.asarray(u[a:b], np.float64))
        dG[a:b] = round_bf16(dg_e)
        dU[a:b] = round_bf16(du_e)
    guq, gus = quantize_mxfp8(np.concatenate([dG, dU], axis=1))
    gu_deq = dequantize_mxfp8(guq, gus)
    dXd = np.zeros((rows, D))
    dWg = np.zeros((E, Hd, D))
    dWu = np.zeros((E, Hd, D))
    dWd = np.zeros((E, D, Hd))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b == a:
            continue
        wgut = dequantize_mxfp8(wqt["wgut_q"][e], wqt["wgut_s"][e])        # [D, 2H]
        dXd[a:b] = round_bf16(gu_deq[a:b] @ wgut.T)
        if wgrad == "bf16":
            dWd[e] = round_bf16(dy[a:b].T @ h_deq[a:b])
            dWg[e] = round_bf16(dG[a:b].T @ x_deq[a:b])
            dWu[e] = round_bf16(dU[a:b].T @ x_deq[a:b])
    if wgrad == "mx":
        if xd is None:
            raise ValueError("the native MXFP8 wgrad takes the bf16 dispatched rows")
        dWd = mx_wgrad(dy, swiglu(g, u), offsets)
        dWg = mx_wgrad(dG, xd, offsets)
        dWu = mx_wgrad(dU, xd, offsets)
    elif wgrad != "bf16":
        raise ValueError("wgrad is 'bf16' or 'mx'")
    return dict(dg=dG, du=dU, dxd=dXd, dw_gate=dWg, dw_up=dWu, dw_down=dWd,
                dyq=dyq, dys=dys, guq=guq, gus=gus)


def layer_bwd_mxfp8(fwd: dict, dout, wqt, recompute: bool = False, wgrad: str = "bf16"):
    """MXFP8 layer backward: the bf16 adjoint sequence around the experts
    (weighted dY dispatch, route-weight gradient, fold of the K rows) with
    experts_bwd_mxfp8 in the middle.  fwd is layer_fwd_mxfp8's result; wqt
    comes from quantize_weights_mxfp8_dgrad.  recompute: the saved H codes are
    not read (SwiGLU-recompute mode).  wgrad = "mx": native MXFP8 weight
    gradients (experts_bwd_mxfp8)."""
    hq = None if recompute else fwd["hq"]
    return _layer_bwd_around(
        fwd, dout, lambda dyd: experts_bwd_mxfp8(dyd, fwd["xq"], fwd["xs"], fwd["g"], fwd["u"], hq,
                                                 fwd["hs"], fwd["offsets"], wqt, wgrad, fwd.get("xd")))

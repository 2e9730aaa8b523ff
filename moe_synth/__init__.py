"""Seeded synthetic inputs for the routed MoE expert layer.

This module is shared by the CPU oracle, the tests and the benchmark.  It only
draws random numbers and stores them as bf16 bit patterns; it holds none of the
layer's arithmetic.  No dataset or trained weight is involved: the shapes are the
five workloads below and the values follow the init scheme they state.

Recipe (one independent PCG64 stream per (seed, tensor, expert) so that experts
can be drawn in parallel threads and any subset can be regenerated alone):

* ``x``      [N, D]    ~ N(0, 1)
* ``w_r``    [E, D]    ~ N(0, 1/D)       router weight, stored expert-major
* ``w_gate`` [E, H, D] ~ N(0, 1/D)       stored [expert][out][in] (in contiguous)
* ``w_up``   [E, H, D] ~ N(0, 1/D)
* ``w_down`` [E, D, H] ~ N(0, 1/H)
* ``bias``   [E] fp32 = -s * ln(rank_e), rank = 1 + a seeded permutation of 0..E-1
  (only for workloads with a Zipf exponent s; none otherwise)
* ``drop``   [N, K] u8 Bernoulli(p_drop) (only where p_drop > 0)
* ``dout``   [N, D]    ~ N(0, 1)         upstream gradient of the layer output

Normals are drawn in fp32 and rounded to nearest-even bf16.  The weights are
i.i.d., so drawing them directly in storage layout has the same distribution as
drawing the logical [E, D, H] tensor and transposing it.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field, asdict
from typing import Optional

import numpy as np

# tensor ids for the per-tensor streams
_T_X, _T_WR, _T_WG, _T_WU, _T_WD, _T_PERM, _T_DROP, _T_DOUT = range(8)


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    D: int
    E: int
    K: int
    H: int
    zipf_s: Optional[float] = None   # Zipf exponent of the expert bias (None = no bias)
    p_drop: float = 0.0              # fraction of routes marked invalid
    mxfp8: bool = False              # MXFP8 expert GEMMs (groups padded to 32 rows)
    bwd: bool = False                # workload includes the backward pass
    renorm: int = 0

    @property
    def align(self) -> int:
        return 32 if self.mxfp8 else 1

    @property
    def rows_cap(self) -> int:
        return self.N * self.K + self.E * (self.align - 1)

    def as_dict(self):
        d = asdict(self)
        d["align"] = self.align
        d["rows_cap"] = self.rows_cap
        return d


WORKLOADS = {
    "tiny_bf16": Workload("tiny_bf16", N=256, D=128, E=8, K=2, H=256),
    "mixtral_bf16": Workload("mixtral_bf16", N=8192, D=4096, E=8, K=2, H=14336),
    "dsv3_bf16": Workload("dsv3_bf16", N=4096, D=7168, E=256, K=8, H=2048, zipf_s=1.1),
    "qwen3_235b_bf16_fwdbwd": Workload("qwen3_235b_bf16_fwdbwd", N=16384, D=4096, E=128, K=8,
                                       H=1536, zipf_s=1.2, p_drop=0.05, bwd=True),
    "dsv3_mxfp8": Workload("dsv3_mxfp8", N=4096, D=7168, E=256, K=8, H=2048, zipf_s=1.1,
                           mxfp8=True),
}


def scaled(w: Workload, name: str = None, **kw) -> Workload:
    """Same workload structure at other sizes (small parity and edge cases)."""
    d = {k: getattr(w, k) for k in ("N", "D", "E", "K", "H", "zipf_s", "p_drop", "mxfp8",
                                     "bwd", "renorm")}
    d.update(kw)
    return Workload(name or (w.name + "_scaled"), **d)


def _rng(seed: int, tensor: int, expert: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor, expert])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    u = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(g: np.random.Generator, shape, std: float) -> np.ndarray:
    v = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return f32_to_bf16_bits(v)


@dataclass
class Inputs:
    wl: Workload
    seed: int
    x: np.ndarray                    # u16 [N, D]
    w_r: np.ndarray                  # u16 [E, D]
    bias: Optional[np.ndarray]       # f32 [E]
    drop: Optional[np.ndarray]       # u8 [N, K]
    dout: Optional[np.ndarray]       # u16 [N, D]
    w_gate: Optional[np.ndarray] = None   # u16 [E, H, D]
    w_up: Optional[np.ndarray] = None     # u16 [E, H, D]
    w_down: Optional[np.ndarray] = None   # u16 [E, D, H]
    extra: dict = field(default_factory=dict)


def expert_weights(wl: Workload, seed: int, e: int):
    """(w_gate[e] [H,D], w_up[e] [H,D], w_down[e] [D,H]) as bf16 bits."""
    sd = 1.0 / np.sqrt(wl.D)
    sh = 1.0 / np.sqrt(wl.H)
    wg = _normal_bf16(_rng(seed, _T_WG, e), (wl.H, wl.D), sd)
    wu = _normal_bf16(_rng(seed, _T_WU, e), (wl.H, wl.D), sd)
    wd = _normal_bf16(_rng(seed, _T_WD, e), (wl.D, wl.H), sh)
    return wg, wu, wd


def zipf_bias(wl: Workload, seed: int) -> Optional[np.ndarray]:
    if wl.zipf_s is None:
        return None
    perm = _rng(seed, _T_PERM).permutation(wl.E)
    rank = 1.0 + perm.astype(np.float64)
    return (-wl.zipf_s * np.log(rank)).astype(np.float32)


def make_inputs(wl: Workload, seed: int = 0, weights: bool = True, threads: int = None,
                weight_out=None) -> Inputs:
    """Draw every input of the workload.

    ``weight_out`` (optional) is a tuple of preallocated u16 arrays
    (w_gate [E,H,D], w_up [E,H,D], w_down [E,D,H]) to fill in place, so that a
    caller may put them in pinned memory.
    """
    N, D, E, K, H = wl.N, wl.D, wl.E, wl.K, wl.H
    x = _normal_bf16(_rng(seed, _T_X), (N, D), 1.0)
    w_r = _normal_bf16(_rng(seed, _T_WR), (E, D), 1.0 / np.sqrt(D))
    bias = zipf_bias(wl, seed)
    drop = None
    if wl.p_drop > 0:
        drop = (_rng(seed, _T_DROP).random((N, K)) < wl.p_drop).astype(np.uint8)
    dout = _normal_bf16(_rng(seed, _T_DOUT), (N, D), 1.0) if wl.bwd else None
    inp = Inputs(wl, seed, x, w_r, bias, drop, dout)
    if weights:
        if weight_out is None:
            wg = np.empty((E, H, D), np.uint16)
            wu = np.empty((E, H, D), np.uint16)
            wd = np.empty((E, D, H), np.uint16)
        else:
            wg, wu, wd = weight_out

        def one(e):
            a, b, c = expert_weights(wl, seed, e)
            wg[e], wu[e], wd[e] = a, b, c

        nthr = threads or min(16, os.cpu_count() or 1)
        if nthr > 1 and E > 1:
            with _cf.ThreadPoolExecutor(nthr) as ex:
                list(ex.map(one, range(E)))
        else:
            for e in range(E):
                one(e)
        inp.w_gate, inp.w_up, inp.w_down = wg, wu, wd
    return inp


def random_logits(N: int, E: int, seed: int, scale: float = 1.0) -> np.ndarray:
    """Standalone fp32 router logits for route-map tests (same law as x.W_r)."""
    return (np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99])))
            .standard_normal((N, E), dtype=np.float32) * np.float32(scale))


def random_bf16(shape, seed: int, tag: int, std: float = 1.0) -> np.ndarray:
    """Extra seeded bf16 tensors (e.g. expert outputs fed straight to combine)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1000 + tag])))
    return _normal_bf16(g, shape, std)


def random_f32(shape, seed: int, tag: int, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 2000 + tag])))
    return (g.random(shape, dtype=np.float32) * np.float32(hi - lo) + np.float32(lo)).astype(np.float32)

"""Host-side accounting of bench.py pinned to numbers the pages print."""
import os

import numpy as np
import pytest

import bench

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    for line in open(os.path.join(GOLD, name)):
        if line.strip() and not line.startswith("#"):
            out.append(line.split())
    return out


def test_routed_flop_convention_reproduces_kosmos_tables():
    """TFLOPS = 6 T K d h (forward) or 12 T K d h (backward) / time, T = 8192."""
    rows = _rows("kosmos_moe_tflops.txt")
    assert len(rows) == 7
    for model, routing, direction, d, h, k, ms, tf in rows:
        R = 8192 * int(k)
        F = bench.routed_flops(R, int(d), int(h), backward=(direction == "bwd"))
        got = F / (float(ms) * 1e-3) / 1e12
        # the table prints ms to 3 decimals and TFLOPS to 1
        tol = got * 0.0005 / float(ms) + 0.05
        assert abs(got - float(tf)) <= tol, (model, direction, got, tf)


def test_imax_worked_example():
    g = dict((r[0], r[1]) for r in _rows("olmo_a9_imax.txt"))
    E, R, align = int(g["experts"]), int(g["rows"]), int(g["align"])
    spike = round(float(g["spike_fraction"]) * R)
    single = np.zeros(E, np.int64)
    single[0] = spike
    single[1:] = (R - spike) // (E - 1)
    single[1: 1 + (R - spike) % (E - 1)] += 1
    three = np.zeros(E, np.int64)
    three[[0, 5, 10]] = spike
    rest = R - 3 * spike
    others = [i for i in range(E) if i not in (0, 5, 10)]
    three[others] = rest // len(others)
    three[others[: rest % len(others)]] += 1
    assert single.sum() == R == three.sum()
    assert three[[0, 5, 10]].sum() / R == pytest.approx(float(g["three_hot_total_fraction"]), abs=0.005)
    a = bench.load_stats(single, align)["I_max"]
    b = bench.load_stats(three, align)["I_max"]
    tol = float(g["imax_tolerance"])
    assert a == pytest.approx(float(g["imax"]), abs=tol)
    assert b == pytest.approx(float(g["imax"]), abs=tol)
    # same I_max, different histograms: the top-3 share tells them apart
    assert bench.load_stats(three, align)["top3_share"] > 0.9 > bench.load_stats(single, align)["top3_share"]


def test_roofline_accounting_matches_table_43():
    """eq. 93 per-GEMM bytes for balanced routing with every expert used equal
    the GEMM1/GEMM2 byte counts here when G/U/H stores are counted as in
    Table 43 (up/gate writes + down input reads = 6 T K h)."""
    T, K, N, d, h = 4096, 4, 64, 4096, 4096
    R = T * K
    F1, Q1 = bench.gemm1_work(R, d, h, N)
    F2, Q2 = bench.gemm2_work(R, d, h, N)
    assert F1 + F2 == 6 * T * K * d * h                      # eq. 92
    q_up = 2 * (T * K * d + 2 * N * d * h + 2 * T * K * h)   # eq. 93, MoE up
    q_down = 2 * (T * K * h + N * h * d + T * K * d)         # eq. 93, MoE down
    # GEMM1 here also stores H (2 R h bytes) besides G and U
    assert Q1 == q_up + 2 * R * h
    assert Q2 == q_down
    assert bench.t_star(1e12, 8e9, 2500.0) == pytest.approx(max(1e12 / 2.5e15, 8e9 / 8e12))


def test_bench_refuses_multi_gpu(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err

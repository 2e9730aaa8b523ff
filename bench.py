"""Benchmark of one GPU's routed MoE expert layer on MI355X.

One step = one forward pass of the whole layer over one batch of seeded
synthetic input: router logits -> softmax/top-K/route map -> dispatch ->
GEMM1 (gate/up, SwiGLU) -> GEMM2 (down) -> weighted combine.  The default
workload is the DeepSeek-V3-shaped layer (N=4096 tokens, D=7168, E=256 experts,
top-8, H=2048, Zipf(1.1) expert bias), bf16 with fp32 accumulation.  Inputs are
resident in HBM before the timed region starts.

Prints ONE JSON line (rank 0).  Usage:
  python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload dsv3_bf16]
"""
from __future__ import annotations

import argparse
import csv
import ctypes as C
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import moe_synth as S  # noqa: E402

METRIC = "MoE layer fwd tokens/s; grouped-GEMM TFLOP/s (% MFMA peak); dispatch GB/s"

PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "mixture_experts_expert_router_amd", "csrc")
# sources of the persistent grouped GEMM: HBM counters taken on another
# version of these no longer describe the kernel
GEMM_SOURCES = ("gemm_fwd.hip", "mfma_tile.h", "common.h", "sched.h")

# MI355X published peaks (dense)
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_MXFP8_TFLOPS = 5000.0


# ---------------------------------------------------------------------------
# accounting (algorithmic work; OLMo-core Appendix A, A.8 eqs. 89-94 and
# Table 43; routed FLOPs as in KOSMOS section 4.1.1)
# ---------------------------------------------------------------------------

def routed_flops(R, D, H, backward=False):
    """Useful expert FLOPs: 6 R D H forward (eq. 92), 12 R D H backward."""
    return (12 if backward else 6) * R * D * H


def gemm1_work(R, D, H, E_act, b=2.0):
    """GEMM1 with SwiGLU: F = 4RDH; bytes = X_d read + gate/up weights of the
    active experts + G, U written (bf16) + H written (b bytes per element)."""
    F = 4 * R * D * H
    Q = b * R * D + b * 2 * E_act * D * H + 4 * R * H + b * R * H
    return F, Q


def gemm2_work(R, D, H, E_act, b=2.0):
    F = 2 * R * D * H
    Q = b * R * H + b * E_act * H * D + 2 * R * D
    return F, Q


def dispatch_bytes(N, D, K, R, b=2.0, pad_rows=0):
    """Each token row read once and written to each of its valid routes; with
    32-row groups (MXFP8) the padding rows of each group are part of the
    output (zero codes and scales) and are written too."""
    return 2 * N * D + b * (R + pad_rows) * D + 4 * N * K


def combine_bytes(N, D, K, R):
    return 2 * R * D + 8 * N * K + 2 * N * D


def router_work(N, D, E):
    return 2 * N * D * E, 2 * N * D + 2 * D * E + 4 * N * E


def t_star(F, Q, peak_tflops, peak_gbs=PEAK_HBM_GBS):
    """Roofline lower bound (eq. 89): max(F / C, Q / B) in seconds."""
    return max(F / (peak_tflops * 1e12), Q / (peak_gbs * 1e9))


# ---------------------------------------------------------------------------
# HBM traffic from rocprofv3 counters
# ---------------------------------------------------------------------------

def gemm_source_hash():
    """Hash of the GEMM kernel sources with comments and blank space taken
    out, so that a change of wording alone keeps recorded counters valid."""
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _pmc_per_dispatch(run_dir, counter):
    """{dispatch id: (kernel name, summed counter value in KiB)} from one
    rocprofv3 --pmc CSV run (values are summed over the counter's instances)."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    out = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                k = (f, r["Dispatch_Id"])
                name, v = out.get(k, (r["Kernel_Name"], 0.0))
                out[k] = (name, v + float(r["Counter_Value"]))
    return out


def pmc_report(fetch_dir, write_dir, copy_mib, workload):
    """Traffic per kernel from a FETCH_SIZE run and a WRITE_SIZE run of
    `bench.py --copy-probe copy_mib`: each counter is scaled by what it reads
    for the plain device copy of copy_mib MiB in the same run."""
    fetch = _pmc_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_dispatch(write_dir, "WRITE_SIZE")
    copy_bytes = copy_mib * 1024.0 * 1024.0

    def copy_kib(d):
        vals = [v for (n, v) in d.values() if "copyBuffer" in n]
        if not vals:
            raise RuntimeError("no device copy kernel in the counter run (use --copy-probe)")
        return max(vals)

    f_fetch = copy_bytes / (copy_kib(fetch) * 1024.0)
    f_write = copy_bytes / (copy_kib(write) * 1024.0)

    def per_kernel(d):
        agg = {}
        for n, v in d.values():
            agg.setdefault(n, []).append(v)
        return {n: float(np.mean(v)) for n, v in agg.items()}

    fk, wk = per_kernel(fetch), per_kernel(write)
    rows = []
    for n in sorted(set(fk) | set(wk), key=lambda n: -(fk.get(n, 0) * f_fetch + wk.get(n, 0) * f_write)):
        rb = fk.get(n, 0.0) * 1024 * f_fetch
        wb = wk.get(n, 0.0) * 1024 * f_write
        rows.append(dict(kernel=n, fetch_kib=fk.get(n), write_kib=wk.get(n), read_bytes=rb, write_bytes=wb,
                         traffic_bytes=rb + wb))
    gemm1 = [r for r in rows if re.search(r"gemm_fwd_kernel<true", r["kernel"])]
    summary = dict(workload=workload, fetch_factor=f_fetch, write_factor=f_write,
                   gemm_source_hash=gemm_source_hash(),
                   gemm1_kernel=gemm1[0]["kernel"] if gemm1 else None,
                   gemm1_traffic_bytes=gemm1[0]["traffic_bytes"] if gemm1 else None)
    return summary, rows


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                 "SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_INSTS_VALU_MFMA_MOPS_F6F4")


def mfma_report(run_dir, cus=256, xcds=8):
    """MFMA utilisation per GEMM kernel from one rocprofv3 --pmc run with
    MFMA_COUNTERS.  rocprofv3 reports each counter summed over its instances:
    GRBM_GUI_ACTIVE over the xcds XCDs, the SQ counters over every SIMD.  So
    busy share = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / xcds * cus * 4
    SIMDs), and the clock the kernel ran at = GRBM_GUI_ACTIVE / xcds / duration.
    Achieved FLOP/s = 512 FLOP per MFMA MOP over the dispatch's duration.
    Averaged over each kernel's dispatches; durations are the counted runs' own."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    disp = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                d = disp.setdefault((f, r["Dispatch_Id"]), {"name": r["Kernel_Name"], "ns": int(r["End_Timestamp"]) -
                                                              int(r["Start_Timestamp"])})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    per = {}
    for d in disp.values():
        if "gemm" not in d["name"] or not d.get("GRBM_GUI_ACTIVE"):
            continue
        gui = d["GRBM_GUI_ACTIVE"] / xcds
        busy = d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (gui * cus * 4)
        ghz = gui / d["ns"]
        mops_bf = d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
        mops_f8 = d.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0) + d.get("SQ_INSTS_VALU_MFMA_MOPS_F6F4", 0.0)
        s_ = d["ns"] * 1e-9
        per.setdefault(d["name"], []).append((busy, 512 * mops_bf / s_ / 1e12, 512 * mops_f8 / s_ / 1e12, d["ns"], ghz))
    rows = []
    for name, v in per.items():
        n = len(v)
        busy, tf_bf, tf_f8, ns, ghz = (sum(x[i] for x in v) / n for i in range(5))
        mx = tf_f8 > tf_bf
        peak = PEAK_MXFP8_TFLOPS if mx else PEAK_BF16_TFLOPS
        rows.append(dict(kernel=name, dispatches=n, busy_pct=100 * busy, tflops=tf_f8 if mx else tf_bf,
                         pct_peak=100 * (tf_f8 if mx else tf_bf) / peak, dtype="mxfp8" if mx else "bf16",
                         us=ns / 1e3, ghz=ghz))
    rows.sort(key=lambda r: -r["us"] * r["dispatches"])
    return rows


STALL_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_LDS",
                  "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_VMEM", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")


def stall_report(run_dir, cus=256, xcds=8):
    """Where the GEMM kernels' waves spend their cycles, from one rocprofv3
    --pmc run with STALL_COUNTERS.  SQ_WAVE_CYCLES, SQ_WAIT_ANY (waiting on a
    dependency: s_waitcnt or a barrier), SQ_WAIT_INST_ANY (ready but not
    issued), SQ_WAIT_INST_LDS and the SQ_ACTIVE_INST_* counters share one unit
    (wave quad-cycles), so each is reported as a share of SQ_WAVE_CYCLES; the
    shares overlap and need not sum to 100.  MFMA busy is per SIMD, as in
    mfma_report.  Averaged over each kernel's dispatches."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    disp = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                d = disp.setdefault((f, r["Dispatch_Id"]), {"name": r["Kernel_Name"], "ns": int(r["End_Timestamp"]) -
                                                              int(r["Start_Timestamp"])})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    keys = ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS",
            "SQ_ACTIVE_INST_VMEM")
    per = {}
    for d in disp.values():
        wc = d.get("SQ_WAVE_CYCLES", 0.0)
        if "gemm" not in d["name"] or not wc or not d.get("GRBM_GUI_ACTIVE"):
            continue
        gui = d["GRBM_GUI_ACTIVE"] / xcds
        v = [100.0 * d.get(k, 0.0) / wc for k in keys]
        v.append(100.0 * d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (gui * cus * 4))
        v.append(d["ns"] / 1e3)
        per.setdefault(d["name"], []).append(v)
    rows = []
    for name, vs in per.items():
        n = len(vs)
        m = [sum(x[i] for x in vs) / n for i in range(len(vs[0]))]
        rows.append(dict(kernel=name, dispatches=n, wait_dep=m[0], wait_issue=m[1], active=m[2], lds_active=m[3],
                         lds_issue_wait=m[4], vmem_active=m[5], mfma_busy=m[6], us=m[7]))
    rows.sort(key=lambda r: -r["us"] * r["dispatches"])
    return rows


def recorded_traffic(workload, seed=0):
    """Bytes per launch of GEMM1 from the committed counter summary of this
    workload, or None when there is none, the GEMM sources changed since, or
    the inputs differ (the counters were taken at seed 0)."""
    if seed != 0:
        return None
    path = os.path.join(PROFILES, f"gemm1_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        m = re.search(r"```json\n(.*?)\n```", fh.read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("gemm_source_hash") != gemm_source_hash() or rec.get("workload") != workload:
        return None
    return rec.get("gemm1_traffic_bytes")


def load_stats(counts, align=1):
    """Expert-load statistics: I_max = the largest aligned expert load over the
    mean rows per expert (OLMo-core Appendix A, A.9), active and empty
    experts, the top-3 share of rows."""
    c = np.asarray(counts, dtype=np.int64)
    a = ((c + align - 1) // align) * align
    tot = c.sum()
    srt = np.sort(c)[::-1]
    return dict(I_max=float(a.max() / (tot / len(c))) if tot else 0.0,
                active=int((c > 0).sum()), empty=int((c == 0).sum()), max_rows=int(c.max()),
                top3_share=float(srt[:3].sum() / max(1, c.sum())))


# ---------------------------------------------------------------------------
# the staged forward (same kernels as moe_layer_fwd, one C-ABI call per stage)
# ---------------------------------------------------------------------------

class StagedForward:
    STAGES = ("router", "route", "dispatch", "gemm1", "gemm2", "combine")

    def __init__(self, M, layer, x):
        import torch
        self.M, self.layer, self.x = M, layer, x
        lib = M.load()
        self.lib = lib
        d = layer.d
        sv = layer.saved
        self.d = d
        P = M._ptr
        self.mx = layer.mxfp8
        wts = layer.wts
        rc = M.rows_cap(d)
        self.ws_route = M.workspace(M.MOE_OP_ROUTE, d)
        self.ws_router = M.workspace(M.MOE_OP_ROUTER, d)
        self.ws_gemm = M._gemm_ws(rc, d.E, x.device)
        q = wts.wq or {}
        dtype = M.MOE_MXFP8 if self.mx else M.MOE_BF16
        if self.mx:
            self.g1 = M.GemmFwdArgs(dtype, M.MOE_EPI_SWIGLU, d.E, rc, d.D, d.H, P(sv["offsets"]),
                                    P(sv["xd_q"]), P(sv["xd_s"]), P(q["wg_q"]), P(q["wg_s"]),
                                    P(q["wu_q"]), P(q["wu_s"]), P(sv["g"]), P(sv["u"]), P(sv.get("h")),
                                    P(sv["h_q"]), P(sv["h_s"]))
            self.g2 = M.GemmFwdArgs(dtype, M.MOE_EPI_NONE, d.E, rc, d.H, d.D, P(sv["offsets"]),
                                    P(sv["h_q"]), P(sv["h_s"]), P(q["wd_q"]), P(q["wd_s"]), None, None,
                                    P(sv["y"]), None, None, None, None)
        else:
            self.g1 = M.GemmFwdArgs(dtype, M.MOE_EPI_SWIGLU, d.E, rc, d.D, d.H, P(sv["offsets"]),
                                    P(sv["xd"]), None, P(wts.w_gate), None, P(wts.w_up), None,
                                    P(sv["g"]), P(sv["u"]), P(sv["h"]), None, None)
            self.g2 = M.GemmFwdArgs(dtype, M.MOE_EPI_NONE, d.E, rc, d.H, d.D, P(sv["offsets"]),
                                    P(sv["h"]), None, P(wts.w_down), None, None, None, P(sv["y"]),
                                    None, None, None, None)
        self.ev = None

    def run(self, events=None):
        M, lib, d, sv, P = self.M, self.lib, self.d, self.layer.saved, self.M._ptr
        s = M._stream()
        chk = M._check
        wts = self.layer.wts

        def mark(i):
            if events is not None:
                events[i].record()

        mark(0)
        chk(lib.moe_router_logits(P(self.x), P(wts.w_r), P(wts.bias), C.byref(d), P(sv["logits"]),
                                  P(self.ws_router), self.ws_router.numel(), s), "router")
        mark(1)
        chk(lib.moe_route(P(sv["logits"]), P(self.layer.drop), C.byref(d), P(sv["topk_idx"]),
                          P(sv["topk_prob"]), P(sv["counts"]), P(sv["offsets"]), P(sv["dst_rows"]),
                          P(sv["row_route"]), P(self.ws_route), self.ws_route.numel(), s), "route")
        mark(2)
        if self.mx:
            chk(lib.moe_dispatch(P(self.x), P(sv["dst_rows"]), None, P(sv["counts"]), P(sv["offsets"]),
                                 C.byref(d), M.MOE_MXFP8, P(sv["xd_q"]), P(sv["xd_s"]), s), "dispatch")
        else:
            chk(lib.moe_dispatch(P(self.x), P(sv["dst_rows"]), None, P(sv["counts"]), P(sv["offsets"]),
                                 C.byref(d), M.MOE_BF16, P(sv["xd"]), None, s), "dispatch")
        mark(3)
        chk(lib.moe_grouped_gemm_fwd(C.byref(self.g1), P(self.ws_gemm), self.ws_gemm.numel(), s), "gemm1")
        mark(4)
        chk(lib.moe_grouped_gemm_fwd(C.byref(self.g2), P(self.ws_gemm), self.ws_gemm.numel(), s), "gemm2")
        mark(5)
        chk(lib.moe_combine(P(sv["y"]), P(sv["dst_rows"]), P(sv["topk_prob"]), C.byref(d),
                            P(self.layer.out), s), "combine")
        mark(6)


def device_inputs(M, inp, mxfp8, torch, backward=False):
    def b(u):
        return torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).view(torch.bfloat16).cuda()

    w = M.LayerWeights(w_r=b(inp.w_r), bias=torch.from_numpy(inp.bias).cuda() if inp.bias is not None else None)
    if mxfp8:
        wg, wu, wd = b(inp.w_gate), b(inp.w_up), b(inp.w_down)
        w.wq = M.quantize_weights_mxfp8(wg, wu, wd)
        if backward:
            # the data gradients' weight copies, quantized along the other dimension
            w.wq.update(M.quantize_weights_mxfp8_dgrad(wg, wu, wd))
        torch.cuda.synchronize()
        del wg, wu, wd
    else:
        w.w_gate, w.w_up, w.w_down = b(inp.w_gate), b(inp.w_up), b(inp.w_down)
    drop = torch.from_numpy(inp.drop).cuda() if inp.drop is not None else None
    return b(inp.x), w, drop


def shared_expert_weights(M, w, wl, seed, torch):
    """The workload's expert weights plus one shared expert, the last, drawn like
    the others (N(0, 1/D) for gate/up, N(0, 1/H) for down)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 7919)
    D, H = wl.D, wl.H
    ws = M.LayerWeights(w_r=w.w_r, bias=w.bias)
    mk = lambda *shape, std: (torch.randn(shape, device="cuda", generator=g) * std).bfloat16()
    sg, su, sd = mk(1, H, D, std=D ** -0.5), mk(1, H, D, std=D ** -0.5), mk(1, D, H, std=H ** -0.5)
    if w.wq:
        q = M.quantize_weights_mxfp8(sg, su, sd)
        if "wdt_q" in w.wq:
            q.update(M.quantize_weights_mxfp8_dgrad(sg, su, sd))
        ws.wq = {k: torch.cat([w.wq[k], q[k]]) for k in w.wq}
    else:
        ws.w_gate, ws.w_up, ws.w_down = (torch.cat([a, b]) for a, b in ((w.w_gate, sg), (w.w_up, su), (w.w_down, sd)))
    return ws


def cpu_baseline(inp, wl, budget_s=20.0):
    """The oracle as it stands, on the first tokens of the same workload (a
    bounded sample); returns tokens/s on the host cores."""
    import oracle as O
    n = 4
    t_used = 0.0
    res = None
    while True:
        t0 = time.perf_counter()
        drop = inp.drop[:n] if inp.drop is not None else None
        if wl.mxfp8:
            wq = _sample_mxfp8_weights(O, inp, wl, n, drop)     # setup, not timed
            t0 = time.perf_counter()
            O.layer_fwd_mxfp8(inp.x[:n], inp.w_r, inp.bias, wq, wl.K, drop=drop)
        else:
            O.layer_fwd(inp.x[:n], inp.w_r, inp.bias, inp.w_gate, inp.w_up, inp.w_down, wl.K, drop=drop)
        dt = time.perf_counter() - t0
        res = (n, dt)
        t_used += dt
        if dt > budget_s / 2 or n >= wl.N or t_used > 2 * budget_s:
            break
        n = min(wl.N, n * 2)
    n, dt = res
    return dict(value=n / dt, unit="tokens/s", cores=_host_threads(), kind="oracle",
                sample=f"first {n} of {wl.N} tokens of the same workload, full expert weights, "
                       f"numpy float64 ({dt:.1f} s)",
                host_cpus=os.cpu_count(), cpu_model=_cpu_model(),
                note="cores = the BLAS threads the oracle ran on; host_cpus = os.cpu_count()")


def _sample_mxfp8_weights(O, inp, wl, n, drop):
    """Pre-quantized weights (the untimed setup step) for the experts the
    sample routes to; the others stay zero and are never read."""
    L = O.router_logits(inp.x[:n], inp.w_r, inp.bias)
    idx = O.topk_select(L, wl.K)
    used = np.unique(idx[O.route_valid(idx, drop, wl.E)])
    E, H, D = wl.E, wl.H, wl.D
    wq = dict(wg_q=np.zeros((E, H, D), np.uint8), wg_s=np.zeros((E, H, D // 32), np.uint8),
              wu_q=np.zeros((E, H, D), np.uint8), wu_s=np.zeros((E, H, D // 32), np.uint8),
              wd_q=np.zeros((E, D, H), np.uint8), wd_s=np.zeros((E, D, H // 32), np.uint8))
    for e in used:
        for name, w in (("wg", inp.w_gate), ("wu", inp.w_up), ("wd", inp.w_down)):
            wq[name + "_q"][e], wq[name + "_s"][e] = O.quantize_mxfp8(w[e])
    return wq


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _host_threads():
    try:
        from threadpoolctl import threadpool_info
        th = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        if th:
            return int(max(th))
    except Exception:
        pass
    return os.cpu_count() or 1


# the workloads measured after the headline in the same run (their step
# times, GEMM rates and permute bandwidths; the tiny case is a parity case)
EXTRA_WORKLOADS = ("mixtral_bf16", "qwen3_235b_bf16_fwdbwd", "dsv3_mxfp8")


def single_launch_ok(wl, bwd):
    """The single-launch layer's rules (bf16 routed experts; the tiled router,
    16 <= E <= 512; D, H multiples of 64; with the router backward E % 64)."""
    return (not wl.mxfp8 and 16 <= wl.E <= 512 and wl.D % 64 == 0 and wl.H % 64 == 0 and wl.K <= 32
            and (not bwd or wl.E % 64 == 0))


def ready_queue_ok(wl):
    """The readiness-gated launch's rules (routed experts; bf16 with D and H
    multiples of 64, MXFP8 with D and H multiples of 128)."""
    m = 128 if wl.mxfp8 else 64
    return wl.D % m == 0 and wl.H % m == 0


def measure(M, torch, wl, inp, steps, warmup, seed, backward=False, layer_call=False, shared_expert=False,
            mx_wgrad=False, single=False):
    """Time `steps` steps of one workload (after `warmup`), inputs resident in
    HBM; returns the result dict of the JSON line (without cpu_baseline)."""
    bwd = wl.bwd or backward
    t0 = time.perf_counter()
    x, w, drop = device_inputs(M, inp, wl.mxfp8, torch, backward=bwd)
    layer = M.MoeLayer(w, wl.N, wl.K, mxfp8=wl.mxfp8, drop=drop, renorm=wl.renorm, with_bwd=bwd,
                       router_bwd=bwd, mx_wgrad=mx_wgrad)
    dout_bits = inp.dout if inp.dout is not None else (S.random_bf16((wl.N, wl.D), seed, 9) if bwd else None)
    dout = (torch.from_numpy(np.ascontiguousarray(dout_bits).view(np.int16)).view(torch.bfloat16).cuda()
            if bwd else None)
    st = StagedForward(M, layer, x)
    torch.cuda.synchronize()
    print(f"# {wl.name}: resident on the GPU in {time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)

    # one step: the staged forward, and for a forward+backward workload the
    # layer backward (combine-bwd, down dgrad/wgrad with the SwiGLU backward,
    # gate/up dgrad/wgrad, router-prob grads, the router backward: dlogits,
    # dX_r, dW_r, db_r; dispatch-bwd folding in dX_r) after it
    def step(ev=None, ev_b=None):
        st.run(ev)
        if bwd:
            layer.backward(x, dout)
            if ev_b is not None:
                ev_b.record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    nst = len(StagedForward.STAGES)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(steps)]
    evb = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(steps):
        step(evs[k], evb[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    stage_ms = {name: float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(steps)]))
                for i, name in enumerate(StagedForward.STAGES)}
    fwd_ms = float(np.mean([evs[k][0].elapsed_time(evs[k][nst]) for k in range(steps)]))
    bwd_ms = (float(np.mean([evs[k][nst].elapsed_time(evb[k]) for k in range(steps)])) if bwd else 0.0)
    total_ms = fwd_ms + bwd_ms
    gpu_ms = evs[0][0].elapsed_time(evb[-1] if bwd else evs[-1][nst]) / steps

    def time_layer(lay):
        for _ in range(2):
            lay.forward(x)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            lay.forward(x)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    layer_ms = time_layer(layer) if (layer_call or shared_expert or single) else None

    def time_graph(lay):
        # the same forward call captured once in a HIP graph and replayed
        # (every step of the call is a kernel, so it captures whole)
        lay.forward(x)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            lay.forward(x)
        for _ in range(2):
            g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        assert int(lay.saved["status"].item()) == 0
        return e0.elapsed_time(e1) / steps

    graph_ms, graph_err = None, None
    if single:
        try:
            graph_ms = time_graph(layer)
        except Exception as ex:   # a capture the runtime refuses: reported, never fatal to the bench
            graph_err = f"{type(ex).__name__}: {ex}"
            torch.cuda.synchronize()
    ready_out = None
    if single and ready_queue_ok(wl):
        # dispatch, GEMM1 and GEMM2 in one readiness-gated launch (outputs
        # bitwise the staged launches'), timed call by call like layer_call_ms
        lay_r = M.MoeLayer(w, wl.N, wl.K, mxfp8=wl.mxfp8, drop=drop, renorm=wl.renorm, sched=M.MOE_SCHED_READY)
        ready_out = {"layer_fwd_ms": time_layer(lay_r), "staged_layer_fwd_ms": layer_ms,
                     "note": "moe_layer_fwd with MOE_SCHED_READY: router and route launches, then dispatch, "
                             "GEMM1 and GEMM2 in one persistent launch (GEMM2 tiles gated per GEMM1 row "
                             "block), then the combine"}
        del lay_r
    single_out = None
    if single and single_launch_ok(wl, bwd):
        # the same layer in one persistent launch per direction (outputs bitwise
        # the staged launches'), timed call by call like layer_call_ms
        lay_1 = M.MoeLayer(w, wl.N, wl.K, mxfp8=False, drop=drop, renorm=wl.renorm, with_bwd=bwd, router_bwd=bwd,
                           sched=M.MOE_SCHED_SINGLE)
        single_out = {"layer_fwd_ms": time_layer(lay_1), "staged_layer_fwd_ms": layer_ms}
        if bwd:
            def time_bwd(lay):
                for _ in range(2):
                    lay.backward(x, dout)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(steps):
                    lay.backward(x, dout)
                e1.record()
                torch.cuda.synchronize()
                return e0.elapsed_time(e1) / steps
            single_out["layer_bwd_ms"] = time_bwd(lay_1)
            single_out["staged_layer_bwd_ms"] = time_bwd(layer)
        single_out["note"] = ("moe_layer_fwd / moe_layer_bwd with MOE_SCHED_SINGLE: router to fold in one "
                              "persistent launch per direction, grid barriers between its phases")
        del lay_1
    shared = None
    if shared_expert:
        ws = shared_expert_weights(M, w, wl, seed, torch)
        lay_s = M.MoeLayer(ws, wl.N, wl.K, mxfp8=wl.mxfp8, drop=drop, renorm=wl.renorm)
        shared = {"layer_fwd_ms": time_layer(lay_s), "routed_only_layer_fwd_ms": layer_ms,
                  "note": "moe_layer_fwd with one shared expert (expert E over every token) in the same "
                          "grouped-GEMM launches"}
        del lay_s, ws

    counts = layer.saved["counts"].cpu().numpy()
    stats = load_stats(counts, wl.align)
    R = int(counts.sum())
    E_act = stats["active"]
    N, D, E, K, H = wl.N, wl.D, wl.E, wl.K, wl.H
    b = (1 + 1 / 32) if wl.mxfp8 else 2.0
    peak = PEAK_MXFP8_TFLOPS if wl.mxfp8 else PEAK_BF16_TFLOPS
    F1, Q1 = gemm1_work(R, D, H, E_act, b)
    F2, Q2 = gemm2_work(R, D, H, E_act, b)
    t1 = stage_ms["gemm1"] / 1e3
    t2 = stage_ms["gemm2"] / 1e3
    bound1 = "hbm" if Q1 / (PEAK_HBM_GBS * 1e9) >= F1 / (peak * 1e12) else "mfma"
    if bound1 == "hbm":
        roof = dict(bound="hbm", achieved=Q1 / t1 / 1e9, peak=PEAK_HBM_GBS, unit="GB/s")
    else:
        roof = dict(bound="mfma", achieved=F1 / t1 / 1e12, peak=peak, unit="TFLOP/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = recorded_traffic(wl.name, seed)
    roof["kernel"] = "gemm1 (grouped gate/up GEMM with SwiGLU epilogue)"
    roof["per_launch_algorithmic"] = dict(flops=F1, bytes=Q1, t_star_ms=t_star(F1, Q1, peak) * 1e3)

    gemm_tflops = routed_flops(R, D, H) / (t1 + t2) / 1e12
    pad = int((((counts + wl.align - 1) // wl.align) * wl.align - counts).sum()) if wl.align > 1 else 0
    qd = dispatch_bytes(N, D, K, R, b, pad)
    qc = combine_bytes(N, D, K, R)
    tstar_layer = sum([t_star(*router_work(N, D, E), peak), qd / (PEAK_HBM_GBS * 1e9), t_star(F1, Q1, peak),
                       t_star(F2, Q2, peak), qc / (PEAK_HBM_GBS * 1e9)])
    out = {
        "metric": METRIC,
        "value": N / (total_ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": total_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8-e4m3/bf16" if wl.mxfp8 else "bf16",
        "data": "synthetic (seeded; random-init weights of the stated shape)",
        "config": {"workload": wl.name, "N": N, "D": D, "E": E, "K": K, "H": H, "zipf_s": wl.zipf_s,
                   "p_drop": wl.p_drop, "align": wl.align, "seed": seed,
                   "pass": "fwd+bwd" if bwd else "fwd"},
        "roofline": roof,
        "grouped_gemm": {"tflops": gemm_tflops, "pct_mfma_peak": 100 * gemm_tflops / peak,
                         "gemm1_ms": stage_ms["gemm1"], "gemm2_ms": stage_ms["gemm2"],
                         "pct_of_roofline": 100 * (t_star(F1, Q1, peak) + t_star(F2, Q2, peak)) / (t1 + t2)},
        "dispatch": {"gbs": qd / (stage_ms["dispatch"] / 1e3) / 1e9,
                     "pct_hbm": 100 * qd / (stage_ms["dispatch"] / 1e3) / 1e9 / PEAK_HBM_GBS,
                     "ms": stage_ms["dispatch"]},
        "combine": {"gbs": qc / (stage_ms["combine"] / 1e3) / 1e9,
                    "pct_hbm": 100 * qc / (stage_ms["combine"] / 1e3) / 1e9 / PEAK_HBM_GBS,
                    "ms": stage_ms["combine"]},
        "stage_ms": stage_ms,
        "layer_fwd_pct_of_roofline": 100 * tstar_layer / (fwd_ms / 1e3),
        "load": dict(stats, routes=R),
        "wall_ms_per_step": 1e3 * wall / steps,
        "gpu_span_ms_per_step": gpu_ms,
    }
    out["fwd_ms"] = fwd_ms
    if bwd:
        tf_b = routed_flops(R, D, H, backward=True) / (bwd_ms / 1e3) / 1e12
        out["backward"] = {"ms": bwd_ms, "routed_tflops": tf_b, "pct_mfma_peak": 100 * tf_b / PEAK_BF16_TFLOPS,
                           "note": "value and ms_per_step cover forward + backward, router backward included; "
                                   "routed_tflops counts the expert GEMMs only; pct_mfma_peak against the bf16 "
                                   "peak" + ((" (MXFP8: block-scaled dgrads and wgrads)" if mx_wgrad else
                                              " (MXFP8: block-scaled dgrads, bf16 wgrads)") if wl.mxfp8 else "")}
    if layer_ms is not None:
        out["layer_call_ms"] = layer_ms
    if graph_ms is not None:
        out["graph_replay"] = {"layer_fwd_ms": graph_ms, "layer_call_ms": layer_ms,
                               "note": "the staged moe_layer_fwd call captured in one HIP graph and replayed"}
    elif graph_err is not None:
        out["graph_replay"] = {"error": graph_err}
    if shared is not None:
        out["shared_expert"] = shared
    if single_out is not None:
        out["single_launch"] = single_out
    if ready_out is not None:
        out["ready_queue"] = ready_out
    del layer, st, x, w, drop, dout
    return out


def summary_of(r):
    """The keys of a non-headline workload's result kept in the JSON line."""
    keep = ("value", "unit", "ms_per_step", "fwd_ms", "dtype", "config", "roofline", "grouped_gemm", "dispatch",
            "combine", "stage_ms", "layer_fwd_pct_of_roofline", "load", "backward", "single_launch", "ready_queue",
            "graph_replay")
    return {k: r[k] for k in keep if k in r}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3_bf16", choices=sorted(S.WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only --workload (by default the Mixtral-shaped forward, the Qwen3-shaped "
                         "forward + backward and the MXFP8 forward follow, as extra keys)")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--layer-call", action="store_true", help="also time moe_layer_fwd as one call")
    ap.add_argument("--backward", action="store_true",
                    help="time forward + backward (moe_layer_bwd with the router backward) on a forward "
                         "workload; dOut is N(0, 1) bf16 from the seed")
    ap.add_argument("--mx-wgrad", action="store_true",
                    help="MXFP8 backward: native block-scaled weight gradients on column-wise copies")
    ap.add_argument("--shared-expert", action="store_true",
                    help="also time moe_layer_fwd with one shared expert (N(0,1/D), N(0,1/H) weights) in the same "
                         "grouped-GEMM launches, beside the routed-only layer call")
    ap.add_argument("--single-only", action="store_true",
                    help="run only the workload's single-launch layer (MOE_SCHED_SINGLE: forward, and backward "
                         "with the router backward for a fwd+bwd workload) warmup + steps times and print its "
                         "times (for a kernel trace of that launch)")
    ap.add_argument("--ready-only", action="store_true",
                    help="run only the workload's readiness-gated forward (MOE_SCHED_READY; bf16 or MXFP8) "
                         "warmup + steps times and print its time (for a kernel trace of that launch)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="before timing, copy MIB MiB device-to-device once: a kernel of known traffic "
                         "that calibrates the HBM byte counters of a profiler run")
    ap.add_argument("--pmc-mfma-report", metavar="DIR",
                    help="print MFMA utilisation per GEMM kernel from one rocprofv3 --pmc run with the counters "
                         + " ".join(MFMA_COUNTERS) + ", and exit")
    ap.add_argument("--pmc-stall-report", metavar="DIR",
                    help="print where each GEMM kernel's waves spend their cycles from one rocprofv3 --pmc run "
                         "with the counters " + " ".join(STALL_COUNTERS) + ", and exit")
    ap.add_argument("--pmc-report", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the HBM traffic summary of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) "
                         "of this script with --copy-probe, and exit")
    args = ap.parse_args(argv)

    if args.pmc_mfma_report:
        print("| kernel | dispatches | avg us (counted run) | clock GHz | MFMA busy % | TFLOP/s (MOPS x 512) "
              "| % of dense peak at 2.4 GHz |")
        print("|---|---|---|---|---|---|---|")
        for r in mfma_report(args.pmc_mfma_report):
            print(f"| `{r['kernel'][:100]}` | {r['dispatches']} | {r['us']:.1f} | {r['ghz']:.2f} | {r['busy_pct']:.1f} | "
                  f"{r['tflops']:.0f} ({r['dtype']}) | {r['pct_peak']:.1f} |")
        return 0

    if args.pmc_stall_report:
        print("| kernel | dispatches | avg us (counted run) | dependency wait % | issue wait % | active % "
              "| LDS active % | LDS issue wait % | VMEM active % | MFMA busy % |")
        print("|---|---|---|---|---|---|---|---|---|---|")
        for r in stall_report(args.pmc_stall_report):
            print(f"| `{r['kernel'][:100]}` | {r['dispatches']} | {r['us']:.1f} | {r['wait_dep']:.1f} | "
                  f"{r['wait_issue']:.1f} | {r['active']:.1f} | {r['lds_active']:.1f} | {r['lds_issue_wait']:.1f} | "
                  f"{r['vmem_active']:.1f} | {r['mfma_busy']:.1f} |")
        return 0

    if args.pmc_report:
        summary, rows = pmc_report(args.pmc_report[0], args.pmc_report[1], args.copy_probe or 1024, args.workload)
        print("| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB | HBM write MB |")
        print("|---|---|---|---|---|")
        for r in rows[:16]:
            print(f"| `{r['kernel'][:110]}` | {r['fetch_kib'] or 0:.0f} | {r['write_kib'] or 0:.0f} | "
                  f"{r['read_bytes'] / 1e6:.1f} | {r['write_bytes'] / 1e6:.1f} |")
        print()
        print("```json")
        print(json.dumps(summary, indent=1))
        print("```")
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(expert parallelism is a design note, not code); run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import mixture_experts_expert_router_amd as M

    wl = S.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    t0 = time.perf_counter()
    inp = S.make_inputs(wl, args.seed)
    print(f"# inputs generated in {time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)

    if args.ready_only:
        if not ready_queue_ok(wl):
            print(f"{wl.name}: outside the readiness-gated launch's rules", file=sys.stderr)
            return 2
        x, w, drop = device_inputs(M, inp, wl.mxfp8, torch)
        lay = M.MoeLayer(w, wl.N, wl.K, mxfp8=wl.mxfp8, drop=drop, renorm=wl.renorm, sched=M.MOE_SCHED_READY)
        ev = []
        for i in range(args.warmup + args.steps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record()
            lay.forward(x)
            e[1].record()
            if i >= args.warmup:
                ev.append(e)
        torch.cuda.synchronize()
        assert int(lay.saved["status"].item()) == 0
        print(json.dumps({"workload": wl.name, "sched": "ready", "steps": args.steps,
                          "fwd_ms": float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))}), flush=True)
        return 0
    if args.single_only:
        bwd = wl.bwd or args.backward
        if not single_launch_ok(wl, bwd):
            print(f"{wl.name}: outside the single-launch layer's rules", file=sys.stderr)
            return 2
        x, w, drop = device_inputs(M, inp, False, torch, backward=bwd)
        dout_bits = inp.dout if inp.dout is not None else S.random_bf16((wl.N, wl.D), args.seed, 9)
        dout = torch.from_numpy(np.ascontiguousarray(dout_bits).view(np.int16)).view(torch.bfloat16).cuda()
        lay = M.MoeLayer(w, wl.N, wl.K, drop=drop, renorm=wl.renorm, with_bwd=bwd, router_bwd=bwd,
                         sched=M.MOE_SCHED_SINGLE)
        ev = []
        for i in range(args.warmup + args.steps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record()
            lay.forward(x)
            e[1].record()
            if bwd:
                lay.backward(x, dout)
            e[2].record()
            if i >= args.warmup:
                ev.append(e)
        torch.cuda.synchronize()
        assert int(lay.saved["status"].item()) == 0
        res = {"workload": wl.name, "sched": "single", "steps": args.steps,
               "fwd_ms": float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))}
        if bwd:
            res["bwd_ms"] = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
        print(json.dumps(res), flush=True)
        return 0

    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    out = measure(M, torch, wl, inp, args.steps, args.warmup, args.seed, backward=args.backward,
                  layer_call=args.layer_call, shared_expert=args.shared_expert, mx_wgrad=args.mx_wgrad,
                  single=not args.headline_only)
    if not args.headline_only:
        # the other workloads of the same run, each its own step (parity cases
        # aside from the headline): keys only, the headline value is above
        extra = {}
        for name in EXTRA_WORKLOADS:
            if name == wl.name:
                continue
            wx = S.WORKLOADS[name]
            t0 = time.perf_counter()
            same_inputs = (wx.N, wx.D, wx.E, wx.K, wx.H, wx.zipf_s, wx.p_drop) == \
                (wl.N, wl.D, wl.E, wl.K, wl.H, wl.zipf_s, wl.p_drop)
            ix = inp if same_inputs else S.make_inputs(wx, args.seed)
            print(f"# {name}: inputs in {time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)
            r = measure(M, torch, wx, ix, args.steps, args.warmup, args.seed, single=True)
            extra[name] = summary_of(r)
            print(f"# {name}: {extra[name]['ms_per_step']:.3f} ms/step", file=sys.stderr, flush=True)
            del ix
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
        out["workloads"] = extra
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, wl, args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

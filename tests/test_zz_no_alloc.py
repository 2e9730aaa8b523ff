"""The allocation-free forward (moe_layer_fwd_noalloc) against moe_layer_fwd:
the same kernels on the library's static per-GPU scratch instead of a
caller workspace, so every saved tensor and the output must be bitwise equal.
Two calls in a row, the second with a smaller input, so the second runs on
the scratch contents the first left behind."""
import numpy as np
import pytest
import torch

import mixture_experts_expert_router_amd as M
import moe_synth as S
import oracle as O
from gpu_util import dev, dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.load()


def _weights(inp, mxfp8):
    w = M.LayerWeights(w_r=dev_bf16(inp.w_r), bias=dev(inp.bias) if inp.bias is not None else None)
    if mxfp8:
        w.wq = {k: dev(v) for k, v in O.quantize_weights_mxfp8(inp.w_gate, inp.w_up, inp.w_down).items()}
    else:
        w.w_gate, w.w_up, w.w_down = dev_bf16(inp.w_gate), dev_bf16(inp.w_up), dev_bf16(inp.w_down)
    return w


def _same(a, b, what):
    assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), what


@pytest.mark.parametrize("base,mxfp8,sched", [("dsv3_bf16", False, M.MOE_SCHED_STAGED),
                                              ("qwen3_235b_bf16_fwdbwd", False, M.MOE_SCHED_STAGED),
                                              ("dsv3_mxfp8", True, M.MOE_SCHED_STAGED),
                                              ("dsv3_bf16", False, M.MOE_SCHED_READY),
                                              ("dsv3_mxfp8", True, M.MOE_SCHED_READY),
                                              ("qwen3_235b_bf16_fwdbwd", False, M.MOE_SCHED_SINGLE)])
def test_noalloc_forward_equals_layer_fwd_on_two_calls(base, mxfp8, sched):
    """Under each schedule: the readiness queue's state and the single
    launch's barrier words also live in the scratch, reset by each call."""
    shapes = [dict(N=640, D=512, E=32, K=8, H=256), dict(N=96, D=256, E=16, K=4, H=128)]
    for i, shp in enumerate(shapes):
        wl = S.scaled(S.WORKLOADS[base], f"noalloc_{i}", **shp)
        print(f"noalloc {base} sched {sched} call {i}: {shp}", flush=True)
        inp = S.make_inputs(wl, 40 + i)
        w = _weights(inp, mxfp8)
        drop = dev(inp.drop) if inp.drop is not None else None
        x = dev_bf16(inp.x)
        ref = M.MoeLayer(w, wl.N, wl.K, mxfp8=mxfp8, drop=drop, sched=sched)
        ref.forward(x)
        got = M.MoeLayer(w, wl.N, wl.K, mxfp8=mxfp8, drop=drop, sched=sched)
        got.saved["_buf"].fill_(0xFF)                 # every saved tensor poisoned
        got.out.view(torch.int16).fill_(0x7FA0)
        got.forward_noalloc(x)
        torch.cuda.synchronize()
        _same(got.out, ref.out, "out")
        n = int(ref.saved["offsets"][-1].item())
        for k, t in M.saved_tensors(ref.saved).items():
            if k in ("aux", "status"):
                continue
            if t.dim() == 2 and t.shape[0] == M.rows_cap(ref.d):
                _same(got.saved[k][:n], t[:n], k)       # rows past the segments are never written
            else:
                _same(got.saved[k], t, k)
        assert int(got.saved["status"].item()) == 0

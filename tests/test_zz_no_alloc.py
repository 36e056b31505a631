"""The allocation-free layer path (ada_lora_layer_static): the unmerged routed layer
with its fp32 intermediates in the library's static device array instead of a
caller-owned workspace, for callers that cannot allocate.  It must give exactly what
ada_lora_layer gives, call after call on the shared array (the second call smaller
than the first), and refuse layers whose intermediates exceed the array."""
import ctypes

import numpy as np
import pytest
import torch

from helpers import to64
from oracle import adafuse as O
from weight_merge_amd import _lib
from weight_merge_amd import api as A
from weight_merge_amd import synth
from weight_merge_amd._lib import ADA_BF16, ADA_ESHAPE, AdaLoraProj

DEV = "cuda"
TD = {"fp32": torch.float32, "bf16": torch.bfloat16}


def group(seed, E, r, shapes, dt):
    banks = [synth.adapter_bank(seed + i, E, r, do, di, dt) for i, (do, di) in enumerate(shapes)]
    xs = [synth.host_normal(synth.tensor_seed(seed, "x", i), (di,), 1.0, dt) for i, (_, di) in enumerate(shapes)]
    return banks, xs


def run_both(banks, xs, idx, gate, dt):
    dev = [tuple(t.to(DEV) for t in b) for b in banks]
    xd = [x.to(DEV) for x in xs]
    y_ws = [torch.full((W.shape[0],), float("nan"), dtype=TD[dt], device=DEV) for W, _, _ in banks]
    y_st = [torch.full((W.shape[0],), float("nan"), dtype=TD[dt], device=DEV) for W, _, _ in banks]
    A.ada_lora_layer([(w, a, b, x, y) for (w, a, b), x, y in zip(dev, xd, y_ws)], idx.to(DEV), gate.to(DEV), 2.0)
    A.ada_lora_layer_static([(w, a, b, x, y) for (w, a, b), x, y in zip(dev, xd, y_st)], idx.to(DEV), gate.to(DEV),
                            2.0)
    torch.cuda.synchronize()
    return y_ws, y_st


@pytest.mark.gpu
def test_static_layer_path_equals_the_workspace_path_twice():
    # call 1: three projections, bf16, k*r = 32; call 2 (smaller, other dtype): one
    # projection, fp32, k*r = 8 -- both on the same static array
    cases = [
        (8, 16, 2, [(1032, 520), (264, 1032), (520, 264)], "bf16", 3),
        (4, 8, 1, [(136, 264)], "fp32", 9),
    ]
    for E, r, k, shapes, dt, seed in cases:
        banks, xs = group(300 + seed, E, r, shapes, dt)
        h, R = synth.small_router(seed, E, 64, dt)
        idx_np, g_np = O.pregate(to64(h), to64(R), k)
        idx = torch.tensor(idx_np, dtype=torch.int32)
        gate = torch.tensor(g_np, dtype=torch.float32)
        y_ws, y_st = run_both(banks, xs, idx, gate, dt)
        for (W, Aw, Bw), x, a, b in zip(banks, xs, y_ws, y_st):
            assert torch.equal(a, b), (E, r, k, dt, W.shape)
            # and both are the routed forward (the GEMV bound of the layer tests)
            ref = O.routed_lora_forward(to64(W), to64(Aw), to64(Bw), idx_np, g_np.astype(np.float32).astype(np.float64),
                                        2.0, to64(x))
            bound = (8e-3 if dt == "bf16" else 1e-6) * np.abs(ref) + \
                (1e-4 if dt == "bf16" else 1e-5) * (np.abs(to64(W)) @ np.abs(to64(x)))
            assert np.all(np.abs(to64(b) - ref) <= bound), (dt, W.shape)


def test_static_layer_path_refuses_intermediates_beyond_its_array():
    """Checked on the host before any HIP call (fake, aligned device addresses): a
    projection of 2^20 + 8 rows needs 4 * (2^20 + 8 + k r) bytes, over the 4 MiB array."""
    lib = _lib.load()
    P = 1 << 20  # never dereferenced
    arr = (AdaLoraProj * 1)(AdaLoraProj(P, P, P, P, P, (1 << 20) + 8, 64, 64))
    idx = ctypes.c_void_p(P)
    assert lib.ada_lora_layer_static(arr, 1, 4, 8, idx, idx, 2, 2.0, ADA_BF16, None) == ADA_ESHAPE
    arr_ok_size = (AdaLoraProj * 1)(AdaLoraProj(P, P, P, P, None, 1024, 64, 64))
    assert lib.ada_lora_layer_static(arr_ok_size, 1, 4, 8, idx, idx, 2, 2.0, ADA_BF16, None) == _lib.ADA_EINVAL


@pytest.mark.gpu
def test_static_layer_path_replays_under_graph_capture():
    """The callers it is for include code under HIP graph capture: captured once, the
    call replays with the same results as eager calls, replay after replay, with eager
    work on the same static array in between (a different layer shape each time)."""
    E, r, k = 8, 16, 2
    banks, xs = group(700, E, r, [(264, 520), (520, 264)], "bf16")
    h, R = synth.small_router(7, E, 64, "bf16")
    idx_np, g_np = O.pregate(to64(h), to64(R), k)
    idx = torch.tensor(idx_np, dtype=torch.int32, device=DEV)
    gate = torch.tensor(g_np, dtype=torch.float32, device=DEV)
    dev = [tuple(t.to(DEV) for t in b) for b in banks]
    xd = [x.to(DEV) for x in xs]
    eager = [torch.empty(W.shape[0], dtype=torch.bfloat16, device=DEV) for W, _, _ in banks]
    A.ada_lora_layer([(w, a, b, x, y) for (w, a, b), x, y in zip(dev, xd, eager)], idx, gate, 2.0)
    ys = [torch.full_like(y, float("nan")) for y in eager]
    call = [(w, a, b, x, y) for (w, a, b), x, y in zip(dev, xd, ys)]
    A.ada_lora_layer_static(call, idx, gate, 2.0)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        A.ada_lora_layer_static(call, idx, gate, 2.0)
    other, other_x = group(900, E, r, [(136, 1032)], "bf16")
    o_dev = [tuple(t.to(DEV) for t in b) for b in other]
    o_y = torch.empty(136, dtype=torch.bfloat16, device=DEV)
    for rep in range(4):
        for y in ys:
            y.fill_(float("nan"))
        # eager use of the same static array between replays
        A.ada_lora_layer_static([(o_dev[0][0], o_dev[0][1], o_dev[0][2], other_x[0].to(DEV), o_y)], idx, gate, 2.0)
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(eager, ys):
            assert torch.equal(a, b), rep

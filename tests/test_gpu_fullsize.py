"""Full-size parity: the 7B- and 70B-shaped stacks in the launch configuration the
benchmark times (pregate, then one in-place merge launch over every layer and
projection, then one unmerge launch), checked against the oracle on sampled rows of
every projection and on every element of selected projections."""
import numpy as np
import pytest
import torch

from helpers import (BF16_ATOL, BF16_RTOL, GATE_ATOL, GATE_RTOL, check_close, gapped_router, gapped_stack_router,
                     merge_tile_rows, oracle_selection, sample_rows, to64)
from oracle import adafuse as O
from weight_merge_amd import api as A
from weight_merge_amd import synth
from weight_merge_amd.configs import LLAMA7B_E8R16K2, LLAMA7B_E16R64K4, LLAMA70B_E8R16K2, LLAMA70B_TP8_E8R16K2

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_stack(cfg, seed, full_check, decode_check=False, band_layer=None):
    """full_check(l, p, proj) -> True for the projections compared element by element;
    every other projection is compared on sampled rows at the launch's tile height
    (band edges of 8 random bands plus 64 random rows), and in layer `band_layer` (if
    given) the first projection of each distinct shape on the first and last row of
    every tile band.  decode_check: also decode every fully kept projection on the
    merged weights and compare with the oracle's routed forward on the original ones
    (relative L2 <= 5e-3, the merged-vs-routed criterion)."""
    h, R, seed = gapped_stack_router(cfg, seed)
    ridx, rg = O.pregate(to64(h), to64(R), cfg.k, cfg.renorm)
    st = synth.make_stack(cfg, seed, device=DEV)
    rng = np.random.default_rng(seed)
    tile = merge_tile_rows(cfg.kr)
    keep = []  # (l, p, rows, W rows before the merge)
    banded = set()
    for l, p, proj in st.items():
        if full_check(l, p, proj):
            rows = np.arange(proj.d_out)
        elif l == band_layer and (proj.d_out, proj.d_in) not in banded:
            banded.add((proj.d_out, proj.d_in))
            rows = sample_rows(proj.d_out, rng, tile, all_bands=True)
        else:
            rows = sample_rows(proj.d_out, rng, tile)
        keep.append((l, p, rows, st.W[l][p][torch.from_numpy(rows).to(DEV)].cpu()))
    model = A.AdaModel([(st.W[l][p], None, st.A[l][p], st.B[l][p]) for l, p, _ in st.items()], cfg.E, cfg.r)
    idx, gate = A.ada_pregate(h.to(DEV), R.to(DEV), cfg.k, cfg.renorm)
    A.ada_merge(model, idx, gate, cfg.scale)
    torch.cuda.synchronize()
    assert idx.cpu().tolist() == ridx.tolist()
    check_close(gate, rg, GATE_RTOL, GATE_ATOL, "gates")

    n_checked = 0
    for l, p, rows, w0 in keep:
        rows_t = torch.from_numpy(rows).to(DEV)
        got = st.W[l][p][rows_t]
        Bsel = st.B[l][p][:, rows_t, :]
        ref = O.merge(to64(w0), to64(st.A[l][p]), to64(Bsel), ridx, rg, cfg.scale)
        check_close(got, ref, BF16_RTOL, BF16_ATOL, f"merge layer {l} proj {cfg.projections[p].name}")
        n_checked += got.numel()

    if decode_check:
        for l, p, rows, w0 in keep:
            if len(rows) != cfg.projections[p].d_out:
                continue
            x = synth.host_normal(synth.tensor_seed(seed, "x", l, p), (w0.shape[1],), 1.0, "bf16")
            y = A.ada_decode_gemv(st.W[l][p], x.to(DEV))
            torch.cuda.synchronize()
            ref = O.routed_lora_forward(to64(w0), to64(st.A[l][p]), to64(st.B[l][p]), ridx, rg, cfg.scale, to64(x))
            rel = np.linalg.norm(to64(y) - ref) / np.linalg.norm(ref)
            assert rel <= 5e-3, (l, cfg.projections[p].name, rel)

    A.ada_unmerge(model, idx, gate, cfg.scale)
    torch.cuda.synchronize()
    exact = total = 0
    for l, p, rows, w0 in keep:
        got = st.W[l][p][torch.from_numpy(rows).to(DEV)].cpu()
        check_close(got, to64(w0), BF16_RTOL, BF16_ATOL, f"unmerge layer {l} proj {cfg.projections[p].name}")
        exact += int((got.view(torch.int16) == w0.view(torch.int16)).sum())
        total += got.numel()
    model.destroy()
    del st
    torch.cuda.empty_cache()
    print(f"{cfg.name}: {n_checked} merged elements checked, unmerge bit-exact fraction {exact / total:.4f}")
    return exact / total


def test_llama7b_e8r16k2_stack():
    frac = run_stack(LLAMA7B_E8R16K2, 1000, lambda l, p, proj: l == 0, decode_check=True, band_layer=17)
    assert frac > 0.8


def test_llama7b_e16r64k4_stack():
    frac = run_stack(LLAMA7B_E16R64K4, 2000, lambda l, p, proj: l == 31, band_layer=5)
    assert frac > 0.8


def test_llama70b_e8r16k2_stack():
    # element by element: the k and v projections (1024 x 8192) of layer 0
    frac = run_stack(LLAMA70B_E8R16K2, 3000, lambda l, p, proj: l == 0 and proj.name in ("k", "v"),
                     band_layer=57)
    assert frac > 0.8


def test_llama70b_tp8_shard_stack():
    # one GPU's tensor-parallel shard: element by element, the 128-row k and v projections
    # and the 1024-column o projection of layer 0
    frac = run_stack(LLAMA70B_TP8_E8R16K2, 4000, lambda l, p, proj: l == 0 and proj.name in ("k", "v", "o"),
                     band_layer=41)
    assert frac > 0.8


def test_llama7b_e8r16k2_fused_switch():
    """The fused switch over the whole 7B-shaped stack in one launch (undo one selection
    and apply another with one read and one write of every weight), from the pristine
    weights: sampled rows of every projection, and every element of layer 0, against
    the oracle's W - delta(prev) + delta(cur)."""
    cfg = LLAMA7B_E8R16K2
    h1, R1, seed = gapped_stack_router(cfg, 6000)
    h2, R2, _ = gapped_stack_router(cfg, 7000)
    sels = []
    for h, R in ((h1, R1), (h2, R2)):
        i, g = O.pregate(to64(h), to64(R), cfg.k, cfg.renorm)
        g32 = np.asarray(g, dtype=np.float32)  # the values the kernel reads
        sels.append((np.asarray(i), g32.astype(np.float64),
                     torch.tensor(i, dtype=torch.int32, device=DEV), torch.from_numpy(g32).to(DEV)))
    assert sels[0][0].tolist() != sels[1][0].tolist(), "the two selections must differ"
    st = synth.make_stack(cfg, seed, device=DEV)
    rng = np.random.default_rng(seed)
    keep = []
    for l, p, proj in st.items():
        rows = np.arange(proj.d_out) if l == 0 else sample_rows(proj.d_out, rng, merge_tile_rows(2 * cfg.kr))
        keep.append((l, p, rows, st.W[l][p][torch.from_numpy(rows).to(DEV)].cpu()))
    model = A.AdaModel([(st.W[l][p], None, st.A[l][p], st.B[l][p]) for l, p, _ in st.items()], cfg.E, cfg.r)
    A.ada_switch(model, (sels[0][2], sels[0][3]), (sels[1][2], sels[1][3]), cfg.scale)
    torch.cuda.synchronize()
    for l, p, rows, w0 in keep:
        rows_t = torch.from_numpy(rows).to(DEV)
        ref = O.switch(to64(w0), to64(st.A[l][p]), to64(st.B[l][p][:, rows_t, :]), sels[0][:2], sels[1][:2],
                       cfg.scale)
        check_close(st.W[l][p][rows_t], ref, BF16_RTOL, BF16_ATOL, f"switch layer {l} proj {cfg.projections[p].name}")
    model.destroy()
    del st
    torch.cuda.empty_cache()


def test_unmerged_paths_at_7b_layer_shapes():
    """One decoder layer of the 7B-shaped stack (q, k, v, o 4096 x 4096; gate, up
    11008 x 4096; down 4096 x 11008) through the unmerged routed paths at full shape,
    in the decode groups ({q, k, v}, {o}, {gate, up}, {down}): the batched path with
    16 requests, each with its own selection, and the single-request layer path;
    every output within the GEMV bound of the oracle's routed forward."""
    E, r, k, nb = 8, 16, 2, 16
    shapes = {"q": (4096, 4096), "k": (4096, 4096), "v": (4096, 4096), "o": (4096, 4096),
              "gate": (11008, 4096), "up": (11008, 4096), "down": (4096, 11008)}
    groups = [["q", "k", "v"], ["o"], ["gate", "up"], ["down"]]
    banks = {n: synth.adapter_bank(800 + i, E, r, do, di, "bf16") for i, (n, (do, di)) in enumerate(shapes.items())}
    xs = {n: synth.host_normal(synth.tensor_seed(900 + i, di), (nb, di), 1.0, "bf16")
          for i, (n, (_, di)) in enumerate(shapes.items())}
    sels = []
    for b in range(nb):
        h, R, _ = gapped_router(E, 64, "bf16", 60 + 7 * b)
        sels.append(oracle_selection(h, R, k))
    idx = torch.stack([s[0] for s in sels]).contiguous()
    gate = torch.stack([s[1] for s in sels]).contiguous()
    assert len({tuple(row) for row in idx.tolist()}) > 1, "the batch must mix selections"
    dev = {n: tuple(t.to(DEV) for t in banks[n]) for n in shapes}
    xd = {n: xs[n].to(DEV) for n in shapes}
    ys = {n: torch.full((nb, shapes[n][0]), float("nan"), dtype=torch.bfloat16, device=DEV) for n in shapes}
    y1 = {n: torch.full((shapes[n][0],), float("nan"), dtype=torch.bfloat16, device=DEV) for n in shapes}
    didx, dgate = idx.to(DEV), gate.to(DEV)
    for gr in groups:
        A.ada_lora_batch([(dev[n][0], dev[n][1], dev[n][2], xd[n], ys[n]) for n in gr], didx, dgate, 2.0)
        A.ada_lora_layer([(dev[n][0], dev[n][1], dev[n][2], xd[n][0].contiguous(), y1[n]) for n in gr],
                         didx[0].contiguous(), dgate[0].contiguous(), 2.0)
    torch.cuda.synchronize()
    for n, (W, Aw, Bw) in banks.items():
        W64, A64, B64 = to64(W), to64(Aw), to64(Bw)
        got = to64(ys[n])
        for b in range(nb):
            x64 = to64(xs[n][b])
            ref = O.routed_lora_forward(W64, A64, B64, idx[b].numpy(), gate[b].numpy().astype(np.float64), 2.0, x64)
            bound = 8e-3 * np.abs(ref) + 1e-4 * (np.abs(W64) @ np.abs(x64))
            assert np.all(np.abs(got[b] - ref) <= bound), (n, b, float(np.max(np.abs(got[b] - ref) / bound)))
            if b == 0:
                assert np.all(np.abs(to64(y1[n]) - ref) <= bound), (n, "single request")

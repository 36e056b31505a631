"""Per-token switching ("AdaFuse", Portuguese summary page, technical summary 2.B: the
SGMM kernel undoes the previous token's fusion and fuses the current one; 2.A: the
router decides per input token) over chains of tokens, each pre-gated on the GPU from
its own hidden state.

Two ways to switch, and what each guarantees:
  * re-merge from the untouched weights (an out-of-place model: ada_merge reads W and
    writes W'): one read and one write of every weight per token, like a fused switch,
    and every token's W' is the stated tolerance away from W + delta(token), however
    long the chain;
  * the fused in-place switch (ada_switch: W <- RNE(W - delta(prev) + delta(cur))):
    each switch rounds W to bf16 again, so rounding errors accumulate along the chain
    (measured here against a CPU emulation of that rounding)."""
import numpy as np
import pytest
import torch

from helpers import BF16_ATOL, BF16_RTOL, GATE_ATOL, GATE_RTOL, check_close, gapped_router, to64
from oracle import adafuse as O
from weight_merge_amd import api as A
from weight_merge_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def token_routers(E, d, n, seed):
    """n hidden states sharing one router, each with logits >= 1e-3 apart."""
    _, R = synth.small_router(seed, E, d, "bf16")
    hs, s = [], seed * 1000
    R64 = to64(R)
    while len(hs) < n:
        h = synth.host_normal(synth.tensor_seed(s, "h"), (d,), 1.0, "bf16")
        z = np.sort(O.router_logits(to64(h), R64))
        if np.min(np.diff(z)) >= 1e-3:
            hs.append(h)
        s += 1
    return hs, R


CHAIN_STACKS = [
    # E, r, k, projection shapes (d_out, d_in): two layers of three ragged projections
    (8, 16, 2, [(264, 520), (136, 264), (520, 136)]),     # k r = 32
    (16, 64, 4, [(136, 264), (264, 136), (200, 392)]),    # k r = 256: long contraction
]


@pytest.mark.parametrize("E,r,k,shapes", CHAIN_STACKS)
def test_per_token_remerge_chain_stays_within_tolerance(E, r, k, shapes):
    """12 tokens: pregate on the GPU from each token's hidden state, re-merge every
    projection of the stack from the untouched W into W' (one launch), decode each
    projection on W'.  Every element of every W' is compared with the oracle's
    W + delta(token), and every decode output with the oracle's routed forward on W."""
    n_tok, d, s = 12, 256, 2.0
    hs, R = token_routers(E, d, n_tok, 31 + r)
    layers = []
    for l in range(2):
        for i, (do, di) in enumerate(shapes):
            W, Aw, Bw = synth.adapter_bank(500 + 10 * l + i, E, r, do, di, "bf16")
            layers.append((W, Aw, Bw, W.to(DEV), torch.full((do, di), float("nan"), dtype=torch.bfloat16,
                                                           device=DEV), Aw.to(DEV), Bw.to(DEV)))
    model = A.AdaModel([(w, wo, a, b) for _, _, _, w, wo, a, b in layers], E, r)
    Rd = R.to(DEV)
    seen = set()
    for t, h in enumerate(hs):
        ridx, rg = O.pregate(to64(h), to64(R), k)
        idx, gate = A.ada_pregate(h.to(DEV), Rd, k)
        A.ada_merge(model, idx, gate, s)
        xs = [synth.host_normal(synth.tensor_seed(t, "x", j), (lay[0].shape[1],), 1.0, "bf16")
              for j, lay in enumerate(layers)]
        ys = [A.ada_decode_gemv(lay[4], x.to(DEV)) for lay, x in zip(layers, xs)]
        torch.cuda.synchronize()
        assert idx.cpu().tolist() == ridx.tolist(), (t, idx.cpu().tolist(), ridx.tolist())
        check_close(gate, rg, GATE_RTOL, GATE_ATOL, f"gates, token {t}")
        seen.add(tuple(ridx.tolist()))
        for j, ((W, Aw, Bw, _, wo, _, _), x, y) in enumerate(zip(layers, xs, ys)):
            W64, A64, B64 = to64(W), to64(Aw), to64(Bw)
            check_close(wo, O.merge(W64, A64, B64, ridx, rg, s), BF16_RTOL, BF16_ATOL, f"token {t} projection {j}")
            ref = O.routed_lora_forward(W64, A64, B64, ridx, rg, s, to64(x))
            rel = np.linalg.norm(to64(y) - ref) / np.linalg.norm(ref)
            assert rel <= 5e-3, (t, j, rel)
    for lay in layers:
        assert torch.equal(lay[3].cpu(), lay[0]), "re-merging must never write W"
    assert len(seen) >= 3, f"the chain should visit several selections, saw {seen}"
    model.destroy()


def emulated_switch_chain(W0, A64, B64, sels, s):
    """The in-place chain's rounding on the CPU: merge sel_0, then switch sel_{t-1} ->
    sel_t, each step W <- RNE_bf16(W - delta(prev) + delta(cur)) with exact deltas (the
    kernels carry the coefficients at fp32 accuracy; only the bf16 roundings of W remain)."""
    def bf(x):
        return torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    deltas = [O.adapter_delta(A64, B64, i, s * g) for i, g in sels]
    w = bf(W0 + deltas[0])
    out = [w]
    for t in range(1, len(sels)):
        w = bf(w - deltas[t - 1] + deltas[t])
        out.append(w)
    return out


def test_in_place_switch_chain_drift_matches_its_emulation():
    """32 tokens on one in-place projection (512 x 4096, E = 8, r = 16, top-2): merge
    the first token's selection, then one fused switch per token.  After each switch the
    fraction of weights outside the stated tolerance of W + delta(token) is measured on
    the GPU and must match the CPU emulation of the chain's bf16 roundings; the first
    merge and the first switch are within tolerance everywhere.  (The fractions are
    printed: a serving loop that switches in place must restore W periodically.)"""
    E, r, k, d_out, d_in, s, n_tok = 8, 16, 2, 512, 4096, 2.0, 32
    W, Aw, Bw = synth.adapter_bank(77, E, r, d_out, d_in, "bf16")
    hs, R = token_routers(E, 256, n_tok, 91)
    sels = [O.pregate(to64(h), to64(R), k) for h in hs]
    W0, A64, B64 = to64(W), to64(Aw), to64(Bw)
    emu = emulated_switch_chain(W0, A64, B64, sels, s)
    w = W.to(DEV)
    model = A.AdaModel([(w, None, Aw.to(DEV), Bw.to(DEV))], E, r)
    Rd = R.to(DEV)
    prev = A.ada_pregate(hs[0].to(DEV), Rd, k)
    A.ada_merge(model, *prev, s)
    rows = []
    for t in range(n_tok):
        if t:
            cur = A.ada_pregate(hs[t].to(DEV), Rd, k)
            A.ada_switch(model, prev, cur, s)
            prev = cur
        torch.cuda.synchronize()
        ref = O.merge(W0, A64, B64, *sels[t], s)
        bound = BF16_RTOL * np.abs(ref) + BF16_ATOL
        got = to64(w)
        f_gpu = float(np.mean(np.abs(got - ref) > bound))
        f_emu = float(np.mean(np.abs(emu[t] - ref) > bound))
        worst = float(np.max(np.abs(got - ref) / bound))
        rows.append((t, f_gpu, f_emu, worst))
        if t <= 1:
            assert f_gpu == 0.0, (t, f_gpu, worst)
        assert abs(f_gpu - f_emu) <= 2e-3 + 0.1 * f_emu, (t, f_gpu, f_emu)
    print("\nin-place switch chain (512 x 4096, E8 r16 k2): token, fraction out of tolerance (GPU, emulated), "
          "worst element / bound")
    for t, fg, fe, wr in rows:
        print(f"  {t:3d}  {fg:.5f}  {fe:.5f}  {wr:.3f}")
    model.destroy()

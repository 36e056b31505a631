"""GPU parity: the HIP path through the C ABI against the fp64 oracle, element by
element, on seeded inputs that span several tiles and ragged tails."""
import numpy as np
import pytest
import torch

from helpers import (BF16_ATOL, BF16_RTOL, GATE_ATOL, GATE_RTOL, check_close, fp32_accumulation_bound,
                     gapped_router, kernel_error_bound, merge_tile_rows, min_gap, oracle_selection, sample_rows, to64,
                     tol)
from oracle import adafuse as O
from weight_merge_amd import api as A
from weight_merge_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"fp32": torch.float32, "bf16": torch.bfloat16}


def sync():
    torch.cuda.synchronize()


# ---------------------------------------------------------------- pre-gating

PREGATE_CASES = [
    # E, k, d, dtype, renorm
    (4, 2, 256, "fp32", True),
    (8, 2, 4096, "bf16", True),
    (16, 4, 4096, "bf16", True),
    (8, 2, 8192, "bf16", True),
    (1, 1, 8, "bf16", True),
    (2, 2, 16, "fp32", True),
    (64, 8, 1032, "bf16", True),
    (64, 64, 520, "fp32", True),
    (33, 5, 264, "bf16", False),
    (16, 4, 4096, "bf16", False),
]


@pytest.mark.parametrize("E,k,d,dt,renorm", PREGATE_CASES)
def test_pregate_matches_oracle(E, k, d, dt, renorm):
    for seed in (11, 12, 13):
        h, R, _ = gapped_router(E, d, dt, seed * 1000)
        idx, gate = A.ada_pregate(h.to(DEV), R.to(DEV), k, renorm=renorm)
        sync()
        ridx, rg = O.pregate(to64(h), to64(R), k, renorm)
        assert idx.cpu().numpy().tolist() == ridx.tolist(), (seed, E, k, d)
        check_close(gate, rg, GATE_RTOL, GATE_ATOL, "gates")


def _random_pregate_cases(n: int = 16, seed: int = 20261205):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        E = int(rng.integers(1, 65))
        out.append((E, int(rng.integers(1, E + 1)), 8 * int(rng.integers(1, 1100)),
                    "bf16" if rng.random() < 0.7 else "fp32", bool(rng.random() < 0.8)))
    return out


@pytest.mark.parametrize("E,k,d,dt,renorm", _random_pregate_cases())
def test_pregate_matches_oracle_on_random_shapes(E, k, d, dt, renorm):
    """Seeded draws of (E, k, d, dtype, renorm), d up to 8792 (ragged batches of the
    row loads): indices bit-exact, gates within tolerance."""
    h, R, _ = gapped_router(E, d, dt, 7000 + d)
    idx, gate = A.ada_pregate(h.to(DEV), R.to(DEV), k, renorm=renorm)
    sync()
    ridx, rg = O.pregate(to64(h), to64(R), k, renorm)
    assert idx.cpu().numpy().tolist() == ridx.tolist(), (E, k, d)
    check_close(gate, rg, GATE_RTOL, GATE_ATOL, "gates")


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_pregate_with_nan_scores_still_selects_distinct_in_range_experts(dt):
    """A NaN in the hidden state makes every logit NaN, and NaN rows of the router make
    some of them NaN: the selection is then unspecified, but it must still be k
    distinct indices in [0, E), so a merge never reads outside the adapter banks."""
    E, k, d = 16, 4, 256
    h, R, _ = gapped_router(E, d, dt, 77)
    h_nan = h.clone()
    h_nan[3] = float("nan")
    R_nan = R.clone()
    R_nan[[2, 9]] = float("nan")
    for hh, RR in ((h_nan, R), (h, R_nan)):
        idx, _ = A.ada_pregate(hh.to(DEV), RR.to(DEV), k)
        sync()
        got = idx.cpu().tolist()
        assert len(set(got)) == k and all(0 <= e < E for e in got), got


def test_pregate_ties_go_to_the_lower_index():
    # identical router rows give identical logits (same summation order per row)
    E, d = 8, 512
    h, R, _ = gapped_router(E, d, "bf16", 5)
    R[5] = R[2]
    R[7] = R[2]
    z = O.router_logits(to64(h), to64(R))
    top = int(np.argmax(z))
    idx, gate = A.ada_pregate(h.to(DEV), R.to(DEV), E)
    sync()
    got = idx.cpu().tolist()
    assert got == O.select_topk(z, E).tolist()
    assert got.index(2) < got.index(5) < got.index(7)
    assert top in got


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_pregate_zero_scores_tie_to_the_lower_index(dt):
    """Rows of zeros give zero scores whatever h holds (products of -0.0 and +0.0 when h
    has both signs); equal scores, zero included, go to the lower index, and the zeros
    here are the largest scores (every other row scores below zero)."""
    E, d, k = 8, 256, 5
    h = synth.host_normal(synth.tensor_seed(71, "h"), (d,), 1.0, dt)
    assert (h < 0).any() and (h > 0).any()
    R = torch.zeros(E, d, dtype=TD[dt])
    for e in (0, 2, 4, 7):
        R[e] = (-(0.1 + 0.05 * e) * h.float()).to(TD[dt])
    z = O.router_logits(to64(h), to64(R))
    assert np.all(z[[1, 3, 5, 6]] == 0.0) and np.all(z[[0, 2, 4, 7]] < 0.0)
    idx, gate = A.ada_pregate(h.to(DEV), R.to(DEV), k)
    sync()
    assert idx.cpu().tolist()[:4] == [1, 3, 5, 6]
    assert idx.cpu().tolist() == O.select_topk(z, k).tolist()
    ref = O.gate_weights(z, O.select_topk(z, k))
    check_close(gate, ref, GATE_RTOL, GATE_ATOL, "gates over tied zero scores")


# ---------------------------------------------------------------- merge

MERGE_CASES = [
    # E, r, k, d_out, d_in, dtype, inplace
    (4, 8, 2, 256, 256, "fp32", True),
    (5, 3, 2, 40, 48, "fp32", False),
    (8, 16, 2, 384, 520, "bf16", False),
    (8, 16, 2, 136, 1000, "bf16", True),
    (16, 64, 4, 136, 264, "bf16", True),
    (8, 4, 3, 200, 72, "bf16", False),
    (6, 12, 2, 128, 128, "bf16", True),
    (64, 8, 64, 96, 40, "bf16", False),
    (1, 16, 1, 8, 8, "bf16", True),
    (16, 128, 4, 264, 1032, "bf16", True),
    (3, 1, 3, 24, 16, "bf16", False),
    # every (tile, rank mode) kernel: r a multiple of 8 but not a power of two, and
    # r not a multiple of 8, on both the 64-row and the 128-row tiles
    (4, 24, 2, 136, 264, "bf16", True),
    (6, 40, 3, 264, 392, "bf16", False),
    (8, 12, 8, 136, 264, "bf16", True),
    (8, 16, 4, 200, 136, "bf16", False),
    # r a power of two and a multiple of the K chunk: one slot per chunk
    (4, 64, 1, 136, 264, "bf16", True),
    (6, 32, 1, 72, 136, "bf16", False),
    (5, 128, 3, 200, 392, "bf16", True),
    # long contractions (128 x 128 tiles, 64-deep chunks): two slots per chunk (r = 32),
    # a slot ending inside a half-empty last chunk on a matrix narrower than a tile
    # (r = 96), eight one-slot chunks, and a matrix smaller than a tile
    (8, 32, 3, 136, 264, "bf16", False),
    (4, 96, 1, 72, 40, "bf16", True),
    (16, 64, 8, 264, 1032, "bf16", False),
    (3, 64, 2, 8, 64, "bf16", True),
    # every rank mode of each tile class: k*r <= 32 (32 x 256 tiles) with r = 24, and
    # k*r <= 64 (64 x 128) with r = 20
    (5, 24, 1, 72, 520, "bf16", True),
    (4, 20, 3, 136, 264, "bf16", False),
]


def make_selection(E, k, d, dt, seed):
    h, R, _ = gapped_router(E, d, dt, seed)
    return oracle_selection(h, R, k)


@pytest.mark.parametrize("E,r,k,d_out,d_in,dt,inplace", MERGE_CASES)
def test_merge_matches_oracle(E, r, k, d_out, d_in, dt, inplace):
    W, Aw, Bw = synth.adapter_bank(7, E, r, d_out, d_in, dt)
    idx, gate = make_selection(E, k, 64, dt, 3)
    s = 2.0
    ref = O.merge(to64(W), to64(Aw), to64(Bw), idx.numpy(), gate.numpy().astype(np.float64), s)
    w = W.to(DEV)
    out = None if inplace else torch.full_like(w, float("nan"))
    m = A.AdaModel([(w, out, Aw.to(DEV), Bw.to(DEV))], E, r)
    A.ada_merge(m, idx.to(DEV), gate.to(DEV), s)
    sync()
    got = w if inplace else out
    check_close(got, ref, *tol(TD[dt]), "merge")
    if not inplace:
        assert torch.equal(w.cpu(), W), "out-of-place merge must not write W"


def _random_merge_cases(n: int = 32, seed: int = 20261203):
    """Seeded draws over the whole admitted range: E up to 64, ranks from 1 to 256
    (every rank mode), k up to min(E, 512 / r) (every tile class), ragged shapes, both
    storage types, in and out of place."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        E = int(rng.integers(1, 65))
        r = int(rng.choice([1, 3, 5, 8, 12, 16, 20, 24, 32, 40, 48, 64, 96, 128, 256]))
        kmax = min(E, 512 // r)
        k = int(rng.integers(1, kmax + 1))
        d_out, d_in = 8 * int(rng.integers(1, 90)), 8 * int(rng.integers(1, 90))
        dt = "bf16" if rng.random() < 0.75 else "fp32"
        cases.append((E, r, k, d_out, d_in, dt, bool(rng.random() < 0.5)))
    return cases


def _merge_within_tolerance(E, r, k, d_out, d_in, dt, inplace, seed):
    W, Aw, Bw = synth.adapter_bank(seed, E, r, d_out, d_in, dt)
    idx, gate = make_selection(E, k, 64, dt, 5)
    g64 = gate.numpy().astype(np.float64)
    ref = O.merge(to64(W), to64(Aw), to64(Bw), idx.numpy(), g64, 2.0)
    w = W.to(DEV)
    out = None if inplace else torch.full_like(w, float("nan"))
    m = A.AdaModel([(w, out, Aw.to(DEV), Bw.to(DEV))], E, r)
    A.ada_merge(m, idx.to(DEV), gate.to(DEV), 2.0)
    sync()
    got = to64(w if inplace else out)
    rtol, atol = tol(TD[dt])
    bound = rtol * np.abs(ref) + atol
    if dt == "fp32":
        bound = bound + fp32_accumulation_bound(Aw, Bw, [(e, g, 2.0) for e, g in zip(idx.tolist(), gate.tolist())])
    err = np.abs(got - ref)
    assert (err <= bound).all(), (float(np.max(err / bound)), int((err > bound).sum()))
    if not inplace:
        assert torch.equal(w.cpu(), W), "out-of-place merge must not write W"
    m.destroy()


@pytest.mark.parametrize("E,r,k,d_out,d_in,dt,inplace", _random_merge_cases())
def test_merge_matches_oracle_on_random_shapes(E, r, k, d_out, d_in, dt, inplace):
    """bf16: the stated tolerance, nothing added.  fp32 storage: its tolerance plus the
    fp32 accumulation of k r products (which small d_in, hence large A, can reach)."""
    _merge_within_tolerance(E, r, k, d_out, d_in, dt, inplace, 17 + d_out + d_in)


def _small_input_cases(n: int = 16, seed: int = 20261205):
    """Long contractions on narrow inputs: d_in from 8 to 64 makes A ~ N(0, 1/sqrt(d_in))
    large, so the delta's terms reach the size of the weights and merged weights cancel;
    k r >= 128 (every long rank mode: r a multiple of 64, r = 32, and r not a multiple
    of 32), bf16 only."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        r = int(rng.choice([8, 16, 24, 32, 40, 64, 128, 256]))
        E = int(rng.integers(max(2, -(-128 // r)), 65))
        kmin = -(-128 // r)
        kmax = min(E, 512 // r)
        if kmin > kmax:
            continue
        k = int(rng.integers(kmin, kmax + 1))
        d_in = 8 * int(rng.integers(1, 9))
        d_out = 8 * int(rng.integers(1, 40))
        cases.append((E, r, k, d_out, d_in, "bf16", bool(rng.random() < 0.5)))
    return cases


@pytest.mark.parametrize("E,r,k,d_out,d_in,dt,inplace", _small_input_cases())
def test_long_contractions_on_narrow_inputs_meet_the_stated_tolerance(E, r, k, d_out, d_in, dt, inplace):
    _merge_within_tolerance(E, r, k, d_out, d_in, dt, inplace, 101 + d_out + d_in)


# W and each adapter bank are addressed with 32-bit byte offsets; the library admits
# operands of fewer than 2^31 elements and dimensions up to 2^22.  One operand or
# dimension per case sits at its limit.
LIMIT_CASES = [
    # E, r, k, d_out, d_in, operand at the limit
    (2, 16, 2, 32768, 65528, "W"),   # W: 2,147,221,504 elements (32 x 256 tiles)
    (64, 256, 1, 8, 131064, "A"),    # A: 64 x 256 x 131064 = 2,147,352,576 elements (128 x 128 tiles)
    (64, 256, 1, 131064, 8, "B"),    # B: the same count
    (1, 8, 1, 8, 4194304, "d_in"),   # the largest dimension accepted (2^22 columns)
    (1, 8, 1, 4194304, 8, "d_out"),  # and rows
]


@pytest.mark.parametrize("E,r,k,d_out,d_in,big", LIMIT_CASES)
def test_operands_at_the_32_bit_offset_limit(E, r, k, d_out, d_in, big):
    """The last expert is selected, so the gathers reach the top of the banks; the
    checked rows include the last rows of W."""
    assert max(d_out * d_in, E * r * d_in, E * r * d_out) < 2 ** 31
    seed = 11
    w = synth.device_normal(synth.tensor_seed(seed, "limit", big, "W"), (d_out, d_in), 0.02, "bf16", DEV)
    a = synth.device_normal(synth.tensor_seed(seed, "limit", big, "A"), (E, r, d_in), 1.0 / np.sqrt(d_in), "bf16", DEV)
    b = synth.device_normal(synth.tensor_seed(seed, "limit", big, "B"), (E, d_out, r), 0.01, "bf16", DEV)
    sel = [E - 1, 0][:k]
    idx = torch.tensor(sel, dtype=torch.int32)
    gate = torch.tensor([0.625, 0.375][:k] if k == 2 else [1.0], dtype=torch.float32)
    rows = np.arange(d_out) if d_out * d_in <= (1 << 21) else \
        sample_rows(d_out, np.random.default_rng(seed), merge_tile_rows(k * r))
    rows_t = torch.from_numpy(rows).to(DEV)
    w0 = to64(w[rows_t])
    a_sel = to64(a[idx.long().to(DEV)])                 # the selected experts only
    b_sel = to64(b[idx.long().to(DEV)][:, rows_t, :])
    s = 2.0
    ref = O.merge(w0, a_sel, b_sel, np.arange(k), gate.numpy().astype(np.float64), s)
    m = A.AdaModel([(w, None, a, b)], E, r)
    A.ada_merge(m, idx.to(DEV), gate.to(DEV), s)
    sync()
    check_close(w[rows_t], ref, BF16_RTOL, BF16_ATOL, f"merge with {big} at the offset limit")
    m.destroy()
    del w, a, b
    torch.cuda.empty_cache()


def test_heavy_cancellation_meets_the_stated_tolerance():
    """d_in = 16 makes A ~ N(0, 1/4), so k*r = 128 terms of |s g b a| sum to ~0.2
    against weights of ~0.02: some merged weights cancel to ~1e-3.  A gate folded into
    B in a single bf16 plane (error up to 2^-8 of that sum) put one weight at 1.06x the
    stated bound here; the kernels carry the coefficient at fp32 accuracy and must meet
    the stated tolerance itself."""
    E, r, k, d_out, d_in = 3, 64, 2, 8, 16
    W, Aw, Bw = synth.adapter_bank(7, E, r, d_out, d_in, "bf16")
    idx, gate = make_selection(E, k, 64, "bf16", 3)
    g64 = gate.numpy().astype(np.float64)
    ref = O.merge(to64(W), to64(Aw), to64(Bw), idx.numpy(), g64, 2.0)
    w = W.to(DEV)
    m = A.AdaModel([(w, None, Aw.to(DEV), Bw.to(DEV))], E, r)
    A.ada_merge(m, idx.to(DEV), gate.to(DEV), 2.0)
    sync()
    check_close(w, ref, BF16_RTOL, BF16_ATOL, "merge with cancelling weights")


ARITH_CASES = [
    # E, r, k, d_out, d_in: each tile class and rank mode, and the cancelling case above
    (8, 16, 2, 384, 520),     # k r = 32: single chunk, split fold
    (5, 24, 1, 72, 520),      # r not a multiple of 8: element gather
    (8, 16, 4, 200, 136),     # k r = 64: two chunks, split fold
    (4, 20, 3, 136, 264),     # k r = 60, element gather
    (16, 64, 4, 136, 264),    # long, r a multiple of 64: scaled accumulators
    (8, 32, 6, 136, 264),     # long, r = 32: scaled accumulators on 32-deep chunks
    (8, 12, 8, 136, 264),     # long, r not a multiple of 32: split fold
    (3, 64, 2, 8, 16),        # cancelling weights
]


@pytest.mark.parametrize("E,r,k,d_out,d_in", ARITH_CASES)
def test_merge_error_is_one_rounding(E, r, k, d_out, d_in):
    """Tighter than the stated tolerance: |W'_gpu - ref| <= 2^-8 |ref| + ~(2^-16 +
    fp32 accumulation) of the terms' magnitude (kernel_error_bound), ref the oracle's
    exact merge: only the final bf16 rounding is visible, the coefficient is carried at
    fp32 accuracy.  The same for a fused switch (both selections in one accumulation)."""
    W, Aw, Bw = synth.adapter_bank(7, E, r, d_out, d_in, "bf16")
    idx, gate = make_selection(E, k, 64, "bf16", 3)
    s = 2.0
    g64 = gate.numpy().astype(np.float64)
    ref = O.merge(to64(W), to64(Aw), to64(Bw), idx.numpy(), g64, s)
    w = W.to(DEV)
    m = A.AdaModel([(w, None, Aw.to(DEV), Bw.to(DEV))], E, r)
    A.ada_merge(m, idx.to(DEV), gate.to(DEV), s)
    sync()
    slots = [(e, g, s) for e, g in zip(idx.tolist(), gate.tolist())]
    bound = kernel_error_bound(W, Aw, Bw, slots, ref)
    err = np.abs(to64(w) - ref)
    assert (err <= bound).all(), float(np.max(err / bound))
    m.destroy()
    # the fused switch on a fresh copy of W: both selections' slots in one accumulation
    ci, cg = make_selection(E, k, 64, "bf16", 4)
    if (2 * k) * r > 512:
        return
    ref2 = O.switch(to64(W), to64(Aw), to64(Bw), (idx.numpy(), g64), (ci.numpy(), cg.numpy().astype(np.float64)), s)
    w2 = W.to(DEV)
    m2 = A.AdaModel([(w2, None, Aw.to(DEV), Bw.to(DEV))], E, r)
    A.ada_switch(m2, (idx.to(DEV), gate.to(DEV)), (ci.to(DEV), cg.to(DEV)), s)
    sync()
    slots2 = [(e, g, -s) for e, g in zip(idx.tolist(), gate.tolist())] + \
        [(e, g, s) for e, g in zip(ci.tolist(), cg.tolist())]
    bound2 = kernel_error_bound(W, Aw, Bw, slots2, ref2)
    err2 = np.abs(to64(w2) - ref2)
    assert (err2 <= bound2).all(), float(np.max(err2 / bound2))
    m2.destroy()


COEF_CASES = [
    # r, gates of the first selection, gates of the second (None: a merge, else a switch)
    (64, [1.0, 1e-30, 0.5], None),                 # ratio 1e-30 between neighbours in |c| order
    (64, [1e-39, 1.0], None),                      # a subnormal gate
    (64, [0.25, 0.25, 0.25, 0.25], None),          # equal magnitudes: ties keep their order
    (64, [0.7, 0.3], [0.3, 0.7]),                  # a switch: equal |c| with opposite signs
    (128, [0.6, 0.4], [0.9, 0.1]),                 # two 64-deep chunks per slot
    (32, [0.5, 0.3, 0.2], [0.6, 0.4]),             # rank 32: 32-deep chunks, one slot each
    (64, [0.5, 0.3, 0.2], None),                   # three slots: a half-empty last pair of chunks
]


@pytest.mark.parametrize("r,g1,g2", COEF_CASES)
def test_scaled_accumulators_on_extreme_and_tied_coefficients(r, g1, g2):
    """Long contractions whose chunks each hold one slot keep B raw and rescale the fp32
    accumulators between slots in order of increasing |c|: extreme ratios must neither
    overflow nor lose the large slot, ties and opposite signs must not drop a slot, and
    the result is the stated tolerance away from the exact merge (or switch)."""
    E, d_out, d_in = 8, 136, 264
    W, Aw, Bw = synth.adapter_bank(61 + r, E, r, d_out, d_in, "bf16")
    i1 = torch.tensor([1, 4, 6, 0][:len(g1)], dtype=torch.int32)
    t1 = torch.tensor(g1, dtype=torch.float32)
    W64, A64, B64 = to64(W), to64(Aw), to64(Bw)
    w = W.to(DEV)
    m = A.AdaModel([(w, None, Aw.to(DEV), Bw.to(DEV))], E, r)
    if g2 is None:
        assert len(g1) * r > 64
        ref = O.merge(W64, A64, B64, i1.numpy(), t1.numpy().astype(np.float64), 2.0)
        A.ada_merge(m, i1.to(DEV), t1.to(DEV), 2.0)
    else:
        i2 = torch.tensor([2, 1, 7][:len(g2)], dtype=torch.int32)
        t2 = torch.tensor(g2, dtype=torch.float32)
        assert (len(g1) + len(g2)) * r > 64
        ref = O.switch(W64, A64, B64, (i1.numpy(), t1.numpy().astype(np.float64)),
                       (i2.numpy(), t2.numpy().astype(np.float64)), 2.0)
        A.ada_switch(m, (i1.to(DEV), t1.to(DEV)), (i2.to(DEV), t2.to(DEV)), 2.0)
    sync()
    got = to64(w)
    assert np.all(np.isfinite(got))
    check_close(got, ref, BF16_RTOL, BF16_ATOL, f"scaled accumulators r={r} gates {g1} {g2}")
    m.destroy()


@pytest.mark.parametrize("E,r,k", [(8, 16, 2), (8, 16, 4), (16, 64, 4)])  # each tile class
def test_stack_of_mixed_shapes_in_one_launch(E, r, k):
    """Several projections of different shapes in one model (one launch): every
    projection gets its own adapters and the same selection."""
    dt = "bf16"
    shapes = [(256, 256), (64, 256), (688, 256), (256, 688), (8, 8), (136, 1000)] * 2
    banks = [synth.adapter_bank(100 + i, E, r, do, di, dt) for i, (do, di) in enumerate(shapes)]
    idx, gate = make_selection(E, k, 256, dt, 9)
    dev = [(W.to(DEV), None, Aw.to(DEV), Bw.to(DEV)) for W, Aw, Bw in banks]
    m = A.AdaModel(dev, E, r)
    A.ada_merge(m, idx.to(DEV), gate.to(DEV), 2.0)
    sync()
    for (W, Aw, Bw), (w, _, _, _) in zip(banks, dev):
        ref = O.merge(to64(W), to64(Aw), to64(Bw), idx.numpy(), gate.numpy().astype(np.float64), 2.0)
        check_close(w, ref, *tol(torch.bfloat16), f"merge {tuple(W.shape)}")


@pytest.mark.parametrize("E,r,k", [(8, 16, 2), (8, 16, 4), (16, 64, 4)])  # each tile class
@pytest.mark.parametrize("inplace", [True, False])
def test_row_strided_weights(E, r, k, inplace):
    """W (and W') with a row stride larger than d_in (column slices of wider matrices)."""
    big, Aw, Bw = synth.adapter_bank(21, E, r, 264, 512, "bf16")
    W = big[:, :392]  # ld 512, d_in 392
    Aw = Aw[:, :, :392].contiguous()
    idx, gate = make_selection(E, k, 64, "bf16", 4)
    ref = O.merge(to64(W), to64(Aw), to64(Bw), idx.numpy(), gate.numpy().astype(np.float64), 2.0)
    wbig = big.to(DEV)
    w = wbig[:, :392]
    obig = torch.full_like(wbig, float("nan"))
    out = None if inplace else obig[:, :392]
    m = A.AdaModel([(w, out, Aw.to(DEV), Bw.to(DEV))], E, r)
    A.ada_merge(m, idx.to(DEV), gate.to(DEV), 2.0)
    sync()
    check_close(w if inplace else out, ref, *tol(torch.bfloat16), f"strided merge, k*r = {k * r}")
    assert torch.equal(wbig[:, 392:].cpu(), big[:, 392:]), "columns past d_in must stay untouched"
    if not inplace:
        assert torch.equal(wbig.cpu(), big), "an out-of-place merge must not write W"
        assert torch.isnan(obig[:, 392:]).all(), "columns past d_in of W' must stay untouched"
    m.destroy()


@pytest.mark.parametrize("dt,r", [("bf16", 16), ("bf16", 64), ("fp32", 16)])
def test_zero_gates_leave_w_bit_identical(dt, r):
    E, k = 4, 2
    W, Aw, Bw = synth.adapter_bank(31, E, r, 200, 264, dt)
    W[0, :8] = -0.0
    w = W.to(DEV)
    out = torch.full_like(w, float("nan"))
    idx = torch.tensor([1, 3], dtype=torch.int32, device=DEV)
    gate = torch.zeros(2, dtype=torch.float32, device=DEV)
    m_in = A.AdaModel([(w, None, Aw.to(DEV), Bw.to(DEV))], E, r)
    m_out = A.AdaModel([(w, out, Aw.to(DEV), Bw.to(DEV))], E, r)
    A.ada_merge(m_in, idx, gate, 2.0)
    A.ada_merge(m_out, idx, gate, 2.0)
    sync()
    assert w.cpu().view(torch.int16 if dt == "bf16" else torch.int32).equal(
        W.view(torch.int16 if dt == "bf16" else torch.int32))
    assert out.cpu().view(torch.int16 if dt == "bf16" else torch.int32).equal(
        W.view(torch.int16 if dt == "bf16" else torch.int32))


@pytest.mark.parametrize("r", [16, 64])
def test_zero_gated_slot_is_dropped(r):
    E = 4
    W, Aw, Bw = synth.adapter_bank(32, E, r, 128, 128, "bf16")
    Aw[1, 0, 5] = float("inf")
    idx = torch.tensor([1, 2], dtype=torch.int32)
    gate = torch.tensor([0.0, 0.7], dtype=torch.float32)
    ref = O.merge(to64(W), to64(Aw), to64(Bw), idx.numpy(), gate.numpy().astype(np.float64), 2.0)
    w = W.to(DEV)
    m = A.AdaModel([(w, None, Aw.to(DEV), Bw.to(DEV))], E, r)
    A.ada_merge(m, idx.to(DEV), gate.to(DEV), 2.0)
    sync()
    assert torch.isfinite(w).all()
    check_close(w, ref, *tol(torch.bfloat16), "zero-gated slot")


def test_single_expert_unit_gate_is_static_lora():
    E, r = 3, 16
    W, Aw, Bw = synth.adapter_bank(33, E, r, 256, 384, "bf16")
    ref = to64(W) + 2.0 * to64(Bw[2]) @ to64(Aw[2])
    w = W.to(DEV)
    m = A.AdaModel([(w, None, Aw.to(DEV), Bw.to(DEV))], E, r)
    A.ada_merge(m, torch.tensor([2], dtype=torch.int32, device=DEV), torch.ones(1, device=DEV), 2.0)
    sync()
    check_close(w, ref, *tol(torch.bfloat16), "k=1 static merge")


def test_out_of_range_index_is_skipped():
    E, r = 4, 8
    W, Aw, Bw = synth.adapter_bank(34, E, r, 64, 64, "bf16")
    idx = torch.tensor([7, 1], dtype=torch.int32)
    gate = torch.tensor([0.5, 0.5], dtype=torch.float32)
    ref = O.merge(to64(W), to64(Aw), to64(Bw), [1], [0.5], 2.0)
    w = W.to(DEV)
    m = A.AdaModel([(w, None, Aw.to(DEV), Bw.to(DEV))], E, r)
    A.ada_merge(m, idx.to(DEV), gate.to(DEV), 2.0)
    sync()
    check_close(w, ref, *tol(torch.bfloat16), "out-of-range slot")


# ---------------------------------------------------------------- unmerge / switch


@pytest.mark.parametrize("dt,E,r,k", [("bf16", 8, 16, 2), ("bf16", 16, 64, 4), ("fp32", 4, 8, 2)])
def test_unmerge_matches_oracle(dt, E, r, k):
    W, Aw, Bw = synth.adapter_bank(41, E, r, 264, 392, dt)
    idx, gate = make_selection(E, k, 64, dt, 5)
    ref = O.unmerge(to64(W), to64(Aw), to64(Bw), idx.numpy(), gate.numpy().astype(np.float64), 2.0)
    w = W.to(DEV)
    m = A.AdaModel([(w, None, Aw.to(DEV), Bw.to(DEV))], E, r)
    A.ada_unmerge(m, idx.to(DEV), gate.to(DEV), 2.0)
    sync()
    check_close(w, ref, *tol(TD[dt]), "unmerge")


@pytest.mark.parametrize("inplace", [True, False])
def test_merge_then_unmerge_returns_w(inplace):
    E, r, k = 8, 16, 2
    W, Aw, Bw = synth.adapter_bank(42, E, r, 520, 392, "bf16")
    idx, gate = make_selection(E, k, 64, "bf16", 6)
    w = W.to(DEV)
    out = None if inplace else torch.empty_like(w)
    m = A.AdaModel([(w, out, Aw.to(DEV), Bw.to(DEV))], E, r)
    A.ada_merge(m, idx.to(DEV), gate.to(DEV), 2.0)
    A.ada_unmerge(m, idx.to(DEV), gate.to(DEV), 2.0)
    sync()
    buf = w if inplace else out
    check_close(buf, to64(W), *tol(torch.bfloat16), "merge->unmerge")
    # bf16 subtraction does not undo bf16 addition exactly; the bit-exact fraction
    # must match two round-to-nearest steps simulated on the oracle's delta
    delta = O.adapter_delta(to64(Aw), to64(Bw), idx.numpy(), 2.0 * gate.numpy().astype(np.float64))
    w1 = torch.from_numpy(to64(W) + delta).to(torch.bfloat16)
    w2 = torch.from_numpy(to64(w1) - delta).to(torch.bfloat16)
    expect = (w2.view(torch.int16) == W.view(torch.int16)).float().mean().item()
    exact = (buf.cpu().view(torch.int16) == W.view(torch.int16)).float().mean().item()
    assert exact >= expect - 0.02, (exact, expect)
    if not inplace:
        assert torch.equal(w.cpu(), W)


@pytest.mark.parametrize("r,E,kp,kc", [(8, 8, 2, 2), (16, 8, 2, 2), (16, 8, 2, 3), (32, 8, 2, 3), (128, 4, 2, 2),
                                        (8, 64, 32, 32)])
def test_switch_matches_oracle(r, E, kp, kc):
    """Undo one selection and apply another in one pass, in every tile class ((k_prev +
    k_cur) * r = 32, 64, 80 and up) up to the largest contraction one launch takes
    (512, in 4 or in 64 slots)."""
    W, Aw, Bw = synth.adapter_bank(43, E, r, 264, 520, "bf16")
    pi, pg = make_selection(E, kp, 64, "bf16", 7)
    ci, cg = make_selection(E, kc, 64, "bf16", 8)
    ref = O.switch(to64(W), to64(Aw), to64(Bw), (pi.numpy(), pg.numpy().astype(np.float64)),
                   (ci.numpy(), cg.numpy().astype(np.float64)), 2.0)
    w = W.to(DEV)
    m = A.AdaModel([(w, None, Aw.to(DEV), Bw.to(DEV))], E, r)
    A.ada_switch(m, (pi.to(DEV), pg.to(DEV)), (ci.to(DEV), cg.to(DEV)), 2.0)
    sync()
    check_close(w, ref, *tol(torch.bfloat16), "switch")


def _random_switch_cases(n: int = 12, seed: int = 20261204):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        E = int(rng.integers(2, 65))
        r = int(rng.choice([1, 5, 8, 12, 16, 24, 32, 48, 64, 128]))
        kp = int(rng.integers(1, min(E, max(1, 512 // r - 1)) + 1))
        kc = int(rng.integers(1, min(E, 512 // r - kp) + 1)) if 512 // r - kp >= 1 else 0
        if kc < 1:
            continue
        cases.append((E, r, kp, kc, 8 * int(rng.integers(1, 60)), 8 * int(rng.integers(1, 60))))
    return cases


@pytest.mark.parametrize("E,r,kp,kc,d_out,d_in", _random_switch_cases())
def test_switch_matches_oracle_on_random_shapes(E, r, kp, kc, d_out, d_in):
    """Seeded draws of the fused switch: (k_prev + k_cur) r up to 512, ragged shapes;
    the stated tolerance, nothing added."""
    W, Aw, Bw = synth.adapter_bank(29 + d_out + d_in, E, r, d_out, d_in, "bf16")
    pi, pg = make_selection(E, kp, 64, "bf16", 11)
    ci, cg = make_selection(E, kc, 64, "bf16", 13)
    p64, c64 = pg.numpy().astype(np.float64), cg.numpy().astype(np.float64)
    ref = O.switch(to64(W), to64(Aw), to64(Bw), (pi.numpy(), p64), (ci.numpy(), c64), 2.0)
    w = W.to(DEV)
    m = A.AdaModel([(w, None, Aw.to(DEV), Bw.to(DEV))], E, r)
    A.ada_switch(m, (pi.to(DEV), pg.to(DEV)), (ci.to(DEV), cg.to(DEV)), 2.0)
    sync()
    check_close(w, ref, BF16_RTOL, BF16_ATOL, "switch")
    m.destroy()


# ---------------------------------------------------------------- invariants


def test_merge_is_deterministic():
    E, r, k = 16, 64, 4
    W, Aw, Bw = synth.adapter_bank(51, E, r, 392, 520, "bf16")
    idx, gate = make_selection(E, k, 64, "bf16", 9)
    w = W.to(DEV)
    o1, o2 = torch.empty_like(w), torch.empty_like(w)
    a, b = Aw.to(DEV), Bw.to(DEV)
    m1 = A.AdaModel([(w, o1, a, b)], E, r)
    m2 = A.AdaModel([(w, o2, a, b)], E, r)
    A.ada_merge(m1, idx.to(DEV), gate.to(DEV), 2.0)
    A.ada_merge(m2, idx.to(DEV), gate.to(DEV), 2.0)
    sync()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_expert_relabelling_is_bit_identical():
    """Permute the adapter banks together with the router rows: the GPU selects the
    permuted experts in the same order and writes bit-identical weights."""
    E, r, k, d = 8, 16, 2, 256
    W, Aw, Bw = synth.adapter_bank(52, E, r, 256, 256, "bf16")
    h, R, _ = gapped_router(E, d, "bf16", 77)
    perm = torch.tensor(np.random.default_rng(0).permutation(E))
    outs = []
    for P in (torch.arange(E), perm):
        w = W.to(DEV)
        idx, gate = A.ada_pregate(h.to(DEV), R[P].contiguous().to(DEV), k)
        m = A.AdaModel([(w, None, Aw[P].contiguous().to(DEV), Bw[P].contiguous().to(DEV))], E, r)
        A.ada_merge(m, idx, gate, 2.0)
        sync()
        outs.append((w.cpu(), P[idx.cpu().long()]))
    assert torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))


def test_pregate_then_merge_chain():
    """GPU pregate feeding GPU merge (no host round trip) vs oracle pregate + merge."""
    E, r, k, d = 16, 64, 4, 1024
    W, Aw, Bw = synth.adapter_bank(53, E, r, 264, 1024, "bf16")
    h, R, _ = gapped_router(E, d, "bf16", 99)
    ridx, rg = O.pregate(to64(h), to64(R), k)
    ref = O.merge(to64(W), to64(Aw), to64(Bw), ridx, rg, 2.0)
    w = W.to(DEV)
    m = A.AdaModel([(w, None, Aw.to(DEV), Bw.to(DEV))], E, r)
    idx, gate = A.ada_pregate(h.to(DEV), R.to(DEV), k)
    A.ada_merge(m, idx, gate, 2.0)
    sync()
    check_close(w, ref, *tol(torch.bfloat16), "pregate->merge")


# ---------------------------------------------------------------- decode GEMV and baseline

GEMV_CASES = [(4096, 4096, "bf16"), (11008, 4096, "bf16"), (4096, 11008, "bf16"), (8, 8, "bf16"),
              (264, 1000, "bf16"), (256, 256, "fp32"), (520, 72, "fp32"), (1024, 8192, "bf16")]


def gemv_bound(W64, x64, y_ref, dt):
    mag = np.abs(W64) @ np.abs(x64)
    if dt == "bf16":
        return 8e-3 * np.abs(y_ref) + 1e-4 * mag
    return 1e-6 * np.abs(y_ref) + 1e-5 * mag


@pytest.mark.parametrize("d_out,d_in,dt", GEMV_CASES)
def test_decode_gemv_matches_oracle(d_out, d_in, dt):
    W, _, _ = synth.adapter_bank(61, 1, 8, d_out, d_in, dt)
    x = synth.host_normal(synth.tensor_seed(62, d_in), (d_in,), 1.0, dt)
    y = A.ada_decode_gemv(W.to(DEV), x.to(DEV))
    sync()
    W64, x64 = to64(W), to64(x)
    ref = O.gemv(W64, x64)
    err = np.abs(to64(y) - ref)
    assert np.all(err <= gemv_bound(W64, x64, ref, dt)), float(err.max())


@pytest.mark.parametrize("dt,E,r,k", [("bf16", 8, 16, 2), ("bf16", 16, 64, 4), ("fp32", 4, 8, 2)])
def test_lora_apply_matches_oracle(dt, E, r, k):
    d_out, d_in = 1032, 520
    W, Aw, Bw = synth.adapter_bank(63, E, r, d_out, d_in, dt)
    x = synth.host_normal(synth.tensor_seed(64, d_in), (d_in,), 1.0, dt)
    idx, gate = make_selection(E, k, 64, dt, 10)
    y = A.ada_lora_apply(W.to(DEV), Aw.to(DEV), Bw.to(DEV), idx.to(DEV), gate.to(DEV), 2.0, x.to(DEV))
    sync()
    ref = O.routed_lora_forward(to64(W), to64(Aw), to64(Bw), idx.numpy(), gate.numpy().astype(np.float64),
                                2.0, to64(x))
    W64, x64 = to64(W), to64(x)
    mag = np.abs(W64) @ np.abs(x64)
    err = np.abs(to64(y) - ref)
    assert np.all(err <= gemv_bound(W64, x64, ref, dt) + 1e-4 * mag), float(err.max())


def test_merged_decode_equals_routed_baseline():
    """Linearity through bf16 rounding: GEMV on the merged weights vs the unmerged
    routed projection, relative L2 within 5e-3 (a dropped adapter gives ~4%)."""
    E, r, k = 8, 16, 2
    W, Aw, Bw = synth.adapter_bank(65, E, r, 4096, 4096, "bf16")
    x = synth.host_normal(synth.tensor_seed(66, 4096), (4096,), 1.0, "bf16").to(DEV)
    idx, gate = make_selection(E, k, 64, "bf16", 11)
    w = W.to(DEV)
    a, b = Aw.to(DEV), Bw.to(DEV)
    y_base = A.ada_lora_apply(w, a, b, idx.to(DEV), gate.to(DEV), 2.0, x)
    m = A.AdaModel([(w, None, a, b)], E, r)
    A.ada_merge(m, idx.to(DEV), gate.to(DEV), 2.0)
    y_m = A.ada_decode_gemv(w, x)
    sync()
    yb, ym = to64(y_base), to64(y_m)
    rel = np.linalg.norm(ym - yb) / np.linalg.norm(yb)
    assert rel <= 5e-3, rel


# ---------------------------------------------------------------- API errors on a live model


def test_live_model_rejects_bad_selections():
    E, r = 4, 128
    W, Aw, Bw = synth.adapter_bank(71, E, r, 64, 64, "bf16")
    m = A.AdaModel([(W.to(DEV), None, Aw.to(DEV), Bw.to(DEV))], E, r)
    idx = torch.zeros(4, dtype=torch.int32, device=DEV)
    gate = torch.zeros(4, dtype=torch.float32, device=DEV)
    with pytest.raises(A.AdaError) as ei:
        A.ada_merge(m, idx, gate, 2.0)  # k*r = 512 is fine
        A.ada_switch(m, (idx, gate), (idx, gate), 2.0)  # 8*128 > 512
    assert ei.value.status == -2
    with pytest.raises(A.AdaError):
        A.ada_merge(m, idx[:0], gate[:0], 2.0)
    m.destroy()
    with pytest.raises(RuntimeError):
        A.ada_merge(m, idx, gate, 2.0)


def test_binding_rejects_tensors_the_c_calls_would_misread():
    """The binding hands the C calls bare pointers, so a strided view, a wrong shape or
    a wrong dtype must be refused before any launch; nothing below reaches the GPU."""
    E, r, k, d_out, d_in = 4, 8, 2, 16, 24
    W, Aw, Bw = synth.adapter_bank(72, E, r, d_out, d_in, "bf16")
    w, a, b = W.to(DEV), Aw.to(DEV), Bw.to(DEV)
    m = A.AdaModel([(w, None, a, b)], E, r)
    idx = torch.tensor([0, 1, 2, 3], dtype=torch.int32, device=DEV)
    gate = torch.full((4,), 0.25, dtype=torch.float32, device=DEV)
    before = w.clone()
    with pytest.raises(ValueError):
        A.ada_merge(m, idx[::2], gate[:2], 2.0)  # strided idx
    with pytest.raises(ValueError):
        A.ada_merge(m, idx.view(2, 2), gate.view(2, 2), 2.0)  # not one-dimensional
    with pytest.raises(TypeError):
        A.ada_merge(m, idx.long(), gate, 2.0)
    x = torch.ones(d_in, dtype=torch.bfloat16, device=DEV)
    for y in (torch.empty(d_out + 8, dtype=torch.bfloat16, device=DEV),
              torch.empty(2 * d_out, dtype=torch.bfloat16, device=DEV)[::2],
              torch.empty(d_out, dtype=torch.float32, device=DEV)):
        with pytest.raises(ValueError):
            A.ada_decode_gemv(w, x, y)
        with pytest.raises(ValueError):
            A.ada_lora_apply(w, a, b, idx[:k], gate[:k], 2.0, x, y)
    with pytest.raises(ValueError):
        A.ada_lora_apply(w, a, b, idx[:k], gate[:k], 2.0, x[:8])
    with pytest.raises(TypeError):
        A.ada_lora_apply(w, a, b.float(), idx[:k], gate[:k], 2.0, x)
    y = torch.empty(d_out, dtype=torch.float32, device=DEV)
    with pytest.raises(TypeError):
        A.ada_lora_layer([(w, a, b, x, y)], idx[:k], gate[:k], 2.0)
    with pytest.raises(ValueError):
        A.ada_pregate(x, w[:, :d_in].contiguous()[:E], k, idx_out=torch.empty(k, dtype=torch.int64, device=DEV))
    sync()
    assert torch.equal(w, before)
    m.destroy()


# ---------------------------------------------------------------- fused unmerged layer (comparator)


@pytest.mark.parametrize("dt,E,r,k", [("bf16", 8, 16, 2), ("bf16", 16, 64, 4), ("fp32", 4, 8, 2)])
def test_lora_layer_matches_oracle_and_the_three_launch_path(dt, E, r, k):
    shapes = [(264, 520), (1032, 264), (8, 8), (520, 1032), (136, 136)]
    idx, gate = make_selection(E, k, 64, dt, 12)
    banks = [synth.adapter_bank(200 + i, E, r, do, di, dt) for i, (do, di) in enumerate(shapes)]
    xs = [synth.host_normal(synth.tensor_seed(300 + i, di), (di,), 1.0, dt) for i, (_, di) in enumerate(shapes)]
    dev = [(W.to(DEV), Aw.to(DEV), Bw.to(DEV), x.to(DEV)) for (W, Aw, Bw), x in zip(banks, xs)]
    ys = [torch.full((W.shape[0],), float("nan"), dtype=TD[dt], device=DEV) for W, _, _ in banks]
    A.ada_lora_layer([(w, a, b, x, y) for (w, a, b, x), y in zip(dev, ys)], idx.to(DEV), gate.to(DEV), 2.0)
    ref3 = [A.ada_lora_apply(w, a, b, idx.to(DEV), gate.to(DEV), 2.0, x) for w, a, b, x in dev]
    sync()
    for (W, Aw, Bw), x, y, y3 in zip(banks, xs, ys, ref3):
        assert torch.equal(y.cpu().view(torch.int16 if dt == "bf16" else torch.int32),
                           y3.cpu().view(torch.int16 if dt == "bf16" else torch.int32))
        ref = O.routed_lora_forward(to64(W), to64(Aw), to64(Bw), idx.numpy(), gate.numpy().astype(np.float64),
                                    2.0, to64(x))
        W64, x64 = to64(W), to64(x)
        mag = np.abs(W64) @ np.abs(x64)
        err = np.abs(to64(y) - ref)
        assert np.all(err <= gemv_bound(W64, x64, ref, dt) + 1e-4 * mag), float(err.max())


# ---------------------------------------------------------------- batch, mixed selections


@pytest.mark.parametrize("dt,E,r,k,nb", [("bf16", 8, 16, 2, 1), ("bf16", 8, 16, 2, 3), ("bf16", 16, 64, 4, 8),
                                         ("bf16", 8, 16, 2, 16), ("fp32", 4, 8, 2, 5)])
def test_lora_batch_serves_a_selection_per_request(dt, E, r, k, nb):
    """A batch of requests with different selections through one layer: request b is
    within the GEMV bound of the oracle's routed forward with that request's selection,
    and agrees with the single-request layer path on (x_b, idx_b, gate_b) to rounding
    (the batched base product sums on MFMA, in another order).  One request carries an
    out-of-range index and a zero gate, both skipped."""
    shapes = [(264, 520), (1032, 264), (8, 8), (136, 136)]
    sels = [make_selection(E, k, 64, dt, 40 + 7 * b) for b in range(nb)]
    idx = torch.stack([s[0] for s in sels]).contiguous()
    gate = torch.stack([s[1] for s in sels]).contiguous()
    if nb > 1:
        idx[1, 0] = E + 3
        gate[1, k - 1] = 0.0
        assert len({tuple(row) for row in idx.tolist()}) > 1, "the batch must mix selections"
    banks = [synth.adapter_bank(400 + i, E, r, do, di, dt) for i, (do, di) in enumerate(shapes)]
    xs = [synth.host_normal(synth.tensor_seed(500 + i, di), (nb, di), 1.0, dt) for i, (_, di) in enumerate(shapes)]
    dev = [(W.to(DEV), Aw.to(DEV), Bw.to(DEV), x.to(DEV)) for (W, Aw, Bw), x in zip(banks, xs)]
    ys = [torch.full((nb, W.shape[0]), float("nan"), dtype=TD[dt], device=DEV) for W, _, _ in banks]
    didx, dgate = idx.to(DEV), gate.to(DEV)
    A.ada_lora_batch([(w, a, b, x, y) for (w, a, b, x), y in zip(dev, ys)], didx, dgate, 2.0)
    singles = []
    for bq in range(nb):
        y1 = [torch.full((W.shape[0],), float("nan"), dtype=TD[dt], device=DEV) for W, _, _ in banks]
        A.ada_lora_layer([(w, a, b, x[bq].contiguous(), y) for (w, a, b, x), y in zip(dev, y1)],
                         didx[bq].contiguous(), dgate[bq].contiguous(), 2.0)
        singles.append(y1)
    sync()
    for bq in range(nb):
        keep = [(e, g) for e, g in zip(idx[bq].tolist(), gate[bq].tolist()) if 0 <= e < E]
        for pi, ((W, Aw, Bw), x) in enumerate(zip(banks, xs)):
            got = ys[pi][bq].cpu()
            W64, x64 = to64(W), to64(x[bq])
            one = to64(singles[bq][pi])
            assert np.all(np.abs(to64(got) - one) <= gemv_bound(W64, x64, one, dt)), (bq, pi)
            ref = O.routed_lora_forward(to64(W), to64(Aw), to64(Bw), [e for e, _ in keep],
                                        np.array([g for _, g in keep], dtype=np.float64), 2.0, to64(x[bq]))
            err = np.abs(to64(got) - ref)
            assert np.all(err <= gemv_bound(W64, x64, ref, dt) + 1e-4 * (np.abs(W64) @ np.abs(x64))), (bq, pi)


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_decode_gemv_layer_is_the_per_projection_gemv(dt):
    """Independent GEMVs in one launch: each bit-identical to its own ada_decode_gemv
    and within the GEMV bound of the oracle."""
    shapes = [(264, 520), (1032, 264), (8, 8), (136, 1000), (520, 136)]
    mats = [synth.adapter_bank(600 + i, 1, 8, do, di, dt)[0] for i, (do, di) in enumerate(shapes)]
    xs = [synth.host_normal(synth.tensor_seed(700 + i, di), (di,), 1.0, dt) for i, (_, di) in enumerate(shapes)]
    dev = [(W.to(DEV), x.to(DEV)) for W, x in zip(mats, xs)]
    ys = [torch.full((W.shape[0],), float("nan"), dtype=TD[dt], device=DEV) for W in mats]
    A.ada_decode_gemv_layer([(w, x, y) for (w, x), y in zip(dev, ys)])
    one = [A.ada_decode_gemv(w, x) for w, x in dev]
    sync()
    iv = torch.int16 if dt == "bf16" else torch.int32
    for W, x, y, y1 in zip(mats, xs, ys, one):
        assert torch.equal(y.cpu().view(iv), y1.cpu().view(iv))
        W64, x64 = to64(W), to64(x)
        ref = O.gemv(W64, x64)
        assert np.all(np.abs(to64(y) - ref) <= gemv_bound(W64, x64, ref, dt))


def _random_layer_cases(n: int = 8, seed: int = 20261206):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        n_proj = int(rng.integers(1, 17))
        shapes = [(8 * int(rng.integers(1, 200)), 8 * int(rng.integers(1, 200))) for _ in range(n_proj)]
        out.append((c, "bf16" if rng.random() < 0.75 else "fp32", shapes))
    return out


@pytest.mark.parametrize("case,dt,shapes", _random_layer_cases())
def test_gemv_layer_and_lora_paths_on_random_groups(case, dt, shapes):
    """Seeded draws of 1 to 16 projections of ragged shapes in one group: the GEMV-layer
    launch bit-identical to per-projection GEMVs and within the oracle's bound; the
    fused unmerged layer path and the batched path (3 requests) within the bound of the
    oracle's routed forward."""
    E, r, k, nb = 6, 8, 2, 3
    banks = [synth.adapter_bank(1300 + 37 * case + i, E, r, do, di, dt) for i, (do, di) in enumerate(shapes)]
    xs = [synth.host_normal(synth.tensor_seed(1400 + 37 * case + i, di), (nb, di), 1.0, dt)
          for i, (_, di) in enumerate(shapes)]
    dev = [tuple(t.to(DEV) for t in b) for b in banks]
    xd = [x.to(DEV) for x in xs]
    sels = [make_selection(E, k, 64, dt, 80 + 7 * b) for b in range(nb)]
    idx = torch.stack([s_[0] for s_ in sels]).contiguous()
    gate = torch.stack([s_[1] for s_ in sels]).contiguous()
    didx, dgate = idx.to(DEV), gate.to(DEV)
    yl = [torch.full((do,), float("nan"), dtype=TD[dt], device=DEV) for do, _ in shapes]
    A.ada_decode_gemv_layer([(w, x[0], y) for (w, _, _), x, y in zip(dev, xd, yl)])
    one = [A.ada_decode_gemv(w, x[0]) for (w, _, _), x in zip(dev, xd)]
    yf = [torch.full((do,), float("nan"), dtype=TD[dt], device=DEV) for do, _ in shapes]
    A.ada_lora_layer([(w, a, b, x[0], y) for (w, a, b), x, y in zip(dev, xd, yf)], didx[0].contiguous(),
                     dgate[0].contiguous(), 2.0)
    yb = [torch.full((nb, do), float("nan"), dtype=TD[dt], device=DEV) for do, _ in shapes]
    A.ada_lora_batch([(w, a, b, x, y) for (w, a, b), x, y in zip(dev, xd, yb)], didx, dgate, 2.0)
    sync()
    iv = torch.int16 if dt == "bf16" else torch.int32
    for (W, Aw, Bw), x, y, y1, f, bt in zip(banks, xs, yl, one, yf, yb):
        assert torch.equal(y.cpu().view(iv), y1.cpu().view(iv))
        W64, A64, B64 = to64(W), to64(Aw), to64(Bw)
        x64 = to64(x[0])
        ref = O.gemv(W64, x64)
        assert np.all(np.abs(to64(y) - ref) <= gemv_bound(W64, x64, ref, dt))
        for b in range(nb):
            xb = to64(x[b])
            rb = O.routed_lora_forward(W64, A64, B64, idx[b].numpy(), gate[b].numpy().astype(np.float64), 2.0, xb)
            lim = gemv_bound(W64, xb, rb, dt) + 1e-4 * (np.abs(W64) @ np.abs(xb))
            assert np.all(np.abs(to64(bt[b]) - rb) <= lim), ("batch", b)
            if b == 0:
                assert np.all(np.abs(to64(f) - rb) <= lim), "layer"


def test_calls_run_in_order_on_the_callers_streams():
    """Every call enqueues on the stream it is given (torch's current stream by
    default): two models merged concurrently on two side streams, each followed on its
    own stream by a copy of its result, match the oracle; a third call given an
    explicit stream that waits on the others sees both merges."""
    E, r, k = 8, 16, 2
    banks = [synth.adapter_bank(1500 + i, E, r, 520, 264, "bf16") for i in range(2)]
    idx, gate = make_selection(E, k, 64, "bf16", 21)
    refs = [O.merge(to64(W), to64(Aw), to64(Bw), idx.numpy(), gate.numpy().astype(np.float64), 2.0)
            for W, Aw, Bw in banks]
    ws = [W.to(DEV) for W, _, _ in banks]
    models = [A.AdaModel([(w, None, Aw.to(DEV), Bw.to(DEV))], E, r) for w, (_, Aw, Bw) in zip(ws, banks)]
    didx, dgate = idx.to(DEV), gate.to(DEV)
    sync()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    copies = []
    for m, w, st in zip(models, ws, streams):
        with torch.cuda.stream(st):
            A.ada_merge(m, didx, dgate, 2.0)
            copies.append(w.clone())
    joined = torch.cuda.Stream()
    for st in streams:
        joined.wait_stream(st)
    A.ada_unmerge(models[0], didx, dgate, 2.0, stream=joined)
    sync()
    for c, ref in zip(copies, refs):
        check_close(c, ref, *tol(torch.bfloat16), "merge on a side stream")
    check_close(ws[0], to64(banks[0][0]), *tol(torch.bfloat16), "unmerge on an explicit stream")
    for m in models:
        m.destroy()


def test_model_table_upload_is_ordered_on_its_stream():
    """ada_model_create uploads the work table asynchronously on the stream it is given:
    a merge enqueued right after it on that stream (no host synchronisation between
    them) sees the whole table.  Many small projections make the table large (tens of
    KB per tile class), and a kernel queued ahead on the stream delays the upload."""
    E, r, k = 4, 16, 2
    banks = [synth.adapter_bank(1700 + i, E, r, 8 * (1 + i % 9), 8 * (1 + (5 * i) % 11), "bf16") for i in range(600)]
    idx, gate = make_selection(E, k, 64, "bf16", 23)
    ws = [W.to(DEV) for W, _, _ in banks]
    dev = [(w, None, Aw.to(DEV), Bw.to(DEV)) for w, (_, Aw, Bw) in zip(ws, banks)]
    didx, dgate = idx.to(DEV), gate.to(DEV)
    big = torch.randn(1 << 26, device=DEV)
    sync()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        for _ in range(4):
            big.mul_(1.0001)  # keep the stream busy when the upload is enqueued
        m = A.AdaModel(dev, E, r, stream=st)
        A.ada_merge(m, didx, dgate, 2.0, stream=st)
    sync()
    g64 = gate.numpy().astype(np.float64)
    for w, (W, Aw, Bw) in zip(ws, banks):
        check_close(w, O.merge(to64(W), to64(Aw), to64(Bw), idx.numpy(), g64, 2.0), *tol(torch.bfloat16),
                    "merge right after an asynchronous table upload")
    m.destroy()


# ---------------------------------------------------------------- graph capture


def test_captured_decode_paths_replay_like_eager():
    """The decode-time paths as the benchmark captures them in HIP graphs (merged-weight
    GEMVs in groups, the routed baseline with its per-layer pre-gating, the fused
    unmerged layer path and the batched path): every replay, with unrelated eager work
    and synchronisation between replays, gives bit-identical outputs to the eager run."""
    E, r, k, nb, L = 8, 16, 2, 4, 2
    shapes = [(264, 520), (136, 264), (520, 136)]
    groups = [[0, 1], [2]]
    banks = [[tuple(t.to(DEV) for t in synth.adapter_bank(1000 + 10 * l + i, E, r, do, di, "bf16"))
              for i, (do, di) in enumerate(shapes)] for l in range(L)]
    xs = [synth.host_normal(synth.tensor_seed(1100 + i, di), (nb, di), 1.0, "bf16").to(DEV)
          for i, (_, di) in enumerate(shapes)]
    h, R, _ = gapped_router(E, 256, "bf16", 5)
    h, R = h.to(DEV), R.to(DEV)
    idx, gate = A.ada_pregate(h, R, k)
    bidx = torch.stack([oracle_selection(*gapped_router(E, 64, "bf16", 70 + 7 * b)[:2], k)[0] for b in range(nb)])
    bgate = torch.stack([oracle_selection(*gapped_router(E, 64, "bf16", 70 + 7 * b)[:2], k)[1] for b in range(nb)])
    bidx, bgate = bidx.contiguous().to(DEV), bgate.contiguous().to(DEV)
    lidx = [torch.empty(k, dtype=torch.int32, device=DEV) for _ in range(L)]
    lgate = [torch.empty(k, dtype=torch.float32, device=DEV) for _ in range(L)]
    ys = {name: [[torch.empty(nb, do, dtype=torch.bfloat16, device=DEV) for do, _ in shapes] for _ in range(L)]
          for name in ("merged", "baseline", "fused", "batch")}
    ws_apply = [[torch.empty(A.lora_layer_workspace_elems([do], k, r), dtype=torch.float32, device=DEV)
                 for do, _ in shapes] for _ in range(L)]
    ws_layer = [[torch.empty(A.lora_layer_workspace_elems([shapes[p][0] for p in g], k, r), dtype=torch.float32,
                             device=DEV) for g in groups] for _ in range(L)]
    ws_batch = [[torch.empty(A.lora_batch_workspace_elems([shapes[p][0] for p in g], nb, k, r),
                             dtype=torch.float32, device=DEV) for g in groups] for _ in range(L)]

    def merged():
        for l in range(L):
            for g in groups:
                A.ada_decode_gemv_layer([(banks[l][p][0], xs[p][0], ys["merged"][l][p][0]) for p in g])

    def baseline():
        for l in range(L):
            A.ada_pregate(h, R, k, True, lidx[l], lgate[l])
            for p in range(len(shapes)):
                w, a, b = banks[l][p]
                A.ada_lora_apply(w, a, b, lidx[l], lgate[l], 2.0, xs[p][0], ys["baseline"][l][p][0], ws_apply[l][p])

    def fused():
        for l in range(L):
            A.ada_pregate(h, R, k, True, lidx[l], lgate[l])
            for gi, g in enumerate(groups):
                A.ada_lora_layer([(*banks[l][p], xs[p][0], ys["fused"][l][p][0]) for p in g], lidx[l], lgate[l],
                                 2.0, ws_layer[l][gi])

    def batch():
        for l in range(L):
            for gi, g in enumerate(groups):
                A.ada_lora_batch([(*banks[l][p], xs[p], ys["batch"][l][p]) for p in g], bidx, bgate, 2.0,
                                 ws_batch[l][gi])

    paths = {"merged": merged, "baseline": baseline, "fused": fused, "batch": batch}
    eager = {}
    for name, fn in paths.items():
        fn()
        sync()
        eager[name] = [[y.clone() for y in row] for row in ys[name]]
    graphs = {}
    for name, fn in paths.items():
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        graphs[name] = g
    other = torch.randn(1 << 20, device=DEV)
    for rep in range(3):
        for name, g in graphs.items():
            for row in ys[name]:
                for y in row:
                    y.fill_(float("nan"))
            other.mul_(1.0001).add_(0.5)  # unrelated eager work between replays
            sync()
            g.replay()
            sync()
            for l in range(L):
                for p in range(len(shapes)):
                    got, want = ys[name][l][p], eager[name][l][p]
                    rows = slice(None) if name == "batch" else slice(0, 1)
                    assert torch.equal(got[rows].view(torch.int16), want[rows].view(torch.int16)), (name, rep, l, p)


@pytest.mark.parametrize("E,r,k", [(8, 16, 2), (8, 16, 4), (16, 64, 4)])  # each tile class
def test_captured_pregate_and_merge_replay_like_eager(E, r, k):
    """Pre-gating plus an out-of-place merge captured in one HIP graph: each replay,
    with unrelated eager work and synchronisation between replays, rewrites W' from the
    untouched W bit-identically to the eager run."""
    shapes = [(264, 520), (136, 264)]
    banks = [tuple(t.to(DEV) for t in synth.adapter_bank(1200 + i, E, r, do, di, "bf16"))
             for i, (do, di) in enumerate(shapes)]
    outs = [torch.empty_like(w) for w, _, _ in banks]
    model = A.AdaModel([(w, o, a, b) for (w, a, b), o in zip(banks, outs)], E, r)
    h, R, _ = gapped_router(E, 256, "bf16", 11)
    h, R = h.to(DEV), R.to(DEV)
    idx = torch.empty(k, dtype=torch.int32, device=DEV)
    gate = torch.empty(k, dtype=torch.float32, device=DEV)

    def step():
        A.ada_pregate(h, R, k, True, idx, gate)
        A.ada_merge(model, idx, gate, 2.0)

    step()
    sync()
    eager = [o.clone() for o in outs]
    w_before = [w.clone() for w, _, _ in banks]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = torch.randn(1 << 20, device=DEV)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        idx.fill_(-1)
        other.mul_(1.0001).add_(0.5)
        sync()
        g.replay()
        sync()
        for o, want in zip(outs, eager):
            assert torch.equal(o.view(torch.int16), want.view(torch.int16)), rep
    for (w, _, _), w0 in zip(banks, w_before):
        assert torch.equal(w.view(torch.int16), w0.view(torch.int16))
    model.destroy()

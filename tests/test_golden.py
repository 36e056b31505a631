"""The oracle still reproduces its stored tiny-stack fixture, and the GPU path
matches it."""
import json
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = json.load(open(os.path.join(HERE, "golden", "tiny_oracle.json")))


def test_oracle_reproduces_the_fixture():
    import importlib.util

    spec = importlib.util.spec_from_file_location("mk", os.path.join(HERE, "golden", "make_tiny_golden.py"))
    mk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mk)
    now = mk.build()
    assert now["idx"] == GOLDEN["idx"]
    np.testing.assert_allclose(now["gate"], GOLDEN["gate"], rtol=1e-13)
    for a, b in zip(now["layers"], GOLDEN["layers"]):
        np.testing.assert_allclose(np.array(a["samples"]), np.array(b["samples"]), rtol=1e-13, atol=1e-15)
        assert abs(a["sum"] - b["sum"]) <= 1e-10 * b["abs_sum"]


def test_fixture_is_self_consistent():
    # the stored gates are a softmax over the stored logits at the stored indices
    z = np.array(GOLDEN["logits"])
    idx = GOLDEN["idx"]
    e = np.exp(z[idx] - z[idx].max())
    np.testing.assert_allclose(GOLDEN["gate"], e / e.sum(), rtol=1e-13)
    assert list(np.argsort(-z, kind="stable")[: len(idx)]) == idx


@pytest.mark.gpu
def test_gpu_matches_the_fixture():
    import torch

    from weight_merge_amd import api as A
    from weight_merge_amd import synth
    from weight_merge_amd.configs import TINY

    h, R = synth.router_inputs(TINY, GOLDEN["seed"])
    st = synth.make_stack(TINY, GOLDEN["seed"])
    ws = [st.W[l][p].cuda() for l, p, _ in st.items()]
    m = A.AdaModel([(w, None, st.A[l][p].cuda(), st.B[l][p].cuda()) for w, (l, p, _) in zip(ws, st.items())],
                   TINY.E, TINY.r)
    idx, gate = A.ada_pregate(h.cuda(), R.cuda(), TINY.k)
    A.ada_merge(m, idx, gate, TINY.scale)
    torch.cuda.synchronize()
    assert idx.cpu().tolist() == GOLDEN["idx"]
    np.testing.assert_allclose(gate.cpu().double().numpy(), GOLDEN["gate"], rtol=1e-4, atol=1e-6)
    for w, lay in zip(ws, GOLDEN["layers"]):
        got = w.cpu().double().numpy()
        for r, c, v in lay["samples"]:
            assert abs(got[r, c] - v) <= 1e-6 * abs(v) + 1e-7, (r, c, got[r, c], v)

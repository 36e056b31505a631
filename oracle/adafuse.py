"""Plain fp64 CPU oracle for AdaFuse token-level pre-gating and the fused adapter merge.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The product path (the HIP library and
its Python binding) never imports it, and this module imports nothing from the
product: the two share no code.  Every function is slow on purpose and follows the
definition it cites with no blocking, fusion or reordering beyond that definition.

Sources (cited by page title and section; both pages summarise the same paper,
"AdaFuse: Accelerating Dynamic Adapter Inference via Token-Level Pre-Gating and
Fused Kernel Optimization"):

  [pt]  the Portuguese summary page (gist.science/pt/paper/2603.11873),
        "Resumo tecnico" sections 1 (problem), 2.A (token-level pre-gating),
        2.B (adapter fusion and the SGMM kernel), 4 (results).
  [ja]  the Japanese summary page (gist.science/ja/paper/2603.11873),
        "技術概要" sections 1, 2.1 (pre-gating), 2.2 (fused switching, SGMM).

What the pages fix, restated:
  * One light Top-2 router runs once, at the first expanded layer, and its choice of
    experts (LoRA adapters) holds for every later layer ([pt] 2.A; [ja] 2.1).
  * The chosen adapters are fused into the backbone weights before decoding, so no
    routing runs while decoding ([pt] 2.B).
  * The chosen adapters' down and up projections are concatenated and merged with
    the base weight matrix in one kernel call, across all layers ([ja] 2.2).
  * Fusion is undone ("de-fused") when the selection changes; a switch undoes the
    previous token's fusion and applies the current one ([pt] 2.B).
  * Fusing a static LoRA adapter into the weights is the operation the dynamic
    methods could not use ([pt] 1).

Readings where the pages are silent (each listed with its reason in the design
notes of the repository):
  * LoRA convention: down projection A_e is r x d_in, up projection B_e is d_out x r,
    the adapter's weight update is B_e @ A_e, so a layer computes W x + B_e (A_e x).
  * Router: a bias-free linear map R (E x d); logits z = R h.
  * Selection: the k largest logits, in descending order, equal logits taken lower
    index first.  The decision compares the logits rounded to fp32, the precision
    the GPU kernel decides in; the logits themselves and the gates are fp64.
  * Gates: softmax over the k selected logits (equivalently the full softmax
    renormalised over the top-k).  ``renorm=False`` gives the full-softmax
    probabilities of the selected experts instead.  Parity unpinned by the pages:
    they print no gate formula.
  * Merged weights: W' = W + s * sum_j g_j * B_{e_j} @ A_{e_j}, slots with g_j == 0
    dropped (so a zero gate leaves W bit-identical and 0 * inf never appears).
  * Unmerge: W'' = W' - (the same sum).  Switch: W - delta(prev) + delta(cur).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "router_logits",
    "select_topk",
    "gate_weights",
    "pregate",
    "adapter_delta",
    "merge",
    "unmerge",
    "switch",
    "gemv",
    "routed_lora_forward",
]


def _f64(x) -> np.ndarray:
    """Exact upcast of stored values (fp32, or bf16 already widened) to fp64."""
    return np.asarray(x, dtype=np.float64)


def router_logits(h, R) -> np.ndarray:
    """Router scores z = R h for the leading token's hidden state h.

    [pt] 2.A and [ja] 2.1: a single light router, run once, scores the E experts.
    R is E x d, h has d entries; the result has E entries (fp64).
    """
    R = _f64(R)
    h = _f64(h)
    if R.ndim != 2 or h.ndim != 1 or R.shape[1] != h.shape[0]:
        raise ValueError(f"router shape mismatch: R{R.shape} h{h.shape}")
    return R @ h


def select_topk(z, k: int) -> np.ndarray:
    """Indices of the k largest scores, largest first, equal scores lower index first.

    [pt] 2.A, [ja] 2.1: a Top-k (Top-2 on the pages) router picks the experts.
    The comparison is made on the scores rounded to fp32 (the kernel's precision);
    Python's sort is stable, so sorting by the negated key keeps lower indices first
    among equal keys.
    """
    z = _f64(z)
    E = z.shape[0]
    if not 1 <= k <= E:
        raise ValueError(f"need 1 <= k <= E, got k={k}, E={E}")
    key = z.astype(np.float32)
    order = sorted(range(E), key=lambda e: -float(key[e]))
    return np.asarray(order[:k], dtype=np.int32)


def gate_weights(z, idx, renorm: bool = True) -> np.ndarray:
    """Gate weight of each selected expert, in selection order (fp64).

    renorm=True: softmax over the selected logits only.
    renorm=False: the full softmax over all E logits, read at the selected experts.
    Both subtract the largest logit first so exp never overflows.
    """
    z = _f64(z)
    idx = np.asarray(idx, dtype=np.int64)
    pool = z[idx] if renorm else z
    m = pool.max()
    denom = np.exp(pool - m).sum()
    return np.exp(z[idx] - m) / denom


def pregate(h, R, k: int, renorm: bool = True):
    """Token-level pre-gating: one router pass giving (indices, gates) for all layers.

    [pt] 2.A ("decide once, apply everywhere"), [ja] 2.1.
    """
    z = router_logits(h, R)
    idx = select_topk(z, k)
    return idx, gate_weights(z, idx, renorm)


def adapter_delta(A, B, idx, coef) -> np.ndarray:
    """sum_j coef_j * B[idx_j] @ A[idx_j], skipping slots whose coefficient is zero.

    A: E x r x d_in (down projections), B: E x d_out x r (up projections).
    [ja] 2.2: the selected down and up projections are concatenated; the product of
    the concatenated factors is exactly this sum of per-expert products.
    """
    A = _f64(A)
    B = _f64(B)
    if A.ndim != 3 or B.ndim != 3 or A.shape[0] != B.shape[0] or A.shape[1] != B.shape[2]:
        raise ValueError(f"adapter bank shape mismatch: A{A.shape} B{B.shape}")
    d_out, d_in = B.shape[1], A.shape[2]
    delta = np.zeros((d_out, d_in), dtype=np.float64)
    for e, c in zip(np.asarray(idx, dtype=np.int64), _f64(coef)):
        if c == 0.0:
            continue
        delta += c * (B[e] @ A[e])
    return delta


def merge(W, A, B, idx, gate, scale: float) -> np.ndarray:
    """Merged weights W + s * sum_j g_j B_{e_j} A_{e_j}, unrounded fp64.

    [pt] 2.B: the activated adapters are fused into the backbone weights before
    decoding; [pt] 1: the same weight fusion static LoRA uses.  A zero-gated slot is
    dropped; with every gate zero the result is W itself.
    """
    W = _f64(W)
    coef = float(scale) * _f64(gate)
    if not np.any(coef != 0.0):
        return W.copy()
    return W + adapter_delta(A, B, idx, coef)


def unmerge(W, A, B, idx, gate, scale: float) -> np.ndarray:
    """De-fused weights W - s * sum_j g_j B_{e_j} A_{e_j} ([pt] 2.B, de-fusion)."""
    W = _f64(W)
    coef = -float(scale) * _f64(gate)
    if not np.any(coef != 0.0):
        return W.copy()
    return W + adapter_delta(A, B, idx, coef)


def switch(W, A, B, prev, cur, scale: float) -> np.ndarray:
    """Undo the previous selection's fusion and apply the current one ([pt] 2.B).

    prev and cur are (indices, gates) pairs.  Both deltas are formed in fp64 and
    added to W once.
    """
    W = _f64(W)
    (pi, pg), (ci, cg) = prev, cur
    d_prev = adapter_delta(A, B, pi, float(scale) * _f64(pg))
    d_cur = adapter_delta(A, B, ci, float(scale) * _f64(cg))
    return W - d_prev + d_cur


def gemv(W, x) -> np.ndarray:
    """Decode-step projection y = W x on the merged backbone ([pt] 2.B: after fusion,
    decoding runs the backbone with no routing)."""
    W = _f64(W)
    x = _f64(x)
    if W.ndim != 2 or x.ndim != 1 or W.shape[1] != x.shape[0]:
        raise ValueError(f"gemv shape mismatch: W{W.shape} x{x.shape}")
    return W @ x


def routed_lora_forward(W, A, B, idx, gate, scale: float, x) -> np.ndarray:
    """One projection of the unmerged, routed baseline: W x + s * sum_j g_j B_j (A_j x).

    [pt] 1 and [ja] 1: conventional dynamic adapters route and apply the selected
    adapters at every layer, keeping them separate from the backbone weights.
    """
    W = _f64(W)
    A = _f64(A)
    B = _f64(B)
    x = _f64(x)
    y = W @ x
    for e, g in zip(np.asarray(idx, dtype=np.int64), _f64(gate)):
        c = float(scale) * g
        if c == 0.0:
            continue
        y = y + c * (B[e] @ (A[e] @ x))
    return y

"""Python binding of libadafuse: argument marshalling only.

Every computation runs in the HIP kernels behind the C ABI; this module turns torch
tensors (device memory) and the current torch stream into the pointers and sizes the
C calls take, and turns negative status codes into exceptions.  Output tensors a
caller does not pass are allocated here with torch, outside the C calls.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import ADA_BF16, ADA_F32, AdaGemvProj, AdaLoraProj, AdaProj

_DT = {torch.float32: ADA_F32, torch.bfloat16: ADA_BF16}


class AdaError(RuntimeError):
    def __init__(self, status: int, call: str):
        msg = _lib.load().ada_status_string(status).decode()
        super().__init__(f"{call} failed with status {status}: {msg}")
        self.status = status


def _check(status: int, call: str):
    if status != 0:
        raise AdaError(status, call)


def _dtype(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16") from None


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _contig(t: torch.Tensor, name: str):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _out(t: torch.Tensor, shape, dtype, name: str):
    """A caller-provided output: the C call writes numel(shape) contiguous elements."""
    _contig(t, name)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


def ada_pregate(h: torch.Tensor, router: torch.Tensor, k: int, renorm: bool = True,
                idx_out: torch.Tensor | None = None, gate_out: torch.Tensor | None = None,
                stream=None):
    """Router GEMV + top-k + gates (one kernel).  Returns (idx int32[k], gate fp32[k])
    on the device."""
    _contig(h, "h")
    _contig(router, "router")
    E, d = router.shape
    if h.shape != (d,) or h.dtype != router.dtype:
        raise ValueError("h must be [d] with the router's dtype")
    if idx_out is None:
        idx_out = torch.empty(k, dtype=torch.int32, device=h.device)
    if gate_out is None:
        gate_out = torch.empty(k, dtype=torch.float32, device=h.device)
    _out(idx_out, (k,), torch.int32, "idx_out")
    _out(gate_out, (k,), torch.float32, "gate_out")
    st = _lib.load().ada_pregate(_dev(h, "h"), _dev(router, "router"), d, E, k, _dtype(h), int(bool(renorm)),
                                 _dev(idx_out, "idx_out"), _dev(gate_out, "gate_out"), _stream(stream))
    _check(st, "ada_pregate")
    return idx_out, gate_out


class AdaModel:
    """A registered stack of adapted projections (owns the device work table).

    projs: iterable of (w, w_out, a, b) with w [d_out, d_in] (row stride w.stride(0)),
    w_out None (merge in place) or a tensor like w, a [E, r, d_in], b [E, d_out, r].
    The tensors must outlive the model; the model keeps references to them.  The
    work table is uploaded on `stream` (default: torch's current stream), which
    orders it before the merges enqueued there.
    """

    def __init__(self, projs, E: int, r: int, stream=None):
        projs = list(projs)
        if not projs:
            raise ValueError("no projections")
        dt = projs[0][0].dtype
        arr = (AdaProj * len(projs))()
        keep = []
        for i, (w, w_out, a, b) in enumerate(projs):
            d_out, d_in = w.shape
            if w.stride(1) != 1 or (w_out is not None and (w_out.shape != w.shape or w_out.stride() != w.stride())):
                raise ValueError("w must have unit column stride; w_out must match w's layout")
            _contig(a, "a")
            _contig(b, "b")
            if a.shape != (E, r, d_in) or b.shape != (E, d_out, r):
                raise ValueError(f"adapter bank shapes {tuple(a.shape)}, {tuple(b.shape)} do not match "
                                 f"E={E}, r={r}, W {tuple(w.shape)}")
            for t in (w, a, b) + ((w_out,) if w_out is not None else ()):
                if t.dtype != dt:
                    raise TypeError("all tensors of a model share one dtype")
            arr[i] = AdaProj(_dev(w, "w"), _dev(w_out, "w_out") if w_out is not None else None,
                             _dev(a, "a"), _dev(b, "b"), d_out, d_in, w.stride(0))
            keep.append((w, w_out, a, b))
        handle = ctypes.c_void_p()
        st = _lib.load().ada_model_create(arr, len(projs), E, r, _DT[dt], _stream(stream), ctypes.byref(handle))
        _check(st, "ada_model_create")
        self._h = handle
        self._keep = keep
        self.E, self.r, self.dtype = E, r, dt
        self.n_proj = len(projs)

    @property
    def handle(self):
        if self._h is None:
            raise RuntimeError("model destroyed")
        return self._h

    @property
    def tiles(self) -> int:
        return int(_lib.load().ada_model_tiles(self.handle))

    @property
    def device_bytes(self) -> int:
        """Device memory the model owns (its work tables)."""
        return int(_lib.load().ada_model_device_bytes(self.handle))

    def destroy(self):
        if getattr(self, "_h", None) is not None:
            _lib.load().ada_model_destroy(self._h)
            self._h = None
            self._keep = []

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def _sel(idx: torch.Tensor, gate: torch.Tensor):
    if idx.dtype != torch.int32 or gate.dtype != torch.float32:
        raise TypeError("idx must be int32 and gate float32")
    if idx.dim() != 1 or gate.dim() != 1 or idx.numel() != gate.numel():
        raise ValueError("idx and gate must be one-dimensional and of the same length")
    _contig(idx, "idx")
    _contig(gate, "gate")
    return _dev(idx, "idx"), _dev(gate, "gate"), idx.numel()


def ada_merge(model: AdaModel, idx: torch.Tensor, gate: torch.Tensor, scale: float, stream=None):
    """Fuse the selected adapters into every registered projection (one launch)."""
    pi, pg, k = _sel(idx, gate)
    _check(_lib.load().ada_merge(model.handle, pi, pg, k, float(scale), _stream(stream)), "ada_merge")


def ada_unmerge(model: AdaModel, idx: torch.Tensor, gate: torch.Tensor, scale: float, stream=None):
    """De-fuse the selection from the merged buffer (one launch)."""
    pi, pg, k = _sel(idx, gate)
    _check(_lib.load().ada_unmerge(model.handle, pi, pg, k, float(scale), _stream(stream)), "ada_unmerge")


def ada_switch(model: AdaModel, prev, cur, scale: float, stream=None):
    """Undo selection `prev` and apply `cur` in one pass; prev, cur = (idx, gate)."""
    pi, pg, pk = _sel(*prev)
    ci, cg, ck = _sel(*cur)
    _check(_lib.load().ada_switch(model.handle, pi, pg, pk, ci, cg, ck, float(scale), _stream(stream)),
           "ada_switch")


def ada_decode_gemv(w: torch.Tensor, x: torch.Tensor, y: torch.Tensor | None = None, stream=None):
    """y = W x on the device (fp32 accumulation, one rounding)."""
    d_out, d_in = w.shape
    if w.stride(1) != 1:
        raise ValueError("w must have unit column stride")
    _contig(x, "x")
    if x.shape != (d_in,) or x.dtype != w.dtype:
        raise ValueError("x must be [d_in] with w's dtype")
    if y is None:
        y = torch.empty(d_out, dtype=w.dtype, device=w.device)
    _out(y, (d_out,), w.dtype, "y")
    st = _lib.load().ada_decode_gemv(_dev(w, "w"), d_out, d_in, w.stride(0), _dev(x, "x"), _dev(y, "y"),
                                     _dtype(w), _stream(stream))
    _check(st, "ada_decode_gemv")
    return y


def ada_decode_gemv_layer(projs, stream=None):
    """Independent GEMVs y_p = W_p x_p in one launch; projs: list of (w, x, y) with w
    [d_out, d_in], x [d_in], y [d_out] (written), all of one dtype."""
    projs = list(projs)
    arr = (AdaGemvProj * len(projs))()
    dt = projs[0][0].dtype
    for i, (w, x, y) in enumerate(projs):
        d_out, d_in = w.shape
        if w.stride(1) != 1:
            raise ValueError("w must have unit column stride")
        _contig(x, "x")
        _contig(y, "y")
        if x.shape != (d_in,) or y.shape != (d_out,):
            raise ValueError("x must be [d_in] and y [d_out]")
        if w.dtype != dt or x.dtype != dt or y.dtype != dt:
            raise TypeError("all tensors share one dtype")
        arr[i] = AdaGemvProj(_dev(w, "w"), _dev(x, "x"), _dev(y, "y"), d_out, d_in, w.stride(0))
    st = _lib.load().ada_decode_gemv_layer(arr, len(projs), _DT[dt], _stream(stream))
    _check(st, "ada_decode_gemv_layer")


def ada_lora_apply(w, a, b, idx, gate, scale: float, x, y=None, workspace=None, stream=None):
    """Unmerged routed projection y = W x + s sum_j g_j B_j (A_j x) (three launches)."""
    d_out, d_in = w.shape
    E, r, _ = a.shape
    pi, pg, k = _sel(idx, gate)
    if w.stride(1) != 1:
        raise ValueError("w must have unit column stride")
    for t, n in ((a, "a"), (b, "b"), (x, "x")):
        _contig(t, n)
    if a.shape != (E, r, d_in) or b.shape != (E, d_out, r) or x.shape != (d_in,):
        raise ValueError("projection shapes do not match")
    if a.dtype != w.dtype or b.dtype != w.dtype or x.dtype != w.dtype:
        raise TypeError("all tensors share one dtype")
    if y is None:
        y = torch.empty(d_out, dtype=w.dtype, device=w.device)
    _out(y, (d_out,), w.dtype, "y")
    need = (d_out + k * r) * 4
    if workspace is None:
        workspace = torch.empty((need + 15) // 16 * 4, dtype=torch.float32, device=w.device)
    _contig(workspace, "workspace")
    st = _lib.load().ada_lora_apply(_dev(w, "w"), d_out, d_in, w.stride(0), _dev(a, "a"), _dev(b, "b"),
                                    E, r, pi, pg, k, float(scale), _dev(x, "x"), _dev(y, "y"),
                                    _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                    _dtype(w), _stream(stream))
    _check(st, "ada_lora_apply")
    return y


def lora_layer_workspace_elems(d_outs, k: int, r: int) -> int:
    """fp32 elements of workspace ada_lora_layer needs for these projections."""
    n = 0
    for d in d_outs:
        n = (n + d + k * r + 3) // 4 * 4
    return n


def _lora_layer_projs(projs):
    w0, a0 = projs[0][0], projs[0][1]
    E, r, _ = a0.shape
    arr = (AdaLoraProj * len(projs))()
    for i, (w, a, b, x, y) in enumerate(projs):
        d_out, d_in = w.shape
        if w.stride(1) != 1:
            raise ValueError("w must have unit column stride")
        for t, n in ((a, "a"), (b, "b"), (x, "x"), (y, "y")):
            _contig(t, n)
        if a.shape != (E, r, d_in) or b.shape != (E, d_out, r) or x.shape != (d_in,) or y.shape != (d_out,):
            raise ValueError("projection shapes do not match")
        if any(t.dtype != w0.dtype for t in (w, a, b, x, y)):
            raise TypeError("all tensors share one dtype")
        arr[i] = AdaLoraProj(_dev(w, "w"), _dev(a, "a"), _dev(b, "b"), _dev(x, "x"), _dev(y, "y"), d_out, d_in,
                             w.stride(0))
    return arr, w0, E, r


def ada_lora_layer(projs, idx, gate, scale: float, workspace=None, stream=None):
    """One layer of the unmerged routed path (two launches for all projections).

    projs: list of (w, a, b, x, y) with w [d_out, d_in], a [E, r, d_in], b [E, d_out, r],
    x [d_in], y [d_out] (written)."""
    projs = list(projs)
    arr, w0, E, r = _lora_layer_projs(projs)
    pi, pg, k = _sel(idx, gate)
    need = lora_layer_workspace_elems([p[0].shape[0] for p in projs], k, r)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.float32, device=w0.device)
    _contig(workspace, "workspace")
    st = _lib.load().ada_lora_layer(arr, len(projs), E, r, pi, pg, k, float(scale), _dev(workspace, "workspace"),
                                    workspace.numel() * workspace.element_size(), _dtype(w0), _stream(stream))
    _check(st, "ada_lora_layer")


def ada_lora_layer_static(projs, idx, gate, scale: float, stream=None):
    """ada_lora_layer with its intermediates in the library's static device array (4 MiB
    per GPU): the C call allocates nothing.  Calls overlapping in time on one GPU race."""
    projs = list(projs)
    arr, w0, E, r = _lora_layer_projs(projs)
    pi, pg, k = _sel(idx, gate)
    st = _lib.load().ada_lora_layer_static(arr, len(projs), E, r, pi, pg, k, float(scale), _dtype(w0),
                                           _stream(stream))
    _check(st, "ada_lora_layer_static")


def lora_batch_workspace_elems(d_outs, nb: int, k: int, r: int) -> int:
    """fp32 elements of workspace ada_lora_batch needs for these projections."""
    n = 0
    for d in d_outs:
        n = (n + nb * (d + k * r) + 3) // 4 * 4
    return n


def ada_lora_batch(projs, idx, gate, scale: float, workspace=None, stream=None):
    """One layer of the unmerged routed path for a batch of requests with a selection
    each (two launches for all projections and requests).

    projs: list of (w, a, b, x, y) with w [d_out, d_in], a [E, r, d_in], b [E, d_out, r],
    x [nb, d_in], y [nb, d_out] (written); idx int32 [nb, k], gate fp32 [nb, k]."""
    projs = list(projs)
    w0, a0 = projs[0][0], projs[0][1]
    E, r, _ = a0.shape
    if idx.dim() != 2 or idx.shape != gate.shape:
        raise ValueError("idx and gate must be [nb, k] and of equal shape")
    if idx.dtype != torch.int32 or gate.dtype != torch.float32:
        raise TypeError("idx must be int32 and gate float32")
    _contig(idx, "idx")
    _contig(gate, "gate")
    nb, k = idx.shape
    arr = (AdaLoraProj * len(projs))()
    for i, (w, a, b, x, y) in enumerate(projs):
        d_out, d_in = w.shape
        if w.stride(1) != 1:
            raise ValueError("w must have unit column stride")
        for t, n in ((a, "a"), (b, "b"), (x, "x"), (y, "y")):
            _contig(t, n)
        if a.shape != (E, r, d_in) or b.shape != (E, d_out, r) or x.shape != (nb, d_in) or y.shape != (nb, d_out):
            raise ValueError("projection shapes do not match")
        if any(t.dtype != w0.dtype for t in (w, a, b, x, y)):
            raise TypeError("all tensors share one dtype")
        arr[i] = AdaLoraProj(_dev(w, "w"), _dev(a, "a"), _dev(b, "b"), _dev(x, "x"), _dev(y, "y"), d_out, d_in,
                             w.stride(0))
    need = lora_batch_workspace_elems([p[0].shape[0] for p in projs], nb, k, r)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.float32, device=w0.device)
    _contig(workspace, "workspace")
    st = _lib.load().ada_lora_batch(arr, len(projs), nb, E, r, _dev(idx, "idx"), _dev(gate, "gate"), k,
                                    float(scale), _dev(workspace, "workspace"),
                                    workspace.numel() * workspace.element_size(), _dtype(w0), _stream(stream))
    _check(st, "ada_lora_batch")

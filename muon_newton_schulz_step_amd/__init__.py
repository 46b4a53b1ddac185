"""Muon optimizer step on MI355X (gfx950): momentum, Newton-Schulz and the
flat-partition writeback as HIP kernels behind a C ABI (include/muon.h).

This package is the Python face of that library: ``_lib`` binds the C entry
points by name; ``MuonGroup`` is a small convenience wrapper that owns a plan.
Device memory and streams come from the caller (e.g. torch tensors).
"""

from __future__ import annotations

from . import _lib
from ._lib import (DTYPE, EXPORTS, NS_METHOD, PRECISION, SCHEDULE, MuonError, load, muon_accumulate,  # noqa: F401
                   muon_apply_update, muon_check_finite, muon_default_options, muon_last_error, muon_layout,
                   muon_plan_create, muon_plan_destroy, muon_plan_phase_ms, muon_plan_problems, muon_plan_runs,
                   muon_plan_set_timing, muon_plan_stats, muon_plan_workspace_bytes, muon_scatter,
                   muon_status_string, muon_step, muon_step_ex, muon_step_noalloc)

__all__ = ["MuonGroup", "pack_layout", "MuonError", "load"] + list(EXPORTS)


def pack_layout(shapes, num_partitions: int, align: int = 16, interior_align: bool = False):
    """Flat layout of a group: matrices back to back in order (each start
    rounded up to `align` if interior_align), the total padded at the tail so
    the partition size is a multiple of `align`.  Returns (offsets, P)."""
    offsets, f = [], 0
    for r, c in shapes:
        if interior_align:
            f = -(-f // align) * align
        offsets.append(f)
        f += int(r) * int(c)
    per = -(-f // (num_partitions * align)) * align
    return offsets, max(per, align)


_TORCH_DT = {"fp32": "torch.float32", "bf16": "torch.bfloat16"}


def _check_bufs(xs, numels, dtype, what: str) -> None:
    """Refuse tensors the library would misread: wrong count, dtype, size,
    a non-contiguous view or a host tensor.  Integers (raw device addresses)
    are the caller's responsibility and pass through."""
    xs = list(xs)
    if len(xs) != len(numels):
        raise ValueError(f"{what}: {len(xs)} buffers, the plan has {len(numels)}")
    for i, (x, n) in enumerate(zip(xs, numels)):
        if x is None or isinstance(x, int) or not hasattr(x, "is_contiguous"):
            continue
        if dtype is not None and str(x.dtype) != _TORCH_DT[dtype]:
            raise ValueError(f"{what}[{i}]: dtype {x.dtype}, expected {_TORCH_DT[dtype]}")
        if not x.is_contiguous():
            raise ValueError(f"{what}[{i}]: not contiguous (a transposed or strided view?)")
        if int(x.numel()) != int(n):
            raise ValueError(f"{what}[{i}]: {int(x.numel())} elements, expected {int(n)}")


def _check_device(**lists) -> None:
    """Every tensor among the arguments lives in device memory."""
    for what, xs in lists.items():
        for i, x in enumerate(xs if isinstance(xs, (list, tuple)) else [xs]):
            if getattr(x, "is_cuda", True) is False:
                raise ValueError(f"{what}[{i}]: a host tensor; the library needs device memory")


class MuonGroup:
    """A plan over one group of matrices (host memory only until used).
    Its methods check every tensor argument against the plan before the
    call: count, dtype, element count and contiguity."""

    def __init__(self, shapes, heads=None, offsets=None, num_partitions: int = 1, partition_numel=None,
                 align: int = 16, method: str = "standard", precision: str = "bf16", grad_dtype: str = "bf16",
                 ns_steps: int = 5, beta: float = 0.95, nesterov: bool = True, coeffs=None, eps=None,
                 max_inflight_bytes=None, schedule: str = "launches"):
        self.shapes = [(int(r), int(c)) for r, c in shapes]
        self.heads = list(heads) if heads is not None else [0] * len(self.shapes)
        if offsets is None or partition_numel is None:
            offs, P = pack_layout(self.shapes, num_partitions, align)
            offsets = offsets if offsets is not None else offs
            partition_numel = partition_numel if partition_numel is not None else P
        self.offsets = [int(o) for o in offsets]
        self.num_partitions = int(num_partitions)
        self.partition_numel = int(partition_numel)
        self.grad_dtype = grad_dtype
        self.precision = precision
        self.method = method
        o = muon_default_options()
        o.beta = beta
        o.nesterov = int(bool(nesterov))
        o.method = NS_METHOD[method]
        o.ns_steps = int(ns_steps)
        if coeffs is not None:
            o.a, o.b, o.c = coeffs
        if eps is not None:
            o.eps = eps
        o.precision = PRECISION[precision]
        o.grad_dtype = DTYPE[grad_dtype]
        if max_inflight_bytes is not None:  # None: the library's default cap; 0: no cap
            o.max_inflight_bytes = int(max_inflight_bytes)
        o.schedule = SCHEDULE[schedule]
        self.options = o
        lay = muon_layout(self.partition_numel, self.num_partitions, 0)
        mats = [(r, c, h, off) for (r, c), h, off in zip(self.shapes, self.heads, self.offsets)]
        self.plan = muon_plan_create(mats, o, lay)
        self.workspace_bytes = muon_plan_workspace_bytes(self.plan)

    # element counts of the per-matrix and per-partition buffers
    def _mat_numels(self):
        return [r * c for r, c in self.shapes]

    def _part_numels(self):
        return [self.partition_numel] * self.num_partitions

    def _ws(self, ws) -> int:
        """Bytes of the workspace: a tensor's own size, or, for a raw device
        address, the plan's requirement (the caller vouches for it)."""
        if hasattr(ws, "numel") and hasattr(ws, "element_size"):
            if not ws.is_contiguous():
                raise ValueError("workspace: not contiguous")
            return int(ws.numel()) * int(ws.element_size())
        return self.workspace_bytes

    def _flag(self, flag, what: str):
        if flag is not None and not isinstance(flag, int):
            if str(flag.dtype) != "torch.int32" or int(flag.numel()) < 1:
                raise ValueError(f"{what}: needs a device int32 tensor")

    def step(self, grads, momenta, partitions, ws, stream=None, skip_flag=None, grad_scale: float = 1.0):
        _check_bufs(grads, self._mat_numels(), self.grad_dtype, "grads")
        _check_bufs(momenta, self._mat_numels(), "fp32", "momenta")
        _check_bufs(partitions, self._part_numels(), "fp32", "partitions")
        self._flag(skip_flag, "skip_flag")
        _check_device(grads=grads, momenta=momenta, partitions=partitions, skip_flag=skip_flag, ws=ws)
        if skip_flag is None and grad_scale == 1.0:
            muon_step(self.plan, grads, momenta, partitions, ws, self._ws(ws), stream)
        else:
            muon_step_ex(self.plan, grads, momenta, partitions, skip_flag, grad_scale, ws, self._ws(ws), stream)

    def step_noalloc(self, grads, momenta, partitions, stream=None, skip_flag=None, grad_scale: float = 1.0):
        """The step on the library's static workspace (no caller workspace)."""
        _check_bufs(grads, self._mat_numels(), self.grad_dtype, "grads")
        _check_bufs(momenta, self._mat_numels(), "fp32", "momenta")
        _check_bufs(partitions, self._part_numels(), "fp32", "partitions")
        self._flag(skip_flag, "skip_flag")
        _check_device(grads=grads, momenta=momenta, partitions=partitions, skip_flag=skip_flag)
        muon_step_noalloc(self.plan, grads, momenta, partitions, skip_flag, grad_scale, stream)

    def check_finite(self, grads, dtype: str, flag, ws, stream=None):
        _check_bufs(grads, self._mat_numels(), dtype, "grads")
        self._flag(flag, "flag")
        _check_device(grads=grads, flag=flag, ws=ws)
        muon_check_finite(self.plan, grads, dtype, flag, ws, self._ws(ws), stream)

    def apply_update(self, params, partitions, lr: float, weight_decay: float, max_norm: float, ws,
                     skip_flag=None, norm_clip_out=None, stream=None):
        _check_bufs(params, self._part_numels(), "fp32", "params")
        _check_bufs(partitions, self._part_numels(), "fp32", "partitions")
        self._flag(skip_flag, "skip_flag")
        if norm_clip_out is not None and not isinstance(norm_clip_out, int):
            _check_bufs([norm_clip_out], [2], "fp32", "norm_clip_out")
        _check_device(params=params, partitions=partitions, skip_flag=skip_flag, norm_clip_out=norm_clip_out, ws=ws)
        muon_apply_update(self.plan, params, partitions, lr, weight_decay, max_norm, skip_flag, norm_clip_out, ws,
                          self._ws(ws), stream)

    def accumulate(self, acc, grad_mb, mb_dtype: str, first: bool, ws, stream=None):
        _check_bufs(acc, self._mat_numels(), "fp32", "acc")
        _check_bufs(grad_mb, self._mat_numels(), mb_dtype, "grad_mb")
        _check_device(acc=acc, grad_mb=grad_mb, ws=ws)
        muon_accumulate(self.plan, acc, grad_mb, mb_dtype, first, ws, self._ws(ws), stream)

    def scatter(self, updates, dtype: str, partitions, ws, stream=None):
        _check_bufs(updates, self._mat_numels(), dtype, "updates")
        _check_bufs(partitions, self._part_numels(), "fp32", "partitions")
        _check_device(updates=updates, partitions=partitions, ws=ws)
        muon_scatter(self.plan, updates, dtype, partitions, ws, self._ws(ws), stream)

    def stats(self) -> dict:
        return muon_plan_stats(self.plan)

    def runs(self, matrix: int) -> list:
        return muon_plan_runs(self.plan, matrix)

    def problems(self) -> list:
        return muon_plan_problems(self.plan)

    def set_timing(self, enable: bool = True):
        muon_plan_set_timing(self.plan, enable)

    def phase_ms(self):
        return muon_plan_phase_ms(self.plan)

    def close(self):
        if getattr(self, "plan", None):
            muon_plan_destroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

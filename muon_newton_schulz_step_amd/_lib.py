"""ctypes binding of libmuon_mi355x.so, with the C ABI's names.

Argument marshalling only: every step of the Muon path runs in the library's
HIP kernels.  There is no fallback: if the compiled library is missing the
import of any entry point raises.  Device buffers are passed as integers
(device addresses) or as objects with a ``data_ptr()`` method (torch tensors);
streams as integers (hipStream_t) or objects with a ``cuda_stream``
attribute.
"""

from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libmuon_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

MUON_OK = 0
STATUS = {0: "MUON_OK", 1: "MUON_ERR_INVALID_ARG", 2: "MUON_ERR_UNSUPPORTED", 3: "MUON_ERR_LAYOUT",
          4: "MUON_ERR_ALIAS", 5: "MUON_ERR_WORKSPACE", 6: "MUON_ERR_HIP"}
NS_METHOD = {"standard": 0, "gram": 1}
PRECISION = {"fp32": 0, "bf16": 1}
DTYPE = {"fp32": 0, "bf16": 1}
SCHEDULE = {"launches": 0, "persistent": 1}

# every symbol include/muon.h declares
EXPORTS = ("muon_default_options", "muon_plan_create", "muon_plan_workspace_bytes", "muon_accumulate",
           "muon_step", "muon_step_ex", "muon_step_noalloc", "muon_check_finite", "muon_apply_update", "muon_scatter",
           "muon_plan_stats", "muon_plan_runs", "muon_plan_problems", "muon_plan_set_timing",
           "muon_plan_phase_ms", "muon_plan_destroy", "muon_status_string", "muon_last_error")


class muon_matrix(C.Structure):
    _fields_ = [("rows", C.c_int64), ("cols", C.c_int64), ("num_heads", C.c_int32),
                ("reserved", C.c_int32), ("flat_offset", C.c_int64)]


class muon_options(C.Structure):
    _fields_ = [("beta", C.c_float), ("nesterov", C.c_int32), ("method", C.c_int32), ("ns_steps", C.c_int32),
                ("a", C.c_float), ("b", C.c_float), ("c", C.c_float), ("eps", C.c_float),
                ("precision", C.c_int32), ("grad_dtype", C.c_int32), ("max_inflight_bytes", C.c_uint64),
                ("schedule", C.c_int32), ("reserved", C.c_int32)]


class muon_layout(C.Structure):
    _fields_ = [("partition_numel", C.c_int64), ("num_partitions", C.c_int32), ("reserved", C.c_int32)]


class muon_stats(C.Structure):
    _fields_ = [("steps", C.c_uint64), ("ns_invocations", C.c_uint64), ("accumulations", C.c_uint64),
                ("waves", C.c_uint64), ("flagged_steps", C.c_uint64)]


class muon_run(C.Structure):
    _fields_ = [("matrix", C.c_int32), ("partition", C.c_int32), ("offset", C.c_int64), ("first", C.c_int64),
                ("length", C.c_int64)]


class muon_problem_info(C.Structure):
    _fields_ = [("matrix", C.c_int32), ("head", C.c_int32), ("m", C.c_int32), ("n", C.c_int32),
                ("transposed", C.c_int32), ("wave", C.c_int32), ("flops", C.c_double)]


_lib = None


def load(path: str | None = None) -> C.CDLL:
    """Load the compiled library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{LIB_NAME} is not built ({p} missing); run "
                          "`python -m muon_newton_schulz_step_amd.build` or __graft_entry__.build()")
    lib = C.CDLL(p)
    vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
    sig = {
        "muon_default_options": (i32, [C.POINTER(muon_options)]),
        "muon_plan_create": (i32, [C.POINTER(vp), C.POINTER(muon_matrix), i32, C.POINTER(muon_options),
                                   C.POINTER(muon_layout)]),
        "muon_plan_workspace_bytes": (i32, [vp, C.POINTER(sz)]),
        "muon_accumulate": (i32, [vp, C.POINTER(vp), C.POINTER(vp), i32, i32, vp, sz, vp]),
        "muon_step": (i32, [vp, C.POINTER(vp), C.POINTER(vp), C.POINTER(vp), vp, sz, vp]),
        "muon_step_ex": (i32, [vp, C.POINTER(vp), C.POINTER(vp), C.POINTER(vp), vp, C.c_float, vp, sz, vp]),
        "muon_step_noalloc": (i32, [vp, C.POINTER(vp), C.POINTER(vp), C.POINTER(vp), vp, C.c_float, vp]),
        "muon_check_finite": (i32, [vp, C.POINTER(vp), i32, vp, vp, sz, vp]),
        "muon_apply_update": (i32, [vp, C.POINTER(vp), C.POINTER(vp), C.c_float, C.c_float, C.c_float, vp, vp,
                                    vp, sz, vp]),
        "muon_scatter": (i32, [vp, C.POINTER(vp), i32, C.POINTER(vp), vp, sz, vp]),
        "muon_plan_stats": (i32, [vp, C.POINTER(muon_stats)]),
        "muon_plan_runs": (i32, [vp, i32, C.POINTER(muon_run), i32, C.POINTER(i32)]),
        "muon_plan_problems": (i32, [vp, C.POINTER(muon_problem_info), i32, C.POINTER(i32)]),
        "muon_plan_set_timing": (i32, [vp, i32]),
        "muon_plan_phase_ms": (i32, [vp, C.POINTER(C.c_float), C.POINTER(i32)]),
        "muon_plan_destroy": (None, [vp]),
        "muon_status_string": (C.c_char_p, [i32]),
        "muon_last_error": (C.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if path is None:
        _lib = lib
    return lib


class MuonError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{where}: {self.name}: {detail}")


def _check(st: int, where: str) -> None:
    if st != MUON_OK:
        detail = load().muon_last_error()
        raise MuonError(st, where, detail.decode() if detail else "")


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(s) -> int:
    if s is None:
        try:
            import torch  # only for the caller's current stream
            if torch.cuda.is_available():
                return int(torch.cuda.current_stream().cuda_stream)
        except ImportError:
            pass
        return 0
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


def _dt(x) -> int:
    return x if isinstance(x, int) else DTYPE[x]


# (matrices, partitions) of every live plan made by muon_plan_create, so a
# pointer table of the wrong length is refused here instead of being read
# past its end by the library
_PLAN_COUNTS: dict = {}


def _counts(plan):
    key = plan.value if isinstance(plan, C.c_void_p) else int(plan or 0)
    return _PLAN_COUNTS.get(key)


def _ptr_table(xs, expect=None, what: str = "table"):
    xs = list(xs)
    if expect is not None and len(xs) != expect:
        raise ValueError(f"{what}: {len(xs)} entries, the plan has {expect}")
    arr = (C.c_void_p * max(1, len(xs)))()
    for i, x in enumerate(xs):
        arr[i] = _ptr(x)
    return arr


def _nmat(plan):
    c = _counts(plan)
    return None if c is None else c[0]


def _nparts(plan):
    c = _counts(plan)
    return None if c is None else c[1]


def _ws_bytes(ws, ws_bytes: int) -> int:
    """The byte count handed to the library: the caller's figure, refused if
    it claims more than a tensor workspace holds past its data pointer."""
    ws_bytes = int(ws_bytes)
    if hasattr(ws, "numel") and hasattr(ws, "element_size"):
        have = int(ws.numel()) * int(ws.element_size())
        if ws_bytes > have:
            raise ValueError(f"workspace: ws_bytes {ws_bytes} exceeds the tensor's {have} bytes")
    return ws_bytes


def muon_default_options() -> muon_options:
    o = muon_options()
    _check(load().muon_default_options(C.byref(o)), "muon_default_options")
    return o


def muon_plan_create(matrices, options: muon_options, layout: muon_layout) -> C.c_void_p:
    """matrices: sequence of (rows, cols, num_heads, flat_offset)."""
    mats = (muon_matrix * max(1, len(matrices)))()
    for i, (r, c, h, off) in enumerate(matrices):
        mats[i] = muon_matrix(int(r), int(c), int(h or 0), 0, int(off))
    out = C.c_void_p()
    _check(load().muon_plan_create(C.byref(out), mats, len(matrices), C.byref(options), C.byref(layout)),
           "muon_plan_create")
    _PLAN_COUNTS[out.value] = (len(matrices), int(layout.num_partitions))
    return out


def muon_plan_workspace_bytes(plan) -> int:
    v = C.c_size_t()
    _check(load().muon_plan_workspace_bytes(plan, C.byref(v)), "muon_plan_workspace_bytes")
    return int(v.value)


def muon_accumulate(plan, acc, grad_mb, mb_dtype: str, first: bool, ws, ws_bytes: int, stream=None) -> None:
    n = _nmat(plan)
    _check(load().muon_accumulate(plan, _ptr_table(acc, n, "acc"), _ptr_table(grad_mb, n, "grad_mb"),
                                  _dt(mb_dtype), int(bool(first)), _ptr(ws), _ws_bytes(ws, ws_bytes),
                                  _stream(stream)), "muon_accumulate")


def muon_step(plan, grads, momenta, partitions, ws, ws_bytes: int, stream=None) -> None:
    n, r = _nmat(plan), _nparts(plan)
    _check(load().muon_step(plan, _ptr_table(grads, n, "grads"), _ptr_table(momenta, n, "momenta"),
                            _ptr_table(partitions, r, "partitions"), _ptr(ws), _ws_bytes(ws, ws_bytes),
                            _stream(stream)), "muon_step")


def muon_step_ex(plan, grads, momenta, partitions, skip_flag, grad_scale: float, ws, ws_bytes: int,
                 stream=None) -> None:
    n, r = _nmat(plan), _nparts(plan)
    _check(load().muon_step_ex(plan, _ptr_table(grads, n, "grads"), _ptr_table(momenta, n, "momenta"),
                               _ptr_table(partitions, r, "partitions"), _ptr(skip_flag), float(grad_scale),
                               _ptr(ws), _ws_bytes(ws, ws_bytes), _stream(stream)), "muon_step_ex")


# size of the library's static workspace array (MUON_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


def muon_step_noalloc(plan, grads, momenta, partitions, skip_flag=None, grad_scale: float = 1.0,
                      stream=None) -> None:
    n, r = _nmat(plan), _nparts(plan)
    _check(load().muon_step_noalloc(plan, _ptr_table(grads, n, "grads"), _ptr_table(momenta, n, "momenta"),
                                    _ptr_table(partitions, r, "partitions"), _ptr(skip_flag), float(grad_scale),
                                    _stream(stream)), "muon_step_noalloc")


def muon_check_finite(plan, grads, dtype: str, flag, ws, ws_bytes: int, stream=None) -> None:
    _check(load().muon_check_finite(plan, _ptr_table(grads, _nmat(plan), "grads"), _dt(dtype), _ptr(flag),
                                    _ptr(ws), _ws_bytes(ws, ws_bytes), _stream(stream)), "muon_check_finite")


def muon_apply_update(plan, params, partitions, lr: float, weight_decay: float, max_norm: float, skip_flag,
                      norm_clip_out, ws, ws_bytes: int, stream=None) -> None:
    r = _nparts(plan)
    _check(load().muon_apply_update(plan, _ptr_table(params, r, "params"), _ptr_table(partitions, r, "partitions"),
                                    float(lr), float(weight_decay), float(max_norm), _ptr(skip_flag),
                                    _ptr(norm_clip_out), _ptr(ws), _ws_bytes(ws, ws_bytes), _stream(stream)),
           "muon_apply_update")


def muon_scatter(plan, updates, dtype: str, partitions, ws, ws_bytes: int, stream=None) -> None:
    _check(load().muon_scatter(plan, _ptr_table(updates, _nmat(plan), "updates"), _dt(dtype),
                               _ptr_table(partitions, _nparts(plan), "partitions"), _ptr(ws),
                               _ws_bytes(ws, ws_bytes), _stream(stream)), "muon_scatter")


def muon_plan_stats(plan) -> dict:
    s = muon_stats()
    _check(load().muon_plan_stats(plan, C.byref(s)), "muon_plan_stats")
    return {"steps": s.steps, "ns_invocations": s.ns_invocations, "accumulations": s.accumulations,
            "waves": s.waves, "flagged_steps": s.flagged_steps}


def muon_plan_runs(plan, matrix: int) -> list:
    n = C.c_int32()
    _check(load().muon_plan_runs(plan, matrix, None, 0, C.byref(n)), "muon_plan_runs")
    arr = (muon_run * max(1, n.value))()
    _check(load().muon_plan_runs(plan, matrix, arr, n.value, C.byref(n)), "muon_plan_runs")
    return [(r.partition, r.offset, r.first, r.length) for r in arr[:n.value]]


def muon_plan_problems(plan) -> list:
    n = C.c_int32()
    _check(load().muon_plan_problems(plan, None, 0, C.byref(n)), "muon_plan_problems")
    arr = (muon_problem_info * max(1, n.value))()
    _check(load().muon_plan_problems(plan, arr, n.value, C.byref(n)), "muon_plan_problems")
    return [dict(matrix=q.matrix, head=q.head, m=q.m, n=q.n, transposed=bool(q.transposed), wave=q.wave,
                 flops=q.flops) for q in arr[:n.value]]


def muon_plan_set_timing(plan, enable: bool) -> None:
    _check(load().muon_plan_set_timing(plan, int(bool(enable))), "muon_plan_set_timing")


def muon_plan_phase_ms(plan):
    """(k1_ms, ns_ms, k3_ms, ns_launches) of the last timed step."""
    out = (C.c_float * 3)()
    n = C.c_int32()
    _check(load().muon_plan_phase_ms(plan, out, C.byref(n)), "muon_plan_phase_ms")
    return float(out[0]), float(out[1]), float(out[2]), int(n.value)


def muon_plan_destroy(plan) -> None:
    if plan:
        c = _counts(plan)
        if c is not None:
            _PLAN_COUNTS.pop(plan.value if isinstance(plan, C.c_void_p) else int(plan), None)
        load().muon_plan_destroy(plan)


def muon_status_string(status: int) -> str:
    return load().muon_status_string(status).decode()


def muon_last_error() -> str:
    v = load().muon_last_error()
    return v.decode() if v else ""

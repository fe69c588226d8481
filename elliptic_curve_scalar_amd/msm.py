"""ctypes binding of libmsm (include/msm.h): argument marshalling only.

Every step of the multi-scalar multiplication runs in the library's HIP kernels;
torch provides device memory and the stream. Tensors are contiguous 4-byte-element
(uint32 or int32) device tensors: points [n, 16], scalars [n, 8]. There is no CPU
fallback: if ``libmsm.so`` is missing this module raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsm.so")

MSM_OK, MSM_ERR_ARG, MSM_ERR_HIP, MSM_ERR_OOM, MSM_ERR_RANGE, MSM_ERR_OFF_CURVE = 0, -1, -2, -3, -4, -5
MSM_SCHED_PAIR_TREE, MSM_SCHED_WALKER = 0, 1
MSM_SCALARS_INTEGER, MSM_SCALARS_MONTGOMERY = 0, 1
MSM_MAX_N = 1 << 26
MSM_NOALLOC_MAX_BYTES = 64 << 20
VALID_S = (4, 8, 16, 32)

# Exported C symbols, each with (restype, argtypes).
_P, _S, _I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
SYMBOLS = {
    "msm_version": (_I, []),
    "msm_last_error": (ctypes.c_char_p, []),
    "msm_ctx_create": (_I, [_I, ctypes.POINTER(_P)]),
    "msm_ctx_destroy": (None, [_P]),
    "msm_workspace_bytes": (_S, [_S, _I, _I]),
    "msm_run": (_I, [_P, _P, _P, _S, _I, _I, _I, _I, _P, _S, _P, _P]),
    "msm": (_I, [_P, _P, _S, _I, _P]),
    "msm_run_noalloc": (_I, [_P, _P, _P, _S, _I, _I, _I, _I, _P, _P]),
    "msm_g1_from_scalars": (_I, [_P, _S, _P, _P]),
    "msm_ctx_set_affine_levels": (_I, [_P, _I]),
    "msm_ctx_set_walker_state": (_I, [_P, _I]),
    "msm_ctx_set_prefix_store": (_I, [_P, _I]),
    "msm_ctx_set_scalar_form": (_I, [_P, _I]),
    "msm_ctx_set_timing": (_I, [_P, _I]),
    "msm_ctx_timing_read": (_I, [_P, _P]),
    "msm_test_fp": (_I, [_I, _P, _P, _P, _S, _P]),
    "msm_test_fp_mul": (_I, [_P, _P, _P, _S, _P]),
    "msm_test_fp_add": (_I, [_P, _P, _P, _S, _P]),
    "msm_test_fp_sub": (_I, [_P, _P, _P, _S, _P]),
    "msm_test_fp_sqr": (_I, [_P, _P, _S, _P]),
    "msm_test_fp_inv": (_I, [_P, _P, _S, _P]),
    "msm_test_batched_add": (_I, [_P, _P, _P, _S, _I, _P]),
    "msm_test_glv": (_I, [_P, _S, _P, _P]),
    "msm_test_issue_rate": (_I, [_I, ctypes.c_uint32, ctypes.c_uint32, _P, _P]),
    "msm_test_row": (_I, [_I, _P, _P, _P, _S, ctypes.c_uint32, _P]),
}

_lib = None
_lock = threading.Lock()


class Timing(ctypes.Structure):
    _fields_ = [("sort_ms", ctypes.c_double), ("accumulate_ms", ctypes.c_double),
                ("level_kernel_ms", ctypes.c_double), ("reduce_ms", ctypes.c_double),
                ("final_ms", ctypes.c_double), ("runs", ctypes.c_int),
                ("level_launches", ctypes.c_int), ("level_pairs", ctypes.c_uint64),
                ("level_lanes", ctypes.c_uint64), ("xyzz_level_ms", ctypes.c_double)]


class MsmError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libmsm error {code}: {msg}")
        self.code = code


def lib():
    """Load libmsm.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
            L = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SYMBOLS.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
    return _lib


def _check(rc: int):
    if rc != MSM_OK:
        raise MsmError(rc, lib().msm_last_error().decode(errors="replace"))


def _dev_ptr(t: torch.Tensor | None, cols: int | None = None, name: str = "tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.element_size() != 4 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 32-bit tensor")
    if cols is not None and (t.dim() != 2 or t.shape[1] != cols):
        raise ValueError(f"{name} must have shape [n, {cols}]")
    return ctypes.c_void_p(t.data_ptr())


def _stream_handle(device: torch.device, stream=None):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def workspace_bytes(n: int, c: int, S: int = 8) -> int:
    return int(lib().msm_workspace_bytes(n, c, S))


class Context:
    """A libmsm context on one device. Workspace comes from torch's allocator.

    The C context orders consecutive runs on the device even across streams, so one
    workspace serves every stream; the workspace tensor is also marked as in use on
    each run's stream, so torch's allocator does not hand it out again (after it has
    grown, say) before the kernels queued there have finished with it.
    """

    def __init__(self, device=None):
        self.device = torch.device("cuda", torch.cuda.current_device() if device is None else
                                   torch.device(device).index or 0)
        h = ctypes.c_void_p()
        _check(lib().msm_ctx_create(self.device.index, ctypes.byref(h)))
        self._h = h
        self._ws = None
        self._need = {}  # workspace bytes per (n, c, S)

    def close(self):
        if getattr(self, "_h", None):
            lib().msm_ctx_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_affine_levels(self, levels: int):
        """Leading pair-tree levels done with batched affine adds (-1: all)."""
        _check(lib().msm_ctx_set_affine_levels(self._h, int(levels)))

    def set_walker_state(self, device_state: int):
        """Stream walker's accumulators: 1 in a device buffer, 0 in private memory."""
        _check(lib().msm_ctx_set_walker_state(self._h, int(device_state)))

    def set_prefix_store(self, store: int):
        """Pair-tree level-0 slot state: 0 private, 1 LDS, 2 private and 3 LDS with the
        denominators cached, 4 one prefix in four stored (checkpoints)."""
        _check(lib().msm_ctx_set_prefix_store(self._h, int(store)))

    def set_scalar_form(self, form: int):
        """MSM_SCALARS_INTEGER (default) or MSM_SCALARS_MONTGOMERY (x * 2^256 mod r)."""
        _check(lib().msm_ctx_set_scalar_form(self._h, int(form)))

    def set_timing(self, level: int = 2):
        """0 off, 1 the batched-affine level kernels only, 2 every phase (True = 2)."""
        level = 2 if level is True else 0 if level is False else int(level)
        _check(lib().msm_ctx_set_timing(self._h, level))

    def timing_read(self) -> dict:
        """Per-phase HIP-event times summed since the last read (waits for them)."""
        t = Timing()
        _check(lib().msm_ctx_timing_read(self._h, ctypes.byref(t)))
        return {name: getattr(t, name) for name, _ in Timing._fields_}

    def workspace(self, n: int, c: int, S: int) -> torch.Tensor:
        key = (n, c, S)
        need = self._need.get(key)
        if need is None:
            need = workspace_bytes(n, c, S)
            if need == 0:
                raise MsmError(MSM_ERR_ARG, "invalid n or c")
            self._need[key] = need
        if self._ws is None or self._ws.numel() < need + 256:
            self._ws = None  # the old block returns to the allocator, guarded by record_stream
            self._ws = torch.empty(need + 256, dtype=torch.uint8, device=self.device)
        return self._ws

    def run(self, points: torch.Tensor, scalars: torch.Tensor, c: int, S: int = 8,
            out: torch.Tensor | None = None, stream=None, sched: int = MSM_SCHED_PAIR_TREE,
            verify: bool = False) -> torch.Tensor:
        """Q = sum_i s_i P_i on the current (or given) stream; returns a [16] device
        tensor (affine x, y in Montgomery form; zeros for infinity)."""
        n = points.shape[0]
        if scalars.shape[0] != n:
            raise ValueError("points and scalars differ in length")
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        if out is None:
            out = torch.empty(16, dtype=torch.uint32, device=self.device)
        ws = self.workspace(n, c, S)
        base = ws.data_ptr()
        aligned = (base + 255) // 256 * 256
        rc = lib().msm_run(self._h, _dev_ptr(points, 16, "points"), _dev_ptr(scalars, 8, "scalars"),
                           n, c, S, int(sched), int(bool(verify)), ctypes.c_void_p(aligned),
                           ws.numel() - (aligned - base), ctypes.c_void_p(s.cuda_stream),
                           _dev_ptr(out, None, "out"))
        for t in (ws, out, points, scalars):
            t.record_stream(s)
        _check(rc)
        return out


_contexts: dict[int, Context] = {}


def context(device=None) -> Context:
    idx = torch.cuda.current_device() if device is None else torch.device(device).index or 0
    if idx not in _contexts:
        _contexts[idx] = Context(idx)
    return _contexts[idx]


def msm(points: torch.Tensor, scalars: torch.Tensor, c: int, S: int = 8, stream=None,
        sched: int = MSM_SCHED_PAIR_TREE, verify: bool = False) -> torch.Tensor:
    return context(points.device).run(points, scalars, c, S, stream=stream, sched=sched,
                                      verify=verify)


def msm_sync(points: torch.Tensor, scalars: torch.Tensor, c: int):
    """The synchronous C entry point ``msm`` (default context, S = 8): host result."""
    out = (ctypes.c_uint32 * 16)()
    _check(lib().msm(_dev_ptr(points, 16, "points"), _dev_ptr(scalars, 8, "scalars"),
                     points.shape[0], c, ctypes.cast(out, ctypes.c_void_p)))
    return list(out)


def g1_from_scalars(k: torch.Tensor, stream=None) -> torch.Tensor:
    """k [n, 8] device u32 -> points k_i * G as [n, 16] device u32."""
    n = k.shape[0]
    out = torch.empty((n, 16), dtype=torch.uint32, device=k.device)
    _check(lib().msm_g1_from_scalars(_dev_ptr(k, 8, "k"), n, _dev_ptr(out, 16, "out"),
                                     _stream_handle(k.device, stream)))
    return out


def test_fp(op: int, a: torch.Tensor, b: torch.Tensor | None = None) -> torch.Tensor:
    """Element-wise F_p operation ``op`` of msm_test_fp on [n, 8] device tensors."""
    out = torch.empty_like(a)
    _check(lib().msm_test_fp(op, _dev_ptr(a, 8, "a"), _dev_ptr(b, 8, "b"), _dev_ptr(out, 8, "out"),
                             a.shape[0], _stream_handle(a.device)))
    return out


def test_fp_named(name: str, a: torch.Tensor, b: torch.Tensor | None = None) -> torch.Tensor:
    """The named hooks msm_test_fp_{mul, sqr, add, sub, inv}."""
    out = torch.empty_like(a)
    fn = getattr(lib(), "msm_test_fp_" + name)
    if name in ("sqr", "inv"):
        rc = fn(_dev_ptr(a, 8, "a"), _dev_ptr(out, 8, "out"), a.shape[0], _stream_handle(a.device))
    else:
        rc = fn(_dev_ptr(a, 8, "a"), _dev_ptr(b, 8, "b"), _dev_ptr(out, 8, "out"), a.shape[0],
                _stream_handle(a.device))
    _check(rc)
    return out


def test_glv(scalars: torch.Tensor) -> torch.Tensor:
    """GLV halves of n scalars: (2n, 4) uint32, |k1| rows then |k2| rows, sign in bit 127."""
    n = scalars.shape[0]
    out = torch.empty((2 * n, 4), dtype=torch.uint32, device=scalars.device)
    _check(lib().msm_test_glv(_dev_ptr(scalars, 8, "scalars"), n, _dev_ptr(out, 4, "out"),
                              _stream_handle(scalars.device)))
    return out


def test_batched_add(a: torch.Tensor, b: torch.Tensor, S: int = 8) -> torch.Tensor:
    """a[i] + b[i] by the batched-affine adder, S slots per lane."""
    out = torch.empty_like(a)
    _check(lib().msm_test_batched_add(_dev_ptr(a, 16, "a"), _dev_ptr(b, 16, "b"),
                                      _dev_ptr(out, 16, "out"), a.shape[0], S,
                                      _stream_handle(a.device)))
    return out


def test_row(op: int, a: torch.Tensor, b: torch.Tensor | None = None, d: int = 0,
             stream=None) -> torch.Tensor:
    """Row-form hooks of msm_test_row: ops 0..2 field ops on [n, 8] tensors, ops 3 and 4
    2^d P on [n, 32] XYZZ points (row runs, quad runs), ops 5 and 6 the latency probe on
    four elements, op 7 P + Q and op 8 2P on [n, 32] XYZZ points in row form, op 9 the
    affine form ([n, 16]) of [n, 32] XYZZ points."""
    words = 32 if op in (3, 4, 7, 8, 9) else 8
    if b is not None and b.shape[0] < a.shape[0]:
        raise ValueError("b must have at least as many rows as a")
    if op == 9:
        out = torch.empty((a.shape[0], 16), dtype=a.dtype, device=a.device)
    else:
        out = torch.empty_like(a)
    _check(lib().msm_test_row(op, _dev_ptr(a, words, "a"), _dev_ptr(b, words, "b"),
                              _dev_ptr(out, 16 if op == 9 else words, "out"), a.shape[0], d,
                              _stream_handle(a.device, stream)))
    return out


def test_issue_rate(op: int, blocks: int, iters: int, out: torch.Tensor, stream=None):
    """Enqueue the instruction-rate probe (msm_test_issue_rate) writing into out
    (blocks * 256 uint32 words on the device)."""
    if out.numel() < blocks * 256:
        raise ValueError("out holds fewer than blocks * 256 words")
    _check(lib().msm_test_issue_rate(op, blocks, iters, _dev_ptr(out, None, "out"),
                                     _stream_handle(out.device, stream)))

"""Python binding of libzero_shard: one data-parallel rank's sharded ZeRO optimizer step on MI355X.

Argument marshalling only. Every step of the path runs in the HIP kernels of libzero_shard.so;
torch supplies device memory and the stream. The entry points carry the names of the C ABI in
``include/zero_shard.h``, where each one's arithmetic, layout, ownership and errors are stated.

The library must be built (``python -m zero_partition_plan_amd.build``); importing this package
without it raises, there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loaded first so the library binds to the HIP runtime torch uses)

__all__ = [
    "ZeroError", "ZeroPlan", "ZeroAdamHParams", "ZeroAdamScalars", "ZeroStageChoice",
    "ZeroOffloadBuffers", "lib", "lib_path", "offload_buffers",
    "ZERO_MAX_REPLICAS", "ZERO_MAX_SHARDS", "ZERO_F32", "ZERO_F16", "ZERO_BF16",
    "ZERO_ADAMW", "ZERO_ADAM_L2", "ZERO_DEV_T_OUT_OF_TABLE", "adam_hparams",
    "zero_partition_plan", "zero_shard_range", "zero_stage_bytes", "zero_stage_comm_bytes",
    "zero_choose_stage",
    "zero_adam_derive", "ZeroArenaArray", "zero_arena_layout", "zero_arena_alloc", "zero_arena_free",
    "arena",
    "zero_sq_partials_len", "zero_reduce_shard", "zero_shard_sqnorm", "zero_reduce_shard_static",
    "ZERO_STATIC_SQ_PARTIALS", "ZERO_STATIC_MAX_ELEMS", "zero_adam_shard_step",
    "zero_adam_shard_step_dev_scale", "zero_clip_scale", "zero_adam_derive_table", "adam_table",
    "zero_adam_shard_step_dev_t",
    "AdamStep", "ReduceCall",
    "zero_gather_params", "zero_host_adam_step", "zero_offload_step",
    "zero_status_str", "zero_last_error",
]

ZERO_MAX_REPLICAS = 64
ZERO_MAX_SHARDS = 64
ZERO_OK, ZERO_E_INVAL, ZERO_E_OVERFLOW, ZERO_E_UNSUPPORTED, ZERO_E_HIP = range(5)
ZERO_F32, ZERO_F16, ZERO_BF16 = 0, 1, 2
ZERO_ADAMW, ZERO_ADAM_L2 = 0, 1
ZERO_DEV_T_OUT_OF_TABLE = 1
ZERO_STATIC_SQ_PARTIALS = 4 << 20
ZERO_STATIC_MAX_ELEMS = (ZERO_STATIC_SQ_PARTIALS - 1024) * 256

_TORCH_DT = {torch.float32: ZERO_F32, torch.float16: ZERO_F16, torch.bfloat16: ZERO_BF16}


class ZeroError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        self.status = status
        super().__init__(f"{fn}: {zero_status_str(status)} ({detail})")


class ZeroPlan(ctypes.Structure):
    _fields_ = [("n", ctypes.c_uint64), ("padded_n", ctypes.c_uint64),
                ("shard_elems", ctypes.c_uint64), ("pad", ctypes.c_uint64),
                ("nd", ctypes.c_uint32), ("align_elems", ctypes.c_uint32)]

    def __repr__(self):
        return (f"ZeroPlan(n={self.n}, padded_n={self.padded_n}, shard_elems={self.shard_elems}, "
                f"pad={self.pad}, nd={self.nd}, align_elems={self.align_elems})")


class _GradSrc(ctypes.Structure):
    _fields_ = [("ptrs", ctypes.POINTER(ctypes.c_void_p)), ("count", ctypes.c_uint32),
                ("dtype", ctypes.c_int32)]


class ZeroAdamHParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double),
                ("wd_mode", ctypes.c_int32), ("reserved", ctypes.c_int32), ("step", ctypes.c_int64)]


class ZeroStageChoice(ctypes.Structure):
    _fields_ = [("stage", ctypes.c_uint32), ("offload_advised", ctypes.c_uint32),
                ("bytes", ctypes.c_uint64 * 4)]


class ZeroOffloadBuffers(ctypes.Structure):
    _fields_ = [("d_grad", ctypes.c_void_p), ("h_grad", ctypes.c_void_p), ("h_param", ctypes.c_void_p),
                ("chunk_elems", ctypes.c_uint64), ("threads", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32), ("h2d_stream", ctypes.c_void_p),
                ("events", ctypes.c_void_p * 4)]


class ZeroArenaArray(ctypes.Structure):
    _fields_ = [("bytes", ctypes.c_uint64), ("hot_offset", ctypes.c_uint64), ("group", ctypes.c_uint32),
                ("elem_bytes", ctypes.c_uint32)]


class ZeroAdamScalars(ctypes.Structure):
    _fields_ = [(k, ctypes.c_float) for k in ("b1", "b2", "c1", "c2", "ss", "bc", "e", "dec", "w")]


def adam_hparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, wd_mode="adamw",
                 step=1) -> ZeroAdamHParams:
    mode = {"adamw": ZERO_ADAMW, "l2": ZERO_ADAM_L2}.get(wd_mode, wd_mode)
    return ZeroAdamHParams(lr, beta1, beta2, eps, weight_decay, int(mode), 0, int(step))


_lib = None


def lib_path() -> str:
    return os.environ.get("ZERO_SHARD_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                            "libzero_shard.so")


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built: run `python -m zero_partition_plan_amd.build`")
        L = ctypes.CDLL(path)
        u64, u32, i32, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int32, ctypes.c_void_p
        P = ctypes.POINTER
        sig = {
            "zero_partition_plan": [u64, u32, u32, P(ZeroPlan)],
            "zero_shard_range": [P(ZeroPlan), u32, P(u64), P(u64)],
            "zero_stage_bytes": [P(ZeroPlan), u32, u32, u32, u32, P(u64)],
            "zero_stage_comm_bytes": [P(ZeroPlan), u32, u32, u32, P(u64)],
            "zero_choose_stage": [P(ZeroPlan), u64, u32, u32, u32, P(ZeroStageChoice)],
            "zero_adam_derive": [P(ZeroAdamHParams), P(ZeroAdamScalars)],
            "zero_arena_layout": [P(ZeroArenaArray), u32, P(u64), P(u64)],
            "zero_arena_alloc": [u64, P(vp), P(i32)],
            "zero_arena_free": [vp],
            "zero_reduce_shard": [P(_GradSrc), u64, vp, vp, vp, ctypes.c_double, vp],
            "zero_shard_sqnorm": [vp, u64, ctypes.c_double, vp, vp, vp],
            "zero_reduce_shard_static": [P(_GradSrc), u64, vp, vp, ctypes.c_double, vp, vp],
            "zero_adam_shard_step": [P(_GradSrc), u64, ctypes.c_float, vp, vp, vp,
                                     P(ZeroAdamHParams), vp, i32, vp, vp],
            "zero_adam_shard_step_dev_scale": [P(_GradSrc), u64, vp, vp, vp, vp,
                                               P(ZeroAdamHParams), vp, i32, vp, vp],
            "zero_clip_scale": [vp, ctypes.c_double, ctypes.c_double, ctypes.c_double, vp, vp],
            "zero_adam_derive_table": [P(ZeroAdamHParams), u32, P(ZeroAdamScalars)],
            "zero_adam_shard_step_dev_t": [P(_GradSrc), u64, vp, vp, u32, vp, vp, i32, vp, vp, vp,
                                           vp, i32, vp, vp],
            "zero_gather_params": [P(vp), u32, u64, u32, u64, u64, vp, vp],
            "zero_host_adam_step": [vp, u64, ctypes.c_float, vp, vp, vp, P(ZeroAdamHParams), vp, i32,
                                    u32],
            "zero_offload_step": [P(_GradSrc), u64, ctypes.c_float, vp, vp, vp, P(ZeroAdamHParams),
                                  vp, i32, P(ZeroOffloadBuffers), vp],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.zero_sq_partials_len.argtypes = [u64]
        L.zero_sq_partials_len.restype = u64
        L.zero_status_str.argtypes = [ctypes.c_int]
        L.zero_status_str.restype = ctypes.c_char_p
        L.zero_last_error.argtypes = []
        L.zero_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def zero_status_str(status: int) -> str:
    return lib().zero_status_str(status).decode()


def zero_last_error() -> str:
    return lib().zero_last_error().decode()


def _check(status: int, fn: str):
    if status != ZERO_OK:
        raise ZeroError(status, fn, zero_last_error())


# ------------------------------------------------------------------------------ host-only calls

def zero_partition_plan(n: int, nd: int, align_elems: int = 1) -> ZeroPlan:
    p = ZeroPlan()
    _check(lib().zero_partition_plan(n, nd, align_elems, ctypes.byref(p)), "zero_partition_plan")
    return p


def zero_shard_range(plan: ZeroPlan, rank: int) -> tuple[int, int]:
    b, v = ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib().zero_shard_range(ctypes.byref(plan), rank, ctypes.byref(b), ctypes.byref(v)),
           "zero_shard_range")
    return b.value, v.value


def zero_stage_bytes(plan: ZeroPlan, stage: int, param_b: int = 2, grad_b: int = 2,
                     opt_b: int = 12) -> tuple[int, int, int, int]:
    out = (ctypes.c_uint64 * 4)()
    _check(lib().zero_stage_bytes(ctypes.byref(plan), stage, param_b, grad_b, opt_b, out),
           "zero_stage_bytes")
    return tuple(int(x) for x in out)


def zero_stage_comm_bytes(plan: ZeroPlan, stage: int, param_b: int = 2,
                          grad_b: int = 2) -> tuple[int, int, int]:
    """(gradient, parameter, total) bytes one rank sends per step; stage 0 = DP, 1..3."""
    out = (ctypes.c_uint64 * 3)()
    _check(lib().zero_stage_comm_bytes(ctypes.byref(plan), stage, param_b, grad_b, out),
           "zero_stage_comm_bytes")
    return tuple(int(x) for x in out)


def zero_choose_stage(plan: ZeroPlan, usable_bytes: int, param_b: int = 2, grad_b: int = 2,
                      opt_b: int = 12) -> tuple[int, bool, tuple[int, int, int, int]]:
    """(stage 1..3, offload advised, the stage's per-rank bytes) for a usable byte budget."""
    out = ZeroStageChoice()
    _check(lib().zero_choose_stage(ctypes.byref(plan), usable_bytes, param_b, grad_b, opt_b,
                                   ctypes.byref(out)), "zero_choose_stage")
    return int(out.stage), bool(out.offload_advised), tuple(int(x) for x in out.bytes)


def zero_adam_derive(hp: ZeroAdamHParams) -> ZeroAdamScalars:
    out = ZeroAdamScalars()
    _check(lib().zero_adam_derive(ctypes.byref(hp), ctypes.byref(out)), "zero_adam_derive")
    return out


def zero_adam_derive_table(hp: ZeroAdamHParams, count: int):
    """The constants of steps 1..count (hp.step ignored) as a ctypes array of ZeroAdamScalars."""
    out = (ZeroAdamScalars * count)()
    _check(lib().zero_adam_derive_table(ctypes.byref(hp), count, out), "zero_adam_derive_table")
    return out


def adam_table(hp: ZeroAdamHParams, count: int, device="cuda") -> torch.Tensor:
    """zero_adam_derive_table's constants as a (count, 9) float32 tensor on ``device``, laid out
    as the device table of zero_adam_shard_step_dev_t expects (one zero_adam_scalars per row)."""
    tab = zero_adam_derive_table(hp, count)
    host = torch.frombuffer(bytearray(tab), dtype=torch.float32).view(count, 9)
    return host.to(device)


def zero_arena_layout(arrays) -> tuple[list[int], int]:
    """arrays: sequence of (bytes, hot_offset, group, elem_bytes) -> (byte offsets, total bytes)."""
    n = len(arrays)
    arr = (ZeroArenaArray * max(n, 1))(*[ZeroArenaArray(int(b), int(h), int(g), int(e))
                                         for b, h, g, e in arrays])
    offs = (ctypes.c_uint64 * max(n, 1))()
    total = ctypes.c_uint64()
    _check(lib().zero_arena_layout(arr, n, offs, ctypes.byref(total)), "zero_arena_layout")
    return [int(offs[i]) for i in range(n)], int(total.value)


def zero_arena_alloc(nbytes: int) -> tuple[int | None, bool]:
    """(device pointer, physically contiguous?) of a new allocation on the current device."""
    ptr, contig = ctypes.c_void_p(), ctypes.c_int32()
    _check(lib().zero_arena_alloc(nbytes, ctypes.byref(ptr), ctypes.byref(contig)), "zero_arena_alloc")
    return ptr.value, bool(contig.value)


def zero_arena_free(ptr: int | None):
    _check(lib().zero_arena_free(ptr), "zero_arena_free")


class _ArenaMemory:
    """Owner of one zero_arena_alloc allocation, handed to torch as a uint8 array. torch keeps this
    object alive while any tensor on the memory lives, and the memory is freed with it."""

    def __init__(self, nbytes: int):
        self.ptr, self.contiguous = zero_arena_alloc(nbytes)
        self.__cuda_array_interface__ = {"shape": (nbytes,), "typestr": "|u1", "strides": None,
                                         "data": (self.ptr, False), "version": 2}

    def __del__(self):
        # a destructor does not raise; hipFree waits for the device before releasing the memory
        ptr, self.ptr = getattr(self, "ptr", None), None
        if ptr and _lib is not None:
            _lib.zero_arena_free(ptr)


def arena(specs, device="cuda", contiguous: bool = True):
    """One device allocation holding every array of ``specs`` where zero_arena_layout places it.

    specs: sequence of (name, numel, dtype, group, hot_elem): hot_elem is the element at which the
    kernels' walk over the array starts (0, or r*S for rank r's slot in a gathered buffer). With
    ``contiguous`` (device memory only) the allocation comes from zero_arena_alloc, physically
    contiguous when the device can give it; otherwise from torch. Returns (storage, {name: 1-D
    view}); the views live as long as the storage, and ``storage.zero_arena_contiguous`` says
    whether the memory is physically contiguous.
    """
    specs = list(specs)
    es = [torch.empty(0, dtype=dt).element_size() for _, _, dt, _, _ in specs]
    offs, total = zero_arena_layout([(n * e, h * e, g, e) for (_, n, _, g, h), e in zip(specs, es)])
    dev = torch.device(device)
    if contiguous and dev.type == "cuda":
        with torch.cuda.device(dev):
            mem = _ArenaMemory(max(total, 1))
            storage = torch.as_tensor(mem, device=dev)
        if storage.data_ptr() != mem.ptr or storage.numel() != max(total, 1):
            raise RuntimeError("torch did not wrap the arena allocation in place")
        storage.zero_arena_contiguous = mem.contiguous
    else:
        storage = torch.empty(max(total, 1), dtype=torch.uint8, device=dev)
        storage.zero_arena_contiguous = False
    views = {name: storage[o:o + n * e].view(dt) for (name, n, dt, _, _), o, e in zip(specs, offs, es)}
    return storage, views


# ------------------------------------------------------------------------------ device calls

def _ptr(t, n: int, what: str, dtype=None, pinned_ok: bool = False) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not (t.is_cuda or (pinned_ok and t.is_pinned())):
        raise TypeError(f"{what} must be a device tensor" + (" or pinned host memory" if pinned_ok else ""))
    if dtype is not None and t.dtype not in dtype:
        raise TypeError(f"{what}: dtype {t.dtype} not in {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if t.numel() < n:
        raise ValueError(f"{what} holds {t.numel()} elements, {n} needed")
    return t.data_ptr()


def _src(reps, n: int):
    """Replica list (or a 2-D tensor whose rows are replicas) -> C gradient source."""
    rows = list(reps.unbind(0)) if isinstance(reps, torch.Tensor) and reps.dim() == 2 else list(reps)
    if not rows:
        raise ValueError("no gradient replicas")
    dt = rows[0].dtype
    if dt not in _TORCH_DT or any(r.dtype != dt for r in rows):
        raise TypeError("replicas must share one of float32, float16, bfloat16")
    arr = (ctypes.c_void_p * len(rows))(*[_ptr(r, n, f"replica {k}") for k, r in enumerate(rows)])
    return _GradSrc(ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), len(rows), _TORCH_DT[dt]), arr


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def zero_sq_partials_len(n: int) -> int:
    """Doubles the squared-norm partials buffer needs for a shard of n elements."""
    return int(lib().zero_sq_partials_len(n))


def zero_reduce_shard(reps, n: int, out_grad=None, nonfinite=None, sq_partials=None,
                      sq_scale: float = 1.0, stream=None):
    """``out_grad`` may also be pinned host memory, which the kernel then writes over the host link."""
    src, keep = _src(reps, n)
    _check(lib().zero_reduce_shard(
        ctypes.byref(src), n, _ptr(out_grad, n, "out_grad", (torch.float32,), pinned_ok=True),
        _ptr(nonfinite, 1, "nonfinite", (torch.int32,)),
        _ptr(sq_partials, zero_sq_partials_len(n), "sq_partials", (torch.float64,)),
        float(sq_scale), _stream(stream)), "zero_reduce_shard")


def zero_shard_sqnorm(grad, n: int, sq_scale: float, partials, out, stream=None):
    _check(lib().zero_shard_sqnorm(
        _ptr(grad, n, "grad", (torch.float32,)), n, float(sq_scale),
        _ptr(partials, zero_sq_partials_len(n), "partials", (torch.float64,)),
        _ptr(out, 1, "out", (torch.float64,)), _stream(stream)), "zero_shard_sqnorm")


def zero_reduce_shard_static(reps, n: int, out_grad=None, nonfinite=None, sq=None,
                             sq_scale: float = 1.0, stream=None):
    """zero_reduce_shard then the squared-norm finish into ``sq`` (float64 device tensor), with the
    partials in the library's own device scratch: no workspace argument, nothing allocated."""
    src, keep = _src(reps, n)
    _check(lib().zero_reduce_shard_static(
        ctypes.byref(src), n, _ptr(out_grad, n, "out_grad", (torch.float32,)),
        _ptr(nonfinite, 1, "nonfinite", (torch.int32,)), float(sq_scale),
        _ptr(sq, 1, "sq", (torch.float64,)), _stream(stream)), "zero_reduce_shard_static")


def _out_dtype(out) -> int:
    if out is None:
        return ZERO_F32
    if out.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("out must be bfloat16 or float16")
    return _TORCH_DT[out.dtype]


def zero_adam_shard_step(reps, n: int, grad_scale: float, master, m, v, hp: ZeroAdamHParams,
                         out=None, skip=None, stream=None):
    """``out``: bf16/fp16 device tensor view starting at the rank's slot (or None)."""
    src, keep = _src(reps, n)
    f32 = (torch.float32,)
    out_dt = _out_dtype(out)
    _check(lib().zero_adam_shard_step(
        ctypes.byref(src), n, float(grad_scale), _ptr(master, n, "master", f32),
        _ptr(m, n, "m", f32), _ptr(v, n, "v", f32), ctypes.byref(hp),
        _ptr(out, n, "out"), out_dt, _ptr(skip, 1, "skip", (torch.int32,)), _stream(stream)),
        "zero_adam_shard_step")


def zero_adam_shard_step_dev_scale(reps, n: int, grad_scale, master, m, v, hp: ZeroAdamHParams,
                                   out=None, skip=None, stream=None):
    """zero_adam_shard_step with ``grad_scale`` a float32 device tensor, read on the device (as
    zero_clip_scale writes it)."""
    src, keep = _src(reps, n)
    f32 = (torch.float32,)
    out_dt = _out_dtype(out)
    _check(lib().zero_adam_shard_step_dev_scale(
        ctypes.byref(src), n, _ptr(grad_scale, 1, "grad_scale", f32), _ptr(master, n, "master", f32),
        _ptr(m, n, "m", f32), _ptr(v, n, "v", f32), ctypes.byref(hp),
        _ptr(out, n, "out"), out_dt, _ptr(skip, 1, "skip", (torch.int32,)), _stream(stream)),
        "zero_adam_shard_step_dev_scale")


def zero_adam_shard_step_dev_t(reps, n: int, grad_scale, table, step, status, master, m, v,
                               wd_mode="adamw", out=None, skip=None, stream=None):
    """The step with its grad scale (float32 device tensor), constants table ((len, 9) float32
    device tensor, e.g. adam_table) and step counter (int64 device tensor) all on the device; the
    counter advances on the device unless ``skip`` is set. A counter outside the table refuses the
    update (nothing written, no advance) and sets ``status`` (int32 device tensor, zeroed by the
    caller) to ZERO_DEV_T_OUT_OF_TABLE."""
    src, keep = _src(reps, n)
    f32 = (torch.float32,)
    out_dt = _out_dtype(out)
    mode = {"adamw": ZERO_ADAMW, "l2": ZERO_ADAM_L2}.get(wd_mode, wd_mode)
    if not isinstance(table, torch.Tensor) or table.dim() != 2 or table.shape[1] != 9:
        raise ValueError("table must be a (len, 9) float32 device tensor")
    _check(lib().zero_adam_shard_step_dev_t(
        ctypes.byref(src), n, _ptr(grad_scale, 1, "grad_scale", f32),
        _ptr(table, table.numel(), "table", f32), table.shape[0],
        _ptr(step, 1, "step", (torch.int64,)), _ptr(status, 1, "status", (torch.int32,)), int(mode),
        _ptr(master, n, "master", f32), _ptr(m, n, "m", f32), _ptr(v, n, "v", f32),
        _ptr(out, n, "out"), out_dt, _ptr(skip, 1, "skip", (torch.int32,)), _stream(stream)),
        "zero_adam_shard_step_dev_t")


def zero_clip_scale(sq, max_norm: float, clip_eps: float, inv_loss_scale: float, grad_scale,
                    stream=None):
    """grad_scale[0] = fp32(min(1, max_norm / (sqrt(sq[0]) + clip_eps)) * inv_loss_scale), on the
    device: ``sq`` a float64 device tensor (zero_shard_sqnorm's output), ``grad_scale`` float32."""
    _check(lib().zero_clip_scale(
        _ptr(sq, 1, "sq", (torch.float64,)), float(max_norm), float(clip_eps), float(inv_loss_scale),
        _ptr(grad_scale, 1, "grad_scale", (torch.float32,)), _stream(stream)), "zero_clip_scale")


class AdamStep:
    """zero_adam_shard_step with its arrays and stream marshalled once; a call passes only the grad
    scale and the hyper-parameters (which change every step). For loops whose steps are short enough
    that per-call marshalling shows. The tensors must stay alive and in place while it is used."""

    def __init__(self, reps, n: int, master, m, v, out=None, skip=None, stream=None):
        self._src, self._keep = _src(reps, n)
        f32 = (torch.float32,)
        out_dt = _out_dtype(out)
        self._tensors = (reps, master, m, v, out, skip)
        self._fn = lib().zero_adam_shard_step
        self._args = (n, _ptr(master, n, "master", f32), _ptr(m, n, "m", f32), _ptr(v, n, "v", f32))
        self._tail = (_ptr(out, n, "out"), out_dt, _ptr(skip, 1, "skip", (torch.int32,)), _stream(stream))
        self._ref = ctypes.byref(self._src)

    def __call__(self, grad_scale: float, hp: ZeroAdamHParams):
        n, p, m, v = self._args
        _check(self._fn(self._ref, n, grad_scale, p, m, v, ctypes.byref(hp), *self._tail),
               "zero_adam_shard_step")


class ReduceCall:
    """zero_reduce_shard with its arrays and stream marshalled once; a call passes only sq_scale.
    For loops of launches short enough that per-call marshalling shows. The tensors must stay alive
    and in place while it is used."""

    def __init__(self, reps, n: int, out_grad=None, nonfinite=None, sq_partials=None, stream=None):
        self._src, self._keep = _src(reps, n)
        self._tensors = (reps, out_grad, nonfinite, sq_partials)
        self._fn = lib().zero_reduce_shard
        self._args = (ctypes.byref(self._src), n,
                      _ptr(out_grad, n, "out_grad", (torch.float32,), pinned_ok=True),
                      _ptr(nonfinite, 1, "nonfinite", (torch.int32,)),
                      _ptr(sq_partials, zero_sq_partials_len(n), "sq_partials", (torch.float64,)))
        self._stream = _stream(stream)

    def __call__(self, sq_scale: float = 1.0):
        _check(self._fn(*self._args, float(sq_scale), self._stream), "zero_reduce_shard")


def zero_gather_params(shards, begin: int, count: int, out, stream=None):
    """out[:count] = the rank shards laid end to end, elements [begin, begin + count).

    ``shards``: list of equally sized 1-D device tensors (one per rank; 16-bit or fp32), or a 2-D
    tensor whose rows are the shards. Shards the range does not touch may be None.
    """
    rows = list(shards.unbind(0)) if isinstance(shards, torch.Tensor) and shards.dim() == 2 else list(shards)
    if not rows or len(rows) > ZERO_MAX_SHARDS:
        raise ValueError(f"1..{ZERO_MAX_SHARDS} shards")
    ref = next((r for r in rows if r is not None), None)
    if ref is None:
        raise ValueError("every shard is None")
    S, dt = ref.numel(), ref.dtype
    eb = {torch.float16: 2, torch.bfloat16: 2, torch.int16: 2, torch.float32: 4, torch.int32: 4}.get(dt)
    if eb is None:
        raise TypeError(f"shard dtype {dt} is not a 2- or 4-byte type")
    ptrs = []
    for k, r in enumerate(rows):
        if r is None:
            ptrs.append(None)
            continue
        if r.dtype != dt or r.numel() != S:
            raise ValueError("shards must share one dtype and length")
        ptrs.append(_ptr(r, S, f"shard {k}"))
    if out is not None and out.element_size() != eb:
        raise TypeError("out must have the shards' element size")
    arr = (ctypes.c_void_p * len(rows))(*ptrs)
    _check(lib().zero_gather_params(ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), len(rows), S, eb,
                                    begin, count, _ptr(out, count, "out"), _stream(stream)),
           "zero_gather_params")


# ------------------------------------------------------------------------------ host (offload) calls

def _hptr(a, n: int, what: str, itemsize: int):
    """Host array (numpy array or CPU torch tensor) -> address, checked for size and layout."""
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        if a.is_cuda:
            raise TypeError(f"{what} must be host memory")
        if not a.is_contiguous() or a.element_size() != itemsize:
            raise ValueError(f"{what}: contiguous {itemsize}-byte elements expected")
        if a.numel() < n:
            raise ValueError(f"{what} holds {a.numel()} elements, {n} needed")
        return a.data_ptr()
    import numpy as np
    if not isinstance(a, np.ndarray) or not a.flags["C_CONTIGUOUS"] or a.itemsize != itemsize:
        raise ValueError(f"{what}: contiguous numpy array of {itemsize}-byte elements expected")
    if a.size < n:
        raise ValueError(f"{what} holds {a.size} elements, {n} needed")
    return a.ctypes.data


def zero_host_adam_step(grad, n: int, grad_scale: float, master, m, v, hp: ZeroAdamHParams,
                        out=None, out_dtype: int = ZERO_BF16, threads: int = 0):
    """The host update on host arrays (numpy or CPU tensors); ``out`` holds 16-bit patterns."""
    _check(lib().zero_host_adam_step(
        _hptr(grad, n, "grad", 4), n, float(grad_scale), _hptr(master, n, "master", 4),
        _hptr(m, n, "m", 4), _hptr(v, n, "v", 4), ctypes.byref(hp), _hptr(out, n, "out", 2),
        out_dtype, threads), "zero_host_adam_step")


def offload_buffers(chunk_elems: int, device="cuda", threads: int = 0, h2d_stream=None,
                    direct: bool = False) -> dict:
    """Caller-side staging for zero_offload_step: device and pinned host chunk buffers (x2) and
    the four events the step records and waits on (torch events, created here by recording each
    once). ``direct``: no device staging; the reduce kernel writes each chunk into the pinned host
    buffer itself."""
    events = [torch.cuda.Event(enable_timing=False) for _ in range(4)]
    for ev in events:
        ev.record()                    # torch creates an event's handle on its first record
    bufs = {
        "d_grad": None if direct else torch.empty(2 * chunk_elems, dtype=torch.float32, device=device),
        "h_grad": torch.empty(2 * chunk_elems, dtype=torch.float32, pin_memory=True),
        "h_param": torch.empty(2 * chunk_elems, dtype=torch.int16, pin_memory=True),
        "chunk_elems": chunk_elems, "threads": threads, "h2d_stream": h2d_stream, "events": events,
    }
    return bufs


def zero_offload_step(reps, n: int, grad_scale: float, h_master, h_m, h_v, hp: ZeroAdamHParams,
                      out, buffers: dict, stream=None):
    """Offloaded step: device replicas -> host Adam on host state -> 16-bit params into ``out``."""
    src, keep = _src(reps, n)
    if out is None or out.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("out must be a bfloat16 or float16 device tensor")
    C = int(buffers["chunk_elems"])
    b = ZeroOffloadBuffers(_ptr(buffers["d_grad"], 2 * C, "d_grad", (torch.float32,)),
                           _hptr(buffers["h_grad"], 2 * C, "h_grad", 4),
                           _hptr(buffers["h_param"], 2 * C, "h_param", 2), C, int(buffers["threads"]), 0,
                           None if buffers.get("h2d_stream") is None else _stream(buffers["h2d_stream"]),
                           (ctypes.c_void_p * 4)(*[ev.cuda_event for ev in buffers["events"]]))
    _check(lib().zero_offload_step(
        ctypes.byref(src), n, float(grad_scale), _hptr(h_master, n, "master", 4), _hptr(h_m, n, "m", 4),
        _hptr(h_v, n, "v", 4), ctypes.byref(hp), _ptr(out, n, "out"), _TORCH_DT[out.dtype],
        ctypes.byref(b), _stream(stream)), "zero_offload_step")

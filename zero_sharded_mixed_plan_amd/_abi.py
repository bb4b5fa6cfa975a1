"""ctypes binding of libzero_shard.so: the C ABI declared in include/zero_shard.h.

Argument marshalling only; every step of the computation runs in the library.
Functions keep the C names.  Device pointers are plain integers (e.g. a torch
tensor's data_ptr()); `stream` is a hipStream_t as an integer (0 = null stream).
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Tuple

# ZERO_SHARD_LIB selects another build of the same library (e.g. a tuning variant)
LIB_PATH = os.environ.get("ZERO_SHARD_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libzero_shard.so")

ZERO_OK, ZERO_EINVAL, ZERO_EALIGN, ZERO_ENOMEM, ZERO_EHIP, ZERO_EIO = 0, -1, -2, -3, -4, -5
ZERO_F32, ZERO_BF16, ZERO_F16 = 0, 1, 2
ZERO_STATE_SEPARATE, ZERO_STATE_TILED = 0, 1
ZERO_STATE_TILE = 2048
ZERO_GRAD_SHARD, ZERO_GRAD_FULL = 0, 1
DTYPE_CODES = {"f32": ZERO_F32, "bf16": ZERO_BF16, "f16": ZERO_F16}
DTYPE_BYTES = {ZERO_F32: 4, ZERO_BF16: 2, ZERO_F16: 2}

# every symbol the header declares
EXPORTS = [
    "zero_plan", "zero_plan_dim0", "zero_plan_free", "zero_plan_shard_numel", "zero_plan_total_numel",
    "zero_plan_padded_numel", "zero_plan_world", "zero_plan_num_buckets", "zero_plan_num_tensors",
    "zero_plan_bucket", "zero_plan_tensor", "zero_plan_rank_segment", "zero_plan_bytes",
    "zero_state_numel", "zero_workspace_bytes", "zero_plan_piece_table_bytes", "zero_plan_attach_piece_table",
    "zero_reduce_shard", "zero_shard_norm", "zero_noalloc_max_shard", "zero_reduce_norm_noalloc",
    "zero_adam_step", "zero_scaler_init", "zero_scaler_update", "zero_scaler_inv_scale", "zero_plan_hash",
    "zero_checkpoint_save", "zero_checkpoint_load", "zero_stream_copy", "zero_last_error", "zero_version",
]


class ZeroError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class zero_adam_args_t(ctypes.Structure):
    _fields_ = [
        ("rank", ctypes.c_int32),
        ("grad", ctypes.c_void_p),
        ("grad_ld", ctypes.c_int64),
        ("grad_dtype", ctypes.c_int),
        ("grad_count", ctypes.c_int32),
        ("grad_layout", ctypes.c_int32),
        ("inv_scale", ctypes.c_float),
        ("g_stash", ctypes.c_void_p),
        ("clip_coef", ctypes.c_void_p),
        ("state_layout", ctypes.c_int32),
        ("master_in", ctypes.c_void_p),
        ("m_in", ctypes.c_void_p),
        ("v_in", ctypes.c_void_p),
        ("master_out", ctypes.c_void_p),
        ("m_out", ctypes.c_void_p),
        ("v_out", ctypes.c_void_p),
        ("gather", ctypes.c_void_p),
        ("param_dtype", ctypes.c_int),
        ("lr", ctypes.c_double),
        ("beta1", ctypes.c_double),
        ("beta2", ctypes.c_double),
        ("eps", ctypes.c_double),
        ("weight_decay", ctypes.c_double),
        ("step", ctypes.c_int64),
        ("skip_in", ctypes.c_void_p),
        ("overflow_out", ctypes.c_void_p),
        ("ev_begin", ctypes.c_void_p),
        ("ev_end", ctypes.c_void_p),
        ("ctl", ctypes.c_void_p),
    ]


class zero_scaler_t(ctypes.Structure):
    _fields_ = [
        ("scale", ctypes.c_float),
        ("growth_tracker", ctypes.c_int32),
        ("growth_factor", ctypes.c_float),
        ("backoff_factor", ctypes.c_float),
        ("growth_interval", ctypes.c_int32),
    ]


class zero_step_ctl_t(ctypes.Structure):
    """Step control kept in device memory (this is its host image)."""
    _fields_ = [
        ("step", ctypes.c_int64),
        ("skipped", ctypes.c_int64),
        ("lr", ctypes.c_double),
        ("scaler", zero_scaler_t),
        ("dynamic", ctypes.c_int32),
        ("k", ctypes.c_float * 8),
    ]


class zero_ckpt_meta_t(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int64), ("scaler", zero_scaler_t)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the library once.  Fails loudly when it has not been built."""
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


def load(path: str, required: bool = True) -> ctypes.CDLL:
    """Load one build of the library from `path` and declare its C signatures
    (required=False skips entry points an older build does not export)."""
    # torch first: the library must bind to the HIP runtime torch already uses
    # for the device memory and streams it hands over (one runtime per process)
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m zero_sharded_mixed_plan_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(path)
    i32, i64, vp, f32, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_double
    P64, P32 = ctypes.POINTER(i64), ctypes.POINTER(i32)
    sig = {
        "zero_plan": (ctypes.c_int, [P64, i32, i32, i64, ctypes.POINTER(vp)]),
        "zero_plan_dim0": (ctypes.c_int, [P64, P64, i32, i32, ctypes.POINTER(vp)]),
        "zero_plan_free": (None, [vp]),
        "zero_plan_shard_numel": (i64, [vp]),
        "zero_plan_total_numel": (i64, [vp]),
        "zero_plan_padded_numel": (i64, [vp]),
        "zero_plan_world": (i32, [vp]),
        "zero_plan_num_buckets": (i32, [vp]),
        "zero_plan_num_tensors": (i32, [vp]),
        "zero_plan_bucket": (ctypes.c_int, [vp, i32, P64, P64, P64, P64, P32, P32]),
        "zero_plan_tensor": (ctypes.c_int, [vp, i32, P32, P64]),
        "zero_plan_rank_segment": (ctypes.c_int, [vp, i32, i32, P64, P64, P64]),
        "zero_plan_bytes": (ctypes.c_int, [vp, i32, ctypes.POINTER(f64), P64]),
        "zero_state_numel": (i64, [vp, i32]),
        "zero_workspace_bytes": (ctypes.c_size_t, [vp]),
        "zero_plan_piece_table_bytes": (i64, [vp]),
        "zero_plan_attach_piece_table": (ctypes.c_int, [vp, i32, vp, i64]),
        "zero_reduce_shard": (ctypes.c_int, [vp, i32, vp, i64, i32, i32, ctypes.c_int, f32, vp, vp, i32, vp, vp]),
        "zero_shard_norm": (ctypes.c_int, [vp, vp, f64, f64, vp, vp, vp, vp]),
        "zero_noalloc_max_shard": (i64, []),
        "zero_reduce_norm_noalloc": (ctypes.c_int, [vp, i32, vp, i64, i32, i32, ctypes.c_int, f32, vp, f64, f64,
                                                    vp, vp, vp, vp, vp]),
        "zero_adam_step": (ctypes.c_int, [vp, ctypes.POINTER(zero_adam_args_t), vp]),
        "zero_scaler_init": (ctypes.c_int, [ctypes.POINTER(zero_scaler_t), f32, f32, f32, i32]),
        "zero_scaler_update": (ctypes.c_int, [ctypes.POINTER(zero_scaler_t), i32]),
        "zero_scaler_inv_scale": (f32, [ctypes.POINTER(zero_scaler_t)]),
        "zero_plan_hash": (ctypes.c_uint64, [vp]),
        "zero_checkpoint_save": (ctypes.c_int, [vp, i32, ctypes.c_char_p, i32, vp, vp, vp,
                                                ctypes.POINTER(zero_ckpt_meta_t), vp]),
        "zero_checkpoint_load": (ctypes.c_int, [vp, i32, ctypes.c_char_p, i32, vp, vp, vp,
                                                ctypes.POINTER(zero_ckpt_meta_t), vp]),
        "zero_stream_copy": (ctypes.c_int, [vp, vp, i64, vp]),
        "zero_last_error": (ctypes.c_char_p, []),
        "zero_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        if not required and not hasattr(L, name):
            continue
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def _check(rc: int) -> None:
    if rc != ZERO_OK:
        raise ZeroError(rc, lib().zero_last_error().decode())


def zero_last_error() -> str:
    return lib().zero_last_error().decode()


def zero_version() -> str:
    return lib().zero_version().decode()


# ---------------------------------------------------------------------------
# planner
# ---------------------------------------------------------------------------

class Plan:
    """Owner of a zero_plan_t handle."""

    def __init__(self, numels, world: int, bucket_cap: int = 0, *, _handle=None):
        L = lib()
        if _handle is None:
            arr = (ctypes.c_int64 * len(numels))(*[int(n) for n in numels])
            h = ctypes.c_void_p()
            _check(L.zero_plan(arr, len(numels), int(world), int(bucket_cap), ctypes.byref(h)))
            _handle = h
        self._h = _handle
        self.world = int(world)

    @classmethod
    def dim0(cls, shapes, world: int) -> "Plan":
        """Per-parameter dim-0 layout (zero_plan_dim0) of parameters of the given shapes."""
        rows, row_numel = [], []
        for sh in shapes:
            sh = tuple(int(x) for x in sh)
            rows.append(sh[0] if sh else 1)
            k = 1
            for x in sh[1:]:
                k *= x
            row_numel.append(k)
        n = len(rows)
        h = ctypes.c_void_p()
        _check(lib().zero_plan_dim0((ctypes.c_int64 * n)(*rows), (ctypes.c_int64 * n)(*row_numel), n,
                                    int(world), ctypes.byref(h)))
        return cls(None, world, _handle=h)

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise ValueError("plan already freed")
        return self._h

    def free(self) -> None:
        if getattr(self, "_h", None) is not None:
            lib().zero_plan_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass

    @property
    def shard_numel(self) -> int:
        return lib().zero_plan_shard_numel(self.handle)

    @property
    def total_numel(self) -> int:
        return lib().zero_plan_total_numel(self.handle)

    @property
    def padded_numel(self) -> int:
        return lib().zero_plan_padded_numel(self.handle)

    @property
    def num_buckets(self) -> int:
        return lib().zero_plan_num_buckets(self.handle)

    @property
    def num_tensors(self) -> int:
        return lib().zero_plan_num_tensors(self.handle)

    def bucket(self, b: int) -> Tuple[int, int, int, int, int, int]:
        """(base, numel, padded, shard, first_tensor, n_tensors)"""
        o = [ctypes.c_int64() for _ in range(4)] + [ctypes.c_int32() for _ in range(2)]
        _check(lib().zero_plan_bucket(self.handle, b, *[ctypes.byref(x) for x in o]))
        return tuple(x.value for x in o)

    def tensor(self, i: int) -> Tuple[int, int]:
        """(bucket, flat offset)"""
        b, off = ctypes.c_int32(), ctypes.c_int64()
        _check(lib().zero_plan_tensor(self.handle, i, ctypes.byref(b), ctypes.byref(off)))
        return b.value, off.value

    def rank_segment(self, rank: int, b: int) -> Tuple[int, int, int]:
        """(gather_off, local_off, valid)"""
        o = [ctypes.c_int64() for _ in range(3)]
        _check(lib().zero_plan_rank_segment(self.handle, rank, b, *[ctypes.byref(x) for x in o]))
        return tuple(x.value for x in o)

    def segments(self, rank: int) -> List[Tuple[int, int, int, int]]:
        """(gather_off, local_off, seg_len, valid) per bucket."""
        out = []
        for b in range(self.num_buckets):
            go, lo, valid = self.rank_segment(rank, b)
            out.append((go, lo, self.bucket(b)[3], valid))
        return out

    def tensor_offsets(self) -> List[int]:
        return [self.tensor(i)[1] for i in range(self.num_tensors)]

    def bytes(self, stage: int) -> Tuple[float, int]:
        f, p = ctypes.c_double(), ctypes.c_int64()
        _check(lib().zero_plan_bytes(self.handle, stage, ctypes.byref(f), ctypes.byref(p)))
        return f.value, p.value

    def piece_table_bytes(self) -> int:
        """Device bytes of one rank's piece table (16 per piece)."""
        return lib().zero_plan_piece_table_bytes(self.handle)

    def attach_piece_table(self, rank: int, table: int, nbytes: int) -> None:
        """Write rank's piece table into device memory `table` and attach it
        (one launch per step for any number of pieces); table=0 detaches."""
        _check(lib().zero_plan_attach_piece_table(self.handle, int(rank), table or None, int(nbytes)))

    def workspace_bytes(self) -> int:
        return lib().zero_workspace_bytes(self.handle)

    def state_numel(self, layout: int) -> int:
        n = lib().zero_state_numel(self.handle, layout)
        if n < 0:
            raise ZeroError(ZERO_EINVAL, "unknown state layout")
        return n


# ---------------------------------------------------------------------------
# device operations
# ---------------------------------------------------------------------------

def zero_reduce_shard(plan: Plan, grad: int, grad_ld: int, grad_dtype: int, inv_scale: float,
                      g_out: int, ws: int, want_sumsq: bool, stream: int = 0,
                      grad_count: int = 0, grad_layout: int = ZERO_GRAD_SHARD, rank: int = 0,
                      ctl: int = 0) -> None:
    """grad_count: gradient buffers summed (0 = N, one per rank; 1 = a stored
    reduce-scatter output, or with grad_layout ZERO_GRAD_FULL one all-reduced
    full gradient read at `rank`'s pieces).  ctl: device address of a
    zero_step_ctl_t whose loss scale replaces inv_scale (0 = none)."""
    _check(lib().zero_reduce_shard(plan.handle, int(rank), grad, grad_ld, grad_count, grad_layout, grad_dtype,
                                   inv_scale, g_out or None, ws, 1 if want_sumsq else 0, ctl or None,
                                   stream or None))


def zero_shard_norm(plan: Plan, ws: int, other_ranks_sumsq: float, max_norm: float,
                    overflow_out: int, sumsq_out: int, clip_coef_out: int, stream: int = 0) -> None:
    _check(lib().zero_shard_norm(plan.handle, ws, other_ranks_sumsq, max_norm, overflow_out or None,
                                 sumsq_out or None, clip_coef_out or None, stream or None))


ZERO_NOALLOC_SCRATCH_BYTES = 4 * 1024 * 1024


def zero_noalloc_max_shard() -> int:
    return int(lib().zero_noalloc_max_shard())


def zero_reduce_norm_noalloc(plan: Plan, grad: int, grad_ld: int, grad_dtype: int, inv_scale: float,
                             g_out: int, other_ranks_sumsq: float, max_norm: float, overflow_out: int,
                             sumsq_out: int, clip_coef_out: int, stream: int = 0, grad_count: int = 0,
                             grad_layout: int = ZERO_GRAD_SHARD, rank: int = 0, ctl: int = 0) -> None:
    """zero_reduce_shard + zero_shard_norm with the library's fixed workspace
    (for callers that cannot allocate device memory)."""
    _check(lib().zero_reduce_norm_noalloc(plan.handle, int(rank), grad, grad_ld, grad_count, grad_layout,
                                          grad_dtype, inv_scale, g_out or None, other_ranks_sumsq, max_norm,
                                          overflow_out or None, sumsq_out or None, clip_coef_out or None,
                                          ctl or None, stream or None))


def zero_adam_step(plan: Plan, args: zero_adam_args_t, stream: int = 0) -> None:
    _check(lib().zero_adam_step(plan.handle, ctypes.byref(args), stream or None))


# ---------------------------------------------------------------------------
# loss scale and sharded checkpoints (host)
# ---------------------------------------------------------------------------

class Scaler:
    """Dynamic loss scale (zero_scaler_t): update() after every step with its
    overflow flag; inv_scale is what the step multiplies the gradient by."""

    def __init__(self, init_scale: float = 65536.0, growth_factor: float = 2.0,
                 backoff_factor: float = 0.5, growth_interval: int = 2000):
        self.s = zero_scaler_t()
        _check(lib().zero_scaler_init(ctypes.byref(self.s), init_scale, growth_factor, backoff_factor,
                                      int(growth_interval)))

    def update(self, overflow: bool) -> None:
        _check(lib().zero_scaler_update(ctypes.byref(self.s), 1 if overflow else 0))

    @property
    def scale(self) -> float:
        return self.s.scale

    @property
    def growth_tracker(self) -> int:
        return self.s.growth_tracker

    @property
    def inv_scale(self) -> float:
        return lib().zero_scaler_inv_scale(ctypes.byref(self.s))


def zero_plan_hash(plan: Plan) -> int:
    return lib().zero_plan_hash(plan.handle)


def zero_checkpoint_save(plan: Plan, rank: int, path: str, state_layout: int, master: int, m: int, v: int,
                         step: int, scaler: zero_scaler_t, stream: int = 0) -> None:
    meta = zero_ckpt_meta_t(step=int(step), scaler=scaler)
    _check(lib().zero_checkpoint_save(plan.handle, int(rank), os.fsencode(path), int(state_layout),
                                      master or None, m or None, v or None, ctypes.byref(meta),
                                      stream or None))


def zero_checkpoint_load(plan: Plan, rank: int, path: str, state_layout: int, master: int, m: int, v: int,
                         stream: int = 0) -> zero_ckpt_meta_t:
    """Returns the saved metadata (step and scaler)."""
    meta = zero_ckpt_meta_t()
    _check(lib().zero_checkpoint_load(plan.handle, int(rank), os.fsencode(path), int(state_layout),
                                      master or None, m or None, v or None, ctypes.byref(meta),
                                      stream or None))
    return meta


def zero_stream_copy(dst: int, src: int, nbytes: int, stream: int = 0) -> None:
    _check(lib().zero_stream_copy(dst, src, int(nbytes), stream or None))


def adam_args(**kw) -> zero_adam_args_t:
    """Build a zero_adam_args_t; unspecified pointers are NULL, inv_scale 1."""
    a = zero_adam_args_t()
    a.inv_scale = 1.0
    for k, v in kw.items():
        if not hasattr(a, k):
            raise TypeError(f"unknown field {k}")
        setattr(a, k, v)
    return a

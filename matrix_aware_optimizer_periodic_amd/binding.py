"""ctypes binding of the C ABI declared in include/muon.h.

Argument marshalling only: every function here forwards to the function of
the same name in ``libmuon_hip.so``; every step of the optimizer runs in the
library's HIP kernels.  A non-OK status raises ``MuonError`` carrying it.
PyTorch is used by callers for device memory and streams.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmuon_hip.so")

MUON_OK, MUON_E_ARG, MUON_E_SHAPE, MUON_E_DTYPE, MUON_E_ALIGN, MUON_E_WORKSPACE, \
    MUON_E_STATE, MUON_E_HIP = range(8)
MUON_F32, MUON_BF16 = 0, 1
MUON_KIND_MATRIX, MUON_KIND_ADAMW = 0, 1
MUON_BRANCH_ROWNORM, MUON_BRANCH_NS5, MUON_BRANCH_BLOCK_NS5 = 0, 1, 2
MUON_NS_BF16, MUON_NS_F32, MUON_NS_BF16_COMP = 0, 1, 2

EXPORTED = ("muon_config_default", "muon_state_bytes", "muon_init", "muon_step", "muon_state",
            "muon_branch", "muon_free", "muon_status_str", "muon_last_error",
            "muon_timing_enable", "muon_timing_read", "muon_sync", "muon_tall_poll_limit",
            "muon_tall_giveups", "muon_step_noalloc")

# muon_kernel_class, in enum order
KERNEL_CLASSES = ("rownorm_rows", "rownorm_cols1", "rownorm_cols2", "ns_prep", "ns_scale",
                  "ns_gram", "ns_poly", "ns_product", "ns_product_last", "adamw", "rownorm_coef",
                  "rownorm_tall", "rownorm_repair")


class MuonTensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ld", ctypes.c_int64), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class MuonConfig(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta", ctypes.c_float), ("gamma", ctypes.c_float),
                ("eps_row", ctypes.c_float), ("K", ctypes.c_int32), ("ns_iters", ctypes.c_int32),
                ("ns_a", ctypes.c_float), ("ns_b", ctypes.c_float), ("ns_c", ctypes.c_float),
                ("ns_eps", ctypes.c_float), ("ns_precision", ctypes.c_int32),
                ("rownorm_axis", ctypes.c_int32), ("bp_blocks", ctypes.c_int32),
                ("bp_period", ctypes.c_int32), ("bp_lr_ratio", ctypes.c_float),
                ("muon_wd", ctypes.c_float), ("adam_lr", ctypes.c_float),
                ("adam_b1", ctypes.c_float), ("adam_b2", ctypes.c_float),
                ("adam_eps", ctypes.c_float), ("adam_wd", ctypes.c_float),
                ("ns_workspace_max", ctypes.c_uint64), ("tall_single_pass", ctypes.c_int32),
                ("reserved0", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class MuonError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_LIB = None


def _hip_runtimes() -> set:
    """Paths of the HIP runtime libraries mapped into this process (Linux)."""
    try:
        with open("/proc/self/maps") as f:
            return {ln.split()[-1] for ln in f if "libamdhip64" in ln}
    except OSError:
        return set()


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built.

    torch is imported first on purpose: torch ships its own HIP runtime, and
    libmuon_hip.so must bind to that same runtime (they share the SONAME
    libamdhip64.so.7) so that torch's device memory and streams are used by
    one runtime.  Loading the library first would map a second HIP runtime
    into the process; that state is refused here.
    """
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m matrix_aware_optimizer_periodic_amd.build`")
        import torch  # noqa: F401  (see docstring)
        L = ctypes.CDLL(LIB_PATH)
        runtimes = _hip_runtimes()
        if len(runtimes) > 1:
            raise RuntimeError("two HIP runtimes are mapped into this process "
                               f"({sorted(runtimes)}); import torch before loading "
                               "libmuon_hip.so through any other route")
        P = ctypes.POINTER
        L.muon_config_default.argtypes = [P(MuonConfig)]
        L.muon_config_default.restype = ctypes.c_int
        L.muon_state_bytes.argtypes = [P(MuonConfig), P(MuonTensor), P(ctypes.c_int32),
                                       ctypes.c_int32, P(ctypes.c_size_t)]
        L.muon_state_bytes.restype = ctypes.c_int
        L.muon_init.argtypes = [P(ctypes.c_void_p), P(MuonConfig), P(MuonTensor), P(MuonTensor),
                                P(ctypes.c_int32), ctypes.c_int32, ctypes.c_void_p,
                                ctypes.c_size_t, ctypes.c_void_p]
        L.muon_init.restype = ctypes.c_int
        L.muon_step.argtypes = [ctypes.c_void_p, P(MuonTensor), P(MuonTensor), ctypes.c_int64]
        L.muon_step.restype = ctypes.c_int
        L.muon_state.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, P(MuonTensor)]
        L.muon_state.restype = ctypes.c_int
        L.muon_branch.argtypes = [P(MuonConfig), ctypes.c_int64]
        L.muon_branch.restype = ctypes.c_int32
        L.muon_free.argtypes = [ctypes.c_void_p]
        L.muon_free.restype = None
        L.muon_status_str.argtypes = [ctypes.c_int32]
        L.muon_status_str.restype = ctypes.c_char_p
        L.muon_last_error.argtypes = [ctypes.c_void_p]
        L.muon_last_error.restype = ctypes.c_char_p
        L.muon_timing_enable.argtypes = [ctypes.c_void_p, ctypes.c_int32]
        L.muon_timing_enable.restype = ctypes.c_int
        L.muon_timing_read.argtypes = [ctypes.c_void_p, P(ctypes.c_double), P(ctypes.c_int64)]
        L.muon_timing_read.restype = ctypes.c_int
        L.muon_sync.argtypes = [ctypes.c_void_p]
        L.muon_sync.restype = ctypes.c_int
        L.muon_tall_poll_limit.argtypes = [ctypes.c_void_p, ctypes.c_uint32]
        L.muon_tall_poll_limit.restype = ctypes.c_int
        L.muon_tall_giveups.argtypes = [ctypes.c_void_p, P(ctypes.c_uint64)]
        L.muon_tall_giveups.restype = ctypes.c_int
        L.muon_step_noalloc.argtypes = [P(MuonConfig), P(MuonTensor), P(MuonTensor),
                                        P(MuonTensor), ctypes.c_int32, ctypes.c_int64,
                                        ctypes.c_void_p]
        L.muon_step_noalloc.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _check(status: int, ctx=None) -> None:
    if status != MUON_OK:
        raise MuonError(status, muon_last_error(ctx))


def _array(cls, items):
    arr = (cls * max(1, len(items)))()
    for i, it in enumerate(items):
        arr[i] = it
    return arr


def tensor_desc(t, rows: int | None = None, cols: int | None = None) -> MuonTensor:
    """Descriptor of a contiguous torch tensor (2-D, or flattened to 1 x N)."""
    import torch
    if t.dtype == torch.float32:
        dt = MUON_F32
    elif t.dtype == torch.bfloat16:
        dt = MUON_BF16
    else:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if rows is None:
        if t.dim() == 2:
            rows, cols = t.shape
        else:
            rows, cols = 1, t.numel()
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return MuonTensor(t.data_ptr(), int(rows), int(cols), int(cols), dt, 0)


# ---------------------------------------------------------------- C ABI calls
def muon_config_default(**overrides) -> MuonConfig:
    cfg = MuonConfig()
    _check(lib().muon_config_default(ctypes.byref(cfg)))
    for k, v in overrides.items():
        if not hasattr(cfg, k):
            raise AttributeError(k)
        setattr(cfg, k, v)
    return cfg


def muon_state_bytes(cfg: MuonConfig, params, kinds) -> int:
    n = len(params)
    out = ctypes.c_size_t(0)
    _check(lib().muon_state_bytes(ctypes.byref(cfg), _array(MuonTensor, params),
                                  _array(ctypes.c_int32, kinds), n, ctypes.byref(out)))
    return out.value


def muon_init(cfg: MuonConfig, params, grads, kinds, state_ptr: int, state_bytes: int,
              stream: int = 0) -> ctypes.c_void_p:
    ctx = ctypes.c_void_p()
    _check(lib().muon_init(ctypes.byref(ctx), ctypes.byref(cfg), _array(MuonTensor, params),
                           _array(MuonTensor, grads), _array(ctypes.c_int32, kinds), len(params),
                           ctypes.c_void_p(state_ptr), state_bytes, ctypes.c_void_p(stream)))
    return ctx


def muon_step(ctx, params, grads, step: int) -> None:
    _check(lib().muon_step(ctx, _array(MuonTensor, params), _array(MuonTensor, grads), step), ctx)


def muon_state(ctx, i: int, which: int = 0) -> MuonTensor:
    view = MuonTensor()
    _check(lib().muon_state(ctx, i, which, ctypes.byref(view)), ctx)
    return view


def muon_branch(cfg: MuonConfig, step: int) -> int:
    return int(lib().muon_branch(ctypes.byref(cfg), step))


def muon_free(ctx) -> None:
    lib().muon_free(ctx)


def muon_status_str(status: int) -> str:
    return lib().muon_status_str(status).decode()


def muon_last_error(ctx=None) -> str:
    return lib().muon_last_error(ctx).decode()


def muon_timing_enable(ctx, enable: bool = True) -> None:
    _check(lib().muon_timing_enable(ctx, int(bool(enable))), ctx)


def muon_timing_read(ctx) -> dict:
    """{kernel class name: (total ms, launches)} since the last read."""
    n = len(KERNEL_CLASSES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(lib().muon_timing_read(ctx, ms, cnt), ctx)
    return {k: (ms[i], cnt[i]) for i, k in enumerate(KERNEL_CLASSES)}


def muon_sync(ctx) -> None:
    """Wait for the context's stream; raises MuonError if the wait failed."""
    _check(lib().muon_sync(ctx), ctx)


def muon_step_noalloc(cfg: MuonConfig, params, grads, moms, step: int, stream: int = 0) -> None:
    n = len(params)
    _check(lib().muon_step_noalloc(ctypes.byref(cfg), _array(MuonTensor, params),
                                   _array(MuonTensor, grads), _array(MuonTensor, moms), n, step,
                                   ctypes.c_void_p(stream)))


def muon_tall_poll_limit(ctx, polls: int) -> None:
    _check(lib().muon_tall_poll_limit(ctx, int(polls)), ctx)


def muon_tall_giveups(ctx) -> int:
    out = ctypes.c_uint64(0)
    _check(lib().muon_tall_giveups(ctx, ctypes.byref(out)), ctx)
    return out.value

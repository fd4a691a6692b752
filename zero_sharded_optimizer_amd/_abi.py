"""ctypes declarations of the C ABI in include/zero_adam.h.

Loading the library touches no GPU: libzero.so makes no HIP call until a
function that enqueues device work is called with valid arguments.
"""
import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libzero.so")

ZERO_OK = 0
ZERO_EINVAL = -1
ZERO_EUNSUPPORTED = -2
ZERO_EHIP = -3

ZERO_MODE_F64 = 0
ZERO_MODE_F32 = 1
ZERO_MODE_MIXED_BF16 = 2
ZERO_MODE_MIXED_F16 = 3

ZERO_OPT_ADAM = 0
ZERO_OPT_SGD = 1

ZERO_MAX_WORKERS = 256

STATUS_NAMES = {ZERO_OK: "ZERO_OK", ZERO_EINVAL: "ZERO_EINVAL",
                ZERO_EUNSUPPORTED: "ZERO_EUNSUPPORTED", ZERO_EHIP: "ZERO_EHIP"}


class zero_hparams(C.Structure):
    _fields_ = [
        ("n", C.c_int64),
        ("n_workers", C.c_int32),
        ("rank", C.c_int32),
        ("mode", C.c_int32),
        ("optimizer", C.c_int32),
        ("lr", C.c_double),
        ("beta1", C.c_double),
        ("beta2", C.c_double),
        ("eps", C.c_double),
        ("weight_decay", C.c_double),
        ("wd_mask", C.c_void_p),
        ("momentum", C.c_double),
        ("dampening", C.c_double),
        ("nesterov", C.c_int32),
        ("reserved", C.c_int32),
    ]


class zero_states(C.Structure):
    _fields_ = [("master", C.c_void_p), ("m", C.c_void_p), ("v", C.c_void_p)]


class zero_step_scalars(C.Structure):
    _fields_ = [("bias1", C.c_double), ("bias2", C.c_double), ("t", C.c_int64)]


class zero_mem(C.Structure):
    _fields_ = [("params", C.c_int64), ("grads", C.c_int64), ("optimizer", C.c_int64),
                ("total", C.c_int64)]


EXPORTED = ("zero_init_states", "zero_step", "zero_memory_bytes", "zero_shard_bounds",
            "zero_last_error", "zero_mean_grad_workspace_bytes", "zero_mean_grad",
            "zero_step_mean", "zero_step_clipped_workspace_bytes", "zero_step_clipped",
            "zero_step_range", "zero_step_scalars_fill", "zero_step_range_dev", "zero_min_stage",
            "zero_step_buckets", "zero_step_with_mean", "zero_mean_grad_noalloc")

_lib = None


def _torch_runtime_first():
    """Load torch (and with it the HIP runtime its wheel ships) before the
    library. libzero.so links the runtime by its soname, libamdhip64.so.7; torch
    links the file name libamdhip64.so from its own directory. Loaded in that
    order, the library binds to torch's runtime, the one that owns the tensors
    and streams it is given. Loaded the other way round, the process would hold
    two HIP runtimes, and launches with torch's streams and memory would fail."""
    try:
        import torch  # noqa: F401
    except ImportError:  # no torch: the library binds the system runtime alone
        pass


def load(path=None):
    """Load libzero.so (once). Raises if it has not been built: there is no
    fallback path."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python zero_sharded_optimizer_amd/build_lib.py`")
    _torch_runtime_first()
    lib = C.CDLL(p)
    lib.zero_init_states.argtypes = [C.POINTER(zero_hparams), C.c_void_p,
                                     C.POINTER(zero_states), C.c_void_p]
    lib.zero_init_states.restype = C.c_int
    lib.zero_step.argtypes = [C.POINTER(zero_hparams), C.c_void_p, C.POINTER(C.c_void_p),
                              C.POINTER(zero_states), C.c_int64, C.c_void_p]
    lib.zero_step.restype = C.c_int
    lib.zero_step_with_mean.argtypes = [C.POINTER(zero_hparams), C.c_void_p,
                                        C.POINTER(C.c_void_p), C.POINTER(zero_states), C.c_int64,
                                        C.c_void_p, C.c_void_p]
    lib.zero_step_with_mean.restype = C.c_int
    lib.zero_memory_bytes.argtypes = [C.c_int64, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                      C.c_int32, C.POINTER(zero_mem)]
    lib.zero_memory_bytes.restype = C.c_int
    lib.zero_shard_bounds.argtypes = [C.c_int64, C.c_int32, C.c_int32, C.POINTER(C.c_int64),
                                      C.POINTER(C.c_int64)]
    lib.zero_shard_bounds.restype = C.c_int
    lib.zero_step_range.argtypes = [C.POINTER(zero_hparams), C.c_void_p, C.POINTER(C.c_void_p),
                                    C.POINTER(zero_states), C.c_int64, C.c_int64, C.c_int64,
                                    C.c_void_p]
    lib.zero_step_range.restype = C.c_int
    lib.zero_mean_grad_workspace_bytes.argtypes = [C.POINTER(zero_hparams), C.POINTER(C.c_size_t)]
    lib.zero_mean_grad_workspace_bytes.restype = C.c_int
    lib.zero_mean_grad.argtypes = [C.POINTER(zero_hparams), C.POINTER(C.c_void_p), C.c_void_p,
                                   C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    lib.zero_mean_grad.restype = C.c_int
    lib.zero_mean_grad_noalloc.argtypes = [C.POINTER(zero_hparams), C.POINTER(C.c_void_p),
                                           C.c_void_p, C.c_void_p, C.c_void_p]
    lib.zero_mean_grad_noalloc.restype = C.c_int
    lib.zero_step_mean.argtypes = [C.POINTER(zero_hparams), C.c_void_p, C.c_void_p,
                                   C.POINTER(zero_states), C.c_int64, C.c_void_p, C.c_double,
                                   C.c_void_p]
    lib.zero_step_mean.restype = C.c_int
    lib.zero_step_clipped_workspace_bytes.argtypes = [C.POINTER(zero_hparams),
                                                      C.POINTER(C.c_size_t)]
    lib.zero_step_clipped_workspace_bytes.restype = C.c_int
    lib.zero_step_clipped.argtypes = [C.POINTER(zero_hparams), C.c_void_p, C.POINTER(C.c_void_p),
                                      C.POINTER(zero_states), C.c_int64, C.c_double, C.c_void_p,
                                      C.c_void_p, C.c_size_t, C.c_void_p]
    lib.zero_step_clipped.restype = C.c_int
    lib.zero_step_scalars_fill.argtypes = [C.POINTER(zero_hparams), C.c_int64,
                                           C.POINTER(zero_step_scalars)]
    lib.zero_step_scalars_fill.restype = C.c_int
    lib.zero_step_range_dev.argtypes = [C.POINTER(zero_hparams), C.c_void_p,
                                        C.POINTER(C.c_void_p), C.POINTER(zero_states), C.c_void_p,
                                        C.c_int64, C.c_int64, C.c_void_p]
    lib.zero_step_range_dev.restype = C.c_int
    lib.zero_step_buckets.argtypes = [C.POINTER(zero_hparams), C.c_void_p, C.POINTER(C.c_void_p),
                                      C.POINTER(zero_states), C.c_int64, C.POINTER(C.c_int64),
                                      C.c_int32, C.POINTER(C.c_void_p), C.c_void_p]
    lib.zero_step_buckets.restype = C.c_int
    lib.zero_min_stage.argtypes = [C.c_int64, C.c_int32, C.c_int32, C.c_int64, C.c_int64,
                                    C.POINTER(C.c_int32)]
    lib.zero_min_stage.restype = C.c_int
    lib.zero_last_error.argtypes = []
    lib.zero_last_error.restype = C.c_char_p
    if path is None:
        _lib = lib
    return lib

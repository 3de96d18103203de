"""ctypes declarations of the C ABI in include/lmoe.h (argument marshalling only)."""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# LMOE_LIBRARY may name another build of the same library (e.g. to compare two builds)
LIB_PATH = os.environ.get("LMOE_LIBRARY") or os.path.join(HERE, "liblmoe.so")

LMOE_F32 = 0
LMOE_BF16 = 1

STATUS = {0: "LMOE_OK", -1: "LMOE_ERR_NULL", -2: "LMOE_ERR_SHAPE", -3: "LMOE_ERR_DTYPE", -4: "LMOE_ERR_ALIGN",
          -5: "LMOE_ERR_WORKSPACE", -6: "LMOE_ERR_HIP", -7: "LMOE_ERR_VALUE", -8: "LMOE_ERR_SCRATCH"}

STATIC_SCRATCH_BYTES = 64 << 20  # LMOE_STATIC_SCRATCH_BYTES

WS_REGIONS = {"z": 0, "counts": 1, "offs": 2, "row_token": 3, "row_slot": 4, "hidden": 5, "rows": 6, "v": 7}

# every function the header declares
EXPORTS = ("lmoe_workspace_size", "lmoe_workspace_offset", "lmoe_forward", "lmoe_forward_timed", "lmoe_forward_static",
           "lmoe_backward", "lmoe_backward_workspace_size",
           "lmoe_qb_update", "lmoe_qb_workspace_size", "lmoe_qb_margin_update", "lmoe_qb_margin_workspace_size",
           "lmoe_bias_signsgd", "lmoe_strerror")

N_STAGES = 8
STAGES = ("down_proj", "router", "topk", "permute", "experts_w12", "experts_w3", "combine_norm", "up_proj")


class Dims(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int64) for f in ("T", "d", "L", "n", "k", "n_shared", "D")]


class Weights(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in ("w_down", "w_router", "router_bias", "router_logit_offset", "w1",
                                               "w2", "w3", "ws1", "ws2", "ws3", "rms_gain", "w_up")] + \
               [("beta1", ctypes.c_float), ("beta2", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("gate", ctypes.c_int32), ("norm", ctypes.c_int32)]

GRAD_FIELDS = ("dx", "dw_down", "dw_router", "dw1", "dw2", "dw3", "dws1", "dws2", "dws3", "dgamma", "dw_up")


class Grads(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in GRAD_FIELDS]


GATES = {"tanh": 0, "clip": 1}  # lmoe_gate
NORMS = {"rms": 0, "none": 1, "both": 2}   # lmoe_norm


_lib = None


def lib():
    """Load liblmoe.so; raise if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(the HIP library is the only implementation)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.lmoe_workspace_size.restype = ctypes.c_size_t
        L.lmoe_workspace_size.argtypes = [P(Dims), ctypes.c_int]
        L.lmoe_workspace_offset.restype = ctypes.c_int64
        L.lmoe_workspace_offset.argtypes = [P(Dims), ctypes.c_int, ctypes.c_int]
        L.lmoe_forward.restype = ctypes.c_int
        L.lmoe_forward.argtypes = [P(Dims), P(Weights), ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_size_t, ctypes.c_void_p]
        L.lmoe_forward_timed.restype = ctypes.c_int
        L.lmoe_forward_timed.argtypes = [P(Dims), P(Weights), ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        L.lmoe_forward_static.restype = ctypes.c_int
        L.lmoe_forward_static.argtypes = [P(Dims), P(Weights), ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.lmoe_backward_workspace_size.restype = ctypes.c_size_t
        L.lmoe_backward_workspace_size.argtypes = [P(Dims), ctypes.c_int]
        L.lmoe_backward.restype = ctypes.c_int
        L.lmoe_backward.argtypes = [P(Dims), P(Weights), ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_size_t, P(Grads), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.lmoe_qb_update.restype = ctypes.c_int
        L.lmoe_qb_update.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_int32, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.lmoe_qb_workspace_size.restype = ctypes.c_size_t
        L.lmoe_qb_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int32]
        L.lmoe_qb_margin_update.restype = ctypes.c_int
        L.lmoe_qb_margin_update.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int32, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                            ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.lmoe_qb_margin_workspace_size.restype = ctypes.c_size_t
        L.lmoe_qb_margin_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]
        L.lmoe_bias_signsgd.restype = ctypes.c_int
        L.lmoe_bias_signsgd.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
        L.lmoe_strerror.restype = ctypes.c_char_p
        L.lmoe_strerror.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def strerror(rc):
    return lib().lmoe_strerror(rc).decode()


def check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed: {STATUS.get(rc, rc)} ({strerror(rc)})")

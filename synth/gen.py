"""Host / device fillers for the counter-based generator of ``synth_core.h``."""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsynth_host.so")
DEV_LIB = os.path.join(_HERE, "libsynth_dev.so")

# tensor ids of the generator streams
TID = {
    "x": 0, "w_down": 1, "w_router": 2, "w1": 3, "w2": 4, "w3": 5,
    "ws1": 6, "ws2": 7, "ws3": 8, "w_up": 9, "bias": 10, "scores": 13, "dy": 14,
}

_host = None
_dev = None


def load_host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_LIB)
        for name, ptr_t in (("synth_fill_f32", ctypes.c_void_p), ("synth_fill_bf16", ctypes.c_void_p)):
            fn = getattr(lib, name)
            fn.restype = None
            fn.argtypes = [ptr_t, ctypes.c_size_t, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                           ctypes.c_float, ctypes.c_void_p, ctypes.c_uint64]
        lib.synth_splitmix_output.restype = ctypes.c_uint64
        lib.synth_splitmix_output.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        _host = lib
    return _host


def _load_dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"{DEV_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(DEV_LIB)
        lib.synth_fill_device.restype = ctypes.c_int
        lib.synth_fill_device.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_uint64,
                                          ctypes.c_uint64, ctypes.c_uint64, ctypes.c_float,
                                          ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
        _dev = lib
    return _dev


def scale_for(std):
    """fp32 multiplier that gives standard deviation ``std``."""
    return np.float32(float(std) / 65536.0)


def splitmix_output(state, j):
    return int(load_host_lib().synth_splitmix_output(state, j))


def host_fill(n, seed, tid, start=0, std=1.0, bf16=False, row_mult=None, row_len=0):
    """Elements start..start+n-1 of stream (seed, tid); float32 array or bf16 bit patterns (uint16)."""
    lib = load_host_lib()
    out = np.empty(int(n), dtype=np.uint16 if bf16 else np.float32)
    rm = None
    if row_mult is not None:
        rm = np.ascontiguousarray(row_mult, dtype=np.float32)
        assert row_len > 0
    fn = lib.synth_fill_bf16 if bf16 else lib.synth_fill_f32
    fn(out.ctypes.data, int(n), int(seed), int(tid), int(start), float(scale_for(std)),
       rm.ctypes.data if rm is not None else None, int(row_len))
    return out


def bf16_bits_to_f64(u16):
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(a):
    """Bit patterns of values that are already exactly bf16 (no rounding performed)."""
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    bits = f.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0), "values are not bf16-representable"
    return (bits >> 16).astype(np.uint16)


def host_fill_values(shape, seed, tid, start=0, std=1.0, dtype="bf16", row_mult=None, row_len=0):
    """float64 array of the generated values, already in the work dtype's value set."""
    n = int(np.prod(shape))
    if dtype == "bf16":
        return bf16_bits_to_f64(host_fill(n, seed, tid, start, std, True, row_mult, row_len)).reshape(shape)
    return host_fill(n, seed, tid, start, std, False, row_mult, row_len).astype(np.float64).reshape(shape)


# ----------------------------------------------------------------------------
# A slow pure-numpy restatement of the same definition, used only to check the
# C filler (small n).

_M64 = (1 << 64) - 1


def _mix64_np(z):
    z = z.astype(np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def numpy_fill_f32(n, seed, tid, start=0, std=1.0):
    g = np.uint64(0x9E3779B97F4A7C15)
    with np.errstate(over="ignore"):
        key = _mix64_np(_mix64_np(np.array([seed], dtype=np.uint64) + g) + np.uint64(tid))[0]
        idx = np.arange(start, start + n, dtype=np.uint64)
        s = np.zeros(n, dtype=np.int64)
        for d in range(3):
            r = _mix64_np(key + (np.uint64(3) * idx + np.uint64(d + 1)) * g)
            for sh in (0, 16, 32, 48):
                s += ((r >> np.uint64(sh)) & np.uint64(0xFFFF)).astype(np.int64)
    c = (s - 393210).astype(np.float32)
    return c * scale_for(std)


def device_fill(t, seed, tid, start=0, std=1.0, row_mult=None, row_len=0, stream=None):
    """Fill a contiguous CUDA tensor (float32 or bfloat16) in place."""
    import torch
    assert t.is_cuda and t.is_contiguous()
    if t.dtype == torch.bfloat16:
        bf = 1
    elif t.dtype == torch.float32:
        bf = 0
    else:
        raise TypeError(t.dtype)
    rm = None
    if row_mult is not None:
        rm = torch.as_tensor(np.ascontiguousarray(row_mult, dtype=np.float32)).to(t.device)
    if stream is None:
        stream = torch.cuda.current_stream(t.device).cuda_stream
    rc = _load_dev_lib().synth_fill_device(t.data_ptr(), t.numel(), bf, int(seed), int(tid), int(start),
                                           float(scale_for(std)), rm.data_ptr() if rm is not None else None,
                                           int(row_len), stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill_device failed ({rc})")
    if rm is not None:
        torch.cuda.current_stream(t.device).synchronize()
    return t

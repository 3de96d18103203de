"""Stable LatentMoE forward + Quantile Balancing on AMD MI355X.

Thin Python binding over the C ABI of ``liblmoe.so`` (include/lmoe.h): it
only reads shapes and device pointers off torch tensors and passes them with
the current HIP stream.  Every step of the layer runs in the library's HIP
kernels; there is no other implementation behind these functions.
"""
import ctypes

import torch

from ._abi import (Dims, Weights, Grads, GRAD_FIELDS, GATES, NORMS, LMOE_BF16, LMOE_F32, WS_REGIONS, EXPORTS, N_STAGES, STAGES, lib,  # noqa: F401
                   STATIC_SCRATCH_BYTES,
                   check, strerror)

__all__ = ["dims_of", "workspace_size", "workspace_view", "forward", "forward_static", "backward", "backward_workspace_size", "qb_update", "qb_workspace_size",
           "qb_margin_update", "qb_margin_workspace_size", "bias_signsgd",
           "strerror", "make_workspace"]


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return LMOE_BF16
    if dt == torch.float32:
        return LMOE_F32
    raise TypeError(f"unsupported work dtype {dt}")


def dims_of(x, weights, k):
    T, d = x.shape
    n, D, L = weights["w1"].shape
    ws1 = weights.get("ws1")
    return Dims(T, d, weights["w_down"].shape[0], n, int(k), 0 if ws1 is None else ws1.shape[0], D)


def workspace_size(dims, dtype):
    return int(lib().lmoe_workspace_size(dims, _dtype_code(dtype) if isinstance(dtype, torch.dtype) else dtype))


def make_workspace(dims, dtype, device="cuda"):
    return torch.empty(max(workspace_size(dims, dtype), 256), dtype=torch.uint8, device=device)


def workspace_view(workspace, dims, dtype, region, capped=True):
    """A typed view of one inspectable workspace region (see lmoe_ws_region).

    ``capped``: both expert caps finite (the staged rows are fp16 for bf16 work
    dtype only then, fp32 otherwise)."""
    code = _dtype_code(dtype)
    off = int(lib().lmoe_workspace_offset(dims, code, WS_REGIONS[region]))
    if off < 0:
        raise ValueError(region)
    T, L, n, k, D, ns = dims.T, dims.L, dims.n, dims.k, dims.D, dims.n_shared
    R = T * (k + ns)  # expert rows: dispatched, then each shared expert's T
    stage_dt = torch.float16 if (dtype == torch.bfloat16 and capped) else torch.float32
    shapes = {"z": ((T, L), dtype), "counts": ((n,), torch.int32), "offs": ((n + 1,), torch.int32),
              "row_token": ((R,), torch.int32), "row_slot": ((T * k,), torch.int32),
              "hidden": ((R, D), dtype), "rows": ((R, L), stage_dt), "v": ((T, L), dtype)}
    shape, dt = shapes[region]
    nbytes = torch.tensor([], dtype=dt).element_size()
    cnt = 1
    for s in shape:
        cnt *= s
    return workspace[off:off + cnt * nbytes].view(dt).view(*shape)


def _weights_struct(w, beta1, beta2, eps, gate="tanh", norm="rms"):
    return Weights(_ptr(w["w_down"]), _ptr(w["w_router"]), _ptr(w["router_bias"]),
                   _ptr(w.get("router_logit_offset")), _ptr(w["w1"]), _ptr(w["w2"]), _ptr(w["w3"]),
                   _ptr(w.get("ws1")), _ptr(w.get("ws2")), _ptr(w.get("ws3")), _ptr(w["rms_gain"]),
                   _ptr(w["w_up"]), float(beta1), float(beta2), float(eps), GATES[gate],
                   NORMS[norm])


def forward(x, weights, k, y=None, topk_idx=None, topk_w=None, scores=None, workspace=None, beta1=4.0,
            beta2=25.0, eps=1e-6, stream=None, stage_events=None, gate="tanh", norm="rms"):
    """y = LatentMoE(x) via lmoe_forward on the current stream; returns y.

    ``gate`` is "tanh" (SiTU-GLU) or "clip" (both caps a hard clip: the ablation);
    ``norm`` is "rms" (the layer's one RMSNorm), "none" (v = u) or "both" (an
    extra RMSNorm on z after the down-projection); the last two are ablations.

    ``weights`` holds device tensors named as in include/lmoe.h (w_down, w_router,
    router_bias, router_logit_offset, w1, w2, w3, ws1, ws2, ws3, rms_gain, w_up).
    """
    dims = dims_of(x, weights, k)
    if y is None:
        y = torch.empty_like(x)
    if workspace is None:
        workspace = make_workspace(dims, x.dtype, x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    W = _weights_struct(weights, beta1, beta2, eps, gate, norm)
    if stage_events is None:
        rc = lib().lmoe_forward(dims, W, _dtype_code(x.dtype), _ptr(x), _ptr(y), _ptr(topk_idx), _ptr(topk_w),
                                _ptr(scores), _ptr(workspace), workspace.numel(), stream)
        check(rc, "lmoe_forward")
    else:
        # stage_events: N_STAGES + 1 entries, each a torch.cuda.Event(enable_timing=True) or None
        # (that stage boundary is not recorded); their hipEvent_t handles
        for ev in stage_events:
            if ev is not None:
                ev.record()  # materialise the underlying hipEvent_t on this device
        handles = (ctypes.c_void_p * len(stage_events))(*[None if ev is None else ev.cuda_event
                                                           for ev in stage_events])
        rc = lib().lmoe_forward_timed(dims, W, _dtype_code(x.dtype), _ptr(x), _ptr(y), _ptr(topk_idx),
                                      _ptr(topk_w), _ptr(scores), _ptr(workspace), workspace.numel(), handles,
                                      len(stage_events), stream)
        check(rc, "lmoe_forward_timed")
    return y


def forward_static(x, weights, k, y=None, topk_idx=None, topk_w=None, scores=None, beta1=4.0, beta2=25.0,
                   eps=1e-6, stream=None, gate="tanh", norm="rms"):
    """y = LatentMoE(x) via lmoe_forward_static: no workspace argument, nothing allocated by
    the library (it uses its own static device scratch); y must be given to allocate nothing here
    either.  Calls on one device share that scratch and must not overlap."""
    dims = dims_of(x, weights, k)
    if y is None:
        y = torch.empty_like(x)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    W = _weights_struct(weights, beta1, beta2, eps, gate, norm)
    rc = lib().lmoe_forward_static(dims, W, _dtype_code(x.dtype), _ptr(x), _ptr(y), _ptr(topk_idx), _ptr(topk_w),
                                   _ptr(scores), stream)
    check(rc, "lmoe_forward_static")
    return y


def backward_workspace_size(dims, dtype):
    return int(lib().lmoe_backward_workspace_size(dims, _dtype_code(dtype) if isinstance(dtype, torch.dtype) else dtype))


def backward(x, dy, weights, k, topk_idx, topk_w, scores, fwd_workspace, grads=None, workspace=None, beta1=4.0,
             beta2=25.0, eps=1e-6, stream=None, gate="tanh", norm="rms"):
    """Gradients of the layer for dy via lmoe_backward, after a forward on the same stream that
    returned topk_idx, topk_w and scores and used fwd_workspace (untouched since).  Returns a dict
    of gradient tensors (allocated here unless given): dx and one per weight (dw_down,
    dw_router, dw1, dw2, dw3, dws1, dws2, dws3 when there are shared experts, dgamma, dw_up)."""
    dims = dims_of(x, weights, k)
    if grads is None:
        like = {"dx": x, "dw_down": weights["w_down"], "dw_router": weights["w_router"], "dw1": weights["w1"],
                "dw2": weights["w2"], "dw3": weights["w3"], "dws1": weights.get("ws1"),
                "dws2": weights.get("ws2"), "dws3": weights.get("ws3"), "dgamma": weights["rms_gain"],
                "dw_up": weights["w_up"]}
        grads = {kk: (None if t is None else torch.empty_like(t)) for kk, t in like.items()}
    if workspace is None:
        workspace = torch.empty(max(backward_workspace_size(dims, x.dtype), 256), dtype=torch.uint8, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    W = _weights_struct(weights, beta1, beta2, eps, gate, norm)
    G = Grads(*[_ptr(grads.get(f)) for f in GRAD_FIELDS])
    rc = lib().lmoe_backward(dims, W, _dtype_code(x.dtype), _ptr(x), _ptr(dy), _ptr(topk_idx), _ptr(topk_w),
                             _ptr(scores), _ptr(fwd_workspace), fwd_workspace.numel(), G, _ptr(workspace),
                             workspace.numel(), stream)
    check(rc, "lmoe_backward")
    return grads


def qb_workspace_size(n, nbins):
    return int(lib().lmoe_qb_workspace_size(int(n), int(nbins)))


def qb_update(scores, k, hist, bias=None, accumulate=False, solve=True, workspace=None, stream=None):
    """Quantile Balancing: update the per-expert histogram and (optionally) solve the bias in place."""
    T, n = scores.shape
    nbins = hist.shape[1]
    if workspace is None and (solve or T > 0):
        workspace = torch.empty(qb_workspace_size(n, nbins), dtype=torch.uint8, device=hist.device)
    if stream is None:
        stream = torch.cuda.current_stream(hist.device).cuda_stream
    rc = lib().lmoe_qb_update(_ptr(scores), T, n, int(k), int(nbins), _ptr(hist), int(bool(accumulate)),
                              _ptr(bias), int(bool(solve)), _ptr(workspace),
                              0 if workspace is None else workspace.numel(), stream)
    check(rc, "lmoe_qb_update")
    return hist, bias


def qb_margin_workspace_size(T, n, nbins):
    return int(lib().lmoe_qb_margin_workspace_size(int(T), int(n), int(nbins)))


def qb_margin_update(scores, k, hist, bias, accumulate=False, solve=True, workspace=None, stream=None):
    """Margin form of Quantile Balancing: histogram each (token, expert) margin against the
    token's top-k threshold under `bias`, then (optionally) move `bias` in place."""
    T, n = scores.shape
    nbins = hist.shape[1]
    if workspace is None and T > 0:
        workspace = torch.empty(qb_margin_workspace_size(T, n, nbins), dtype=torch.uint8, device=hist.device)
    if stream is None:
        stream = torch.cuda.current_stream(hist.device).cuda_stream
    rc = lib().lmoe_qb_margin_update(_ptr(scores), T, n, int(k), int(nbins), _ptr(hist), int(bool(accumulate)),
                                     _ptr(bias), int(bool(solve)), _ptr(workspace),
                                     0 if workspace is None else workspace.numel(), stream)
    check(rc, "lmoe_qb_margin_update")
    return hist, bias


def bias_signsgd(topk_idx, n, step, bias, stream=None):
    """K2-style fixed-step bias update from the top-k lists [T, k] (in place on `bias`)."""
    T, k = topk_idx.shape
    if stream is None:
        stream = torch.cuda.current_stream(bias.device).cuda_stream
    rc = lib().lmoe_bias_signsgd(_ptr(topk_idx) if T > 0 else None, T, int(n), int(k), float(step), _ptr(bias),
                                 stream)
    check(rc, "lmoe_bias_signsgd")
    return bias

"""lmoe_forward_static, the entry point that allocates nothing (its workspace is
the library's static device scratch), against lmoe_forward with a caller's
workspace: the same kernels, so every output is bit-identical.  Two calls in a
row on each shape, the second with fewer tokens, so the second runs on scratch
that still holds the first call's contents."""
import pytest
import torch

import sparse_moe_layer_down_amd as lmoe
import synth

pytestmark = pytest.mark.gpu


def _both(cfg, w, x):
    dev = x.device
    T, k, n = x.shape[0], cfg.k, cfg.n
    outs = []
    for static in (False, True):
        idx = torch.full((T, k), -1, dtype=torch.int32, device=dev)
        g = torch.zeros((T, k), dtype=torch.float32, device=dev)
        s = torch.zeros((T, n), dtype=torch.float32, device=dev)
        y = torch.zeros_like(x)
        if static:
            lmoe.forward_static(x, w, k, y=y, topk_idx=idx, topk_w=g, scores=s, beta1=cfg.beta1, beta2=cfg.beta2)
        else:
            lmoe.forward(x, w, k, y=y, topk_idx=idx, topk_w=g, scores=s, beta1=cfg.beta1, beta2=cfg.beta2)
        outs.append((y, idx, g, s))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("name,t1,t2", [("C3", 64, 7), ("C1", 512, 77), ("C0", 64, 5)])
def test_static_forward_matches_forward_twice(name, t1, t2):
    cfg = synth.get_config(name)
    dev = torch.device("cuda:0")
    w = synth.device_params(cfg, device=dev, with_x=False)
    for T in (t1, t2):
        c = cfg.with_(T=T)
        assert lmoe.workspace_size(lmoe.dims_of(torch.empty(T, c.d), w, c.k), 1 if c.dtype == "bf16" else 0) \
            <= lmoe.STATIC_SCRATCH_BYTES
        x = synth.params.device_x(c, dev)
        _both(c, w, x)
    del w
    torch.cuda.empty_cache()


def test_static_forward_rejects_a_call_beyond_its_scratch():
    """A call whose workspace would exceed the scratch fails before anything is
    launched (the output stays as it was)."""
    cfg = synth.get_config("C1")
    dev = torch.device("cuda:0")
    w = synth.device_params(cfg, device=dev)
    x = w.pop("x")
    y = torch.zeros_like(x)
    with pytest.raises(RuntimeError, match="LMOE_ERR_SCRATCH"):
        lmoe.forward_static(x, w, cfg.k, y=y)
    torch.cuda.synchronize()
    assert not y.any()

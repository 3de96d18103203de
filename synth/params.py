"""Weights and tokens of a workload, on the host (float64 values, lazily per
expert) and in device memory (torch tensors filled in place)."""
import math

import numpy as np

from .gen import TID, host_fill, bf16_bits_to_f64, device_fill


def outlier_rows(cfg):
    """Token rows scaled by cfg.outlier_mult (round(frac*T) rows, seeded choice)."""
    cnt = int(round(cfg.outlier_frac * cfg.T))
    if cnt == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(np.random.default_rng([cfg.x_seed, 11]).choice(cfg.T, cnt, replace=False))


def zipf_logit_offset(cfg):
    """Per-expert additive router-logit skew alpha * r_e^-s, r = 1 + seeded permutation; None if off."""
    if cfg.zipf_alpha == 0.0:
        return None
    r = 1 + np.random.default_rng([cfg.x_seed, 12]).permutation(cfg.n)
    return (cfg.zipf_alpha * r.astype(np.float64) ** (-cfg.zipf_s)).astype(np.float32)


def _row_mult(cfg):
    rows = outlier_rows(cfg)
    if rows.size == 0:
        return None
    m = np.ones(cfg.T, dtype=np.float32)
    m[rows] = np.float32(cfg.outlier_mult)
    return m


def _x_tid(step):
    return TID["x"] if step is None else 100 + int(step)


class HostParams:
    """Host-side view of a workload's inputs as float64 arrays of work-dtype values.

    Expert weights are generated on demand; ``cache=True`` keeps the compact
    (bf16 bit / fp32) form of what was generated so later calls only convert.
    ``cache`` may also be a dict, shared by workloads with the same weights
    (same w_seed, shapes and dtype).
    """

    def __init__(self, cfg, cache=False):
        self.cfg = cfg
        self.bf16 = cfg.dtype == "bf16"
        self._cache = cache if isinstance(cache, dict) else ({} if cache else None)

    def _gen(self, name, tid, count, start, std):
        key = (name, start, count)
        if self._cache is not None and key in self._cache:
            raw = self._cache[key]
        else:
            raw = host_fill(count, self.cfg.w_seed, tid, start, std, self.bf16)
            if self._cache is not None:
                self._cache[key] = raw
        return bf16_bits_to_f64(raw) if self.bf16 else raw.astype(np.float64)

    # dense weights, PyTorch [out, in] layout
    def w_down(self):
        c = self.cfg
        return self._gen("w_down", TID["w_down"], c.L * c.d, 0, math.sqrt(1.0 / c.d)).reshape(c.L, c.d)

    def w_router(self):
        c = self.cfg
        return self._gen("w_router", TID["w_router"], c.n * c.L, 0, math.sqrt(1.0 / c.L)).reshape(c.n, c.L)

    def w_up(self):
        c = self.cfg
        return self._gen("w_up", TID["w_up"], c.d * c.L, 0, math.sqrt(1.0 / c.L)).reshape(c.d, c.L)

    def w1(self, e):
        c = self.cfg
        return self._gen("w1", TID["w1"], c.D * c.L, e * c.D * c.L, math.sqrt(1.0 / c.L)).reshape(c.D, c.L)

    def w2(self, e):
        c = self.cfg
        return self._gen("w2", TID["w2"], c.D * c.L, e * c.D * c.L, math.sqrt(1.0 / c.L)).reshape(c.D, c.L)

    def w3(self, e):
        c = self.cfg
        return self._gen("w3", TID["w3"], c.L * c.D, e * c.L * c.D, math.sqrt(1.0 / c.D)).reshape(c.L, c.D)

    def ws1(self, j):
        c = self.cfg
        return self._gen("ws1", TID["ws1"], c.D * c.L, j * c.D * c.L, math.sqrt(1.0 / c.L)).reshape(c.D, c.L)

    def ws2(self, j):
        c = self.cfg
        return self._gen("ws2", TID["ws2"], c.D * c.L, j * c.D * c.L, math.sqrt(1.0 / c.L)).reshape(c.D, c.L)

    def ws3(self, j):
        c = self.cfg
        return self._gen("ws3", TID["ws3"], c.L * c.D, j * c.L * c.D, math.sqrt(1.0 / c.D)).reshape(c.L, c.D)

    def bias(self):
        c = self.cfg
        if c.bias_std == 0.0:
            return np.zeros(c.n, dtype=np.float64)
        return host_fill(c.n, c.w_seed, TID["bias"], 0, c.bias_std, False).astype(np.float64)

    def logit_offset(self):
        o = zipf_logit_offset(self.cfg)
        return None if o is None else o.astype(np.float64)

    def gamma(self):
        return np.ones(self.cfg.L, dtype=np.float64)

    def x_rows(self, rows, step=None):
        """Token rows (float64 [len(rows), d]); the outlier multiplier applies to C2-style configs."""
        c = self.cfg
        rows = np.asarray(rows, dtype=np.int64)
        mult = None
        rm = _row_mult(c) if step is None else None
        out = np.empty((rows.size, c.d), dtype=np.float64)
        for i, r in enumerate(rows):
            if rm is not None:
                mult = rm[r:r + 1]
            raw = host_fill(c.d, c.x_seed, _x_tid(step), int(r) * c.d, 1.0, self.bf16, mult, c.d if mult is not None else 0)
            out[i] = bf16_bits_to_f64(raw) if self.bf16 else raw
        return out

    def x(self, step=None):
        c = self.cfg
        rm = _row_mult(c) if step is None else None
        raw = host_fill(c.T * c.d, c.x_seed, _x_tid(step), 0, 1.0, self.bf16, rm, c.d if rm is not None else 0)
        v = bf16_bits_to_f64(raw) if self.bf16 else raw.astype(np.float64)
        return v.reshape(c.T, c.d)


def device_params(cfg, device="cuda", step=None, with_x=True):
    """Allocate and fill every input of the layer on ``device``; returns a dict of torch tensors."""
    import torch
    c = cfg
    wdt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
    g = {}

    def mk(name, shape, tid, std):
        t = torch.empty(shape, dtype=wdt, device=device)
        device_fill(t, c.w_seed, tid, 0, std)
        g[name] = t

    mk("w_down", (c.L, c.d), TID["w_down"], math.sqrt(1.0 / c.d))
    mk("w_router", (c.n, c.L), TID["w_router"], math.sqrt(1.0 / c.L))
    mk("w1", (c.n, c.D, c.L), TID["w1"], math.sqrt(1.0 / c.L))
    mk("w2", (c.n, c.D, c.L), TID["w2"], math.sqrt(1.0 / c.L))
    mk("w3", (c.n, c.L, c.D), TID["w3"], math.sqrt(1.0 / c.D))
    if c.n_shared > 0:
        mk("ws1", (c.n_shared, c.D, c.L), TID["ws1"], math.sqrt(1.0 / c.L))
        mk("ws2", (c.n_shared, c.D, c.L), TID["ws2"], math.sqrt(1.0 / c.L))
        mk("ws3", (c.n_shared, c.L, c.D), TID["ws3"], math.sqrt(1.0 / c.D))
    mk("w_up", (c.d, c.L), TID["w_up"], math.sqrt(1.0 / c.L))
    g["rms_gain"] = torch.ones(c.L, dtype=wdt, device=device)
    bias = torch.zeros(c.n, dtype=torch.float32, device=device)
    if c.bias_std != 0.0:
        device_fill(bias, c.w_seed, TID["bias"], 0, c.bias_std)
    g["router_bias"] = bias
    o = zipf_logit_offset(c)
    g["router_logit_offset"] = None if o is None else torch.as_tensor(o).to(device)
    if with_x:
        g["x"] = device_x(c, device, step)
    return g


def device_x(cfg, device="cuda", step=None):
    import torch
    c = cfg
    wdt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
    x = torch.empty((c.T, c.d), dtype=wdt, device=device)
    rm = _row_mult(c) if step is None else None
    device_fill(x, c.x_seed, _x_tid(step), 0, 1.0, rm, c.d if rm is not None else 0)
    return x

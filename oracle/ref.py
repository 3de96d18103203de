"""Plain CPU oracle of the Stable LatentMoE forward pass and of Quantile Balancing.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module;
only the tests, the smoke check and the CPU-baseline leg of the benchmark call
it.  It shares no code with the HIP library.

Everything is computed in float64 with NumPy.  The only rounding applied is to
the work dtype (bf16 with round-to-nearest-even, or fp32) at the points where
the layer stores a tensor in that dtype: the latent z, the gated hidden a, the
normalised latent v and the output y.  Scores used for histogram binning are
taken in fp32 because the binning rule is defined on fp32 scores.

Sources (the three web pages on the Kimi K3 architecture):
  [DD]  "Kimi K3 Architecture Deep Dive" (jianyuh.github.io):
        §1 SiTU-GLU, §2 Stable LatentMoE, §3 Quantile Balancing.
  [IK]  "Inside K3: How Stable Latent MoE and MLA Attention Are Designed"
        (besthub.dev): sections "SiTU-GLU", "RMSNorm insertion",
        "Quantile Balancing (QB)".
  [RB]  LeiPhone report on Su Jianlin's K3 notes (robotbelt.com):
        "LatentMoE: paying for a bigger pool", "Keeping the numbers in range".

Readings of points the pages leave open are marked READING; each is also
listed in the design notes.  Parity pins: every function here is pinned by
the CPU tests (closed forms, library special cases, brute force, invariants);
the full forward has no printed numeric example on the pages, so its
end-to-end values are pinned only through those properties and special cases.
"""
import numpy as np

# ---------------------------------------------------------------------------
# rounding to the work dtype


def round_bf16(a):
    """Round float64 values to the nearest bf16 value (ties to even), returned as float64.

    Rounds the float64 value directly (no double rounding through fp32).
    """
    a = np.asarray(a, dtype=np.float64)
    out = np.empty_like(a)
    bits = a.view(np.uint64)
    mag = np.abs(a)
    finite = np.isfinite(a)
    normal = finite & (mag >= 2.0 ** -126)
    # normal range: keep 7 explicit mantissa bits of the 52 -> drop 45 bits, ties to even
    b = bits[normal]
    lsb = (b >> np.uint64(45)) & np.uint64(1)
    b = (b + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    r = b.view(np.float64)
    # beyond the largest finite bf16 (0x7F7F -> 3.3895e38) rounding overflows to inf
    big = np.abs(r) > 3.3895313892515355e38
    r = np.where(big, np.copysign(np.inf, r), r)
    out[normal] = r
    # bf16 subnormals: spacing 2^-133, round half to even
    sub = finite & ~normal
    q = 2.0 ** -133
    out[sub] = np.round(a[sub] / q) * q
    out[~finite] = a[~finite]
    return out


def round_to(a, dtype):
    """Store-rounding to the work dtype: 'bf16', 'f32' or 'f64' (none)."""
    if dtype == "bf16":
        return round_bf16(a)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(a, dtype=np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# SiTU-GLU  ([DD] §1 SiTU-GLU, softcap and SiTU equations and the SiTU-GLU
# equation with beta1 = 4, beta2 = 25; [IK] "SiTU-GLU")


def sigmoid(x):
    """Logistic function 1 / (1 + e^-x)."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=np.float64)))


def softcap(x, beta):
    """softcap(x; beta) = beta * tanh(x / beta)  ([DD] §1).

    READING: beta = +inf is the limit of that expression, the identity (the
    uncapped gate; with both caps at +inf SiTU-GLU is SwiGLU).
    """
    x = np.asarray(x, dtype=np.float64)
    if beta == np.inf:
        return x.copy()
    return beta * np.tanh(x / beta)


def hard_clip(x, beta):
    """clamp(x; beta) = min(max(x, -beta), beta): the hard clip that the tanh
    softcap replaces at the same ceiling ([DD] §1; [IK] section SiTU-GLU).

    READING: the hard-clip ablation puts this in place of softcap in both
    branches, with the same beta1 and beta2.
    """
    return np.clip(np.asarray(x, dtype=np.float64), -beta, beta)


def cap(x, beta, gate="tanh"):
    """The branch cap: softcap for gate "tanh" (the pages' choice), hard_clip for "clip"."""
    if gate == "tanh":
        return softcap(x, beta)
    if gate == "clip":
        return hard_clip(x, beta)
    raise ValueError(f"unknown gate {gate!r}")


def situ(x, beta, gate="tanh"):
    """SiTU(x; beta) = softcap(x; beta) * sigmoid(x)  ([DD] §1)."""
    return cap(x, beta, gate) * sigmoid(x)


def situ_glu_hidden(p1, p2, beta1, beta2, gate="tanh"):
    """Gated hidden of SiTU-GLU: SiTU(W1 x; beta1) (.) softcap(W2 x; beta2)  ([DD] §1).

    READING: W1 is the gate branch (SiTU), W2 the linear branch (softcap), as
    the pages state; the W3 product is applied by the caller.
    """
    return situ(p1, beta1, gate) * cap(p2, beta2, gate)


def expert_hidden(zr, w1, w2, beta1, beta2, dtype, gate="tanh"):
    """a = rnd(SiTU(zr W1^T; b1) * softcap(zr W2^T; b2)) for the rows routed to one expert."""
    p1 = zr @ w1.T
    p2 = zr @ w2.T
    return round_to(situ_glu_hidden(p1, p2, beta1, beta2, gate), dtype)


# ---------------------------------------------------------------------------
# router  ([DD] §2 LatentMoE structure: route after the d -> d/2 projection;
# [DD] §3 and [RB] "Keeping the numbers in range": loss-free selection bias)


def router_scores(z, w_router, logit_offset=None):
    """s = sigmoid(z W_r^T + o).

    READING: scores are sigmoid of the router logits (the [0,1] map of QB is
    then the identity); o is an optional per-expert logit offset used only to
    make routing skewed in synthetic workloads.
    """
    logits = z @ w_router.T
    if logit_offset is not None:
        logits = logits + np.asarray(logit_offset, dtype=np.float64)[None, :]
    return sigmoid(logits)


def biased_topk(s, bias, k):
    """Top-k experts per token by the biased score s + b; ties go to the lower expert index.

    Returns (idx [T,k] ordered by decreasing biased score, then index; gap [T]
    = k-th minus (k+1)-th biased score, +inf when k == n).
    READING: the bias acts on selection only ([RB]: balancing steers selection
    through a bias rather than a loss).
    """
    s = np.asarray(s, dtype=np.float64)
    sel = s + np.asarray(bias, dtype=np.float64)[None, :]
    order = np.argsort(-sel, axis=1, kind="stable")
    idx = order[:, :k]
    T, n = sel.shape
    if k < n:
        srt = np.take_along_axis(sel, order[:, :k + 1], axis=1)
        gap = srt[:, k - 1] - srt[:, k]
    else:
        gap = np.full(T, np.inf)
    return idx.astype(np.int64), gap


def routing_weights(s, idx):
    """g_ie = s_ie / sum_{e' in K_i} s_ie' on the unbiased scores.

    READING: renormalised sigmoid scores over the chosen k ([RB]: the router
    assigns per-expert weights to the chosen experts' outputs); no extra
    routed scale ([DD] §2 effect 1: no hand-tuned scaling factor).
    """
    sk = np.take_along_axis(np.asarray(s, dtype=np.float64), idx, axis=1)
    return sk / sk.sum(axis=1, keepdims=True)


def dispatch(idx, n):
    """Token permutation to experts: rows ordered by (expert, token).

    Returns counts [n], offs [n+1] (exclusive prefix sum), row_token [T*k],
    row_slot [T*k].  Each token lists distinct experts, so within one expert
    the rows are in increasing token order.
    """
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    flat = idx.reshape(-1)
    counts = np.bincount(flat, minlength=n).astype(np.int64)
    offs = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(counts, out=offs[1:])
    order = np.argsort(flat, kind="stable")
    return counts, offs, order // k, order % k


# ---------------------------------------------------------------------------
# RMSNorm  ([DD] §2 "one RMS Norm before up-projection"; [IK] "RMSNorm
# insertion"; [RB]: after aggregation, before projecting back up)


def rms_norm(u, gamma, eps):
    """v = gamma * u / sqrt(mean(u^2) + eps) over the latent dimension."""
    u = np.asarray(u, dtype=np.float64)
    ms = np.mean(u * u, axis=-1, keepdims=True)
    return np.asarray(gamma, dtype=np.float64)[None, :] * u / np.sqrt(ms + eps)


# ---------------------------------------------------------------------------
# the layer


class ArrayParams:
    """Adapter giving plain arrays the accessor interface the forward uses."""

    def __init__(self, w_down, w_router, w1, w2, w3, w_up, ws1=None, ws2=None, ws3=None,
                 bias=None, logit_offset=None, gamma=None):
        self._d = dict(w_down=w_down, w_router=w_router, w1=w1, w2=w2, w3=w3, w_up=w_up,
                       ws1=ws1, ws2=ws2, ws3=ws3)
        self._bias = bias
        self._o = logit_offset
        self._gamma = gamma

    def w_down(self):
        return np.asarray(self._d["w_down"], dtype=np.float64)

    def w_router(self):
        return np.asarray(self._d["w_router"], dtype=np.float64)

    def w_up(self):
        return np.asarray(self._d["w_up"], dtype=np.float64)

    def w1(self, e):
        return np.asarray(self._d["w1"][e], dtype=np.float64)

    def w2(self, e):
        return np.asarray(self._d["w2"][e], dtype=np.float64)

    def w3(self, e):
        return np.asarray(self._d["w3"][e], dtype=np.float64)

    def ws1(self, j):
        return np.asarray(self._d["ws1"][j], dtype=np.float64)

    def ws2(self, j):
        return np.asarray(self._d["ws2"][j], dtype=np.float64)

    def ws3(self, j):
        return np.asarray(self._d["ws3"][j], dtype=np.float64)

    def bias(self):
        n = self._d["w_router"].shape[0]
        return np.zeros(n) if self._bias is None else np.asarray(self._bias, dtype=np.float64)

    def logit_offset(self):
        return None if self._o is None else np.asarray(self._o, dtype=np.float64)

    def gamma(self):
        L = self._d["w_down"].shape[0]
        return np.ones(L) if self._gamma is None else np.asarray(self._gamma, dtype=np.float64)


def forward(x, P, k, n_shared, dtype, beta1=4.0, beta2=25.0, eps=1e-6, forced_idx=None, gate="tanh",
            norm="rms"):
    """Stable LatentMoE forward for the token rows x [T, d].

    Steps ([DD] §2 LatentMoE: d -(down)-> d/2 -(route/gate)-> D -> d/2 -(up)-> d;
    [RB] "LatentMoE: paying for a bigger pool" and "Keeping the numbers in range"):
      1. z = rnd(x W_down^T)                      pure linear map, no norm after it
      2. s = sigmoid(z W_r^T + o)
      3. top-k on s + b (ties -> lower index)     loss-free selection bias
      4. g = s / sum over the chosen k
      5. dispatch rows to experts (stable by token)
      6. a = rnd(SiTU(z W1_e^T; b1) * softcap(z W2_e^T; b2)) per expert
      7. u_i += g_ie * (a W3_e^T)                 router-weighted aggregation
      8. u_i += shared_j(z_i) for every shared expert (weight 1, same SiTU-GLU)
      9. v = rnd(RMSNorm(u))                       the single retained norm
     10. y = rnd(v W_up^T)
    READING: shared experts run in the latent space and are summed into u
    before the norm; the residual add of the surrounding block is not part of
    the layer.  forced_idx replaces step 3 (used to compare expert math on
    tokens whose k-th/(k+1)-th scores are too close to call).  gate="clip"
    puts hard_clip in place of softcap in steps 6 and 8 (the hard-clip
    ablation).  norm="none" drops step 9's norm, v = rnd(u) (the ablation of
    the one retained norm, [DD] §2); norm="both" keeps it and adds the norm
    the pages leave out after the down-projection: step 1 becomes
    z = rnd(RMSNorm(rnd(x W_down^T))), unit gain, the same eps (READING: the
    stored z is normed in place, so the router and the experts both see it).
    """
    if norm not in ("rms", "none", "both"):
        raise ValueError(f"unknown norm {norm!r}")
    x = np.asarray(x, dtype=np.float64)
    w_router = P.w_router()
    n = w_router.shape[0]
    z_pre = x @ P.w_down().T
    if norm == "both":
        z_pre = rms_norm(round_to(z_pre, dtype), np.ones(z_pre.shape[1]), eps)
    z = round_to(z_pre, dtype)
    s = router_scores(z, w_router, P.logit_offset())
    if forced_idx is None:
        idx, gap = biased_topk(s, P.bias(), k)
    else:
        idx = np.asarray(forced_idx, dtype=np.int64)
        gap = np.full(idx.shape[0], np.nan)
    g = routing_weights(s, idx)
    counts, offs, row_token, row_slot = dispatch(idx, n)
    T = x.shape[0]
    L = z.shape[1]
    u = np.zeros((T, L), dtype=np.float64)
    for e in range(n):
        lo, hi = offs[e], offs[e + 1]
        if lo == hi:
            continue
        toks = row_token[lo:hi]
        a = expert_hidden(z[toks], P.w1(e), P.w2(e), beta1, beta2, dtype, gate)
        u[toks] += g[toks, row_slot[lo:hi]][:, None] * (a @ P.w3(e).T)
    for j in range(n_shared):
        a = expert_hidden(z, P.ws1(j), P.ws2(j), beta1, beta2, dtype, gate)
        u += a @ P.ws3(j).T
    v_pre = u if norm == "none" else rms_norm(u, P.gamma(), eps)
    v = round_to(v_pre, dtype)
    y_pre = v @ P.w_up().T
    y = round_to(y_pre, dtype)
    # *_pre: the same tensors before their store rounding (for tolerance checks)
    return dict(z=z, s=s, s32=s.astype(np.float32), idx=idx, gap=gap, g=g, counts=counts, offs=offs,
                row_token=row_token, row_slot=row_slot, u=u, v=v, y=y, z_pre=z_pre, v_pre=v_pre, y_pre=y_pre)


# ---------------------------------------------------------------------------
# Quantile Balancing  ([DD] §3 Quantile Balancing: map scores into [0,1],
# keep a B-bin histogram, aggregate by summing histograms, read the quantile;
# B = 1000 by default.  [IK] "Quantile Balancing (QB)".  [RB] "Keeping the
# numbers in range": read the score distribution against the top-k threshold
# and move each expert's threshold to its target share.)


def qb_bins(s32, nbins):
    """Bin of each fp32 score: floor(fp32(s * B)) clamped to [0, B-1].

    READING: left-closed bins of width 1/B; the product is one fp32 multiply
    (round to nearest even); s = 1 and anything above lands in the last bin;
    negative scores and NaN land in bin 0.
    """
    t = np.asarray(s32, dtype=np.float32) * np.float32(nbins)
    with np.errstate(invalid="ignore"):
        ge1 = t >= np.float32(1.0)
        top = t >= np.float32(nbins - 1)
    tf = np.where(ge1 & ~top, t, np.float32(0.0))
    b = np.floor(tf).astype(np.int64)
    b[top] = nbins - 1
    b[~ge1] = 0
    return b


def qb_histogram(s32, nbins):
    """H[e][j] = number of tokens whose score for expert e falls in bin j (int64 [n, B]).

    READING: all T*n unbiased scores are counted, one histogram per expert.
    """
    b = qb_bins(s32, nbins)
    T, n = b.shape
    H = np.zeros((n, nbins), dtype=np.int64)
    for e in range(n):
        H[e] = np.bincount(b[:, e], minlength=nbins)
    return H


def qb_read(h, c):
    """Score level above which a count c of the histogram's mass lies (upper-tail quantile).

    G(j) = sum_{j' >= j} h[j'], G(B) = 0; j* = max{j : G(j) >= c};
    q = (j* + 1 - (c - G(j*+1)) / h[j*]) / B   (linear inside the crossing bin).
    Requires 0 < c <= sum(h).
    """
    h = np.asarray(h, dtype=np.int64)
    B = h.size
    G = np.zeros(B + 1, dtype=np.int64)
    G[:B] = np.cumsum(h[::-1])[::-1]
    above = np.nonzero(G[:B] >= c)[0]
    jstar = int(above.max())
    frac = (float(c) - float(G[jstar + 1])) / float(h[jstar])
    return (float(jstar + 1) - frac) / float(B)


def qb_solve(H, k, n, bias_in):
    """Bias that gives each expert its target share k/n of the tokens.

    q_e = upper-(k/n) quantile of expert e's histogram; tau = the same read on
    the pooled histogram sum_e H[e] (the global top-k threshold);
    b_e = fp32(tau - q_e).  READING: the bias is set directly (no step size),
    which is what makes the rule free of hyper-parameters.  An empty
    histogram carries no information and leaves the bias unchanged.
    """
    H = np.asarray(H, dtype=np.int64)
    out = np.array(bias_in, dtype=np.float32, copy=True)
    pooled = H.sum(axis=0)
    Np = int(pooled.sum())
    if Np == 0:
        return out
    tau = qb_read(pooled, Np * k / n)
    for e in range(H.shape[0]):
        Ne = int(H[e].sum())
        if Ne == 0:
            continue
        q = qb_read(H[e], Ne * k / n)
        out[e] = np.float32(tau - q)
    return out


def qb_update(s32, nbins, k, hist=None, accumulate=False, bias=None, solve=True):
    """One QB call: (optionally accumulate into) the histogram, then optionally solve the bias.

    Summing histograms is how the estimator aggregates across devices ([DD] §3
    step 3); on one device the sum is local.
    """
    s32 = np.asarray(s32, dtype=np.float32)
    n = s32.shape[1]
    Hb = qb_histogram(s32, nbins)
    H = Hb + np.asarray(hist, dtype=np.int64) if (accumulate and hist is not None) else Hb
    b = None
    if solve:
        b = qb_solve(H, k, n, np.zeros(n, np.float32) if bias is None else bias)
    return H, b


def expert_loads(idx, n):
    """Tokens routed to each expert."""
    return np.bincount(np.asarray(idx).reshape(-1), minlength=n)



# ---------------------------------------------------------------------------
# Bias-update baselines and variants compared with Quantile Balancing
# ([DD] §3: K2's loss-free balancing used a SignSGD-style bias update that
# becomes unstable at 896 experts; [RB] "Keeping the numbers in range": K2
# nudged each expert's selection up or down by a fixed step; QB instead reads
# the router scores against the top-k threshold and solves where each expert's
# threshold should move to get its target share; [IK] Quantile Balancing.)


def signsgd_update(loads, T, k, bias, step):
    """K2-style bias step: b_e <- fp32(b_e + step * sign(T k / n - load_e)).

    READING: the pages give the rule's form (a fixed step up for under-loaded,
    down for over-loaded experts) but no step size; `step` is the caller's.
    The comparison with the target share is exact in integers
    (load_e * n against T * k); an expert exactly at its share keeps its bias.
    """
    loads = np.asarray(loads, dtype=np.int64)
    n = loads.size
    target = int(T) * int(k)
    sgn = np.sign(target - loads * n).astype(np.float32)
    return (np.asarray(bias, dtype=np.float32) + np.float32(step) * sgn).astype(np.float32)


def selection_keys(s32, bias):
    """The keys the top-k compares: fp32(s + b), one fp32 add per element."""
    return (np.asarray(s32, dtype=np.float32) + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)


def margin_thresholds(sel, k):
    """Per token, the k-th and (k+1)-th largest selection keys (tau_k, tau_k1);
    tau_k1 = -inf when k equals the expert count."""
    srt = -np.sort(-np.asarray(sel, dtype=np.float32), axis=1)
    tk = srt[:, k - 1]
    tk1 = srt[:, k] if k < srt.shape[1] else np.full(srt.shape[0], -np.inf, dtype=np.float32)
    return tk.astype(np.float32), tk1.astype(np.float32)


def margins(s32, bias, k):
    """Margin of every (token, expert) against the threshold that expert must cross.

    READING of "reads the distribution of router scores against the top-k
    threshold" ([RB]): an expert whose key is at or above the token's k-th key
    is in the token's top-k and leaves it when its key falls below the (k+1)-th
    key; any other expert enters when its key passes the k-th.  So
      m_ie = fp32(sel_ie - tau_k1(i))   if sel_ie >= tau_k(i)
      m_ie = fp32(sel_ie - tau_k(i))    otherwise,
    and, away from ties, shifting expert e's bias alone by delta keeps it in
    (or brings it into) token i's top-k exactly when m_ie + delta > 0.
    """
    sel = selection_keys(s32, bias)
    tk, tk1 = margin_thresholds(sel, k)
    with np.errstate(invalid="ignore"):
        above = sel >= tk[:, None]
    thr = np.where(above, tk1[:, None], tk[:, None]).astype(np.float32)
    return (sel - thr).astype(np.float32)


def margin_bins(m32, nbins):
    """Bin of each fp32 margin: the margin mapped to [0, 1] as u = fp32(m + 1) * 0.5
    (margins of sigmoid scores under small biases lie in (-1, 1); the halving is
    exact), then the score binning rule of qb_bins (clamped to the end bins)."""
    m32 = np.asarray(m32, dtype=np.float32)
    u = ((m32 + np.float32(1.0)).astype(np.float32) * np.float32(0.5)).astype(np.float32)
    return qb_bins(u, nbins)


def margin_histogram(s32, bias, k, nbins):
    """H[e][j]: tokens whose margin for expert e falls in bin j (int64 [n, B])."""
    b = margin_bins(margins(s32, bias, k), nbins)
    T, n = b.shape
    H = np.zeros((n, nbins), dtype=np.int64)
    for e in range(n):
        H[e] = np.bincount(b[:, e], minlength=nbins)
    return H


def margin_solve(H, k, n, bias_in):
    """Move each expert's bias so that its target share k/n of tokens clears its threshold.

    q_e = upper-(k/n) quantile of expert e's margin histogram (in [0, 1]
    units), i.e. the margin 2 q_e - 1 that N_e k / n of its tokens reach;
    b_e <- fp32(b_e - (2 q_e - 1)), computed in fp64.  No step size: the shift
    is read off the distribution.  Experts with an empty histogram keep their
    bias.  READING: iterated batch after batch, since every expert moves at once
    and the tokens' thresholds move with them.
    """
    H = np.asarray(H, dtype=np.int64)
    out = np.array(bias_in, dtype=np.float32, copy=True)
    for e in range(H.shape[0]):
        Ne = int(H[e].sum())
        if Ne == 0:
            continue
        q = qb_read(H[e], Ne * k / n)
        out[e] = np.float32(float(out[e]) - (2.0 * q - 1.0))
    return out


def margin_update(s32, nbins, k, bias, hist=None, accumulate=False, solve=True):
    """One margin-QB call: histogram this batch's margins (optionally added to
    `hist`), then optionally solve the new bias."""
    s32 = np.asarray(s32, dtype=np.float32)
    n = s32.shape[1]
    Hb = margin_histogram(s32, bias, k, nbins)
    H = Hb + np.asarray(hist, dtype=np.int64) if (accumulate and hist is not None) else Hb
    b = margin_solve(H, k, n, bias) if solve else None
    return H, b


# ---------------------------------------------------------------------------
# Backward pass  ([DD] §2, effect 6: with the norm before the up-projection the
# up-projection's weight gradient takes the normalised form g (h / |h|_RMS)^T;
# [DD] §1: the softcap's gradient, unlike a clip's, never vanishes abruptly)


def softcap_grad(x, beta, gate="tanh"):
    """d/dx of the branch cap: 1 - tanh^2(x / beta) for the softcap (1 at beta = +inf);
    for the hard clip 1 inside (-beta, beta) and 0 outside."""
    x = np.asarray(x, dtype=np.float64)
    if gate == "clip":
        return (np.abs(x) < beta).astype(np.float64)
    if beta == np.inf:
        return np.ones_like(x)
    t = np.tanh(x / beta)
    return 1.0 - t * t


def situ_grad(x, beta, gate="tanh"):
    """d/dx SiTU(x; beta) = cap'(x) sigmoid(x) + cap(x) sigmoid(x) (1 - sigmoid(x))."""
    sg = sigmoid(x)
    return softcap_grad(x, beta, gate) * sg + cap(x, beta, gate) * sg * (1.0 - sg)


def backward(x, P, k, n_shared, dtype, dy, beta1=4.0, beta2=25.0, eps=1e-6, forced_idx=None, gate="tanh",
             norm="rms"):
    """Gradients of the layer for the upstream gradient dy [T, d] of y.

    The forward is recomputed as `forward` computes it (z, a, v rounded where it
    stores them).  The backward stores, in the work dtype, the tensors that feed
    a matrix product: the latent gradient du (and g du, the routed rows'
    output gradient), the gated hidden's gradient da, the gate inputs'
    gradients dp1, dp2, the router logits' gradient dl, the latent's gradient
    dz and the rows it is summed from (one per routed slot, shared expert and
    the router); every product is then taken in fp64 of those rounded values.
    dv, the norm's backward, the routing weights' gradient and the sum of the dz
    rows stay unrounded.
    Steps (chain rule, the forward's notation):
      dv = dy W_up;  dW_up = dy^T v
      norm "rms": u_hat = u / r, r = sqrt(mean(u^2) + eps); dgamma = sum_i dv (.) u_hat;
                  du = (gamma (.) dv - u_hat mean(gamma (.) dv (.) u_hat)) / r
      norm "none": du = dv
      routed row (token i, slot j, expert e), with du stored as rnd(du):
                  o = a W3_e^T; dg_ij = du_i . o (unrounded du);
                  da = rnd(g_ij (rnd(du_i) W3_e));  dW3_e += rnd(g rnd(du_i))^T a
      shared expert s: da = rnd(rnd(du_i) W3s_s);  dW3s_s += rnd(du_i)^T a
      gate: dp1 = rnd(da) C(p2) SiTU'(p1);  dp2 = rnd(da) SiTU(p1) C'(p2)
            with p1 = z W1^T, p2 = z W2^T recomputed from the stored z
      dz_i += rnd(rnd(dp1) W1_e + rnd(dp2) W2_e);  dW1_e += rnd(dp1)^T z;  dW2_e += rnd(dp2)^T z
      router, chosen experts only (selection is not differentiable; the bias b
      gets no gradient): g_j = s_j / S, S = sum_j s_j:
            ds_j = (dg_j - sum_j' dg_j' g_j') / S;  dl_j = ds_j s_j (1 - s_j)
            dz += rnd(rnd(dl) W_r);  dW_r = rnd(dl)^T z
      dx = rnd(dz) W_down;  dW_down = rnd(dz)^T x
    Returns a dict with the weight gradients (dw_down [L, d], dw_router [n, L],
    dw1, dw2 [n, D, L], dw3 [n, L, D], dws1, dws2 [n_s, D, L], dws3 [n_s, L, D],
    dgamma [L], dw_up [d, L]), dx [T, d] and the intermediates (dv, du, dz, dl
    [T, n] dense with zeros off the chosen experts), each also before its own
    store rounding where it has one (*_pre).
    READING: norm "both" (the extra norm on z) has no backward here.
    """
    if norm not in ("rms", "none"):
        raise ValueError(f"backward has no norm {norm!r}")
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    fw = forward(x, P, k, n_shared, dtype, beta1, beta2, eps, forced_idx=forced_idx, gate=gate, norm=norm)
    z, s, idx, g, u, v = fw["z"], fw["s"], fw["idx"], fw["g"], fw["u"], fw["v"]
    T, L = z.shape
    n = s.shape[1]
    w_up = P.w_up()
    dv = dy @ w_up
    dw_up = dy.T @ v
    if norm == "rms":
        gamma = P.gamma()
        r = np.sqrt(np.mean(u * u, axis=1, keepdims=True) + eps)
        uh = u / r
        dgamma = np.sum(dv * uh, axis=0)
        dh = gamma[None, :] * dv
        du = (dh - uh * np.mean(dh * uh, axis=1, keepdims=True)) / r
    else:
        dgamma = np.zeros(L)
        du = dv
    du_r = round_to(du, dtype)
    counts, offs, row_token, row_slot = dispatch(idx, n)
    dz = np.zeros((T, L))
    dg = np.zeros_like(g)
    D = P.w1(0).shape[0]
    dw1 = np.zeros((n, D, L))
    dw2 = np.zeros((n, D, L))
    dw3 = np.zeros((n, L, D))

    def expert_back(zr, w1, w2, w3, du_rows, gr):
        p1 = zr @ w1.T
        p2 = zr @ w2.T
        a = round_to(situ_glu_hidden(p1, p2, beta1, beta2, gate), dtype)
        da = round_to(gr[:, None] * (du_rows @ w3), dtype)
        dout = round_to(gr[:, None] * du_rows, dtype)
        dp1 = round_to(da * cap(p2, beta2, gate) * situ_grad(p1, beta1, gate), dtype)
        dp2 = round_to(da * situ(p1, beta1, gate) * softcap_grad(p2, beta2, gate), dtype)
        return a, round_to(dp1 @ w1 + dp2 @ w2, dtype), dp1.T @ zr, dp2.T @ zr, dout.T @ a

    for e in range(n):
        lo, hi = offs[e], offs[e + 1]
        if lo == hi:
            continue
        toks, slots = row_token[lo:hi], row_slot[lo:hi]
        w1, w2, w3 = P.w1(e), P.w2(e), P.w3(e)
        gr = g[toks, slots]
        a, dzr, dw1[e], dw2[e], dw3[e] = expert_back(z[toks], w1, w2, w3, du_r[toks], gr)
        dg[toks, slots] = np.sum(du[toks] * (a @ w3.T), axis=1)
        np.add.at(dz, toks, dzr)
    dws1 = np.zeros((n_shared, D, L))
    dws2 = np.zeros((n_shared, D, L))
    dws3 = np.zeros((n_shared, L, D))
    for j in range(n_shared):
        _, dzr, dws1[j], dws2[j], dws3[j] = expert_back(z, P.ws1(j), P.ws2(j), P.ws3(j), du_r, np.ones(T))
        dz += dzr
    # router: g = s_K / S over the chosen experts
    sk = np.take_along_axis(s, idx, axis=1)
    S = sk.sum(axis=1, keepdims=True)
    dsk = (dg - np.sum(dg * g, axis=1, keepdims=True)) / S
    dl_pre = np.zeros((T, n))
    np.put_along_axis(dl_pre, idx, dsk * sk * (1.0 - sk), axis=1)
    dl = round_to(dl_pre, dtype)
    w_r = P.w_router()
    dz += round_to(dl @ w_r, dtype)
    dw_router = dl.T @ z
    dz_r = round_to(dz, dtype)
    dx = dz_r @ P.w_down()
    dw_down = dz_r.T @ x
    return dict(dx=dx, dw_down=dw_down, dw_router=dw_router, dw1=dw1, dw2=dw2, dw3=dw3, dws1=dws1, dws2=dws2,
                dws3=dws3, dgamma=dgamma, dw_up=dw_up, dv=dv, du=du_r, du_pre=du, dz=dz_r, dz_pre=dz, dl=dl,
                dl_pre=dl_pre, dg=dg, fw=fw)

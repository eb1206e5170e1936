"""CPU fp64 oracle of Forgetting Attention.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of
bench.py may import or call anything in this package; the library path never does.

Each function writes out the plain definition of one step of the method, in float64, with no
tiling, fusion or reordering beyond what the definition states. Sources (cited by page and
section; the pages summarise arXiv 2503.02130, "Forgetting Transformer: Softmax Attention with
a Forget Gate"):

  [FoX-pg]  paper-graph-ui.vercel.app summary, section 3.4 "Detailed, Sentence-Based Technical
            Breakdown" with its parts "The Mathematical Form of Forgetting Attention",
            "Forget Gate Computation", "Hardware-Aware Implementation (Modified FlashAttention)",
            "Connection to ALiBi" and "The Pro Block Architecture".
  [FoX-pl]  paperlayer.ai summary (abs/2503.02130v2), sections "3 FORGETTING TRANSFORMER",
            "D DATA-INDEPENDENT FORGET GATE INITIALIZATION" and "E HARDWARE-AWARE
            IMPLEMENTATION OF FORGETTING ATTENTION".

Two independent tiers compute attention:
  T1 (``*_bruteforce``): explicit range sums D_ij = sum_{l=j+1..i} log f_l and per-row loops;
      supports log f = -inf (f = 0). For tiny L only.
  T2 (``attn_fwd`` / ``attn_bwd`` / ``attn_fwd_rows`` / ``attn_bwd_tail``): D_ij = c_i - c_j
      with c = cumsum(log f), vectorised over blocks of query rows (the blocking only groups
      rows; every row still sees all of its keys at once).

Conventions (readings taken where the pages are silent or ambiguous): positions are 0-indexed and
c is the inclusive prefix sum; the softmax scale multiplies q.k only, never the bias; the
causal mask keeps j <= i (D_ii = 0); LSE is the natural-log log-sum-exp of the biased, scaled
logits.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def _f64(a):
    return np.asarray(a, dtype=F64)


# ----------------------------------------------------------------------------------------------
# Forget gate  ([FoX-pg] "Forget Gate Computation"; Pro block Step 4)
# ----------------------------------------------------------------------------------------------
def log_sigmoid(z):
    """log sigma(z) in fp64, evaluated stably: -log1p(exp(-z)) for z >= 0, z - log1p(exp(z)) else.

    The gate is f = sigma(w_f . x + b_f) in (0,1); the path only ever needs log f.
    """
    z = _f64(z)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = -np.log1p(np.exp(-z[pos]))
    out[~pos] = z[~pos] - np.log1p(np.exp(z[~pos]))
    return out


def gate_logf(x, w_f, b_f):
    """Per-head scalar forget gate in log space.

    x: [B, L, d_model] layer input; w_f: [H, d_model]; b_f: [H]  ->  log f: [B, H, L].
    z[b,h,t] = sum_d x[b,t,d] w_f[h,d] + b_f[h]; log f = log sigma(z).
    One (w_f, b_f) pair per head ([FoX-pg] "Forget Gate Computation", multi-head treatment).
    """
    x, w_f, b_f = _f64(x), _f64(w_f), _f64(b_f)
    z = np.matmul(x, w_f.T)                        # [B, L, H]
    z = np.transpose(z, (0, 2, 1)) + b_f[None, :, None]
    return log_sigmoid(z)


def rms_norm(x, eps, weight=None):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) [* weight].

    Used for QK-norm in the Pro block (Step 1 for queries, Step 2 for keys); unit weights
    when ``weight`` is None.
    """
    x = _f64(x)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    if weight is not None:
        y = y * _f64(weight)
    return y


def gate_logf_bwd(x, w_f, b_f, dlog_f):
    """Gradients of the gate through log sigma and the per-head GEMV.

    Given the upstream gradient dlog_f [B, H, L] of log f = log sigma(z),
    z[b,h,t] = sum_d x[b,t,d] w_f[h,d] + b_f[h]:
      dz   = dlog_f * d(log sigma)/dz = dlog_f * sigma(-z)        (1 - sigma(z) = sigma(-z))
      db_f = sum_{b,t} dz[b,h,t]
      dw_f = sum_{b,t} dz[b,h,t] x[b,t,:]
      dx   = sum_h dz[b,h,t] w_f[h,:]
    Returns (dx [B, L, d_model], dw_f [H, d_model], db_f [H]). sigma(-z) is taken as
    exp(log sigma(-z)), so it never rounds to 0 or 1 before the product.
    ([FoX-pg] "Forget Gate Computation"; Pro block Step 4.)
    """
    x, w_f, b_f, g = _f64(x), _f64(w_f), _f64(b_f), _f64(dlog_f)
    z = np.transpose(np.matmul(x, w_f.T), (0, 2, 1)) + b_f[None, :, None]   # [B, H, L]
    dz = g * np.exp(log_sigmoid(-z))
    db_f = dz.sum(axis=(0, 2))
    dw_f = np.einsum("bhl,bld->hd", dz, x)
    dx = np.einsum("bhl,hd->bld", dz, w_f)
    return dx, dw_f, db_f


def rms_norm_bwd(x, dy, eps, weight=None):
    """Gradients of y = x / r * w, r = sqrt(mean(x^2) + eps), over the last axis.

    With xh = x / r and g = dy * w (g = dy for unit weights):
      dx = (g - xh * mean(g * xh)) / r
      dw = sum over rows of dy * xh          (None for unit weights)
    Returns (dx, dw). ([FoX-pg] "The Pro Block Architecture", Steps 1-2, QK-norm.)
    """
    x, dy = _f64(x), _f64(dy)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    xh = x / r
    g = dy if weight is None else dy * _f64(weight)
    dx = (g - xh * np.mean(g * xh, axis=-1, keepdims=True)) / r
    dw = None if weight is None else (dy * xh).reshape(-1, x.shape[-1]).sum(axis=0)
    return dx, dw


# ----------------------------------------------------------------------------------------------
# Pro block: KV-shift and output norm + gate  ([FoX-pg] "The Pro Block Architecture", Steps 2,
# 3, 5 and 7). The equations of these steps are missing from the page; the readings below take
# the plainest form its words support (see the readings table of the design notes).
# ----------------------------------------------------------------------------------------------
def shift_gate(x, w):
    """Shift gate alpha[b, h, t] = sigma(x[b, t, :] . w[h, :]) in (0, 1), one learned vector per
    head and no bias (Step 2: "an additional learned vector for the shift gate")."""
    z = np.transpose(np.matmul(_f64(x), _f64(w).T), (0, 2, 1))
    return np.exp(log_sigmoid(z))


def shift_gate_bwd(x, w, dalpha):
    """Gradients of shift_gate for the upstream gradient dalpha [B, H, L]:
    dz = dalpha sigma(z) sigma(-z), dw = sum_{b,t} dz x, dx = sum_h dz w. Returns (dx, dw)."""
    x, w, g = _f64(x), _f64(w), _f64(dalpha)
    z = np.transpose(np.matmul(x, w.T), (0, 2, 1))
    dz = g * np.exp(log_sigmoid(z) + log_sigmoid(-z))
    return np.einsum("bhl,hd->bld", dz, w), np.einsum("bhl,bld->hd", dz, x)


def kv_shift(x_cand, alpha):
    """Data-dependent token shift over positions (Steps 2-3): the shift gate interpolates between
    the previous position's candidate and the current one,
        y_t = alpha_t x_{t-1} + (1 - alpha_t) x_t,   x_{-1} = 0,
    with alpha_t weighting the carried-forward previous candidate. x_cand [..., L, D],
    alpha [..., L]."""
    x, a = _f64(x_cand), _f64(alpha)[..., None]
    prev = np.concatenate([np.zeros_like(x[..., :1, :]), x[..., :-1, :]], axis=-2)
    return a * prev + (1.0 - a) * x


def kv_shift_bwd(x_cand, alpha, dy):
    """Gradients of kv_shift: dx_t = (1 - alpha_t) dy_t + alpha_{t+1} dy_{t+1} (the last
    position has no successor) and dalpha_t = sum_d dy_t (x_{t-1} - x_t)."""
    x, a, g = _f64(x_cand), _f64(alpha), _f64(dy)
    prev = np.concatenate([np.zeros_like(x[..., :1, :]), x[..., :-1, :]], axis=-2)
    nxt = np.concatenate([(a[..., 1:, None] * g[..., 1:, :]), np.zeros_like(g[..., :1, :])], axis=-2)
    dx = (1.0 - a[..., None]) * g + nxt
    da = np.sum(g * (prev - x), axis=-1)
    return dx, da


def out_norm_gate(o, g_lin, eps, weight=None):
    """Output normalisation and gating (Steps 5 and 7): y = RMSNorm(o) [* weight] * sigma(g_lin),
    the per-dimension output gate sigma(W_g x) applied to the normalised attention output
    before the output projection."""
    return rms_norm(o, eps, weight) * np.exp(log_sigmoid(_f64(g_lin)))


def out_norm_gate_bwd(o, g_lin, eps, dy, weight=None):
    """Gradients of out_norm_gate: with n = RMSNorm(o) [* weight] and s = sigma(g_lin),
    dg_lin = dy n s (1 - s) and do = RMSNorm backward of dy s (rms_norm_bwd)."""
    gl, dy = _f64(g_lin), _f64(dy)
    s = np.exp(log_sigmoid(gl))
    n = rms_norm(o, eps, weight)
    dg = dy * n * s * np.exp(log_sigmoid(-gl))
    do, _ = rms_norm_bwd(o, dy * s, eps, weight)
    return do, dg


def fixed_gate_logf(t_min, t_max, H):
    """Data-independent gate initialisation ([FoX-pl] D; [FoX-pg] "Connection to ALiBi").

    The decay horizons T_h are geometrically spaced from t_min to t_max; the bias is
    b_h = logit(exp(-1/T_h)), so sigma(b_h)^T_h = 1/e. Returns (T_h, b_h, log f_h = log sigma(b_h)).
    Used only to build structured test inputs (a fixed gate is ALiBi with slope 1/T_h).
    """
    if H == 1:
        T = np.array([float(t_min)])
    else:
        T = float(t_min) * (float(t_max) / float(t_min)) ** (np.arange(H, dtype=F64) / (H - 1))
    f = np.exp(-1.0 / T)
    b = np.log(f) - np.log1p(-f)
    return T, b, log_sigmoid(b)


# ----------------------------------------------------------------------------------------------
# Cumulative log decay  ([FoX-pg] "Hardware-Aware Implementation": c = cumsum(log f))
# ----------------------------------------------------------------------------------------------
def cumsum_logf(log_f):
    """c_i = sum_{l <= i} log f_l (inclusive, 0-indexed), fp64, along the last axis."""
    return np.cumsum(_f64(log_f), axis=-1)


def reverse_cumsum(dc):
    """d log f_l = sum_{t >= l} dc_t: the adjoint of the inclusive prefix sum."""
    dc = _f64(dc)
    return np.flip(np.cumsum(np.flip(dc, axis=-1), axis=-1), axis=-1)


# ----------------------------------------------------------------------------------------------
# T1: brute force from the definition  ([FoX-pg] "The Mathematical Form of Forgetting Attention")
# ----------------------------------------------------------------------------------------------
def decay_bias_bruteforce(log_f_row):
    """D[i, j] = sum_{l=j+1..i} log f_l for j <= i (so D_ii = 0), -inf for j > i.

    Explicit range sums; log f may hold -inf (f = 0, log 0 = -inf cuts off every key before it).
    """
    lf = _f64(log_f_row)
    L = lf.shape[0]
    D = np.full((L, L), -np.inf)
    for i in range(L):
        for j in range(i + 1):
            D[i, j] = lf[j + 1:i + 1].sum() if i > j else 0.0
    return D


def attn_probs_bruteforce(q, k, log_f, scale):
    """P[i, :] = softmax_j(scale * q_i . k_j + D_ij) for one (b, h): [L, L], zeros above the diagonal."""
    q, k = _f64(q), _f64(k)
    L = q.shape[0]
    D = decay_bias_bruteforce(log_f)
    P = np.zeros((L, L))
    for i in range(L):
        s = scale * (k[:i + 1] @ q[i]) + D[i, :i + 1]
        m = np.max(s)
        p = np.exp(s - m)
        P[i, :i + 1] = p / p.sum()
    return P


def attn_fwd_bruteforce(q, k, v, log_f, scale):
    """T1 forward. q, k, v: [B, H, L, D]; log_f: [B, H, L]  ->  (O [B,H,L,D], LSE [B,H,L]).

    Per row: s_j = scale q_i.k_j + D_ij (j <= i); m = max s; p = exp(s - m); l = sum p;
    O_i = sum_j p_j v_j / l; LSE_i = m + log l.
    """
    q, k, v, log_f = _f64(q), _f64(k), _f64(v), _f64(log_f)
    B, H, L, Dh = q.shape
    O = np.zeros((B, H, L, Dh))
    LSE = np.zeros((B, H, L))
    for b in range(B):
        for h in range(H):
            D = decay_bias_bruteforce(log_f[b, h])
            for i in range(L):
                s = scale * (k[b, h, :i + 1] @ q[b, h, i]) + D[i, :i + 1]
                m = np.max(s)
                p = np.exp(s - m)
                ell = p.sum()
                O[b, h, i] = (p @ v[b, h, :i + 1]) / ell
                LSE[b, h, i] = m + np.log(ell)
    return O, LSE


def attn_bwd_bruteforce(q, k, v, log_f, do, scale):
    """T1 backward for the loss sum(dO * O): returns (dQ, dK, dV, dlog_f).

    P from attn_probs_bruteforce; dV = P^T dO; dP = dO V^T; dS = P * (dP - rowsum(dP * P));
    dQ = scale dS K; dK = scale dS^T Q. The log-gate gradient is taken straight from the
    definition: log f_l enters D_ij exactly when j < l <= i, so d log f_l = sum_{i >= l} sum_{j < l} dS_ij.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, L, Dh = q.shape
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    dlf = np.zeros((B, H, L))
    for b in range(B):
        for h in range(H):
            P = attn_probs_bruteforce(q[b, h], k[b, h], log_f[b, h], scale)
            dV[b, h] = P.T @ do[b, h]
            dP = do[b, h] @ v[b, h].T
            dS = P * (dP - np.sum(dP * P, axis=1, keepdims=True))
            dQ[b, h] = scale * (dS @ k[b, h])
            dK[b, h] = scale * (dS.T @ q[b, h])
            for l in range(L):
                dlf[b, h, l] = dS[l:, :l].sum()
    return dQ, dK, dV, dlf


# ----------------------------------------------------------------------------------------------
# T2: the c_i - c_j form  ([FoX-pg] "Hardware-Aware Implementation"; [FoX-pl] E)
# ----------------------------------------------------------------------------------------------
def _rows_logits(q_rows, k_keys, c_rows, c_keys, rows, scale):
    """s[r, j] = scale q_r . k_j + c_r - c_j for the given query rows; -inf where j > row."""
    s = scale * (q_rows @ k_keys.T) + (c_rows[:, None] - c_keys[None, :])
    j = np.arange(k_keys.shape[0])
    s[j[None, :] > rows[:, None]] = -np.inf
    return s


def attn_fwd(q, k, v, log_f=None, *, c=None, scale, block=512):
    """T2 forward. Either log_f or c ([B, H, L]) gives the decay. Returns (O, LSE) in fp64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    c = cumsum_logf(log_f) if c is None else _f64(c)
    B, H, L, Dh = q.shape
    O = np.zeros((B, H, L, Dh))
    LSE = np.zeros((B, H, L))
    for b in range(B):
        for h in range(H):
            for i0 in range(0, L, block):
                i1 = min(L, i0 + block)
                rows = np.arange(i0, i1)
                s = _rows_logits(q[b, h, i0:i1], k[b, h, :i1], c[b, h, i0:i1], c[b, h, :i1], rows,
                                 scale)
                m = s.max(axis=1)
                p = np.exp(s - m[:, None])
                ell = p.sum(axis=1)
                O[b, h, i0:i1] = (p @ v[b, h, :i1]) / ell[:, None]
                LSE[b, h, i0:i1] = m + np.log(ell)
    return O, LSE


def attn_fwd_rows(q, k, v, c, rows, *, scale):
    """O and LSE of selected rows of one (b, h): q, k, v [L, D], c [L] -> (O [n, D], LSE [n]).

    Each listed row i sees keys 0..i only; the cost is O(i * D) per row, so full-length
    sequences can be checked on a sample of rows.
    """
    q, k, v, c = _f64(q), _f64(k), _f64(v), _f64(c)
    rows = np.asarray(rows, dtype=np.int64)
    O = np.zeros((rows.size, q.shape[1]))
    LSE = np.zeros(rows.size)
    for n, i in enumerate(rows):
        s = scale * (k[:i + 1] @ q[i]) + (c[i] - c[:i + 1])
        m = s.max()
        p = np.exp(s - m)
        ell = p.sum()
        O[n] = (p @ v[:i + 1]) / ell
        LSE[n] = m + np.log(ell)
    return O, LSE


def attn_bwd_tail(q, k, v, c, do, n, *, scale):
    """Forward and backward of the last n positions of one (b, h): q, k, v, dO [L, D], c [L].

    Only the last n query rows reach the gradients of the last n positions: key j is seen by
    queries i >= j, and d log f_l = sum_{t >= l} dc_t sums over positions t >= l. So the
    definition written for rows i in [L - n, L) alone gives, exactly, O and LSE of those rows,
    their dQ, and dK, dV and d log f of those positions, whatever L is. Returns
    (O, LSE, dQ, dK, dV, dlog_f), each for the last n positions.
    """
    k, v, c = _f64(k), _f64(v), _f64(c)
    L = k.shape[0]
    i0 = L - n
    qt, dot = _f64(q[i0:]), _f64(do[i0:])
    rows = np.arange(i0, L)
    s = _rows_logits(qt, k, c[i0:], c, rows, scale)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    ell = p.sum(axis=1)
    P = p / ell[:, None]
    O = P @ v
    LSE = m + np.log(ell)
    Delta = np.sum(dot * O, axis=1)
    dP = dot @ v.T
    dS = P * (dP - Delta[:, None])
    dQ = scale * (dS @ k)
    dV = P[:, i0:].T @ dot
    dK = scale * (dS[:, i0:].T @ qt)
    dc = dS.sum(axis=1) - dS[:, i0:].sum(axis=0)  # dc^q_t + dc^k_t of the tail positions
    return O, LSE, dQ, dK, dV, reverse_cumsum(dc)


def attn_bwd(q, k, v, log_f=None, do=None, *, c=None, scale, O=None, LSE=None, block=512):
    """T2 backward for the loss sum(dO * O). Returns (dQ, dK, dV, dlog_f, dc_q, dc_k).

    Recompute P_ij = exp(s_ij - LSE_i) with the same bias; Delta_i = dO_i . O_i;
    dV_j = sum_i P_ij dO_i; dP_ij = dO_i . v_j; dS_ij = P_ij (dP_ij - Delta_i);
    dQ_i = scale sum_j dS_ij k_j; dK_j = scale sum_i dS_ij q_i;
    dc^q_i = sum_j dS_ij; dc^k_j = -sum_i dS_ij; dc = dc^q + dc^k; d log f = reverse cumsum(dc).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    c = cumsum_logf(log_f) if c is None else _f64(c)
    if O is None or LSE is None:
        O, LSE = attn_fwd(q, k, v, c=c, scale=scale, block=block)
    B, H, L, Dh = q.shape
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    dcq = np.zeros((B, H, L))
    dck = np.zeros((B, H, L))
    Delta = np.sum(do * O, axis=-1)
    for b in range(B):
        for h in range(H):
            for i0 in range(0, L, block):
                i1 = min(L, i0 + block)
                rows = np.arange(i0, i1)
                s = _rows_logits(q[b, h, i0:i1], k[b, h, :i1], c[b, h, i0:i1], c[b, h, :i1], rows,
                                 scale)
                P = np.exp(s - LSE[b, h, i0:i1, None])
                dV[b, h, :i1] += P.T @ do[b, h, i0:i1]
                dP = do[b, h, i0:i1] @ v[b, h, :i1].T
                dS = P * (dP - Delta[b, h, i0:i1, None])
                dQ[b, h, i0:i1] = scale * (dS @ k[b, h, :i1])
                dK[b, h, :i1] += scale * (dS.T @ q[b, h, i0:i1])
                dcq[b, h, i0:i1] = dS.sum(axis=1)
                dck[b, h, :i1] -= dS.sum(axis=0)
    dlf = reverse_cumsum(dcq + dck)
    return dQ, dK, dV, dlf, dcq, dck


# ----------------------------------------------------------------------------------------------
# Exact tile skipping  ([FoX-pl] section 6 "CONCLUSION", limitations and future work: pruning
# computation by the forget-gate values; [FoX-pg] "Follow-Up Research": eviction of tokens
# before sharp forget gates). The pages leave the method open; the reading here skips only work
# that contributes exact zeros, so the attention output is unchanged.
# ----------------------------------------------------------------------------------------------
def _group_max_norms(x, g):
    """Largest row norm |x_r| of every g-row group, [..., L, D] -> [..., ceil(L / g)]."""
    x = _f64(x)
    L = x.shape[-2]
    n = np.sqrt(np.sum(x * x, axis=-1))
    pad = (-L) % g
    n = np.concatenate([n, np.zeros(n.shape[:-1] + (pad,))], axis=-1)
    return n.reshape(n.shape[:-1] + (-1, g)).max(axis=-1)


def _group_extrema(c, g):
    """Smallest and largest value of c in every g-position group, [..., L] -> two
    [..., ceil(L / g)] arrays."""
    c = _f64(c)
    pad = (-c.shape[-1]) % g
    lo = np.concatenate([c, np.full(c.shape[:-1] + (pad,), np.inf)], axis=-1)
    hi = np.concatenate([c, np.full(c.shape[:-1] + (pad,), -np.inf)], axis=-1)
    shape = c.shape[:-1] + (-1, g)
    return lo.reshape(shape).min(axis=-1), hi.reshape(shape).max(axis=-1)


def skip_bounds(q, k, c, *, scale, g=64):
    """Upper bounds, in log2 units, on the weight of every key of a key tile for every query of
    a query tile, relative to the query's diagonal logit scale q_i.k_i.

    For a query i and an earlier key j the logit difference is
        scale q_i.(k_j - k_i) - (c_j - c_i) <= scale |q_i| (|k_j| + |k_i|) - (c_j - c_i)
    (Cauchy-Schwarz), and over a query range and an earlier key range
    c_j - c_i >= Cmin_keys - Cmax_queries, the smallest c of the key range less the largest c
    of the query range. With Qmax, Kmax and Kdiag the largest |q_i|, |k_j| and |k_i| of the
    ranges (taken over g-row groups):
        bound = log2(e) (scale Qmax (Kmax + Kdiag) - (Cmin_keys - Cmax_queries)).
    The forget gate lies in (0, 1), so c does not increase and the extremes are c at the key
    range's last position and at the query range's first; taking them over the groups keeps the
    bound valid for any finite c.

    Two tilings, both in g-row groups:
      fwd[b, h, t, T] : query tile t of 4g rows, key tile T of g rows, for the key tiles before
                        the tile's four diagonal key tiles (T < (last query of t) // g - 3);
                        +inf elsewhere.
      kv[b, h, kb, u] : key block kb of 2g rows, query tile u of g rows counted from the block's
                        first row, for u >= 2 (entirely after the block); +inf elsewhere.
    """
    q, k, c = _f64(q), _f64(k), _f64(c)
    B, H, L, _ = q.shape
    qn, kn = _group_max_norms(q, g), _group_max_norms(k, g)
    cmin, cmax = _group_extrema(c, g)
    n_qt, n_g, n_kb = -(-L // (4 * g)), -(-L // g), -(-L // (2 * g))
    fwd = np.full((B, H, n_qt, n_g), np.inf)
    kv = np.full((B, H, n_kb, n_g), np.inf)
    for t in range(n_qt):
        qa, qb = 4 * g * t, min(4 * g * t + 4 * g - 1, L - 1)
        groups = slice(qa // g, qb // g + 1)
        qmax, kdiag = qn[..., groups].max(axis=-1), kn[..., groups].max(axis=-1)
        cq = cmax[..., groups].max(axis=-1)
        for T in range(qb // g - 3):
            fwd[..., t, T] = np.log2(np.e) * (scale * qmax * (kn[..., T] + kdiag)
                                              - (cmin[..., T] - cq))
    for blk in range(n_kb):
        ka, kb = 2 * g * blk, min(2 * g * blk + 2 * g - 1, L - 1)
        kgroups = slice(ka // g, kb // g + 1)
        kmax, ck = kn[..., kgroups].max(axis=-1), cmin[..., kgroups].min(axis=-1)
        for u in range(2, -(-(L - ka) // g)):
            grp = (ka + g * u) // g
            kv[..., blk, u] = np.log2(np.e) * (scale * qn[..., grp] * (kmax + kn[..., grp])
                                               - (ck - cmax[..., grp]))
    return fwd, kv


def skip_plan(q, k, c, *, scale, threshold_log2=-160.0, g=64):
    """The tiles whose bound (skip_bounds) lies below threshold_log2.

    q_skip[b, h, t]    : the number of leading key tiles (from key 0) a query tile skips: the
                         longest prefix of its candidate tiles that all lie below the threshold.
    kv_tiles[b, h, kb] : the number of query tiles a key block walks from its first row: one more
                         than its last tile not below the threshold (at least 2, the diagonal),
                         capped at the tiles up to the sequence end.
    """
    fwd, kv = skip_bounds(q, k, c, scale=scale, g=g)
    B, H, L, _ = _f64(q).shape
    n_qt, n_kb = fwd.shape[2], kv.shape[2]
    q_skip = np.zeros((B, H, n_qt), np.int64)
    kv_tiles = np.zeros((B, H, n_kb), np.int64)
    for b in range(B):
        for h in range(H):
            for t in range(n_qt):
                qb = min(4 * g * t + 4 * g - 1, L - 1)
                n = 0
                while n < qb // g - 3 and fwd[b, h, t, n] < threshold_log2:
                    n += 1
                q_skip[b, h, t] = n
            for blk in range(n_kb):
                n_full = -(-(L - 2 * g * blk) // g)
                keep = [u for u in range(2, n_full) if not kv[b, h, blk, u] < threshold_log2]
                kv_tiles[b, h, blk] = min(n_full, max(keep, default=1) + 1)
    return q_skip, kv_tiles

"""Pins of the fp64 oracle against facts fixed outside it (CPU only).

Every check compares the oracle with something it does not compute itself: a library routine
(torch's causal scaled-dot-product attention, torch autograd, scipy's log_expit), a closed form
the pages state (ALiBi as a constant gate, the hard reset of log 0 = -inf, the printed gate
initialisation), an invariant of softmax attention, or central finite differences. The last
block plants mistakes into a copy of the oracle's source and checks that some pin catches each.
"""
import json
import math
import os
import types

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import fox_inputs as fi
import oracle
from oracle import fox_oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _case(B=2, H=2, L=64, D=32, seed=50, gate="normal"):
    return fi.make_case(B, H, L, D, "f32", seed=seed, gate=gate, with_do=True)


def _t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def _sdpa_causal(q, k, v, scale, bias=None):
    """torch's scaled_dot_product_attention (fp64, CPU) with causal masking and optional float bias."""
    L = q.shape[-2]
    mask = torch.full((L, L), -math.inf, dtype=torch.float64).triu(1)
    if bias is not None:
        mask = mask + _t(bias)
    return F.scaled_dot_product_attention(_t(q), _t(k), _t(v), attn_mask=mask, scale=scale).numpy()


def _lse_ref(q, k, scale, bias):
    L = q.shape[-2]
    s = torch.matmul(_t(q), _t(k).transpose(-1, -2).contiguous()) * scale + _t(bias)
    s = s + torch.full((L, L), -math.inf, dtype=torch.float64).triu(1)
    return torch.logsumexp(s, dim=-1).numpy()


# ---------------------------------------------------------------- two independent tiers agree
def test_t1_equals_t2_forward():
    c = _case()
    s = 1 / math.sqrt(c.D)
    O1, L1 = oracle.attn_fwd_bruteforce(c.q, c.k, c.v, c.log_f, s)
    O2, L2 = oracle.attn_fwd(c.q, c.k, c.v, c.log_f, scale=s, block=16)
    assert np.abs(O1 - O2).max() < 1e-12 and np.abs(L1 - L2).max() < 1e-12


def test_t1_equals_t2_backward():
    c = _case()
    s = 1 / math.sqrt(c.D)
    g1 = oracle.attn_bwd_bruteforce(c.q, c.k, c.v, c.log_f, c.do, s)
    g2 = oracle.attn_bwd(c.q, c.k, c.v, c.log_f, c.do, scale=s, block=16)
    for a, b in zip(g1, g2[:4]):
        assert np.abs(a - b).max() < 1e-11 * max(1.0, np.abs(a).max())


def test_range_sum_is_difference_of_prefix_sums():
    lf = fi.make_case(1, 1, 40, 4, "f32", seed=3).log_f[0, 0]
    D = oracle.decay_bias_bruteforce(lf)
    c = oracle.cumsum_logf(lf)
    ii, jj = np.tril_indices(40)
    assert np.abs(D[ii, jj] - (c[ii] - c[jj])).max() < 1e-12
    assert np.all(np.isneginf(D[np.triu_indices(40, 1)]))
    assert np.all(np.diag(D) == 0.0)


def test_rows_match_full_forward():
    c = _case(B=1, H=1, L=300, D=16, seed=7)
    s = 0.25
    O, LSE = oracle.attn_fwd(c.q, c.k, c.v, c.log_f, scale=s, block=64)
    cc = oracle.cumsum_logf(c.log_f)
    rows = np.array([0, 1, 63, 64, 200, 299])
    Or, Lr = oracle.attn_fwd_rows(c.q[0, 0], c.k[0, 0], c.v[0, 0], cc[0, 0], rows, scale=s)
    assert np.abs(Or - O[0, 0, rows]).max() < 1e-12 and np.abs(Lr - LSE[0, 0, rows]).max() < 1e-12
    # and against torch's attention with the explicit bias c_i - c_j, independently of attn_fwd
    bias = cc[0, 0][:, None] - cc[0, 0][None, :]
    ref = _sdpa_causal(c.q[:, :1], c.k[:, :1], c.v[:, :1], s, bias)[0, 0, rows]
    assert np.abs(Or - ref).max() < 1e-12
    assert np.abs(Lr - _lse_ref(c.q[:, :1], c.k[:, :1], s, bias)[0, 0, rows]).max() < 1e-12


# ---------------------------------------------------------------- closed forms and library routines
def test_all_gates_open_is_causal_softmax_attention():
    c = _case(gate="zero")
    s = 1 / math.sqrt(c.D)
    O, LSE = oracle.attn_fwd(c.q, c.k, c.v, c.log_f, scale=s, block=16)
    ref = _sdpa_causal(c.q, c.k, c.v, s)
    assert np.abs(O - ref).max() < 1e-12
    assert np.abs(LSE - _lse_ref(c.q, c.k, s, np.zeros((c.L, c.L)))).max() < 1e-12


@pytest.mark.parametrize("tier", ["T1", "T2"])
def test_constant_gate_is_alibi(tier):
    """log f = -m_h at every position gives the bias -m_h (i - j) exactly."""
    B, H, L, D = 1, 4, 48, 16
    c = fi.make_case(B, H, L, D, "f32", seed=11)
    m = 2.0 ** (-8.0 * np.arange(1, H + 1) / H)
    log_f = np.broadcast_to(-m[None, :, None], (B, H, L)).astype(np.float64)
    s = 1 / math.sqrt(D)
    if tier == "T1":
        O, LSE = oracle.attn_fwd_bruteforce(c.q, c.k, c.v, log_f, s)
    else:
        O, LSE = oracle.attn_fwd(c.q, c.k, c.v, log_f, scale=s, block=16)
    i = np.arange(L)
    for h in range(H):
        bias = -m[h] * (i[:, None] - i[None, :])
        bias = np.where(i[None, :] <= i[:, None], bias, 0.0)
        ref = _sdpa_causal(c.q[:, h:h + 1], c.k[:, h:h + 1], c.v[:, h:h + 1], s, bias)
        assert np.abs(O[:, h:h + 1] - ref).max() < 1e-12
        assert np.abs(LSE[0, h] - _lse_ref(c.q[0, h], c.k[0, h], s, bias)).max() < 1e-11


def test_fixed_gate_init_matches_printed_values():
    g = json.load(open(os.path.join(GOLDEN, "fixed_gate_init.json")))
    T, b, log_f = oracle.fixed_gate_logf(g["t_min"], g["t_max"], g["H"])
    assert np.allclose(T, g["horizons"], rtol=1e-12)
    f = np.exp(log_f)
    # the pages give three decimals without saying whether they round or truncate: allow one unit
    tol = 10.0 ** -g["printed_decimals"]
    assert abs(f[0] - g["f_at_t_min_approx"]) <= tol
    assert abs(f[-1] - g["f_at_t_max_approx"]) <= tol
    assert np.allclose(f ** T, math.exp(-1.0), rtol=1e-12)
    # a fixed gate is ALiBi with slope 1/T_h
    assert np.allclose(-log_f, 1.0 / T, rtol=1e-12)


@pytest.mark.parametrize("cut", [1, 17, 40])
def test_hard_reset_cuts_off_the_past(cut):
    """log f_l = -inf (f = 0): rows i >= l attend only to keys l..i (T1); -1e4 does the same in T2."""
    B, H, L, D = 1, 1, 48, 8
    c = fi.make_case(B, H, L, D, "f32", seed=5)
    s = 1 / math.sqrt(D)
    for val, tier in ((-np.inf, "T1"), (-1e4, "T2")):
        lf = c.log_f.astype(np.float64).copy()
        lf[..., cut] = val
        if tier == "T1":
            O, LSE = oracle.attn_fwd_bruteforce(c.q, c.k, c.v, lf, s)
        else:
            O, LSE = oracle.attn_fwd(c.q, c.k, c.v, lf, scale=s, block=16)
        lf_tail = lf[..., cut:].copy()
        lf_tail[..., 0] = 0.0
        O_tail, LSE_tail = oracle.attn_fwd_bruteforce(c.q[..., cut:, :], c.k[..., cut:, :],
                                                      c.v[..., cut:, :], lf_tail, s)
        assert np.abs(O[..., cut:, :] - O_tail).max() < 1e-12
        assert np.abs(LSE[..., cut:] - LSE_tail).max() < 1e-12


def test_first_row_sees_only_itself():
    c = _case()
    s = 0.3
    O, LSE = oracle.attn_fwd(c.q, c.k, c.v, c.log_f, scale=s)
    assert np.abs(O[..., 0, :] - c.v[..., 0, :]).max() < 1e-15
    assert np.abs(LSE[..., 0] - s * np.sum(c.q[..., 0, :].astype(np.float64) * c.k[..., 0, :], -1)).max() < 1e-12


def test_rows_are_distributions():
    c = _case(B=1, H=1, L=40)
    P = oracle.attn_probs_bruteforce(c.q[0, 0], c.k[0, 0], c.log_f[0, 0], 0.2)
    assert np.abs(P.sum(1) - 1).max() < 1e-14
    assert np.all(P >= 0) and np.all(np.triu(P, 1) == 0)


def test_shift_and_first_gate_invariance():
    c = _case()
    s = 1 / math.sqrt(c.D)
    cc = oracle.cumsum_logf(c.log_f)
    O, LSE = oracle.attn_fwd(c.q, c.k, c.v, c=cc, scale=s)
    O2, LSE2 = oracle.attn_fwd(c.q, c.k, c.v, c=cc + 123.25, scale=s)
    assert np.abs(O - O2).max() < 1e-12 and np.abs(LSE - LSE2).max() < 1e-10
    lf = c.log_f.astype(np.float64).copy()
    lf[..., 0] -= 7.0
    O3, LSE3 = oracle.attn_fwd(c.q, c.k, c.v, lf, scale=s)
    assert np.abs(O - O3).max() < 1e-12 and np.abs(LSE - LSE3).max() < 1e-10


def test_log_sigmoid_against_scipy():
    z = np.concatenate([np.linspace(-60, 60, 2001), [-800.0, -40.0, 0.0, 40.0, 800.0]])
    ref = scipy.special.log_expit(z)
    got = oracle.log_sigmoid(z)
    assert np.all(np.isfinite(got))
    assert np.abs(got - ref).max() <= 1e-15 * np.maximum(1.0, np.abs(ref)).max()
    assert oracle.log_sigmoid(np.array([0.0]))[0] == -math.log(2.0)


def test_gate_against_torch():
    c = fi.make_pro_case(2, 3, 40, 8, 96, seed=9)
    got = oracle.gate_logf(c.x, c.w_f, c.b_f)
    z = torch.einsum("bld,hd->bhl", _t(c.x), _t(c.w_f)) + _t(c.b_f)[None, :, None]
    assert np.abs(got - F.logsigmoid(z).numpy()).max() < 1e-13


def test_rms_norm_against_torch():
    x = np.random.default_rng(0).standard_normal((5, 7, 128))
    got = oracle.rms_norm(x, 1e-6)
    ref = F.rms_norm(_t(x), (128,), eps=1e-6).numpy()
    assert np.abs(got - ref).max() < 1e-13


def test_reverse_cumsum_is_adjoint_of_cumsum():
    rng = np.random.default_rng(1)
    a, b = rng.standard_normal(57), rng.standard_normal(57)
    assert abs(np.dot(oracle.cumsum_logf(a), b) - np.dot(a, oracle.reverse_cumsum(b))) < 1e-12


# ---------------------------------------------------------------- gradients
def _torch_grads(c, scale):
    """Gradients of sum(dO * O) through torch autograd, bias built as c_i - c_j in torch."""
    q, k, v = (_t(a).requires_grad_(True) for a in (c.q, c.k, c.v))
    lf = _t(c.log_f).requires_grad_(True)
    cc = torch.cumsum(lf, dim=-1)
    bias = cc[..., :, None] - cc[..., None, :]
    L = c.L
    bias = bias + torch.full((L, L), -math.inf, dtype=torch.float64).triu(1)
    O = F.scaled_dot_product_attention(q, k, v, attn_mask=bias, scale=scale)
    (O * _t(c.do)).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy(), lf.grad.numpy()


def test_gradients_against_torch_autograd():
    c = _case()
    s = 1 / math.sqrt(c.D)
    ref = _torch_grads(c, s)
    got = oracle.attn_bwd(c.q, c.k, c.v, c.log_f, c.do, scale=s, block=16)
    for g, r in zip(got[:4], ref):
        assert np.abs(g - r).max() < 1e-11 * max(1.0, np.abs(r).max())


def test_gradients_against_finite_differences():
    """Central differences along random directions, loss = sum(dO * O), fp64."""
    c = _case()
    s = 1 / math.sqrt(c.D)
    grads = oracle.attn_bwd(c.q, c.k, c.v, c.log_f, c.do, scale=s, block=32)[:4]
    base = [c.q.astype(np.float64), c.k.astype(np.float64), c.v.astype(np.float64),
            c.log_f.astype(np.float64)]
    rng = np.random.default_rng(123)

    def loss(args):
        O, _ = oracle.attn_fwd(args[0], args[1], args[2], args[3], scale=s, block=32)
        return float(np.sum(O * c.do))

    h = 1e-5
    for which in range(4):
        for _ in range(3):
            u = rng.standard_normal(base[which].shape)
            plus = list(base)
            minus = list(base)
            plus[which] = base[which] + h * u
            minus[which] = base[which] - h * u
            fd = (loss(plus) - loss(minus)) / (2 * h)
            an = float(np.sum(grads[which] * u))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (which, fd, an)


@pytest.mark.parametrize("n", [1, 5, 40, 64])
@pytest.mark.parametrize("gate", ["normal", "zero"])
def test_tail_backward_against_torch_autograd(n, gate):
    """attn_bwd_tail (the last n positions alone) against torch autograd of the whole sequence,
    and its forward part against torch's attention: exact where only the tail rows reach."""
    c = _case(B=1, H=1, L=64, D=16, seed=71, gate=gate)
    s = 1 / math.sqrt(c.D)
    dq, dk, dv, dlf = _torch_grads(c, s)
    cc = oracle.cumsum_logf(c.log_f)[0, 0]
    O, LSE, dQ, dK, dV, dLF = oracle.attn_bwd_tail(c.q[0, 0], c.k[0, 0], c.v[0, 0], cc,
                                                   c.do[0, 0], n, scale=s)
    bias = cc[:, None] - cc[None, :]
    ref_o = _sdpa_causal(c.q, c.k, c.v, s, bias)[0, 0, -n:]
    ref_lse = _lse_ref(c.q, c.k, s, bias)[0, 0, -n:]
    tol = 1e-11
    assert np.abs(O - ref_o).max() < tol and np.abs(LSE - ref_lse).max() < tol
    for got, ref in ((dQ, dq), (dK, dk), (dV, dv), (dLF, dlf)):
        ref = ref[0, 0, -n:]
        assert np.abs(got - ref).max() < tol * max(1.0, np.abs(ref).max())


def test_tail_backward_with_a_hard_reset():
    """A reset (log f = -1e4) inside the tail: rows after it see nothing before it."""
    c = _case(B=1, H=1, L=48, D=8, seed=72)
    c.log_f[0, 0, 40] = -1e4
    s = 0.3
    dq, dk, dv, dlf = _torch_grads(c, s)
    cc = oracle.cumsum_logf(c.log_f)[0, 0]
    got = oracle.attn_bwd_tail(c.q[0, 0], c.k[0, 0], c.v[0, 0], cc, c.do[0, 0], 12, scale=s)
    for g, r in zip(got[2:], (dq, dk, dv, dlf)):
        r = r[0, 0, -12:]
        assert np.abs(g - r).max() < 1e-10 * max(1.0, np.abs(r).max())


def test_gradient_invariants():
    c = _case()
    s = 1 / math.sqrt(c.D)
    dQ, dK, dV, dlf, dcq, dck = oracle.attn_bwd(c.q, c.k, c.v, c.log_f, c.do, scale=s)
    # adding a constant vector to every key shifts each row's logits by a constant
    assert np.abs(dK.sum(axis=2)).max() < 1e-12
    # rows of P sum to one, so the total value gradient is the total output gradient
    assert np.abs(dV.sum(axis=2) - c.do.astype(np.float64).sum(axis=2)).max() < 1e-12
    # each row of dS sums to zero, and log f_0 never reaches an output
    assert np.abs(dcq).max() < 1e-12
    assert np.abs(dlf[..., 0]).max() < 1e-12


# ---------------------------------------------------------------- planted mistakes are caught
MUTATIONS = {
    "bias_sign": ("(c_rows[:, None] - c_keys[None, :])", "(c_keys[None, :] - c_rows[:, None])"),
    "scaled_bias": ("s = scale * (q_rows @ k_keys.T) + (c_rows[:, None] - c_keys[None, :])",
                    "s = scale * (q_rows @ k_keys.T + (c_rows[:, None] - c_keys[None, :]))"),
    "mask_diagonal": ("s[j[None, :] > rows[:, None]] = -np.inf",
                      "s[j[None, :] >= rows[:, None]] = -1e30"),
    # (dropping dc^q is not a mistake in exact arithmetic: every row of dS sums to zero)
    "dck_sign": ("dlf = reverse_cumsum(dcq + dck)", "dlf = reverse_cumsum(dcq - dck)"),
    "exclusive_reverse_scan": ("dlf = reverse_cumsum(dcq + dck)",
                               "dlf = reverse_cumsum(dcq + dck) - (dcq + dck)"),
    "dk_transpose": ("dK[b, h, :i1] += scale * (dS.T @ q[b, h, i0:i1])",
                     "dK[b, h, :i1] += scale * (P.T @ q[b, h, i0:i1])"),
    "forward_scan": ("return np.flip(np.cumsum(np.flip(dc, axis=-1), axis=-1), axis=-1)",
                     "return np.cumsum(dc, axis=-1)"),
}


def _mutant(name):
    src = open(fox_oracle.__file__).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType("oracle_mutant_" + name)
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    return mod


def _pins_hold(mod):
    c = _case(B=1, H=2, L=48, D=16)
    s = 1 / math.sqrt(c.D)
    O, LSE = mod.attn_fwd(c.q, c.k, c.v, c.log_f, scale=s, block=16)
    O1, L1 = oracle.attn_fwd_bruteforce(c.q, c.k, c.v, c.log_f, s)
    if np.abs(O - O1).max() > 1e-10 or np.abs(LSE - L1).max() > 1e-10:
        return False
    got = mod.attn_bwd(c.q, c.k, c.v, c.log_f, c.do, scale=s, block=16)[:4]
    ref = _torch_grads(c, s)
    return all(np.abs(g - r).max() < 1e-9 for g, r in zip(got, ref))


def test_unmutated_oracle_passes_the_pin_harness():
    assert _pins_hold(fox_oracle)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    assert not _pins_hold(_mutant(name))


TAIL_MUTATIONS = {
    "tail_drops_dck": ("dc = dS.sum(axis=1) - dS[:, i0:].sum(axis=0)", "dc = dS.sum(axis=1)"),
    "tail_dk_unscaled": ("dK = scale * (dS[:, i0:].T @ qt)", "dK = dS[:, i0:].T @ qt"),
    "tail_dv_keys_shifted": ("dV = P[:, i0:].T @ dot", "dV = P[:, i0 - 1:-1].T @ dot"),
    "tail_row_term_unnormalised": ("P = p / ell[:, None]", "P = p"),
}


def _tail_pins_hold(mod):
    """The tail of a 40-position sequence (n = 9, with a reset inside it) against autograd."""
    c = _case(B=1, H=1, L=40, D=8, seed=73)
    c.log_f[0, 0, 35] = -30.0
    s = 0.4
    ref = _torch_grads(c, s)
    cc = oracle.cumsum_logf(c.log_f)[0, 0]
    try:
        got = mod.attn_bwd_tail(c.q[0, 0], c.k[0, 0], c.v[0, 0], cc, c.do[0, 0], 9, scale=s)
    except ValueError:
        return False
    return all(g.shape == r[0, 0, -9:].shape and np.abs(g - r[0, 0, -9:]).max() < 1e-9
               for g, r in zip(got[2:], ref))


def test_tail_pin_harness():
    assert _tail_pins_hold(fox_oracle)


@pytest.mark.parametrize("name", sorted(TAIL_MUTATIONS))
def test_planted_tail_mistake_is_caught(name):
    old, new = TAIL_MUTATIONS[name]
    src = open(fox_oracle.__file__).read()
    assert src.count(old) == 1, name
    mod = types.ModuleType("oracle_mutant_" + name)
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    assert not _tail_pins_hold(mod)


# ---------------------------------------------------------------- Pro block backward (gate, QK-norm)
def _pro_small(seed=11):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((2, 7, 24))
    w = 0.3 * rng.standard_normal((3, 24))
    b = rng.uniform(1, 6, size=3) * np.array([1.0, -1.0, 1.0])  # both signs of z
    g = rng.standard_normal((2, 3, 7))
    return x, w, b, g


def _fd_dir(f, args, which, u, h=1e-6):
    p = list(args)
    m = list(args)
    p[which] = args[which] + h * u
    m[which] = args[which] - h * u
    return (f(*p) - f(*m)) / (2 * h)


def _gate_pins_hold(mod):
    """Finite differences of sum(g * log f) for x, w_f, b_f, and torch autograd."""
    x, w, b, g = _pro_small()
    dx, dw, db = mod.gate_logf_bwd(x, w, b, g)
    loss = lambda x_, w_, b_: float(np.sum(g * oracle.gate_logf(x_, w_, b_)))
    rng = np.random.default_rng(5)
    for which, grad in enumerate((dx, dw, db)):
        for _ in range(2):
            u = rng.standard_normal(grad.shape)
            fd = _fd_dir(loss, (x, w, b), which, u)
            if abs(fd - float(np.sum(grad * u))) > 1e-7 * max(1.0, abs(fd)):
                return False
    xt, wt, bt = (_t(a).requires_grad_(True) for a in (x, w, b))
    z = torch.einsum("bld,hd->bhl", xt, wt) + bt[None, :, None]
    (F.logsigmoid(z) * _t(g)).sum().backward()
    return all(np.abs(a - r.grad.numpy()).max() < 1e-12 for a, r in ((dx, xt), (dw, wt), (db, bt)))


def _rms_pins_hold(mod):
    """Finite differences of sum(dy * rms_norm(x)) for x and the weights, and torch autograd."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 32)) * rng.uniform(0.1, 3.0, size=(5, 1))
    dy = rng.standard_normal((5, 32))
    wgt = rng.uniform(0.5, 1.5, size=32)
    for weight in (None, wgt):
        dx, dw = mod.rms_norm_bwd(x, dy, 1e-3, weight)
        loss = lambda x_, w_: float(np.sum(dy * oracle.rms_norm(x_, 1e-3, w_)))
        u = rng.standard_normal(x.shape)
        fd = _fd_dir(loss, (x, weight), 0, u)
        if abs(fd - float(np.sum(dx * u))) > 1e-7 * max(1.0, abs(fd)):
            return False
        if weight is not None:
            u = rng.standard_normal(32)
            fd = _fd_dir(loss, (x, weight), 1, u)
            if abs(fd - float(np.sum(dw * u))) > 1e-7 * max(1.0, abs(fd)):
                return False
    xt = _t(x).requires_grad_(True)
    wt = _t(wgt).requires_grad_(True)
    (F.rms_norm(xt, (32,), weight=wt, eps=1e-3) * _t(dy)).sum().backward()
    dx, dw = mod.rms_norm_bwd(x, dy, 1e-3, wgt)
    return np.abs(dx - xt.grad.numpy()).max() < 1e-12 and np.abs(dw - wt.grad.numpy()).max() < 1e-12


def test_gate_backward_pins():
    assert _gate_pins_hold(fox_oracle)


def test_rms_norm_backward_pins():
    assert _rms_pins_hold(fox_oracle)


def test_gate_backward_linear_and_zero():
    x, w, b, g = _pro_small()
    a = oracle.gate_logf_bwd(x, w, b, g)
    a2 = oracle.gate_logf_bwd(x, w, b, -2.5 * g)
    for p, q in zip(a, a2):
        assert np.abs(q + 2.5 * p).max() < 1e-12
    for z in oracle.gate_logf_bwd(x, w, b, 0 * g):
        assert np.abs(z).max() == 0.0


def test_rms_norm_backward_scale_invariance():
    """With eps = 0 and unit weights the output ignores the row's scale, so x . dx = 0."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((9, 64))
    dx, dw = oracle.rms_norm_bwd(x, rng.standard_normal((9, 64)), 0.0)
    assert dw is None
    assert np.abs(np.sum(x * dx, axis=-1)).max() < 1e-12


PRO_MUTATIONS = {
    "gate_sigmoid_sign": ("dz = g * np.exp(log_sigmoid(-z))", "dz = g * np.exp(log_sigmoid(z))"),
    "gate_dx_transpose": ('dx = np.einsum("bhl,hd->bld", dz, w_f)', 'dx = np.einsum("bhl,hd->bld", g, w_f)'),
    "gate_db_axis": ("db_f = dz.sum(axis=(0, 2))", "db_f = g.sum(axis=(0, 2))"),
    "rms_mean_term": ("dx = (g - xh * np.mean(g * xh, axis=-1, keepdims=True)) / r", "dx = g / r"),
    "rms_dw_unnormalised": ("dw = None if weight is None else (dy * xh).reshape(-1, x.shape[-1]).sum(axis=0)",
                            "dw = None if weight is None else (dy * x).reshape(-1, x.shape[-1]).sum(axis=0)"),
}


@pytest.mark.parametrize("name", sorted(PRO_MUTATIONS))
def test_planted_pro_backward_mistake_is_caught(name):
    src = open(fox_oracle.__file__).read()
    old, new = PRO_MUTATIONS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType("oracle_pro_mutant_" + name)
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    assert not (_gate_pins_hold(mod) and _rms_pins_hold(mod))


# ------------------------------------------------------------------------- exact tile skipping
# The skip bound is checked against brute force (it may never lie below the largest logit
# difference of a tile), against a construction where Cauchy-Schwarz is tight (it must equal
# it), against hand-derived plans for that construction, and against the real attention weights
# (every weight in a skipped tile is below the threshold).
def _skip_case(seed, L=150, D=8, lam=(5.0, 20.0), rising=False):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(1, 2, L, D)) * rng.uniform(0.5, 3.0, size=(1, 2, L, 1))
    k = rng.normal(size=(1, 2, L, D)) * rng.uniform(0.5, 3.0, size=(1, 2, L, 1))
    log_f = -rng.uniform(*lam, size=(1, 2, L)) * np.array([1.0, 0.05])[None, :, None]
    if rising:  # positive log f inside tiles: c rises there, so no tile end bounds its range
        for a in (21, 70, 103):
            log_f[..., a:a + 7] = rng.uniform(10.0, 40.0, size=(1, 2, 7))
    return q, k, log_f


def _exact_tile_max(q, k, c, scale, g):
    """max over each candidate tile of log2(e) (logit_ij - logit_ii), by brute force."""
    B, H, L, _ = q.shape
    diag = scale * np.einsum("bhld,bhld->bhl", q, k)
    lg = scale * np.einsum("bhid,bhjd->bhij", q, k) + c[..., :, None] - c[..., None, :]
    diff = (lg - diag[..., :, None]) * math.log2(math.e)
    n_qt, n_g, n_kb = -(-L // (4 * g)), -(-L // g), -(-L // (2 * g))
    fwd = np.full((B, H, n_qt, n_g), -np.inf)
    kv = np.full((B, H, n_kb, n_g), -np.inf)
    for t in range(n_qt):
        qa, qb = 4 * g * t, min(4 * g * t + 4 * g - 1, L - 1)
        for T in range(qb // g - 3):
            fwd[..., t, T] = diff[..., qa:qb + 1, g * T:g * T + g].max(axis=(-1, -2))
    for blk in range(n_kb):
        ka, kb = 2 * g * blk, min(2 * g * blk + 2 * g - 1, L - 1)
        for u in range(2, -(-(L - ka) // g)):
            qa = ka + g * u
            kv[..., blk, u] = diff[..., qa:min(qa + g, L), ka:kb + 1].max(axis=(-1, -2))
    return fwd, kv


def _tight_case(g=4, D=8, lam=20.0):
    """All queries a u, keys a u before row 4g and -a u from it on (u a unit vector), constant
    gate log f = -lam: for query rows >= 4g and keys < 4g, q_i.(k_j - k_i) = |q_i| (|k_j| + |k_i|)
    and the bound is attained at the tile's first query and last key."""
    L = 8 * g
    scale = 1.0 / math.sqrt(D)
    a = math.sqrt(10.0 / scale)  # scale a^2 = 10
    u = np.zeros(D)
    u[0] = 1.0
    q = np.broadcast_to(a * u, (1, 1, L, D)).copy()
    k = q.copy()
    k[..., 4 * g:, :] *= -1.0
    c = np.cumsum(np.full((1, 1, L), -lam), axis=-1)
    return q, k, c, scale


def _skip_pins_hold(mod):
    ok = True
    g = 4
    for seed in (1, 2, 3, 4, 5):
        q, k, log_f = _skip_case(seed, rising=seed > 3)
        c = np.cumsum(log_f, axis=-1)
        s = 1.0 / math.sqrt(q.shape[-1])
        fb, kb = mod.skip_bounds(q, k, c, scale=s, g=g)
        fe, ke = _exact_tile_max(q, k, c, s, g)
        ok &= bool(np.all(np.isfinite(fb) == np.isfinite(fe)))
        ok &= bool(np.all(np.isfinite(kb) == np.isfinite(ke)))
        ok &= bool(np.all(fb[np.isfinite(fb)] >= fe[np.isfinite(fe)] - 1e-9))
        ok &= bool(np.all(kb[np.isfinite(kb)] >= ke[np.isfinite(ke)] - 1e-9))
        # every weight of a skipped tile lies below the threshold
        q_skip, kv_tiles = mod.skip_plan(q, k, c, scale=s, threshold_log2=-60.0, g=g)
        n_full = -(-(150 - 8 * np.arange(kv_tiles.shape[-1])) // 4)  # tiles up to the end
        ok &= bool(q_skip.sum() > 0 and np.any(kv_tiles < n_full))  # the case does skip
        for h in range(2):
            P = fox_oracle.attn_probs_bruteforce(q[0, h], k[0, h], log_f[0, h], s)
            lp = np.log2(np.maximum(P, 1e-300))
            for t, n in enumerate(q_skip[0, h]):
                rows = slice(16 * t, min(16 * t + 16, 150))
                if n:
                    ok &= bool(lp[rows, :4 * n].max() < -60.0)
            for blk, n in enumerate(kv_tiles[0, h]):
                if 8 * blk + 4 * n < 150:
                    ok &= bool(lp[8 * blk + 4 * n:, 8 * blk:8 * blk + 8].max() < -60.0)
    # tight construction: equality, and the plans derived by hand. Bounds (log2 e times
    # 20 - lam (qa - kb)) put qa - kb >= 9 below -160 and qa - kb <= 5 above it.
    q, k, c, s = _tight_case(g=g)
    fb, kb = mod.skip_bounds(q, k, c, scale=s, g=g)
    fe, ke = _exact_tile_max(q, k, c, s, g)
    ok &= bool(np.allclose(fb[0, 0, 1, :4], fe[0, 0, 1, :4], rtol=0, atol=1e-9))
    ok &= bool(np.allclose(kb[0, 0, 0, 4:8], ke[0, 0, 0, 4:8], rtol=0, atol=1e-9))
    ok &= bool(np.allclose(kb[0, 0, 1, 2:6], ke[0, 0, 1, 2:6], rtol=0, atol=1e-9))
    q_skip, kv_tiles = mod.skip_plan(q, k, c, scale=s, g=g)
    ok &= q_skip[0, 0].tolist() == [0, 2]
    ok &= kv_tiles[0, 0].tolist() == [4, 4, 4, 2]
    # no decay: nothing is skipped
    q_skip, kv_tiles = mod.skip_plan(q, k, np.zeros_like(c), scale=s, g=g)
    ok &= q_skip[0, 0].tolist() == [0, 0] and kv_tiles[0, 0].tolist() == [8, 6, 4, 2]
    return ok


def test_skip_bound_pins():
    assert _skip_pins_hold(fox_oracle)


SKIP_MUTATIONS = {
    "skip_drop_diag_norm": ("(kn[..., T] + kdiag)", "(kn[..., T])"),
    "skip_largest_key_c": ("- (cmin[..., T] - cq))", "- (cmax[..., T] - cq))"),
    "skip_smallest_query_c": ("cq = cmax[..., groups].max(axis=-1)",
                              "cq = cmin[..., groups].min(axis=-1)"),
    "skip_tile_ends_only": ("- (cmin[..., T] - cq))", "- (c[..., g * T + g - 1] - c[..., qa]))"),
    "skip_kv_block_ends_only": ("- (ck - cmax[..., grp]))", "- (c[..., kb] - c[..., ka + g * u]))"),
    "skip_kv_walk_short": ("max(keep, default=1) + 1", "max(keep, default=1)"),
    "skip_prefix_too_long": ("while n < qb // g - 3 and fwd[b, h, t, n] < threshold_log2:",
                             "while n < qb // g - 3 and fwd[b, h, t, n] < threshold_log2 + 100:"),
}


@pytest.mark.parametrize("name", sorted(SKIP_MUTATIONS))
def test_planted_skip_mistake_is_caught(name):
    src = open(fox_oracle.__file__).read()
    old, new = SKIP_MUTATIONS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType("oracle_skip_mutant_" + name)
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    assert not _skip_pins_hold(mod)


# ------------------------------------------------------- Pro block: KV-shift and output norm + gate
# Forward pins: torch's sigmoid and matmul for the shift gate; special gate values where the
# shift is the identity, a pure one-position shift, or the mean of neighbours; the output gate
# saturated open (RMSNorm, pinned above against torch) and half open. Backward pins: central
# finite differences of the oracle's own forward, in every input.
def _pro_shift_pins_hold(mod):
    rng = np.random.default_rng(31)
    B, H, L, D, dm = 2, 3, 9, 8, 16
    x = rng.standard_normal((B, L, dm))
    w = rng.standard_normal((H, dm)) * 0.3
    a = mod.shift_gate(x, w)
    ref = torch.sigmoid(_t(x) @ _t(w).T).permute(0, 2, 1).numpy()
    if np.abs(a - ref).max() > 1e-14:
        return False
    da = rng.standard_normal((B, H, L))
    gx, gw = mod.shift_gate_bwd(x, w, da)
    loss = lambda x_, w_: float(np.sum(da * oracle.shift_gate(x_, w_)))
    for which, grad in ((0, gx), (1, gw)):
        u = rng.standard_normal(x.shape if which == 0 else w.shape)
        fd = _fd_dir(loss, (x, w), which, u)
        if abs(fd - float(np.sum(grad * u))) > 1e-7 * max(1.0, abs(fd)):
            return False
    xc = rng.standard_normal((B, H, L, D))
    zero, one = np.zeros((B, H, L)), np.ones((B, H, L))
    shifted = np.concatenate([np.zeros((B, H, 1, D)), xc[:, :, :-1]], axis=2)
    if not (np.allclose(mod.kv_shift(xc, zero), xc, rtol=0, atol=1e-15)
            and np.allclose(mod.kv_shift(xc, one), shifted, rtol=0, atol=1e-15)
            and np.allclose(mod.kv_shift(xc, one / 2), (xc + shifted) / 2, rtol=0, atol=1e-15)):
        return False
    dy = rng.standard_normal((B, H, L, D))
    al = rng.uniform(0.05, 0.95, size=(B, H, L))
    dx, da = mod.kv_shift_bwd(xc, al, dy)
    loss = lambda x_, a_: float(np.sum(dy * oracle.kv_shift(x_, a_)))
    for which, grad in ((0, dx), (1, da)):
        u = rng.standard_normal(xc.shape if which == 0 else al.shape)
        fd = _fd_dir(loss, (xc, al), which, u)
        if abs(fd - float(np.sum(grad * u))) > 1e-7 * max(1.0, abs(fd)):
            return False
    return True


def _pro_out_pins_hold(mod):
    rng = np.random.default_rng(32)
    o = rng.standard_normal((6, 16)) * rng.uniform(0.1, 3.0, size=(6, 1))
    g = rng.standard_normal((6, 16))
    wgt = rng.uniform(0.5, 1.5, size=16)
    for weight in (None, wgt):
        if not np.allclose(mod.out_norm_gate(o, np.full_like(g, 60.0), 1e-3, weight),
                           oracle.rms_norm(o, 1e-3, weight), rtol=1e-15, atol=1e-15):
            return False
        if not np.allclose(mod.out_norm_gate(o, np.zeros_like(g), 1e-3, weight),
                           0.5 * oracle.rms_norm(o, 1e-3, weight), rtol=1e-15, atol=1e-15):
            return False
        dy = rng.standard_normal(o.shape)
        do, dg = mod.out_norm_gate_bwd(o, g, 1e-3, dy, weight)
        loss = lambda o_, g_: float(np.sum(dy * oracle.out_norm_gate(o_, g_, 1e-3, weight)))
        for which, grad in ((0, do), (1, dg)):
            u = rng.standard_normal(o.shape)
            fd = _fd_dir(loss, (o, g), which, u)
            if abs(fd - float(np.sum(grad * u))) > 1e-7 * max(1.0, abs(fd)):
                return False
    return True


def test_pro_shift_and_output_pins():
    assert _pro_shift_pins_hold(fox_oracle)
    assert _pro_out_pins_hold(fox_oracle)


PRO2_MUTATIONS = {
    "shift_gate_sides_swapped": ("return a * prev + (1.0 - a) * x", "return (1.0 - a) * prev + a * x"),
    "shift_gate_bwd_derivative": ("dz = g * np.exp(log_sigmoid(z) + log_sigmoid(-z))",
                                  "dz = g * np.exp(log_sigmoid(-z))"),
    "shift_bwd_next_gate": ("(a[..., 1:, None] * g[..., 1:, :])", "(a[..., :-1, None] * g[..., 1:, :])"),
    "shift_bwd_dalpha_sign": ("da = np.sum(g * (prev - x), axis=-1)", "da = np.sum(g * (x - prev), axis=-1)"),
    "out_gate_derivative": ("dg = dy * n * s * np.exp(log_sigmoid(-gl))", "dg = dy * n * s"),
    "out_norm_bwd_ungated": ("do, _ = rms_norm_bwd(o, dy * s, eps, weight)", "do, _ = rms_norm_bwd(o, dy, eps, weight)"),
}


@pytest.mark.parametrize("name", sorted(PRO2_MUTATIONS))
def test_planted_pro_shift_output_mistake_is_caught(name):
    src = open(fox_oracle.__file__).read()
    old, new = PRO2_MUTATIONS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType("oracle_pro2_mutant_" + name)
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    assert not (_pro_shift_pins_hold(mod) and _pro_out_pins_hold(mod))

"""Pins of the fp64 oracle to facts other than itself.

Each ``pin_*`` function takes an :class:`oracle.Oracle` and raises
AssertionError when the oracle disagrees with what the pages and the
mathematics fix.  ``tests/test_oracle_pins.py`` runs them on the oracle;
``tests/test_oracle_mutations.py`` runs them on builds with planted mistakes
and requires every mistake to fail at least one pin.

Kinds of pin used (none re-types the oracle's own loops):
  * closed forms of special cases (identity and shift conv taps, beta = 0 pure
    decay, g = 0 / beta = 1 overwrite with orthonormal keys, constant-vector
    gated norm, tiny-vector L2 with eps);
  * exact rational brute force of the recurrence in its transition-product
    form S_t = S_{t-1} diag(a_t) (I - beta_t k k^T) + beta_t v k^T, a formula
    different from the oracle's decay/predict/write sequence;
  * invariants: chunked WY arm == token arm, split calls == one call, decode
    steps == prefill, per-channel decay with equal channels == scalar decay,
    linearity in v, packed varlen == separate sequences;
  * geometry printed by the golden PR (tests/golden/golden_pr_geometry.txt);
  * gates from the a / b projections: closed forms of softplus and the sigmoid at
    ln-rational points, the identities softplus(x) - softplus(-x) = x and
    sigmoid(x) + sigmoid(-x) = 1, and the far tails.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(got, want, tol, what):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    scale = max(1.0, float(np.max(np.abs(want))) if want.size else 1.0)
    err = float(np.max(np.abs(got - want))) if want.size else 0.0
    assert err <= tol * scale, f"{what}: max abs err {err:.3e} > {tol:.1e} * {scale:.3g}"


# ---------------------------------------------------------------------------
# conv (depthwise causal, width 4)
# ---------------------------------------------------------------------------

def pin_conv_identity_and_shift(orc):
    """Taps (0,0,0,1) give y = x; taps (1,0,0,0) give y_t = x_{t-3} with the
    three carried rows in front (catches the one-position shift fault named by
    the GLM ledger's conv slice)."""
    rng = np.random.default_rng(11)
    T, C = 7, 5
    x = rng.standard_normal((T, C))
    st = rng.standard_normal((1, 3, C))
    ident = np.tile([0.0, 0.0, 0.0, 1.0], (C, 1))
    y, so = orc.conv1d(x, ident, [0, T], st, act=0)
    assert np.array_equal(y, x), "identity taps must reproduce x exactly"
    assert np.array_equal(so[0], x[T - 3:]), "state out = last three inputs, oldest first"
    shift = np.tile([1.0, 0.0, 0.0, 0.0], (C, 1))
    y, _ = orc.conv1d(x, shift, [0, T], st, act=0)
    want = np.concatenate([st[0], x[: T - 3]], axis=0)
    assert np.array_equal(y, want), "taps (1,0,0,0) must delay by exactly three tokens"
    mid = np.tile([0.0, 1.0, 0.0, 0.0], (C, 1))
    y, _ = orc.conv1d(x, mid, [0, T], st, act=0)
    want = np.concatenate([st[0, 1:], x[: T - 2]], axis=0)
    assert np.array_equal(y, want), "taps (0,1,0,0) must delay by exactly two tokens"


def pin_conv_worked_example(orc):
    """Hand-computed single channel: x = 1..5, taps (1, -1, 2, 1/2), zero state.
    y0 = .5, y1 = 2 + 1 = 3, y2 = -1 + 4 + 1.5 = 4.5, y3 = 1 - 2 + 6 + 2 = 7,
    y4 = 2 - 3 + 8 + 2.5 = 9.5; state out (3, 4, 5)."""
    x = np.arange(1.0, 6.0).reshape(5, 1)
    w = np.array([[1.0, -1.0, 2.0, 0.5]])
    y, so = orc.conv1d(x, w, [0, 5], None, act=0)
    assert np.array_equal(y[:, 0], [0.5, 3.0, 4.5, 7.0, 9.5])
    assert np.array_equal(so[0, :, 0], [3.0, 4.0, 5.0])


def pin_conv_short_sequences_state(orc):
    """Sequences shorter than the window: the state out mixes carried rows and
    inputs; an empty sequence hands its state through unchanged."""
    C = 3
    st = np.arange(2 * 3 * C, dtype=np.float64).reshape(2, 3, C) + 100.0
    x = np.array([[1.0, 2.0, 3.0]])            # sequence 0 has 1 token, sequence 1 none
    ident = np.tile([0.0, 0.0, 0.0, 1.0], (C, 1))
    _, so = orc.conv1d(x, ident, [0, 1, 1], st, act=0)
    assert np.array_equal(so[0], np.stack([st[0, 1], st[0, 2], x[0]]))
    assert np.array_equal(so[1], st[1])


def pin_silu_closed_form(orc):
    """SiLU after the conv: act(0) = 0, act(1) = e/(e+1), act(-1) = -1/(e+1),
    act(30) = 30 - 30 e^-30 to fp64 precision (first term of the series)."""
    x = np.array([[0.0], [1.0], [-1.0], [30.0]])
    ident = np.array([[0.0, 0.0, 0.0, 1.0]])
    y, _ = orc.conv1d(x, ident, [0, 4], None, act=1)
    e = math.e
    want = [0.0, e / (e + 1.0), -1.0 / (e + 1.0), 30.0 - 30.0 * math.exp(-30.0)]
    _close(y[:, 0], want, 1e-15, "silu")


def pin_conv_step_equals_full(orc):
    """A conv step applied token by token equals the full conv (GLM ledger,
    conv slice), with and without SiLU; split calls carry the state."""
    rng = np.random.default_rng(12)
    T, C = 9, 6
    x = rng.standard_normal((T, C))
    w = 0.5 * rng.standard_normal((C, 4))
    st = rng.standard_normal((1, 3, C))
    for act in (0, 1):
        y_full, so_full = orc.conv1d(x, w, [0, T], st, act=act)
        state = st.copy()
        for t in range(T):
            y_t, state = orc.conv1d_step(x[t:t + 1], w, state, act=act)
            _close(y_t[0], y_full[t], 1e-15, f"step {t}")
        assert np.array_equal(state, so_full), "step state == prefill state out"
        y_a, so_a = orc.conv1d(x[:4], w, [0, 4], st, act=act)
        y_b, so_b = orc.conv1d(x[4:], w, [0, T - 4], so_a, act=act)
        assert np.array_equal(np.concatenate([y_a, y_b]), y_full)
        assert np.array_equal(so_b, so_full)


def pin_conv_varlen_isolation(orc):
    """Packed sequences never read each other's inputs."""
    rng = np.random.default_rng(13)
    C = 4
    lens = [5, 2, 7]
    x = rng.standard_normal((sum(lens), C))
    w = rng.standard_normal((C, 4))
    st = rng.standard_normal((3, 3, C))
    cu = np.concatenate([[0], np.cumsum(lens)])
    y, so = orc.conv1d(x, w, cu, st, act=1)
    for n in range(3):
        ys, ss = orc.conv1d(x[cu[n]:cu[n + 1]], w, [0, lens[n]], st[n:n + 1], act=1)
        assert np.array_equal(ys, y[cu[n]:cu[n + 1]])
        assert np.array_equal(ss[0], so[n])


# ---------------------------------------------------------------------------
# recurrence
# ---------------------------------------------------------------------------

def _rand_rule_inputs(rng, T, Hk, Hv, dk, dv, per_channel=False):
    q = rng.standard_normal((T, Hk, dk))
    k = rng.standard_normal((T, Hk, dk))
    v = rng.standard_normal((T, Hv, dv))
    gshape = (T, Hv, dk) if per_channel else (T, Hv)
    g = -np.logaddexp(0.0, -rng.standard_normal(gshape))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, Hv))))
    return q, k, v, g, beta


def pin_pure_decay(orc):
    """beta = 0: nothing is written, so S_t = exp(sum_{s<=t} g_s) S0 and
    o_t = S_t qtil_t (scalar and per-key-channel decay)."""
    rng = np.random.default_rng(21)
    T, Hk, Hv, d = 6, 1, 2, 8
    for per_channel in (False, True):
        q, k, v, g, _ = _rand_rule_inputs(rng, T, Hk, Hv, d, d, per_channel)
        beta = np.zeros((T, Hv))
        S0 = rng.standard_normal((1, Hv, d, d))
        o, sT = orc.delta_rule(q, k, v, g, beta, [0, T], S0, l2_eps=0.0)
        for h in range(Hv):
            for t in range(T):
                qn = q[t, 0] / np.linalg.norm(q[t, 0]) / math.sqrt(d)
                if per_channel:
                    decay = np.exp(g[: t + 1, h].sum(axis=0))          # [dk]
                    want = S0[0, h] @ (decay * qn)
                else:
                    want = math.exp(g[: t + 1, h].sum()) * (S0[0, h] @ qn)
                _close(o[t, h], want, 1e-13, f"pure decay o t={t} h={h}")
            if per_channel:
                want_s = S0[0, h] * np.exp(g[:, h].sum(axis=0))[None, :]
            else:
                want_s = math.exp(g[:, h].sum()) * S0[0, h]
            _close(sT[0, h], want_s, 1e-13, "pure decay final state")


def pin_overwrite_orthonormal(orc):
    """g = 0, beta = 1, one-hot keys: each token overwrites column pi(t) of S
    with v_t and leaves the others; reading with q = e_j returns column j
    scaled by 1/sqrt(dk)."""
    rng = np.random.default_rng(22)
    d, T = 8, 5
    perm = [3, 0, 6, 3, 1]                      # column 3 written twice
    k = np.zeros((T, 1, d))
    for t, j in enumerate(perm):
        k[t, 0, j] = 2.5                         # normalises to exactly e_j
    q = np.zeros((T, 1, d))
    reads = [3, 0, 6, 5, 3]
    for t, j in enumerate(reads):
        q[t, 0, j] = 0.75
    v = rng.standard_normal((T, 1, d))
    g = np.zeros((T, 1))
    beta = np.ones((T, 1))
    S0 = rng.standard_normal((1, 1, d, d))
    o, sT = orc.delta_rule(q, k, v, g, beta, [0, T], S0, l2_eps=0.0)
    S = S0[0, 0].copy()
    for t in range(T):
        S[:, perm[t]] = v[t, 0]
        _close(o[t, 0], S[:, reads[t]] / math.sqrt(d), 1e-14, f"overwrite read t={t}")
    _close(sT[0, 0], S, 1e-14, "overwrite final state")


def _frac_vec(xs):
    return [Fraction(x) for x in xs]


def _brute_force(S0, steps, per_channel):
    """Exact transition-product form in rationals.  steps: (a, beta, k, v, q) with
    a a scalar or a per-channel list; k, q unit vectors; returns outputs and S."""
    dv, dk = len(S0), len(S0[0])
    S = [row[:] for row in S0]
    outs = []
    for a, beta, k, v, q in steps:
        avec = a if per_channel else [a] * dk
        # M = diag(a) (I - beta k k^T)
        M = [[avec[i] * ((1 if i == j else 0) - beta * k[i] * k[j]) for j in range(dk)]
             for i in range(dk)]
        S = [[sum(S[r][m] * M[m][c] for m in range(dk)) + beta * v[r] * k[c] for c in range(dk)]
             for r in range(dv)]
        half = Fraction(1, 2)                    # q scale 1/sqrt(4)
        outs.append([sum(S[r][c] * q[c] for c in range(dk)) * half for r in range(dv)])
    return outs, S


def pin_brute_force_rational(orc):
    """1 head, dk = dv = 4, decay in {1, 1/2, 1/4}, beta in {1, 1/2, 1/4},
    Pythagorean unit keys: the fp64 oracle equals the exact rational
    transition-product form to 1e-14 (scalar and per-channel decay)."""
    units = [
        _frac_vec([Fraction(3, 5), Fraction(4, 5), 0, 0]),
        _frac_vec([0, 0, Fraction(3, 5), Fraction(4, 5)]),
        _frac_vec([Fraction(1, 2)] * 4),
        _frac_vec([Fraction(1, 2), Fraction(-1, 2), Fraction(1, 2), Fraction(-1, 2)]),
        _frac_vec([Fraction(2, 3), Fraction(2, 3), Fraction(1, 3), 0]),
        _frac_vec([0, Fraction(4, 5), 0, Fraction(-3, 5)]),
    ]
    S0 = [[Fraction(i - 2 * j, 4) for j in range(4)] for i in range(4)]
    vs = [_frac_vec(r) for r in ([1, -2, 3, 0], [Fraction(1, 2), 0, -1, 2], [2, 2, -1, 1],
                                 [0, 1, 0, -3], [-1, Fraction(3, 2), 1, 0])]
    betas = [Fraction(1), Fraction(1, 2), Fraction(1, 4), Fraction(1, 2), Fraction(1)]
    a_scalar = [Fraction(1), Fraction(1, 2), Fraction(1, 4), Fraction(1, 2), Fraction(1)]
    a_chan = [[Fraction(1), Fraction(1, 2), Fraction(1, 4), Fraction(1)],
              [Fraction(1, 2)] * 4,
              [Fraction(1, 4), Fraction(1), Fraction(1, 2), Fraction(1, 2)],
              [Fraction(1), Fraction(1), Fraction(1, 4), Fraction(1, 2)],
              [Fraction(1, 2), Fraction(1, 4), Fraction(1), Fraction(1)]]
    kidx = [0, 2, 3, 4, 1]
    qidx = [2, 5, 0, 1, 3]
    T = len(betas)
    for per_channel in (False, True):
        a_list = a_chan if per_channel else a_scalar
        steps = [(a_list[t], betas[t], units[kidx[t]], vs[t], units[qidx[t]]) for t in range(T)]
        outs, S = _brute_force(S0, steps, per_channel)
        q = np.array([[[float(x) for x in units[qidx[t]]]] for t in range(T)])
        k = np.array([[[float(x) for x in units[kidx[t]]]] for t in range(T)])
        v = np.array([[[float(x) for x in vs[t]]] for t in range(T)])
        if per_channel:
            g = np.log(np.array([[[float(x) for x in a_list[t]]] for t in range(T)]))
        else:
            g = np.log(np.array([[float(a_list[t])] for t in range(T)]))
        beta = np.array([[float(b)] for b in betas])
        S0f = np.array([[[[float(x) for x in row] for row in S0]]])
        o, sT = orc.delta_rule(q, k, v, g, beta, [0, T], S0f, l2_eps=0.0)
        want_o = np.array([[[float(x) for x in outs[t]]] for t in range(T)])
        _close(o, want_o, 1e-14, f"brute force outputs (per_channel={per_channel})")
        _close(sT[0, 0], np.array([[float(x) for x in row] for row in S]), 1e-14,
               f"brute force state (per_channel={per_channel})")


def pin_worked_example_2x2(orc):
    """Hand-computed dk = dv = 2, q scale 1, eps 0.  S0 = [[1,0],[0,2]].
    Token 1: a = 1/2, beta = 1/2, k = (3,4) -> (3/5,4/5), v = (1,-1), q = (0,2) -> (0,1).
      decayed S = [[1/2,0],[0,1]]; p = (3/10, 4/5); u = (7/20, -9/10);
      S = [[71/100, 7/25], [-27/50, 7/25]]; o = (7/25, 7/25).
    Token 2: a = 1, beta = 1, k = (0,-1), v = (2,0), q = (1,0).
      p = (-7/25, -7/25); u = (57/25, 7/25); S = [[71/100, -2], [-27/50, 0]];
      o = (71/100, -27/50)."""
    q = np.array([[[0.0, 2.0]], [[1.0, 0.0]]])
    k = np.array([[[3.0, 4.0]], [[0.0, -1.0]]])
    v = np.array([[[1.0, -1.0]], [[2.0, 0.0]]])
    g = np.log(np.array([[0.5], [1.0]]))
    beta = np.array([[0.5], [1.0]])
    S0 = np.array([[[[1.0, 0.0], [0.0, 2.0]]]])
    o, sT = orc.delta_rule(q, k, v, g, beta, [0, 2], S0, l2_eps=0.0, q_scale=1.0)
    _close(o[:, 0], [[7 / 25, 7 / 25], [71 / 100, -27 / 50]], 1e-15, "worked example outputs")
    _close(sT[0, 0], [[71 / 100, -2.0], [-27 / 50, 0.0]], 1e-15, "worked example state")


def pin_l2_eps_and_scale(orc):
    """Single token from a zero state with g = 0, beta = 1 and q = k: the
    output is v * scale * |k|^2 / (|k|^2 + eps).  A large key gives v/sqrt(dk)
    (catches an RMS norm, which is sqrt(dk) larger, and a missing q scale); a
    key of norm 1e-4 with eps = 1e-6 gives v/sqrt(dk)/101 (catches max(norm,eps))."""
    d = 16
    rng = np.random.default_rng(23)
    v = rng.standard_normal((1, 1, d))
    for norm, eps in ((3.0, 0.0), (3.0, 1e-6), (1e-4, 1e-6)):
        k = rng.standard_normal((1, 1, d))
        k *= norm / np.linalg.norm(k)
        o, _ = orc.delta_rule(k.copy(), k, v, np.zeros((1, 1)), np.ones((1, 1)), [0, 1], None,
                              l2_eps=eps)
        ss = norm * norm
        want = v[0, 0] / math.sqrt(d) * ss / (ss + eps)
        _close(o[0, 0], want, 1e-13, f"l2 norm={norm} eps={eps}")


def pin_l2norm_off_takes_keys_as_given(orc):
    """qk_l2norm = 0 (the L2 stage bound outside the call) uses q and k as given: fed the
    unit-normalised rows it reproduces the qk_l2norm = 1 result (eps 0); fed the raw rows of
    norm c it differs (beta k k^T grows as c^2), and on a single token from a zero state with
    g = 0, beta = 1 and q = k it gives v * scale * |k|^2 (the closed form without the division)."""
    rng = np.random.default_rng(41)
    T, hk, hv, d = 9, 2, 4, 8
    q = rng.standard_normal((T, hk, d))
    k = rng.standard_normal((T, hk, d))
    v = rng.standard_normal((T, hv, d))
    g = -np.abs(rng.standard_normal((T, hv))) * 0.3
    beta = rng.random((T, hv))
    s0 = rng.standard_normal((1, hv, d, d)) * 0.1
    o1, s1 = orc.delta_rule(q, k, v, g, beta, [0, T], s0, l2_eps=0.0)
    qu = q / np.linalg.norm(q, axis=-1, keepdims=True)
    ku = k / np.linalg.norm(k, axis=-1, keepdims=True)
    o0, s0_ = orc.delta_rule(qu, ku, v, g, beta, [0, T], s0, l2norm=0, l2_eps=0.0)
    _close(o0, o1, 1e-12, "l2norm=0 on unit rows == l2norm=1")
    _close(s0_, s1, 1e-12, "l2norm=0 on unit rows == l2norm=1 (state)")
    o2, _ = orc.delta_rule(q, k, v, g, beta, [0, T], s0, l2norm=0, l2_eps=0.0)
    assert np.max(np.abs(o2 - o1)) > 1e-3, "l2norm=0 must not normalise"
    kk = rng.standard_normal((1, 1, d)) * 2.0
    vv = rng.standard_normal((1, 1, d))
    o3, _ = orc.delta_rule(kk.copy(), kk, vv, np.zeros((1, 1)), np.ones((1, 1)), [0, 1], None, l2norm=0)
    _close(o3[0, 0], vv[0, 0] / math.sqrt(d) * float(np.sum(kk * kk)), 1e-12, "l2norm=0 closed form")


def pin_head_repeat_interleave(orc):
    """Value head h reads key head h // (Hv/Hk): running each value head alone
    with its key head reproduces the packed multi-head result."""
    rng = np.random.default_rng(24)
    T, Hk, Hv, d = 5, 2, 6, 8
    q, k, v, g, beta = _rand_rule_inputs(rng, T, Hk, Hv, d, d)
    S0 = 0.1 * rng.standard_normal((1, Hv, d, d))
    o, sT = orc.delta_rule(q, k, v, g, beta, [0, T], S0)
    for h in range(Hv):
        kh = h // (Hv // Hk)
        o1, s1 = orc.delta_rule(q[:, kh:kh + 1], k[:, kh:kh + 1], v[:, h:h + 1], g[:, h:h + 1],
                                beta[:, h:h + 1], [0, T], S0[:, h:h + 1])
        assert np.array_equal(o1[:, 0], o[:, h]), f"head {h} must read key head {kh}"
        assert np.array_equal(s1[0, 0], sT[0, h])


def pin_linearity_in_v(orc):
    """From a zero state the outputs are linear in v."""
    rng = np.random.default_rng(25)
    T, d = 7, 8
    q, k, v1, g, beta = _rand_rule_inputs(rng, T, 1, 1, d, d)
    v2 = rng.standard_normal(v1.shape)
    o1, _ = orc.delta_rule(q, k, v1, g, beta, [0, T])
    o2, _ = orc.delta_rule(q, k, v2, g, beta, [0, T])
    o3, _ = orc.delta_rule(q, k, v1 + 2.0 * v2, g, beta, [0, T])
    _close(o3, o1 + 2.0 * o2, 1e-13, "linearity")


def pin_per_channel_equal_is_scalar(orc):
    """Per-key-channel decay with all channels equal is the scalar-decay rule."""
    rng = np.random.default_rng(26)
    T, Hk, Hv, d = 9, 1, 3, 8
    q, k, v, g, beta = _rand_rule_inputs(rng, T, Hk, Hv, d, d)
    S0 = 0.1 * rng.standard_normal((1, Hv, d, d))
    o1, s1 = orc.delta_rule(q, k, v, g, beta, [0, T], S0)
    gc = np.repeat(g[:, :, None], d, axis=2)
    o2, s2 = orc.delta_rule(q, k, v, gc, beta, [0, T], S0)
    _close(o2, o1, 1e-15, "per-channel equal outputs")
    _close(s2, s1, 1e-15, "per-channel equal state")


def pin_chunked_equals_sequential(orc):
    """The chunked WY arm equals the token arm at lengths around the chunk
    boundary (GLM ledger prefill slice: 63/64/65), scalar and per-channel."""
    rng = np.random.default_rng(27)
    Hk, Hv, d = 1, 2, 16
    for per_channel in (False, True):
        for T in (1, 63, 64, 65, 127, 128, 129):
            q, k, v, g, beta = _rand_rule_inputs(rng, T, Hk, Hv, d, d, per_channel)
            S0 = 0.1 * rng.standard_normal((1, Hv, d, d))
            o1, s1 = orc.delta_rule(q, k, v, g, beta, [0, T], S0)
            o2, s2 = orc.delta_rule(q, k, v, g, beta, [0, T], S0, chunk=64)
            _close(o2, o1, 1e-12, f"chunked o T={T} pc={per_channel}")
            _close(s2, s1, 1e-12, f"chunked state T={T} pc={per_channel}")


def pin_state_carry_and_varlen(orc):
    """Split calls carrying the state equal one call; packed sequences equal
    separate calls (each with its own initial state)."""
    rng = np.random.default_rng(28)
    Hk, Hv, d = 1, 3, 8
    T = 20
    q, k, v, g, beta = _rand_rule_inputs(rng, T, Hk, Hv, d, d)
    S0 = 0.1 * rng.standard_normal((1, Hv, d, d))
    o, s = orc.delta_rule(q, k, v, g, beta, [0, T], S0)
    oa, sa = orc.delta_rule(q[:8], k[:8], v[:8], g[:8], beta[:8], [0, 8], S0)
    ob, sb = orc.delta_rule(q[8:], k[8:], v[8:], g[8:], beta[8:], [0, T - 8], sa)
    assert np.array_equal(np.concatenate([oa, ob]), o)
    assert np.array_equal(sb, s)
    S2 = 0.1 * rng.standard_normal((2, Hv, d, d))
    op, sp = orc.delta_rule(q, k, v, g, beta, [0, 8, T], S2)
    o0, s0 = orc.delta_rule(q[:8], k[:8], v[:8], g[:8], beta[:8], [0, 8], S2[:1])
    o1, s1 = orc.delta_rule(q[8:], k[8:], v[8:], g[8:], beta[8:], [0, T - 8], S2[1:])
    assert np.array_equal(op, np.concatenate([o0, o1]))
    assert np.array_equal(sp, np.concatenate([s0, s1]))


# ---------------------------------------------------------------------------
# gated RMSNorm (sigmoid gate)
# ---------------------------------------------------------------------------

def pin_gated_norm_closed_forms(orc):
    """o = (3, 4), w = (1, 2), z = (0, ln 3): mean square 12.5, sigmoid gates
    1/2 and 3/4, out = (3 sqrt2/10, 6 sqrt2/5).  A constant vector c*1 with
    eps = 0 gives sign(c) w sigmoid(z); with c = 1e-3 and eps = 1e-6 it gives
    w sigmoid(z) / sqrt(2) (eps inside the root).  Scaling o leaves the output."""
    out = orc.gated_rmsnorm([[3.0, 4.0]], [[0.0, math.log(3.0)]], [1.0, 2.0], eps=0.0)
    _close(out[0], [3 * math.sqrt(2) / 10, 6 * math.sqrt(2) / 5], 1e-15, "norm worked example")
    rng = np.random.default_rng(31)
    d = 16
    z = rng.standard_normal((1, d))
    w = 1 + 0.1 * rng.standard_normal(d)
    sig = 1 / (1 + np.exp(-z[0]))
    out = orc.gated_rmsnorm(np.full((1, d), -2.5), z, w, eps=0.0)
    _close(out[0], -w * sig, 1e-15, "constant vector")
    out = orc.gated_rmsnorm(np.full((1, d), 1e-3), z, w, eps=1e-6)
    _close(out[0], w * sig / math.sqrt(2.0), 1e-12, "eps inside the root")
    o = rng.standard_normal((3, d))
    a = orc.gated_rmsnorm(o, np.tile(z, (3, 1)), w, eps=0.0)
    b = orc.gated_rmsnorm(7.0 * o, np.tile(z, (3, 1)), w, eps=0.0)
    _close(a, b, 1e-14, "scale invariance")


# ---------------------------------------------------------------------------
# composition: decode steps == prefill (chunk/decode equivalence)
# ---------------------------------------------------------------------------

def pin_decode_equals_prefill(orc):
    """T fused decode steps reproduce the prefill path over the same T tokens
    (conv state, recurrent state and gated-norm output), which the TDD ledger's
    method names as the GDN localisation step."""
    rng = np.random.default_rng(41)
    Hk, Hv, d, T = 2, 6, 8, 6
    C = 2 * Hk * d + Hv * d
    x = rng.standard_normal((T, C))
    w = 0.5 * rng.standard_normal((C, 4))
    cs = rng.standard_normal((1, 3, C))
    g = -np.logaddexp(0.0, -rng.standard_normal((T, Hv)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, Hv))))
    z = rng.standard_normal((T, Hv, d))
    nw = 1 + 0.1 * rng.standard_normal(d)
    S0 = 0.1 * rng.standard_normal((1, Hv, d, d))
    out, o, sT, csT, _ = orc.prefill(x, w, [0, T], g, beta, z, nw, Hk=Hk, Hv=Hv, dk=d, dv=d,
                                     conv_state_in=cs, state_in=S0)
    c_state, s_state = cs.copy(), S0.copy()
    for t in range(T):
        ot, c_state, s_state = orc.decode_step(x[t:t + 1], w, c_state, g[t:t + 1], beta[t:t + 1],
                                               z[t:t + 1], nw, s_state, Hk=Hk, Hv=Hv, dk=d, dv=d)
        _close(ot[0], out[t], 1e-13, f"decode step {t}")
    _close(s_state, sT, 1e-13, "decode final state")
    assert np.array_equal(c_state, csT), "decode conv state == prefill conv state"


def pin_verify_transaction_equals_prefill(orc):
    """A verify of K rows per sequence and a commit of c of them reproduce the prefill path
    over each sequence's first c tokens (outputs for every verified row, and both states),
    with c = 0 (abort: the prior states bit for bit), a middle prefix and all K rows; the
    verify leaves its inputs unchanged."""
    rng = np.random.default_rng(43)
    Hk, Hv, d, B, K = 2, 6, 8, 3, 4
    C = 2 * Hk * d + Hv * d
    x = rng.standard_normal((B, K, C))
    w = 0.5 * rng.standard_normal((C, 4))
    cs = rng.standard_normal((B, 3, C))
    g = -np.logaddexp(0.0, -rng.standard_normal((B, K, Hv)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, K, Hv))))
    z = rng.standard_normal((B, K, Hv, d))
    nw = 1 + 0.1 * rng.standard_normal(d)
    S0 = 0.1 * rng.standard_normal((B, Hv, d, d))
    cs_keep, S0_keep = cs.copy(), S0.copy()
    out, snaps = orc.verify(x, w, cs, g, beta, z, nw, S0, Hk=Hk, Hv=Hv, dk=d, dv=d)
    assert np.array_equal(cs, cs_keep) and np.array_equal(S0, S0_keep), "verify must not touch its inputs"
    accepted = [0, 2, K]
    cs_c, st_c = orc.commit(snaps, accepted)
    for b, c in enumerate(accepted):
        ref_out, _, ref_s, ref_cs, _ = orc.prefill(x[b], w, [0, K], g[b], beta[b], z[b], nw, Hk=Hk, Hv=Hv,
                                                   dk=d, dv=d, conv_state_in=cs[b:b + 1], state_in=S0[b:b + 1])
        _close(out[b], ref_out, 1e-13, f"verified rows of sequence {b}")
        if c == 0:
            assert np.array_equal(st_c[b], S0[b]) and np.array_equal(cs_c[b], cs[b]), "abort keeps the prior states"
            continue
        _, _, pre_s, pre_cs, _ = orc.prefill(x[b, :c], w, [0, c], g[b, :c], beta[b, :c], z[b, :c], nw, Hk=Hk,
                                             Hv=Hv, dk=d, dv=d, conv_state_in=cs[b:b + 1], state_in=S0[b:b + 1])
        _close(st_c[b], pre_s[0], 1e-13, f"committed state, {c} rows")
        assert np.array_equal(cs_c[b], pre_cs[0]), f"committed conv state, {c} rows"
        if c == K:
            _close(st_c[b], ref_s[0], 1e-13, "commit of every row == prefill final state")


# ---------------------------------------------------------------------------
# geometry the golden PR prints
# ---------------------------------------------------------------------------

# ---------------------------------------------------------------------------
# gates from the a / b projections
# ---------------------------------------------------------------------------

def pin_gates_closed_forms(orc):
    """Points where softplus and the sigmoid have closed forms: softplus(0) = ln 2,
    softplus(ln 3) = ln 4, softplus(-ln 3) = ln(4/3); sigmoid(0) = 1/2, sigmoid(+-ln 3) =
    3/4, 1/4.  Head 1 has A_log = ln 5 (g scales by 5), head 2 has dt_bias = ln 3 (it
    shifts a), so a dropped exp, a dropped or negated bias and a sign slip each miss."""
    ln3 = math.log(3.0)
    A_log = np.array([0.0, math.log(5.0), 0.0])
    dt_bias = np.array([0.0, 0.0, ln3])
    a = np.array([[0.0, ln3, -2.0 * ln3]])
    b = np.array([[0.0, ln3, -ln3]])
    g, beta = orc.gates(a, b, A_log, dt_bias)
    _close(g, [[-math.log(2.0), -5.0 * math.log(4.0), -math.log(4.0 / 3.0)]], 1e-14, "g closed forms")
    _close(beta, [[0.5, 0.75, 0.25]], 1e-14, "beta closed forms")


def pin_gates_identities_and_tails(orc):
    """softplus(x) - softplus(-x) = x and sigmoid(x) + sigmoid(-x) = 1 on random points;
    far tails: softplus(40) = 40 + e^-40, softplus(-40) = e^-40 (relative), so a ReLU or
    an exp in place of softplus fails; g <= 0 everywhere and heads are not mixed up."""
    rng = np.random.default_rng(23)
    Hv = 4
    A_log = rng.uniform(0.0, 2.7, Hv)
    dt_bias = rng.uniform(-4.0, 1.0, Hv)
    x = rng.standard_normal((9, Hv)) * 3.0
    g_pos, b_pos = orc.gates(x - dt_bias, x, A_log, dt_bias)
    g_neg, b_neg = orc.gates(-x - dt_bias, -x, A_log, dt_bias)
    A = np.exp(A_log)
    _close((g_neg - g_pos) / A, x, 1e-13, "softplus(x) - softplus(-x) = x")
    _close(b_pos + b_neg, np.ones_like(x), 1e-14, "sigmoid(x) + sigmoid(-x) = 1")
    assert np.all(g_pos <= 0.0) and np.all(g_neg <= 0.0), "g must be a log decay (<= 0)"
    tail = np.array([[40.0, -40.0, 0.0, 0.0]])
    g, _ = orc.gates(tail - dt_bias, np.zeros((1, Hv)), A_log, dt_bias)
    assert abs(g[0, 0] / -(A[0] * (40.0 + math.exp(-40.0))) - 1.0) < 1e-14, "softplus(40)"
    assert abs(g[0, 1] / -(A[1] * math.exp(-40.0)) - 1.0) < 1e-12, "softplus(-40) = e^-40 (relative)"
    _close(g[0, 2:], -A[2:] * math.log(2.0), 1e-14, "per-head A at softplus(0)")


def pin_round_f16_ieee_half(orc):
    """The fp16 rounding step at IEEE half facts: 1 + 2^-11 is a tie and goes to 1 (even),
    1 + 3 * 2^-11 goes up to 1 + 2^-9, 65504 is the largest finite half, 2^-24 the smallest
    subnormal and 2^-26 rounds to zero."""
    import oracle as oracle_pkg
    got = oracle_pkg.round_f16([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 65504.0, 2.0 ** -24, 2.0 ** -26, -1.5])
    assert np.array_equal(got, [1.0, 1 + 2.0 ** -9, 65504.0, 2.0 ** -24, 0.0, -1.5])


def read_golden_geometry():
    cases = {}
    path = os.path.join(GOLDEN, "golden_pr_geometry.txt")
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            fields = dict(tok.split("=") for tok in line.split())
            cases[int(fields["S"])] = {k: float(v) for k, v in fields.items() if k != "S"}
    return cases


def pin_golden_pr_geometry(orc):
    """The measured table of the golden PR counts, per case, the elements of
    the gated-norm output (its out-of-bound denominators), the chunks run, and
    in the tolerance derivation the conv-leg elements over all cases (2.9M).
    The oracle's prefill at the pages' geometry (16 K / 48 V heads of 128,
    conv 4) must produce outputs of exactly those sizes."""
    cases = read_golden_geometry()
    Hk, Hv, d = 16, 48, 128
    C = 2 * Hk * d + Hv * d
    total_conv = 0
    for S, fields in sorted(cases.items()):
        rng = np.random.default_rng(S)
        x = rng.standard_normal((S, C))
        w = 0.5 * rng.standard_normal((C, 4))
        g = -np.logaddexp(0.0, -rng.standard_normal((S, Hv)))
        beta = 1 / (1 + np.exp(-rng.standard_normal((S, Hv))))
        z = rng.standard_normal((S, Hv, d))
        nw = np.ones(d)
        if S > 16:        # the full path is exercised once; the rest checks shapes only
            assert (S * Hv * d) == int(fields["elements"])
            total_conv += S * C
            assert math.ceil(S / 64) == int(fields["chunks"])
            continue
        out, o, sT, cso, y = orc.prefill(x, w, [0, S], g, beta, z, nw, Hk=Hk, Hv=Hv, dk=d, dv=d)
        assert out.size == int(fields["elements"]), f"S={S}: output elements"
        assert math.ceil(S / 64) == int(fields["chunks"])
        assert np.all(np.isfinite(out))
        total_conv += y.size
    assert round(total_conv / 1e6, 1) == 2.9, f"conv-leg elements {total_conv}"


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]

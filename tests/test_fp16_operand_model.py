"""CPU check of the precision budget behind the register-resident chunk spines.

Those spines round every operand of the state and output products -- the
normalised key and query rows, the chunk-start state, R, Vnew, c Vnew, Tt and
Pt -- once to fp16 and accumulate in fp32, with the state itself kept in fp32
between chunks.  This test writes that chunk form in numpy (fp64 arithmetic,
each operand rounded to fp16 where the kernels round it; the per-chunk solve
and the Gram products exact) and checks it against the fp64 oracle on the
workload's distributions, at a length that crosses several chunks, with and
without decay: the rounding alone must stay well inside the 2e-3 max-relative
bound the GPU parity tests hold the library to.  It also checks that rounding
the same operands to bf16 instead would not (the reason for fp16).  Test
infrastructure only: nothing here runs on or is used by the library.
"""
import numpy as np

import gdn_inputs as gi
import oracle

T = 512
HEADS = (0, 40)


def _f16(x):
    return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def _bf16(x):
    return oracle.round_bf16(x)


def _chunked(q, k, v, g, beta, s0, rnd, L=64, eps=1e-6):
    """One value head: q, k [T, dk], v [T, dv], g, beta [T], s0 [dv, dk] -> (o, S)."""
    dk = k.shape[1]
    rk = 1.0 / np.sqrt((k * k).sum(1) + eps)
    rq = (1.0 / np.sqrt(dk)) / np.sqrt((q * q).sum(1) + eps)
    S = s0.astype(np.float64).copy()
    o = np.zeros((len(k), v.shape[1]))
    for c0 in range(0, len(k), L):
        c1 = min(len(k), c0 + L)
        n = c1 - c0
        K, Q, V = k[c0:c1], q[c0:c1], v[c0:c1]
        gam = np.cumsum(g[c0:c1])
        b = beta[c0:c1]
        D = np.exp(gam[:, None] - gam[None, :])
        A = np.tril(np.ones((n, n)), -1) * (b[:, None] * D * rk[c0:c1, None] * rk[None, c0:c1] * (K @ K.T))
        Tt = np.linalg.solve(np.eye(n) + A, np.diag(b))
        Pt = np.tril(np.ones((n, n))) * (rq[c0:c1, None] * rk[None, c0:c1] * D * (Q @ K.T))
        kh, qh = rnd(K * rk[c0:c1, None]), rnd(Q * rq[c0:c1, None])
        eg = np.exp(gam)
        Sr = rnd(S)
        R = V - eg[:, None] * (kh @ Sr.T)
        Vn = rnd(Tt) @ rnd(R)
        o[c0:c1] = eg[:, None] * (qh @ Sr.T) + rnd(Pt) @ rnd(Vn)
        W = np.exp(gam[-1] - gam)[:, None] * Vn
        S = np.exp(gam[-1]) * S + rnd(W).T @ kh
    return o, S


def _errors(decay):
    d = gi.gen_prefill(11, [T])
    orc = oracle.Oracle()
    y, _ = orc.conv1d(d["x"], d["conv_w"], d["cu"], None, act=1)
    y = oracle.round_bf16(y)
    hkd = gi.HK * gi.DK
    q = y[:, :hkd].reshape(T, gi.HK, gi.DK)
    k = y[:, hkd:2 * hkd].reshape(T, gi.HK, gi.DK)
    v = y[:, 2 * hkd:].reshape(T, gi.HV, gi.DV)
    g = d["g"] if decay else np.zeros_like(d["g"])
    o_ref, s_ref = orc.delta_rule(q, k, v, g, d["beta"], d["cu"], d["state_in"])
    out = {}
    for name, rnd in (("f16", _f16), ("bf16", _bf16)):
        eo = es = 0.0
        for h in HEADS:
            o, S = _chunked(q[:, h // 3], k[:, h // 3], v[:, h], g[:, h].astype(np.float64),
                            d["beta"][:, h].astype(np.float64), d["state_in"][0, h], rnd)
            eo = max(eo, np.abs(o - o_ref[:, h]).max() / np.abs(o_ref[:, h]).max())
            es = max(es, np.abs(S - s_ref[0, h]).max() / np.abs(s_ref[0, h]).max())
        out[name] = (eo, es)
    return out


def test_fp16_operands_within_bound_with_decay():
    e = _errors(decay=True)
    assert max(e["f16"]) < 1.2e-3, e
    assert max(e["bf16"]) > 2e-3, e


def test_fp16_operands_within_bound_without_decay():
    e = _errors(decay=False)
    assert max(e["f16"]) < 1.2e-3, e

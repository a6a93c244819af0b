"""fp64 CPU oracle for the Gated DeltaNet sublayer -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does, and the oracle never imports the product.

The arithmetic lives in ``gdn_oracle.c`` (plain C, fp64, direct loops); this
module only builds it with gcc, marshals numpy arrays through ctypes and adds
the one rounding step the oracle needs at boundaries where the library stores
bf16 (round-to-nearest-even to 8 significant bits).  See the C file's header
for the passages of the pages each routine follows.

Parity status: every routine here is pinned by ``tests/test_oracle_pins.py``
(closed forms, exact brute force in rational arithmetic, chunked == sequential,
decode == prefill) and ``tests/test_oracle_mutations.py`` (each planted mistake
fails a pin).  No routine is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "gdn_oracle.c")
LIBRARY = os.path.join(_HERE, "libgdn_oracle.so")

_c_double_p = ctypes.POINTER(ctypes.c_double)
_c_int32_p = ctypes.POINTER(ctypes.c_int32)


def compile_oracle(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc (OpenMP, -O2, no fast-math) into a shared library."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", source, "-o", output, "-lm"]
    subprocess.run(cmd, check=True)
    return output


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    i32, i64, dbl, dp, ip = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, _c_double_p, _c_int32_p
    lib.gdn_oracle_conv1d.argtypes = [dp, i32, ip, i32, dp, dp, i32, dp, dp]
    lib.gdn_oracle_conv1d_step.argtypes = [dp, i32, i32, dp, dp, i32, dp]
    rule = [i32, i32, i32, i32, i32, i32, dbl, dbl, dp, dp, i64, dp, i64, dp, dp, ip, i32, dp]
    lib.gdn_oracle_delta_rule.argtypes = rule + [dp, dp]
    lib.gdn_oracle_delta_rule_chunked.argtypes = rule + [i32, dp, dp]
    lib.gdn_oracle_gated_rmsnorm.argtypes = [dp, dp, dp, i64, i32, dbl, dp]
    lib.gdn_oracle_decode_step.argtypes = [i32, i32, i32, i32, i32, i32, dbl, dbl, dbl, i32,
                                           dp, dp, dp, dp, dp, dp, dp, dp, dp]
    lib.gdn_oracle_gates.argtypes = [dp, dp, dp, dp, i64, i32, dp, dp]
    for name in ("gdn_oracle_conv1d", "gdn_oracle_conv1d_step", "gdn_oracle_delta_rule",
                 "gdn_oracle_delta_rule_chunked", "gdn_oracle_gated_rmsnorm",
                 "gdn_oracle_decode_step", "gdn_oracle_gates"):
        getattr(lib, name).restype = None
    return lib


_LIB: Optional[ctypes.CDLL] = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the compiled oracle (building it first if absent).  ``path`` loads another
    build of the same source, e.g. a mutant compiled by the mutation tests."""
    global _LIB
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _LIB is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            compile_oracle()
        _LIB = _bind(ctypes.CDLL(LIBRARY))
    return _LIB


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(_c_double_p)


def _iptr(a: np.ndarray):
    return a.ctypes.data_as(_c_int32_p)


def round_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 value (8 significant bits, ties to
    even), returned as fp64.  Used only where the library stores bf16.

    On the fp64 bit pattern: 8 significant bits keep the top 7 of the 52 stored
    fraction bits, so the low 45 bits are rounded away to nearest, ties to the
    even kept bit (a carry into the exponent is the correct rounding up to the
    next binade).  Finite, normal fp64 inputs; equal to rint(m * 256) / 256 * 2^e
    with x = m 2^e, 1/2 <= |m| < 1."""
    u = np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)
    half = np.uint64((1 << 44) - 1)
    r = (u + half + ((u >> np.uint64(45)) & np.uint64(1))) & ~np.uint64((1 << 45) - 1)
    return r.view(np.float64)


def round_f16(x) -> np.ndarray:
    """Round fp64 values to the nearest IEEE half (ties to even, subnormals kept),
    returned as fp64.  Used only where the library stores an fp16 recurrent state."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


class Oracle:
    """Thin numpy front end over the C routines.  ``lib`` selects a build (the
    default oracle, or a mutant in the mutation tests)."""

    def __init__(self, lib: Optional[ctypes.CDLL] = None):
        self.lib = lib if lib is not None else load()

    def set_threads(self, n: int) -> None:
        """OpenMP threads for the routines' parallel loops (the runtime the oracle is
        built against; its independent (sequence, head) or channel loops only)."""
        self.lib.omp_set_num_threads.argtypes = [ctypes.c_int]
        self.lib.omp_set_num_threads.restype = None
        self.lib.omp_set_num_threads(int(n))

    def max_threads(self) -> int:
        self.lib.omp_get_max_threads.restype = ctypes.c_int
        return int(self.lib.omp_get_max_threads())

    # -- conv (a1) ---------------------------------------------------------
    def conv1d(self, x, w, cu, state_in=None, act: int = 1) -> Tuple[np.ndarray, np.ndarray]:
        """x [T,C], w [C,4], cu [N+1] -> (y [T,C], state_out [N,3,C])."""
        x, w = _f64(x), _f64(w)
        cu = np.ascontiguousarray(np.asarray(cu, dtype=np.int32))
        T, C = x.shape
        N = len(cu) - 1
        si = None if state_in is None else _f64(state_in).reshape(N, 3, C)
        y = np.empty((T, C))
        so = np.empty((N, 3, C))
        self.lib.gdn_oracle_conv1d(_ptr(x), C, _iptr(cu), N, _ptr(w), _ptr(si), act, _ptr(y), _ptr(so))
        return y, so

    def conv1d_step(self, x, w, state, act: int = 1) -> Tuple[np.ndarray, np.ndarray]:
        """x [B,C], state [B,3,C] -> (y [B,C], new state)."""
        x, w = _f64(x), _f64(w)
        st = _f64(state).copy()
        B, C = x.shape
        y = np.empty((B, C))
        self.lib.gdn_oracle_conv1d_step(_ptr(x), B, C, _ptr(w), _ptr(st), act, _ptr(y))
        return y, st

    # -- gated delta rule (a2-a8, a11, a12) ---------------------------------
    def delta_rule(self, q, k, v, g, beta, cu, state_in=None, *, l2norm: int = 1,
                   l2_eps: float = 1e-6, q_scale: Optional[float] = None,
                   chunk: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
        """q, k [T,Hk,dk]; v [T,Hv,dv]; g [T,Hv] or [T,Hv,dk]; beta [T,Hv];
        state_in [N,Hv,dv,dk] or None -> (o [T,Hv,dv], final state).
        ``chunk`` selects the chunked WY arm instead of the token-by-token one."""
        q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
        cu = np.ascontiguousarray(np.asarray(cu, dtype=np.int32))
        T, Hk, dk = k.shape
        _, Hv, dv = v.shape
        N = len(cu) - 1
        per_channel = 1 if g.ndim == 3 else 0
        if q_scale is None:
            q_scale = 1.0 / np.sqrt(dk)
        si = None if state_in is None else _f64(state_in).reshape(N, Hv, dv, dk)
        o = np.zeros((T, Hv, dv))
        so = np.empty((N, Hv, dv, dk))
        args = [Hk, Hv, dk, dv, per_channel, l2norm, l2_eps, float(q_scale),
                _ptr(q), _ptr(k), Hk * dk, _ptr(v), Hv * dv, _ptr(g), _ptr(beta),
                _iptr(cu), N, _ptr(si)]
        if chunk is None:
            self.lib.gdn_oracle_delta_rule(*args, _ptr(o), _ptr(so))
        else:
            self.lib.gdn_oracle_delta_rule_chunked(*args, int(chunk), _ptr(o), _ptr(so))
        return o, so

    # -- gates from the a / b projections ------------------------------------
    def gates(self, a, b, A_log, dt_bias) -> Tuple[np.ndarray, np.ndarray]:
        """a, b [..., Hv]; A_log, dt_bias [Hv] -> (g, beta) [..., Hv]:
        g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b)."""
        a, b, A_log, dt_bias = _f64(a), _f64(b), _f64(A_log), _f64(dt_bias)
        Hv = A_log.shape[0]
        assert a.shape == b.shape and a.shape[-1] == Hv and dt_bias.shape == (Hv,)
        g = np.empty_like(a)
        beta = np.empty_like(b)
        self.lib.gdn_oracle_gates(_ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), a.size // Hv, Hv,
                                  _ptr(g), _ptr(beta))
        return g, beta

    # -- gated norm (a9) ----------------------------------------------------
    def gated_rmsnorm(self, o, z, w, eps: float = 1e-6) -> np.ndarray:
        """o, z [..., d]; w [d] -> out [..., d]."""
        o, z, w = _f64(o), _f64(z), _f64(w)
        d = o.shape[-1]
        out = np.empty_like(o)
        self.lib.gdn_oracle_gated_rmsnorm(_ptr(o), _ptr(z), _ptr(w), o.size // d, d, eps, _ptr(out))
        return out

    # -- fused decode (a10) -------------------------------------------------
    def decode_step(self, x, conv_w, conv_state, g, beta, z, norm_w, state, *, Hk: int, Hv: int,
                    dk: int, dv: int, act: int = 1, l2_eps: float = 1e-6,
                    q_scale: Optional[float] = None, rms_eps: float = 1e-6, state_f16: bool = False):
        """x [B,Cc]; conv_state [B,3,Cc]; g [B,Hv] (or [B,Hv,dk]); beta [B,Hv]; z [B,Hv,dv];
        state [B,Hv,dv,dk] -> (out [B,Hv,dv], new conv_state, new state).  ``state_f16``: the
        new state is rounded to fp16, as where the library stores an fp16 state (once per
        token)."""
        x, conv_w, g, beta, z, norm_w = map(_f64, (x, conv_w, g, beta, z, norm_w))
        cs = _f64(conv_state).copy()
        st = _f64(state).copy()
        B = x.shape[0]
        per_channel = 1 if g.ndim == 3 else 0
        if q_scale is None:
            q_scale = 1.0 / np.sqrt(dk)
        out = np.empty((B, Hv, dv))
        self.lib.gdn_oracle_decode_step(Hk, Hv, dk, dv, per_channel, act, l2_eps, float(q_scale),
                                        rms_eps, B, _ptr(x), _ptr(conv_w), _ptr(cs), _ptr(g),
                                        _ptr(beta), _ptr(z), _ptr(norm_w), _ptr(st), _ptr(out))
        if state_f16:
            st = round_f16(st)
        return out, cs, st

    # -- speculative verify transaction --------------------------------------
    def verify(self, x, conv_w, conv_state, g, beta, z, norm_w, state, *, Hk: int, Hv: int,
               dk: int, dv: int, **kw):
        """The verify half of a speculative transaction (the TDD ledger's transaction rules:
        the K verified rows are computed from the prior logical state, which only a commit
        may change).  x [B,K,Cc]; g, beta [B,K,Hv] (g [B,K,Hv,dk] per channel); z [B,K,Hv,dv].
        Row t of each sequence is decode step t from (conv_state, state); the inputs are left
        unchanged.  Returns (out [B,K,Hv,dv], snaps) with snaps[c] = (conv state, state)
        after the first c rows of every sequence, c = 0..K."""
        K = np.asarray(x).shape[1]
        cs, st = _f64(conv_state).copy(), _f64(state).copy()
        snaps = [(cs, st)]
        outs = []
        for t in range(K):
            o, cs, st = self.decode_step(np.asarray(x)[:, t], conv_w, cs, np.asarray(g)[:, t],
                                         np.asarray(beta)[:, t], np.asarray(z)[:, t], norm_w, st,
                                         Hk=Hk, Hv=Hv, dk=dk, dv=dv, **kw)
            outs.append(o)
            snaps.append((cs, st))
        return np.stack(outs, axis=1), snaps

    @staticmethod
    def commit(snaps, accepted) -> Tuple[np.ndarray, np.ndarray]:
        """The commit half: sequence b keeps the states after its first accepted[b] rows
        (0 = abort: the prior states).  Returns (conv state, state)."""
        cs = np.stack([snaps[int(c)][0][b] for b, c in enumerate(accepted)])
        st = np.stack([snaps[int(c)][1][b] for b, c in enumerate(accepted)])
        return cs, st

    # -- composition of the whole prefill path ------------------------------
    def prefill(self, x, conv_w, cu, g, beta, z, norm_w, *, Hk: int, Hv: int, dk: int, dv: int,
                conv_state_in=None, state_in=None, act: int = 1, l2_eps: float = 1e-6,
                rms_eps: float = 1e-6, round_y_bf16: bool = False, chunk: Optional[int] = None):
        """conv -> split q|k|v -> gated delta rule -> gated norm over packed sequences.
        ``round_y_bf16`` rounds the conv output where the library stores it as bf16.
        Returns (out, o, final_state, conv_state_out, y)."""
        y, cso = self.conv1d(x, conv_w, cu, conv_state_in, act)
        if round_y_bf16:
            y = round_bf16(y)
        T = y.shape[0]
        q = y[:, : Hk * dk].reshape(T, Hk, dk)
        k = y[:, Hk * dk: 2 * Hk * dk].reshape(T, Hk, dk)
        v = y[:, 2 * Hk * dk:].reshape(T, Hv, dv)
        o, so = self.delta_rule(q, k, v, g, beta, cu, state_in, l2_eps=l2_eps, chunk=chunk)
        out = self.gated_rmsnorm(o, z, norm_w, rms_eps)
        return out, o, so, cso, y


def default() -> Oracle:
    return Oracle()

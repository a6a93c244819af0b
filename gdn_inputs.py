"""Seeded synthetic inputs for the Gated DeltaNet sublayer.

This module is shared by the tests, the benchmark and the smoke check, and
serves both the HIP library and the CPU oracle.  It holds none of the method's
arithmetic: it only draws random numbers with the value distributions of the
workloads and rounds them to bf16 where the workload is bf16, so that both
sides see the very same values.

Value distributions (the second parameter of N is a standard deviation):
  pre-conv activations x (q|k|v)    N(0, 1)
  conv weight                        N(0, 0.5)
  log decay g                        logsigmoid(N(0, 1))   (always < 0)
  beta                               sigmoid(N(0, 1))
  output gate z                      N(0, 1)
  norm weight                        1 + N(0, 0.1)
  recurrent state                    N(0, 0.1)
  conv state                         N(0, 1)
Geometry of the pages' model: 16 key heads and 48 value heads of 128, conv
width 4, conv channels 2*16*128 + 48*128 = 10240.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional

import numpy as np

HK, HV, DK, DV, CONV_W, CHUNK = 16, 48, 128, 128, 4, 64


def bf16_round(a: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value (ties to even), kept as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _logsigmoid(x: np.ndarray) -> np.ndarray:
    return -np.logaddexp(0.0, -x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def conv_channels(hk: int = HK, hv: int = HV, dk: int = DK, dv: int = DV) -> int:
    return 2 * hk * dk + hv * dv


@dataclass
class Geometry:
    hk: int = HK
    hv: int = HV
    dk: int = DK
    dv: int = DV

    @property
    def channels(self) -> int:
        return conv_channels(self.hk, self.hv, self.dk, self.dv)


def seqlens_to_cu(lengths: List[int]) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def varlen_lengths(lo_total: int = 31000, hi_total: int = 33000):
    """Lengths for the varlen workload: 63, 64, 65 plus five draws from
    uniform[1, 8192], using the smallest seed >= 0 whose total lies in
    [lo_total, hi_total].  Returns (lengths, seed)."""
    seed = 0
    while True:
        rng = np.random.default_rng(seed)
        extra = rng.integers(1, 8193, size=5).tolist()
        lengths = [63, 64, 65] + [int(e) for e in extra]
        if lo_total <= sum(lengths) <= hi_total:
            return lengths, seed
        seed += 1


def gen_prefill(seed: int, lengths: List[int], geo: Geometry = Geometry(), *, bf16: bool = True,
                init_state: bool = True, conv_state: bool = False, per_channel: bool = False,
                state_sd: float = 0.1) -> Dict[str, np.ndarray]:
    """Inputs for the prefill path over packed sequences of the given lengths.

    Returns float32 arrays (bf16-representable where ``bf16``):
      x [T, Cc], conv_w [Cc, 4], g [T, Hv] (or [T, Hv, dk]), beta [T, Hv],
      z [T, Hv, dv], norm_w [dv], state_in [N, Hv, dv, dk] or None,
      conv_state_in [N, 3, Cc] or None, cu [N+1] int32.
    """
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    N = len(lengths)
    C = geo.channels
    act_round = bf16_round if bf16 else (lambda a: a.astype(np.float32))
    x = act_round(rng.standard_normal((T, C), dtype=np.float32))
    conv_w = (0.5 * rng.standard_normal((C, CONV_W))).astype(np.float32)
    gshape = (T, geo.hv, geo.dk) if per_channel else (T, geo.hv)
    g = _logsigmoid(rng.standard_normal(gshape)).astype(np.float32)
    beta = _sigmoid(rng.standard_normal((T, geo.hv))).astype(np.float32)
    z = act_round(rng.standard_normal((T, geo.hv, geo.dv), dtype=np.float32))
    norm_w = (1.0 + 0.1 * rng.standard_normal(geo.dv)).astype(np.float32)
    state_in = None
    if init_state:
        state_in = (state_sd * rng.standard_normal((N, geo.hv, geo.dv, geo.dk), dtype=np.float32)
                    ).astype(np.float32)
    cs = None
    if conv_state:
        cs = act_round(rng.standard_normal((N, CONV_W - 1, C), dtype=np.float32))
    return dict(x=x, conv_w=conv_w, g=g, beta=beta, z=z, norm_w=norm_w, state_in=state_in,
                conv_state_in=cs, cu=seqlens_to_cu(lengths))


def gen_qkv(seed: int, lengths: List[int], geo: Geometry = Geometry(), *, bf16: bool = True,
            init_state: bool = True, per_channel: bool = False,
            state_sd: float = 0.1) -> Dict[str, np.ndarray]:
    """Inputs for the chunk call alone: q, k [T, Hk, dk], v [T, Hv, dv] ~ N(0, 1), plus
    g, beta, state_in and cu as in :func:`gen_prefill`."""
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    N = len(lengths)
    act_round = bf16_round if bf16 else (lambda a: a.astype(np.float32))
    q = act_round(rng.standard_normal((T, geo.hk, geo.dk), dtype=np.float32))
    k = act_round(rng.standard_normal((T, geo.hk, geo.dk), dtype=np.float32))
    v = act_round(rng.standard_normal((T, geo.hv, geo.dv), dtype=np.float32))
    gshape = (T, geo.hv, geo.dk) if per_channel else (T, geo.hv)
    g = _logsigmoid(rng.standard_normal(gshape)).astype(np.float32)
    beta = _sigmoid(rng.standard_normal((T, geo.hv))).astype(np.float32)
    state_in = None
    if init_state:
        state_in = (state_sd * rng.standard_normal((N, geo.hv, geo.dv, geo.dk), dtype=np.float32)
                    ).astype(np.float32)
    return dict(q=q, k=k, v=v, g=g, beta=beta, state_in=state_in, cu=seqlens_to_cu(lengths))


STRONG_DECAY_PATTERNS = ("quarter_m10", "all_m3", "all_m30", "bursts_m30")


def strong_channel_decay(g: np.ndarray, pattern: str, seed: int) -> np.ndarray:
    """A per-key-channel log decay g [T, Hv, dk] with strong decays written in:
      quarter_m10  g = -10 in a random quarter of each head's channels (the rest as drawn)
      all_m3       g = -3 everywhere
      all_m30      g = -30 everywhere (every in-chunk factor between tokens underflows)
      bursts_m30   g = -30 on 8-token runs (aligned to 8) of random channels, about one run in 8
    All values stay <= 0, the method's range for g.  A scalar decay g [T, Hv] takes the
    same patterns with the heads in the place of the channels."""
    if np.ndim(g) == 2:
        return strong_channel_decay(np.asarray(g)[:, None, :], pattern, seed)[:, 0, :]
    rng = np.random.default_rng(seed)
    g = np.array(g, dtype=np.float32, copy=True)
    T, hv, dk = g.shape
    if pattern == "quarter_m10":
        for h in range(hv):
            g[:, h, rng.permutation(dk)[: dk // 4]] = -10.0
    elif pattern == "all_m3":
        g[:] = -3.0
    elif pattern == "all_m30":
        g[:] = -30.0
    elif pattern == "bursts_m30":
        runs = (T + 7) // 8
        hit = rng.random((runs, hv, dk)) < 0.125
        g[np.repeat(hit, 8, axis=0)[:T]] = -30.0
    else:
        raise ValueError(f"unknown pattern {pattern!r}")
    return g


def gen_decode(seed: int, batch: int, geo: Geometry = Geometry(), *, bf16: bool = True,
               per_channel: bool = False, state_sd: float = 0.1) -> Dict[str, np.ndarray]:
    """Inputs for one fused decode step of ``batch`` sequences:
      x [B, Cc], conv_w [Cc, 4], conv_state [B, 3, Cc], g [B, Hv] (or [B, Hv, dk]),
      beta [B, Hv], z [B, Hv, dv], norm_w [dv], state [B, Hv, dv, dk]."""
    rng = np.random.default_rng(seed)
    C = geo.channels
    act_round = bf16_round if bf16 else (lambda a: a.astype(np.float32))
    x = act_round(rng.standard_normal((batch, C), dtype=np.float32))
    conv_w = (0.5 * rng.standard_normal((C, CONV_W))).astype(np.float32)
    conv_state = act_round(rng.standard_normal((batch, CONV_W - 1, C), dtype=np.float32))
    gshape = (batch, geo.hv, geo.dk) if per_channel else (batch, geo.hv)
    g = _logsigmoid(rng.standard_normal(gshape)).astype(np.float32)
    beta = _sigmoid(rng.standard_normal((batch, geo.hv))).astype(np.float32)
    z = act_round(rng.standard_normal((batch, geo.hv, geo.dv), dtype=np.float32))
    norm_w = (1.0 + 0.1 * rng.standard_normal(geo.dv)).astype(np.float32)
    state = (state_sd * rng.standard_normal((batch, geo.hv, geo.dv, geo.dk), dtype=np.float32)
             ).astype(np.float32)
    return dict(x=x, conv_w=conv_w, conv_state=conv_state, g=g, beta=beta, z=z, norm_w=norm_w,
                state=state)


def gen_gate_projections(seed: int, rows: int, hv: int = HV, *, bf16: bool = True) -> Dict[str, np.ndarray]:
    """Raw gate inputs for ``rows`` tokens (or sequences): the a / b projection outputs
    a, b [rows, Hv] ~ N(0, 1) (bf16-representable where ``bf16``), and per head
    A_log = log(U[1, 16]) and dt_bias = log(expm1(U[0.001, 0.1])) (the bias that makes
    softplus(dt_bias) a step in [0.001, 0.1]), fp32."""
    rng = np.random.default_rng(seed)
    act_round = bf16_round if bf16 else (lambda a: a.astype(np.float32))
    a = act_round(rng.standard_normal((rows, hv), dtype=np.float32))
    b = act_round(rng.standard_normal((rows, hv), dtype=np.float32))
    A_log = np.log(rng.uniform(1.0, 16.0, hv)).astype(np.float32)
    dt_bias = np.log(np.expm1(rng.uniform(0.001, 0.1, hv))).astype(np.float32)
    return dict(a=a, b=b, A_log=A_log, dt_bias=dt_bias)


# The five workloads, by what they are.
WORKLOADS = {
    "prefill_s80_fp32": dict(lengths=[80], bf16=False, init_state=False, seed=1001),
    "decode_b64_bf16": dict(batch=64, bf16=True, seed=1002),
    "prefill_s4096_bf16": dict(lengths=[4096], bf16=True, init_state=True, seed=1003),
    "varlen8_32k_bf16": dict(bf16=True, init_state=True, seed=1004),
    "kda_h64_s16384_bf16": dict(lengths=[16384], bf16=True, init_state=True, per_channel=True,
                                seed=1005, geo=Geometry(hk=64, hv=64)),
}

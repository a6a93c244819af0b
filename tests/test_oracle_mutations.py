"""Planted mistakes in the oracle must each fail at least one pin.

Every case below edits one expression of ``oracle/gdn_oracle.c`` (in a
temporary copy), compiles the mutant with gcc and runs the whole pin suite
against it.  The mistakes are the plausible ones: the faults the pages name
(wrong decay sign, missing beta or q scale, transposed state, RMS or
max(norm, eps) in place of L2, one-position conv shift, SiLU in place of the
sigmoid gate, dropped state carry) and slips of sign, index or order.  CPU
only; no GPU code is involved.
"""

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTANTS = [
    # (id, exact source text, replacement)
    ("decay_sign", "exp(g[t * Hv + h]);", "exp(-g[t * Hv + h]);"),
    ("decay_sign_per_channel", "exp(g[(t * Hv + h) * dk + j])", "exp(-g[(t * Hv + h) * dk + j])"),
    ("per_channel_wrong_channel", "exp(g[(t * Hv + h) * dk + j])", "exp(g[(t * Hv + h) * dk])"),
    ("missing_beta", "u[i] = b * (vt[i] - p);", "u[i] = (vt[i] - p);"),
    ("missing_q_scale", "qn[j] *= q_scale;", "qn[j] *= 1.0;"),
    ("transposed_state_predict", "p += S[(int64_t)i * dk + j] * kn[j];",
     "p += S[(int64_t)j * dk + i] * kn[j];"),
    ("transposed_state_read", "acc += S[(int64_t)i * dk + j] * qn[j];",
     "acc += S[(int64_t)j * dk + i] * qn[j];"),
    ("predict_before_decay", "p += S[(int64_t)i * dk + j] * kn[j];",
     "p += S[(int64_t)i * dk + j] / a[j] * kn[j];"),
    ("write_sign", "S[(int64_t)i * dk + j] += u[i] * kn[j];", "S[(int64_t)i * dk + j] -= u[i] * kn[j];"),
    ("rms_instead_of_l2", "1.0 / sqrt(ss + eps)", "1.0 / sqrt(ss / d + eps)"),
    ("max_norm_eps", "1.0 / sqrt(ss + eps)", "1.0 / fmax(sqrt(ss), eps)"),
    ("eps_outside_l2_root", "1.0 / sqrt(ss + eps)", "1.0 / (sqrt(ss) + eps)"),
    ("head_tile_not_interleave", "const int32_t kh = h / ratio;\n      double* S = (double*)calloc",
     "const int32_t kh = h % Hk;\n      double* S = (double*)calloc"),
    ("conv_one_position_shift", "conv_input(x, C, t0, n, state_in, t - 3 + i, c)",
     "conv_input(x, C, t0, n, state_in, t - 2 + i, c)"),
    ("conv_taps_reversed", "acc += w[c * 4 + i] * conv_input", "acc += w[c * 4 + 3 - i] * conv_input"),
    ("conv_state_out_reversed", "state_out[((int64_t)n * 3 + r) * C + c] = keep[r];",
     "state_out[((int64_t)n * 3 + r) * C + c] = keep[2 - r];"),
    ("conv_step_shift", "st[0 * C + c] = window[1];", "st[0 * C + c] = window[0];"),
    ("conv_state_rows_newest_first", "return state_in[((int64_t)n * 3 + (3 + s)) * C + c];",
     "return state_in[((int64_t)n * 3 + (-1 - s)) * C + c];"),
    ("silu_instead_of_sigmoid_gate", "w[i] * sigmoid(zrow[i])", "w[i] * zrow[i] * sigmoid(zrow[i])"),
    ("norm_eps_outside_root", "1.0 / sqrt(ss / d + eps)", "1.0 / (sqrt(ss / d) + eps)"),
    ("norm_sum_not_mean", "1.0 / sqrt(ss / d + eps)", "1.0 / sqrt(ss + eps)"),
    ("silu_wrong", "return act ? y * sigmoid(y) : y;", "return act ? sigmoid(y) : y;"),
    ("chunk_dropped_carry", "memcpy(S, S1, sizeof(double) * dv * dk);", "/* carry dropped */"),
    ("chunk_solve_sign", "acc -= A[r * chunk + j] * Tm[j * chunk + col];",
     "acc += A[r * chunk + j] * Tm[j * chunk + col];"),
    ("chunk_A_missing_beta", "A[r * chunk + j] = bet[r] * acc;", "A[r * chunk + j] = acc;"),
    ("chunk_A_decay_sign", "exp(gam[(int64_t)r * dk + c] - gam[(int64_t)j * dk + c]);",
     "exp(gam[(int64_t)j * dk + c] - gam[(int64_t)r * dk + c]);"),
    ("chunk_output_exclusive", "for (int32_t j = 0; j <= r; ++j) {", "for (int32_t j = 0; j < r; ++j) {"),
    ("chunk_factorised_decay_sign", "exp(gl - gam[(int64_t)j * dk + c]);", "exp(gam[(int64_t)j * dk + c] - gl);"),
    ("gate_sign", "g[t * Hv + h] = -exp(A_log[h])", "g[t * Hv + h] = exp(A_log[h])"),
    ("gate_A_not_exponentiated", "g[t * Hv + h] = -exp(A_log[h]) * softplus", "g[t * Hv + h] = -A_log[h] * softplus"),
    ("gate_dt_bias_dropped", "softplus(a[t * Hv + h] + dt_bias[h])", "softplus(a[t * Hv + h])"),
    ("gate_dt_bias_negated", "softplus(a[t * Hv + h] + dt_bias[h])", "softplus(a[t * Hv + h] - dt_bias[h])"),
    ("gate_relu_for_softplus", "return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));",
     "return x > 0.0 ? x : 0.0;"),
    ("gate_softplus_branch_sign", "return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));",
     "return x > 0.0 ? x - log1p(exp(-x)) : log1p(exp(x));"),
    ("gate_exp_for_softplus", "return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));", "return exp(x);"),
    ("gate_beta_silu", "beta[t * Hv + h] = sigmoid(b[t * Hv + h]);",
     "beta[t * Hv + h] = b[t * Hv + h] * sigmoid(b[t * Hv + h]);"),
    ("gate_beta_sign", "beta[t * Hv + h] = sigmoid(b[t * Hv + h]);", "beta[t * Hv + h] = sigmoid(-b[t * Hv + h]);"),
    ("gate_head_index", "-exp(A_log[h]) * softplus(a[t * Hv + h] + dt_bias[h])",
     "-exp(A_log[0]) * softplus(a[t * Hv + h] + dt_bias[h])"),
    ("decode_skips_conv_state_update", "gdn_oracle_conv1d_step(x, B, Cc, conv_w, conv_state, act, y);",
     "{ double* tmp = (double*)malloc(sizeof(double) * B * 3 * Cc); "
     "memcpy(tmp, conv_state, sizeof(double) * B * 3 * Cc); "
     "gdn_oracle_conv1d_step(x, B, Cc, conv_w, tmp, act, y); free(tmp); }"),
]


def _run_pins(orc):
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError as e:
            failed.append((pin.__name__, (str(e) or "assertion").splitlines()[0][:120]))
    return failed


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


def test_unmutated_build_passes_every_pin(source, tmp_path):
    path = str(tmp_path / "liboracle_copy.so")
    src = tmp_path / "copy.c"
    src.write_text(source)
    oracle.compile_oracle(str(src), path)
    assert _run_pins(oracle.Oracle(oracle.load(path))) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_fails_a_pin(source, tmp_path, name, old, new):
    assert source.count(old) >= 1, f"mutation site for {name} not found in the oracle"
    mutated = source.replace(old, new, 1)
    src = tmp_path / f"{name}.c"
    src.write_text(mutated)
    lib = str(tmp_path / f"lib_{name}.so")
    oracle.compile_oracle(str(src), lib)
    failed = _run_pins(oracle.Oracle(oracle.load(lib)))
    assert failed, f"planted mistake '{name}' passed every pin"


# The verify / commit transaction of the oracle is Python composing the C decode step; its
# plausible slips are planted in subclasses and must fail the transaction pin.
class _CommitOffByOne(oracle.Oracle):
    @staticmethod
    def commit(snaps, accepted):
        return oracle.Oracle.commit(snaps, [min(int(c) + 1, len(snaps) - 1) for c in accepted])


class _CommitKeepsLast(oracle.Oracle):
    @staticmethod
    def commit(snaps, accepted):
        return oracle.Oracle.commit(snaps, [len(snaps) - 1 for _ in accepted])


class _VerifyInPlace(oracle.Oracle):
    def verify(self, x, conv_w, conv_state, g, beta, z, norm_w, state, **kw):
        out, snaps = super().verify(x, conv_w, conv_state, g, beta, z, norm_w, state, **kw)
        conv_state[...] = snaps[-1][0]
        state[...] = snaps[-1][1]
        return out, snaps


class _VerifyRowsFromPriorState(oracle.Oracle):
    """Every verified row decoded from the prior state (no chaining inside the window)."""
    def verify(self, x, conv_w, conv_state, g, beta, z, norm_w, state, *, Hk, Hv, dk, dv, **kw):
        outs = [self.decode_step(x[:, t], conv_w, conv_state, g[:, t], beta[:, t], z[:, t], norm_w, state,
                                 Hk=Hk, Hv=Hv, dk=dk, dv=dv, **kw) for t in range(x.shape[1])]
        snaps = [(conv_state.copy(), state.copy())] + [(o[1], o[2]) for o in outs]
        return __import__("numpy").stack([o[0] for o in outs], axis=1), snaps


@pytest.mark.parametrize("mutant", [_CommitOffByOne, _CommitKeepsLast, _VerifyInPlace, _VerifyRowsFromPriorState],
                         ids=lambda m: m.__name__.strip("_"))
def test_transaction_mutant_fails_the_pin(mutant):
    from oracle_pins import pin_verify_transaction_equals_prefill
    with pytest.raises(AssertionError):
        pin_verify_transaction_equals_prefill(mutant())

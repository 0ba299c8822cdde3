"""Plant plausible mistakes in copies of the oracle (on the CPU) and require
every broken copy to fail at least one pin.  This shows the pins constrain
every part of the oracle: the decay, the projection, the write, the output
read, checkpoints, initial state, the conv filter and state, and the norm."""
import os
import re

import pytest

import oracle
from oracle import build as obuild
from tests.oracle_pins import ALL_PINS

with open(obuild.SOURCE) as _f:
    SOURCE = _f.read()


def _swap_decay_and_projection(src):
    a = src.index("    /* S <- Diag(alpha) S")
    b = src.index("    /* S <- (I - beta k k^T) S")
    c = src.index("    /* S <- S + beta k v^T. */")
    return src[:a] + src[b:c] + src[a:b] + src[c:]


def _output_before_update(src):
    a = src.index("    /* o = scale * S^T q. */")
    end = src.index("\n}\n", a)
    block = src[a:end + 1]
    body = src[:a] + src[end + 1:]
    start = body.index("    /* S <- Diag(alpha) S")
    return body[:start] + block + body[start:]


def _sub(old, new, count=1):
    def f(src):
        assert src.count(old) >= 1, old
        return src.replace(old, new, count)
    return f


MUTANTS = {
    "decay_sign": _sub("double a = exp(g[i]);", "double a = exp(-g[i]);"),
    "decay_after_projection": _swap_decay_and_projection,
    "output_before_update": _output_before_update,
    "projection_without_beta": _sub("S[i * dv + j] -= beta * k[i] * work[j];",
                                    "S[i * dv + j] -= k[i] * work[j];"),
    "write_without_beta": _sub("S[i * dv + j] += beta * k[i] * v[j];",
                               "S[i * dv + j] += k[i] * v[j];"),
    "projection_uses_q": _sub("s += k[i] * S[i * dv + j];", "s += q[i] * S[i * dv + j];"),
    "scale_dropped": _sub("o[j] = scale * s;", "o[j] = s;"),
    "checkpoint_off_by_one": _sub("const int64_t pos = p0 + r + 1;", "const int64_t pos = p0 + r;"),
    "checkpoint_ignores_start": _sub("const int64_t pos = p0 + r + 1;", "const int64_t pos = r + 1;"),
    "checkpoint_rows_ignore_start": _sub("pos / ckpt_interval - p0 / ckpt_interval - 1",
                                         "pos / ckpt_interval - 1"),
    "initial_state_ignored": _sub("if (!has_init || has_init[i]) memcpy(S, home",
                                  "if (1) memcpy(S, home"),
    "state_not_written": _sub("memcpy(home, S,", "if (0) memcpy(home, S,"),
    "padding_not_zeroed": _sub("memset(o + (t * H + h) * dv, 0,", "if (0) memset(o + (t * H + h) * dv, 0,"),
    "l2norm_skipped_for_k": _sub("kt = kn;", "kt = kt;"),
    "conv_taps_reversed": _sub("acc += w[c * W + j] * ext", "acc += w[c * W + (W - 1 - j)] * ext"),
    "conv_state_not_updated": _sub("memcpy(st, ext + L * Cch,", "if (0) memcpy(st, ext + L * Cch,"),
    "conv_state_ignored": _sub("if (!has_init || has_init[i]) memcpy(ext, st,",
                               "if (0) memcpy(ext, st,"),
    "spec_state_saved_before_token": _sub(
        "            kda_token(S, dk, dv, qt, kt, v + (row * H + h) * dv, g + (row * H + h) * dk,\n"
        "                      beta[row * H + h], scale, o + (row * H + h) * dv, work);\n"
        "            memcpy(token_states + ((b * ntok + t) * H + h) * dk * dv, S,\n"
        "                   (size_t)(dk * dv) * sizeof(double));",
        "            memcpy(token_states + ((b * ntok + t) * H + h) * dk * dv, S,\n"
        "                   (size_t)(dk * dv) * sizeof(double));\n"
        "            kda_token(S, dk, dv, qt, kt, v + (row * H + h) * dv, g + (row * H + h) * dk,\n"
        "                      beta[row * H + h], scale, o + (row * H + h) * dv, work);"),
    "spec_token_rows_interleaved": _sub("const int64_t row = b * ntok + t;", "const int64_t row = t * B + b;"),
    "spec_commit_takes_last_draft": _sub("token_states + ((b * ntok + accepted[b] - 1) * H + h)",
                                         "token_states + ((b * ntok + ntok - 1) * H + h)"),
    "rmsnorm_sum_not_mean": _sub("ss / (double)dim + eps", "ss + eps"),
    "rmsnorm_sigmoid_not_silu": _sub(": z / (1.0 + exp(-z));", ": 1.0 / (1.0 + exp(-z));"),
    "rmsnorm_silu_for_sigmoid": _sub("sigmoid ? 1.0 / (1.0 + exp(-z))", "sigmoid ? z / (1.0 + exp(-z))"),
    "rmsnorm_residual_dropped": _sub("x[r * dim + c] + (residual ? residual[r * dim + c] : 0.0)",
                                     "x[r * dim + c]"),
    "rmsnorm_bias_after_gate": _sub(
        "(h[c] * inv * (w ? w[c] : 1.0) + (b ? b[c] : 0.0)) * act",
        "h[c] * inv * (w ? w[c] : 1.0) * act + (b ? b[c] : 0.0)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name, tmp_path):
    src = MUTANTS[name](SOURCE)
    assert src != SOURCE
    path = tmp_path / f"mutant_{name}.c"
    path.write_text(src)
    lib = obuild.build(str(path), str(tmp_path / f"libmutant_{name}.so"))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"

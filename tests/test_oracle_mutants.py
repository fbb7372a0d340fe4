"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of the oracle's C source (a wrong order of
decay / read / write, a sign, a dropped term, a wrong index or snapshot), builds the copy,
and runs the pin suite against it in a separate process. The pins must fail for every
mutant; a mutant that survives means a part of the oracle is not pinned by anything but
itself.
"""
import os
import shutil
import subprocess
import sys

import pytest

from oracle.build import SRC, build_oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_DECAY = """    /* decay */
    for (int i = 0; i < dk; i++) {
        double a = exp(c->perkey ? g[i] : g[0]);
        double* row = S + (size_t)i * dv;
        for (int j = 0; j < dv; j++) row[j] *= a;
    }
"""
_WRITE_MARK = "    /* residual write: S += k r^T with r = beta (v - vhat) */\n"
_READOUT = """    /* read after write */
    for (int j = 0; j < dv; j++) o[j] = 0.0;
    for (int i = 0; i < dk; i++) {
        const double* row = S + (size_t)i * dv;
        for (int j = 0; j < dv; j++) o[j] += row[j] * q[i];
    }
    for (int j = 0; j < dv; j++) o[j] *= c->scale;
"""


def _move_before(src, block, mark):
    assert src.count(block) == 1 and src.count(mark) == 1
    src = src.replace(block, "")
    return src.replace(mark, block + mark)


def _sub(old, new):
    def f(src):
        assert src.count(old) == 1, old
        return src.replace(old, new)
    return f


MUTANTS = {
    # gated delta rule, one token
    "read_before_decay": lambda s: _swap_decay_read(s),
    "residual_sign": _sub("vhat[j] = beta * (v[j] - vhat[j]);",
                          "vhat[j] = beta * (v[j] + vhat[j]);"),
    "beta_dropped": _sub("vhat[j] = beta * (v[j] - vhat[j]);",
                         "vhat[j] = (v[j] - vhat[j]);"),
    "output_before_write": lambda s: _move_before(s, _READOUT, _WRITE_MARK),
    "scale_dropped": _sub("o[j] *= c->scale;", "o[j] *= 1.0;"),
    "perkey_gate_first_channel": _sub("exp(c->perkey ? g[i] : g[0])",
                                      "exp(c->perkey ? g[0] : g[0])"),
    "gate_not_log": _sub("double a = exp(c->perkey ? g[i] : g[0]);",
                         "double a = 1.0 + (c->perkey ? g[i] : g[0]);"),
    "write_transposed_key": _sub("row[j] += k[i] * vhat[j];",
                                 "row[j] += k[j % dk] * vhat[i % dv];"),
    "l2norm_skips_q": _sub("l2n(q_in, q, dk, c->l2norm, c->eps);",
                           "l2n(q_in, q, dk, 0, c->eps);"),
    # DeltaLog bookkeeping
    "deltalog_read_before_decay": _sub("for (int d = 0; d < dl; d++) lp[d] = lb[d] + g[d];",
                                       "for (int d = 0; d < dl; d++) lp[d] = lb[d];"),
    "deltalog_lambda_snapshot_old": _sub("for (int d = 0; d < dl; d++) Le[d] = lp[d];",
                                         "for (int d = 0; d < dl; d++) Le[d] = lb[d];"),
    "deltalog_merge_drops_current": _sub("for (int j = 0; j < dv; j++) row[j] += k[i] * b[j];",
                                         "for (int j = 0; j < dv; j++) row[j] += 0.0 * b[j];"),
    "deltalog_output_drops_current": _sub("o[j] = J->cfg.scale * (qs[j] + kq * b[j]);",
                                          "o[j] = J->cfg.scale * qs[j];"),
    "deltalog_replay_undecayed": _sub("coef += x[i] * exp(lp[di] - Le[di]) * Ke[i];",
                                      "coef += x[i] * Ke[i];"),
    "deltalog_merge_keeps_lbar": _sub("for (int d = 0; d < dl; d++) lb[d] = 0.0;",
                                      "for (int d = 0; d < dl; d++) lb[d] = lb[d];"),
    "deltalog_key_not_rounded": _sub(
        "Ke[i] = J->klog_bf16 ? round_bf16(k[i]) : k[i];", "Ke[i] = k[i];"),
    # short convolution
    "conv_taps_reversed": _sub("acc += w[(size_t)c * width + j] * x[(size_t)src * channels + c];",
                               "acc += w[(size_t)c * width + (width - 1 - j)] * "
                               "x[(size_t)src * channels + c];"),
    "conv_crosses_sequences": _sub("if (src < cu_seqlens[n]) continue;",
                                   "if (src < 0) continue;"),
    "conv_no_silu": _sub("y[(size_t)t * channels + c] = acc / (1.0 + exp(-acc));",
                         "y[(size_t)t * channels + c] = acc;"),
}


def _swap_decay_read(src):
    """Read vhat from the undecayed state, then decay, then write."""
    read = """    /* read against the decayed state */
    for (int j = 0; j < dv; j++) vhat[j] = 0.0;
    for (int i = 0; i < dk; i++) {
        const double* row = S + (size_t)i * dv;
        for (int j = 0; j < dv; j++) vhat[j] += row[j] * k[i];
    }
"""
    assert src.count(read) == 1 and src.count(_DECAY) == 1
    return src.replace(_DECAY + read, read + _DECAY)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_kill_mutant(name, tmp_path):
    src = open(SRC).read()
    mutated = MUTANTS[name](src)
    assert mutated != src
    c = tmp_path / "mutant.c"
    c.write_text(mutated)
    lib = build_oracle(src=str(c), out=str(tmp_path / "libmutant.so"))
    env = dict(os.environ, GDN_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1 and "failed" in r.stdout, (
        f"mutant {name} survived the pins:\n{r.stdout[-2000:]}\n{r.stderr[-2000:]}")


# Mistakes planted in the gate formula (oracle/gates.py); the pins run against a copy of the
# oracle package that holds the mutated module.
GATE_MUTANTS = {
    "A_log_not_exponentiated": ("np.exp(np.asarray(A_log, dtype=np.float64))[:, None] * x",
                                "np.asarray(A_log, dtype=np.float64)[:, None] * x"),
    "dt_bias_dropped": ("x = fb + np.asarray(dt_bias, dtype=np.float64)", "x = fb"),
    "sigmoid_sign": ("return 1.0 / (1.0 + np.exp(-x))", "return 1.0 / (1.0 + np.exp(x))"),
    "A_log_per_channel": ("np.exp(np.asarray(A_log, dtype=np.float64))[:, None] * x",
                          "np.exp(np.asarray(A_log, dtype=np.float64))[None, :] * x"),
}


@pytest.mark.parametrize("name", sorted(GATE_MUTANTS))
def test_gate_pins_kill_mutant(name, tmp_path):
    old, new = GATE_MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "gates.py")).read()
    assert src.count(old) == 1
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("__pycache__"))
    (tmp_path / "oracle" / "gates.py").write_text(src.replace(old, new))
    (tmp_path / "tests").mkdir()
    for f in ("conftest.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tmp_path / "tests" / "golden")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-k", "kda_gate", str(tmp_path / "tests" / "test_oracle_pins.py")],
                       cwd=str(tmp_path), capture_output=True, text=True, timeout=600)
    assert r.returncode == 1 and "failed" in r.stdout, (
        f"gate mutant {name} survived the pins:\n{r.stdout[-2000:]}\n{r.stderr[-2000:]}")


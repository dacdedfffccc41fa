"""Each plausible mistake planted in the oracle must fail at least one pin.

The mistakes are planted on the CPU only: the test rewrites a copy of
``oracle/kda_oracle.c`` (a dropped term, a wrong sign, a wrong operand, a
transposed index, a swapped order of steps), builds it with gcc into a
temporary directory, and runs every pin of ``oracle_pins`` against it.
"""
import os
import subprocess

import pytest

import oracle
from oracle_pins import ALL_PINS

DECAY = "    /* S' = diag(exp(max(g, floor))) S */\n"
ERR_W = "    /* w = S'^T k */\n"
ERR_U = "    /* u = beta (v - w) */\n"
WRITE = "    /* S = S' + k u^T */\n"
READ = "    /* o = S^T q */\n"
END = "  }\n}\n\n/* Returns"


def _blocks(src):
    i = [src.index(m) for m in (DECAY, ERR_W, ERR_U, WRITE, READ)] + [src.index(END)]
    names = ["decay", "w", "u", "write", "read"]
    return src[:i[0]], {n: src[i[j]:i[j + 1]] for j, n in enumerate(names)}, src[i[-1]:]


def _reorder(order):
    def f(src):
        head, b, tail = _blocks(src)
        return head + "".join(b[n] for n in order) + tail
    return f


def _replace(old, new):
    def f(src):
        assert src.count(old) == 1, old
        return src.replace(old, new)
    return f


MUTANTS = {
    "no_decay": _replace("S[c * dv + j] *= a;", "S[c * dv + j] *= 1.0 + 0.0 * a;"),
    "no_floor": _replace("if (gc < g_floor) gc = g_floor;", ""),
    "decay_sign": _replace("const double a = exp(gc);", "const double a = exp(-gc);"),
    "error_sign": _replace("u[j] = bt * ((double)vt[j] - w[j]);",
                           "u[j] = bt * ((double)vt[j] + w[j]);"),
    "no_beta": _replace("u[j] = bt * ((double)vt[j] - w[j]);",
                        "u[j] = 1.0 * ((double)vt[j] - w[j]);"),
    "erase_with_q": _replace("w[j] += S[c * dv + j] * kc;",
                             "w[j] += S[c * dv + j] * (double)qt[c];"),
    "erase_transposed": _replace("w[j] += S[c * dv + j] * kc;",
                                 "w[j] += S[(j % dk) * dv + (c % dv)] * kc;"),
    "write_with_q": _replace("S[c * dv + j] += kc * u[j];",
                             "S[c * dv + j] += (double)qt[c] * u[j];"),
    "read_with_k": _replace("ot[j] += S[c * dv + j] * qc;",
                            "ot[j] += S[c * dv + j] * (double)kt[c];"),
    "read_transposed": _replace("ot[j] += S[c * dv + j] * qc;",
                                "ot[j] += S[(j % dk) * dv + (c % dv)] * qc;"),
    "read_before_write": _reorder(["decay", "w", "u", "read", "write"]),
    "decay_after_write": _reorder(["w", "u", "write", "decay", "read"]),
    "ignore_h0": _replace("if (S0)\n", "if (0 && S0)\n"),
    "drop_last_token": _replace("for (int64_t t = t0; t < t1; ++t) {",
                                "for (int64_t t = t0; t + 1 < t1; ++t) {"),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    src = MUTANTS[name](source)
    assert src != source
    c_path = os.path.join(tmp_path, f"{name}.c")
    so_path = os.path.join(tmp_path, f"{name}.so")
    with open(c_path, "w") as f:
        f.write(src)
    subprocess.run(["gcc", *oracle.CFLAGS, "-w", "-o", so_path, c_path, "-lm"], check=True)
    mutant = oracle.Oracle(so_path)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except Exception:  # AssertionError, or numbers so wrong they break the pin
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"

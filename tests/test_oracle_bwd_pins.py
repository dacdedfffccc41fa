"""The oracle's gradient against its pins, and planted mistakes in a copy of
its source against the same pins.  CPU only."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle_bwd_pins import ALL_BWD_PINS, tiny_case


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle()


@pytest.mark.parametrize("pin", ALL_BWD_PINS, ids=[p.__name__ for p in ALL_BWD_PINS])
def test_bwd_pin(orc, pin):
    pin(orc)


def test_bwd_thread_count_does_not_change_result(orc):
    c = tiny_case()
    a = orc.backward(c["q"], c["k"], c["v"], c["g"], c["beta"], c["do"], h0=c["h0"],
                     dht=c["dht"], cu_seqlens=c["cu"], n_threads=1)
    b = orc.backward(c["q"], c["k"], c["v"], c["g"], c["beta"], c["do"], h0=c["h0"],
                     dht=c["dht"], cu_seqlens=c["cu"], n_threads=4)
    for key in a:
        assert (a[key] == b[key]).all(), key


def test_bwd_long_sequence_crosses_replay_blocks(orc):
    """Sequences longer than the replay block (64 tokens) give the same
    gradient as the same tokens split at a block boundary and resumed with
    the state and its gradient handed across (split/resume of the reverse
    pass)."""
    from oracle_pins import rand_inputs
    q, k, v, g, beta, S0 = rand_inputs(np.random.default_rng(9), 1, 200, 2, 8, 8, g_mode="weak")
    rng = np.random.default_rng(10)
    do = rng.standard_normal(v.shape)
    dht = rng.standard_normal(S0.shape)
    full = orc.backward(q, k, v, g, beta, do, h0=S0, dht=dht)
    t1 = 130
    _, mid = orc.forward(q[:, :t1], k[:, :t1], v[:, :t1], g[:, :t1], beta[:, :t1], h0=S0)
    tail = orc.backward(q[:, t1:], k[:, t1:], v[:, t1:], g[:, t1:], beta[:, t1:], do[:, t1:],
                        h0=mid, dht=dht)
    head = orc.backward(q[:, :t1], k[:, :t1], v[:, :t1], g[:, :t1], beta[:, :t1], do[:, :t1],
                        h0=S0, dht=tail["dh0"])
    for key in ("dq", "dk", "dv", "dg", "dbeta"):
        joined = np.concatenate([head[key], tail[key]], axis=1)
        assert np.max(np.abs(joined - full[key])) <= 1e-9 * np.max(np.abs(full[key])), key
    assert np.max(np.abs(head["dh0"] - full["dh0"])) <= 1e-9 * np.max(np.abs(full["dh0"]))


# plausible mistakes in the reverse pass, planted in a copy of its source
MUTANTS = {
    "dq_from_previous_state": ("acc += St[c * dv + j] * dot[j];", "acc += Sprev[c * dv + j] * dot[j];"),
    "no_write_term_in_dk": ("acc += dS[c * dv + j] * u[j];", "acc += 0.0 * u[j];"),
    "dw_sign": ("du[j] = -bt * du[j];", "du[j] = bt * du[j];"),
    "no_erase_term_in_dS": ("dS[c * dv + j] += (double)kt[c] * du[j];", "(void)0;"),
    "no_decay_on_dS": ("dS[c * dv + j] *= a[c];", "(void)a;"),
    "dbeta_uses_v_only": ("db += du[j] * ((double)vt[j] - w[j]);", "db += du[j] * (double)vt[j];"),
    "floor_blocks_ties": ("(double)gt[c] >= in->g_floor ?", "(double)gt[c] > in->g_floor ?"),
    "dg_without_alpha": ("a[c] * acc : 0.0;", "acc : 0.0;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bwd_mutant_is_caught(name, tmp_path):
    with open(oracle.SOURCE_BWD) as f:
        src = f.read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, old
    c_path = os.path.join(tmp_path, f"{name}.c")
    so_path = os.path.join(tmp_path, f"{name}.so")
    with open(c_path, "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc", *oracle.CFLAGS, "-w", "-o", so_path, oracle.SOURCE, c_path, "-lm"],
                   check=True)
    mutant = oracle.Oracle(so_path)
    failed = []
    for pin in ALL_BWD_PINS:
        try:
            pin(mutant)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every gradient pin"

"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that the pins catch
every one: a dropped term, a wrong sign, a wrong index or operand, a wrong order of steps."""
import os
import subprocess
import tempfile

import pytest

import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "kda_oracle.c")

FORGET = """    for (int i = 0; i < dk; ++i) {
        double alpha = exp(ld(g, g_dt, qk_off + i));
        for (int j = 0; j < dv; ++j) S[i * dv + j] *= alpha;
    }
"""
READOUT_START = "    /* read-out o = scale * S^T q */\n"
INNOV_START = "    /* innovation u = v - S^T k */\n"


def _swap_forget_after_write(s):
    assert FORGET in s
    s = s.replace(FORGET, "", 1)
    return s.replace(READOUT_START, FORGET + READOUT_START, 1)


def _readout_before_write(s):
    a, b = s.index(INNOV_START), s.index(READOUT_START)
    end = s.index("\n}\n", b)
    readout = s[b:end] + "\n"
    return s[:a] + readout + s[a:b] + s[end:]


MUTANTS = {
    "no_forget": lambda s: s.replace("S[i * dv + j] *= alpha;", "S[i * dv + j] *= 1.0;"),
    "forget_wrong_channel": lambda s: s.replace("exp(ld(g, g_dt, qk_off + i));",
                                                "exp(ld(g, g_dt, qk_off + (i + 1) % dk));"),
    "innovation_sign": lambda s: s.replace("u[j] -= S[i * dv + j] * ki;",
                                           "u[j] += S[i * dv + j] * ki;"),
    "no_beta": lambda s: s.replace("double bk = b * ld(k, in_dt, qk_off + i);",
                                   "double bk = ld(k, in_dt, qk_off + i);"),
    "write_with_q": lambda s: s.replace("double bk = b * ld(k, in_dt, qk_off + i);",
                                        "double bk = b * ld(q, in_dt, qk_off + i);"),
    "readout_with_k": lambda s: s.replace("double qi = ld(q, in_dt, qk_off + i);",
                                          "double qi = ld(k, in_dt, qk_off + i);"),
    "no_scale": lambda s: s.replace("o_row[j] *= scale;", "o_row[j] *= 1.0;"),
    "forget_after_write": _swap_forget_after_write,
    "readout_before_write": _readout_before_write,
    "gate_sign": lambda s: s.replace("1.0 / (1.0 + exp(-x));", "1.0 / (1.0 + exp(x));"),
    "gate_no_exp_A": lambda s: s.replace("double x = exp(ld(A, a_dt, (int64_t)h * dk + c))",
                                         "double x = (ld(A, a_dt, (int64_t)h * dk + c))"),
    "bf16_upcast_shift": lambda s: s.replace("[i]) << 16;", "[i]) << 15;"),
    "decode_wrong_unit": lambda s: s.replace("uidx * dv, uidx, scale, u, o ? o + uidx * dv",
                                             "uidx * dv, (uidx + 1) % units, scale, u, o ? o + uidx * dv"),
}


@pytest.fixture(scope="module")
def mutant_dir():
    with tempfile.TemporaryDirectory() as d:
        yield d


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, mutant_dir):
    src = open(SRC).read()
    mutated = MUTANTS[name](src)
    assert mutated != src, f"mutation {name} did not apply"
    cpath = os.path.join(mutant_dir, f"{name}.c")
    lpath = os.path.join(mutant_dir, f"lib{name}.so")
    with open(cpath, "w") as f:
        f.write(mutated)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", lpath, cpath,
                    "-lm"], check=True)
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(lpath)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"no pin caught mutant {name}"

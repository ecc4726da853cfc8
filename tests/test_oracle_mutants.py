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


# ---- oracle.forward_units: deliberately broken copies of the Python wrapper, each of which the
# forward_units pin must reject (the C loop is the real one, so only the unit bookkeeping changes)
UNIT_MUTANTS = {
    "packed_tok0_off_by_one": ("tok0 = int(cu[n]) if", "tok0 = max(int(cu[n]) - 1, 0) if"),
    "fixed_tok0_off_by_one": ("else n * T\n        length", "else max(n * T - 1, 0)\n        length"),
    "short_length": ("length = int(cu[n + 1] - cu[n]) if cu is not None else T",
                     "length = max(int(cu[n + 1] - cu[n]) - 1, 0) if cu is not None else T - 1"),
    "wrong_S0_sequence": ("np.array(s0[n, h], dtype", "np.array(s0[(n + 1) % s0.shape[0], h], dtype"),
    "wrong_S0_head": ("np.array(s0[n, h], dtype", "np.array(s0[n, (h + 1) % H], dtype"),
    "S0_ignored": ("S = np.array(s0[n, h], dtype=np.float64) if sdt != _BF16 else None",
                   "S = np.zeros((dk, dv)) if sdt != _BF16 else None"),
    "wrong_head": ("tok0, length, H, h,", "tok0, length, H, (h + 1) % H,"),
    "no_scale": ("dk, dv, float(scale), _p(S), _p(o_u)", "dk, dv, 1.0, _p(S), _p(o_u)"),
}


@pytest.mark.parametrize("name", sorted(UNIT_MUTANTS))
def test_forward_units_pin_catches_mutant(name):
    import inspect

    import oracle
    src = inspect.getsource(oracle.forward_units)
    old, new = UNIT_MUTANTS[name]
    assert src.count(old) == 1, f"mutation {name} did not apply"
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new), f"<forward_units mutant {name}>", "exec"), ns)
    with pytest.raises(AssertionError):
        oracle_pins.check_forward_units(None, forward_units=ns["forward_units"])


def test_forward_units_pin_passes_unmodified_copy():
    """The same recompilation without a mutation passes, so the rejections above come from the
    mutations themselves."""
    import inspect

    import oracle
    ns = dict(vars(oracle))
    exec(compile(inspect.getsource(oracle.forward_units), "<forward_units copy>", "exec"), ns)
    oracle_pins.check_forward_units(None, forward_units=ns["forward_units"])

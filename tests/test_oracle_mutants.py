"""The oracle's pins catch plausible mistakes (CPU only).

Each case copies ``oracle/disco_oracle.c``, plants one mistake in one function
(a reversed longitude shift, a dropped subsampling factor, a flipped latitude, a
dropped CSR entry, a transposed or reversed weight index, a dropped basis term,
a scatter to the wrong column, a missing absolute value), builds the copy with
gcc, and runs the pin suite (``test_oracle_pins.py``) against it in a
subprocess through ``DISCO_ORACLE_LIB``.  The case passes when at least one pin
fails on the mutant.  Every planted mistake keeps all indices in range, so a
mutant fails by value, never by a crash.  The oracle itself is untouched.
"""
import os
import re
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "disco_oracle.c")

SHIFT = "(int64_t)col_wi[e] + (int64_t)s * wo) % Wi"
W_IDX = "W[((int64_t)o * C + c) * K + k]"

# (function, text in that function, replacement)
MUTANTS = {
    "fwd_shift_reversed": ("oracle_fwd", SHIFT, "(int64_t)col_wi[e] + (int64_t)(Wi - s) * wo) % Wi"),
    "fwd_subsampling_dropped": ("oracle_fwd", SHIFT, "(int64_t)col_wi[e] + (int64_t)wo) % Wi"),
    "fwd_latitude_flipped": ("oracle_fwd", "xp + (int64_t)col_hi[e] * Wi", "xp + (int64_t)(Hi - 1 - col_hi[e]) * Wi"),
    "fwd_first_entry_dropped": ("oracle_fwd", "for (int64_t e = row_ptr[r]; e", "for (int64_t e = row_ptr[r] + 1; e"),
    "fwd_abs_of_x_dropped": ("oracle_fwd", "opnd((double)xrow[wi], abs_mode)", "(double)xrow[wi]"),
    "bwd_shift_reversed": ("oracle_bwd", SHIFT, "(int64_t)col_wi[e] + (int64_t)(Wi - s) * wo) % Wi"),
    "bwd_output_index_off_by_one": ("oracle_bwd", "opnd((double)go[wo], abs_mode)",
                                    "opnd((double)go[(wo + 1) % Wo], abs_mode)"),
    "fused_basis_reversed": ("oracle_fused", W_IDX, "W[((int64_t)o * C + c) * K + (K - 1 - k)]"),
    "fused_channel_reversed": ("oracle_fused", W_IDX, "W[((int64_t)o * C + (C - 1 - c)) * K + k]"),
    "einsum_first_basis_dropped": ("oracle_einsum", "for (int k = 0; k < K; ++k) {", "for (int k = 1; k < K; ++k) {"),
    "einsum_basis_reversed": ("oracle_einsum", W_IDX, "W[((int64_t)o * C + c) * K + (K - 1 - k)]"),
    "fused_bwd_gx_shifted": ("oracle_fused_bwd", "grow[wi] += v * gr[wo];", "grow[wi] += v * gr[(wo + 1) % Wo];"),
    "fused_bwd_dw_basis_reversed": ("oracle_fused_bwd", "dW[((int64_t)o * C + c) * K + k] += acc;",
                                    "dW[((int64_t)o * C + c) * K + (K - 1 - k)] += acc;"),
    "fused_bwd_g_sign": ("oracle_fused_bwd", "const double wv = opnd(", "const double wv = -opnd("),
}


def _mutate(src: str, func: str, old: str, new: str) -> str:
    """Replace `old` by `new` once, inside the body of C function `func` only."""
    m = re.search(r"^void " + func + r"\(", src, flags=re.M)
    assert m, func
    end = src.index("\n}\n", m.start())
    body = src[m.start():end]
    assert body.count(old) >= 1, (func, old)
    return src[:m.start()] + body.replace(old, new, 1) + src[end:]


def _run_pins(src: str, tmp_path):
    c = tmp_path / "mutant.c"
    c.write_text(src)
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
                    str(c), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, DISCO_ORACLE_LIB=str(lib), OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle_pins.py")], env=env, cwd=os.path.dirname(HERE),
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def test_unmodified_copy_passes(tmp_path):
    # control: the harness itself (copy, gcc -O1, subprocess, DISCO_ORACLE_LIB) changes nothing
    rc, tail = _run_pins(open(SRC).read(), tmp_path)
    assert rc == 0, tail


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    func, old, new = MUTANTS[name]
    rc, tail = _run_pins(_mutate(open(SRC).read(), func, old, new), tmp_path)
    assert rc == 1, f"pins did not fail cleanly on mutant {name} (rc {rc}):\n{tail}"
    assert re.search(r"\b1 failed\b", tail), tail

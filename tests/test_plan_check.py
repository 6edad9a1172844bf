"""Host plan code under the address and undefined-behaviour sanitizers (CPU only).

`sparse_gather_contraction_amd/csrc/plan_check.cpp` builds every plan that
disco_psi_create builds (plain, LDS-staged for 4- and 2-byte elements, register-tiled;
the phase-split matrix-core plans of the fused conv, the forward and the backward over
the row-inverted CSR), replays each kernel's indexing on the CPU and checks that every
index stays inside the buffer it addresses (for the matrix-core plans: descriptors, every
lane's psi words and x runs, stage sizes against the LDS budgets), that every destination
element of the gathers is written exactly once, that the replay reproduces the CSR
definition in fp64 (the matrix-core replay sums each block's 16 offsets per A row and B
column as v_mfma_f32_32x32x16 does), that the row-inverted CSR reproduces the backward,
and that the tiled kernel's workgroup decode serves every (task, plane) pair.  A plan bug
would otherwise surface as a GPU memory fault.  The checker is compiled here with g++ and
-fsanitize=address,undefined.
"""
import os
import subprocess

import numpy as np
import pytest

from disco_inputs import WORKLOADS, workload_psi
from disco_inputs.psi import build_psi, random_psi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_gather_contraction_amd", "csrc")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("plan_check") / "plan_check")
    cmd = ["g++", "-O2", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-I", CSRC,
           os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "plan_fused.cpp"), os.path.join(CSRC, "plan_tile.cpp"),
           os.path.join(CSRC, "plan_check.cpp"), "-o", out]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    return out


def _write_csr(p, path):
    with open(path, "wb") as f:
        np.array([p.K, p.Ho, p.Wo, p.Hi, p.Wi], np.int32).tofile(f)
        np.array([int(np.asarray(p.row_ptr)[-1])], np.int64).tofile(f)
        np.asarray(p.row_ptr, np.int64).tofile(f)
        np.asarray(p.col_hi, np.int32).tofile(f)
        np.asarray(p.col_wi, np.int32).tofile(f)
        np.asarray(p.val, np.float32).tofile(f)


def _run(checker, psi, tmp_path):
    path = str(tmp_path / "psi.csr")
    _write_csr(psi, path)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([checker, path], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env,
                       timeout=600)
    assert r.returncode == 0, r.stdout
    return r.stdout


CASES = {
    # Hi, Wi, Ho, Wo, theta_c, n_r, n_a (generated hat-basis psi)
    "caps_s3": lambda: build_psi(31, 60, 16, 20, 0.5, 2, 2),
    "whole_rings_k12": lambda: build_psi(31, 60, 31, 20, 1.5, 3, 4),
    "k8_s3": lambda: build_psi(37, 72, 19, 24, 0.9, 4, 2),
    "k16_s1": lambda: build_psi(31, 64, 31, 64, 1.5, 4, 4),
    # random CSRs: empty rows, dense rows (long runs), odd row lengths, the row-length limits of
    # the tiled kernel (192 / 193 and 384), rows longer than every staged plan
    "rand_long": lambda: random_psi(3, 4, 1100, 5, 2200, 0.05, seed=11, empty_rows=(0, 5, 11)),
    "rand_dense": lambda: random_psi(2, 3, 40, 4, 80, 0.9, seed=12, empty_rows=(1,)),
    "rand_empty": lambda: random_psi(2, 5, 16, 6, 32, 0.2, seed=13, empty_rows=(0, 3, 7)),
    "rand_odd_s1": lambda: random_psi(3, 7, 15, 9, 15, 0.3, seed=5),
    "rand_odd_s2": lambda: random_psi(2, 7, 13, 9, 26, 0.3, seed=6),
    "rand_L384": lambda: random_psi(2, 3, 384, 4, 768, 0.02, seed=7),
    "rand_L193": lambda: random_psi(2, 3, 193, 4, 386, 0.05, seed=8),
    "rand_L192": lambda: random_psi(3, 3, 192, 4, 384, 0.05, seed=9),
    # matrix-core plans: K = 16 at s = 1 with resident latitudes (two psi copies) and streamed
    # ones (rows cut into sub-rows, realigned psi reads); K = 8 at s = 2
    "phase_k16_s1_resident_and_streamed": lambda: build_psi(33, 512, 33, 512, 0.5, 4, 4),
    "phase_k8_s2": lambda: build_psi(25, 768, 25, 384, 0.5, 4, 2),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_plans_of_generated_and_random_psi(checker, name, tmp_path):
    _run(checker, CASES[name](), tmp_path)


@pytest.mark.parametrize("name", ["tiny_fwd_f32_16x32", "fwdbwd_f32_181x360"])
def test_plans_of_the_fp32_workloads(checker, name, tmp_path):
    out = _run(checker, workload_psi(WORKLOADS[name]), tmp_path)
    assert "tiled fwd on" in out and "bwd on" in out  # both fp32 workloads run the tiled kernel


def test_checker_catches_a_bad_plan_index(checker, tmp_path):
    """The checker must fail on a CSR it rejects (a column outside the grid): exit status 3."""
    p = random_psi(2, 3, 16, 4, 32, 0.3, seed=21)
    col_wi = np.asarray(p.col_wi).copy()
    col_wi[0] = 32  # == Wi: outside [0, Wi)
    bad = type(p)(p.K, p.Ho, p.Wo, p.Hi, p.Wi, p.row_ptr, p.col_hi, col_wi, p.val)
    path = str(tmp_path / "bad.csr")
    _write_csr(bad, path)
    r = subprocess.run([checker, path], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=60)
    assert r.returncode == 3 and "CSR rejected" in r.stdout


MUTANTS = {
    # each replaces one line of plan_tile.cpp with a plausible mistake the checker must catch
    "window offset drops the residue row": ("rec.a = 4 * ((slot * out.deint + rho) * out.lrow + rec.j0);",
                                            "rec.a = 4 * ((slot * out.deint) * out.lrow + rec.j0);"),
    "first shift off by one": ("rec.j0 = (sg.j0 + off) % L;", "rec.j0 = (sg.j0 + off + 1) % L;"),
    "wrap threshold off by one": ("rec.w = L - rec.j0;", "rec.w = L - rec.j0 + 1;"),
    "halo too short for the longest record": ("out.lrow = (L + kTileHalo + 3) / 4 * 4;",
                                              "out.lrow = (L + 4 + 3) / 4 * 4;"),
    "first-stage descriptor of the last stage": (
        "out.task_first.push_back(t.stage_begin < t.stage_end ? out.stages[t.stage_begin]",
        "out.task_first.push_back(t.stage_begin < t.stage_end ? out.stages[t.stage_end - 1]"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_checker_catches_planted_plan_mistakes(name, tmp_path):
    """Sensitivity: a copy of plan_tile.cpp with one planted mistake must fail the checker on the
    181x360 workload's psi (built without sanitizers, only the outcome matters)."""
    old, new = MUTANTS[name]
    src = open(os.path.join(CSRC, "plan_tile.cpp")).read()
    assert src.count(old) == 1, name
    mut = tmp_path / "plan_tile_mut.cpp"
    mut.write_text(src.replace(old, new))
    exe = str(tmp_path / "plan_check_mut")
    cmd = ["g++", "-O1", "-std=c++17", "-I", CSRC, os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "plan_fused.cpp"),
           str(mut), os.path.join(CSRC, "plan_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    path = str(tmp_path / "psi.csr")
    _write_csr(workload_psi(WORKLOADS["fwdbwd_f32_181x360"]), path)
    r = subprocess.run([exe, path], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    assert r.returncode == 1 and "FAIL:" in r.stdout, r.stdout[-2000:]


WINDOW_MUTANTS = {
    # each replaces one line of plan.cpp's window builder with a plausible mistake the checker must catch
    "window arc one shift short": ("span = std::max(span, (sg.j0 - a + L) % L + sg.m);",
                                   "span = std::max(span, (sg.j0 - a + L) % L + sg.m - 1);"),
    "window offset ignores the arc start": ("out.seg_off[q] = base + (p.segs[q].j0 - best_a + L) % L;",
                                            "out.seg_off[q] = base + p.segs[q].j0 % L;"),
    "window misses the tile's last longitude": ("w.len = best_span + px - 1;", "w.len = best_span + px - 2;"),
}


@pytest.mark.parametrize("name", sorted(WINDOW_MUTANTS))
def test_checker_catches_planted_window_mistakes(name, tmp_path):
    """Sensitivity of the fused kernels' window replay: a copy of plan.cpp with one planted mistake in
    the window builder must fail the checker on the 181x360 workload's psi."""
    old, new = WINDOW_MUTANTS[name]
    src = open(os.path.join(CSRC, "plan.cpp")).read()
    assert src.count(old) == 1, name
    mut = tmp_path / "plan_mut.cpp"
    mut.write_text(src.replace(old, new))
    exe = str(tmp_path / "plan_check_mut")
    cmd = ["g++", "-O1", "-std=c++17", "-I", CSRC, str(mut), os.path.join(CSRC, "plan_fused.cpp"),
           os.path.join(CSRC, "plan_tile.cpp"), os.path.join(CSRC, "plan_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    path = str(tmp_path / "psi.csr")
    _write_csr(workload_psi(WORKLOADS["fwdbwd_f32_181x360"]), path)
    r = subprocess.run([exe, path], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    assert r.returncode == 1 and "fused windows" in r.stdout, r.stdout[-2000:]


FUSED_MUTANTS = {
    # each replaces one line of plan_fused.cpp with a plausible mistake the checker must catch
    "psi offset drops the 8s lead": ("out.descs.push_back(2 * kr * (a_row_e + (t0 - first) + 8 * s));",
                                     "out.descs.push_back(2 * kr * (a_row_e + (t0 - first)));"),
    "window offset one run late": ("out.descs.push_back((s == 2 ? 1 : 2) * (win_off + (t0 - first)));",
                                   "out.descs.push_back((s == 2 ? 1 : 2) * (win_off + (t0 - first) + 8));"),
    "second psi copy not shifted": ("if (copies == 2) put_pairs(copy1, copy1_16, m, first - 8 * s, ra, 1);",
                                    "if (copies == 2) put_pairs(copy1, copy1_16, m, first - 8 * s, ra, 0);"),
    "realigned psi tail too short": ("tail = realign ? 18 : 16;", "tail = 16;"),
    "inverse CSR shift sign": ("out.col_wi[dst] = (c.Wo - (wi - rho) / s) % c.Wo;",
                               "out.col_wi[dst] = (c.Wo + (wi - rho) / s) % c.Wo;"),
    "last block of a row dropped": ("for (int32_t t0 = T0; t0 == T0 || t0 - 1 - smax < tmax; t0 += kBlkJ) {",
                                    "for (int32_t t0 = T0; t0 == T0 || t0 + 15 - smax < tmax; t0 += kBlkJ) {"),
    "transposed CSR offset not negated": ("out.col_wi[dst] = (c.Wo - c.col_wi[e]) % c.Wo;",
                                          "out.col_wi[dst] = c.col_wi[e];"),
    "transposed CSR column keeps the input latitude": ("out.col_hi[dst] = ho;", "out.col_hi[dst] = c.col_hi[e];"),
}


@pytest.mark.parametrize("name", sorted(FUSED_MUTANTS))
def test_checker_catches_planted_matrix_core_plan_mistakes(name, tmp_path):
    """Sensitivity of the matrix-core replay: a copy of plan_fused.cpp with one planted mistake must
    fail the checker on a K = 16 psi with both resident and streamed latitudes."""
    old, new = FUSED_MUTANTS[name]
    src = open(os.path.join(CSRC, "plan_fused.cpp")).read()
    assert src.count(old) == 1, name
    mut = tmp_path / "plan_fused_mut.cpp"
    mut.write_text(src.replace(old, new))
    exe = str(tmp_path / "plan_check_mut")
    cmd = ["g++", "-O1", "-std=c++17", "-I", CSRC, os.path.join(CSRC, "plan.cpp"), str(mut),
           os.path.join(CSRC, "plan_tile.cpp"), os.path.join(CSRC, "plan_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    path = str(tmp_path / "psi.csr")
    _write_csr(CASES["phase_k16_s1_resident_and_streamed"](), path)
    r = subprocess.run([exe, path], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    assert r.returncode == 1 and "FAIL:" in r.stdout, r.stdout[-2000:]

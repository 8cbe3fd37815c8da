"""Host checks (no GPU) that the quantize kernels' FMA-corrected quotient decides every
FP8 / INT8 code exactly as the IEEE fp32 division x / s does: over all bf16 inputs and the
per-row scales amax / qmax, and over all significand pairs for an arbitrary scale."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "quotient_shortcut.c")


@pytest.fixture(scope="module")
def binary(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    out = str(tmp_path_factory.mktemp("qs") / "quotient_shortcut")
    # -ffp-contract=off keeps x * r and the FMAs exactly as written (no extra fusion).
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", SRC, "-o", out, "-lm"], check=True)
    return out


@pytest.mark.parametrize("qmax", ["448", "127"])
def test_shortcut_matches_ieee_division(binary, qmax):
    env = dict(os.environ)
    env.setdefault("OMP_NUM_THREADS", str(min(16, os.cpu_count() or 1)))
    r = subprocess.run([binary, qmax], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "harmful=0" in r.stdout and "signflip=0" in r.stdout


SRC_ANY = os.path.join(HERE, "native", "quotient_any_scale.c")


def test_shortcut_is_ieee_for_any_scale(tmp_path):
    """Every bf16 significand of x against every fp32 significand of s: the static
    quantizer's FMA-corrected quotient equals x / s bit for bit."""
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    out = str(tmp_path / "quotient_any_scale")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", SRC_ANY, "-o", out, "-lm"], check=True)
    env = dict(os.environ)
    env.setdefault("OMP_NUM_THREADS", str(min(16, os.cpu_count() or 1)))
    r = subprocess.run([out], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "differ=0" in r.stdout

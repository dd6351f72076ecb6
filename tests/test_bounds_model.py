"""CPU check of the kernels' addressing: tests/bounds/bounds_model.cpp writes
out on the host every global load and store, buffer-descriptor range and LDS
index of the decode step, the window close / encode and the FP32 baseline,
for every thread, and checks them against the C ABI's buffer sizes and the LDS
arrays over all
(d, bits, decay, activation) instantiations, r = 0..8, buffer capacities up to
64 and every buffer length a launch accepts. Planted mistakes (an LDS array one
row short, a state one entry row short per head, a compensator's G row
addressed inside its descriptor, the baseline's pieces shifted by one) must be
caught."""
import os
import shutil
import subprocess

import pytest

SRC = os.path.join(os.path.dirname(__file__), "bounds", "bounds_model.cpp")


def _run(tmp_path, *defs):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "bounds_model")
    subprocess.run([gxx, "-O2", "-std=c++17", *defs, SRC, "-o", exe], check=True)
    return subprocess.run([exe], capture_output=True, text=True, timeout=300)


def test_kernel_addressing_stays_inside_every_buffer(tmp_path):
    res = _run(tmp_path)
    print(res.stdout)
    assert res.returncode == 0, res.stdout
    assert "all inside their buffers" in res.stdout


@pytest.mark.parametrize("define,what", [("-DMODEL_KAPPA_ROWS=71", "lds kappa"),
                                         ("-DMODEL_ENTRY_SLACK=1", ""),
                                         ("-DMODEL_G_COMP_OFF=0", "compensator G offset"),
                                         ("-DMODEL_BL_PIECE_OFF=1", "baseline state piece")])
def test_planted_mistakes_are_caught(tmp_path, define, what):
    res = _run(tmp_path, define)
    assert res.returncode == 1
    assert res.stdout.startswith("VIOLATION") and what in res.stdout, res.stdout

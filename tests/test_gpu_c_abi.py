"""The C ABI from plain C (tests/c/abi_solve.c, built with the library): a
2D Poisson CSR in caller-owned device memory through create, PCG, matvec,
adjoint, BiCGStab on a non-symmetric variant and a refused call; the PCG
solution it writes is compared with the oracle's on the same matrix, and the
path the solve took (sla_csr_get_last_path) is checked for consistency."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from workloads import poisson2d_coo

pytestmark = pytest.mark.gpu
BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "abi_solve")


def test_plain_c_program(tmp_path):
    N = 48
    out = tmp_path / "x.bin"
    res = subprocess.run([BIN, str(N), str(out)], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0, (res.returncode, res.stdout, res.stderr)
    fields = dict(kv.split("=", 1) for kv in res.stdout.split() if "=" in kv)
    assert fields["status"] == "0" and fields["refused"] == "1"
    # the 48^2 Poisson system fits the single-kernel solve; if the per-step
    # kernels ran instead, it must be because the cooperative launch was
    # refused (a process started by one that made cooperative launches can
    # be refused on this GPU), and the library must say so
    path, fallbacks = int(fields["path"]), int(fields["fallbacks"])
    assert path in (1, 2)
    if path == 1:
        assert fallbacks == 0
    else:
        assert fallbacks == 1
    x = np.fromfile(out, dtype=np.float64)
    r, c, v = poisson2d_coo(N)
    ref = oracle.coo_to_csr(N * N, r, c, v)
    b = np.sin(0.1 * np.arange(N * N)) + 0.5
    xo, ito, _, _ = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, 1e-10, 5000)
    assert abs(int(fields["iterations"]) - ito) <= 2
    assert np.linalg.norm(x - xo) <= 1e-8 * np.linalg.norm(xo)

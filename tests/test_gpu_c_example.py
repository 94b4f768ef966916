"""The route from plain C: tests/c_abi/route_example.c (built by build() next
to the library) prepares a decode plan, runs route_fused and the two-call
route on an 8-row batch through the C ABI and the HIP runtime API, and checks
what holds for any inputs: fused equals two calls bit for bit, each row's
selection is a valid top-16 of the returned logits with weights summing to
1, sampled latent values are within one BF16 ULP of a host double dot, and a
call above the plan's rows is rejected without writing."""
import os
import subprocess

import pytest

from latent_projection_top_amd import build as route_build
from tests.routekit import log

pytestmark = pytest.mark.gpu


def test_c_example_runs():
    exe = route_build.EXAMPLE_EXE
    if not os.path.exists(exe):
        pytest.skip(f"{exe} is not built (build() links it next to the library)")
    log(f"running {exe}")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    log(r.stdout.strip())
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c example ok" in r.stdout

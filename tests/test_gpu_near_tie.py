"""Near-tie gate of the standalone top-16 on the GPU.

Page "Kimi K3.1 recipe: route 9..20 decode rows through the pushed pair gather
and standalone top-16", "Claims and caveats": a near-tie gate over 3.2M rows at
9/12/16/20 rows per call found every set difference to be a 1-for-1 swap within
2 fp32 ULP. Here the logits are fed straight to route_topk16 (no projection in
front), so the selection must be bit-exact: 3.24M synthetic rows with the 17th
value planted 0..4 ULP under the 16th, exact 3- and 5-way ties across the
boundary, +0.0/-0.0 boundaries and all-equal rows, in 9/12/16/20-row calls."""
import concurrent.futures as cf
import ctypes

import numpy as np
import pytest
import torch

from oracle import compare
from oracle import route_oracle as orc
from synth import generators as gen
from tests.routekit import log

pytestmark = pytest.mark.gpu

route = pytest.importorskip("latent_projection_top_amd.route")

CHUNK = 18000            # a multiple of 9, 12, 16 and 20
CHUNKS_PER_WIDTH = 45    # 45 x 18000 = 810,000 rows per width, 3.24M in all


def _prepare(width: int, c: int):
    L = gen.near_tie_logits(CHUNK, chunk=width * 1000 + c)
    ids = orc.topk16_ref(L)
    return L, ids, orc.route_weights_ref(L, ids)


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("width", [9, 12, 16, 20])
def test_near_tie_gate(width):
    log(f"near-tie gate width={width}: {CHUNK * CHUNKS_PER_WIDTH} rows")
    plan = route.Plan(route.MODE_DECODE, width)
    h = ctypes.c_void_p(plan.handle)
    lg = torch.empty((CHUNK, 896), dtype=torch.float32, device="cuda")
    ids = torch.empty((CHUNK, 16), dtype=torch.int32, device="cuda")
    wts = torch.empty((CHUNK, 16), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream or None
    bad_rows = 0
    max_w_ulp = 0
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        futs = [ex.submit(_prepare, width, c) for c in range(CHUNKS_PER_WIDTH)]
        for c, f in enumerate(futs):
            L, ref_ids, ref_w = f.result()
            lg.copy_(torch.from_numpy(L))
            ids.fill_(-1)
            base_l, base_i, base_w = lg.data_ptr(), ids.data_ptr(), wts.data_ptr()
            for s in range(0, CHUNK, width):
                st = route.LIB.route_topk16(h, base_l + s * 896 * 4, base_i + s * 64,
                                            base_w + s * 64, width, stream)
                assert st == 0
            got_ids = ids.cpu().numpy()
            got_w = wts.cpu().numpy()
            bad = (got_ids != ref_ids).any(axis=1)
            bad_rows += int(bad.sum())
            fin = np.isfinite(ref_w).all(axis=1)
            d = compare.f32_ulp_distance(got_w[fin], ref_w[fin])
            max_w_ulp = max(max_w_ulp, int(d.max()))
            if c % 15 == 0:
                log(f"  chunk {c}: bad rows so far {bad_rows}, weights max ulp {max_w_ulp}")
    assert bad_rows == 0
    assert max_w_ulp <= 5

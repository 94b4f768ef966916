"""GPU parity of the prefill route (up to 3072 rows) through the C ABI.

Workload: 3072-row chunks (page "Optionally gather the Kimi3 prefill latent
instead of reducing it", timing table) with 1 % of hidden channels scaled x20
as outliers. At this size the float64 oracle still runs on the host in
seconds, so every output is compared, for several banks; ragged row counts
check the M tail of the tiles."""
import numpy as np
import pytest
import torch

from oracle import compare
from oracle import route_oracle as orc
from synth import generators as gen
from tests.routekit import Outputs, assert_prefill_logit_error, bf16_dev, log, oracle_rows, weights_dev

pytestmark = pytest.mark.gpu

route = pytest.importorskip("latent_projection_top_amd.route")


def run_prefill(x_bits, cap=3072, fused=False):
    w, wr = weights_dev(0)
    rows = x_bits.shape[0]
    plan = route.Plan(route.MODE_PREFILL, cap)
    ws = plan.new_workspace()
    xd = bf16_dev(x_bits)
    out = Outputs(rows)
    out.poison()
    if fused:
        route.fused(plan, xd, w, wr, out.latent, out.logits, out.ids, out.weights, ws, rows=rows)
    else:
        route.latent_router(plan, xd, w, wr, out.latent, out.logits, ws, rows=rows)
        route.topk16(plan, out.logits, out.ids, out.weights, rows=rows)
    torch.cuda.synchronize()
    return out.host()


def check_outputs(xs, got, tag):
    ref = oracle_rows(xs)
    lc = compare.latent_check(got["latent"], ref["latent"], ref["exact"], ref["abs_terms"])
    gc = compare.logits_check(got["logits"], ref["logits"], ref["logits_exact"],
                              ref["logits_abs_terms"])
    ld = compare.f32_ulp_distance(got["logits"], ref["logits"])
    top = np.abs(ref["logits_exact"]) >= 1.0
    ic = compare.ids_check(got["ids"], ref["ids"], ref["logits"])
    wc = compare.weights_check(got["weights"], orc.route_weights_ref(got["logits"], got["ids"]))
    same = (got["ids"] == ref["ids"]).all(axis=1)
    wc2 = compare.weights_check(got["weights"][same], ref["weights"][same])
    log(f"{tag}: latent {lc} | logits {gc}, |l|>=1 ulp max {ld[top].max()} mean "
        f"{ld[top].mean():.3g} | ids equal {ic['equal']} swaps {ic['swaps']} viol "
        f"{ic['violations']} | weights max {wc['max_ulp']} / e2e {wc2['max_ulp']}")
    assert lc["fail"] == 0
    assert lc["rel_rms"] <= 2.0e-3
    assert lc["band"] <= max(4, 1e-4 * lc["n"])
    assert gc["fail"] == 0
    assert_prefill_logit_error(gc)
    assert ic["violations"] == 0, ic["bad_rows"][:5]
    assert wc["fail"] == 0 and wc2["fail"] == 0


@pytest.mark.timeout(900)
@pytest.mark.parametrize("bank", [0, 1, 2, 3])
def test_prefill_chunk_3072_outliers(bank):
    log(f"prefill 3072 rows, outliers, bank={bank}")
    xs = gen.hidden(3072, bank=500 + bank, outliers=True)
    got = run_prefill(xs, fused=(bank % 2 == 1))
    check_outputs(xs, got, f"prefill 3072 bank {bank}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("rows", [1, 77, 130, 191, 192, 193, 384, 700, 768, 769, 1000, 1536, 1537, 1700,
                                  1729, 2048, 2500, 2880, 3071])
def test_prefill_ragged(rows):
    """Row counts around the 192-row block tile and across the K splits of
    chunks with few row tiles: one row, a partial first tile, one row short
    of a tile, a whole tile (14 splits), one row into the second tile and two
    whole tiles (7), four tiles (4), six tiles (2), nine tiles (the router
    alone split in 2), then 10 to 16 row tiles (unsplit, fewer tiles than
    CUs: 11, 14, 15 and 16 here). Each change of split is tested on both
    sides: 768 / 769 rows (4 ways, then 2), 1,536 / 1,537 (both GEMMs in 2,
    then the router alone) and 1,700 / 1,729 (the router in 2, then
    neither)."""
    log(f"prefill ragged rows={rows}")
    xs = gen.hidden(rows, bank=600 + rows, outliers=True)
    got = run_prefill(xs, cap=3072)
    check_outputs(xs, got, f"prefill rows={rows}")


def test_prefill_fused_equals_two_calls():
    log("prefill fused == two calls")
    xs = gen.hidden(300, bank=9)
    a = run_prefill(xs, cap=512, fused=True)
    b = run_prefill(xs, cap=512, fused=False)
    for k in ("latent", "logits", "ids"):
        assert np.array_equal(a[k], b[k]), k
    assert np.array_equal(a["weights"].view(np.uint32), b["weights"].view(np.uint32))


def test_prefill_zero_rows_degenerate_case():
    """All-zero hidden rows inside a ragged chunk (200 rows, tile edges at 192):
    latent +0.0, logits all 0.0, ids 0..15, weights exactly 1/16."""
    log("prefill with all-zero hidden rows")
    xs = gen.hidden(200, bank=95, outliers=True)
    zero = [0, 100, 191, 192, 199]
    xs[zero] = 0
    got = run_prefill(xs, cap=256, fused=True)
    for r in zero:
        assert (got["latent"][r] == 0).all()
        assert (got["logits"][r].view(np.uint32) == 0).all()
        assert np.array_equal(got["ids"][r], np.arange(16))
        assert (got["weights"][r] == np.float32(1.0 / 16.0)).all()
    check_outputs(xs, got, "prefill rows=200 with zero rows")


@pytest.mark.parametrize("cap", [1, 100, 700])
def test_prefill_plan_at_its_capacity(cap):
    """Plans prepared for few rows size their workspace's K-split area for
    their own capacity (14, 14 and 4 splits here): a call at the capacity
    matches the oracle, packed and [K][N] alike, and the two agree bitwise."""
    log(f"prefill plan of capacity {cap}, call at capacity")
    w, wr = weights_dev(0)
    xs = gen.hidden(cap, bank=650 + cap, outliers=True)
    got = run_prefill(xs, cap=cap, fused=True)
    check_outputs(xs, got, f"prefill cap={cap}")
    plan = route.Plan(route.MODE_PREFILL, cap)
    ws = plan.new_workspace()
    pk = route.pack_weights(plan, w, wr)
    o = Outputs(cap)
    o.poison()
    route.fused_packed(plan, bf16_dev(xs), pk, o.latent, o.logits, o.ids, o.weights, ws)
    torch.cuda.synchronize()
    h = o.host()
    for k in ("latent", "ids"):
        assert np.array_equal(h[k], got[k]), k
    assert np.array_equal(h["logits"].view(np.uint32), got["logits"].view(np.uint32))

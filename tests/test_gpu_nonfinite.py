"""Hidden rows holding an infinity or a NaN: a degenerate input the route
passes through instead of hiding, with the other rows of the call untouched.

With x[r, k] = +-inf and no zero weight, every exact dot of row r is an
infinity with the sign of the weight (one infinite term, the rest finite), so
the latent row is BF16 +-inf, the logits are FP32 +-inf, the top-16 is the 16
lowest-indexed experts whose logit is +inf and each weight is exactly 1/16
(sigmoid(+inf) = 1). With x[r, k] = NaN the whole row is NaN, the top-16 is
experts 0..15 (NaN orders below -inf, ties go to the lower index) and the
weights are NaN. Both routes must give exactly the oracle's values on such
rows: the decode route's FP64 sums keep the single infinite term, and the
prefill route recomputes every logit its GEMM returned non-finite as an exact
FP64 dot (the GEMM's three BF16 parts of a weight would turn an infinite term
into inf - inf)."""
import numpy as np
import pytest
import torch

from oracle import compare
from oracle import route_oracle as orc
from synth import generators as gen
from tests.routekit import (Outputs, assert_fp64_logits, assert_prefill_logit_error, bf16_dev, bits_host, log, oracle_rows,
                            weights_dev)

pytestmark = pytest.mark.gpu

route = pytest.importorskip("latent_projection_top_amd.route")

BF16_POS_INF, BF16_NEG_INF, BF16_NAN = 0x7F80, 0xFF80, 0x7FC0


def poisoned_rows(rows: int, bank: int):
    """Rows 1, 3, 5 and (from 18 rows) 17 and 19, whose decode router logits
    run on the FP64 VALU at 17..20 rows; past 20 rows also the chunk's last
    rows."""
    xs = gen.hidden(rows, bank=bank)
    bad = {1: (100, BF16_POS_INF), 3: (5000, BF16_NEG_INF), 5: (7, BF16_NAN),
           17: (3000, BF16_NEG_INF), 19: (7100, BF16_NAN)}
    if rows > 20:
        bad.update({rows - 6: (7167, BF16_POS_INF), rows - 1: (0, BF16_NAN)})
    bad = {r: kv for r, kv in bad.items() if r < rows}
    for r, (k, v) in bad.items():
        xs[r, k] = v
    return xs, sorted(bad)


def bf16_is_nan(bits):
    return ((bits & 0x7F80) == 0x7F80) & ((bits & 0x007F) != 0)


def check_bad_rows(got, ref, bad, exact_logits: bool):
    for r in bad:
        gl, rl = got["latent"][r], ref["latent"][r]
        assert np.array_equal(bf16_is_nan(gl), bf16_is_nan(rl)), r
        fin = ~bf16_is_nan(rl)
        assert np.array_equal(gl[fin], rl[fin]), r
        g, e = got["logits"][r], ref["logits"][r]
        if exact_logits:
            assert np.array_equal(np.isnan(g), np.isnan(e)), r
            assert np.array_equal(g[~np.isnan(e)], e[~np.isnan(e)]), r
            assert np.array_equal(got["ids"][r], ref["ids"][r]), r
        else:
            assert np.array_equal(np.isfinite(g), np.isfinite(e)), r
            assert np.array_equal(got["ids"][r], orc.topk16_ref(g[None])[0]), r
        w = got["weights"][r]
        if np.isnan(e).all():
            assert np.isnan(w).all() and np.array_equal(got["ids"][r], np.arange(16)), r
        elif exact_logits:
            assert (w == np.float32(1.0 / 16.0)).all(), r


def check_good_rows(got, ref, good, logits_ulp: bool):
    sub = {k: v[good] for k, v in got.items()}
    rsub = {k: v[good] for k, v in ref.items()}
    lc = compare.latent_check(sub["latent"], rsub["latent"], rsub["exact"], rsub["abs_terms"])
    assert lc["fail"] == 0 and lc["rel_rms"] <= 2.0e-3, lc
    if logits_ulp:
        assert_fp64_logits(sub["logits"], rsub["logits"])
    else:
        gc = compare.logits_check(sub["logits"], rsub["logits"], rsub["logits_exact"],
                                  rsub["logits_abs_terms"])
        assert gc["fail"] == 0, gc
        assert_prefill_logit_error(gc)
    ic = compare.ids_check(sub["ids"], rsub["ids"], rsub["logits"])
    assert ic["violations"] == 0, ic["bad_rows"][:5]
    wc = compare.weights_check(sub["weights"], orc.route_weights_ref(sub["logits"], sub["ids"]))
    assert wc["fail"] == 0


@pytest.mark.parametrize("packed", [False, True])
def test_decode_nonfinite_rows(packed):
    log(f"decode with inf / NaN hidden values, packed={packed}")
    w, wr = weights_dev(0)
    for width in (4, 8, 20):
        xs, bad = poisoned_rows(width, bank=600 + width)
        plan = route.Plan(route.MODE_DECODE, width)
        ws = plan.new_workspace()
        o = Outputs(width)
        o.poison()
        if packed:
            pk = route.pack_weights(plan, w, wr)
            route.fused_packed(plan, bf16_dev(xs), pk, o.latent, o.logits, o.ids, o.weights, ws)
        else:
            route.fused(plan, bf16_dev(xs), w, wr, o.latent, o.logits, o.ids, o.weights, ws)
        torch.cuda.synchronize()
        got = {"latent": bits_host(o.latent), "logits": o.logits.cpu().numpy(),
               "ids": o.ids.cpu().numpy(), "weights": o.weights.cpu().numpy()}
        with np.errstate(invalid="ignore", over="ignore"):
            ref = oracle_rows(xs)
        check_bad_rows(got, ref, bad, exact_logits=True)
        good = np.array([r for r in range(width) if r not in bad])
        check_good_rows(got, ref, good, logits_ulp=True)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("rows", [96, 700, 2112])
@pytest.mark.parametrize("packed", [False, True])
def test_prefill_nonfinite_rows(packed, rows):
    """Both weight layouts, on a chunk whose GEMMs split K in 14 (96 rows) or
    4 (700 rows), where the router's combine pass recomputes the non-finite
    logits, and on one that does not split (2112 rows), where the router
    GEMM's own epilogue does."""
    log(f"prefill with inf / NaN hidden values, packed={packed}, rows={rows}")
    w, wr = weights_dev(0)
    xs, bad = poisoned_rows(rows, bank=700 + rows)
    plan = route.Plan(route.MODE_PREFILL, rows)
    ws = plan.new_workspace()
    o = Outputs(rows)
    o.poison()
    if packed:
        pk = route.pack_weights(plan, w, wr)
        route.fused_packed(plan, bf16_dev(xs), pk, o.latent, o.logits, o.ids, o.weights, ws)
    else:
        route.fused(plan, bf16_dev(xs), w, wr, o.latent, o.logits, o.ids, o.weights, ws)
    torch.cuda.synchronize()
    got = {"latent": bits_host(o.latent), "logits": o.logits.cpu().numpy(),
           "ids": o.ids.cpu().numpy(), "weights": o.weights.cpu().numpy()}
    with np.errstate(invalid="ignore", over="ignore"):
        ref = oracle_rows(xs)
    check_bad_rows(got, ref, bad, exact_logits=True)
    good = np.array([r for r in range(rows) if r not in bad])
    check_good_rows(got, ref, good, logits_ulp=False)


def test_prefill_nonfinite_latent_router_two_tiles():
    """route_latent_router alone (no top-16) on a 200-row chunk whose bad rows
    sit in two 64-row blocks of the recompute and two 192-row GEMM tiles: the
    same exact logits as the fused call."""
    log("prefill latent_router with inf / NaN hidden values, 200 rows")
    w, wr = weights_dev(0)
    rows = 200
    xs, bad = poisoned_rows(rows, bank=701)
    plan = route.Plan(route.MODE_PREFILL, rows)
    ws = plan.new_workspace()
    o = Outputs(rows)
    o.poison()
    route.latent_router(plan, bf16_dev(xs), w, wr, o.latent, o.logits, ws)
    torch.cuda.synchronize()
    g = o.logits.cpu().numpy()
    with np.errstate(invalid="ignore", over="ignore"):
        ref = oracle_rows(xs)
    for r in bad:
        e = ref["logits"][r]
        assert np.array_equal(np.isnan(g[r]), np.isnan(e)), r
        assert np.array_equal(g[r][~np.isnan(e)], e[~np.isnan(e)]), r
    assert np.isfinite(np.delete(g, bad, axis=0)).all()

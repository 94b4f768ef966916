"""The allocation-free entry point (route_fused_packed_noalloc) against the
entry point it varies (route_fused_packed with a caller workspace), on calls
in a row, each with fewer rows than the one before, for decode and prefill
plans, and both against the oracle: bitwise the same outputs wherever both
run the same launches (every decode call; prefill calls of more than 1,728
rows). Prefill calls of fewer rows split K in route_fused_packed, whose
workspace holds the split partials, and not in the allocation-free call, so
there the two are compared through the oracle's bounds. Nothing here
allocates between the calls but the test's own output tensors."""
import numpy as np
import pytest
import torch

from oracle import compare
from oracle import route_oracle as orc
from synth import generators as gen
from tests.routekit import Outputs, assert_fp64_logits, bf16_dev, log, oracle_rows, weights_dev

pytestmark = pytest.mark.gpu

route = pytest.importorskip("latent_projection_top_amd.route")


def run_pair(plan, xd, packed, rows, ws, with_logits):
    ref, got = Outputs(rows), Outputs(rows)
    ref.poison()
    got.poison()
    route.fused_packed(plan, xd, packed, ref.latent, ref.logits, ref.ids, ref.weights, ws, rows=rows)
    route.fused_packed_noalloc(plan, xd, packed, got.latent, got.logits if with_logits else None,
                               got.ids, got.weights, rows=rows)
    torch.cuda.synchronize()
    return ref.host(), got.host()


def assert_bitwise(r, g, with_logits):
    assert np.array_equal(r["latent"], g["latent"])
    assert np.array_equal(r["ids"], g["ids"])
    assert np.array_equal(r["weights"].view(np.uint32), g["weights"].view(np.uint32))
    if with_logits:
        assert np.array_equal(r["logits"].view(np.uint32), g["logits"].view(np.uint32))


def check_oracle(xs, g, decode):
    ref = oracle_rows(xs)
    lc = compare.latent_check(g["latent"], ref["latent"], ref["exact"], ref["abs_terms"])
    ic = compare.ids_check(g["ids"], ref["ids"], ref["logits"])
    assert lc["fail"] == 0 and lc["rel_rms"] <= 2.0e-3, lc
    assert ic["violations"] == 0, ic["bad_rows"][:5]
    if decode:
        assert_fp64_logits(g["logits"], ref["logits"])
        wc = compare.weights_check(g["weights"], orc.route_weights_ref(g["logits"], g["ids"]))
        assert wc["fail"] == 0


@pytest.mark.parametrize("with_logits", [True, False])
def test_noalloc_decode_two_calls(with_logits):
    w, wr = weights_dev(0)
    plan = route.Plan(route.MODE_DECODE, 20)
    ws = plan.new_workspace()
    packed = route.pack_weights(plan, w, wr)
    for rows, bank in ((20, 8100), (8, 8101), (1, 8102)):
        log(f"noalloc decode rows={rows} logits={'given' if with_logits else 'scratch'}")
        xs = gen.hidden(rows, bank=bank)
        r, g = run_pair(plan, bf16_dev(xs), packed, rows, ws, with_logits)
        assert_bitwise(r, g, with_logits)
        check_oracle(xs, r if not with_logits else g, decode=True)


def test_noalloc_prefill_two_calls_and_capacity():
    w, wr = weights_dev(0)
    plan = route.Plan(route.MODE_PREFILL, 3072)
    ws = plan.new_workspace()
    packed = route.pack_weights(plan, w, wr)
    for rows, bank, with_logits in ((3072, 8203, True), (2112, 8204, True), (300, 8202, True),
                                    (200, 8200, False), (77, 8201, False)):
        log(f"noalloc prefill rows={rows} logits={'given' if with_logits else 'scratch'}")
        xs = gen.hidden(rows, bank=bank, outliers=True)
        r, g = run_pair(plan, bf16_dev(xs), packed, rows, ws, with_logits)
        if rows > 1728:
            assert_bitwise(r, g, with_logits)
            if rows <= 2112:
                check_oracle(xs, g, decode=False)
        else:
            check_oracle(xs, g, decode=False)
            check_oracle(xs, r, decode=False)
    # the static scratch holds the logits of at most this many rows; one more
    # is rejected before anything is launched
    fit = (route.STATIC_SCRATCH_BYTES - 512) // (route.EXPERTS * 4)
    o = Outputs(fit + 1)
    x = torch.zeros((fit + 1, route.HIDDEN), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(route.RouteError) as e:
        route.fused_packed_noalloc(plan, x, packed, o.latent, None, o.ids, o.weights)
    assert e.value.status == route.E_SCRATCH
    route.fused_packed_noalloc(plan, x[:fit], packed, o.latent[:fit], None, o.ids[:fit], o.weights[:fit])
    torch.cuda.synchronize()
    assert (o.ids[:fit].cpu().numpy() == np.arange(16)).all()


def test_noalloc_decode_counters_survive_mixed_calls():
    """Decode calls through the static scratch interleaved with prefill calls
    that keep their logits there: the decode counters sit below the area a
    prefill call may use, so the decode results stay exact."""
    w, wr = weights_dev(0)
    dplan = route.Plan(route.MODE_DECODE, 12)
    pplan = route.Plan(route.MODE_PREFILL, 512)
    dws = dplan.new_workspace()
    dpk = route.pack_weights(dplan, w, wr)
    ppk = route.pack_weights(pplan, w, wr)
    for i in range(3):
        xs = gen.hidden(12, bank=8300 + i)
        r, g = run_pair(dplan, bf16_dev(xs), dpk, 12, dws, with_logits=False)
        assert_bitwise(r, g, with_logits=False)
        xp = bf16_dev(gen.hidden(512, bank=8310 + i))
        o = Outputs(512)
        route.fused_packed_noalloc(pplan, xp, ppk, o.latent, None, o.ids, o.weights)
    torch.cuda.synchronize()

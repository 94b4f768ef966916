"""Parity in the configuration bench.py times, through bench.py's own setup.

Decode: 8-row route_fused calls captured in one HIP graph over 8 distinct
weight copies (617 MB of weights, more than the 256 MB Infinity Cache) and
8 input banks, replayed several times; every output of every copy is checked
against the oracle on that copy's weights, and the same for the graph of
route_fused_packed calls on the packed copies. Prefill: the
3072-row chunk with outlier channels that bench.py times, one route_fused
call and one route_fused_packed call (bitwise equal); a seeded sample of rows
is checked against the oracle row by row (the full chunk is checked in the
prefill parity tests). Criteria as in the decode and prefill parity tests:
latent within 1 BF16 ULP or the cancellation band, relative RMS <= 2.0e-3;
logits within 2 FP32 ULP; ids equal up to a 1-for-1 swap within 2 FP32 ULP;
weights within 5 FP32 ULP."""
import numpy as np
import pytest
import torch

import bench
from oracle import compare
from oracle import route_oracle as orc
from synth import generators as gen
from tests.routekit import assert_fp64_logits, assert_prefill_logit_error, bits_host, log, oracle_rows

pytestmark = pytest.mark.gpu

route = pytest.importorskip("latent_projection_top_amd.route")

COPIES = 8


def bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def check(got, ref, tag, logits_ulp=True):
    lc = compare.latent_check(got["latent"], ref["latent"], ref["exact"], ref["abs_terms"])
    ld = compare.f32_ulp_distance(got["logits"], ref["logits"])
    ic = compare.ids_check(got["ids"], ref["ids"], ref["logits"])
    wc = compare.weights_check(got["weights"], orc.route_weights_ref(got["logits"], got["ids"]))
    log(f"{tag}: latent {lc} | logits ulp max {ld.max()} | ids equal {ic['equal']} swaps "
        f"{ic['swaps']} viol {ic['violations']} | weights max {wc['max_ulp']}")
    assert lc["fail"] == 0
    assert lc["rel_rms"] <= 2.0e-3
    if logits_ulp:
        assert_fp64_logits(got["logits"], ref["logits"])
    else:
        gc = compare.logits_check(got["logits"], ref["logits"], ref["logits_exact"],
                                  ref["logits_abs_terms"])
        log(f"{tag}: logits {gc}")
        assert gc["fail"] == 0, gc
        assert_prefill_logit_error(gc)
    assert ic["violations"] == 0, ic["bad_rows"][:5]
    assert wc["fail"] == 0


@pytest.mark.timeout(600)
def test_decode_graph_over_weight_copies():
    log("bench decode configuration: 8 rows, graph over 8 weight copies")
    copies = [(bf16(gen.latent_weight(c)), torch.from_numpy(gen.router_weight(c)).cuda())
              for c in range(COPIES)]
    xs = [gen.hidden(20, bank=4000 + b) for b in range(COPIES)]
    banks = [bf16(x) for x in xs]
    d = bench.DecodeSetup(8, copies, banks, route, torch)
    g = d.capture()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    for i in range(COPIES):
        got = {"latent": bits_host(d.lat[i]), "logits": d.lg[i].cpu().numpy(),
               "ids": d.ids[i].cpu().numpy(), "weights": d.wt[i].cpu().numpy()}
        check(got, oracle_rows(xs[i][:8], copy=i), f"copy {i}")

    pplan = route.Plan(route.MODE_DECODE, 20)
    packs = [route.pack_weights(pplan, w, wr) for w, wr in copies]
    p = bench.PackedDecodeSetup(8, copies, banks, route, torch, packs)
    gp = p.capture()
    for _ in range(3):
        gp.replay()
    torch.cuda.synchronize()
    for i in range(COPIES):
        got = {"latent": bits_host(p.lat[i]), "logits": p.lg[i].cpu().numpy(),
               "ids": p.ids[i].cpu().numpy(), "weights": p.wt[i].cpu().numpy()}
        check(got, oracle_rows(xs[i][:8], copy=i), f"packed copy {i}")


@pytest.mark.timeout(600)
def test_prefill_chunk_sampled_rows():
    log("bench prefill configuration: 3072 rows with outliers, sampled rows")
    w, wr = bf16(gen.latent_weight(0)), torch.from_numpy(gen.router_weight(0)).cuda()
    x = gen.hidden(3072, bank=4100, outliers=True)
    plan = route.Plan(route.MODE_PREFILL, 3072)
    ws = plan.new_workspace()
    lat = torch.empty((3072, route.LATENT), dtype=torch.bfloat16, device="cuda")
    lg = torch.empty((3072, route.EXPERTS), dtype=torch.float32, device="cuda")
    ids = torch.empty((3072, 16), dtype=torch.int32, device="cuda")
    wt = torch.empty((3072, 16), dtype=torch.float32, device="cuda")
    xd = bf16(x)
    packed = route.pack_weights(plan, w, wr)
    lat_p, lg_p = torch.empty_like(lat), torch.empty_like(lg)
    ids_p, wt_p = torch.empty_like(ids), torch.empty_like(wt)
    route.fused_packed(plan, xd, packed, lat_p, lg_p, ids_p, wt_p, ws)
    route.fused(plan, xd, w, wr, lat, lg, ids, wt, ws)
    torch.cuda.synchronize()
    assert torch.equal(lat_p.view(torch.int16), lat.view(torch.int16))
    assert torch.equal(lg_p.view(torch.int32), lg.view(torch.int32))
    assert torch.equal(ids_p, ids) and torch.equal(wt_p.view(torch.int32), wt.view(torch.int32))
    rows = np.sort(np.random.default_rng(7).choice(3072, 128, replace=False))
    got = {"latent": bits_host(lat)[rows], "logits": lg.cpu().numpy()[rows],
           "ids": ids.cpu().numpy()[rows], "weights": wt.cpu().numpy()[rows]}
    # prefill logits: the error bound of the prefill parity tests
    check(got, oracle_rows(x[rows], copy=0), "prefill sample", logits_ulp=False)

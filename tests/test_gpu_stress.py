"""Graph-replay stress and the cancelling-partials accuracy set on the GPU.

Stress (page "Optionally gather the Kimi3 prefill latent instead of reducing
it", Tests: CUDA-graph replays with a new input bank every replay and outputs
poisoned inside the graph, 0 mismatches): route_fused is captured in a HIP
graph once; every replay takes a new bank, the outputs are poisoned inside the
graph before the route runs, and each replay must equal the eager result for
its bank. The workspace counters must be back in their idle state afterwards.

Cancelling set (same page, Description, numerics bullet: on cancelling partials
one rounding keeps its accuracy while per-shard rounding loses it): 1024 rows
whose two halves of K cancel; relative RMS of the latent against float64 stays
<= 2.0e-3 through the decode and the prefill kernels."""
import numpy as np
import pytest
import torch

from oracle import compare
from oracle import route_oracle as orc
from synth import generators as gen
from tests.routekit import Outputs, bf16_dev, bits_host, decode_counters_idle, log, weights_dev

pytestmark = pytest.mark.gpu

route = pytest.importorskip("latent_projection_top_amd.route")

REPLAYS = 2000


@pytest.mark.timeout(600)
@pytest.mark.parametrize("width", [8, 20])
def test_graph_replay_with_new_banks_and_poisoned_outputs(width):
    log(f"graph replay stress width={width} replays={REPLAYS}")
    w, wr = weights_dev(0)
    plan = route.Plan(route.MODE_DECODE, width)
    ws = plan.new_workspace()
    nb = 64
    banks = [bf16_dev(gen.hidden(width, bank=20000 + b)) for b in range(nb)]
    # eager references
    refs = []
    for b in range(nb):
        o = Outputs(width)
        route.fused(plan, banks[b], w, wr, o.latent, o.logits, o.ids, o.weights, ws)
        refs.append(o)
    torch.cuda.synchronize()

    x_static = torch.empty_like(banks[0])
    x_static.copy_(banks[0])
    out = Outputs(width)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        # warm-up on the capture stream
        out.poison()
        route.fused(plan, x_static, w, wr, out.latent, out.logits, out.ids, out.weights, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out.poison()
        route.fused(plan, x_static, w, wr, out.latent, out.logits, out.ids, out.weights, ws)
    torch.cuda.synchronize()

    mismatches = 0
    for i in range(REPLAYS):
        b = (i * 7 + 3) % nb
        x_static.copy_(banks[b])
        g.replay()
        r = refs[b]
        same = (torch.equal(out.latent, r.latent) and torch.equal(out.logits, r.logits)
                and torch.equal(out.ids, r.ids)
                and torch.equal(out.weights.view(torch.int32), r.weights.view(torch.int32)))
        mismatches += 0 if same else 1
        if i % 500 == 0:
            log(f"  replay {i}: mismatches so far {mismatches}")
    torch.cuda.synchronize()
    assert mismatches == 0
    assert decode_counters_idle(ws)


@pytest.mark.timeout(600)
def test_cancelling_partials_single_rounding():
    log("cancel set: 1024 rows through decode (20-row calls) and prefill")
    xs, wc = gen.cancel_set(1024)
    w = bf16_dev(wc)
    _, wr = weights_dev(0)
    exact = orc.latent_exact(xs, wc)
    two = orc.bf16_bits_to_f64(orc.two_round_latent_ref(xs, wc))
    rr_two = compare.rel_rms(two, exact)
    xd = bf16_dev(xs)

    dplan = route.Plan(route.MODE_DECODE, 20)
    ws = dplan.new_workspace()
    out = Outputs(1024)
    for s in range(0, 1024, 20):
        n = min(20, 1024 - s)
        route.latent_router(dplan, xd[s:s + n], w, wr, out.latent[s:s + n], out.logits[s:s + n],
                            ws, rows=n)
    torch.cuda.synchronize()
    dec = bits_host(out.latent)

    pplan = route.Plan(route.MODE_PREFILL, 1024)
    pws = pplan.new_workspace()
    out2 = Outputs(1024)
    route.latent_router(pplan, xd, w, wr, out2.latent, out2.logits, pws)
    torch.cuda.synchronize()
    pre = bits_host(out2.latent)

    terms = orc.latent_abs_terms(xs, wc)
    ref = orc.round_f64_to_bf16_bits(exact)
    for tag, got in (("decode", dec), ("prefill", pre)):
        lc = compare.latent_check(got, ref, exact, terms)
        log(f"cancel {tag}: {lc} | two-round relRMS {rr_two:.4g}")
        assert lc["fail"] == 0
        assert lc["rel_rms"] <= 2.0e-3
        assert lc["rel_rms"] <= 0.1 * rr_two

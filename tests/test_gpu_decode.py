"""GPU parity of the decode route (1..20 rows) through the C ABI against the
CPU oracle, on seeded banks of the pages' decode widths.

Widths: 1 (single row), 8 (the fused single-exchange width) and 9/12/16/20
(two- and four-stream speculative verify rounds), page "Kimi K3.1 recipe:
route 9..20 decode rows through the pushed pair gather and standalone top-16",
"What / why". Criteria: latent within 1 BF16 ULP or the cancellation band,
relative RMS <= 2.0e-3 against float64; ids equal up to a 1-for-1 swap within
2 FP32 ULP; weights within 5 FP32 ULP."""
import numpy as np
import pytest
import torch

from oracle import compare
from oracle import route_oracle as orc
from synth import generators as gen
from tests.routekit import (Outputs, assert_fp64_logits, bf16_dev, bits_host, decode_counters_idle, log, oracle_rows,
                            weights_dev)

pytestmark = pytest.mark.gpu

route = pytest.importorskip("latent_projection_top_amd.route")

BANKS = 200


def bank_rows(width: int, banks: int) -> np.ndarray:
    return np.concatenate([gen.hidden(width, bank=1000 * width + b) for b in range(banks)])


def run_banks(width: int, banks: int, fused: bool):
    w, wr = weights_dev(0)
    plan = route.Plan(route.MODE_DECODE, width)
    ws = plan.new_workspace()
    xs = bank_rows(width, banks)
    xd = bf16_dev(xs)
    out = Outputs(width * banks)
    for b in range(banks):
        s = slice(b * width, (b + 1) * width)
        if fused:
            route.fused(plan, xd[s], w, wr, out.latent[s], out.logits[s], out.ids[s],
                        out.weights[s], ws, rows=width)
        else:
            route.latent_router(plan, xd[s], w, wr, out.latent[s], out.logits[s], ws, rows=width)
            route.topk16(plan, out.logits[s], out.ids[s], out.weights[s], rows=width)
    torch.cuda.synchronize()
    return xs, out.host(), ws


def check_outputs(xs, got, tag):
    ref = oracle_rows(xs)
    lc = compare.latent_check(got["latent"], ref["latent"], ref["exact"], ref["abs_terms"])
    ld = compare.f32_ulp_distance(got["logits"], ref["logits"])
    ic = compare.ids_check(got["ids"], ref["ids"], ref["logits"])
    wc = compare.weights_check(got["weights"], orc.route_weights_ref(got["logits"], got["ids"]))
    same = (got["ids"] == ref["ids"]).all(axis=1)
    wc2 = compare.weights_check(got["weights"][same], ref["weights"][same])
    log(f"{tag}: latent {lc} | logits ulp max {ld.max()} mean {ld.mean():.3g} | ids "
        f"equal {ic['equal']} swaps {ic['swaps']} viol {ic['violations']} | weights max "
        f"{wc['max_ulp']} / e2e {wc2['max_ulp']}")
    assert lc["fail"] == 0
    assert lc["rel_rms"] <= 2.0e-3
    assert lc["band"] <= max(2, 1e-4 * lc["n"])
    assert_fp64_logits(got["logits"], ref["logits"])
    assert ic["violations"] == 0, ic["bad_rows"][:5]
    assert wc["fail"] == 0 and wc2["fail"] == 0


@pytest.mark.parametrize("width", [1, 8, 9, 12, 16, 20])
def test_decode_banks(width):
    log(f"decode parity width={width} banks={BANKS}")
    xs, got, ws = run_banks(width, BANKS, fused=(width % 2 == 0))
    check_outputs(xs, got, f"decode w={width}")
    # the tile counters are back at zero and the next call's pair is cleared
    assert decode_counters_idle(ws)


@pytest.mark.parametrize("width", [w for w in range(1, 21) if w not in (1, 8, 9, 12, 16, 20)])
def test_decode_other_widths(width):
    """Every other call width of the 1..20 envelope, 10 banks each, fused
    route on [K][N] weights against the oracle."""
    log(f"decode parity width={width} banks=10")
    xs, got, ws = run_banks(width, 10, fused=True)
    check_outputs(xs, got, f"decode w={width}")
    assert decode_counters_idle(ws)


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("width", [8, 20])
def test_decode_outlier_channels(width, packed):
    """Hidden rows with the prefill workload's outlier channels (1 % of the
    channels scaled x20), where the FP32 accumulation of the latent has the
    largest terms: 20 banks, fused route, both weight layouts."""
    log(f"decode with outlier channels width={width} packed={packed}")
    w, wr = weights_dev(0)
    plan = route.Plan(route.MODE_DECODE, width)
    ws = plan.new_workspace()
    pk = route.pack_weights(plan, w, wr) if packed else None
    banks = 20
    xs = np.concatenate([gen.hidden(width, bank=3000 + 100 * width + b, outliers=True) for b in range(banks)])
    xd = bf16_dev(xs)
    out = Outputs(width * banks)
    out.poison()
    for b in range(banks):
        s = slice(b * width, (b + 1) * width)
        if packed:
            route.fused_packed(plan, xd[s], pk, out.latent[s], out.logits[s], out.ids[s], out.weights[s], ws,
                               rows=width)
        else:
            route.fused(plan, xd[s], w, wr, out.latent[s], out.logits[s], out.ids[s], out.weights[s], ws,
                        rows=width)
    torch.cuda.synchronize()
    check_outputs(xs, out.host(), f"decode outliers w={width} packed={packed}")
    assert decode_counters_idle(ws)


@pytest.mark.parametrize("width", list(range(1, 21)))
def test_fused_equals_two_calls_bitwise(width):
    log(f"fused == latent_router + topk16, width={width}")
    xs_a, got_a, _ = run_banks(width, 3, fused=True)
    xs_b, got_b, _ = run_banks(width, 3, fused=False)
    for k in ("latent", "logits", "ids"):
        assert np.array_equal(got_a[k], got_b[k]), k
    assert np.array_equal(got_a["weights"].view(np.uint32), got_b["weights"].view(np.uint32))
    if width in (2, 3, 5, 17):
        check_outputs(xs_a, got_a, f"decode w={width}")


def test_rows_below_plan_capacity_and_repeat_determinism():
    log("decode rows < plan rows, repeated calls bit-identical")
    w, wr = weights_dev(0)
    plan = route.Plan(route.MODE_DECODE, 20)
    ws = plan.new_workspace()
    xs = gen.hidden(20, bank=77)
    xd = bf16_dev(xs)
    outs = []
    for i, rows in enumerate((20, 5, 20, 13, 1, 20, 7, 20)):
        o = Outputs(20)
        o.poison()
        if i == 4:
            # a projection-only call on the same workspace, then the
            # workspace zero-filled again: both leave it usable
            route.latent_router(plan, xd, w, wr, o.latent, o.logits, ws, rows=20)
            torch.cuda.synchronize()
            assert decode_counters_idle(ws)
            ws.zero_()
            o.poison()
        route.fused(plan, xd, w, wr, o.latent, o.logits, o.ids, o.weights, ws, rows=rows)
        torch.cuda.synchronize()
        assert decode_counters_idle(ws)
        h = o.host()
        outs.append((rows, h))
        # rows beyond `rows` are untouched
        assert (h["ids"][rows:] == -1).all()
    full = [h for r, h in outs if r == 20]
    for h in full[1:]:
        for k in ("latent", "logits", "ids"):
            assert np.array_equal(h[k], full[0][k])
    check_outputs(xs, full[0], "decode w=20 cap")
    # a row's outputs do not depend on how many rows share the call
    for rows, h in outs:
        assert np.array_equal(h["latent"][:rows], full[0]["latent"][:rows])
        assert np.array_equal(h["ids"][:rows], full[0]["ids"][:rows])


def test_fused_without_logits_buffer():
    log("fused with logits == NULL")
    w, wr = weights_dev(0)
    for width in (4, 12):
        plan = route.Plan(route.MODE_DECODE, width)
        ws = plan.new_workspace()
        xd = bf16_dev(gen.hidden(width, bank=5))
        a, b = Outputs(width), Outputs(width)
        route.fused(plan, xd, w, wr, a.latent, a.logits, a.ids, a.weights, ws)
        route.fused(plan, xd, w, wr, b.latent, None, b.ids, b.weights, ws)
        torch.cuda.synchronize()
        assert torch.equal(a.ids, b.ids) and torch.equal(a.latent, b.latent)
        assert torch.equal(a.weights.view(torch.int32), b.weights.view(torch.int32))


def test_run_call_validation_launches_nothing():
    w, wr = weights_dev(0)
    plan = route.Plan(route.MODE_DECODE, 8)
    ws = plan.new_workspace()
    xd = bf16_dev(gen.hidden(9, bank=1))
    o = Outputs(9)
    o.poison()
    with pytest.raises(route.RouteError) as e:
        route.latent_router(plan, xd, w, wr, o.latent, o.logits, ws, rows=9)
    assert e.value.status == route.E_ROWS
    with pytest.raises(route.RouteError) as e:
        route.latent_router(plan, xd, w, wr, o.latent, o.logits, ws, rows=0)
    assert e.value.status == route.E_ROWS
    # a pointer off the 16-byte grid
    raw = torch.zeros(8 * 896 + 1, dtype=torch.float32, device="cuda")
    st = route.LIB.route_latent_router(
        plan.handle, xd.data_ptr(), w.data_ptr(), wr.data_ptr(), o.latent.data_ptr(),
        raw.data_ptr() + 4, ws.data_ptr(), 8, None)
    assert st == route.E_ALIGN
    torch.cuda.synchronize()
    assert (bits_host(o.latent) == 0xFFFF).all()
    assert int(ws.count_nonzero()) == 0


def test_zero_rows_degenerate_case():
    """All-zero hidden rows among ordinary ones: their latent is +0.0, their
    logits are all 0.0, so the top-16 is experts 0..15 (lowest index on the
    896-way tie) with weights exactly 1/16; the other rows are unaffected."""
    log("decode with all-zero hidden rows")
    w, wr = weights_dev(0)
    for width in (8, 20):
        xs = gen.hidden(width, bank=90 + width)
        zero = [1, width - 1] if width == 8 else [0, 7, 16, 19]
        xs[zero] = 0
        plan = route.Plan(route.MODE_DECODE, width)
        ws = plan.new_workspace()
        o = Outputs(width)
        o.poison()
        route.fused(plan, bf16_dev(xs), w, wr, o.latent, o.logits, o.ids, o.weights, ws)
        torch.cuda.synchronize()
        h = o.host()
        for r in zero:
            assert (h["latent"][r] == 0).all()
            assert (h["logits"][r].view(np.uint32) == 0).all()
            assert np.array_equal(h["ids"][r], np.arange(16))
            assert (h["weights"][r] == np.float32(1.0 / 16.0)).all()
        check_outputs(xs, h, f"decode w={width} with zero rows")


def test_binding_rejects_short_workspace_and_wrong_device():
    """The binding checks what the C ABI cannot see: a workspace shorter than
    route_workspace_bytes, and tensors on another device than the plan's.
    Nothing is launched."""
    w, wr = weights_dev(0)
    plan = route.Plan(route.MODE_DECODE, 8)
    xd = bf16_dev(gen.hidden(8, bank=3))
    o = Outputs(8)
    o.poison()
    short = torch.zeros(plan.workspace_bytes - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="workspace"):
        route.fused(plan, xd, w, wr, o.latent, o.logits, o.ids, o.weights, short)
    with pytest.raises(ValueError, match="workspace"):
        route.latent_router(plan, xd, w, wr, o.latent, o.logits, short)
    pplan = route.Plan(route.MODE_PREFILL, 64)
    pshort = torch.zeros(pplan.workspace_bytes - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="workspace"):
        route.latent_router(pplan, xd, w, wr, o.latent, o.logits, pshort, rows=8)
    torch.cuda.synchronize()
    assert (bits_host(o.latent) == 0xFFFF).all()
    assert int(short.count_nonzero()) == 0
    # a plan for another device index: every tensor here is on the current one
    other = route.Plan.__new__(route.Plan)
    other.__dict__.update(plan.__dict__)
    other.device = plan.device + 1
    other.handle = 0  # never reaches the library
    with pytest.raises(ValueError, match="plan is for"):
        route.fused(other, xd, w, wr, o.latent, o.logits, o.ids, o.weights, plan.new_workspace())

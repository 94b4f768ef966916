"""Packed weights (route_pack_weights, route_latent_router_packed,
route_fused_packed) on the GPU through the C ABI.

A decode buffer holds the same values as the [K][N] weights in the decode
kernel's consumption order; a prefill buffer holds W transposed and the
router weight's three exact BF16 parts, transposed. The packed calls run the
same arithmetic on the same per-lane operands, so their outputs must be
bitwise those of route_latent_router / route_fused on the original weights:
at every decode width (both kernel variants: up to 16 rows, and 17..20 rows
with the router's VALU rows), and at 1, 200 (ragged tile edge) and 3072
prefill rows; and within the oracle's bounds (latent within 1 BF16 ULP or
the cancellation band, ids equal up to a 2-ULP near-tie swap, weights within
5 FP32 ULP)."""
import numpy as np
import pytest
import torch

from oracle import compare
from oracle import route_oracle as orc
from synth import generators as gen
from tests.routekit import Outputs, bf16_dev, decode_counters_idle, log, oracle_rows, weights_dev

pytestmark = pytest.mark.gpu

route = pytest.importorskip("latent_projection_top_amd.route")


def packed_weights(copy: int = 0):
    w, wr = weights_dev(copy)
    plan = route.Plan(route.MODE_DECODE, 20)
    packed = route.pack_weights(plan, w, wr)
    torch.cuda.synchronize()
    return plan, packed


def test_packed_buffer_is_a_permutation_of_the_weights():
    w, wr = weights_dev(0)
    plan, packed = packed_weights(0)
    assert plan.packed_bytes == route.HIDDEN * (route.LATENT * 2 + route.EXPERTS * 4)
    nl = route.HIDDEN * route.LATENT * 2
    lat = packed[:nl].view(torch.int16)
    rt = packed[nl:plan.packed_bytes].view(torch.int32)
    assert torch.equal(torch.sort(lat).values, torch.sort(w.view(torch.int16).reshape(-1)).values)
    assert torch.equal(torch.sort(rt).values, torch.sort(wr.view(torch.int32).reshape(-1)).values)
    # first pieces, by the layout's definition: latent unit 0 (tile 0, split
    # 0), wave 0, step 0, MFMA 0, lane 0 holds W[0..7][0]; lane 1 holds
    # W[0..7][4]; lane 16 W[8..15][0]; router lane 0 holds Wr[0][0], Wr[0][1],
    # Wr[1][0], Wr[1][1]
    wl = w.view(torch.int16)
    assert torch.equal(lat[0:8], wl[0:8, 0])
    assert torch.equal(lat[8:16], wl[0:8, 4])
    assert torch.equal(lat[16 * 8:17 * 8], wl[8:16, 0])
    wi = wr.view(torch.int32)
    assert torch.equal(rt[0:4], torch.stack([wi[0, 0], wi[0, 1], wi[1, 0], wi[1, 1]]))


@pytest.mark.parametrize("width", [1, 8, 16, 17, 20])
def test_packed_bitwise_equal_to_unpacked(width):
    w, wr = weights_dev(0)
    plan, packed = packed_weights(0)
    banks = 8
    xs = np.concatenate([gen.hidden(width, bank=7000 + 100 * width + b) for b in range(banks)])
    xd = bf16_dev(xs)
    ref, got, got2 = Outputs(width * banks), Outputs(width * banks), Outputs(width * banks)
    for o in (ref, got, got2):
        o.poison()
    ws_a, ws_b = plan.new_workspace(), plan.new_workspace()
    for b in range(banks):
        s = slice(b * width, (b + 1) * width)
        route.fused(plan, xd[s], w, wr, ref.latent[s], ref.logits[s], ref.ids[s], ref.weights[s],
                    ws_a, rows=width)
        route.fused_packed(plan, xd[s], packed, got.latent[s], got.logits[s], got.ids[s],
                           got.weights[s], ws_b, rows=width)
        route.latent_router_packed(plan, xd[s], packed, got2.latent[s], got2.logits[s], ws_b,
                                   rows=width)
    torch.cuda.synchronize()
    r, g, g2 = ref.host(), got.host(), got2.host()
    for k in ("latent", "logits", "ids", "weights"):
        assert np.array_equal(r[k].view(np.uint32) if k in ("logits", "weights") else r[k],
                              g[k].view(np.uint32) if k in ("logits", "weights") else g[k]), k
    assert np.array_equal(r["latent"], g2["latent"])
    assert np.array_equal(r["logits"].view(np.uint32), g2["logits"].view(np.uint32))
    assert decode_counters_idle(ws_b)

    ref_o = oracle_rows(xs)
    lc = compare.latent_check(g["latent"], ref_o["latent"], ref_o["exact"], ref_o["abs_terms"])
    ic = compare.ids_check(g["ids"], ref_o["ids"], ref_o["logits"])
    wc = compare.weights_check(g["weights"], orc.route_weights_ref(g["logits"], g["ids"]))
    log(f"packed width {width}: latent {lc} ids equal {ic['equal']} viol {ic['violations']} "
        f"weights max {wc['max_ulp']}")
    assert lc["fail"] == 0 and lc["rel_rms"] <= 2.0e-3
    assert ic["violations"] == 0
    assert wc["fail"] == 0


def test_packed_rejects_share_plans():
    w, wr = weights_dev(0)
    share = route.Plan(route.MODE_DECODE, 8, latent=448, experts=112)
    assert share.packed_bytes == 0
    buf = torch.empty(16, dtype=torch.uint8, device="cuda")
    for plan in (share,):
        st = route.LIB.route_pack_weights(plan.handle, w.data_ptr(), wr.data_ptr(), buf.data_ptr(),
                                          None)
        assert st == route.E_SHAPE
    dec = route.Plan(route.MODE_DECODE, 8)
    st = route.LIB.route_fused_packed(dec.handle, buf.data_ptr(), buf.data_ptr() + 4, buf.data_ptr(),
                                      None, buf.data_ptr(), buf.data_ptr(), buf.data_ptr(), 8, None)
    assert st == route.E_ALIGN
    st = route.LIB.route_fused_packed(dec.handle, buf.data_ptr(), buf.data_ptr(), buf.data_ptr(),
                                      None, buf.data_ptr(), buf.data_ptr(), buf.data_ptr(), 9, None)
    assert st == route.E_ROWS


# ------------------------------------------------------------------ prefill --

def prefill_packed(copy: int = 0):
    w, wr = weights_dev(copy)
    plan = route.Plan(route.MODE_PREFILL, 3072)
    packed = route.pack_weights(plan, w, wr)
    torch.cuda.synchronize()
    return plan, packed


def test_prefill_packed_layout():
    """The prefill buffer is W transposed ([3584][7168]) followed by the three
    exact BF16 parts of Wr, transposed, in rows (e / 64) * 192 + 64 p + e % 64:
    hi + mid + lo == Wr exactly, each part a BF16 value with at most 8
    significant bits."""
    w, wr = weights_dev(0)
    plan, packed = prefill_packed(0)
    assert plan.packed_bytes == route.HIDDEN * (route.LATENT + 3 * route.EXPERTS) * 2
    nl = route.HIDDEN * route.LATENT * 2
    wt = packed[:nl].view(torch.int16).view(route.LATENT, route.HIDDEN)
    assert torch.equal(wt, w.view(torch.int16).t())
    parts = packed[nl:plan.packed_bytes].view(torch.int16).view(14, 3, 64, route.HIDDEN)
    parts = parts.view(torch.bfloat16).double()
    total = (parts[:, 0] + parts[:, 1] + parts[:, 2]).reshape(route.EXPERTS, route.HIDDEN)
    assert torch.equal(total, wr.double().t())
    # the parts are ordered by magnitude (each is the remainder's top bits)
    hi, mid = parts[:, 0].abs(), parts[:, 1].abs()
    nz = mid > 0
    assert bool((mid[nz] <= hi[nz] * 2.0 ** -7).all())


@pytest.mark.parametrize("rows", [1, 200, 3072])
def test_prefill_packed_bitwise_equal_to_unpacked(rows):
    w, wr = weights_dev(0)
    plan, packed = prefill_packed(0)
    xs = gen.hidden(rows, bank=8000 + rows, outliers=True)
    xd = bf16_dev(xs)
    ws = plan.new_workspace()
    ref, got, got2 = Outputs(rows), Outputs(rows), Outputs(rows)
    for o in (ref, got, got2):
        o.poison()
    route.fused(plan, xd, w, wr, ref.latent, ref.logits, ref.ids, ref.weights, ws, rows=rows)
    route.fused_packed(plan, xd, packed, got.latent, got.logits, got.ids, got.weights, ws, rows=rows)
    route.latent_router_packed(plan, xd, packed, got2.latent, got2.logits, ws, rows=rows)
    torch.cuda.synchronize()
    r, g, g2 = ref.host(), got.host(), got2.host()
    log(f"prefill packed rows={rows}: comparing bitwise")
    assert np.array_equal(r["latent"], g["latent"])
    assert np.array_equal(r["logits"].view(np.uint32), g["logits"].view(np.uint32))
    assert np.array_equal(r["ids"], g["ids"])
    assert np.array_equal(r["weights"].view(np.uint32), g["weights"].view(np.uint32))
    assert np.array_equal(r["latent"], g2["latent"])
    assert np.array_equal(r["logits"].view(np.uint32), g2["logits"].view(np.uint32))
    if rows <= 200:
        ref_o = oracle_rows(xs)
        lc = compare.latent_check(g["latent"], ref_o["latent"], ref_o["exact"], ref_o["abs_terms"])
        ic = compare.ids_check(g["ids"], ref_o["ids"], ref_o["logits"])
        assert lc["fail"] == 0 and ic["violations"] == 0

"""Packed weights (route_pack_weights, route_latent_router_packed,
route_fused_packed) on the GPU through the C ABI.

A decode buffer holds the [K][N] weights' values in the packed decode
kernel's consumption order, tile by tile in K order (the kernel splits K 8
ways for both weights up to 4 rows, 4 / 8 ways above); a prefill buffer
holds W transposed and the router
weight's three exact BF16 parts, transposed. Decode: the packed kernel's K
split differs from route_fused's (latent 4, router 16 ways), so its outputs
are checked against the oracle like route_fused's (latent
within 1 BF16 ULP or the cancellation band, relative RMS <= 2.0e-3, logits
within 2 FP32 ULP, ids equal up to a 1-for-1 swap within 2 FP32 ULP, weights
within 5 FP32 ULP) at every decode width of the pages, both kernel variants
(up to 16 rows; 17..20 rows with the router's VALU rows), fused and two-call
forms bitwise equal, and its logits against route_fused's. Prefill: every
GEMM lane receives the same operands as with [K][N] weights, so the outputs
must be bitwise those of route_fused, at 1, 200 (ragged tile edge) and 3072
rows."""
import numpy as np
import pytest
import torch

from oracle import compare
from synth import generators as gen
from tests.routekit import Outputs, bf16_dev, decode_counters_idle, log, oracle_rows, weights_dev
from tests.test_gpu_decode import check_outputs

pytestmark = pytest.mark.gpu

route = pytest.importorskip("latent_projection_top_amd.route")

BANKS = 200


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
    # pieces at known places of the layout (tile-major, K steps in order):
    # latent tile 0, K step 0, MFMA 0: lane 0 holds W[0..7][0], lane 1
    # W[0..7][4], lane 16 W[8..15][0]; MFMA 1, lane 0: W[0..7][1]; K step 7
    # (K 224..) at value offset 7 * 2048, step 28 (K 896..) at 28 * 2048,
    # tile 1 (columns 64..) at 224 * 2048. Router tile 0, step 0, lane 0
    # holds Wr[0][0], Wr[0][1], Wr[1][0], Wr[1][1]; half 1: Wr[2..3][0..1];
    # step 14 (K 224..) at float offset 14 * 512; tile 1 (experts 32..) at
    # 448 * 512.
    wl = w.view(torch.int16)
    assert torch.equal(lat[0:8], wl[0:8, 0])
    assert torch.equal(lat[8:16], wl[0:8, 4])
    assert torch.equal(lat[16 * 8:17 * 8], wl[8:16, 0])
    assert torch.equal(lat[64 * 8:65 * 8], wl[0:8, 1])
    for o, k, n in ((7 * 2048, 224, 0), (28 * 2048, 896, 0), (224 * 2048, 0, 64)):
        assert torch.equal(lat[o:o + 8], wl[k:k + 8, n]), (o, k, n)
    wi = wr.view(torch.int32)

    def quad(k, e):
        return torch.stack([wi[k, e], wi[k, e + 1], wi[k + 1, e], wi[k + 1, e + 1]])

    assert torch.equal(rt[0:4], quad(0, 0))
    assert torch.equal(rt[256:260], quad(2, 0))
    assert torch.equal(rt[14 * 512:14 * 512 + 4], quad(224, 0))
    assert torch.equal(rt[448 * 512:448 * 512 + 4], quad(0, 32))


def run_packed_banks(width: int, banks: int, fused: bool, seed: int = 7000):
    plan, packed = packed_weights(0)
    ws = plan.new_workspace()
    xs = np.concatenate([gen.hidden(width, bank=seed + 100 * width + b) for b in range(banks)])
    xd = bf16_dev(xs)
    out = Outputs(width * banks)
    out.poison()
    for b in range(banks):
        s = slice(b * width, (b + 1) * width)
        if fused:
            route.fused_packed(plan, xd[s], packed, out.latent[s], out.logits[s], out.ids[s],
                               out.weights[s], ws, rows=width)
        else:
            route.latent_router_packed(plan, xd[s], packed, out.latent[s], out.logits[s], ws,
                                       rows=width)
            route.topk16(plan, out.logits[s], out.ids[s], out.weights[s], rows=width)
    torch.cuda.synchronize()
    return xs, out.host(), ws


@pytest.mark.parametrize("width", [1, 4, 5, 8, 9, 12, 16, 17, 20])
def test_packed_decode_banks(width):
    log(f"packed decode parity width={width} banks={BANKS}")
    xs, got, ws = run_packed_banks(width, BANKS, fused=(width % 2 == 0))
    check_outputs(xs, got, f"packed decode w={width}")
    assert decode_counters_idle(ws)


@pytest.mark.parametrize("width", [2, 3, 6, 7, 10, 11, 13, 14, 15, 18, 19])
def test_packed_decode_other_widths(width):
    """Every other call width of the 1..20 envelope, 10 banks each, fused
    route on packed weights against the oracle."""
    log(f"packed decode parity width={width} banks=10")
    xs, got, ws = run_packed_banks(width, 10, fused=True, seed=9000)
    check_outputs(xs, got, f"packed decode w={width}")
    assert decode_counters_idle(ws)


@pytest.mark.parametrize("width", [1, 2, 4, 5, 8, 12, 13, 16, 17, 20])
def test_packed_fused_equals_two_calls_bitwise(width):
    _, a, _ = run_packed_banks(width, 3, fused=True, seed=7500)
    _, b, _ = run_packed_banks(width, 3, fused=False, seed=7500)
    for k in ("latent", "logits", "ids"):
        assert np.array_equal(a[k], b[k]), k
    assert np.array_equal(a["weights"].view(np.uint32), b["weights"].view(np.uint32))


@pytest.mark.parametrize("width", [1, 4, 5, 8, 13, 17, 20])
def test_packed_against_kn_on_one_workspace(width):
    """route_fused and route_fused_packed alternate on one workspace (they
    share its counters): every call's outputs stay right, the counters idle;
    the logits agree within 1 FP32 ULP (both FP64 sums rounded once), the
    latent within the oracle's bounds (checked in the bank tests)."""
    w, wr = weights_dev(0)
    plan, packed = packed_weights(0)
    ws = plan.new_workspace()
    banks = 6
    xs = np.concatenate([gen.hidden(width, bank=7700 + 100 * width + b) for b in range(banks)])
    xd = bf16_dev(xs)
    kn, pk = Outputs(width * banks), Outputs(width * banks)
    for b in range(banks):
        s = slice(b * width, (b + 1) * width)
        for which in ((kn, pk) if b % 2 == 0 else (pk, kn)):
            if which is kn:
                route.fused(plan, xd[s], w, wr, kn.latent[s], kn.logits[s], kn.ids[s], kn.weights[s],
                            ws, rows=width)
            else:
                route.fused_packed(plan, xd[s], packed, pk.latent[s], pk.logits[s], pk.ids[s],
                                   pk.weights[s], ws, rows=width)
    torch.cuda.synchronize()
    assert decode_counters_idle(ws)
    a, b = kn.host(), pk.host()
    ld = compare.f32_ulp_distance(a["logits"], b["logits"])
    lat_same = float((a["latent"] == b["latent"]).mean())
    log(f"packed vs [K][N] width {width}: logits ulp max {ld.max()} ({int((ld > 0).sum())} differ); "
        f"latent identical {lat_same:.5f}")
    assert ld.max() <= 1
    same_rows = (ld == 0).all(axis=1)
    assert np.array_equal(a["ids"][same_rows], b["ids"][same_rows])
    check_outputs(xs, b, f"packed/[K][N] alternating w={width}")


def test_packed_rejects_share_plans():
    w, wr = weights_dev(0)
    share = route.Plan(route.MODE_DECODE, 8, latent=448, experts=112)
    assert share.packed_bytes == 0
    buf = torch.empty(16, dtype=torch.uint8, device="cuda")
    st = route.LIB.route_pack_weights(share.handle, w.data_ptr(), wr.data_ptr(), buf.data_ptr(), None)
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


@pytest.mark.parametrize("rows", [1, 191, 193, 200, 2881, 3072])
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


@pytest.mark.timeout(900)
@pytest.mark.parametrize("rows", [128, 129, 256, 257, 512, 513, 1024, 1025, 1152, 1153, 2049, 2304, 2305])
def test_prefill_tile_plan_boundaries(rows):
    """Both sides of every change between 128- and 192-row block tiles in
    the prefill plan (the latent GEMM switches at 128 / 192 / 256 / 384 /
    512 / 768 / 1024 / 1536 / 2048 rows, the router at 128 / 192 / 256 /
    384 / 512 / 768 / 1152 / 1728 / 2304): the packed call against the
    oracle, and bitwise against the [K][N] call, which takes the same plan."""
    from tests.test_gpu_prefill import check_outputs
    w, wr = weights_dev(0)
    plan, packed = prefill_packed(0)
    xs = gen.hidden(rows, bank=8600 + rows, outliers=True)
    xd = bf16_dev(xs)
    ws = plan.new_workspace()
    ref, got = Outputs(rows), Outputs(rows)
    for o in (ref, got):
        o.poison()
    route.fused(plan, xd, w, wr, ref.latent, ref.logits, ref.ids, ref.weights, ws, rows=rows)
    route.fused_packed(plan, xd, packed, got.latent, got.logits, got.ids, got.weights, ws, rows=rows)
    torch.cuda.synchronize()
    r, g = ref.host(), got.host()
    log(f"prefill tile plan rows={rows}")
    assert np.array_equal(r["latent"], g["latent"])
    assert np.array_equal(r["logits"].view(np.uint32), g["logits"].view(np.uint32))
    assert np.array_equal(r["ids"], g["ids"])
    assert np.array_equal(r["weights"].view(np.uint32), g["weights"].view(np.uint32))
    check_outputs(xs, g, f"prefill tile plan rows={rows}")

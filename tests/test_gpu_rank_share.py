"""GPU parity of the decode kernel at one tensor-parallel rank's share of the
route, through the C ABI, against the CPU oracle on the same weight columns.

Shares: 448 latent columns x 112 experts (8 ranks) and 224 x 56 (16 ranks),
the per-rank outputs of page "Optionally gather the Kimi3 prefill latent
instead of reducing it" (448 columns per rank at 8 ranks) and page "Use two row
blocks for eight-row Kimi paired gathers" (BF16 [8, 224] latent and FP32
[8, 56] router per rank at 16 ranks). A rank's weights are its contiguous
column slices of the full weights. Every output is one full-K dot product, so
the oracle is the whole route's oracle restricted to those columns. Criteria
as for the whole route: latent within 1 BF16 ULP or the cancellation band,
relative RMS <= 2.0e-3; logits within 2 FP32 ULP of the float64 dot rounded
once."""
import numpy as np
import pytest
import torch

from oracle import compare
from oracle import route_oracle as orc
from synth import generators as gen
from tests.routekit import assert_fp64_logits, bf16_dev, bits_host, log, weights_f64, weights_host

pytestmark = pytest.mark.gpu

route = pytest.importorskip("latent_projection_top_amd.route")

BANKS = 40
RANKS = sorted(route.RANK_SHARES)


def share_weights(ranks: int, rank: int, copy: int = 0):
    """Rank `rank`'s contiguous column slices of the full weights (host bits
    and device tensors)."""
    lat, exp = route.RANK_SHARES[ranks]
    w, wr = weights_host(copy)
    ws = np.ascontiguousarray(w[:, rank * lat:(rank + 1) * lat])
    wrs = np.ascontiguousarray(wr[:, rank * exp:(rank + 1) * exp])
    return ws, wrs, bf16_dev(ws), torch.from_numpy(wrs).cuda()


def share_oracle(x_bits: np.ndarray, ranks: int, rank: int, copy: int = 0) -> dict:
    lat, exp = route.RANK_SHARES[ranks]
    w64, wr64 = weights_f64(copy)
    w64 = w64[:, rank * lat:(rank + 1) * lat]
    wr64 = wr64[:, rank * exp:(rank + 1) * exp]
    # the oracle's route restricted to the share's columns (its top-16 over
    # the share's experts goes unused)
    return orc.route_detail_widened(x_bits, w64, wr64)


class ShareOutputs:
    """Outputs of a share call, each followed by a poisoned guard area that no
    call may touch (the partial tiles at a share's edge are masked)."""
    GUARD = 4096

    def __init__(self, rows: int, lat: int, exp: int):
        self.rows, self.lat, self.exp = rows, lat, exp
        self._lat = torch.empty(rows * lat + self.GUARD, dtype=torch.bfloat16, device="cuda")
        self._lg = torch.empty(rows * exp + self.GUARD, dtype=torch.float32, device="cuda")
        self._lat.view(torch.int16).fill_(-1)
        self._lg.view(torch.int32).fill_(-1)
        self.latent = self._lat[:rows * lat].view(rows, lat)
        self.logits = self._lg[:rows * exp].view(rows, exp)

    def guards_intact(self) -> bool:
        a = bits_host(self._lat[self.rows * self.lat:])
        b = self._lg[self.rows * self.exp:].view(torch.int32).cpu().numpy()
        return bool((a == 0xFFFF).all() and (b == -1).all())

    def host(self):
        return bits_host(self.latent), self.logits.cpu().numpy()


def check_outputs(xs, got_latent, got_logits, ref, tag):
    lc = compare.latent_check(got_latent, ref["latent"], ref["exact"], ref["abs_terms"])
    ld = compare.f32_ulp_distance(got_logits, ref["logits"])
    log(f"{tag}: latent {lc} | logits ulp max {ld.max()} mean {ld.mean():.3g}")
    assert lc["fail"] == 0
    assert lc["rel_rms"] <= 2.0e-3
    assert lc["band"] <= max(2, 1e-4 * lc["n"])
    assert_fp64_logits(got_logits, ref["logits"])


@pytest.mark.parametrize("ranks", RANKS)
@pytest.mark.parametrize("width", [1, 4, 8, 16, 17, 20])
def test_share_banks(ranks, width):
    """40 banks at 1 / 8 / 20 rows, 10 at 4 / 16 / 17 (either side of the
    16-row step where rows 16..19 of the router move to the VALU), each width
    on another rank."""
    lat, exp = route.RANK_SHARES[ranks]
    rank = {1: 0, 4: 1, 8: ranks - 1, 16: 2, 17: ranks - 2, 20: ranks // 2 + 1}[width]
    banks = BANKS if width in (1, 8, 20) else 10
    log(f"share parity ranks={ranks} rank={rank} width={width} banks={banks}")
    _, _, w, wr = share_weights(ranks, rank)
    plan = route.Plan(route.MODE_DECODE, width, latent=lat, experts=exp)
    ws = plan.new_workspace()
    xs = np.concatenate([gen.hidden(width, bank=7000 + 100 * width + b) for b in range(banks)])
    xd = bf16_dev(xs)
    lat_h, lg_h = [], []
    for b in range(banks):
        o = ShareOutputs(width, lat, exp)
        route.latent_router(plan, xd[b * width:(b + 1) * width], w, wr, o.latent, o.logits, ws,
                            rows=width)
        torch.cuda.synchronize()
        assert o.guards_intact()
        a, l_ = o.host()
        lat_h.append(a)
        lg_h.append(l_)
    check_outputs(xs, np.concatenate(lat_h), np.concatenate(lg_h), share_oracle(xs, ranks, rank),
          f"share {ranks} ranks w={width}")
    assert int(ws[:512].count_nonzero()) == 0


@pytest.mark.parametrize("ranks", RANKS)
def test_share_rows_below_capacity_and_determinism(ranks):
    lat, exp = route.RANK_SHARES[ranks]
    log(f"share ranks={ranks}: rows < plan rows, repeated calls bit-identical")
    _, _, w, wr = share_weights(ranks, 1)
    plan = route.Plan(route.MODE_DECODE, 20, latent=lat, experts=exp)
    ws = plan.new_workspace()
    xs = gen.hidden(20, bank=78)
    xd = bf16_dev(xs)
    outs = []
    for rows in (20, 7, 20, 16, 17, 20):
        o = ShareOutputs(20, lat, exp)
        route.latent_router(plan, xd, w, wr, o.latent, o.logits, ws, rows=rows)
        torch.cuda.synchronize()
        a, l_ = o.host()
        assert (a[rows:] == 0xFFFF).all() and (l_[rows:].view(np.int32) == -1).all()
        assert o.guards_intact()
        outs.append((rows, a, l_))
    full = [(a, l_) for r, a, l_ in outs if r == 20]
    for a, l_ in full[1:]:
        assert np.array_equal(a, full[0][0]) and np.array_equal(l_.view(np.int32), full[0][1].view(np.int32))
    for rows, a, l_ in outs:
        assert np.array_equal(a[:rows], full[0][0][:rows])
        assert np.array_equal(l_[:rows].view(np.int32), full[0][1][:rows].view(np.int32))
    check_outputs(xs, full[0][0], full[0][1], share_oracle(xs, ranks, 1), f"share {ranks} ranks cap 20")
    assert int(ws[:512].count_nonzero()) == 0


@pytest.mark.parametrize("ranks", RANKS)
def test_share_plan_has_no_topk(ranks):
    """A share has no top-16: the select calls reject its plan and launch
    nothing."""
    lat, exp = route.RANK_SHARES[ranks]
    plan = route.Plan(route.MODE_DECODE, 8, latent=lat, experts=exp)
    ws = plan.new_workspace()
    lg = torch.zeros((8, route.EXPERTS), dtype=torch.float32, device="cuda")
    ids = torch.full((8, 16), -1, dtype=torch.int32, device="cuda")
    wt = torch.zeros((8, 16), dtype=torch.float32, device="cuda")
    x = torch.zeros((8, route.HIDDEN), dtype=torch.bfloat16, device="cuda")
    wl = torch.zeros((route.HIDDEN, lat), dtype=torch.bfloat16, device="cuda")
    wrt = torch.zeros((route.HIDDEN, exp), dtype=torch.float32, device="cuda")
    latent = torch.zeros((8, lat), dtype=torch.bfloat16, device="cuda")
    st = route.LIB.route_topk16(plan.handle, lg.data_ptr(), ids.data_ptr(), wt.data_ptr(), 8, None)
    assert st == route.E_SHAPE
    st = route.LIB.route_topk16_sharded(plan.handle, lg.data_ptr(), 8, ids.data_ptr(), wt.data_ptr(),
                                        ws.data_ptr(), 8, None)
    assert st == route.E_SHAPE
    st = route.LIB.route_fused(plan.handle, x.data_ptr(), wl.data_ptr(), wrt.data_ptr(),
                               latent.data_ptr(), None, ids.data_ptr(), wt.data_ptr(), ws.data_ptr(),
                               8, None)
    assert st == route.E_SHAPE
    torch.cuda.synchronize()
    assert (ids.cpu().numpy() == -1).all()
    assert int(ws.count_nonzero()) == 0

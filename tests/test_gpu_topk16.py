"""GPU parity of the standalone top-16 (route_topk16) through the C ABI: ids
bit-exact against the oracle on identical logits, weights within 5 FP32 ULP.
Page "Kimi K3.1 recipe: route 9..20 decode rows through the pushed pair gather
and standalone top-16", "Claims and caveats": ids identical on identical
inputs, weights within 5 fp32 ULP."""
import numpy as np
import pytest
import torch

from oracle import compare
from oracle import route_oracle as orc
from synth import generators as gen
from tests.routekit import log

pytestmark = pytest.mark.gpu

route = pytest.importorskip("latent_projection_top_amd.route")


def run_topk(plan, logits_np, rows=None):
    rows = logits_np.shape[0] if rows is None else rows
    lg = torch.from_numpy(np.ascontiguousarray(logits_np, dtype=np.float32)).cuda()
    ids = torch.full((rows, 16), -7, dtype=torch.int32, device="cuda")
    w = torch.full((rows, 16), -7.0, dtype=torch.float32, device="cuda")
    route.topk16(plan, lg, ids, w, rows=rows)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def check(logits_np, ids, w):
    ref = orc.topk16_ref(logits_np)
    bad = np.nonzero((ids != ref).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows differ, first {bad[:5]}: {ids[bad[0]]} vs {ref[bad[0]]}"
    wc = compare.weights_check(w, orc.route_weights_ref(logits_np, ref))
    assert wc["fail"] == 0, wc


@pytest.mark.parametrize("rows", list(range(1, 21)))
def test_topk16_decode_widths(rows):
    log(f"topk16 decode rows={rows}")
    plan = route.Plan(route.MODE_DECODE, rows)
    L = np.random.default_rng(1000 + rows).standard_normal((rows, 896)).astype(np.float32)
    check(L, *run_topk(plan, L))


def test_topk16_prefill_chunk():
    log("topk16 prefill rows=3072")
    plan = route.Plan(route.MODE_PREFILL, 3072)
    L = (np.random.default_rng(7).standard_normal((3072, 896)) * 2).astype(np.float32)
    check(L, *run_topk(plan, L))


def test_topk16_dense_ties_and_specials():
    log("topk16 dense ties / specials")
    plan = route.Plan(route.MODE_PREFILL, 512)
    r = np.random.default_rng(8)
    pool = np.array([-1.0, -0.0, 0.0, 1.0, 2.0, np.inf, -np.inf, np.nan], dtype=np.float32)
    rows = []
    for probs in ([.2, .2, .2, .2, .1, .0, .05, .05], [.05, .3, .3, .3, .05, 0, 0, 0],
                  [.1, .1, .1, .1, .1, .2, .1, .2], [0, 0, 0, 0, 0, 0, .01, .99],
                  [0, 0, 0, 0, 0, 0, 0, 1.0], [0, .5, .5, 0, 0, 0, 0, 0]):
        for _ in range(40):
            rows.append(r.choice(pool, size=896, p=probs))
    L = np.array(rows, dtype=np.float32)
    ids, w = run_topk(plan, L)
    ref = orc.topk16_ref(L)
    assert np.array_equal(ids, ref)
    # weights: compare where the oracle's weights are finite (rows of NaN
    # logits have NaN weights)
    with np.errstate(invalid="ignore"):
        rw = orc.route_weights_ref(L, ref)
    fin = np.isfinite(rw).all(axis=1)
    assert compare.weights_check(w[fin], rw[fin])["fail"] == 0


def test_topk16_subnormals_and_signed_zeros():
    """Rows made of FP32 subnormals of both signs, signed zeros and a few
    normal numbers: subnormals order as numbers (not as zero), -0.0 ties with
    +0.0 and the lower index wins."""
    log("topk16 subnormals and signed zeros")
    plan = route.Plan(route.MODE_PREFILL, 256)
    r = np.random.default_rng(13)
    tiny = np.float32(np.finfo(np.float32).smallest_subnormal)
    sub = (r.integers(1, 1 << 23, size=(256, 896)).astype(np.float32) * tiny).astype(np.float32)
    sign = np.where(r.random((256, 896)) < 0.5, -1.0, 1.0).astype(np.float32)
    L = (sub * sign).astype(np.float32)
    z = r.random((256, 896))
    L[z < 0.1] = np.float32(-0.0)
    L[(z >= 0.1) & (z < 0.2)] = np.float32(0.0)
    L[z > 0.999] = np.float32(1e-30)
    # rows 0..63: only 20 positive subnormals, the rest zeros of both signs,
    # so the zero ties decide the last places
    L[:64] = np.where(r.random((64, 896)) < 0.5, np.float32(-0.0), np.float32(0.0))
    for i in range(64):
        L[i, r.permutation(896)[:12]] = tiny * r.integers(1, 100, size=12).astype(np.float32)
    assert (np.abs(L[L != 0]) < np.finfo(np.float32).tiny).mean() > 0.99
    check(L, *run_topk(plan, L))


def test_topk16_quantised_logits():
    """Logits on coarse grids (steps 1/2, 1/8, 1/64, 1/1024 over a normal
    spread): many equal values within and across lanes, so the threshold
    often falls on a value several lane maxima share (the index-half search)
    and the exact-count stop of the logit-half search fires rarely. ids must
    equal the oracle's (lowest index first among equal logits)."""
    log("topk16 quantised logits")
    plan = route.Plan(route.MODE_PREFILL, 3072)
    r = np.random.default_rng(14)
    parts = []
    for step in (0.5, 0.125, 1 / 64, 1 / 1024):
        L = r.standard_normal((768, 896)) * 1.5
        parts.append((np.round(L / step) * step).astype(np.float32))
    L = np.concatenate(parts)
    check(L, *run_topk(plan, L))


def clustered_rows(n, seed):
    """Rows whose largest logits sit in 16 of the 64 lanes (expert index mod
    64): one lane all 10.0, fifteen lanes uniform in [10.5, 11]. The 16th
    largest lane maximum is then 10.0 and about 210 keys lie above it, more
    than the 64 the threshold path compacts, so these rows take the
    sort-and-rounds path."""
    r = np.random.default_rng(seed)
    L = r.standard_normal((n, 896)).astype(np.float32)
    e = np.arange(896)
    for i in range(n):
        lanes = r.permutation(64)[:16]
        for j, l in enumerate(lanes):
            m = (e % 64) == l
            L[i, m] = 10.0 if j == 0 else (10.5 + 0.5 * r.random(m.sum())).astype(np.float32)
    return L


def test_topk16_clustered_lanes():
    log("topk16 clustered lanes (more than 64 keys above the threshold)")
    plan = route.Plan(route.MODE_PREFILL, 256)
    L = np.concatenate([clustered_rows(128, 11), np.random.default_rng(12).standard_normal((128, 896))
                        .astype(np.float32)])
    check(L, *run_topk(plan, L))


def test_topk16_near_tie_sample():
    log("topk16 near-tie sample 20000 rows")
    plan = route.Plan(route.MODE_PREFILL, 3072)
    L = gen.near_tie_logits(20000, chunk=0)
    for s in range(0, 20000, 3072):
        part = L[s:s + 3072]
        check(part, *run_topk(plan, part))


def test_topk16_ragged_and_bounds():
    log("topk16 ragged rows within a larger plan")
    plan = route.Plan(route.MODE_PREFILL, 3072)
    L = np.random.default_rng(9).standard_normal((3072, 896)).astype(np.float32)
    for rows in (1, 3, 4, 5, 767, 3071):
        ids, w = run_topk(plan, L[:rows], rows=rows)
        check(L[:rows], ids, w)


def test_topk16_rows_above_plan_rejected_and_nothing_written():
    plan = route.Plan(route.MODE_DECODE, 8)
    L = torch.zeros((9, 896), dtype=torch.float32, device="cuda")
    ids = torch.full((9, 16), -7, dtype=torch.int32, device="cuda")
    w = torch.full((9, 16), -7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(route.RouteError) as e:
        route.topk16(plan, L, ids, w, rows=9)
    assert e.value.status == route.E_ROWS
    torch.cuda.synchronize()
    assert (ids == -7).all()

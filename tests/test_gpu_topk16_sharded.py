"""GPU parity of the sharded top-16 (route_topk16_sharded) through the C ABI:
a local top-16 per expert shard plus an exact merge must give, bitwise, the
ids and weights of route_topk16 on the same logits, and the oracle's ids
(topk16_sharded_ref, itself pinned equal to topk16_ref).

Shard counts: every divisor of 896 with at least 16 experts per shard; 8 and
16 are the tensor-parallel widths of page "Use two row blocks for eight-row
Kimi paired gathers" (56 experts per rank over 16 ranks). Inputs: the decode
widths and a 3072-row chunk of N(0,1) logits, the near-tie generator's rows,
rows whose largest logits crowd into one shard or into a few lanes (the
selection's fallback path), and dense ties with special values."""
import numpy as np
import pytest
import torch

from oracle import route_oracle as orc
from synth import generators as gen
from tests.routekit import log

pytestmark = pytest.mark.gpu

route = pytest.importorskip("latent_projection_top_amd.route")

SHARDS = (1, 2, 4, 7, 8, 14, 16, 28, 32, 56)


def run(plan, ws, L, shards=None):
    rows = L.shape[0]
    lg = torch.from_numpy(np.ascontiguousarray(L, dtype=np.float32)).cuda()
    ids = torch.full((rows, 16), -7, dtype=torch.int32, device="cuda")
    w = torch.full((rows, 16), -7.0, dtype=torch.float32, device="cuda")
    if shards is None:
        route.topk16(plan, lg, ids, w, rows=rows)
    else:
        route.topk16_sharded(plan, lg, shards, ids, w, ws, rows=rows)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy().view(np.uint32)


def check_all_shards(plan, ws, L, tag):
    ids0, w0 = run(plan, ws, L)
    ref = orc.topk16_ref(L)
    assert np.array_equal(ids0, ref), tag
    for s in SHARDS:
        ids, w = run(plan, ws, L, s)
        assert np.array_equal(ids, ids0), (tag, s)
        assert np.array_equal(w, w0), (tag, s)
        assert np.array_equal(ids, orc.topk16_sharded_ref(L, s)), (tag, s)
    log(f"{tag}: {L.shape[0]} rows, {len(SHARDS)} shard counts bitwise equal")


def shard_clustered(n, seed):
    r = np.random.default_rng(seed)
    L = r.standard_normal((n, 896)).astype(np.float32)
    for i in range(n):
        s = r.integers(0, 16)
        L[i, 56 * s:56 * s + 40] += 6.0
    return L


def lane_clustered(n, seed):
    r = np.random.default_rng(seed)
    L = r.standard_normal((n, 896)).astype(np.float32)
    e = np.arange(896)
    for i in range(n):
        lanes = r.permutation(64)[:16]
        for j, l in enumerate(lanes):
            m = (e % 64) == l
            L[i, m] = 10.0 if j == 0 else (10.5 + 0.5 * r.random(m.sum())).astype(np.float32)
    return L


@pytest.mark.parametrize("rows", [1, 8, 20])
def test_sharded_decode_widths(rows):
    plan = route.Plan(route.MODE_DECODE, rows)
    ws = plan.new_workspace()
    L = np.random.default_rng(500 + rows).standard_normal((rows, 896)).astype(np.float32)
    check_all_shards(plan, ws, L, f"decode rows={rows}")


def test_sharded_prefill_chunk_and_hard_rows():
    plan = route.Plan(route.MODE_PREFILL, 3072)
    ws = plan.new_workspace()
    L = (np.random.default_rng(510).standard_normal((3072, 896)) * 2).astype(np.float32)
    check_all_shards(plan, ws, L, "prefill 3072")
    nt = gen.near_tie_logits(512, chunk=0)
    check_all_shards(plan, ws, np.asarray(nt, dtype=np.float32), "near-tie 512")
    check_all_shards(plan, ws, np.concatenate([shard_clustered(128, 511), lane_clustered(128, 512)]),
                     "clustered 256")
    r = np.random.default_rng(513)
    pool = np.array([-1.0, -0.0, 0.0, 1.0, 2.0, np.inf, -np.inf, np.nan], dtype=np.float32)
    L = np.array([r.choice(pool, size=896, p=p) for p in
                  ([.2, .2, .2, .2, .1, .0, .05, .05], [.05, .3, .3, .3, .05, 0, 0, 0],
                   [0, 0, 0, 0, 0, 0, .01, .99]) for _ in range(20)], dtype=np.float32)
    check_all_shards(plan, ws, L, "dense ties / specials 60")


def test_sharded_rejects_bad_shard_counts_and_writes_nothing():
    plan = route.Plan(route.MODE_DECODE, 4)
    ws = plan.new_workspace()
    lg = torch.zeros((4, 896), dtype=torch.float32, device="cuda")
    ids = torch.full((4, 16), -7, dtype=torch.int32, device="cuda")
    w = torch.full((4, 16), -7.0, dtype=torch.float32, device="cuda")
    for s in (0, 3, 5, 64, 112, 896, -8):
        with pytest.raises(route.RouteError) as e:
            route.topk16_sharded(plan, lg, s, ids, w, ws)
        assert e.value.status == route.E_ARG
    # rows above the plan's: rejected by the C ABI before any launch
    st = route.LIB.route_topk16_sharded(plan.handle, lg.data_ptr(), 8, ids.data_ptr(), w.data_ptr(),
                                        ws.data_ptr(), 5, None)
    assert st == route.E_ROWS
    torch.cuda.synchronize()
    assert (ids == -7).all() and (w == -7.0).all()

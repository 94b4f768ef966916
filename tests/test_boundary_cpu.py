"""Host-side tests of the C ABI that need no GPU: the library loads, exports
every function include/route.h declares, and route_prepare rejects every
malformed configuration before touching the HIP runtime."""
import ctypes
import json
import os
import re

import pytest

from latent_projection_top_amd import route

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "route.h")
FACTS = json.load(open(os.path.join(ROOT, "tests", "golden", "page_facts.json")))


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(route_[a-z0-9_]+)\s*\(", src)))


def header_defines():
    out = {}
    for name, val in re.findall(r"#define\s+(ROUTE_\w+)\s+\(?(-?\d+)u?\)?", open(HEADER).read()):
        out[name] = int(val)
    return out


def test_library_exports_every_declared_function():
    declared = header_functions()
    assert set(declared) == set(route.SYMBOLS)
    lib = ctypes.CDLL(route.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_binding_constants_match_header():
    d = header_defines()
    assert d["ROUTE_HIDDEN"] == route.HIDDEN == FACTS["hidden"]["value"]
    assert d["ROUTE_LATENT"] == route.LATENT == FACTS["latent"]["value"]
    assert d["ROUTE_EXPERTS"] == route.EXPERTS
    assert d["ROUTE_TOPK"] == route.TOPK
    assert d["ROUTE_DECODE_MAX_ROWS"] == route.DECODE_MAX_ROWS == FACTS["decode_rows_accepted"]["max"]
    assert d["ROUTE_PREFILL_MAX_ROWS"] == route.PREFILL_MAX_ROWS == FACTS["prefill_chunk_rows"]["value"]
    assert d["ROUTE_ABI_VERSION"] == route.ABI_VERSION
    for k in ("OK", "E_ARG", "E_ROWS", "E_SHAPE", "E_ALIGN", "E_DEVICE", "E_HIP", "E_SCRATCH"):
        assert d["ROUTE_" + k] == getattr(route, k)
    assert d["ROUTE_STATIC_SCRATCH_BYTES"] == route.STATIC_SCRATCH_BYTES


def test_experts_match_page_shards():
    f = FACTS["router_fp32_per_rank_tp16"]
    assert route.EXPERTS == 16 * f["cols"]
    assert route.LATENT == 16 * f["latent_cols"] == 8 * FACTS["latent_columns_per_rank_tp8"]["value"]


def test_strerror_distinct():
    msgs = {route.strerror(s) for s in (0, -1, -2, -3, -4, -5, -6, -7)}
    assert len(msgs) == 8
    assert route.strerror(-99) == "unknown status"


def _prep(**kw):
    mode = kw.pop("mode", route.MODE_DECODE)
    rows = kw.pop("rows", 8)
    device = kw.pop("device", 0)
    cfg = route.make_config(mode, rows, device, **kw)
    return route.prepare_raw(cfg)


def test_prepare_null_arguments():
    assert route.LIB.route_prepare(None, None) == route.E_ARG
    out = ctypes.c_void_p(1234)
    assert route.LIB.route_prepare(None, ctypes.byref(out)) == route.E_ARG
    assert not out.value


@pytest.mark.parametrize("kw,status", [
    ({"abi_version": 2}, route.E_ARG),
    ({"mode": 7}, route.E_ARG),
    ({"hidden": 7169}, route.E_SHAPE),
    ({"latent": 448}, route.E_SHAPE),
    ({"experts": 56}, route.E_SHAPE),
    ({"latent": 448, "experts": 56}, route.E_SHAPE),
    ({"latent": 224, "experts": 112}, route.E_SHAPE),
    ({"latent": 896, "experts": 224}, route.E_SHAPE),
    ({"mode": route.MODE_PREFILL, "latent": 448, "experts": 112}, route.E_SHAPE),
    ({"mode": route.MODE_PREFILL, "latent": 224, "experts": 56}, route.E_SHAPE),
    ({"topk": 8}, route.E_SHAPE),
    ({"rows": 0}, route.E_ROWS),
    ({"rows": -3}, route.E_ROWS),
    ({"rows": 21}, route.E_ROWS),
    ({"mode": route.MODE_PREFILL, "rows": 0}, route.E_ROWS),
    ({"mode": route.MODE_PREFILL, "rows": 3073}, route.E_ROWS),
    ({"device": -1}, route.E_DEVICE),
    ({"device": 4096}, route.E_DEVICE),
])
def test_prepare_rejects(kw, status):
    st, handle = _prep(**kw)
    assert st == status
    assert handle == 0


def test_shape_checked_before_rows():
    st, _ = _prep(hidden=1, rows=99)
    assert st == route.E_SHAPE


def test_decode_envelope_matches_page():
    """1..20 decode rows pass validation, 21 does not. On a host with no GPU
    the accepted widths stop at the device check (E_DEVICE), which comes after
    every argument check."""
    f = FACTS["decode_rows_accepted"]
    have_gpu = False
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:
        pass
    for rows in range(f["min"], f["max"] + 1):
        st, handle = _prep(rows=rows)
        if have_gpu:
            assert st == route.OK
            route.LIB.route_destroy(ctypes.c_void_p(handle))
        else:
            assert st == route.E_DEVICE and handle == 0
    assert _prep(rows=f["rejected"])[0] == route.E_ROWS


def _have_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def test_rank_shares_match_pages():
    """The decode share shapes are the per-rank outputs the pages print: 448
    latent columns per rank at 8 ranks, [8, 224] BF16 latent and [8, 56] FP32
    router per rank at 16 ranks."""
    f = FACTS["router_fp32_per_rank_tp16"]
    assert route.RANK_SHARES[16] == (f["latent_cols"], f["cols"])
    assert route.RANK_SHARES[8][0] == FACTS["latent_columns_per_rank_tp8"]["value"]
    for ranks, (lat, exp) in route.RANK_SHARES.items():
        assert lat * ranks == route.LATENT and exp * ranks == route.EXPERTS


@pytest.mark.parametrize("ranks", sorted(route.RANK_SHARES))
def test_rank_share_passes_validation(ranks):
    """A decode share (1..20 rows) passes every argument check; without a GPU
    it stops at the device check."""
    lat, exp = route.RANK_SHARES[ranks]
    for rows in (1, 8, 20):
        st, handle = _prep(rows=rows, latent=lat, experts=exp)
        if _have_gpu():
            assert st == route.OK
            route.LIB.route_destroy(ctypes.c_void_p(handle))
        else:
            assert st == route.E_DEVICE and handle == 0
    assert _prep(rows=21, latent=lat, experts=exp)[0] == route.E_ROWS


def test_run_calls_reject_null_plan():
    assert route.LIB.route_latent_router(None, None, None, None, None, None, None, 1, None) == route.E_ARG
    assert route.LIB.route_topk16(None, None, None, None, 1, None) == route.E_ARG
    assert route.LIB.route_fused(None, None, None, None, None, None, None, None, None, 1, None) == route.E_ARG
    assert route.LIB.route_topk16_sharded(None, None, 8, None, None, None, 1, None) == route.E_ARG
    assert route.LIB.route_workspace_bytes(None) == 0
    assert route.LIB.route_packed_weight_bytes(None) == 0
    assert route.LIB.route_pack_weights(None, None, None, None, None) == route.E_ARG
    assert route.LIB.route_latent_router_packed(None, None, None, None, None, None, 1, None) == route.E_ARG
    assert route.LIB.route_fused_packed(None, None, None, None, None, None, None, None, 1, None) == route.E_ARG
    assert route.LIB.route_fused_packed_noalloc(None, None, None, None, None, None, None, 1, None) == route.E_ARG
    route.LIB.route_destroy(None)


def test_binding_fails_loudly_without_the_library(tmp_path, monkeypatch):
    """No fallback: with the shared library absent, loading the binding raises
    instead of computing anything another way."""
    monkeypatch.setattr(route, "LIB_PATH", str(tmp_path / "libroute.so"))
    with pytest.raises(ImportError, match="not built"):
        route._load()

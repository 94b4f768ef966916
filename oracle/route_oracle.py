"""Plain CPU oracle of the per-row MoE route: latent down projection, FP32
router logits, standalone top-16 with normalised sigmoid weights.

TEST INFRASTRUCTURE. Only the tests, the smoke entry point and the CPU-baseline
leg of the benchmark import this module. It shares no code with the HIP path and
imports nothing from it. It is slow on purpose: float64 numpy, each step the
plain definition of what the pages say the route computes.

Pages cited:
  [PR24]  "Kimi K3.1 recipe: route 9..20 decode rows through the pushed pair
          gather and standalone top-16" (voipmonitor/flare pull request 24)
  [PR16]  "Optionally gather the Kimi3 prefill latent instead of reducing it"
          (voipmonitor/flare pull request 16)
  [PR265] "Use two row blocks for eight-row Kimi paired gathers"
          (NVIDIA/hyperflare-inference pull request 265)

Readings taken where the pages are silent (each is listed in the design notes):
  * BF16 rounding is round-to-nearest-even, applied once, straight from the
    float64 value (never through float32).
  * Router logits are the float64 dot rounded once to float32.
  * Selection key: (logit descending, expert index ascending); -0.0 equals
    +0.0; NaN ranks below -inf.  Ids are emitted in key order, as int32.
  * Weights: sigmoid of each selected FP32 logit, in float64, divided by the
    sum over the 16 selected, rounded once to float32.  No bias, no grouping,
    no scaling factor.
"""
from __future__ import annotations

import numpy as np

HIDDEN = 7168
LATENT = 3584
EXPERTS = 896
TOPK = 16


# ---------------------------------------------------------------- BF16 bits --

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns (uint16) -> exact float64 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float64 values to BF16, nearest-even, in one step; return bits.

    A BF16 number has an 8-bit significand and float32's exponent range. For
    a finite v with frexp exponent E (2**(E-1) <= |v| < 2**E) the BF16 spacing
    is 2**(E-8); below the smallest normal (2**-126) it stays 2**-133. So
    v / spacing is brought to the nearest integer (ties to even, np.rint) and
    scaled back. Results of magnitude 2**128 or more are infinities. Every
    step but the rint is an exact power-of-two scaling.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    fin = np.isfinite(v)
    vf = v[fin]
    _, e = np.frexp(vf)
    q = np.maximum(e - 8, -133).astype(np.float64)
    r = np.rint(np.ldexp(vf, -q.astype(np.int64)))
    rv = np.ldexp(r, q.astype(np.int64))
    with np.errstate(over="ignore"):
        f32 = rv.astype(np.float32)   # exact: rv is a BF16 value or >= 2**128
    out[fin] = (f32.view(np.uint32) >> 16).astype(np.uint16)
    nan = np.isnan(v)
    out[nan] = 0x7FC0
    pinf = np.isposinf(v)
    ninf = np.isneginf(v)
    out[pinf] = 0x7F80
    out[ninf] = 0xFF80
    return out


# ------------------------------------------------------------ latent (a2) --

def latent_exact(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """float64 latent[r, n] = sum_k x[r, k] * W[k, n].

    [PR16] Description, numerics bullet: with the row-sharded weight each latent
    value is one full-K dot product of the hidden row with a weight column.
    W is stored [K][N] (N contiguous). Every BF16 x BF16 product is exact in
    float64; the float64 sum error is far below a BF16 unit.
    """
    x = bf16_bits_to_f64(x_bits)
    w = bf16_bits_to_f64(w_bits)
    return x @ w


def latent_abs_terms(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """sum_k |x[r, k] * W[k, n]| in float64 (the scale of the accumulation
    error of any FP32 summation order)."""
    return np.abs(bf16_bits_to_f64(x_bits)) @ np.abs(bf16_bits_to_f64(w_bits))


def latent_ref(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """BF16 latent, rounded once from the full-K dot ([PR16] Description,
    numerics bullet: one FP32-accumulated full-K dot, rounded once). Bits."""
    return round_f64_to_bf16_bits(latent_exact(x_bits, w_bits))


def two_round_latent_ref(x_bits: np.ndarray, w_bits: np.ndarray,
                         shards: int = 8) -> np.ndarray:
    """The general (column-sharded) path's latent, for accuracy comparisons.

    [PR16] Description, numerics bullet: today a latent value is 8 BF16-rounded
    K-shard partials, summed in FP32, then rounded to BF16 again. The shards are
    contiguous K ranges of equal width, summed in shard order.
    """
    x = bf16_bits_to_f64(x_bits)
    w = bf16_bits_to_f64(w_bits)
    k = x.shape[1]
    assert k % shards == 0
    step = k // shards
    acc = np.zeros((x.shape[0], w.shape[1]), dtype=np.float32)
    for s in range(shards):
        part = x[:, s * step:(s + 1) * step] @ w[s * step:(s + 1) * step]
        part16 = bf16_bits_to_f64(round_f64_to_bf16_bits(part)).astype(np.float32)
        acc = (acc + part16).astype(np.float32)
    return round_f64_to_bf16_bits(acc.astype(np.float64))


# ------------------------------------------------------------ router (a3) --

def logits_exact(x_bits: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """float64 router logits[r, e] = sum_k x[r, k] * Wr[k, e].

    [PR265] description: the router output exchanged beside the latent rows is
    FP32. BF16 x FP32 products are exact in float64.
    """
    x = bf16_bits_to_f64(x_bits)
    return x @ np.asarray(w_router, dtype=np.float32).astype(np.float64)


def logits_abs_terms(x_bits: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """sum_k |x[r, k] * Wr[k, e]| in float64 (the scale of the accumulation
    error of any FP32 summation order of the logit's terms)."""
    x = bf16_bits_to_f64(x_bits)
    return np.abs(x) @ np.abs(np.asarray(w_router, dtype=np.float32).astype(np.float64))


def logits_ref(x_bits: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """FP32 router logits, the float64 dot rounded once (nearest-even)."""
    return logits_exact(x_bits, w_router).astype(np.float32)


# ----------------------------------------------------------- top-16 (a5) --

def _rank_order(logits: np.ndarray) -> np.ndarray:
    """Expert indices of each row sorted by (logit descending, index
    ascending), with -0.0 equal to +0.0 and NaN after every number.

    A plain lexicographic sort on three keys: whether the logit is NaN, the
    negated logit, the expert index (np.lexsort takes its last key as the
    primary one).
    """
    v = np.atleast_2d(np.asarray(logits, dtype=np.float32)).astype(np.float64) + 0.0  # -0.0 -> +0.0
    nan = np.isnan(v)
    neg = np.where(nan, 0.0, -v)
    idx = np.broadcast_to(np.arange(v.shape[-1]), v.shape)
    return np.lexsort((idx, neg, nan), axis=-1)


def topk16_ref(logits: np.ndarray, k: int = TOPK) -> np.ndarray:
    """Standalone top-16 ids per row, int32 [rows, 16], in selection order.

    [PR24] "What / why" and "Dependency": the standalone top-16 selects each
    row's experts from the router logits for rounds of 1..20 rows. The ids are
    the first k of the full sort of the row's experts by (logit descending,
    index ascending).
    """
    return _rank_order(logits)[:, :k].astype(np.int32)


def topk16_sharded_ref(logits: np.ndarray, shards: int, k: int = TOPK) -> np.ndarray:
    """Top-16 ids as a route whose experts are split over ranks selects them,
    int32 [rows, 16], in selection order.

    [PR24] "What / why": each row keeps its 16 largest experts; [PR265]: the
    router output is split by expert over the ranks (56 experts per rank over
    16 ranks). Step 1: each of `shards` contiguous expert shards keeps its own
    top k (topk16_ref on the shard's columns, mapped back to global expert
    numbers). Step 2: the row's top k among the k * shards candidates, by the
    same order on (logit, global index).
    """
    logits = np.atleast_2d(np.asarray(logits, dtype=np.float32))
    rows, e = logits.shape
    if shards < 1 or e % shards or e // shards < k:
        raise ValueError("shards must divide the experts with at least k per shard")
    size = e // shards
    cand = np.concatenate([s * size + topk16_ref(logits[:, s * size:(s + 1) * size], k)
                           for s in range(shards)], axis=1).astype(np.int64)
    cand.sort(axis=1)        # global index order, so that ties break on the index
    vals = np.take_along_axis(logits, cand, axis=1)
    return np.take_along_axis(cand, _rank_order(vals)[:, :k], axis=1).astype(np.int32)


def route_weights_ref(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Normalised sigmoid weights of the selected experts, float32 [rows, 16].

    Reading of the row's routing weights: s_i = 1 / (1 + exp(-l_i)) in float64
    from the FP32 logit, w_i = s_i / sum_j s_j over the 16 selected, rounded
    once to float32. [PR24] "Claims and caveats" compares these weights across
    paths within 5 fp32 ULP.
    """
    sel = np.take_along_axis(np.atleast_2d(logits).astype(np.float32),
                             np.asarray(ids, dtype=np.int64), axis=1)
    s = 1.0 / (1.0 + np.exp(-sel.astype(np.float64)))
    return (s / s.sum(axis=1, keepdims=True)).astype(np.float32)


# ------------------------------------------------------------- whole route --

def widen_weights(w_bits: np.ndarray, w_router: np.ndarray):
    """float64 copies of the latent and router weights (exact widening), so a
    caller routing many batches through the same layer converts them once."""
    return bf16_bits_to_f64(w_bits), np.asarray(w_router, dtype=np.float32).astype(np.float64)


def route_ref_widened(x_bits: np.ndarray, w64: np.ndarray, wr64: np.ndarray) -> dict:
    """Every output of the route, from weights already widened to float64.
    The same steps as latent_ref, logits_ref, topk16_ref and route_weights_ref."""
    x = bf16_bits_to_f64(x_bits)
    logits = (x @ wr64).astype(np.float32)
    ids = topk16_ref(logits)
    return {
        "latent": round_f64_to_bf16_bits(x @ w64),
        "logits": logits,
        "ids": ids,
        "weights": route_weights_ref(logits, ids),
    }


def route_detail_widened(x_bits: np.ndarray, w64: np.ndarray, wr64: np.ndarray) -> dict:
    """route_ref_widened's outputs plus what the comparators need beside them:
    the float64 latent and logit dots ("exact", "logits_exact") and the sums
    of their terms' magnitudes ("abs_terms", "logits_abs_terms"), the same
    quantities as latent_exact, latent_abs_terms, logits_exact and
    logits_abs_terms, from weights widened once."""
    x = bf16_bits_to_f64(x_bits)
    exact = x @ w64
    lexact = x @ wr64
    logits = lexact.astype(np.float32)
    ids = topk16_ref(logits)
    ax = np.abs(x)
    return {
        "exact": exact,
        "abs_terms": ax @ np.abs(w64),
        "logits_exact": lexact,
        "logits_abs_terms": ax @ np.abs(wr64),
        "latent": round_f64_to_bf16_bits(exact),
        "logits": logits,
        "ids": ids,
        "weights": route_weights_ref(logits, ids),
    }


def route_ref(x_bits: np.ndarray, w_bits: np.ndarray, w_router: np.ndarray) -> dict:
    """Every output of the route for the given rows."""
    return route_ref_widened(x_bits, *widen_weights(w_bits, w_router))

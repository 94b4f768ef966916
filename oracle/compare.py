"""Comparators that check an implementation's route outputs against the oracle.

TEST INFRASTRUCTURE (see route_oracle). Pure numpy; imports nothing from the
HIP path.

Criteria, from the pages' statement of what must match:
  * latent: within 1 BF16 ULP of the correctly rounded value, or, for outputs
    inside the cancellation band, |got - exact| <= ulp_bf16(got)/2 +
    2**-24 * sum_k |x_k W_k| (any FP32 accumulation order has at most this
    error, and one BF16 unit is smaller than it there); relative RMS against
    float64 stays at one BF16 rounding ([PR16] Description, numerics bullet);
  * ids: on identical logits bit-exact; end to end, per row at most one id in /
    one id out, that pair's oracle logits within 2 float32 ULP, and the emitted
    order consistent with the oracle logits within 2 ULP ([PR24] "Claims and
    caveats", near-tie gate);
  * weights: within 5 float32 ULP ([PR24] "Claims and caveats").
"""
from __future__ import annotations

import numpy as np

from .route_oracle import bf16_bits_to_f64

U32 = 2.0 ** -24


def rel_rms(a: np.ndarray, e: np.ndarray) -> float:
    """Aggregate relative RMS: sqrt(sum (a-e)^2 / sum e^2)."""
    a = np.asarray(a, dtype=np.float64)
    e = np.asarray(e, dtype=np.float64)
    return float(np.sqrt(np.sum((a - e) ** 2) / np.sum(e ** 2)))


def _ordered_f32(v: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.int64)
    mag = b & 0x7FFFFFFF
    return np.where(b >> 31 == 1, -mag, mag)


def f32_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Number of float32 values between a and b (0 for -0.0 vs +0.0)."""
    return np.abs(_ordered_f32(a) - _ordered_f32(b))


def _ordered_bf16(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b >> 15 == 1, -mag, mag)


def bf16_ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    return np.abs(_ordered_bf16(a_bits) - _ordered_bf16(b_bits))


def bf16_spacing(bits: np.ndarray) -> np.ndarray:
    """BF16 unit in the last place at each BF16 value."""
    e = (np.asarray(bits, dtype=np.uint16).astype(np.int64) >> 7) & 0xFF
    return np.ldexp(1.0, np.where(e == 0, -133, e - 127 - 7))


def latent_check(got_bits, ref_bits, exact, abs_terms) -> dict:
    """Check BF16 latent bits against the oracle (see module docstring)."""
    got_bits = np.asarray(got_bits, dtype=np.uint16)
    d = bf16_ulp_distance(got_bits, ref_bits)
    within = d <= 1
    g = bf16_bits_to_f64(got_bits)
    band_ok = np.abs(g - exact) <= 0.5 * bf16_spacing(got_bits) + U32 * abs_terms
    band = (~within) & band_ok
    fail = (~within) & (~band_ok)
    return {
        "n": int(d.size),
        "within_1ulp": int(within.sum()),
        "band": int(band.sum()),
        "fail": int(fail.sum()),
        "max_ulp": int(d.max()) if d.size else 0,
        "exact_match": int((d == 0).sum()),
        "rel_rms": rel_rms(g, exact) if d.size else 0.0,
    }


def f32_spacing(v: np.ndarray) -> np.ndarray:
    """float32 unit in the last place at each float32 value."""
    e = (np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.int64) >> 23) & 0xFF
    return np.ldexp(1.0, np.where(e == 0, -149, e - 127 - 23))


def logits_check(got, ref, exact, abs_terms, c: float = 1.0) -> dict:
    """Check FP32 logits: within 1 ULP of the correctly rounded value, or
    |got - exact| <= ulp(got)/2 + c * 2**-24 * sum_k |x_k Wr_k| (the error any
    summation of FP32-rounded partial sums can reach when a logit is small
    against the magnitude of its terms)."""
    got = np.asarray(got, dtype=np.float32)
    d = f32_ulp_distance(got, ref)
    within = d <= 1
    err = np.abs(got.astype(np.float64) - exact)
    band_ok = err <= 0.5 * f32_spacing(got) + c * U32 * abs_terms
    large = np.abs(exact) >= 1.0
    return {
        "n": int(d.size),
        "within_1ulp": int(within.sum()),
        "band": int(((~within) & band_ok).sum()),
        "fail": int(((~within) & (~band_ok)).sum()),
        "max_ulp": int(d.max()) if d.size else 0,
        # ULP distance where the logit is at least 1 in magnitude (the range
        # the top-16 selects from, where a unit is a fixed fraction of it)
        "large_n": int(large.sum()),
        "large_mean_ulp": float(d[large].mean()) if large.any() else 0.0,
        "large_max_ulp": int(d[large].max()) if large.any() else 0,
        # (outputs whose terms are all zero have no scale and are left out)
        "max_err_over_terms": float((err[abs_terms > 0] / (U32 * abs_terms[abs_terms > 0])).max())
        if (abs_terms > 0).any() else 0.0,
    }


def ids_check(got_ids, ref_ids, ref_logits, max_ulp: int = 2) -> dict:
    """End-to-end id rule. Returns counts of equal rows, 1-for-1 swap rows and
    violating rows (with the violating row indices)."""
    got_ids = np.asarray(got_ids, dtype=np.int64)
    ref_ids = np.asarray(ref_ids, dtype=np.int64)
    ref_logits = np.asarray(ref_logits, dtype=np.float32)
    equal = swaps = 0
    bad = []
    for r in range(got_ids.shape[0]):
        g, o = got_ids[r], ref_ids[r]
        if np.array_equal(g, o):
            equal += 1
            continue
        gs, os_ = set(g.tolist()), set(o.tolist())
        ok = len(gs) == len(g)
        extra, missing = gs - os_, os_ - gs
        if ok and len(extra) <= 1 and len(extra) == len(missing):
            if extra:
                i, j = extra.pop(), missing.pop()
                ok = f32_ulp_distance(ref_logits[r, i], ref_logits[r, j]) <= max_ulp
            lg = ref_logits[r, g]
            for a in range(len(g) - 1):
                if lg[a] < lg[a + 1] and f32_ulp_distance(lg[a], lg[a + 1]) > max_ulp:
                    ok = False
        else:
            ok = False
        if ok:
            swaps += int(gs != os_)
            equal += int(gs == os_)
        else:
            bad.append(r)
    return {"rows": int(got_ids.shape[0]), "equal": equal, "swaps": swaps,
            "violations": len(bad), "bad_rows": bad}


def weights_check(got_w, ref_w, max_ulp: int = 5) -> dict:
    d = f32_ulp_distance(got_w, ref_w)
    return {"n": int(d.size), "max_ulp": int(d.max()) if d.size else 0,
            "fail": int((d > max_ulp).sum())}

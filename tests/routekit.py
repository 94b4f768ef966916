"""Shared helpers of the GPU tests: tensor conversion, cached seeded weights,
and a tiny wrapper that runs the route through the C ABI."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

from oracle import compare
from synth import generators as gen


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_dev(bits: np.ndarray, dev="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def bits_host(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@functools.lru_cache(maxsize=2)
def weights_host(copy: int = 0):
    return gen.latent_weight(copy), gen.router_weight(copy)


@functools.lru_cache(maxsize=2)
def weights_dev(copy: int = 0):
    w, wr = weights_host(copy)
    return bf16_dev(w), torch.from_numpy(wr).cuda()


@functools.lru_cache(maxsize=2)
def weights_f64(copy: int = 0):
    """Oracle-side float64 copies of the weights, widened once per session."""
    from oracle import route_oracle as orc
    return orc.widen_weights(*weights_host(copy))


def oracle_rows(x_bits: np.ndarray, copy: int = 0) -> dict:
    """Oracle outputs for many rows at once, with the float64 dots and term
    magnitudes the comparators need (oracle.route_detail_widened on weights
    widened once per session)."""
    from oracle import route_oracle as orc
    return orc.route_detail_widened(x_bits, *weights_f64(copy))


def assert_fp64_logits(got, ref, allowance: float = 1e-5) -> None:
    """Logits the decode route accumulates in FP64 and rounds once: equal to
    the oracle's correctly rounded FP32 values, except that two float64 sums
    of the same exact terms in different orders can fall on either side of an
    FP32 rounding boundary (their difference is about 1e-16 of the sum of the
    terms' magnitudes against an FP32 unit of about 6e-8 of the logit), so at
    most 1 ULP and, counted, at most `allowance` of the outputs may differ."""
    d = compare.f32_ulp_distance(got, ref)
    off = int((d > 0).sum())
    assert d.max() <= 1, f"logit {int(d.max())} ULP from the oracle"
    assert off <= max(2, allowance * d.size), f"{off} of {d.size} logits 1 ULP off"


def assert_prefill_logit_error(gc: dict) -> None:
    """Prefill logits: FP32 MFMA chains of at most 256 K terms folded into
    FP64. Besides compare.logits_check's pass / fail (every logit within
    ulp/2 + 2^-24 * sum_k |x_k Wr_k| of the exact dot), three caps set from
    the measured error of this accumulation (four 3072-row chunks with
    outliers: largest error 0.59 of 2^-24 * sum_k |x_k Wr_k|, 42 % of the
    logits more than 1 ULP from the correctly rounded value, mean distance
    0.99 ULP and largest 15 ULP where |logit| >= 1), each with a margin, so
    that a longer chain or a lost restart fails (one chain over all 7168 K
    reaches about 2.5 units)."""
    assert gc["max_err_over_terms"] <= 0.75, gc
    assert gc["band"] <= 0.5 * gc["n"], gc
    assert gc["large_mean_ulp"] <= 1.5 and gc["large_max_ulp"] <= 32, gc


class Outputs:
    def __init__(self, rows: int, dev="cuda"):
        from latent_projection_top_amd import route
        self.latent = torch.empty((rows, route.LATENT), dtype=torch.bfloat16, device=dev)
        self.logits = torch.empty((rows, route.EXPERTS), dtype=torch.float32, device=dev)
        self.ids = torch.empty((rows, route.TOPK), dtype=torch.int32, device=dev)
        self.weights = torch.empty((rows, route.TOPK), dtype=torch.float32, device=dev)

    def poison(self):
        self.latent.view(torch.int16).fill_(-1)
        self.logits.view(torch.int32).fill_(-1)
        self.ids.fill_(-1)
        self.weights.view(torch.int32).fill_(-1)

    def host(self, rows: int | None = None) -> dict:
        r = slice(None) if rows is None else slice(0, rows)
        return {
            "latent": bits_host(self.latent[r]),
            "logits": self.logits[r].cpu().numpy(),
            "ids": self.ids[r].cpu().numpy(),
            "weights": self.weights[r].cpu().numpy(),
        }


def decode_counters_idle(ws: torch.Tensor) -> bool:
    """State a whole-route decode workspace is left in after every call: the
    84 per-tile counters at zero, the row-phase parity 0 or 1, and the
    counter pair the next call will use cleared."""
    c = ws[:512].view(torch.int32).cpu().numpy()
    par = int(c[84])
    return bool((c[:84] == 0).all() and par in (0, 1) and c[85] == 0
                and c[86 + 2 * par] == 0 and c[87 + 2 * par] == 0 and (c[90:] == 0).all())

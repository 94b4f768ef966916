"""Shared helpers of the GPU tests: tensor conversion, cached seeded weights,
and a tiny wrapper that runs the route through the C ABI."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

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
    """Oracle-side float64 views of the weights, converted once per session."""
    from oracle import route_oracle as orc
    w, wr = weights_host(copy)
    return orc.bf16_bits_to_f64(w), wr.astype(np.float64)


def oracle_rows(x_bits: np.ndarray, copy: int = 0) -> dict:
    """Oracle outputs for many rows at once (float64 dots with cached weights).
    Same arithmetic as oracle.route_ref; the weights are widened once."""
    from oracle import route_oracle as orc
    w64, wr64 = weights_f64(copy)
    x64 = orc.bf16_bits_to_f64(x_bits)
    exact = x64 @ w64
    lexact = x64 @ wr64
    logits = lexact.astype(np.float32)
    ids = orc.topk16_ref(logits)
    return {
        "exact": exact,
        "abs_terms": np.abs(x64) @ np.abs(w64),
        "logits_exact": lexact,
        "logits_abs_terms": np.abs(x64) @ np.abs(wr64),
        "latent": orc.round_f64_to_bf16_bits(exact),
        "logits": logits,
        "ids": ids,
        "weights": orc.route_weights_ref(logits, ids),
    }


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

"""Seeded synthetic inputs for the per-row MoE route.

This module only draws numbers. It holds none of the route's arithmetic (no
projection, no rounding rule of its own, no selection); BF16 tensors are made
by torch's own float32 -> bfloat16 conversion. Both the CPU oracle tests and the
GPU tests / benchmark take their inputs from here, so that the two sides see the
same bits.

Pages (the method's source):
  [PR24]  "Kimi K3.1 recipe: route 9..20 decode rows through the pushed pair
          gather and standalone top-16" (voipmonitor/flare pull request 24)
  [PR16]  "Optionally gather the Kimi3 prefill latent instead of reducing it"
          (voipmonitor/flare pull request 16)

Recipe (no real weights are available, so everything is synthetic):
  * every draw comes from numpy's PCG64 seeded with (seed, tag, index);
  * hidden rows x ~ N(0,1), shape [rows, 7168]  ([PR16] Description: K 7168);
    prefill chunks may scale 1 % of the channels (72, chosen without
    replacement) by 20 before rounding, to model outlier channels;
  * latent weight W ~ N(0, 1/7168), shape [7168, 3584]  ([PR16] Description:
    latent 3584, K 7168), BF16;
  * router weight Wr ~ N(0, 1/7168), shape [7168, 896], FP32 (896 experts:
    16 ranks x 56 router columns per rank, [PR265] description);
  * float64 draws are cast to float32 (round to nearest even), then torch
    converts float32 -> bfloat16 (round to nearest even);
  * the cancelling set and the near-tie logits follow the accuracy and
    near-tie claims of [PR16] Description (cancelling partials) and [PR24]
    "Claims and caveats" (near-tie gate).
"""
from __future__ import annotations

import numpy as np
import torch

HIDDEN = 7168
LATENT = 3584
EXPERTS = 896
TOPK = 16

TAG_HIDDEN = 0
TAG_W_LATENT = 1
TAG_W_ROUTER = 2
TAG_OUTLIER = 3
TAG_CANCEL = 4
TAG_NEAR_TIE = 5
TAG_COPY = 6

OUTLIER_FRACTION = 0.01
OUTLIER_SCALE = 20.0


def rng(tag: int, index: int, seed: int = 0) -> np.random.Generator:
    """PCG64 stream for (seed, tag, index)."""
    return np.random.default_rng([int(seed), int(tag), int(index)])


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float64/float32 array -> BF16 bit patterns (uint16), via torch's cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def outlier_channels(seed: int = 0) -> np.ndarray:
    """The 72 (1 % of 7168) hidden channels scaled x20 in prefill chunks."""
    n = int(round(OUTLIER_FRACTION * HIDDEN))
    return np.sort(rng(TAG_OUTLIER, 0, seed).choice(HIDDEN, size=n, replace=False))


def hidden(rows: int, bank: int = 0, seed: int = 0, outliers: bool = False,
           hidden_dim: int = HIDDEN) -> np.ndarray:
    """Hidden rows x[rows, hidden_dim] as BF16 bits, x ~ N(0,1)."""
    x = rng(TAG_HIDDEN, bank, seed).standard_normal((rows, hidden_dim))
    if outliers:
        ch = outlier_channels(seed)
        ch = ch[ch < hidden_dim]
        x[:, ch] *= OUTLIER_SCALE
    return to_bf16_bits(x)


def latent_weight(copy: int = 0, seed: int = 0, k: int = HIDDEN,
                  n: int = LATENT) -> np.ndarray:
    """Latent down-projection weight W[k, n] ([K][N], N contiguous), BF16 bits."""
    g = rng(TAG_W_LATENT, copy, seed)
    return to_bf16_bits(g.standard_normal((k, n)) * (1.0 / np.sqrt(HIDDEN)))


def router_weight(copy: int = 0, seed: int = 0, k: int = HIDDEN,
                  e: int = EXPERTS) -> np.ndarray:
    """Router weight Wr[k, e] ([K][E], E contiguous), float32."""
    g = rng(TAG_W_ROUTER, copy, seed)
    return (g.standard_normal((k, e)) * (1.0 / np.sqrt(HIDDEN))).astype(np.float32)


def cancel_set(rows: int = 1024, seed: int = 0):
    """Rows whose hidden x latent-weight partials cancel.

    x[:, k + 3584] = x[:, k] and Wc[k + 3584, :] = -Wc[k, :], so the halves of
    K cancel exactly; then 20..35 pairs per row are broken by a fresh N(0,1)
    draw in the upper half, leaving |sum| about 1e-3 of the sum of |terms|.
    The two halves map onto K shards s and s+4 of an 8-way K split, which is the
    case where per-shard rounding loses the most.
    Returns (x_bits [rows, 7168], wc_bits [7168, 3584]).
    """
    half = HIDDEN // 2
    g = rng(TAG_CANCEL, 0, seed)
    w_half = g.standard_normal((half, LATENT)) * (1.0 / np.sqrt(HIDDEN))
    wc = np.concatenate([w_half, -w_half], axis=0)
    xb = rng(TAG_CANCEL, 1, seed).standard_normal((rows, half))
    x = np.concatenate([xb, xb], axis=1)
    gb = rng(TAG_CANCEL, 2, seed)
    for r in range(rows):
        m = int(gb.integers(20, 36))
        ks = gb.choice(half, size=m, replace=False)
        x[r, half + ks] = gb.standard_normal(m)
    return to_bf16_bits(x), to_bf16_bits(wc)


def near_tie_logits(rows: int, chunk: int, seed: int = 0) -> np.ndarray:
    """FP32 router logits [rows, 896] with planted 16th/17th-slot near ties.

    Base rows are N(0,1) float32.  Per row one class is planted:
      * 98 %: the 17th-largest value is set g in {0..4} float32 ULPs below the
        16th (g = 0 is an exact tie decided by the expert index);
      * 0.5 %: a 3-way exact tie on slots 15..17; 0.5 %: a 5-way tie on 14..18;
      * 1 %: slots 16 and 17 are +0.0 and -0.0 (in random order), with the 15
        larger values positive and the rest negative;
      * chunk 0 additionally makes its first 3 rows all-equal.
    """
    g = rng(TAG_NEAR_TIE, chunk, seed)
    L = g.standard_normal((rows, EXPERTS), dtype=np.float32)
    u = g.random(rows)
    gap = g.integers(0, 5, rows)
    flip = g.random(rows) < 0.5
    # positions of the 18 largest values per row, largest first
    top = np.argpartition(-L, 18, axis=1)[:, :18]
    tv = np.take_along_axis(L, top, axis=1)
    o = np.argsort(-tv, axis=1, kind="stable")
    top = np.take_along_axis(top, o, axis=1)
    ar = np.arange(rows)

    gap_rows = u >= 0.02
    if gap_rows.any():
        r = ar[gap_rows]
        v16 = L[r, top[r, 15]]
        v = v16.copy()
        for step in range(4):
            m = gap[r] > step
            v[m] = np.nextafter(v[m], np.float32(-np.inf))
        L[r, top[r, 16]] = v

    tie3 = u < 0.005
    if tie3.any():
        r = ar[tie3]
        v = L[r, top[r, 14]]
        for s in (15, 16):
            L[r, top[r, s]] = v
    tie5 = (u >= 0.005) & (u < 0.01)
    if tie5.any():
        r = ar[tie5]
        v = L[r, top[r, 13]]
        for s in (14, 15, 16, 17):
            L[r, top[r, s]] = v

    zero = (u >= 0.01) & (u < 0.02)
    if zero.any():
        r = ar[zero]
        A = np.abs(L[r])
        A[A == 0] = np.float32(1e-3)
        Lr = -A
        pos_idx = top[r, :15]
        np.put_along_axis(Lr, pos_idx, np.take_along_axis(A, pos_idx, 1), axis=1)
        a = np.where(flip[r], np.float32(0.0), np.float32(-0.0))
        b = np.where(flip[r], np.float32(-0.0), np.float32(0.0))
        Lr[np.arange(len(r)), top[r, 15]] = a
        Lr[np.arange(len(r)), top[r, 16]] = b
        L[r] = Lr

    if chunk == 0:
        for i in range(min(3, rows)):
            L[i, :] = np.float32(0.25 * (i + 1))
    return L

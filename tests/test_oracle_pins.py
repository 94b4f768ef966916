"""Pins of the CPU oracle to things other than itself: exact rational
arithmetic on tiny inputs, closed forms, special cases with known answers,
brute-force sorting, and the accuracy figures the pages print.

Each test is built so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, a wrong rounding rule or tie-break)
fails at least one of them.
"""
import bisect
import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle as o
from oracle import compare as c
from synth import generators as g

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")
FACTS = json.load(open(GOLDEN))

# ------------------------------------------------------------ references --
# Positive finite BF16 magnitudes, bit patterns 0x0000..0x7F7F, increasing.
_POS_BITS = np.arange(0x7F80, dtype=np.uint32)
_POS_VALS = [Fraction(float(v)) for v in
             (_POS_BITS << 16).astype(np.uint32).view(np.float32).astype(np.float64)]
_BF16_OVERFLOW = Fraction(2) ** 128 - Fraction(2) ** 119   # max + half a unit


def rne_bf16_reference(a, negative_zero=False) -> int:
    """Textbook round-to-nearest-even of an exact rational to BF16 bits."""
    a = Fraction(a)
    sign = 0x8000 if (a < 0 or (a == 0 and negative_zero)) else 0
    m = abs(a)
    if m >= _BF16_OVERFLOW:
        return sign | 0x7F80
    i = bisect.bisect_left(_POS_VALS, m)
    if i < len(_POS_VALS) and _POS_VALS[i] == m:
        return sign | int(_POS_BITS[i])
    if i == len(_POS_VALS):          # above the largest finite value,
        return sign | 0x7F7F           # below the overflow threshold
    lo, hi = i - 1, i
    dlo, dhi = m - _POS_VALS[lo], _POS_VALS[hi] - m
    if dlo < dhi:
        pick = lo
    elif dhi < dlo:
        pick = hi
    else:
        pick = lo if int(_POS_BITS[lo]) % 2 == 0 else hi
    return sign | int(_POS_BITS[pick])


def rne_f32_reference(a) -> np.float32:
    """Correct float32 rounding of an exact rational (neighbour search)."""
    a = Fraction(a)
    f = np.float32(float(a))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = None
    for cnd in cands:
        d = abs(Fraction(float(cnd)) - a)
        key = (d, int(np.array(cnd).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cnd)
    return np.float32(best[1])


def to_bits(vals) -> np.ndarray:
    return g.to_bf16_bits(np.asarray(vals, dtype=np.float64))


# ---------------------------------------------------------- BF16 rounding --

def test_bf16_rounding_matches_rational_rne():
    r = np.random.default_rng(11)
    vals = list(r.standard_normal(3000) * np.exp2(r.integers(-140, 130, 3000)))
    # exact halfway points between neighbouring BF16 values, and just off them
    for b in r.integers(1, 0x7F7F, 400):
        lo = float(_POS_VALS[b])
        hi = float(_POS_VALS[b + 1])
        mid = (lo + hi) / 2          # exact in float64
        vals += [mid, -mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf)]
    vals += [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 2.0 ** -133, 2.0 ** -134,
             3 * 2.0 ** -135, 2.0 ** -126 * (1 - 2 ** -9), float(_BF16_OVERFLOW),
             np.nextafter(float(_BF16_OVERFLOW), 0), -float(_BF16_OVERFLOW), 1e300, -1e-300]
    v = np.array(vals, dtype=np.float64)
    got = o.round_f64_to_bf16_bits(v)
    want = [rne_bf16_reference(Fraction(float(x)), negative_zero=math.copysign(1, x) < 0)
            for x in v]
    assert got.tolist() == want


def test_bf16_rounding_specials():
    got = o.round_f64_to_bf16_bits(np.array([np.inf, -np.inf, np.nan]))
    assert got[0] == 0x7F80 and got[1] == 0xFF80
    assert (got[2] & 0x7F80) == 0x7F80 and (got[2] & 0x7F) != 0


def test_bf16_rounding_is_not_through_float32():
    # 1 + 2^-8 + 2^-30 lies just above a BF16 halfway point; a float32 stop
    # would land exactly on the halfway point and round down to 1.0.
    v = np.array([1.0 + 2 ** -8 + 2 ** -30])
    assert o.round_f64_to_bf16_bits(v)[0] == 0x3F81
    assert rne_bf16_reference(Fraction(v[0])) == 0x3F81


# -------------------------------------------------------------- latent --

@pytest.mark.parametrize("k", [2, 7, 64])
def test_latent_bruteforce_rational(k):
    r = np.random.default_rng(k)
    x = to_bits(r.standard_normal((3, k)) * np.exp2(r.integers(-6, 6, (3, k))))
    w = to_bits(r.standard_normal((k, 5)) * 0.1)
    got = o.latent_ref(x, w)
    xf = o.bf16_bits_to_f64(x)
    wf = o.bf16_bits_to_f64(w)
    for i in range(3):
        for n in range(5):
            exact = sum(Fraction(float(xf[i, j])) * Fraction(float(wf[j, n])) for j in range(k))
            assert got[i, n] == rne_bf16_reference(exact), (i, n)


def test_latent_designed_halfway_cases():
    x = to_bits([[1.0, 2 ** -8, 0.0], [1.0, 3 * 2 ** -8, 0.0], [1.0, 2 ** -8, 2 ** -30],
                 [-1.0, -(2 ** -8), -(2 ** -30)]])
    w = to_bits([[1.0], [1.0], [1.0]])
    got = o.latent_ref(x, w)[:, 0].tolist()
    assert got == [0x3F80, 0x3F82, 0x3F81, 0xBF81]


def test_latent_identity_weight_full_shape():
    x = g.hidden(4, bank=7)
    w = np.zeros((g.HIDDEN, g.LATENT), dtype=np.uint16)
    w[np.arange(g.LATENT), np.arange(g.LATENT)] = 0x3F80      # 1.0
    got = o.latent_ref(x, w)
    ref = x[:, :g.LATENT].copy()
    ref[ref == 0x8000] = 0x0000      # -0.0 * 1 + (+0 terms) sums to +0.0
    assert np.array_equal(got, ref)


def test_latent_one_hot_rows_pin_orientation():
    w = g.latent_weight(0)
    ks = [0, 1, 3583, 3584, 7167]
    x = np.zeros((len(ks), g.HIDDEN), dtype=np.uint16)
    x[np.arange(len(ks)), ks] = 0x3F80
    got = o.latent_ref(x, w)
    want = w[ks].copy()
    want[want == 0x8000] = 0
    assert np.array_equal(got, want)


def test_latent_minus_sign_and_column_independence():
    r = np.random.default_rng(3)
    x = to_bits(r.standard_normal((2, 64)))
    w = to_bits(r.standard_normal((64, 6)))
    neg_w = w ^ np.uint16(0x8000)
    a = o.latent_ref(x, w)
    b = o.latent_ref(x, neg_w)
    nz = (a & 0x7FFF) != 0
    assert np.array_equal(a[nz] ^ np.uint16(0x8000), b[nz])
    # dropping a column of W changes only that column of the output
    assert np.array_equal(o.latent_ref(x, w[:, :3]), a[:, :3])


# ---------------------------------------------------- accuracy page facts --

@pytest.fixture(scope="module")
def accuracy_set():
    x = g.hidden(32, bank=0)
    w = g.latent_weight(0)
    e = o.latent_exact(x, w)
    one = o.latent_ref(x, w)
    two = o.two_round_latent_ref(x, w)
    return x, w, e, one, two


def test_one_rounding_rel_rms_matches_page(accuracy_set):
    _, _, e, one, _ = accuracy_set
    page = FACTS["latent_rel_rms_one_rounding"]["value"]
    assert abs(c.rel_rms(o.bf16_bits_to_f64(one), e) / page - 1) < 0.05


def test_two_roundings_rel_rms_matches_page(accuracy_set):
    _, _, e, one, two = accuracy_set
    page = FACTS["latent_rel_rms_two_roundings"]["value"]
    rr_two = c.rel_rms(o.bf16_bits_to_f64(two), e)
    assert abs(rr_two / page - 1) < 0.05
    assert rr_two > c.rel_rms(o.bf16_bits_to_f64(one), e)
    page_vs = FACTS["latent_rel_rms_route_vs_general"]["value"]
    assert abs(c.rel_rms(o.bf16_bits_to_f64(one), o.bf16_bits_to_f64(two)) / page_vs - 1) < 0.05


def test_two_roundings_miss_rate_matches_page(accuracy_set):
    _, _, _, one, two = accuracy_set
    page = FACTS["correctly_rounded_misses_two_roundings"]["value"]
    assert abs(np.mean(one != two) - page) < 0.03


def test_two_round_with_one_shard_is_one_rounding():
    x = g.hidden(3, bank=2)
    w = g.latent_weight(0)
    assert np.array_equal(o.two_round_latent_ref(x, w, shards=1), o.latent_ref(x, w))


def test_cancelling_partials_single_rounding_holds():
    x, w = g.cancel_set(64)
    e = o.latent_exact(x, w)
    terms = o.latent_abs_terms(x, w)
    assert 5e-4 < np.median(np.abs(e) / terms) < 2e-3
    one = c.rel_rms(o.bf16_bits_to_f64(o.latent_ref(x, w)), e)
    two = c.rel_rms(o.bf16_bits_to_f64(o.two_round_latent_ref(x, w)), e)
    assert one <= 2.0e-3
    # the page reports 0.025x on its real cancelling data; the ratio depends on
    # how deep the cancellation is, so the pin is the inequality one <= 0.1 two
    assert one <= 0.1 * two


# -------------------------------------------------------------- logits --

@pytest.mark.parametrize("k", [3, 33, 96])
def test_logits_bruteforce_rational(k):
    r = np.random.default_rng(100 + k)
    x = to_bits(r.standard_normal((2, k)))
    wr = (r.standard_normal((k, 7)) * np.exp2(r.integers(-10, 3, (k, 7)))).astype(np.float32)
    got = o.logits_ref(x, wr)
    xf = o.bf16_bits_to_f64(x)
    for i in range(2):
        for e in range(7):
            exact = sum(Fraction(float(xf[i, j])) * Fraction(float(wr[j, e])) for j in range(k))
            assert got[i, e] == rne_f32_reference(exact), (i, e)


def test_logits_k_permutation_invariant():
    x = g.hidden(3, bank=4)
    wr = g.router_weight(0)
    p = np.random.default_rng(5).permutation(g.HIDDEN)
    assert np.array_equal(o.logits_ref(x, wr), o.logits_ref(x[:, p], wr[p]))


def test_logits_one_hot_pins_orientation():
    wr = g.router_weight(0)
    x = np.zeros((2, g.HIDDEN), dtype=np.uint16)
    x[0, 5] = 0x3F80
    x[1, 7000] = 0xBF80      # -1
    got = o.logits_ref(x, wr)
    assert np.array_equal(got[0], wr[5]) and np.array_equal(got[1], -wr[7000])


# -------------------------------------------------------------- top-16 --

def _brute_top16(row):
    def key(i):
        v = float(row[i])
        if math.isnan(v):
            return (1, 0.0, i)
        return (0, -v, i)
    return sorted(range(len(row)), key=key)[:16]


def test_top16_bruteforce_dense_ties():
    r = np.random.default_rng(21)
    pool = np.array([-1.0, -0.0, 0.0, 1.0, 2.0, np.inf, -np.inf, np.nan], dtype=np.float32)
    rows = []
    for probs in ([.2, .2, .2, .2, .1, .0, .05, .05], [.05, .3, .3, .3, .05, 0, 0, 0],
                  [.1, .1, .1, .1, .1, .2, .1, .2], [0, 0, 0, 0, 0, 0, .01, .99]):
        for _ in range(10):
            rows.append(r.choice(pool, size=g.EXPERTS, p=probs))
    L = np.array(rows, dtype=np.float32)
    got = o.topk16_ref(L)
    for i in range(L.shape[0]):
        assert got[i].tolist() == _brute_top16(L[i]), i


def test_top16_bruteforce_random_rows():
    L = np.random.default_rng(22).standard_normal((50, g.EXPERTS)).astype(np.float32)
    got = o.topk16_ref(L)
    for i in range(L.shape[0]):
        assert got[i].tolist() == _brute_top16(L[i])


def test_top16_all_equal_row():
    L = np.full((3, g.EXPERTS), 0.7, dtype=np.float32)
    ids = o.topk16_ref(L)
    assert (ids == np.arange(16)).all()
    w = o.route_weights_ref(L, ids)
    assert (w == np.float32(0.0625)).all()


def test_top16_relabel_experts():
    L = np.random.default_rng(23).standard_normal((40, g.EXPERTS)).astype(np.float32)
    p = np.random.default_rng(24).permutation(g.EXPERTS)
    ids = o.topk16_ref(L)
    ids2 = o.topk16_ref(L[:, p])
    assert np.array_equal(p[ids2], ids)


SHARD_COUNTS = (1, 2, 4, 7, 8, 14, 16, 28, 32, 56)


def _clustered_rows(n, seed):
    """Rows whose largest logits crowd into few expert shards."""
    r = np.random.default_rng(seed)
    L = r.standard_normal((n, g.EXPERTS)).astype(np.float32)
    for i in range(n):
        s = r.integers(0, 16)
        L[i, 56 * s:56 * s + 40] += 6.0
    return L


def test_top16_sharded_matches_sorted_on_dense_ties():
    # tiny value pools (many exact ties, specials) against Python sorted()
    r = np.random.default_rng(25)
    pool = np.array([-1.0, -0.0, 0.0, 1.0, 2.0, np.inf, -np.inf, np.nan], dtype=np.float32)
    L = np.array([r.choice(pool, size=g.EXPERTS, p=[.2, .2, .2, .2, .1, .0, .05, .05])
                  for _ in range(12)], dtype=np.float32)
    for shards in SHARD_COUNTS:
        got = o.topk16_sharded_ref(L, shards)
        for i in range(L.shape[0]):
            assert got[i].tolist() == _brute_top16(L[i]), (shards, i)


def test_top16_sharded_equals_unsharded():
    # the merge is exact for every shard count, also when the largest logits
    # crowd into one shard
    L = np.concatenate([np.random.default_rng(26).standard_normal((200, g.EXPERTS)).astype(np.float32),
                        _clustered_rows(100, 27)])
    ref = o.topk16_ref(L)
    for shards in SHARD_COUNTS:
        assert np.array_equal(o.topk16_sharded_ref(L, shards), ref), shards


def test_top16_sharded_rejects_bad_shard_counts():
    L = np.zeros((1, g.EXPERTS), dtype=np.float32)
    for shards in (0, 3, 5, 64, 112, 896):
        with pytest.raises(ValueError):
            o.topk16_sharded_ref(L, shards)


def test_top16_near_tie_generator_structure():
    L = g.near_tie_logits(2000, chunk=0)
    ids = o.topk16_ref(L)
    for i in range(0, 2000, 97):
        assert ids[i].tolist() == _brute_top16(L[i])


# ------------------------------------------------------------- weights --

def _decimal_weights(logits):
    getcontext().prec = 60
    s = [Decimal(1) / (Decimal(1) + (-Decimal(float(v))).exp()) for v in logits]
    tot = sum(s)
    return [rne_f32_reference(Fraction(x / tot)) for x in s]


def test_weights_against_decimal_sigmoid():
    L = (np.random.default_rng(31).standard_normal((6, g.EXPERTS)) * 2).astype(np.float32)
    ids = o.topk16_ref(L)
    w = o.route_weights_ref(L, ids)
    for i in range(L.shape[0]):
        want = np.array(_decimal_weights(L[i, ids[i]]), dtype=np.float32)
        assert c.f32_ulp_distance(w[i], want).max() <= 1


def test_weights_closed_forms():
    L = np.zeros((1, g.EXPERTS), dtype=np.float32)
    w = o.route_weights_ref(L, o.topk16_ref(L))
    assert (w == np.float32(1 / 16)).all()
    # eight at a, eight at b: w_a = sigmoid(a) / (8 sigmoid(a) + 8 sigmoid(b))
    a, b = 1.5, -0.25
    L = np.full((1, g.EXPERTS), -9.0, dtype=np.float32)
    L[0, :8] = a
    L[0, 8:16] = b
    w = o.route_weights_ref(L, o.topk16_ref(L))
    sa, sb = 1 / (1 + math.exp(-a)), 1 / (1 + math.exp(-b))
    assert abs(w[0, 0] - sa / (8 * sa + 8 * sb)) < 1e-7
    assert abs(w[0, 15] - sb / (8 * sa + 8 * sb)) < 1e-7
    assert w[0, 0] > w[0, 15]


def test_weights_sum_to_one():
    L = (np.random.default_rng(32).standard_normal((500, g.EXPERTS)) * 3).astype(np.float32)
    w = o.route_weights_ref(L, o.topk16_ref(L))
    s = w.astype(np.float64).sum(axis=1)
    assert np.all(np.abs(s - 1.0) <= 16 * 2 ** -24)


# --------------------------------------------------------- comparators --

def test_comparator_ulp_helpers():
    a = np.float32(1.0)
    b = np.nextafter(np.nextafter(a, np.float32(2)), np.float32(2))
    assert c.f32_ulp_distance(a, b) == 2
    assert c.f32_ulp_distance(np.float32(0.0), np.float32(-0.0)) == 0
    assert c.bf16_ulp_distance(np.uint16(0x3F80), np.uint16(0x3F82)) == 2
    assert c.bf16_spacing(np.uint16(0x3F80)) == 2.0 ** -7
    assert c.bf16_spacing(np.uint16(0x0001)) == 2.0 ** -133


def test_f32_spacing_against_numpy():
    """The FP32 unit in the last place at a value (the logits band's
    half-ULP term) equals numpy's spacing above |v|, for normals of every
    exponent, powers of two, subnormals and zero, either sign."""
    r = np.random.default_rng(5)
    bits = r.integers(0, 0x7F800000, 4000, dtype=np.uint32)
    v = np.concatenate([bits.view(np.float32),
                        np.float32([0.0, 1.0, 2.0, 0.5, 3.0e38, np.finfo(np.float32).tiny,
                                    np.finfo(np.float32).smallest_subnormal])])
    v = np.concatenate([v, -v])
    ref = np.abs(np.spacing(np.abs(v))).astype(np.float64)
    assert np.array_equal(c.f32_spacing(v), ref)


def test_weights_check_counts_ulps():
    """Weights exactly 5 FP32 ULP away pass, 6 away fail (the window of the
    weights criterion); signed zeros are equal; the counts and the largest
    distance are reported."""
    ref = np.float32([0.0625, 0.3, 1e-6, 0.0])
    got = ref.copy()
    for _ in range(5):
        got[0] = np.nextafter(got[0], np.float32(1))
        got[1] = np.nextafter(got[1], np.float32(-1))
    got[3] = np.float32(-0.0)
    r = c.weights_check(got, ref)
    assert r == {"n": 4, "max_ulp": 5, "fail": 0}
    got[2] = ref[2]
    for _ in range(6):
        got[2] = np.nextafter(got[2], np.float32(1))
    r = c.weights_check(got, ref)
    assert r["fail"] == 1 and r["max_ulp"] == 6
    assert c.weights_check(got, ref, max_ulp=6)["fail"] == 0


def test_latent_check_flags_a_wrong_value():
    x = g.hidden(2, bank=1)
    w = g.latent_weight(0)
    e = o.latent_exact(x, w)
    t = o.latent_abs_terms(x, w)
    ref = o.latent_ref(x, w)
    assert c.latent_check(ref, ref, e, t)["fail"] == 0
    bad = ref.copy()
    bad[0, 0] ^= np.uint16(0x0004)       # 4 units off
    assert c.latent_check(bad, ref, e, t)["fail"] == 1


def test_ids_check_rules():
    L = np.random.default_rng(41).standard_normal((2, g.EXPERTS)).astype(np.float32)
    ids = o.topk16_ref(L)
    assert c.ids_check(ids, ids, L)["violations"] == 0
    swapped = ids.copy()
    outside = [i for i in range(g.EXPERTS) if i not in set(ids[0].tolist())][0]
    swapped[0, 15] = outside
    assert c.ids_check(swapped, ids, L)["violations"] == 1


def test_route_ref_widened_matches_parts():
    x = g.hidden(3, bank=11)
    w, wr = g.latent_weight(0), g.router_weight(0)
    a = o.route_ref(x, w, wr)
    assert np.array_equal(a["latent"], o.latent_ref(x, w))
    assert np.array_equal(a["logits"], o.logits_ref(x, wr))
    assert np.array_equal(a["ids"], o.topk16_ref(o.logits_ref(x, wr)))


# ------------------------------------------- error scales and comparators --

@pytest.mark.parametrize("k", [3, 16, 64])
def test_abs_terms_against_rational_sums(k):
    """latent_abs_terms / logits_abs_terms are sum_k |x_k w_k| (not |sum_k x_k
    w_k|, not sum |x| * sum |w|): checked against exact rational sums, on rows
    built so that the signed sum cancels to exactly zero."""
    r = np.random.default_rng(100 + k)
    x = to_bits(r.standard_normal((3, k)) * np.exp2(r.integers(-4, 4, (3, k))))
    w = to_bits(r.standard_normal((k, 6)) * 0.05)
    wr = (r.standard_normal((k, 5)) * 0.05).astype(np.float32)
    # row 2: x = (a, a, ...) against a column whose two halves cancel
    half = k // 2
    x[2, :] = x[2, 0]
    w[half:2 * half, 5] = w[:half, 5] ^ np.uint16(0x8000)
    w[2 * half:, 5] = 0
    wr[half:2 * half, 4] = -wr[:half, 4]
    wr[2 * half:, 4] = 0
    xf, wf = o.bf16_bits_to_f64(x), o.bf16_bits_to_f64(w)
    lat, lgt = o.latent_abs_terms(x, w), o.logits_abs_terms(x, wr)
    for i in range(3):
        for n in range(6):
            want = sum(abs(Fraction(xf[i, j]) * Fraction(wf[j, n])) for j in range(k))
            assert abs(Fraction(lat[i, n]) - want) <= want * k * Fraction(2) ** -52
        for e in range(5):
            want = sum(abs(Fraction(xf[i, j]) * Fraction(float(wr[j, e]))) for j in range(k))
            assert abs(Fraction(lgt[i, e]) - want) <= want * k * Fraction(2) ** -52
    # the cancelling column: the signed dot is zero, the magnitudes are not
    assert o.latent_exact(x, w)[2, 5] == 0.0 and lat[2, 5] > 0.0
    assert o.logits_exact(x, wr)[2, 4] == 0.0 and lgt[2, 4] > 0.0


def _logits_case(err_units):
    """One logit whose float64 value is exact = 2^-10 (f32 unit 2^-33), with
    sum |terms| = 64 (so 2^-24 * 64 = 2^-18), and a returned value
    err_units * (ulp/2 + 2^-18) above it."""
    exact = np.array([2.0 ** -10])
    terms = np.array([64.0])
    ref = exact.astype(np.float32)
    bound = 0.5 * 2.0 ** -33 + 2.0 ** -18
    got = np.array([exact[0] + err_units * bound], dtype=np.float32)
    return got, ref, exact, terms


def test_logits_check_band_edges():
    # within 1 ULP: passes as within
    got, ref, exact, terms = _logits_case(0.0)
    near = np.nextafter(ref, np.float32(1))
    r = c.logits_check(near, ref, exact, terms)
    assert r["within_1ulp"] == 1 and r["fail"] == 0
    # far more than 1 ULP off but inside ulp/2 + 2^-24 sum|terms|: a band output
    got, ref, exact, terms = _logits_case(0.9)
    r = c.logits_check(got, ref, exact, terms)
    assert r["within_1ulp"] == 0 and r["band"] == 1 and r["fail"] == 0
    assert 0.85 <= r["max_err_over_terms"] <= 0.95
    # just outside the bound: fails (a unit of 2^-23 instead of 2^-24, or a
    # factor c of 2, would let it pass)
    got, ref, exact, terms = _logits_case(1.1)
    r = c.logits_check(got, ref, exact, terms)
    assert r["fail"] == 1 and r["band"] == 0
    # c scales the band: c = 2 admits the same value, c = 0.5 rejects 0.9
    assert c.logits_check(got, ref, exact, terms, c=2.0)["fail"] == 0
    got, ref, exact, terms = _logits_case(0.9)
    assert c.logits_check(got, ref, exact, terms, c=0.5)["fail"] == 1


def test_logits_check_without_terms_needs_half_ulp():
    # no terms (sum |terms| = 0): only ulp(got)/2 is allowed, and 2 ULPs fail
    exact = np.array([1.0 + 2.0 ** -24])     # halfway between 1 and 1 + 2^-23
    ref = np.array([1.0], dtype=np.float32)   # ties to even
    up = np.nextafter(np.float32(1.0), np.float32(2))
    assert c.logits_check(np.array([up]), ref, exact, np.zeros(1))["fail"] == 0
    up2 = np.nextafter(up, np.float32(2))
    up3 = np.nextafter(up2, np.float32(2))
    assert c.logits_check(np.array([up3]), ref, exact, np.zeros(1))["fail"] == 1


def test_latent_check_band_edges():
    # exact = 2^-6, BF16 unit there 2^-13; sum |terms| = 2^14 gives a band of
    # ulp/2 + 2^-10; 3 BF16 units off (3 * 2^-13 < 2^-10) is a band output,
    # 12 units off (12 * 2^-13 > 2^-14 + 2^-10) fails
    exact = np.array([2.0 ** -6])
    ref = o.round_f64_to_bf16_bits(exact)
    terms = np.array([2.0 ** 14])
    r = c.latent_check(ref + np.uint16(3), ref, exact, terms)
    assert r["band"] == 1 and r["fail"] == 0
    r = c.latent_check(ref + np.uint16(12), ref, exact, terms)
    assert r["fail"] == 1


def test_route_detail_equals_plain_parts():
    x = g.hidden(4, bank=12)
    w, wr = g.latent_weight(0), g.router_weight(0)
    d = o.route_detail_widened(x, *o.widen_weights(w, wr))
    ref = o.route_ref(x, w, wr)
    for key in ("latent", "logits", "ids", "weights"):
        assert np.array_equal(d[key], ref[key]), key
    assert np.array_equal(d["exact"], o.latent_exact(x, w))
    assert np.array_equal(d["abs_terms"], o.latent_abs_terms(x, w))
    assert np.array_equal(d["logits_exact"], o.logits_exact(x, wr))
    assert np.array_equal(d["logits_abs_terms"], o.logits_abs_terms(x, wr))


def test_gpu_tests_oracle_rows_equal_route_ref():
    """The helper every GPU parity test compares against (tests/routekit.py)
    returns the oracle's route."""
    from tests.routekit import oracle_rows
    w, wr = g.latent_weight(0), g.router_weight(0)
    for bank, rows in ((0, 1), (1, 8), (2, 20)):
        x = g.hidden(rows, bank=bank)
        got = oracle_rows(x)
        ref = o.route_ref(x, w, wr)
        for key in ("latent", "logits", "ids", "weights"):
            assert np.array_equal(got[key], ref[key]), (bank, key)
        assert np.array_equal(got["abs_terms"], o.latent_abs_terms(x, w))
        assert np.array_equal(got["logits_abs_terms"], o.logits_abs_terms(x, wr))


def test_logits_check_large_logit_statistics():
    # |exact| >= 1 only: 2.0 (got 3 ULP above) and -1.5 (exact); 0.25 is left out
    exact = np.array([2.0, -1.5, 0.25])
    ref = exact.astype(np.float32)
    got = ref.copy()
    for _ in range(3):
        got[0] = np.nextafter(got[0], np.float32(3))
    got[2] = np.nextafter(got[2], np.float32(1))
    r = c.logits_check(got, ref, exact, np.full(3, 1e6))
    assert r["large_n"] == 2 and r["large_max_ulp"] == 3 and r["large_mean_ulp"] == 1.5

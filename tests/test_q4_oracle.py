"""Pins of the oracle's q4_0 cache, CPU only.

The pages name q4_0 beside q8_0 among the KV cache types whose decode was not yet exercised
(1bit-MONSTER/engine issue #115, comment "Closing the remaining half of this issue") and do not
define it; the oracle reads it as the published ggml q4_0 block: 32 elements, one f16 scale d,
4-bit codes c with value (c - 8) * d, byte i of the block's 16 code bytes holding element i in
its low nibble and element i + 16 in its high nibble; and quantizes by ggml's rule (m the
element of largest magnitude, first on a tie; d = m / -8; c = min(15, trunc(x / d + 8.5)) in
f32, the scale stored as f16(d)).

Each pin ties the oracle to something other than itself: blocks whose values the definition
fixes in closed form, torch's fp64 SDPA over the dense values a paged q4_0 cache was packed
from (packing written on the test side), the rule's exact round trip for groups on its grid, its
error bound, its tie and first-maximum decisions on hand-computed groups, and the decode of what
the append wrote. Mutants with a planted mistake must fail a pin.
"""
import os
import tempfile

import numpy as np
import pytest

import oracle
from tests.paged import dense_reference, paged_from_dense, q4_pack, q4_values


def _q4_problem(rng, B, T, Hq, Hkv, D, P, lens, extra_heads=1):
    """A paged q4_0 problem from random codes and power-of-two-times-small-integer scales, with
    the dense fp64 values it holds."""
    Lmax = max(lens)
    ck = rng.integers(0, 16, (B, Lmax, Hkv, D))
    cv = rng.integers(0, 16, (B, Lmax, Hkv, D))
    ks = (rng.integers(1, 64, (B, Lmax, Hkv, D // 32)) * 2.0 ** -9).astype(np.float16)
    vs = (rng.integers(1, 64, (B, Lmax, Hkv, D // 32)) * 2.0 ** -9).astype(np.float16)
    ks[rng.random(ks.shape) < 0.1] *= -1  # negative scales occur (d = m / -8 for m > 0)
    xk = (ck - 8) * np.repeat(ks.astype(np.float64), 32, axis=-1)
    xv = (cv - 8) * np.repeat(vs.astype(np.float64), 32, axis=-1)
    q = rng.standard_normal((B * T, Hq, D), dtype=np.float32).astype(np.float16)
    prob = paged_from_dense(rng, q, q4_pack(ck), q4_pack(cv), lens, P, T=T, q4=True,
                            extra_heads=extra_heads, Ks=ks, Vs=vs)
    return prob, (q, xk, xv)


def check_block_closed_form(lib):
    """One position, one KV head, q = one-hot e_d: lse = sm_scale * K[d], so every element's
    value is read back through the decode. Bytes i | (15 - i) << 4 with d = 0.5 give element i
    the value (i - 8) / 2 and element i + 16 the value (7 - i) / 2; a second group with d = -2
    and all bytes 0x80 gives elements 0..15 the value 16 and 16..31 the value 0."""
    D = 64
    g0 = np.array([i | ((15 - i) << 4) for i in range(16)], np.uint8)
    g1 = np.full(16, 0x80, np.uint8)
    k = np.concatenate([g0, g1]).reshape(1, 1, 1, 32)
    s = np.array([0.5, -2.0], np.float16).reshape(1, 1, 1, 2)
    want = np.concatenate([(np.arange(16) - 8) / 2, (7 - np.arange(16)) / 2,
                           np.full(16, 16.0), np.zeros(16)])
    q = np.zeros((1, D, D), np.float16)
    q[0, np.arange(D), np.arange(D)] = 1.0
    prob = dict(q=q, k_pages=k, v_pages=k.copy(), k_scales=s, v_scales=s.copy(),
                page_table=np.zeros((1, 1), np.int32), kv_len=np.array([1], np.int32),
                q_per_seq=1, sm_scale=1.0)
    o, lse = oracle.decode(prob, lib=lib)
    # a single position: o is that position's V row for every query head
    return bool(np.array_equal(lse, want) and np.array_equal(o[0], want))


def check_sdpa_q4(lib, seed=2):
    rng = np.random.default_rng(seed)
    ok = True
    for (B, T, Hq, Hkv, D, P, lens) in ((2, 1, 8, 2, 64, 4, (37, 90)),
                                        (2, 3, 4, 4, 128, 16, (3, 70)),
                                        (1, 2, 4, 1, 256, 8, (41,))):
        prob, (q, xk, xv) = _q4_problem(rng, B, T, Hq, Hkv, D, P, lens)
        o, lse = oracle.decode(prob, lib=lib)
        ro, rl = dense_reference(q, xk, xv, np.asarray(lens), T, prob["sm_scale"])
        ok &= np.abs(o - ro.reshape(o.shape)).max() <= 1e-12
        ok &= np.abs(lse - rl.reshape(lse.shape)).max() <= 1e-12
    return bool(ok)


def check_gather_q4(lib, seed=3):
    """The gather returns each visible row's code bytes and scales as packed."""
    rng = np.random.default_rng(seed)
    prob, (q, xk, xv) = _q4_problem(rng, 2, 1, 4, 2, 128, 16, (20, 33))
    dk, dv, dks, dvs = oracle.gather(prob, 40, lib=lib)
    ok = dk.shape == (2, 40, 2, 64) and dks.shape == (2, 40, 2, 4)
    for b, n in enumerate((20, 33)):
        ok &= np.array_equal(q4_values(dk[b, :n], dks[b, :n]), xk[b, :n])
        ok &= np.array_equal(q4_values(dv[b, :n], dvs[b, :n]), xv[b, :n])
    return bool(ok)


def _quant(lib, x):
    c, s = oracle.quantize_q4_group(np.asarray(x, np.float16), lib=lib)
    return np.concatenate([c & 15, c >> 4]).astype(int), s


def check_exact_groups(lib, seed=4):
    """Groups on the rule's grid: x = k * d with integers k in [-8, 7] and k = -8 at the largest
    magnitude (d of either sign, f16-exact). The rule returns d and codes k + 8 exactly."""
    rng = np.random.default_rng(seed)
    ok = True
    for _ in range(300):
        d = float(rng.integers(1, 128)) * 2.0 ** int(rng.integers(-16, -4))
        d = float(np.float16(d)) * (1 if rng.random() < 0.5 else -1)
        k = rng.integers(-7, 8, 32)
        k[rng.integers(0, 32)] = -8
        x = (k * d).astype(np.float16)
        assert np.array_equal(x.astype(np.float64), k * d)  # on the f16 grid
        c, s = _quant(lib, x)
        ok &= float(s) == d and np.array_equal(c, k + 8)
    return bool(ok)


def check_error_bound(lib, seed=5):
    """For N(0,1) groups: the extreme element gets code 0, the stored scale is f16(m / -8), and
    every element is within |d| / 2 of its value (|d| where the code is clipped at 15), up to
    the f16 rounding of the scale."""
    rng = np.random.default_rng(seed)
    ok = True
    for _ in range(400):
        x = (rng.standard_normal(32) * rng.uniform(0.01, 100)).astype(np.float16)
        xf = x.astype(np.float64)
        c, s = _quant(lib, x)
        i = int(np.argmax(np.abs(xf)))             # first index of the largest magnitude
        d = xf[i] / -8
        ok &= c[i] == 0 and float(s) == float(np.float16(d))
        val = (c - 8) * float(s)
        slack = 8 * abs(float(s) - d) + 1e-12
        bound = np.where(c == 15, abs(d), abs(d) / 2) + slack
        ok &= bool((np.abs(xf - val) <= bound).all())
    return bool(ok)


def check_ties_and_first_max(lib):
    """Hand-computed groups. m = 8 (d = -1, 1/d = -1): x / d + 8.5 = 8.5 - x, truncated, so
    x = 1.5 -> 7 and x = 2.5 -> 6, x = -0.5 -> 9, x = -1.5 -> 10, x = 0.5 -> 8, x = -7.5 -> 15
    (16 clipped); the half-way points round up, not to even. A tie of magnitudes takes the first
    element: +3 at index 2 before -3 at index 5 gives d = -0.375, codes 0 and 15. An all-zero
    group stores d = -0 (0 / -8) and codes 8."""
    x = np.zeros(32, np.float16)
    x[:7] = [8, 1.5, 2.5, -0.5, -1.5, 0.5, -7.5]
    c, s = _quant(lib, x)
    ok = float(s) == -1.0 and list(c[:7]) == [0, 7, 6, 9, 10, 8, 15] and (c[7:] == 8).all()
    y = np.zeros(32, np.float16)
    y[2], y[5] = 3, -3
    c, s = _quant(lib, y)
    ok &= float(s) == -0.375 and c[2] == 0 and c[5] == 15 and (np.delete(c, [2, 5]) == 8).all()
    c, s = _quant(lib, np.zeros(32, np.float16))
    ok &= np.float16(s).view(np.uint16) == 0x8000 and (c == 8).all()
    return bool(ok)


def check_append_decodes(lib, seed=6, P=4):
    """Append f16 rows into a q4_0 cache, then decode: the result equals SDPA over the values
    the rule gives (rebuilt on the test side from the written bytes and scales, which must
    match a per-group quantization), and untouched slots keep their bytes."""
    rng = np.random.default_rng(seed)
    B, Hkv, D, L = 2, 2, 64, (9, 14)
    prob, _ = _q4_problem(rng, B, 1, 4, Hkv, D, P, L, extra_heads=0)
    N = sum(L)
    xk = (rng.standard_normal((N, Hkv, D)) * 3).astype(np.float16)
    xv = (rng.standard_normal((N, Hkv, D)) * 3).astype(np.float16)
    bi = np.concatenate([np.full(n, b) for b, n in enumerate(L)]).astype(np.int32)
    pos = np.concatenate([np.arange(n) for n in L]).astype(np.int32)
    order = rng.permutation(N)
    k, v, ks, vs, skipped = oracle.append(xk[order], xv[order], bi[order], pos[order],
                                          prob["page_table"], max(L), prob["k_pages"],
                                          prob["v_pages"], prob["k_scales"], prob["v_scales"],
                                          lib=lib)
    ok = skipped == 0
    tab = prob["page_table"]
    touched = np.zeros(k.shape[:2], bool)
    Kd = np.zeros((B, max(L), Hkv, D))
    Vd = np.zeros_like(Kd)
    for i in range(N):
        b, j = bi[i], pos[i]
        pg, sl = tab[b, j // P], j % P
        touched[pg, sl] = True
        for h in range(Hkv):
            for grp in range(D // 32):
                ck, sk = oracle.quantize_q4_group(xk[i, h, 32 * grp:32 * grp + 32], lib=lib)
                ok &= np.array_equal(k[pg, sl, h, 16 * grp:16 * grp + 16], ck)
                ok &= np.float16(ks[pg, sl, h, grp]).view(np.uint16) == np.float16(sk).view(
                    np.uint16)
        Kd[b, j] = q4_values(k[pg, sl], ks[pg, sl])
        Vd[b, j] = q4_values(v[pg, sl], vs[pg, sl])
        # the written values are the inputs to within the rule's bound
        ok &= bool((np.abs(Kd[b, j] - xk[i].astype(np.float64)) <=
                    np.repeat(np.abs(ks[pg, sl].astype(np.float64)), 32, -1) * 1.01).all())
    ok &= np.array_equal(k[~touched], prob["k_pages"][~touched])
    new = dict(prob, k_pages=k, v_pages=v, k_scales=ks, v_scales=vs)
    o, lse = oracle.decode(new, lib=lib)
    ro, rl = dense_reference(prob["q"], Kd, Vd, np.asarray(L), 1, prob["sm_scale"])
    ok &= np.abs(o - ro.reshape(o.shape)).max() <= 1e-12
    ok &= np.abs(lse - rl.reshape(lse.shape)).max() <= 1e-12
    return bool(ok)


def check_non_finite(lib):
    """NaN elements take no part in the maximum and store code 8; an infinite element makes the
    scale infinite and every code 8."""
    x = (np.arange(32) - 10).astype(np.float16)
    x[3] = np.nan
    c, s = _quant(lib, x)
    x2 = x.copy()
    x2[3] = 0
    c2, s2 = _quant(lib, x2)
    ok = c[3] == 8 and float(s) == float(s2) and np.array_equal(np.delete(c, 3), np.delete(c2, 3))
    y = np.ones(32, np.float16)
    y[7] = np.inf
    c, s = _quant(lib, y)
    ok &= np.isinf(s) and float(s) < 0 and (c == 8).all()
    y[7] = -np.inf
    c, s = _quant(lib, y)
    ok &= np.isinf(s) and float(s) > 0 and (c == 8).all()
    return bool(ok)


ALL_PINS = [
    ("block_closed_form", check_block_closed_form),
    ("sdpa_q4", check_sdpa_q4),
    ("gather_q4", check_gather_q4),
    ("exact_groups", check_exact_groups),
    ("error_bound", check_error_bound),
    ("ties_and_first_max", check_ties_and_first_max),
    ("append_decodes", check_append_decodes),
    ("non_finite", check_non_finite),
]


@pytest.mark.parametrize("name,fn", ALL_PINS, ids=[n for n, _ in ALL_PINS])
def test_q4_pin(name, fn):
    assert fn(oracle.load())


MUTANTS = {20: "nibble order swapped on read", 21: "code offset 7 instead of 8",
           22: "last element of largest magnitude wins a tie",
           23: "scale from the magnitude, not the signed extreme",
           24: "nearest-even rounding instead of the +8.5 truncation"}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=[MUTANTS[m] for m in sorted(MUTANTS)])
def test_q4_pins_catch_planted_mistake(mutant):
    with tempfile.TemporaryDirectory() as d:
        lib = oracle.load(oracle.build(os.path.join(d, f"liboracle_m{mutant}.so"), mutant=mutant))
        failed = [n for n, fn in ALL_PINS if not fn(lib)]
        assert failed, f"no pin catches mutant {mutant} ({MUTANTS[mutant]})"


def test_q4_generator_recipe():
    """The q4_0 inputs follow their recipe: live scales finite and f16(max|x| / 8) of N(0,1)-sized
    groups, unread slots NaN-poisoned, dequantized values N(0,1) draws to within the rounding."""
    import workloads
    s = workloads.spec(name="q4_recipe", batch=3, q_per_seq=1, num_qo_heads=8, num_kv_heads=2,
                       head_dim=128, page_size=16, kv_dtype="q4", lens=("list", (5, 300, 64)))
    prob = workloads.generate(s, 9)
    k, ks, table, L, P = prob["k_pages"], prob["k_scales"], prob["page_table"], prob["kv_len"], 16
    assert k.dtype == np.uint8 and k.shape[3] == 64 and ks.shape[3] == 4
    live = np.zeros(k.shape[:2], bool)
    for b in range(3):
        for j in range(int(L[b])):
            live[table[b, j // P], j % P] = True
    assert np.isfinite(ks[live]).all() and np.isnan(ks[~live]).all()
    x = q4_values(k[live], ks[live])
    assert abs(x.mean()) < 0.05 and 0.9 < x.std() < 1.1

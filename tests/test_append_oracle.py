"""Pins of the oracle's append (writing new tokens into the paged cache, int8 quantize-on-write)
against what the mathematics and the format fix (CPU only).

Each pin ties the oracle's append to something other than itself: numpy's f32 -> f16
conversion (a library routine), closed forms of the int8 rule (exactly representable groups
come back exactly, every element within half a scale step, ties to even, an all-zero group),
and round trips through the already-pinned decode and gather: a dense cache appended position
by position into permuted pages must decode like torch's fp64 SDPA on the dense cache, and
positions that were not appended must keep their bytes. The last test builds mutants of the
oracle with one planted mistake in the append each and checks that some pin fails for every
one of them.
"""
import math
import os
import tempfile

import numpy as np
import pytest

import oracle
from tests.paged import dense_reference

# --------------------------------------------------------------------------- helpers


def empty_paged(rng, B, L, Hkv, D, P, int8, spare=3, extra_heads=0):
    """NaN-poisoned pools (int8: codes 0x55, NaN scales) with a random page table covering
    positions < L[b]; entries past them are -1. Returns (k, v, ks, vs, table)."""
    L = np.asarray(L, np.int64)
    npages = (L + P - 1) // P
    N = int(npages.sum()) + spare
    perm = rng.permutation(N)
    Hs = Hkv + extra_heads
    if int8:
        k = np.full((N, P, Hs, D), 0x55, np.int8)[:, :, :Hkv]
        v = np.full((N, P, Hs, D), 0x55, np.int8)[:, :, :Hkv]
        ks = np.full((N, P, Hs, D // 32), np.nan, np.float16)[:, :, :Hkv]
        vs = np.full((N, P, Hs, D // 32), np.nan, np.float16)[:, :, :Hkv]
    else:
        k = np.full((N, P, Hs, D), np.nan, np.float16)[:, :, :Hkv]
        v = np.full((N, P, Hs, D), np.nan, np.float16)[:, :, :Hkv]
        ks = vs = None
    table = np.full((B, int(npages.max()) + 1), -1, np.int32)
    off = 0
    for b in range(B):
        table[b, :npages[b]] = perm[off:off + npages[b]]
        off += int(npages[b])
    return k, v, ks, vs, table


def exact_groups(rng, shape):
    """f16 data whose every 32-element group is c * 2^e with integer c in [-127, 127], the
    group's largest |c| = 127 and e per group in [-10, 0]: the int8 rule must return s = 2^e
    and the codes c exactly."""
    c = rng.integers(-127, 128, size=shape[:-1] + (shape[-1] // 32, 32))
    pick = rng.integers(0, 32, size=c.shape[:-1])
    np.put_along_axis(c, pick[..., None], np.where(rng.random(pick.shape) < 0.5, 127, -127)[..., None],
                      axis=-1)
    e = rng.integers(-10, 1, size=c.shape[:-1])
    x = c * np.exp2(e)[..., None]
    return x.reshape(shape).astype(np.float16), c.reshape(shape).astype(np.int8), \
        np.exp2(e).astype(np.float16)


def append_all(rng, lib, B, L, Hkv, D, P, int8, x_k, x_v, order=None, extra_heads=0, q_T=1):
    """Append every position j < L[b] of dense [B, Lmax, Hkv, D] f16 rows (tokens in a random
    order) into empty permuted pools; returns the decode problem dict over the written pools."""
    k, v, ks, vs, table = empty_paged(rng, B, L, Hkv, D, P, int8, extra_heads=extra_heads)
    bi = np.concatenate([np.full(int(L[b]), b) for b in range(B)]).astype(np.int32)
    pos = np.concatenate([np.arange(int(L[b])) for b in range(B)]).astype(np.int32)
    perm = rng.permutation(bi.shape[0]) if order is None else order
    bi, pos = bi[perm], pos[perm]
    kn = np.ascontiguousarray(x_k[bi, pos])
    vn = np.ascontiguousarray(x_v[bi, pos])
    k2, v2, ks2, vs2, skipped = oracle.append(kn, vn, bi, pos, table, int(max(L)), k, v, ks, vs,
                                              lib=lib)
    assert skipped == 0
    q = rng.standard_normal((B * q_T, 2 * Hkv, D), dtype=np.float32).astype(np.float16)
    return dict(q=q, k_pages=k2, v_pages=v2, k_scales=ks2, v_scales=vs2, page_table=table,
                kv_len=np.asarray(L, np.int32), q_per_seq=q_T,
                sm_scale=float(np.float32(1 / math.sqrt(D))))


# --------------------------------------------------------------------------- pins


def check_half_conversion(lib, seed=1):
    """f32 -> f16 (nearest even) equals numpy's astype on every f16 value, on every midpoint
    between neighbouring f16 values (ties), just off the midpoints, across the subnormal range,
    at overflow, and on random f32 bit patterns."""
    rng = np.random.default_rng(seed)
    h = np.arange(0, 0x7c00, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    mids = (h[:-1] + h[1:]) / 2  # exact in f32 (12 significant bits at most)
    vals = [h, mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
            np.nextafter(mids.astype(np.float32), np.float32(0)),
            np.array([65504.0, 65519.0, 65520.0, 1e6, 2.0 ** -25, 2.0 ** -26, 3 * 2.0 ** -26]),
            rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32).view(np.float32)]
    x = np.concatenate([np.asarray(v, np.float32).ravel() for v in vals])
    x = x[np.isfinite(x)]
    x = np.concatenate([x, -x[::7]])
    with np.errstate(over="ignore"):  # values past f16's range convert to infinity
        ref = x.astype(np.float16).view(np.uint16)
    mine = np.array([lib.oracle_float_to_half(float(v)) for v in x], np.uint16)
    return np.array_equal(mine, ref)


def _quant(lib, g):
    return oracle.quantize_group(g, lib=lib)


def check_exact_groups(lib, seed=2):
    """Groups c * 2^e (largest |c| = 127) come back as scale 2^e and codes c, exactly."""
    rng = np.random.default_rng(seed)
    x, c, s = exact_groups(rng, (300, 32))
    for i in range(x.shape[0]):
        codes, sc = _quant(lib, x[i])
        if not (np.array_equal(codes, c[i]) and sc == s[i, 0]):
            return False
    return True


def check_half_step_bound(lib, seed=3):
    """Every element lies within half a scale step of code * scale (up to the f32 quotient's
    rounding, < 1e-5 of a step), codes stay in [-127, 127], and the largest-magnitude element
    gets a code of magnitude 127."""
    rng = np.random.default_rng(seed)
    for i in range(400):
        mag = 10.0 ** rng.uniform(-3, 3)
        g = (mag * rng.standard_normal(32)).astype(np.float16)
        codes, sc = _quant(lib, g)
        s = float(sc)
        xf = g.astype(np.float64)
        if s <= 0 or np.abs(codes.astype(np.int64)).max() > 127:
            return False
        if np.abs(xf - codes * s).max() > s * (0.5 + 1e-5):
            return False
        if abs(int(codes[np.argmax(np.abs(xf))])) != 127:
            return False
        # the scale is the f16 nearest to the f32 quotient max|x| / 127
        if sc != np.float16(np.float32(np.abs(g).max()) / np.float32(127)):
            return False
    return True


def check_ties_and_zero(lib):
    """x / s exactly halfway between integers rounds to the even integer; an all-zero group,
    and a group below f16's scale range, get scale 0 and codes 0."""
    g = np.zeros(32, np.float16)
    g[0] = 127.0  # s = 1 exactly
    halves = [0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, -3.5, 100.5, -126.5, 126.5]
    g[1:1 + len(halves)] = halves
    codes, sc = _quant(lib, g)
    want = [127, 0, 2, 2, 4, 0, -2, -2, -4, 100, -126, 126]
    if sc != 1.0 or list(codes[:len(want)]) != want:
        return False
    codes, sc = _quant(lib, np.zeros(32, np.float16))
    if sc.view(np.uint16) != 0 or codes.any():
        return False
    tiny = np.zeros(32, np.float16)
    tiny[5] = np.float16(2.0 ** -24)  # max/127 rounds to f16 zero
    codes, sc = _quant(lib, tiny)
    return sc == 0 and not codes.any()


def check_append_decodes_f16(lib, seed=4, P=4, extra_heads=1):
    """A dense f16 cache appended token by token (random order) into empty permuted pages
    decodes like torch's fp64 SDPA on the dense cache."""
    rng = np.random.default_rng(seed)
    B, Hkv, D, L = 2, 2, 64, (37, 90)
    K = rng.standard_normal((B, max(L), Hkv, D), dtype=np.float32).astype(np.float16)
    V = rng.standard_normal((B, max(L), Hkv, D), dtype=np.float32).astype(np.float16)
    prob = append_all(rng, lib, B, L, Hkv, D, P, False, K, V, extra_heads=extra_heads)
    o, lse = oracle.decode(prob)
    ro, rl = dense_reference(prob["q"], K, V, np.asarray(L), 1, prob["sm_scale"])
    return (np.abs(o - ro.reshape(o.shape)).max() <= 1e-12
            and np.abs(lse - rl.reshape(lse.shape)).max() <= 1e-12)


def check_append_decodes_int8(lib, seed=5, P=4):
    """Exactly representable groups appended into an int8 cache decode like torch's fp64 SDPA
    on the f16 values (the quantization is exact there, so any misplaced code or scale shows)."""
    rng = np.random.default_rng(seed)
    B, Hkv, D, L = 2, 2, 64, (29, 70)
    K, _, _ = exact_groups(rng, (B, max(L), Hkv, D))
    V, _, _ = exact_groups(rng, (B, max(L), Hkv, D))
    prob = append_all(rng, lib, B, L, Hkv, D, P, True, K, V, extra_heads=1)
    o, lse = oracle.decode(prob)
    ro, rl = dense_reference(prob["q"], K, V, np.asarray(L), 1, prob["sm_scale"])
    return (np.abs(o - ro.reshape(o.shape)).max() <= 1e-12
            and np.abs(lse - rl.reshape(lse.shape)).max() <= 1e-12)


def check_untouched(lib, seed=6, int8=False):
    """Appending half the positions leaves every other position's bytes (read back by the
    pinned gather) as they were, and writes the appended ones verbatim (f16) or as the group
    rule gives them (int8)."""
    rng = np.random.default_rng(seed)
    B, Hkv, D, P, L = 2, 2, 64, 4, (30, 45)
    k, v, ks, vs, table = empty_paged(rng, B, L, Hkv, D, P, int8)
    X = rng.standard_normal((B, max(L), Hkv, D), dtype=np.float32).astype(np.float16)
    bi = np.concatenate([np.full(int(L[b]), b) for b in range(B)]).astype(np.int32)
    pos = np.concatenate([np.arange(int(L[b])) for b in range(B)]).astype(np.int32)
    pick = rng.random(bi.shape[0]) < 0.5
    k2, v2, ks2, vs2, skipped = oracle.append(X[bi[pick], pos[pick]], X[bi[pick], pos[pick]],
                                              bi[pick], pos[pick], table, max(L), k, v, ks, vs,
                                              lib=lib)
    prob0 = dict(q=np.zeros((B, 2, D), np.float16), k_pages=k, v_pages=v, k_scales=ks,
                 v_scales=vs, page_table=table, kv_len=np.asarray(L, np.int32), q_per_seq=1,
                 sm_scale=1.0)
    prob1 = dict(prob0, k_pages=k2, v_pages=v2, k_scales=ks2, v_scales=vs2)
    g0 = oracle.gather(prob0, max(L))
    g1 = oracle.gather(prob1, max(L))
    for b, j, w in zip(bi, pos, pick):
        if not w:
            for a0, a1 in zip(g0, g1):
                if a0 is not None and not np.array_equal(a0[b, j].view(np.uint8),
                                                         a1[b, j].view(np.uint8)):
                    return False
        elif not int8:
            if not (np.array_equal(g1[0][b, j].view(np.uint16), X[b, j].view(np.uint16))
                    and np.array_equal(g1[1][b, j].view(np.uint16), X[b, j].view(np.uint16))):
                return False
        else:
            for h in range(Hkv):
                for grp in range(D // 32):
                    c, sc = _quant(lib, X[b, j, h, 32 * grp:32 * grp + 32])
                    for dk, ds in ((g1[0], g1[2]), (g1[1], g1[3])):
                        if not (np.array_equal(dk[b, j, h, 32 * grp:32 * grp + 32], c)
                                and ds[b, j, h, grp].view(np.uint16) == sc.view(np.uint16)):
                            return False
    return skipped == 0


def check_skips(lib, seed=7, int8=True):
    """Tokens with a sequence index outside [0, batch), a position outside [0, max_len), or a
    page id outside the pool are skipped: nothing in the pools changes."""
    rng = np.random.default_rng(seed)
    B, Hkv, D, P, L = 2, 2, 64, 4, (8, 12)
    k, v, ks, vs, table = empty_paged(rng, B, L, Hkv, D, P, int8)
    table = table.copy()
    table[1, 0] = k.shape[0]      # one past the pool
    table[1, 1] = -5
    bi = np.array([-1, 2, 0, 0, 1, 1, 7], np.int32)
    pos = np.array([0, 0, -1, 12, 1, 5, 3], np.int32)
    X = rng.standard_normal((bi.shape[0], Hkv, D), dtype=np.float32).astype(np.float16)
    k2, v2, ks2, vs2, skipped = oracle.append(X, X, bi, pos, table, 12, k, v, ks, vs, lib=lib)
    same = all(np.array_equal(a.view(np.uint8), b_.view(np.uint8))
               for a, b_ in ((k, k2), (v, v2)) + (((ks, ks2), (vs, vs2)) if int8 else ()))
    return same and skipped == 5


def check_non_finite(lib, seed=12):
    """Non-finite inputs follow the formulas: f16 infinity converts like numpy's; a NaN element
    is left out of the group maximum (the scale and the other codes are those of the group
    without it) and stores code 0; an infinite element gives the scale f16(inf) and all codes
    0."""
    ok = lib.oracle_float_to_half(float("inf")) == np.float16(np.inf).view(np.uint16)
    ok &= lib.oracle_float_to_half(float("-inf")) == np.float16(-np.inf).view(np.uint16)
    rng = np.random.default_rng(seed)
    x, c, sc = exact_groups(rng, (40, 32))
    for i in range(x.shape[0]):
        g = x[i].astype(np.float16)
        j = int(rng.integers(32))
        if int(np.abs(c[i, j])) == 127:
            continue  # the maximum itself: removing it changes the scale
        gn = g.copy()
        gn[j] = np.float16(np.nan)
        codes, s = _quant(lib, gn)
        ref_codes, ref_s = _quant(lib, g)
        ok &= codes[j] == 0 and s.view(np.uint16) == ref_s.view(np.uint16)
        ok &= np.array_equal(np.delete(codes, j), np.delete(ref_codes, j))
        gi = g.copy()
        gi[j] = np.float16(np.inf if i % 2 else -np.inf)
        codes, s = _quant(lib, gi)
        ok &= bool(np.isinf(s)) and not codes.any()
    return bool(ok)


ALL_PINS = [
    ("non_finite", check_non_finite),
    ("half_conversion", check_half_conversion),
    ("exact_groups", check_exact_groups),
    ("half_step_bound", check_half_step_bound),
    ("ties_and_zero", check_ties_and_zero),
    ("append_decodes_f16", check_append_decodes_f16),
    ("append_decodes_f16_P1", lambda lib: check_append_decodes_f16(lib, seed=8, P=1, extra_heads=0)),
    ("append_decodes_int8", check_append_decodes_int8),
    ("untouched_f16", check_untouched),
    ("untouched_int8", lambda lib: check_untouched(lib, seed=9, int8=True)),
    ("skips", check_skips),
    ("skips_f16", lambda lib: check_skips(lib, seed=10, int8=False)),
]


@pytest.mark.parametrize("name,fn", ALL_PINS, ids=[n for n, _ in ALL_PINS])
def test_append_pin(name, fn):
    assert fn(oracle.load())


MUTANTS = {11: "divisor 128", 12: "truncation instead of rounding", 13: "scale in the wrong slot",
           14: "row under the next KV head"}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=[MUTANTS[m] for m in sorted(MUTANTS)])
def test_append_pins_catch_planted_mistake(mutant):
    with tempfile.TemporaryDirectory() as d:
        path = oracle.build(os.path.join(d, f"liboracle_m{mutant}.so"), mutant=mutant)
        lib = oracle.load(path)
        failed = []
        for name, fn in ALL_PINS:
            try:
                if not fn(lib):
                    failed.append(name)
            except AssertionError:
                failed.append(name)
        assert failed, f"no pin catches mutant {mutant} ({MUTANTS[mutant]})"

"""Pins of the fp64 oracle against what the mathematics and the pages fix (CPU only).

Each pin ties the oracle to something other than itself: a library routine (numpy's f16
decode, torch's fp64 SDPA and logsumexp), a closed form (identical keys, one dominant key, a
single position), an invariant (split-form merge = one-pass softmax; causal row t = a T=1 call
on the shorter prefix; int8 with power-of-two scales = the equivalent f16 cache), or a round
trip (a dense cache scattered into permuted pages comes back exactly). The last test builds
mutants of the oracle with one planted mistake each and checks that some pin fails for every
one of them.
"""
import math
import os
import tempfile

import numpy as np
import pytest

import oracle
from tests.paged import dense_reference, paged_from_dense, random_dense, dequant

# --------------------------------------------------------------------------- helpers


def _problem(seed, B=2, T=1, Hq=4, Hkv=2, D=64, P=4, lens=(37, 90), int8=False, extra_heads=1,
             q_mult=1.0):
    rng = np.random.default_rng(seed)
    Lmax = max(lens)
    K, V, Ks, Vs = random_dense(rng, B, Lmax, Hkv, D, int8)
    q = (q_mult * rng.standard_normal((B * T, Hq, D), dtype=np.float32)).astype(np.float16)
    prob = paged_from_dense(rng, q, K, V, lens, P, T=T, extra_heads=extra_heads, Ks=Ks, Vs=Vs)
    return prob, (q, K, V, Ks, Vs)


CASES = [
    # (B, T, Hq, Hkv, D, P, lens, int8)
    (1, 1, 4, 4, 32, 1, (5,), False),
    (2, 1, 4, 2, 64, 2, (37, 90), False),
    (2, 1, 8, 2, 128, 16, (200, 17), False),
    (2, 4, 4, 2, 64, 4, (23, 64), False),
    (1, 2, 6, 3, 32, 16, (150,), False),
    (2, 1, 4, 2, 64, 4, (37, 90), True),
    (2, 4, 8, 2, 128, 16, (100, 33), True),
    (2, 37, 4, 2, 64, 16, (37, 120), False),   # many query tokens (the prefill route's reading)
    (1, 20, 8, 2, 64, 4, (90,), True),
    (2, 2, 8, 2, 192, 16, (70, 33), False),    # head_dim 192
    (2, 1, 4, 2, 512, 4, (41, 66), False),     # head_dim 512
    (2, 3, 4, 1, 512, 16, (80, 17), True),     # head_dim 512, int8 (16 scale groups per row)
]


def check_sdpa(lib, case, seed):
    B, T, Hq, Hkv, D, P, lens, int8 = case
    prob, (q, K, V, Ks, Vs) = _problem(seed, B, T, Hq, Hkv, D, P, lens, int8)
    o, lse = oracle.decode(prob, lib=lib)
    ro, rlse = dense_reference(q, K, V, np.asarray(lens), T, prob["sm_scale"], Ks, Vs)
    return (np.abs(o - ro.reshape(o.shape)).max() <= 1e-12
            and np.abs(lse - rlse.reshape(lse.shape)).max() <= 1e-12)


def check_identical_keys(lib, seed=5):
    """All visible keys equal => o = mean of the visible V rows, lse = s + ln n."""
    rng = np.random.default_rng(seed)
    B, T, Hq, Hkv, D, P = 1, 1, 4, 2, 64, 4
    L = 77
    K, V, _, _ = random_dense(rng, B, L, Hkv, D)
    K[:] = K[:, :1]
    q = rng.standard_normal((B * T, Hq, D), dtype=np.float32).astype(np.float16)
    prob = paged_from_dense(rng, q, K, V, (L,), P)
    o, lse = oracle.decode(prob, lib=lib)
    ok = True
    for h in range(Hq):
        g = h // (Hq // Hkv)
        s = prob["sm_scale"] * float(np.dot(q[0, h].astype(np.float64), K[0, 0, g].astype(np.float64)))
        mean = V[0, :L, g].astype(np.float64).mean(axis=0)
        ok &= np.abs(o[h] - mean).max() <= 1e-12
        ok &= abs(lse[h] - (s + math.log(L))) <= 1e-12
    return bool(ok)


def check_one_hot(lib, seed=6, int8=False):
    """One key aligned with q and a logit gap >= 40 => o = that position's V row."""
    rng = np.random.default_rng(seed)
    B, T, Hq, Hkv, D, P = 1, 1, 2, 1, 64, 16
    L, pos = 120, 83
    q = rng.standard_normal((1, Hq, D), dtype=np.float32).astype(np.float16)
    q[0, 1] = q[0, 0]
    if int8:
        K, V, Ks, Vs = random_dense(rng, B, L, Hkv, D, True)
        K[:] = rng.integers(-2, 3, size=K.shape)
        K[0, pos, 0] = np.where(q[0, 0] > 0, 127, -127)
        Ks[:] = np.float16(0.03125)
        Ks[0, pos, 0] = np.float16(0.125)
    else:
        K, V, Ks, Vs = random_dense(rng, B, L, Hkv, D)
        K *= np.float16(0.01)
        K[0, pos, 0] = q[0, 0] * np.float16(4.0)
    prob = paged_from_dense(rng, q, K, V, (L,), P, Ks=Ks, Vs=Vs)
    o, lse = oracle.decode(prob, lib=lib)
    Vf = dequant(V, Vs)
    Kf = dequant(K, Ks)
    s = prob["sm_scale"] * (Kf[0, :L, 0] @ q[0, 0].astype(np.float64))
    gap = s[pos] - np.delete(s, pos).max()
    assert gap >= 40, gap
    return bool(np.abs(o - Vf[0, pos, 0]).max() <= 1e-12)


def check_single_position(lib, seed=7):
    """kv_len 1 => o is exactly V row 0 and lse exactly its logit."""
    rng = np.random.default_rng(seed)
    K, V, _, _ = random_dense(rng, 2, 1, 2, 64)
    q = rng.standard_normal((2, 4, 64), dtype=np.float32).astype(np.float16)
    prob = paged_from_dense(rng, q, K, V, (1, 1), 16)
    o, lse = oracle.decode(prob, lib=lib)
    ok = True
    for r in range(8):
        b, h = r // 4, r % 4
        g = h // 2
        ok &= bool(np.array_equal(o[r], V[b, 0, g].astype(np.float64)))
        s = prob["sm_scale"] * float(np.dot(q[b, h].astype(np.float64), K[b, 0, g].astype(np.float64)))
        ok &= abs(lse[r] - s) <= 1e-14
    return bool(ok)


def check_causal_prefix(lib, seed=8, int8=False):
    """Causal T > 1: row t equals a T = 1 decode of the same cache with kv_len L - T + t + 1."""
    T = 4
    prob, (q, K, V, Ks, Vs) = _problem(seed, B=2, T=T, Hq=4, Hkv=2, D=64, P=4, lens=(23, 64),
                                       int8=int8)
    o, lse = oracle.decode(prob, lib=lib)
    ok = True
    for t in range(T):
        p1 = dict(prob)
        p1["q_per_seq"] = 1
        p1["q"] = np.ascontiguousarray(q.reshape(2, T, 4, 64)[:, t])
        p1["kv_len"] = (np.asarray(prob["kv_len"]) - T + t + 1).astype(np.int32)
        o1, l1 = oracle.decode(p1, lib=lib)
        ot = o.reshape(2, T, 4, 64)[:, t].reshape(-1, 64)
        lt = lse.reshape(2, T, 4)[:, t].reshape(-1)
        ok &= bool(np.array_equal(ot, o1)) and bool(np.array_equal(lt, l1))
    return bool(ok)


def check_int8_pow2_equivalence(lib, seed=9):
    """int8 values times power-of-two f16 scales are exact f16 values: an int8 cache and the
    equivalent f16 cache give bit-identical results."""
    rng = np.random.default_rng(seed)
    B, Hkv, D, L = 2, 2, 64, 50
    K = rng.integers(-127, 128, size=(B, L, Hkv, D)).astype(np.int8)
    V = rng.integers(-127, 128, size=(B, L, Hkv, D)).astype(np.int8)
    Ks = (2.0 ** rng.integers(-9, -4, size=(B, L, Hkv, D // 32))).astype(np.float16)
    Vs = (2.0 ** rng.integers(-9, -4, size=(B, L, Hkv, D // 32))).astype(np.float16)
    q = rng.standard_normal((B, 4, D), dtype=np.float32).astype(np.float16)
    r1 = np.random.default_rng(1)
    p8 = paged_from_dense(r1, q, K, V, (L, 31), 4, Ks=Ks, Vs=Vs)
    Kh = dequant(K, Ks).astype(np.float16)
    Vh = dequant(V, Vs).astype(np.float16)
    assert np.array_equal(Kh.astype(np.float64), dequant(K, Ks))
    r2 = np.random.default_rng(2)
    p16 = paged_from_dense(r2, q, Kh, Vh, (L, 31), 4)
    o8, l8 = oracle.decode(p8, lib=lib)
    o16, l16 = oracle.decode(p16, lib=lib)
    return bool(np.array_equal(o8, o16) and np.array_equal(l8, l16))


def check_gather_roundtrip(lib, seed=10, int8=False, P=4):
    prob, (q, K, V, Ks, Vs) = _problem(seed, B=3, T=1, Hq=4, Hkv=2, D=64, P=P, lens=(1, 45, 70),
                                       int8=int8, extra_heads=2)
    Lmax = 70
    dk, dv, dks, dvs = oracle.gather(prob, Lmax, lib=lib)
    ok = True
    for b, n in enumerate((1, 45, 70)):
        ok &= np.array_equal(dk[b, :n].view(np.uint8), K[b, :n].view(np.uint8))
        ok &= np.array_equal(dv[b, :n].view(np.uint8), V[b, :n].view(np.uint8))
        if int8:
            ok &= np.array_equal(dks[b, :n].view(np.uint16), Ks[b, :n].view(np.uint16))
            ok &= np.array_equal(dvs[b, :n].view(np.uint16), Vs[b, :n].view(np.uint16))
    return bool(ok)


def check_split_identity(lib, seed=11):
    prob, _ = _problem(seed, B=2, T=2, Hq=4, Hkv=2, D=64, P=16, lens=(700, 1300), q_mult=2.0)
    o, lse = oracle.decode(prob, lib=lib)
    ok = True
    for blk in (1, 64, 128, 1024, 4096):
        ob, lb = oracle.decode_blocked(prob, blk, lib=lib)
        ok &= np.abs(ob - o).max() <= 1e-12 and np.abs(lb - lse).max() <= 1e-12
    return bool(ok)


def check_empty_rows(lib, seed=12):
    rng = np.random.default_rng(seed)
    K, V, _, _ = random_dense(rng, 2, 9, 1, 32)
    q = rng.standard_normal((2, 2, 32), dtype=np.float32).astype(np.float16)
    prob = paged_from_dense(rng, q, K, V, (0, 9), 4)
    o, lse = oracle.decode(prob, lib=lib)
    return bool(np.all(o[:2] == 0) and np.all(np.isneginf(lse[:2])) and np.all(np.isfinite(lse[2:])))


ALL_PINS = [
    ("sdpa", lambda lib: all(check_sdpa(lib, c, 100 + i) for i, c in enumerate(CASES))),
    ("identical_keys", check_identical_keys),
    ("one_hot", check_one_hot),
    ("one_hot_int8", lambda lib: check_one_hot(lib, int8=True)),
    ("single_position", check_single_position),
    ("causal_prefix", check_causal_prefix),
    ("causal_prefix_int8", lambda lib: check_causal_prefix(lib, int8=True)),
    ("int8_pow2", check_int8_pow2_equivalence),
    ("gather_f16", check_gather_roundtrip),
    ("gather_i8_P1", lambda lib: check_gather_roundtrip(lib, int8=True, P=1)),
    ("split_identity", check_split_identity),
    ("empty_rows", check_empty_rows),
]

# --------------------------------------------------------------------------- tests


def test_half_decode_all_patterns():
    """The oracle's f16 -> f64 decode equals numpy's on all 65536 bit patterns."""
    lib = oracle.load()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = np.array([lib.oracle_half_to_double(int(b)) for b in bits])
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])


@pytest.mark.parametrize("i", range(len(CASES)))
def test_matches_sdpa(i):
    assert check_sdpa(oracle.load(), CASES[i], 100 + i)


@pytest.mark.parametrize("name,fn", ALL_PINS[1:], ids=[n for n, _ in ALL_PINS[1:]])
def test_pin(name, fn):
    assert fn(oracle.load())


def test_oracle_row_subset_matches_full():
    prob, _ = _problem(13, B=2, T=2, Hq=4, Hkv=2, D=64, P=4, lens=(23, 64))
    o, lse = oracle.decode(prob)
    rows = np.array([15, 0, 7, 3])
    os_, ls = oracle.decode(prob, rows=rows)
    assert np.array_equal(os_, o[rows]) and np.array_equal(ls, lse[rows])


MUTANTS = {
    1: "interleaved head map", 2: "scale dropped", 3: "causal off by one", 4: "wrong slot",
    5: "wrong int8 scale group", 6: "max dropped from lse", 7: "o not normalized",
    8: "V used as K", 9: "exp sign flipped", 10: "query token ignored",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=[MUTANTS[m] for m in sorted(MUTANTS)])
def test_pins_catch_planted_mistake(mutant):
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

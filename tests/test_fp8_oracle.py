"""Pins of the oracle's fp8 cache (OCP E4M3 bytes times a per-tensor f32 scale for K and one
for V, the fp8 caches with k_scale / v_scale that the AMD-Ecosystem/flashinfer PR #397 commit
messages name), CPU only.

Each pin ties the oracle to something other than itself: torch's float8_e4m3fn decoding of all
256 bytes and its nearest-even encoding (library routines), values the format fixes (448 the
largest, 2^-6 the smallest normal, 2^-9 the smallest subnormal), torch's fp64 SDPA over the
dequantized cache, and the decode of what the fp8 append wrote. Mutants with a planted mistake
must fail a pin.
"""
import os
import tempfile

import numpy as np
import pytest
import torch

import oracle
from tests.paged import dense_reference, e4m3_values, paged_from_dense


def check_decode_all_bytes(lib):
    codes = np.arange(256, dtype=np.uint8)
    mine = np.array([lib.oracle_e4m3_to_double(int(c)) for c in codes])
    ref = e4m3_values(codes)
    nan = np.isnan(ref)
    ok = np.array_equal(np.isnan(mine), nan) and nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    ok &= np.array_equal(mine[~nan], ref[~nan])
    # values the format fixes
    ok &= mine[0x7E] == 448.0 and mine[0x08] == 2.0 ** -6 and mine[0x01] == 2.0 ** -9
    ok &= mine[0x38] == 1.0 and mine[0xB8] == -1.0 and mine[0x80] == 0.0
    return bool(ok)


def _torch_encode(x):
    """f32 -> E4M3 bytes by torch (nearest even); inputs already within +-448."""
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def check_encode_against_torch(lib, seed=1):
    rng = np.random.default_rng(seed)
    vals = np.concatenate([
        rng.standard_normal(3000).astype(np.float32) * np.float32(8),
        rng.uniform(-448, 448, 2000).astype(np.float32),
        (rng.standard_normal(1000) * 2.0 ** -8).astype(np.float32),   # subnormal range
    ])
    # every midpoint between consecutive magnitudes (exact ties), and one f32 ulp either side
    mags = np.array([lib.oracle_e4m3_to_double(c) for c in range(0x7F)])
    mid = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    vals = np.concatenate([vals, mid, -mid, np.nextafter(mid, np.float32(0)),
                           np.nextafter(mid, np.float32(1000)), mags.astype(np.float32)])
    mine = np.array([lib.oracle_e4m3_from_float(float(v)) for v in vals], np.uint8)
    return bool(np.array_equal(mine, _torch_encode(vals)))


def check_encode_special(lib):
    ok = lib.oracle_e4m3_from_float(1e6) == 0x7E and lib.oracle_e4m3_from_float(-1e6) == 0xFE
    ok &= lib.oracle_e4m3_from_float(float("inf")) == 0x7E
    ok &= lib.oracle_e4m3_from_float(float("nan")) == 0x00
    ok &= lib.oracle_e4m3_from_float(-0.0) == 0x80 and lib.oracle_e4m3_from_float(0.0) == 0x00
    ok &= lib.oracle_e4m3_from_float(464.0) == 0x7E  # above 448 saturates (no overflow to NaN)
    ok &= lib.oracle_e4m3_from_float(2.0 ** -10) == 0x00  # half of 2^-9: tie to even (zero)
    ok &= lib.oracle_e4m3_from_float(3 * 2.0 ** -10) == 0x02  # 1.5 * 2^-9: tie to even (2)
    return bool(ok)


def _fp8_problem(rng, B, T, Hq, Hkv, D, P, lens, extra_heads=1):
    Lmax = max(lens)
    K = rng.integers(0, 256, (B, Lmax, Hkv, D)).astype(np.uint8)
    V = rng.integers(0, 256, (B, Lmax, Hkv, D)).astype(np.uint8)
    K[(K & 0x7F) == 0x7F] ^= 1   # no NaN bytes in the live cache
    V[(V & 0x7F) == 0x7F] ^= 1
    ks = np.float32(rng.uniform(0.001, 0.01))
    vs = np.float32(rng.uniform(0.001, 0.01))
    q = rng.standard_normal((B * T, Hq, D), dtype=np.float32).astype(np.float16)
    prob = paged_from_dense(rng, q, K, V, lens, P, T=T, extra_heads=extra_heads, Ks=ks, Vs=vs)
    return prob, (q, K, V, ks, vs)


def check_sdpa_fp8(lib, seed=2):
    rng = np.random.default_rng(seed)
    ok = True
    for (B, T, Hq, Hkv, D, P, lens) in ((2, 1, 8, 2, 64, 4, (37, 90)),
                                        (2, 3, 4, 4, 128, 16, (3, 70))):
        prob, (q, K, V, ks, vs) = _fp8_problem(rng, B, T, Hq, Hkv, D, P, lens)
        o, lse = oracle.decode(prob, lib=lib)
        ro, rl = dense_reference(q, K, V, np.asarray(lens), T, prob["sm_scale"], ks, vs)
        ok &= np.abs(o - ro.reshape(o.shape)).max() <= 1e-12
        ok &= np.abs(lse - rl.reshape(lse.shape)).max() <= 1e-12
    return bool(ok)


def check_append_fp8(lib, seed=3):
    """The fp8 append writes torch's nearest-even E4M3 of clip(x / s) at the slots the decode
    reads, and nothing else; the decode of the written cache equals SDPA over those bytes."""
    rng = np.random.default_rng(seed)
    B, Hkv, D, P, L = 2, 2, 64, 4, (9, 14)
    prob, _ = _fp8_problem(rng, B, 1, 4, Hkv, D, P, L, extra_heads=0)
    N = sum(L)
    xk = (rng.standard_normal((N, Hkv, D)) * 3).astype(np.float16)
    xv = (rng.standard_normal((N, Hkv, D)) * 3).astype(np.float16)
    bi = np.concatenate([np.full(n, b) for b, n in enumerate(L)]).astype(np.int32)
    pos = np.concatenate([np.arange(n) for n in L]).astype(np.int32)
    order = rng.permutation(N)
    ks, vs = prob["k_scales"], prob["v_scales"]
    k, v, _, _, skipped = oracle.append(xk[order], xv[order], bi[order], pos[order],
                                        prob["page_table"], max(L), prob["k_pages"],
                                        prob["v_pages"], ks, vs, lib=lib)
    ok = skipped == 0
    ek = _torch_encode(np.clip(xk.astype(np.float32) / ks[0], -448, 448))
    ev = _torch_encode(np.clip(xv.astype(np.float32) / vs[0], -448, 448))
    tab = prob["page_table"]
    touched = np.zeros(k.shape[:2], bool)
    for i in range(N):
        b, j = bi[i], pos[i]
        pg, sl = tab[b, j // P], j % P
        ok &= np.array_equal(k[pg, sl], ek[i]) and np.array_equal(v[pg, sl], ev[i])
        touched[pg, sl] = True
    ok &= np.array_equal(k[~touched], prob["k_pages"][~touched])
    new = dict(prob, k_pages=k, v_pages=v)
    o, lse = oracle.decode(new, lib=lib)
    Kd = np.zeros((B, max(L), Hkv, D), np.uint8)
    Vd = np.zeros_like(Kd)
    Kd[bi, pos], Vd[bi, pos] = ek, ev
    ro, rl = dense_reference(prob["q"], Kd, Vd, np.asarray(L), 1, prob["sm_scale"], ks, vs)
    ok &= np.abs(o - ro.reshape(o.shape)).max() <= 1e-12
    return bool(ok)


def check_non_finite(lib):
    """The rule's clip at +-448 makes an infinite quotient the nearest value to +-448 (the
    largest finite E4M3 magnitude), and a NaN quotient stores 0."""
    b = oracle.e4m3_from_float(np.array([np.inf, -np.inf, np.nan, 448.0, -448.0], np.float32),
                               lib=lib)
    v = oracle.e4m3_to_float(b[:2], lib=lib)
    return bool(b[0] == b[3] and b[1] == b[4] and b[2] == 0 and v[0] == 448.0 and v[1] == -448.0)


ALL_PINS = [
    ("non_finite", check_non_finite),
    ("decode_all_bytes", check_decode_all_bytes),
    ("encode_against_torch", check_encode_against_torch),
    ("encode_special", check_encode_special),
    ("sdpa_fp8", check_sdpa_fp8),
    ("append_fp8", check_append_fp8),
]


@pytest.mark.parametrize("name,fn", ALL_PINS, ids=[n for n, _ in ALL_PINS])
def test_fp8_pin(name, fn):
    assert fn(oracle.load())


MUTANTS = {17: "subnormal exponent off by one", 18: "tensor scale dropped",
           19: "ties to the smaller magnitude"}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=[MUTANTS[m] for m in sorted(MUTANTS)])
def test_fp8_pins_catch_planted_mistake(mutant):
    with tempfile.TemporaryDirectory() as d:
        lib = oracle.load(oracle.build(os.path.join(d, f"liboracle_m{mutant}.so"), mutant=mutant))
        failed = [n for n, fn in ALL_PINS if not fn(lib)]
        assert failed, f"no pin catches mutant {mutant} ({MUTANTS[mutant]})"


def test_fp8_generator_recipe():
    """The fp8 inputs follow their recipe: scales in [1/80, 1/64]; every byte a decode reads is a
    finite E4M3 value and every slot it must not read holds the NaN byte; dequantized values are
    N(0,1) draws to within E4M3's rounding."""
    import workloads
    s = workloads.spec(name="f8_recipe", batch=3, q_per_seq=1, num_qo_heads=8, num_kv_heads=2,
                       head_dim=128, page_size=16, kv_dtype="f8", lens=("list", (5, 300, 64)))
    prob = workloads.generate(s, 9)
    ks, vs = float(prob["k_scales"][0]), float(prob["v_scales"][0])
    assert 1 / 80 <= ks <= 1 / 64 and 1 / 80 <= vs <= 1 / 64
    k, table, L, P = prob["k_pages"], prob["page_table"], prob["kv_len"], 16
    live = np.zeros(k.shape[:2], bool)
    for b in range(3):
        for j in range(int(L[b])):
            live[table[b, j // P], j % P] = True
    assert not ((k[live] & 0x7F) == 0x7F).any()
    assert ((k[~live] & 0x7F) == 0x7F).all()
    x = e4m3_values(k[live]) * ks
    assert abs(x.mean()) < 0.05 and 0.93 < x.std() < 1.07

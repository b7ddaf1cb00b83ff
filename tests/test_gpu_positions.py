"""GPU tests that see which cache position the decode hot path read.

* The hot path's own addressing, bit for bit: skvd_gather_debug runs the plan's partial-kernel
  variant in a debug form that stores every K/V element and scale at the point where the decode
  consumes it (after the int8 / q4_0 lane transposes), at the position the kernel attributes it
  to. Compared with the oracle's gather for every variant: f16 / int8 / fp8 / q4_0, head_dim
  128, 192, 256 and 512, one to four row quarters, row tiles (more than 16 query rows per KV
  head) and row groups (more than 64), 1 / 2 / 4 / 8 KV heads per workgroup, page sizes 1, 4, 16 and 64 (per-token
  and per-tile page lookups), static and balanced schedules.
* A one-hot dominant key (logit gap >= 40 over every other visible key, checked on the stored
  values) at the first and last token of pages, 16-token tiles, 32-token chunks, 64-token
  blocks, splits and balanced shares, and at the ends of the sequence, up to 65536 tokens:
  o must be that position's V row (a misread position moves o by O(1)).
* Identical keys: o = the mean of the visible V rows, lse = s + ln n (closed form).
Tolerances: max|do| <= 2e-3 against the oracle and against the dominant V row / the mean,
max|dlse| <= 1e-3.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from tests import paged
from tests.gpu_util import compare, make_plan, run, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_kv_cache_page_amd as skvd
    skvd.lib()
    yield
    torch.cuda.synchronize()


def _seed(*parts):
    return zlib.crc32(repr(parts).encode()) % 100000


# ------------------------------------------------------------------ hot-path gather, bit-exact
# (D, T, Hq, Hkv): query rows R = Hq / Hkv * T per KV head select the variant
SHAPES = [
    (128, 1, 32, 8),   # R 4: one row quarter, vector P.V (1 / 2 / 4 / 8 KV heads per workgroup)
    (128, 2, 16, 4),   # R 8: two quarters, MFMA P.V
    (128, 4, 16, 4),   # R 16: four quarters
    (128, 3, 32, 4),   # R 24: two row tiles
    (128, 8, 32, 4),   # R 64: four row tiles
    (128, 8, 64, 4),   # R 128: two row groups of four row tiles
    (256, 1, 8, 4),    # R 2 at head_dim 256
    (256, 4, 16, 4),   # R 16 at head_dim 256
    (256, 8, 16, 2),   # R 64 at head_dim 256
    (192, 1, 16, 4),   # head_dim 192 (24-lane V rows, two per load step; fp8 K zero-padded)
    (192, 8, 16, 2),   # R 64 at head_dim 192
    (512, 1, 16, 4),   # head_dim 512
    (512, 4, 16, 4),   # R 16 at head_dim 512
]


def _gather_case(kv, D, T, Hq, Hkv, P, schedule, hw=0, lens=(1, 190, 700, 2100)):
    rng = np.random.default_rng(_seed(kv, D, T, Hq, Hkv, P, schedule, hw))
    B = len(lens)
    Lmax = max(lens)
    K = rng.standard_normal((B, Lmax, Hkv, D)).astype(np.float32)
    V = rng.standard_normal((B, Lmax, Hkv, D)).astype(np.float32)
    Kd, Ks = paged.quantize_dense(K, kv)
    Vd, Vs = paged.quantize_dense(V, kv)
    q = rng.standard_normal((B * T, Hq, D)).astype(np.float16)
    prob = paged.paged_from_dense(rng, q, Kd, Vd, np.array(lens, np.int32), P, T=T, Ks=Ks, Vs=Vs)
    dev = to_dev(prob)
    kw = dict(schedule=schedule, force_blocks_per_split=2)
    if hw:
        kw["heads_per_wg"] = hw
    plan = make_plan(prob, **kw)
    dk, dv, dks, dvs = plan.gather_debug(dev["q"], dev["k_pages"], dev["v_pages"],
                                         dev["page_table"], dev["kv_len"], Lmax,
                                         dev["k_scales"], dev["v_scales"], q_per_seq=T)
    torch.cuda.synchronize()
    ok, ov, oks, ovs = oracle.gather(prob, Lmax)
    tag = f"gather {kv} D={D} T={T} Hq={Hq} Hkv={Hkv} P={P} {schedule} hw={hw}: {plan.describe()}"
    assert np.array_equal(dk.cpu().numpy().view(np.uint8), ok.view(np.uint8)), tag + " K"
    assert np.array_equal(dv.cpu().numpy().view(np.uint8), ov.view(np.uint8)), tag + " V"
    if kv in ("i8", "q4"):
        assert np.array_equal(dks.cpu().numpy().view(np.uint16), oks.view(np.uint16)), tag + " Ks"
        assert np.array_equal(dvs.cpu().numpy().view(np.uint16), ovs.view(np.uint16)), tag + " Vs"
    say(f"  {tag}: bit-exact")


@pytest.mark.parametrize("schedule", ["balanced", "static"])
@pytest.mark.parametrize("P", [16, 1, 64, 4])
@pytest.mark.parametrize("kv", ["f16", "i8", "f8", "q4"])
def test_hot_path_gather_bit_exact(kv, P, schedule):
    for D, T, Hq, Hkv in SHAPES:
        if D == 192 and kv in ("i8", "q4"):
            continue  # (the plan refuses int8 and q4_0 at head_dim 192)
        _gather_case(kv, D, T, Hq, Hkv, P, schedule)
    for hw in (1, 2, 8):
        _gather_case(kv, 128, 1, 32, 8, P, schedule, hw=hw)


def test_hot_path_gather_large_balanced_batch():
    """Balanced shares over more than 64 sequences (several sequences per lane of the share
    computation)."""
    rng = np.random.default_rng(7)
    for B in (65, 130, 300):
        lens = tuple(int(x) for x in rng.integers(0, 300, B))
        for kv in ("f16", "i8", "q4"):
            _gather_case(kv, 128, 1, 32, 8, 16, "balanced", lens=lens)


# ------------------------------------------------------------------ one-hot dominant key
def _boundary_blocks(plan, lens, Hkv, hw, R):
    """Per (sequence, KV head): 64-token block indices where a split (static) or a share
    (balanced) of the plan starts, computed from the plan's shape by the schedule's integer
    rule (share w starts at global block floor(w N / W); the schedule's heads are the KV head
    groups times the row groups of R query rows)."""
    info = plan.info
    rt = 1 if R <= 16 else (2 if R <= 32 else 4)
    nrg = -(-R // min(R, 16 * rt))
    nb = [(int(L) + 63) // 64 for L in lens]
    out = {(b, g): set() for b in range(len(lens)) for g in range(Hkv)}
    if plan.schedule == "static":
        step = int(info.blocks_per_split)
        for b in range(len(lens)):
            for g in range(Hkv):
                out[(b, g)].update(range(step, nb[b], step))
        return out
    Hg = Hkv // hw * nrg
    N = Hg * sum(nb)
    W = max(1, min(int(info.grid_wgs), N))
    pre = np.concatenate([[0], np.cumsum(nb)])
    for w in range(1, W):
        x = w * N // W
        xq = x // Hg
        b = int(np.searchsorted(pre, xq, side="right") - 1)
        off = x - Hg * int(pre[b])
        grp, blk = off // nb[b], off % nb[b]
        kg = grp // nrg
        for g in range(kg * hw, kg * hw + hw):
            out[(b, g)].add(int(blk))
    return out


EDGE = [0, 1, 15, 16, 17, 31, 32, 33, 47, 48, 63, 64, 65, 127, 128]


def _positions(plan, lens, Hkv, hw, T, P, variant, R):
    """One dominant position per (sequence, KV head): variant 0 takes the first token of a
    split/share boundary block (else a tile/chunk/page edge), variant 1 the token before it
    (else the sequence's last visible position), variant 2 a page edge."""
    bnd = _boundary_blocks(plan, lens, Hkv, hw, R)
    pos = []
    for b, L in enumerate(lens):
        row = []
        for g in range(Hkv):
            lim = int(L) - T
            cands = sorted(bnd[(b, g)])
            k = b * Hkv + g
            if variant == 0:
                p = 64 * cands[k % len(cands)] if cands else EDGE[k % len(EDGE)]
            elif variant == 1:
                p = 64 * cands[k % len(cands)] - 1 if cands else lim
            else:
                p = P * (1 + k) - (k % 2)
            row.append(int(min(max(p, 0), lim)))
        pos.append(row)
    return pos


DOM = [
    # (name, B, T, Hq, Hkv, D, P, kv, lens, plan kw)
    ("f16_long", 2, 1, 32, 8, 128, 16, "f16", (65536, 777), {}),
    ("i8_long", 2, 1, 32, 8, 128, 16, "i8", (65536, 777), {}),
    ("f8_long", 2, 1, 32, 8, 128, 16, "f8", (65536, 777), {}),
    ("f16_p64", 3, 1, 32, 8, 128, 64, "f16", (9000, 4100, 2049), {}),
    ("i8_p1", 2, 1, 8, 2, 128, 1, "i8", (5000, 129), {}),
    ("f16_p1", 2, 1, 8, 2, 128, 1, "f16", (3000, 2048), {}),
    ("f8_p4", 2, 1, 16, 4, 128, 4, "f8", (3000, 700), {}),
    ("i8_hw1", 3, 1, 32, 8, 128, 16, "i8", (5000, 2100, 300), dict(heads_per_wg=1)),
    ("f16_hw8", 3, 1, 32, 8, 128, 16, "f16", (5000, 2100, 300), dict(heads_per_wg=8)),
    ("i8_t2_rb2", 2, 2, 16, 4, 128, 16, "i8", (4000, 600), {}),
    ("i8_d256_t2", 2, 2, 8, 4, 256, 16, "i8", (3000, 700), {}),
    ("f8_d256_t4", 2, 4, 16, 4, 256, 16, "f8", (3000, 700), {}),
    ("f16_g8_t8", 2, 8, 32, 4, 128, 16, "f16", (3000, 900), {}),
    ("i8_g8_t8", 2, 8, 32, 4, 128, 16, "i8", (3000, 900), {}),
    ("f8_g16_t8", 2, 8, 64, 4, 128, 16, "f8", (2500, 600), {}),
    ("i8_g8_t8_d256", 2, 8, 16, 2, 256, 16, "i8", (2000, 700), {}),
    ("f16_d192", 2, 1, 16, 4, 192, 16, "f16", (3000, 700), {}),
    ("f8_d192_t2", 2, 2, 8, 4, 192, 16, "f8", (3000, 700), {}),
    ("i8_d512", 2, 1, 16, 4, 512, 16, "i8", (3000, 700), {}),
    ("f16_d512_t4", 2, 4, 16, 4, 512, 16, "f16", (2500, 700), {}),
    ("q4_long", 2, 1, 32, 8, 128, 16, "q4", (65536, 777), {}),
    ("q4_p1", 2, 1, 8, 2, 128, 1, "q4", (5000, 129), {}),
    ("q4_hw1", 3, 1, 32, 8, 128, 16, "q4", (5000, 2100, 300), dict(heads_per_wg=1)),
    ("q4_t2_rb2", 2, 2, 16, 4, 128, 16, "q4", (4000, 600), {}),
    ("q4_d256_t2", 2, 2, 8, 4, 256, 16, "q4", (3000, 700), {}),
    ("q4_g8_t8", 2, 8, 32, 4, 128, 16, "q4", (3000, 900), {}),
    ("q4_d512", 2, 1, 16, 4, 512, 16, "q4", (3000, 700), {}),
]


@pytest.mark.parametrize("variant", [0, 1, 2])
@pytest.mark.parametrize("schedule", ["auto", "static"])
@pytest.mark.parametrize("case", DOM, ids=[c[0] for c in DOM])
def test_dominant_key_position(case, schedule, variant):
    name, B, T, Hq, Hkv, D, P, kv, lens, kw = case
    G = Hq // Hkv
    rng = np.random.default_rng(_seed(name, schedule, variant))
    # the plan first (its shape fixes the boundaries), then the problem
    probe = dict(q=np.zeros((B * T, Hq, D), np.float16),
                 k_pages=np.zeros((1, P, Hkv, D // 2 if kv == "q4" else D),
                                  {"f16": np.float16, "i8": np.int8, "f8": np.uint8,
                                   "q4": np.uint8}[kv]),
                 kv_len=np.array(lens, np.int32), q_per_seq=T,
                 page_table=np.zeros((B, -(-max(lens) // P) + 2), np.int32))
    plan = make_plan(probe, schedule=schedule, **kw)
    hw = int(plan.info.heads_per_wg)
    pos = _positions(plan, lens, Hkv, hw, T, P, variant, G * T)
    prob, dom = paged.dominant_problem(rng, B, T, Hq, Hkv, D, P, lens, kv, pos)
    say(f"case {name} {schedule} v{variant}: {plan.describe()} positions {pos[0][:4]}...")
    dev = to_dev(prob)
    plan = make_plan(prob, schedule=schedule, **kw)
    o, lse = run(plan, prob, dev)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(prob)
    compare(o, lse, ro, rl, what=f"{name} {schedule} v{variant}")
    go = o.float().cpu().numpy().astype(np.float64).reshape(B, T, Hq, D)
    for b in range(B):
        for h in range(Hq):
            err = np.abs(go[b, :, h] - dom[b, h // G][None]).max()
            assert err <= 2e-3, (name, b, h, pos[b][h // G], err)


# ------------------------------------------------------------------ identical keys
IDENT = [
    ("f16", 3, 1, 32, 8, 128, 16, (1, 2047, 5000)),
    ("i8", 3, 1, 32, 8, 128, 16, (64, 2049, 5000)),
    ("f8", 2, 1, 16, 4, 128, 16, (700, 4097)),
    ("i8", 2, 4, 8, 4, 256, 16, (4, 3000)),
    ("f16", 2, 8, 32, 4, 128, 1, (8, 1500)),
    ("i8", 2, 8, 32, 4, 128, 16, (9, 2500)),
    ("q4", 3, 1, 32, 8, 128, 16, (64, 2049, 5000)),
    ("q4", 2, 4, 8, 4, 256, 16, (4, 3000)),
]


@pytest.mark.parametrize("schedule", ["auto", "static"])
@pytest.mark.parametrize("case", IDENT, ids=[f"{c[0]}_T{c[2]}_D{c[5]}_P{c[6]}" for c in IDENT])
def test_identical_keys_mean_of_v(case, schedule):
    kv, B, T, Hq, Hkv, D, P, lens = case
    G = Hq // Hkv
    rng = np.random.default_rng(_seed("ident", case, schedule))
    prob, Kf, Vf = paged.identical_key_problem(rng, B, T, Hq, Hkv, D, P, lens, kv)
    dev = to_dev(prob)
    plan = make_plan(prob, schedule=schedule)
    say(f"case identical keys {case} {schedule}: {plan.describe()}")
    o, lse = run(plan, prob, dev)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(prob)
    compare(o, lse, ro, rl, what=f"identical keys {kv}")
    go = o.float().cpu().numpy().astype(np.float64).reshape(B, T, Hq, D)
    gl = lse.cpu().numpy().astype(np.float64).reshape(B, T, Hq)
    q = prob["q"].astype(np.float64).reshape(B, T, Hq, D)
    for b, L in enumerate(lens):
        for t in range(T):
            n = int(L) - T + t + 1
            for h in range(Hq):
                g = h // G
                mean = Vf[b, :n, g].mean(axis=0)
                s = prob["sm_scale"] * float(q[b, t, h] @ Kf[b, 0, g])
                assert np.abs(go[b, t, h] - mean).max() <= 2e-3, (b, t, h)
                assert abs(gl[b, t, h] - (s + math.log(n))) <= 1e-3, (b, t, h)

"""GPU parity: the HIP path through the C ABI against the fp64 oracle on seeded inputs.

Small and mid-size problems are compared on every output; the full-size workloads on sampled
rows. Tolerances: max|do| <= 2e-3, max|dlse| <= 1e-3; page gather bit-exact.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
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


def spec(**kw):
    return workloads.spec(**kw)


def check(s, seed, plan_kw=None, rows=None, what=None):
    prob = workloads.generate(s, seed)
    what = what or f"{s.name} seed={seed} {plan_kw or ''}"
    say(f"case {what}: B={s.batch} T={s.q_per_seq} Hq={s.num_qo_heads} Hkv={s.num_kv_heads} "
        f"D={s.head_dim} P={s.page_size} kv={s.kv_dtype} L={list(prob['kv_len'])[:8]}")
    dev = to_dev(prob)
    plan = make_plan(prob, **(plan_kw or {}))
    say(f"  {plan.describe()}")
    o, lse = run(plan, prob, dev)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(prob, rows=rows)
    compare(o, lse, ro, rl, rows=rows, what=what)
    return prob, dev, plan, o, lse


# ------------------------------------------------------------------ small/mid shapes, all rows
SMALL = [
    # (name, batch, T, Hq, Hkv, D, P, kv, lens)
    ("mha_one_tile", 1, 1, 8, 8, 128, 16, "f16", ("list", (256,))),
    ("gqa4_ragged", 5, 1, 32, 8, 128, 16, "f16", ("list", (1, 63, 64, 65, 1000))),
    ("gqa4_p1", 3, 1, 8, 2, 128, 1, "f16", ("list", (17, 130, 300))),
    ("gqa4_p4", 3, 1, 8, 2, 128, 4, "f16", ("list", (5, 64, 257))),
    ("gqa2_t4_d256", 3, 4, 8, 4, 256, 16, "f16", ("list", (4, 100, 700))),
    ("gqa2_t4_d256_p2", 2, 4, 4, 2, 256, 2, "f16", ("list", (9, 333))),
    ("mha_t2_d256", 2, 2, 4, 4, 256, 64, "f16", ("list", (2, 1500))),
    ("gqa8_t2", 2, 2, 16, 2, 128, 16, "f16", ("list", (40, 900))),
    ("int8_gqa4", 4, 1, 32, 8, 128, 16, "i8", ("list", (1, 65, 512, 2049))),
    ("int8_p1", 2, 1, 8, 2, 128, 1, "i8", ("list", (33, 200))),
    ("int8_t4_d256", 2, 4, 8, 4, 256, 16, "i8", ("list", (4, 600))),
    ("int8_t3_g2", 2, 3, 4, 2, 128, 8, "i8", ("list", (3, 400))),
    ("int8_t4_g4", 2, 4, 16, 4, 128, 16, "i8", ("list", (4, 900))),     # 16 rows: 4 quarters
    ("int8_t4_g4_p4", 3, 4, 8, 2, 128, 4, "i8", ("list", (5, 64, 333))),
    ("int8_t2_g4", 2, 2, 8, 2, 128, 16, "i8", ("list", (2, 1500))),     # 8 rows: 2 quarters
    ("d192_gqa4", 3, 1, 16, 4, 192, 16, "f16", ("list", (1, 700, 2100))),  # head_dim 192
    ("d192_t4_p2", 2, 4, 8, 4, 192, 2, "f16", ("list", (4, 333))),
    ("d192_f8", 3, 1, 16, 4, 192, 16, "f8", ("list", (65, 700, 1500))),
    ("d512_gqa4", 3, 1, 16, 4, 512, 16, "f16", ("list", (1, 700, 2100))),  # head_dim 512
    ("d512_t2_p4", 2, 2, 8, 4, 512, 4, "f16", ("list", (2, 400))),
    ("d512_i8", 3, 1, 16, 4, 512, 16, "i8", ("list", (64, 900, 1700))),
    ("d512_i8_t4_p1", 2, 4, 8, 2, 512, 1, "i8", ("list", (5, 300))),
    ("d512_f8", 3, 1, 16, 4, 512, 16, "f8", ("list", (129, 800, 1300))),
    ("q4_gqa4", 4, 1, 32, 8, 128, 16, "q4", ("list", (1, 65, 512, 2049))),  # q4_0 cache
    ("q4_p1", 2, 1, 8, 2, 128, 1, "q4", ("list", (33, 200))),
    ("q4_t4_d256", 2, 4, 8, 4, 256, 16, "q4", ("list", (4, 600))),
    ("q4_t3_g2", 2, 3, 4, 2, 128, 8, "q4", ("list", (3, 400))),        # 6 rows: MFMA P.V
    ("q4_t4_g4", 2, 4, 16, 4, 128, 16, "q4", ("list", (4, 900))),
    ("q4_t2_g4_p4", 3, 2, 8, 2, 128, 4, "q4", ("list", (5, 64, 333))),
    ("d512_q4", 3, 1, 16, 4, 512, 16, "q4", ("list", (64, 900, 1700))),
    ("d512_q4_t4_p1", 2, 4, 8, 2, 512, 1, "q4", ("list", (5, 300))),
]


@pytest.mark.parametrize("schedule", ["auto", "static"])
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_all_rows(case, schedule):
    name, B, T, Hq, Hkv, D, P, kv, lens = case
    s = spec(name=name, batch=B, q_per_seq=T, num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D,
             page_size=P, kv_dtype=kv, lens=lens)
    check(s, seed=zlib.crc32(name.encode()) % 1000, plan_kw=dict(schedule=schedule))


_rng = np.random.default_rng(2024)
BALANCED = [
    # (name, B, T, Hq, Hkv, D, kv, lens, plan kw): shares that cover many short rows, empty
    # sequences, one long row among short ones, tiny and large grids
    ("tiny_rows", 64, 1, 8, 2, 128, "f16", tuple(int(x) for x in _rng.integers(0, 140, 64)),
     dict(force_blocks_per_split=1, wgs_per_cu=1, num_cus=8)),
    ("tiny_rows_i8", 64, 1, 8, 2, 128, "i8", tuple(int(x) for x in _rng.integers(0, 140, 64)),
     dict(force_blocks_per_split=2, wgs_per_cu=1, num_cus=5)),
    ("half_empty", 64, 1, 16, 4, 128, "f16", tuple([0, 333] * 32), dict(force_blocks_per_split=1)),
    ("one_long", 17, 2, 8, 4, 128, "f16", (5000,) + (70,) * 16, dict(force_blocks_per_split=2)),
    ("big_grid", 3, 1, 16, 16, 128, "f16", (64, 1000, 129), dict(force_blocks_per_split=1,
                                                                 wgs_per_cu=64)),
    ("mqa_d256", 9, 1, 4, 1, 256, "f16", (1, 300, 64, 65, 1200, 7, 0, 640, 2),
     dict(force_blocks_per_split=1, wgs_per_cu=2, num_cus=3)),
    ("t4_i8_d256", 5, 4, 8, 4, 256, "i8", (700, 4, 129, 1100, 64), dict(force_blocks_per_split=3)),
    ("tiny_rows_q4", 64, 1, 8, 2, 128, "q4", tuple(int(x) for x in _rng.integers(0, 140, 64)),
     dict(force_blocks_per_split=2, wgs_per_cu=1, num_cus=5)),
]


@pytest.mark.parametrize("case", BALANCED, ids=[c[0] for c in BALANCED])
def test_balanced_schedule_edges(case):
    name, B, T, Hq, Hkv, D, kv, lens, kw = case
    s = spec(name=name, batch=B, q_per_seq=T, num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D,
             page_size=16, kv_dtype=kv, lens=("list", lens))
    _, _, plan, _, _ = check(s, seed=zlib.crc32(name.encode()) % 1000,
                             plan_kw=dict(schedule="balanced", **kw))
    assert plan.schedule == "balanced"


@pytest.mark.parametrize("kv", ["i8", "f16", "q4"])
@pytest.mark.parametrize("hw", [1, 2, 4, 8])
@pytest.mark.parametrize("schedule", ["balanced", "static"])
@pytest.mark.parametrize("P", [16, 1])
def test_heads_per_workgroup(kv, hw, schedule, P):
    """Workgroups serving 1, 2, 4 or 8 KV heads (one wave each) over the same blocks."""
    s = spec(name="hw", batch=5, q_per_seq=1, num_qo_heads=32, num_kv_heads=8, head_dim=128,
             page_size=P, kv_dtype=kv, lens=("list", (1, 700, 64, 2100, 333)))
    _, _, plan, _, _ = check(s, seed=hw * 10 + P, plan_kw=dict(heads_per_wg=hw, schedule=schedule,
                                                              force_blocks_per_split=2))
    assert plan.info.heads_per_wg == hw


def test_balanced_all_empty():
    s = spec(name="all_empty", batch=4, q_per_seq=1, num_qo_heads=8, num_kv_heads=2,
             head_dim=128, page_size=16, lens=("list", (0, 0, 0, 0)))
    prob = workloads.generate(s, 1)
    prob["page_table"] = np.zeros((4, 300), np.int32)  # plan for up to 300 pages per row
    dev = to_dev(prob)
    plan = make_plan(prob, schedule="balanced")
    o, lse = run(plan, prob, dev)
    torch.cuda.synchronize()
    assert plan.schedule == "balanced"
    assert (o.float() == 0).all() and torch.isneginf(lse).all()


@pytest.mark.parametrize("kv", ["f16", "i8", "q4"])
@pytest.mark.parametrize("red,bps", [("direct", 1), ("cooperative", 1), ("multipass", 1),
                                     ("hierarchical", 1), ("direct", 3), ("multipass", 7),
                                     ("hierarchical", 2), ("none", 1000)])
@pytest.mark.parametrize("schedule", ["auto", "static"])
def test_forced_reducers_and_splits(kv, red, bps, schedule):
    s = spec(name="forced", batch=3, q_per_seq=1, num_qo_heads=16, num_kv_heads=4, head_dim=128,
             page_size=16, kv_dtype=kv, lens=("list", (70, 1300, 5000)))
    if red == "cooperative":
        s = spec(name="forced", batch=3, q_per_seq=1, num_qo_heads=16, num_kv_heads=4,
                 head_dim=128, page_size=16, kv_dtype=kv, lens=("list", (70, 1300, 4000)))
    check(s, seed=7, plan_kw=dict(force_reducer=red, force_blocks_per_split=bps,
                                  schedule=schedule))


@pytest.mark.parametrize("schedule", ["auto", "static"])
@pytest.mark.parametrize("red", ["cooperative", "multipass", "hierarchical"])
@pytest.mark.parametrize("D", [192, 256, 512])
def test_forced_reducers_wide_heads(D, red, schedule):
    """The merge's rounds of output-slice loads at every head_dim (64 / PER per round for more
    than 8 partials: 21, 16 and 8 loads), one block per split so that rows carry from 3 to
    beyond 64 partials (cooperative: up to 63), under both schedules."""
    lens = (130, 1100, 4000) if red == "cooperative" else (130, 1100, 5000)
    s = spec(name=f"wide{D}", batch=3, q_per_seq=1, num_qo_heads=8, num_kv_heads=2, head_dim=D,
             page_size=16, lens=("list", lens))
    check(s, seed=D, plan_kw=dict(force_reducer=red, force_blocks_per_split=1, schedule=schedule))


@pytest.mark.parametrize("L", [2047, 2048, 2049, 4095, 4096, 4097])
def test_2048_4096_boundaries(L):
    """Partial counts 32/33/64/65 around the pages' cooperative ceiling, at one block per
    split, with every reducer that covers them."""
    s = spec(name=f"boundary{L}", batch=2, q_per_seq=1, num_qo_heads=32, num_kv_heads=8,
             head_dim=128, page_size=16, lens=("list", (L, L - 1000)))
    for red in ("multipass", "hierarchical", "direct"):
        check(s, seed=L, plan_kw=dict(force_blocks_per_split=1, force_reducer=red,
                                      schedule="static"), what=f"L={L} {red} static")
    check(s, seed=L, plan_kw=dict(force_blocks_per_split=1), what=f"L={L} balanced")


def test_no_ceiling_262208():
    """One sequence of 262208 tokens = 4097 blocks, above the pages' 262144 cap."""
    s = spec(name="beyond_cap", batch=1, q_per_seq=1, num_qo_heads=8, num_kv_heads=2,
             head_dim=128, page_size=64, lens=("list", (262208,)))
    rows = np.arange(8)
    check(s, seed=11, plan_kw=dict(force_blocks_per_split=1, force_reducer="hierarchical",
                                   schedule="static"), rows=rows)
    check(s, seed=11, plan_kw=dict(force_blocks_per_split=1, force_reducer="multipass",
                                   schedule="static"), rows=rows)
    check(s, seed=11, plan_kw=dict(force_reducer="hierarchical"), rows=rows)
    check(s, seed=11, rows=rows)


def test_split_invariance():
    """Same input, every split size and reducer: all within tolerance of the oracle and of
    each other (LSE merge of partials = one-pass softmax)."""
    s = spec(name="inv", batch=2, q_per_seq=2, num_qo_heads=8, num_kv_heads=4, head_dim=128,
             page_size=16, lens=("list", (3000, 777)), q_mult=2.0)
    outs = []
    for bps, red, sch in [(1, "multipass", "auto"), (2, "hierarchical", "auto"),
                          (8, "cooperative", "auto"), (0, "auto", "auto"), (47, "direct", "auto"),
                          (1000, "none", "auto"), (1, "multipass", "static"),
                          (3, "auto", "static")]:
        _, _, _, o, lse = check(s, seed=3, plan_kw=dict(force_blocks_per_split=bps,
                                                         force_reducer=red, schedule=sch))
        outs.append((o.float().cpu(), lse.cpu()))
    for o, l in outs[1:]:
        assert (o - outs[0][0]).abs().max().item() <= 2e-3
        assert (l - outs[0][1]).abs().max().item() <= 1e-3


def test_gather_bit_exact():
    for kv, P in (("f16", 16), ("f16", 1), ("i8", 4), ("i8", 64), ("q4", 16), ("q4", 2)):
        s = spec(name="gather", batch=3, q_per_seq=1, num_qo_heads=4, num_kv_heads=2,
                 head_dim=128, page_size=P, kv_dtype=kv, lens=("list", (1, 190, 700)))
        prob = workloads.generate(s, 5)
        dev = to_dev(prob)
        plan = make_plan(prob)
        maxl = int(prob["kv_len"].max())
        dk, dv, dks, dvs = plan.gather_debug(dev["q"], dev["k_pages"], dev["v_pages"],
                                             dev["page_table"], dev["kv_len"], maxl,
                                             dev["k_scales"], dev["v_scales"])
        ok, ov, oks, ovs = oracle.gather(prob, maxl)
        assert np.array_equal(dk.cpu().numpy().view(np.uint8), ok.view(np.uint8))
        assert np.array_equal(dv.cpu().numpy().view(np.uint8), ov.view(np.uint8))
        if kv in ("i8", "q4"):
            assert np.array_equal(dks.cpu().numpy().view(np.uint16), oks.view(np.uint16))
            assert np.array_equal(dvs.cpu().numpy().view(np.uint16), ovs.view(np.uint16))
        say(f"  gather {kv} P={P}: bit-exact")


def test_single_position_exact():
    """kv_len 1: o is exactly the V row (weight 1), on the single-split and merged paths."""
    for kw in (dict(), dict(force_blocks_per_split=1, force_reducer="multipass")):
        s = spec(name="one", batch=3, q_per_seq=1, num_qo_heads=8, num_kv_heads=2, head_dim=128,
                 page_size=16, lens=("list", (1, 1, 1)))
        prob, dev, plan, o, lse = check(s, seed=9, plan_kw=kw)
        v = prob["v_pages"]
        for b in range(3):
            pg = prob["page_table"][b, 0]
            for h in range(8):
                assert np.array_equal(o[b, h].cpu().numpy().view(np.uint16),
                                      v[pg, 0, h // 4].view(np.uint16))


def test_empty_sequence():
    s = spec(name="empty", batch=3, q_per_seq=1, num_qo_heads=8, num_kv_heads=2, head_dim=128,
             page_size=16, lens=("list", (0, 50, 0)))
    for kw in (dict(max_kv_len=64), dict(force_blocks_per_split=1, force_reducer="cooperative")):
        prob, dev, plan, o, lse = check(s, seed=2, plan_kw=kw)
        assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))


def test_strided_q_and_shorter_v_pool():
    """q sliced from a fused QKV buffer (token stride > Hq*D) and a V pool with fewer pages
    than K (only indexed pages are read)."""
    s = spec(name="strided", batch=3, q_per_seq=1, num_qo_heads=16, num_kv_heads=4,
             head_dim=128, page_size=16, lens=("list", (33, 500, 1200)), spare_frac=0.0)
    prob = workloads.generate(s, 4)
    ref_o, ref_l = oracle.decode(prob)
    dev = to_dev(prob)
    qkv = torch.zeros((3, 16 + 8, 128), dtype=torch.float16, device="cuda")
    qkv[:, :16] = dev["q"]
    dev["q"] = qkv[:, :16]
    extra = torch.full((7,) + tuple(dev["k_pages"].shape[1:]), float("nan"),
                       dtype=torch.float16, device="cuda")
    dev["k_pages"] = torch.cat([dev["k_pages"], extra])  # K pool longer than V pool
    plan = make_plan(prob)
    o, lse = run(plan, prob, dev)
    torch.cuda.synchronize()
    compare(o, lse, ref_o, ref_l, what="strided q, unequal pools")


HND_CASES = [
    # (kv, B, T, Hq, Hkv, D, P, lens)
    ("f16", 3, 1, 32, 8, 128, 16, (33, 1500, 4100)),
    ("f16", 2, 4, 32, 16, 256, 16, (700, 3000)),
    ("i8", 3, 1, 32, 8, 128, 16, (33, 1500, 4100)),
    ("i8", 2, 2, 16, 8, 256, 64, (129, 2049)),
    ("f8", 3, 1, 32, 8, 128, 64, (64, 1500, 4100)),
    ("q4", 3, 1, 32, 8, 128, 16, (33, 1500, 4100)),
    ("q4", 2, 4, 32, 16, 256, 16, (700, 3000)),
    ("f16", 2, 1, 8, 2, 128, 4, (5, 300)),
]


@pytest.mark.parametrize("case", HND_CASES, ids=[f"{c[0]}_D{c[5]}_P{c[6]}_T{c[2]}" for c in
                                                 HND_CASES])
@pytest.mark.parametrize("sched", ["auto", "static"])
def test_hnd_pools(case, sched):
    """K/V pools (and int8 / q4_0 scale pools) in HND memory order: each KV head's page rows
    contiguous, passed as the permuted [N, P, Hkv, X] view; the decode reads them through the
    strides alone (the results depend only on the values)."""
    kv, B, T, Hq, Hkv, D, P, lens = case
    s = spec(name=f"hnd_{kv}", batch=B, q_per_seq=T, num_qo_heads=Hq, num_kv_heads=Hkv,
             head_dim=D, page_size=P, kv_dtype=kv, lens=("list", lens))
    prob = workloads.generate(s, 91)
    dev = to_dev(prob, layout="hnd")
    assert dev["k_pages"].stride(1) != dev["k_pages"].shape[2] * dev["k_pages"].shape[3]
    plan = make_plan(prob, schedule=sched)
    say(f"case hnd {kv} D={D} P={P} T={T} {sched}: {plan.describe()}")
    o, lse = run(plan, prob, dev)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.decode(prob)
    compare(o, lse, ref_o, ref_l, what=f"hnd {kv} {sched}")


def test_read_only_and_canaries():
    """Inputs bit-identical after the call; nothing written outside o and lse."""
    s = spec(name="ro", batch=4, q_per_seq=2, num_qo_heads=8, num_kv_heads=4, head_dim=128,
             page_size=16, lens=("list", (5, 300, 2500, 64)))
    prob = workloads.generate(s, 8)
    dev = to_dev(prob)
    before = {k: (v.clone() if v is not None else None) for k, v in dev.items()}
    plan = make_plan(prob, force_blocks_per_split=2)
    n = 8 * 8
    canary = torch.full((n * 128 + 2 * 4096,), 12345.0, dtype=torch.float16, device="cuda")
    out = canary[4096:4096 + n * 128].view(8, 8, 128)
    lcan = torch.full((n + 2 * 64,), -7.0, dtype=torch.float32, device="cuda")
    lse = lcan[64:64 + n].view(8, 8)
    run(plan, prob, dev, out=out, lse=lse)
    torch.cuda.synchronize()
    for k, v in dev.items():
        if v is not None:
            assert torch.equal(v.view(torch.uint8) if v.dtype != torch.int32 else v,
                               before[k].view(torch.uint8) if v.dtype != torch.int32 else before[k]), k
    assert torch.all(canary[:4096] == 12345.0) and torch.all(canary[4096 + n * 128:] == 12345.0)
    assert torch.all(lcan[:64] == -7.0) and torch.all(lcan[64 + n:] == -7.0)
    ro, rl = oracle.decode(prob)
    compare(out, lse, ro, rl, what="canaries")


def test_deterministic():
    s = spec(name="det", batch=4, q_per_seq=1, num_qo_heads=32, num_kv_heads=8, head_dim=128,
             page_size=16, lens=("list", (100, 3000, 5000, 9000)))
    prob = workloads.generate(s, 12)
    dev = to_dev(prob)
    plan = make_plan(prob)
    o1, l1 = run(plan, prob, dev)
    o1, l1 = o1.clone(), l1.clone()
    for _ in range(3):
        o2, l2 = run(plan, prob, dev)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_partial_timed_matches_partial():
    """skvd_decode_partial_timed writes what skvd_decode_partial writes, and its kernel-stamped
    events bound a positive duration no longer than a marker pair around the same launch."""
    s = spec(name="timed", batch=4, q_per_seq=1, num_qo_heads=32, num_kv_heads=8, head_dim=128,
             page_size=16, lens=("list", (100, 3000, 5000, 9000)))
    prob = workloads.generate(s, 13)
    dev = to_dev(prob)
    plan = make_plan(prob)
    o1, l1 = run(plan, prob, dev, stage="partial")
    run(plan, prob, dev, out=o1, lse=l1, stage="merge")
    o1, l1 = o1.clone(), l1.clone()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    torch.cuda.synchronize()
    for _ in range(2):
        m0.record()
        o2, l2 = plan.run(dev["q"], dev["k_pages"], dev["v_pages"], dev["page_table"],
                          dev["kv_len"], prob["sm_scale"], stage="partial", events=(e0, e1))
        m1.record()
        run(plan, prob, dev, out=o2, lse=l2, stage="merge")
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
        t_kernel, t_marker = e0.elapsed_time(e1), m0.elapsed_time(m1)
        say(f"  kernel-stamped {t_kernel * 1e3:.1f} us, marker pair {t_marker * 1e3:.1f} us")
        assert 0 < t_kernel <= t_marker * 1.05 + 1e-3
    with pytest.raises(ValueError):
        plan.run(dev["q"], dev["k_pages"], dev["v_pages"], dev["page_table"], dev["kv_len"],
                 prob["sm_scale"], stage="all", events=(e0, e1))


def test_debug_status_clamps():
    """kv_len above max_kv_len and out-of-range page ids are clamped, flagged, never faulted."""
    import quantized_kv_cache_page_amd as skvd
    s = spec(name="dbg", batch=2, q_per_seq=1, num_qo_heads=8, num_kv_heads=2, head_dim=128,
             page_size=16, lens=("list", (100, 200)))
    prob = workloads.generate(s, 6)
    dev = to_dev(prob)
    plan = make_plan(prob, debug=True, max_kv_len=256)
    plan.clear_status()
    dev["kv_len"][1] = 100000  # above max_kv_len: clamped to 256
    t = torch.full((2, 16), -1, dtype=torch.int32, device="cuda")
    t[:, :dev["page_table"].shape[1]] = dev["page_table"]
    t[0, 3] = 10 ** 6          # beyond the pool: clamped into it
    dev["page_table"] = t
    run(plan, prob, dev)
    torch.cuda.synchronize()
    st = plan.status_word()
    assert st & skvd.STATUS_KV_LEN_CLAMPED and st & skvd.STATUS_PAGE_CLAMPED


# ------------------------------------------------------------------ graph capture
def test_graph_capture_replay():
    """First call made under capture; replays equal the eager result bit for bit, with eager
    work between replays; a new plan re-records at a new shape."""
    for lens in ((700, 3000, 20), (64, 128, 4100)):
        s = spec(name="graph", batch=3, q_per_seq=1, num_qo_heads=16, num_kv_heads=4,
                 head_dim=128, page_size=16, lens=("list", lens))
        prob = workloads.generate(s, 21)
        dev = to_dev(prob)
        plan = make_plan(prob)
        plan.ensure_workspace()
        out = torch.empty((3, 16, 128), dtype=torch.float16, device="cuda")
        lse = torch.empty((3, 16), dtype=torch.float32, device="cuda")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run(plan, prob, dev, out=out, lse=lse)
        eo, el = run(plan, prob, dev)
        torch.cuda.synchronize()
        eo, el = eo.clone(), el.clone()
        for i in range(4):
            out.zero_()
            lse.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), eo.view(torch.int16)), f"replay {i}"
            assert torch.equal(lse, el)
            _ = run(plan, prob, dev)  # eager work between replays
        ro, rl = oracle.decode(prob)
        compare(out, lse, ro, rl, what=f"graph {lens}")


# ------------------------------------------------------------------ more than 16 query rows
ROWTILES = [
    # (name, B, T, Hq, Hkv, D, P, kv, lens): G*T > 16 query rows per KV head
    ("g8_t8", 3, 8, 32, 4, 128, 16, "f16", (8, 700, 3000)),        # 64 rows: 4 row tiles
    ("g8_t8_i8", 3, 8, 32, 4, 128, 16, "i8", (8, 700, 3000)),
    ("g8_t8_f8", 3, 8, 32, 4, 128, 16, "f8", (8, 700, 3000)),
    ("g8_t3", 2, 3, 32, 4, 128, 16, "f16", (3, 2100)),              # 24 rows: 2 row tiles
    ("g8_t5_i8", 2, 5, 32, 4, 128, 16, "i8", (5, 2100)),            # 40 rows: a 4th tile idle
    ("g16_t8", 2, 8, 64, 4, 128, 16, "f16", (8, 1500)),             # 128 rows: 2 row groups
    ("g16_t8_i8", 2, 8, 64, 4, 128, 16, "i8", (8, 1500)),
    ("g8_t8_p1", 2, 8, 16, 2, 128, 1, "i8", (9, 400)),              # per-token page lookups
    ("g8_t8_d256", 2, 8, 16, 2, 256, 16, "f16", (8, 1200)),
    ("g8_t8_d256_i8", 2, 8, 16, 2, 256, 16, "i8", (8, 1200)),
    ("g4_t8_d256_f8", 2, 8, 8, 2, 256, 4, "f8", (8, 800)),          # 32 rows at head_dim 256
    ("g8_t8_d192", 2, 8, 16, 2, 192, 16, "f16", (8, 900)),          # 64 rows at head_dim 192
    ("g8_t8_d512_i8", 2, 8, 16, 2, 512, 16, "i8", (8, 700)),        # 64 rows at head_dim 512
    ("g8_t8_q4", 3, 8, 32, 4, 128, 16, "q4", (8, 700, 3000)),
    ("g8_t8_d256_q4", 2, 8, 16, 2, 256, 16, "q4", (8, 1200)),
    ("g32_t1", 2, 1, 64, 2, 128, 16, "f16", (1, 3000)),             # 32 rows from a large group
]


@pytest.mark.parametrize("schedule", ["auto", "static"])
@pytest.mark.parametrize("case", ROWTILES, ids=[c[0] for c in ROWTILES])
def test_row_tiles_all_rows(case, schedule):
    """More than 16 query rows per KV head (large groups, multi-token drafts up to 8 tokens):
    row tiles of 16 rows per wave, several waves per KV head, row groups beyond 64 rows."""
    name, B, T, Hq, Hkv, D, P, kv, lens = case
    s = spec(name=name, batch=B, q_per_seq=T, num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D,
             page_size=P, kv_dtype=kv, lens=("list", lens))
    check(s, seed=zlib.crc32(name.encode()) % 1000, plan_kw=dict(schedule=schedule))
    check(s, seed=zlib.crc32(name.encode()) % 1000 + 1,
          plan_kw=dict(schedule=schedule, force_blocks_per_split=1, force_reducer="multipass"),
          what=f"{name} {schedule} one block per split")


def test_mtp_draft_32q_4kv_t8_all_reducers():
    """The pages' attention shape (32 query / 4 KV heads) with an 8-token draft: every reducer
    and schedule on the same input, each within tolerance."""
    s = spec(name="mtp8", batch=4, q_per_seq=8, num_qo_heads=32, num_kv_heads=4, head_dim=128,
             page_size=16, kv_dtype="i8", lens=("list", (8, 2047, 2049, 5000)), q_mult=2.0)
    for red, bps, sch in [("auto", 0, "auto"), ("direct", 20, "static"),
                          ("cooperative", 2, "static"), ("multipass", 1, "static"),
                          ("hierarchical", 1, "static"), ("multipass", 1, "balanced")]:
        check(s, seed=88, plan_kw=dict(force_reducer=red, force_blocks_per_split=bps,
                                       schedule=sch), what=f"mtp8 {red} bps={bps} {sch}")


# ------------------------------------------------------------------ more than 64 sequences
@pytest.mark.parametrize("B", [65, 128, 256, 1000])
@pytest.mark.parametrize("kv", ["f16", "i8", "q4"])
def test_balanced_large_batch(kv, B):
    """Balanced shares over more than 64 sequences: several sequences per lane of the share
    computation, ragged lengths including empty sequences."""
    rng = np.random.default_rng(B)
    lens = tuple(int(x) for x in rng.integers(0, 700 if B < 1000 else 200, B))
    s = spec(name=f"batch{B}", batch=B, q_per_seq=1, num_qo_heads=32, num_kv_heads=8,
             head_dim=128, page_size=16, kv_dtype=kv, lens=("list", lens))
    # (the plan's own choice for so many short rows is one split per row: the balanced
    # schedule is forced, with one-block shares, to cover the share arithmetic)
    _, _, plan, _, _ = check(s, seed=B, plan_kw=dict(schedule="balanced",
                                                     force_blocks_per_split=1))
    assert plan.schedule == "balanced"


# ------------------------------------------------------------------ the workloads
_WORKLOADS = {}


def workload(cfg):
    """The generated workload (kept for the module: the large ones take seconds to draw)."""
    if cfg not in _WORKLOADS:
        _WORKLOADS[cfg] = workloads.generate(workloads.config(cfg), cfg)
    return _WORKLOADS[cfg]


def test_config1_all_rows():
    check(workloads.config(1), 1)


@pytest.mark.parametrize("qmult", [1, 8])
@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_config_all_rows(cfg, qmult):
    """Every row of the workload, in the benchmark's launch configuration; qmult 8 scales q by
    8 (exact in f16) so that the softmax is peaked and a misread position or a lost bit of a
    logit moves the output beyond the tolerance."""
    prob = dict(workload(cfg))
    if qmult != 1:
        prob["q"] = (prob["q"].astype(np.float32) * qmult).astype(np.float16)
    s = prob["spec"]
    say(f"case config {cfg} ({s.name}) q x{qmult}: L={list(prob['kv_len'])[:8]}...")
    dev = to_dev(prob)
    plan = make_plan(prob, max_kv_len=s.max_kv_len)
    say(f"  {plan.describe()}")
    o, lse = run(plan, prob, dev)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(prob)
    compare(o, lse, ro, rl, what=f"config {cfg} q x{qmult} all {ro.shape[0]} rows")
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("qmult", [1, 8])
def test_q4_batch_all_rows(qmult):
    """The int8 batch's shape (64 sequences, Zipf lengths 512..65536) over a q4_0 cache: every
    row, in the benchmark's launch configuration."""
    key = "q4_batch"
    if key not in _WORKLOADS:
        _WORKLOADS[key] = workloads.generate(workloads.VARIANT_CONFIGS[key], 5)
    prob = dict(_WORKLOADS[key])
    if qmult != 1:
        prob["q"] = (prob["q"].astype(np.float32) * qmult).astype(np.float16)
    s = prob["spec"]
    say(f"case {key} q x{qmult}: L={list(prob['kv_len'])[:8]}...")
    dev = to_dev(prob)
    plan = make_plan(prob, max_kv_len=s.max_kv_len)
    say(f"  {plan.describe()}")
    o, lse = run(plan, prob, dev)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(prob)
    compare(o, lse, ro, rl, what=f"{key} q x{qmult} all {ro.shape[0]} rows")

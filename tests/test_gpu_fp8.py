"""GPU parity of the fp8 cache (OCP E4M3 bytes times one f32 scale per tensor for K and for V)
through the C ABI against the fp64 oracle, which is pinned to torch's float8_e4m3fn decoding.
Every kernel variant the one-byte layout reaches: one query-row quarter (vector P.V, 1 to 8 KV
heads per workgroup), several quarters and head_dim 256 (P.V on the MFMA), page size 1 (per-token
page lookups), one split (o and lse from the partial kernel), the static and balanced schedules,
the full-size int8-batch shape, the raw gather, and scales changed between graph replays.
Tolerances as for the decode: max|do| <= 2e-3, max|dlse| <= 1e-3.
"""
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


def check(s, seed, plan_kw=None, rows=None):
    prob = workloads.generate(s, seed)
    say(f"case {s.name} seed={seed} {plan_kw or ''}: B={s.batch} T={s.q_per_seq} "
        f"Hq={s.num_qo_heads} Hkv={s.num_kv_heads} D={s.head_dim} P={s.page_size} kv=f8 "
        f"L={list(prob['kv_len'])[:8]} k_scale={prob['k_scales'][0]:.4f}")
    dev = to_dev(prob)
    plan = make_plan(prob, **(plan_kw or {}))
    say(f"  {plan.describe()}")
    o, lse = run(plan, prob, dev)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(prob, rows=rows)
    compare(o, lse, ro, rl, rows=rows, what=s.name)
    return prob, dev, plan, o, lse


CASES = [
    # (name, B, T, Hq, Hkv, D, P, lens)
    ("f8_gqa4", 4, 1, 32, 8, 128, 16, (1, 65, 512, 2049)),
    ("f8_p1", 2, 1, 8, 2, 128, 1, (33, 200)),
    ("f8_p4_mha", 3, 1, 8, 8, 128, 4, (5, 64, 257)),
    ("f8_t2_g4", 2, 2, 8, 2, 128, 16, (2, 900)),        # two row quarters: P.V on the MFMA
    ("f8_t4_d256", 2, 4, 8, 4, 256, 16, (4, 600)),
    ("f8_d256_p2", 2, 1, 4, 2, 256, 2, (9, 333)),
    ("f8_g8_t2", 2, 2, 16, 2, 128, 8, (40, 900)),       # 16 rows
    ("f8_short", 1, 1, 8, 8, 128, 16, (100,)),          # one split
]


@pytest.mark.parametrize("schedule", ["auto", "static"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fp8_all_rows(case, schedule):
    name, B, T, Hq, Hkv, D, P, lens = case
    s = workloads.spec(name=name, batch=B, q_per_seq=T, num_qo_heads=Hq, num_kv_heads=Hkv,
                       head_dim=D, page_size=P, kv_dtype="f8", lens=("list", lens))
    check(s, zlib.crc32(name.encode()) % 1000, plan_kw=dict(schedule=schedule))


@pytest.mark.parametrize("hw", [1, 2, 4, 8])
@pytest.mark.parametrize("P", [16, 1])
def test_fp8_heads_per_workgroup(hw, P):
    s = workloads.spec(name="f8_hw", batch=5, q_per_seq=1, num_qo_heads=32, num_kv_heads=8,
                       head_dim=128, page_size=P, kv_dtype="f8", lens=("list", (1, 700, 64, 2100, 333)))
    _, _, plan, _, _ = check(s, hw * 10 + P, plan_kw=dict(heads_per_wg=hw, force_blocks_per_split=2))
    assert plan.info.heads_per_wg == hw


@pytest.mark.parametrize("red", ["direct", "cooperative", "multipass", "hierarchical"])
def test_fp8_reducers(red):
    s = workloads.spec(name=f"f8_{red}", batch=3, q_per_seq=1, num_qo_heads=16, num_kv_heads=4,
                       head_dim=128, page_size=16, kv_dtype="f8", lens=("list", (1, 1000, 3000)))
    check(s, 7, plan_kw=dict(force_reducer=red, force_blocks_per_split=1, schedule="static"))


def test_fp8_int8_batch_shape_sampled():
    """The int8 batch's shape (64 sequences, Zipf lengths up to 65536) with an fp8 cache, in the
    benchmark's launch configuration, on sampled rows."""
    base = workloads.config(5)
    s = workloads.Spec("f8_batch", base.batch, 1, 32, 8, 128, 16, "f8", base.lens)
    prob = workloads.generate(s, 5)
    dev = to_dev(prob)
    plan = make_plan(prob, max_kv_len=s.max_kv_len)
    say(f"case f8_batch: {plan.describe()}")
    o, lse = run(plan, prob, dev)
    torch.cuda.synchronize()
    total = prob["q"].shape[0] * prob["q"].shape[1]
    rows = np.unique(np.concatenate([np.random.default_rng(5).choice(total, 96, replace=False),
                                     [0, total - 1]]))
    ro, rl = oracle.decode(prob, rows=rows)
    compare(o, lse, ro, rl, rows=rows, what="f8_batch sampled")
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_fp8_gather_bit_exact():
    for P in (16, 1, 64):
        s = workloads.spec(name="f8_gather", batch=3, q_per_seq=1, num_qo_heads=4, num_kv_heads=2,
                           head_dim=128, page_size=P, kv_dtype="f8", lens=("list", (1, 190, 700)))
        prob = workloads.generate(s, 5)
        dev = to_dev(prob)
        plan = make_plan(prob)
        maxl = int(prob["kv_len"].max())
        dk, dv, dks, dvs = plan.gather_debug(dev["q"], dev["k_pages"], dev["v_pages"],
                                             dev["page_table"], dev["kv_len"], maxl,
                                             dev["k_scales"], dev["v_scales"])
        ok, ov, _, _ = oracle.gather(prob, maxl)
        assert dks is None and dvs is None
        assert np.array_equal(dk.cpu().numpy(), ok) and np.array_equal(dv.cpu().numpy(), ov)
        say(f"  gather f8 P={P}: bit-exact")


def test_fp8_scales_read_at_each_replay():
    """The tensor scales are read on the device at each call: a graph captured once follows
    new k_scale / v_scale values written into the same one-element tensors."""
    s = workloads.spec(name="f8_graph", batch=3, q_per_seq=1, num_qo_heads=16, num_kv_heads=4,
                       head_dim=128, page_size=16, kv_dtype="f8", lens=("list", (700, 3000, 20)))
    prob = workloads.generate(s, 21)
    dev = to_dev(prob)
    plan = make_plan(prob)
    plan.ensure_workspace()
    out = torch.empty((3, 16, 128), dtype=torch.float16, device="cuda")
    lse = torch.empty((3, 16), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(plan, prob, dev, out=out, lse=lse)
    k0, v0 = float(prob["k_scales"][0]), float(prob["v_scales"][0])
    # new scales near the drawn ones (outputs stay N(0,1)-sized, as the tolerance assumes)
    for i, (ks, vs) in enumerate(((3 * k0, 0.5 * v0), (0.25 * k0, v0), (k0, 0.75 * v0))):
        ks, vs = float(np.float32(ks)), float(np.float32(vs))
        dev["k_scales"].fill_(ks)
        dev["v_scales"].fill_(vs)
        g.replay()
        torch.cuda.synchronize()
        p = dict(prob, k_scales=np.array([ks], np.float32), v_scales=np.array([vs], np.float32))
        ro, rl = oracle.decode(p)
        compare(out, lse, ro, rl, what=f"replay {i} k_scale={ks:.5f} v_scale={vs:.5f}")
        torch.ones(1 << 20, device="cuda").sum()  # eager work between replays


def test_fp8_deterministic_and_read_only():
    s = workloads.spec(name="f8_det", batch=4, q_per_seq=1, num_qo_heads=32, num_kv_heads=8,
                       head_dim=128, page_size=16, kv_dtype="f8", lens=("list", (10, 3000, 700, 64)))
    prob, dev, plan, o1, l1 = check(s, 31)
    before = [dev[k].clone() for k in ("k_pages", "v_pages", "k_scales", "v_scales")]
    o2, l2 = run(plan, prob, dev)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for b, k in zip(before, ("k_pages", "v_pages", "k_scales", "v_scales")):
        assert torch.equal(b, dev[k]), k


@pytest.mark.parametrize("route", ["decode", "prefill"])
def test_fp8_scale_edges(route):
    """Tensor scales that are negative (the scores change sign: on the multi-token route the
    sign is carried by q) or zero (k_scale 0: uniform weights; v_scale 0: o = 0)."""
    T = 2 if route == "decode" else 24
    s = workloads.spec(name=f"f8_edges_{route}", batch=2, q_per_seq=T, num_qo_heads=8,
                       num_kv_heads=2, head_dim=128, page_size=16, kv_dtype="f8",
                       lens=("list", (T, 700)))
    prob = workloads.generate(s, 41)
    k0, v0 = float(prob["k_scales"][0]), float(prob["v_scales"][0])
    for ks, vs in ((-k0, v0), (0.0, v0), (k0, 0.0), (-2 * k0, -v0)):
        p = dict(prob, k_scales=np.array([ks], np.float32), v_scales=np.array([vs], np.float32))
        dev = to_dev(p)
        plan = make_plan(p, max_q_per_seq=T if route == "decode" else 1)
        args = (dev["q"], dev["k_pages"], dev["v_pages"], dev["page_table"], dev["kv_len"],
                p["sm_scale"], dev["k_scales"], dev["v_scales"])
        o, lse = (plan.run if route == "decode" else plan.prefill)(*args, q_per_seq=T)
        torch.cuda.synchronize()
        ro, rl = oracle.decode(p)
        compare(o, lse, ro, rl, what=f"{route} k_scale={ks:.4f} v_scale={vs:.4f}")
        if vs == 0.0:
            assert not o.float().abs().max().item()

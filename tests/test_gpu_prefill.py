"""GPU parity of the multi-token (prefill) route: the MFMA tile kernel through the C ABI against
the fp64 oracle, whose causal reading (token t of T sees positions j <= kv_len - T + t) is the
decode's and is pinned at long T against torch's SDPA. Tolerances as for the decode: max|do| <=
2e-3, max|dlse| <= 1e-3.
"""
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


def prefill(plan, prob, dev, out=None, lse=None):
    return plan.prefill(dev["q"], dev["k_pages"], dev["v_pages"], dev["page_table"],
                        dev["kv_len"], prob["sm_scale"], dev["k_scales"], dev["v_scales"],
                        out=out, lse=lse, q_per_seq=int(prob["q_per_seq"]))


def check(s, seed, rows=None):
    prob = workloads.generate(s, seed)
    say(f"case {s.name}: B={s.batch} T={s.q_per_seq} Hq={s.num_qo_heads} Hkv={s.num_kv_heads} "
        f"D={s.head_dim} P={s.page_size} kv={s.kv_dtype} L={list(prob['kv_len'])[:8]}")
    dev = to_dev(prob)
    plan = make_plan(prob, max_q_per_seq=1)  # the prefill route is not bounded by max_q_per_seq
    o, lse = prefill(plan, prob, dev)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(prob, rows=rows)
    compare(o, lse, ro, rl, rows=rows, what=s.name)
    return prob, dev, plan, o, lse


CASES = [
    # (name, B, T, Hq, Hkv, D, P, kv, lens)
    ("gqa4_full_causal", 2, 37, 8, 2, 128, 16, "f16", (37, 300)),
    ("gqa4_i8", 1, 100, 32, 8, 128, 16, "i8", (1000,)),
    ("mha_p1", 3, 9, 4, 4, 128, 1, "f16", (9, 64, 129)),
    ("gqa8_d256", 2, 64, 16, 2, 256, 16, "f16", (64, 500)),
    ("mha_d256_i8_p4", 2, 50, 8, 8, 256, 4, "i8", (50, 777)),
    ("gqa16", 1, 20, 32, 2, 128, 16, "f16", (700,)),
    ("gqa4_t1", 2, 1, 8, 2, 128, 16, "f16", (1, 200)),
    ("gqa4_i8_p64_ragged", 4, 70, 16, 4, 128, 64, "i8", (70, 71, 135, 2049)),
    ("gqa2_many_tiles", 1, 300, 8, 4, 128, 16, "f16", (4100,)),
    ("gqa4_f8", 2, 100, 32, 8, 128, 16, "f8", (100, 1000)),
    ("gqa8_d256_f8_p4", 2, 50, 16, 2, 256, 4, "f8", (50, 777)),
    ("mha_f8_p1_ragged", 3, 40, 4, 4, 128, 1, "f8", (40, 41, 300)),
    ("gqa4_q4", 2, 100, 32, 8, 128, 16, "q4", (100, 1000)),
    ("mha_d256_q4_p4", 2, 50, 8, 8, 256, 4, "q4", (50, 777)),
    ("gqa8_q4_p64_ragged", 3, 70, 32, 4, 128, 64, "q4", (70, 71, 2049)),
    ("mha_f16_p16", 2, 150, 8, 8, 128, 16, "f16", (150, 900)),
    ("g3_f16_p16", 2, 50, 12, 4, 128, 16, "f16", (50, 700)),
    ("g64_f16_p16", 1, 20, 64, 1, 128, 16, "f16", (300,)),
    ("g3_d256_f16_p32", 2, 33, 6, 2, 256, 32, "f16", (33, 400)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_matches_oracle(case):
    name, B, T, Hq, Hkv, D, P, kv, lens = case
    s = workloads.spec(name=name, batch=B, q_per_seq=T, num_qo_heads=Hq, num_kv_heads=Hkv,
                       head_dim=D, page_size=P, kv_dtype=kv, lens=("list", lens))
    check(s, 61)


def test_prefill_rows_without_positions():
    """kv_len below T (a contract violation): rows that see no position get o = 0, lse = -inf."""
    s = workloads.spec(name="short", batch=2, q_per_seq=8, num_qo_heads=8, num_kv_heads=2,
                       head_dim=128, page_size=16, kv_dtype="f16", lens=("list", (5, 40)))
    prob, dev, plan, o, lse = check(s, 62)
    ls = lse.cpu().numpy().reshape(2, 8, 8)
    assert np.isneginf(ls[0, :3]).all() and np.isfinite(ls[0, 3:]).all()
    assert (o.reshape(2, 8, 8, 128)[0, :3] == 0).all()


@pytest.mark.parametrize("kv", ["i8", "f8", "q4"])
def test_prefill_equals_decode_route(kv):
    """For T <= 8 both routes compute the same attention: each matches the oracle, and they agree
    with each other within the tolerance."""
    s = workloads.spec(name=f"routes_{kv}", batch=3, q_per_seq=4, num_qo_heads=16, num_kv_heads=4,
                       head_dim=128, page_size=16, kv_dtype=kv, lens=("list", (4, 900, 3000)))
    prob, dev, plan, o1, l1 = check(s, 63)
    plan2 = make_plan(prob)
    o2, l2 = run(plan2, prob, dev)
    torch.cuda.synchronize()
    assert float((o1.float() - o2.float()).abs().max()) <= 2e-3
    assert float((l1 - l2).abs().max()) <= 1e-3


@pytest.mark.parametrize("kv,P", [("f16", 16), ("f16", 64), ("i8", 16), ("f8", 16),
                                  ("q4", 16)])
def test_prefill_hnd_pools(kv, P):
    """The multi-token route over HND pools (each KV head's page rows contiguous, passed as the
    permuted view): f16 copies tiles into LDS through the HND strides, the one-byte formats load
    and widen them."""
    s = workloads.spec(name=f"pf_hnd_{kv}", batch=2, q_per_seq=70, num_qo_heads=32,
                       num_kv_heads=8, head_dim=128, page_size=P, kv_dtype=kv,
                       lens=("list", (70, 2100)))
    prob = workloads.generate(s, 93)
    dev = to_dev(prob, layout="hnd")
    plan = make_plan(prob, max_q_per_seq=1)
    o, lse = prefill(plan, prob, dev)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(prob)
    compare(o, lse, ro, rl, what=f"prefill hnd {kv} P={P}")


@pytest.mark.parametrize("kv", ["f16", "i8", "q4"])
@pytest.mark.parametrize("form", ["halves", "interleaved", "layer"])
def test_prefill_cache_views(kv, form):
    """The multi-token route with K and V as views of one tensor (the halves of [2, pages, ...],
    the interleaved [pages, 2, ...], layer 1 of a [layers, 2, pages, ...] pool): addressed
    through the views' strides alone (f16: the copies into LDS), the result matches the oracle
    and the tensor keeps its bytes."""
    s = workloads.spec(name=f"pf_views_{form}_{kv}", batch=2, q_per_seq=40, num_qo_heads=16,
                       num_kv_heads=4, head_dim=128, page_size=16, kv_dtype=kv,
                       lens=("list", (40, 1500)))
    prob = workloads.generate(s, 95)

    def combined(k, v):
        if k is None:
            return None, None, None
        if form == "halves":
            big = np.stack([k, v])                       # [2, N, P, H, X]
            return big, big[0], big[1]
        if form == "interleaved":
            big = np.ascontiguousarray(np.stack([k, v], axis=1))  # [N, 2, P, H, X]
            return big, big[:, 0], big[:, 1]
        big = np.stack([np.stack([v, k]), np.stack([k, v])])     # [layers=2, 2, N, P, H, X]
        return big, big[1, 0], big[1, 1]

    def dev_view(t, npview, base):
        off = (npview.__array_interface__["data"][0] - base.__array_interface__["data"][0])
        st = [x // npview.itemsize for x in npview.strides]
        return torch.as_strided(t, npview.shape, st, off // npview.itemsize)

    bkv, kview, vview = combined(prob["k_pages"], prob["v_pages"])
    bsc, ksview, vsview = combined(prob["k_scales"], prob["v_scales"])
    tk = torch.from_numpy(bkv).cuda()
    ts = None if bsc is None else torch.from_numpy(bsc).cuda()
    dev = to_dev(prob)
    dev["k_pages"], dev["v_pages"] = dev_view(tk, kview, bkv), dev_view(tk, vview, bkv)
    if ts is not None:
        dev["k_scales"], dev["v_scales"] = dev_view(ts, ksview, bsc), dev_view(ts, vsview, bsc)
    before = tk.clone()
    plan = make_plan(prob, max_q_per_seq=1)
    o, lse = prefill(plan, prob, dev)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(prob)
    compare(o, lse, ro, rl, what=f"prefill views {form} {kv}")
    assert torch.equal(tk.view(torch.uint8), before.view(torch.uint8))


@pytest.mark.parametrize("kv", ["f16", "i8"])
def test_prefill_strided_q_unequal_pools_read_only(kv):
    """q sliced from a fused QKV buffer (token stride > Hq*D), a K pool longer than the V pool
    (only indexed pages are read), outputs inside larger canary buffers: o and lse match the
    oracle, every input and every canary keeps its bytes."""
    s = workloads.spec(name=f"pf_strided_{kv}", batch=3, q_per_seq=24, num_qo_heads=16,
                       num_kv_heads=4, head_dim=128, page_size=16, kv_dtype=kv,
                       lens=("list", (24, 500, 1300)), spare_frac=0.0)
    prob = workloads.generate(s, 97)
    ro, rl = oracle.decode(prob)
    dev = to_dev(prob)
    rows = dev["q"].shape[0]
    qkv = torch.randn((rows, 16 + 8, 128), device="cuda").to(torch.float16)
    qkv[:, :16] = dev["q"]
    dev["q"] = qkv[:, :16]
    extra = torch.full((5,) + tuple(dev["k_pages"].shape[1:]), 0x7F, dtype=torch.uint8,
                       device="cuda").view(dev["k_pages"].dtype) if kv != "f16" else \
        torch.full((5,) + tuple(dev["k_pages"].shape[1:]), float("nan"), dtype=torch.float16,
                   device="cuda")
    dev["k_pages"] = torch.cat([dev["k_pages"], extra])  # K pool longer than V pool
    inputs = {k: v.clone() for k, v in dev.items() if v is not None}
    qkv_before = qkv.clone()
    o_buf = torch.full((rows + 2, 16, 128), 7.0, dtype=torch.float16, device="cuda")
    l_buf = torch.full((rows + 2, 16), 7.0, dtype=torch.float32, device="cuda")
    o, lse = o_buf[1:-1], l_buf[1:-1]
    plan = make_plan(prob, max_q_per_seq=1)
    prefill(plan, prob, dev, out=o, lse=lse)
    torch.cuda.synchronize()
    compare(o, lse, ro, rl, what=f"prefill strided {kv}")
    for k, v in inputs.items():
        assert torch.equal(dev[k].view(torch.uint8), v.view(torch.uint8)), k
    assert torch.equal(qkv.view(torch.uint8), qkv_before.view(torch.uint8))
    assert torch.all(o_buf[0] == 7.0) and torch.all(o_buf[-1] == 7.0)
    assert torch.all(l_buf[0] == 7.0) and torch.all(l_buf[-1] == 7.0)


def test_prefill_deterministic():
    s = workloads.spec(name="det", batch=2, q_per_seq=33, num_qo_heads=8, num_kv_heads=2,
                       head_dim=128, page_size=16, kv_dtype="f16", lens=("list", (33, 500)))
    prob, dev, plan, o1, l1 = check(s, 64)
    o2, l2 = prefill(plan, prob, dev)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("kv", ["i8", "f16", "q4"])
def test_prefill_graph_capture_replay(kv):
    """Replays of a captured multi-token call (f16: the kernel that copies tiles straight into
    LDS; int8 / q4_0: the register-staged one) match the oracle and each other bit for bit,
    with eager work between the replays."""
    s = workloads.spec(name=f"graph_prefill_{kv}", batch=2, q_per_seq=40, num_qo_heads=8,
                       num_kv_heads=2, head_dim=128, page_size=16, kv_dtype=kv,
                       lens=("list", (40, 1000)))
    prob = workloads.generate(s, 65)
    dev = to_dev(prob)
    plan = make_plan(prob, max_q_per_seq=1)
    out = torch.empty(dev["q"].shape, dtype=torch.float16, device="cuda")
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        prefill(plan, prob, dev, out=out, lse=lse)
    ro, rl = oracle.decode(prob)
    ref = None
    for i in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        compare(out, lse, ro, rl, what=f"replay {i}")
        if ref is None:
            ref = (out.clone(), lse.clone())
        else:
            assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1])
        torch.ones(1 << 20, device="cuda").sum()


@pytest.mark.parametrize("name", sorted(workloads.PREFILL_CONFIGS))
def test_prefill_workloads_sampled(name):
    """The benchmark's prefill workloads at full size, in its launch configuration, on 256
    sampled rows (spread over sequences, tokens and heads, incl. the first and last token)."""
    s = workloads.PREFILL_CONFIGS[name]
    rng = np.random.default_rng(66)
    total = s.batch * s.q_per_seq * s.num_qo_heads
    rows = np.unique(np.concatenate([rng.integers(0, total, 250),
                                     [0, s.num_qo_heads - 1, total - 1,
                                      (s.q_per_seq - 1) * s.num_qo_heads]]))
    check(s, 67, rows=rows)


def test_prefill_long_prompt_sampled():
    """One 8192-token prompt over its own 8192 positions (128 KV tiles for the last query tile),
    and a ragged batch whose pair count is not a multiple of 8 (the other work order)."""
    s = workloads.spec(name="long_prompt", batch=1, q_per_seq=8192, num_qo_heads=32,
                       num_kv_heads=8, head_dim=128, page_size=16, kv_dtype="f16",
                       lens=("list", (8192,)))
    rng = np.random.default_rng(68)
    total = 8192 * 32
    rows = np.unique(np.concatenate([rng.integers(0, total, 200), [0, total - 1]]))
    check(s, 69, rows=rows)
    s = workloads.spec(name="odd_pairs", batch=3, q_per_seq=300, num_qo_heads=6, num_kv_heads=3,
                       head_dim=128, page_size=16, kv_dtype="i8", lens=("list", (300, 1000, 700)))
    check(s, 70)


@pytest.mark.parametrize("kv", ["i8", "f8", "q4"])
def test_attention_routing(kv):
    """skvd_attention: T = 4 takes the decode (bit-identical to run()), T = 40 the tiled route
    (bit-identical to prefill())."""
    for T, lens in ((4, (4, 900, 3000)), (40, (40, 900, 3000))):
        s = workloads.spec(name=f"route_T{T}_{kv}", batch=3, q_per_seq=T, num_qo_heads=16,
                           num_kv_heads=4, head_dim=128, page_size=16, kv_dtype=kv,
                           lens=("list", lens))
        prob = workloads.generate(s, 76)
        dev = to_dev(prob)
        plan = make_plan(prob, max_q_per_seq=min(T, 4))
        args = (dev["q"], dev["k_pages"], dev["v_pages"], dev["page_table"], dev["kv_len"],
                prob["sm_scale"], dev["k_scales"], dev["v_scales"])
        o1, l1 = plan.attend(*args, q_per_seq=T)
        o2, l2 = (plan.run if T <= 4 else plan.prefill)(*args, q_per_seq=T)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), T
        ro, rl = oracle.decode(prob)
        compare(o1, l1, ro, rl, what=f"attend T={T}")


@pytest.mark.parametrize("scale", [-0.08, 0.0])
def test_prefill_scale_sign(scale):
    """A negative softmax scale (carried by q) and a zero scale (uniform weights)."""
    s = workloads.spec(name="scale", batch=2, q_per_seq=24, num_qo_heads=8, num_kv_heads=2,
                       head_dim=128, page_size=16, kv_dtype="f16", lens=("list", (24, 300)))
    prob = dict(workloads.generate(s, 77), sm_scale=float(np.float32(scale)))
    dev = to_dev(prob)
    plan = make_plan(prob, max_q_per_seq=1)
    o, lse = prefill(plan, prob, dev)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(prob)
    compare(o, lse, ro, rl, what=f"scale {scale}")

"""GPU parity of the append (new K/V rows into the paged cache, int8 quantized on write): the HIP
kernel through the C ABI against the oracle's append on the same seeded inputs.

Append is byte work (f16 rows copied, int8 codes and f16 scales decided in f32 on both sides),
so every comparison is bit-exact over the whole pools, written slots and untouched ones alike.
The decode over an appended cache is compared with the fp64 oracle at the decode's tolerance.
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


def _dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _pool_dev(x, layout):
    """A pool [N, P, Hkv, X] on the device in NHD (as given) or HND memory order (the same
    logical view over [N, Hkv, P, X] storage)."""
    if x is None:
        return None
    if layout == "nhd" or x.ndim != 4:  # (fp8 scales: one f32 per tensor)
        return torch.from_numpy(x).cuda()
    return torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))).cuda().permute(0, 2, 1, 3)


def gpu_append(plan, prob, new, layout="nhd", batch=None, table=None):
    """Append on the GPU into device copies of the problem's pools; returns them on the host."""
    k = _pool_dev(prob["k_pages"], layout)
    v = _pool_dev(prob["v_pages"], layout)
    ks = _pool_dev(prob["k_scales"], layout)
    vs = _pool_dev(prob["v_scales"], layout)
    tab = _dev(prob["page_table"] if table is None else table)
    plan.append(_dev(new["k_new"]), _dev(new["v_new"]), _dev(new["batch_idx"]),
                _dev(new["positions"]), k, v, tab, ks, vs, batch=batch)
    torch.cuda.synchronize()
    return [None if t is None else t.cpu().numpy() for t in (k, v, ks, vs)]


def oracle_append(prob, new, max_len, batch=None, table=None):
    k, v, ks, vs, _ = oracle.append(new["k_new"], new["v_new"], new["batch_idx"],
                                    new["positions"],
                                    prob["page_table"] if table is None else table, max_len,
                                    prob["k_pages"], prob["v_pages"], prob["k_scales"],
                                    prob["v_scales"], batch=batch)
    return [k, v, ks, vs]


def assert_pools_equal(got, want, what):
    for name, g, w in zip(("K", "V", "K scales", "V scales"), got, want):
        if w is None:
            assert g is None
            continue
        gb, wb = np.ascontiguousarray(g).view(np.uint8), np.ascontiguousarray(w).view(np.uint8)
        bad = int((gb != wb).sum())
        assert bad == 0, f"{what}: {name} differs in {bad} bytes"
    say(f"  {what}: pools bit-identical")


CASES = [
    # (name, B, Hkv, D, P, kv, lens, new per sequence, layout)
    ("f16_d128_p16", 3, 8, 128, 16, "f16", (17, 300, 64), 40, "nhd"),
    ("f16_d256_p1", 2, 2, 256, 1, "f16", (9, 130), 130, "nhd"),
    ("f16_d128_p64_hnd", 3, 4, 128, 64, "f16", (1, 200, 129), 70, "hnd"),
    ("i8_d128_p16", 4, 8, 128, 16, "i8", (1, 65, 512, 33), 64, "nhd"),
    ("i8_d256_p4", 2, 2, 256, 4, "i8", (7, 300), 300, "nhd"),
    ("i8_d128_p1_mha", 2, 1, 128, 1, "i8", (50, 3), 50, "nhd"),
    ("i8_d128_p16_hnd", 3, 8, 128, 16, "i8", (40, 16, 100), 25, "hnd"),
    ("f8_d128_p16", 3, 8, 128, 16, "f8", (17, 300, 64), 40, "nhd"),
    ("f8_d256_p1", 2, 2, 256, 1, "f8", (9, 130), 130, "nhd"),
    ("f8_d128_p64_hnd", 3, 4, 128, 64, "f8", (1, 200, 129), 70, "hnd"),
    ("f16_d192_p16", 2, 4, 192, 16, "f16", (17, 300), 40, "nhd"),
    ("f8_d192_p4", 2, 2, 192, 4, "f8", (9, 130), 60, "nhd"),
    ("f16_d512_p16", 2, 2, 512, 16, "f16", (17, 300), 40, "nhd"),
    ("i8_d512_p16", 2, 4, 512, 16, "i8", (1, 65, 200)[:2], 64, "nhd"),
    ("f8_d512_p1", 2, 2, 512, 1, "f8", (9, 130), 130, "nhd"),
    ("q4_d128_p16", 4, 8, 128, 16, "q4", (1, 65, 512, 33), 64, "nhd"),
    ("q4_d256_p4", 2, 2, 256, 4, "q4", (7, 300), 300, "nhd"),
    ("q4_d128_p1_mha", 2, 1, 128, 1, "q4", (50, 3), 50, "nhd"),
    ("q4_d128_p16_hnd", 3, 8, 128, 16, "q4", (40, 16, 100), 25, "hnd"),
    ("q4_d512_p16", 2, 4, 512, 16, "q4", (1, 65), 64, "nhd"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_append_matches_oracle(case):
    name, B, Hkv, D, P, kv, lens, n, layout = case
    s = workloads.spec(name=name, batch=B, num_qo_heads=2 * Hkv, num_kv_heads=Hkv, head_dim=D,
                       page_size=P, kv_dtype=kv, lens=("list", lens))
    prob = workloads.generate(s, 31)
    new = workloads.append_tokens(prob, 31, n)
    say(f"case {name}: N={new['k_new'].shape[0]} B={B} Hkv={Hkv} D={D} P={P} {kv} {layout}")
    plan = make_plan(prob)
    got = gpu_append(plan, prob, new, layout)
    want = oracle_append(prob, new, plan.params.max_kv_len)
    assert_pools_equal(got, want, name)


def test_append_special_values():
    """Groups that stress the int8 rule: exact multiples of powers of two, quotients halfway
    between integers, all-zero groups, groups whose scale underflows f16, f16 subnormals,
    values near f16's maximum, and NaN and infinite elements."""
    B, Hkv, D, P = 1, 2, 128, 16
    s = workloads.spec(name="special", batch=B, num_qo_heads=4, num_kv_heads=Hkv, head_dim=D,
                       page_size=P, kv_dtype="i8", lens=("list", (64,)))
    prob = workloads.generate(s, 32)
    rng = np.random.default_rng(32)
    N = 64
    x = np.zeros((N, Hkv, D // 32, 32), np.float64)
    for i in range(N):
        for h in range(Hkv):
            for g in range(D // 32):
                kind = (i * 7 + h * 3 + g) % 8
                c = rng.integers(-127, 128, size=32).astype(np.float64)
                if kind == 0:    # exact: c * 2^e with |c| = 127 present
                    c[rng.integers(32)] = 127
                    x[i, h, g] = c * 2.0 ** rng.integers(-12, 3)
                elif kind == 1:  # halfway quotients at scale 1
                    x[i, h, g] = np.round(c) + 0.5
                    x[i, h, g, 0] = 127
                elif kind == 2:  # all zero
                    x[i, h, g] = 0
                elif kind == 3:  # scale below f16's range
                    x[i, h, g] = 0
                    x[i, h, g, 3] = 2.0 ** -24
                elif kind == 4:  # subnormal inputs
                    x[i, h, g] = c * 2.0 ** -24
                elif kind == 5:  # near f16's maximum
                    x[i, h, g] = rng.uniform(-65504, 65504, 32)
                elif kind == 6:  # wide dynamic range in one group
                    x[i, h, g] = rng.standard_normal(32) * 10.0 ** rng.uniform(-4, 4, 32)
                else:            # non-finite elements: NaN (left out of the maximum, code 0),
                    x[i, h, g] = c  # and on odd tokens an infinity (scale inf, codes 0)
                    x[i, h, g, int(rng.integers(32))] = np.nan
                    if i % 2:
                        x[i, h, g, int(rng.integers(32))] = np.inf * (1 if h else -1)
    kn = x.reshape(N, Hkv, D).astype(np.float16)
    vn = (-x[:, ::-1]).reshape(N, Hkv, D).astype(np.float16)
    new = dict(k_new=kn, v_new=np.ascontiguousarray(vn), batch_idx=np.zeros(N, np.int32),
               positions=rng.permutation(64).astype(np.int32))
    plan = make_plan(prob)
    got = gpu_append(plan, prob, new)
    want = oracle_append(prob, new, plan.params.max_kv_len)
    assert_pools_equal(got, want, "special values")


def test_append_q4_special_values():
    """Groups that stress the q4_0 rule: grids of the rule (k * d with k = -8 at the extreme,
    either sign of d), quotients x / d exactly halfway between integers (8.5 - x / |d| rounding
    up), magnitude ties between elements of opposite sign (the first one wins), all-zero
    groups (scale -0), f16 subnormals, values near f16's maximum, wide dynamic ranges, and NaN
    and infinite elements."""
    B, Hkv, D, P = 1, 2, 128, 16
    s = workloads.spec(name="special_q4", batch=B, num_qo_heads=4, num_kv_heads=Hkv, head_dim=D,
                       page_size=P, kv_dtype="q4", lens=("list", (64,)))
    prob = workloads.generate(s, 39)
    rng = np.random.default_rng(39)
    N = 64
    x = np.zeros((N, Hkv, D // 32, 32), np.float64)
    for i in range(N):
        for h in range(Hkv):
            for g in range(D // 32):
                kind = (i * 7 + h * 3 + g) % 8
                k = rng.integers(-7, 8, size=32).astype(np.float64)
                sgn = 1.0 if rng.random() < 0.5 else -1.0
                if kind == 0:    # on the grid: k * d, the extreme -8 * d
                    k[rng.integers(32)] = -8
                    x[i, h, g] = k * sgn * 2.0 ** rng.integers(-12, 3)
                elif kind == 1:  # halfway quotients: m = 8 (d = -1), x = k + 0.5
                    x[i, h, g] = np.clip(k, -8, 6) + 0.5
                    x[i, h, g, int(rng.integers(32))] = 8 * sgn
                elif kind == 2:  # all zero, or a magnitude tie of opposite signs
                    x[i, h, g] = 0
                    if i % 2:
                        a, b = rng.choice(32, 2, replace=False)
                        x[i, h, g, a], x[i, h, g, b] = 3.0, -3.0
                elif kind == 3:  # subnormal inputs
                    x[i, h, g] = k * 2.0 ** -24
                elif kind == 4:  # near f16's maximum
                    x[i, h, g] = rng.uniform(-65504, 65504, 32)
                elif kind == 5:  # wide dynamic range in one group
                    x[i, h, g] = rng.standard_normal(32) * 10.0 ** rng.uniform(-4, 4, 32)
                elif kind == 6:  # N(0, 1)
                    x[i, h, g] = rng.standard_normal(32)
                else:            # non-finite: NaN (left out of the maximum, code 8), and on
                    x[i, h, g] = k  # odd tokens an infinity (scale -+inf, codes 8)
                    x[i, h, g, int(rng.integers(32))] = np.nan
                    if i % 2:
                        x[i, h, g, int(rng.integers(32))] = np.inf * (1 if h else -1)
    kn = x.reshape(N, Hkv, D).astype(np.float16)
    vn = (-x[:, ::-1]).reshape(N, Hkv, D).astype(np.float16)
    new = dict(k_new=kn, v_new=np.ascontiguousarray(vn), batch_idx=np.zeros(N, np.int32),
               positions=rng.permutation(64).astype(np.int32))
    plan = make_plan(prob)
    got = gpu_append(plan, prob, new)
    want = oracle_append(prob, new, plan.params.max_kv_len)
    assert_pools_equal(got, want, "q4_0 special values")


@pytest.mark.parametrize("scale", [2.0 ** -6, 3.0 / 16])
def test_append_fp8_special_values(scale):
    """The fp8 rule at its edges: every E4M3 magnitude and every midpoint between neighbours
    (exact ties when the scale is a power of two), one f16 step either side, values past 448 *
    scale (saturation), zeros of both signs, f16 subnormals, NaN (stores 0) and infinities
    (saturate)."""
    B, Hkv, D, P = 1, 2, 128, 16
    s = workloads.spec(name="special_f8", batch=B, num_qo_heads=4, num_kv_heads=Hkv, head_dim=D,
                       page_size=P, kv_dtype="f8", lens=("list", (64,)))
    prob = workloads.generate(s, 37)
    prob = dict(prob, k_scales=np.array([scale], np.float32),
                v_scales=np.array([scale * 1.25], np.float32))
    mags = oracle.e4m3_to_float(np.arange(0x7F, dtype=np.uint8))
    mid = (mags[:-1] + mags[1:]) / 2
    base = np.concatenate([mags, mid]) * scale
    h = base.astype(np.float16)
    vals = np.concatenate([h, -h, np.nextafter(h, np.float16(np.inf)),
                           np.nextafter(h, np.float16(0)),
                           np.array([0.0, -0.0, 500 * scale, -600 * scale, 65504, -65504,
                                     2.0 ** -24, -3 * 2.0 ** -24, 2.0 ** -14, np.nan, np.inf,
                                     -np.inf, -np.nan], np.float16)])
    rng = np.random.default_rng(37)
    N = 64
    x = np.resize(rng.permutation(vals), 2 * N * Hkv * D).astype(np.float16)
    kn = x[:N * Hkv * D].reshape(N, Hkv, D)
    vn = x[N * Hkv * D:].reshape(N, Hkv, D)
    new = dict(k_new=kn, v_new=vn, batch_idx=np.zeros(N, np.int32),
               positions=rng.permutation(64).astype(np.int32))
    plan = make_plan(prob)
    got = gpu_append(plan, prob, new)
    want = oracle_append(prob, new, plan.params.max_kv_len)
    assert_pools_equal(got, want, f"fp8 special values, scale {scale}")


def test_append_skips_invalid_tokens():
    """Tokens naming a sequence outside [0, batch), a position outside [0, max_kv_len), or a page
    id outside the pool write nothing (the kernel's own bounds checks); the rest are written."""
    s = workloads.spec(name="skips", batch=3, num_qo_heads=8, num_kv_heads=4, head_dim=128,
                       page_size=16, kv_dtype="i8", lens=("list", (40, 64, 20)))
    prob = workloads.generate(s, 33)
    new = workloads.append_tokens(prob, 33, 20)
    N = new["k_new"].shape[0]
    bi, pos = new["batch_idx"].copy(), new["positions"].copy()
    bi[0], bi[1], pos[2], pos[3] = -1, 3, -7, 64  # 64 = max_kv_len of the plan below
    table = prob["page_table"].copy()
    table[2, 0] = prob["k_pages"].shape[0]        # one past the pool
    table[2, 1] = -3
    new = dict(new, batch_idx=bi, positions=pos)
    plan = make_plan(prob, max_kv_len=64)
    got = gpu_append(plan, prob, new, table=table)
    want = oracle_append(prob, new, 64, table=table)
    say(f"  N={N}")
    assert_pools_equal(got, want, "skips")


def test_append_empty_launches_nothing():
    s = workloads.spec(name="empty", batch=1, num_qo_heads=2, num_kv_heads=1, head_dim=128,
                       page_size=16, kv_dtype="f16", lens=("list", (32,)))
    prob = workloads.generate(s, 34)
    new = dict(k_new=np.zeros((0, 1, 128), np.float16), v_new=np.zeros((0, 1, 128), np.float16),
               batch_idx=np.zeros(0, np.int32), positions=np.zeros(0, np.int32))
    plan = make_plan(prob)
    got = gpu_append(plan, prob, new)
    assert_pools_equal(got, [prob["k_pages"], prob["v_pages"], None, None], "empty")


@pytest.mark.parametrize("name", sorted(workloads.APPEND_CONFIGS))
def test_append_workloads_full_size(name):
    """The benchmark's append workloads at full size, in its launch configuration."""
    s, n = workloads.APPEND_CONFIGS[name]
    prob = workloads.generate(s, 35)
    new = workloads.append_tokens(prob, 35, n)
    say(f"case {name}: N={new['k_new'].shape[0]}")
    plan = make_plan(prob, max_kv_len=s.max_kv_len)
    got = gpu_append(plan, prob, new)
    want = oracle_append(prob, new, s.max_kv_len)
    assert_pools_equal(got, want, name)


@pytest.mark.parametrize("kv", ["f16", "i8", "f8", "q4"])
def test_append_then_decode(kv):
    """A decode step: append T new tokens per sequence at the end of each cache, then decode
    over the result on the GPU; the pools match the oracle's append bit for bit and the decode
    matches the fp64 oracle on those pools."""
    s = workloads.spec(name=f"step_{kv}", batch=6, q_per_seq=2, num_qo_heads=32, num_kv_heads=8,
                       head_dim=128, page_size=16, kv_dtype=kv,
                       lens=("list", (2, 70, 1000, 2049, 31, 4096)))
    prob = workloads.generate(s, 36)
    new = workloads.append_tokens(prob, 36, 2)
    plan = make_plan(prob)
    dev = to_dev(prob)
    plan.append(_dev(new["k_new"]), _dev(new["v_new"]), _dev(new["batch_idx"]),
                _dev(new["positions"]), dev["k_pages"], dev["v_pages"], dev["page_table"],
                dev["k_scales"], dev["v_scales"])
    o, lse = run(plan, prob, dev)
    torch.cuda.synchronize()
    want = oracle_append(prob, new, plan.params.max_kv_len)
    got = [None if dev[k] is None else dev[k].cpu().numpy()
           for k in ("k_pages", "v_pages", "k_scales", "v_scales")]
    assert_pools_equal(got, want, f"append {kv}")
    p2 = dict(prob, k_pages=want[0], v_pages=want[1], k_scales=want[2], v_scales=want[3])
    ro, rl = oracle.decode(p2)
    compare(o, lse, ro, rl, what=f"decode after append {kv}")


def test_append_graph_capture_replay():
    """Append + decode captured into one HIP graph (first calls of the plan under capture);
    replays with eager work between them give the eager results bit for bit."""
    s = workloads.spec(name="graph_append", batch=3, q_per_seq=1, num_qo_heads=16,
                       num_kv_heads=4, head_dim=128, page_size=16, kv_dtype="i8",
                       lens=("list", (100, 1500, 3000)))
    prob = workloads.generate(s, 37)
    new = workloads.append_tokens(prob, 37, 1)
    args = [_dev(new[k]) for k in ("k_new", "v_new", "batch_idx", "positions")]
    plan = make_plan(prob)
    plan.ensure_workspace()
    dev = to_dev(prob)
    out = torch.empty(dev["q"].shape, dtype=torch.float16, device="cuda")
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.append(*args, dev["k_pages"], dev["v_pages"], dev["page_table"], dev["k_scales"],
                    dev["v_scales"])
        run(plan, prob, dev, out=out, lse=lse)
    want = oracle_append(prob, new, plan.params.max_kv_len)
    p2 = dict(prob, k_pages=want[0], v_pages=want[1], k_scales=want[2], v_scales=want[3])
    ro, rl = oracle.decode(p2)
    ref = None
    for i in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = [dev[k].cpu().numpy() for k in ("k_pages", "v_pages", "k_scales", "v_scales")]
        assert_pools_equal(got, want, f"replay {i}")
        compare(out, lse, ro, rl, what=f"replay {i}")
        if ref is None:
            ref = (out.clone(), lse.clone())
        else:
            assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1])
        torch.ones(1 << 20, device="cuda").sum()  # eager work between replays


@pytest.mark.parametrize("kv", ["f16", "i8", "f8", "q4"])
@pytest.mark.parametrize("form", ["halves", "interleaved", "layer"])
def test_cache_views(kv, form):
    """K and V as views of one tensor -- the two halves of [2, pages, ...], the interleaved
    [pages, 2, ...], layer 1 of a [layers, 2, pages, ...] pool (the layouts AMD-Ecosystem/
    flashinfer PR #397 tests under "Test plan") -- are addressed through their strides: an
    append into the views and a decode over them match the oracle, and the other layer and
    the unused halves keep their bytes."""
    s = workloads.spec(name=f"views_{form}_{kv}", batch=3, q_per_seq=1, num_qo_heads=16,
                       num_kv_heads=4, head_dim=128, page_size=16, kv_dtype=kv,
                       lens=("list", (33, 700, 1500)))
    prob = workloads.generate(s, 38)
    new = workloads.append_tokens(prob, 38, 3)

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

    bkv, kview, vview = combined(prob["k_pages"], prob["v_pages"])
    bsc, ksview, vsview = combined(prob["k_scales"], prob["v_scales"])
    tk = torch.from_numpy(bkv).cuda()
    ts = None if bsc is None else torch.from_numpy(bsc).cuda()

    def dev_view(t, npview, base):
        if t is None:
            return None
        off = (npview.__array_interface__["data"][0] - base.__array_interface__["data"][0])
        st = [x // npview.itemsize for x in npview.strides]
        return torch.as_strided(t, npview.shape, st, off // npview.itemsize)

    dk, dv = dev_view(tk, kview, bkv), dev_view(tk, vview, bkv)
    dks = None if ts is None else dev_view(ts, ksview, bsc)
    dvs = None if ts is None else dev_view(ts, vsview, bsc)
    plan = make_plan(prob)
    tab, kvl, q = _dev(prob["page_table"]), _dev(prob["kv_len"]), _dev(prob["q"])
    plan.append(_dev(new["k_new"]), _dev(new["v_new"]), _dev(new["batch_idx"]),
                _dev(new["positions"]), dk, dv, tab, dks, dvs)
    o, lse = plan.run(q, dk, dv, tab, kvl, prob["sm_scale"], dks, dvs)
    torch.cuda.synchronize()
    want = oracle_append(prob, new, plan.params.max_kv_len)
    got = [None if t is None else t.cpu().numpy() for t in (dk, dv, dks, dvs)]
    assert_pools_equal(got, want, f"views {form} {kv}")
    if form == "layer":  # layer 0 untouched
        assert np.array_equal(tk[0].cpu().numpy().view(np.uint8), bkv[0].view(np.uint8))
        if ts is not None:
            assert np.array_equal(ts[0].cpu().numpy().view(np.uint8), bsc[0].view(np.uint8))
    p2 = dict(prob, k_pages=want[0], v_pages=want[1], k_scales=want[2], v_scales=want[3])
    ro, rl = oracle.decode(p2)
    compare(o, lse, ro, rl, what=f"decode over views {form} {kv}")

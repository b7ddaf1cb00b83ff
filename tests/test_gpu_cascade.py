"""GPU parity of the merge of attention states (cascade / shared-prefix attention) through the
C ABI against the fp64 oracle, and a cascade built from the library's own calls: decode a
shared prefix, decode each sequence's suffix, merge, compare with the oracle's decode over the
whole sequence. Tolerances as for the decode (max|do| <= 2e-3, max|dlse| <= 1e-3)."""
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


def random_states(rng, S, rows, D, empty_frac=0.1):
    o = rng.standard_normal((S, rows, D), dtype=np.float32).astype(np.float16)
    lse = (5 * rng.standard_normal((S, rows))).astype(np.float32)
    lse[rng.random((S, rows)) < empty_frac] = -np.inf
    lse[:, :3] = -np.inf  # the first rows: every state empty
    return o, lse


@pytest.mark.parametrize("S,rows,D", [(1, 100, 128), (2, 1000, 128), (3, 4097, 64),
                                      (5, 257, 256), (2, 130, 512), (4, 1, 128)])
def test_merge_states_matches_oracle(S, rows, D):
    import quantized_kv_cache_page_amd as skvd
    rng = np.random.default_rng(71 + S + D)
    o_s, l_s = random_states(rng, S, rows, D)
    say(f"case S={S} rows={rows} D={D}")
    o, lse = skvd.merge_states(torch.from_numpy(o_s).cuda(), torch.from_numpy(l_s).cuda())
    torch.cuda.synchronize()
    ro, rl = oracle.merge_states(o_s.astype(np.float64), l_s.astype(np.float64))
    compare(o.reshape(rows, 1, D), lse.reshape(rows, 1), ro, rl, what=f"merge S={S} D={D}")
    assert (o[:3] == 0).all() and torch.isneginf(lse[:3]).all()


def test_merge_states_strided():
    """States stored row-major by row ([rows, S, D] memory, viewed as [S, rows, D])."""
    import quantized_kv_cache_page_amd as skvd
    rng = np.random.default_rng(72)
    o_s, l_s = random_states(rng, 3, 500, 128, empty_frac=0.0)
    od = torch.from_numpy(np.ascontiguousarray(o_s.transpose(1, 0, 2))).cuda().permute(1, 0, 2)
    lse_buf = torch.full((3, 512), float("nan"), device="cuda")
    lse_buf[:, :500] = torch.from_numpy(l_s).cuda()
    o, lse = skvd.merge_states(od, lse_buf[:, :500])
    torch.cuda.synchronize()
    ro, rl = oracle.merge_states(o_s.astype(np.float64), l_s.astype(np.float64))
    compare(o.reshape(500, 1, 128), lse.reshape(500, 1), ro, rl, what="merge strided")


@pytest.mark.parametrize("kv", ["f16", "i8"])
def test_cascade_prefix_suffix(kv):
    """Sequences that share a prefix of pages: decode the prefix for every sequence, decode each
    sequence's own suffix, merge the two states = the oracle's decode over the whole sequence."""
    import quantized_kv_cache_page_amd as skvd
    P, prefix_pages = 16, 40
    s = workloads.spec(name=f"cascade_{kv}", batch=6, num_qo_heads=32, num_kv_heads=8,
                       head_dim=128, page_size=P, kv_dtype=kv,
                       lens=("list", (700, 2000, 3000, 645, 1300, 4096)))
    prob = workloads.generate(s, 73)
    table = prob["page_table"].copy()
    table[:, :prefix_pages] = table[0, :prefix_pages]  # every sequence starts with sequence 0's pages
    prob = dict(prob, page_table=table)
    L = prob["kv_len"].astype(np.int64)
    pre = prefix_pages * P
    assert (L > pre).all()
    # the oracle over whole sequences (shared prefix + own suffix)
    ro, rl = oracle.decode(prob)
    dev = to_dev(prob)
    plan = make_plan(prob)
    pre_len = torch.full_like(dev["kv_len"], pre)
    o_pre, l_pre = plan.run(dev["q"], dev["k_pages"], dev["v_pages"], dev["page_table"], pre_len,
                            prob["sm_scale"], dev["k_scales"], dev["v_scales"])
    suf_table = torch.from_numpy(np.ascontiguousarray(
        np.concatenate([table[:, prefix_pages:], np.full((6, prefix_pages), -1, np.int32)], 1))).cuda()
    suf_len = dev["kv_len"] - pre
    o_suf, l_suf = plan.run(dev["q"], dev["k_pages"], dev["v_pages"], suf_table, suf_len,
                            prob["sm_scale"], dev["k_scales"], dev["v_scales"])
    rows = o_pre.shape[0] * o_pre.shape[1]
    o_s = torch.stack([o_pre.reshape(rows, 128), o_suf.reshape(rows, 128)])
    l_s = torch.stack([l_pre.reshape(rows), l_suf.reshape(rows)])
    o, lse = skvd.merge_states(o_s, l_s)
    torch.cuda.synchronize()
    compare(o.reshape(o_pre.shape), lse.reshape(l_pre.shape), ro, rl, what=f"cascade {kv}")


def test_merge_states_graph_capture_replay():
    import quantized_kv_cache_page_amd as skvd
    rng = np.random.default_rng(74)
    o_s, l_s = random_states(rng, 3, 2000, 128)
    od, ld = torch.from_numpy(o_s).cuda(), torch.from_numpy(l_s).cuda()
    out = torch.empty((2000, 128), dtype=torch.float16, device="cuda")
    lse = torch.empty((2000,), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        skvd.merge_states(od, ld, out=out, lse=lse)
    ro, rl = oracle.merge_states(o_s.astype(np.float64), l_s.astype(np.float64))
    ref = None
    for i in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        compare(out.reshape(2000, 1, 128), lse.reshape(2000, 1), ro, rl, what=f"replay {i}")
        if ref is None:
            ref = (out.clone(), lse.clone())
        else:
            assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1])
        torch.ones(1 << 20, device="cuda").sum()


def test_merge_many_states():
    """Nine states (rounds of four loads plus a partial one)."""
    import quantized_kv_cache_page_amd as skvd
    rng = np.random.default_rng(75)
    o_s, l_s = random_states(rng, 9, 777, 256)
    o, lse = skvd.merge_states(torch.from_numpy(o_s).cuda(), torch.from_numpy(l_s).cuda())
    torch.cuda.synchronize()
    ro, rl = oracle.merge_states(o_s.astype(np.float64), l_s.astype(np.float64))
    compare(o.reshape(777, 1, 256), lse.reshape(777, 1), ro, rl, what="merge S=9")

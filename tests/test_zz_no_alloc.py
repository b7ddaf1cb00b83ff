"""The allocation-free decode (skvd_decode_noalloc, the library's own device workspace) through
the C ABI against skvd_decode with a caller workspace: bit-identical outputs on two calls in a
row, the second with a smaller batch and shorter sequences (the array keeps the first call's
contents), over f16, int8, fp8 and q4_0 caches at head_dim 128 and the one-byte formats at 256;
plans whose workspace exceeds the array's size and debug plans are refused."""
import numpy as np
import pytest
import torch

import workloads
from tests.gpu_util import make_plan, run, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_kv_cache_page_amd as skvd
    skvd.lib()
    yield
    torch.cuda.synchronize()


def _noalloc(plan, prob, dev):
    out = torch.empty(dev["q"].shape, dtype=torch.float16, device="cuda")
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
    plan.run_noalloc(dev["q"], dev["k_pages"], dev["v_pages"], dev["page_table"], dev["kv_len"],
                     prob["sm_scale"], dev["k_scales"], dev["v_scales"], out=out, lse=lse,
                     q_per_seq=int(prob["q_per_seq"]))
    return out, lse


@pytest.mark.parametrize("kv,T,Hq,Hkv,sched,D", [("f16", 1, 32, 8, "auto", 128),
                                                 ("i8", 1, 32, 8, "auto", 128),
                                                 ("i8", 4, 16, 4, "static", 128),
                                                 ("f8", 8, 32, 4, "auto", 128),
                                                 ("q4", 2, 32, 8, "auto", 128),
                                                 ("i8", 4, 32, 16, "auto", 256),
                                                 ("f8", 2, 16, 8, "auto", 256)])
def test_noalloc_matches_decode(kv, T, Hq, Hkv, sched, D):
    big = workloads.spec(name="na_big", batch=6, q_per_seq=T, num_qo_heads=Hq, num_kv_heads=Hkv,
                         head_dim=D, page_size=16, kv_dtype=kv,
                         lens=("list", (9000, 700, 2049, 64, 3000, 8)))
    small = workloads.spec(name="na_small", batch=3, q_per_seq=T, num_qo_heads=Hq,
                           num_kv_heads=Hkv, head_dim=D, page_size=16, kv_dtype=kv,
                           lens=("list", (100, 1500, 9)))
    pb = workloads.generate(big, 31)
    ps = workloads.generate(small, 32)
    # one plan for both calls, sized for the larger
    plan = make_plan(pb, schedule=sched)
    say(f"case noalloc {kv} T={T}: {plan.describe()}")
    for prob in (pb, ps):
        dev = to_dev(prob)
        if prob is ps:  # the plan's table width
            t = torch.full((3, dev_big_table_w), -1, dtype=torch.int32, device="cuda")
            t[:, :dev["page_table"].shape[1]] = dev["page_table"]
            dev["page_table"] = t
        else:
            dev_big_table_w = dev["page_table"].shape[1]
        o_ref, l_ref = run(plan, prob, dev)
        o_na, l_na = _noalloc(plan, prob, dev)
        torch.cuda.synchronize()
        assert torch.equal(o_ref.view(torch.int16), o_na.view(torch.int16)), prob["spec"].name
        assert torch.equal(l_ref, l_na), prob["spec"].name
        say(f"  {prob['spec'].name}: bit-identical to skvd_decode")


def test_noalloc_refusals():
    import quantized_kv_cache_page_amd as skvd
    s = workloads.spec(name="na_err", batch=2, q_per_seq=1, num_qo_heads=8, num_kv_heads=2,
                       head_dim=128, page_size=16, lens=("list", (100, 200)))
    prob = workloads.generate(s, 3)
    dev = to_dev(prob)
    dbg = make_plan(prob, debug=True)
    with pytest.raises(skvd.SkvdError) as e:
        _noalloc(dbg, prob, dev)
    assert e.value.status == 7
    huge = skvd.Plan(64, 64, 256, 16, "f16", max_batch=1024, max_q_per_seq=8, max_kv_len=65536,
                     device=0, schedule="static")
    assert huge.workspace_bytes > (32 << 20)
    # arguments of the huge plan's shape (one sequence, two pages): refused for the workspace
    q = torch.zeros((1, 64, 256), dtype=torch.float16, device="cuda")
    pool = torch.zeros((2, 16, 64, 256), dtype=torch.float16, device="cuda")
    table = torch.zeros((1, 4096), dtype=torch.int32, device="cuda")
    kv_len = torch.full((1,), 20, dtype=torch.int32, device="cuda")
    with pytest.raises(skvd.SkvdError) as e:
        huge.run_noalloc(q, pool, pool, table, kv_len, 0.0625)
    assert e.value.status == 5

"""The torch operators on the GPU (AMD-Ecosystem/flashinfer PR #397, "Test plan": the cache
bit-identical after the call under torch.compile over [2, pages] views and a layer of a pool;
"Architecture / design notes": nothing the decode only reads is copied on a graph replay).

* torch.library.opcheck on skvd::decode_v1 and skvd::decode_out_v1 (schema -- including that
  no input not declared written is changed --, fake implementation, AOT dispatch) over f16,
  int8, fp8 and q4_0 caches.
* torch.compile(fullgraph=True) with the aot_eager backend and with a backend that keeps the
  functionalized forward graph, over the cache as one half of a [2, pages, ...] tensor, one
  slot of an interleaved [pages, 2, ...] tensor and one layer of a multi-layer pool: outputs
  equal the eager Plan.run bit for bit, every cache tensor is bit-identical afterwards, and the
  graph copies nothing into any cache tensor.
* The compiled decode captured in a CUDA graph and replayed with eager work in between:
  bit-identical replays, caches untouched.
* skvd::append_v1 under torch.compile writes what the eager append writes.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import compare, make_plan, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_kv_cache_page_amd as skvd
    skvd.lib()
    yield
    torch.cuda.synchronize()


def _problem(kv, T=1, seed=5):
    s = workloads.spec(name=f"ops_{kv}", batch=3, q_per_seq=T, num_qo_heads=16, num_kv_heads=4,
                       head_dim=128, page_size=16, kv_dtype=kv, lens=("list", (T, 900, 2100)))
    return workloads.generate(s, seed)


def _layout(dev, layout):
    """Rebuild the pools as views of one larger tensor; returns (base, k, v, k_scales, v_scales)."""
    k, v = dev["k_pages"], dev["v_pages"]
    if layout == "two_halves":
        base = torch.stack([k, v])
        kk, vv = base[0], base[1]
    elif layout == "interleaved":
        base = torch.stack([k, v], dim=1)
        kk, vv = base[:, 0], base[:, 1]
    else:  # layer 1 of a 3-layer pool
        base = torch.zeros((3, 2) + tuple(k.shape), dtype=k.dtype, device=k.device)
        base[1, 0], base[1, 1] = k, v
        kk, vv = base[1, 0], base[1, 1]
    ks, vs = dev["k_scales"], dev["v_scales"]
    if ks is not None and ks.dim() == 4:  # int8 scale pools as views too
        sbase = torch.stack([ks, vs])
        ks, vs = sbase[0], sbase[1]
    return base, kk, vv, ks, vs


@pytest.mark.parametrize("kv", ["f16", "i8", "f8", "q4"])
def test_opcheck(kv):
    from quantized_kv_cache_page_amd import ops
    prob = _problem(kv)
    dev = to_dev(prob)
    plan = make_plan(prob)
    pid = ops.register_plan(plan)
    args = (dev["q"], dev["k_pages"], dev["v_pages"], dev["page_table"], dev["kv_len"],
            dev["k_scales"], dev["v_scales"], float(prob["sm_scale"]), 1, pid)
    torch.library.opcheck(torch.ops.skvd.decode_v1.default, args)
    out = torch.empty(dev["q"].shape, dtype=torch.float16, device="cuda")
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
    torch.library.opcheck(torch.ops.skvd.decode_out_v1.default, args + (out, lse))
    o, l = torch.ops.skvd.decode_v1.default(*args)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(prob)
    compare(o, l, ro, rl, what=f"decode_v1 {kv}")
    ops.unregister_plan(pid)


def _capturing_backend(found):
    """A torch.compile backend that functionalizes the captured graph the way AOT autograd does
    (aot_export_module) and records which of the graph's inputs it must write back -- the
    inputs an op declares mutated -- and any in-graph copy, then runs the graph as captured."""
    from torch._functorch.aot_autograd import aot_export_module

    def backend(gm, example_inputs):
        names = [n.name for n in gm.graph.nodes if n.op == "placeholder"]
        fx_g, sig = aot_export_module(gm, example_inputs, trace_joint=False)
        inputs = list(sig.user_inputs)
        found["mutated"] = sorted(names[inputs.index(i)] for i in sig.user_inputs_to_mutate.values())
        found["copies"] = [str(n.args[0]) for n in fx_g.graph.nodes
                           if n.op == "call_function" and n.target is torch.ops.aten.copy_.default]
        return gm.forward
    return backend


@pytest.mark.parametrize("with_out", [False, True])
@pytest.mark.parametrize("layout", ["two_halves", "interleaved", "layer_of_pool"])
@pytest.mark.parametrize("kv", ["f16", "i8", "q4"])
def test_compile_over_cache_views(kv, layout, with_out):
    from quantized_kv_cache_page_amd import ops
    prob = _problem(kv, seed=7)
    dev = to_dev(prob)
    base, k, v, ks, vs = _layout(dev, layout)
    plan = make_plan(prob)
    pid = ops.register_plan(plan)
    sm = float(prob["sm_scale"])
    before = base.clone()
    sbefore = None if ks is None else (ks.clone(), vs.clone())
    eo, el = plan.run(dev["q"], k, v, dev["page_table"], dev["kv_len"], sm, ks, vs)

    def fn(q, k, v, table, kv_len, ks, vs, out, lse):
        if with_out:
            torch.ops.skvd.decode_out_v1(q, k, v, table, kv_len, ks, vs, sm, 1, pid, out, lse)
            return out * 1, lse * 1
        return torch.ops.skvd.decode_v1(q, k, v, table, kv_len, ks, vs, sm, 1, pid)

    found = {}
    for backend in ("aot_eager", _capturing_backend(found)):
        torch._dynamo.reset()
        cfn = torch.compile(fn, backend=backend, fullgraph=True)
        out = torch.empty_like(eo)
        lse = torch.empty_like(el)
        for _ in range(2):
            co, cl = cfn(dev["q"], k, v, dev["page_table"], dev["kv_len"], ks, vs, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(co.view(torch.int16), eo.view(torch.int16)) and torch.equal(cl, el)
        assert torch.equal(base.view(torch.uint8), before.view(torch.uint8)), "cache changed"
        if sbefore is not None:  # (bit views: the unread scale slots hold NaN)
            assert torch.equal(ks.view(torch.int16), sbefore[0].view(torch.int16))
            assert torch.equal(vs.view(torch.int16), sbefore[1].view(torch.int16))
    say(f"  {kv} {layout} out={with_out}: written inputs {found['mutated']}, in-graph copies "
        f"{found['copies']}")
    assert found["copies"] == []
    if with_out:
        assert len(found["mutated"]) == 2 and "out" in found["mutated"][1]
        assert "lse" in found["mutated"][0]
    else:
        assert found["mutated"] == []
    ops.unregister_plan(pid)


def test_compiled_decode_in_cuda_graph():
    from quantized_kv_cache_page_amd import ops
    prob = _problem("i8", seed=9)
    dev = to_dev(prob)
    base, k, v, ks, vs = _layout(dev, "layer_of_pool")
    plan = make_plan(prob)
    pid = ops.register_plan(plan)
    sm = float(prob["sm_scale"])
    out = torch.empty(dev["q"].shape, dtype=torch.float16, device="cuda")
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")

    def fn():
        torch.ops.skvd.decode_out_v1(dev["q"], k, v, dev["page_table"], dev["kv_len"], ks, vs,
                                     sm, 1, pid, out, lse)

    cfn = torch.compile(fn, backend="aot_eager", fullgraph=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            cfn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eo, el = out.clone(), lse.clone()
    before = base.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cfn()
    for i in range(3):
        out.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eo.view(torch.int16)), f"replay {i}"
        assert torch.equal(lse, el)
        plan.run(dev["q"], k, v, dev["page_table"], dev["kv_len"], sm, ks, vs)  # eager work
    assert torch.equal(base.view(torch.uint8), before.view(torch.uint8))
    ro, rl = oracle.decode(prob)
    compare(out, lse, ro, rl, what="graph-replayed compiled decode")
    ops.unregister_plan(pid)


def test_compiled_append_writes_the_cache():
    from quantized_kv_cache_page_amd import ops
    prob = _problem("i8", seed=11)
    new = workloads.append_tokens(prob, 11, 64)
    dev = to_dev(prob)
    nd = {kk: torch.from_numpy(np.ascontiguousarray(vv)).cuda() for kk, vv in new.items()}
    plan = make_plan(prob)
    pid = ops.register_plan(plan)
    ref = [dev[x].clone() for x in ("k_pages", "v_pages", "k_scales", "v_scales")]
    plan.append(nd["k_new"], nd["v_new"], nd["batch_idx"], nd["positions"], ref[0], ref[1],
                dev["page_table"], ref[2], ref[3])

    def fn(kp, vp, ksp, vsp):
        torch.ops.skvd.append_v1(nd["k_new"], nd["v_new"], nd["batch_idx"], nd["positions"], kp,
                                 vp, dev["page_table"], ksp, vsp, pid)

    torch.compile(fn, backend="aot_eager", fullgraph=True)(dev["k_pages"], dev["v_pages"],
                                                          dev["k_scales"], dev["v_scales"])
    torch.cuda.synchronize()
    for a, b in zip(ref, (dev["k_pages"], dev["v_pages"], dev["k_scales"], dev["v_scales"])):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    ops.unregister_plan(pid)

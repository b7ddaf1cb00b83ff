"""The torch operators on the GPU (AMD-Ecosystem/flashinfer PR #397, "Test plan": the cache
bit-identical after the call under torch.compile over [2, pages] views, an interleaved tensor
under dynamic shapes and a layer of a pool, for the decode and the paged prefill; an append
before and after each route in one graph; "Architecture / design notes": nothing the decode
only reads is copied on a graph replay).

* torch.library.opcheck on skvd::decode_v1, skvd::decode_out_v1, skvd::prefill_v1 and
  skvd::prefill_out_v1 (schema -- including that no input not declared written is changed --,
  fake implementation, AOT dispatch) over f16, int8, fp8 and q4_0 caches.
* torch.compile(fullgraph=True) with the aot_eager backend (static shapes for the [2, pages]
  halves, dynamic for the interleaved tensor, both for a layer of a pool) and with a backend
  that keeps the functionalized forward graph, over the cache as one half of a [2, pages, ...]
  tensor, one slot of an interleaved [pages, 2, ...] tensor and one layer of a multi-layer
  pool, for the decode and the multi-token route: outputs equal the eager call bit for bit,
  every cache tensor is bit-identical afterwards, and the graph copies nothing into any cache
  tensor.
* The compiled decode and multi-token route captured in a CUDA graph and replayed with eager
  work in between: bit-identical replays, caches untouched.
* skvd::append_v1 under torch.compile writes what the eager append writes; an append of half
  the new rows before each route and of the other half after it, in one compiled graph (over
  separate caches, and over views of one tensor with dynamic shapes), gives what the same
  calls give eagerly, in that order.
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


@pytest.mark.parametrize("kv", ["f16", "i8", "f8", "q4"])
def test_opcheck_prefill(kv):
    from quantized_kv_cache_page_amd import ops
    prob = _problem(kv, T=4, seed=6)
    dev = to_dev(prob)
    plan = make_plan(prob, max_q_per_seq=1)
    pid = ops.register_plan(plan)
    args = (dev["q"], dev["k_pages"], dev["v_pages"], dev["page_table"], dev["kv_len"],
            dev["k_scales"], dev["v_scales"], float(prob["sm_scale"]), 4, pid)
    torch.library.opcheck(torch.ops.skvd.prefill_v1.default, args)
    out = torch.empty(dev["q"].shape, dtype=torch.float16, device="cuda")
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
    torch.library.opcheck(torch.ops.skvd.prefill_out_v1.default, args + (out, lse))
    o, l = ops.prefill(pid, *args[:5], args[7], args[5], args[6], q_per_seq=4)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(prob)
    compare(o, l, ro, rl, what=f"prefill_v1 {kv}")
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


# the compile modes of each cache form: static shapes for the [2, pages] halves, dynamic for the
# interleaved tensor, both for a layer of a pool
_DYNAMIC = {"two_halves": (False,), "interleaved": (True,), "layer_of_pool": (False, True)}


def _route_ops(route):
    if route == "decode":
        return torch.ops.skvd.decode_v1, torch.ops.skvd.decode_out_v1, 1
    return torch.ops.skvd.prefill_v1, torch.ops.skvd.prefill_out_v1, 4


@pytest.mark.parametrize("route", ["decode", "prefill"])
@pytest.mark.parametrize("with_out", [False, True])
@pytest.mark.parametrize("layout", ["two_halves", "interleaved", "layer_of_pool"])
@pytest.mark.parametrize("kv", ["f16", "i8", "q4"])
def test_compile_over_cache_views(kv, layout, with_out, route):
    from quantized_kv_cache_page_amd import ops
    op, op_out, T = _route_ops(route)
    prob = _problem(kv, T=T, seed=7)
    dev = to_dev(prob)
    base, k, v, ks, vs = _layout(dev, layout)
    plan = make_plan(prob)
    pid = ops.register_plan(plan)
    sm = float(prob["sm_scale"])
    before = base.clone()
    sbefore = None if ks is None else (ks.clone(), vs.clone())
    eager = plan.run if route == "decode" else plan.prefill
    eo, el = eager(dev["q"], k, v, dev["page_table"], dev["kv_len"], sm, ks, vs, q_per_seq=T)

    def fn(q, k, v, table, kv_len, ks, vs, out, lse):
        if with_out:
            op_out(q, k, v, table, kv_len, ks, vs, sm, T, pid, out, lse)
            return out * 1, lse * 1
        return op(q, k, v, table, kv_len, ks, vs, sm, T, pid)

    found = {}
    modes = [("aot_eager", d) for d in _DYNAMIC[layout]] + [(_capturing_backend(found), False)]
    for backend, dynamic in modes:
        torch._dynamo.reset()
        cfn = torch.compile(fn, backend=backend, fullgraph=True, dynamic=dynamic)
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
    say(f"  {route} {kv} {layout} out={with_out} dynamic={_DYNAMIC[layout]}: written inputs "
        f"{found['mutated']}, in-graph copies {found['copies']}")
    assert found["copies"] == []
    if with_out:
        assert len(found["mutated"]) == 2 and "out" in found["mutated"][1]
        assert "lse" in found["mutated"][0]
    else:
        assert found["mutated"] == []
    ops.unregister_plan(pid)


@pytest.mark.parametrize("route", ["decode", "prefill"])
def test_compiled_decode_in_cuda_graph(route):
    from quantized_kv_cache_page_amd import ops
    _, op_out, T = _route_ops(route)
    prob = _problem("i8", T=T, seed=9)
    dev = to_dev(prob)
    base, k, v, ks, vs = _layout(dev, "layer_of_pool")
    plan = make_plan(prob)
    pid = ops.register_plan(plan)
    sm = float(prob["sm_scale"])
    out = torch.empty(dev["q"].shape, dtype=torch.float16, device="cuda")
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")

    def fn():
        op_out(dev["q"], k, v, dev["page_table"], dev["kv_len"], ks, vs, sm, T, pid, out, lse)

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
        plan.run(dev["q"], k, v, dev["page_table"], dev["kv_len"], sm, ks, vs,
                 q_per_seq=T)  # eager work
    assert torch.equal(base.view(torch.uint8), before.view(torch.uint8))
    ro, rl = oracle.decode(prob)
    compare(out, lse, ro, rl, what=f"graph-replayed compiled {route}")
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


@pytest.mark.parametrize("form", ["separate", "views_dynamic"])
@pytest.mark.parametrize("route", ["decode", "prefill"])
def test_compiled_append_and_attention_order(route, form):
    """append(first half) -> attend -> append(second half) -> attend in one fullgraph graph:
    the attention ops declare the cache only read, so what orders them after each append is
    the append's own declaration; each output must equal the eager sequence's."""
    from quantized_kv_cache_page_amd import ops
    op, _, T = _route_ops(route)
    prob = _problem("i8", T=T, seed=13)
    new = workloads.append_tokens(prob, 13, 64)
    dev = to_dev(prob)
    nd = {kk: torch.from_numpy(np.ascontiguousarray(vv)).cuda() for kk, vv in new.items()}
    N = nd["k_new"].shape[0]
    halves = [{kk: vv[:N // 2] for kk, vv in nd.items()}, {kk: vv[N // 2:] for kk, vv in nd.items()}]
    plan = make_plan(prob)
    pid = ops.register_plan(plan)
    sm = float(prob["sm_scale"])
    table, kv_len = dev["page_table"], dev["kv_len"]
    eager = plan.run if route == "decode" else plan.prefill

    # the eager sequence on copies of the cache
    ref = [dev[x].clone() for x in ("k_pages", "v_pages", "k_scales", "v_scales")]
    outs = []
    for h in halves:
        plan.append(h["k_new"], h["v_new"], h["batch_idx"], h["positions"], ref[0], ref[1],
                    table, ref[2], ref[3])
        outs += [t.clone() for t in eager(dev["q"], ref[0], ref[1], table, kv_len, sm, ref[2],
                                          ref[3], q_per_seq=T)]
    torch.cuda.synchronize()
    assert not torch.equal(outs[0], outs[2]), "the second append must change the output"

    def steps(q, kp, vp, ksp, vsp):
        res = []
        for h in halves:
            torch.ops.skvd.append_v1(h["k_new"], h["v_new"], h["batch_idx"], h["positions"], kp,
                                     vp, table, ksp, vsp, pid)
            res += list(op(q, kp, vp, table, kv_len, ksp, vsp, sm, T, pid))
        return tuple(res)

    if form == "separate":
        cache = [dev[x].clone() for x in ("k_pages", "v_pages", "k_scales", "v_scales")]
        fn = torch.compile(steps, backend="aot_eager", fullgraph=True)
        torch._dynamo.reset()
        got = fn(dev["q"], *cache)
        final = cache
    else:
        base = torch.stack([dev["k_pages"], dev["v_pages"]])
        sbase = torch.stack([dev["k_scales"], dev["v_scales"]])

        def from_base(q, base, sbase):
            return steps(q, base[0], base[1], sbase[0], sbase[1])

        torch._dynamo.reset()
        fn = torch.compile(from_base, backend="aot_eager", fullgraph=True, dynamic=True)
        got = fn(dev["q"], base, sbase)
        final = [base[0], base[1], sbase[0], sbase[1]]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(outs, got)):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.float16 else a,
                           b.view(torch.int16) if b.dtype == torch.float16 else b), i
    for a, b in zip(ref, final):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    say(f"  {route} {form}: {N} rows appended in two halves, both outputs equal the eager order")
    ops.unregister_plan(pid)

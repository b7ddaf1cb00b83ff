"""The torch operators' declarations, checked without a GPU: what each op's schema marks as
written, and what torch's functionalization (the pass torch.compile and torch.export run) makes
of a decode (and of the multi-token route) over cache views -- one half of a [2, pages, ...] tensor, one slot of an
interleaved [pages, 2, ...] tensor, one layer of a multi-layer pool
(AMD-Ecosystem/flashinfer PR #397, "What changed" and "Test plan"). The graphs are traced
with meta tensors through the ops' fake implementations; nothing runs. A planted wrong
declaration (an op that registers the cache as mutated) is shown to be caught by the same
check."""
import pytest
import torch

from quantized_kv_cache_page_amd import ops  # noqa: F401  (registers torch.ops.skvd.*)

M = "meta"


def _mutable(schema):
    return sorted(a.name for a in schema.arguments if a.alias_info is not None and a.alias_info.is_write)


def test_schemas_declare_only_real_outputs():
    assert _mutable(torch.ops.skvd.decode_v1.default._schema) == []
    assert _mutable(torch.ops.skvd.decode_out_v1.default._schema) == ["lse", "out"]
    assert _mutable(torch.ops.skvd.prefill_v1.default._schema) == []
    assert _mutable(torch.ops.skvd.prefill_out_v1.default._schema) == ["lse", "out"]
    # the append really writes the cache and says so
    assert _mutable(torch.ops.skvd.append_v1.default._schema) == [
        "k_pages", "k_scales", "v_pages", "v_scales"]
    # versioned names: a schema change gets a new name, never a stale cache entry
    assert str(torch.ops.skvd.decode_v1.default._schema).startswith("skvd::decode_v1(")


def _views(layout, pages=40, P=16, Hkv=8, D=128, dtype=torch.float16):
    if layout == "two_halves":       # [2, pages, P, Hkv, D]
        base = torch.empty(2, pages, P, Hkv, D, dtype=dtype, device=M)
        return base, base[0], base[1]
    if layout == "interleaved":      # [pages, 2, P, Hkv, D]
        base = torch.empty(pages, 2, P, Hkv, D, dtype=dtype, device=M)
        return base, base[:, 0], base[:, 1]
    if layout == "layer_of_pool":    # [layers, 2, pages, P, Hkv, D]
        base = torch.empty(3, 2, pages, P, Hkv, D, dtype=dtype, device=M)
        return base, base[1, 0], base[1, 1]
    raise ValueError(layout)


class _Decode(torch.nn.Module):
    def __init__(self, layout, with_out, route="decode"):
        super().__init__()
        self.layout, self.with_out, self.route = layout, with_out, route

    def forward(self, q, base, table, kv_len, out, lse):
        if self.layout == "two_halves":
            k, v = base[0], base[1]
        elif self.layout == "interleaved":
            k, v = base[:, 0], base[:, 1]
        else:
            k, v = base[1, 0], base[1, 1]
        T = 1 if self.route == "decode" else 2
        if self.with_out:
            op = torch.ops.skvd.decode_out_v1 if self.route == "decode" else \
                torch.ops.skvd.prefill_out_v1
            op(q, k, v, table, kv_len, None, None, 0.1, T, 1, out, lse)
            return out.sum(), lse.sum()
        op = torch.ops.skvd.decode_v1 if self.route == "decode" else torch.ops.skvd.prefill_v1
        return op(q, k, v, table, kv_len, None, None, 0.1, T, 1)


def _inputs(layout):
    base, _, _ = _views(layout)
    q = torch.empty(4, 32, 128, dtype=torch.float16, device=M)
    table = torch.empty(4, 10, dtype=torch.int32, device=M)
    kv_len = torch.empty(4, dtype=torch.int32, device=M)
    out = torch.empty(4, 32, 128, dtype=torch.float16, device=M)
    lse = torch.empty(4, 32, dtype=torch.float32, device=M)
    return q, base, table, kv_len, out, lse


def _functional_graph(mod, args):
    ep = torch.export.export(mod, args).run_decompositions({})
    return ep, ep.graph_signature.user_inputs_to_mutate


@pytest.mark.parametrize("route", ["decode", "prefill"])
@pytest.mark.parametrize("with_out", [False, True])
@pytest.mark.parametrize("layout", ["two_halves", "interleaved", "layer_of_pool"])
def test_functionalized_decode_writes_no_cache(layout, with_out, route):
    ep, mutated = _functional_graph(_Decode(layout, with_out, route), _inputs(layout))
    assert "base" not in mutated.values(), (layout, mutated)
    assert set(mutated.values()) == ({"out", "lse"} if with_out else set()), mutated
    # no copy of anything back into the cache's base
    for n in ep.graph.nodes:
        if n.op == "call_function" and n.target is torch.ops.aten.copy_.default:
            assert n.args[0].name != "base", n


def test_planted_wrong_declaration_is_caught():
    """An op that declares the cache mutated (the mistake the pages fix) makes the
    functionalized graph write the whole base tensor back: the check above would fail."""
    lib = torch.library.Library("skvd_planted", "FRAGMENT")  # test-only namespace
    lib.define("decode_declares_cache(Tensor q, Tensor(a!) k_pages, Tensor(b!) v_pages) -> Tensor")
    lib.impl("decode_declares_cache", lambda q, k, v: torch.empty_like(q), "Meta")

    class Bad(torch.nn.Module):
        def forward(self, q, base):
            return torch.ops.skvd_planted.decode_declares_cache(q, base[0], base[1])

    base, _, _ = _views("two_halves")
    q = torch.empty(4, 32, 128, dtype=torch.float16, device=M)
    _, mutated = _functional_graph(Bad(), (q, base))
    assert "base" in mutated.values()


def test_append_declares_the_pools_it_writes():
    class App(torch.nn.Module):
        def forward(self, kn, vn, bi, pos, base, table):
            torch.ops.skvd.append_v1(kn, vn, bi, pos, base[0], base[1], table, None, None, 1)
            return kn.sum()

    base, _, _ = _views("two_halves")
    kn = torch.empty(5, 8, 128, dtype=torch.float16, device=M)
    args = (kn, kn.clone(), torch.empty(5, dtype=torch.int32, device=M),
            torch.empty(5, dtype=torch.int32, device=M), base,
            torch.empty(4, 10, dtype=torch.int32, device=M))
    _, mutated = _functional_graph(App(), args)
    assert set(mutated.values()) == {"base"}

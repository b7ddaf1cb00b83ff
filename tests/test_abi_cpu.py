"""The C ABI on the CPU: the library loads and exports every declared symbol, plans resolve
as specified, and every host-checkable error path returns its status without any HIP call
(skvd_decode_check and plan creation with an explicit CU count touch no GPU)."""
import math
import os
import re

import pytest

import quantized_kv_cache_page_amd as skvd
from quantized_kv_cache_page_amd import _binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    txt = open(os.path.join(ROOT, "include", "skvd.h")).read()
    return sorted(set(re.findall(r"^\S[^\n(]*?\b(skvd_\w+)\(", txt, re.M)))


def test_exports_every_declared_symbol():
    L = skvd.lib()
    syms = declared_symbols()
    assert len(syms) >= 12
    for s in syms:
        assert hasattr(L, s), s
    assert set(syms) == set(bd.SIGNATURES), set(syms) ^ set(bd.SIGNATURES)
    assert L.skvd_abi_version() == bd.ABI_VERSION == 11


def plan(**kw):
    base = dict(num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16, kv_dtype="f16",
                max_batch=32, max_q_per_seq=1, max_kv_len=4096, device=0, num_cus=256)
    base.update(kw)
    return skvd.Plan(**base)


def test_golden_capacity_blocks():
    """Forced one block per split, the partial count is the page's capacity / 64."""
    path = os.path.join(ROOT, "tests", "golden", "capacity_blocks.txt")
    for ln in open(path):
        if ln.startswith("#") or not ln.strip():
            continue
        n, cap, blocks = map(int, ln.split())
        assert cap == -(-n // 64) * 64 and blocks == cap // 64
        p = plan(max_batch=1, max_kv_len=n, force_blocks_per_split=1, force_reducer="multipass")
        assert p.info.splits_cap == blocks


@pytest.mark.parametrize("maxlen", [1, 63, 64, 65, 256, 257, 2047, 2048, 2049, 4096, 4864,
                                    131072, 262144, 262208])
@pytest.mark.parametrize("bps", [0, 1, 3, 8])
def test_plan_splits_and_total_reducer(maxlen, bps):
    p = plan(max_kv_len=maxlen, force_blocks_per_split=bps)
    i = p.info
    blocks = -(-maxlen // 64)
    assert 1 <= i.blocks_per_split <= blocks
    if bps:
        assert i.blocks_per_split == min(bps, blocks)
    assert i.splits_cap == -(-blocks // i.blocks_per_split)
    # the reducer choice is total: every partial count has one
    assert p.reducer in ("none", "direct", "cooperative", "multipass", "hierarchical")
    if i.splits_cap == 1:
        assert p.reducer == "none" and p.schedule == "static" and i.part_stride == 1
    else:  # max_batch 32 <= 64: the balanced schedule; a row meets at most min(grid, pieces + 1)
        # shares, a piece being one block (or the forced split size)
        assert p.schedule == "balanced" and i.heads_per_wg == 4
        assert i.grid_wgs == 256  # 4 KV heads per workgroup, one workgroup per CU
        piece = min(bps, blocks) if bps else 1
        assert i.part_stride == min(i.grid_wgs, -(-blocks // piece) + 1)
    if p.reducer == "cooperative":
        assert i.part_stride <= 64
    if p.reducer == "hierarchical":
        assert i.hier_groups_cap == -(-i.part_stride // 64)
    # workspace holds the status word plus (m, l, D floats) per partial: static, per output row
    # and split; balanced, per compact slot (schedule rows + shares), head and query row
    rows = 32 * 1 * 32
    if p.reducer == "none":
        need = 0
    elif p.schedule == "static":
        need = rows * i.part_stride * (2 + 128) * 4
    else:
        need = (32 * 2 + i.grid_wgs) * 4 * 4 * (2 + 128) * 4
    assert i.workspace_bytes >= need + 4


def test_schedule_choice():
    for b in (64, 65, 256, 1024):
        assert plan(max_batch=b).schedule == "balanced"
    p = plan(max_batch=1025)
    assert p.schedule == "static" and p.info.part_stride == p.info.splits_cap
    assert p.info.grid_wgs == (p.info.splits_cap | 1) * (8 // p.info.heads_per_wg) * 1025
    s = plan(schedule="static")
    assert s.schedule == "static" and s.info.part_stride == s.info.splits_cap
    w = plan(wgs_per_cu=7, num_cus=100)
    assert w.schedule == "balanced" and w.info.grid_wgs == 700 and w.info.heads_per_wg == 4
    assert "schedule=balanced" in w.describe()
    # defaults per variant: 4 per CU, 3 at head_dim 256 (f16), 8 for the one-byte formats at
    # head_dim 192 / 256 (two waves per SIMD), 4 at 512; one-byte single-quarter tiles:
    # workgroups of 4 KV heads, three per CU (else 2 or 1 heads, 12 waves per CU)
    assert plan(head_dim=256, num_kv_heads=16).info.grid_wgs == 3 * 256
    for kv in ("i8", "f8", "q4"):
        assert plan(head_dim=256, num_kv_heads=16, kv_dtype=kv).info.grid_wgs == 8 * 256, kv
        assert plan(head_dim=512, num_kv_heads=16, kv_dtype=kv).info.grid_wgs == 4 * 256, kv
    assert plan(head_dim=192, num_kv_heads=16, kv_dtype="f8").info.grid_wgs == 8 * 256
    assert plan(head_dim=192, num_kv_heads=16).info.grid_wgs == 3 * 256
    i8 = plan(kv_dtype="i8")
    assert i8.info.heads_per_wg == 4 and i8.info.grid_wgs == 3 * 256
    i8_4 = plan(kv_dtype="i8", num_kv_heads=4, num_qo_heads=16)
    assert i8_4.info.heads_per_wg == 4 and i8_4.info.grid_wgs == 3 * 256
    assert plan(kv_dtype="i8", heads_per_wg=8).info.grid_wgs == 1 * 256
    assert plan(kv_dtype="i8", num_kv_heads=2, num_qo_heads=8).info.heads_per_wg == 2
    assert plan(heads_per_wg=8).info.grid_wgs == 256
    assert plan(kv_dtype="i8", num_kv_heads=3, num_qo_heads=12).info.heads_per_wg == 1
    assert plan(kv_dtype="i8", heads_per_wg=1).info.grid_wgs == 12 * 256
    assert plan(kv_dtype="i8", max_q_per_seq=2).info.grid_wgs == 4 * 256
    assert plan(kv_dtype="i8", max_q_per_seq=2).info.heads_per_wg == 1
    assert plan().info.heads_per_wg == 4 and plan().info.grid_wgs == 256
    assert plan(heads_per_wg=1).info.grid_wgs == 4 * 256
    assert plan(num_kv_heads=2, num_qo_heads=8).info.grid_wgs == 2 * 256
    st = plan(kv_dtype="i8", schedule="static")
    assert st.info.grid_wgs == (st.info.splits_cap | 1) * (8 // st.info.heads_per_wg) * 32


@pytest.mark.parametrize("red", ["direct", "multipass", "hierarchical"])
def test_forced_reducers_cover_any_count(red):
    p = plan(max_kv_len=262208, force_blocks_per_split=1, force_reducer=red, schedule="static")
    assert p.info.splits_cap == 4097 and p.info.part_stride == 4097 and p.reducer == red
    b = plan(max_kv_len=262208, force_blocks_per_split=1, force_reducer=red)
    assert b.schedule == "balanced" and b.info.part_stride == b.info.grid_wgs == 256
    assert b.reducer == red


def test_heuristic_configs():
    """The workloads' plans: one split up to 128 tokens; small decodes spread one KV head per
    workgroup; no 2048/32-block ceiling anywhere."""
    assert plan(num_qo_heads=8, num_kv_heads=8, max_batch=1, max_kv_len=128).reducer == "none"
    c1 = plan(num_qo_heads=8, num_kv_heads=8, max_batch=1, max_kv_len=256)
    assert c1.reducer in ("direct", "cooperative") and c1.schedule == "balanced"
    # 32 (sequence, KV head, block) units on 256 CUs: one block per split fills the most CUs
    assert c1.info.heads_per_wg == 1 and c1.info.blocks_per_split == 1
    # many query rows per KV head (32 query / 4 KV heads, 8-token drafts, 64 rows): the partial
    # traffic rule alone would give one split per row; the plan still fills the CUs
    mtp = plan(num_qo_heads=32, num_kv_heads=4, max_batch=2, max_q_per_seq=8, max_kv_len=2544,
               kv_dtype="i8")
    assert mtp.schedule == "balanced" and mtp.info.splits_cap >= 32
    assert "rows_per_wg=64" in mtp.describe()
    # (sequence, KV head, block) units <= CUs: one head per workgroup; beyond, four
    assert plan(max_batch=1, max_kv_len=1024).info.heads_per_wg == 1
    assert plan(max_batch=1, max_kv_len=8192).info.heads_per_wg == 4
    c3 = plan(max_batch=1, page_size=64, max_kv_len=131072)
    assert c3.info.splits_cap > 64 and c3.reducer in ("multipass", "hierarchical")
    for p in (plan(), c3, plan(num_kv_heads=16, head_dim=256, max_batch=8, max_q_per_seq=4,
                               max_kv_len=32768), plan(kv_dtype="i8", max_batch=64,
                                                       max_kv_len=65536)):
        i = p.info
        assert i.blocks_per_split * 64 * i.splits_cap >= p.params.max_kv_len


def test_balanced_limits_fall_back_to_static():
    """Where the balanced schedule's 32-bit share arithmetic would not hold, the automatic
    choice is the static schedule; just inside the limits it stays balanced."""
    assert plan(max_batch=1024, max_kv_len=1 << 27).schedule == "static"
    assert plan(num_cus=600).schedule == "static"
    assert plan(max_batch=1024, max_kv_len=1 << 21).schedule == "balanced"  # 2^26 blocks
    assert plan(num_cus=512).schedule == "balanced"


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), 2), (dict(num_qo_heads=30), 2), (dict(page_size=24), 2),
    (dict(max_q_per_seq=9), 2), (dict(max_q_per_seq=1, num_qo_heads=2048, num_kv_heads=1), 2),
    (dict(max_batch=0), 2), (dict(max_kv_len=0), 2), (dict(kv_dtype=7), 4),
    (dict(force_reducer="cooperative", max_kv_len=131072, max_batch=1, force_blocks_per_split=1), 7),
    (dict(force_reducer="none", max_kv_len=4096), 7),
    (dict(schedule="balanced", max_batch=1025), 7), (dict(schedule="balanced", max_kv_len=128), 7),
    (dict(schedule="balanced", force_reducer="none", max_kv_len=200), 7),
    # the device cuts balanced shares in 32-bit arithmetic: blocks x schedule heads x max_batch
    # below 2^31 (here 1024 x 2 x 2^21), and the grid's square below 2^30 (num_cus <= 512)
    (dict(schedule="balanced", max_batch=1024, max_kv_len=1 << 27), 7),
    (dict(schedule="balanced", num_cus=600), 7),
    (dict(schedule=3), 7), (dict(wgs_per_cu=65), 7), (dict(wgs_per_cu=-1), 7),
    (dict(heads_per_wg=2, max_q_per_seq=2), 7), (dict(kv_dtype="i8", heads_per_wg=3), 7),
    (dict(kv_dtype="i8", heads_per_wg=8, num_kv_heads=4, num_qo_heads=16), 7), (dict(kv_dtype="i8", heads_per_wg=4, num_kv_heads=2,
                                                   num_qo_heads=8), 7),
    (dict(kv_dtype="i8", heads_per_wg=2, head_dim=256), 7),
])
def test_plan_errors(kw, status):
    with pytest.raises(skvd.SkvdError) as e:
        if kw.get("kv_dtype") == 7:
            prm = bd.skvd_plan_params(32, 8, 128, 16, 32, 1, 4096, 7, 0, 256, 0, 0, 0)
            bd.skvd_plan_create(prm)
        else:
            plan(**kw)
    assert e.value.status == status
    assert skvd.last_error()


FAKE = 1 << 40  # an aligned address; skvd_decode_check never dereferences it


def good_args(p, i8=False, **over):
    a = bd.skvd_decode_args()
    a.q, a.q_tok_stride, a.q_head_stride = FAKE, 32 * 128, 128
    a.k_pages, a.v_pages = FAKE, FAKE + (1 << 30)
    a.page_stride, a.tok_stride, a.head_stride = 16 * 8 * 128, 8 * 128, 128
    a.num_k_pages = a.num_v_pages = 100
    if i8:
        a.k_scales, a.v_scales = FAKE + (2 << 30), FAKE + (3 << 30)
        a.scale_page_stride, a.scale_tok_stride, a.scale_head_stride = 16 * 8 * 4, 8 * 4, 4
    a.page_table, a.table_stride, a.kv_len = FAKE, 256, FAKE
    a.batch, a.q_per_seq, a.sm_scale = 32, 1, 1 / math.sqrt(128)
    a.o, a.lse = FAKE, FAKE
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("over,status", [
    ({}, 0), (dict(lse=None), 0), (dict(batch=0), 0),
    (dict(q=None), 1), (dict(o=None), 1), (dict(kv_len=None), 1), (dict(page_table=None), 1),
    (dict(batch=33), 2), (dict(batch=-1), 2), (dict(q_per_seq=2), 2), (dict(q_per_seq=0), 2),
    (dict(sm_scale=float("nan")), 2), (dict(reserved=1), 2), (dict(num_v_pages=0), 2),
    (dict(q=FAKE + 2), 3), (dict(q_head_stride=100), 3), (dict(tok_stride=1020), 3),
    (dict(k_pages=FAKE + 8), 3), (dict(table_stride=255), 3), (dict(o=FAKE + 4), 3),
    (dict(page_stride=-8), 3),
    (dict(k_scales=FAKE), 4),
])
def test_decode_check_f16(over, status):
    p = plan()
    assert bd.skvd_decode_check(p.handle, good_args(p, **over), p.workspace_bytes) == status


@pytest.mark.parametrize("over,status", [
    ({}, 0), (dict(k_scales=None), 4), (dict(v_scales=None), 4), (dict(k_pages=FAKE + 8), 3),
    (dict(k_pages=FAKE + 16), 0),
    (dict(k_pages=FAKE + 4), 3), (dict(k_scales=FAKE + 1), 3), (dict(v_scales=FAKE + 4), 3),
    (dict(tok_stride=8 * 128 + 8), 3), (dict(tok_stride=8 * 128 + 16), 0),
    (dict(scale_tok_stride=34), 3), (dict(scale_head_stride=2), 3),
    (dict(scale_page_stride=16 * 8 * 4 + 2), 3), (dict(scale_tok_stride=36), 0),
])
def test_decode_check_int8(over, status):
    p = plan(kv_dtype="i8")
    assert bd.skvd_decode_check(p.handle, good_args(p, i8=True, **over), p.workspace_bytes) == status


@pytest.mark.parametrize("over,status", [
    ({}, 0), (dict(k_scales=None), 4), (dict(v_scales=None), 4), (dict(k_scales=FAKE + 2), 3),
    (dict(v_scales=FAKE + 4), 0), (dict(k_pages=FAKE + 8), 3),
    (dict(tok_stride=8 * 128 + 8), 3), (dict(tok_stride=8 * 128 + 16), 0),
    (dict(scale_tok_stride=3, scale_head_stride=1), 0),  # fp8 has no per-row scale strides
])
def test_decode_check_fp8(over, status):
    """fp8 E4M3 cache: one-byte elements like int8, and one f32 scale per tensor (4-byte
    aligned pointers; the scale strides are ignored)."""
    p = plan(kv_dtype="f8")
    a = good_args(p, **dict(dict(k_scales=FAKE + (2 << 30), v_scales=FAKE + (3 << 30)), **over))
    assert bd.skvd_decode_check(p.handle, a, p.workspace_bytes) == status


def test_fp8_plan_and_unsupported_routes():
    """fp8 plans: 4 KV heads per workgroup, three workgroups per CU (as int8); appends and the
    multi-token route take the two tensor scales."""
    p8, pi = plan(kv_dtype="f8"), plan(kv_dtype="i8")
    assert p8.kv_dtype == "f8" and p8.info.heads_per_wg == 4 and pi.info.heads_per_wg == 4
    assert "grid=768" in p8.describe() and "grid=768" in pi.describe()
    a = good_append_args(k_scales=FAKE + (2 << 32), v_scales=FAKE + (3 << 32))
    assert bd.skvd_append_check(p8.handle, a) == 0
    for over, st in ((dict(k_scales=None), 4), (dict(v_scales=FAKE + 2), 3),
                     (dict(tok_stride=8 * 128 + 8), 3), (dict(scale_tok_stride=3), 0)):
        a = good_append_args(**dict(dict(k_scales=FAKE + (2 << 32), v_scales=FAKE + (3 << 32)),
                                    **over))
        assert bd.skvd_append_check(p8.handle, a) == st, over
    d = good_args(p8, q_per_seq=512, k_scales=FAKE + (2 << 30), v_scales=FAKE + (3 << 30))
    assert bd.skvd_prefill_check(p8.handle, d) == 0
    assert bd.skvd_prefill_check(p8.handle, good_args(p8, q_per_seq=512)) == 4  # no scales
    with pytest.raises(ValueError):
        plan(kv_dtype="q5")


def test_workspace_too_small():
    p = plan()
    assert bd.skvd_decode_check(p.handle, good_args(p), p.workspace_bytes - 1) == 5
    assert "workspace" in skvd.last_error()


def test_status_strings():
    for s in range(9):
        assert skvd.status_string(s)
    assert skvd.status_string(0) == "ok"


def good_append_args(i8=False, **over):
    a = bd.skvd_append_args()
    a.k_new, a.v_new = FAKE, FAKE + (1 << 29)
    a.new_tok_stride, a.new_head_stride = 8 * 128, 128
    a.batch_idx, a.positions = FAKE + (1 << 28), FAKE + (1 << 27)
    a.num_tokens, a.batch = 64, 32
    a.k_pages, a.v_pages = FAKE + (1 << 31), FAKE + (1 << 32)
    a.page_stride, a.tok_stride, a.head_stride = 16 * 8 * 128, 8 * 128, 128
    a.num_k_pages = a.num_v_pages = 100
    if i8:
        a.k_scales, a.v_scales = FAKE + (2 << 32), FAKE + (3 << 32)
        a.scale_page_stride, a.scale_tok_stride, a.scale_head_stride = 16 * 8 * 4, 8 * 4, 4
    a.page_table, a.table_stride = FAKE, 256
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("over,status", [
    ({}, 0), (dict(num_tokens=0), 0), (dict(batch=0), 0),
    (dict(num_tokens=0, k_new=None, v_new=None, batch_idx=None, positions=None), 0),
    (dict(k_new=None), 1), (dict(v_new=None), 1), (dict(batch_idx=None), 1),
    (dict(positions=None), 1), (dict(k_pages=None), 1), (dict(page_table=None), 1),
    (dict(num_tokens=-1), 2), (dict(batch=-1), 2), (dict(num_k_pages=0), 2),
    (dict(k_new=FAKE + 8), 3), (dict(new_head_stride=100), 3), (dict(new_tok_stride=-8), 3),
    (dict(v_pages=FAKE + 8), 3), (dict(tok_stride=1020), 3), (dict(table_stride=255), 3),
    (dict(k_scales=FAKE), 4),
])
def test_append_check_f16(over, status):
    p = plan()
    assert bd.skvd_append_check(p.handle, good_append_args(**over)) == status


@pytest.mark.parametrize("over,status", [
    ({}, 0), (dict(k_scales=None), 4), (dict(v_scales=None), 4), (dict(k_pages=FAKE + 8), 3),
    (dict(tok_stride=8 * 128 + 8), 3), (dict(tok_stride=8 * 128 + 16), 0),
    (dict(k_scales=FAKE + 2), 3), (dict(scale_tok_stride=34), 3),
])
def test_append_check_int8(over, status):
    p = plan(kv_dtype="i8")
    assert bd.skvd_append_check(p.handle, good_append_args(i8=True, **over)) == status


def test_append_check_null_plan():
    assert bd.skvd_append_check(None, good_append_args()) == 1


@pytest.mark.parametrize("over,status", [
    ({}, 0), (dict(q_per_seq=8), 0), (dict(q_per_seq=4096), 0), (dict(q_per_seq=1), 0),
    (dict(q_per_seq=0), 2), (dict(q_per_seq=4097), 2), (dict(batch=33), 2),
    (dict(q=None), 1), (dict(q_head_stride=100), 3), (dict(k_scales=FAKE), 4),
])
def test_prefill_check(over, status):
    """The prefill route takes any token count up to max_kv_len and needs no workspace."""
    p = plan()
    a = good_args(p, **dict(dict(q_per_seq=512), **over))
    assert bd.skvd_prefill_check(p.handle, a) == status


@pytest.mark.parametrize("over,status", [
    (dict(o_states=None), 1), (dict(lse_states=None), 1), (dict(o=None), 1),
    (dict(num_states=0), 2), (dict(rows=-1), 2), (dict(head_dim=96), 2),
    (dict(o_states=FAKE + 8), 3), (dict(o_row_stride=132), 3), (dict(o=FAKE + 8), 3),
    (dict(lse_states=FAKE + 2), 3), (dict(o_state_stride=-128), 3),
])
def test_merge_states_errors(over, status):
    """Invalid merges are refused before any launch (the error paths need no GPU)."""
    a = dict(o_states=FAKE, o_state_stride=1024 * 128, o_row_stride=128, lse_states=FAKE,
             lse_state_stride=1024, num_states=2, rows=1024, head_dim=128, o=FAKE, lse=FAKE,
             stream=None)
    a.update(over)
    assert bd.skvd_merge_states(*a.values()) == status
    assert skvd.last_error()


def test_attention_routes_errors():
    """skvd_attention reports the errors of the route it takes (no launch on the CPU)."""
    p = plan()
    assert bd.skvd_attention(None, good_args(p), None, 0, None) == 1
    # T <= max_q_per_seq: the decode route, which wants its workspace
    assert bd.skvd_attention(p.handle, good_args(p), None, p.workspace_bytes, None) == 5
    # T above the plan's bound: the tiled route; its checks (here a bad q stride) apply
    assert bd.skvd_attention(p.handle, good_args(p, q_per_seq=64, q_head_stride=100), None, 0,
                             None) == 3


@pytest.mark.parametrize("over,status", [
    ({}, 0), (dict(k_scales=None), 4), (dict(v_scales=None), 4), (dict(k_pages=FAKE + 8), 3),
    (dict(tok_stride=8 * 64 + 8), 3), (dict(tok_stride=8 * 64 + 16), 0),
    (dict(head_stride=64 + 4), 3), (dict(scale_tok_stride=34), 3), (dict(k_scales=FAKE + 4), 3),
])
def test_decode_check_q4(over, status):
    """q4_0 cache: pools addressed in bytes (rows of D/2 = 64 code bytes, strides multiples of
    16 bytes), f16 scale pools laid out as int8's."""
    p = plan(kv_dtype="q4")
    a = good_args(p, i8=True, **dict(dict(page_stride=16 * 8 * 64, tok_stride=8 * 64,
                                          head_stride=64), **over))
    assert bd.skvd_decode_check(p.handle, a, p.workspace_bytes) == status


def test_q4_plan_and_routes():
    """q4_0 plans at head_dim 128, 256 and 512 (not 192); the append takes the scale pools;
    so does the multi-token route (head_dim 128 and 256)."""
    p = plan(kv_dtype="q4")
    assert p.kv_dtype == "q4" and "kv=q4_0" in p.describe() and p.info.heads_per_wg == 4
    for D in (256, 512):
        assert plan(kv_dtype="q4", head_dim=D).kv_dtype == "q4"
    with pytest.raises(skvd.SkvdError) as e:
        plan(kv_dtype="q4", head_dim=192)
    assert e.value.status == 2
    a = good_append_args(i8=True, page_stride=16 * 8 * 64, tok_stride=8 * 64, head_stride=64)
    assert bd.skvd_append_check(p.handle, a) == 0
    assert bd.skvd_append_check(p.handle, good_append_args(page_stride=16 * 8 * 64,
                                                           tok_stride=8 * 64,
                                                           head_stride=64)) == 4  # no scales
    d = good_args(p, i8=True, q_per_seq=512, page_stride=16 * 8 * 64, tok_stride=8 * 64,
                  head_stride=64)
    assert bd.skvd_prefill_check(p.handle, d) == 0
    p512 = plan(kv_dtype="q4", head_dim=512)
    d512 = good_args(p512, i8=True, q_per_seq=512, page_stride=16 * 8 * 256, tok_stride=8 * 256,
                     head_stride=256)
    assert bd.skvd_prefill_check(p512.handle, d512) == 2  # head_dim 512: not on this route


def test_plan_waves_per_cu_by_format():
    """Workgroups per CU chosen per format (256 CUs): at head_dim 128 with one query-row quarter,
    f16 4 KV heads x 1 workgroup, int8 and fp8 4 x 3; at head_dim 256, f16 three workgroups
    per CU (one wave per SIMD), the one-byte formats eight (two waves per SIMD)."""
    def grid(**kw):
        d = plan(**kw).describe()
        return int(d.split("grid=")[1].split()[0]), int(d.split("heads_per_wg=")[1].split()[0])
    assert grid(kv_dtype="f16") == (256, 4)
    assert grid(kv_dtype="i8") == (768, 4)
    assert grid(kv_dtype="f8") == (768, 4)
    wide = dict(num_qo_heads=32, num_kv_heads=16, head_dim=256, max_batch=8, max_q_per_seq=4,
                max_kv_len=32768)
    assert grid(kv_dtype="f16", **wide) == (768, 1)
    assert grid(kv_dtype="i8", **wide) == (2048, 1)
    assert grid(kv_dtype="f8", **wide) == (2048, 1)
    assert grid(kv_dtype="q4", **wide) == (2048, 1)

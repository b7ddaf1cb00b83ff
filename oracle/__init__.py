"""fp64 CPU oracle for paged decode attention, and for appending to the paged cache (test
infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package. The HIP library never calls it and shares no code with it. The
arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over rows); this module only builds
that file with gcc and marshals numpy arrays into it.

The decode functions take the problem as the dict that ``workloads.generate`` returns (numpy
arrays: q, k_pages, v_pages, k_scales, v_scales, page_table, kv_len; ints: q_per_seq; float:
sm_scale). ``append`` takes new K/V rows and their (sequence, position) pairs and returns
written copies of the pools; ``merge_states`` merges attention states over disjoint key sets. Strides are read from the arrays themselves, in elements.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


class OracleProblem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("q_per_seq", ctypes.c_int32),
        ("num_qo_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("kv_int8", ctypes.c_int32), ("pad0", ctypes.c_int32),
        ("sm_scale", ctypes.c_double),
        ("q", ctypes.c_void_p), ("q_tok_stride", ctypes.c_int64), ("q_head_stride", ctypes.c_int64),
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("page_stride", ctypes.c_int64), ("tok_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64),
        ("s_page_stride", ctypes.c_int64), ("s_tok_stride", ctypes.c_int64), ("s_head_stride", ctypes.c_int64),
        ("table", ctypes.c_void_p), ("table_stride", ctypes.c_int64),
        ("kv_len", ctypes.c_void_p),
        ("k_fp8_scale", ctypes.c_double), ("v_fp8_scale", ctypes.c_double),
    ]


class OracleAppendProblem(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("kv_int8", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("max_len", ctypes.c_int32), ("pad0", ctypes.c_int32),
        ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
        ("new_tok_stride", ctypes.c_int64), ("new_head_stride", ctypes.c_int64),
        ("batch_idx", ctypes.c_void_p), ("positions", ctypes.c_void_p),
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("page_stride", ctypes.c_int64), ("tok_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64),
        ("num_k_pages", ctypes.c_int64), ("num_v_pages", ctypes.c_int64),
        ("s_page_stride", ctypes.c_int64), ("s_tok_stride", ctypes.c_int64), ("s_head_stride", ctypes.c_int64),
        ("table", ctypes.c_void_p), ("table_stride", ctypes.c_int64),
        ("k_fp8_scale", ctypes.c_float), ("v_fp8_scale", ctypes.c_float),
    ]


def build(out_path: str = _LIB_PATH, mutant: int = 0) -> str:
    """Compile oracle.c with gcc (-O2 -fopenmp, no fast-math). mutant > 0 plants the
    numbered deliberate mistake (used only to show that the pins catch it)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
           f"-DORACLE_MUTANT={int(mutant)}", _SRC, "-o", out_path + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out_path + ".tmp", out_path)
    return out_path


def load(path: str | None = None):
    """Load the oracle library (building it if it is missing)."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p) or (path is None and os.path.getmtime(p) < os.path.getmtime(_SRC)):
        build(p)
    lib = ctypes.CDLL(p)
    P = ctypes.POINTER(OracleProblem)
    lib.oracle_decode.argtypes = [P, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_int]
    lib.oracle_decode.restype = ctypes.c_int
    lib.oracle_decode_blocked.argtypes = [P, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_void_p, ctypes.c_void_p]
    lib.oracle_decode_blocked.restype = ctypes.c_int
    lib.oracle_gather.argtypes = [P, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p]
    lib.oracle_gather.restype = ctypes.c_int
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = ctypes.c_double
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_append.argtypes = [ctypes.POINTER(OracleAppendProblem)]
    lib.oracle_append.restype = ctypes.c_int64
    lib.oracle_float_to_half.argtypes = [ctypes.c_float]
    lib.oracle_float_to_half.restype = ctypes.c_uint16
    lib.oracle_quantize_group.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p]
    lib.oracle_quantize_group.restype = None
    lib.oracle_quantize_q4_group.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.oracle_quantize_q4_group.restype = None
    lib.oracle_merge_states.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.oracle_merge_states.restype = ctypes.c_int
    lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_to_double.restype = ctypes.c_double
    lib.oracle_e4m3_from_float.argtypes = [ctypes.c_float]
    lib.oracle_e4m3_from_float.restype = ctypes.c_uint8
    if path is None:
        _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def kv_format(k_pages, head_dim: int) -> int:
    """Cache format code of a pool: 0 f16, 1 int8 (int8 elements), 2 fp8 E4M3 (uint8, one
    byte per element), 3 q4_0 (uint8 rows of head_dim / 2 bytes: two 4-bit codes per byte)."""
    if k_pages.dtype == np.float16:
        return 0
    if k_pages.dtype == np.int8:
        return 1
    assert k_pages.dtype == np.uint8
    if k_pages.shape[3] * 2 == head_dim:
        return 3
    assert k_pages.shape[3] == head_dim
    return 2


def _problem(prob: dict):
    """Build the ctypes problem struct; returns (struct, keep-alive list)."""
    q, k, v = prob["q"], prob["k_pages"], prob["v_pages"]
    fmt = kv_format(k, q.shape[2])
    int8, fp8, q4 = fmt == 1, fmt == 2, fmt == 3
    assert q.dtype == np.float16 and q.ndim == 3 and q.strides[2] == 2
    assert k.shape == v.shape and k.strides == v.strides and k.ndim == 4
    table = np.ascontiguousarray(prob["page_table"], dtype=np.int32)
    kv_len = np.ascontiguousarray(prob["kv_len"], dtype=np.int32)
    es = k.itemsize
    B = kv_len.shape[0]
    T = int(prob["q_per_seq"])
    s = OracleProblem()
    s.batch, s.q_per_seq = B, T
    s.num_qo_heads, s.num_kv_heads, s.head_dim = q.shape[1], k.shape[2], q.shape[2]
    s.page_size = k.shape[1]
    s.kv_int8 = fmt
    s.sm_scale = float(np.float32(prob["sm_scale"]))
    if fp8:
        s.k_fp8_scale = float(np.float32(np.asarray(prob["k_scales"]).reshape(-1)[0]))
        s.v_fp8_scale = float(np.float32(np.asarray(prob["v_scales"]).reshape(-1)[0]))
    s.q = q.ctypes.data
    s.q_tok_stride, s.q_head_stride = q.strides[0] // 2, q.strides[1] // 2
    s.k, s.v = k.ctypes.data, v.ctypes.data
    s.page_stride, s.tok_stride, s.head_stride = (k.strides[0] // es, k.strides[1] // es,
                                                  k.strides[2] // es)
    keep = [q, k, v, table, kv_len]
    if int8 or q4:
        ks, vs = prob["k_scales"], prob["v_scales"]
        assert ks.dtype == np.float16 and ks.strides == vs.strides
        s.k_scale, s.v_scale = ks.ctypes.data, vs.ctypes.data
        s.s_page_stride, s.s_tok_stride, s.s_head_stride = (ks.strides[0] // 2, ks.strides[1] // 2,
                                                            ks.strides[2] // 2)
        keep += [ks, vs]
    s.table = table.ctypes.data
    s.table_stride = table.shape[1]
    s.kv_len = kv_len.ctypes.data
    return s, keep


def decode(prob: dict, rows=None, nthreads: int = 0, lib=None):
    """fp64 o [nrows, D] and lse [nrows] for the given flat rows r = (b*T + t)*Hq + h
    (all rows when None)."""
    lib = lib or load()
    s, keep = _problem(prob)
    D = s.head_dim
    total = s.batch * s.q_per_seq * s.num_qo_heads
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = total if r is None else r.shape[0]
    o = np.empty((n, D), np.float64)
    lse = np.empty((n,), np.float64)
    rc = lib.oracle_decode(ctypes.byref(s), _ptr(r), n, o.ctypes.data, lse.ctypes.data, nthreads)
    if rc != 0:
        raise RuntimeError("oracle_decode failed")
    return o, lse


def decode_blocked(prob: dict, block: int, rows=None, lib=None):
    """The same rows in split form over blocks of `block` tokens (self-check of the merge)."""
    lib = lib or load()
    s, keep = _problem(prob)
    D = s.head_dim
    total = s.batch * s.q_per_seq * s.num_qo_heads
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = total if r is None else r.shape[0]
    o = np.empty((n, D), np.float64)
    lse = np.empty((n,), np.float64)
    rc = lib.oracle_decode_blocked(ctypes.byref(s), _ptr(r), n, int(block), o.ctypes.data,
                                   lse.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle_decode_blocked failed")
    return o, lse


def gather(prob: dict, max_len: int, lib=None):
    """Raw dense copies of every visible K/V row: (dense_k, dense_v, dense_ks, dense_vs) of
    shape [B, max_len, Hkv, D] (q4_0: D/2 code bytes; and [B, max_len, Hkv, D/32] scales for
    int8 and q4_0); positions at or beyond kv_len are zero."""
    lib = lib or load()
    s, keep = _problem(prob)
    B, Hkv, D = s.batch, s.num_kv_heads, s.head_dim
    dt = prob["k_pages"].dtype
    row = D // 2 if s.kv_int8 == 3 else D
    dk = np.zeros((B, max_len, Hkv, row), dt)
    dv = np.zeros((B, max_len, Hkv, row), dt)
    dks = dvs = None
    if s.kv_int8 in (1, 3):
        dks = np.zeros((B, max_len, Hkv, D // 32), np.float16)
        dvs = np.zeros((B, max_len, Hkv, D // 32), np.float16)
    rc = lib.oracle_gather(ctypes.byref(s), int(max_len), dk.ctypes.data, dv.ctypes.data,
                           _ptr(dks), _ptr(dvs))
    if rc != 0:
        raise RuntimeError("oracle_gather failed")
    return dk, dv, dks, dvs


def num_threads() -> int:
    return int(load().oracle_num_threads())


def append(k_new, v_new, batch_idx, positions, page_table, max_len, k_pages, v_pages,
           k_scales=None, v_scales=None, batch=None, lib=None):
    """Write new K/V rows into copies of the pools. k_new, v_new: f16 [N, Hkv, D] (same
    strides); batch_idx, positions: int [N]; page_table [B, stride] int32; pools as in the
    decode problem (int8 and q4_0 pools take f16 scale pools; fp8 pools, uint8 E4M3 bytes, take
    one f32 scale each; q4_0 pools are uint8 rows of D/2 bytes). Returns (k, v, ks, vs,
    skipped): the written copies (ks, vs None for f16, the scales unchanged for fp8) and the
    number of tokens skipped."""
    lib = lib or load()
    kn, vn = k_new, v_new
    assert kn.dtype == np.float16 and kn.shape == vn.shape and kn.strides == vn.strides
    assert kn.ndim == 3 and kn.strides[2] == 2
    fmt = kv_format(k_pages, kn.shape[2])
    int8, fp8, q4 = fmt == 1, fmt == 2, fmt == 3
    k, v = k_pages.copy(), v_pages.copy()
    bi = np.ascontiguousarray(batch_idx, dtype=np.int32)
    ps = np.ascontiguousarray(positions, dtype=np.int32)
    table = np.ascontiguousarray(page_table, dtype=np.int32)
    es = k.itemsize
    s = OracleAppendProblem()
    s.num_tokens, s.num_kv_heads, s.head_dim = kn.shape[0], k.shape[2], kn.shape[2]
    s.page_size, s.kv_int8 = k.shape[1], fmt
    s.batch = table.shape[0] if batch is None else int(batch)
    s.max_len = int(max_len)
    s.k_new, s.v_new = kn.ctypes.data, vn.ctypes.data
    s.new_tok_stride, s.new_head_stride = kn.strides[0] // 2, kn.strides[1] // 2
    s.batch_idx, s.positions = bi.ctypes.data, ps.ctypes.data
    s.k, s.v = k.ctypes.data, v.ctypes.data
    s.page_stride, s.tok_stride, s.head_stride = (k.strides[0] // es, k.strides[1] // es,
                                                  k.strides[2] // es)
    s.num_k_pages, s.num_v_pages = k.shape[0], v.shape[0]
    ks = vs = None
    if int8 or q4:
        ks, vs = k_scales.copy(), v_scales.copy()
        s.k_scale, s.v_scale = ks.ctypes.data, vs.ctypes.data
        s.s_page_stride, s.s_tok_stride, s.s_head_stride = (ks.strides[0] // 2, ks.strides[1] // 2,
                                                            ks.strides[2] // 2)
    if fp8:
        ks = np.asarray(k_scales, np.float32).reshape(-1).copy()
        vs = np.asarray(v_scales, np.float32).reshape(-1).copy()
        s.k_fp8_scale, s.v_fp8_scale = float(ks[0]), float(vs[0])
    s.table, s.table_stride = table.ctypes.data, table.shape[1]
    skipped = lib.oracle_append(ctypes.byref(s))
    return k, v, ks, vs, int(skipped)


def float_to_half_bits(x: float, lib=None) -> int:
    """f32 -> f16 bits, nearest even (the oracle's own conversion)."""
    return int((lib or load()).oracle_float_to_half(float(np.float32(x))))


def e4m3_to_float(codes, lib=None):
    """OCP E4M3 bytes -> their values (fp64), by the oracle's own decoding."""
    lib = lib or load()
    c = np.asarray(codes, np.uint8).reshape(-1)
    return np.array([lib.oracle_e4m3_to_double(int(x)) for x in c]).reshape(np.shape(codes))


def e4m3_from_float(x, lib=None):
    """f32 values -> E4M3 bytes by the oracle's fp8 append rule (nearest, ties to even,
    saturating at +-448, NaN -> 0)."""
    lib = lib or load()
    a = np.asarray(x, np.float32).reshape(-1)
    return np.array([lib.oracle_e4m3_from_float(float(v)) for v in a],
                    np.uint8).reshape(np.shape(x))


def quantize_group(x, lib=None):
    """One group of f16 elements -> (int8 codes, f16 scale) by the oracle's int8 append rule."""
    lib = lib or load()
    xb = np.ascontiguousarray(x, dtype=np.float16)
    codes = np.empty(xb.shape[0], np.int8)
    sb = np.empty(1, np.uint16)
    lib.oracle_quantize_group(xb.ctypes.data, xb.shape[0], codes.ctypes.data, sb.ctypes.data)
    return codes, sb.view(np.float16)[0]


def quantize_q4_group(x, lib=None):
    """One group of 32 f16 elements -> (16 code bytes, f16 scale) by the oracle's q4_0 append
    rule (byte i: element i in the low nibble, element i + 16 in the high nibble)."""
    lib = lib or load()
    xb = np.ascontiguousarray(x, dtype=np.float16)
    assert xb.shape == (32,)
    codes = np.empty(16, np.uint8)
    sb = np.empty(1, np.uint16)
    lib.oracle_quantize_q4_group(xb.ctypes.data, codes.ctypes.data, sb.ctypes.data)
    return codes, sb.view(np.float16)[0]


def merge_states(o_states, lse_states, lib=None):
    """Merge S attention states per row: o_states [S, rows, D] (any float dtype, widened to
    fp64 exactly), lse_states [S, rows] (natural log). Returns fp64 (o [rows, D], lse [rows])."""
    lib = lib or load()
    o_s = np.ascontiguousarray(o_states, dtype=np.float64)
    l_s = np.ascontiguousarray(lse_states, dtype=np.float64)
    S, rows, D = o_s.shape
    assert l_s.shape == (S, rows)
    o = np.empty((rows, D), np.float64)
    lse = np.empty((rows,), np.float64)
    rc = lib.oracle_merge_states(S, rows, D, o_s.ctypes.data, l_s.ctypes.data, o.ctypes.data,
                                 lse.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle_merge_states failed")
    return o, lse

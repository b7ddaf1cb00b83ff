"""Seeded synthetic inputs for paged decode attention.

This module only builds inputs: it draws lengths, page permutations and N(0,1) values, and
for the int8 cache it builds the stored int8 values and f16 scales from N(0,1) data (the
scale pools stored head-major within each page, see head_major), and for
the fp8 cache the E4M3 bytes of N(0,1) data under a drawn per-tensor scale. It holds
none of the decode's arithmetic, so both the HIP path and the CPU oracle consume its arrays.

Workloads (synthetic stand-ins; the pages measure whole models whose weights are absent):

  1 tiny_mha         B=1,  T=1, Hq=8,  Hkv=8,  D=128, P=16, kv_len 256, identity page table
  2 gqa_batch        B=32, T=1, Hq=32, Hkv=8,  D=128, P=16, kv_len uniform [1024, 4096]
  3 long_ctx         B=1,  T=1, Hq=32, Hkv=8,  D=128, P=64, kv_len 131072, q scaled x2
  4 wide_multitoken  B=8,  T=4, Hq=32, Hkv=16, D=256, P=16, kv_len uniform [8192, 32768]
  5 int8_batch       B=64, T=1, Hq=32, Hkv=8,  D=128, P=16, kv_len Zipf(1.1) clipped
                     to [512, 65536], int8 K/V with one f16 scale per 32 elements

Recipe: numpy.random.default_rng(seed) draws (1) kv_len, then (2) the page permutation. Then
(3) q, (4) the K pool and (5) the V pool are N(0,1) values drawn in float32 and rounded to f16
(round to nearest even), each array from its own streams: chunk c of 4 Mi elements of array k
comes from PCG64(SeedSequence(seed, spawn_key=(k, c))), so the values do not depend on the
thread count. For the int8 cache the same float32 draws are quantized, which draws nothing.
Pools hold sum_b ceil(L_b/P) live pages plus ceil(live/16) spare pages; page ids are a random
permutation consumed in sequence order.
fp8 cache (kv_dtype "f8", uint8 OCP E4M3 bytes): k_scale and v_scale (one f32 each, arrays of
shape [1]) are uniform in [1/80, 1/64] from default_rng((seed, 8)); the pools' N(0,1) draws
(streams 4 and 5, as for f16) divided by the scale, clipped to +-448, become E4M3 bytes by
torch's float8_e4m3fn cast (nearest even), which draws nothing.
q4_0 cache (kv_dtype "q4", uint8 rows of D/2 bytes, two 4-bit codes per byte; value =
(c - 8) * d, one f16 d per 32 elements, scale pools head-major as int8's): the N(0,1) draws
(streams 4 and 5) made into codes by quantize_q4, which draws nothing.
Spare pages and the tail slots past kv_len of each sequence's last page are NaN-poisoned
(for int8 and q4_0: their scales are NaN; fp8: the NaN byte 0x7F), so any read of them shows
up in the output.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Spec:
    name: str
    batch: int
    q_per_seq: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    kv_dtype: str = "f16"           # "f16", "i8", "f8" or "q4"
    lens: tuple = ("fixed", 256)     # ("fixed", L) | ("uniform", lo, hi) | ("zipf", s, lo, hi) | ("list", (..))
    q_mult: float = 1.0
    identity_table: bool = False
    spare_frac: float = 1.0 / 16.0
    poison: bool = True

    @property
    def max_kv_len(self) -> int:
        kind = self.lens[0]
        if kind == "fixed":
            return int(self.lens[1])
        if kind == "uniform":
            return int(self.lens[2])
        if kind == "zipf":
            return int(self.lens[3])
        return int(max(self.lens[1]))

    @property
    def group(self) -> int:
        return self.num_qo_heads // self.num_kv_heads


CONFIGS = {
    1: Spec("tiny_mha", 1, 1, 8, 8, 128, 16, "f16", ("fixed", 256), identity_table=True),
    2: Spec("gqa_batch", 32, 1, 32, 8, 128, 16, "f16", ("uniform", 1024, 4096)),
    3: Spec("long_ctx", 1, 1, 32, 8, 128, 64, "f16", ("fixed", 131072), q_mult=2.0),
    4: Spec("wide_multitoken", 8, 4, 32, 16, 256, 16, "f16", ("uniform", 8192, 32768)),
    5: Spec("int8_batch", 64, 1, 32, 8, 128, 16, "i8", ("zipf", 1.1, 512, 65536)),
}


# The int8 batch's shape over the other quantized cache: q4_0 codes with the same f16 scales
# per 32 elements (the cache type the pages name beside q8_0).
VARIANT_CONFIGS = {
    "q4_batch": Spec("q4_batch", 64, 1, 32, 8, 128, 16, "q4", ("zipf", 1.1, 512, 65536)),
}


def config(i: int) -> Spec:
    return CONFIGS[int(i)]


def spec(name="custom", batch=1, q_per_seq=1, num_qo_heads=4, num_kv_heads=2, head_dim=128,
         page_size=16, kv_dtype="f16", lens=("fixed", 64), **kw) -> Spec:
    return Spec(name, batch, q_per_seq, num_qo_heads, num_kv_heads, head_dim, page_size,
                kv_dtype, tuple(lens), **kw)


def draw_lengths(s: Spec, rng) -> np.ndarray:
    kind = s.lens[0]
    if kind == "fixed":
        L = np.full(s.batch, int(s.lens[1]), np.int64)
    elif kind == "uniform":
        L = rng.integers(int(s.lens[1]), int(s.lens[2]) + 1, size=s.batch)
    elif kind == "zipf":
        L = np.clip(rng.zipf(float(s.lens[1]), size=s.batch), int(s.lens[2]), int(s.lens[3]))
    elif kind == "list":
        L = np.asarray(s.lens[1], np.int64)
        assert L.shape == (s.batch,)
    else:
        raise ValueError(kind)
    return L.astype(np.int32)


_CHUNK = 1 << 22  # elements per independently seeded chunk (a multiple of 32 and of D)


def _chunk_rng(seed: int, stream: int, chunk: int):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(stream, chunk))))


def _parallel(fn, n):
    from concurrent.futures import ThreadPoolExecutor
    import os
    workers = max(1, min(16, os.cpu_count() or 1))
    if n <= 1 or workers == 1:
        for i in range(n):
            fn(i)
        return
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(fn, range(n)))


def _normal_f16(seed, stream, shape, mult=1.0):
    """N(0,1) (times mult) drawn in float32 and rounded to f16. Chunk c of the flattened array
    comes from its own generator seeded by (seed, stream, c), so the values do not depend on
    how many threads fill them."""
    out = np.empty(shape, np.float16)
    flat = out.reshape(-1)
    n = flat.shape[0]

    def fill(c):
        a, b = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        x = _chunk_rng(seed, stream, c).standard_normal(b - a, dtype=np.float32)
        if mult != 1.0:
            x *= np.float32(mult)
        flat[a:b] = x.astype(np.float16)

    _parallel(fill, -(-n // _CHUNK))
    return out


def quantize_int8(x: np.ndarray):
    """Symmetric int8 with one f16 scale per 32 contiguous elements of the last axis:
    scale = f16(max|x| / 127), q = clip(rint(x / scale), -127, 127); an all-zero group gets
    scale 0 and q 0. Returns (q int8 [..., D], scale f16 [..., D/32])."""
    D = x.shape[-1]
    g = x.reshape(x.shape[:-1] + (D // 32, 32)).astype(np.float32)
    amax = np.abs(g).max(axis=-1)
    scale = (amax / np.float32(127.0)).astype(np.float16)
    sf = scale.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        qv = np.where(sf > 0, np.rint(g / np.where(sf > 0, sf, 1)), 0)
    qv = np.clip(qv, -127, 127).astype(np.int8)
    return qv.reshape(x.shape), scale


def quantize_q4(x: np.ndarray):
    """4-bit codes with one f16 scale per 32 contiguous elements of the last axis (the q4_0
    layout: value = (c - 8) * d, codes 0..15): d = f16(max|x| / 8), c = clip(rint(x / d) + 8,
    0, 15), an all-zero group d = 0 and c = 8 -- a plain input recipe, not the append's rule.
    Returns (packed uint8 [..., D/2]: byte i of a group holds element i in its low nibble and
    element i + 16 in its high nibble, scale f16 [..., D/32])."""
    D = x.shape[-1]
    g = x.reshape(x.shape[:-1] + (D // 32, 32)).astype(np.float32)
    amax = np.abs(g).max(axis=-1)
    scale = (amax / np.float32(8.0)).astype(np.float16)
    sf = scale.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.where(sf > 0, np.rint(g / np.where(sf > 0, sf, 1)), 0) + 8
    c = np.clip(c, 0, 15).astype(np.uint8)
    packed = c[..., :16] | (c[..., 16:] << 4)
    return packed.reshape(x.shape[:-1] + (D // 2,)), scale


def _normal_q4(seed, stream, shape):
    """N(0,1) data (drawn as in _normal_f16) as q4_0 codes + f16 scales."""
    D = shape[-1]
    q = np.empty(tuple(shape[:-1]) + (D // 2,), np.uint8)
    sc = np.empty(tuple(shape[:-1]) + (D // 32,), np.float16)
    qf, sf = q.reshape(-1), sc.reshape(-1)
    n = int(np.prod(shape))

    def fill(c):
        a, b = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        x = _chunk_rng(seed, stream, c).standard_normal(b - a, dtype=np.float32)
        qq, ss = quantize_q4(x.reshape(-1, 32))
        qf[a // 2:b // 2] = qq.reshape(-1)
        sf[a // 32:b // 32] = ss.reshape(-1)

    _parallel(fill, -(-n // _CHUNK))
    return q, sc


def _normal_int8(seed, stream, shape):
    """N(0,1) data (drawn as in _normal_f16) quantized to int8 + f16 scales."""
    q = np.empty(shape, np.int8)
    sc = np.empty(tuple(shape[:-1]) + (shape[-1] // 32,), np.float16)
    qf, sf = q.reshape(-1), sc.reshape(-1)
    n = qf.shape[0]

    def fill(c):
        a, b = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        x = _chunk_rng(seed, stream, c).standard_normal(b - a, dtype=np.float32)
        qq, ss = quantize_int8(x.reshape(-1, 32))
        qf[a:b] = qq.reshape(-1)
        sf[a // 32:b // 32] = ss.reshape(-1)

    _parallel(fill, -(-n // _CHUNK))
    return q, sc


def head_major(sc: np.ndarray) -> np.ndarray:
    """The same [pages, P, Hkv, D/32] scales stored head-major within each page (memory order
    [pages, Hkv, P, D/32]): the int8 cache's scale layout, in which one KV head's scales of a
    16-token tile are 128 contiguous bytes. Returns a strided view; the values are unchanged."""
    return np.ascontiguousarray(sc.transpose(0, 2, 1, 3)).transpose(0, 2, 1, 3)


def _normal_e4m3(seed, stream, shape, scale):
    """N(0,1) data (drawn as in _normal_f16) over a per-tensor scale, as E4M3 bytes: x / scale
    in f32, clipped to +-448, cast by torch to float8_e4m3fn (nearest even)."""
    import torch
    out = np.empty(shape, np.uint8)
    flat = out.reshape(-1)
    n = flat.shape[0]
    sc = np.float32(scale)

    def fill(c):
        a, b = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        x = _chunk_rng(seed, stream, c).standard_normal(b - a, dtype=np.float32)
        y = np.clip(x / sc, np.float32(-448), np.float32(448))
        flat[a:b] = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()

    _parallel(fill, -(-n // _CHUNK))
    return out


def fp8_scales(seed):
    """(k_scale, v_scale): one f32 each, arrays of shape [1], uniform in [1/80, 1/64]."""
    r = np.random.default_rng((seed, 8)).uniform(1 / 80, 1 / 64, 2).astype(np.float32)
    return r[:1].copy(), r[1:].copy()


def generate(s: Spec, seed: int) -> dict:
    """Build one problem. Returns a dict of numpy arrays and ints:
    q [B*T, Hq, D] f16; k_pages, v_pages [N, P, Hkv, D] f16, int8 or uint8 (E4M3), or
    [N, P, Hkv, D/2] uint8 (q4_0 codes); k_scales, v_scales [N, P, Hkv, D/32] f16 (int8, q4_0),
    [1] f32 (fp8) or None; page_table [B, ceil(max_kv_len/P)] int32 (-1 past each
    sequence's pages); kv_len [B] int32; q_per_seq; sm_scale (f32 value 1/sqrt(D)); spec."""
    rng = np.random.default_rng(seed)
    B, T, Hq, Hkv, D, P = (s.batch, s.q_per_seq, s.num_qo_heads, s.num_kv_heads, s.head_dim,
                           s.page_size)
    # (1) lengths
    L = draw_lengths(s, rng)
    maxL = max(s.max_kv_len, int(L.max()) if L.size else 0, 1)
    max_pages = -(-maxL // P)
    npages = (L.astype(np.int64) + P - 1) // P
    live = int(npages.sum())
    # (2) page permutation
    table = np.full((B, max_pages), -1, np.int32)
    if s.identity_table:
        N = max(live, 1)
        perm = np.arange(N)
    else:
        spare = int(math.ceil(live * s.spare_frac)) if s.spare_frac > 0 else 0
        N = max(live + spare, 1)
        perm = rng.permutation(N)
    off = 0
    for b in range(B):
        table[b, :npages[b]] = perm[off:off + npages[b]]
        off += int(npages[b])
    # (3) q
    q = _normal_f16(seed, 3, (B * T, Hq, D), s.q_mult)
    # (4), (5) pools, then (6) quantization for int8
    ks = vs = None
    if s.kv_dtype == "f16":
        k = _normal_f16(seed, 4, (N, P, Hkv, D))
        v = _normal_f16(seed, 5, (N, P, Hkv, D))
    elif s.kv_dtype == "i8":
        k, ks = _normal_int8(seed, 4, (N, P, Hkv, D))
        v, vs = _normal_int8(seed, 5, (N, P, Hkv, D))
        ks, vs = head_major(ks), head_major(vs)
    elif s.kv_dtype == "q4":
        k, ks = _normal_q4(seed, 4, (N, P, Hkv, D))
        v, vs = _normal_q4(seed, 5, (N, P, Hkv, D))
        ks, vs = head_major(ks), head_major(vs)
    elif s.kv_dtype == "f8":
        ks, vs = fp8_scales(seed)
        k = _normal_e4m3(seed, 4, (N, P, Hkv, D), ks[0])
        v = _normal_e4m3(seed, 5, (N, P, Hkv, D), vs[0])
    else:
        raise ValueError(s.kv_dtype)
    if s.poison:
        poison_unread(k, v, ks, vs, table, L, P, perm[off:] if not s.identity_table else [])
    return dict(q=q, k_pages=k, v_pages=v, k_scales=ks, v_scales=vs, page_table=table,
                kv_len=L, q_per_seq=T, sm_scale=float(np.float32(1.0 / math.sqrt(D))), spec=s)


def poison_unread(k, v, ks, vs, table, L, P, spare_pages):
    """NaN-poison what a correct decode never reads: spare pages and tail slots."""
    spare = np.asarray(spare_pages, np.int64)
    if ks is not None and ks.dtype == np.float16:  # int8 and q4_0: NaN scales
        nan = np.float16(np.nan)
        if spare.size:
            ks[spare] = nan
            vs[spare] = nan
            k[spare] = 127 if k.dtype == np.int8 else 0xFF
            v[spare] = 127 if k.dtype == np.int8 else 0xFF
        for b in range(L.shape[0]):
            if L[b] % P:
                last = table[b, (L[b] - 1) // P]
                ks[last, L[b] % P:] = nan
                vs[last, L[b] % P:] = nan
    elif k.dtype == np.uint8:
        nan = np.uint8(0x7F)  # the E4M3 NaN byte
        if spare.size:
            k[spare] = nan
            v[spare] = nan
        for b in range(L.shape[0]):
            if L[b] % P:
                last = table[b, (L[b] - 1) // P]
                k[last, L[b] % P:] = nan
                v[last, L[b] % P:] = nan
    else:
        nan = np.float16(np.nan)
        if spare.size:
            k[spare] = nan
            v[spare] = nan
        for b in range(L.shape[0]):
            if L[b] % P:
                last = table[b, (L[b] - 1) // P]
                k[last, L[b] % P:] = nan
                v[last, L[b] % P:] = nan


def append_tokens(prob: dict, seed: int, new_per_seq: int):
    """New K/V rows for an append: the last new_per_seq positions of every sequence (positions
    kv_len_b - n .. kv_len_b - 1 that exist), visited in a random order. Values are N(0,1)
    rounded to f16 from streams 6 (K) and 7 (V) of `seed`; the order comes from
    default_rng((seed, 7)). Returns dict(k_new, v_new [N, Hkv, D] f16, batch_idx, positions
    [N] int32)."""
    k = prob["k_pages"]
    Hkv, D = k.shape[2], prob["q"].shape[2]
    L = np.asarray(prob["kv_len"], np.int64)
    n = np.minimum(L, int(new_per_seq))
    bi = np.concatenate([np.full(int(n[b]), b) for b in range(L.shape[0])] + [np.zeros(0)])
    pos = np.concatenate([np.arange(L[b] - n[b], L[b]) for b in range(L.shape[0])] + [np.zeros(0)])
    order = np.random.default_rng((seed, 7)).permutation(bi.shape[0])
    N = int(bi.shape[0])
    return dict(k_new=_normal_f16(seed, 6, (N, Hkv, D)), v_new=_normal_f16(seed, 7, (N, Hkv, D)),
                batch_idx=bi[order].astype(np.int32), positions=pos[order].astype(np.int32))


# Append workloads: (cache spec, new tokens per sequence). A prefill chunk of 1024 tokens for
# each of 32 sequences (the GQA batch's cache shape; int8, f16, fp8 and q4_0 caches), and one decode
# step (one token for each of 64 sequences, the int8 batch's cache shape).
APPEND_CONFIGS = {
    "prefill_i8": (Spec("append_prefill_i8", 32, 1, 32, 8, 128, 16, "i8", ("fixed", 1024)), 1024),
    "prefill_f16": (Spec("append_prefill_f16", 32, 1, 32, 8, 128, 16, "f16", ("fixed", 1024)), 1024),
    "decode_i8": (Spec("append_decode_i8", 64, 1, 32, 8, 128, 16, "i8", ("fixed", 1024)), 1),
    "prefill_f8": (Spec("append_prefill_f8", 32, 1, 32, 8, 128, 16, "f8", ("fixed", 1024)), 1024),
    "prefill_q4": (Spec("append_prefill_q4", 32, 1, 32, 8, 128, 16, "q4", ("fixed", 1024)), 1024),
}


# Prefill workloads (the multi-token route): 4 prompts of 2048 tokens each processed at once
# against their own 2048 cached positions (full causal), the GQA batch's head shape; int8 and
# f16 caches. T = 2048 query tokens per sequence.
PREFILL_CONFIGS = {
    "prompt_i8": Spec("prefill_prompt_i8", 4, 2048, 32, 8, 128, 16, "i8", ("fixed", 2048)),
    "prompt_f16": Spec("prefill_prompt_f16", 4, 2048, 32, 8, 128, 16, "f16", ("fixed", 2048)),
    "prompt_f8": Spec("prefill_prompt_f8", 4, 2048, 32, 8, 128, 16, "f8", ("fixed", 2048)),
    "prompt_q4": Spec("prefill_prompt_q4", 4, 2048, 32, 8, 128, 16, "q4", ("fixed", 2048)),
}


def attention_flops(prob: dict) -> int:
    """Algorithmic FLOPs of one attention call: 4*D per (query row, visible position) pair
    (2*D for q.k, 2*D for p*v), visible positions per the causal reading."""
    D = prob["q"].shape[2]
    Hq = prob["q"].shape[1]
    T = int(prob["q_per_seq"])
    L = np.asarray(prob["kv_len"], np.int64)
    t = np.arange(T, dtype=np.int64)
    vis = np.clip(L[:, None] - T + t[None, :] + 1, 0, None).sum()
    return int(4 * D * Hq * vis)


def _row_pair_bytes(k, D: int) -> int:
    if k.dtype == np.float16:
        return 4 * D
    if k.dtype == np.uint8 and k.shape[3] * 2 == D:  # q4_0: D/2 code bytes + D/32 f16 scales
        return 2 * (D // 2 + 2 * (D // 32))
    if k.dtype == np.uint8:
        return 2 * D
    return 2 * (D + 2 * (D // 32))


def append_bytes(prob: dict, new: dict) -> int:
    """Algorithmic bytes of one append: the new K and V rows read (2*D*2 bytes per token-head)
    plus the cache written (2*D*2 bytes for f16; 2*(D + 2*D/32) for int8 with f16 scales; 2*D
    for fp8; 2*(D/2 + 2*D/32) for q4_0)."""
    k = prob["k_pages"]
    Hkv, D = k.shape[2], new["k_new"].shape[2]
    written = _row_pair_bytes(k, D)
    return int(new["k_new"].shape[0]) * Hkv * (4 * D + written)


def kv_bytes(prob: dict) -> int:
    """Algorithmic K+V bytes one decode reads: sum_b kv_len_b * Hkv * row bytes, where a row
    pair is 2*D*2 bytes for f16, 2*(D + 2*D/32) bytes for int8 with f16 scales, 2*D bytes
    for fp8 (its two per-tensor scales are not per row) and 2*(D/2 + 2*D/32) for q4_0."""
    k = prob["k_pages"]
    Hkv, D = k.shape[2], prob["q"].shape[2]
    row = _row_pair_bytes(k, D)
    return int(np.asarray(prob["kv_len"], np.int64).sum()) * Hkv * row


def with_lengths(s: Spec, lens) -> Spec:
    return replace(s, lens=("list", tuple(int(x) for x in lens)), batch=len(lens))

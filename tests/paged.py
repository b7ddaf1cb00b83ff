"""Test-side builders: scatter dense K/V into a paged pool and dense references.

``paged_from_dense`` is the construction a pin needs: it writes a known dense cache into
randomly permuted pages (optionally with extra heads so that the pool is a strided view), so
that a correct gather must give the dense cache back. ``dense_reference`` computes attention
on the dense cache with torch's fp64 CPU ``scaled_dot_product_attention`` (a library routine,
independent of the oracle's C code).
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F


def paged_from_dense(rng, q, Kd, Vd, L, P, *, T=1, spare=3, extra_heads=0, Ks=None, Vs=None,
                     sm_scale=None, table_pad=2):
    """q [B*T, Hq, D] f16; Kd, Vd [B, Lmax, Hkv, D] (f16, int8, or uint8 E4M3 bytes); Ks, Vs
    [B, Lmax, Hkv, D/32] f16 scales for int8, or the [1] f32 tensor scales for E4M3. Returns a problem dict whose pools hold position j of sequence b at
    page table[b, j // P], slot j % P, with pages randomly permuted among spare NaN pages."""
    B, Lmax, Hkv, D = Kd.shape
    L = np.asarray(L, np.int32)
    npages = (L.astype(np.int64) + P - 1) // P
    live = int(npages.sum())
    N = live + spare
    perm = rng.permutation(N)
    Hs = Hkv + extra_heads
    int8 = Kd.dtype == np.int8
    if Kd.dtype == np.uint8:
        kbig = np.full((N, P, Hs, D), 0x7F, np.uint8)  # the E4M3 NaN byte
        vbig = np.full((N, P, Hs, D), 0x7F, np.uint8)
    elif int8:
        kbig = np.full((N, P, Hs, D), 127, np.int8)
        vbig = np.full((N, P, Hs, D), 127, np.int8)
        ksb = np.full((N, P, Hs, D // 32), np.nan, np.float16)
        vsb = np.full((N, P, Hs, D // 32), np.nan, np.float16)
    else:
        kbig = np.full((N, P, Hs, D), np.nan, np.float16)
        vbig = np.full((N, P, Hs, D), np.nan, np.float16)
    maxp = int(max(npages.max() if B else 0, 1)) + table_pad
    table = np.full((B, maxp), -1, np.int32)
    off = 0
    for b in range(B):
        for i in range(npages[b]):
            pg = perm[off + i]
            table[b, i] = pg
            j0, j1 = i * P, min((i + 1) * P, int(L[b]))
            kbig[pg, :j1 - j0, :Hkv] = Kd[b, j0:j1]
            vbig[pg, :j1 - j0, :Hkv] = Vd[b, j0:j1]
            if int8:
                ksb[pg, :j1 - j0, :Hkv] = Ks[b, j0:j1]
                vsb[pg, :j1 - j0, :Hkv] = Vs[b, j0:j1]
        off += int(npages[b])
    prob = dict(q=q, k_pages=kbig[:, :, :Hkv], v_pages=vbig[:, :, :Hkv], k_scales=None,
                v_scales=None, page_table=table, kv_len=L, q_per_seq=T,
                sm_scale=float(np.float32(sm_scale if sm_scale is not None else 1 / math.sqrt(D))))
    if int8:
        prob["k_scales"] = ksb[:, :, :Hkv]
        prob["v_scales"] = vsb[:, :, :Hkv]
    if Kd.dtype == np.uint8:
        prob["k_scales"] = np.asarray(Ks, np.float32).reshape(1)
        prob["v_scales"] = np.asarray(Vs, np.float32).reshape(1)
    return prob


def e4m3_values(x):
    """OCP E4M3 bytes -> fp64 values by torch's float8_e4m3fn decoding (a library routine)."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def dequant(x, s):
    """Stored int8 values times their f16 scale (one per 32 elements), or E4M3 bytes times the
    tensor's f32 scale, in fp64."""
    if x.dtype == np.uint8:
        return e4m3_values(x) * float(np.asarray(s, np.float32).reshape(-1)[0])
    if s is None:
        return x.astype(np.float64)
    return x.astype(np.float64) * np.repeat(s.astype(np.float64), 32, axis=-1)


def dense_reference(q, Kd, Vd, L, T, sm_scale, Ks=None, Vs=None):
    """fp64 o [B*T, Hq, D] and lse [B*T, Hq] by torch SDPA on the dense cache, with the query
    tokens as the last T positions (token t sees positions j <= L - T + t)."""
    Kf, Vf = dequant(Kd, Ks), dequant(Vd, Vs)
    BT, Hq, D = q.shape
    B = BT // T
    Hkv = Kd.shape[2]
    o = np.zeros((BT, Hq, D))
    lse = np.full((BT, Hq), -np.inf)
    for b in range(B):
        n = int(L[b])
        if n == 0:
            continue
        qb = torch.from_numpy(q[b * T:(b + 1) * T].astype(np.float64)).permute(1, 0, 2)[None]
        kb = torch.from_numpy(Kf[b, :n]).permute(1, 0, 2)[None].contiguous()
        vb = torch.from_numpy(Vf[b, :n]).permute(1, 0, 2)[None].contiguous()
        mask = torch.from_numpy(np.arange(n)[None, :] <= (n - T + np.arange(T))[:, None])
        ob = F.scaled_dot_product_attention(qb, kb, vb, attn_mask=mask, scale=float(sm_scale),
                                            enable_gqa=True)
        o[b * T:(b + 1) * T] = ob[0].permute(1, 0, 2).numpy()
        kr = kb.repeat_interleave(Hq // Hkv, dim=1)
        logits = float(sm_scale) * (qb @ kr.transpose(-1, -2))
        logits = logits.masked_fill(~mask, -math.inf)
        lse[b * T:(b + 1) * T] = torch.logsumexp(logits, dim=-1)[0].permute(1, 0).numpy()
    return o, lse


def random_dense(rng, B, Lmax, Hkv, D, int8=False):
    if not int8:
        K = rng.standard_normal((B, Lmax, Hkv, D), dtype=np.float32).astype(np.float16)
        V = rng.standard_normal((B, Lmax, Hkv, D), dtype=np.float32).astype(np.float16)
        return K, V, None, None
    K = rng.integers(-127, 128, size=(B, Lmax, Hkv, D)).astype(np.int8)
    V = rng.integers(-127, 128, size=(B, Lmax, Hkv, D)).astype(np.int8)
    Ks = (rng.uniform(0.005, 0.05, size=(B, Lmax, Hkv, D // 32))).astype(np.float16)
    Vs = (rng.uniform(0.005, 0.05, size=(B, Lmax, Hkv, D // 32))).astype(np.float16)
    return K, V, Ks, Vs

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
                     sm_scale=None, table_pad=2, q4=False):
    """q [B*T, Hq, D] f16; Kd, Vd [B, Lmax, Hkv, D] (f16, int8, or uint8 E4M3 bytes; with q4,
    [B, Lmax, Hkv, D/2] uint8 q4_0 code bytes); Ks, Vs [B, Lmax, Hkv, D/32] f16 scales for int8
    and q4_0, or the [1] f32 tensor scales for E4M3. Returns a problem dict whose pools hold
    position j of sequence b at page table[b, j // P], slot j % P, with pages randomly permuted
    among spare NaN pages."""
    B, Lmax, Hkv, D = Kd.shape
    L = np.asarray(L, np.int32)
    npages = (L.astype(np.int64) + P - 1) // P
    live = int(npages.sum())
    N = live + spare
    perm = rng.permutation(N)
    Hs = Hkv + extra_heads
    q4 = q4 or (Kd.dtype == np.uint8 and 2 * D == q.shape[2])  # D/2 code bytes per row
    int8 = Kd.dtype == np.int8 or q4
    if q4:
        kbig = np.full((N, P, Hs, D), 0xFF, np.uint8)
        vbig = np.full((N, P, Hs, D), 0xFF, np.uint8)
        ksb = np.full((N, P, Hs, 2 * D // 32), np.nan, np.float16)
        vsb = np.full((N, P, Hs, 2 * D // 32), np.nan, np.float16)
    elif Kd.dtype == np.uint8:
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
    Dq = 2 * D if q4 else D
    prob = dict(q=q, k_pages=kbig[:, :, :Hkv], v_pages=vbig[:, :, :Hkv], k_scales=None,
                v_scales=None, page_table=table, kv_len=L, q_per_seq=T,
                sm_scale=float(np.float32(sm_scale if sm_scale is not None else 1 / math.sqrt(Dq))))
    if int8:
        prob["k_scales"] = ksb[:, :, :Hkv]
        prob["v_scales"] = vsb[:, :, :Hkv]
    if Kd.dtype == np.uint8 and not q4:
        prob["k_scales"] = np.asarray(Ks, np.float32).reshape(1)
        prob["v_scales"] = np.asarray(Vs, np.float32).reshape(1)
    return prob


def e4m3_values(x):
    """OCP E4M3 bytes -> fp64 values by torch's float8_e4m3fn decoding (a library routine)."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def dequant(x, s):
    """Stored int8 values times their f16 scale (one per 32 elements), q4_0 code bytes (uint8
    with f16 scales) as (c - 8) * scale, or E4M3 bytes times the tensor's f32 scale, in fp64."""
    if x.dtype == np.uint8 and s is not None and np.asarray(s).dtype == np.float16:
        return q4_values(x, s)
    if x.dtype == np.uint8:
        return e4m3_values(x) * float(np.asarray(s, np.float32).reshape(-1)[0])
    if s is None:
        return x.astype(np.float64)
    return x.astype(np.float64) * np.repeat(s.astype(np.float64), 32, axis=-1)


def q4_pack(c):
    """4-bit codes [..., D] (0..15) -> q4_0 bytes [..., D/2]: in each group of 32, byte i holds
    code i in its low nibble and code i + 16 in its high nibble."""
    c = np.asarray(c, np.uint8)
    g = c.reshape(c.shape[:-1] + (c.shape[-1] // 32, 2, 16))
    return (g[..., 0, :] | (g[..., 1, :] << 4)).reshape(c.shape[:-1] + (c.shape[-1] // 2,))


def q4_values(codes, scales):
    """q4_0 bytes [..., D/2] and f16 scales [..., D/32] -> fp64 values (c - 8) * scale."""
    b = np.asarray(codes, np.uint8)
    g = b.reshape(b.shape[:-1] + (b.shape[-1] // 16, 1, 16))
    c = np.concatenate([g & 15, g >> 4], axis=-2).reshape(b.shape[:-1] + (2 * b.shape[-1],))
    return (c.astype(np.float64) - 8) * np.repeat(np.asarray(scales).astype(np.float64), 32,
                                                  axis=-1)


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


def quantize_dense(x, kv, rng_scale=None):
    """f32 dense rows -> the stored form of cache format kv: f16 values; int8 codes and f16
    scales (the workload generator's quantizer); q4_0 code bytes and f16 scales (likewise); or
    E4M3 bytes (torch's nearest-even cast of x / scale, clipped to +-448) with a [1] f32 tensor
    scale. Returns (stored, scales)."""
    import workloads
    if kv == "f16":
        return x.astype(np.float16), None
    if kv == "i8":
        return workloads.quantize_int8(x.astype(np.float32))
    if kv == "q4":
        return workloads.quantize_q4(x.astype(np.float32))
    scale = np.float32(1 / 64 if rng_scale is None else rng_scale)
    y = np.clip(x.astype(np.float32) / scale, np.float32(-448), np.float32(448))
    b = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return b, np.array([scale], np.float32)


def dominant_problem(rng, B, T, Hq, Hkv, D, P, L, kv, positions, *, beta=32.0, noise=0.25,
                     spare=3):
    """A problem whose every (sequence b, KV head g) has one dominant key: K rows are
    noise * N(0,1) except row positions[b][g] = alpha * u[b,g], and every query row of the
    group is beta * u[b,g] plus 0.3 * N(0,1), u a random unit vector. alpha is set so that the
    dominant logit exceeds every other visible one by >= 40 (checked on the stored values), so
    o is that position's V row to within e^-40 * L. positions[b][g] <= L[b] - T. Returns the
    problem dict and the dequantized dominant V rows [B, Hkv, D] (fp64)."""
    L = np.asarray(L, np.int32)
    G = Hq // Hkv
    Lmax = int(L.max())
    sm = 1.0 / math.sqrt(D)
    u = rng.standard_normal((B, Hkv, D))
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    K = (noise * rng.standard_normal((B, Lmax, Hkv, D))).astype(np.float32)
    V = rng.standard_normal((B, Lmax, Hkv, D)).astype(np.float32)
    # the noise keys' largest logit is about sm * beta * noise * 4.5; the dominant one
    # sm * beta * alpha
    alpha = (44.0 + sm * beta * noise * 5.0) / (sm * beta)
    for b in range(B):
        for g in range(Hkv):
            p = int(positions[b][g])
            assert 0 <= p <= L[b] - T, (b, g, p, L[b])
            K[b, p, g] = alpha * u[b, g]
    q = np.empty((B * T, Hq, D), np.float32)
    for b in range(B):
        for h in range(Hq):
            q[b * T:(b + 1) * T, h] = beta * u[b, h // G] + 0.3 * rng.standard_normal((T, D))
    q = q.astype(np.float16)
    Kd, Ks = quantize_dense(K, kv)
    Vd, Vs = quantize_dense(V, kv)
    prob = paged_from_dense(rng, q, Kd, Vd, L, P, T=T, spare=spare, Ks=Ks, Vs=Vs, sm_scale=sm)
    Kf, Vf = dequant(Kd, Ks), dequant(Vd, Vs)
    dom = np.empty((B, Hkv, D))
    q64 = q.astype(np.float64)
    for b in range(B):
        for g in range(Hkv):
            p = int(positions[b][g])
            dom[b, g] = Vf[b, p, g]
            for t in range(T):
                n = int(L[b]) - T + t + 1
                s = sm * (Kf[b, :n, g] @ q64[b * T + t, g * G:(g + 1) * G].T)  # [n, G]
                gap = s[p] - np.delete(s, p, axis=0).max(axis=0) if n > 1 else np.full(G, 99.0)
                assert gap.min() >= 40.0, (b, g, t, gap.min())
    return prob, dom


def identical_key_problem(rng, B, T, Hq, Hkv, D, P, L, kv, spare=3):
    """Every visible K row of (sequence b, KV head g) is the same vector; V rows random. The
    softmax is then uniform over a row's n visible positions: o = mean of its n V rows and
    lse = s + ln n with s the one logit. Returns the problem and the dequantized dense K, V."""
    L = np.asarray(L, np.int32)
    Lmax = int(L.max())
    k0 = rng.standard_normal((B, 1, Hkv, D)).astype(np.float32)
    K = np.repeat(k0, Lmax, axis=1)
    V = rng.standard_normal((B, Lmax, Hkv, D)).astype(np.float32)
    q = (2.0 * rng.standard_normal((B * T, Hq, D))).astype(np.float16)
    Kd, Ks = quantize_dense(K, kv)
    Vd, Vs = quantize_dense(V, kv)
    prob = paged_from_dense(rng, q, Kd, Vd, L, P, T=T, spare=spare, Ks=Ks, Vs=Vs,
                            sm_scale=1.0 / math.sqrt(D))
    return prob, dequant(Kd, Ks), dequant(Vd, Vs)

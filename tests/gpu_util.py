"""Helpers for the GPU tests: move a generated problem to the device, run the library through
its C ABI (via the binding), and compare with the oracle at the decode's tolerance."""
from __future__ import annotations

import sys

import numpy as np
import torch

O_TOL = 2e-3    # max |o_gpu - o_oracle|   (f16 output, f32 accumulation)
LSE_TOL = 1e-3  # max |lse_gpu - lse_oracle|


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(prob, device="cuda:0", layout="nhd"):
    """The problem's arrays on the device. layout "hnd": the K/V pools and int8 / q4_0 scale
    pools [N, P, Hkv, X] are stored as [N, Hkv, P, X] (each KV head's page rows contiguous) and
    passed as the permuted view, so the kernels see the HND strides with the same values."""
    d = {}
    for k in ("q", "k_pages", "v_pages", "k_scales", "v_scales", "page_table", "kv_len"):
        v = prob.get(k)
        if v is None:
            d[k] = None
        elif layout == "hnd" and k in ("k_pages", "v_pages", "k_scales", "v_scales") and v.ndim == 4:
            d[k] = torch.from_numpy(np.ascontiguousarray(v.transpose(0, 2, 1, 3))).to(
                device).permute(0, 2, 1, 3)
        else:
            d[k] = torch.from_numpy(np.ascontiguousarray(v) if k in
                                    ("page_table", "kv_len") else v).to(device)
    return d


def make_plan(prob, **kw):
    import quantized_kv_cache_page_amd as skvd
    k = prob["k_pages"]
    D = prob["q"].shape[2]
    s = dict(num_qo_heads=prob["q"].shape[1], num_kv_heads=k.shape[2], head_dim=D,
             page_size=k.shape[1],
             kv_dtype="q4" if k.dtype == np.uint8 and 2 * k.shape[3] == D else
             {np.dtype(np.float16): "f16", np.dtype(np.int8): "i8",
              np.dtype(np.uint8): "f8"}[k.dtype],
             max_batch=len(prob["kv_len"]), max_q_per_seq=int(prob["q_per_seq"]),
             max_kv_len=max(int(prob["page_table"].shape[1] * k.shape[1]), 1), device=0)
    s.update(kw)
    return skvd.Plan(**s)


def run(plan, prob, dev, out=None, lse=None, stage="all"):
    return plan.run(dev["q"], dev["k_pages"], dev["v_pages"], dev["page_table"], dev["kv_len"],
                    prob["sm_scale"], dev["k_scales"], dev["v_scales"], out=out, lse=lse,
                    q_per_seq=int(prob["q_per_seq"]), stage=stage)


def compare(o, lse, ref_o, ref_lse, rows=None, what=""):
    """o [B*T, Hq, D] f16 and lse [B*T, Hq] from the GPU vs fp64 oracle rows."""
    D = o.shape[-1]
    go = o.reshape(-1, D).float().cpu().numpy().astype(np.float64)
    gl = lse.reshape(-1).cpu().numpy().astype(np.float64)
    if rows is not None:
        go, gl = go[rows], gl[rows]
    do = np.abs(go - ref_o)
    finite = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(gl), finite), f"{what}: lse finiteness differs"
    dl = np.abs(gl[finite] - ref_lse[finite]) if finite.any() else np.zeros(1)
    mo, ml = float(np.nanmax(do)) if do.size else 0.0, float(dl.max()) if dl.size else 0.0
    say(f"  {what}: max|do|={mo:.2e} max|dlse|={ml:.2e}")
    assert np.isfinite(go).all(), f"{what}: non-finite o"
    assert mo <= O_TOL, f"{what}: max|do|={mo}"
    assert ml <= LSE_TOL, f"{what}: max|dlse|={ml}"
    return mo, ml

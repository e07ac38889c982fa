"""Independent float64 reference built from library routines (torch CPU), used
only to pin the oracle.  It shares nothing with the oracle's C code: the
append uses torch's own fp32 add, its RNE casts to float16/bfloat16 and
torch.round (half-to-even); the attention uses torch's float64 matmul and
softmax, or scaled_dot_product_attention.

Conventions it encodes (the readings the oracle also takes): L_b counts the
appended token, the new row goes to position L_b - 1, the bias is one
[b_q | b_k | b_v] vector, query head h reads KV head h // (H / H_kv), the
softmax scale is 1/sqrt(D), and the new row enters the attention as stored.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


def to_torch(a: np.ndarray, dt: str) -> torch.Tensor:
    if dt == "bf16":
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    return torch.from_numpy(a.copy())


def from_torch(t: torch.Tensor, dt: str) -> np.ndarray:
    if dt == "bf16":
        return t.contiguous().view(torch.int16).numpy().view(np.uint16).copy()
    return t.contiguous().numpy().copy()


def ref_step(q, k_new, v_new, bias, k_cache, v_cache, seq_lens, step, H, Hkv, D, kv_dtype,
             kv_scales=None, use_sdpa=False):
    """Returns (out float64 [B,H,D], k_cache', v_cache', kv_scales') with the
    caches as numpy arrays in their stored types."""
    act = "f16" if kv_dtype == "i8" else kv_dtype
    B = q.shape[0]
    G = H // Hkv
    qt = to_torch(q, act).double()
    kn = to_torch(k_new, act).float()
    vn = to_torch(v_new, act).float()
    if bias is not None:
        bt = to_torch(bias, act).float()
        bq = bt[: H * D].view(H, D).double()
        bk = bt[H * D:(H + Hkv) * D].view(Hkv, D)
        bv = bt[(H + Hkv) * D:].view(Hkv, D)
    else:
        bq = torch.zeros(H, D, dtype=torch.float64)
        bk = bv = None
    kc = to_torch(k_cache, kv_dtype)
    vc = to_torch(v_cache, kv_dtype)
    sc = torch.from_numpy(kv_scales.copy()) if kv_scales is not None else None
    lens = [int(x) for x in (seq_lens if seq_lens is not None else [step] * B)]
    out = torch.full((B, H, D), float("nan"), dtype=torch.float64)
    for b in range(B):
        L = lens[b]
        if L < 1 or L > step:
            continue
        p = L - 1
        for which, (src, bb, cache) in enumerate(((kn, bk, kc), (vn, bv, vc))):
            x = src[b] + bb if bb is not None else src[b]          # fp32 add
            if kv_dtype == "f32":
                cache[b, :, p] = x
            elif kv_dtype == "f16":
                cache[b, :, p] = x.to(torch.float16)
            elif kv_dtype == "bf16":
                cache[b, :, p] = x.to(torch.bfloat16)
            else:
                s = x.abs().amax(dim=-1) / 127.0                   # fp32 divide
                codes = torch.where(s[:, None] > 0, torch.round(x / s[:, None]).clamp(-127, 127),
                                    torch.zeros_like(x))
                cache[b, :, p] = codes.to(torch.int8)
                sc[which, b, :, p] = s
        for h in range(H):
            j = h // G
            if kv_dtype == "i8":
                K = kc[b, j, :L].double() * sc[0, b, j, :L].double()[:, None]
                V = vc[b, j, :L].double() * sc[1, b, j, :L].double()[:, None]
            else:
                K = kc[b, j, :L].double()
                V = vc[b, j, :L].double()
            qh = qt[b, h] + bq[h]
            if use_sdpa:
                o = F.scaled_dot_product_attention(qh.view(1, 1, 1, D), K.view(1, 1, L, D),
                                                   V.view(1, 1, L, D))
                out[b, h] = o.view(D)
            else:
                s = (K @ qh) / np.sqrt(D)
                out[b, h] = torch.softmax(s, dim=0) @ V
    return (out.numpy(), from_torch(kc, kv_dtype), from_torch(vc, kv_dtype),
            sc.numpy() if sc is not None else None)

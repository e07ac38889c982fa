"""Pins of the QKV projection oracle (oracle.qkv_proj).  CPU only.

The projection is y = x W^T (+ bias) followed by a three-way split of the
features into Q [B, H, D], K [B, Hkv, D] and V [B, Hkv, D]
([lpnh.cn/news/2765398] section 2.1).  Each pin ties it to something other
than its own matmul:
  * routing: rows of W that pick one input element move that element,
    exactly, to the output position the split assigns;
  * a brute-force sum in pure Python (math.fsum, exact rounding of the sum);
  * bias: adding a bias adds it, and scaling W by 2 scales y by 2 exactly;
  * rounding to the activation type matches torch's casts."""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import to_np


def rand_act(shape, dt, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    t = (torch.randn(shape, generator=g) * scale).to({"f16": torch.float16, "bf16": torch.bfloat16}[dt])
    return to_np(t, dt)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("H,Hkv,D", [(4, 4, 8), (8, 2, 16), (6, 3, 4)])
def test_routing_places_each_feature(dt, H, Hkv, D):
    B, hidden = 3, 64
    N = (H + 2 * Hkv) * D
    x = rand_act((B, hidden), dt, seed=1)
    perm = np.random.default_rng(2).integers(0, hidden, N)
    one = np.float16(1.0) if dt == "f16" else np.uint16(0x3F80)     # 1.0 (bfloat16 bit pattern)
    w = np.zeros((N, hidden), dtype=x.dtype)
    w[np.arange(N), perm] = one
    q, k, v = oracle.qkv_proj(x, w, None, H, Hkv, D, dt)
    xf = oracle.cache_to_f64(x, dt)
    for b in range(B):
        for f in range(N):
            want = xf[b, perm[f]]
            if f < H * D:
                got = q[b, f // D, f % D]
            elif f < (H + Hkv) * D:
                got = k[b, (f - H * D) // D, f % D]
            else:
                got = v[b, (f - (H + Hkv) * D) // D, f % D]
            assert got == want, (b, f)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_brute_force_sum(dt):
    B, H, Hkv, D, hidden = 2, 2, 1, 4, 24
    N = (H + 2 * Hkv) * D
    x = rand_act((B, hidden), dt, seed=3)
    w = rand_act((N, hidden), dt, seed=4, scale=0.2)
    bias = rand_act((N,), dt, seed=5)
    q, k, v = oracle.qkv_proj(x, w, bias, H, Hkv, D, dt)
    y = np.concatenate([q.reshape(B, -1), k.reshape(B, -1), v.reshape(B, -1)], axis=1)
    xf, wf, bf = (oracle.cache_to_f64(a, dt) for a in (x, w, bias))
    for b in range(B):
        for f in range(N):
            exact = math.fsum([float(xf[b, i]) * float(wf[f, i]) for i in range(hidden)] + [float(bf[f])])
            assert abs(y[b, f] - exact) <= 1e-12 * max(1.0, abs(exact)), (b, f)


def test_bias_and_scaling():
    dt = "bf16"
    B, H, Hkv, D, hidden = 4, 4, 2, 8, 32
    N = (H + 2 * Hkv) * D
    x = rand_act((B, hidden), dt, seed=6)
    w = rand_act((N, hidden), dt, seed=7)
    bias = rand_act((N,), dt, seed=8)
    y0 = np.concatenate([a.reshape(B, -1) for a in oracle.qkv_proj(x, w, None, H, Hkv, D, dt)], axis=1)
    y1 = np.concatenate([a.reshape(B, -1) for a in oracle.qkv_proj(x, w, bias, H, Hkv, D, dt)], axis=1)
    assert np.allclose(y1 - y0, oracle.cache_to_f64(bias, dt)[None, :], rtol=0, atol=1e-12)
    # doubling every weight doubles every output exactly (a power of two)
    w2 = (torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).float() * 2).to(torch.bfloat16)
    y2 = np.concatenate([a.reshape(B, -1) for a in oracle.qkv_proj(x, to_np(w2, dt), None, H, Hkv, D, dt)],
                        axis=1)
    assert np.array_equal(y2, 2 * y0)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_round_to_act_matches_torch(dt):
    y = np.random.default_rng(9).standard_normal(5000) * 3
    y = np.concatenate([y, [0.0, -0.0, 1e-9, 65504.0, 1e5]])
    got = oracle.round_to_act(y, dt)
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    # torch rounds float64 -> fp32 -> target; via fp32 is exact for both here
    want = to_np(torch.from_numpy(y).float().to(tdt), dt)
    assert got.view(np.uint16).tobytes() == want.view(np.uint16).tobytes()

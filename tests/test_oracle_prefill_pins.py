"""Pins of the prefill oracle (oracle.prefill_mha).  CPU only.

Prefill computes, for every prompt position t, what a decode step at length
t + 1 computes ([lpnh.cn/news/2765398] section 1.1: the prompt is processed
in parallel, then decode goes token by token).  So the strongest pin is the
decode oracle itself, which is pinned on its own (tests/test_oracle_pins.py):
running S decode steps one position at a time must give the same outputs at
every position and byte-identical caches.  Closed forms add two more: the
first position sees only itself (out = stored V row, exactly), and identical
keys give the running mean of V."""
import numpy as np
import pytest

import oracle
from decode_step_attention_amd import workloads as W
from tests.helpers import to_np


def prompt(dt, B, H, Hkv, D, S, Lmax, seed):
    case = W.Case("pf", B, H, Hkv, D, dt, ctx=S, max_seq_len=Lmax, value_scale=0.5, seed=seed)
    import torch
    g = torch.Generator().manual_seed(seed)
    tdt = W.TORCH_DTYPES[dt]
    r = lambda *shape: to_np((torch.randn(shape, generator=g) * 0.5).to(tdt), dt)
    q, kn, vn = r(B, S, H, D), r(B, S, Hkv, D), r(B, S, Hkv, D)
    bias = r((H + 2 * Hkv) * D)
    poison = np.uint16(0x7fc0) if dt == "bf16" else np.float16(np.nan)
    kc = np.full((B, Hkv, Lmax, D), poison, dtype=q.dtype)
    vc = kc.copy()
    return case, q, kn, vn, bias, kc, vc


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("H,Hkv", [(4, 4), (4, 2), (6, 1)])
def test_prefill_is_successive_decode_steps(oracle_mod, dt, H, Hkv):
    B, D, S, Lmax = 2, 8, 9, 12
    case, q, kn, vn, bias, kc, vc = prompt(dt, B, H, Hkv, D, S, Lmax, seed=11 + H + Hkv)
    lens = np.array([S, 5], np.int32)
    kd, vd = kc.copy(), vc.copy()           # the same poisoned caches, for the decode steps
    out = oracle_mod.prefill_mha(q, kn, vn, bias, kc, vc, lens, H, Hkv, D, dt)
    for t in range(S):
        step_lens = np.minimum(lens, t + 1).astype(np.int32)
        active = lens > t
        # sequences past their prompt repeat their last step (same inputs,
        # same slot: the step is idempotent)
        idx = np.minimum(t, lens - 1)
        qt = np.ascontiguousarray(q[np.arange(B), idx])
        kt = np.ascontiguousarray(kn[np.arange(B), idx])
        vt = np.ascontiguousarray(vn[np.arange(B), idx])
        o, _ = oracle_mod.decode_mha(qt, kt, vt, bias, kd, vd, step_lens, int(step_lens.max()), H, Hkv, D, dt)
        for b in range(B):
            if active[b]:
                assert np.allclose(out[b, t], o[b], rtol=1e-12, atol=1e-14), (b, t)
    assert kd.tobytes() == kc.tobytes() and vd.tobytes() == vc.tobytes()
    assert np.all(out[1, 5:] == 0)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_first_position_is_its_own_value(oracle_mod, dt):
    B, H, Hkv, D, S = 2, 4, 2, 16, 6
    case, q, kn, vn, bias, kc, vc = prompt(dt, B, H, Hkv, D, S, S, seed=3)
    out = oracle_mod.prefill_mha(q, kn, vn, bias, kc, vc, None, H, Hkv, D, dt)
    for b in range(B):
        for h in range(H):
            assert np.array_equal(out[b, 0, h], oracle_mod.cache_to_f64(vc[b, h // (H // Hkv), 0], dt))


def test_identical_keys_give_running_mean(oracle_mod):
    dt = "f16"
    B, H, Hkv, D, S = 1, 2, 1, 8, 7
    case, q, kn, vn, bias, kc, vc = prompt(dt, B, H, Hkv, D, S, S, seed=5)
    kn[:] = kn[:, :1]                       # every key the same (no bias)
    out = oracle_mod.prefill_mha(q, kn, vn, None, kc, vc, None, H, Hkv, D, dt)
    V = oracle_mod.cache_to_f64(vc[0, 0], dt)
    for t in range(S):
        assert np.allclose(out[0, t, 0], V[:t + 1].mean(axis=0), rtol=0, atol=1e-15)


@pytest.mark.parametrize("H,Hkv", [(4, 4), (6, 2)])
def test_int8_prefill_is_successive_decode_steps(oracle_mod, H, Hkv):
    """INT8 cache: the same pin against the decode oracle's INT8 steps (fp16
    activations, codes and one fp32 scale per stored row); caches and scales
    must match byte for byte, poison included."""
    import torch
    B, D, S, Lmax = 2, 8, 9, 12
    g = torch.Generator().manual_seed(31 + H)
    r = lambda *shape: to_np(torch.randn(shape, generator=g).to(torch.float16), "f16")
    q, kn, vn = r(B, S, H, D), r(B, S, Hkv, D), r(B, S, Hkv, D)
    bias = r((H + 2 * Hkv) * D)
    kc = np.full((B, Hkv, Lmax, D), 77, dtype=np.int8)
    vc = kc.copy()
    sc = np.full((2, B, Hkv, Lmax), np.nan, dtype=np.float32)
    kd, vd, sd = kc.copy(), vc.copy(), sc.copy()
    lens = np.array([S, 5], np.int32)
    out = oracle_mod.prefill_mha(q, kn, vn, bias, kc, vc, lens, H, Hkv, D, "i8", sc)
    for t in range(S):
        step_lens = np.minimum(lens, t + 1).astype(np.int32)
        idx = np.minimum(t, lens - 1)
        qt = np.ascontiguousarray(q[np.arange(B), idx])
        kt = np.ascontiguousarray(kn[np.arange(B), idx])
        vt = np.ascontiguousarray(vn[np.arange(B), idx])
        o, _ = oracle_mod.decode_mha(qt, kt, vt, bias, kd, vd, step_lens, int(step_lens.max()), H, Hkv, D, "i8",
                                     sd)
        for b in range(B):
            if lens[b] > t:
                assert np.allclose(out[b, t], o[b], rtol=1e-12, atol=1e-14), (b, t)
    assert kd.tobytes() == kc.tobytes() and vd.tobytes() == vc.tobytes()
    assert np.array_equal(sd, sc, equal_nan=True)

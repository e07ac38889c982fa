"""Pins of the CPU oracle against things other than itself: exhaustive
comparisons with library number-format routines, closed forms, invariants,
special cases that reduce to a library routine, and brute force on tiny
inputs.  CPU only."""
import itertools
import math

import numpy as np
import pytest
import torch

from decode_step_attention_amd import workloads as W
from tests import torch_ref
from tests.helpers import inputs_to_np, run_oracle


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

def test_f16_decode_all_patterns(oracle_mod):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle_mod.f16_bits_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_decode_all_patterns(oracle_mod):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    got = np.array([oracle_mod.bf16_bits_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def _float_probe_values(fmt):
    """fp32 values that exercise round-to-nearest-even: random values across
    the range, exact midpoints between neighbours, the subnormal range and
    the overflow threshold."""
    rng = np.random.default_rng(7)
    vals = [rng.standard_normal(20000).astype(np.float32) * s for s in (1e-6, 1e-3, 1.0, 300.0)]
    if fmt == "f16":
        grid = np.arange(0, 65536, 97, dtype=np.uint32).astype(np.uint16).view(np.float16)
        grid = grid[np.isfinite(grid)].astype(np.float64)
        grid = np.sort(np.abs(grid))
        mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)
        vals.append(mids)
        vals.append(np.array([65504, 65519.99, 65520, 65535, 65536, 1e6, 2 ** -24, 2 ** -25,
                              3 * 2 ** -26, 2 ** -26, 5.960464477539063e-08, 0.0, -0.0,
                              np.inf, -np.inf], dtype=np.float32))
    else:
        bits = np.arange(0, 65536, 97, dtype=np.uint32) << 16
        grid = bits.view(np.float32)
        grid = np.sort(np.abs(grid[np.isfinite(grid)].astype(np.float64)))
        vals.append(((grid[:-1] + grid[1:]) / 2).astype(np.float32))
        vals.append(np.array([3.3895314e38, 3.39e38, 3.4028235e38, 1e-40, 1e-45, 0.0, -0.0,
                              np.inf, -np.inf], dtype=np.float32))
    v = np.concatenate(vals).astype(np.float32)
    return np.concatenate([v, -v])


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_float_to_half_rne_matches_library(oracle_mod, fmt):
    x = _float_probe_values(fmt)
    tdt = torch.float16 if fmt == "f16" else torch.bfloat16
    ref = torch.from_numpy(x).to(tdt).view(torch.int16).numpy().view(np.uint16)
    fn = oracle_mod.float_to_f16_rne if fmt == "f16" else oracle_mod.float_to_bf16_rne
    got = np.array([fn(float(v)) for v in x], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]
    if fmt == "f16":   # numpy's own RNE cast agrees too
        with np.errstate(over="ignore"):
            assert np.array_equal(got, x.astype(np.float16).view(np.uint16))


def test_quantize_row_matches_torch_ops(oracle_mod):
    rng = np.random.default_rng(11)
    rows = [rng.standard_normal(128).astype(np.float32) * s for s in (1.0, 1e-3, 50.0)]
    rows.append(np.zeros(128, np.float32))
    rows.append(np.full(128, -0.0, np.float32))
    # exact half-way codes: absmax = 127 * 2^-5 gives scale 2^-5 exactly, and
    # x = (k + 1/2) * 2^-5 lands on k + 1/2 after the division
    k = np.arange(-126, 126)
    tie = ((k + 0.5) * 2.0 ** -5).astype(np.float32)
    tie = np.concatenate([tie, np.array([127 * 2.0 ** -5], np.float32)])
    rows.append(tie)
    for x in rows:
        codes, s = oracle_mod.quantize_row_i8(x)
        xt = torch.from_numpy(x)
        st = xt.abs().amax() / 127.0
        ct = torch.round(xt / st).clamp(-127, 127) if st > 0 else torch.zeros_like(xt)
        assert np.float32(s).tobytes() == st.numpy().astype(np.float32).tobytes()
        assert np.array_equal(codes, ct.numpy().astype(np.int8))
    # half-to-even: k + 1/2 goes to the even neighbour
    codes, s = oracle_mod.quantize_row_i8(tie)
    assert s == 2.0 ** -5
    expect = np.where((k % 2) == 0, k, k + 1)
    assert np.array_equal(codes[:-1], expect.astype(np.int8))


# ---------------------------------------------------------------------------
# Small problems
# ---------------------------------------------------------------------------

def small_case(kv_dtype="f32", B=2, H=4, Hkv=2, D=8, ctx=6, Lmax=8, lens=None, seed=5, scale=0.5):
    return W.Case("t", B, H, Hkv, D, kv_dtype, ctx=ctx, max_seq_len=Lmax, value_scale=scale,
                  lens=lens, seed=seed)


def gen(case, poison=True):
    return inputs_to_np(W.make_inputs(case, "cpu", poison=poison), case.kv_dtype)


@pytest.mark.parametrize("kv_dtype", ["f32", "f16", "bf16", "i8"])
def test_single_token_output_is_v(oracle_mod, kv_dtype):
    """t = 1: one position, weight exactly 1, so out equals the stored new V
    row widened to double."""
    case = small_case(kv_dtype, ctx=1)
    npi = gen(case)
    out, probs = run_oracle(oracle_mod, case, npi, want_probs=True)
    G = case.group
    for b in range(case.batch):
        for h in range(case.n_heads):
            j = h // G
            if kv_dtype == "i8":
                v = npi["v_cache"][b, j, 0].astype(np.float64) * np.float64(npi["kv_scales"][1, b, j, 0])
            else:
                v = oracle_mod.cache_to_f64(npi["v_cache"][b, j, 0], kv_dtype)
            assert np.array_equal(out[b, h], v)
            assert probs[b, h, 0] == 1.0


def test_identical_keys_give_mean_of_v(oracle_mod):
    case = small_case("f32", ctx=6)
    npi = gen(case, poison=False)
    key = np.float32(np.linspace(-1, 1, case.head_dim))
    npi["k_cache"][:] = key
    npi["k_new"][:] = key
    npi["bias"][case.n_heads * case.head_dim:(case.n_heads + case.n_kv_heads) * case.head_dim] = 0
    out, probs = run_oracle(oracle_mod, case, npi, want_probs=True)
    L = case.ctx
    for b in range(case.batch):
        for h in range(case.n_heads):
            j = h // case.group
            mean = npi["v_cache"][b, j, :L].astype(np.float64).mean(axis=0)
            np.testing.assert_allclose(out[b, h], mean, rtol=0, atol=1e-15)
            np.testing.assert_allclose(probs[b, h, :L], 1.0 / L, rtol=1e-15)


@pytest.mark.parametrize("kv_dtype", ["f32", "f16", "bf16", "i8"])
def test_weights_sum_to_one_and_vanish_past_length(oracle_mod, kv_dtype):
    case = small_case(kv_dtype, B=3, ctx=7, Lmax=9, lens=(1, 7))
    npi = gen(case)
    out, probs = run_oracle(oracle_mod, case, npi, want_probs=True)
    for b in range(case.batch):
        L = int(npi["seq_lens"][b])
        assert np.all(np.abs(probs[b, :, :L].sum(axis=-1) - 1.0) <= 1e-12)
        assert np.all(probs[b, :, L:] == 0.0)
        assert np.all(probs[b, :, :L] > 0)
    assert np.isfinite(out).all()


def test_closed_form_three_positions(oracle_mod):
    """Scores 0, 1, 2 against one-hot values give
    out = (1, e, e^2, 0) / (1 + e + e^2)."""
    D = 4
    case = small_case("f32", B=1, H=1, Hkv=1, D=D, ctx=3, Lmax=3)
    npi = gen(case, poison=False)
    npi["q"][:] = np.array([2.0, 0, 0, 0], np.float32)      # q.k/sqrt(4) = k_0
    npi["bias"][:] = 0
    npi["k_cache"][0, 0, :2] = np.array([[0, 5, 5, 5], [1, -3, 2, 7]], np.float32)
    npi["k_new"][0, 0] = np.array([2, 0.5, 0.25, 9], np.float32)
    npi["v_cache"][0, 0, :2] = np.eye(4, dtype=np.float32)[:2]
    npi["v_new"][0, 0] = np.eye(4, dtype=np.float32)[2]
    out, _ = run_oracle(oracle_mod, case, npi)
    e = math.e
    ref = np.array([1, e, e * e, 0]) / (1 + e + e * e)
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-15, atol=1e-16)


SWEEP = [(B, H, Hkv, D, L, dt)
         for B in (1, 2) for H in (1, 2, 4) for Hkv in (1, 2, 4) if H % Hkv == 0
         for D in (1, 2, 4, 8) for L in (1, 2, 3, 6)
         for dt in ("f32", "f16", "bf16", "i8")]


def _sweep_subset():
    # every combination would be ~1.5k oracle calls and twice that in torch;
    # a fixed stride keeps every axis value covered
    return SWEEP[::3]


@pytest.mark.parametrize("B,H,Hkv,D,L,dt", _sweep_subset())
def test_brute_force_against_torch_float64(oracle_mod, B, H, Hkv, D, L, dt):
    case = small_case(dt, B=B, H=H, Hkv=Hkv, D=D, ctx=L, Lmax=L + 1, seed=100 + D * 7 + L)
    npi = gen(case)
    ref = torch_ref.ref_step(npi["q"], npi["k_new"], npi["v_new"], npi["bias"], npi["k_cache"],
                             npi["v_cache"], npi["seq_lens"], npi["step"], H, Hkv, D, dt,
                             npi["kv_scales"], use_sdpa=(L % 2 == 0))
    out, _ = run_oracle(oracle_mod, case, npi)
    # append: bytewise equal to torch's fp32 add + RNE cast / quantiser
    assert npi["k_cache"].tobytes() == ref[1].tobytes()
    assert npi["v_cache"].tobytes() == ref[2].tobytes()
    if dt == "i8":
        assert npi["kv_scales"].tobytes() == ref[3].tobytes()
    np.testing.assert_allclose(out, ref[0], rtol=1e-12, atol=1e-14)


def test_textbook_formula_longdouble(oracle_mod):
    """Softmax written without the max subtraction, in extended precision,
    for scores of moderate size."""
    case = small_case("f32", B=2, H=4, Hkv=2, D=8, ctx=6, Lmax=6)
    npi = gen(case, poison=False)
    snap_k, snap_v = npi["k_cache"].copy(), npi["v_cache"].copy()
    out, _ = run_oracle(oracle_mod, case, npi)
    ld = np.longdouble
    H, Hkv, D, G = 4, 2, 8, 2
    for b in range(2):
        L = 6
        for h in range(H):
            j = h // G
            K = npi["k_cache"][b, j, :L].astype(ld)
            V = npi["v_cache"][b, j, :L].astype(ld)
            qh = npi["q"][b, h].astype(ld) + npi["bias"][h * D:(h + 1) * D].astype(ld)
            s = (K * qh).sum(axis=1) / np.sqrt(ld(D))
            w = np.exp(s)
            ref = (w[:, None] * V).sum(axis=0) / w.sum()
            np.testing.assert_allclose(out[b, h], ref.astype(np.float64), rtol=1e-13, atol=1e-15)
    # prefilled rows untouched
    assert np.array_equal(npi["k_cache"][:, :, :5], snap_k[:, :, :5])
    assert np.array_equal(npi["v_cache"][:, :, :5], snap_v[:, :, :5])


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16", "i8"])
def test_permutation_invariance(oracle_mod, kv_dtype):
    """Permuting the history positions together with their V rows (and
    scales) leaves the output unchanged."""
    case = small_case(kv_dtype, B=2, H=4, Hkv=2, D=8, ctx=9, Lmax=9)
    npi = gen(case)
    base = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in npi.items()}
    out0, _ = run_oracle(oracle_mod, case, npi)
    perm = np.random.default_rng(3).permutation(8)
    per = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in base.items()}
    per["k_cache"][:, :, :8] = base["k_cache"][:, :, perm]
    per["v_cache"][:, :, :8] = base["v_cache"][:, :, perm]
    if kv_dtype == "i8":
        per["kv_scales"][:, :, :, :8] = base["kv_scales"][:, :, :, perm]
    out1, _ = run_oracle(oracle_mod, case, per)
    np.testing.assert_allclose(out1, out0, rtol=1e-13, atol=1e-15)


def test_shift_invariance_needs_stable_softmax(oracle_mod):
    """Adding one vector u to every key adds q.u/sqrt(D) to every score and
    must not change the output.  With q.u/sqrt(D) = 8192 a softmax without
    the maximum subtracted overflows double precision."""
    D = 4
    case = small_case("f32", B=1, H=1, Hkv=1, D=D, ctx=5, Lmax=5)
    npi = gen(case, poison=False)
    rng = np.random.default_rng(1)
    # dyadic keys so that adding the shift is exact in fp32
    npi["k_cache"][:] = (rng.integers(-64, 64, size=npi["k_cache"].shape) / 64.0).astype(np.float32)
    npi["k_new"][:] = (rng.integers(-64, 64, size=npi["k_new"].shape) / 64.0).astype(np.float32)
    npi["bias"][:] = 0
    npi["q"][:] = np.array([1.0, 0.5, -0.25, 0.125], np.float32)
    base = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in npi.items()}
    out0, _ = run_oracle(oracle_mod, case, npi)
    sh = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in base.items()}
    sh["k_cache"][..., 0] += np.float32(16384.0)
    sh["k_new"][..., 0] += np.float32(16384.0)
    out1, _ = run_oracle(oracle_mod, case, sh)
    assert np.isfinite(out1).all()
    np.testing.assert_allclose(out1, out0, rtol=1e-12, atol=1e-14)


def test_one_hot_limit(oracle_mod):
    """A key equal to lambda * q for large lambda takes all the weight."""
    D = 8
    case = small_case("f32", B=1, H=1, Hkv=1, D=D, ctx=6, Lmax=6)
    npi = gen(case, poison=False)
    npi["bias"][:] = 0
    qv = npi["q"][0, 0].astype(np.float64)
    npi["k_cache"][0, 0, 2] = (200.0 * qv / np.dot(qv, qv) * np.sqrt(D)).astype(np.float32)
    out, probs = run_oracle(oracle_mod, case, npi, want_probs=True)
    others = np.delete(probs[0, 0, :6], 2)
    assert probs[0, 0, 2] >= 1 - 1e-15 and np.all(others < 1e-50)
    np.testing.assert_allclose(out[0, 0], npi["v_cache"][0, 0, 2].astype(np.float64), atol=1e-12)


@pytest.mark.parametrize("kv_dtype", ["f16", "i8"])
def test_gqa_equals_mha_with_replicated_kv(oracle_mod, kv_dtype):
    """Query head h of a grouped problem reads KV head h // G: the result
    equals plain multi-head attention on a cache whose KV heads are each
    repeated G times."""
    B, H, Hkv, D = 2, 8, 2, 8
    G = H // Hkv
    case = small_case(kv_dtype, B=B, H=H, Hkv=Hkv, D=D, ctx=7, Lmax=8)
    npi = gen(case)
    rep = dict(npi)
    rep["k_cache"] = np.repeat(npi["k_cache"], G, axis=1).copy()
    rep["v_cache"] = np.repeat(npi["v_cache"], G, axis=1).copy()
    rep["k_new"] = np.repeat(npi["k_new"], G, axis=1).copy()
    rep["v_new"] = np.repeat(npi["v_new"], G, axis=1).copy()
    bq = npi["bias"][:H * D]
    bk = np.repeat(npi["bias"][H * D:(H + Hkv) * D].reshape(Hkv, D), G, axis=0).reshape(-1)
    bv = np.repeat(npi["bias"][(H + Hkv) * D:].reshape(Hkv, D), G, axis=0).reshape(-1)
    rep["bias"] = np.concatenate([bq, bk, bv])
    if kv_dtype == "i8":
        rep["kv_scales"] = np.repeat(npi["kv_scales"], G, axis=2).copy()
    out_g, _ = run_oracle(oracle_mod, case, npi)
    case_m = case.with_(n_kv_heads=H)
    out_m, _ = run_oracle(oracle_mod, case_m, rep)
    assert np.array_equal(out_g, out_m)


def test_invalid_length_gives_nan_and_no_append(oracle_mod):
    case = small_case("f16", B=3, ctx=5, Lmax=6)
    npi = gen(case, poison=False)
    npi["seq_lens"] = np.array([5, 0, 7], np.int32)   # 0 and 7 (> step 5) are invalid
    k0, v0 = npi["k_cache"].copy(), npi["v_cache"].copy()
    out, _ = run_oracle(oracle_mod, case, npi)
    assert np.isfinite(out[0]).all()
    assert np.isnan(out[1]).all() and np.isnan(out[2]).all()
    assert np.array_equal(npi["k_cache"][1:], k0[1:]) and np.array_equal(npi["v_cache"][1:], v0[1:])


@pytest.mark.parametrize("kv_dtype", ["f32", "i8"])
def test_poisoned_rows_are_never_read(oracle_mod, kv_dtype):
    """Rows past each length (and the append slot) hold NaN before the step;
    the output stays finite and equals that of a clean cache."""
    case = small_case(kv_dtype, B=3, ctx=9, Lmax=12, lens=(2, 9))
    dirty = gen(case, poison=True)
    clean = gen(case, poison=False)
    out_d, _ = run_oracle(oracle_mod, case, dirty)
    out_c, _ = run_oracle(oracle_mod, case, clean)
    assert np.isfinite(out_d).all()
    assert np.array_equal(out_d, out_c)


def test_append_touches_only_the_new_row(oracle_mod):
    case = small_case("bf16", B=2, H=4, Hkv=2, D=8, ctx=5, Lmax=8, lens=(2, 5))
    npi = gen(case, poison=False)
    k0, v0 = npi["k_cache"].copy(), npi["v_cache"].copy()
    run_oracle(oracle_mod, case, npi)
    for b in range(2):
        p = int(npi["seq_lens"][b]) - 1
        mask = np.ones(k0.shape[2], bool)
        mask[p] = False
        assert np.array_equal(npi["k_cache"][b][:, mask], k0[b][:, mask])
        assert np.array_equal(npi["v_cache"][b][:, mask], v0[b][:, mask])


def test_threads_do_not_change_the_result(oracle_mod):
    case = small_case("f16", B=4, H=8, Hkv=4, D=16, ctx=20, Lmax=24, lens=(3, 20))
    a = gen(case)
    b = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in a.items()}
    out1, _ = run_oracle(oracle_mod, case, a, n_threads=1)
    out4, _ = run_oracle(oracle_mod, case, b, n_threads=4)
    assert np.array_equal(out1, out4)
    assert a["k_cache"].tobytes() == b["k_cache"].tobytes()

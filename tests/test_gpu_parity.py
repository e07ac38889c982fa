"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.

Bar: the appended cache rows (and INT8 scales) are bit-exact and every other
byte of the caches is unchanged; out is within max-abs 1e-5 / row-rel 1e-5
for an fp32 cache and max-abs 2e-3 / row-rel 1e-2 for fp16, bf16 and INT8
caches (fp32 accumulation).  Row-rel is max_d |err| / max_d |ref| per
(b, h) row, the normwise form (outputs near zero make an elementwise
relative error meaningless).  Cosine similarity is reported and must stay
above 0.99 as a diagnostic."""
import numpy as np
import pytest
import torch

import oracle
from decode_step_attention_amd import workloads as W
from tests.helpers import errors, inputs_to_np, out_to_f64, run_oracle, to_np

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "f16": (2e-3, 1e-2), "bf16": (2e-3, 1e-2), "i8": (2e-3, 1e-2)}


@pytest.fixture(scope="module")
def ftm():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from decode_step_attention_amd import ftm as m
    yield m
    m.ftm_set_split_chunk(0)


def gpu_call(ftm, inp, case, with_bias=True, with_lens=True, stream=None):
    out = torch.empty((case.batch, case.n_heads, case.head_dim), dtype=W.TORCH_DTYPES[case.act_dtype],
                      device=inp["q"].device)
    ftm.ftm_decode_mha(inp["q"], inp["k_new"], inp["v_new"], inp["bias"] if with_bias else None,
                       inp["k_cache"], inp["v_cache"], inp["seq_lens"] if with_lens else None,
                       inp["step"], out, inp.get("kv_scales"), stream=stream)
    return out


def bits(t: torch.Tensor) -> torch.Tensor:
    """Bit pattern view, so that equality is bitwise (signed zeros, NaNs)."""
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()])


FRAC_BITS = {"f32": 23, "f16": 10, "bf16": 7, "i8": 10}   # of the output (activation) type


def ulp(x: np.ndarray, dt: str) -> np.ndarray:
    """One unit in the last place of the output type at |x| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -14)))
    return 2.0 ** (e - FRAC_BITS[dt])


def check(case, out, ref, tag="", tol=None):
    """out is stored in the activation type, and that rounding to nearest
    adds at most half a unit in the last place of the stored value on top
    of the error of the fp32 result: the absolute bar is the stated
    tolerance plus half an ulp of the output type at the larger of |out|
    and |ref| (the larger one, since the rounded value can sit in the next
    binade up)."""
    atol, rtol = tol or TOL[case.kv_dtype]
    got = out if isinstance(out, np.ndarray) else out_to_f64(out)
    finite = np.isfinite(ref).all(axis=-1)
    assert np.array_equal(np.isfinite(got).all(axis=-1), finite), f"{tag}: NaN rows differ"
    a, r, cos = errors(got[finite], ref[finite]) if finite.any() else (0, 0, 1)
    print(f"[{tag}] max_abs={a:.3e} row_rel={r:.3e} min_cos={cos:.6f}", flush=True)
    if finite.any():
        g, f = got[finite], ref[finite]
        bar = atol + 0.5 * ulp(np.maximum(np.abs(g), np.abs(f)), case.act_dtype)
        excess = np.abs(g - f) - bar
        assert excess.max() <= 0, f"{tag}: max abs err {a} beyond {atol} + half an ulp"
    assert r <= rtol, f"{tag}: max row-rel err {r}"
    assert cos > 0.99, f"{tag}: cosine {cos}"


def run_and_compare(ftm, case, chunk=0, device="cuda", poison=True, with_bias=True,
                    with_lens=True, lens=None, mutate=None, tag="", tol=None, waves=0):
    """Full comparison at a size the oracle finishes quickly."""
    inp = W.make_inputs(case, "cpu", poison=poison, lens=lens)
    if mutate:
        mutate(inp)
    npi = inputs_to_np(inp, case.kv_dtype)
    if not with_bias:
        npi["bias"] = None
    if not with_lens:
        npi["seq_lens"] = None
    ref_out, _ = run_oracle(oracle, case, npi, n_threads=8)
    g = {k: (v.to(device) if torch.is_tensor(v) else v) for k, v in inp.items()}
    ftm.ftm_set_split_chunk(chunk)
    ftm.ftm_set_workgroup_waves(waves)
    try:
        out = gpu_call(ftm, g, case, with_bias, with_lens)
        torch.cuda.synchronize()
    finally:
        ftm.ftm_set_split_chunk(0)
        ftm.ftm_set_workgroup_waves(0)
    # caches: every byte equals the oracle's (appended rows bit-exact, the
    # rest untouched); NaN-poisoned rows compare as bytes too
    assert to_np(g["k_cache"], case.kv_dtype).tobytes() == npi["k_cache"].tobytes(), f"{tag}: k_cache"
    assert to_np(g["v_cache"], case.kv_dtype).tobytes() == npi["v_cache"].tobytes(), f"{tag}: v_cache"
    if case.kv_dtype == "i8":
        assert to_np(g["kv_scales"], "f32").tobytes() == npi["kv_scales"].tobytes(), f"{tag}: scales"
    check(case, out, ref_out, tag, tol)
    return out, ref_out


def small(kv, D=128, B=3, H=8, Hkv=4, Lmax=1100, lens=(1, 1033), seed=7):
    scale = 1.0 if kv == "i8" else 1 / np.sqrt(D)
    return W.Case("p", B, H, Hkv, D, kv, ctx=Lmax, max_seq_len=Lmax, value_scale=scale,
                  lens=lens, seed=seed)


# ---- dtype x head_dim x grouping, ragged lengths, several tiles ----------
GRID = [(kv, D, H, Hkv) for kv in ("f32", "f16", "bf16", "i8") for D in (64, 128)
        for (H, Hkv) in ((4, 4), (8, 4), (8, 2), (8, 1))]


@pytest.mark.parametrize("kv,D,H,Hkv", GRID)
def test_parity_grid(ftm, kv, D, H, Hkv):
    case = small(kv, D=D, H=H, Hkv=Hkv, seed=11 + D + H * 3 + Hkv)
    run_and_compare(ftm, case, tag=f"{kv} D{D} H{H}/{Hkv}")


WIDE = [(kv, D, H, Hkv, chunk) for kv in ("f32", "f16", "bf16", "i8") for D in (64, 128)
        for (H, Hkv) in ((4, 4), (8, 4)) for chunk in (0, 256)]


@pytest.mark.parametrize("kv,D,H,Hkv,chunk", WIDE)
def test_parity_wide_workgroups(ftm, kv, D, H, Hkv, chunk):
    """The 16-wave workgroup (one or two query heads per pass), single pass
    and split."""
    case = small(kv, D=D, H=H, Hkv=Hkv, seed=21 + D + H + Hkv + chunk)
    run_and_compare(ftm, case, chunk=chunk, waves=16, tag=f"wide {kv} D{D} H{H}/{Hkv} c{chunk}")


@pytest.mark.parametrize("waves", [4, 16])
def test_parity_forced_narrow_and_wide_on_7b_shape(ftm, waves):
    """The 7B-shaped layer (fp16, 32 heads x 128) at a shorter context, both
    workgroup shapes."""
    case = W.Case("7b-short", 8, 32, 32, 128, "f16", ctx=640, max_seq_len=640,
                  value_scale=1 / np.sqrt(128), seed=22)
    run_and_compare(ftm, case, waves=waves, tag=f"7b-short waves{waves}")


def test_prepared_call_matches_plain_call(ftm):
    case = small("bf16", B=2, H=8, Hkv=2, Lmax=900, lens=(500, 900), seed=23)
    inp = W.make_inputs(case, "cuda")
    a = gpu_call(ftm, inp, case)
    out = torch.empty_like(a)
    call = ftm.ftm_decode_mha_prepared(inp["q"], inp["k_new"], inp["v_new"], inp["bias"],
                                       inp["k_cache"], inp["v_cache"], inp["seq_lens"], inp["step"],
                                       out, inp.get("kv_scales"))
    call()
    torch.cuda.synchronize()
    assert torch.equal(bits(a), bits(out))


@pytest.mark.parametrize("vector_alu", [False, True])
@pytest.mark.parametrize("kv,D,G,scale", [("bf16", 128, 8, None), ("f16", 128, 8, None),
                                           ("bf16", 64, 4, None), ("f16", 64, 8, None),
                                           ("bf16", 128, 8, 1.0), ("f16", 128, 4, 1.0)])
def test_grouped_heads_matrix_core_and_vector_paths(ftm, tuning, vector_alu, kv, D, G, scale):
    """Groups of 4 and 8 heads over fp16/bf16 caches run q.K on the matrix
    cores with the query split into two halves; FTM_GQA_VALU=1 selects the
    vector-ALU pass.  Both meet the bar, also with unit-scale data, where
    scores reach several units and the query split matters."""
    if vector_alu:
        tuning.set("FTM_GQA_VALU", "1")
    case = small(kv, D=D, H=2 * G, Hkv=2, B=3, seed=50 + G + D)
    if scale is not None:
        case = case.with_(value_scale=scale)
    for chunk in (0, 256):
        run_and_compare(ftm, case, chunk=chunk, tag=f"gqa {kv} D{D} G{G} s{scale} valu{vector_alu} c{chunk}")


@pytest.mark.parametrize("B,Lmax,lens,kv", [(1, 8192, (8192, 8192), "bf16"),   # one unit, many slices
                                             (2, 3000, (1, 3000), "f16"),
                                             (37, 700, (1, 700), "bf16"),      # many short units
                                             (5, 64, (1, 64), "f16"),           # less work than one slice
                                             (256, 96, (1, 96), "bf16"),        # the largest batch of the pass
                                             (257, 96, (1, 96), "f16")])        # one more: the vector path
def test_grouped_heads_balanced_schedule(ftm, B, Lmax, lens, kv):
    """The grouped-query pass splits the total work evenly over a fixed grid;
    slices cross unit boundaries and a unit may be merged from many slices
    in the same launch.  Repeated calls must give identical bits (the
    per-unit counts are cleared for the next call)."""
    case = small(kv, B=B, H=16, Hkv=2, Lmax=Lmax, lens=lens, seed=60 + B)
    out, ref = run_and_compare(ftm, case, tag=f"balanced B{B} L{lens} {kv}")
    inp = W.make_inputs(case, "cuda")
    outs = [gpu_call(ftm, inp, case) for _ in range(4)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(bits(o), bits(outs[0]))


@pytest.mark.parametrize("cost,per_cu", [(0, 1), (5, 1), (14, 2), (3, 3)])
def test_grouped_heads_range_boundaries(ftm, tuning, cost, per_cu):
    """The grouped-query schedule hands equal tile ranges to the workgroups;
    the per-unit charge and the workgroups per CU move the range boundaries
    inside units, so that ranges start and end mid-unit, hold several whole
    units, or begin in one unit's charge.  Every placement meets the bar and
    repeated calls give identical bits."""
    tuning.set("FTM_GQA_UNIT_COST", str(cost))
    tuning.set("FTM_GQA_BLOCKS_PER_CU", str(per_cu))
    case = small("bf16", B=23, H=16, Hkv=2, Lmax=2500, lens=(1, 2500), seed=70 + cost)
    run_and_compare(ftm, case, tag=f"ranges cost{cost} per_cu{per_cu}")
    inp = W.make_inputs(case, "cuda")
    outs = [gpu_call(ftm, inp, case) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(bits(o), bits(outs[0]))


@pytest.mark.parametrize("skew", ["1,1", "2,1", "8,7", "1,4"])
def test_grouped_heads_wave_shares(ftm, tuning, skew):
    """The grouped-query pass deals each round of tiles out unevenly between
    the older and the younger waves of a workgroup; every split covers each
    tile once, meets the bar and gives identical bits on repeated calls."""
    tuning.set("FTM_GQA_SKEW", skew)
    case = small("f16", B=9, H=16, Hkv=2, Lmax=3000, lens=(1, 3000), seed=80)
    run_and_compare(ftm, case, tag=f"wave shares {skew}")
    inp = W.make_inputs(case, "cuda")
    outs = [gpu_call(ftm, inp, case) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(bits(o), bits(outs[0]))


def test_grouped_heads_invalid_lengths(ftm):
    case = small("bf16", B=6, H=16, Hkv=2, Lmax=900, lens=(100, 800), seed=61)
    lens = W.seq_lens(case).clone()
    lens[0] = 0
    lens[4] = -3
    inp = W.make_inputs(case, "cpu", lens=lens)
    npi = inputs_to_np(inp, case.kv_dtype)
    ref, _ = run_oracle(oracle, case, npi)
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp.items()}
    out = gpu_call(ftm, g, case)
    torch.cuda.synchronize()
    o = out_to_f64(out)
    assert np.isnan(o[0]).all() and np.isnan(o[4]).all()
    check(case, out, ref, "gqa invalid lens")
    assert to_np(g["k_cache"], "bf16").tobytes() == npi["k_cache"].tobytes()
    assert to_np(g["v_cache"], "bf16").tobytes() == npi["v_cache"].tobytes()


@pytest.mark.parametrize("G", [3, 5, 12, 16])
def test_parity_odd_and_large_groups(ftm, G):
    """Group sizes that are not a power of two, and groups above 8 heads
    (served by several passes)."""
    case = small("f16", H=2 * G, Hkv=2, B=2, seed=40 + G)
    run_and_compare(ftm, case, tag=f"G{G}")


@pytest.mark.parametrize("chunk", [1, 128, 256, 384, 1024, 4096])
@pytest.mark.parametrize("kv", ["f32", "bf16", "i8"])
def test_split_count_invariance(ftm, kv, chunk):
    """Every chunk length (one tile up to a single pass) matches the oracle,
    and the outputs of different splittings agree to fp32 rounding."""
    case = small(kv, B=2, H=4, Hkv=2, Lmax=1500, lens=(900, 1500), seed=3)
    run_and_compare(ftm, case, chunk=chunk, tag=f"{kv} chunk{chunk}")


def test_split_outputs_agree_with_each_other(ftm):
    case = small("f32", B=2, H=4, Hkv=2, Lmax=2000, lens=(1900, 2000), seed=4)
    outs = []
    for chunk in (128, 512, 4096):
        o, _ = run_and_compare(ftm, case, chunk=chunk, tag=f"agree chunk{chunk}")
        outs.append(out_to_f64(o))
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 2e-6


@pytest.mark.parametrize("kv", ["f32", "f16", "bf16"])
def test_single_position_output_is_the_appended_v(ftm, kv):
    """t = 1: the only weight is exactly 1, so out equals the stored new V
    row bit for bit when the output type equals the cache type."""
    case = small(kv, B=4, H=8, Hkv=4, Lmax=16, lens=(1, 1), seed=9)
    inp = W.make_inputs(case, "cpu")
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp.items()}
    out = gpu_call(ftm, g, case)
    torch.cuda.synchronize()
    G = case.group
    v_rows = g["v_cache"][:, :, 0, :]                        # [B, Hkv, D]
    expect = v_rows.repeat_interleave(G, dim=1)               # query head h -> KV head h // G
    assert torch.equal(bits(out), bits(expect.contiguous()))


def test_single_position_int8(ftm):
    case = small("i8", B=2, H=4, Hkv=2, Lmax=8, lens=(1, 1), seed=10)
    run_and_compare(ftm, case, tag="i8 t=1")


def test_identical_keys_give_mean_of_v(ftm):
    case = small("f32", B=2, H=4, Hkv=2, Lmax=700, lens=(650, 700), seed=12)

    def same_keys(inp):
        key = torch.linspace(-1, 1, case.head_dim)
        inp["k_cache"][:] = key
        inp["k_new"][:] = key
        H, Hkv, D = case.n_heads, case.n_kv_heads, case.head_dim
        inp["bias"][H * D:(H + Hkv) * D] = 0
    out, ref = run_and_compare(ftm, case, poison=False, mutate=same_keys, tag="same keys")
    # equal weights: out is the plain mean of the V rows (oracle's cache
    # after the append, widened to double)
    inp = W.make_inputs(case, "cpu", poison=False)
    same_keys(inp)
    npi = inputs_to_np(inp, case.kv_dtype)
    run_oracle(oracle, case, npi)
    got = out_to_f64(out)
    for b in range(case.batch):
        L = int(npi["seq_lens"][b])
        for h in range(case.n_heads):
            mean = npi["v_cache"][b, h // case.group, :L].astype(np.float64).mean(axis=0)
            np.testing.assert_allclose(got[b, h], mean, rtol=0, atol=1e-6)


@pytest.mark.parametrize("kv", ["f32", "f16"])
@pytest.mark.parametrize("v_mean", [1.0, 0.0])
def test_large_scores_stay_stable(ftm, kv, v_mean):
    """Keys sharing a large component put every score near 100, where exp()
    overflows fp32: the softmax must subtract the running maximum.

    With values of mean 1 the outputs are of order 1 and both cache types
    meet their usual bars (fp32: 1e-5 max-abs and row-relative).  With
    zero-mean values the output, a weighted mean over ~800 values of
    spread 0.125, falls to ~0.01, far below the values it averages; the
    max-abs bar is unchanged, and for fp32 the row-relative bar is derived
    from the score sizes: each score s (log2 units, |s| up to S ~ 145)
    carries a few fp32 roundings of 2^-24 |s|, a weight moves by ln 2 times
    that relative to itself, and the output of a row by that times the
    largest |v| it averages: rel <= 1e-5 + 4 ln2 2^-24 S max|v| / max|out|."""
    case = small(kv, B=2, H=4, Hkv=2, D=64, Lmax=900, lens=(800, 900), seed=13)

    def big(inp):
        inp["k_cache"][..., 0] += 100.0
        inp["k_new"][..., 0] += 100.0
        inp["q"][..., 0] = 8.0
        inp["v_cache"] += v_mean
        inp["v_new"] += v_mean
    if v_mean or kv != "f32":
        run_and_compare(ftm, case, poison=True, mutate=big, tag=f"large scores {kv} v_mean {v_mean}")
        return
    # zero-mean values, fp32: max-abs 1e-5, the derived row-relative bound
    inp = W.make_inputs(case, "cpu", poison=True)
    big(inp)
    npi = inputs_to_np(inp, "f32")
    ref, _ = run_oracle(oracle, case, npi)
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp.items()}
    got = out_to_f64(gpu_call(ftm, g, case))
    torch.cuda.synchronize()
    G, D = case.group, case.head_dim
    qh = (npi["q"].astype(np.float64) + npi["bias"][:case.n_heads * D].reshape(case.n_heads, D))
    S, vmax = 0.0, np.zeros((case.batch, case.n_heads))
    for b in range(case.batch):
        L = int(npi["seq_lens"][b])
        for h in range(case.n_heads):
            k = npi["k_cache"][b, h // G, :L].astype(np.float64)
            S = max(S, float(np.abs(k @ qh[b, h]).max()) * np.log2(np.e) / np.sqrt(D))
            vmax[b, h] = np.abs(npi["v_cache"][b, h // G, :L]).max()
    err = np.abs(got - ref)
    rel = err.max(axis=-1) / np.abs(ref).max(axis=-1)
    bound = 1e-5 + 4 * np.log(2) * 2.0 ** -24 * S * vmax / np.abs(ref).max(axis=-1)
    print(f"[large scores f32 v_mean 0] S={S:.1f} max_abs={err.max():.3e} row_rel={rel.max():.3e} "
          f"bound={bound.min():.3e}..{bound.max():.3e}", flush=True)
    assert err.max() <= 1e-5
    assert (rel <= bound).all()


def test_int8_dequantisation_in_isolation(ftm):
    """An INT8 step equals an fp32-cache step whose cache holds code x scale
    exactly.  History scales get five significant bits and the new rows are
    built so that absmax / 127 is a power of two, so every code x scale
    product is exact in fp32 and the two steps differ only in where the
    dequantisation happens (and the fp16 rounding of the INT8 step's
    output): |out_i8 - out_f32| <= 1e-5 + half an fp16 ulp."""
    case = small("i8", B=3, H=8, Hkv=4, D=128, Lmax=700, lens=(1, 700), seed=91)
    B, H, Hkv, D = case.batch, case.n_heads, case.n_kv_heads, case.head_dim
    inp = W.make_inputs(case, "cpu", poison=True)
    gen = torch.Generator().manual_seed(91)
    # history scales 2^-5 x (16 + k) / 16, k in 0..15 (poisoned rows stay NaN)
    nice = 2.0 ** -5 * (16 + torch.randint(0, 16, inp["kv_scales"].shape, generator=gen)).float() / 16
    inp["kv_scales"] = torch.where(torch.isnan(inp["kv_scales"]), inp["kv_scales"], nice)
    # new rows: codes in [-127, 127] with |code| = 127 somewhere, times 2^-4,
    # and no K/V bias, so s = absmax / 127 = 2^-4 exactly
    for name in ("k_new", "v_new"):
        codes = torch.randint(-127, 128, (B, Hkv, D), generator=gen)
        codes[..., 5] = 127
        inp[name] = (codes.float() * 2.0 ** -4).half()
    inp["bias"][H * D:] = 0
    g8 = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp.items()}
    f32 = case.with_(kv_dtype="f32")
    g32 = {"q": g8["q"].float(), "k_new": g8["k_new"].float(), "v_new": g8["v_new"].float(),
           "bias": g8["bias"].float(), "seq_lens": g8["seq_lens"], "step": g8["step"],
           "k_cache": (g8["k_cache"].float() * g8["kv_scales"][0][..., None]).contiguous(),
           "v_cache": (g8["v_cache"].float() * g8["kv_scales"][1][..., None]).contiguous()}
    out8 = gpu_call(ftm, g8, case)
    out32 = gpu_call(ftm, g32, f32)
    torch.cuda.synchronize()
    # the appended rows agree: code x 2^-4 in both caches
    pos = (g8["seq_lens"] - 1).long()
    bi = torch.arange(B, device="cuda")
    assert torch.equal(g8["kv_scales"][0][bi, :, pos], torch.full((B, Hkv), 2.0 ** -4, device="cuda"))
    assert torch.equal(g8["k_cache"][bi, :, pos].float() * 2.0 ** -4, g32["k_cache"][bi, :, pos])
    assert torch.equal(g8["v_cache"][bi, :, pos].float() * 2.0 ** -4, g32["v_cache"][bi, :, pos])
    a, b32 = out_to_f64(out8), out_to_f64(out32)
    assert np.isfinite(a).all() and np.isfinite(b32).all()
    bar = 1e-5 + 0.5 * ulp(np.maximum(np.abs(a), np.abs(b32)), "f16")
    err = np.abs(a - b32)
    print(f"[int8 isolation] max |i8 - f32| = {err.max():.3e}", flush=True)
    assert (err <= bar).all(), f"max {err.max()}"


@pytest.mark.parametrize("step,D", [(512, 128), (513, 128), (1024, 64), (1025, 64)])
def test_default_launch_shape_at_the_short_pass_limit(ftm, step, D):
    """The 7B-shaped layer with the launch shape left to the library: a step
    that fits four 4-wave iterations takes the 4-wave single pass, one
    position more takes the 16-wave pass.  Ragged lengths up to the step and
    one invalid length (NaN rows, no append)."""
    case = W.Case("7b-step", 8, 32, 32, D, "f16", ctx=step, max_seq_len=step + 8,
                  value_scale=1 / np.sqrt(D), lens=(1, step), seed=95 + step + D)
    lens = W.seq_lens(case).clone()
    lens[0] = step
    lens[5] = 0
    run_and_compare(ftm, case, lens=lens, tag=f"default shape step{step} D{D}")


def test_no_bias_and_no_lengths(ftm):
    case = small("f16", B=3, H=8, Hkv=4, Lmax=600, lens=None, seed=14).with_(ctx=600)
    run_and_compare(ftm, case, with_bias=False, with_lens=False, tag="no bias, no lens")


def test_invalid_lengths_give_nan_rows_and_no_append(ftm):
    case = small("bf16", B=4, H=4, Hkv=2, Lmax=600, lens=(300, 500), seed=15)
    lens = W.seq_lens(case).clone()
    lens[1] = 0
    lens[3] = int(lens.max()) + 7           # above `step` once step is the valid max
    inp = W.make_inputs(case, "cpu", lens=lens)
    inp["step"] = int(max(lens[0], lens[2]))
    npi = inputs_to_np(inp, case.kv_dtype)
    ref, _ = run_oracle(oracle, case, npi)
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp.items()}
    for chunk in (0, 128):
        ftm.ftm_set_split_chunk(chunk)
        out = gpu_call(ftm, g, case)
        torch.cuda.synchronize()
        ftm.ftm_set_split_chunk(0)
        o = out_to_f64(out)
        assert np.isnan(o[1]).all() and np.isnan(o[3]).all()
        check(case, out, ref, f"invalid lens chunk{chunk}")
    assert to_np(g["k_cache"], "bf16").tobytes() == npi["k_cache"].tobytes()
    assert to_np(g["v_cache"], "bf16").tobytes() == npi["v_cache"].tobytes()


def test_deterministic(ftm):
    case = small("f16", B=2, H=8, Hkv=2, Lmax=2048, lens=(1500, 2048), seed=16)
    inp = W.make_inputs(case, "cuda")
    a = gpu_call(ftm, inp, case)
    b = gpu_call(ftm, inp, case)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_side_stream(ftm):
    case = small("f16", B=2, H=4, Hkv=4, Lmax=800, lens=(1, 800), seed=17)
    inp = W.make_inputs(case, "cpu")
    npi = inputs_to_np(inp, case.kv_dtype)
    ref, _ = run_oracle(oracle, case, npi)
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp.items()}
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        out = gpu_call(ftm, g, case)
    s.synchronize()
    check(case, out, ref, "side stream")


# ---- full-size workloads, sampled against the oracle ----------------------
def sub_problem(case, host, b, j):
    """Inputs of one (sequence, KV head) unit as a B=1, Hkv=1 problem."""
    G, D, H, Hkv = case.group, case.head_dim, case.n_heads, case.n_kv_heads
    bias = host["bias"]
    sub_bias = np.concatenate([bias[j * G * D:(j + 1) * G * D],
                               bias[(H + j) * D:(H + j + 1) * D],
                               bias[(H + Hkv + j) * D:(H + Hkv + j + 1) * D]])
    L = int(host["seq_lens"][b])
    sub = {"q": host["q"][b:b + 1, j * G:(j + 1) * G].copy(),
           "k_new": host["k_new"][b:b + 1, j:j + 1].copy(),
           "v_new": host["v_new"][b:b + 1, j:j + 1].copy(),
           "bias": sub_bias.copy(),
           "k_cache": host["k_slab"][(b, j)].copy(), "v_cache": host["v_slab"][(b, j)].copy(),
           "seq_lens": np.array([L], np.int32), "step": L,
           "kv_scales": host["s_slab"][(b, j)].copy() if case.kv_dtype == "i8" else None}
    return sub, case.with_(batch=1, n_heads=G, n_kv_heads=1)


@pytest.mark.parametrize("name", ["tiny", "7b", "sizing32", "gqa", "int8"])
def test_full_size_workload(ftm, name):
    """The five workloads at full size, in the launch configuration the
    benchmark times (automatic split).  Appended rows of every (b, j) are
    checked bytewise, the rest of the caches must be unchanged, and sampled
    (b, j) units are recomputed by the oracle."""
    import oracle
    case = W.CASES[name]
    print(f"[full {name}] generating", flush=True)
    inp = W.make_inputs(case, "cuda", poison=False)
    kvd, act = case.kv_dtype, case.act_dtype
    B, Hkv = case.batch, case.n_kv_heads
    rng = np.random.default_rng(case.seed)
    units = sorted({(int(b), int(j)) for b, j in zip(rng.integers(0, B, 6), rng.integers(0, Hkv, 6))}
                   | {(0, 0), (B - 1, Hkv - 1)})
    host = {k: to_np(inp[k], act) for k in ("q", "k_new", "v_new", "bias")}
    host["seq_lens"] = inp["seq_lens"].cpu().numpy().astype(np.int32)
    host["k_slab"] = {u: to_np(inp["k_cache"][u[0]:u[0] + 1, u[1]:u[1] + 1], kvd) for u in units}
    host["v_slab"] = {u: to_np(inp["v_cache"][u[0]:u[0] + 1, u[1]:u[1] + 1], kvd) for u in units}
    if kvd == "i8":
        host["s_slab"] = {u: to_np(inp["kv_scales"][:, u[0]:u[0] + 1, u[1]:u[1] + 1], "f32")
                          for u in units}
    k_before = inp["k_cache"].clone()
    v_before = inp["v_cache"].clone()
    s_before = inp["kv_scales"].clone() if kvd == "i8" else None
    print(f"[full {name}] running", flush=True)
    out = gpu_call(ftm, inp, case)
    torch.cuda.synchronize()
    # expected appended rows for every (b, j): the oracle on a one-slot cache
    one = case.with_(max_seq_len=1)
    tiny_k = np.zeros((B, Hkv, 1, case.head_dim), dtype=host["k_slab"][units[0]].dtype)
    tiny_v = tiny_k.copy()
    tiny_s = np.zeros((2, B, Hkv, 1), np.float32) if kvd == "i8" else None
    oracle.decode_mha(host["q"], host["k_new"], host["v_new"], host["bias"], tiny_k, tiny_v,
                      np.ones(B, np.int32), 1, case.n_heads, Hkv, case.head_dim, kvd, tiny_s,
                      n_threads=8)
    pos = torch.as_tensor(host["seq_lens"] - 1, device="cuda").long()
    bi = torch.arange(B, device="cuda")
    got_k = inp["k_cache"][bi, :, pos]            # [B, Hkv, D]
    got_v = inp["v_cache"][bi, :, pos]
    assert to_np(got_k, kvd).tobytes() == tiny_k[:, :, 0].tobytes(), "appended K rows"
    assert to_np(got_v, kvd).tobytes() == tiny_v[:, :, 0].tobytes(), "appended V rows"
    k_before[bi, :, pos] = got_k
    v_before[bi, :, pos] = got_v
    assert torch.equal(bits(k_before), bits(inp["k_cache"])), "other K rows changed"
    assert torch.equal(bits(v_before), bits(inp["v_cache"])), "other V rows changed"
    if kvd == "i8":
        # (index each plane separately: non-adjacent index tensors would move
        # the batch axis first)
        got_s = torch.stack([inp["kv_scales"][w][bi, :, pos] for w in range(2)])   # [2, B, Hkv]
        assert got_s.cpu().numpy().tobytes() == tiny_s[:, :, :, 0].tobytes(), "appended scales"
        for w in range(2):
            s_before[w][bi, :, pos] = got_s[w]
        assert torch.equal(bits(s_before), bits(inp["kv_scales"])), "other scales changed"
    del k_before, v_before
    out_h = out_to_f64(out)
    for (b, j) in units:
        sub, sc = sub_problem(case, host, b, j)
        ref, _ = oracle.decode_mha(sub["q"], sub["k_new"], sub["v_new"], sub["bias"],
                                   sub["k_cache"], sub["v_cache"], sub["seq_lens"], sub["step"],
                                   sc.n_heads, 1, sc.head_dim, kvd, sub["kv_scales"])
        G = case.group
        check(case, out_h[b:b + 1, j * G:(j + 1) * G], ref,
              f"full {name} b{b} j{j} L{int(host['seq_lens'][b])}")

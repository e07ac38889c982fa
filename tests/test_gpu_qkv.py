"""GPU parity of the fused QKV projection (ftm_qkv_proj) through the C ABI.

Bar: the projection accumulates in fp32 and rounds once to the activation
type, so |got - ref| <= 1 ulp of the output type at |ref| (half an ulp for
the rounding, doubled to cover a binade edge) + hidden * 2^-24 * sum_k
|x_k w_k| (the worst-case growth of an fp32 sum of `hidden` products,
which are exact in fp32), with ref the float64 oracle.  Every output
element is checked.  A routing case, one-hot weight rows that copy input
elements, must be bitwise exact, which pins where every feature lands in
q, k_new and v_new.  A chained case runs the projection and then the
attention step, against the oracle's projection, rounded by the oracle,
and the oracle's attention."""
import numpy as np
import pytest
import torch

import oracle
from decode_step_attention_amd import workloads as W
from tests.helpers import out_to_f64, to_np
from tests.test_gpu_parity import bits, check

pytestmark = pytest.mark.gpu

FRAC = {"f16": 10, "bf16": 7}
MIN_EXP = {"f16": -14, "bf16": -126}


@pytest.fixture(scope="module")
def ftm():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from decode_step_attention_amd import ftm as m
    return m


def run(ftm, inp, case, with_bias=True):
    dt = W.TORCH_DTYPES[case.dtype]
    B, H, Hkv, D = case.batch, case.n_heads, case.n_kv_heads, case.head_dim
    g = {k: v.cuda() for k, v in inp.items()}
    q = torch.empty((B, H, D), dtype=dt, device="cuda")
    k = torch.empty((B, Hkv, D), dtype=dt, device="cuda")
    v = torch.empty((B, Hkv, D), dtype=dt, device="cuda")
    ftm.ftm_qkv_proj(g["x"], g["w"], g["bias"] if with_bias else None, q, k, v)
    torch.cuda.synchronize()
    return q, k, v


def reference(inp, case, with_bias=True):
    dt = case.dtype
    x, w = to_np(inp["x"], dt), to_np(inp["w"], dt)
    b = to_np(inp["bias"], dt) if with_bias else None
    ref = oracle.qkv_proj(x, w, b, case.n_heads, case.n_kv_heads, case.head_dim, dt)
    absdot = np.abs(oracle.cache_to_f64(x, dt)) @ np.abs(oracle.cache_to_f64(w, dt)).T   # [B, N]
    return ref, absdot


def check_proj(case, got, ref, absdot, tag):
    dt = case.dtype
    B = case.batch
    g = np.concatenate([out_to_f64(t).reshape(B, -1) for t in got], axis=1)
    r = np.concatenate([a.reshape(B, -1) for a in ref], axis=1)
    e = np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** MIN_EXP[dt])))
    ulp = 2.0 ** (e - FRAC[dt])
    bound = ulp + case.hidden * 2.0 ** -24 * absdot
    err = np.abs(g - r)
    worst = float((err / bound).max())
    print(f"[{tag}] max abs err {err.max():.3e}, worst err/bound {worst:.3f}", flush=True)
    assert np.isfinite(g).all(), f"{tag}: non-finite output"
    assert worst <= 1.0, f"{tag}: error beyond the bound ({worst:.3f} of it)"


SHAPES = [
    # dtype, B, H, Hkv, D, hidden
    ("f16", 1, 8, 8, 64, 512),
    ("bf16", 8, 8, 2, 128, 1024),
    ("f16", 16, 16, 16, 128, 2048),
    ("bf16", 17, 8, 8, 64, 768),       # a second batch tile, ragged; three k iterations over four waves
    ("f16", 33, 4, 4, 128, 256),       # one k iteration: three waves idle
    ("bf16", 64, 8, 1, 128, 4096),
    ("f16", 5, 12, 4, 80, 1280),       # head_dim not a power of two
]


@pytest.mark.parametrize("dt,B,H,Hkv,D,hidden", SHAPES)
@pytest.mark.parametrize("with_bias", [True, False])
def test_projection_parity(ftm, dt, B, H, Hkv, D, hidden, with_bias):
    case = W.ProjCase("t", B, H, Hkv, D, hidden, dt, seed=17 + B + hidden)
    inp = W.make_proj_inputs(case)
    got = run(ftm, inp, case, with_bias)
    ref, absdot = reference(inp, case, with_bias)
    check_proj(case, got, ref, absdot, f"{dt} B{B} H{H}/{Hkv} D{D} hidden{hidden} bias{with_bias}")


@pytest.mark.parametrize("ft", ["1", "2", "3", "4"])
@pytest.mark.parametrize("dt,B,hidden", [("bf16", 16, 1024), ("f16", 40, 768), ("bf16", 64, 2048)])
def test_column_tiles(ftm, tuning, ft, dt, B, hidden):
    """Every number of column tiles per workgroup (forced), with one to four
    batch tiles."""
    tuning.set("FTM_QKV_COLUMN_TILES", ft)
    case = W.ProjCase("t", B, 8, 2, 128, hidden, dt, seed=31 + B)
    inp = W.make_proj_inputs(case)
    got = run(ftm, inp, case)
    ref, absdot = reference(inp, case)
    check_proj(case, got, ref, absdot, f"{dt} B{B} hidden{hidden} column tiles {ft}")


@pytest.mark.parametrize("ft", ["3", "4"])
@pytest.mark.parametrize("dt,B,H,Hkv,D,hidden", [("bf16", 9, 8, 1, 64, 768),     # 640 features
                                                 ("f16", 33, 6, 2, 80, 512),     # 800 features
                                                 ("bf16", 64, 5, 5, 128, 1024)]) # 1920: 48 x 40
def test_partial_last_workgroup(ftm, tuning, ft, dt, B, H, Hkv, D, hidden):
    """Feature counts that are not a multiple of the workgroup's 16 FT
    columns: the last workgroup's rows past the end read as zero and its
    tiles past the end are not written (every output is checked, and the
    buffers past the outputs are not touched)."""
    tuning.set("FTM_QKV_COLUMN_TILES", ft)
    case = W.ProjCase("t", B, H, Hkv, D, hidden, dt, seed=41 + B + D)
    inp = W.make_proj_inputs(case)
    tdt = W.TORCH_DTYPES[dt]
    g = {k: v.cuda() for k, v in inp.items()}
    # each output is the head of a buffer whose tail holds a sentinel
    sizes = [B * H * D, B * Hkv * D, B * Hkv * D]
    bufs = [torch.full((n + 4096,), 12345.0, dtype=tdt, device="cuda") for n in sizes]
    q, k, v = (bufs[0][:sizes[0]].view(B, H, D), bufs[1][:sizes[1]].view(B, Hkv, D),
               bufs[2][:sizes[2]].view(B, Hkv, D))
    ftm.ftm_qkv_proj(g["x"], g["w"], g["bias"], q, k, v)
    torch.cuda.synchronize()
    for buf, n in zip(bufs, sizes):
        assert bool((buf[n:] == 12345.0).all()), f"ft {ft}: a write past an output buffer"
    ref, absdot = reference(inp, case)
    check_proj(case, (q, k, v), ref, absdot, f"{dt} B{B} H{H}/{Hkv} D{D} partial last workgroup ft {ft}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_routing_is_exact(ftm, dt):
    """One-hot weight rows: feature f copies x[:, perm[f]] exactly."""
    B, H, Hkv, D, hidden = 9, 8, 2, 64, 1024
    case = W.ProjCase("r", B, H, Hkv, D, hidden, dt, seed=5)
    inp = W.make_proj_inputs(case)
    N = case.n_out
    perm = torch.from_numpy(np.random.default_rng(3).integers(0, hidden, N))
    w = torch.zeros((N, hidden), dtype=W.TORCH_DTYPES[dt])
    w[torch.arange(N), perm] = 1.0
    inp["w"] = w
    q, k, v = run(ftm, inp, case, with_bias=False)
    y = torch.cat([q.reshape(B, -1), k.reshape(B, -1), v.reshape(B, -1)], dim=1).cpu()
    want = inp["x"][:, perm]
    assert torch.equal(bits(y), bits(want))


@pytest.mark.parametrize("name", sorted(W.PROJ_CASES))
def test_full_size_projection(ftm, name):
    """The benchmark's projections at full size, every output checked."""
    case = W.PROJ_CASES[name]
    inp = W.make_proj_inputs(case)
    got = run(ftm, inp, case)
    ref, absdot = reference(inp, case)
    check_proj(case, got, ref, absdot, f"full {name}")


@pytest.mark.parametrize("dt,H,Hkv", [("f16", 8, 8), ("bf16", 8, 2)])
def test_projection_then_attention(ftm, dt, H, Hkv):
    """x -> projection -> decode step, against the oracle's projection
    (float64, rounded to the activation type by the oracle) and the oracle's
    step.  The appended rows may differ from the oracle's by the rounding of
    k_new/v_new (fp32 against float64 sums): within one ulp."""
    B, D = 3, 128
    hidden = H * D
    pc = W.ProjCase("c", B, H, Hkv, D, hidden, dt, seed=23)
    inp = W.make_proj_inputs(pc)
    ac = W.Case("c", B, H, Hkv, D, dt, ctx=700, max_seq_len=720, value_scale=1 / np.sqrt(D),
                lens=(1, 700), seed=29)
    ai = W.make_inputs(ac, "cpu", poison=True)
    # oracle chain
    (qr, kr, vr), _ = reference(inp, pc, with_bias=False)
    qn, kn, vn = (oracle.round_to_act(a, dt) for a in (qr, kr, vr))
    kc, vc = to_np(ai["k_cache"], dt), to_np(ai["v_cache"], dt)
    lens = ai["seq_lens"].numpy().astype(np.int32)
    ref, _ = oracle.decode_mha(qn, kn, vn, to_np(ai["bias"], dt), kc, vc, lens, ai["step"], H, Hkv, D, dt,
                               n_threads=8)
    # GPU chain
    q, k, v = run(ftm, inp, pc, with_bias=False)
    g = {kk: (t.cuda() if torch.is_tensor(t) else t) for kk, t in ai.items()}
    out = torch.empty((B, H, D), dtype=W.TORCH_DTYPES[dt], device="cuda")
    ftm.ftm_decode_mha(q, k, v, g["bias"], g["k_cache"], g["v_cache"], g["seq_lens"], g["step"], out)
    torch.cuda.synchronize()
    check(ac, out, ref, f"projection + attention {dt} H{H}/{Hkv}")
    gk = oracle.cache_to_f64(to_np(g["k_cache"], dt), dt)
    rk = oracle.cache_to_f64(kc, dt)
    for b in range(B):
        p = int(lens[b]) - 1
        d = np.abs(gk[b, :, p] - rk[b, :, p])
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(rk[b, :, p]), 2.0 ** MIN_EXP[dt]))) - FRAC[dt])
        assert (d <= ulp).all(), f"appended K row of sequence {b} beyond one ulp"


# k split: dtype, B, H, Hkv, D, hidden.  Feature counts that leave the last
# 128-feature column partial, iteration counts (hidden / 256) that do not
# divide by the split, and one to four batch tiles.
SPLIT_SHAPES = [
    ("bf16", 9, 8, 1, 64, 768),         # 640 features (5 columns), 3 iterations
    ("f16", 33, 6, 2, 80, 1280),        # 800: the last column has 32 features, 5 iterations
    ("f16", 48, 8, 8, 128, 1536),       # three batch tiles, 6 iterations
    ("bf16", 64, 5, 5, 128, 2048),      # 1920 features, 8 iterations
    ("bf16", 20, 4, 4, 64, 256),        # one iteration: every split clamps to one pass
]


def sentinel_outputs(case, g, tdt):
    B, H, Hkv, D = case.batch, case.n_heads, case.n_kv_heads, case.head_dim
    sizes = [B * H * D, B * Hkv * D, B * Hkv * D]
    bufs = [torch.full((n + 4096,), 12345.0, dtype=tdt, device="cuda") for n in sizes]
    outs = (bufs[0][:sizes[0]].view(B, H, D), bufs[1][:sizes[1]].view(B, Hkv, D),
            bufs[2][:sizes[2]].view(B, Hkv, D))
    return bufs, sizes, outs


@pytest.mark.parametrize("ks", ["1", "2", "3", "4"])
@pytest.mark.parametrize("dt,B,H,Hkv,D,hidden", SPLIT_SHAPES)
def test_k_split(ftm, tuning, ks, dt, B, H, Hkv, D, hidden):
    """Every k split (forced) of the 128-feature-column variant: each
    workgroup's fp32 partial goes through the workspace and the last one
    of its column adds them.  Every output is checked, and nothing is
    written past the output buffers."""
    tuning.set("FTM_QKV_K_SPLIT", ks)
    case = W.ProjCase("t", B, H, Hkv, D, hidden, dt, seed=53 + B + D)
    inp = W.make_proj_inputs(case)
    g = {k: v.cuda() for k, v in inp.items()}
    bufs, sizes, (q, k, v) = sentinel_outputs(case, g, W.TORCH_DTYPES[dt])
    ftm.ftm_qkv_proj(g["x"], g["w"], g["bias"], q, k, v)
    torch.cuda.synchronize()
    for buf, n in zip(bufs, sizes):
        assert bool((buf[n:] == 12345.0).all()), f"k split {ks}: a write past an output buffer"
    ref, absdot = reference(inp, case)
    check_proj(case, (q, k, v), ref, absdot, f"{dt} B{B} H{H}/{Hkv} D{D} hidden{hidden} k split {ks}")


@pytest.mark.parametrize("ks", ["2", "3"])
def test_k_split_is_repeatable(ftm, tuning, ks):
    """The partials are added in split order whichever workgroup finishes
    last, and the column counts return to zero: repeated calls, with a call
    of another shape between them, give the same bits."""
    tuning.set("FTM_QKV_K_SPLIT", ks)
    case = W.ProjCase("t", 64, 8, 2, 128, 2048, "f16", seed=61)
    other = W.ProjCase("t", 40, 4, 4, 64, 1024, "f16", seed=62)
    inp, inp2 = W.make_proj_inputs(case), W.make_proj_inputs(other)
    first = [t.clone() for t in run(ftm, inp, case)]
    for _ in range(3):
        run(ftm, inp2, other)
        again = run(ftm, inp, case)
        for a, b in zip(first, again):
            assert torch.equal(bits(a.cpu()), bits(b.cpu()))
    ref, absdot = reference(inp, case)
    check_proj(case, first, ref, absdot, f"repeat k split {ks}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_k_split_routing_is_exact(ftm, tuning, dt):
    """One-hot weight rows through the k split: each feature's one product
    lands in one split's partial and the others add exact zeros."""
    tuning.set("FTM_QKV_K_SPLIT", "3")
    B, H, Hkv, D, hidden = 64, 8, 2, 64, 1536
    case = W.ProjCase("r", B, H, Hkv, D, hidden, dt, seed=7)
    inp = W.make_proj_inputs(case)
    N = case.n_out
    perm = torch.from_numpy(np.random.default_rng(4).integers(0, hidden, N))
    w = torch.zeros((N, hidden), dtype=W.TORCH_DTYPES[dt])
    w[torch.arange(N), perm] = 1.0
    inp["w"] = w
    q, k, v = run(ftm, inp, case, with_bias=False)
    y = torch.cat([q.reshape(B, -1), k.reshape(B, -1), v.reshape(B, -1)], dim=1).cpu()
    want = inp["x"][:, perm]
    assert torch.equal(bits(y), bits(want))

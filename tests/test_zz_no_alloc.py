"""The allocation-free decode call (ftm_decode_mha_static) through the C ABI,
against ftm_decode_mha on the same inputs.

The two run the same kernels and differ only in where the scratch lives
(a fixed device array instead of the per-stream workspace), so the outputs
must be bitwise equal and so must the caches after the append.  Each case
makes calls in a row on one stream: a larger step, a smaller one, then the
larger again, so that a partial or a counter left over from the previous
call would show.  The cases cover every kernel path that uses scratch: the
grouped-query pass whose units are cut into pieces (partials and counters),
and the split single-head pass (partials and the combine)."""
import numpy as np
import pytest
import torch

from decode_step_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ftm():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from decode_step_attention_amd import ftm as m
    yield m
    m.ftm_set_split_chunk(0)


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()])


def case(kv, B, H, Hkv, Lmax, lens, seed, D=128):
    scale = 1.0 if kv == "i8" else 1 / np.sqrt(D)
    return W.Case("na", B, H, Hkv, D, kv, ctx=Lmax, max_seq_len=Lmax, value_scale=scale, lens=lens, seed=seed)


def both(ftm, c):
    """One step through each entry point on copies of the same inputs."""
    inp = W.make_inputs(c, "cuda")
    copy = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in inp.items()}
    outs = []
    for f, d in ((ftm.ftm_decode_mha, inp), (ftm.ftm_decode_mha_static, copy)):
        out = torch.empty((c.batch, c.n_heads, c.head_dim), dtype=W.TORCH_DTYPES[c.act_dtype], device="cuda")
        f(d["q"], d["k_new"], d["v_new"], d["bias"], d["k_cache"], d["v_cache"], d["seq_lens"], d["step"], out,
          d.get("kv_scales"))
        outs.append(out)
    torch.cuda.synchronize()
    tag = f"{c.kv_dtype} B{c.batch} H{c.n_heads}/{c.n_kv_heads} L{c.lens}"
    assert torch.equal(bits(outs[0]), bits(outs[1])), f"{tag}: outputs differ"
    for k in ("k_cache", "v_cache", "kv_scales"):
        if k in inp:
            assert torch.equal(bits(inp[k]), bits(copy[k])), f"{tag}: {k} differs"
    assert torch.isfinite(outs[1].float()).all(), f"{tag}: non-finite output"
    print(f"[{tag}] bitwise equal", flush=True)


# (larger, smaller) steps of one kernel path each
PAIRS = {
    # grouped heads on the matrix cores: long units cut into pieces
    "grouped pieces": (case("bf16", 2, 16, 2, 8192, (4000, 8192), 301),
                       case("bf16", 1, 16, 2, 3000, (100, 3000), 302)),
    "grouped many units": (case("f16", 37, 8, 1, 700, (1, 700), 303),
                           case("f16", 5, 8, 1, 300, (1, 300), 304)),
    # one query head per pass, split into chunks + combine (automatic shape)
    "single head split": (case("f16", 1, 4, 4, 6000, (6000, 6000), 305),
                          case("f16", 1, 2, 2, 3000, (2000, 3000), 306)),
    "fp32 split": (case("f32", 2, 2, 2, 5000, (3000, 5000), 307, D=64),
                   case("f32", 1, 2, 2, 2000, (100, 2000), 308, D=64)),
    "int8 split": (case("i8", 1, 8, 8, 4096, (4096, 4096), 309),
                   case("i8", 1, 4, 4, 1500, (800, 1500), 310)),
}


@pytest.mark.parametrize("path", sorted(PAIRS))
def test_static_equals_workspace_call(ftm, path):
    big, small = PAIRS[path]
    both(ftm, big)
    both(ftm, small)
    both(ftm, big)


def test_static_forced_split_chunks(ftm):
    """Many chunks per sequence (a forced short chunk), then fewer."""
    ftm.ftm_set_split_chunk(128)
    try:
        both(ftm, case("bf16", 3, 8, 8, 3000, (1, 3000), 311))
        both(ftm, case("bf16", 2, 4, 4, 1000, (1, 1000), 312))
    finally:
        ftm.ftm_set_split_chunk(0)


def test_static_refuses_steps_beyond_its_scratch(ftm, tuning):
    """Sixteen ranges per CU need more partial slots than the fixed array
    holds: the call returns FTM_ERR_UNSUPPORTED and writes nothing."""
    tuning.set("FTM_GQA_BLOCKS_PER_CU", 16)
    c = case("bf16", 2, 16, 2, 4096, (2000, 4096), 313)
    inp = W.make_inputs(c, "cuda")
    k0 = inp["k_cache"].clone()
    out = torch.full((c.batch, c.n_heads, c.head_dim), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="status 2: .*fixed scratch"):
        ftm.ftm_decode_mha_static(inp["q"], inp["k_new"], inp["v_new"], inp["bias"], inp["k_cache"],
                                  inp["v_cache"], inp["seq_lens"], inp["step"], out)
    torch.cuda.synchronize()
    assert torch.equal(bits(inp["k_cache"]), bits(k0))
    assert (out == 7.0).all()

"""GPU parity of prefill into a paged cache (ftm_prefill_mha_paged) through
the C ABI, against the paged prefill oracle on the same seeded inputs.

Bar: the page pools must equal the oracle's bytewise over the whole pools
(the prompt rows at the page and row the table names, every other row, NaN
poison included, untouched); every output row t < S_b meets the decode
bar.  With an identity table the outputs must equal the contiguous
prefill's bit for bit (the same arithmetic, only the addressing differs)."""
import numpy as np
import pytest
import torch

import oracle
from decode_step_attention_amd import workloads as W
from tests.helpers import out_to_f64, to_np
from tests.test_gpu_parity import bits, check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ftm():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from decode_step_attention_amd import ftm as m
    return m


def run_paged(ftm, inp, case):
    g = {k: v.cuda() for k, v in inp.items()}
    out = torch.zeros((case.batch, case.prompt, case.n_heads, case.head_dim), dtype=W.TORCH_DTYPES[case.dtype],
                      device="cuda")
    ftm.ftm_prefill_mha_paged(g["q"], g["k_new"], g["v_new"], g["bias"], g["k_pages"], g["v_pages"],
                              g["block_table"], g["seq_lens"], out)
    torch.cuda.synchronize()
    return g, out


def compare_paged(ftm, case, inp, tag):
    dt = case.dtype
    npi = {k: to_np(v, dt) for k, v in inp.items() if k not in ("seq_lens", "block_table")}
    lens = inp["seq_lens"].numpy().astype(np.int32)
    table = inp["block_table"].numpy()
    print(f"[{tag}] oracle", flush=True)
    ref = oracle.prefill_mha_paged(npi["q"], npi["k_new"], npi["v_new"], npi["bias"], npi["k_pages"],
                                   npi["v_pages"], table, lens, case.n_heads, case.n_kv_heads, case.head_dim, dt)
    print(f"[{tag}] gpu", flush=True)
    g, out = run_paged(ftm, inp, case)
    assert to_np(g["k_pages"], dt).tobytes() == npi["k_pages"].tobytes(), f"{tag}: k_pages"
    assert to_np(g["v_pages"], dt).tobytes() == npi["v_pages"].tobytes(), f"{tag}: v_pages"
    got = out_to_f64(out)
    ac = W.Case("p", case.batch, case.n_heads, case.n_kv_heads, case.head_dim, dt, ctx=case.prompt,
                max_seq_len=case.max_seq_len, value_scale=1.0)
    for b in range(case.batch):
        Sb = int(lens[b])
        if np.isnan(ref[b, :Sb]).all():
            assert np.isnan(got[b, :Sb]).all(), f"{tag}: sequence {b} must give NaN rows"
            continue
        check(ac, got[b, :Sb], ref[b, :Sb], f"{tag} b{b} S{Sb}")
    return g, out


SHAPES = [
    # dtype, B, S, H, Hkv, D, Lmax, lens, P
    ("f16", 2, 200, 4, 4, 128, 208, (1, 200), 16),
    ("bf16", 3, 150, 8, 2, 64, 160, (20, 150), 64),
    ("f16", 2, 333, 12, 4, 128, 512, (300, 333), 256),
    ("bf16", 1, 64, 2, 1, 128, 64, None, 32),
    ("f16", 2, 700, 2, 2, 64, 768, (1, 700), 128),
]


@pytest.mark.parametrize("dt,B,S,H,Hkv,D,Lmax,lens,P", SHAPES)
def test_paged_prefill_parity(ftm, dt, B, S, H, Hkv, D, Lmax, lens, P):
    case = W.PrefillCase("t", B, S, H, Hkv, D, dt, Lmax, lens=lens, seed=91 + S + P)
    inp = W.prefill_to_paged(W.make_prefill_inputs(case, "cpu", poison=True), case, P)
    compare_paged(ftm, case, inp, f"paged prefill {dt} B{B} S{S} H{H}/{Hkv} D{D} P{P}")


@pytest.mark.parametrize("dt,P", [("f16", 16), ("bf16", 64)])
def test_identity_table_matches_the_contiguous_prefill(ftm, dt, P):
    B, S, H, Hkv, D = 2, 300, 8, 2, 128
    npp = (S + P - 1) // P
    case = W.PrefillCase("t", B, S, H, Hkv, D, dt, npp * P, lens=(150, 300), seed=97)
    inp = W.make_prefill_inputs(case, "cpu", poison=True)
    g = {k: v.cuda() for k, v in inp.items()}
    ref_out = torch.zeros((B, S, H, D), dtype=W.TORCH_DTYPES[dt], device="cuda")
    ftm.ftm_prefill_mha(g["q"], g["k_new"], g["v_new"], g["bias"], g["k_cache"], g["v_cache"], g["seq_lens"],
                        ref_out)
    pools = {k: torch.full((B * npp, Hkv, P, D), float("nan"), dtype=W.TORCH_DTYPES[dt], device="cuda")
             for k in ("k", "v")}
    table = torch.arange(B * npp, dtype=torch.int32, device="cuda").reshape(B, npp)
    out = torch.zeros_like(ref_out)
    ftm.ftm_prefill_mha_paged(g["q"], g["k_new"], g["v_new"], g["bias"], pools["k"], pools["v"], table,
                              g["seq_lens"], out)
    torch.cuda.synchronize()
    lens = inp["seq_lens"].tolist()
    for b in range(B):
        assert torch.equal(bits(out[b, :lens[b]]), bits(ref_out[b, :lens[b]])), f"sequence {b}"
        for name, cache in (("k", g["k_cache"]), ("v", g["v_cache"])):
            as_cache = pools[name].reshape(B, npp, Hkv, P, D).transpose(1, 2).reshape(B, Hkv, npp * P, D)
            assert torch.equal(bits(as_cache[b, :, :lens[b]]), bits(cache[b, :, :lens[b]])), f"{name} {b}"


def test_pages_outside_the_pool(ftm):
    case = W.PrefillCase("t", 3, 260, 4, 2, 128, "bf16", 320, lens=(200, 260), seed=101)
    inp = W.prefill_to_paged(W.make_prefill_inputs(case, "cpu", poison=True), case, 64)
    n_pages = inp["k_pages"].shape[0]
    inp["block_table"][1, 1] = n_pages + 5                  # sequence 1: its second page is outside the pool
    inp["block_table"][2, 0] = -7                           # sequence 2: its first page
    compare_paged(ftm, case, inp, "paged prefill, pages outside the pool")


@pytest.mark.parametrize("name", ["prefill_7b_paged"])
def test_full_size_paged_prefill_sampled_heads(ftm, name):
    """The benchmark's paged prefill at full size: the pools are checked whole
    against the contiguous kernel's caches through the table, and two
    (sequence, head) pairs of the output are recomputed by the oracle."""
    case = W.PREFILL_CASES[name]
    inp = W.make_prefill_inputs(case, "cuda", poison=False)
    contiguous = {k: v.clone() for k, v in inp.items()}
    inp = W.prefill_to_paged(inp, case, case.page_size)
    print(f"[full {name}] gpu", flush=True)
    g, out = run_paged(ftm, inp, case)
    ref_out = torch.zeros_like(out)
    c = contiguous
    ftm.ftm_prefill_mha(c["q"], c["k_new"], c["v_new"], c["bias"], c["k_cache"], c["v_cache"], c["seq_lens"],
                        ref_out)
    torch.cuda.synchronize()
    assert torch.equal(bits(out), bits(ref_out)), "paged and contiguous prefill outputs differ"
    P = case.page_size
    table = g["block_table"].cpu()
    for b in range(case.batch):
        for i in range((case.prompt + P - 1) // P):
            pg = int(table[b, i])
            assert torch.equal(bits(g["k_pages"][pg]), bits(c["k_cache"][b, :, i * P:(i + 1) * P])), (b, i)
            assert torch.equal(bits(g["v_pages"][pg]), bits(c["v_cache"][b, :, i * P:(i + 1) * P])), (b, i)

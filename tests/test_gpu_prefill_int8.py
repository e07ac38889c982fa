"""GPU parity of prefill into an INT8 cache (ftm_prefill_mha and
ftm_prefill_mha_paged with kv_dtype FTM_I8) through the C ABI, against the
INT8 prefill oracle on the same seeded inputs.

Bar: codes and scales must equal the oracle's bytewise over the whole cache
and scale buffers (every prompt row quantised by the decode step's rule,
every other byte, poison included, untouched); every output row t < S_b
meets the decode bar."""
import numpy as np
import pytest
import torch

import oracle
from decode_step_attention_amd import workloads as W
from tests.helpers import out_to_f64, to_np
from tests.test_gpu_parity import check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ftm():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from decode_step_attention_amd import ftm as m
    return m


def host(inp):
    out = {}
    for k, v in inp.items():
        if k in ("seq_lens", "block_table"):
            continue
        out[k] = to_np(v, "f16") if v.dtype == torch.float16 else v.cpu().numpy().copy()
    return out


def run_and_compare(ftm, case, inp, tag, paged):
    npi = host(inp)
    lens = inp["seq_lens"].numpy().astype(np.int32)
    H, Hkv, D = case.n_heads, case.n_kv_heads, case.head_dim
    print(f"[{tag}] oracle", flush=True)
    if paged:
        ref = oracle.prefill_mha_paged(npi["q"], npi["k_new"], npi["v_new"], npi["bias"], npi["k_pages"],
                                       npi["v_pages"], inp["block_table"].numpy(), lens, H, Hkv, D, "i8",
                                       npi["kv_scales"])
    else:
        ref = oracle.prefill_mha(npi["q"], npi["k_new"], npi["v_new"], npi["bias"], npi["k_cache"],
                                 npi["v_cache"], lens, H, Hkv, D, "i8", npi["kv_scales"])
    print(f"[{tag}] gpu", flush=True)
    g = {k: v.cuda() for k, v in inp.items()}
    out = torch.zeros((case.batch, case.prompt, H, D), dtype=torch.float16, device="cuda")
    if paged:
        ftm.ftm_prefill_mha_paged(g["q"], g["k_new"], g["v_new"], g["bias"], g["k_pages"], g["v_pages"],
                                  g["block_table"], g["seq_lens"], out, kv_scales=g["kv_scales"])
        names = ("k_pages", "v_pages", "kv_scales")
    else:
        ftm.ftm_prefill_mha(g["q"], g["k_new"], g["v_new"], g["bias"], g["k_cache"], g["v_cache"], g["seq_lens"],
                            out, kv_scales=g["kv_scales"])
        names = ("k_cache", "v_cache", "kv_scales")
    torch.cuda.synchronize()
    for name in names:
        assert g[name].cpu().numpy().tobytes() == npi[name].tobytes(), f"{tag}: {name}"
    got = out_to_f64(out)
    ac = W.Case("p", case.batch, H, Hkv, D, "i8", ctx=case.prompt, max_seq_len=case.max_seq_len, value_scale=1.0)
    for b in range(case.batch):
        Sb = int(lens[b])
        if np.isnan(ref[b, :Sb]).all():
            assert np.isnan(got[b, :Sb]).all(), f"{tag}: sequence {b} must give NaN rows"
            continue
        check(ac, got[b, :Sb], ref[b, :Sb], f"{tag} b{b} S{Sb}")


SHAPES = [
    # B, S, H, Hkv, D, Lmax, lens
    (2, 200, 4, 4, 128, 208, (1, 200)),
    (3, 150, 8, 2, 64, 160, (20, 150)),
    (2, 333, 12, 4, 128, 400, (300, 333)),
    (1, 64, 2, 1, 128, 64, None),
]


@pytest.mark.parametrize("B,S,H,Hkv,D,Lmax,lens", SHAPES)
def test_int8_prefill_parity(ftm, B, S, H, Hkv, D, Lmax, lens):
    case = W.PrefillCase("t", B, S, H, Hkv, D, "i8", Lmax, lens=lens, seed=121 + S)
    inp = W.make_prefill_inputs(case, "cpu", poison=True)
    run_and_compare(ftm, case, inp, f"int8 prefill B{B} S{S} H{H}/{Hkv} D{D}", paged=False)


@pytest.mark.parametrize("P", [16, 128])
def test_int8_paged_prefill_parity(ftm, P):
    case = W.PrefillCase("t", 3, 260, 8, 4, 128, "i8", 320, lens=(1, 260), seed=131 + P)
    inp = W.prefill_to_paged(W.make_prefill_inputs(case, "cpu", poison=True), case, P)
    run_and_compare(ftm, case, inp, f"int8 paged prefill P{P}", paged=True)


def test_int8_prefill_without_bias_and_lengths(ftm):
    case = W.PrefillCase("t", 2, 170, 6, 2, 128, "i8", 176, seed=141)
    inp = W.make_prefill_inputs(case, "cpu", poison=True)
    npi = host(inp)
    ref = oracle.prefill_mha(npi["q"], npi["k_new"], npi["v_new"], None, npi["k_cache"], npi["v_cache"], None,
                             case.n_heads, case.n_kv_heads, case.head_dim, "i8", npi["kv_scales"])
    g = {k: v.cuda() for k, v in inp.items()}
    out = torch.zeros((2, 170, 6, 128), dtype=torch.float16, device="cuda")
    ftm.ftm_prefill_mha(g["q"], g["k_new"], g["v_new"], None, g["k_cache"], g["v_cache"], None, out,
                        kv_scales=g["kv_scales"])
    torch.cuda.synchronize()
    for name in ("k_cache", "v_cache", "kv_scales"):
        assert g[name].cpu().numpy().tobytes() == npi[name].tobytes(), name
    ac = W.Case("p", 2, 6, 2, 128, "i8", ctx=170, max_seq_len=176, value_scale=1.0)
    got = out_to_f64(out)
    for b in range(2):
        check(ac, got[b], ref[b], f"int8 prefill no bias/lengths b{b}")


def test_int8_prefill_then_decode(ftm):
    """The cache an INT8 prefill wrote is the one an INT8 decode step reads:
    prefill the first S - 1 positions, then decode position S - 1, and the
    decode output must match the prefill output at that position within the
    decode bar (both are the same function of the same codes)."""
    case = W.PrefillCase("t", 2, 240, 8, 8, 128, "i8", 256, seed=151)
    inp = W.make_prefill_inputs(case, "cpu", poison=True)
    g = {k: v.cuda() for k, v in inp.items()}
    S = case.prompt
    full = torch.zeros((2, S, 8, 128), dtype=torch.float16, device="cuda")
    ftm.ftm_prefill_mha(g["q"], g["k_new"], g["v_new"], g["bias"], g["k_cache"].clone(), g["v_cache"].clone(),
                        None, full, kv_scales=g["kv_scales"].clone())
    kc, vc, sc = g["k_cache"], g["v_cache"], g["kv_scales"]
    part = torch.zeros((2, S - 1, 8, 128), dtype=torch.float16, device="cuda")
    ftm.ftm_prefill_mha(g["q"][:, :S - 1].contiguous(), g["k_new"][:, :S - 1].contiguous(),
                        g["v_new"][:, :S - 1].contiguous(), g["bias"], kc, vc, None, part, kv_scales=sc)
    dec = torch.empty((2, 8, 128), dtype=torch.float16, device="cuda")
    ftm.ftm_decode_mha(g["q"][:, S - 1].contiguous(), g["k_new"][:, S - 1].contiguous(),
                       g["v_new"][:, S - 1].contiguous(), g["bias"], kc, vc, None, S, dec, kv_scales=sc)
    torch.cuda.synchronize()
    d = (dec.float() - full[:, S - 1].float()).abs().max().item()
    assert d <= 2e-3, d
    assert torch.equal(part, full[:, :S - 1])


def test_int8_paged_prefill_pages_outside_the_pool(ftm):
    case = W.PrefillCase("t", 3, 260, 4, 2, 128, "i8", 320, lens=(200, 260), seed=161)
    inp = W.prefill_to_paged(W.make_prefill_inputs(case, "cpu", poison=True), case, 64)
    n_pages = inp["k_pages"].shape[0]
    inp["block_table"][1, 1] = n_pages + 5                  # sequence 1: its second page is outside the pool
    inp["block_table"][2, 0] = -7                           # sequence 2: its first page
    run_and_compare(ftm, case, inp, "int8 paged prefill, pages outside the pool", paged=True)


def test_int8_prefill_invalid_lengths(ftm):
    case = W.PrefillCase("t", 3, 100, 4, 2, 128, "i8", 128, seed=171)
    inp = W.make_prefill_inputs(case, "cpu", poison=True)
    inp["seq_lens"] = torch.tensor([100, 0, 101], dtype=torch.int32)
    run_and_compare(ftm, case, inp, "int8 prefill invalid lengths", paged=False)


def test_full_size_int8_prefill_sampled_heads(ftm):
    """The INT8 benchmark prefill at full size: codes and scales of two
    (sequence, KV head) pairs are checked bytewise and their outputs
    recomputed by the oracle; the paged call with the same inputs gives the
    same outputs bit for bit."""
    case = W.PREFILL_CASES["prefill_int8"]
    inp = W.make_prefill_inputs(case, "cuda", poison=False)
    contiguous = {k: v.clone() for k, v in inp.items()}
    H, Hkv, D, S = case.n_heads, case.n_kv_heads, case.head_dim, case.prompt
    out = torch.zeros((case.batch, S, H, D), dtype=torch.float16, device="cuda")
    print("[full prefill_int8] gpu", flush=True)
    c = contiguous
    ftm.ftm_prefill_mha(c["q"], c["k_new"], c["v_new"], c["bias"], c["k_cache"], c["v_cache"], c["seq_lens"], out,
                        kv_scales=c["kv_scales"])
    paged = W.prefill_to_paged(inp, case, 256)
    pout = torch.zeros_like(out)
    ftm.ftm_prefill_mha_paged(paged["q"], paged["k_new"], paged["v_new"], paged["bias"], paged["k_pages"],
                              paged["v_pages"], paged["block_table"], paged["seq_lens"], pout,
                              kv_scales=paged["kv_scales"])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), pout.view(torch.int16)), "paged and contiguous INT8 prefill differ"
    G = H // Hkv
    bias = c["bias"].cpu()
    for b, h in ((0, 0), (case.batch - 1, H - 1)):
        j = h // G
        sub_bias = torch.cat([bias[h * D:(h + 1) * D], bias[(H + j) * D:(H + j + 1) * D],
                              bias[(H + Hkv + j) * D:(H + Hkv + j + 1) * D]])
        q = to_np(c["q"][b:b + 1, :, h:h + 1].cpu(), "f16")
        kn = to_np(c["k_new"][b:b + 1, :, j:j + 1].cpu(), "f16")
        vn = to_np(c["v_new"][b:b + 1, :, j:j + 1].cpu(), "f16")
        kc = np.zeros((1, 1, case.max_seq_len, D), dtype=np.int8)
        vc = kc.copy()
        sc = np.zeros((2, 1, 1, case.max_seq_len), dtype=np.float32)
        print(f"[full prefill_int8] oracle b{b} h{h}", flush=True)
        ref = oracle.prefill_mha(q, kn, vn, to_np(sub_bias, "f16"), kc, vc, None, 1, 1, D, "i8", sc)
        assert c["k_cache"][b, j].cpu().numpy().tobytes() == kc.tobytes(), "K codes"
        assert c["v_cache"][b, j].cpu().numpy().tobytes() == vc.tobytes(), "V codes"
        assert c["kv_scales"][:, b, j].cpu().numpy().tobytes() == sc.tobytes(), "scales"
        ac = W.Case("p", 1, 1, 1, D, "i8", ctx=S, max_seq_len=case.max_seq_len, value_scale=1.0)
        check(ac, out_to_f64(out[b:b + 1, :, h:h + 1]).reshape(S, 1, D), ref.reshape(S, 1, D),
              f"full prefill_int8 b{b} h{h}")


def test_int8_prefill_quantisation_ties(ftm):
    """Rows whose quotients x / s fall exactly on half-integers (absmax 127,
    so s = 1) or within a few ulps of them (absmax 127 (1 + 2^-10)): the
    codes must still equal the oracle's, which rounds the IEEE quotient to
    even."""
    case = W.PrefillCase("t", 2, 96, 4, 2, 128, "i8", 96, seed=181)
    inp = W.make_prefill_inputs(case, "cpu", poison=True)
    inp["bias"].zero_()                     # x = the stored value exactly
    g = torch.Generator().manual_seed(5)
    for name in ("k_new", "v_new"):
        t = inp[name]
        for pos in range(0, 96, 3):
            row = (torch.randint(-126, 126, (128,), generator=g).float() + 0.5)
            row[pos % 128] = 127.0 if pos % 2 == 0 else 127.0 * (1 + 2 ** -10)
            t[pos % 2, pos, pos % 2] = row.to(torch.float16)
    run_and_compare(ftm, case, inp, "int8 prefill quantisation ties", paged=False)


def test_int8_prefill_v_rows_of_any_fp16_size(ftm):
    """V rows whose absolute maximum is far past 32496, where a weight (up to
    2^8 against the running reference) times the V scale would leave the
    fp16 range if the staging held the plain scale: one row at 40000, and
    every row of another KV head shifted by a bias of up to 30000 with one
    of them reaching 60000 (outputs stay inside the fp16 range).  Every
    output row meets the bar against the oracle and the cache holds its
    codes and scales."""
    case = W.PrefillCase("t", 2, 200, 8, 2, 128, "i8", 208, lens=(150, 200), seed=151)
    inp = W.make_prefill_inputs(case, "cpu", poison=True)
    H, Hkv, D = case.n_heads, case.n_kv_heads, case.head_dim
    inp["v_new"][0, 77, 1, :] = torch.linspace(-40000.0, 40000.0, D).half()
    inp["v_new"][1, 30, 0, :] = torch.linspace(-30000.0, 30000.0, D).half()
    inp["bias"][(H + Hkv) * D:(H + Hkv + 1) * D] = torch.linspace(-30000.0, 30000.0, D).half()
    npi = host(inp)
    lens = inp["seq_lens"].numpy().astype(np.int32)
    ref = oracle.prefill_mha(npi["q"], npi["k_new"], npi["v_new"], npi["bias"], npi["k_cache"], npi["v_cache"],
                             lens, H, Hkv, D, "i8", npi["kv_scales"])
    g = {k: v.cuda() for k, v in inp.items()}
    out = torch.zeros((case.batch, case.prompt, H, D), dtype=torch.float16, device="cuda")
    ftm.ftm_prefill_mha(g["q"], g["k_new"], g["v_new"], g["bias"], g["k_cache"], g["v_cache"], g["seq_lens"],
                        out, kv_scales=g["kv_scales"])
    torch.cuda.synchronize()
    for name in ("k_cache", "v_cache", "kv_scales"):
        assert g[name].cpu().numpy().tobytes() == npi[name].tobytes(), name
    assert npi["kv_scales"][1, 0, 1, 77] > 65504.0 / 256 and npi["kv_scales"][1, 1, 0, 30] > 450
    got = out_to_f64(out)
    ac = W.Case("p", case.batch, H, Hkv, D, "i8", ctx=case.prompt, max_seq_len=case.max_seq_len, value_scale=1.0)
    for b in range(case.batch):
        Sb = int(lens[b])
        assert np.isfinite(got[b, :Sb]).all()
        # the absolute bar grows with the values: an fp32 sum of at most Sb
        # weighted values errs by up to Sb 2^-24 max|v|, far above 2e-3 at
        # |v| ~ 6e4; the row-relative bar (1e-2) stays as it is
        vmax = 127.0 * float(npi["kv_scales"][1, b, :, :Sb].max())
        check(ac, got[b, :Sb], ref[b, :Sb], f"int8 prefill large V rows b{b}",
              tol=(2e-3 + Sb * 2.0 ** -24 * vmax, 1e-2))

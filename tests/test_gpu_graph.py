"""GPU: a decode step of several layers captured into a HIP graph through
the C ABI (ftm_graph_begin / ftm_graph_end / ftm_graph_launch) and replayed.

Each replay runs with new query values written into the captured buffers
between replays, with the program's own eager work and synchronisations in
between, and every replay's outputs must be bitwise those of the eager
calls on the same inputs (the graph holds the same kernels on the same
pointers).  The layers cover every kernel kind: the single pass, the split
pass with its combine kernel, the grouped-query pass with its per-unit
counters, INT8, and a paged cache.  No memset is recorded: the library's
counters are cleared by the kernel that uses them."""
import numpy as np
import pytest
import torch

import oracle
from decode_step_attention_amd import workloads as W
from tests.helpers import inputs_to_np, run_oracle
from tests.test_gpu_parity import bits, check, small

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ftm():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from decode_step_attention_amd import ftm as m
    yield m
    m.ftm_set_split_chunk(0)


def layer_cases():
    return [
        ("mha f16", small("f16", D=128, H=8, Hkv=8, seed=101), 0),
        ("split f16", small("f16", D=64, H=4, Hkv=4, B=2, seed=102), 256),
        ("gqa bf16", small("bf16", D=128, H=8, Hkv=1, B=3, seed=103).with_(lens=(600, 1100)), 0),
        ("int8", small("i8", D=128, H=8, Hkv=8, seed=104), 0),
        ("paged f16", small("f16", D=128, H=8, Hkv=2, seed=105), 0),
    ]


def build_layers():
    layers = []
    for name, case, chunk in layer_cases():
        inp = W.make_inputs(case, "cpu", poison=True)
        if name.startswith("paged"):
            inp = W.to_paged(inp, case, 32)
        host = inp
        g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp.items()}
        out = torch.empty((case.batch, case.n_heads, case.head_dim),
                          dtype=W.TORCH_DTYPES[case.act_dtype], device="cuda")
        layers.append(dict(name=name, case=case, chunk=chunk, g=g, out=out, host=host))
    return layers


def call(ftm, L, out, stream):
    g = L["g"]
    ftm.ftm_set_split_chunk(L["chunk"])
    try:
        if "k_pages" in g:
            ftm.ftm_decode_mha_paged(g["q"], g["k_new"], g["v_new"], g["bias"], g["k_pages"],
                                     g["v_pages"], g["block_table"], g["seq_lens"], g["step"], out,
                                     g.get("kv_scales"), stream=stream)
        else:
            ftm.ftm_decode_mha(g["q"], g["k_new"], g["v_new"], g["bias"], g["k_cache"], g["v_cache"],
                               g["seq_lens"], g["step"], out, g.get("kv_scales"), stream=stream)
    finally:
        ftm.ftm_set_split_chunk(0)


def test_graph_replays_match_eager_calls(ftm):
    layers = build_layers()
    s = torch.cuda.Stream()
    sp = s.cuda_stream
    refs = [torch.empty_like(L["out"]) for L in layers]
    # one eager call per layer grows this stream's workspace before capture
    for L, r in zip(layers, refs):
        call(ftm, L, r, sp)
    s.synchronize()
    print("[graph] capturing", flush=True)
    ftm.ftm_graph_begin(sp)
    try:
        for L in layers:
            call(ftm, L, L["out"], sp)
    finally:
        graph = ftm.ftm_graph_end(sp)
    try:
        gen = torch.Generator().manual_seed(7)
        for rep in range(3):
            with torch.cuda.stream(s):
                for L in layers:
                    q = L["g"]["q"]
                    fresh = (torch.randn(q.shape, generator=gen) / np.sqrt(q.shape[-1])).to(q.dtype)
                    q.copy_(fresh.cuda(), non_blocking=False)
                    L["out"].fill_(float("nan"))
            print(f"[graph] replay {rep}", flush=True)
            ftm.ftm_graph_launch(graph, sp)
            s.synchronize()
            got = [L["out"].clone() for L in layers]
            for L, r in zip(layers, refs):
                call(ftm, L, r, sp)
            s.synchronize()
            torch.cuda.synchronize()
            for L, gt, r in zip(layers, got, refs):
                assert torch.equal(bits(gt), bits(r)), f"replay {rep}: {L['name']} differs from eager"
        # the last replay of the first layer against the oracle as well
        L = layers[0]
        case = L["case"]
        npi = inputs_to_np({**L["host"], "q": L["g"]["q"].cpu()}, case.kv_dtype)
        ref, _ = run_oracle(oracle, case, npi, n_threads=8)
        check(case, got[0], ref, "graph replay vs oracle")
    finally:
        ftm.ftm_graph_destroy(graph)


def test_capture_refuses_to_grow_the_workspace(ftm):
    """A split call on a stream whose workspace is too small is refused under
    capture (nothing recorded, the capture stays valid); a single-pass call
    recorded after it replays correctly."""
    s = torch.cuda.Stream()
    sp = s.cuda_stream
    split = small("f16", D=128, H=8, Hkv=8, B=2, seed=111)
    ins = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in W.make_inputs(split, "cpu").items()}
    out_s = torch.empty((2, 8, 128), dtype=torch.float16, device="cuda")
    direct = W.Case("direct", 8, 32, 32, 128, "f16", ctx=512, max_seq_len=512,
                    value_scale=1 / np.sqrt(128), seed=112)
    ind = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in W.make_inputs(direct, "cpu").items()}
    out_d = torch.empty((8, 32, 128), dtype=torch.float16, device="cuda")
    ref_d = torch.empty_like(out_d)
    ftm.ftm_decode_mha(ind["q"], ind["k_new"], ind["v_new"], ind["bias"], ind["k_cache"],
                       ind["v_cache"], ind["seq_lens"], ind["step"], ref_d, stream=sp)
    s.synchronize()
    ftm.ftm_graph_begin(sp)
    err = None
    try:
        ftm.ftm_set_split_chunk(256)
        try:
            ftm.ftm_decode_mha(ins["q"], ins["k_new"], ins["v_new"], ins["bias"], ins["k_cache"],
                               ins["v_cache"], ins["seq_lens"], ins["step"], out_s, stream=sp)
        except RuntimeError as e:
            err = str(e)
        finally:
            ftm.ftm_set_split_chunk(0)
        ftm.ftm_decode_mha(ind["q"], ind["k_new"], ind["v_new"], ind["bias"], ind["k_cache"],
                           ind["v_cache"], ind["seq_lens"], ind["step"], out_d, stream=sp)
    finally:
        graph = ftm.ftm_graph_end(sp)
    try:
        assert err is not None and "captured" in err, err
        out_d.fill_(float("nan"))
        torch.cuda.synchronize()
        ftm.ftm_graph_launch(graph, sp)
        s.synchronize()
        assert torch.equal(bits(out_d), bits(ref_d))
    finally:
        ftm.ftm_graph_destroy(graph)


@pytest.mark.parametrize("dt", ["bf16", "i8"])
@pytest.mark.parametrize("paged", [False, True])
def test_prefill_graph_replays_match_eager_calls(ftm, paged, dt):
    """A prefill (append + attention) captured into a graph: every replay,
    with new query values between replays and eager work in between, must
    give the eager call's outputs and caches bit for bit.  A prefill with a
    bias keeps its bias terms (float caches) or its staged codes (INT8) in
    the stream's workspace, so one eager call on the stream sizes it before
    the capture."""
    case = W.PrefillCase("t", 2, 200, 8, 2, 128, dt, 256, lens=(120, 200), seed=111)
    inp = W.make_prefill_inputs(case, "cpu", poison=True)
    if paged:
        inp = W.prefill_to_paged(inp, case, 64)
    g = {k: v.cuda() for k, v in inp.items()}
    ck, cv = ("k_pages", "v_pages") if paged else ("k_cache", "v_cache")
    act = torch.float16 if dt == "i8" else torch.bfloat16
    out = torch.zeros((case.batch, case.prompt, case.n_heads, case.head_dim), dtype=act, device="cuda")
    stream = torch.cuda.Stream()

    def prefill(o):
        sc = g.get("kv_scales")
        if paged:
            ftm.ftm_prefill_mha_paged(g["q"], g["k_new"], g["v_new"], g["bias"], g[ck], g[cv], g["block_table"],
                                      g["seq_lens"], o, stream=stream.cuda_stream, kv_scales=sc)
        else:
            ftm.ftm_prefill_mha(g["q"], g["k_new"], g["v_new"], g["bias"], g[ck], g[cv], g["seq_lens"], o,
                                stream=stream.cuda_stream, kv_scales=sc)

    prefill(torch.zeros_like(out))
    stream.synchronize()
    ftm.ftm_graph_begin(stream.cuda_stream)
    try:
        prefill(out)
    finally:
        graph = ftm.ftm_graph_end(stream.cuda_stream)
    try:
        gen = torch.Generator().manual_seed(5)
        for rep in range(3):
            scale = 1.0 if dt == "i8" else 1.0 / np.sqrt(case.head_dim)
            q_new = (torch.randn(g["q"].shape, generator=gen) * scale).to(act)
            g["q"].copy_(q_new.cuda())
            torch.cuda.synchronize()
            ftm.ftm_graph_launch(graph, stream.cuda_stream)
            stream.synchronize()
            got, got_k = out.clone(), g[ck].clone()
            got_s = g["kv_scales"].clone() if dt == "i8" else None
            _ = (g["q"].float() * 2).sum().item()          # eager work between replays
            ref = torch.zeros_like(out)
            with torch.cuda.stream(stream):
                prefill(ref)
            stream.synchronize()
            assert torch.equal(bits(got), bits(ref)), f"replay {rep}: outputs"
            assert torch.equal(bits(got_k), bits(g[ck])), f"replay {rep}: caches"
            if dt == "i8":
                assert torch.equal(got_s.view(torch.int32), g["kv_scales"].view(torch.int32)), f"replay {rep}: scales"
    finally:
        ftm.ftm_graph_destroy(graph)


@pytest.mark.parametrize("ks", ["1", "2", "3"])
def test_projection_graph_replays_match_eager_calls(ftm, tuning, ks):
    """The fused QKV projection captured into a graph, in one pass and with
    the hidden dimension split over two or three workgroups (their partial
    sums go through the stream's workspace and a per-column count that the
    kernel clears): every replay, with new x between replays and eager work
    in between, must give the eager call's q, k_new and v_new bit for bit.
    One eager call on the stream sizes the workspace before the capture."""
    tuning.set("FTM_QKV_K_SPLIT", ks)
    case = W.ProjCase("g", 64, 8, 2, 128, 2048, "f16", seed=121)
    g = {k: v.cuda() for k, v in W.make_proj_inputs(case).items()}
    B, H, Hkv, D = case.batch, case.n_heads, case.n_kv_heads, case.head_dim
    outs = [torch.empty((B, H, D), dtype=torch.float16, device="cuda"),
            torch.empty((B, Hkv, D), dtype=torch.float16, device="cuda"),
            torch.empty((B, Hkv, D), dtype=torch.float16, device="cuda")]
    refs = [torch.empty_like(o) for o in outs]
    stream = torch.cuda.Stream()

    def proj(dst):
        ftm.ftm_qkv_proj(g["x"], g["w"], g["bias"], *dst, stream=stream.cuda_stream)

    proj(refs)
    stream.synchronize()
    ftm.ftm_graph_begin(stream.cuda_stream)
    try:
        proj(outs)
    finally:
        graph = ftm.ftm_graph_end(stream.cuda_stream)
    try:
        gen = torch.Generator().manual_seed(9)
        for rep in range(3):
            x_new = torch.randn(g["x"].shape, generator=gen).to(torch.float16)
            g["x"].copy_(x_new.cuda())
            for o in outs:
                o.fill_(float("nan"))
            torch.cuda.synchronize()
            ftm.ftm_graph_launch(graph, stream.cuda_stream)
            stream.synchronize()
            got = [o.clone() for o in outs]
            _ = (g["x"].float() * 2).sum().item()          # eager work between replays
            proj(refs)
            stream.synchronize()
            for name, a, r in zip(("q", "k_new", "v_new"), got, refs):
                assert torch.equal(bits(a), bits(r)), f"replay {rep}: {name} differs from eager"
    finally:
        ftm.ftm_graph_destroy(graph)


def test_projection_capture_needs_a_sized_workspace(ftm, tuning):
    """A k-split projection captured before any eager call has sized the
    stream's workspace is refused (nothing recorded, the capture stays
    valid); a one-pass projection recorded after it replays correctly."""
    torch.cuda.synchronize()
    ftm.ftm_release_workspaces()            # torch may hand out a stream a previous test used
    case = W.ProjCase("g", 48, 4, 4, 64, 1024, "bf16", seed=122)
    g = {k: v.cuda() for k, v in W.make_proj_inputs(case).items()}
    B, H, Hkv, D = case.batch, case.n_heads, case.n_kv_heads, case.head_dim

    def buffers():
        return [torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda"),
                torch.empty((B, Hkv, D), dtype=torch.bfloat16, device="cuda"),
                torch.empty((B, Hkv, D), dtype=torch.bfloat16, device="cuda")]
    outs, refs = buffers(), buffers()
    stream = torch.cuda.Stream()
    tuning.set("FTM_QKV_K_SPLIT", "1")
    ftm.ftm_qkv_proj(g["x"], g["w"], g["bias"], *refs, stream=stream.cuda_stream)
    stream.synchronize()
    err = None
    ftm.ftm_graph_begin(stream.cuda_stream)
    try:
        tuning.set("FTM_QKV_K_SPLIT", "2")
        try:
            ftm.ftm_qkv_proj(g["x"], g["w"], g["bias"], *outs, stream=stream.cuda_stream)
        except RuntimeError as e:
            err = str(e)
        tuning.set("FTM_QKV_K_SPLIT", "1")
        ftm.ftm_qkv_proj(g["x"], g["w"], g["bias"], *outs, stream=stream.cuda_stream)
    finally:
        graph = ftm.ftm_graph_end(stream.cuda_stream)
    try:
        assert err is not None and "captured" in err, err
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        ftm.ftm_graph_launch(graph, stream.cuda_stream)
        stream.synchronize()
        for name, a, r in zip(("q", "k_new", "v_new"), outs, refs):
            assert torch.equal(bits(a), bits(r)), f"{name} differs from eager"
    finally:
        ftm.ftm_graph_destroy(graph)

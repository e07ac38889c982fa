"""Host-side logic of libftm, runnable without a GPU: the library loads and
exports every symbol of include/ftm.h, argument errors are reported before
anything touches the device, and the cache sizing matches the pages'
worked examples (tests/golden/kv_cache_sizing.json)."""
import ctypes
import json
import os
import re

import pytest

from decode_step_attention_amd import ftm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "ftm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ftm_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_exactly_the_binding_exports():
    assert header_functions() == sorted(ftm.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(ftm.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name


def test_version_and_empty_error():
    assert "gfx950" in ftm.ftm_version()


def test_kv_cache_bytes_pages_examples():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "kv_cache_sizing.json")))
    ex1, ex2 = g["examples"]
    per_layer = ftm.ftm_kv_cache_bytes(ex1["batch"], ex1["n_kv_heads"], ex1["context"],
                                       ex1["head_dim"], ftm.FTM_F16)
    assert per_layer * ex1["layers"] == ex1["expected_kv_bytes_all_layers"]
    # the page's own product is one of K and V
    assert per_layer * ex1["layers"] == 2 * ex1["page_product_bytes"]
    # "about 32 GB": 32 GiB is 34.4 GB, within the page's rounding
    assert abs(per_layer * ex1["layers"] / 2 ** 30 - 32) < 1e-9
    one_tok = ftm.ftm_kv_cache_bytes(1, ex2["n_kv_heads"], 1, ex2["head_dim"], ftm.FTM_F16)
    assert one_tok // 2 * ex2["layers"] == ex2["expected_k_only_per_token_all_layers"]
    assert one_tok // 2 * ex2["layers"] == ex2["page_per_token_bytes"]
    assert one_tok // 2 * ex2["layers"] * ex2["context"] == ex2["expected_k_only_per_request"]


def test_kv_cache_bytes_dtypes_and_invalid():
    assert ftm.ftm_kv_cache_bytes(2, 3, 5, 64, ftm.FTM_F32) == 2 * 2 * 3 * 5 * 64 * 4
    assert ftm.ftm_kv_cache_bytes(2, 3, 5, 64, ftm.FTM_BF16) == 2 * 2 * 3 * 5 * 64 * 2
    assert ftm.ftm_kv_cache_bytes(2, 3, 5, 128, ftm.FTM_I8) == 2 * 2 * 3 * 5 * (128 + 4)
    assert ftm.ftm_kv_cache_bytes(0, 3, 5, 64, ftm.FTM_F16) == 0
    assert ftm.ftm_kv_cache_bytes(1, 1, 1, 64, 9) == 0


A = 0x10000  # a 16-byte aligned fake device address; never dereferenced


def call(**kw):
    args = dict(q=A, k_new=A, v_new=A, qkv_bias=A, k_cache=A, v_cache=A, seq_lens=A, batch=2,
                max_seq_len=16, step=8, n_heads=4, n_kv_heads=2, head_dim=128,
                kv_dtype=ftm.FTM_F16, kv_scales=None, out=A, stream=None)
    args.update(kw)
    rc = ftm.ftm_decode_mha_raw(**args)
    return rc, ftm.ftm_last_error()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), 1, "NULL"),
    (dict(out=None), 1, "NULL"),
    (dict(k_cache=None), 1, "NULL"),
    (dict(batch=0), 1, ">= 1"),
    (dict(n_heads=5), 1, "multiple"),
    (dict(step=0), 1, "step"),
    (dict(step=17), 1, "step"),
    (dict(kv_dtype=7), 1, "kv_dtype"),
    (dict(kv_dtype=ftm.FTM_I8), 1, "kv_scales"),
    (dict(kv_scales=A), 1, "kv_scales"),
    (dict(q=A + 2), 1, "aligned"),
    (dict(k_cache=A + 8), 1, "aligned"),
    (dict(seq_lens=A + 2), 1, "aligned"),
    (dict(head_dim=96), 2, "head_dim"),
    (dict(head_dim=256), 2, "head_dim"),
])
def test_argument_errors_return_before_any_device_call(kw, status, needle):
    rc, msg = call(**kw)
    assert rc == status
    assert needle in msg


def test_split_chunk_setting_roundtrip():
    prev = ftm.ftm_set_split_chunk(512)
    assert ftm.ftm_set_split_chunk(prev) == 512
    assert ftm.ftm_set_split_chunk(-1) == -1


def test_binding_rejects_mismatched_tensors():
    import torch
    q = torch.zeros(2, 4, 128, dtype=torch.float16)
    kc = torch.zeros(2, 2, 16, 128, dtype=torch.float16)
    kn = torch.zeros(2, 2, 128, dtype=torch.float16)
    with pytest.raises(TypeError):
        ftm.ftm_decode_mha(q.float(), kn, kn, None, kc, kc, None, 8, q)
    with pytest.raises(ValueError):
        ftm.ftm_decode_mha(q, kn[:, :1], kn, None, kc, kc, None, 8, q)
    with pytest.raises(ValueError):
        ftm.ftm_decode_mha(q, kn, kn, None, kc, kc.transpose(2, 3), None, 8, q)


def call_paged(**kw):
    args = [("q", A), ("k_new", A), ("v_new", A), ("qkv_bias", A), ("k_pages", A), ("v_pages", A),
            ("block_table", A), ("n_pages", 10), ("page_size", 16), ("max_pages_per_seq", 4),
            ("seq_lens", A), ("batch", 2), ("step", 40), ("n_heads", 4), ("n_kv_heads", 2),
            ("head_dim", 128), ("kv_dtype", ftm.FTM_F16), ("kv_scales", None), ("out", A),
            ("stream", None)]
    vals = [kw.get(k, v) for k, v in args]
    rc = ftm.lib.ftm_decode_mha_paged(*vals)
    return rc, ftm.ftm_last_error()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(block_table=None), 1, "block_table"),
    (dict(block_table=A + 2), 1, "aligned"),
    (dict(n_pages=0), 1, "n_pages"),
    (dict(max_pages_per_seq=0), 1, "max_pages_per_seq"),
    (dict(page_size=8), 1, "page_size"),
    (dict(page_size=48), 1, "power of two"),
    (dict(page_size=1 << 17), 1, "page_size"),
    (dict(step=65), 1, "max_pages_per_seq * page_size"),
    (dict(max_pages_per_seq=1 << 20, page_size=1 << 12), 2, "2^31"),
    (dict(k_pages=A + 8), 1, "aligned"),
    (dict(q=None), 1, "NULL"),
    (dict(kv_dtype=ftm.FTM_I8), 1, "kv_scales"),
    (dict(head_dim=96), 2, "head_dim"),
])
def test_paged_argument_errors_return_before_any_device_call(kw, status, needle):
    rc, msg = call_paged(**kw)
    assert rc == status
    assert needle in msg


def test_graph_argument_errors():
    assert ftm.lib.ftm_graph_begin(None) == 1
    assert "null stream" in ftm.ftm_last_error()
    assert ftm.lib.ftm_graph_end(None, None) == 1
    assert ftm.lib.ftm_graph_launch(None, None) == 1
    assert "graph is NULL" in ftm.ftm_last_error()
    assert ftm.lib.ftm_graph_destroy(None) == 0


def test_binding_rejects_mismatched_paged_tensors():
    import torch
    q = torch.zeros(2, 4, 128, dtype=torch.float16)
    kn = torch.zeros(2, 2, 128, dtype=torch.float16)
    kp = torch.zeros(6, 2, 16, 128, dtype=torch.float16)
    tbl = torch.zeros(2, 3, dtype=torch.int32)
    with pytest.raises(TypeError):
        ftm.ftm_decode_mha_paged(q, kn, kn, None, kp, kp, tbl.long(), None, 8, q)
    with pytest.raises(ValueError):
        ftm.ftm_decode_mha_paged(q, kn, kn, None, kp, kp[:, :1], tbl, None, 8, q)
    with pytest.raises(ValueError):
        ftm.ftm_decode_mha_paged(q, kn, kn, None, kp, kp, tbl[:1], None, 8, q)


def call_qkv(**kw):
    args = [("x", A), ("w", A), ("bias", None), ("q", A), ("k_new", A), ("v_new", A), ("batch", 8),
            ("hidden", 4096), ("n_heads", 32), ("n_kv_heads", 32), ("head_dim", 128),
            ("act_dtype", ftm.FTM_F16), ("stream", None)]
    vals = [kw.get(k, v) for k, v in args]
    rc = ftm.lib.ftm_qkv_proj(*vals)
    return rc, ftm.ftm_last_error()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(x=None), 1, "NULL"),
    (dict(v_new=None), 1, "NULL"),
    (dict(batch=0), 1, ">= 1"),
    (dict(n_heads=31), 1, "multiple"),
    (dict(act_dtype=ftm.FTM_F32), 2, "fp16 or bf16"),
    (dict(act_dtype=ftm.FTM_I8), 1, "fp16 or bf16"),
    (dict(w=A + 4), 1, "aligned"),
    (dict(bias=A + 2), 1, "aligned"),
    (dict(batch=65), 2, "batch"),
    (dict(hidden=4000), 2, "hidden"),
    (dict(hidden=1 << 17), 2, "hidden"),
    (dict(head_dim=72), 2, "head_dim"),
])
def test_projection_argument_errors_return_before_any_device_call(kw, status, needle):
    rc, msg = call_qkv(**kw)
    assert rc == status
    assert needle in msg


def test_binding_rejects_mismatched_projection_tensors():
    import torch
    x = torch.zeros(2, 256, dtype=torch.bfloat16)
    w = torch.zeros((4 + 2 * 2) * 16, 256, dtype=torch.bfloat16)
    q = torch.zeros(2, 4, 16, dtype=torch.bfloat16)
    k = torch.zeros(2, 2, 16, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        ftm.ftm_qkv_proj(x.float(), w, None, q, k, k)
    with pytest.raises(ValueError):
        ftm.ftm_qkv_proj(x, w[:-16], None, q, k, k)
    with pytest.raises(TypeError):
        ftm.ftm_qkv_proj(x, w.half(), None, q, k, k)


def call_prefill(**kw):
    args = [("q", A), ("k_new", A), ("v_new", A), ("bias", None), ("k_cache", A), ("v_cache", A),
            ("seq_lens", None), ("batch", 4), ("max_seq_len", 2048), ("prompt_len", 2048), ("n_heads", 32),
            ("n_kv_heads", 32), ("head_dim", 128), ("kv_dtype", ftm.FTM_F16), ("kv_scales", None), ("out", A),
            ("stream", None)]
    vals = [kw.get(k, v) for k, v in args]
    rc = ftm.lib.ftm_prefill_mha(*vals)
    return rc, ftm.ftm_last_error()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), 1, "NULL"),
    (dict(out=None), 1, "NULL"),
    (dict(batch=0), 1, ">= 1"),
    (dict(n_heads=31), 1, "multiple"),
    (dict(prompt_len=0), 1, "prompt_len"),
    (dict(prompt_len=2049), 1, "prompt_len"),
    (dict(kv_dtype=ftm.FTM_F32), 2, "fp16, bf16 or INT8"),
    (dict(kv_dtype=ftm.FTM_I8), 1, "kv_scales"),
    (dict(kv_scales=A), 1, "kv_scales"),
    (dict(kv_dtype=ftm.FTM_I8, kv_scales=A + 2), 1, "4-byte aligned"),
    (dict(kv_dtype=7), 1, "kv_dtype"),
    (dict(k_cache=A + 8), 1, "aligned"),
    (dict(seq_lens=A + 2), 1, "aligned"),
    (dict(head_dim=96), 2, "head_dim"),
    (dict(batch=65536, n_heads=1, n_kv_heads=1), 2, "grid"),
    (dict(batch=40000, n_heads=65536, n_kv_heads=1), 2, "grid"),
    (dict(max_seq_len=1 << 23, prompt_len=1), 2, "2 GiB"),
    (dict(max_seq_len=1 << 23, prompt_len=(1 << 23) - 64), 2, "grid"),
    (dict(kv_dtype=ftm.FTM_I8, kv_scales=A, max_seq_len=1 << 22, prompt_len=1 << 22, n_heads=64, n_kv_heads=64),
     2, "INT8 prefill"),
])
def test_prefill_argument_errors_return_before_any_device_call(kw, status, needle):
    rc, msg = call_prefill(**kw)
    assert rc == status
    assert needle in msg


def call_prefill_paged(**kw):
    args = [("q", A), ("k_new", A), ("v_new", A), ("bias", None), ("k_pages", A), ("v_pages", A),
            ("block_table", A), ("n_pages", 64), ("page_size", 256), ("max_pages", 8), ("seq_lens", None),
            ("batch", 4), ("prompt_len", 2048), ("n_heads", 32), ("n_kv_heads", 32), ("head_dim", 128),
            ("kv_dtype", ftm.FTM_F16), ("kv_scales", None), ("out", A), ("stream", None)]
    vals = [kw.get(k, v) for k, v in args]
    rc = ftm.lib.ftm_prefill_mha_paged(*vals)
    return rc, ftm.ftm_last_error()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(block_table=None), 1, "block_table is NULL"),
    (dict(block_table=A + 2), 1, "4-byte aligned"),
    (dict(n_pages=0), 1, "n_pages"),
    (dict(max_pages=0), 1, "max_pages_per_seq"),
    (dict(page_size=8), 1, "power of two"),
    (dict(page_size=96), 1, "power of two"),
    (dict(page_size=1 << 17), 1, "power of two"),
    (dict(prompt_len=2049), 1, "prompt_len"),
    (dict(max_pages=1 << 16, page_size=1 << 16), 2, "2^31"),
    (dict(kv_dtype=ftm.FTM_I8), 1, "kv_scales"),
    (dict(kv_dtype=ftm.FTM_I8, kv_scales=A, max_pages=1 << 15, prompt_len=(1 << 23) - 128, n_heads=64,
          n_kv_heads=64), 2, "INT8 prefill"),
    (dict(kv_dtype=ftm.FTM_F32), 2, "fp16, bf16 or INT8"),
    (dict(q=None), 1, "NULL"),
    (dict(head_dim=96), 2, "head_dim"),
])
def test_paged_prefill_argument_errors_return_before_any_device_call(kw, status, needle):
    rc, msg = call_prefill_paged(**kw)
    assert rc == status, msg
    assert needle in msg


def _compile(tmp_path, compiler, lang_flags, body, extra=()):
    import subprocess
    src = tmp_path / ("probe.c" if compiler == "gcc" else "probe.cpp")
    src.write_text(body)
    cmd = [compiler, *lang_flags, "-fsyntax-only", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
           *extra, str(src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_header_is_plain_c11(tmp_path):
    """include/ftm.h compiles as C11 on its own: plain pointers, sizes and the
    two enums, with HIP's stream handle declared as HIP declares it."""
    _compile(tmp_path, "gcc", ["-std=c11"], '#include "ftm.h"\n'
             "static int (*p)(const void*, const void*, const void*, const void*, void*, void*,\n"
             "              const int32_t*, int, int, int, int, int, int, ftm_dtype, float*, void*,\n"
             "              hipStream_t) = ftm_decode_mha;\n"
             "int main(void) { return p == 0; }\n")


def test_header_next_to_hip_runtime(tmp_path):
    """The header's stream typedef is HIP's own: including both compiles."""
    _compile(tmp_path, "g++", ["-std=c++17", "-D__HIP_PLATFORM_AMD__"],
             '#include <hip/hip_runtime_api.h>\n#include "ftm.h"\n'
             "int main() { hipStream_t s = nullptr; ftm_dtype d = FTM_F16;\n"
             "  return ftm_decode_mha(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,\n"
             "                        1, 1, 1, 1, 1, 64, d, nullptr, nullptr, s); }\n",
             extra=("-I", "/opt/rocm/include"))


def test_compute_calls_never_wait_for_the_device():
    """The compute path of the C ABI holds no host synchronisation and no
    hipFree: the only waits are the documented ones (ftm_release_workspaces,
    ftm_timing_read, the FTM_VALIDATE check)."""
    src = open(os.path.join(ROOT, "decode_step_attention_amd", "csrc", "ftm_api.cpp")).read()
    assert "hipDeviceSynchronize" not in src
    assert "hipMemset" not in src
    waits = [m.start() for m in re.finditer(r"hipStreamSynchronize|hipEventSynchronize|hipFree\(", src)]
    allowed = {
        "hipStreamSynchronize": "FTM_VALIDATE",
        "hipEventSynchronize": "int ftm_timing_read(",
        "hipFree(": "void ftm_release_workspaces(",
    }
    for pos in waits:
        name = next(k for k in allowed if src.startswith(k, pos))
        owner = src.rfind(allowed[name], 0, pos)
        assert owner >= 0 and pos - owner < 1500, f"{name} at offset {pos} outside {allowed[name]}"

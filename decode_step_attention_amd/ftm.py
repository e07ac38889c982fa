"""Python binding of libftm (include/ftm.h): argument marshalling only.

Each function has the C entry point's name.  Tensors supply device pointers
and shapes; torch supplies the current HIP stream.  Every step of the
computation runs in the library's gfx950 kernels; there is no fallback, and
importing this module fails loudly if the built library is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Callable, Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libftm.so")

FTM_F32, FTM_F16, FTM_BF16, FTM_I8 = 0, 1, 2, 3
KV_DTYPES = {"f32": FTM_F32, "f16": FTM_F16, "bf16": FTM_BF16, "i8": FTM_I8}
_TORCH_TO_KV = {torch.float32: FTM_F32, torch.float16: FTM_F16, torch.bfloat16: FTM_BF16,
                torch.int8: FTM_I8}
_ACT = {FTM_F32: torch.float32, FTM_F16: torch.float16, FTM_BF16: torch.bfloat16,
        FTM_I8: torch.float16}

# Every symbol include/ftm.h declares.
EXPORTS = ("ftm_decode_mha", "ftm_decode_mha_static", "ftm_decode_mha_paged", "ftm_qkv_proj", "ftm_prefill_mha", "ftm_prefill_mha_paged",
           "ftm_kv_cache_bytes",
           "ftm_last_error",
           "ftm_version", "ftm_set_split_chunk", "ftm_set_workgroup_waves", "ftm_release_workspaces",
           "ftm_tuning_reload",
           "ftm_graph_begin", "ftm_graph_end", "ftm_graph_launch", "ftm_graph_destroy",
           "ftm_timing_enable", "ftm_timing_disable", "ftm_timing_read")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libftm.so is not built ({LIB_PATH}); run "
                          "`python -m decode_step_attention_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.ftm_decode_mha.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                   i32, vp, vp, vp]
    lib.ftm_decode_mha.restype = i32
    lib.ftm_decode_mha_static.argtypes = lib.ftm_decode_mha.argtypes
    lib.ftm_decode_mha_static.restype = i32
    lib.ftm_decode_mha_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, vp, i32, i32,
                                         i32, i32, i32, i32, vp, vp, vp]
    lib.ftm_decode_mha_paged.restype = i32
    lib.ftm_qkv_proj.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    lib.ftm_qkv_proj.restype = i32
    lib.ftm_prefill_mha.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp]
    lib.ftm_prefill_mha.restype = i32
    lib.ftm_prefill_mha_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, vp, i32, i32, i32, i32, i32,
                                          i32, vp, vp, vp]
    lib.ftm_prefill_mha_paged.restype = i32
    lib.ftm_graph_begin.argtypes = [vp]
    lib.ftm_graph_begin.restype = i32
    lib.ftm_graph_end.argtypes = [vp, ctypes.POINTER(vp)]
    lib.ftm_graph_end.restype = i32
    lib.ftm_graph_launch.argtypes = [vp, vp]
    lib.ftm_graph_launch.restype = i32
    lib.ftm_graph_destroy.argtypes = [vp]
    lib.ftm_graph_destroy.restype = i32
    lib.ftm_kv_cache_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.ftm_kv_cache_bytes.restype = ctypes.c_size_t
    lib.ftm_last_error.argtypes = []
    lib.ftm_last_error.restype = ctypes.c_char_p
    lib.ftm_version.argtypes = []
    lib.ftm_version.restype = ctypes.c_char_p
    lib.ftm_set_split_chunk.argtypes = [i32]
    lib.ftm_set_split_chunk.restype = i32
    lib.ftm_set_workgroup_waves.argtypes = [i32]
    lib.ftm_set_workgroup_waves.restype = i32
    lib.ftm_release_workspaces.argtypes = []
    lib.ftm_release_workspaces.restype = None
    lib.ftm_tuning_reload.argtypes = []
    lib.ftm_tuning_reload.restype = None
    lib.ftm_timing_enable.argtypes = [i32]
    lib.ftm_timing_enable.restype = i32
    lib.ftm_timing_disable.argtypes = []
    lib.ftm_timing_disable.restype = i32
    lib.ftm_timing_read.argtypes = [i32, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_double)]
    lib.ftm_timing_read.restype = i32
    return lib


lib = _load()


def ftm_last_error() -> str:
    return lib.ftm_last_error().decode()


def ftm_version() -> str:
    return lib.ftm_version().decode()


def ftm_kv_cache_bytes(batch: int, n_kv_heads: int, max_seq_len: int, head_dim: int,
                       kv_dtype: int) -> int:
    return int(lib.ftm_kv_cache_bytes(batch, n_kv_heads, max_seq_len, head_dim, kv_dtype))


def ftm_set_split_chunk(positions: int) -> int:
    return int(lib.ftm_set_split_chunk(positions))


def ftm_set_workgroup_waves(waves: int) -> int:
    return int(lib.ftm_set_workgroup_waves(waves))


def ftm_release_workspaces() -> None:
    lib.ftm_release_workspaces()


def ftm_tuning_reload() -> None:
    """Makes the library read the FTM_* tuning variables of os.environ again."""
    lib.ftm_tuning_reload()


def _check(rc: int) -> None:
    if rc != 0:
        raise RuntimeError(f"libftm status {rc}: {ftm_last_error()}")


def ftm_timing_enable(capacity: int) -> None:
    _check(lib.ftm_timing_enable(capacity))


def ftm_timing_disable() -> None:
    _check(lib.ftm_timing_disable())


def ftm_timing_read(kind: int) -> Tuple[int, float]:
    n = ctypes.c_int(0)
    ms = ctypes.c_double(0.0)
    _check(lib.ftm_timing_read(kind, ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def ftm_decode_mha_raw(q, k_new, v_new, qkv_bias, k_cache, v_cache, seq_lens, batch,
                       max_seq_len, step, n_heads, n_kv_heads, head_dim, kv_dtype, kv_scales,
                       out, stream) -> int:
    """The C entry point with integer pointers, unchanged status code."""
    return int(lib.ftm_decode_mha(q, k_new, v_new, qkv_bias, k_cache, v_cache, seq_lens, batch,
                                  max_seq_len, step, n_heads, n_kv_heads, head_dim, kv_dtype,
                                  kv_scales, out, stream))


def _check_tensors(tensors, dev) -> None:
    for name, (t, dt, shape) in tensors.items():
        if t.dtype != dt:
            raise TypeError(f"{name}: dtype {t.dtype}, expected {dt}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the cache on {dev}")


def _step_tensors(q, k_new, v_new, qkv_bias, k_cache, seq_lens, out):
    """Checks of the per-step tensors shared by both cache layouts."""
    if k_cache.dim() != 4 or q.dim() != 3:
        raise ValueError("q must be [B, H, D] and the cache 4-dimensional")
    B, H, D = q.shape
    Hkv = k_cache.shape[1]
    kv = _TORCH_TO_KV.get(k_cache.dtype)
    if kv is None:
        raise TypeError(f"unsupported cache dtype {k_cache.dtype}")
    act = _ACT[kv]
    tensors = {"q": (q, act, (B, H, D)), "k_new": (k_new, act, (B, Hkv, D)),
               "v_new": (v_new, act, (B, Hkv, D)), "out": (out, act, (B, H, D))}
    if qkv_bias is not None:
        tensors["qkv_bias"] = (qkv_bias, act, ((H + 2 * Hkv) * D,))
    if seq_lens is not None:
        tensors["seq_lens"] = (seq_lens, torch.int32, (B,))
    return B, H, Hkv, D, kv, tensors


def _stream_ptr(stream, dev):
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    return ctypes.c_void_p(stream)


def _marshal(q, k_new, v_new, qkv_bias, k_cache, v_cache, seq_lens, step, out, kv_scales, stream):
    B, H, Hkv, D, kv, tensors = _step_tensors(q, k_new, v_new, qkv_bias, k_cache, seq_lens, out)
    Lmax = k_cache.shape[2]
    tensors["k_cache"] = (k_cache, k_cache.dtype, (B, Hkv, Lmax, D))
    tensors["v_cache"] = (v_cache, k_cache.dtype, (B, Hkv, Lmax, D))
    if kv_scales is not None:
        tensors["kv_scales"] = (kv_scales, torch.float32, (2, B, Hkv, Lmax))
    _check_tensors(tensors, k_cache.device)
    return (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(qkv_bias), _ptr(k_cache), _ptr(v_cache),
            _ptr(seq_lens), B, Lmax, int(step), H, Hkv, D, kv, _ptr(kv_scales), _ptr(out),
            _stream_ptr(stream, k_cache.device))


def _marshal_paged(q, k_new, v_new, qkv_bias, k_pages, v_pages, block_table, seq_lens, step, out,
                   kv_scales, stream):
    B, H, Hkv, D, kv, tensors = _step_tensors(q, k_new, v_new, qkv_bias, k_pages, seq_lens, out)
    n_pages, _, P, _ = k_pages.shape
    if block_table.dim() != 2:
        raise ValueError("block_table must be [B, max_pages_per_seq]")
    max_pages = block_table.shape[1]
    tensors["k_pages"] = (k_pages, k_pages.dtype, (n_pages, Hkv, P, D))
    tensors["v_pages"] = (v_pages, k_pages.dtype, (n_pages, Hkv, P, D))
    tensors["block_table"] = (block_table, torch.int32, (B, max_pages))
    if kv_scales is not None:
        tensors["kv_scales"] = (kv_scales, torch.float32, (2, n_pages, Hkv, P))
    _check_tensors(tensors, k_pages.device)
    return (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(qkv_bias), _ptr(k_pages), _ptr(v_pages),
            _ptr(block_table), n_pages, P, max_pages, _ptr(seq_lens), B, int(step), H, Hkv, D, kv,
            _ptr(kv_scales), _ptr(out), _stream_ptr(stream, k_pages.device))


def ftm_decode_mha(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                   qkv_bias: Optional[torch.Tensor], k_cache: torch.Tensor, v_cache: torch.Tensor,
                   seq_lens: Optional[torch.Tensor], step: int, out: torch.Tensor,
                   kv_scales: Optional[torch.Tensor] = None, stream=None) -> None:
    """One decode step (see include/ftm.h).  Shapes: q/out [B, H, D],
    k_new/v_new [B, Hkv, D], k_cache/v_cache [B, Hkv, Lmax, D],
    qkv_bias [(H + 2 Hkv) D] or None, seq_lens int32 [B] or None,
    kv_scales fp32 [2, B, Hkv, Lmax] for an int8 cache.  Caches and scales
    are updated in place; out is written."""
    _check(lib.ftm_decode_mha(*_marshal(q, k_new, v_new, qkv_bias, k_cache, v_cache, seq_lens,
                                        step, out, kv_scales, stream)))


def ftm_decode_mha_static(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                          qkv_bias: Optional[torch.Tensor], k_cache: torch.Tensor, v_cache: torch.Tensor,
                          seq_lens: Optional[torch.Tensor], step: int, out: torch.Tensor,
                          kv_scales: Optional[torch.Tensor] = None, stream=None) -> None:
    """ftm_decode_mha with its scratch in the library's fixed device array:
    no allocation (see include/ftm.h for the limit, and for why calls that
    overlap on one GPU race)."""
    _check(lib.ftm_decode_mha_static(*_marshal(q, k_new, v_new, qkv_bias, k_cache, v_cache, seq_lens,
                                               step, out, kv_scales, stream)))


def _prepared(f, args, keep) -> Callable[[], None]:
    def call() -> None:
        rc = f(*args)
        if rc != 0:
            raise RuntimeError(f"libftm status {rc}: {ftm_last_error()}")
    call.tensors = keep
    return call


def ftm_decode_mha_prepared(q, k_new, v_new, qkv_bias, k_cache, v_cache, seq_lens, step, out,
                            kv_scales=None, stream=None) -> Callable[[], None]:
    """Checks and marshals the arguments once and returns a callable that
    issues the same ftm_decode_mha call, for loops that repeat a call on
    fixed buffers.  The tensors must stay alive and in place."""
    args = _marshal(q, k_new, v_new, qkv_bias, k_cache, v_cache, seq_lens, step, out, kv_scales,
                    stream)
    keep = (q, k_new, v_new, qkv_bias, k_cache, v_cache, seq_lens, out, kv_scales)
    return _prepared(lib.ftm_decode_mha, args, keep)


def ftm_decode_mha_paged(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                         qkv_bias: Optional[torch.Tensor], k_pages: torch.Tensor,
                         v_pages: torch.Tensor, block_table: torch.Tensor,
                         seq_lens: Optional[torch.Tensor], step: int, out: torch.Tensor,
                         kv_scales: Optional[torch.Tensor] = None, stream=None) -> None:
    """One decode step over a paged cache (see include/ftm.h).  Shapes:
    k_pages/v_pages [n_pages, Hkv, P, D], block_table int32 [B, max_pages],
    kv_scales fp32 [2, n_pages, Hkv, P] for an int8 cache; the rest as for
    ftm_decode_mha."""
    _check(lib.ftm_decode_mha_paged(*_marshal_paged(q, k_new, v_new, qkv_bias, k_pages, v_pages,
                                                    block_table, seq_lens, step, out, kv_scales,
                                                    stream)))


def ftm_decode_mha_paged_prepared(q, k_new, v_new, qkv_bias, k_pages, v_pages, block_table,
                                  seq_lens, step, out, kv_scales=None,
                                  stream=None) -> Callable[[], None]:
    """ftm_decode_mha_paged with the arguments marshalled once."""
    args = _marshal_paged(q, k_new, v_new, qkv_bias, k_pages, v_pages, block_table, seq_lens, step,
                          out, kv_scales, stream)
    keep = (q, k_new, v_new, qkv_bias, k_pages, v_pages, block_table, seq_lens, out, kv_scales)
    return _prepared(lib.ftm_decode_mha_paged, args, keep)


def _marshal_qkv(x, w, bias, q, k_new, v_new, stream):
    if x.dim() != 2 or q.dim() != 3 or k_new.dim() != 3:
        raise ValueError("x must be [B, hidden], q [B, H, D] and k_new/v_new [B, Hkv, D]")
    B, hidden = x.shape
    _, H, D = q.shape
    Hkv = k_new.shape[1]
    act = {torch.float16: FTM_F16, torch.bfloat16: FTM_BF16}.get(x.dtype)
    if act is None:
        raise TypeError(f"unsupported activation dtype {x.dtype}")
    N = (H + 2 * Hkv) * D
    tensors = {"x": (x, x.dtype, (B, hidden)), "w": (w, x.dtype, (N, hidden)),
               "q": (q, x.dtype, (B, H, D)), "k_new": (k_new, x.dtype, (B, Hkv, D)),
               "v_new": (v_new, x.dtype, (B, Hkv, D))}
    if bias is not None:
        tensors["bias"] = (bias, x.dtype, (N,))
    _check_tensors(tensors, x.device)
    return (_ptr(x), _ptr(w), _ptr(bias), _ptr(q), _ptr(k_new), _ptr(v_new), B, hidden, H, Hkv, D, act,
            _stream_ptr(stream, x.device))


def ftm_qkv_proj(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor], q: torch.Tensor,
                 k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> None:
    """The fused QKV projection (see include/ftm.h): q, k_new, v_new =
    split(x @ w.T + bias).  x [B, hidden], w [(H + 2 Hkv) D, hidden]."""
    _check(lib.ftm_qkv_proj(*_marshal_qkv(x, w, bias, q, k_new, v_new, stream)))


def ftm_qkv_proj_prepared(x, w, bias, q, k_new, v_new, stream=None) -> Callable[[], None]:
    """ftm_qkv_proj with the arguments marshalled once."""
    args = _marshal_qkv(x, w, bias, q, k_new, v_new, stream)
    return _prepared(lib.ftm_qkv_proj, args, (x, w, bias, q, k_new, v_new))


def _prefill_types(cache):
    kv = _TORCH_TO_KV.get(cache.dtype)
    if kv is None:
        raise TypeError(f"unsupported cache dtype {cache.dtype}")
    act = torch.float16 if cache.dtype == torch.int8 else cache.dtype
    return kv, act


def _marshal_prefill(q, k_new, v_new, qkv_bias, k_cache, v_cache, seq_lens, out, stream, kv_scales=None):
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q must be [B, S, H, D] and the caches [B, Hkv, Lmax, D]")
    B, S, H, D = q.shape
    _, Hkv, Lmax, _ = k_cache.shape
    kv, act = _prefill_types(k_cache)
    tensors = {"q": (q, act, (B, S, H, D)), "k_new": (k_new, act, (B, S, Hkv, D)),
               "v_new": (v_new, act, (B, S, Hkv, D)), "k_cache": (k_cache, k_cache.dtype, (B, Hkv, Lmax, D)),
               "v_cache": (v_cache, k_cache.dtype, (B, Hkv, Lmax, D)), "out": (out, act, (B, S, H, D))}
    if qkv_bias is not None:
        tensors["qkv_bias"] = (qkv_bias, act, ((H + 2 * Hkv) * D,))
    if seq_lens is not None:
        tensors["seq_lens"] = (seq_lens, torch.int32, (B,))
    if kv_scales is not None:
        tensors["kv_scales"] = (kv_scales, torch.float32, (2, B, Hkv, Lmax))
    _check_tensors(tensors, k_cache.device)
    return (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(qkv_bias), _ptr(k_cache), _ptr(v_cache),
            _ptr(seq_lens), B, Lmax, S, H, Hkv, D, kv, _ptr(kv_scales), _ptr(out),
            _stream_ptr(stream, k_cache.device))


def ftm_prefill_mha(q, k_new, v_new, qkv_bias, k_cache, v_cache, seq_lens, out, stream=None,
                    kv_scales=None) -> None:
    """Prefill (see include/ftm.h): q/out [B, S, H, D], k_new/v_new
    [B, S, Hkv, D], caches [B, Hkv, Lmax, D], seq_lens int32 [B] or None;
    an int8 cache takes fp16 activations and kv_scales fp32 [2, B, Hkv, Lmax]."""
    _check(lib.ftm_prefill_mha(*_marshal_prefill(q, k_new, v_new, qkv_bias, k_cache, v_cache, seq_lens,
                                                 out, stream, kv_scales)))


def ftm_prefill_mha_prepared(q, k_new, v_new, qkv_bias, k_cache, v_cache, seq_lens, out,
                             stream=None, kv_scales=None) -> Callable[[], None]:
    """ftm_prefill_mha with the arguments marshalled once."""
    args = _marshal_prefill(q, k_new, v_new, qkv_bias, k_cache, v_cache, seq_lens, out, stream, kv_scales)
    return _prepared(lib.ftm_prefill_mha, args,
                     (q, k_new, v_new, qkv_bias, k_cache, v_cache, seq_lens, out, kv_scales))


def _marshal_prefill_paged(q, k_new, v_new, qkv_bias, k_pages, v_pages, block_table, seq_lens, out, stream,
                           kv_scales=None):
    if q.dim() != 4 or k_pages.dim() != 4 or block_table.dim() != 2:
        raise ValueError("q must be [B, S, H, D], the pools [n_pages, Hkv, P, D] and block_table "
                         "[B, max_pages_per_seq]")
    B, S, H, D = q.shape
    n_pages, Hkv, P, _ = k_pages.shape
    max_pages = block_table.shape[1]
    kv, act = _prefill_types(k_pages)
    tensors = {"q": (q, act, (B, S, H, D)), "k_new": (k_new, act, (B, S, Hkv, D)),
               "v_new": (v_new, act, (B, S, Hkv, D)), "k_pages": (k_pages, k_pages.dtype, (n_pages, Hkv, P, D)),
               "v_pages": (v_pages, k_pages.dtype, (n_pages, Hkv, P, D)),
               "block_table": (block_table, torch.int32, (B, max_pages)), "out": (out, act, (B, S, H, D))}
    if qkv_bias is not None:
        tensors["qkv_bias"] = (qkv_bias, act, ((H + 2 * Hkv) * D,))
    if seq_lens is not None:
        tensors["seq_lens"] = (seq_lens, torch.int32, (B,))
    if kv_scales is not None:
        tensors["kv_scales"] = (kv_scales, torch.float32, (2, n_pages, Hkv, P))
    _check_tensors(tensors, k_pages.device)
    return (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(qkv_bias), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
            n_pages, P, max_pages, _ptr(seq_lens), B, S, H, Hkv, D, kv, _ptr(kv_scales), _ptr(out),
            _stream_ptr(stream, k_pages.device))


def ftm_prefill_mha_paged(q, k_new, v_new, qkv_bias, k_pages, v_pages, block_table, seq_lens, out,
                          stream=None, kv_scales=None) -> None:
    """Prefill into a paged cache (see include/ftm.h): pools [n_pages, Hkv, P, D],
    block_table int32 [B, max_pages_per_seq], kv_scales fp32 [2, n_pages, Hkv, P]
    for an int8 pool, the rest as ftm_prefill_mha."""
    _check(lib.ftm_prefill_mha_paged(*_marshal_prefill_paged(q, k_new, v_new, qkv_bias, k_pages, v_pages,
                                                             block_table, seq_lens, out, stream, kv_scales)))


def ftm_prefill_mha_paged_prepared(q, k_new, v_new, qkv_bias, k_pages, v_pages, block_table, seq_lens, out,
                                   stream=None, kv_scales=None) -> Callable[[], None]:
    """ftm_prefill_mha_paged with the arguments marshalled once."""
    args = _marshal_prefill_paged(q, k_new, v_new, qkv_bias, k_pages, v_pages, block_table, seq_lens, out, stream,
                                  kv_scales)
    return _prepared(lib.ftm_prefill_mha_paged, args,
                     (q, k_new, v_new, qkv_bias, k_pages, v_pages, block_table, seq_lens, out, kv_scales))


def ftm_graph_begin(stream: int) -> None:
    """Starts capturing `stream` (a created stream's handle, not 0)."""
    _check(lib.ftm_graph_begin(ctypes.c_void_p(stream)))


def ftm_graph_end(stream: int) -> int:
    """Ends the capture and returns the instantiated graph's handle."""
    g = ctypes.c_void_p(None)
    _check(lib.ftm_graph_end(ctypes.c_void_p(stream), ctypes.byref(g)))
    return g.value


def ftm_graph_launch(graph: int, stream: int) -> None:
    _check(lib.ftm_graph_launch(ctypes.c_void_p(graph), ctypes.c_void_p(stream)))


def ftm_graph_destroy(graph: Optional[int]) -> None:
    _check(lib.ftm_graph_destroy(ctypes.c_void_p(graph)))


# The boundary's calls without the C prefix (ftm.decode_mha, ...): the same
# functions under the names the Python side of the boundary uses.
decode_mha = ftm_decode_mha
decode_mha_prepared = ftm_decode_mha_prepared
decode_mha_static = ftm_decode_mha_static
decode_mha_paged = ftm_decode_mha_paged
decode_mha_paged_prepared = ftm_decode_mha_paged_prepared
qkv_proj = ftm_qkv_proj
prefill_mha = ftm_prefill_mha
prefill_mha_paged = ftm_prefill_mha_paged
last_error = ftm_last_error
version = ftm_version
kv_cache_bytes = ftm_kv_cache_bytes
release_workspaces = ftm_release_workspaces
tuning_reload = ftm_tuning_reload

"""CPU oracle for one decode step of masked multi-head attention over a KV cache.

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The GPU library never imports, links
or runs anything here, and nothing here imports the GPU library.

The arithmetic lives in ``ftm_oracle.c`` (plain C, fp64 attention, fp32
append); this module only builds it with gcc and marshals numpy arrays.

Element types are passed as numpy arrays holding the raw values: float32,
float16, bfloat16 as its uint16 bit pattern, int8.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ftm_oracle.c")
_LIB = os.path.join(_HERE, "libftm_oracle.so")

DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "i8": 3}
_NP = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "i8": np.int8}

_lib = None


def build() -> str:
    """Compile the oracle with IEEE semantics (no fast-math, no contraction)."""
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11",
           "-Wall", "-Wextra", "-shared", "-fPIC", "-pthread",
           _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.orc_decode_mha.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                   i32, i32, i32, i32, vp, vp, vp, i32]
    lib.orc_decode_mha.restype = i32
    lib.orc_f16_bits_to_double.argtypes = [ctypes.c_uint16]
    lib.orc_f16_bits_to_double.restype = ctypes.c_double
    lib.orc_bf16_bits_to_double.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_bits_to_double.restype = ctypes.c_double
    lib.orc_float_to_f16_rne.argtypes = [ctypes.c_float]
    lib.orc_float_to_f16_rne.restype = ctypes.c_uint16
    lib.orc_float_to_bf16_rne.argtypes = [ctypes.c_float]
    lib.orc_float_to_bf16_rne.restype = ctypes.c_uint16
    lib.orc_quantize_row_i8.argtypes = [vp, i32, vp]
    lib.orc_quantize_row_i8.restype = ctypes.c_float
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _need(a, dtype, shape, name, writable=False):
    if a.dtype != np.dtype(dtype):
        raise TypeError(f"{name}: dtype {a.dtype}, expected {np.dtype(dtype)}")
    if tuple(a.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {a.shape}, expected {tuple(shape)}")
    if not a.flags.c_contiguous or (writable and not a.flags.writeable):
        raise ValueError(f"{name}: must be C-contiguous" + (" and writable" if writable else ""))


def act_dtype_of(kv_dtype: str) -> str:
    """Activation type: the cache type for float caches, fp16 for INT8."""
    return "f16" if kv_dtype == "i8" else kv_dtype


def decode_mha(q, k_new, v_new, qkv_bias, k_cache, v_cache, seq_lens, step,
               n_heads, n_kv_heads, head_dim, kv_dtype, kv_scales=None,
               n_threads=1, want_probs=False) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """One decode step; appends into k_cache/v_cache/kv_scales in place.

    Returns (out[B,H,D] float64, probs[B,H,step] float64 or None)."""
    lib = _load()
    B, Hkv, Lmax, D = k_cache.shape
    H = n_heads
    if D != head_dim or Hkv != n_kv_heads:
        raise ValueError("cache shape does not match head_dim / n_kv_heads")
    act = _NP[act_dtype_of(kv_dtype)]
    _need(q, act, (B, H, D), "q")
    _need(k_new, act, (B, Hkv, D), "k_new")
    _need(v_new, act, (B, Hkv, D), "v_new")
    if qkv_bias is not None:
        _need(qkv_bias, act, ((H + 2 * Hkv) * D,), "qkv_bias")
    _need(k_cache, _NP[kv_dtype], (B, Hkv, Lmax, D), "k_cache", True)
    _need(v_cache, _NP[kv_dtype], (B, Hkv, Lmax, D), "v_cache", True)
    if seq_lens is not None:
        _need(seq_lens, np.int32, (B,), "seq_lens")
    if kv_scales is not None:
        _need(kv_scales, np.float32, (2, B, Hkv, Lmax), "kv_scales", True)
    out = np.empty((B, H, D), dtype=np.float64)
    probs = np.empty((B, H, step), dtype=np.float64) if want_probs else None
    rc = lib.orc_decode_mha(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(qkv_bias),
                            _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                            B, Lmax, int(step), H, Hkv, D, DTYPES[kv_dtype],
                            _ptr(kv_scales), _ptr(out), _ptr(probs), int(n_threads))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out, probs


def decode_mha_paged(q, k_new, v_new, qkv_bias, k_pages, v_pages, block_table, seq_lens, step,
                     n_heads, n_kv_heads, head_dim, kv_dtype, kv_scales=None,
                     n_threads=1) -> np.ndarray:
    """One decode step over a paged cache; appends into k_pages/v_pages/kv_scales
    in place and returns out[B,H,D] float64.

    Paging is address translation only ([intelliparadigm.com
    .../2131745] section 5.1: the cache cut into fixed-size pages;
    [framerc.cn/news/4453289] section 3.2: blocks taken on demand, located
    through a table as in virtual memory): position i of sequence b is row
    i mod P of page block_table[b, i // P].  The step is therefore the
    contiguous step above on the cache that the table describes: this
    function gathers that cache, runs ``decode_mha`` on it and writes the
    one appended row per (b, KV head) back to its page.

    Contract for a table entry outside [0, n_pages) among the pages of
    positions [0, L_b): the sequence's output rows are NaN, and its new row
    is appended only if the new row's own page is valid.

    Layouts: k_pages/v_pages [n_pages, Hkv, P, D], block_table int32
    [B, max_pages], kv_scales float32 [2, n_pages, Hkv, P] (INT8 only)."""
    n_pages, Hkv, P, D = k_pages.shape
    B, max_pages = block_table.shape
    if Hkv != n_kv_heads or D != head_dim or v_pages.shape != k_pages.shape:
        raise ValueError("page pool shape does not match n_kv_heads / head_dim")
    cap = max_pages * P
    lens = (np.full(B, step, dtype=np.int64) if seq_lens is None
            else np.asarray(seq_lens, dtype=np.int64))
    tbl = np.asarray(block_table, dtype=np.int64)
    ok_entry = (tbl >= 0) & (tbl < n_pages)
    page_of = np.where(ok_entry, tbl, 0)

    def gather(pool):
        # [B, max_pages, Hkv, P, ...] -> [B, Hkv, max_pages * P, ...]
        g = pool[page_of]
        g = np.swapaxes(g, 1, 2)
        return np.ascontiguousarray(g.reshape((B, Hkv, cap) + pool.shape[3:]))

    kc, vc = gather(k_pages), gather(v_pages)
    sc = None
    if kv_scales is not None:
        sc = np.ascontiguousarray(np.stack([gather(kv_scales[0]), gather(kv_scales[1])]))
    out, _ = decode_mha(q, k_new, v_new, qkv_bias, kc, vc,
                        None if seq_lens is None else np.ascontiguousarray(seq_lens, dtype=np.int32),
                        step, n_heads, n_kv_heads, head_dim, kv_dtype, sc, n_threads=n_threads)
    for b in range(B):
        L = int(lens[b])
        if L < 1 or L > step:
            continue                        # the contiguous step already wrote NaN, no append
        pages_used = (L - 1) // P + 1
        if not ok_entry[b, :pages_used].all():
            out[b] = np.nan
        last = (L - 1) // P
        if not ok_entry[b, last]:
            continue
        pg, row = int(tbl[b, last]), (L - 1) % P
        k_pages[pg, :, row] = kc[b, :, L - 1]
        v_pages[pg, :, row] = vc[b, :, L - 1]
        if kv_scales is not None:
            kv_scales[0, pg, :, row] = sc[0, b, :, L - 1]
            kv_scales[1, pg, :, row] = sc[1, b, :, L - 1]
    return out


def qkv_proj(x, w, bias, n_heads, n_kv_heads, head_dim, act_dtype):
    """The fused QKV projection of one decode step, in float64.

    One projection produces Q, K and V together, and its output is split
    three ways ([lpnh.cn/news/2765398] section 2.1): y = x W^T (+ bias)
    with x [B, hidden] and W [(H + 2 Hkv) D, hidden] (one row of weights
    per output feature), then features [0, H D) are Q as [B, H, D], the next
    Hkv D are K and the last Hkv D are V, each [B, Hkv, D].

    x, w, bias hold act_dtype values (bfloat16 as uint16 bit patterns).
    Returns (q, k, v) float64 arrays, unrounded."""
    xf = cache_to_f64(np.asarray(x), act_dtype)
    wf = cache_to_f64(np.asarray(w), act_dtype)
    B = xf.shape[0]
    H, Hkv, D = n_heads, n_kv_heads, head_dim
    N = (H + 2 * Hkv) * D
    if wf.shape != (N, xf.shape[1]):
        raise ValueError(f"w must be [{N}, {xf.shape[1]}]")
    y = xf @ wf.T
    if bias is not None:
        y = y + cache_to_f64(np.asarray(bias), act_dtype)[None, :]
    q = y[:, :H * D].reshape(B, H, D)
    k = y[:, H * D:(H + Hkv) * D].reshape(B, Hkv, D)
    v = y[:, (H + Hkv) * D:].reshape(B, Hkv, D)
    return q, k, v


def prefill_mha(q, k_new, v_new, qkv_bias, k_cache, v_cache, seq_lens, n_heads, n_kv_heads,
                head_dim, kv_dtype, kv_scales=None):
    """Prefill: the whole prompt of every sequence in one step.  Writes the
    prompt's K/V rows into the cache in place and returns out[B, S, H, D]
    float64 (rows past a sequence's prompt are 0).

    The prompt is processed in parallel where decode goes token by token
    ([lpnh.cn/news/2765398] section 1.1): for sequence b with prompt length
    S_b, position t of every query head attends to positions [0, t] of its
    KV head, causally.  Each position is what a decode step at length t + 1
    computes, with the same readings: the bias added in fp32 before the K/V
    rows are stored (rounded to the cache type, or quantised to INT8 codes
    with one fp32 scale per row by the decode step's rule), the stored rows
    used in the attention (code x scale for INT8), the query with its bias
    unrounded, scale 1/sqrt(D), the maximum subtracted before exp.

    Layouts: q [B, S, H, D]; k_new, v_new [B, S, Hkv, D]; qkv_bias
    [(H + 2 Hkv) D] or None; caches [B, Hkv, Lmax, D] with Lmax >= S;
    seq_lens [B] int32 (1 <= S_b <= S) or None for every S_b = S.  fp16,
    bf16 (as uint16 bit patterns) and INT8 caches; with INT8 the
    activations are fp16 and kv_scales float32 [2, B, Hkv, Lmax] (K first)
    is written in place."""
    import torch
    if kv_dtype not in ("f16", "bf16", "i8"):
        raise ValueError("prefill takes fp16, bf16 or INT8 caches")
    i8 = kv_dtype == "i8"
    if i8 and kv_scales is None:
        raise ValueError("an INT8 cache needs kv_scales")
    act = act_dtype_of(kv_dtype)
    B, S, H, D = q.shape
    Hkv = n_kv_heads
    G = H // Hkv
    if H != n_heads or D != head_dim or k_new.shape != (B, S, Hkv, D):
        raise ValueError("shapes do not match n_heads / n_kv_heads / head_dim")
    lens = np.full(B, S) if seq_lens is None else np.asarray(seq_lens, dtype=np.int64)
    tdt = torch.float16 if act == "f16" else torch.bfloat16

    def f32(a):
        return torch.from_numpy(cache_to_f64(np.asarray(a), act).astype(np.float32))

    bias = None if qkv_bias is None else f32(qkv_bias)
    out = np.zeros((B, S, H, D), dtype=np.float64)
    inv = 1.0 / np.sqrt(D)
    for b in range(B):
        Sb = int(lens[b])
        if Sb < 1 or Sb > S:
            out[b] = np.nan
            continue
        for which, src, cache in ((0, k_new, k_cache), (1, v_new, v_cache)):
            x = f32(src[b, :Sb])                              # [Sb, Hkv, D]
            if bias is not None:
                x = x + bias[(H + which * Hkv) * D:(H + (which + 1) * Hkv) * D].reshape(Hkv, D)
            if i8:
                xs = x.numpy()
                for t in range(Sb):
                    for j in range(Hkv):
                        codes, sc = quantize_row_i8(xs[t, j])
                        cache[b, j, t] = codes
                        kv_scales[which, b, j, t] = sc
                continue
            stored = x.to(tdt)                                # round to nearest even
            if kv_dtype == "bf16":
                cache[b, :, :Sb] = stored.view(torch.int16).numpy().view(np.uint16).transpose(1, 0, 2)
            else:
                cache[b, :, :Sb] = stored.numpy().transpose(1, 0, 2)
        if i8:
            K = cache_to_f64(k_cache[b, :, :Sb], "i8", kv_scales[0, b, :, :Sb])
            V = cache_to_f64(v_cache[b, :, :Sb], "i8", kv_scales[1, b, :, :Sb])
        else:
            K = cache_to_f64(k_cache[b, :, :Sb], kv_dtype)   # [Hkv, Sb, D]
            V = cache_to_f64(v_cache[b, :, :Sb], kv_dtype)
        causal = np.tril(np.ones((Sb, Sb), dtype=bool))
        for h in range(H):
            j = h // G
            qh = cache_to_f64(np.asarray(q[b, :Sb, h]), act)
            if bias is not None:
                qh = qh + bias[h * D:(h + 1) * D].double().numpy()[None, :]
            s = (qh @ K[j].T) * inv                            # [Sb, Sb]
            s = np.where(causal, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            w = np.exp(s)
            p = w / w.sum(axis=1, keepdims=True)
            out[b, :Sb, h] = p @ V[j]
    return out


def prefill_mha_paged(q, k_new, v_new, qkv_bias, k_pages, v_pages, block_table, seq_lens, n_heads,
                      n_kv_heads, head_dim, kv_dtype, kv_scales=None):
    """Prefill into a paged cache: writes the prompt's K/V rows into their
    pages in place and returns out[B, S, H, D] float64.

    Position i of sequence b is row i mod P of page block_table[b, i // P]
    (paging is address translation only: [intelliparadigm.com .../2131745]
    section 5.1, [framerc.cn/news/4453289] section 3.2).  A prefill reads
    only the rows it writes itself, so it is the contiguous prefill above run
    on a fresh contiguous cache, whose rows [0, S_b) are then written to the
    pages the table names.

    Contract for a table entry outside [0, n_pages) among the pages of
    positions [0, S_b): the sequence's output rows [0, S_b) are NaN, and
    only the rows whose page is valid are appended.

    Layouts: k_pages/v_pages [n_pages, Hkv, P, D]; block_table int32
    [B, max_pages] with max_pages P >= S; INT8: kv_scales float32
    [2, n_pages, Hkv, P] (K first), written with the codes."""
    n_pages, Hkv, P, D = k_pages.shape
    B, S = q.shape[0], q.shape[1]
    _, max_pages = block_table.shape
    if Hkv != n_kv_heads or D != head_dim or v_pages.shape != k_pages.shape:
        raise ValueError("page pool shape does not match n_kv_heads / head_dim")
    if max_pages * P < S:
        raise ValueError("the table has too few pages for the prompt")
    lens = np.full(B, S) if seq_lens is None else np.asarray(seq_lens, dtype=np.int64)
    kc = np.zeros((B, Hkv, S, D), dtype=k_pages.dtype)
    vc = np.zeros_like(kc)
    sc = None if kv_scales is None else np.zeros((2, B, Hkv, S), dtype=np.float32)
    out = prefill_mha(q, k_new, v_new, qkv_bias, kc, vc, seq_lens, n_heads, n_kv_heads, head_dim, kv_dtype, sc)
    tbl = np.asarray(block_table, dtype=np.int64)
    for b in range(B):
        Sb = int(lens[b])
        if Sb < 1 or Sb > S:
            continue                        # NaN rows already, no append
        entries = tbl[b, :(Sb + P - 1) // P]
        ok = (entries >= 0) & (entries < n_pages)
        if not ok.all():
            out[b, :Sb] = np.nan
        for t in range(Sb):
            if ok[t // P]:
                pg = int(entries[t // P])
                k_pages[pg, :, t % P] = kc[b, :, t]
                v_pages[pg, :, t % P] = vc[b, :, t]
                if sc is not None:
                    kv_scales[:, pg, :, t % P] = sc[:, b, :, t]
    return out


def round_to_act(y, act_dtype):
    """float64 values rounded to nearest even in the activation type, as the
    array type the oracle takes (bfloat16 as uint16 bit patterns)."""
    y = np.asarray(y, dtype=np.float64)
    if act_dtype == "f32":
        return y.astype(np.float32)
    if act_dtype == "f16":
        with np.errstate(over="ignore"):
            return y.astype(np.float16)       # numpy rounds float64 to binary16 to nearest even
    # via fp32 (exact double rounding: 24 >= 2 * 8 + 2), then the oracle's RNE
    f = _load().orc_float_to_bf16_rne
    flat = y.astype(np.float32).ravel()
    return np.array([f(float(v)) for v in flat], dtype=np.uint16).reshape(y.shape)


def f16_bits_to_double(bits: int) -> float:
    return _load().orc_f16_bits_to_double(bits)


def bf16_bits_to_double(bits: int) -> float:
    return _load().orc_bf16_bits_to_double(bits)


def float_to_f16_rne(x: float) -> int:
    return _load().orc_float_to_f16_rne(x)


def float_to_bf16_rne(x: float) -> int:
    return _load().orc_float_to_bf16_rne(x)


def quantize_row_i8(x: np.ndarray) -> Tuple[np.ndarray, float]:
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.empty(x.shape[0], dtype=np.int8)
    s = _load().orc_quantize_row_i8(_ptr(x), x.shape[0], _ptr(codes))
    return codes, float(np.float32(s))


def cache_to_f64(cache: np.ndarray, kv_dtype: str, scales: Optional[np.ndarray] = None) -> np.ndarray:
    """Stored cache values widened exactly to float64 (INT8: code * scale).
    ``scales`` is broadcast over the last axis."""
    if kv_dtype == "f32":
        return cache.astype(np.float64)
    if kv_dtype == "f16":
        return cache.astype(np.float64)
    if kv_dtype == "bf16":
        return (cache.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return cache.astype(np.float64) * scales.astype(np.float64)[..., None]

"""Seeded synthetic inputs for decode-step attention, shared by the tests, the
smoke check and the benchmark.

This module draws numbers and lays them out; it holds none of the
attention's arithmetic (no bias add, no rounding rule of the cache, no
quantiser, no softmax).  Both the GPU path and the CPU oracle receive the
very same bytes from here.

Workloads (shapes, types, value distributions) follow the pages' decode
setting: a pre-allocated [B, H_kv, L_max, D] cache per layer
([intelliparadigm.com .../2131745] section 2.1), fp16 caches of a
7B/13B-class model with hidden 4096 ([pptc.cn/news/144085] section 3.1, the
32-sequence / 2048-token / 32-layer sizing example), grouped KV heads
([pptc.cn/news/144085] section 3.4) and an INT8 cache ([pptc.cn/news/144085]
section 3.1).

Generation: one ``torch.Generator`` per (seed, tensor tag, layer), on the
device the tensor is made on.  Small cases are generated on the host and
copied; full-size cases are generated on the GPU and the oracle receives
copies of those bytes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import torch

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "i8": torch.int8}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1}

_TAGS = {"q": 1, "k_new": 2, "v_new": 3, "bias": 4, "k_cache": 5, "v_cache": 6,
         "k_scale": 7, "v_scale": 8, "lens": 9, "pages": 10}


def act_dtype(kv_dtype: str) -> str:
    """Activation type (q, k_new, v_new, bias, out): the cache type for float
    caches and fp16 next to an INT8 cache."""
    return "f16" if kv_dtype == "i8" else kv_dtype


@dataclass(frozen=True)
class Case:
    """One decode-step problem.

    ``lens``: None for every sequence at ``ctx`` tokens (after the append),
    or (lo, hi) for lengths drawn uniformly from [lo, hi] per sequence.
    ``value_scale``: standard deviation of every drawn real value.
    ``int8_code_gain``: prefilled INT8 rows hold codes round(gain * N(0,1))
    clamped to +-127, with a per-row scale of (1 +- 5%) / gain, so that the
    dequantised values are again about N(0,1) * value_scale-free.
    ``page_size``: 0 for the contiguous [B, Hkv, Lmax, D] cache, else the
    tokens per page of a paged cache (``make_paged_inputs``)."""
    name: str
    batch: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    kv_dtype: str
    ctx: int
    max_seq_len: int
    value_scale: float
    lens: Optional[tuple] = None
    layers: int = 1
    rotate: int = 1
    seed: int = 1000
    int8_code_gain: float = 127.0 / 3.0
    page_size: int = 0

    @property
    def act_dtype(self) -> str:
        return act_dtype(self.kv_dtype)

    @property
    def group(self) -> int:
        return self.n_heads // self.n_kv_heads

    def with_(self, **kw) -> "Case":
        return replace(self, **kw)


# The five workloads.  Value scales: N(0,1)/sqrt(D) where stated; the INT8
# workload states N(0,1) data (absmax/127 scales) and no 1/sqrt(D) factor.
CASES: Dict[str, Case] = {
    "tiny": Case("tiny", 1, 8, 8, 64, "f32", ctx=128, max_seq_len=128,
                 value_scale=1 / 8.0, seed=1000),
    "7b": Case("7b", 8, 32, 32, 128, "f16", ctx=2048, max_seq_len=2048,
               value_scale=1 / math.sqrt(128), rotate=32, seed=1001),
    "sizing32": Case("sizing32", 32, 32, 32, 128, "f16", ctx=2048, max_seq_len=2048,
                     value_scale=1 / math.sqrt(128), layers=32, seed=1002),
    "gqa": Case("gqa", 16, 64, 8, 128, "bf16", ctx=8192, max_seq_len=8192,
                value_scale=1 / math.sqrt(128), lens=(512, 8192), rotate=8, seed=1003),
    "int8": Case("int8", 64, 40, 40, 128, "i8", ctx=4096, max_seq_len=4096,
                 value_scale=1.0, rotate=2, seed=1004),
}
# The same layer shapes over a paged cache of 256-token pages (the page size
# [intelliparadigm.com .../2131745] section 5.1 gives as its example), pages
# handed out in a seeded random order.
CASES["7b_paged"] = CASES["7b"].with_(name="7b_paged", page_size=256)
CASES["gqa_paged"] = CASES["gqa"].with_(name="gqa_paged", page_size=256)


def _gen(case: Case, tag: str, layer: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((case.seed * 1_000_003 + _TAGS[tag] * 10_007 + layer * 101) % (2 ** 62))
    return g


def seq_lens(case: Case) -> torch.Tensor:
    """Per-sequence lengths after the append (host int32 tensor)."""
    if case.lens is None:
        return torch.full((case.batch,), case.ctx, dtype=torch.int32)
    lo, hi = case.lens
    g = _gen(case, "lens", 0, "cpu")
    return torch.randint(lo, hi + 1, (case.batch,), generator=g, dtype=torch.int32)


def _normal(case: Case, tag: str, layer: int, shape, dtype: str, device) -> torch.Tensor:
    g = _gen(case, tag, layer, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x.mul_(case.value_scale)
    return x.to(TORCH_DTYPES[dtype])


def _fill_cache_float(t: torch.Tensor, case: Case, tag: str, layer: int) -> None:
    """Fill a [B, Hkv, Lmax, D] float cache one (b) slab at a time so the
    fp32 temporary stays small."""
    g = _gen(case, tag, layer, t.device)
    tmp = torch.empty(t.shape[1:], device=t.device, dtype=torch.float32)
    for b in range(t.shape[0]):
        tmp.normal_(generator=g).mul_(case.value_scale)
        t[b].copy_(tmp)


def _fill_cache_int8(codes: torch.Tensor, scales: torch.Tensor, case: Case, tag: str,
                     stag: str, layer: int) -> None:
    g = _gen(case, tag, layer, codes.device)
    tmp = torch.empty(codes.shape[1:], device=codes.device, dtype=torch.float32)
    for b in range(codes.shape[0]):
        tmp.normal_(generator=g).mul_(case.int8_code_gain).round_().clamp_(-127, 127)
        codes[b].copy_(tmp)
    gs = _gen(case, stag, layer, codes.device)
    u = torch.rand(scales.shape, generator=gs, device=codes.device, dtype=torch.float32)
    scales.copy_((0.95 + 0.1 * u) / case.int8_code_gain)


def make_inputs(case: Case, device="cpu", layer: int = 0, poison: bool = True,
                lens: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """All inputs of one layer's decode step.

    Cache rows [0, L_b - 1) hold prefilled history; row L_b - 1 is the slot
    the step appends into.  With ``poison`` every row >= L_b - 1 is NaN (float
    caches) or has a NaN scale (INT8), so a read of anything but the history
    shows up in the output."""
    B, H, Hkv, D, Lmax = case.batch, case.n_heads, case.n_kv_heads, case.head_dim, case.max_seq_len
    act = case.act_dtype
    L = (seq_lens(case) if lens is None else lens.to(torch.int32).cpu())
    t: Dict[str, torch.Tensor] = {}
    t["q"] = _normal(case, "q", layer, (B, H, D), act, device)
    t["k_new"] = _normal(case, "k_new", layer, (B, Hkv, D), act, device)
    t["v_new"] = _normal(case, "v_new", layer, (B, Hkv, D), act, device)
    t["bias"] = _normal(case, "bias", layer, ((H + 2 * Hkv) * D,), act, device)
    shape = (B, Hkv, Lmax, D)
    kvt = TORCH_DTYPES[case.kv_dtype]
    k = torch.empty(shape, dtype=kvt, device=device)
    v = torch.empty(shape, dtype=kvt, device=device)
    if case.kv_dtype == "i8":
        sc = torch.empty((2, B, Hkv, Lmax), dtype=torch.float32, device=device)
        _fill_cache_int8(k, sc[0], case, "k_cache", "k_scale", layer)
        _fill_cache_int8(v, sc[1], case, "v_cache", "v_scale", layer)
        t["kv_scales"] = sc
    else:
        _fill_cache_float(k, case, "k_cache", layer)
        _fill_cache_float(v, case, "v_cache", layer)
    if poison:
        for b in range(B):
            p = int(L[b]) - 1
            if case.kv_dtype == "i8":
                t["kv_scales"][:, b, :, max(p, 0):] = float("nan")
            else:
                k[b, :, max(p, 0):, :] = float("nan")
                v[b, :, max(p, 0):, :] = float("nan")
    t["k_cache"] = k
    t["v_cache"] = v
    t["seq_lens"] = L.to(device)
    t["step"] = int(L.max())
    return t


def to_paged(t: Dict[str, torch.Tensor], case: Case, page_size: int, layer: int = 0,
             poison: bool = True) -> Dict[str, torch.Tensor]:
    """Moves the contiguous cache of ``make_inputs`` into a page pool.

    Sequence b takes ceil(L_b / P) pages, enough for positions [0, L_b); the
    pool holds those plus max(1, B / 4) spare pages, all handed out in a
    seeded random order.  Adds ``k_pages``/``v_pages`` [n_pages, Hkv, P, D],
    ``block_table`` int32 [B, ceil(Lmax / P)] (-1 past a sequence's pages)
    and, for INT8, ``kv_scales`` [2, n_pages, Hkv, P]; removes the
    contiguous cache.  Rows the pool holds that no position maps to are NaN
    (NaN scales for INT8) with ``poison``, else zero."""
    P = page_size
    k, v = t.pop("k_cache"), t.pop("v_cache")
    B, Hkv, Lmax, D = k.shape
    dev = k.device
    L = t["seq_lens"].cpu().tolist()
    max_pages = (Lmax + P - 1) // P
    need = [min(max(0, (int(x) + P - 1) // P), max_pages) for x in L]
    n_pages = sum(need) + max(1, B // 4)
    perm = torch.randperm(n_pages, generator=_gen(case, "pages", layer, "cpu")).tolist()
    table = torch.full((B, max_pages), -1, dtype=torch.int32)
    fill = float("nan") if poison else 0.0
    i8 = case.kv_dtype == "i8"
    kp = torch.empty((n_pages, Hkv, P, D), dtype=k.dtype, device=dev)
    vp = torch.empty_like(kp)
    if i8:
        kp.zero_()
        vp.zero_()
        sc = t.pop("kv_scales")
        sp = torch.full((2, n_pages, Hkv, P), fill, dtype=torch.float32, device=dev)
    else:
        kp.fill_(fill)
        vp.fill_(fill)
    n = 0
    for b in range(B):
        for i in range(need[b]):
            pg = perm[n]
            n += 1
            table[b, i] = pg
            lo, hi = i * P, min((i + 1) * P, Lmax)
            kp[pg, :, :hi - lo] = k[b, :, lo:hi]
            vp[pg, :, :hi - lo] = v[b, :, lo:hi]
            if i8:
                sp[:, pg, :, :hi - lo] = sc[:, b, :, lo:hi]
    t["k_pages"], t["v_pages"] = kp, vp
    t["block_table"] = table.to(dev)
    if i8:
        t["kv_scales"] = sp
    return t


def make_paged_inputs(case: Case, device="cpu", layer: int = 0, poison: bool = True,
                      lens: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """``make_inputs`` with the cache in a page pool of ``case.page_size``."""
    return to_paged(make_inputs(case, device, layer, poison, lens), case, case.page_size, layer, poison)


def kv_bytes(case: Case, lens: Optional[List[int]] = None) -> int:
    """Bytes of K and V (and INT8 scales) that one step must read: every
    position [0, L_b) of every (sequence, KV head), K and V."""
    L = seq_lens(case).tolist() if lens is None else list(lens)
    row = case.head_dim * ELEM_BYTES[case.kv_dtype] + (4 if case.kv_dtype == "i8" else 0)
    return sum(L) * case.n_kv_heads * 2 * row


@dataclass(frozen=True)
class ProjCase:
    """A fused QKV projection: x [batch, hidden] times W [(H + 2 Hkv) D, hidden].
    x ~ N(0, 1) and W ~ N(0, 1/hidden), so each output is about N(0, 1);
    the bias ~ N(0, 1/8)."""
    name: str
    batch: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    hidden: int
    dtype: str
    rotate: int = 1
    seed: int = 2000

    @property
    def n_out(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim

    def with_(self, **kw) -> "ProjCase":
        return replace(self, **kw)


# The projections that feed the attention workloads' layers (hidden = H D):
# the 7B-shaped layer, the 13B-shaped layer of the INT8 workload, and the
# grouped-query layer.  Weight sets rotate so the 256 MB last-level cache
# cannot serve repeated reads.
PROJ_CASES: Dict[str, ProjCase] = {
    "qkv_7b": ProjCase("qkv_7b", 8, 32, 32, 128, 4096, "f16", rotate=8, seed=2001),
    "qkv_13b": ProjCase("qkv_13b", 64, 40, 40, 128, 5120, "f16", rotate=4, seed=2004),
    "qkv_gqa": ProjCase("qkv_gqa", 16, 64, 8, 128, 8192, "bf16", rotate=4, seed=2003),
}


def make_proj_inputs(case: ProjCase, device="cpu", layer: int = 0) -> Dict[str, torch.Tensor]:
    """x, w, bias of one projection (``case.seed`` and ``layer`` pick the draw)."""
    dt = TORCH_DTYPES[case.dtype]

    def draw(tag, shape, scale):
        g = torch.Generator(device=device)
        g.manual_seed((case.seed * 1_000_003 + tag * 10_007 + layer * 101) % (2 ** 62))
        return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * scale).to(dt)

    return {"x": draw(1, (case.batch, case.hidden), 1.0),
            "w": draw(2, (case.n_out, case.hidden), 1.0 / math.sqrt(case.hidden)),
            "bias": draw(3, (case.n_out,), 1.0 / math.sqrt(8.0))}


def proj_bytes(case: ProjCase) -> int:
    """Bytes one projection must move: the weights, x and the outputs."""
    e = ELEM_BYTES[case.dtype]
    return (case.n_out * case.hidden + case.batch * case.hidden + case.batch * case.n_out) * e


@dataclass(frozen=True)
class PrefillCase:
    """Prefill of a batch of prompts: q [B, S, H, D], k_new/v_new [B, S, Hkv, D],
    all values N(0, 1) / sqrt(D) like the decode workloads; ``lens`` None for
    every prompt at S, or (lo, hi) drawn per sequence."""
    name: str
    batch: int
    prompt: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    max_seq_len: int
    lens: Optional[tuple] = None
    seed: int = 3000
    page_size: int = 0                      # 0: contiguous cache; else a paged one (pages of this many rows)

    def with_(self, **kw) -> "PrefillCase":
        return replace(self, **kw)


# Prefill of 2048-token prompts for the 7B-shaped layer and the grouped-query layer.
PREFILL_CASES: Dict[str, PrefillCase] = {
    "prefill_7b": PrefillCase("prefill_7b", 4, 2048, 32, 32, 128, "f16", 2048, seed=3001),
    "prefill_gqa": PrefillCase("prefill_gqa", 4, 2048, 64, 8, 128, "bf16", 2048, seed=3003),
    "prefill_7b_paged": PrefillCase("prefill_7b_paged", 4, 2048, 32, 32, 128, "f16", 2048, seed=3001,
                                    page_size=256),
    # the INT8 decode workload's layer (40 heads x 128, fp16 activations)
    "prefill_int8": PrefillCase("prefill_int8", 4, 2048, 40, 40, 128, "i8", 2048, seed=3005),
}


def make_prefill_inputs(case: PrefillCase, device="cpu", poison: bool = True) -> Dict[str, torch.Tensor]:
    """Inputs of one prefill step; caches are NaN (poison) or zero before it.

    INT8 caches follow the INT8 decode workload: fp16 activations drawn
    N(0, 1) without the 1/sqrt(D) factor, codes poisoned with 99 and
    ``kv_scales`` [2, B, Hkv, Lmax] with NaN (or all zero)."""
    dt = TORCH_DTYPES[case.dtype]
    i8 = case.dtype == "i8"
    act = torch.float16 if i8 else dt
    B, S, H, Hkv, D = case.batch, case.prompt, case.n_heads, case.n_kv_heads, case.head_dim
    scale = 1.0 if i8 else 1.0 / math.sqrt(D)

    def draw(tag, shape):
        g = torch.Generator(device=device)
        g.manual_seed((case.seed * 1_000_003 + tag * 10_007) % (2 ** 62))
        return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * scale).to(act)

    t = {"q": draw(1, (B, S, H, D)), "k_new": draw(2, (B, S, Hkv, D)), "v_new": draw(3, (B, S, Hkv, D)),
         "bias": draw(4, ((H + 2 * Hkv) * D,))}
    fill = float("nan") if poison else 0.0
    if i8:
        t["k_cache"] = torch.full((B, Hkv, case.max_seq_len, D), 99 if poison else 0, dtype=dt, device=device)
        t["kv_scales"] = torch.full((2, B, Hkv, case.max_seq_len), fill, dtype=torch.float32, device=device)
    else:
        t["k_cache"] = torch.full((B, Hkv, case.max_seq_len, D), fill, dtype=dt, device=device)
    t["v_cache"] = torch.full_like(t["k_cache"], t["k_cache"].flatten()[0].item())
    if case.lens is None:
        L = torch.full((B,), S, dtype=torch.int32)
    else:
        g = torch.Generator().manual_seed(case.seed + 77)
        L = torch.randint(case.lens[0], case.lens[1] + 1, (B,), generator=g, dtype=torch.int32)
    t["seq_lens"] = L.to(device)
    return t


def prefill_to_paged(t: Dict[str, torch.Tensor], case: PrefillCase, page_size: int) -> Dict[str, torch.Tensor]:
    """Replaces the contiguous caches of ``make_prefill_inputs`` by page pools.

    Sequence b takes ceil(S_b / P) pages; the pool holds those plus
    max(1, B / 4) spare pages, handed out in a seeded random order.  Adds
    ``k_pages``/``v_pages`` [n_pages, Hkv, P, D] filled like the caches
    they replace (NaN or zero) and ``block_table`` int32
    [B, ceil(max_seq_len / P)] (-1 past a sequence's pages)."""
    P = page_size
    k = t.pop("k_cache")
    t.pop("v_cache")
    B, Hkv, Lmax, D = k.shape
    L = t["seq_lens"].cpu().tolist()
    max_pages = (Lmax + P - 1) // P
    need = [min(max(0, (int(x) + P - 1) // P), max_pages) for x in L]
    n_pages = sum(need) + max(1, B // 4)
    g = torch.Generator().manual_seed((case.seed * 7919 + P) % (2 ** 62))
    perm = torch.randperm(n_pages, generator=g).tolist()
    table = torch.full((B, max_pages), -1, dtype=torch.int32)
    n = 0
    for b in range(B):
        for i in range(need[b]):
            table[b, i] = perm[n]
            n += 1
    fill = k.flatten()[0].item()
    t["k_pages"] = torch.full((n_pages, Hkv, P, D), fill, dtype=k.dtype, device=k.device)
    t["v_pages"] = torch.full_like(t["k_pages"], fill)
    t["block_table"] = table.to(k.device)
    if "kv_scales" in t:                    # INT8: the scale pool [2, n_pages, Hkv, P]
        sfill = t.pop("kv_scales").flatten()[0].item()
        t["kv_scales"] = torch.full((2, n_pages, Hkv, P), sfill, dtype=torch.float32, device=k.device)
    return t


def prefill_append_bytes(case: PrefillCase, lens: Optional[List[int]] = None) -> int:
    """Bytes the append moves: every prompt row of K and V read once (bias
    aside) and written once to the cache."""
    L = [case.prompt] * case.batch if lens is None else list(lens)
    if case.dtype == "i8":                  # fp16 rows in, codes and one fp32 scale per row out
        return sum(L) * case.n_kv_heads * (case.head_dim * 3 + 4) * 2
    return sum(L) * case.n_kv_heads * case.head_dim * ELEM_BYTES[case.dtype] * 2 * 2


def prefill_flops(case: PrefillCase, lens: Optional[List[int]] = None) -> int:
    """Multiply-adds x 2 of the causal attention: q.k and p.v over positions
    [0, t] for every prompt position t and query head."""
    L = [case.prompt] * case.batch if lens is None else list(lens)
    return sum(4 * (l * (l + 1) // 2) * case.n_heads * case.head_dim for l in L)

"""Small shared test utilities: tensor <-> numpy marshalling and error metrics.
No attention arithmetic lives here."""
from __future__ import annotations

import numpy as np
import torch


def to_np(t: torch.Tensor, dt: str) -> np.ndarray:
    """Torch tensor (any device) -> C-contiguous numpy array in the oracle's
    representation (bfloat16 as uint16 bit patterns)."""
    t = t.detach().contiguous().cpu()
    if dt == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def inputs_to_np(inp: dict, kv_dtype: str) -> dict:
    act = "f16" if kv_dtype == "i8" else kv_dtype
    r = {k: to_np(inp[k], act) for k in ("q", "k_new", "v_new", "bias")}
    r["k_cache"] = to_np(inp["k_cache"], kv_dtype)
    r["v_cache"] = to_np(inp["v_cache"], kv_dtype)
    r["seq_lens"] = to_np(inp["seq_lens"], "i32").astype(np.int32)
    r["kv_scales"] = to_np(inp["kv_scales"], "f32") if "kv_scales" in inp else None
    r["step"] = inp["step"]
    return r


def run_oracle(oracle, case, npi: dict, n_threads=1, want_probs=False):
    return oracle.decode_mha(npi["q"], npi["k_new"], npi["v_new"], npi["bias"],
                             npi["k_cache"], npi["v_cache"], npi["seq_lens"], npi["step"],
                             case.n_heads, case.n_kv_heads, case.head_dim, case.kv_dtype,
                             npi["kv_scales"], n_threads=n_threads, want_probs=want_probs)


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray):
    """(max abs error, max over rows of the row-normwise relative error,
    min cosine similarity over rows).  Rows are the last axis."""
    g = got.reshape(-1, got.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    d = np.abs(g - r)
    abs_err = float(d.max()) if d.size else 0.0
    scale = np.maximum(np.abs(r).max(axis=1), 1e-30)
    rel = float((d.max(axis=1) / scale).max()) if d.size else 0.0
    num = (g * r).sum(axis=1)
    den = np.linalg.norm(g, axis=1) * np.linalg.norm(r, axis=1)
    cos = float(np.min(np.where(den > 0, num / np.maximum(den, 1e-300), 1.0))) if d.size else 1.0
    return abs_err, rel, cos

"""Algorithmic bytes and flops of one batched decode step, per step and per
kernel class, for rooflines.

"Algorithmic" means what the method has to move or compute, counted once:
every streamed weight byte once per step (the point of the panel step,
"MODEL-BATCHING-RESULTS — multi-user batched decode, measured", section "The
lever": each weight row is read once for all B users), each lane's KV history
once per layer, the new K/V written once, activations in and out once, and
the logits written once.  Re-reads, padding and split-K partials are not
counted.  Flops count 2 per multiply-add of the projections and of attention
(q.k and p.v).

HBM peak 8 TB/s and the dense bf16 MFMA peak 2.5 PFLOP/s are MI355X's
published figures.
"""
from __future__ import annotations

from typing import Dict, Sequence

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}


def _wbytes_per_elem(wtype: int) -> float:
    return {0: 4.0, 1: 2.0, 2: 34.0 / 32.0}[wtype]


def act_bytes(wtype: int) -> int:
    return 4 if wtype == 0 else 2


def kv_bytes(wtype: int) -> int:
    return 2 if wtype == 1 else 4


def streamed_params(cfg) -> int:
    """Parameters one step streams: the four projection matrices of every layer plus the head."""
    per_layer = cfg.n_qkv * cfg.d + cfg.d * cfg.q_dim + 2 * cfg.ffn * cfg.d + cfg.d * cfg.ffn
    return cfg.n_layers * per_layer + cfg.vocab * cfg.d


def weight_bytes(cfg) -> float:
    return streamed_params(cfg) * _wbytes_per_elem(cfg.wtype)


def kv_bytes_per_token(cfg) -> int:
    """K and V of one position, all layers."""
    return 2 * cfg.n_layers * cfg.kv_dim * kv_bytes(cfg.wtype)


def step_bytes(cfg, positions: Sequence[int]) -> float:
    """Weights once + embedding rows + KV history reads + new KV writes + logits."""
    B = len(positions)
    kvt = kv_bytes_per_token(cfg)
    return (weight_bytes(cfg) + B * cfg.d * _wbytes_per_elem(cfg.wtype) + sum(positions) * kvt + B * kvt
            + B * cfg.vocab * 4)


def step_flops(cfg, positions: Sequence[int]) -> float:
    B = len(positions)
    attn = sum(4 * cfg.n_heads * cfg.head_dim * cfg.n_layers * (p + 1) for p in positions)
    return 2.0 * streamed_params(cfg) * B + attn


def roofline_time_s(cfg, positions: Sequence[int], dtype: str = "bf16") -> float:
    return max(step_bytes(cfg, positions) / (HBM_PEAK_GBS * 1e9),
               step_flops(cfg, positions) / (MFMA_PEAK_TFLOPS[dtype] * 1e12))


def kernel_bytes(cfg, cls: str, positions: Sequence[int]) -> float:
    """Algorithmic bytes of one launch of a kernel class (one layer for per-layer classes)."""
    B = len(positions)
    wb = _wbytes_per_elem(cfg.wtype)
    ab = act_bytes(cfg.wtype)
    d, F, V = cfg.d, cfg.ffn, cfg.vocab
    # projections that consume the normalised stream read it in the activation
    # format; the residual projections read and write the f32 residual x
    if cls == "gemm_qkv":
        return cfg.n_qkv * d * wb + B * d * ab + B * cfg.n_qkv * 4
    if cls == "gemm_o":
        return d * cfg.q_dim * wb + B * cfg.q_dim * ab + 2 * B * d * 4
    if cls == "gemm_gu":
        return 2 * F * d * wb + B * d * ab + B * F * ab
    if cls == "gemm_down":
        return d * F * wb + B * F * ab + 2 * B * d * 4
    if cls == "gemm_head":
        return V * d * wb + B * d * ab + B * V * 4
    if cls == "attention":
        # K and V of every cached position read once, the new K/V written, q/k/v read
        per_pos = 2 * cfg.kv_dim * kv_bytes(cfg.wtype)  # K and V of one position, one layer
        return sum(positions) * per_pos + B * per_pos + B * cfg.n_qkv * 4
    if cls == "attn_combine":
        return B * cfg.q_dim * ab  # the attention output
    if cls == "rmsnorm":
        return B * d * 4 + B * d * ab + d * 4
    if cls == "embed":
        return B * d * (wb + 4)
    return 0.0


def kernel_flops(cfg, cls: str, positions: Sequence[int]) -> float:
    B = len(positions)
    d, F = cfg.d, cfg.ffn
    n = {"gemm_qkv": cfg.n_qkv * d, "gemm_o": d * cfg.q_dim, "gemm_gu": 2 * F * d, "gemm_down": d * F,
         "gemm_head": cfg.vocab * d}.get(cls)
    if n is not None:
        return 2.0 * n * B
    if cls == "attention":
        return float(sum(4 * cfg.n_heads * cfg.head_dim * (p + 1) for p in positions))
    return 0.0


def per_class_summary(cfg, prof: Dict[str, tuple], positions: Sequence[int]) -> Dict[str, dict]:
    """From {class: (total ms, launches)} to per-class average launch time and achieved GB/s."""
    out = {}
    for cls, (ms, n) in prof.items():
        if n <= 0:
            continue
        avg_ms = ms / n
        b = kernel_bytes(cfg, cls, positions)
        out[cls] = {"total_ms": ms, "launches": n, "avg_us": avg_ms * 1e3,
                    "alg_bytes": b, "achieved_GBs": (b / (avg_ms * 1e-3) / 1e9) if b else None}
    return out

"""Seeded synthetic inputs for the batched decode step.

This package produces every input the decode step and its CPU oracle consume:
model weights (f32, bf16 or Q8_0 planes), prompts, per-lane KV contents,
KV lengths and arrival traces.  It holds none of the decode arithmetic.  All
numbers come from ``libsynth.so`` (Philox4x32-10 + Box-Muller, see
``synth.c``), so the same (seed, stream, index) gives the same value here, on
the GPU machine and in every test.

Model shapes follow the dense Llama decoder the pages name ("dense-Llama",
SwiGLU FFN, RMSNorm, rotary positions, grouped KV heads).  Storage layout of a
model (one array per tensor, row-major, ``[N_out, K_in]``):

* ``embed``     ``[vocab, d]``
* ``lm_head``   ``[vocab, d]`` (absent when tied to ``embed``)
* ``final_norm``, ``attn_norm[l]``, ``ffn_norm[l]``  ``[d]`` f32 gains (1.0)
* ``w_qkv[l]``  ``[(Hq + 2 Hkv) * hd, d]`` — query rows, then key rows, then value rows
* ``w_o[l]``    ``[d, Hq * hd]``
* ``w_gu[l]``   ``[2 F, d]`` — gate rows, then up rows
* ``w_down[l]`` ``[d, F]``

Stream ids under the weight seed: embed 1, lm_head 2, and for layer ``l``:
w_qkv ``16 + 8 l``, w_o ``17 + 8 l``, w_gu ``18 + 8 l``, w_down ``19 + 8 l``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None

WTYPE_F32, WTYPE_BF16, WTYPE_Q8_0 = 0, 1, 2
WTYPE_NAMES = {WTYPE_F32: "f32", WTYPE_BF16: "bf16", WTYPE_Q8_0: "q8_0"}

# Seeds of the synthetic workloads.
SEED_WEIGHTS = 0
SEED_TOKENS = 1
SEED_LENGTHS = 2
SEED_KV = 3
SEED_TRACE = 4


def build(force: bool = False) -> str:
    """Compile libsynth.so with gcc (OpenMP; fixed-order double arithmetic)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.synth_normal_f32.argtypes = [u64, u64, u64, i64, dbl, vp]
        L.synth_normal_bf16.argtypes = [u64, u64, u64, i64, dbl, vp]
        L.synth_words.argtypes = [u64, u64, u64, i64, vp]
        L.synth_uniform_int.argtypes = [u64, u64, u64, i64, i64, ctypes.c_uint32, vp]
        L.synth_uniform_open01.argtypes = [u64, u64, u64, i64, vp]
        for f in (L.synth_f32_to_bf16, L.synth_bf16_to_f32, L.synth_f32_to_f16, L.synth_f16_to_f32):
            f.argtypes = [vp, vp, i64]
        L.synth_q8_0_quantize.argtypes = [vp, i64, i64, vp, vp]
        for f in (L.synth_normal_f32, L.synth_normal_bf16, L.synth_words, L.synth_uniform_int,
                  L.synth_uniform_open01, L.synth_f32_to_bf16, L.synth_bf16_to_f32,
                  L.synth_f32_to_f16, L.synth_f16_to_f32, L.synth_q8_0_quantize):
            f.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ---- primitive draws ---------------------------------------------------------

def normal_f32(seed: int, stream: int, shape, scale: float = 1.0, first: int = 0) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    lib().synth_normal_f32(seed, stream, first, out.size, scale, _ptr(out))
    return out


def normal_bf16(seed: int, stream: int, shape, scale: float = 1.0, first: int = 0) -> np.ndarray:
    """bf16 bit patterns (uint16) of the f32 draws ``normal_f32`` gives, rounded to nearest even."""
    out = np.empty(shape, dtype=np.uint16)
    lib().synth_normal_bf16(seed, stream, first, out.size, scale, _ptr(out))
    return out


def words(seed: int, stream: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint32)
    lib().synth_words(seed, stream, first, n, _ptr(out))
    return out


def uniform_int(seed: int, stream: int, n: int, lo: int, hi_inclusive: int, first: int = 0) -> np.ndarray:
    span = hi_inclusive - lo + 1
    assert 0 < span < 2 ** 32
    out = np.empty(n, dtype=np.int32)
    lib().synth_uniform_int(seed, stream, first, n, lo, span, _ptr(out))
    return out


def uniform_open01(seed: int, stream: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    lib().synth_uniform_open01(seed, stream, first, n, _ptr(out))
    return out


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().synth_f32_to_bf16(_ptr(a), _ptr(out), a.size)
    return out


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.uint16)
    out = np.empty(a.shape, dtype=np.float32)
    lib().synth_bf16_to_f32(_ptr(a), _ptr(out), a.size)
    return out


def f32_to_f16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().synth_f32_to_f16(_ptr(a), _ptr(out), a.size)
    return out


def f16_to_f32(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.uint16)
    out = np.empty(a.shape, dtype=np.float32)
    lib().synth_f16_to_f32(_ptr(a), _ptr(out), a.size)
    return out


def q8_0_quantize(w: np.ndarray):
    """Q8_0 planes of an f32 ``[rows, k]`` matrix: (int8 ``[rows, k]``, f16 bits ``[rows, k/32]``)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, k = w.shape
    assert k % 32 == 0, "Q8_0 needs k % 32 == 0"
    q = np.empty((rows, k), dtype=np.int8)
    s = np.empty((rows, k // 32), dtype=np.uint16)
    lib().synth_q8_0_quantize(_ptr(w), rows, k, _ptr(q), _ptr(s))
    return q, s


# ---- model shapes ------------------------------------------------------------

@dataclass(frozen=True)
class ModelConfig:
    name: str
    d: int
    n_layers: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    tied: bool = False
    wtype: int = WTYPE_F32

    @property
    def n_qkv(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def with_wtype(self, wtype: int) -> "ModelConfig":
        return replace(self, wtype=wtype)


# Tiny dense Llama: d=64, 2 layers, 4 heads of 16, FFN 172, vocab 256.
TINY = ModelConfig("tiny-f32", d=64, n_layers=2, n_heads=4, n_kv_heads=4, head_dim=16, ffn=172, vocab=256)
# SmolLM2-135M shape: d=576, 30 layers, 9 query / 3 KV heads of 64, FFN 1536, vocab 49152, tied.
SMOL135M = ModelConfig("smollm2-135m-f32", d=576, n_layers=30, n_heads=9, n_kv_heads=3, head_dim=64,
                       ffn=1536, vocab=49152, tied=True)
SMOL135M_Q8 = replace(SMOL135M, name="smollm2-135m-q8_0", wtype=WTYPE_Q8_0)
# Mistral-7B shape: d=4096, 32 layers, 32 query / 8 KV heads of 128, FFN 14336, vocab 32000, bf16.
MISTRAL7B = ModelConfig("mistral-7b-bf16", d=4096, n_layers=32, n_heads=32, n_kv_heads=8, head_dim=128,
                        ffn=14336, vocab=32000, wtype=WTYPE_BF16)

CONFIGS = {c.name: c for c in (TINY, SMOL135M, SMOL135M_Q8, MISTRAL7B)}


def stream_id(tensor: str, layer: int = -1) -> int:
    if tensor == "embed":
        return 1
    if tensor == "lm_head":
        return 2
    off = {"w_qkv": 0, "w_o": 1, "w_gu": 2, "w_down": 3}[tensor]
    return 16 + 8 * layer + off


def matrix_shapes(cfg: ModelConfig):
    return {
        "w_qkv": (cfg.n_qkv, cfg.d),
        "w_o": (cfg.d, cfg.q_dim),
        "w_gu": (2 * cfg.ffn, cfg.d),
        "w_down": (cfg.d, cfg.ffn),
    }


@dataclass
class Matrix:
    """One weight matrix in its storage format.

    ``data``: f32 ``[N, K]`` (f32), uint16 bf16 bits ``[N, K]`` (bf16), or int8 ``[N, K]`` (Q8_0);
    ``scale``: f16 bits ``[N, K/32]`` for Q8_0, else None.
    """
    wtype: int
    data: np.ndarray
    scale: Optional[np.ndarray] = None

    @property
    def shape(self):
        return self.data.shape

    @property
    def nbytes(self) -> int:
        return self.data.nbytes + (self.scale.nbytes if self.scale is not None else 0)


@dataclass
class Weights:
    cfg: ModelConfig
    embed: Matrix
    lm_head: Optional[Matrix]
    final_norm: np.ndarray
    attn_norm: List[np.ndarray] = field(default_factory=list)
    ffn_norm: List[np.ndarray] = field(default_factory=list)
    w_qkv: List[Matrix] = field(default_factory=list)
    w_o: List[Matrix] = field(default_factory=list)
    w_gu: List[Matrix] = field(default_factory=list)
    w_down: List[Matrix] = field(default_factory=list)

    def head(self) -> Matrix:
        return self.embed if self.cfg.tied else self.lm_head

    def streamed_bytes(self) -> int:
        """Bytes of every matrix one decode step streams: the layer projections plus the head."""
        n = self.head().nbytes
        for l in range(self.cfg.n_layers):
            n += self.w_qkv[l].nbytes + self.w_o[l].nbytes + self.w_gu[l].nbytes + self.w_down[l].nbytes
        return n


def _make_matrix(cfg: ModelConfig, seed: int, stream: int, shape, wtype: int, std: float) -> Matrix:
    if wtype == WTYPE_F32:
        return Matrix(wtype, normal_f32(seed, stream, shape, std))
    if wtype == WTYPE_BF16:
        return Matrix(wtype, normal_bf16(seed, stream, shape, std))
    w = normal_f32(seed, stream, shape, std)
    q, s = q8_0_quantize(w)
    return Matrix(wtype, q, s)


def make_weights(cfg: ModelConfig, seed: int = SEED_WEIGHTS, std: float = 0.02,
                 wtype: Optional[int] = None) -> Weights:
    """Seeded synthetic weights: every matrix ~ N(0, std^2); RMSNorm gains 1.0.

    ``wtype`` overrides the storage type (the f32 weights a Q8_0 model was quantised
    from are ``make_weights(cfg, wtype=WTYPE_F32)``: the same draws).
    """
    wt = cfg.wtype if wtype is None else wtype
    cfg = cfg.with_wtype(wt)
    ones = np.ones(cfg.d, dtype=np.float32)
    W = Weights(cfg=cfg,
                embed=_make_matrix(cfg, seed, stream_id("embed"), (cfg.vocab, cfg.d), wt, std),
                lm_head=None if cfg.tied else _make_matrix(cfg, seed, stream_id("lm_head"),
                                                           (cfg.vocab, cfg.d), wt, std),
                final_norm=ones.copy())
    shapes = matrix_shapes(cfg)
    for l in range(cfg.n_layers):
        W.attn_norm.append(ones.copy())
        W.ffn_norm.append(ones.copy())
        for name in ("w_qkv", "w_o", "w_gu", "w_down"):
            getattr(W, name).append(_make_matrix(cfg, seed, stream_id(name, l), shapes[name], wt, std))
    return W


# ---- token, length, KV and trace draws ------------------------------------------

def prompt_tokens(cfg: ModelConfig, lane: int, length: int, seed: int = SEED_TOKENS) -> np.ndarray:
    """Uniform token ids in [0, vocab) for lane/job ``lane`` (stream = lane)."""
    return uniform_int(seed, lane, length, 0, cfg.vocab - 1)


def step_tokens(cfg: ModelConfig, n_lanes: int, seed: int = SEED_TOKENS) -> np.ndarray:
    """One input token per lane for a single decode step, uniform in [0, vocab) (stream 999)."""
    return uniform_int(seed, 999, n_lanes, 0, cfg.vocab - 1)


def kv_lengths(n_lanes: int, lo: int = 128, hi: int = 4096, seed: int = SEED_LENGTHS) -> np.ndarray:
    """Per-lane KV lengths uniform in [lo, hi] (stream 0, element = lane)."""
    return uniform_int(seed, 0, n_lanes, lo, hi)


def lane_kv_bf16(cfg: ModelConfig, lane: int, length: int, seed: int = SEED_KV):
    """Synthetic post-rotary K and V ~ N(0, 1) in bf16, layout ``[L, Hkv, length, hd]``.

    K of lane ``b`` is stream ``2 b``, V is stream ``2 b + 1``.
    """
    shape = (cfg.n_layers, cfg.n_kv_heads, length, cfg.head_dim)
    return normal_bf16(seed, 2 * lane, shape, 1.0), normal_bf16(seed, 2 * lane + 1, shape, 1.0)


def lane_kv_f32(cfg: ModelConfig, lane: int, length: int, seed: int = SEED_KV):
    shape = (cfg.n_layers, cfg.n_kv_heads, length, cfg.head_dim)
    return normal_f32(seed, 2 * lane, shape, 1.0), normal_f32(seed, 2 * lane + 1, shape, 1.0)


@dataclass
class Job:
    job_id: int
    arrival_step: int
    prompt: np.ndarray
    max_new_tokens: int


def make_trace(cfg: ModelConfig, n_jobs: int = 64, mean_gap: float = 4.0, prompt_lo: int = 32,
               prompt_hi: int = 1024, new_lo: int = 16, new_hi: int = 256,
               seed: int = SEED_TRACE) -> List[Job]:
    """Poisson arrivals (exponential gaps of mean ``mean_gap`` steps; arrival = floor of the
    running sum), prompt lengths and max_new_tokens uniform in the given ranges, prompt tokens
    uniform in [0, vocab).  Streams: gaps 0, prompt lengths 1, new-token counts 2, prompt of
    job j is stream 100 + j."""
    u = uniform_open01(seed, 0, n_jobs)
    gaps = -mean_gap * np.log(u)
    arrivals = np.floor(np.cumsum(gaps)).astype(np.int64)
    plens = uniform_int(seed, 1, n_jobs, prompt_lo, prompt_hi)
    news = uniform_int(seed, 2, n_jobs, new_lo, new_hi)
    jobs = []
    for j in range(n_jobs):
        toks = uniform_int(seed, 100 + j, int(plens[j]), 0, cfg.vocab - 1)
        jobs.append(Job(j, int(arrivals[j]), toks, int(news[j])))
    return jobs

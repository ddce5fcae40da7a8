"""CPU oracle for the batched decode step — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU product path never imports,
links or calls it, and it shares no code with the GPU path.

``liboracle.so`` (``oracle.c``) computes the plain f32 definition of a dense
Llama decode step, lane by lane, with fixed-order scalar arithmetic; see the
header of ``oracle.c`` for the math, the precision modes and the passages of
the pages it follows.  This module adds ctypes marshalling and the greedy
driver loop of the continuous-batching decode thread ("Fat-station continuous
batching", section "Components", item 3): a cleared lane is fed its prompt one
token per step, the step that feeds the last prompt token yields generated
token 1, and every generated token but the last is fed back, so a job with a
prompt of P tokens and n new tokens takes P + n - 1 steps.

Two builds of the same source: the default accumulates every sum in double
(sums exact up to double rounding, rounded to f32 where a value is stored);
``accumulate="f32"`` builds it with f32 accumulators instead.  The second is a
plain f32 evaluation of the same definition; comparing the two measures how
far any correct f32-accumulating implementation can drift from the exact
result at a given shape (used to size bf16 parity bars at full depth).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIBS = {"exact": os.path.join(_HERE, "liboracle.so"), "f32": os.path.join(_HERE, "liboracle_f32acc.so")}
_DEFS = {"exact": [], "f32": ["-DORC_ACC=float"]}
_lib = {}

ORC_F32, ORC_BF16, ORC_Q8_0 = 0, 1, 2


def build(force: bool = False, accumulate: str = "exact") -> str:
    """Compile the oracle library with gcc: -O2, no fast-math, no FMA contraction, OpenMP."""
    out = _LIBS[accumulate]
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(_SRC):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp"]
                              + _DEFS[accumulate] + ["-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, out)
    return out


class _Config(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int), ("n_layers", ctypes.c_int), ("n_heads", ctypes.c_int),
                ("n_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int), ("ffn", ctypes.c_int),
                ("vocab", ctypes.c_int), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("tied", ctypes.c_int), ("wtype", ctypes.c_int)]


class _Mat(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("scale", ctypes.c_void_p)]


class _Weights(ctypes.Structure):
    _fields_ = [("embed", _Mat), ("lm_head", _Mat), ("final_norm", ctypes.c_void_p),
                ("attn_norm", ctypes.POINTER(ctypes.c_void_p)), ("ffn_norm", ctypes.POINTER(ctypes.c_void_p)),
                ("w_qkv", ctypes.POINTER(_Mat)), ("w_o", ctypes.POINTER(_Mat)),
                ("w_gu", ctypes.POINTER(_Mat)), ("w_down", ctypes.POINTER(_Mat))]


def lib(accumulate: str = "exact"):
    if accumulate not in _lib:
        L = ctypes.CDLL(build(accumulate=accumulate))
        vp, i32, f32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_int64
        L.orc_model_create.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_Weights)]
        L.orc_model_create.restype = vp
        L.orc_model_destroy.argtypes = [vp]
        L.orc_lane_create.argtypes = [vp, i32]
        L.orc_lane_create.restype = vp
        L.orc_lane_destroy.argtypes = [vp]
        L.orc_lane_clear.argtypes = [vp]
        L.orc_lane_length.argtypes = [vp]
        L.orc_lane_length.restype = i32
        L.orc_lane_set_kv.argtypes = [vp, i32, i32, vp, vp]
        L.orc_lane_set_kv.restype = i32
        L.orc_lane_get_kv.argtypes = [vp, i32, vp, vp]
        L.orc_lane_get_kv.restype = i32
        L.orc_lane_evict_span.argtypes = [vp, vp, i32, i32]
        L.orc_lane_evict_span.restype = i32
        L.orc_step.argtypes = [vp, vp, i32, vp]
        L.orc_step.restype = i32
        L.orc_step_batch.argtypes = [vp, vp, i32, vp, vp]
        L.orc_step_batch.restype = i32
        L.orc_matvec.argtypes = [ctypes.POINTER(_Mat), i32, i32, i32, i32, vp, vp]
        L.orc_rmsnorm.argtypes = [vp, vp, i32, f32, vp]
        L.orc_rope_cs.argtypes = [i32, i32, f32, vp, vp]
        L.orc_rope.argtypes = [vp, i32, i32, f32]
        L.orc_silu.argtypes = [f32]
        L.orc_silu.restype = f32
        L.orc_attention.argtypes = [vp, vp, vp, i64, i32, i32, i32, i32, vp]
        L.orc_argmax.argtypes = [vp, i32]
        L.orc_argmax.restype = i32
        L.orc_round_bf16.argtypes = [f32]
        L.orc_round_bf16.restype = f32
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f32.restype = f32
        L.orc_num_threads.restype = i32
        for f in (L.orc_model_destroy, L.orc_lane_destroy, L.orc_lane_clear, L.orc_matvec, L.orc_rmsnorm,
                  L.orc_rope_cs, L.orc_rope, L.orc_attention):
            f.restype = None
        _lib[accumulate] = L
    return _lib[accumulate]


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


# ---- pieces ------------------------------------------------------------------

def _mat(data: np.ndarray, scale=None) -> _Mat:
    return _Mat(_p(data), _p(scale) if scale is not None else None)


def matvec(data: np.ndarray, x: np.ndarray, wtype: int = ORC_F32, scale=None, row0: int = 0,
           nrows: int = None) -> np.ndarray:
    K = data.shape[1]
    nrows = data.shape[0] - row0 if nrows is None else nrows
    x = _f32(x)
    y = np.empty(nrows, dtype=np.float32)
    m = _mat(data, scale)
    lib().orc_matvec(ctypes.byref(m), wtype, row0, nrows, K, _p(x), _p(y))
    return y


def rmsnorm(x, g, eps: float) -> np.ndarray:
    x, g = _f32(x), _f32(g)
    out = np.empty_like(x)
    lib().orc_rmsnorm(_p(x), _p(g), x.size, eps, _p(out))
    return out


def rope_cs(hd: int, pos: int, theta: float):
    c = np.empty(hd // 2, dtype=np.float32)
    s = np.empty(hd // 2, dtype=np.float32)
    lib().orc_rope_cs(hd, pos, theta, _p(c), _p(s))
    return c, s


def rope(v, pos: int, theta: float) -> np.ndarray:
    v = _f32(v).copy()
    lib().orc_rope(_p(v), v.size, pos, theta)
    return v


def silu(u: float) -> float:
    return lib().orc_silu(u)


def attention(q, K, V, n_heads: int, n_kv_heads: int, hd: int) -> np.ndarray:
    """q [Hq*hd]; K, V [n_keys, Hkv*hd] -> [Hq*hd]."""
    q, K, V = _f32(q), _f32(K), _f32(V)
    out = np.empty(n_heads * hd, dtype=np.float32)
    lib().orc_attention(_p(q), _p(K), _p(V), K.shape[1], K.shape[0], n_heads, n_kv_heads, hd, _p(out))
    return out


def argmax(x) -> int:
    x = _f32(x)
    return lib().orc_argmax(_p(x), x.size)


def round_bf16(x: float) -> float:
    return lib().orc_round_bf16(x)


def f16_to_f32(h: int) -> float:
    return lib().orc_f16_to_f32(h)


def num_threads() -> int:
    return lib().orc_num_threads()


# ---- model -------------------------------------------------------------------

class Model:
    """Borrows the arrays of a ``synth.Weights`` (kept alive by this object).

    accumulate: "exact" (double accumulators, the oracle) or "f32" (the same
    definition with f32 accumulators)."""

    def __init__(self, W, accumulate: str = "exact"):
        self.L = lib(accumulate)
        c = W.cfg
        self.cfg = c
        self.W = W
        self._cfg = _Config(c.d, c.n_layers, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn, c.vocab,
                            c.rms_eps, c.rope_theta, int(c.tied), c.wtype)
        L = c.n_layers
        mk = lambda m: _mat(m.data, m.scale)
        self._attn = (ctypes.c_void_p * L)(*[_p(a) for a in W.attn_norm])
        self._ffn = (ctypes.c_void_p * L)(*[_p(a) for a in W.ffn_norm])
        self._qkv = (_Mat * L)(*[mk(m) for m in W.w_qkv])
        self._o = (_Mat * L)(*[mk(m) for m in W.w_o])
        self._gu = (_Mat * L)(*[mk(m) for m in W.w_gu])
        self._down = (_Mat * L)(*[mk(m) for m in W.w_down])
        head = W.lm_head if W.lm_head is not None else W.embed
        self._w = _Weights(mk(W.embed), mk(head), _p(W.final_norm),
                           ctypes.cast(self._attn, ctypes.POINTER(ctypes.c_void_p)),
                           ctypes.cast(self._ffn, ctypes.POINTER(ctypes.c_void_p)),
                           self._qkv, self._o, self._gu, self._down)
        self.h = self.L.orc_model_create(ctypes.byref(self._cfg), ctypes.byref(self._w))
        if not self.h:
            raise ValueError("oracle rejected the model config")

    def __del__(self):
        if getattr(self, "h", None):
            self.L.orc_model_destroy(self.h)
            self.h = None

    def lane(self, max_seq: int) -> "Lane":
        return Lane(self, max_seq)

    def step(self, lane: "Lane", token: int) -> np.ndarray:
        out = np.empty(self.cfg.vocab, dtype=np.float32)
        rc = self.L.orc_step(self.h, lane.h, int(token), _p(out))
        if rc != 0:
            raise ValueError("oracle step rejected (token out of range or lane full)")
        return out

    def step_batch(self, lanes: Sequence["Lane"], tokens) -> np.ndarray:
        B = len(lanes)
        toks = np.ascontiguousarray(tokens, dtype=np.int32)
        arr = (ctypes.c_void_p * B)(*[ln.h for ln in lanes])
        out = np.empty((B, self.cfg.vocab), dtype=np.float32)
        rc = self.L.orc_step_batch(self.h, arr, B, _p(toks), _p(out))
        if rc != 0:
            raise ValueError("oracle batch step rejected (rc=%d)" % rc)
        return out


class Lane:
    def __init__(self, model: Model, max_seq: int):
        self.model = model
        self.L = model.L
        self.max_seq = max_seq
        self.h = self.L.orc_lane_create(model.h, max_seq)
        if not self.h:
            raise MemoryError("oracle lane allocation failed")

    def __del__(self):
        if getattr(self, "h", None):
            self.L.orc_lane_destroy(self.h)
            self.h = None

    def clear(self):
        self.L.orc_lane_clear(self.h)

    def evict_span(self, begin: int, end: int):
        """Drop positions [begin, end); later entries move down, keys rotated to their new positions."""
        if self.L.orc_lane_evict_span(self.model.h, self.h, int(begin), int(end)) != 0:
            raise ValueError("span outside the lane")

    @property
    def length(self) -> int:
        return self.L.orc_lane_length(self.h)

    def set_kv(self, k: np.ndarray, v: np.ndarray):
        """k, v: f32 ``[L, Hkv, length, hd]`` (post-rotary keys)."""
        k, v = _f32(k), _f32(v)
        c = self.model.cfg
        if self.L.orc_lane_set_kv(self.h, k.shape[2], c.head_dim, _p(k), _p(v)) != 0:
            raise ValueError("length exceeds the lane capacity")

    def get_kv(self):
        c = self.model.cfg
        n = self.length
        shape = (c.n_layers, c.n_kv_heads, n, c.head_dim)
        k = np.empty(shape, dtype=np.float32)
        v = np.empty(shape, dtype=np.float32)
        self.L.orc_lane_get_kv(self.h, c.head_dim, _p(k), _p(v))
        return k, v


# ---- greedy driver -------------------------------------------------------------

def generate(model: Model, prompt, n_new: int, max_seq: int = None, return_logits: bool = False):
    """Serial greedy generation of one job on a fresh lane: P + n - 1 steps."""
    prompt = [int(t) for t in prompt]
    assert len(prompt) >= 1 and n_new >= 1
    lane = model.lane(max_seq or (len(prompt) + n_new))
    out, logits_seq = [], []
    tok = prompt[0]
    for step in range(len(prompt) + n_new - 1):
        lg = model.step(lane, tok)
        if return_logits:
            logits_seq.append(lg)
        if step + 1 < len(prompt):
            tok = prompt[step + 1]
        else:
            tok = argmax(lg)
            out.append(tok)
    return (out, logits_seq) if return_logits else out


def generate_lockstep(model: Model, prompts: Sequence[Sequence[int]], n_new, max_seq: int = None,
                      return_logits: bool = False):
    """Lockstep greedy generation: every step is one panel step over the lanes still live.

    Returns per-lane generated tokens (and per-lane logits of every step they took)."""
    B = len(prompts)
    n_new = [n_new] * B if np.isscalar(n_new) else list(n_new)
    lanes = [model.lane(max_seq or (len(p) + n)) for p, n in zip(prompts, n_new)]
    feed = [0] * B
    last = [int(p[0]) for p in prompts]
    gen: List[List[int]] = [[] for _ in range(B)]
    logs: List[list] = [[] for _ in range(B)]
    while True:
        live = [b for b in range(B) if len(gen[b]) < n_new[b]]
        if not live:
            break
        toks = [int(prompts[b][feed[b]]) if feed[b] < len(prompts[b]) else last[b] for b in live]
        lg = model.step_batch([lanes[b] for b in live], toks)
        for i, b in enumerate(live):
            feed[b] += 1
            if return_logits:
                logs[b].append(lg[i])
            if feed[b] >= len(prompts[b]):
                last[b] = argmax(lg[i])
                gen[b].append(last[b])
    return (gen, logs) if return_logits else gen

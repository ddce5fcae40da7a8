"""Python binding of libcbd.so, the batched decode step for MI355X (gfx950).

Argument marshalling only: every step of the decode runs in the HIP kernels
behind the C-ABI of ``include/cbd.h``; the names here mirror it.  PyTorch is
used for device memory and streams.  There is no CPU fallback: without the
built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcbd.so")

CBD_F32, CBD_BF16, CBD_Q8_0 = 0, 1, 2
ERRORS = {
    -1: "CBD_E_ARG", -2: "CBD_E_DUP_LANE", -3: "CBD_E_LANE_NOT_LIVE", -4: "CBD_E_POS_MISMATCH",
    -5: "CBD_E_KV_FULL", -6: "CBD_E_TOKEN", -7: "CBD_E_NO_FREE_LANE", -8: "CBD_E_HIP",
    -9: "CBD_E_WORKSPACE", -10: "CBD_E_UNSUPPORTED",
}
# Every symbol include/cbd.h declares.
SYMBOLS = [
    "cbd_version", "cbd_last_error", "cbd_model_create", "cbd_model_destroy", "cbd_arena_bytes",
    "cbd_arena_create", "cbd_arena_destroy", "cbd_lane_alloc", "cbd_lane_clear", "cbd_lane_evict",
    "cbd_lane_length", "cbd_arena_used_bytes", "cbd_arena_live_lanes", "cbd_workspace_bytes",
    "cbd_decode_step_batch", "cbd_decode_step", "cbd_lane_kv_export", "cbd_lane_kv_import", "cbd_set_variant",
    "cbd_lane_truncate", "cbd_profile_enable", "cbd_profile_reset", "cbd_profile_read", "cbd_profile_classes",
    "cbd_profile_class_name", "cbd_set_graph_replay", "cbd_arena_block_bytes", "cbd_arena_n_blocks",
    "cbd_arena_free_blocks", "cbd_prefill_batch", "cbd_sched_create", "cbd_sched_create_device",
    "cbd_sched_destroy", "cbd_sched_submit", "cbd_sched_tick", "cbd_sched_run", "cbd_sched_get_telemetry",
    "cbd_sched_job_tokens", "cbd_lane_clone", "cbd_lane_evict_span", "cbd_debug_alloc_count",
    "cbd_decode_step_batch_noalloc", "cbd_noalloc_scratch_bytes", "cbd_packed_bytes", "cbd_pack_matrix",
]


class CbdError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s (%d): %s" % (ERRORS.get(code, "?"), code, msg))
        self.code = code
        self.name = ERRORS.get(code, "?")


class Config(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int), ("n_layers", ctypes.c_int), ("n_heads", ctypes.c_int),
                ("n_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int), ("ffn_dim", ctypes.c_int),
                ("vocab", ctypes.c_int), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("tied_embeddings", ctypes.c_int), ("wtype", ctypes.c_int), ("packed", ctypes.c_int)]


class _Matrix(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("scale", ctypes.c_void_p)]


class _Weights(ctypes.Structure):
    _fields_ = [("embed", _Matrix), ("lm_head", _Matrix), ("final_norm", ctypes.c_void_p),
                ("attn_norm", ctypes.POINTER(ctypes.c_void_p)), ("ffn_norm", ctypes.POINTER(ctypes.c_void_p)),
                ("w_qkv", ctypes.POINTER(_Matrix)), ("w_o", ctypes.POINTER(_Matrix)),
                ("w_gu", ctypes.POINTER(_Matrix)), ("w_down", ctypes.POINTER(_Matrix))]


# scheduler (host policy over the step)
SCHED_DECISIONS = {0: "QUEUED", 1: "REJECTED_KV_BUDGET", 2: "REJECTED_SCRATCH_BUDGET", 3: "REJECTED_DUPLICATE",
                   4: "REJECTED_QUEUE_FULL"}
_P32 = ctypes.POINTER(ctypes.c_int32)
PREFILL_FN = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int, _P32, _P32, _P32, _P32, _P32)
DECODE_FN = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int, _P32, _P32, _P32, _P32)
ALLOC_FN = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, _P32)
EVICT_FN = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int32)


class SchedBudget(ctypes.Structure):
    _fields_ = [("weight_bytes", ctypes.c_size_t), ("kv_budget_bytes", ctypes.c_size_t),
                ("kv_bytes_per_token", ctypes.c_size_t), ("scratch_per_session", ctypes.c_size_t),
                ("scratch_budget_bytes", ctypes.c_size_t), ("max_active", ctypes.c_int),
                ("max_queue", ctypes.c_int), ("max_batch", ctypes.c_int),
                ("max_prefill_tokens_per_tick", ctypes.c_int)]


class SchedEngine(ctypes.Structure):
    _fields_ = [("ctx", ctypes.c_void_p), ("prefill", PREFILL_FN), ("decode", DECODE_FN),
                ("lane_alloc", ALLOC_FN), ("lane_evict", EVICT_FN)]


class SchedTelemetry(ctypes.Structure):
    _fields_ = [("ticks", ctypes.c_longlong), ("decode_ticks", ctypes.c_longlong), ("active", ctypes.c_int),
                ("queued", ctypes.c_int), ("finished", ctypes.c_int), ("effective_active_cap", ctypes.c_int),
                ("occupancy_last", ctypes.c_int), ("occupancy_max", ctypes.c_int),
                ("occupancy_avg", ctypes.c_double), ("kv_bytes", ctypes.c_size_t),
                ("kv_peak_bytes", ctypes.c_size_t), ("kv_budget_bytes", ctypes.c_size_t),
                ("scratch_bytes", ctypes.c_size_t), ("scratch_budget_bytes", ctypes.c_size_t),
                ("weight_bytes", ctypes.c_size_t), ("prefill_tokens", ctypes.c_longlong),
                ("decode_tokens", ctypes.c_longlong), ("rejected", ctypes.c_longlong),
                ("rejected_kv", ctypes.c_longlong), ("rejected_scratch", ctypes.c_longlong),
                ("rejected_duplicate", ctypes.c_longlong), ("rejected_queue_full", ctypes.c_longlong)]


_lib = None


def lib():
    """Load libcbd.so (built in-tree by build.py); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libcbd.so is not built (%s); run continuous_batching_decode_step_amd/build.py"
                               % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        pi32 = ctypes.POINTER(ctypes.c_int32)
        L.cbd_version.restype = ctypes.c_char_p
        L.cbd_last_error.restype = ctypes.c_char_p
        L.cbd_model_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(_Weights), ctypes.POINTER(vp)]
        L.cbd_model_destroy.argtypes = [vp]
        L.cbd_model_destroy.restype = None
        L.cbd_packed_bytes.argtypes = [i32, i32, i32, i32]
        L.cbd_packed_bytes.restype = sz
        L.cbd_pack_matrix.argtypes = [i32, vp, vp, i32, i32, i32, vp]
        L.cbd_arena_bytes.argtypes = [ctypes.POINTER(Config), i32, i32]
        L.cbd_arena_bytes.restype = sz
        L.cbd_arena_block_bytes.argtypes = [ctypes.POINTER(Config)]
        L.cbd_arena_block_bytes.restype = sz
        L.cbd_arena_n_blocks.argtypes = [vp]
        L.cbd_arena_free_blocks.argtypes = [vp]
        L.cbd_arena_create.argtypes = [vp, i32, i32, vp, sz, ctypes.POINTER(vp)]
        L.cbd_arena_destroy.argtypes = [vp]
        L.cbd_arena_destroy.restype = None
        L.cbd_lane_alloc.argtypes = [vp, pi32]
        L.cbd_lane_clear.argtypes = [vp, i32]
        L.cbd_lane_evict.argtypes = [vp, i32]
        L.cbd_lane_length.argtypes = [vp, i32]
        L.cbd_arena_used_bytes.argtypes = [vp]
        L.cbd_arena_used_bytes.restype = sz
        L.cbd_arena_live_lanes.argtypes = [vp]
        L.cbd_workspace_bytes.argtypes = [vp, i32, i32]
        L.cbd_workspace_bytes.restype = sz
        L.cbd_decode_step_batch.argtypes = [vp, vp, i32, pi32, pi32, pi32, vp, vp, vp, sz, vp]
        L.cbd_prefill_batch.argtypes = [vp, vp, i32, pi32, pi32, pi32, pi32, vp, vp, vp, sz, vp]
        L.cbd_decode_step.argtypes = [vp, vp, i32, pi32, ctypes.c_int32, vp, vp, vp, sz, vp]
        L.cbd_lane_kv_export.argtypes = [vp, i32, vp, vp, vp]
        L.cbd_lane_kv_import.argtypes = [vp, i32, i32, vp, vp, vp]
        L.cbd_set_variant.argtypes = [vp, i32]
        L.cbd_lane_truncate.argtypes = [vp, i32, i32]
        L.cbd_set_graph_replay.argtypes = [vp, i32]
        L.cbd_profile_enable.argtypes = [vp, i32]
        L.cbd_profile_reset.argtypes = [vp]
        L.cbd_profile_read.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_longlong)]
        L.cbd_profile_classes.argtypes = []
        L.cbd_profile_class_name.argtypes = [i32]
        L.cbd_profile_class_name.restype = ctypes.c_char_p
        L.cbd_decode_step_batch_noalloc.argtypes = [vp, vp, i32, pi32, pi32, pi32, vp, vp, vp]
        L.cbd_noalloc_scratch_bytes.argtypes = []
        L.cbd_noalloc_scratch_bytes.restype = sz
        L.cbd_debug_alloc_count.argtypes = []
        L.cbd_debug_alloc_count.restype = ctypes.c_longlong
        L.cbd_lane_clone.argtypes = [vp, i32, i32, i32, vp]
        L.cbd_lane_evict_span.argtypes = [vp, i32, i32, i32, vp]
        L.cbd_sched_create.argtypes = [ctypes.POINTER(SchedBudget), ctypes.POINTER(SchedEngine), ctypes.POINTER(vp)]
        L.cbd_sched_create_device.argtypes = [ctypes.POINTER(SchedBudget), vp, vp, vp, sz, vp, vp, vp,
                                              ctypes.POINTER(vp)]
        L.cbd_sched_destroy.argtypes = [vp]
        L.cbd_sched_destroy.restype = None
        L.cbd_sched_submit.argtypes = [vp, ctypes.c_longlong, pi32, i32, i32, ctypes.POINTER(ctypes.c_int)]
        L.cbd_sched_tick.argtypes = [vp, ctypes.POINTER(ctypes.c_int)]
        L.cbd_sched_run.argtypes = [vp, ctypes.c_longlong]
        L.cbd_sched_get_telemetry.argtypes = [vp, ctypes.POINTER(SchedTelemetry)]
        L.cbd_sched_job_tokens.argtypes = [vp, ctypes.c_longlong, pi32, i32, ctypes.POINTER(ctypes.c_int),
                                           ctypes.POINTER(ctypes.c_int)]
        _lib = L
    return _lib


def _check(rc: int) -> int:
    if rc < 0:
        raise CbdError(rc, lib().cbd_last_error().decode())
    return rc


def _ptr(t) -> Optional[int]:
    """Device address of a torch tensor (or an int / None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        assert t.flags["C_CONTIGUOUS"]
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _pi32(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def config_of(cfg, packed: bool = False) -> Config:
    """C config from any object with the fields of a model shape (d, n_layers, ...); packed: the
    layer matrices (and an untied LM head) are in the packed tile layout."""
    return Config(cfg.d, cfg.n_layers, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn, cfg.vocab,
                  cfg.rms_eps, cfg.rope_theta, int(cfg.tied), int(cfg.wtype), int(packed))


# ---- device weights -------------------------------------------------------------

@dataclass
class DeviceMatrix:
    data: "object"                    # torch tensor [N, K] (float32 / int16 bf16 bits / int8)
    scale: Optional["object"] = None  # torch int16 tensor of binary16 bits [N, K/32] (Q8_0)


@dataclass
class DeviceWeights:
    embed: DeviceMatrix
    lm_head: Optional[DeviceMatrix]
    final_norm: "object"
    attn_norm: List["object"]
    ffn_norm: List["object"]
    w_qkv: List[DeviceMatrix]
    w_o: List[DeviceMatrix]
    w_gu: List[DeviceMatrix]
    w_down: List[DeviceMatrix]
    packed: bool = False              # layer matrices and an untied head in the packed tile layout

    def nbytes(self) -> int:
        n = 0
        for m in [self.embed, self.lm_head] + self.w_qkv + self.w_o + self.w_gu + self.w_down:
            if m is not None:
                n += m.data.numel() * m.data.element_size()
                if m.scale is not None:
                    n += m.scale.numel() * m.scale.element_size()
        return n


def packable(cfg) -> bool:
    """Whether a model shape's layer matrices have the packed tile layout (bf16, every K a multiple of 32)."""
    return int(cfg.wtype) == CBD_BF16 and all(k % 32 == 0 for k in (cfg.d, cfg.ffn, cfg.n_heads * cfg.head_dim))


def pack_matrix(data, rows: int, halves: int = 1, stream=None):
    """The packed tile layout (cbd_pack_matrix) of a bf16 device matrix [halves * rows, K] (int16 bits),
    as a new device tensor of int16 bits."""
    import torch
    K = int(data.shape[1])
    nb = lib().cbd_packed_bytes(CBD_BF16, rows, K, halves)
    if nb == 0:
        raise CbdError(-10, "no packed layout for %d x %d rows, K %d" % (halves, rows, K))
    out = torch.empty(nb // 2, dtype=torch.int16, device=data.device)
    _check(lib().cbd_pack_matrix(CBD_BF16, _ptr(data), _ptr(out), rows, K, halves, _stream(stream)))
    return out


def upload_weights(W, device="cuda", pack: Optional[bool] = None) -> DeviceWeights:
    """Copy host weight arrays (numpy, in the layout of include/cbd.h) to device tensors.  pack (default:
    whenever the shape allows it, see packable): bf16 layer matrices and an untied LM head go to the
    device in the packed tile layout, which the weight-streaming kernels load in whole kilobytes."""
    import torch

    def t(a):
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    def m(x):
        return None if x is None else DeviceMatrix(t(x.data), None if x.scale is None else t(x.scale))

    cfg = W.cfg
    if pack is None:
        pack = packable(cfg)
    elif pack and not packable(cfg):
        raise CbdError(-10, "model shape has no packed layout")

    def mp(x, halves=1):
        if x is None or not pack:
            return m(x)
        d = t(x.data)
        p = pack_matrix(d, d.shape[0] // halves, halves)
        torch.cuda.synchronize()
        del d
        return DeviceMatrix(p, None)

    return DeviceWeights(embed=m(W.embed), lm_head=mp(W.lm_head), final_norm=t(W.final_norm),
                         attn_norm=[t(a) for a in W.attn_norm], ffn_norm=[t(a) for a in W.ffn_norm],
                         w_qkv=[mp(x) for x in W.w_qkv], w_o=[mp(x) for x in W.w_o],
                         w_gu=[mp(x, 2) for x in W.w_gu], w_down=[mp(x) for x in W.w_down], packed=bool(pack))


# ---- objects ------------------------------------------------------------------------

class Model:
    """cbd_model over device weights (kept referenced by this object)."""

    def __init__(self, cfg, weights: DeviceWeights):
        self.cfg = cfg
        self.weights = weights
        self._c = config_of(cfg, weights.packed)
        L = cfg.n_layers
        mat = lambda x: _Matrix(_ptr(x.data), _ptr(x.scale)) if x is not None else _Matrix(None, None)
        self._attn = (ctypes.c_void_p * L)(*[_ptr(a) for a in weights.attn_norm])
        self._ffn = (ctypes.c_void_p * L)(*[_ptr(a) for a in weights.ffn_norm])
        self._qkv = (_Matrix * L)(*[mat(x) for x in weights.w_qkv])
        self._o = (_Matrix * L)(*[mat(x) for x in weights.w_o])
        self._gu = (_Matrix * L)(*[mat(x) for x in weights.w_gu])
        self._down = (_Matrix * L)(*[mat(x) for x in weights.w_down])
        self._w = _Weights(mat(weights.embed), mat(weights.lm_head), _ptr(weights.final_norm),
                           ctypes.cast(self._attn, ctypes.POINTER(ctypes.c_void_p)),
                           ctypes.cast(self._ffn, ctypes.POINTER(ctypes.c_void_p)),
                           self._qkv, self._o, self._gu, self._down)
        h = ctypes.c_void_p()
        _check(lib().cbd_model_create(ctypes.byref(self._c), ctypes.byref(self._w), ctypes.byref(h)))
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            lib().cbd_model_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_bytes(self, max_batch: int, max_seq: int) -> int:
        return lib().cbd_workspace_bytes(self.h, max_batch, max_seq)

    def set_variant(self, variant: int):
        _check(lib().cbd_set_variant(self.h, variant))

    def set_graph_replay(self, on: bool = True):
        _check(lib().cbd_set_graph_replay(self.h, int(on)))

    def profile_enable(self, on: bool = True):
        _check(lib().cbd_profile_enable(self.h, int(on)))

    def profile_reset(self):
        _check(lib().cbd_profile_reset(self.h))

    def profile_read(self) -> dict:
        """{class name: (total ms, launches)} since the last reset."""
        out = {}
        for c in range(lib().cbd_profile_classes()):
            ms, n = ctypes.c_double(), ctypes.c_longlong()
            _check(lib().cbd_profile_read(self.h, c, ctypes.byref(ms), ctypes.byref(n)))
            out[lib().cbd_profile_class_name(c).decode()] = (ms.value, n.value)
        return out

    def decode_step_batch_noalloc(self, arena: "Arena", lanes: Sequence[int], positions: np.ndarray, tokens,
                                  logits, argmax=None, stream=None) -> None:
        """cbd_decode_step_batch_noalloc: the step over the device's static scratch, allocating nothing.
        positions: np.int32 array, advanced in place on success."""
        ln = _i32(lanes)
        assert isinstance(positions, np.ndarray) and positions.dtype == np.int32 and positions.flags["C_CONTIGUOUS"]
        tk = _i32(tokens)
        B = len(ln)
        assert len(positions) == B and len(tk) == B
        _check(lib().cbd_decode_step_batch_noalloc(self.h, arena.h, B, _pi32(ln), _pi32(positions), _pi32(tk),
                                                   _ptr(logits), _ptr(argmax), _stream(stream)))

    def decode_step_batch(self, arena: "Arena", lanes: Sequence[int], positions: np.ndarray, tokens,
                          logits, argmax=None, workspace=None, workspace_bytes: Optional[int] = None,
                          stream=None) -> None:
        """positions: np.int32 array, advanced in place on success."""
        ln = _i32(lanes)
        assert isinstance(positions, np.ndarray) and positions.dtype == np.int32 and positions.flags["C_CONTIGUOUS"]
        tk = _i32(tokens)
        B = len(ln)
        assert len(positions) == B and len(tk) == B
        wsb = workspace_bytes if workspace_bytes is not None else (
            0 if workspace is None else workspace.numel() * workspace.element_size())
        _check(lib().cbd_decode_step_batch(self.h, arena.h, B, _pi32(ln), _pi32(positions), _pi32(tk),
                                           _ptr(logits), _ptr(argmax), _ptr(workspace), wsb, _stream(stream)))

    def prefill_batch(self, arena: "Arena", lanes: Sequence[int], positions: np.ndarray, counts, tokens,
                      logits, argmax=None, workspace=None, workspace_bytes: Optional[int] = None,
                      stream=None) -> None:
        """counts[i] tokens for lane i, tokens concatenated lane by lane; logits [len(lanes), vocab] of each
        lane's last token.  positions: np.int32 array, advanced in place by counts on success."""
        ln = _i32(lanes)
        assert isinstance(positions, np.ndarray) and positions.dtype == np.int32 and positions.flags["C_CONTIGUOUS"]
        ct = _i32(counts)
        tk = _i32(tokens)
        n = len(ln)
        assert len(positions) == n and len(ct) == n and len(tk) == int(ct.astype(np.int64).sum())
        wsb = workspace_bytes if workspace_bytes is not None else (
            0 if workspace is None else workspace.numel() * workspace.element_size())
        _check(lib().cbd_prefill_batch(self.h, arena.h, n, _pi32(ln), _pi32(positions), _pi32(ct), _pi32(tk),
                                       _ptr(logits), _ptr(argmax), _ptr(workspace), wsb, _stream(stream)))

    def decode_step(self, arena: "Arena", lane: int, position: np.ndarray, token: int, logits, argmax=None,
                    workspace=None, workspace_bytes: Optional[int] = None, stream=None) -> None:
        """position: np.int32 array of one element, advanced in place on success."""
        assert isinstance(position, np.ndarray) and position.dtype == np.int32 and position.size == 1
        wsb = workspace_bytes if workspace_bytes is not None else (
            0 if workspace is None else workspace.numel() * workspace.element_size())
        _check(lib().cbd_decode_step(self.h, arena.h, lane, _pi32(position), int(token), _ptr(logits),
                                     _ptr(argmax), _ptr(workspace), wsb, _stream(stream)))


def alloc_count() -> int:
    """Device and pinned host allocations the library has made so far (cbd_debug_alloc_count)."""
    return int(lib().cbd_debug_alloc_count())


def arena_bytes(cfg, n_lanes: int, max_seq: int) -> int:
    """Bytes for every one of n_lanes lanes to hold max_seq positions at once."""
    c = config_of(cfg)
    return lib().cbd_arena_bytes(ctypes.byref(c), n_lanes, max_seq)


def arena_block_bytes(cfg) -> int:
    """Bytes of one KV block (64 positions of one lane, every layer and KV head, K and V)."""
    c = config_of(cfg)
    return lib().cbd_arena_block_bytes(ctypes.byref(c))


class Arena:
    """cbd_arena over caller-owned device memory (kept referenced by this object)."""

    def __init__(self, model: Model, n_lanes: int, max_seq: int, dev_mem, dev_bytes: Optional[int] = None):
        self.model = model
        self.n_lanes = n_lanes
        self.max_seq = max_seq
        self.mem = dev_mem
        nbytes = dev_bytes if dev_bytes is not None else dev_mem.numel() * dev_mem.element_size()
        h = ctypes.c_void_p()
        _check(lib().cbd_arena_create(model.h, n_lanes, max_seq, _ptr(dev_mem), nbytes, ctypes.byref(h)))
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            lib().cbd_arena_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def lane_alloc(self) -> int:
        out = ctypes.c_int32()
        _check(lib().cbd_lane_alloc(self.h, ctypes.byref(out)))
        return out.value

    def lane_clear(self, lane: int):
        _check(lib().cbd_lane_clear(self.h, lane))

    def lane_evict(self, lane: int):
        _check(lib().cbd_lane_evict(self.h, lane))

    def lane_truncate(self, lane: int, length: int):
        _check(lib().cbd_lane_truncate(self.h, lane, length))

    def lane_length(self, lane: int) -> int:
        return _check(lib().cbd_lane_length(self.h, lane))

    @property
    def used_bytes(self) -> int:
        return lib().cbd_arena_used_bytes(self.h)

    @property
    def live_lanes(self) -> int:
        return lib().cbd_arena_live_lanes(self.h)

    @property
    def n_blocks(self) -> int:
        return lib().cbd_arena_n_blocks(self.h)

    @property
    def free_blocks(self) -> int:
        return lib().cbd_arena_free_blocks(self.h)

    def lane_evict_span(self, lane: int, begin: int, end: int, stream=None):
        """Drop positions [begin, end) of a lane; later entries move down, keys rotated to their new positions."""
        _check(lib().cbd_lane_evict_span(self.h, lane, begin, end, _stream(stream)))

    def lane_clone(self, src: int, dst: int, n: int, stream=None):
        """dst := the first n positions of src (prefix reuse); synchronous with respect to stream."""
        _check(lib().cbd_lane_clone(self.h, src, dst, n, _stream(stream)))

    def kv_export(self, lane: int, k_dst, v_dst, stream=None):
        _check(lib().cbd_lane_kv_export(self.h, lane, _ptr(k_dst), _ptr(v_dst), _stream(stream)))

    def kv_import(self, lane: int, length: int, k_src, v_src, stream=None):
        _check(lib().cbd_lane_kv_import(self.h, lane, length, _ptr(k_src), _ptr(v_src), _stream(stream)))


class Scheduler:
    """cbd_sched: the continuous-batching host policy (admission budgets, decode first then bounded
    prefill, release on completion, telemetry).  engine: a dict of Python callables
    {prefill(n, lanes, positions, counts, tokens, next) -> int, decode(B, lanes, positions, tokens, next) -> int,
    lane_alloc(lane_out) -> int, lane_evict(lane) -> int} taking ctypes int32 pointers, or None with
    device=(model, arena, workspace, logits, argmax, stream) for the decode path of this library."""

    def __init__(self, budget: dict, engine: Optional[dict] = None, device=None):
        b = SchedBudget(**budget)
        h = ctypes.c_void_p()
        if engine is not None:
            self._cb = SchedEngine(None, PREFILL_FN(lambda c, *a: engine["prefill"](*a)),
                                   DECODE_FN(lambda c, *a: engine["decode"](*a)),
                                   ALLOC_FN(lambda c, *a: engine["lane_alloc"](*a)),
                                   EVICT_FN(lambda c, *a: engine["lane_evict"](*a)))
            _check(lib().cbd_sched_create(ctypes.byref(b), ctypes.byref(self._cb), ctypes.byref(h)))
        else:
            model, arena, ws, logits, argmax, stream = device
            self._keep = device
            wsb = ws.numel() * ws.element_size()
            _check(lib().cbd_sched_create_device(ctypes.byref(b), model.h, arena.h, _ptr(ws), wsb, _ptr(logits),
                                                 _ptr(argmax), _stream(stream), ctypes.byref(h)))
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            lib().cbd_sched_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def submit(self, job_id: int, prompt, max_new: int) -> str:
        p = _i32(prompt)
        d = ctypes.c_int()
        _check(lib().cbd_sched_submit(self.h, int(job_id), _pi32(p), len(p), int(max_new), ctypes.byref(d)))
        return SCHED_DECISIONS[d.value]

    def tick(self) -> bool:
        w = ctypes.c_int()
        _check(lib().cbd_sched_tick(self.h, ctypes.byref(w)))
        return bool(w.value)

    def run(self, max_ticks: int = 1 << 40):
        _check(lib().cbd_sched_run(self.h, int(max_ticks)))

    def telemetry(self) -> dict:
        t = SchedTelemetry()
        _check(lib().cbd_sched_get_telemetry(self.h, ctypes.byref(t)))
        return {k: getattr(t, k) for k, _ in SchedTelemetry._fields_}

    def job_tokens(self, job_id: int):
        n, done = ctypes.c_int(), ctypes.c_int()
        _check(lib().cbd_sched_job_tokens(self.h, int(job_id), None, 0, ctypes.byref(n), ctypes.byref(done)))
        out = np.zeros(max(1, n.value), np.int32)
        _check(lib().cbd_sched_job_tokens(self.h, int(job_id), _pi32(out), n.value, ctypes.byref(n),
                                          ctypes.byref(done)))
        return out[:n.value].tolist(), bool(done.value)

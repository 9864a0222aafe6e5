"""ctypes binding of libla_pbd.so (include/la_pbd.h).

Argument marshalling only: every step of the PBD window step runs in the HIP
library.  torch supplies device memory and the current stream.  There is no
fallback: if the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_size_t, c_void_p
from typing import Optional

import torch

from . import synth

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libla_pbd.so")

LA_W_BF16, LA_W_INT4, LA_W_W8A8 = 0, 1, 2
_FMT = {"bf16": LA_W_BF16, "int4": LA_W_INT4, "w8a8": LA_W_W8A8}
LA_EPI_NONE, LA_EPI_SILU_GATE = 0, 1
LA_DERR_TOKEN_ID, LA_DERR_CAPACITY, LA_DERR_BLOCK_ID, LA_DERR_WINDOW = 1, 2, 4, 8
LA_LAYOUT_ROWS, LA_LAYOUT_TILED, LA_LAYOUT_TILED_GU, LA_LAYOUT_TILED_QKV = 0, 1, 2, 3
LA_MASK_BIDIRECTIONAL, LA_MASK_CAUSAL = 0, 1

EXPORTED = [
    "la_int4_embed_gather", "la_wgemm_workspace", "la_wgemm", "la_pbd_attention_workspace",
    "la_pbd_attention", "la_lm_head_argmax_workspace", "la_lm_head_argmax", "la_pbd_layer",
    "la_pbd_step_workspace", "la_pbd_step", "la_status_str", "la_pack_weight_bytes",
    "la_pack_weight", "la_packed_rows_bytes", "la_pack_rows", "la_wgemm_packed", "la_pbd_commit",
    "la_pbd_attention_masked", "la_pbd_attention_refeed", "la_pbd_step_refeed",
    "la_pbd_commit_refeed", "la_pbd_step_opts", "la_lm_head_argmax_penalized", "la_pbd_mark_tokens",
    "la_pbd_prefill_workspace", "la_pbd_prefill", "la_pbd_step_noalloc", "la_sample_logits",
]


class LaWeight(ctypes.Structure):
    _fields_ = [("fmt", c_int32), ("n", c_int32), ("k", c_int32), ("group", c_int32),
                ("layout", c_int32), ("reserved", c_int32), ("data", c_void_p), ("scales", c_void_p)]


class LaLayer(ctypes.Structure):
    _fields_ = [("in_norm", c_void_p), ("post_norm", c_void_p), ("qkv", LaWeight),
                ("qkv_bias", c_void_p), ("o", LaWeight), ("gate_up", LaWeight),
                ("down", LaWeight)]


class LaModel(ctypes.Structure):
    _fields_ = [("hidden", c_int32), ("n_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("inter", c_int32), ("n_layers", c_int32),
                ("vocab", c_int32), ("rms_eps", c_float), ("rope_theta", c_float),
                ("layers", POINTER(LaLayer)), ("embed", LaWeight), ("lm_head", LaWeight),
                ("final_norm", c_void_p), ("window_mask", c_int32)]


class LaKvCache(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("block_table", c_void_p),
                ("num_blocks", c_int32), ("max_blocks", c_int32), ("block_size", c_int32),
                ("n_layers", c_int32)]


class LaSampling(ctypes.Structure):
    _fields_ = [("temperature", c_float), ("top_p", c_float), ("seed", ctypes.c_uint64),
                ("offset", ctypes.c_uint64), ("offset_dev", c_void_p), ("logits", c_void_p)]


class LaStepOpts(ctypes.Structure):
    _fields_ = [("causal_rows", c_void_p), ("window_len", c_void_p), ("rep_bits", c_void_p),
                ("rep_words", c_int32), ("rep_penalty", c_float),
                ("sampling", POINTER(LaSampling)), ("block_events", c_void_p)]


class LaError(RuntimeError):
    pass


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libla_pbd.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise LaError(f"{_LIB_PATH} is missing: build it with box_decoding_amd.build.build()")
    lib = ctypes.CDLL(_LIB_PATH)
    W = POINTER(LaWeight)
    sig = {
        "la_int4_embed_gather": (c_int32, [c_void_p, c_int32, W, c_void_p, c_void_p, c_void_p]),
        "la_wgemm_workspace": (c_size_t, [c_int32, W, c_int32]),
        "la_wgemm": (c_int32, [c_void_p, c_int32, W, c_void_p, c_float, c_void_p, c_void_p, c_int32,
                               c_void_p, c_void_p, c_size_t, c_void_p]),
        "la_pbd_attention_workspace": (c_size_t, [c_int32] * 6),
        "la_pbd_attention": (c_int32, [c_void_p, POINTER(LaKvCache), c_int32, c_int32, c_int32,
                                       c_int32, c_void_p, c_int32, c_int32, c_int32, c_void_p,
                                       c_void_p, c_size_t, c_void_p]),
        "la_lm_head_argmax_workspace": (c_size_t, [c_int32, W]),
        "la_lm_head_argmax": (c_int32, [c_void_p, c_int32, W, c_void_p, c_float, c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
        "la_pbd_layer": (c_int32, [POINTER(LaModel), c_int32, POINTER(LaKvCache), c_void_p,
                                   c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                   c_void_p, c_size_t, c_void_p]),
        "la_pbd_step_workspace": (c_size_t, [POINTER(LaModel), c_int32, c_int32, c_int32]),
        "la_pbd_step": (c_int32, [POINTER(LaModel), POINTER(LaKvCache), c_void_p, c_void_p,
                                  c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                  c_void_p, c_size_t, c_void_p, c_void_p]),
        "la_status_str": (ctypes.c_char_p, [c_int32]),
        "la_pack_weight_bytes": (c_size_t, [W, c_int32, c_int32]),
        "la_pack_weight": (c_int32, [W, c_int32, c_void_p, c_void_p, c_void_p]),
        "la_packed_rows_bytes": (c_size_t, [c_int32, c_int32]),
        "la_pack_rows": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_float, c_int32, c_void_p,
                                   c_size_t, c_void_p]),
        "la_wgemm_packed": (c_int32, [c_void_p, c_int32, W, c_void_p, c_void_p, c_int32, c_void_p,
                                      c_void_p]),
        "la_pbd_commit": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                    c_void_p]),
        "la_pbd_attention_masked": (c_int32, [c_void_p, POINTER(LaKvCache), c_int32, c_int32,
                                              c_int32, c_int32, c_void_p, c_int32, c_int32,
                                              c_int32, c_int32, c_void_p, c_void_p, c_size_t,
                                              c_void_p]),
        "la_pbd_attention_refeed": (c_int32, [c_void_p, POINTER(LaKvCache), c_int32, c_int32,
                                              c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                              c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                              c_size_t, c_void_p]),
        "la_pbd_step_refeed": (c_int32, [POINTER(LaModel), POINTER(LaKvCache), c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_int32, c_int32, c_int32, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_size_t, c_void_p,
                                         c_void_p]),
        "la_pbd_commit_refeed": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                           c_void_p, c_int32, c_int32, c_int32, c_int32,
                                           c_void_p]),
        "la_pbd_step_opts": (c_int32, [POINTER(LaModel), POINTER(LaKvCache), c_void_p, c_void_p,
                                       POINTER(LaStepOpts), c_int32, c_int32, c_int32, c_void_p,
                                       c_void_p, c_void_p, c_void_p, c_size_t, c_void_p, c_void_p]),
        "la_lm_head_argmax_penalized": (c_int32, [c_void_p, c_int32, W, c_void_p, c_float, c_void_p,
                                                  c_int32, c_int32, c_float, c_void_p, c_void_p,
                                                  c_void_p, c_void_p, c_size_t, c_void_p]),
        "la_pbd_mark_tokens": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                         c_int32, c_int32, c_void_p]),
        "la_pbd_step_noalloc": (c_int32, [POINTER(LaModel), POINTER(LaKvCache), c_void_p, c_void_p,
                                          c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                          c_void_p, c_void_p]),
        "la_sample_logits": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_int32, c_int32,
                                       c_float, POINTER(LaSampling), c_void_p, c_void_p, c_void_p]),
        "la_pbd_prefill_workspace": (c_size_t, [POINTER(LaModel), c_int32, c_int32, c_int32]),
        "la_pbd_prefill": (c_int32, [POINTER(LaModel), POINTER(LaKvCache), c_void_p, c_void_p,
                                     c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_size_t, c_void_p, c_void_p]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != 0:
        msg = load().la_status_str(status).decode()
        raise LaError(f"{what} failed: {msg} ({status})")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else c_void_p(t.data_ptr())


def _stream():
    return c_void_p(torch.cuda.current_stream().cuda_stream)


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise LaError("every tensor handed to the library must live on the GPU")


def weight_desc(w: dict) -> LaWeight:
    if w is None:
        return LaWeight(LA_W_BF16, 0, 0, 0, 0, 0, None, None)
    fmt = _FMT[w["fmt"]]
    _require_cuda(w["data"], w.get("scales"))
    return LaWeight(fmt, int(w["n"]), int(w["k"]), int(w.get("group") or 0),
                    int(w.get("layout", LA_LAYOUT_ROWS)), 0, _ptr(w["data"]), _ptr(w.get("scales")))


def pack_weight(w: dict, layout: int) -> dict:
    """Tiled copy of a row-major weight (device memory from torch)."""
    lib = load()
    src = weight_desc(w)
    nd = lib.la_pack_weight_bytes(ctypes.byref(src), layout, 0)
    ns = lib.la_pack_weight_bytes(ctypes.byref(src), layout, 1)
    if nd == 0:
        raise LaError("la_pack_weight_bytes rejected the weight")
    dev = w["data"].device
    data = torch.empty(nd, dtype=torch.uint8, device=dev)
    scales = torch.empty(ns, dtype=torch.uint8, device=dev) if ns else None
    _check(lib.la_pack_weight(ctypes.byref(src), layout, _ptr(data), _ptr(scales), _stream()),
           "la_pack_weight")
    out = dict(w)
    out.update(data=data, scales=scales, layout=layout)
    return out


def pack_model(model: dict) -> dict:
    """Model dict whose linears and lm_head use the tiled layouts (the INT4
    group-32 embedding stays row-major: it is only gathered; a w8a8 model's
    bf16 embedding is tiled too, the gather reads either)."""
    out = dict(model)
    layers = []
    for lay in model["layers"]:
        nl = dict(lay)
        nl["qkv"] = pack_weight(lay["qkv"], LA_LAYOUT_TILED_QKV)
        nl["o"] = pack_weight(lay["o"], LA_LAYOUT_TILED)
        nl["gate_up"] = pack_weight(lay["gate_up"], LA_LAYOUT_TILED_GU)
        nl["down"] = pack_weight(lay["down"], LA_LAYOUT_TILED)
        layers.append(nl)
    out["layers"] = layers
    if model["wfmt"] in ("bf16", "w8a8"):
        out["embed"] = pack_weight(model["embed"], LA_LAYOUT_TILED)  # tied lm_head (bf16)
    if model["wfmt"] != "bf16":
        out["lm_head"] = pack_weight(model["lm_head"], LA_LAYOUT_TILED)
    return out


class Workspace:
    """Grow-only device workspace."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, nbytes: int) -> torch.Tensor:
        nbytes = max(int(nbytes), 256)
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self.buf


_default_ws = {}


def _ws(ws: Optional[Workspace]) -> Workspace:
    if ws is not None:
        return ws
    dev = torch.cuda.current_device()
    if dev not in _default_ws:
        _default_ws[dev] = Workspace(f"cuda:{dev}")
    return _default_ws[dev]


class DeviceModel:
    """A model dict (from synth.make_model, tensors on the GPU) plus its ABI struct."""

    def __init__(self, model: dict, causal_window: bool = False):
        # causal_window: window row j sees the prefix and window rows 0..j (the
        # RK3588 conversion's mask) instead of the whole window
        d: synth.ModelDims = model["dims"]
        self.model = model
        self.dims = d
        self.layers = (LaLayer * d.n_layers)()
        for i, lay in enumerate(model["layers"]):
            _require_cuda(lay["in_norm"], lay["post_norm"], lay.get("qkv_bias"))
            self.layers[i] = LaLayer(_ptr(lay["in_norm"]), _ptr(lay["post_norm"]),
                                     weight_desc(lay["qkv"]), _ptr(lay.get("qkv_bias")),
                                     weight_desc(lay["o"]), weight_desc(lay["gate_up"]),
                                     weight_desc(lay["down"]))
        self.struct = LaModel(d.hidden, d.n_heads, d.n_kv_heads, d.head_dim, d.inter, d.n_layers,
                              d.vocab, d.rms_eps, d.rope_theta,
                              ctypes.cast(self.layers, POINTER(LaLayer)),
                              weight_desc(model["embed"]), weight_desc(model.get("lm_head")),
                              _ptr(model["final_norm"]),
                              LA_MASK_CAUSAL if causal_window else LA_MASK_BIDIRECTIONAL)


class DeviceCache:
    """A paged cache dict (from synth.make_cache, tensors on the GPU) plus its ABI struct."""

    def __init__(self, cache: dict, n_layers: int):
        _require_cuda(cache["k"], cache["v"], cache["block_table"])
        self.cache = cache
        self.struct = LaKvCache(_ptr(cache["k"]), _ptr(cache["v"]), _ptr(cache["block_table"]),
                                int(cache["num_blocks"]), int(cache["max_blocks"]),
                                int(cache["block"]), int(n_layers))


# ---------------------------------------------------------------- entry points

def embed_gather(ids: torch.Tensor, emb: dict, err: Optional[torch.Tensor] = None) -> torch.Tensor:
    lib = load()
    _require_cuda(ids, err)
    ids = ids.to(torch.int32).contiguous().view(-1)
    out = torch.empty((ids.numel(), int(emb["k"])), dtype=torch.float32, device=ids.device)
    wd = weight_desc(emb)
    _check(lib.la_int4_embed_gather(_ptr(ids), ids.numel(), ctypes.byref(wd), _ptr(out), _ptr(err),
                                    _stream()), "la_int4_embed_gather")
    return out


def wgemm(x: torch.Tensor, w: dict, norm_gain=None, eps: float = 1e-6, bias=None, residual=None,
          silu_gate: bool = False, out: Optional[torch.Tensor] = None,
          ws: Optional[Workspace] = None) -> torch.Tensor:
    lib = load()
    _require_cuda(x, norm_gain, bias, residual)
    M = x.shape[0]
    wd = weight_desc(w)
    epi = LA_EPI_SILU_GATE if silu_gate else LA_EPI_NONE
    n_out = int(w["n"]) // 2 if silu_gate else int(w["n"])
    y = out if out is not None else torch.empty((M, n_out), dtype=torch.float32, device=x.device)
    need = lib.la_wgemm_workspace(M, ctypes.byref(wd), epi)
    buf = _ws(ws).get(need)
    _check(lib.la_wgemm(_ptr(x), M, ctypes.byref(wd), _ptr(norm_gain), eps, _ptr(bias),
                        _ptr(residual), epi, _ptr(y), _ptr(buf), buf.numel(), _stream()),
           "la_wgemm")
    return y


def pack_rows(x: torch.Tensor, fmt: str = "bf16", norm_gain=None, eps: float = 1e-6,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The packed matrix-core operand of x (RMSNorm'd when norm_gain is given)
    for a weight of format fmt, as a uint8 device buffer."""
    lib = load()
    _require_cuda(x, norm_gain)
    M, K = x.shape
    need = lib.la_packed_rows_bytes(M, K)
    if need == 0:
        raise LaError(f"no packed layout for M={M}, K={K}")
    buf = out if out is not None else torch.empty(need, dtype=torch.uint8, device=x.device)
    _check(lib.la_pack_rows(_ptr(x), M, K, _ptr(norm_gain), eps,
                            _FMT[fmt], _ptr(buf), buf.numel(),
                            _stream()), "la_pack_rows")
    return buf


def wgemm_packed(packed: torch.Tensor, M: int, w: dict, bias=None, residual=None,
                 silu_gate: bool = False, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """la_wgemm on an operand made by pack_rows."""
    lib = load()
    _require_cuda(packed, bias, residual)
    wd = weight_desc(w)
    n_out = int(w["n"]) // 2 if silu_gate else int(w["n"])
    y = out if out is not None else torch.empty((M, n_out), dtype=torch.float32,
                                                device=packed.device)
    _check(lib.la_wgemm_packed(_ptr(packed), M, ctypes.byref(wd), _ptr(bias), _ptr(residual),
                               LA_EPI_SILU_GATE if silu_gate else LA_EPI_NONE, _ptr(y), _stream()),
           "la_wgemm_packed")
    return y


def pbd_attention(q: torch.Tensor, cache: DeviceCache, layer: int, n_heads: int, n_kv_heads: int,
                  prefix_len: torch.Tensor, B: int, W: int, max_len: int,
                  ws: Optional[Workspace] = None, causal_window: bool = False,
                  causal_rows: Optional[torch.Tensor] = None,
                  window_len: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Window attention; causal_rows / window_len (int32 [B], both or neither)
    make it a re-fed window."""
    lib = load()
    _require_cuda(q, prefix_len, causal_rows, window_len)
    out = torch.empty_like(q)
    need = lib.la_pbd_attention_workspace(B, W, n_heads, n_kv_heads, 128, max_len)
    buf = _ws(ws).get(need)
    if causal_rows is not None or window_len is not None:
        _check(lib.la_pbd_attention_refeed(_ptr(q), ctypes.byref(cache.struct), layer, n_heads,
                                           n_kv_heads, 128, _ptr(prefix_len), _ptr(causal_rows),
                                           _ptr(window_len), B, W, max_len, _ptr(out), _ptr(buf),
                                           buf.numel(), _stream()), "la_pbd_attention_refeed")
    elif causal_window:
        _check(lib.la_pbd_attention_masked(_ptr(q), ctypes.byref(cache.struct), layer, n_heads,
                                           n_kv_heads, 128, _ptr(prefix_len), B, W, max_len,
                                           LA_MASK_CAUSAL, _ptr(out), _ptr(buf), buf.numel(),
                                           _stream()), "la_pbd_attention_masked")
    else:
        _check(lib.la_pbd_attention(_ptr(q), ctypes.byref(cache.struct), layer, n_heads, n_kv_heads,
                                    128, _ptr(prefix_len), B, W, max_len, _ptr(out), _ptr(buf),
                                    buf.numel(), _stream()), "la_pbd_attention")
    return out


def lm_head_argmax(h: torch.Tensor, lm: dict, norm_gain=None, eps: float = 1e-6,
                   ws: Optional[Workspace] = None, rep_bits: Optional[torch.Tensor] = None,
                   rep_rows: int = 1, rep_penalty: float = 1.0):
    """Tied lm_head argmax; rep_bits (int32 [rows / rep_rows, words], the
    vocabulary bitmaps) applies the repetition penalty."""
    lib = load()
    _require_cuda(h, norm_gain, rep_bits)
    M = h.shape[0]
    wd = weight_desc(lm)
    ids = torch.empty(M, dtype=torch.int32, device=h.device)
    top1 = torch.empty(M, dtype=torch.float32, device=h.device)
    gap = torch.empty(M, dtype=torch.float32, device=h.device)
    need = lib.la_lm_head_argmax_workspace(M, ctypes.byref(wd))
    buf = _ws(ws).get(need)
    if rep_bits is not None:
        _check(lib.la_lm_head_argmax_penalized(_ptr(h), M, ctypes.byref(wd), _ptr(norm_gain), eps,
                                               _ptr(rep_bits), rep_bits.shape[1], rep_rows,
                                               float(rep_penalty), _ptr(ids), _ptr(top1), _ptr(gap),
                                               _ptr(buf), buf.numel(), _stream()),
               "la_lm_head_argmax_penalized")
    else:
        _check(lib.la_lm_head_argmax(_ptr(h), M, ctypes.byref(wd), _ptr(norm_gain), eps, _ptr(ids),
                                     _ptr(top1), _ptr(gap), _ptr(buf), buf.numel(), _stream()),
               "la_lm_head_argmax")
    return ids, top1, gap


def pbd_layer(model: DeviceModel, layer: int, cache: DeviceCache, x: torch.Tensor,
              prefix_len: torch.Tensor, B: int, W: int, max_len: int, want_attn: bool = False,
              ws: Optional[Workspace] = None):
    lib = load()
    _require_cuda(x, prefix_len)
    d = model.dims
    y = torch.empty_like(x)
    attn = (torch.empty((B * W, d.n_heads * d.head_dim), dtype=torch.float32, device=x.device)
            if want_attn else None)
    need = lib.la_pbd_step_workspace(ctypes.byref(model.struct), B, W, max_len)
    if need == 0:
        raise LaError("la_pbd_step_workspace rejected the model or shape")
    buf = _ws(ws).get(need)
    _check(lib.la_pbd_layer(ctypes.byref(model.struct), layer, ctypes.byref(cache.struct), _ptr(x),
                            _ptr(prefix_len), B, W, max_len, _ptr(y), _ptr(attn), _ptr(buf),
                            buf.numel(), _stream()), "la_pbd_layer")
    return (y, attn) if want_attn else y


def step_workspace_bytes(model: DeviceModel, B: int, W: int, max_len: int) -> int:
    return int(load().la_pbd_step_workspace(ctypes.byref(model.struct), B, W, max_len))


class BlockEvents:
    """2 * n_layers HIP events for la_step_opts.block_events: the time of each
    layer's attention block in a step (ms() after the step has finished, and
    after a device synchronisation: the events are made for timing only,
    without the system-scope fence whose cache writeback and invalidation
    would add to the interval they bracket)."""

    _DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence

    def __init__(self, n_layers: int):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventElapsedTime.argtypes = [POINTER(c_float), c_void_p, c_void_p]
        self._hip.hipEventCreateWithFlags.argtypes = [POINTER(c_void_p), ctypes.c_uint]
        self.n = 2 * n_layers
        self.events = (c_void_p * self.n)()
        for i in range(self.n):
            h = c_void_p()
            if self._hip.hipEventCreateWithFlags(ctypes.byref(h), self._DISABLE_SYSTEM_FENCE) != 0:
                raise LaError("hipEventCreate failed")
            self.events[i] = h
        self.address = ctypes.addressof(self.events)

    def ms(self) -> list:
        """Elapsed milliseconds of each layer's attention block."""
        out = []
        for l in range(self.n // 2):
            t = c_float()
            if self._hip.hipEventElapsedTime(ctypes.byref(t), self.events[2 * l], self.events[2 * l + 1]) != 0:
                raise LaError("hipEventElapsedTime failed")
            out.append(t.value)
        return out

    def __del__(self):
        hip = getattr(self, "_hip", None)
        if hip is not None:
            for h in getattr(self, "events", []):
                if h:
                    hip.hipEventDestroy(c_void_p(h))


def pbd_step(model: DeviceModel, cache: DeviceCache, window_ids: torch.Tensor,
             prefix_len: torch.Tensor, max_len: int, want_gap: bool = True,
             want_hidden: bool = False, ws: Optional[Workspace] = None, out_ids=None, out_gap=None,
             err: Optional[torch.Tensor] = None, causal_rows: Optional[torch.Tensor] = None,
             window_len: Optional[torch.Tensor] = None, rep_bits: Optional[torch.Tensor] = None,
             rep_penalty: float = 1.0, sampling: Optional["Sampling"] = None,
             block_events: Optional["BlockEvents"] = None):
    """One PBD window step; returns (ids [B,W], gap [B,W] or None, hidden or None).
    causal_rows / window_len (int32 [B]) make it a re-fed window step; rep_bits
    (int32 [B, words] vocabulary bitmaps) applies the repetition penalty;
    sampling (a Sampling) replaces the argmax by the sampled selection (gap
    then holds the selected logit minus the row's largest); block_events (a
    BlockEvents) times every layer's attention block."""
    lib = load()
    _require_cuda(window_ids, prefix_len, err, causal_rows, window_len, rep_bits)
    B, W = window_ids.shape
    dev = window_ids.device
    ids = out_ids if out_ids is not None else torch.empty((B, W), dtype=torch.int32, device=dev)
    gap = out_gap if out_gap is not None else (
        torch.empty((B, W), dtype=torch.float32, device=dev) if want_gap else None)
    hid = (torch.empty((B * W, model.dims.hidden), dtype=torch.float32, device=dev)
           if want_hidden else None)
    need = lib.la_pbd_step_workspace(ctypes.byref(model.struct), B, W, max_len)
    if need == 0:
        raise LaError("la_pbd_step_workspace rejected the model or shape")
    buf = _ws(ws).get(need)
    if rep_bits is not None or sampling is not None or block_events is not None:
        smp = None
        if sampling is not None:
            smp = sampling.struct(B * W, model.dims.vocab, dev)
        if block_events is not None and block_events.n != 2 * model.dims.n_layers:
            raise LaError("block_events must hold 2 events per layer")
        opts = LaStepOpts(_ptr(causal_rows), _ptr(window_len), _ptr(rep_bits),
                          0 if rep_bits is None else rep_bits.shape[1], float(rep_penalty),
                          None if smp is None else ctypes.pointer(smp),
                          None if block_events is None else block_events.address)
        _check(lib.la_pbd_step_opts(ctypes.byref(model.struct), ctypes.byref(cache.struct),
                                    _ptr(window_ids), _ptr(prefix_len), ctypes.byref(opts), B, W,
                                    max_len, _ptr(ids), _ptr(gap), _ptr(hid), _ptr(buf), buf.numel(),
                                    _ptr(err), _stream()), "la_pbd_step_opts")
    elif causal_rows is not None or window_len is not None:
        _check(lib.la_pbd_step_refeed(ctypes.byref(model.struct), ctypes.byref(cache.struct),
                                      _ptr(window_ids), _ptr(prefix_len), _ptr(causal_rows),
                                      _ptr(window_len), B, W, max_len, _ptr(ids), _ptr(gap),
                                      _ptr(hid), _ptr(buf), buf.numel(), _ptr(err), _stream()),
               "la_pbd_step_refeed")
    else:
        _check(lib.la_pbd_step(ctypes.byref(model.struct), ctypes.byref(cache.struct),
                               _ptr(window_ids), _ptr(prefix_len), B, W, max_len, _ptr(ids),
                               _ptr(gap), _ptr(hid), _ptr(buf), buf.numel(), _ptr(err), _stream()),
               "la_pbd_step")
    return ids, gap, hid


def pbd_step_noalloc(model: DeviceModel, cache: DeviceCache, window_ids: torch.Tensor,
                     prefix_len: torch.Tensor, max_len: int, out_ids: torch.Tensor,
                     out_gap: Optional[torch.Tensor] = None, out_hidden: Optional[torch.Tensor] = None,
                     err: Optional[torch.Tensor] = None):
    """la_pbd_step_noalloc: the step on the library's own per-GPU scratch array
    (no workspace argument); outputs go to the caller's tensors."""
    lib = load()
    _require_cuda(window_ids, prefix_len, out_ids, out_gap, out_hidden, err)
    B, W = window_ids.shape
    _check(lib.la_pbd_step_noalloc(ctypes.byref(model.struct), ctypes.byref(cache.struct),
                                   _ptr(window_ids), _ptr(prefix_len), B, W, max_len, _ptr(out_ids),
                                   _ptr(out_gap), _ptr(out_hidden), _ptr(err), _stream()),
           "la_pbd_step_noalloc")


class Sampling:
    """Parameters of the sampled selection (la_sampling): temperature, top_p,
    seed, offset (or offset_dev, an int64 device word the call reads and then
    advances by 1); logits: the step's fp32 [rows, vocab] scratch (allocated on
    first use when not given; it holds the step's logits after a call)."""

    def __init__(self, temperature=0.7, top_p=0.9, seed=0, offset=0,
                 offset_dev: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None):
        self.temperature, self.top_p, self.seed, self.offset = temperature, top_p, seed, offset
        self.offset_dev, self.logits = offset_dev, logits
        self._keep = None

    def struct(self, rows: int = 0, vocab: int = 0, device=None) -> LaSampling:
        if rows and (self.logits is None or self.logits.numel() < rows * vocab):
            self.logits = torch.empty((rows, vocab), dtype=torch.float32, device=device)
        _require_cuda(self.offset_dev, self.logits)
        s = LaSampling(float(self.temperature), float(self.top_p), int(self.seed) & (2 ** 64 - 1),
                       int(self.offset) & (2 ** 64 - 1), _ptr(self.offset_dev), _ptr(self.logits))
        self._keep = s
        return s


def sample_logits(logits: torch.Tensor, sampling: Sampling, rep_bits: Optional[torch.Tensor] = None,
                  rep_rows: int = 1, rep_penalty: float = 1.0):
    """la_sample_logits: sampled ids [M] (and selected logit minus the row max) of logits [M, V]."""
    lib = load()
    _require_cuda(logits, rep_bits)
    M, V = logits.shape
    ids = torch.empty(M, dtype=torch.int32, device=logits.device)
    gap = torch.empty(M, dtype=torch.float32, device=logits.device)
    smp = sampling.struct()
    _check(lib.la_sample_logits(_ptr(logits), M, V, logits.stride(0), _ptr(rep_bits),
                                0 if rep_bits is None else rep_bits.shape[1], rep_rows,
                                float(rep_penalty), ctypes.byref(smp), _ptr(ids), _ptr(gap), _stream()),
           "la_sample_logits")
    return ids, gap


def pbd_commit(out_ids: torch.Tensor, window_ids: torch.Tensor, prefix_len: torch.Tensor,
               mask_id: int):
    """Commit a fully accepted window on the device: prefix_len += W and
    window_ids <- [out_ids[:, W-1], mask_id x (W-1)] (in place)."""
    lib = load()
    _require_cuda(out_ids, window_ids, prefix_len)
    B, W = window_ids.shape
    _check(lib.la_pbd_commit(_ptr(out_ids), _ptr(window_ids), _ptr(prefix_len), B, W, int(mask_id),
                             _stream()), "la_pbd_commit")


def pbd_commit_refeed(out_ids: torch.Tensor, window_ids: torch.Tensor, prefix_len: torch.Tensor,
                      causal_rows: torch.Tensor, window_len: torch.Tensor, block: int, mask_id: int,
                      n_accept: Optional[torch.Tensor] = None):
    """Commit of a re-fed window step on the device (in place): accept the
    first n_accept[b] block outputs (all when None), re-feed them, and open a
    new block of `block` rows."""
    lib = load()
    _require_cuda(out_ids, window_ids, prefix_len, causal_rows, window_len, n_accept)
    B, W = window_ids.shape
    _check(lib.la_pbd_commit_refeed(_ptr(out_ids), _ptr(n_accept), _ptr(window_ids),
                                    _ptr(prefix_len), _ptr(causal_rows), _ptr(window_len), B, W,
                                    int(block), int(mask_id), _stream()), "la_pbd_commit_refeed")


def pbd_prefill(model: DeviceModel, cache: DeviceCache, ids: torch.Tensor, prefix_len: torch.Tensor,
                max_len: int, embeds: Optional[torch.Tensor] = None, want_hidden: bool = False,
                ws: Optional[Workspace] = None, err: Optional[torch.Tensor] = None):
    """Prefill of ids [B, L] (negative ids take their row of embeds [B, L, H]);
    returns (first generated id [B], gap [B], last-row hidden [B, H] or None)."""
    lib = load()
    _require_cuda(ids, prefix_len, embeds, err)
    B, L = ids.shape
    dev = ids.device
    out = torch.empty(B, dtype=torch.int32, device=dev)
    gap = torch.empty(B, dtype=torch.float32, device=dev)
    hid = torch.empty((B, model.dims.hidden), dtype=torch.float32, device=dev) if want_hidden else None
    need = lib.la_pbd_prefill_workspace(ctypes.byref(model.struct), B, L, max_len)
    if need == 0:
        raise LaError("la_pbd_prefill_workspace rejected the model or shape")
    buf = _ws(ws).get(need)
    _check(lib.la_pbd_prefill(ctypes.byref(model.struct), ctypes.byref(cache.struct), _ptr(ids),
                              _ptr(embeds), _ptr(prefix_len), B, L, max_len, _ptr(out), _ptr(gap),
                              _ptr(hid), _ptr(buf), buf.numel(), _ptr(err), _stream()),
           "la_pbd_prefill")
    return out, gap, hid


def mark_tokens(ids: torch.Tensor, rep_bits: torch.Tensor, vocab: int,
                first: Optional[torch.Tensor] = None, count: Optional[torch.Tensor] = None):
    """Set the repetition-bitmap bits of the selected ids (in place, on the device)."""
    lib = load()
    _require_cuda(ids, rep_bits, first, count)
    B, W = ids.shape
    _check(lib.la_pbd_mark_tokens(_ptr(ids), B, W, _ptr(first), _ptr(count), _ptr(rep_bits),
                                  rep_bits.shape[1], int(vocab), _stream()), "la_pbd_mark_tokens")


def rep_words(vocab: int) -> int:
    return (vocab + 31) // 32


class StepGraph:
    """One la_pbd_step call captured in a HIP graph (torch.cuda.CUDAGraph) and
    replayed; inputs and outputs are the tensors given at capture time."""

    def __init__(self, model: DeviceModel, cache: DeviceCache, window_ids: torch.Tensor,
                 prefix_len: torch.Tensor, max_len: int, out_ids: torch.Tensor,
                 out_gap: Optional[torch.Tensor] = None, ws: Optional[Workspace] = None,
                 err: Optional[torch.Tensor] = None, commit_mask_id: Optional[int] = None,
                 refeed: Optional[tuple] = None):
        # commit_mask_id: also capture la_pbd_commit after the step, so each
        # replay is one step of an emission loop (the window and prefix
        # lengths advance on the device).  refeed = (causal_rows, window_len,
        # block, n_accept or None): re-fed window steps, committed with
        # la_pbd_commit_refeed when commit_mask_id is given.
        self.args = (model, cache, window_ids, prefix_len, max_len)
        self.commit_mask_id = commit_mask_id
        self.refeed = refeed
        self.ws = ws or Workspace(window_ids.device)
        self.out_ids, self.out_gap, self.err = out_ids, out_gap, err
        side = torch.cuda.Stream(device=window_ids.device)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self._call(commit=False)  # sizes the workspace before capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self._call()

    def _call(self, commit: bool = True):
        m, c, ids, P, ml = self.args
        cr, wl = (self.refeed[0], self.refeed[1]) if self.refeed else (None, None)
        pbd_step(m, c, ids, P, ml, want_gap=self.out_gap is not None, ws=self.ws,
                 out_ids=self.out_ids, out_gap=self.out_gap, err=self.err, causal_rows=cr,
                 window_len=wl)
        if commit and self.commit_mask_id is not None:
            if self.refeed:
                pbd_commit_refeed(self.out_ids, ids, P, cr, wl, self.refeed[2], self.commit_mask_id,
                                  self.refeed[3])
            else:
                pbd_commit(self.out_ids, ids, P, self.commit_mask_id)

    def replay(self):
        self.graph.replay()

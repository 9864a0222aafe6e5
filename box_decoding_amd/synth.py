"""Seeded synthetic inputs for the PBD window step.

This module only draws random numbers and packs them into the storage formats
the library reads.  It holds none of the step's arithmetic: both the HIP path and
the CPU oracle receive the same tensors from here and each decodes them on its
own.

Storage formats (the library's layouts):
  * bf16 tensors are uint16 bit patterns (round-to-nearest-even of fp32 draws).
  * INT4 tensors are nibble-packed uint8 ``[rows, k/2]`` with the low nibble
    holding the even element and the high nibble the odd one, plus fp16 scales
    ``[rows, k/group]`` stored as uint16 bit patterns (the ONNX WebGPU INT4 page,
    section on the embedding gather/dequant; group 32 for the embedding, group
    128 for the linears).
  * K cache pages are ``[layers, num_blocks, n_kv_heads, block, head_dim]`` and
    V cache pages ``[layers, num_blocks, n_kv_heads, head_dim, block]``
    (dim-major inside a page), both bf16, addressed through an int32 block
    table ``[batch, max_blocks]``.

Value recipes follow the workload descriptions: linear and embedding weights
~N(0, 0.02), norm gains 1 + N(0, 0.02), q/k/v biases ~N(0, 0.02), K/V cache
entries ~N(0, 1), INT4 codes uniform on 0..15 with scales uniform on
[0.005, 0.02].
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

# --------------------------------------------------------------------------
# Model shapes
# --------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class ModelDims:
    hidden: int = 2048
    n_heads: int = 16
    n_kv_heads: int = 2
    head_dim: int = 128
    inter: int = 11008
    n_layers: int = 36
    vocab: int = 152681
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    block: int = 16

    @property
    def qkv_out(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim


QWEN25_3B = ModelDims()


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: model shape, batch, window and prefix lengths."""
    name: str
    dims: ModelDims
    batch: int
    window: int
    prefix: tuple  # ("fixed", P) or ("uniform", lo, hi)
    wfmt: str = "bf16"  # "bf16", "int4" or "w8a8"
    steps: int = 1      # consecutive window steps (emission loop)
    lm_head: bool = True
    model_seed: int = 0
    input_seed: int = 1


WORKLOADS = {
    # One decoder layer, one window, batch 1, prefix 512.
    "layer_b1_p512": Workload("layer_b1_p512", dataclasses.replace(QWEN25_3B, n_layers=1),
                              batch=1, window=6, prefix=("fixed", 512), lm_head=False,
                              model_seed=10, input_seed=1),
    # Full 36-layer step + tied lm_head argmax, batch 1, prefix 1280.
    "step_b1_p1280": Workload("step_b1_p1280", QWEN25_3B, batch=1, window=6,
                              prefix=("fixed", 1280), model_seed=0, input_seed=2),
    # Batched step, 32 ragged sequences, prefix uniform in [300, 4096].
    "step_b32_ragged": Workload("step_b32_ragged", QWEN25_3B, batch=32, window=6,
                                prefix=("uniform", 300, 4096), model_seed=0, input_seed=3),
    # INT4 weight-only variant, batch 8, prefix 1280.
    "step_int4_b8_p1280": Workload("step_int4_b8_p1280", QWEN25_3B, batch=8, window=6,
                                   prefix=("fixed", 1280), wfmt="int4", model_seed=4,
                                   input_seed=4),
    # Dense-scene emission loop: batch 16, prefix 2048, 40 consecutive steps.
    "emit_b16_p2048_x40": Workload("emit_b16_p2048_x40", QWEN25_3B, batch=16, window=6,
                                   prefix=("fixed", 2048), steps=40, model_seed=0,
                                   input_seed=5),
    # w8a8 weights (int8 codes, per-channel scales, int8 activations per row),
    # the RK3588 conversion's format, at the batch-1 shape.
    "step_w8a8_b1_p1280": Workload("step_w8a8_b1_p1280", QWEN25_3B, batch=1, window=6,
                                   prefix=("fixed", 1280), wfmt="w8a8", model_seed=7,
                                   input_seed=2),
    # Long-context probe: batch 1, prefix 32768.
    "probe_b1_p32768": Workload("probe_b1_p32768", QWEN25_3B, batch=1, window=6,
                                prefix=("fixed", 32768), model_seed=0, input_seed=6),
}

# --------------------------------------------------------------------------
# Seeded draws
# --------------------------------------------------------------------------

_MASK64 = (1 << 64) - 1


def _mix(*parts: int) -> int:
    """Deterministic 63-bit seed from integer parts (splitmix64 finaliser)."""
    h = 0x9E3779B97F4A7C15
    for p in parts:
        h = (h ^ (int(p) & _MASK64)) & _MASK64
        h = (h + 0x9E3779B97F4A7C15) & _MASK64
        z = h
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        h = z ^ (z >> 31)
    return h & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_mix(*parts))
    return g


def _bits16(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16)


def normal_bf16(shape, std, mean, device, *seed) -> torch.Tensor:
    """bf16 bit patterns (int16 view) of mean + std * N(0,1) fp32 draws, RNE."""
    g = _gen(device, *seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    return _bits16(x.to(torch.bfloat16))


def int4_tensor(rows, k, group, device, *seed):
    """Nibble-packed INT4 codes uniform on 0..15 and fp16 scales on [0.005, 0.02]."""
    g = _gen(device, *seed)
    q = torch.randint(0, 16, (rows, k), generator=g, device=device, dtype=torch.uint8)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).contiguous()
    del q
    s = torch.rand((rows, k // group), generator=g, device=device, dtype=torch.float32)
    s = (0.005 + 0.015 * s).to(torch.float16)
    return packed, _bits16(s)


def int8_tensor(rows, k, device, *seed):
    """int8 codes uniform on -127..127 and one fp32 scale per row on
    [2e-4, 4e-4] (weights of about 0.02 standard deviation)."""
    g = _gen(device, *seed)
    q = torch.randint(-127, 128, (rows, k), generator=g, device=device, dtype=torch.int8)
    s = 2e-4 + 2e-4 * torch.rand((rows,), generator=g, device=device, dtype=torch.float32)
    return q, s


def _weight(fmt, n, k, device, *seed):
    if fmt == "bf16":
        return {"fmt": "bf16", "n": n, "k": k, "group": 0,
                "data": normal_bf16((n, k), 0.02, 0.0, device, *seed), "scales": None}
    if fmt == "w8a8":
        q, s = int8_tensor(n, k, device, *seed)
        return {"fmt": "w8a8", "n": n, "k": k, "group": 0, "data": q, "scales": s}
    packed, scales = int4_tensor(n, k, 128, device, *seed)
    return {"fmt": "int4", "n": n, "k": k, "group": 128, "data": packed, "scales": scales}


def make_model(dims: ModelDims, wfmt: str = "bf16", seed: int = 0, device="cpu",
               qkv_bias: bool = True) -> dict:
    """Random-init weights of the decoder.

    Layout per layer: ``qkv`` is [q | k | v] stacked along the output dim
    ([Hq*D + 2*Hkv*D, H]); ``gate_up`` is [gate | up] stacked ([2F, H]);
    ``o`` is [H, Hq*D]; ``down`` is [H, F].  The lm_head is tied to the
    embedding in bf16; in INT4 the embedding is a group-32 copy and the lm_head
    a group-128 copy of the tied matrix; in w8a8 the embedding stays bf16 and
    the lm_head is an int8 matrix with its own codes and per-row scales (it
    stands for the quantised copy of the tied matrix).
    """
    d = dims
    H, F = d.hidden, d.inter
    layers = []
    for l in range(d.n_layers):
        lay = {
            "in_norm": normal_bf16((H,), 0.02, 1.0, device, seed, l, 1),
            "post_norm": normal_bf16((H,), 0.02, 1.0, device, seed, l, 2),
            "qkv": _weight(wfmt, d.qkv_out, H, device, seed, l, 3),
            "qkv_bias": normal_bf16((d.qkv_out,), 0.02, 0.0, device, seed, l, 4) if qkv_bias else None,
            "o": _weight(wfmt, H, d.n_heads * d.head_dim, device, seed, l, 5),
            "gate_up": _weight(wfmt, 2 * F, H, device, seed, l, 6),
            "down": _weight(wfmt, H, F, device, seed, l, 7),
        }
        layers.append(lay)
    model = {"dims": d, "wfmt": wfmt, "layers": layers,
             "final_norm": normal_bf16((H,), 0.02, 1.0, device, seed, 1000, 1)}
    if wfmt in ("bf16", "w8a8"):
        model["embed"] = {"fmt": "bf16", "n": d.vocab, "k": H, "group": 0,
                          "data": normal_bf16((d.vocab, H), 0.02, 0.0, device, seed, 1000, 2),
                          "scales": None}
        model["lm_head"] = None  # tied: the embedding matrix itself
        if wfmt == "w8a8":
            q, s = int8_tensor(d.vocab, H, device, seed, 1000, 6)
            model["lm_head"] = {"fmt": "w8a8", "n": d.vocab, "k": H, "group": 0, "data": q, "scales": s}
    else:
        # Tied matrix: one set of INT4 codes, read with group-32 scales by the
        # gather and with group-128 scales by the lm_head.
        p, s = int4_tensor(d.vocab, H, 32, device, seed, 1000, 3)
        model["embed"] = {"fmt": "int4", "n": d.vocab, "k": H, "group": 32, "data": p, "scales": s}
        g = _gen(device, seed, 1000, 5)
        s128 = torch.rand((d.vocab, H // 128), generator=g, device=device, dtype=torch.float32)
        s128 = _bits16((0.005 + 0.015 * s128).to(torch.float16))
        model["lm_head"] = {"fmt": "int4", "n": d.vocab, "k": H, "group": 128, "data": p,
                            "scales": s128}
    return model


def draw_prefix_lens(w: Workload, device="cpu") -> torch.Tensor:
    g = _gen("cpu", w.input_seed, 1)
    if w.prefix[0] == "fixed":
        p = torch.full((w.batch,), int(w.prefix[1]), dtype=torch.int32)
    else:
        lo, hi = int(w.prefix[1]), int(w.prefix[2])
        p = torch.randint(lo, hi + 1, (w.batch,), generator=g, dtype=torch.int32)
    return p.to(device)


def make_cache(dims: ModelDims, prefix_lens, window: int, extra_tokens: int = 0,
               seed: int = 1, device="cpu", spare_blocks: int = 0, fill_all: bool = True) -> dict:
    """Paged bf16 K/V cache with a shuffled block table.

    Each sequence b gets ceil((P_b + window + extra_tokens) / block) blocks from a
    pool whose order is a seeded random permutation.  Every slot is filled with
    N(0,1) bf16 (slots at or beyond P_b hold values the step must overwrite or
    ignore).
    """
    d = dims
    bs = d.block
    P = [int(x) for x in torch.as_tensor(prefix_lens).cpu().tolist()]
    B = len(P)
    need = [-(-(p + window + extra_tokens) // bs) for p in P]
    max_blocks = max(need) if need else 1
    nb = sum(need) + spare_blocks
    g = _gen("cpu", seed, 2)
    perm = torch.randperm(nb, generator=g, dtype=torch.int64).to(torch.int32)
    table = torch.full((B, max_blocks), -1, dtype=torch.int32)
    off = 0
    for b in range(B):
        table[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
    kshape = (d.n_layers, nb, d.n_kv_heads, bs, d.head_dim)
    vshape = (d.n_layers, nb, d.n_kv_heads, d.head_dim, bs)
    if fill_all:
        k = normal_bf16(kshape, 1.0, 0.0, device, seed, 3)
        v = normal_bf16(vshape, 1.0, 0.0, device, seed, 4)
    else:
        k = torch.zeros(kshape, dtype=torch.int16, device=device)
        v = torch.zeros(vshape, dtype=torch.int16, device=device)
    return {"k": k, "v": v, "block_table": table.to(device), "block": bs,
            "num_blocks": nb, "max_blocks": max_blocks}


def draw_window_ids(batch: int, window: int, vocab: int, seed: int, mask_id: Optional[int] = None,
                    device="cpu") -> torch.Tensor:
    """Window ids [batch, window]: a uniform last-accepted id followed by mask ids.

    ``mask_id`` stands for the <text_mask> token, whose id the pages do not give;
    by default it is one fixed seeded id.  ``mask_id=-1`` draws every position
    uniformly instead.
    """
    g = _gen("cpu", seed, 5)
    ids = torch.randint(0, vocab, (batch, window), generator=g, dtype=torch.int32)
    if mask_id is None:
        mask_id = int(torch.randint(0, vocab, (1,), generator=_gen("cpu", 7, 7)).item())
    if mask_id >= 0:
        ids[:, 1:] = mask_id
    return ids.to(device)


def make_hidden(rows: int, hidden: int, seed: int, device="cpu") -> torch.Tensor:
    """fp32 hidden states ~N(0,1) (input of a single decoder layer)."""
    g = _gen(device, seed, 6)
    return torch.randn((rows, hidden), generator=g, device=device, dtype=torch.float32)


def make_workload(name_or_w, device="cpu", dims: Optional[ModelDims] = None) -> dict:
    """All inputs of a named workload: model, cache, window ids, prefix lengths."""
    w = WORKLOADS[name_or_w] if isinstance(name_or_w, str) else name_or_w
    d = dims or w.dims
    P = draw_prefix_lens(w)
    extra = (w.steps - 1) * w.window
    model = make_model(d, w.wfmt, w.model_seed, device)
    cache = make_cache(d, P, w.window, extra, seed=w.input_seed, device=device)
    ids = draw_window_ids(w.batch, w.window, d.vocab, w.input_seed, device=device)
    out = {"workload": w, "dims": d, "model": model, "cache": cache,
           "window_ids": ids, "prefix_len": P.to(device)}
    if not w.lm_head:
        out["hidden"] = make_hidden(w.batch * w.window, d.hidden, w.input_seed, device)
    return out


def to_numpy_tree(x):
    """Copy a nested dict/list of tensors to host numpy arrays (for the oracle)."""
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().numpy()
    if isinstance(x, dict):
        return {k: to_numpy_tree(v) for k, v in x.items()}
    if isinstance(x, list):
        return [to_numpy_tree(v) for v in x]
    return x

"""Plain, slow CPU oracle of the Parallel Box Decoding (PBD) window step.

TEST INFRASTRUCTURE ONLY (see the package docstring).  It shares no code with
the HIP path and imports nothing from it.

What it computes, step by step, in float64 numpy (``dtype`` can lower it to
float32), with every stored input decoded exactly:

* The window is the last accepted token followed by mask tokens; it sits at
  positions P..P+W-1 right after the cached prefix, and its rows attend to the
  whole cached prefix and to every row of the window (bidirectional inside the
  window).  Source: "LocateAnything-3B for RK3588 (RKLLM + RKNN)", section
  "How it differs from the original", item 1; "LocateAnything-3B on Jetson Orin
  Nano", Part 1 section 1.3 (a block mask instead of a strictly causal one).
* The decoder is a plain Qwen2 causal LM (Jetson page, Part 1 section 1.2):
  pre-RMSNorm, GQA attention with half-rotation RoPE and q/k/v biases, a
  SiLU-gated MLP, a final RMSNorm, and an lm_head tied to the input embedding
  ("LocateAnything-3B — ONNX WebGPU (INT4 + 4-bit embeddings)", section "Why
  this repo exists").  GQA K/V have 2 heads of 128 (same page, section
  "KV-cache graph for in-browser use").
* Group-wise symmetric INT4: element j of a row is (q_j - 8) * scale[j // g],
  q_j from the low nibble for even j and the high nibble for odd j (WebGPU
  page, section "Embedding gather / dequant (JS reference)"; g = 32 for the
  embedding; g = 128 along the input dim for the linears, section "Files").
* Greedy selection: the per-position argmax of the logits (Jetson page, Part 1
  section 1.4: temperature 0, no sampling), lowest index on exact ties.
* w8a8 weights, the RK3588 conversion's format ("LocateAnything-3B for RK3588
  (RKLLM + RKNN)", "Files" and "How it differs from the original", item 3,
  which name w8a8 and give no formula).  Read plainly: int8 weight codes with
  one fp32 scale per output channel; the activations entering each linear
  layer are quantised per row, s = max|x| / 127 and q = round-half-even(x / s)
  clamped to [-127, 127], decided in float32 (a zero row has s = 0, q = 0); the
  integer products are summed exactly and scaled by both scales.

Readings taken where the pages are silent (each is listed with its reason in
the design notes): one key bound P+W shared by every window row; the window's
K/V rounded to bf16 (round-to-nearest-even from the fp32 value) before
attention, as they are read back from a bf16 cache; RoPE inv_freq =
theta^(-2i/D) pairing dims i and i+D/2; attention scale 1/sqrt(D); SiLU(z) =
z / (1 + exp(-z)).

Pins (tests/test_oracle_pins.py): INT4 decode against hand-built rows in
tests/golden; window attention against a dense brute-force masked softmax and
torch SDPA; W=1 against textbook causal decode; bidirectionality; paging and
NaN-poisoned-slot invariance; RoPE, RMSNorm, SiLU closed forms; argmax ties
and gaps; structural special cases of the layer and of the whole step.
Whole-step agreement with the trained model: parity unpinned (no trained
weights exist here).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_to_float", "fp16_to_float", "round_to_bf16_bits", "int4_dequant", "decode_weight",
    "quantize_rows_int8", "linear",
    "embed_rows", "rmsnorm", "silu", "rope_angles", "rope_apply", "window_attention",
    "repetition_penalty", "logits_of",
    "cache_read", "decoder_layer", "lm_head_argmax", "pbd_step", "emission_commit", "pbd_emission_loop",
    "refeed_commit", "pbd_refeed_loop", "pbd_prefill",
]


def _dim(d, name):
    return d[name] if isinstance(d, dict) else getattr(d, name)


# ---------------------------------------------------------------------------
# Storage decoding (exact)
# ---------------------------------------------------------------------------

def bf16_to_float(bits, dtype=np.float64):
    """bf16 bit patterns (uint16/int16) -> float (exact: bf16 is the top half of fp32)."""
    u = np.asarray(bits).view(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(dtype)


def fp16_to_float(bits, dtype=np.float64):
    """IEEE fp16 bit patterns (uint16/int16) -> float (exact)."""
    return np.asarray(bits).view(np.uint16).view(np.float16).astype(dtype)


def round_to_bf16_bits(x):
    """Round values to bf16 bit patterns the way the fp32 kernel does.

    The value is first rounded to fp32, then to bf16 with round-to-nearest-even
    (the decision is taken in the kernel's precision, fp32).
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def int4_dequant(packed, scales, group, dtype=np.float64):
    """Group-wise symmetric INT4 -> float.

    packed: uint8 [..., k/2]; scales: fp16 bits [..., k/group].  Element j of a
    row has the 4-bit code q_j = (byte[j // 2] >> (4 * (j % 2))) & 0xF (the even
    element in the low nibble) and decodes to (q_j - 8) * scale[j // group]
    (WebGPU page, section "Embedding gather / dequant (JS reference)").
    """
    packed = np.asarray(packed).view(np.uint8)
    j = np.arange(2 * packed.shape[-1])
    q = (packed[..., j // 2].astype(np.int64) >> (4 * (j % 2))) & 0xF
    return (q - 8).astype(dtype) * fp16_to_float(scales, dtype)[..., j // group]


def decode_weight(w, rows=None, dtype=np.float64):
    """Decode a weight descriptor (bf16, INT4 or w8a8) to a float matrix [n, k]."""
    data = w["data"] if rows is None else w["data"][rows]
    if w["fmt"] == "bf16":
        return bf16_to_float(data, dtype)
    scales = w["scales"] if rows is None else w["scales"][rows]
    if w["fmt"] == "w8a8":
        return np.asarray(data).view(np.int8).astype(dtype) * np.asarray(scales, dtype=np.float32).astype(dtype)[:, None]
    return int4_dequant(data, scales, int(w["group"]), dtype)


def quantize_rows_int8(x):
    """Per-row symmetric int8 quantisation of activations (the w8a8 reading in
    the header), every decision in float32: s = max|x| / 127, q = round half to
    even of x / s (float32 division), clamped to [-127, 127]; a row of zeros
    gets s = 0 and q = 0.  Returns (q int64 [..., K], s float32 [...])."""
    x32 = np.asarray(x, dtype=np.float32)
    s = (np.max(np.abs(x32), axis=-1) / np.float32(127)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1)).astype(np.float32)
    q = np.rint((x32 / safe[..., None]).astype(np.float32))
    q = np.where(s[..., None] > 0, np.clip(q, -127, 127), 0)
    return q.astype(np.int64), s


def linear(x, w, rows=None, dtype=np.float64, quantize_acts=True):
    """x . W^T for a weight descriptor (rows: a subset of W's rows).  bf16 and
    INT4: the exactly decoded weight.  w8a8: the rows of x quantised to int8
    (quantize_rows_int8), the integer dot products summed exactly, then scaled
    by the row's scale and the output channel's scale; with quantize_acts
    False the activations stay unquantised (the decoded weight times x: the
    reference point for the format's own error)."""
    if w["fmt"] != "w8a8" or not quantize_acts:
        return np.asarray(x, dtype=dtype) @ decode_weight(w, rows=rows, dtype=dtype).T
    q, s = quantize_rows_int8(x)
    data = w["data"] if rows is None else w["data"][rows]
    sw = w["scales"] if rows is None else w["scales"][rows]
    # integer products summed in float64: every partial sum is an integer of
    # magnitude below 127 * 127 * K < 2^53, so the sum is exact in any order
    acc = q.astype(np.float64) @ np.asarray(data).view(np.int8).astype(np.float64).T
    return acc.astype(dtype) * s.astype(dtype)[..., None] * np.asarray(sw, dtype=np.float32).astype(dtype)


def embed_rows(ids, emb, dtype=np.float64):
    """x[t] = E[ids[t]] (bf16 row, or INT4 group-32 row dequantized)."""
    ids = np.asarray(ids).reshape(-1).astype(np.int64)
    return decode_weight(emb, rows=ids, dtype=dtype)


# ---------------------------------------------------------------------------
# Elementwise pieces
# ---------------------------------------------------------------------------

def rmsnorm(x, gain, eps):
    """x / sqrt(mean(x^2) + eps) * gain, over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gain


def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    return z / (1.0 + np.exp(-z))


def rope_angles(pos, head_dim, theta, dtype=np.float64):
    """Angles [len(pos), D/2]: pos * theta^(-2i/D), computed in float64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / head_dim)
    return (np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]).astype(dtype)


def rope_apply(x, ang):
    """Half-rotation RoPE on x [T, heads, D] with angles [T, D/2].

    (x_i, x_{i+D/2}) -> (x_i cos a_i - x_{i+D/2} sin a_i, x_{i+D/2} cos a_i + x_i sin a_i).
    """
    h = x.shape[-1] // 2
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# ---------------------------------------------------------------------------
# Attention over the paged cache
# ---------------------------------------------------------------------------

def cache_read(cache, layer, b, n, dtype=np.float64):
    """Token slots 0..n-1 of sequence b from the paged cache -> (K, V) [n, Hkv, D].

    K pages are [blocks, Hkv, block, D]; V pages are [blocks, Hkv, D, block].
    Slot t lives in block block_table[b, t // block] at offset t % block.
    """
    bs = int(cache["block"])
    t = np.arange(n)
    blk = np.asarray(cache["block_table"])[b, t // bs].astype(np.int64)
    off = t % bs
    kl = cache["k"][layer]
    vl = cache["v"][layer]
    k = kl[blk, :, off, :]            # [n, Hkv, D]
    v = vl[blk, :, :, off]            # [n, Hkv, D]
    return bf16_to_float(k, dtype), bf16_to_float(v, dtype)


def window_attention(q, k, v, dtype=np.float64, causal=False, causal_rows=0, window_len=None):
    """Attention of the W window rows over n keys (prefix + window).

    q: [W, Hq, D]; k, v: [n, Hkv, D] with the W window rows' keys last.  Every
    window row sees all n keys: the prefix is before it (causal) and the window
    is bidirectional.  Query head h reads KV head h // (Hq / Hkv).
    softmax(q.k / sqrt(D)) . v.

    causal=True is the causal window of the RK3588 conversion ("LocateAnything-3B
    for RK3588 (RKLLM + RKNN)", "How it differs from the original", item 1):
    window row j sees the prefix and window rows 0..j only, i.e. the first
    n - W + j + 1 keys.

    A re-fed window puts accepted tokens, attended causally, before the
    bidirectional block (the same page, same item: the accepted tokens are
    sent again with the mask tokens each step).  Its first ``causal_rows`` rows
    are the re-fed tokens: row j < causal_rows sees the prefix and window rows
    0..j.  The rows from causal_rows up to ``window_len`` (default W) are the
    block: each sees the prefix and window rows 0..window_len-1.  Rows at or
    past window_len are padding that no real row sees; they see what the block
    sees.  causal=True is causal_rows = W.
    """
    W, Hq, D = q.shape
    Hkv = k.shape[1]
    n = k.shape[0]
    P = n - W
    G = Hq // Hkv
    c = W if causal else int(causal_rows)
    w = W if window_len is None else int(window_len)
    assert 0 <= c <= W and 1 <= w <= W and P >= 0
    out = np.zeros((W, Hq, D), dtype=dtype)
    scale = 1.0 / np.sqrt(D)
    for h in range(Hq):
        kv = h // G
        s = (q[:, h, :] @ k[:, kv, :].T) * scale        # [W, n]
        for j in range(W):
            last = j if j < c else w - 1                 # the last window row row j sees
            s[j, P + last + 1:] = -np.inf
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, kv, :]
    return out


# ---------------------------------------------------------------------------
# Decoder layer, lm_head, step
# ---------------------------------------------------------------------------

def decoder_layer(h, lay, dims, cache, layer, prefix_len, window, dtype=np.float64, parts=None,
                  causal=False, causal_rows=None, window_len=None, window_kv=None, quantize_acts=True):
    """One decoder layer on the window rows of every sequence.

    h: [B*W, H] hidden states (row b*W + j is window position j of sequence b).
    causal_rows / window_len: per-sequence [B] re-fed rows and window lengths
    of a re-fed window (window_attention), None for the plain window.
    window_kv: None, or (k_bits, v_bits) [B*W, Hkv, D] bf16 bit patterns that
    the attention reads for the window rows in place of this layer's own
    rounding of k and v (to follow another implementation's rounding
    decisions; the window's K/V are then inputs, as the prefix's are).
    Returns (h_out, k_bits, v_bits) where k_bits/v_bits [B*W, Hkv, D] are the
    bf16 K/V this layer computes for slots P_b + j (its own rounding).  ``parts`` (a dict) receives
    intermediate values when given.  quantize_acts False: w8a8 linears take
    unquantised activations (see linear).
    """
    H = _dim(dims, "hidden")
    Hq = _dim(dims, "n_heads")
    Hkv = _dim(dims, "n_kv_heads")
    D = _dim(dims, "head_dim")
    F = _dim(dims, "inter")
    eps = float(_dim(dims, "rms_eps"))
    theta = float(_dim(dims, "rope_theta"))
    P = np.asarray(prefix_len).astype(np.int64)
    B = len(P)
    W = int(window)
    T = B * W
    assert h.shape == (T, H)

    a = rmsnorm(h, bf16_to_float(lay["in_norm"], dtype), eps)
    qkv = linear(a, lay["qkv"], dtype=dtype, quantize_acts=quantize_acts)
    if lay.get("qkv_bias") is not None:
        qkv = qkv + bf16_to_float(lay["qkv_bias"], dtype)
    q = qkv[:, :Hq * D].reshape(T, Hq, D)
    k = qkv[:, Hq * D:(Hq + Hkv) * D].reshape(T, Hkv, D)
    v = qkv[:, (Hq + Hkv) * D:].reshape(T, Hkv, D)

    pos = (P[:, None] + np.arange(W)[None, :]).reshape(-1)
    ang = rope_angles(pos, D, theta, dtype)
    q = rope_apply(q, ang)
    k = rope_apply(k, ang)
    k_bits = round_to_bf16_bits(k)
    v_bits = round_to_bf16_bits(v)
    kw = bf16_to_float(k_bits if window_kv is None else window_kv[0], dtype)
    vw = bf16_to_float(v_bits if window_kv is None else window_kv[1], dtype)

    o = np.zeros((T, Hq, D), dtype=dtype)
    for b in range(B):
        rows = slice(b * W, (b + 1) * W)
        kp, vp = cache_read(cache, layer, b, int(P[b]), dtype)
        kk = np.concatenate([kp, kw[rows]], axis=0)
        vv = np.concatenate([vp, vw[rows]], axis=0)
        o[rows] = window_attention(
            q[rows], kk, vv, dtype, causal=causal,
            causal_rows=0 if causal_rows is None else int(causal_rows[b]),
            window_len=None if window_len is None else int(window_len[b]))

    h1 = h + linear(o.reshape(T, Hq * D), lay["o"], dtype=dtype, quantize_acts=quantize_acts)
    a2 = rmsnorm(h1, bf16_to_float(lay["post_norm"], dtype), eps)
    gu = linear(a2, lay["gate_up"], dtype=dtype, quantize_acts=quantize_acts)
    m = silu(gu[:, :F]) * gu[:, F:]
    h2 = h1 + linear(m, lay["down"], dtype=dtype, quantize_acts=quantize_acts)
    if parts is not None:
        parts.update(q=q, k=k, v=v, attn=o.reshape(T, Hq * D), h_mid=h1, mlp=m, qkv=qkv)
    return h2, k_bits, v_bits


def repetition_penalty(z, theta):
    """A logit of a token already in the sequence, penalised: z / theta where
    z > 0, z * theta otherwise (theta > 1 lowers it either way).

    The Jetson page's generate call (Part 1 section 1.4) passes
    repetition_penalty=1.1 with greedy selection; the pages give no formula,
    and this is the plain one: the penalty divides a positive score and
    multiplies a negative one, so the token is always made less likely.
    """
    z = np.asarray(z)
    return np.where(z > 0, z / theta, z * theta)


def logits_of(f, lm, ids, dtype=np.float64, rep_sets=None, rep_penalty=1.0):
    """The logit f[t] . E[ids[t]] of one given vocabulary id per row (after the
    repetition penalty when rep_sets holds the id), for rows whose ranking is
    checked for validity rather than exactly."""
    f = np.asarray(f, dtype=dtype)
    ids = np.asarray(ids).reshape(-1).astype(np.int64)
    z = np.array([linear(f[t:t + 1], lm, rows=ids[t:t + 1], dtype=dtype)[0, 0] for t in range(len(ids))],
                 dtype=dtype)
    if rep_sets is not None:
        for t in range(len(ids)):
            if np.isin(ids[t], np.asarray(rep_sets[t])):
                z[t] = repetition_penalty(z[t], rep_penalty)
    return z


def lm_head_argmax(f, lm, chunk=8192, dtype=np.float64, rep_sets=None, rep_penalty=1.0):
    """Per-row argmax of f . E^T over the vocabulary, with top-1 and top-2 gap.

    Lowest index wins an exact tie.  gap = logit[id] - max_{v != id} logit[v].
    The vocabulary is processed in chunks only to bound memory.  rep_sets: one
    array of vocabulary ids per row (or None); those ids' logits go through
    repetition_penalty(., rep_penalty) before the ranking.
    """
    f = np.asarray(f, dtype=dtype)
    T = f.shape[0]
    V = int(lm["n"]) if "n" in lm else lm["data"].shape[0]
    best = np.full(T, -np.inf)
    best_id = np.full(T, -1, dtype=np.int64)
    second = np.full(T, -np.inf)
    sets = None
    if rep_sets is not None:
        sets = [np.unique(np.asarray(x, dtype=np.int64)) for x in rep_sets]
    for v0 in range(0, V, chunk):
        v1 = min(V, v0 + chunk)
        logits = linear(f, lm, rows=np.arange(v0, v1), dtype=dtype)   # [T, v1-v0]
        if sets is not None:
            for t in range(T):
                idx = sets[t][(sets[t] >= v0) & (sets[t] < v1)] - v0
                logits[t, idx] = repetition_penalty(logits[t, idx], rep_penalty)
        for t in range(T):
            row = logits[t]
            i = int(np.argmax(row))                    # first (lowest) index of the max
            top = row[i]
            rest = np.delete(row, i)
            sec = rest.max() if rest.size else -np.inf
            if top > best[t]:
                second[t] = max(best[t], sec)
                best[t] = top
                best_id[t] = v0 + i
            else:
                second[t] = max(second[t], top)
    return best_id, best, best - second


def pbd_step(model, cache, window_ids, prefix_len, dtype=np.float64, return_hidden=False,
             layers=None, causal=False, causal_rows=None, window_len=None, rep_sets=None,
             rep_penalty=1.0, input_embeds=None, window_kv=None):
    """One PBD window step for every sequence.

    window_ids [B, W] -> per-position argmax ids [B, W] and top-2 gaps [B, W].
    causal_rows / window_len [B] make it a re-fed window (window_attention).
    rep_sets: per sequence, the vocabulary ids already in it (or None); every
    row of the sequence ranks its logits with those penalised
    (repetition_penalty, rep_penalty).  input_embeds [B, W, H] (or None):
    rows whose id is negative take this row instead of an embedding row.
    window_kv: None, or per layer the (k_bits, v_bits) the attention reads for
    the window rows (decoder_layer).
    The step writes nothing into ``cache``; it returns the bf16 K/V it would
    store at slots P_b .. P_b+W-1 of each layer ("kv") and their values
    before the rounding ("kv_exact").
    """
    dims = model["dims"]
    ids = np.asarray(window_ids)
    B, W = ids.shape
    flat = ids.reshape(-1)
    h = embed_rows(np.where(flat < 0, 0, flat), model["embed"], dtype)
    if input_embeds is not None:
        emb_in = np.asarray(input_embeds, dtype=dtype).reshape(B * W, -1)
        h[flat < 0] = emb_in[flat < 0]
    kv, kv_exact = [], []
    n_layers = len(model["layers"]) if layers is None else layers
    for l in range(n_layers):
        parts = {}
        h, kb, vb = decoder_layer(h, model["layers"][l], dims, cache, l, prefix_len, W, dtype,
                                  parts=parts, causal=causal, causal_rows=causal_rows,
                                  window_len=window_len,
                                  window_kv=None if window_kv is None else window_kv[l])
        kv.append((kb, vb))
        kv_exact.append((parts["k"], parts["v"]))
    f = rmsnorm(h, bf16_to_float(model["final_norm"], dtype), float(_dim(dims, "rms_eps")))
    lm = model["lm_head"] if model.get("lm_head") is not None else model["embed"]
    row_sets = None if rep_sets is None else [rep_sets[t // W] for t in range(B * W)]
    out_ids, top1, gap = lm_head_argmax(f, lm, dtype=dtype, rep_sets=row_sets, rep_penalty=rep_penalty)
    res = {"ids": out_ids.reshape(B, W), "top1": top1.reshape(B, W), "gap": gap.reshape(B, W),
           "kv": kv, "kv_exact": kv_exact, "final": f}
    if return_hidden:
        res["hidden"] = h
    return res


def emission_commit(out_ids, prefix_len, mask_id):
    """The next window after a step whose window is accepted as it stands (no
    re-feeding): the prefix grows by W and the next window is [the last
    row's output, mask x (W-1)].  Returns (ids', P')."""
    out = np.asarray(out_ids)
    B, W = out.shape
    ids = np.full((B, W), mask_id, dtype=np.int32)
    ids[:, 0] = out[:, W - 1]
    return ids, np.asarray(prefix_len, dtype=np.int64) + W


def pbd_emission_loop(model, cache, window_ids, prefix_len, steps, mask_id, dtype=np.float64):
    """Consecutive window steps with every window accepted.

    After each step the window's K/V are stored at slots P_b..P_b+W-1, the
    prefix grows by W, and the next window is [last output id, mask x (W-1)].
    ``cache`` is copied, never modified.
    """
    c = {k: (np.array(v, copy=True) if isinstance(v, np.ndarray) else v) for k, v in cache.items()}
    ids = np.array(window_ids, copy=True)
    P = np.array(prefix_len, dtype=np.int64, copy=True)
    B, W = ids.shape
    bs = int(c["block"])
    outs = []
    for _ in range(steps):
        r = pbd_step(model, c, ids, P, dtype)
        outs.append(r["ids"])
        for l, (kb, vb) in enumerate(r["kv"]):
            for b in range(B):
                for j in range(W):
                    t = int(P[b]) + j
                    blk = int(c["block_table"][b, t // bs])
                    c["k"][l, blk, :, t % bs, :] = kb[b * W + j].view(np.int16)
                    c["v"][l, blk, :, :, t % bs] = vb[b * W + j].view(np.int16)
        ids, P = emission_commit(r["ids"], P, mask_id)
    return outs, P, c


def refeed_commit(out_ids, window_ids, prefix_len, causal_rows, window_len, block, mask_id,
                  n_accept=None):
    """The next re-fed window after a step of a decode loop that re-feeds what it accepts.

    Sequence b's block is rows c_b .. w_b - 1 of its window.  Window row i sits
    at position P_b + i and its argmax is read as the token after it, so the
    block's outputs are the tokens at P_b + c_b + 1 onwards.  The first n_b of
    them are accepted (all S_b = w_b - c_b when n_accept is None; n_b is clamped
    to 1 .. S_b).  Every row up to the block's first is then final, and the next
    window starts right after it, re-feeding the accepted tokens; the last of
    them opens a new block of ``block`` rows with block - 1 mask tokens:
        ids'_b = [out_b[c_b] .. out_b[c_b + n_b - 1], mask x (block - 1), mask ...]
        c'_b = n_b - 1,  w'_b = n_b + block - 1,  P'_b = P_b + c_b + 1.
    The window keeps its width W (w'_b <= W is required).  Source: "LocateAnything-3B
    for RK3588 (RKLLM + RKNN)", "How it differs from the original", item 1 (the
    accepted tokens and the mask tokens are sent each step, the cached common
    prefix is reused).  Returns (ids', P', c', w').
    """
    out = np.asarray(out_ids)
    B, W = np.asarray(window_ids).shape
    P = np.asarray(prefix_len, dtype=np.int64)
    c = np.asarray(causal_rows, dtype=np.int64)
    w = np.asarray(window_len, dtype=np.int64)
    ids = np.full((B, W), mask_id, dtype=np.int32)
    P2 = np.zeros(B, dtype=np.int64)
    c2 = np.zeros(B, dtype=np.int64)
    w2 = np.zeros(B, dtype=np.int64)
    for b in range(B):
        S = int(w[b] - c[b])
        n = S if n_accept is None else min(max(int(n_accept[b]), 1), S)
        assert n + block - 1 <= W
        ids[b, :n] = out[b, c[b]:c[b] + n]
        P2[b] = P[b] + c[b] + 1
        c2[b] = n - 1
        w2[b] = n + block - 1
    return ids, P2, c2, w2


def pbd_refeed_loop(model, cache, window_ids, prefix_len, causal_rows, window_len, steps, block,
                    mask_id, n_accept=None, dtype=np.float64):
    """Consecutive re-fed window steps (refeed_commit between them).

    After each step the K/V of every real window row (j < w_b) are stored at
    slots P_b + j; padding rows store nothing.  n_accept: None (accept every
    block output) or one [B] array per step.  ``cache`` is copied, never
    modified.  Returns (per-step ids, final (ids, P, c, w), cache).
    """
    cc = {k: (np.array(v, copy=True) if isinstance(v, np.ndarray) else v) for k, v in cache.items()}
    ids = np.array(window_ids, copy=True)
    P = np.array(prefix_len, dtype=np.int64, copy=True)
    c = np.array(causal_rows, dtype=np.int64, copy=True)
    w = np.array(window_len, dtype=np.int64, copy=True)
    B, W = ids.shape
    bs = int(cc["block"])
    outs = []
    for s in range(steps):
        r = pbd_step(model, cc, ids, P, dtype, causal_rows=c, window_len=w)
        outs.append(r["ids"])
        for l, (kb, vb) in enumerate(r["kv"]):
            for b in range(B):
                for j in range(int(w[b])):
                    t = int(P[b]) + j
                    blk = int(cc["block_table"][b, t // bs])
                    cc["k"][l, blk, :, t % bs, :] = kb[b * W + j].view(np.int16)
                    cc["v"][l, blk, :, :, t % bs] = vb[b * W + j].view(np.int16)
        ids, P, c, w = refeed_commit(r["ids"], ids, P, c, w, block, mask_id,
                                     None if n_accept is None else n_accept[s])
    return outs, (ids, P, c, w), cc


def pbd_prefill(model, cache, ids, prefix_len, input_embeds=None, dtype=np.float64):
    """Prefill of L prompt positions per sequence after a cached prefix of P_b.

    The prompt is the image tokens and the text: rows whose id is negative take
    their input row from input_embeds [B, L, H] (the vision encoder's features
    spliced in over the image-token positions: "LocateAnything-3B — ONNX
    WebGPU (INT4 + 4-bit embeddings)", sections "Why this repo exists" and
    "Embedding gather / dequant (JS reference)"), the others an embedding row.
    The prefill is the fixed cost before decoding in the Jetson page's latency
    breakdown (section 3.1).  Every row attends causally (a plain causal LM pass over
    the prompt: the re-fed window with every row causal).  Returns the argmax
    id, top-2 gap, top-1 logit, final hidden state and final-normed row of
    each sequence's last row, and the bf16 K/V of every row (as pbd_step).
    """
    ids = np.asarray(ids)
    B, L = ids.shape
    r = pbd_step(model, cache, ids, prefix_len, dtype, return_hidden=True, causal=True,
                 input_embeds=input_embeds)
    last = np.arange(B) * L + (L - 1)
    return {"ids": r["ids"][:, L - 1], "gap": r["gap"][:, L - 1], "top1": r["top1"][:, L - 1],
            "hidden": r["hidden"][last], "final": r["final"][last], "kv": r["kv"]}


"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a worked example from the pages
(tests/golden), a closed form, a textbook/library routine, an invariant of the
method, or brute force on a tiny input.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle as O
import oracle.sampling as OS
from box_decoding_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

TINY = synth.ModelDims(hidden=64, n_heads=4, n_kv_heads=2, head_dim=16, inter=96, n_layers=2,
                       vocab=300, rms_eps=1e-6, rope_theta=1e6, block=4)


def _np(x):
    return synth.to_numpy_tree(x)


# ---------------------------------------------------------------- INT4 / bf16 decode

def test_int4_golden_rows():
    g = json.load(open(os.path.join(GOLDEN, "int4_rows.json")))
    for row in g["rows"]:
        packed = np.array([int(b, 16) for b in row["bytes_hex"]], dtype=np.uint8)[None, :]
        scales = np.array([int(s, 16) for s in row["scales_fp16_hex"]], dtype=np.uint16)[None, :]
        assert np.array_equal(O.fp16_to_float(scales)[0], np.array(row["scales_value"]))
        got = O.int4_dequant(packed, scales, g["group"])[0]
        if "all" in row:
            exp = np.array(row["all"])
        else:
            exp = np.zeros(64)
            for j, val in row["nonzero"].items():
                exp[int(j)] = val
        assert np.array_equal(got, exp)


def test_int4_storage_sizes_match_page():
    # WebGPU page, "Files": packed table [152681, 1024] uint8 (~156 MB) and fp16
    # scales [152681, 64] (~19.5 MB) for a 2048-wide, group-32 embedding.
    V, H = 152681, 2048
    assert V * (H // 2) == 156_345_344
    assert V * (H // 32) * 2 == 19_543_168
    # Tied embedding: vocab x hidden in fp32 is ~1.25 GB ("Why this repo exists").
    assert V * H * 4 == 1_250_762_752
    d = synth.QWEN25_3B
    assert (d.vocab, d.hidden) == (V, H)
    # KV graph: 36 layers x (K, V) x [2 heads, 128] bf16 per token.
    assert d.n_layers * 2 * d.n_kv_heads * d.head_dim * 2 == 36_864


def test_int4_dequant_matches_synth_packing_roundtrip():
    # The decoder must invert the packer for every code: pack codes 0..15 in all
    # even/odd positions and read them back with unit scales (value q - 8).
    q = np.array([[a, b] for a in range(16) for b in range(16)], dtype=np.uint8).reshape(1, -1)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    ones = np.full((1, q.shape[1] // 32), 0x3C00, dtype=np.uint16)
    assert np.array_equal(O.int4_dequant(packed, ones, 32), q.astype(np.float64) - 8)


def test_bf16_rounding_textbook():
    for line in open(os.path.join(GOLDEN, "bf16_rne.txt")):
        if line.startswith("#") or not line.strip():
            continue
        _, f32hex, bfhex = line.split()
        f = np.array([int(f32hex, 16)], dtype=np.uint32).view(np.float32)
        assert int(O.round_to_bf16_bits(f)[0]) == int(bfhex, 16), line
    # library routine: torch's fp32 -> bf16 conversion is round-to-nearest-even
    x = torch.randn(100000, generator=torch.Generator().manual_seed(3)) * 10
    ref = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.round_to_bf16_bits(x.numpy()), ref)
    # decode is exact
    assert np.array_equal(O.bf16_to_float(ref), x.to(torch.bfloat16).double().numpy())


# ---------------------------------------------------------------- attention

def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _dense_bruteforce(q, k, v, mask, G):
    """Plain loops: masked softmax attention of every row over every allowed key."""
    N, Hq, D = q.shape
    out = np.zeros_like(q)
    for i in range(N):
        for h in range(Hq):
            kv = h // G
            scores = []
            for t in range(N):
                if mask[i, t]:
                    scores.append(sum(q[i, h, d] * k[t, kv, d] for d in range(D)) / math.sqrt(D))
                else:
                    scores.append(-math.inf)
            mx = max(scores)
            w = [math.exp(s - mx) if s != -math.inf else 0.0 for s in scores]
            z = sum(w)
            for d in range(D):
                out[i, h, d] = sum(w[t] * v[t, kv, d] for t in range(N)) / z
    return out


def _pbd_mask(P, W):
    """Dense mask of a prefix of P tokens followed by a W-token window.

    Prefix rows are causal; every window row sees the prefix and the whole window.
    """
    N = P + W
    m = np.zeros((N, N), dtype=bool)
    for i in range(N):
        for t in range(N):
            m[i, t] = (t <= i) if i < P else True
    return m


@pytest.mark.parametrize("P,W", [(0, 6), (5, 6), (13, 6), (9, 1), (7, 4)])
def test_window_attention_equals_dense_masked_bruteforce(P, W):
    Hq, Hkv, D = 4, 2, 8
    N = P + W
    q = _rand((N, Hq, D), 1)
    k = _rand((N, Hkv, D), 2)
    v = _rand((N, Hkv, D), 3)
    mask = _pbd_mask(P, W)
    ref = _dense_bruteforce(q, k, v, mask, Hq // Hkv)
    got = O.window_attention(q[P:], k, v)
    np.testing.assert_allclose(got, ref[P:], rtol=1e-12, atol=1e-12)
    # library routine: torch SDPA in float64 with the explicit boolean mask
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(np.repeat(k, Hq // Hkv, axis=1)).permute(1, 0, 2)[None]
    vt = torch.from_numpy(np.repeat(v, Hq // Hkv, axis=1)).permute(1, 0, 2)[None]
    sd = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask))
    np.testing.assert_allclose(got, sd[0].permute(1, 0, 2).numpy()[P:], rtol=1e-12, atol=1e-12)


def test_w1_is_textbook_causal_decode():
    Hq, Hkv, D, P = 4, 2, 16, 37
    N = P + 1
    q = _rand((N, Hq, D), 11)
    k = _rand((N, Hkv, D), 12)
    v = _rand((N, Hkv, D), 13)
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(np.repeat(k, 2, axis=1)).permute(1, 0, 2)[None]
    vt = torch.from_numpy(np.repeat(v, 2, axis=1)).permute(1, 0, 2)[None]
    sd = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    got = O.window_attention(q[P:], k, v)
    np.testing.assert_allclose(got[0], sd[0, :, -1, :].numpy(), rtol=1e-12, atol=1e-12)


def test_window_is_bidirectional():
    Hq, Hkv, D, P, W = 4, 2, 8, 10, 6
    N = P + W
    q = _rand((W, Hq, D), 21)
    k = _rand((N, Hkv, D), 22)
    v = _rand((N, Hkv, D), 23)
    base = O.window_attention(q, k, v)
    for j in range(W):
        k2, v2 = k.copy(), v.copy()
        k2[P + j] += 0.5
        v2[P + j] += 0.5
        pert = O.window_attention(q, k2, v2)
        # every window row, including rows before j, sees the changed key
        for r in range(W):
            assert np.abs(pert[r] - base[r]).max() > 1e-6
        # under a causal mask rows before j would not change (control)
        causal = np.tril(np.ones((N, N), dtype=bool))
        a = _dense_bruteforce(np.concatenate([np.zeros((P, Hq, D)), q]), k, v, causal, 2)
        b = _dense_bruteforce(np.concatenate([np.zeros((P, Hq, D)), q]), k2, v2, causal, 2)
        if j > 0:
            assert np.abs(a[P:P + j] - b[P:P + j]).max() == 0.0


@pytest.mark.parametrize("P,W", [(0, 6), (5, 6), (13, 6), (7, 4)])
def test_causal_window_equals_dense_causal_bruteforce(P, W):
    # the RK3588 page's causal window: a plain lower-triangular mask over prefix
    # and window together; brute force and torch SDPA's is_causal (a library
    # routine) fix it
    Hq, Hkv, D = 4, 2, 8
    N = P + W
    q = _rand((N, Hq, D), 61)
    k = _rand((N, Hkv, D), 62)
    v = _rand((N, Hkv, D), 63)
    ref = _dense_bruteforce(q, k, v, np.tril(np.ones((N, N), dtype=bool)), Hq // Hkv)
    got = O.window_attention(q[P:], k, v, causal=True)
    np.testing.assert_allclose(got, ref[P:], rtol=1e-12, atol=1e-12)
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(np.repeat(k, Hq // Hkv, axis=1)).permute(1, 0, 2)[None]
    vt = torch.from_numpy(np.repeat(v, Hq // Hkv, axis=1)).permute(1, 0, 2)[None]
    sd = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    np.testing.assert_allclose(got, sd[0].permute(1, 0, 2).numpy()[P:], rtol=1e-12, atol=1e-12)


def test_causal_window_special_cases():
    Hq, Hkv, D, P, W = 4, 2, 8, 10, 6
    N = P + W
    q = _rand((W, Hq, D), 71)
    k = _rand((N, Hkv, D), 72)
    v = _rand((N, Hkv, D), 73)
    causal = O.window_attention(q, k, v, causal=True)
    bidir = O.window_attention(q, k, v)
    # the last window row sees every key either way; the others differ
    np.testing.assert_array_equal(causal[W - 1], bidir[W - 1])
    assert np.abs(causal[0] - bidir[0]).max() > 1e-6
    # W = 1: the two masks are one
    np.testing.assert_array_equal(O.window_attention(q[:1], k[:P + 1], v[:P + 1], causal=True),
                                  O.window_attention(q[:1], k[:P + 1], v[:P + 1]))
    # changing window key j changes rows j.. only
    for j in range(1, W):
        k2, v2 = k.copy(), v.copy()
        k2[P + j] += 0.5
        v2[P + j] += 0.5
        pert = O.window_attention(q, k2, v2, causal=True)
        assert np.abs(pert[:j] - causal[:j]).max() == 0.0
        assert np.abs(pert[j] - causal[j]).max() > 1e-6


def test_equal_scores_give_mean_of_values():
    Hq, Hkv, D, n = 4, 2, 8, 9
    q = np.zeros((3, Hq, D))
    k = _rand((n, Hkv, D), 31)
    v = _rand((n, Hkv, D), 32)
    got = O.window_attention(q, k, v)
    for h in range(Hq):
        np.testing.assert_allclose(got[:, h, :], np.broadcast_to(v[:, h // 2, :].mean(0), (3, D)),
                                   rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- elementwise closed forms

def test_rope_closed_forms():
    D, theta = 16, 1e6
    x = _rand((1, 3, D), 41)
    # position 0 is the identity
    np.testing.assert_array_equal(O.rope_apply(x, O.rope_angles([0], D, theta)), x)
    # each (i, i + D/2) pair keeps its norm
    ang = O.rope_angles([12345], D, theta)
    y = O.rope_apply(x, ang)
    n0 = x[..., :D // 2] ** 2 + x[..., D // 2:] ** 2
    n1 = y[..., :D // 2] ** 2 + y[..., D // 2:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12)
    # the dot product depends only on the position difference
    q = _rand((1, 1, D), 42)
    k = _rand((1, 1, D), 43)

    def dot(p, pk):
        return float((O.rope_apply(q, O.rope_angles([p], D, theta)) *
                      O.rope_apply(k, O.rope_angles([pk], D, theta))).sum())
    assert abs(dot(100, 37) - dot(1100, 1037)) < 1e-10
    assert abs(dot(100, 37) - dot(37, 100)) > 1e-6
    # textbook RoPE frequencies (RoFormer): pair i turns by theta^(-2i/D) rad per
    # position; the pairing is (i, i + D/2)
    for i in (0, 1, D // 2 - 1):
        e = np.zeros((1, 1, D))
        e[0, 0, i] = 1.0
        w = theta ** (-2.0 * i / D)
        r = O.rope_apply(e, O.rope_angles([3], D, theta))
        assert abs(r[0, 0, i] - math.cos(3 * w)) < 1e-15
        assert abs(r[0, 0, i + D // 2] - math.sin(3 * w)) < 1e-15


def test_rmsnorm_constant_vector():
    g = 1.0 + _rand(32, 51, 0.02)
    for c in (3.0, -0.25, 1e-4):
        eps = 1e-6
        got = O.rmsnorm(np.full((1, 32), c), g, eps)
        np.testing.assert_allclose(got[0], np.sign(c) * g / np.sqrt(1.0 + eps / c ** 2), rtol=1e-14)


def test_silu_library_and_limits():
    z = np.linspace(-30, 30, 2001)
    np.testing.assert_allclose(O.silu(z), z * expit(z), rtol=1e-13, atol=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(O.silu(-z), O.silu(z) - z, atol=1e-12)


# ---------------------------------------------------------------- argmax / gap

def test_lm_head_argmax_planted_max_tie_and_gap():
    rng = np.random.default_rng(61)
    V, H = 20000, 8
    E = rng.standard_normal((V, H)) * 0.02
    E[:, 0] = 0.0
    E[777, 0] = 5.0          # planted maximum for row 0
    E[123, 1] = 9.0          # planted tie for row 1 ...
    E[18001, 1] = 9.0        # ... across two vocab chunks: lowest index wins
    E[4100, 2] = 7.0         # planted tie inside one vocab chunk
    E[4200, 2] = 7.0
    bits = O.round_to_bf16_bits(E)
    lm = {"fmt": "bf16", "n": V, "data": bits}
    f = np.zeros((3, H))
    f[0, 0] = 1.0
    f[1, 1] = 1.0
    f[2, 2] = 1.0
    f2 = np.zeros((1, H))
    f2[0] = rng.standard_normal(H)
    f = np.concatenate([f, f2])
    ids, top1, gap = O.lm_head_argmax(f, lm, chunk=8192)
    assert ids[0] == 777 and ids[1] == 123 and ids[2] == 4100
    assert gap[1] == 0.0 and gap[2] == 0.0
    logits = f @ O.bf16_to_float(bits).T
    for t in range(4):
        s = np.sort(logits[t])[::-1]
        assert top1[t] == s[0]
        assert gap[t] == s[0] - s[1]
        assert ids[t] == int(np.flatnonzero(logits[t] == s[0])[0])


# ---------------------------------------------------------------- layer structure

def _tiny_setup(P_list=(5, 9), W=3, seed=0, dims=TINY):
    model = _np(synth.make_model(dims, "bf16", seed))
    model["dims"] = dims
    cache = _np(synth.make_cache(dims, torch.tensor(P_list), W, seed=seed + 1))
    h = np.random.default_rng(seed).standard_normal((len(P_list) * W, dims.hidden))
    return model, cache, h


def _zero_like_weight(w):
    if w["fmt"] == "int4":  # code 8 decodes to zero
        return {**w, "data": np.full_like(w["data"], 0x88)}
    return {**w, "data": np.zeros_like(w["data"])}


def test_layer_with_zero_weights_is_identity():
    model, cache, h = _tiny_setup()
    lay = dict(model["layers"][0])
    for name in ("qkv", "o", "gate_up", "down"):
        lay[name] = _zero_like_weight(lay[name])
    out, _, _ = O.decoder_layer(h, lay, TINY, cache, 0, [5, 9], 3)
    np.testing.assert_array_equal(out, h)


def test_layer_gqa_head_mapping_and_value_slice():
    # q = k = 0 (uniform attention); every cached and window value of kv head 0 is
    # c0 and of kv head 1 is c1; with W_o = I the attention output of query head h
    # is c_{h // 2} on all its dims, and the MLP is off.
    d = TINY
    model, cache, h = _tiny_setup()
    lay = dict(model["layers"][0])
    c0, c1 = 0.5, -1.25
    lay["qkv"] = _zero_like_weight(lay["qkv"])
    bias = np.zeros(d.qkv_out)
    bias[(d.n_heads + d.n_kv_heads) * d.head_dim:][:d.head_dim] = c0
    bias[(d.n_heads + d.n_kv_heads) * d.head_dim:][d.head_dim:] = c1
    lay["qkv_bias"] = O.round_to_bf16_bits(bias)
    lay["o"] = {"fmt": "bf16", "data": O.round_to_bf16_bits(np.eye(d.hidden))}
    lay["down"] = _zero_like_weight(lay["down"])
    cache = dict(cache)
    v = np.array(cache["v"])
    v[0, :, 0] = O.round_to_bf16_bits(np.full(v[0, :, 0].shape, c0)).view(np.int16)
    v[0, :, 1] = O.round_to_bf16_bits(np.full(v[0, :, 1].shape, c1)).view(np.int16)
    cache["v"] = v
    out, _, vb = O.decoder_layer(h, lay, d, cache, 0, [5, 9], 3)
    expect = np.concatenate([np.full(d.head_dim * 2, c0), np.full(d.head_dim * 2, c1)])
    np.testing.assert_allclose(out - h, np.broadcast_to(expect, h.shape), rtol=0, atol=1e-14)
    assert np.all(O.bf16_to_float(vb)[:, 0] == c0) and np.all(O.bf16_to_float(vb)[:, 1] == c1)


def test_layer_single_key_attention_returns_value():
    # P = 0 and W = 1: the only key is the token itself, softmax is 1, so the
    # attention output of head h is the bf16-rounded value of kv head h // G, and
    # RoPE at position 0 leaves q, k unchanged.
    d = TINY
    model, cache, h = _tiny_setup(P_list=(0,), W=1, seed=3)
    lay = model["layers"][0]
    parts = {}
    O.decoder_layer(h, lay, d, cache, 0, [0], 1, parts=parts)
    a = O.rmsnorm(h, O.bf16_to_float(lay["in_norm"]), d.rms_eps)
    Wqkv = O.bf16_to_float(lay["qkv"]["data"])
    bq = O.bf16_to_float(lay["qkv_bias"])
    HqD, HkvD = d.n_heads * d.head_dim, d.n_kv_heads * d.head_dim
    v = a @ Wqkv[HqD + HkvD:].T + bq[HqD + HkvD:]
    q = a @ Wqkv[:HqD].T + bq[:HqD]
    vr = O.bf16_to_float(O.round_to_bf16_bits(v)).reshape(1, d.n_kv_heads, d.head_dim)
    np.testing.assert_allclose(parts["attn"].reshape(1, d.n_heads, d.head_dim),
                               np.repeat(vr, d.n_heads // d.n_kv_heads, axis=1), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(parts["q"].reshape(1, -1), q, rtol=1e-13, atol=1e-14)


def test_mlp_gate_up_order_and_down_mapping():
    # Attention branch off (W_o = 0) and h constant c, so the post-norm input is
    # a = g / sqrt(1 + eps/c^2) exactly.  With W_gate = diag(alpha), W_up =
    # diag(beta) and W_down = I, the layer adds silu(alpha*a) * (beta*a); swapping
    # gate and up, or misplacing the down columns, changes it.
    d = synth.ModelDims(hidden=16, n_heads=2, n_kv_heads=1, head_dim=8, inter=16, n_layers=1,
                        vocab=40, block=4)
    model, cache, _ = _tiny_setup(P_list=(3,), W=2, seed=5, dims=d)
    lay = dict(model["layers"][0])
    lay["o"] = _zero_like_weight(lay["o"])
    c = 2.0
    h = np.full((2, d.hidden), c)
    g = O.bf16_to_float(lay["post_norm"])
    s = 1.0 / math.sqrt(1.0 + d.rms_eps / c ** 2)
    alpha = np.linspace(-3, 3, d.inter)
    beta = np.linspace(0.5, 2.0, d.inter)
    Wg = np.zeros((d.inter, d.hidden))
    Wu = np.zeros((d.inter, d.hidden))
    for i in range(d.inter):
        Wg[i, i] = 1.0
        Wu[i, i] = 1.0
    lay["gate_up"] = {"fmt": "bf16", "data": O.round_to_bf16_bits(np.concatenate([Wg, Wu]))}
    lay["down"] = {"fmt": "bf16", "data": O.round_to_bf16_bits(np.eye(d.hidden, d.inter))}
    out, _, _ = O.decoder_layer(h, lay, d, cache, 0, [3], 2)
    a = g * s
    np.testing.assert_allclose(out - h, np.broadcast_to(a * expit(a) * a, out.shape), rtol=1e-12)
    # swap gate and up rows: the result must differ (order matters)
    Wg2 = Wg * alpha[:, None]
    Wu2 = Wu * beta[:, None]
    lay["gate_up"] = {"fmt": "bf16", "data": O.round_to_bf16_bits(np.concatenate([Wg2, Wu2]))}
    out2, _, _ = O.decoder_layer(h, lay, d, cache, 0, [3], 2)
    ag = O.bf16_to_float(O.round_to_bf16_bits(alpha)) * a
    bu = O.bf16_to_float(O.round_to_bf16_bits(beta)) * a
    np.testing.assert_allclose(out2 - h, np.broadcast_to(ag * expit(ag) * bu, out.shape), rtol=1e-12)


def test_paging_and_poisoned_slots_do_not_change_layer():
    d = TINY
    model, cache, h = _tiny_setup(P_list=(6, 11), W=3, seed=7)
    ref, kb, vb = O.decoder_layer(h, model["layers"][1], d, cache, 1, [6, 11], 3)
    # the same logical tokens under another block permutation, with every slot
    # at or beyond P_b (and all spare blocks) poisoned with NaN
    bs = cache["block"]
    L, nb = cache["k"].shape[:2]
    nb2 = nb + 5
    rng = np.random.default_rng(9)
    perm = rng.permutation(nb2)
    nan16 = np.uint16(0x7FC0).view(np.int16)
    k2 = np.full((L, nb2) + cache["k"].shape[2:], nan16, dtype=np.int16)
    v2 = np.full((L, nb2) + cache["v"].shape[2:], nan16, dtype=np.int16)
    table2 = np.full_like(cache["block_table"], -1)
    for b, P in enumerate((6, 11)):
        for t in range(P):
            ob = cache["block_table"][b, t // bs]
            nbk = perm[b * 5 + t // bs]
            table2[b, t // bs] = nbk
            k2[:, nbk, :, t % bs, :] = cache["k"][:, ob, :, t % bs, :]
            v2[:, nbk, :, :, t % bs] = cache["v"][:, ob, :, :, t % bs]
    cache2 = {**cache, "k": k2, "v": v2, "block_table": table2}
    out, kb2, vb2 = O.decoder_layer(h, model["layers"][1], d, cache2, 1, [6, 11], 3)
    np.testing.assert_array_equal(out, ref)
    np.testing.assert_array_equal(kb2, kb)


# ---------------------------------------------------------------- whole step

@pytest.mark.parametrize("wfmt", ["bf16", "int4"])
def test_step_with_identity_layers_returns_input_ids(wfmt):
    # With every layer's weights zero the layers are the identity, so the final
    # hidden state of a position is its own (dequantized) embedding row, and the
    # tied lm_head scores that row highest: the step returns the window ids.
    d = synth.ModelDims(hidden=256, n_heads=4, n_kv_heads=2, head_dim=64, inter=128, n_layers=2,
                        vocab=700, block=16)
    model = _np(synth.make_model(d, wfmt, 11))
    model["dims"] = d
    for lay in model["layers"]:
        for name in ("qkv", "o", "gate_up", "down"):
            lay[name] = _zero_like_weight(lay[name])
    cache = _np(synth.make_cache(d, torch.tensor([20, 33]), 6, seed=12))
    ids = synth.draw_window_ids(2, 6, d.vocab, 13, mask_id=-1).numpy()
    r = O.pbd_step(model, cache, ids, [20, 33])
    np.testing.assert_array_equal(r["ids"], ids)
    assert np.all(r["gap"] > 0)


def test_oracle_float32_tracks_float64():
    # Self-consistency of the precision switch (not a pin): the float32 run of a
    # tiny 2-layer step stays close to the float64 run.
    model, cache, _ = _tiny_setup(P_list=(5, 9), W=3, seed=17)
    ids = synth.draw_window_ids(2, 3, TINY.vocab, 19, mask_id=-1).numpy()
    r64 = O.pbd_step(model, cache, ids, [5, 9], return_hidden=True)
    r32 = O.pbd_step(model, cache, ids, [5, 9], dtype=np.float32, return_hidden=True)
    rel = np.linalg.norm(r32["hidden"] - r64["hidden"]) / np.linalg.norm(r64["hidden"])
    assert rel < 1e-5


def test_emission_loop_commits_window_kv():
    model, cache, _ = _tiny_setup(P_list=(5, 9), W=3, seed=23)
    # room for two windows per sequence
    cache = _np(synth.make_cache(TINY, torch.tensor([5, 9]), 3, extra_tokens=3, seed=24))
    ids = synth.draw_window_ids(2, 3, TINY.vocab, 25).numpy()
    outs, P, c2 = O.pbd_emission_loop(model, cache, ids, [5, 9], 2, mask_id=int(ids[0, 1]))
    assert list(P) == [11, 15]
    r0 = O.pbd_step(model, cache, ids, [5, 9])
    np.testing.assert_array_equal(outs[0], r0["ids"])
    bs = cache["block"]
    for l, (kb, vb) in enumerate(r0["kv"]):
        for b, p in enumerate((5, 9)):
            for j in range(3):
                t = p + j
                blk = cache["block_table"][b, t // bs]
                assert np.array_equal(c2["k"][l, blk, :, t % bs, :].view(np.uint16), kb[b * 3 + j])
                assert np.array_equal(c2["v"][l, blk, :, :, t % bs].view(np.uint16), vb[b * 3 + j])
    # the second step reads the committed window as prefix
    nxt = np.full((2, 3), int(ids[0, 1]), dtype=np.int32)
    nxt[:, 0] = r0["ids"][:, 2]
    r1 = O.pbd_step(model, c2, nxt, [8, 12])
    np.testing.assert_array_equal(outs[1], r1["ids"])


# ---------------------------------------------------------------- re-fed window

def _sdpa(q, k, v, G, is_causal=False):
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(np.repeat(k, G, axis=1)).permute(1, 0, 2)[None]
    vt = torch.from_numpy(np.repeat(v, G, axis=1)).permute(1, 0, 2)[None]
    sd = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=is_causal)
    return sd[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("P,W,c,w", [(0, 6, 0, 6), (5, 11, 5, 11), (13, 11, 2, 8), (7, 16, 10, 16),
                                     (9, 8, 3, 3), (4, 12, 0, 6)])
def test_refeed_window_rows_match_library_attention(P, W, c, w):
    # re-fed rows are ordinary causal decode rows (torch SDPA is_causal over the
    # whole sequence); block rows attend, unmasked, to every key before the
    # window's end P + w (torch SDPA without a mask over those keys)
    Hq, Hkv, D = 4, 2, 8
    N = P + W
    q = _rand((N, Hq, D), 81)
    k = _rand((N, Hkv, D), 82)
    v = _rand((N, Hkv, D), 83)
    got = O.window_attention(q[P:], k, v, causal_rows=c, window_len=w)
    causal = _sdpa(q, k, v, Hq // Hkv, is_causal=True)
    for j in range(c):
        np.testing.assert_allclose(got[j], causal[P + j], rtol=1e-12, atol=1e-12)
    block = _sdpa(q[P + c:P + w], k[:P + w], v[:P + w], Hq // Hkv)
    np.testing.assert_allclose(got[c:w], block, rtol=1e-12, atol=1e-12)
    # padding rows' keys and values never reach a real row
    k2, v2 = k.copy(), v.copy()
    k2[P + w:] = 1e3 * _rand(k2[P + w:].shape, 84)
    v2[P + w:] = 1e3 * _rand(v2[P + w:].shape, 85)
    got2 = O.window_attention(q[P:], k2, v2, causal_rows=c, window_len=w)
    np.testing.assert_array_equal(got2[:w], got[:w])


def test_refeed_window_special_cases_and_locality():
    Hq, Hkv, D, P, W = 4, 2, 8, 10, 11
    N = P + W
    q = _rand((W, Hq, D), 91)
    k = _rand((N, Hkv, D), 92)
    v = _rand((N, Hkv, D), 93)
    # no re-fed rows is the PBD window; every row re-fed is the causal window
    np.testing.assert_array_equal(O.window_attention(q, k, v, causal_rows=0),
                                  O.window_attention(q, k, v))
    np.testing.assert_array_equal(O.window_attention(q, k, v, causal_rows=W),
                                  O.window_attention(q, k, v, causal=True))
    c = 5
    base = O.window_attention(q, k, v, causal_rows=c)
    for j in range(W):
        k2, v2 = k.copy(), v.copy()
        k2[P + j] += 0.5
        v2[P + j] += 0.5
        pert = O.window_attention(q, k2, v2, causal_rows=c)
        changed = [bool(np.abs(pert[r] - base[r]).max() > 1e-9) for r in range(W)]
        # a re-fed row sees the rows up to its own; a block row sees them all
        assert changed == [(r >= j) if r < c else True for r in range(W)]


def _store_kv(cache, kv, P, B, W, real_rows):
    bs = int(cache["block"])
    for l, (kb, vb) in enumerate(kv):
        for b in range(B):
            for j in range(real_rows[b]):
                t = int(P[b]) + j
                blk = int(cache["block_table"][b, t // bs])
                cache["k"][l, blk, :, t % bs, :] = kb[b * W + j].view(np.int16)
                cache["v"][l, blk, :, :, t % bs] = vb[b * W + j].view(np.int16)


def test_refeed_step_equals_token_by_token_decode():
    # A re-fed window [r tokens | block of S] at P gives the same K/V for the r
    # tokens and the same block outputs as decoding the r tokens one at a time
    # (W = 1 steps, each storing its K/V) and then running the S-row block at
    # P + r: re-feeding is causal decoding batched into the window.
    d = TINY
    W = 7
    Ps, cs, ws = (5, 9), (2, 1), (6, 4)  # sequence 0: 2 re-fed + 4-block; 1: 1 + 3, 3 padding rows
    model, _, _ = _tiny_setup(seed=31)
    cache = _np(synth.make_cache(d, torch.tensor(list(Ps)), W, seed=32))
    ids = synth.draw_window_ids(2, W, d.vocab, 33, mask_id=-1).numpy()
    r = O.pbd_step(model, cache, ids, Ps, causal_rows=cs, window_len=ws, return_hidden=True)
    for b in range(2):
        sub = {k: (np.array(v, copy=True) if isinstance(v, np.ndarray) else v) for k, v in cache.items()}
        sub["block_table"] = sub["block_table"][[b]]
        P = Ps[b]
        for j in range(cs[b]):
            rj = O.pbd_step(model, sub, ids[b:b + 1, j:j + 1], [P + j])
            for l, (kb, vb) in enumerate(rj["kv"]):
                np.testing.assert_array_equal(r["kv"][l][0][b * W + j], kb[0])
                np.testing.assert_array_equal(r["kv"][l][1][b * W + j], vb[0])
            _store_kv(sub, rj["kv"], [P + j], 1, 1, [1])
        S = ws[b] - cs[b]
        rb = O.pbd_step(model, sub, ids[b:b + 1, cs[b]:ws[b]], [P + cs[b]], return_hidden=True)
        rows = slice(b * W + cs[b], b * W + ws[b])
        np.testing.assert_allclose(r["hidden"][rows], rb["hidden"], rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(r["ids"][b, cs[b]:ws[b]], rb["ids"][0])
        for l, (kb, vb) in enumerate(rb["kv"]):
            assert np.abs(r["kv"][l][0][rows].astype(np.int32) - kb.astype(np.int32)).max() <= 1
            assert np.abs(r["kv"][l][1][rows].astype(np.int32) - vb.astype(np.int32)).max() <= 1
        assert S == rb["ids"].shape[1]


def test_refeed_commit_worked_example():
    out = np.array([[10, 11, 12, 13, 14, 15, 16], [20, 21, 22, 23, 24, 25, 26]])
    win = np.zeros((2, 7), dtype=np.int32)
    ids, P, c, w = O.refeed_commit(out, win, [100, 200], [1, 0], [5, 3], 3, 99)
    # sequence 0: block rows 1..4 accepted (11..14), the last opens a 3-row block
    np.testing.assert_array_equal(ids, [[11, 12, 13, 14, 99, 99, 99], [20, 21, 22, 99, 99, 99, 99]])
    assert list(P) == [102, 201] and list(c) == [3, 2] and list(w) == [6, 5]
    ids, P, c, w = O.refeed_commit(out, win, [100, 200], [1, 0], [5, 3], 3, 99, n_accept=[2, 9])
    np.testing.assert_array_equal(ids, [[11, 12, 99, 99, 99, 99, 99], [20, 21, 22, 99, 99, 99, 99]])
    assert list(P) == [102, 201] and list(c) == [1, 2] and list(w) == [4, 5]
    ids, P, c, w = O.refeed_commit(out, win, [100, 200], [1, 0], [5, 3], 3, 99, n_accept=[0, 1])
    np.testing.assert_array_equal(ids[:, :3], [[11, 99, 99], [20, 99, 99]])
    assert list(c) == [0, 0] and list(w) == [3, 3]


def test_refeed_loop_places_every_accepted_token_at_its_position():
    # Across a loop with partial acceptance, every real window row holds the
    # token predicted for its position (row i of a window is at P + i; the
    # argmax of row i is the token at P + i + 1), and the K/V of committed
    # slots are the ones the step that last held them as a real row computed.
    d = TINY
    W, block, mask = 7, 4, 3
    model, _, _ = _tiny_setup(seed=41)
    cache = _np(synth.make_cache(d, torch.tensor([5, 9]), W, extra_tokens=16, seed=42))
    ids = np.full((2, W), mask, dtype=np.int32)
    ids[:, 0] = [17, 29]
    acc = [np.array([4, 2]), np.array([1, 3]), np.array([2, 4])]
    outs, (ids_f, P_f, c_f, w_f), cc = O.pbd_refeed_loop(
        model, cache, ids, [5, 9], [0, 0], [block, block], 3, block, mask, n_accept=acc)
    tok = {0: {5: 17}, 1: {9: 29}}
    win, P, c, w = ids, np.array([5, 9]), np.array([0, 0]), np.array([block, block])
    for s in range(3):
        for b in range(2):
            for i in range(int(w[b])):
                if win[b, i] != mask or i <= c[b]:
                    assert tok[b][int(P[b]) + i] == win[b, i]
            n = min(max(int(acc[s][b]), 1), int(w[b] - c[b]))
            for i in range(n):
                tok[b][int(P[b] + c[b]) + i + 1] = int(outs[s][b, c[b] + i])
        win, P, c, w = O.refeed_commit(outs[s], win, P, c, w, block, mask, acc[s])
    np.testing.assert_array_equal(win, ids_f)
    assert list(P) == list(P_f)
    # the committed cache is what the next step reads: a fresh step on it
    # gives the loop's next outputs
    r = O.pbd_step(model, cc, ids_f, P_f, causal_rows=c_f, window_len=w_f)
    assert r["ids"].shape == (2, W)


# ---------------------------------------------------------------- repetition penalty

def _lm_of(values):
    """A tied lm_head whose column 0 holds `values` (bf16-exact), so that the
    logits of f = e_0 are exactly those values."""
    V = len(values)
    E = np.zeros((V, 4))
    E[:, 0] = values
    bits = O.round_to_bf16_bits(E)
    assert np.array_equal(O.bf16_to_float(bits)[:, 0], values)
    return {"fmt": "bf16", "data": bits, "n": V}


def test_repetition_penalty_worked_examples():
    # logits 3, 2.75, -1, -0.9375, 0.5 (exact in bf16) for the row f = e_0
    lm = _lm_of(np.array([3.0, 2.75, -1.0, -0.9375, 0.5]))
    f = np.zeros((1, 4))
    f[0, 0] = 1.0
    ids, top1, gap = O.lm_head_argmax(f, lm)
    assert ids[0] == 0 and top1[0] == 3.0 and gap[0] == 0.25
    # id 0 already used: 3 / 1.1 = 2.7272... < 2.75, so id 1 wins by 0.0227...
    ids, top1, gap = O.lm_head_argmax(f, lm, rep_sets=[[0]], rep_penalty=1.1)
    assert ids[0] == 1 and top1[0] == 2.75
    assert abs(gap[0] - (2.75 - 3.0 / 1.1)) < 1e-15
    # ids 0 and 1 used: 2.7272... beats 2.5
    ids, top1, gap = O.lm_head_argmax(f, lm, rep_sets=[[1, 0]], rep_penalty=1.1)
    assert ids[0] == 0 and abs(top1[0] - 3.0 / 1.1) < 1e-15 and abs(gap[0] - (3.0 / 1.1 - 2.5)) < 1e-15
    # a negative logit is multiplied: -0.9375 * 1.1 = -1.03125 falls below -1
    neg = _lm_of(np.array([-1.0, -0.9375, -2.0]))
    ids, top1, gap = O.lm_head_argmax(f, neg)
    assert ids[0] == 1
    ids, top1, gap = O.lm_head_argmax(f, neg, rep_sets=[[1]], rep_penalty=1.1)
    assert ids[0] == 0 and top1[0] == -1.0 and abs(gap[0] - (-1.0 + 1.03125)) < 1e-15
    # zero is not positive: multiplied, and stays zero
    np.testing.assert_array_equal(O.repetition_penalty(np.array([0.0, 2.2, -2.0]), 1.1),
                                  [0.0, 2.2 / 1.1, -2.0 * 1.1])


def test_repetition_penalty_special_cases():
    rng = np.random.default_rng(71)
    V, H = 9000, 16
    bits = O.round_to_bf16_bits(rng.standard_normal((V, H)) * 0.5)
    lm = {"fmt": "bf16", "data": bits, "n": V}
    f = rng.standard_normal((5, H))
    base = O.lm_head_argmax(f, lm, chunk=4096)
    sets = [rng.choice(V, size=300, replace=False) for _ in range(5)]
    # a penalty of 1 changes nothing
    same = O.lm_head_argmax(f, lm, chunk=4096, rep_sets=sets, rep_penalty=1.0)
    for a, b in zip(base, same):
        np.testing.assert_array_equal(a, b)
    # penalising only tokens that are not the argmax never changes the argmax
    # (every penalised logit only goes down)
    others = [np.setdiff1d(s_, [base[0][t]]) for t, s_ in enumerate(sets)]
    got = O.lm_head_argmax(f, lm, chunk=4096, rep_sets=others, rep_penalty=1.3)
    np.testing.assert_array_equal(got[0], base[0])
    np.testing.assert_array_equal(got[1], base[1])
    # penalising the argmax: the new winner is the best of the penalised top-1
    # and the unpenalised rest, found by sorting the full logit row
    logits = f @ O.bf16_to_float(bits).T
    got = O.lm_head_argmax(f, lm, chunk=4096, rep_sets=[[i] for i in base[0]], rep_penalty=1.3)
    for t in range(5):
        row = logits[t].copy()
        i = base[0][t]
        row[i] = row[i] / 1.3 if row[i] > 0 else row[i] * 1.3
        order = np.argsort(-row, kind="stable")
        assert got[0][t] == order[0]
        assert abs(got[2][t] - (row[order[0]] - row[order[1]])) < 1e-12


# ---------------------------------------------------------------- prefill

def test_prefill_equals_token_by_token_decode():
    # A causal pass over L prompt positions gives the K/V of every position
    # and the last position's hidden state and id that L single-token decode
    # steps (W = 1, each storing its K/V) give.
    d = TINY
    L, Ps = 7, (0, 9)
    model, _, _ = _tiny_setup(seed=51)
    cache = _np(synth.make_cache(d, torch.tensor(list(Ps)), L, seed=52))
    ids = synth.draw_window_ids(2, L, d.vocab, 53, mask_id=-1).numpy()
    r = O.pbd_prefill(model, cache, ids, Ps)
    for b in range(2):
        sub = {k: (np.array(v, copy=True) if isinstance(v, np.ndarray) else v) for k, v in cache.items()}
        sub["block_table"] = sub["block_table"][[b]]
        for j in range(L):
            rj = O.pbd_step(model, sub, ids[b:b + 1, j:j + 1], [Ps[b] + j], return_hidden=True)
            for l, (kb, vb) in enumerate(rj["kv"]):
                assert np.abs(r["kv"][l][0][b * L + j].astype(np.int32) - kb[0].astype(np.int32)).max() <= 1
                assert np.abs(r["kv"][l][1][b * L + j].astype(np.int32) - vb[0].astype(np.int32)).max() <= 1
            _store_kv(sub, rj["kv"], [Ps[b] + j], 1, 1, [1])
        np.testing.assert_allclose(r["hidden"][b], rj["hidden"][0], rtol=1e-12, atol=1e-12)
        assert r["ids"][b] == rj["ids"][0, 0]


def test_prefill_spliced_rows_equal_their_embedding_rows():
    # a spliced input row that equals an embedding row gives the same result,
    # bit for bit, as that row's id; another spliced row changes the result
    d = TINY
    L, Ps = 6, (3, 5)
    model, _, _ = _tiny_setup(seed=61)
    cache = _np(synth.make_cache(d, torch.tensor(list(Ps)), L, seed=62))
    ids = synth.draw_window_ids(2, L, d.vocab, 63, mask_id=-1).numpy()
    ref = O.pbd_prefill(model, cache, ids, Ps)
    emb = np.zeros((2, L, d.hidden))
    spliced = ids.copy()
    for b, j in ((0, 1), (0, 2), (1, 0)):
        emb[b, j] = O.embed_rows([ids[b, j]], model["embed"])[0]
        spliced[b, j] = -1
    got = O.pbd_prefill(model, cache, spliced, Ps, input_embeds=emb)
    np.testing.assert_array_equal(got["hidden"], ref["hidden"])
    np.testing.assert_array_equal(got["ids"], ref["ids"])
    emb[0, 2] += 0.5
    other = O.pbd_prefill(model, cache, spliced, Ps, input_embeds=emb)
    assert np.abs(other["hidden"][0] - ref["hidden"][0]).max() > 1e-6
    np.testing.assert_array_equal(other["hidden"][1], ref["hidden"][1])


# ---------------------------------------------------------------- sampling (temperature, top-p)

def test_philox_known_answer_vectors():
    # Philox4x32-10 known-answer vectors of the Random123 distribution
    # (counter, key) -> output
    kat = [
        ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
        ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
        ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
         [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
    ]
    for ctr, key, want in kat:
        assert OS.philox4x32_10(ctr, key) == want
    u = OS.philox_uniform(0, 0, 0)
    assert u == (0x6627E8D5 >> 8) / 2 ** 24 and 0.0 <= u < 1.0


def test_nucleus_hand_worked():
    # probabilities 0.1, 0.5, 0.05, 0.15, 0.2 (T = 1): top_p 0.8 keeps the three
    # largest, ids 1 (0.5), 4 (0.2), 3 (0.15): 0.5 + 0.2 = 0.7 < 0.8 <= 0.85
    p = np.array([0.1, 0.5, 0.05, 0.15, 0.2])
    z = np.log(p)
    kept, pk, total = OS.nucleus(z, 1.0, 0.8)
    assert kept.tolist() == [1, 3, 4]
    np.testing.assert_allclose(pk / total, [0.5, 0.15, 0.2], rtol=1e-12)
    # the draw walks the kept ids in ascending id order (not probability
    # order): cumulative 0.5, 0.65, 0.85 of the kept mass 0.85, i.e. u
    # boundaries at 0.588 and 0.765
    for u, want in ((0.0, 1), (0.58, 1), (0.59, 3), (0.76, 3), (0.77, 4), (0.999, 4)):
        assert OS.sample_row(z, 1.0, 0.8, u) == want, u
    # just below and just above the mass of the first two (0.7)
    assert OS.nucleus(z, 1.0, 0.69)[0].tolist() == [1, 4]
    assert OS.nucleus(z, 1.0, 0.71)[0].tolist() == [1, 3, 4]
    # temperature sharpens: T = 0.5 squares the ratios, 0.25 : 0.04 : 0.0225 :
    # 0.01 : 0.0025, i.e. 0.769, 0.123, 0.069, ... of the total: the first two
    # hold 0.892
    assert OS.nucleus(z, 0.5, 0.88)[0].tolist() == [1, 4]
    assert OS.nucleus(z, 0.5, 0.9)[0].tolist() == [1, 3, 4]


def test_nucleus_ties_take_lower_ids_first():
    z = np.array([0.0, 2.0, 1.0, 2.0, 2.0])
    # three ids tie at the top; top_p small keeps only the lowest of them
    assert OS.nucleus(z, 1.0, 1e-6)[0].tolist() == [1]
    # two thirds of the tied mass needs two of them: ids 1 and 3
    kept, pk, total = OS.nucleus(z, 1.0, 0.5)
    assert kept.tolist() == [1, 3]


def test_sampling_limits():
    rng = np.random.default_rng(3)
    z = rng.standard_normal(1000)
    top = int(np.argmax(z))
    # T <= 0 and T -> 0 select the argmax
    assert OS.sample_row(z, 0.0, 0.9, 0.7) == top
    assert OS.sample_row(z, 1e-4, 0.9, 0.7) == top
    # top_p -> 0 keeps the argmax only
    assert OS.sample_row(z, 1.0, 1e-9, 0.99) == top
    # top_p = 1 keeps everything: the draw is the plain inverse CDF in id order
    kept, pk, total = OS.nucleus(z, 0.7, 1.0)
    assert kept.size == z.size
    p = np.exp((z - z.max()) / 0.7)
    cdf = np.cumsum(p) / p.sum()
    for u in (0.0, 0.3, 0.77, 0.999999):
        assert OS.sample_row(z, 0.7, 1.0, u) == int(np.searchsorted(cdf, u, side="right"))


def test_sampling_frequencies_match_the_nucleus():
    # many draws (Philox over rows) against the renormalised nucleus: chi-square
    rng = np.random.default_rng(4)
    z = rng.standard_normal(12) * 1.5
    T, top_p = 0.7, 0.9
    kept, pk, total = OS.nucleus(z, T, top_p)
    n = 20000
    counts = np.zeros(z.size)
    for t in range(n):
        counts[OS.sample_row(z, T, top_p, OS.philox_uniform(t, 1234, 99))] += 1
    assert counts[np.setdiff1d(np.arange(z.size), kept)].sum() == 0
    expect = n * pk / pk.sum()
    chi2 = float(((counts[kept] - expect) ** 2 / expect).sum())
    # 99.9th percentile of chi-square with up to 11 degrees of freedom is < 32
    assert chi2 < 32.0, (chi2, kept.size)


def test_sample_rows_uses_the_row_counter():
    z = np.zeros((4, 50))
    # uniform logits: the id is floor(u * 50) for each row's own draw
    ids = OS.sample_rows(z, 1.0, 1.0, seed=7, offset=5)
    want = [int(OS.philox_uniform(t, 7, 5) * 50) for t in range(4)]
    assert ids.tolist() == want


def test_window_kv_override():
    # the window's own rounding passed back in reproduces the step bit for bit;
    # one window value changed by one bf16 ulp changes every later layer's output
    d = TINY
    model, cache, _ = _tiny_setup(P_list=(4, 9), W=3, seed=71)
    ids = synth.draw_window_ids(2, 3, d.vocab, 72, mask_id=-1).numpy()
    P = [4, 9]
    ref = O.pbd_step(model, cache, ids, P, return_hidden=True)
    same = O.pbd_step(model, cache, ids, P, return_hidden=True, window_kv=ref["kv"])
    np.testing.assert_array_equal(same["hidden"], ref["hidden"])
    forced = [(k.copy(), v.copy()) for k, v in ref["kv"]]
    forced[0][1][2, 0, 5] ^= 1                      # one V element of layer 0, one ulp
    other = O.pbd_step(model, cache, ids, P, return_hidden=True, window_kv=forced)
    assert np.abs(other["hidden"] - ref["hidden"]).max() > 0
    # the layer's own rounding is still what it returns
    np.testing.assert_array_equal(other["kv"][0][1], ref["kv"][0][1])


# ---------------------------------------------------------------- w8a8

def test_quantize_rows_int8_hand_worked():
    # max |x| = 127 gives s = 1 exactly, so x / s is exact and the rounding is
    # visible: halves go to the even integer (-63.5 -> -64, 31.5 -> 32,
    # 2.5 -> 2, -0.5 -> 0), not away from zero (-64, 32, 3, -1)
    q, s = O.quantize_rows_int8(np.array([[127.0, -63.5, 31.5, 2.5, -0.5, 0.0]]))
    assert s.dtype == np.float32 and s.tolist() == [1.0]
    assert q.tolist() == [[127, -64, 32, 2, 0, 0]]
    # a negative maximum: s = 254 / 127 = 2; 127 / 2 = 63.5 -> 64
    q, s = O.quantize_rows_int8(np.array([[-254.0, 127.0, 1.0]]))
    assert s.tolist() == [2.0] and q.tolist() == [[-127, 64, 0]]
    # a zero row: s = 0, every code 0 (no division by zero)
    q, s = O.quantize_rows_int8(np.zeros((2, 5)))
    assert s.tolist() == [0.0, 0.0] and not q.any()
    # the decision is taken in float32: x / s of the float32 operands
    x = np.array([[1.0, 1.0 / 3.0, -0.7]])
    q, s = O.quantize_rows_int8(x)
    s32 = np.float32(1.0) / np.float32(127)
    assert s[0] == s32
    assert q[0, 1] == int(np.rint(np.float32(np.float32(1.0 / 3.0) / s32)))


def _w8a8_weight(rng, n, k):
    q = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    s = rng.uniform(2e-4, 4e-4, size=n).astype(np.float32)
    return {"fmt": "w8a8", "n": n, "k": k, "group": 0, "data": q, "scales": s}


def test_w8a8_linear_scales_the_integer_products():
    """The integer sum scaled by both scales equals the product of the
    dequantised operands (two different computations of the same number)."""
    rng = np.random.default_rng(11)
    w = _w8a8_weight(rng, 24, 96)
    x = rng.standard_normal((5, 96))
    y = O.linear(x, w)
    qx, sx = O.quantize_rows_int8(x)
    xd = qx.astype(np.float64) * sx.astype(np.float64)[:, None]
    ref = xd @ O.decode_weight(w).T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-15)
    # a subset of output channels (the lm_head's chunks) gives the same columns
    rows = np.array([3, 7, 20])
    np.testing.assert_allclose(O.linear(x, w, rows=rows), y[:, rows], rtol=1e-15)
    # unquantised activations: the decoded weight times x itself
    np.testing.assert_allclose(O.linear(x, w, quantize_acts=False), x @ O.decode_weight(w).T, rtol=1e-15)


def test_w8a8_linear_error_bound_and_exact_grid():
    rng = np.random.default_rng(12)
    w = _w8a8_weight(rng, 16, 128)
    Wd = O.decode_weight(w)
    x = rng.standard_normal((7, 128))
    y = O.linear(x, w)
    _, sx = O.quantize_rows_int8(x)
    # rounding moves each activation by at most s / 2 (plus float32 slack)
    bound = (sx.astype(np.float64)[:, None] * 0.5 * (1 + 1e-6) + 1e-7 * np.abs(x).max(axis=1)[:, None]) \
        * np.abs(Wd).sum(axis=1)[None, :]
    assert np.all(np.abs(y - x @ Wd.T) <= bound)
    # activations already on the grid (s a power of two, max |q| = 127) are kept exactly
    q = rng.integers(-127, 128, size=(3, 128)).astype(np.float64)
    q[:, 0] = 127
    xg = q * 2.0 ** -5
    np.testing.assert_allclose(O.linear(xg, w), xg @ Wd.T, rtol=1e-12)


def test_w8a8_layer_zero_weights_is_identity():
    d = synth.ModelDims(n_layers=1, vocab=64, hidden=256, n_heads=2, n_kv_heads=1, inter=512)
    m = synth.to_numpy_tree(synth.make_model(d, "w8a8", 1, "cpu"))
    lay = m["layers"][0]
    for k in ("qkv", "o", "gate_up", "down"):
        lay[k]["data"] = np.zeros_like(lay[k]["data"])
    P = torch.tensor([9], dtype=torch.int32)
    cache = synth.to_numpy_tree(synth.make_cache(d, P, 6, seed=2, device="cpu"))
    h = np.random.default_rng(3).standard_normal((6, 256))
    out, _, _ = O.decoder_layer(h, lay, d, cache, 0, P.numpy(), 6)
    np.testing.assert_array_equal(out, h)


def test_w8a8_integer_sums_are_exact_at_full_width():
    # K = 11008 with every code at +-127: float64 sums equal the int64 products
    rng = np.random.default_rng(13)
    K = 11008
    qw = np.where(rng.random((4, K)) < 0.5, -127, 127).astype(np.int8)
    w = {"fmt": "w8a8", "n": 4, "k": K, "group": 0, "data": qw, "scales": np.ones(4, np.float32)}
    qx = np.where(rng.random((3, K)) < 0.5, -127, 127).astype(np.int64)
    qx[:, 0] = 127  # max |x| = 127: s = 1, the codes are x itself
    y = O.linear(qx.astype(np.float64), w)
    exact = qx @ qw.astype(np.int64).T
    assert np.array_equal(y, exact.astype(np.float64))

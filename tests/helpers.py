"""Shared helpers of the GPU parity tests (inputs come from box_decoding_amd.synth;
expected values from the oracle only)."""
import numpy as np
import torch

import oracle as O
from box_decoding_amd import synth


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def np_tree(x):
    return synth.to_numpy_tree(x)


def ids_match(gpu_ids, ref_ids, ref_gap, ref_top1, f, lm, row_sets=None, rep_penalty=1.0, thr=1e-3):
    """Argmax ids against the oracle, every row compared.

    Where the oracle's top-2 gap is >= thr the GPU's id must equal the
    oracle's.  Where it is smaller several ids are correct: the GPU's id must
    be a vocabulary id whose oracle logit (computed here from the oracle's
    final-normed rows f, with the repetition penalty of row_sets) is within
    thr of the oracle's top-1.

    Returns (n_compared, n_bad, n_near_tie): every row is compared, n_bad
    counts exact mismatches plus near-tie rows whose id is not valid."""
    g = np.asarray(gpu_ids).reshape(-1).astype(np.int64)
    r = np.asarray(ref_ids).reshape(-1)
    gap = np.asarray(ref_gap).reshape(-1)
    top1 = np.asarray(ref_top1).reshape(-1)
    keep = gap >= thr
    bad = int((g[keep] != r[keep]).sum())
    near = np.flatnonzero(~keep)
    if near.size:
        V = int(lm["n"])
        f = np.asarray(f).reshape(len(g), -1)
        ok_id = (g[near] >= 0) & (g[near] < V)
        z = np.full(near.size, -np.inf)
        if ok_id.any():
            sets = None if row_sets is None else [row_sets[t] for t in near[ok_id]]
            z[ok_id] = O.logits_of(f[near[ok_id]], lm, g[near[ok_id]], rep_sets=sets,
                                   rep_penalty=rep_penalty)
        bad += int((z < top1[near] - thr).sum())
    return len(g), bad, int(near.size)


def step_ids_match(gpu_ids, ref, rows=None):
    """ids_match for an oracle result ``ref`` (pbd_step / pbd_prefill) that the
    test has completed with ref["lm"] (the oracle's lm_head weight) and, for a
    penalised ranking, ref["seq_sets"] (per-sequence repetition sets) and
    ref["rep_penalty"].  ``rows`` selects flat rows (default all)."""
    ids = np.asarray(ref["ids"])
    W = ids.shape[-1] if ids.ndim > 1 else 1
    g = np.asarray(gpu_ids).reshape(-1)
    n = g.size
    rows = np.arange(n) if rows is None else np.asarray(rows)
    seq_sets = ref.get("seq_sets")
    row_sets = None if seq_sets is None else [seq_sets[t // W] for t in rows]
    return ids_match(g[rows], ids.reshape(-1)[rows], np.asarray(ref["gap"]).reshape(-1)[rows],
                     np.asarray(ref["top1"]).reshape(-1)[rows],
                     np.asarray(ref["final"]).reshape(n, -1)[rows], ref["lm"], row_sets,
                     ref.get("rep_penalty", 1.0))


def oracle_lm(mn):
    """The oracle model's lm_head weight (the tied embedding when lm_head is None)."""
    return mn["lm_head"] if mn.get("lm_head") is not None else mn["embed"]


def rel_l2_rows(a, b, width):
    """Largest rel-L2 over the rows of width ``width`` (a row's error against its own norm)."""
    a = np.asarray(a, dtype=np.float64).reshape(-1, width)
    b = np.asarray(b, dtype=np.float64).reshape(-1, width)
    num = np.linalg.norm(a - b, axis=1)
    den = np.maximum(np.linalg.norm(b, axis=1), 1e-300)
    return float(np.max(num / den)) if a.shape[0] else 0.0


def max_abs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def bf16_ulp_diff(a_bits, b_bits):
    """Distance in bf16 units of the last place between two bf16 bit arrays."""
    def ordered(x):
        x = np.asarray(x).view(np.uint16).astype(np.int64)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + x)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def bf16_kv_mismatch(got_bits, ref_bits, rel_floor=1e-4):
    """Largest disagreement between bf16 K/V entries written by the GPU and the
    oracle's rounding of the exact value, in bf16 ulps of the reference value.

    The GPU rounds an fp32 result whose absolute error is a small fraction of
    the tensor's scale; where the reference value is so small that this
    fraction exceeds its bf16 ulp, any entry within rel_floor * rms of the
    reference counts as 0 ulps.  Elsewhere one ulp (a rounding decision taken
    on the other side of a tie point) is the bar."""
    g = np.asarray(got_bits).view(np.uint16).astype(np.uint32) << 16
    r = np.asarray(ref_bits).view(np.uint16).astype(np.uint32) << 16
    gf = g.view(np.float32).astype(np.float64)
    rf = r.view(np.float32).astype(np.float64)
    rms = np.sqrt(np.mean(rf * rf)) if rf.size else 0.0
    ulps = bf16_ulp_diff(got_bits, ref_bits)
    small = np.abs(gf - rf) <= rel_floor * rms
    return int(np.max(np.where(small, 0, ulps))) if ulps.size else 0


def cache_slots(cache_np, layer, b, positions):
    """bf16 bits of K and V at the given token positions of sequence b: [n, Hkv, D]."""
    bs = int(cache_np["block"])
    pos = np.asarray(positions)
    blk = np.asarray(cache_np["block_table"])[b, pos // bs].astype(np.int64)
    off = pos % bs
    k = cache_np["k"][layer][blk, :, off, :]
    v = cache_np["v"][layer][blk, :, :, off]
    return k.view(np.uint16), v.view(np.uint16)


def poison_unused_slots(cache: dict, prefix_len, window: int):
    """Fill every cache slot at or beyond P_b + window (and unreferenced blocks) with NaN."""
    k, v, table = cache["k"], cache["v"], cache["block_table"].cpu().numpy()
    bs = int(cache["block"])
    used = np.zeros((k.shape[1], bs), dtype=bool)
    for b, P in enumerate(torch.as_tensor(prefix_len).cpu().tolist()):
        for t in range(P + window):
            used[table[b, t // bs], t % bs] = True
    mask = torch.from_numpy(~used).to(k.device)  # [NB, bs]
    nan = torch.tensor(0x7FC0, dtype=torch.int32).to(torch.int16).item()
    km = mask[None, :, None, :, None].expand_as(k)
    vm = mask[None, :, None, None, :].expand_as(v)
    k.masked_fill_(km, nan)
    v.masked_fill_(vm, nan)


def bf16_bits_rel_l2(got_bits, ref_bits):
    """rel-L2 between two bf16 bit arrays, as decoded values."""
    def dec(x):
        return (np.asarray(x).view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return rel_l2(dec(got_bits), dec(ref_bits))


def kv_rows_vs_exact(got_bits, exact, row_width):
    """Largest per-row rel-L2 of the bf16 K/V the GPU stored against the
    oracle's values before rounding.  A bf16 store alone moves each value by up
    to half an ulp (2^-9 of it), so a bar on this is a tolerance plus 2^-9."""
    dec = (np.asarray(got_bits).view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    return rel_l2_rows(dec.astype(np.float64), exact, row_width)


BF16_HALF_ULP = 2.0 ** -9

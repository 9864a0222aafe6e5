"""Shared helpers of the GPU parity tests (inputs come from box_decoding_amd.synth;
expected values from the oracle only)."""
import numpy as np
import torch

from box_decoding_amd import synth


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def np_tree(x):
    return synth.to_numpy_tree(x)


def ids_match(gpu_ids, ref_ids, ref_gap, thr=1e-3):
    """Argmax ids must match wherever the oracle's top-2 gap is >= thr.

    Returns (n_compared, n_mismatch, n_excluded)."""
    g = np.asarray(gpu_ids).reshape(-1)
    r = np.asarray(ref_ids).reshape(-1)
    gap = np.asarray(ref_gap).reshape(-1)
    keep = gap >= thr
    return int(keep.sum()), int((g[keep] != r[keep]).sum()), int((~keep).sum())


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

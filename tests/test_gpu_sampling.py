"""GPU parity of the sampled selection (temperature, top-p, Philox draws)
against the oracle (oracle/sampling.py).

The draws are bit-identical on both sides (the same counter-based generator),
so where the oracle's decision does not hang on rounding the ids must be
equal.  The GPU sums probabilities in 40-bit fixed point from fp32 exp2, the
oracle in float64: where u lies within EPS of a boundary of the kept
distribution, or the nucleus boundary within EPS of top_p, several ids are
correct, and the GPU's must be one of them.  With uniform logits every
probability is exact on both sides and the ids must match everywhere, which
pins the generator, the tie order and the draw bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle as O
import oracle.sampling as OS
from box_decoding_amd import binding as B
from box_decoding_amd import synth
from helpers import np_tree, oracle_lm

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
EPS = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()
    torch.cuda.set_device(0)


def _log(msg):
    print(msg, flush=True)


def check_draw(z, T, top_p, u, got, eps=EPS):
    """0 if the GPU's id equals the oracle's, 1 if it differs but is a valid
    draw of the same distribution within eps, else raise."""
    want = OS.sample_row(z, T, top_p, u)
    if got == want:
        return 0
    z = np.asarray(z, dtype=np.float64)
    p = np.exp((z - z.max()) / T)
    order = np.lexsort((np.arange(z.size), -z))
    cum = np.cumsum(p[order]) / p.sum()
    rank = np.empty(z.size, dtype=np.int64)
    rank[order] = np.arange(z.size)
    # every nucleus for a top_p' within eps of top_p, and the draw in each
    n_lo = int(np.searchsorted(cum, top_p - eps, side="left")) + 1
    n_hi = int(np.searchsorted(cum, top_p + eps, side="left")) + 1
    assert 0 <= got < z.size and rank[got] < max(n_hi, 1), (got, want, rank[got], n_hi)
    for n in range(max(n_lo, 1), min(max(n_hi, 1), z.size) + 1):
        kept = np.sort(order[:n])
        if got not in kept:
            continue
        c = np.cumsum(p[kept]) / p[kept].sum()
        i = int(np.searchsorted(kept, got))
        lo = c[i - 1] if i else 0.0
        if lo - eps <= u <= c[i] + eps:
            return 1
    raise AssertionError(f"id {got} is not a valid draw (oracle {want}, u {u})")


@pytest.mark.parametrize("V,sigma,T,top_p,ties", [
    (152681, 0.1, 0.7, 0.9, False),   # flat: the nucleus holds most of the vocabulary
    (152681, 3.0, 0.7, 0.9, False),   # peaked: a handful of ids
    (152681, 1.0, 1.5, 0.5, False),
    (50000, 1.0, 0.7, 0.9, True),     # logits on a 1/4 grid: many exact ties
    (1000, 2.0, 0.3, 0.99, True),
])
def test_sample_logits_matches_oracle(V, sigma, T, top_p, ties):
    M, seed, offset = 48, 1234 + V, 77
    g = torch.Generator(device=DEV).manual_seed(V + int(sigma * 10))
    z = torch.randn((M, V), generator=g, device=DEV) * sigma
    if ties:
        z = torch.round(z * 4) / 4
    ids, sel = B.sample_logits(z, B.Sampling(T, top_p, seed, offset))
    torch.cuda.synchronize()
    zn = z.cpu().numpy().astype(np.float64)
    got = ids.cpu().numpy()
    near = 0
    top_p32 = float(np.float32(top_p))
    for t in range(M):
        u = OS.philox_uniform(t, seed, offset)
        near += check_draw(zn[t], T, top_p32, u, int(got[t]))
    sel_ref = zn[np.arange(M), got] - zn.max(axis=1)
    assert np.max(np.abs(sel.cpu().numpy() - sel_ref)) < 1e-5
    _log(f"sample V={V} sigma={sigma} T={T} top_p={top_p} ties={ties}: {M - near} equal, {near} valid near "
         f"a boundary")
    assert near <= M // 10


@pytest.mark.parametrize("V,top_p", [(1000, 1.0), (4096, 0.9), (152681, 0.37)])
def test_sample_uniform_logits_bit_exact(V, top_p):
    """Equal logits: the nucleus is the lowest ceil(top_p * V) ids, the draw
    floor(u * kept): every id equals the oracle's."""
    M, seed, offset = 256, 99, (1 << 33) + 5
    z = torch.zeros((M, V), device=DEV)
    ids, _ = B.sample_logits(z, B.Sampling(1.0, top_p, seed, offset))
    torch.cuda.synchronize()
    top_p32 = float(np.float32(top_p))
    want = [OS.sample_row(np.zeros(V), 1.0, top_p32, OS.philox_uniform(t, seed, offset)) for t in range(M)]
    assert ids.cpu().numpy().tolist() == want


def test_sample_frequencies():
    """4096 rows with the same logits, one draw each: frequencies against the
    renormalised nucleus (chi-square)."""
    rng = np.random.default_rng(5)
    V, M, T, top_p = 24, 4096, 0.7, 0.9
    zr = rng.standard_normal(V) * 1.5
    z = torch.from_numpy(np.tile(zr.astype(np.float32), (M, 1))).to(DEV)
    ids, _ = B.sample_logits(z, B.Sampling(T, top_p, 31, 0))
    torch.cuda.synchronize()
    counts = np.bincount(ids.cpu().numpy(), minlength=V).astype(np.float64)
    kept, pk, _ = OS.nucleus(zr.astype(np.float32).astype(np.float64), T, top_p)
    assert counts[np.setdiff1d(np.arange(V), kept)].sum() == 0
    expect = M * pk / pk.sum()
    chi2 = float(((counts[kept] - expect) ** 2 / expect).sum())
    _log(f"sample frequencies: {kept.size} kept ids, chi-square {chi2:.1f}")
    assert chi2 < 45.0  # 99.9th percentile of chi-square with <= 23 degrees of freedom is 49


def test_sample_greedy_and_penalty():
    M, V = 12, 3001
    g = torch.Generator(device=DEV).manual_seed(3)
    z = torch.randn((M, V), generator=g, device=DEV)
    ids, sel = B.sample_logits(z, B.Sampling(0.0, 0.9, 1, 1))
    torch.cuda.synchronize()
    assert torch.equal(ids.long(), z.argmax(dim=1)) and float(sel.abs().max()) == 0.0
    # a penalised argmax: every row's winner in its set, penalty 1.1
    rows = 6
    win = z.argmax(dim=1).cpu().numpy()
    words = B.rep_words(V)
    bits = np.zeros((M // rows, words), dtype=np.uint32)
    for t in range(M):
        bits[t // rows, win[t] >> 5] |= np.uint32(1) << np.uint32(win[t] & 31)
    bt = torch.from_numpy(bits.view(np.int32)).to(DEV)
    ids2, _ = B.sample_logits(z, B.Sampling(0.0, 0.9, 1, 1), rep_bits=bt, rep_rows=rows, rep_penalty=1.1)
    # and sampled with the penalty
    ids3, _ = B.sample_logits(z, B.Sampling(0.8, 0.95, 5, 6), rep_bits=bt, rep_rows=rows, rep_penalty=1.1)
    torch.cuda.synchronize()
    zn = z.cpu().numpy().astype(np.float64)
    near = 0
    for t in range(M):
        sset = np.flatnonzero(np.unpackbits(bits[t // rows].view(np.uint8), bitorder="little")[:V])
        zp = zn[t].copy()
        zp[sset] = O.repetition_penalty(zp[sset], 1.1)
        assert int(ids2[t]) == int(np.argmax(zp))
        near += check_draw(zp, 0.8, float(np.float32(0.95)), OS.philox_uniform(t, 5, 6), int(ids3[t]))
    assert near <= 2


def test_sample_offset_dev_advances_and_is_deterministic():
    M, V = 8, 777
    z = torch.randn((M, V), generator=torch.Generator(device=DEV).manual_seed(8), device=DEV)
    off = torch.tensor([41], dtype=torch.int64, device=DEV)
    s = B.Sampling(1.0, 0.9, 3, 0, offset_dev=off)
    a, _ = B.sample_logits(z, s)
    b, _ = B.sample_logits(z, s)
    c, _ = B.sample_logits(z, B.Sampling(1.0, 0.9, 3, 41))
    d, _ = B.sample_logits(z, B.Sampling(1.0, 0.9, 3, 42))
    torch.cuda.synchronize()
    assert int(off.item()) == 43
    assert torch.equal(a, c) and torch.equal(b, d)
    assert not torch.equal(a, b)


@pytest.mark.parametrize("fmt", ["bf16", "int4"])
def test_step_sampling_matches_oracle(fmt):
    """The whole step with sampling (2 layers, V = 5003): the stored logits
    against the oracle's, and every row's id a valid draw of the oracle's
    distribution with the same u; temperature 0 gives the greedy step's ids."""
    d = synth.ModelDims(n_layers=2, vocab=5003)
    model = synth.make_model(d, fmt, 401, DEV)
    P_list, W = [0, 37, 300], 6
    P = torch.tensor(P_list, dtype=torch.int32)
    cache = synth.make_cache(d, P, W, seed=402, device=DEV)
    ids = synth.draw_window_ids(3, W, d.vocab, 403, device=DEV)
    dm, dc = B.DeviceModel(model), B.DeviceCache(cache, d.n_layers)
    mn, cn = np_tree(model), np_tree(cache)
    mn["dims"] = d
    ref = O.pbd_step(mn, cn, ids.cpu().numpy(), P.numpy())
    lm = oracle_lm(mn)
    zref = ref["final"] @ O.decode_weight(lm).T
    T_, top_p, seed = 0.7, 0.9, 2024
    smp = B.Sampling(T_, top_p, seed, 0)
    out, sel, _ = B.pbd_step(dm, dc, ids, P.to(DEV), max(P_list) + W, sampling=smp)
    greedy, _, _ = B.pbd_step(dm, dc, ids, P.to(DEV), max(P_list) + W)
    out0, _, _ = B.pbd_step(dm, dc, ids, P.to(DEV), max(P_list) + W, sampling=B.Sampling(0.0, top_p, seed))
    torch.cuda.synchronize()
    zg = smp.logits.cpu().numpy().astype(np.float64)
    dz = np.max(np.abs(zg - zref))
    got = out.cpu().numpy().reshape(-1)
    near = sum(check_draw(zref[t], T_, float(np.float32(top_p)), OS.philox_uniform(t, seed, 0), int(got[t]),
                          eps=1e-4) for t in range(got.size))
    _log(f"step sampling {fmt}: max |logit diff| {dz:.1e}; {got.size - near} ids equal, {near} valid near a "
         f"boundary")
    assert dz < 1e-3
    assert torch.equal(out0, greedy)

"""GPU parity at the benchmarked shapes, decode loops checked step by step, and
exact ties in the lm_head.

* Full-size steps: the 36-layer decoder with the 152,681-token tied lm_head,
  in the tiled weight layout the benchmark streams, for the batch-1 prefix-1280
  step, the 32 ragged sequences (prefix 300..4096), INT4 weights at batch 8
  and one sequence at prefix 32768.  Sequences are independent, so where the
  oracle checks a subset of a batch it is the same computation as for all.
* Loops are teacher-forced: before every step the oracle takes the cache, the
  window and the prefix lengths the GPU holds, so each step is compared on
  its own (ids, the K/V it writes, the state after the device-side commit
  exactly) with no drift carried from earlier steps.
* K/V written to the bf16 cache: each value is a rounding decision taken on
  an fp32 value.  Layer 0's values carry no earlier rounding, so they are
  held to one bf16 ulp of the oracle's rounding (entries within 1e-4 of the
  tensor's rms excepted).  A decision taken the other way (the GPU's fp32
  value and the oracle's float64 one straddle a rounding point) is correct on
  both sides but moves what follows, most on a short context (attention over
  a handful of keys); the loops therefore run the oracle following the GPU's
  decisions (the window's K/V read back from the cache, as the prefix is),
  which holds every layer of the 2-layer models to one ulp.  Deeper layers
  carry fp32 accumulation over the earlier layers (about 1e-5 relative), which
  also flips roundings of values near zero: every layer's K/V rows (one
  token's K or V of one head) are held to the rel-L2 bar against the
  oracle's values before rounding, plus the half ulp of the bf16 store.
* Exact ties: copies of a row's winning lm_head row planted at lower and
  higher vocabulary ids, in the same tile and in other workgroups' ranges;
  the lowest index must win.
"""
import numpy as np
import pytest
import torch

import oracle as O
from box_decoding_amd import binding as B
from box_decoding_amd import synth
from helpers import (BF16_HALF_ULP, bf16_kv_mismatch, cache_slots, ids_match, kv_rows_vs_exact, max_abs,
                     np_tree, oracle_lm, rel_l2, rel_l2_rows, step_ids_match)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_BF16 = 2e-3
TOL_INT4 = 5e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()
    torch.cuda.set_device(0)


def _log(msg):
    print(msg, flush=True)


_models = {}


def _full_model(wfmt, seed):
    """The full 36-layer model (tiled layout on the GPU, row-major copy on the
    host for the oracle), built once per module."""
    key = (wfmt, seed)
    if key not in _models:
        d = synth.QWEN25_3B
        m = synth.make_model(d, wfmt, seed, DEV)
        mn = np_tree(m)
        mn["dims"] = d
        packed = B.pack_model(m)
        del m
        torch.cuda.synchronize()
        _models.clear()  # one full model on the GPU at a time
        _models[key] = (B.DeviceModel(packed), mn, packed)
    return _models[key]


def sub_cache_np(cache, seqs):
    """Host copy of the pages of sequences ``seqs`` only (block table renumbered)."""
    bt = cache["block_table"][torch.as_tensor(seqs, device=cache["block_table"].device)]
    S, MB = bt.shape
    idx = bt.clamp(min=0).reshape(-1).long()
    return {"k": cache["k"].index_select(1, idx).cpu().numpy(),
            "v": cache["v"].index_select(1, idx).cpu().numpy(),
            "block_table": np.arange(S * MB, dtype=np.int32).reshape(S, MB),
            "block": int(cache["block"])}


def gpu_window_kv(cache_np, seqs, P, W, n_layers):
    """Per layer, the bf16 K/V the GPU wrote at slots P_b .. P_b+W-1 of the
    sequences seqs (row i of cache_np's block table is sequence seqs[i])."""
    out = []
    for layer in range(n_layers):
        ks, vs = zip(*[cache_slots(cache_np, layer, i, np.arange(int(P[b]), int(P[b]) + W))
                       for i, b in enumerate(seqs)])
        out.append((np.concatenate(ks), np.concatenate(vs)))
    return out


def _full_step(wname, seqs=None, tol=TOL_BF16):
    w = synth.WORKLOADS[wname]
    d = w.dims
    dm, mn, _ = _full_model(w.wfmt, w.model_seed)
    P = synth.draw_prefix_lens(w)
    cache = synth.make_cache(d, P, w.window, seed=w.input_seed, device=DEV)
    ids = synth.draw_window_ids(w.batch, w.window, d.vocab, w.input_seed, device=DEV)
    dc = B.DeviceCache(cache, d.n_layers)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out_ids, gap, hid = B.pbd_step(dm, dc, ids, P.to(DEV), int(P.max()) + w.window,
                                   want_hidden=True, err=err)
    torch.cuda.synchronize()
    seqs = list(range(w.batch)) if seqs is None else list(seqs)
    cn = np_tree(cache) if len(seqs) == w.batch else sub_cache_np(cache, seqs)
    ref = O.pbd_step(mn, cn, ids.cpu().numpy()[seqs], P.numpy()[seqs], return_hidden=True)
    ref["lm"] = oracle_lm(mn)
    W = w.window
    rows = np.concatenate([np.arange(b * W, (b + 1) * W) for b in seqs])
    got_ids = out_ids.cpu().numpy().reshape(-1)[rows]
    n, bad, near = step_ids_match(got_ids, ref)
    h = hid.cpu().numpy()[rows]
    e, er = rel_l2(h, ref["hidden"]), rel_l2_rows(h, ref["hidden"], d.hidden)
    # the window's K/V: layer 0 within one ulp, every layer per row
    cg = cn  # the step wrote slots P_b .. P_b+W-1; the oracle read only the slots before
    kd = vd = 0
    kr = 0.0
    for layer in range(d.n_layers):
        kb, vb = ref["kv"][layer]
        ke, ve = ref["kv_exact"][layer]
        for i, b in enumerate(seqs):
            pos = np.arange(int(P[b]), int(P[b]) + W)
            kg, vg = cache_slots(cg, layer, i, pos)
            if layer == 0:
                kd = max(kd, bf16_kv_mismatch(kg, kb[i * W:(i + 1) * W]))
                vd = max(vd, bf16_kv_mismatch(vg, vb[i * W:(i + 1) * W]))
            kr = max(kr, kv_rows_vs_exact(kg, ke[i * W:(i + 1) * W], d.head_dim),
                     kv_rows_vs_exact(vg, ve[i * W:(i + 1) * W], d.head_dim))
    gd = max_abs(gap.cpu().numpy().reshape(-1)[rows][ref["gap"].reshape(-1) >= 1e-3],
                 ref["gap"].reshape(-1)[ref["gap"].reshape(-1) >= 1e-3])
    _log(f"full step {wname} ({len(seqs)} of {w.batch} sequences checked): hidden rel-L2 {e:.2e} "
         f"(worst row {er:.2e}); ids {n} compared, {bad} bad, {near} near-ties; layer-0 K/V ulp {kd}/{vd}, "
         f"worst K/V row rel-L2 against the unrounded values {kr:.2e}; max |gap diff| {gd:.1e}")
    assert int(err.item()) == 0
    assert bad == 0
    assert e <= tol and er <= tol
    assert kd <= 1 and vd <= 1 and kr <= tol + BF16_HALF_ULP
    assert gd < 1e-3


@pytest.mark.timeout(900)
def test_full_step_b1_p1280():
    """The benchmark's headline shape: batch 1, prefix 1280."""
    _full_step("step_b1_p1280")


@pytest.mark.timeout(900)
def test_full_step_b32_ragged():
    """32 ragged sequences, prefix uniform in [300, 4096], every sequence checked."""
    _full_step("step_b32_ragged")


@pytest.mark.timeout(900)
def test_full_step_int4_b8_p1280():
    """INT4 weights (group 128 linears and lm_head, group-32 embedding), batch 8."""
    _full_step("step_int4_b8_p1280", tol=TOL_INT4)


@pytest.mark.timeout(900)
def test_full_step_probe_b1_p32768():
    """One sequence at prefix 32768."""
    _full_step("probe_b1_p32768")


# ---------------------------------------------------------------- loops, teacher-forced

def _teacher_forced_loop(dm, mn, cache, d, ids, Pd, cr, wl, block, mask, steps, acc, graph, max_len,
                         seqs, refeed, ulp_layers=None, tol=TOL_BF16):
    """Run ``steps`` steps (each a step and its device-side commit) and check
    every one against the oracle run on the state the GPU holds before it.

    refeed=False: la_pbd_step + la_pbd_commit (window [last id, mask x (W-1)],
    prefix += W); refeed=True: la_pbd_step_refeed + la_pbd_commit_refeed with
    n_accept = acc[s] (None: the whole block).  seqs: the sequences the oracle
    recomputes (the commit is checked on all); it follows the GPU's K/V
    rounding decisions; the real rows of the layers in ulp_layers (default
    all) are held to one ulp, of every layer to the rel-L2 bar against the
    values before rounding.  Returns the counts."""
    ulp_layers = range(d.n_layers) if ulp_layers is None else ulp_layers
    nb, W = ids.shape
    out_ids = torch.empty((nb, W), dtype=torch.int32, device=DEV)
    out_gap = torch.empty((nb, W), dtype=torch.float32, device=DEV)
    n_acc = torch.zeros(nb, dtype=torch.int32, device=DEV)
    dc = B.DeviceCache(cache, d.n_layers)
    g = None
    if graph:
        g = B.StepGraph(dm, dc, ids, Pd, max_len, out_ids, out_gap, commit_mask_id=mask,
                        refeed=(cr, wl, block, n_acc if acc is not None else None) if refeed else None)
    tot = dict(ids=0, near=0, kd=0, vd=0, kv_row=0.0)
    for s in range(steps):
        win = ids.cpu().numpy()
        P = Pd.cpu().numpy().astype(np.int64)
        c = cr.cpu().numpy().astype(np.int64) if refeed else np.zeros(nb, dtype=np.int64)
        w = wl.cpu().numpy().astype(np.int64) if refeed else np.full(nb, W, dtype=np.int64)
        before = sub_cache_np(cache, seqs)
        if acc is not None:
            n_acc.copy_(torch.from_numpy(np.asarray(acc[s], dtype=np.int32)))
        if graph:
            g.replay()
        elif refeed:
            B.pbd_step(dm, dc, ids, Pd, max_len, out_ids=out_ids, out_gap=out_gap, causal_rows=cr,
                       window_len=wl)
            B.pbd_commit_refeed(out_ids, ids, Pd, cr, wl, block, mask, n_acc if acc is not None else None)
        else:
            B.pbd_step(dm, dc, ids, Pd, max_len, out_ids=out_ids, out_gap=out_gap)
            B.pbd_commit(out_ids, ids, Pd, mask)
        torch.cuda.synchronize()
        got = out_ids.cpu().numpy()
        # the oracle on the GPU's own state before the step, following the
        # GPU's K/V rounding decisions of this step (read back from the cache)
        after = sub_cache_np(cache, seqs)
        kv_gpu = gpu_window_kv(after, seqs, P, W, d.n_layers)
        ref = O.pbd_step(mn, before, win[seqs], P[seqs], causal_rows=c[seqs] if refeed else None,
                         window_len=w[seqs] if refeed else None, window_kv=kv_gpu)
        ref["lm"] = oracle_lm(mn)
        rows = np.concatenate([np.arange(i * W, i * W + int(w[b])) for i, b in enumerate(seqs)])
        n, bad, near = step_ids_match(got[seqs].reshape(-1), ref, rows=rows)
        assert bad == 0, (s, bad)
        tot["ids"] += n
        tot["near"] += near
        # the K/V the step wrote at slots P_b .. P_b + w_b - 1, every layer
        for layer in range(d.n_layers):
            kb, vb = ref["kv"][layer]
            for i, b in enumerate(seqs):
                pos = np.arange(int(P[b]), int(P[b]) + int(w[b]))
                kg, vg = cache_slots(after, layer, i, pos)
                kr, vr = kb[i * W:i * W + int(w[b])], vb[i * W:i * W + int(w[b])]
                ke, ve = (x[i * W:i * W + int(w[b])] for x in ref["kv_exact"][layer])
                if layer in ulp_layers:
                    kd_, vd_ = bf16_kv_mismatch(kg, kr), bf16_kv_mismatch(vg, vr)
                    if max(kd_, vd_) > 1:
                        rowk = [bf16_kv_mismatch(kg[j:j + 1], kr[j:j + 1]) for j in range(len(pos))]
                        rowv = [bf16_kv_mismatch(vg[j:j + 1], vr[j:j + 1]) for j in range(len(pos))]
                        _log(f"K/V mismatch: step {s} layer {layer} seq {b} P {int(P[b])} c {int(c[b])} "
                             f"w {int(w[b])}: K ulps by row {rowk}, V ulps by row {rowv}")
                    tot["kd"] = max(tot["kd"], kd_)
                    tot["vd"] = max(tot["vd"], vd_)
                tot["kv_row"] = max(tot["kv_row"], kv_rows_vs_exact(kg, ke, d.head_dim),
                                    kv_rows_vs_exact(vg, ve, d.head_dim))
        # the device-side commit, from the GPU's own ids, exactly
        gw, gp = ids.cpu().numpy(), Pd.cpu().numpy().astype(np.int64)
        if refeed:
            ew, ep, ec, el = O.refeed_commit(got, win, P, c, w, block, mask,
                                             None if acc is None else acc[s])
            assert np.array_equal(gw, ew) and np.array_equal(gp, ep), s
            assert np.array_equal(cr.cpu().numpy(), ec) and np.array_equal(wl.cpu().numpy(), el), s
        else:
            ew, ep = O.emission_commit(got, P, mask)
            assert np.array_equal(gw, ew) and np.array_equal(gp, ep), s
    assert tot["kd"] <= 1 and tot["vd"] <= 1 and tot["kv_row"] <= tol + BF16_HALF_ULP, tot
    return tot


@pytest.mark.parametrize("graph", [False, True])
def test_emission_loop_teacher_forced(graph):
    """Window steps committed without re-feeding (la_pbd_commit: the window's
    own K/V stay in the cache), 2 layers, 3 sequences, 4 steps."""
    d = synth.ModelDims(n_layers=2, vocab=3001)
    steps, W, mask = 4, 6, 17
    P0 = [0, 33, 200]
    model = synth.make_model(d, "bf16", 101, DEV)
    mn = np_tree(model)
    mn["dims"] = d
    cache = synth.make_cache(d, torch.tensor(P0), W, extra_tokens=steps * W, seed=102, device=DEV)
    ids = synth.draw_window_ids(len(P0), W, d.vocab, 103, mask_id=mask, device=DEV)
    Pd = torch.tensor(P0, dtype=torch.int32, device=DEV)
    tot = _teacher_forced_loop(B.DeviceModel(model), mn, cache, d, ids, Pd, None, None, W, mask, steps,
                               None, graph, max(P0) + (steps + 1) * W, list(range(len(P0))), False)
    _log(f"emission loop (graph={graph}), teacher-forced: {tot}")
    assert np.array_equal(Pd.cpu().numpy(), np.array(P0) + steps * W)


@pytest.mark.parametrize("graph", [False, True])
def test_refeed_loop_teacher_forced(graph):
    """Re-fed window steps (W = 11: up to 5 re-fed rows, a block of 6, padding)
    with partial acceptance, 2 layers, 3 sequences, 4 steps."""
    d = synth.ModelDims(n_layers=2, vocab=3001)
    steps, W, block, mask = 4, 11, 6, 17
    P0 = [0, 33, 200]
    nb = len(P0)
    acc = [[6, 3, 1], [2, 6, 4], [5, 1, 6], [6, 6, 6]]
    model = synth.make_model(d, "bf16", 111, DEV)
    mn = np_tree(model)
    mn["dims"] = d
    cache = synth.make_cache(d, torch.tensor(P0), W, extra_tokens=steps * W, seed=112, device=DEV)
    first = synth.draw_window_ids(nb, 1, d.vocab, 113, device=DEV)
    ids = torch.full((nb, W), mask, dtype=torch.int32, device=DEV)
    ids[:, 0] = first[:, 0]
    cr = torch.zeros(nb, dtype=torch.int32, device=DEV)
    wl = torch.full((nb,), block, dtype=torch.int32, device=DEV)
    Pd = torch.tensor(P0, dtype=torch.int32, device=DEV)
    tot = _teacher_forced_loop(B.DeviceModel(model), mn, cache, d, ids, Pd, cr, wl, block, mask, steps,
                               acc, graph, max(P0) + (steps + 1) * W, list(range(nb)), True)
    _log(f"re-fed loop (graph={graph}), teacher-forced: {tot}")
    assert np.all(Pd.cpu().numpy() > np.array(P0) + steps)


@pytest.mark.timeout(900)
def test_full_refeed_loop_b16_p2048():
    """The dense-scene loop at its full size: 16 sequences from prefix 2048,
    re-fed windows (W = 11, blocks of 6, every block accepted: each step
    appends 6 accepted tokens' K/V), the captured graph the benchmark replays;
    3 steps, 4 sequences recomputed by the oracle, the commit checked on all."""
    w = synth.WORKLOADS["emit_b16_p2048_x40"]
    d = w.dims
    steps, block = 3, w.window
    W = 2 * block - 1
    dm, mn, _ = _full_model(w.wfmt, w.model_seed)
    P = synth.draw_prefix_lens(w)
    cache = synth.make_cache(d, P, W, extra_tokens=steps * block, seed=w.input_seed, device=DEV)
    first = synth.draw_window_ids(w.batch, block, d.vocab, w.input_seed, device=DEV)
    mask = int(first[0, 1].item())
    ids = torch.full((w.batch, W), mask, dtype=torch.int32, device=DEV)
    ids[:, 0] = first[:, 0]
    cr = torch.zeros(w.batch, dtype=torch.int32, device=DEV)
    wl = torch.full((w.batch,), block, dtype=torch.int32, device=DEV)
    Pd = P.to(DEV)
    tot = _teacher_forced_loop(dm, mn, cache, d, ids, Pd, cr, wl, block, mask, steps, None, True,
                               int(P.max()) + W + steps * block, [0, 5, 10, 15], True, ulp_layers=(0,))
    _log(f"full re-fed loop b16 p2048, teacher-forced: {tot}")
    assert np.array_equal(Pd.cpu().numpy(), P.numpy() + 1 + (steps - 1) * block)


# ---------------------------------------------------------------- exact ties

def _full_logits(f, lm, chunk=16384):
    V = int(lm["n"])
    out = np.empty((f.shape[0], V))
    for v0 in range(0, V, chunk):
        v1 = min(V, v0 + chunk)
        out[:, v0:v1] = f @ O.decode_weight(lm, rows=np.arange(v0, v1)).T
    return out


@pytest.mark.parametrize("fmt,M", [("bf16", 6), ("bf16", 48), ("int4", 48)])
def test_lm_head_planted_exact_ties(fmt, M):
    """Each row's winning vocabulary row is copied to other ids (one in the
    same 16-row tile, one far below, one above): the logits tie exactly, and
    where the tied value leads the rest by >= 1e-3 the GPU must return the
    lowest tied id."""
    V = 152681
    d = synth.ModelDims(n_layers=1, vocab=V)
    m = synth.make_model(d, fmt, seed=79, device=DEV)
    lm = m["lm_head"] if m["lm_head"] is not None else m["embed"]
    h = torch.randn((M, d.hidden), device=DEV, generator=torch.Generator(device=DEV).manual_seed(M))
    gain = m["final_norm"]
    f = O.rmsnorm(h.cpu().numpy().astype(np.float64), O.bf16_to_float(gain.cpu().numpy()), d.rms_eps)
    win0, _, _ = O.lm_head_argmax(f, np_tree(lm))
    rng = np.random.default_rng(7 + M)
    used = set(int(x) for x in win0)
    ties = []
    for t in range(M):
        r = int(win0[t])
        cand = [r - 1 - int(rng.integers(0, r % 16)) if r % 16 else -1,   # same tile, below
                int(rng.integers(0, max(1, r - 20000))),                   # far below
                int(rng.integers(min(r + 1, V - 1), V))]                   # above
        group = [r]
        for c in cand:
            if 0 <= c < V and c not in used:
                used.add(c)
                group.append(c)
        ties.append(group)
        for c in group[1:]:
            lm["data"][c].copy_(lm["data"][r])
            if lm["scales"] is not None:
                lm["scales"][c].copy_(lm["scales"][r])
    torch.cuda.synchronize()
    ids, top1, gap = B.lm_head_argmax(h, lm, norm_gain=gain)
    torch.cuda.synchronize()
    lmn = np_tree(lm)
    logits = _full_logits(f, lmn)
    got = ids.cpu().numpy()
    decisive = 0
    for t in range(M):
        grp = ties[t]
        vals = logits[t, grp]
        assert np.all(vals == vals[0]), t          # the copies tie exactly in the oracle too
        rest = logits[t].copy()
        rest[grp] = -np.inf
        if vals[0] - rest.max() >= 1e-3:
            decisive += 1
            assert got[t] == min(grp), (t, got[t], sorted(grp))
            assert gap.cpu().numpy()[t] == 0.0, t  # a tie at the top: no gap on the GPU either
    rid, rtop, rgap = O.lm_head_argmax(f, lmn)
    n, bad, near = ids_match(got, rid, rgap, rtop, f, lmn)
    _log(f"planted ties {fmt} M={M}: {decisive} decisive tied rows, group sizes "
         f"{sorted(set(len(g) for g in ties))}; ids {n} compared, {bad} bad")
    assert bad == 0 and decisive >= M // 2

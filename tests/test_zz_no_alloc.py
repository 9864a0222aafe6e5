"""la_pbd_step_noalloc (the step on the library's own scratch array, for
callers that cannot allocate) against la_pbd_step with a caller workspace:
bit-identical outputs, on two calls in a row, the second with a smaller
input; and a shape past the array's size is refused."""
import numpy as np
import pytest
import torch

from box_decoding_amd import binding as B
from box_decoding_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()
    torch.cuda.set_device(0)


def _case(dm, d, P_list, W, seed):
    P = torch.tensor(P_list, dtype=torch.int32)
    cache = synth.make_cache(d, P, W, seed=seed, device=DEV)
    ids = synth.draw_window_ids(len(P_list), W, d.vocab, seed + 1, device=DEV)
    dc = B.DeviceCache(cache, d.n_layers)
    Pd = P.to(DEV)
    max_len = int(P.max()) + W
    Bn = len(P_list)
    # the reference: la_pbd_step with a caller workspace
    r_ids, r_gap, r_hid = B.pbd_step(dm, dc, ids, Pd, max_len, want_hidden=True)
    torch.cuda.synchronize()
    out_ids = torch.full((Bn, W), -7, dtype=torch.int32, device=DEV)
    out_gap = torch.full((Bn, W), -7.0, dtype=torch.float32, device=DEV)
    out_hid = torch.full((Bn * W, d.hidden), -7.0, dtype=torch.float32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    B.pbd_step_noalloc(dm, dc, ids, Pd, max_len, out_ids, out_gap, out_hid, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(out_ids, r_ids)
    assert torch.equal(out_gap, r_gap)
    assert torch.equal(out_hid, r_hid)
    return out_ids.cpu().numpy()


def test_step_noalloc_matches_step():
    d = synth.ModelDims(n_layers=2, vocab=5003)
    dm = B.DeviceModel(B.pack_model(synth.make_model(d, "bf16", 301, DEV)))
    # a larger call, then a smaller one: the second runs on the scratch the
    # first left behind
    a = _case(dm, d, [0, 17, 300, 1000], 11, 302)
    b = _case(dm, d, [40], 6, 304)
    print(f"noalloc step: ids {a.shape} then {b.shape} bit-identical to la_pbd_step", flush=True)


def test_step_noalloc_refuses_oversized_shapes():
    d = synth.ModelDims(n_layers=1, vocab=1000)
    dm = B.DeviceModel(synth.make_model(d, "bf16", 305, DEV))
    P = torch.tensor([10] * 64, dtype=torch.int32)
    cache = synth.make_cache(d, P, 16, seed=306, device=DEV)
    dc = B.DeviceCache(cache, d.n_layers)
    ids = torch.zeros((64, 16), dtype=torch.int32, device=DEV)
    out = torch.empty((64, 16), dtype=torch.int32, device=DEV)
    # 64 sequences x 16 rows over a 60000-key bound needs far more than the array
    with pytest.raises(B.LaError, match="workspace"):
        B.pbd_step_noalloc(dm, dc, ids, P.to(DEV), 60000, out)

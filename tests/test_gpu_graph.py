"""The sparse forward captured as a HIP graph and replayed (torch.cuda.CUDAGraph
over the library's launches on the capturing stream).

Every replay, with the program's own eager work and synchronisations in
between, must give the eager forward's y bit for bit, and the TwELL as well;
the library records no memset nodes and no host synchronisation in the
forward, so a replay is the same launches as an eager call.
"""
import pytest
import torch

from gpu_util import dev, layer, twell_np, valid_slots
from unstructured_sparse_feedforward_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _eq(a, b):
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("w,T,store", [(wl.GATED_1P5B, 2048, "f32"),
                                       (wl.GATED_1P5B, 1500, "bf16"),
                                       (wl.NONGATED[29], 1024, "f32")])
def test_forward_graph_replays(w, T, store):
    print(f"graph {w.name} T={T} store={store}", flush=True)
    inp = wl.make_inputs(w, seed=31, T=T)
    ffn = layer(inp, store_dtype=torch.bfloat16 if store == "bf16" else torch.float32)
    args = [dev(inp, k) for k in ("x", "w_gate", "w_up", "w_down")]
    tw = ffn.new_twell(T)
    y = torch.empty((T, w.d), dtype=torch.float32, device="cuda")
    ffn.forward(*args, mode="sparse", tw=tw, y=y)          # checked: capacities hold
    torch.cuda.synchronize()
    ref_y = y.clone()
    ref_tw = twell_np(tw)
    assert ref_tw["n_flagged"] > 0 or not w.outlier_frac

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ffn.forward(*args, mode="sparse", tw=tw, y=y, check=False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ffn.forward(*args, mode="sparse", tw=tw, y=y, check=False)

    for rep in range(4):
        # eager work between the replays: clobber the outputs, run an
        # unrelated reduction, synchronise
        y.fill_(float("nan"))
        for k in ("val", "idx", "cnt"):
            tw[k].zero_()
        _ = torch.sum(args[0].float())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _eq(y, ref_y), f"replay {rep}: y differs from the eager forward"
        got = twell_np(tw)
        assert (got["cnt"] == ref_tw["cnt"]).all(), f"replay {rep}: TwELL counts differ"
        m = valid_slots(ref_tw)
        for k in ("idx", "val"):
            assert (got[k][m] == ref_tw[k][m]).all(), f"replay {rep}: TwELL {k} differs"
    # and an eager call after the replays still agrees
    ffn.forward(*args, mode="sparse", tw=tw, y=y)
    assert _eq(y, ref_y)

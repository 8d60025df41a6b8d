"""cf_topk_select_noalloc (the selection entry point that allocates nothing, for callers under HIP
graph capture or in loops that cannot allocate) against cf_topk_select with a caller workspace:
bit-identical selections on two calls in a row, the second with a smaller input, for token top-k
on the whole-GPU path (n >= 65536, which uses the scratch), on the one-workgroup path, and for
document-aligned spans; a selection whose scratch would exceed the fixed array is rejected on the
host before anything is enqueued; and the call captured in a HIP graph replays correctly on new values."""
import numpy as np
import pytest

import selective_recompute_cf_amd as cf
from tests._gpu import say

pytestmark = pytest.mark.gpu


def _pair(d, k, mode, spans=None):
    import torch
    a = torch.full((max(k, 1),), -1, dtype=torch.int32, device="cuda")
    b = torch.full((max(k, 1),), -2, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(cf.topk_workspace_size(d.numel(), mode), 1), dtype=torch.uint8, device="cuda")
    cf.topk_select(d, k, a, mode, spans, ws)
    cf.topk_select_noalloc(d, k, b, mode, spans)
    torch.cuda.synchronize()
    return a.cpu().numpy()[:k], b.cpu().numpy()[:k]


@pytest.mark.parametrize("mode,sizes", [("token", [3_000_017, 200_003]), ("token", [70_000, 65_536]),
                                        ("token", [5000, 333]), ("doc", [500_000, 40_001])])
def test_noalloc_selection_equals_workspace_call(mode, sizes):
    import torch
    for i, n in enumerate(sizes):
        g = torch.Generator().manual_seed(11 + i)
        d = torch.rand(n, generator=g)
        d[torch.randint(0, n, (n // 50,), generator=g)] = 0.5  # heavy ties at one value
        d = d.cuda()
        k = max(1, n * 15 // 100)
        spans = None
        if mode == "doc":
            cuts = np.unique(np.random.default_rng(i).integers(1, n, 200))
            spans = [0] + cuts.tolist() + [n]
        say(f"noalloc {mode} n={n} k={k}")
        want, got = _pair(d, k, mode, spans)
        np.testing.assert_array_equal(got, want)
        assert np.all(np.diff(got) > 0)


def test_noalloc_rejects_selections_beyond_the_scratch():
    import torch
    n = 600_000  # document-aligned spans keep (n + 1) fp64 running sums: beyond the 4 MiB scratch
    d = torch.rand(n, device="cuda")
    out = torch.full((10,), -3, dtype=torch.int32, device="cuda")
    with pytest.raises(cf.CfError) as e:
        cf.topk_select_noalloc(d, 10, out, "doc", [0, n // 2, n])
    assert e.value.status == cf.CF_EWORKSPACE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == -3).all())


@pytest.mark.parametrize("n,k", [(3_000_017, 450_002), (5000, 750)])
def test_noalloc_selection_replays_from_a_hip_graph(n, k):
    """The callers this entry point is for include code under HIP graph capture: captured once (on
    the whole-GPU path and on the one-workgroup path), then replayed three times with new values
    copied into the captured input, with eager calls and syncs in between; every replay equals a
    workspace call on the same values."""
    import torch
    d = torch.empty(n, device="cuda")
    out = torch.full((k,), -1, dtype=torch.int32, device="cuda")
    want = torch.full((k,), -2, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(cf.topk_workspace_size(n, "token"), 1), dtype=torch.uint8, device="cuda")

    def values(seed):
        g = torch.Generator().manual_seed(seed)
        v = torch.rand(n, generator=g)
        v[torch.randint(0, n, (n // 50,), generator=g)] = 0.5  # ties at one value
        return v.cuda()

    d.copy_(values(31))
    side = torch.cuda.Stream()  # warm-up off the capture: the scratch address is looked up here
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        cf.topk_select_noalloc(d, k, out, "token")
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cf.topk_select_noalloc(d, k, out, "token")
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"noalloc graph n={n} replay {rep}")
        d.copy_(values(32 + rep))
        out.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        cf.topk_select(d, k, want, "token", None, ws)  # eager, with a workspace, between replays
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        np.testing.assert_array_equal(got, want.cpu().numpy())
        assert np.all(np.diff(got) > 0)

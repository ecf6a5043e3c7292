"""moe_forward captured in a HIP graph: the library enqueues only kernels on
the caller's stream (no allocation, no host synchronisation, no memset), so
a captured forward replays the whole path.  Every replay, with new inputs
copied into the captured buffers and eager work between replays, must equal
the eager forward on the same inputs bit for bit."""

import pytest
import torch

import mixture_experts_layer_28_amd as moe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# (T, H, I, E, k, renorm): decode-sized segments (32-row tiles) and
# prefill-sized ones (N >= 96 E: the large-tile kernel)
CASES = [(48, 256, 384, 16, 4, False), (400, 256, 384, 4, 2, True)]


@pytest.mark.parametrize("T,H,I,E,k,renorm", CASES)
def test_graph_replays_match_eager(T, H, I, E, k, renorm):
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(T + E)

    def rnd(*shape, scale=1.0):
        return (torch.randn(*shape, device=dev, generator=g) * scale).to(
            torch.bfloat16)

    wg, wu = rnd(E, I, H, scale=H ** -0.5), rnd(E, I, H, scale=H ** -0.5)
    wd = rnd(E, H, I, scale=I ** -0.5)
    x, logits = rnd(T, H), rnd(T, E)
    ws = torch.empty(moe.moe_forward_workspace_size(T, H, I, E, k, x.dtype),
                     dtype=torch.uint8, device=dev)
    out = torch.empty(T, H, dtype=x.dtype, device=dev)

    def fwd():
        moe.moe_forward(x, logits, wg, wu, wd, k, renorm, out=out,
                        workspace=ws)

    fwd()  # first launches outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd()
    torch.cuda.synchronize()

    for rep in range(4):
        x_new, lg_new = rnd(T, H), rnd(T, E)
        if rep == 3:
            lg_new[:3] = float("nan")  # poisoned rows through the graph too
        want = moe.moe_forward(x_new, lg_new, wg, wu, wd, k, renorm)
        torch.cuda.synchronize()
        x.copy_(x_new)
        logits.copy_(lg_new)
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        _ = (want.float() * 2).sum().item()  # eager work between replays
        same = torch.equal(torch.isnan(got), torch.isnan(want)) and torch.equal(
            torch.nan_to_num(got), torch.nan_to_num(want))
        assert same, "replay %d differs from the eager forward" % rep

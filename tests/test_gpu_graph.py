"""The forward under HIP graph capture: a captured fmlp_forward (or
fmlp_forward_noalloc) replays several times, with the program's own eager
work and synchronisations in between, and every replay equals the eager
result bit for bit (the library
clears its split-K counters with a kernel, not a memset, and allocates
nothing, so a captured call is a fixed sequence of kernels)."""
import pytest
import torch

from swiglu_mlp_rmsnorm_amd import fmlp as F
from swiglu_mlp_rmsnorm_amd import synth

from parity_util import Bf16Layer, Int4Layer, bf16_inputs

pytestmark = pytest.mark.gpu
EPS = synth.EPS


def _graph_matches_eager(run, outs, replays=4):
    """run() launches the forward on the current stream into the tensors
    `outs`; capture it, replay it, and compare each replay with eager."""
    run()  # first call outside capture (one-time attribute setup)
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i in range(replays):
        for o in outs:
            o.fill_(float("nan"))              # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o.view(torch.int16), w.view(torch.int16)), f"replay {i} differs"


@pytest.mark.parametrize("d,ff,M", [(1024, 2048, 1),     # decode, split-K down (counters)
                                    (1024, 2048, 20),    # decode, larger-M configuration
                                    (256, 704, 70)])     # prefill
def test_graph_replay_bf16(d, ff, M):
    layer = Bf16Layer(d, ff, 81)
    x, g = bf16_inputs(M, d, 82)
    y = torch.empty((M, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(F.fmlp_workspace_size(M, d, ff, F.FMLP_W_BF16), dtype=torch.uint8,
                     device="cuda")

    def run():
        F.fmlp_forward(x, g, EPS, layer.wgu_t, layer.wd_t, y=y, workspace=ws,
                       stream=torch.cuda.current_stream())
    _graph_matches_eager(run, [y])


@pytest.mark.parametrize("M", [1, 16, 40])
def test_graph_replay_int4_with_residual(M):
    d, ff = 1024, 2048
    layer = Int4Layer(d, ff, 83)
    x, g = bf16_inputs(M, d, 84)
    res = synth.activations(M, d, 85, "cuda")
    y = torch.empty((M, d), dtype=torch.bfloat16, device="cuda")
    h = torch.empty((M, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(F.fmlp_workspace_size(M, d, ff, F.FMLP_W_INT4_G32), dtype=torch.uint8,
                     device="cuda")

    def run():
        layer.forward_ex(x, g, EPS, y=y, workspace=ws, activation=F.FMLP_ACT_GELU_TANH,
                         residual=res, h_out=h, stream=torch.cuda.current_stream())
    _graph_matches_eager(run, [y, h])


@pytest.mark.parametrize("d,ff,M", [(1024, 2048, 1),     # decode, split-K down (counters)
                                    (256, 704, 70)])     # prefill
def test_graph_replay_noalloc(d, ff, M):
    # the entry point without a workspace is meant for captured code: every
    # replay reuses the library's device scratch and equals the eager result
    layer = Bf16Layer(d, ff, 86)
    x, g = bf16_inputs(M, d, 87)
    y = torch.empty((M, d), dtype=torch.bfloat16, device="cuda")

    def run():
        F.fmlp_forward_noalloc(x, g, EPS, layer.wgu_t, layer.wd_t, y=y,
                               stream=torch.cuda.current_stream())
    _graph_matches_eager(run, [y])
    ws = torch.empty(F.fmlp_workspace_size(M, d, ff, F.FMLP_W_BF16), dtype=torch.uint8,
                     device="cuda")
    y_ws = F.fmlp_forward(x, g, EPS, layer.wgu_t, layer.wd_t, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ws.view(torch.int16))

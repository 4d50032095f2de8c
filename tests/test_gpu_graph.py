"""The forward captured in a HIP graph and replayed, through the C ABI.

A caller that captures the layer (torch.cuda.CUDAGraph records the launches libssd makes on
the capture stream) must get, at every replay, what an eager call on the same inputs gives.
Both forward entry points are captured: ssd_fwd with a workspace the caller allocated
before the capture, and ssd_fwd_noalloc, whose stage buffers live in the library's fixed
device array.  Between replays the test copies new inputs into the captured buffers and
runs eager work of its own (filling the outputs with NaN), so a replay that reused stale
state, skipped a kernel or depended on the first replay's memory would show.  The forward
issues no memset, so nothing in the graph is a memset node."""
import numpy as np
import pytest
import torch

from mamba_ssd_chunked_03_amd import binding
from mamba_ssd_chunked_03_amd.workloads import Workload, generate
from parity import say, to_device

pytestmark = pytest.mark.gpu

LN = np.log
# slow decay, so that the state carried across chunks reaches the output; ragged last chunk
W_A = Workload("graph_a", 2, 1024 + 77, 8, 64, 128, 2, 256, init_state=True,
               log_neg_a_range=(LN(0.005), LN(0.05)))
W_B = Workload("graph_b", 2, 1024 + 77, 8, 64, 128, 2, 256, init_state=True, seed=1,
               log_neg_a_range=(LN(0.005), LN(0.05)))


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    binding.library()
    torch.cuda.init()


@pytest.mark.parametrize("entry", ["ssd_fwd", "ssd_fwd_noalloc"])
def test_forward_graph_replays_match_eager_calls(entry):
    say(f"[graph] {entry}: {W_A.describe()}")
    src_a, src_b = to_device(generate(W_A)), to_device(generate(W_B))
    Q = W_A.chunk_len
    inp = {k: v.clone() for k, v in src_a.items() if v is not None}  # the captured buffers
    d = binding.dims_of(inp["x"], inp["B"])
    ws = torch.empty(max(binding.ssd_fwd_workspace_size(d, Q), 1), dtype=torch.uint8,
                     device="cuda")
    y = torch.empty_like(inp["x"])
    fin = torch.empty(W_A.batch, W_A.nheads, W_A.dstate, W_A.headdim, device="cuda")

    def call():
        args = (inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], Q)
        if entry == "ssd_fwd":
            binding.ssd_fwd(*args, init_state=inp["init_state"], y=y, final_state=fin,
                            workspace=ws)
        else:
            binding.ssd_fwd_noalloc(*args, init_state=inp["init_state"], y=y, final_state=fin)

    def load(src):
        for k, v in inp.items():
            v.copy_(src[k])

    refs = []
    for src in (src_a, src_b):
        load(src)
        call()
        torch.cuda.synchronize()
        refs.append((y.clone(), fin.clone()))
    assert not torch.equal(refs[0][0], refs[1][0])  # the two inputs give different outputs

    # a warm-up call on a side stream, then the capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()

    for rep, k in enumerate((0, 1, 0, 1, 1)):
        load(src_a if k == 0 else src_b)
        y.fill_(float("nan"))
        fin.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        same = torch.equal(y, refs[k][0]) and torch.equal(fin, refs[k][1])
        say(f"    replay {rep} (inputs {'ab'[k]}): {'equal' if same else 'DIFFERENT'}")
        assert same, (entry, rep)

"""A block's steps captured into a HIP graph (through torch.cuda.CUDAGraph)
replay bit for bit like the eager calls: the library allocates nothing and
issues no memset, so it is capturable.  Each replay is checked, with eager
work and synchronisations between the replays."""
import numpy as np
import pytest
import torch

from cached_attention_amd import workloads as wl
from cached_attention_amd.session import AttentionStep

pytestmark = pytest.mark.gpu


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device="cuda", dtype=torch.bfloat16)


@pytest.mark.parametrize("shape,sparse", [("text", False), ("text", True), ("frame", False)],
                         ids=["text", "text_sparse", "frame"])
def test_block_graph_replays_match_eager(shape, sparse):
    if shape == "text":
        w = wl.ci_version(wl.WORKLOADS["text_gqa_128k"], prefix_len=1500, hq=8, hkv=2, block_len=16, batch=2)
        w = wl.replace(w, ragged=0.25, steps=4)
    else:   # 16 heads x 1190-token block: the 80-row key-group block pass
        w = wl.ci_version(wl.WORKLOADS["video_1560"], prefix_len=600, hq=16, hkv=16, block_len=1190, n_blocks=1)
        w = wl.replace(w, steps=4)
    prefix, blocks = wl.make_inputs(w)
    blk = blocks[0]
    chunks = torch.tensor([[[0, 7], [3, 11]], [[2, 5], [1, 9]]], dtype=torch.int32) if sparse else None
    kp, vp = dev(prefix.k), dev(prefix.v)
    steps = [(dev(blk.q[s]), dev(blk.k[s]), dev(blk.v[s])) for s in range(w.steps)]

    def make():
        return AttentionStep("bf16", w.batch, w.hq, w.hkv, w.head_dim, w.block_len, prefix.offsets, chunks=chunks)

    def run(st, s, stream=None):
        q, k, v = steps[s]
        st.step(q, k, v, kp, vp, s, 2, stream=stream)

    # eager reference: the output of every step
    eager = make()
    ref = []
    for s in range(w.steps):
        run(eager, s)
        ref.append((eager.o.clone(), eager.lse.clone()))
    torch.cuda.synchronize()
    # one graph per step on a second state
    st = make()
    graphs = []
    cs = torch.cuda.Stream()
    for s in range(w.steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cs):
            with torch.cuda.graph(g, stream=cs):
                run(st, s, stream=torch.cuda.current_stream())
        graphs.append(g)
    torch.cuda.synchronize()
    for rep in range(3):
        for s in range(w.steps):
            graphs[s].replay()
            torch.cuda.synchronize()
            assert torch.equal(st.o, ref[s][0]), f"replay {rep}, step {s}: O differs"
            assert torch.equal(st.lse, ref[s][1]), f"replay {rep}, step {s}: LSE differs"
            # eager work between replays: another state's step, and a torch op
            run(eager, s)
            torch.cuda.synchronize()
            st.o.float().sum().item()

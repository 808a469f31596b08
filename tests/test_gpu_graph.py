"""HIP-graph capture and replay of the C-ABI forward (the way the benchmark
times it).

A graph of several forwards over different inputs, sharing one workspace, is
captured once and replayed several times with eager work of the program
(other forwards, torch kernels, host synchronisations) between the replays.
Every replay must reproduce the eager outputs bit for bit: the kernels are
deterministic for a fixed shape and split count, and the path records no
memset node. Covers split and unsplit shapes, both ring disciplines, the K
repack (N % 8 != 0), the QK-normalised variant and the grouped combine
(32 splits and more).
"""
import numpy as np
import pytest

from gqa_attention_split_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu

CASES = [
    # B, M, N, D, splits, qk_norm
    (16, 256, 4096, 64, 0, False),   # the benchmark workload: 64-row shared ring, 4 splits
    (4, 256, 2048, 64, 1, False),    # 64-row tiles over the whole key range
    (2, 256, 4100, 64, 0, False),    # N % 8 != 0: K repacked into the workspace first
    (3, 8, 3000, 64, 0, False),      # decode rows: 32-row private ring
    (8, 1, 1032, 128, 0, False),     # head dim 128
    (2, 64, 1032, 64, 0, True),      # QK-normalised
    (2, 256, 32768, 64, 0, False),   # long keys: 32 splits, the grouped combine
    (2, 256, 32768, 64, 0, True),    # the same through the QK-normalised (lse) grouped combine
]


@pytest.mark.parametrize("B,M,N,D,splits,qkn", CASES)
def test_graph_replays_match_eager(gpu, B, M, N, D, splits, qkn):
    import torch

    import gqa_attention_split_amd as mga

    dev = gpu
    copies = 3
    inputs = []
    for c in range(copies):
        q, k, v = make_qkv(B, M, N, seed=700 + c, qk_std=1.0 if qkn else 0.25, D=D)
        inputs.append(tuple(torch.from_numpy(x).to(dev) for x in (q, k, v)))
    outs = [torch.empty(B, M, D, dtype=torch.float16, device=dev) for _ in range(copies)]
    ws = mga.workspace_for(B, M, N, D, splits, device=dev, qk_norm=qkn)
    stream = torch.cuda.Stream()

    def step(c):
        q, k, v = inputs[c]
        mga.gqa_forward(q, k, v, out=outs[c], splits=splits, workspace=ws, stream=stream,
                        qk_norm=qkn, eps=1e-6)

    with torch.cuda.stream(stream):
        for c in range(copies):
            step(c)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    assert all(torch.isfinite(o.float()).all().item() for o in eager)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in range(copies):
            step(c)
    torch.cuda.synchronize()

    scratch = torch.randn(1 << 20, device=dev)
    for r in range(4):
        for o in outs:
            o.fill_(float("nan"))
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        for c in range(copies):
            a = outs[c].cpu().numpy().view(np.uint16)
            b = eager[c].cpu().numpy().view(np.uint16)
            assert np.array_equal(a, b), f"replay {r}, input copy {c}: output differs from eager"
        # eager work of the program between replays: another forward on the
        # same workspace, a torch kernel, a host synchronisation
        with torch.cuda.stream(stream):
            step(r % copies)
        scratch.mul_(1.0001)
        torch.cuda.synchronize()

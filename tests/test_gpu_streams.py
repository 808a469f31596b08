"""Several forwards in flight at once on different HIP streams, each with its
own workspace and output: the library keeps no per-call state on the device
(the workspace is the caller's), so every result equals the one the same call
gives alone, bit for bit."""
import numpy as np
import pytest

from gqa_attention_split_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu

CASES = [
    # B, M, N, D, splits, qk_norm
    (16, 256, 4096, 64, 0, False),
    (2, 256, 8192, 64, 0, False),
    (8, 8, 3000, 64, 0, False),
    (16, 1, 2048, 128, 0, False),
    (4, 64, 1032, 64, 0, True),
    (3, 100, 1001, 64, 3, False),
]


def test_concurrent_streams_match_solo_calls(gpu):
    import torch

    import gqa_attention_split_amd as mga

    inputs, outs, wss, solo = [], [], [], []
    for c, (B, M, N, D, s, qkn) in enumerate(CASES):
        q, k, v = make_qkv(B, M, N, seed=900 + c, qk_std=1.0 if qkn else 0.25, D=D)
        inputs.append(tuple(torch.from_numpy(x).to(gpu) for x in (q, k, v)))
        outs.append(torch.empty(B, M, D, dtype=torch.float16, device=gpu))
        wss.append(mga.workspace_for(B, M, N, D, s, device=gpu, qk_norm=qkn))
    for c, (B, M, N, D, s, qkn) in enumerate(CASES):
        q, k, v = inputs[c]
        solo.append(mga.gqa_forward(q, k, v, splits=s, qk_norm=qkn, eps=1e-6).clone())
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in CASES]
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        for c, (B, M, N, D, s, qkn) in enumerate(CASES):
            q, k, v = inputs[c]
            with torch.cuda.stream(streams[c]):
                for _ in range(4):  # several calls queued per stream, overlapping the others
                    mga.gqa_forward(q, k, v, out=outs[c], splits=s, workspace=wss[c],
                                    stream=streams[c], qk_norm=qkn, eps=1e-6)
        torch.cuda.synchronize()
        for c in range(len(CASES)):
            a = outs[c].cpu().numpy().view(np.uint16)
            b = solo[c].cpu().numpy().view(np.uint16)
            assert np.array_equal(a, b), f"case {CASES[c]} repetition {rep}: differs from its solo call"

"""mga_gqa_forward_noalloc, the entry point whose workspace is the library's
own device scratch (for callers that cannot allocate), against
mga_gqa_forward_strided with a caller-owned workspace: the outputs must be
bitwise equal (same kernels, same plan) and within the contract tolerance of
the fp64 oracle, on consecutive calls that reuse the scratch, the later ones
with smaller inputs and other layouts (split partials, the K copy of a
contiguous K with N % 8 != 0, head dim 128)."""
import numpy as np
import pytest

import gqa_attention_split_amd as mga
import oracle
from gqa_attention_split_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu

CALLS = [
    # B, M, N, D, splits -- in this order, one after another on the same scratch
    (16, 256, 4096, 64, 0),   # the benchmark shape: 4 splits, 2.2 MB of partials
    (2, 100, 1000, 64, 3),    # smaller, other split count
    (3, 40, 1003, 64, 0),     # N % 8 != 0: K copied into the scratch first
    (4, 1, 1032, 128, 2),     # head dim 128
]


def test_noalloc_matches_the_workspace_entry_point(gpu):
    import torch

    stream = torch.cuda.Stream()
    for B, M, N, D, splits in CALLS:
        q, k, v = make_qkv(B, M, N, seed=900 + B + N, qk_std=0.25, D=D)
        tq, tk, tv = (torch.from_numpy(x).to(gpu) for x in (q, k, v))
        need = mga.mga_gqa_workspace_bytes(B, M, N, D, splits)
        assert need <= mga.NOALLOC_SCRATCH_BYTES
        print(f"[noalloc] B={B} M={M} N={N} D={D} splits={splits} workspace={need}", flush=True)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=gpu)
        o_ws = torch.full((B, M, D), float("nan"), dtype=torch.float16, device=gpu)
        o_na = torch.full((B, M, D), float("nan"), dtype=torch.float16, device=gpu)
        with torch.cuda.stream(stream):
            rc = mga.mga_gqa_forward_strided(tq, tk, tv, o_ws, B, M, N, D, None, splits, ws, ws.numel(), stream)
            assert rc == mga.MGA_OK, mga.mga_status_string(rc)
            rc = mga.mga_gqa_forward_noalloc(tq, tk, tv, o_na, B, M, N, D, None, splits, stream)
            assert rc == mga.MGA_OK, mga.mga_status_string(rc)
        torch.cuda.synchronize()
        a = o_na.cpu().numpy()
        b = o_ws.cpu().numpy()
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), "noalloc output differs from the workspace path"
        ref = oracle.gqa_f64(q, k, v)
        err = np.abs(a.astype(np.float64) - ref)
        assert np.isfinite(a).all()
        assert (err <= 1e-3 + 5e-3 * np.abs(ref)).all(), f"max err {err.max():.3e}"

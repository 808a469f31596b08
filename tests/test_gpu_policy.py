"""The split policy sizes the grid to the current device's compute units.

On a GPU the planning calls ask the runtime for the compute-unit count; on
MI355X in its default mode that is 256 and the policy's choices at the
benchmark shapes are the ones the tile rule documents (one workgroup per
compute unit, two for the 32-row shape).
"""
import pytest

pytestmark = pytest.mark.gpu


def ceil_div(a, b):
    return -(-a // b)


def test_policy_fills_the_device(gpu):
    import torch

    import gqa_attention_split_amd as mga

    cus = torch.cuda.get_device_properties(gpu).multi_processor_count
    assert cus > 0
    # 64-row tiles over split keys at (16, 256, 4096): 64 tiles, splits fill
    # the chip (at most 8 for 32 key blocks of 128), unless 256- or 128-row
    # tiles alone already fill it (16 or 32 of them) -- then no split
    rc, rows, splits = mga.mga_gqa_plan(16, 256, 4096, 64, 0)
    assert rc == 0
    if cus <= 16:
        assert (rows, splits) == (256, 1)
    elif cus <= 32:
        assert (rows, splits) == (128, 1)
    else:
        assert rows == 64 and splits == min(ceil_div(cus, 64), 8)
    # 32-row tiles, two per compute unit, at (64, 8, 8192): 64 tiles
    rc, rows, splits = mga.mga_gqa_plan(64, 8, 8192, 64, 0)
    assert rc == 0 and rows == 32 and splits == min(ceil_div(2 * cus, 64), 16)
    if cus == 256:  # MI355X, single partition
        assert mga.mga_gqa_plan(16, 256, 4096, 64, 0) == (0, 64, 4)
        assert mga.mga_gqa_plan(2, 256, 32768, 64, 0) == (0, 64, 32)
        assert mga.mga_gqa_plan(128, 256, 16384, 64, 0) == (0, 128, 1)

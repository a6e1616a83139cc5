"""The Python binding rejects bad tensors before reaching the C ABI (no GPU needed)."""

import pytest
import torch

import online_softmax_09_amd as osm


def test_rejects_cpu_tensors():
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        osm.fa_fwd(q, q, q)
    x = torch.zeros(4, 8, dtype=torch.float32)
    with pytest.raises(TypeError):
        osm.online_softmax_rows(x)


def test_rejects_wrong_dtype():
    q = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    with pytest.raises(TypeError):
        osm.fa_fwd(q, q, q)
    with pytest.raises(TypeError):
        osm.fa_fwd_f32(q, q, q)


def test_rejects_non_tensors_and_bad_rank():
    with pytest.raises(TypeError):
        osm.fa_fwd([1.0], [1.0], [1.0])
    q = torch.zeros(1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises((TypeError, ValueError)):
        osm.fa_fwd(q, q, q)


def test_library_path_is_in_tree():
    import os

    assert os.path.dirname(osm.library_path()) == os.path.dirname(osm.__file__)

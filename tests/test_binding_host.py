"""Host-side logic of the ctypes binding (no GPU): outputs allocated beside
a strided input take its row stride (the C ABI passes one stride for both),
and outputs given with other strides are refused before any call."""
import pytest
import torch

import tp_invariant_numerics_amd as tb


def test_rows_like_keeps_the_row_stride():
    x = torch.zeros((3, 10), dtype=torch.bfloat16)[:, :7]
    y = tb._rows_like(x)
    assert y.shape == x.shape and y.stride() == x.stride()
    q = torch.zeros((5, 32), dtype=torch.bfloat16)[:, :16].unflatten(1, (2, 8))
    y = tb._rows_like(q)
    assert y.shape == q.shape and y.stride() == q.stride()
    c = torch.zeros((4, 6), dtype=torch.bfloat16)
    assert tb._rows_like(c).stride() == c.stride()


def test_same_rows_refuses_other_strides():
    x = torch.zeros((3, 10), dtype=torch.bfloat16)[:, :7]
    tb._same_rows(tb._rows_like(x), x, "y")
    with pytest.raises(ValueError):
        tb._same_rows(torch.zeros((3, 7), dtype=torch.bfloat16), x, "y")

"""Host logic of the Python binding (no GPU): the row stride handed to the
C calls for tensors with padded rows, size-1 dimensions of arbitrary stride
and a single row."""
import numpy as np
import pytest
import torch

from proposal_sv_verify_amd import _row_stride


def test_contiguous_and_padded_rows():
    x = torch.zeros(3, 5, 7)
    assert _row_stride(x, 2, "x") == 7
    big = torch.zeros(3, 5, 12)
    assert _row_stride(big[..., :7], 2, "x") == 12
    assert _row_stride(big[..., 2:9], 2, "x") == 12
    tok = torch.zeros(4, 100, dtype=torch.int32)
    assert _row_stride(tok[:, :37], 1, "tok") == 100


def test_size_one_dims_take_any_stride():
    # numpy gives a new axis of size 1 a zero stride; torch keeps it
    a = np.zeros((6, 9), np.float32)
    x = torch.from_numpy(np.ascontiguousarray(a[:, None, :]))
    assert x.shape == (6, 1, 9)
    assert _row_stride(x, 2, "x") == 9
    one = torch.from_numpy(np.zeros(300, np.int32)[None, :])
    assert one.stride(0) in (0, 300)
    assert _row_stride(one, 1, "tok") == 300              # a single context: its length
    single = torch.zeros(1, 1, 5).as_strided((1, 1, 5), (0, 0, 1))
    assert _row_stride(single, 2, "x") == 5
    # K + 1 = 1 rows with the batch stride doing the spacing
    b = torch.zeros(40).as_strided((4, 1, 8), (10, 3, 1))
    assert _row_stride(b, 2, "x") == 10


def test_uneven_rows_and_inner_stride_are_rejected():
    x = torch.zeros(5, 3, 7).transpose(0, 1)               # rows not evenly spaced
    with pytest.raises(ValueError):
        _row_stride(x, 2, "x")
    y = torch.zeros(4, 9)[:, ::2]                          # inner stride 2
    with pytest.raises(ValueError):
        _row_stride(y, 1, "y")
    with pytest.raises(ValueError):
        _row_stride(torch.zeros(4, 9), 2, "z")             # wrong rank


def test_single_row_takes_the_partner_stride():
    """A draft tensor of one row ([1, 1, V]) is passed with a target whose
    rows are padded: its own stride is unconstrained, so it takes the
    target's."""
    big = torch.zeros(1, 3, 12)
    target = big[:, :2, :7]                                # rows 12 apart
    draft = big[:, 2:, :7]                                 # one row
    assert _row_stride(target, 2, "t") == 12
    assert _row_stride(draft, 2, "d") == 7
    assert _row_stride(draft, 2, "d", single=12) == 12
    two = torch.zeros(2, 1, 12)[..., :7]                   # two rows: the stride is fixed
    assert _row_stride(two, 2, "d", single=99) == 12

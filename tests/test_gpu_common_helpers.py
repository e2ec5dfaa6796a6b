"""The bitwise comparison helper of the GPU tests, on CPU tensors: equal tensors pass (NaN
included); a planted difference is reported with its count, first index and values."""
import pytest

from tests.gpu_common import assert_same_bits

torch = pytest.importorskip("torch")


def test_equal_tensors_pass_nan_included():
    a = torch.randn(3, 4, 5)
    a[1, 2, 3] = float("nan")
    assert_same_bits(a, a.clone(), "fp32")
    b = torch.randn(6, 7).to(torch.bfloat16)
    assert_same_bits(b, b.clone(), "bf16")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_a_difference_is_reported_with_its_index_and_values(dtype):
    a = torch.zeros(4, 8, dtype=dtype)
    b = a.clone()
    b[2, 5] = 1.5
    b[3, 0] = -0.0  # differs from +0.0 in its bits only
    with pytest.raises(AssertionError) as e:
        assert_same_bits(a, b, "planted")
    msg = str(e.value)
    assert "planted: 2 of 32 elements differ; first at (2, 5): 0.0" in msg and "1.5" in msg


def test_shape_mismatch_is_reported():
    with pytest.raises(AssertionError, match="shapes"):
        assert_same_bits(torch.zeros(2, 3), torch.zeros(3, 2), "shapes differ")

"""The torch binding's argument checks (raised before anything is
enqueued): tensors of one call on one device, the error word a single int32
element on that device, the combine's row weights covering every row id the
kernel may read, outputs as large as the kernels write."""

import pytest
import torch

from co_activation_amd import ops

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib(built_lib):
    assert torch.cuda.is_available()
    return built_lib


def test_combine_row_weight_must_cover_z():
    z = torch.zeros(16, 128, dtype=torch.bfloat16, device="cuda")
    rows = torch.zeros(4, 2, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="row_weight"):
        ops.combine(z, rows, torch.ones(15, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError, match="row_weight"):
        ops.combine(z, rows, torch.ones(4, 4, dtype=torch.float32, device="cuda"))


def test_error_word_shape_dtype_device():
    z = torch.zeros(16, 128, dtype=torch.bfloat16, device="cuda")
    rows = torch.zeros(4, 2, dtype=torch.int32, device="cuda")
    with pytest.raises(TypeError):
        ops.combine(z, rows, d_err=torch.zeros(1, dtype=torch.int64, device="cuda"))
    with pytest.raises(ValueError, match="single"):
        ops.combine(z, rows, d_err=torch.zeros(2, dtype=torch.int32, device="cuda"))
    x = torch.zeros(4, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        ops.permute(x, rows, 8, d_err=torch.zeros(1, dtype=torch.int32))  # host tensor


@pytest.mark.skipif(torch.cuda.device_count() < 2, reason="needs a second device")
def test_tensors_on_another_device_rejected():
    z = torch.zeros(16, 128, dtype=torch.bfloat16, device="cuda:0")
    rows = torch.zeros(4, 2, dtype=torch.int32, device="cuda:1")
    with pytest.raises(ValueError, match="must be on"):
        ops.combine(z, rows)


def test_row_dot_out_must_match_rows():
    a = torch.zeros(4, 128, dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(8, 128, dtype=torch.bfloat16, device="cuda")
    rows = torch.zeros(4, 2, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="out"):
        ops.row_dot(a, b, rows, out=torch.zeros(4, 1, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError, match="out"):
        ops.row_dot(a, b, rows, out=torch.zeros(6, dtype=torch.float32, device="cuda"))
    ops.row_dot(a, b, rows, out=torch.zeros(4, 2, dtype=torch.float32, device="cuda"))
    ops.row_dot(a, b, rows, out=torch.zeros(8, dtype=torch.float32, device="cuda"))  # same memory


def test_permute_scaled_out_and_scale_shapes():
    x = torch.zeros(4, 128, dtype=torch.bfloat16, device="cuda")
    dest = torch.zeros(4, 2, dtype=torch.int32, device="cuda")
    scale = torch.ones(8, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="out_rows"):
        ops.permute_scaled(x, dest, scale, 8,
                           out=torch.zeros(8 * 128, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError, match="out_rows"):
        ops.permute_scaled(x, dest, torch.ones(2, 4, dtype=torch.float32, device="cuda"), 8)

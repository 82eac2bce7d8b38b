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


def test_bound_calls_replay_on_the_buffers_given():
    """A bound call replays the checked call on the same buffers: after the
    input is overwritten in place, a replay gives what an unbound call on the
    new input gives, bit for bit, on the current stream or a given one."""
    g = torch.Generator().manual_seed(5)
    T, H, G, k = 300, 256, 8, 2
    x = torch.randn(T, H, generator=g).to(torch.bfloat16).cuda()
    dest = torch.stack([torch.arange(T), torch.arange(T) + T], 1).to(torch.int32).cuda()
    send = torch.empty(2 * T, H, dtype=torch.bfloat16, device="cuda")
    out, call = ops.permute(x, dest, 2 * T, out=send, bind=True)
    assert out is send and isinstance(call, ops.Bound)
    call()
    assert torch.equal(send, ops.permute(x, dest, 2 * T))
    x.copy_(torch.randn(T, H, generator=g).to(torch.bfloat16))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())  # the copy above runs on the current stream
    call(s.cuda_stream)
    s.synchronize()
    assert torch.equal(send, ops.permute(x, dest, 2 * T))
    rows = dest
    w = torch.rand(2 * T, generator=g).cuda()
    y = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    _, comb = ops.combine(send, rows, w, out=y, bind=True)
    comb()
    assert torch.equal(y, ops.combine(send, rows, w))


def test_bound_call_reports_data_errors():
    """A replay with a row id past the buffer sets the error word it was
    bound with, as the unbound call does."""
    x = torch.zeros(4, 128, dtype=torch.bfloat16, device="cuda")
    dest = torch.tensor([[0], [1], [2], [3]], dtype=torch.int32, device="cuda")
    err = ops.new_error_word()
    _, call = ops.permute(x, dest, 4, d_err=err, bind=True)
    call()
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    dest[2, 0] = 9  # past the 4 output rows
    call()
    torch.cuda.synchronize()
    assert "ROW_RANGE" in ops.decode_errors(int(err.item()))

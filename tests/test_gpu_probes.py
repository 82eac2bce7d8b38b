"""The HBM probe kernels the benchmark takes its ceilings from move the bytes
they claim to: the fan-out probe stores every source vector into each of its
F regions (and nothing between staggered regions), the fan-in probe stores
the XOR of its F regions, and the copy probe copies.  Small sizes, every
block shape, capped and uncapped."""

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probe_lib(built_lib):
    from co_activation_amd import hbm_probe
    return hbm_probe._load()


def _stream():
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("shape", [0, 1, 2, 3])
@pytest.mark.parametrize("fan,cap", [(1, 0), (3, 0), (3, 8), (7, 2)])
def test_fanout_probe_copies(probe_lib, shape, fan, cap):
    nbytes = 48 * 1024 + 16 * 5  # not a whole number of blocks: the tail is exercised
    stride = nbytes + 4096 + 16
    g = torch.Generator().manual_seed(shape * 100 + fan)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).cuda()
    dst = torch.full(((fan - 1) * stride + nbytes + 64,), 0xAB, dtype=torch.uint8, device="cuda")
    rc = probe_lib.moe_probe_fanout(shape, src.data_ptr(), dst.data_ptr(), nbytes, stride, fan,
                                    cap, _stream())
    assert rc == 0
    torch.cuda.synchronize()
    for f in range(fan):
        assert torch.equal(dst[f * stride:f * stride + nbytes], src), f
        gap = dst[f * stride + nbytes:(f + 1) * stride] if f < fan - 1 else dst[-64:]
        assert bool((gap == 0xAB).all()), f"bytes past region {f} written"


@pytest.mark.parametrize("shape", [0, 1, 2, 3])
@pytest.mark.parametrize("fan,cap", [(1, 0), (2, 0), (5, 6), (8, 2)])
def test_fanin_probe_folds(probe_lib, shape, fan, cap):
    nbytes = 40 * 1024 + 16 * 3
    stride = nbytes + 2048 + 48
    g = torch.Generator().manual_seed(shape * 100 + fan + 7)
    src = torch.randint(0, 256, ((fan - 1) * stride + nbytes,), dtype=torch.uint8,
                        generator=g).cuda()
    dst = torch.full((nbytes + 64,), 0xCD, dtype=torch.uint8, device="cuda")
    rc = probe_lib.moe_probe_fanin(shape, src.data_ptr(), stride, dst.data_ptr(), nbytes, fan,
                                   cap, _stream())
    assert rc == 0
    torch.cuda.synchronize()
    want = src[:nbytes].clone()
    for f in range(1, fan):
        want ^= src[f * stride:f * stride + nbytes]
    assert torch.equal(dst[:nbytes], want)
    assert bool((dst[nbytes:] == 0xCD).all())


@pytest.mark.parametrize("shape", [0, 3])
def test_copy_and_write_probes(probe_lib, shape):
    nbytes = 32 * 1024 + 16
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8).cuda()
    dst = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert probe_lib.moe_probe_stream(2, shape, src.data_ptr(), dst.data_ptr(), nbytes,
                                      sink.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert probe_lib.moe_probe_stream(1, shape, None, dst.data_ptr(), nbytes, None,
                                      _stream()) == 0
    torch.cuda.synchronize()
    assert not torch.equal(dst, src)  # overwritten with the write probe's pattern

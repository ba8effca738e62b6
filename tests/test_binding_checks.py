"""Argument checks of the Python binding, on the CPU: every tensor handed to
the attention calls must be a CUDA tensor of the right dtype, shape and
device before a device address crosses the C ABI.  A stand-in tensor type
and a library that records calls replace torch's CUDA tensors and libkvc.so,
so no call reaches the device."""
import ctypes

import pytest
import torch

import chunked_attention_amd as kv


class FakeCuda:
    """What the binding reads of a tensor: dtype, device, shape, layout."""

    def __init__(self, shape, dtype=torch.bfloat16, cuda=True, device="cuda:0",
                 contiguous=True):
        self.shape = tuple(shape)
        self.dtype = dtype
        self.is_cuda = cuda
        self.device = torch.device(device if cuda else "cpu")
        self._contig = contiguous

    def is_contiguous(self):
        return self._contig

    def data_ptr(self):
        return 0x7F0000001000


class FakeStream:
    cuda_stream = 0


class RecordingLib:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def f(*args):
            self.calls.append(name)
            return kv.KVC_OK
        return f


@pytest.fixture
def fake_lib(monkeypatch):
    rec = RecordingLib()
    monkeypatch.setattr(kv, "_lib", rec)
    return rec


CFG = kv.make_config(4, 128, 100, 16, 2)


def qo():
    return FakeCuda((100, 4, 128)), FakeCuda((100, 4, 128))


def test_valid_call_reaches_the_library(fake_lib):
    q, o = qo()
    kv.chunk_attn_fwd(ctypes.c_void_p(1), CFG, q, o, lse=FakeCuda((4, 100), torch.float32),
                      stream=FakeStream())
    assert fake_lib.calls == ["chunk_attn_fwd"]


@pytest.mark.parametrize("lse", [
    FakeCuda((4, 100), torch.float32, cuda=False),           # host memory
    FakeCuda((4, 100), torch.float32, device="cuda:1"),      # another device
    FakeCuda((4, 100), torch.float16),                       # wrong dtype
    FakeCuda((100, 4), torch.float32),                       # wrong shape
    FakeCuda((4, 100), torch.float32, contiguous=False),
])
def test_bad_lse_is_rejected_before_the_library(fake_lib, lse):
    q, o = qo()
    with pytest.raises(ValueError):
        kv.chunk_attn_fwd(ctypes.c_void_p(1), CFG, q, o, lse=lse)
    assert fake_lib.calls == []


@pytest.mark.parametrize("which", ["q", "o"])
def test_bad_q_or_o_is_rejected(fake_lib, which):
    q, o = qo()
    bad = FakeCuda((100, 4, 128), cuda=False)
    args = (bad, o) if which == "q" else (q, bad)
    with pytest.raises(ValueError):
        kv.chunk_attn_fwd(ctypes.c_void_p(1), CFG, *args)
    o2 = FakeCuda((100, 4, 128), device="cuda:1")
    with pytest.raises(ValueError):
        kv.chunk_attn_fwd(ctypes.c_void_p(1), CFG, q, o2)
    assert fake_lib.calls == []

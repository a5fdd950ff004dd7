"""Host logic of the Python binding that needs no GPU: which device a call
runs on.  Every tensor of a call must sit on one GPU; a CPU tensor (there is
no CPU path) or a second device is rejected before anything is launched."""
import types

import pytest
import torch

from row_normalization_amd import _lib


def _fake(dev: str):
    return types.SimpleNamespace(is_cuda=dev.startswith("cuda"), device=torch.device(dev))


def test_one_device_per_call():
    assert _lib._gpu(_fake("cuda:0"), None, _fake("cuda:0")) == torch.device("cuda:0")
    assert _lib._gpu(_fake("cuda:3")) == torch.device("cuda:3")
    with pytest.raises(ValueError, match="one GPU"):
        _lib._gpu(_fake("cuda:0"), _fake("cuda:1"))
    with pytest.raises(ValueError, match="GPU tensors only"):
        _lib._gpu(_fake("cuda:0"), torch.zeros(1))


def test_explicit_stream_is_passed_through():
    s = types.SimpleNamespace(cuda_stream=1234)
    assert _lib._stream(s, torch.device("cuda:0")) == 1234
    assert _lib._stream(0, torch.device("cuda:0")) == 0

"""The binding's hand-over of the tensors it allocates to a launch stream (CPU only).

A wrapper that allocates o, a workspace or gradients on the current stream and
enqueues the kernels on another stream must mark those tensors as used by that
stream, or the caching allocator may give their memory to the next allocation
on the current stream while the kernels still run.
"""
import torch

from linear_attention_sequence_modality_amd import kda


class _Stream:
    def __init__(self, handle):
        self.cuda_stream = handle


class _Tensor:
    def __init__(self):
        self.recorded = []

    def record_stream(self, s):
        self.recorded.append(s.cuda_stream)


def _fake_streams(monkeypatch, current=7):
    monkeypatch.setattr(torch.cuda, "current_stream", lambda device=None: _Stream(current))
    monkeypatch.setattr(torch.cuda, "ExternalStream", lambda handle, device=None: _Stream(handle))


def test_current_stream_needs_nothing(monkeypatch):
    _fake_streams(monkeypatch)
    t = _Tensor()
    kda._hand_over(None, "cuda:0", t)
    kda._hand_over(7, "cuda:0", t)
    kda._hand_over(_Stream(7), "cuda:0", t)
    assert t.recorded == []


def test_side_stream_marks_every_allocated_tensor(monkeypatch):
    _fake_streams(monkeypatch)
    a, b = _Tensor(), _Tensor()
    kda._hand_over(_Stream(9), "cuda:0", a, None, b)
    assert a.recorded == [9] and b.recorded == [9]


def test_raw_stream_handles_are_wrapped(monkeypatch):
    _fake_streams(monkeypatch)
    a = _Tensor()
    kda._hand_over(11, "cuda:0", a)
    assert a.recorded == [11]

"""The binding's opt-in health check, on the CPU: after a call that used a
workspace it reads the health word (kla_workspace_health) and raises
KlaHealthError when a wait gave up.  The library is replaced by a stand-in
whose health read reports a word set from the host, so the raise path is
exercised without a GPU; the real word is tested on the GPU."""

import ctypes

import pytest

from linear_attention_sequence_kla_amd import kla


class _FakeLib:
    """Just the health read of libkla: reports `word` once, then 0 (the read
    clears it)."""

    def __init__(self, word):
        self.word = word
        self.reads = 0

    def kla_workspace_health(self, ws, out, stream):
        self.reads += 1
        ctypes.cast(out, ctypes.POINTER(ctypes.c_uint32))[0] = self.word
        self.word = 0
        return kla.KLA_OK


class _FakeTensor:
    device = "cpu"

    def data_ptr(self):
        return 0x1000


class _FakeStream:
    cuda_stream = 0


@pytest.fixture
def fake(monkeypatch):
    lib = _FakeLib(word=1)
    monkeypatch.setattr(kla, "library", lambda: lib)
    monkeypatch.setattr(kla.torch.cuda, "current_stream", lambda device=None: _FakeStream())
    prev = kla.set_health_checks(False)
    yield lib
    kla.set_health_checks(prev)


def test_off_by_default_reads_nothing(fake):
    kla._after_call("kla_scan_fwd", _FakeTensor())
    assert fake.reads == 0


def test_nonzero_word_raises_and_is_cleared(fake):
    kla.set_health_checks(True)
    with pytest.raises(kla.KlaHealthError) as e:
        kla._after_call("kla_scan_fwd", _FakeTensor())
    assert e.value.name == "kla_scan_fwd"
    assert "gave up" in e.value.detail
    assert isinstance(e.value, RuntimeError)
    # the read cleared the word: the next call passes
    kla._after_call("kla_scan_fwd", _FakeTensor())
    assert fake.reads == 2


def test_zero_word_passes(fake):
    fake.word = 0
    kla.set_health_checks(True)
    kla._after_call("kla_mixer_bwd", _FakeTensor())
    assert fake.reads == 1


def test_set_health_checks_returns_previous(fake):
    assert kla.set_health_checks(True) is False
    assert kla.health_checks_enabled()
    assert kla.set_health_checks(False) is True
    assert not kla.health_checks_enabled()

"""Host-side behaviour of the Python binding (no GPU): the default workspace
is zeroed on the stream the decode is launched on, and calls on different
streams get different default workspaces.

The C library is replaced by a recorder, so these tests check only what the
binding hands to it.
"""

import ctypes

import pytest
import torch

import paged_kv_decode_block_amd as pad


class FakeStream:
    def __init__(self, ptr):
        self.cuda_stream = ptr


class RecordingLib:
    """Stands in for libpad_attn.so: records the stream of every call."""

    def __init__(self, ws_bytes):
        self.ws_bytes = ws_bytes
        self.events = []

    def pad_decode_attn_workspace_size(self, shape_ref, n_ref):
        n_ref._obj.value = self.ws_bytes
        return pad.PAD_OK

    def pad_decode_attn_workspace_init(self, ptr, nbytes, stream):
        self.events.append(("init", stream.value, ptr.value, nbytes))
        return pad.PAD_OK

    def pad_decode_attn(self, shape, q, kv, bt, lens, scale, window, out, ws, ws_bytes, stream):
        self.events.append(("decode", stream.value, ws.value, ws_bytes.value))
        return pad.PAD_OK


@pytest.fixture
def fake(monkeypatch):
    rec = RecordingLib(4096)
    monkeypatch.setattr(pad, "lib", rec)
    monkeypatch.setattr(pad, "_require_device", lambda **kw: None)
    monkeypatch.setattr(pad, "_default_ws", {})
    return rec


def _tensors(S=2, M=1, Hq=4, Hkv=1, D=64, P=16, nb=8, mb=4):
    q = torch.zeros((S, M, Hq, D), dtype=torch.bfloat16)
    kv = torch.zeros((nb, Hkv, P, 2, D), dtype=torch.bfloat16)
    bt = torch.zeros((S, mb), dtype=torch.int32)
    lens = torch.ones(S, dtype=torch.int32)
    return q, kv, bt, lens, torch.empty_like(q)


def test_default_workspace_zeroed_on_the_launch_stream(fake):
    q, kv, bt, lens, out = _tensors()
    a = FakeStream(0x1111)
    pad.pad_decode_attn(q, kv, bt, lens, 0.125, 0, out, stream=a)
    (init, dec), = [fake.events]
    assert init[0] == "init" and dec[0] == "decode"
    assert init[1] == dec[1] == 0x1111, "the fill must be enqueued on the decode's stream"
    assert init[2] == dec[2] and init[3] >= 4096, "the decode must use the buffer that was zeroed"
    # A second call on the same stream reuses it without a new fill.
    pad.pad_decode_attn(q, kv, bt, lens, 0.125, 0, out, stream=a)
    assert [e[0] for e in fake.events] == ["init", "decode", "decode"]
    assert fake.events[2][2] == dec[2]


def test_streams_get_their_own_default_workspace(fake):
    q, kv, bt, lens, out = _tensors()
    a, b = FakeStream(0x1111), FakeStream(0x2222)
    pad.pad_decode_attn(q, kv, bt, lens, 0.125, 0, out, stream=a)
    pad.pad_decode_attn(q, kv, bt, lens, 0.125, 0, out, stream=b)
    inits = [e for e in fake.events if e[0] == "init"]
    decs = [e for e in fake.events if e[0] == "decode"]
    assert [e[1] for e in inits] == [0x1111, 0x2222]
    assert decs[0][2] != decs[1][2], "calls on different streams must not share a workspace"
    assert {k[1] for k in pad._default_ws} == {0x1111, 0x2222}


def test_growing_workspace_is_zeroed_on_the_launch_stream(fake):
    q, kv, bt, lens, out = _tensors()
    a = FakeStream(0x3333)
    pad.pad_decode_attn(q, kv, bt, lens, 0.125, 0, out, stream=a)
    fake.ws_bytes = 1 << 16  # a larger shape comes along
    pad.pad_decode_attn(q, kv, bt, lens, 0.125, 0, out, stream=a)
    inits = [e for e in fake.events if e[0] == "init"]
    assert len(inits) == 2 and all(e[1] == 0x3333 for e in inits)
    assert inits[1][3] >= 1 << 16
    assert fake.events[-1][0] == "decode" and fake.events[-1][2] == inits[1][2]


def test_varlen_default_workspace_follows_the_stream(fake):
    q, kv, bt, lens, _ = _tensors()
    fake_varlen = []

    def varlen(shape, q_, qs, kv_, bt_, lens_, scale, window, out_, ws, ws_bytes, stream):
        fake_varlen.append((stream.value, ws.value))
        return pad.PAD_OK

    fake.pad_decode_attn_varlen = varlen
    qp = torch.zeros((3, 4, 64), dtype=torch.bfloat16)
    q_start = torch.tensor([0, 1, 3], dtype=torch.int32)
    s = FakeStream(0x4444)
    pad.pad_decode_attn_varlen(qp, q_start, kv, bt, lens, 0.125, 0, torch.empty_like(qp), max_query_len=2, stream=s)
    (init,) = [e for e in fake.events if e[0] == "init"]
    assert init[1] == 0x4444 and fake_varlen == [(0x4444, init[2])]


def test_explicit_workspace_is_passed_through(fake):
    q, kv, bt, lens, out = _tensors()
    ws = torch.zeros(8192, dtype=torch.uint8)
    pad.pad_decode_attn(q, kv, bt, lens, 0.125, 0, out, workspace=ws, stream=FakeStream(5))
    assert fake.events == [("decode", 5, ws.data_ptr(), 8192)]
    assert ctypes.sizeof(ctypes.c_void_p) == 8


def test_packed_cache_default_workspace(fake):
    """The packed-cache calls share one default workspace per (device,
    stream), apart from the plain decode's, zeroed on the launch stream
    and passed to both the uniform and the per-sequence-count entries."""
    calls = []

    def slot_bytes(fmt, head_size, n_ref):
        n_ref._obj.value = 240
        return pad.PAD_OK

    def octave_ws(shape_ref, fmt, n_ref):
        n_ref._obj.value = 2048
        return pad.PAD_OK

    def octave(shape, fmt, q, cache, bt, lens, ks, vs, scale, out, ws, ws_bytes, stream):
        calls.append(("octave", stream.value, ws.value, ws_bytes.value))
        return pad.PAD_OK

    def octave_varlen(shape, fmt, q, qs, cache, bt, lens, ks, vs, scale, out, ws, ws_bytes, stream):
        calls.append(("varlen", stream.value, ws.value, ws_bytes.value))
        return pad.PAD_OK

    fake.pad_octave_slot_bytes = slot_bytes
    fake.pad_decode_attn_octave_workspace_size = octave_ws
    fake.pad_decode_attn_octave = octave
    fake.pad_decode_attn_octave_varlen = octave_varlen
    S, M, Hq, Hkv, D, P = 2, 4, 16, 2, 256, 16
    q = torch.zeros((S, M, Hq, D), dtype=torch.bfloat16)
    cache = torch.zeros((8, Hkv, P, 240), dtype=torch.uint8)
    bt = torch.zeros((S, 4), dtype=torch.int32)
    lens = torch.ones(S, dtype=torch.int32)
    signs = torch.zeros(8, dtype=torch.int32)
    s = FakeStream(0x5150)
    pad.pad_decode_attn_octave(q, cache, bt, lens, signs, signs, 0.1, torch.empty_like(q), 1, stream=s)
    qp = torch.zeros((5, Hq, D), dtype=torch.bfloat16)
    q_start = torch.tensor([0, 2, 5], dtype=torch.int32)
    pad.pad_decode_attn_octave_varlen(qp, q_start, cache, bt, lens, signs, signs, 0.1, torch.empty_like(qp), 1,
                                      max_query_len=M, stream=s)
    (init,) = [e for e in fake.events if e[0] == "init"]
    assert init[1] == 0x5150 and init[3] == 2048
    assert calls == [("octave", 0x5150, init[2], 2048), ("varlen", 0x5150, init[2], 2048)]
    # the plain decode on the same stream gets a workspace of its own
    q2, kv2, bt2, lens2, out2 = _tensors()
    pad.pad_decode_attn(q2, kv2, bt2, lens2, 0.125, 0, out2, stream=s)
    decode = [e for e in fake.events if e[0] == "decode"]
    assert decode and decode[0][2] != init[2]

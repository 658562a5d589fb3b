"""The C-ABI library: it loads, exports every declared symbol, and its host-side
checks and size rules behave as documented.  No GPU: only calls that return
before anything is launched."""
import ctypes
import os
import re

import pytest

import paged_kv_cache_reshape_amd as pa
from paged_kv_cache_reshape_amd import build as pabuild

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "pagedattn.h")

OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pa.LIB_PATH):
        pabuild.build()
    return pa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("pa_reshape_and_cache", "pa_paged_attention_decode", "pa_decode_step",
              "pa_decode_workspace_bytes", "pa_decode_partition_size",
              "pa_debug_gather_kv", "pa_status_string", "pa_last_error_message",
              "pa_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert lib.pa_status_string(0) == b"ok"
    assert lib.pa_status_string(3) == b"workspace too small"
    assert lib.pa_status_string(99) == b"unknown status"
    assert lib.pa_version() >= 100


def _decode(lib, **kw):
    a = dict(out=16, q=16, k=16, v=16, bt=16, cl=16, B=4, Hq=4, Hkv=2, D=64, nb=32,
             bs=16, mb=4, scale=0.125, ps=0, ws=None, wsb=0, cnt=None, ncnt=0, dt=0)
    a.update(kw)
    return lib.pa_paged_attention_decode(
        a["out"], a["q"], a["k"], a["v"], a["bt"], a["cl"], a["B"], a["Hq"], a["Hkv"],
        a["D"], a["nb"], a["bs"], a["mb"], a["scale"], a["ps"], a["ws"], a["wsb"],
        a["cnt"], a["ncnt"], a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=5), INVALID),
    (dict(Hq=6, Hkv=4), INVALID),
    (dict(Hq=12, Hkv=4), UNSUPPORTED),      # group of 3
    (dict(D=96), UNSUPPORTED),
    (dict(bs=8), UNSUPPORTED),
    (dict(ps=24), INVALID),                 # not a multiple of block_size
    (dict(ps=16 * 129), INVALID),           # more than 128 blocks
    (dict(Hkv=0), INVALID),
    (dict(nb=0), INVALID),
    (dict(B=-1), INVALID),
    (dict(q=None), INVALID),
    (dict(k=8), INVALID),                   # misaligned
    (dict(mb=400, ps=16), WS_SMALL),        # needs partials, none given
    (dict(mb=400, ps=16, ws=256, wsb=1 << 30), WS_SMALL),  # no counters
    (dict(mb=400, ps=16, ws=256, wsb=1 << 30, cnt=256, ncnt=7), WS_SMALL),
    (dict(mb=400, ps=16, ws=128, wsb=1 << 30, cnt=256, ncnt=8), INVALID),
    (dict(B=0, q=None, out=None), OK),      # empty batch: nothing to do
])
def test_decode_argument_checks(lib, kw, status):
    assert _decode(lib, **kw) == status
    if status:
        assert lib.pa_last_error_message() != b""


def _step(lib, **kw):
    a = dict(out=16, q=16, key=16, value=16, k=16, v=16, bt=16, cl=16, B=4, Hq=4, Hkv=2, D=64,
             nb=32, bs=16, mb=4, scale=0.125, ps=0, ws=None, wsb=0, cnt=None, ncnt=0, dt=0)
    a.update(kw)
    return lib.pa_decode_step(
        a["out"], a["q"], a["key"], a["value"], a["k"], a["v"], a["bt"], a["cl"], a["B"],
        a["Hq"], a["Hkv"], a["D"], a["nb"], a["bs"], a["mb"], a["scale"], a["ps"], a["ws"],
        a["wsb"], a["cnt"], a["ncnt"], a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(key=None), INVALID),
    (dict(value=None), INVALID),
    (dict(key=24), INVALID),                # misaligned
    (dict(dt=5), INVALID),                  # the decode's own checks come first
    (dict(Hq=12, Hkv=4), UNSUPPORTED),
    (dict(mb=400, ps=16), WS_SMALL),
    (dict(B=0, q=None, out=None, key=None, value=None), OK),  # empty batch
])
def test_decode_step_argument_checks(lib, kw, status):
    assert _step(lib, **kw) == status
    if status:
        assert lib.pa_last_error_message() != b""


def _noalloc(lib, **kw):
    a = dict(out=16, q=16, key=16, value=16, k=16, v=16, bt=16, cl=16, B=4, Hq=4, Hkv=2, D=64,
             nb=32, bs=16, mb=4, scale=0.125, ps=0, dt=0)
    a.update(kw)
    return lib.pa_decode_step_noalloc(
        a["out"], a["q"], a["key"], a["value"], a["k"], a["v"], a["bt"], a["cl"], a["B"],
        a["Hq"], a["Hkv"], a["D"], a["nb"], a["bs"], a["mb"], a["scale"], a["ps"], a["dt"],
        None)


@pytest.mark.parametrize("kw,status", [
    (dict(key=None), INVALID),
    (dict(dt=5), INVALID),
    (dict(Hq=12, Hkv=4), UNSUPPORTED),
    # The 32K-token batch at 512-token partitions needs 8 MiB + 128 KiB of
    # workspace (fits); twice the table needs more than the 16 MiB held.
    (dict(B=8, Hq=32, Hkv=8, D=128, mb=4096, ps=512, dt=1), WS_SMALL),
    (dict(B=256, Hq=32, Hkv=32, D=128, mb=64, ps=128, dt=1), WS_SMALL),
    (dict(B=0, q=None, out=None, key=None, value=None), OK),  # empty batch
])
def test_noalloc_step_rejects_before_launch(lib, kw, status):
    """The entry point without allocation: its own size limit and the checks
    it shares with pa_decode_step, all decided before any device call."""
    assert _noalloc(lib, **kw) == status
    if status:
        msg = lib.pa_last_error_message()
        assert msg != b""
        if status == WS_SMALL:
            assert b"noalloc" in msg


def test_write_argument_checks(lib):
    f = lib.pa_reshape_and_cache
    assert f(16, 16, 16, 16, 16, 0, 2, 64, 32, 16, 0, None) == OK  # no tokens
    assert f(16, 16, 16, 16, 16, -1, 2, 64, 32, 16, 0, None) == INVALID
    assert f(None, 16, 16, 16, 16, 4, 2, 64, 32, 16, 0, None) == INVALID
    assert f(16, 16, 16, 16, 16, 4, 2, 48, 32, 16, 0, None) == UNSUPPORTED
    assert f(16, 16, 16, 16, 16, 4, 2, 64, 32, 64, 0, None) == UNSUPPORTED
    assert f(16, 16, 16, 16, 16, 4, 2, 64, 32, 16, 9, None) == INVALID
    assert f(16, 24, 16, 16, 16, 4, 2, 64, 32, 16, 0, None) == INVALID  # misaligned


def test_copy_blocks_argument_checks(lib):
    f = lib.pa_copy_blocks
    assert f(16, 16, 16, 0, 2, 64, 32, 16, 0, None) == OK          # no pairs
    assert f(16, 16, 16, -1, 2, 64, 32, 16, 0, None) == INVALID
    assert f(16, 16, None, 3, 2, 64, 32, 16, 0, None) == INVALID
    assert f(16, 24, 16, 3, 2, 64, 32, 16, 0, None) == INVALID     # misaligned
    assert f(16, 16, 16, 3, 2, 64, 32, 8, 0, None) == UNSUPPORTED
    assert f(16, 16, 16, 3, 0, 64, 32, 16, 0, None) == INVALID


def test_prefill_argument_checks(lib):
    f = lib.pa_paged_attention_prefill

    def call(**kw):
        a = dict(out=16, q=16, k=16, v=16, bt=16, cl=16, qs=16, B=2, T=8, Hq=4, Hkv=2, D=64,
                 nb=32, bs=16, mb=4, mq=4, scale=0.125, dt=1)
        a.update(kw)
        return f(a["out"], a["q"], a["k"], a["v"], a["bt"], a["cl"], a["qs"], a["B"], a["T"],
                 a["Hq"], a["Hkv"], a["D"], a["nb"], a["bs"], a["mb"], a["mq"], a["scale"],
                 a["dt"], None)
    assert call(dt=0) == UNSUPPORTED            # float32 prefill is not built
    assert call(dt=7) == INVALID
    assert call(Hq=6, Hkv=2) == UNSUPPORTED     # group of 3
    assert call(Hq=6, Hkv=4) == INVALID
    assert call(D=96) == UNSUPPORTED
    assert call(bs=64) == UNSUPPORTED
    assert call(T=-1) == INVALID
    assert call(qs=None) == INVALID
    assert call(q=24) == INVALID                # misaligned
    assert call(mq=1 << 30) == INVALID          # launch too large
    # 2^20 sequences x 8 kv heads x 256 row groups: more workgroups than a
    # 32-bit workgroup number holds
    assert call(B=1 << 20, Hq=8, Hkv=8, mq=65536) == INVALID
    assert call(T=0, q=None, out=None) == OK    # nothing to do
    assert call(B=0, qs=None) == OK


def test_gather_argument_checks(lib):
    f = lib.pa_debug_gather_kv
    assert f(16, 16, 16, 16, 16, 16, 0, 2, 64, 32, 16, 4, 0, None) == OK
    assert f(16, 16, 16, 16, 16, 16, 4, 2, 64, 32, 16, 0, 0, None) == INVALID
    assert f(None, 16, 16, 16, 16, 16, 4, 2, 64, 32, 16, 4, 0, None) == INVALID


def test_partition_size_rule(lib):
    # explicit sizes are honoured when valid
    assert pa.decode_partition_size(8, 32, 8, 128, 2048, 16, 512) == 512
    assert pa.decode_partition_size(8, 32, 8, 128, 2048, 16, 500) == -1
    assert pa.decode_partition_size(8, 32, 8, 128, 2048, 16, 16 * 64) == 1024
    assert pa.decode_partition_size(8, 32, 8, 128, 2048, 16, 16 * 128) == 2048
    assert pa.decode_partition_size(8, 32, 8, 128, 2048, 16, 16 * 129) == -1
    # left to the library: the balanced schedule (reported as 0) for at most
    # 1024 (sequence, kv head) pairs with 1 or 2 query heads per kv head, or
    # 4 at head_dim 64 over tables of at most 4096 tokens; otherwise 1024
    # tokens at head_dim 128 (2048 for tables of more than 4096 tokens) and
    # 1024 at head_dim 64 for groups of 4 or more
    assert pa.decode_partition_size(32, 16, 8, 128, 128, 16, 0) == 0
    assert pa.decode_partition_size(64, 16, 8, 64, 256, 16, 0) == 0
    assert pa.decode_partition_size(4, 4, 2, 64, 4, 16, 0) == 0
    assert pa.decode_partition_size(64, 32, 8, 64, 256, 16, 0) == 0     # Llama-3.2 shape
    assert pa.decode_partition_size(64, 32, 8, 64, 128, 32, 0) == 0     # 32-token blocks
    assert pa.decode_partition_size(64, 32, 8, 64, 257, 16, 0) == 1024  # > 4096 tokens
    assert pa.decode_partition_size(8, 32, 8, 128, 256, 16, 0) == 1024  # G = 4 at D = 128
    assert pa.decode_partition_size(8, 32, 8, 128, 2048, 16, 0) == 2048  # 32K tokens
    assert pa.decode_partition_size(8, 32, 8, 128, 257, 16, 0) == 2048
    assert pa.decode_partition_size(8, 32, 8, 128, 128, 32, 0) == 1024
    assert pa.decode_partition_size(8, 32, 8, 128, 129, 32, 0) == 2048
    assert pa.decode_partition_size(256, 32, 32, 128, 32, 32, 0) == 1024
    assert pa.decode_partition_size(256, 32, 8, 64, 256, 16, 0) == 1024  # 2048 pairs
    assert pa.decode_partition_size(8, 64, 8, 64, 256, 16, 0) == 1024   # G = 8
    assert pa.decode_partition_size(600, 16, 8, 64, 256, 16, 0) == 512  # 4800 pairs


def test_schedule_override_is_read_once_and_reloaded(lib, monkeypatch):
    """PAGEDATTN_SCHEDULE takes effect after pa_reload_options, not before."""
    monkeypatch.setenv("PAGEDATTN_SCHEDULE", "fixed")
    assert pa.decode_partition_size(32, 16, 8, 128, 128, 16, 0) == 0  # not re-read yet
    pa.reload_options()
    assert pa.decode_partition_size(32, 16, 8, 128, 128, 16, 0) == 1024
    monkeypatch.setenv("PAGEDATTN_SCHEDULE", "stream")
    pa.reload_options()
    assert pa.decode_partition_size(8, 32, 8, 128, 256, 16, 0) == 0
    assert pa.decode_partition_size(8, 64, 8, 128, 256, 16, 0) == 1024  # G = 8: not built


def test_workspace_size_rule(lib):
    def al(x):
        return (x + 255) // 256 * 256
    # library choice for the Qwen3 shape: the balanced schedule, 128 workers
    # per kv head (1024 in all), two partial states each of G rows
    B, Hq, Hkv, D, mb, bs = 32, 16, 8, 128, 128, 16
    rows = Hkv * 128 * 2 * (Hq // Hkv)
    assert pa.decode_workspace_bytes(B, Hq, Hkv, D, mb, bs, 0) == \
        al(rows * D * 4) + al(rows * 2 * 4)
    # the Llama-3.2 shape (4 query heads per kv head): 2048 workers, 256 per
    # kv head
    rows = 8 * 256 * 2 * 4
    assert pa.decode_workspace_bytes(64, 32, 8, 64, 256, 16, 0) == \
        al(rows * 64 * 4) + al(rows * 2 * 4)
    # the workers are enough that no range exceeds 128 blocks: 500 sequences
    # of 2048-token tables need 8000 workers per kv head
    rows = 2 * 8000 * 2 * 2
    assert pa.decode_workspace_bytes(500, 4, 2, 128, 2048, 16, 0) == \
        al(rows * 128 * 4) + al(rows * 2 * 4)
    # with a fixed partition size: 1024-token partitions of a 2048-token
    # table -> 2 partitions per sequence
    rows = B * Hkv * 2 * (Hq // Hkv)
    assert pa.decode_workspace_bytes(B, Hq, Hkv, D, mb, bs, 1024) == \
        al(rows * D * 4) + al(rows * 2 * 4)
    # no workspace when every sequence fits one partition
    assert pa.decode_workspace_bytes(4, 4, 2, 64, 4, 16, 64) == 0
    # otherwise: G*D floats of output + 2 floats per (seq, kv head, partition,
    # head), each region 256-byte aligned (the counters are a separate array)
    B, Hq, Hkv, D, mb, bs, ps = 8, 32, 8, 128, 2048, 16, 512
    parts = mb * bs // ps
    rows = B * Hkv * parts * (Hq // Hkv)

    def al(x):
        return (x + 255) // 256 * 256
    want = al(rows * D * 4) + al(rows * 2 * 4)
    assert pa.decode_workspace_bytes(B, Hq, Hkv, D, mb, bs, ps) == want
    assert pa.decode_workspace_bytes(B, Hq, Hkv, D, mb, bs, 24) == 0  # invalid


def test_binding_refuses_cpu_tensors(lib):
    import torch
    q = torch.zeros(1, 2, 64)
    with pytest.raises(ValueError):
        pa.paged_attention_decode(q, torch.zeros(1, 16, 1, 64), torch.zeros(1, 16, 1, 64),
                                  torch.zeros(1, 1, dtype=torch.int32),
                                  torch.ones(1, dtype=torch.int32), 0.1)


def test_one_hip_runtime_in_process(lib):
    """The library binds to the HIP runtime PyTorch already loaded: the process
    maps exactly one libamdhip64, PyTorch's own copy."""
    maps = open("/proc/self/maps").read()
    hips = sorted(set(re.findall(r"\S*libamdhip64\S*", maps)))
    assert len(hips) == 1, hips
    assert hips[0].startswith(pabuild.torch_lib_dir()), hips


def test_ctypes_signatures_match_header(lib):
    assert lib.pa_decode_workspace_bytes.restype is ctypes.c_size_t
    assert len(lib.pa_paged_attention_decode.argtypes) == 21
    assert len(lib.pa_decode_step.argtypes) == 23
    assert len(lib.pa_decode_step_noalloc.argtypes) == 19
    assert len(lib.pa_reshape_and_cache.argtypes) == 12
    assert len(lib.pa_debug_gather_kv.argtypes) == 14
    assert len(lib.pa_copy_blocks.argtypes) == 10
    assert len(lib.pa_paged_attention_prefill.argtypes) == 19

"""The C-ABI library loads and exports every symbol include/pa.h declares; host
validation returns the documented codes (CPU only: no call reaches a kernel)."""
import ctypes
import os
import re

import pytest

import paged_kv_cache_85_amd as pa
from paged_kv_cache_85_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from paged_kv_cache_85_amd import build
        build.build(verbose=False)
    return pa.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert getattr(lib, name) is not None


def test_status_strings(lib):
    for code in (pa.PA_OK, pa.PA_E_INVAL, pa.PA_E_UNSUPPORTED, pa.PA_E_WORKSPACE, pa.PA_E_HIP):
        s = pa.pa_status_string(code)
        assert s and s != "unknown status"
    assert pa.pa_status_string(12345) == "unknown status"


def test_workspace_bytes(lib):
    assert pa.pa_decode_workspace_bytes(0, 16, 128, 2048) == 0
    n = pa.pa_decode_workspace_bytes(256, 16, 128, 2048)
    # partials for at least 2048 / 512 partitions of (D outputs + max + sum) per head
    assert n >= 256 * 16 * 4 * (128 + 2) * 4
    assert pa.pa_decode_workspace_bytes(1, 1, 64, 1) >= (64 + 2) * 4


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def _decode(lib, **kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, cl=FAKE, B=4, hq=16, hkv=8, d=128,
             nb=64, bs=16, mb=8, maxl=128, scale=0.125, dtype=1, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.pa_decode(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["cl"], a["B"], a["hq"],
                         a["hkv"], a["d"], a["nb"], a["bs"], a["mb"], a["maxl"], a["scale"],
                         a["dtype"], a["ws"], a["wsb"], a["stream"])


def test_decode_validation(lib):
    assert _decode(lib, hq=12, hkv=8) == pa.PA_E_INVAL            # Hq % Hkv != 0
    assert _decode(lib, d=96) == pa.PA_E_UNSUPPORTED
    assert _decode(lib, dtype=7) == pa.PA_E_UNSUPPORTED
    assert _decode(lib, out=None) == pa.PA_E_INVAL
    assert _decode(lib, bs=0) == pa.PA_E_INVAL
    assert _decode(lib, maxl=200, mb=8, bs=16) == pa.PA_E_INVAL     # table too short
    assert _decode(lib, scale=float("nan")) == pa.PA_E_INVAL
    assert _decode(lib, scale=0.0) == pa.PA_E_INVAL                # scale must be > 0
    assert _decode(lib, scale=-0.125) == pa.PA_E_INVAL
    assert _decode(lib, maxl=1000, mb=64, ws=None) == pa.PA_E_WORKSPACE
    assert _decode(lib, maxl=1000, mb=64, ws=FAKE, wsb=16) == pa.PA_E_WORKSPACE
    assert _decode(lib, B=0) == pa.PA_OK                           # empty batch: no-op
    for name in ("out", "q", "kc", "vc"):                          # 16-byte element rows
        assert _decode(lib, **{name: ctypes.c_void_p(0x1008)}) == pa.PA_E_INVAL


def _prefill(lib, **kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, cq=FAKE, ck=FAKE, B=3, tq=30, mq=20,
             mk=40, hq=16, hkv=8, d=128, nb=64, bs=16, mb=4, scale=0.1, dtype=1, ws=None,
             wsb=0, stream=None)
    a.update(kw)
    return lib.pa_prefill_varlen(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["cq"], a["ck"],
                                 a["B"], a["tq"], a["mq"], a["mk"], a["hq"], a["hkv"], a["d"],
                                 a["nb"], a["bs"], a["mb"], a["scale"], a["dtype"], a["ws"],
                                 a["wsb"], a["stream"])


def test_prefill_validation(lib):
    assert _prefill(lib, hq=15) == pa.PA_E_INVAL
    assert _prefill(lib, d=80) == pa.PA_E_UNSUPPORTED
    assert _prefill(lib, mq=50, mk=40) == pa.PA_E_INVAL            # Lq may not exceed Lk
    assert _prefill(lib, mk=100, mb=4, bs=16) == pa.PA_E_INVAL      # table too short
    assert _prefill(lib, cq=None) == pa.PA_E_INVAL
    assert _prefill(lib, scale=-1.0) == pa.PA_E_INVAL
    assert _prefill(lib, tq=0) == pa.PA_OK
    assert _prefill(lib, B=0) == pa.PA_OK
    assert _prefill(lib, ws=FAKE, wsb=16) == pa.PA_E_WORKSPACE     # counter area too small
    assert _prefill(lib, ws=ctypes.c_void_p(0x1010), wsb=256) == pa.PA_E_INVAL   # unaligned
    for name in ("out", "q", "kc", "vc"):                          # 16-byte element rows
        assert _prefill(lib, **{name: ctypes.c_void_p(0x1008)}) == pa.PA_E_INVAL
    assert binding.PREFILL_WORKSPACE_BYTES == 256


def test_store_validation(lib):
    f = lib.pa_store_kv
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 8, 128, 64, 16, 1, None) == pa.PA_E_INVAL
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 64, 16, 5, None) == pa.PA_E_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, None, FAKE, 4, 8, 128, 64, 16, 1, None) == pa.PA_E_INVAL
    assert f(None, None, None, None, None, 0, 8, 128, 64, 16, 1, None) == pa.PA_OK
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 1 << 20, 1 << 12, 1, None) == pa.PA_E_INVAL


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(ImportError):
        binding.lib()


def _prologue(lib, **kw):
    a = dict(qo=FAKE, q=FAKE, k=FAKE, v=FAKE, qw=FAKE, kw=FAKE, cs=FAKE, pos=FAKE, kc=FAKE,
             vc=FAKE, sm=FAKE, T=4, hq=16, hkv=8, d=128, nb=64, bs=16, mp=4096, eps=1e-6,
             dtype=1, stream=None)
    a.update(kw)
    return lib.pa_qk_norm_rope_store(a["qo"], a["q"], a["k"], a["v"], a["qw"], a["kw"], a["cs"],
                                     a["pos"], a["kc"], a["vc"], a["sm"], a["T"], a["hq"],
                                     a["hkv"], a["d"], a["nb"], a["bs"], a["mp"], a["eps"],
                                     a["dtype"], a["stream"])


def test_prologue_validation(lib):
    assert _prologue(lib, d=96) == pa.PA_E_UNSUPPORTED
    assert _prologue(lib, dtype=3) == pa.PA_E_UNSUPPORTED
    assert _prologue(lib, eps=-1.0) == pa.PA_E_INVAL
    assert _prologue(lib, eps=float("inf")) == pa.PA_E_INVAL
    assert _prologue(lib, mp=0) == pa.PA_E_INVAL
    assert _prologue(lib, kc=None) == pa.PA_E_INVAL
    assert _prologue(lib, q=ctypes.c_void_p(0x1008)) == pa.PA_E_INVAL   # not 16-byte aligned
    assert _prologue(lib, T=-1) == pa.PA_E_INVAL
    assert _prologue(lib, T=0, q=None) == pa.PA_OK


def test_decode_noalloc_validation(lib):
    f = lib.pa_decode_noalloc

    def call(B=4, hq=16, hkv=8, d=128, nb=64, bs=16, mb=8, maxl=128, out=FAKE):
        return f(out, FAKE, FAKE, FAKE, FAKE, FAKE, B, hq, hkv, d, nb, bs, mb, maxl, 0.125, 1,
                 None)

    # a batch whose partials exceed the library's scratch array: refused
    # before any device call
    big = pa.pa_decode_workspace_bytes(4096, 64, 128, 8192)
    assert big > binding.NOALLOC_SCRATCH_BYTES
    assert call(B=4096, hq=64, hkv=8, mb=512, maxl=8192) == pa.PA_E_WORKSPACE
    # one-partition contexts need no scratch: the argument checks answer
    assert call(hq=12, hkv=8) == pa.PA_E_INVAL
    assert call(d=96) == pa.PA_E_UNSUPPORTED
    assert call(out=None) == pa.PA_E_INVAL
    assert call(B=0) == pa.PA_OK
    # the Qwen3-shaped decode batch fits the scratch array
    assert pa.pa_decode_workspace_bytes(256, 16, 128, 2048) <= binding.NOALLOC_SCRATCH_BYTES


def test_header_constants_match_binding():
    src = open(HEADER).read()
    got = {k: v for k, v in re.findall(r"#define\s+(PA_[A-Z_]+)\s+(\d+)\b", src)}
    assert int(got["PA_DECODE_PARTITION_TOKENS"]) == binding.DECODE_PARTITION_TOKENS
    assert int(got["PA_PREFILL_WORKSPACE_BYTES"]) == binding.PREFILL_WORKSPACE_BYTES
    m = re.search(r"#define\s+PA_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == binding.NOALLOC_SCRATCH_BYTES


def test_decode_workspace_sized_for_its_partitions(lib):
    # [256 B counter][B*Hq*parts*D fp32, 256-aligned][B*Hq*parts*2 fp32], parts = ceil(L / 512)
    B, hq, d, L = 256, 16, 128, 2048
    parts = -(-L // binding.DECODE_PARTITION_TOKENS)
    o = B * hq * parts * d * 4
    ml_off = (256 + o + 255) // 256 * 256
    assert pa.pa_decode_workspace_bytes(B, hq, d, L) == ml_off + B * hq * parts * 2 * 4

"""C-ABI boundary tests that need no GPU: the library loads, exports every
function include/spa.h declares, and rejects bad arguments on the host
before launching anything (fake non-null pointers are never dereferenced)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import split_paged_attention_amd as spa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spa.h")

FAKE = ctypes.c_void_p(0x100000)       # aligned, never dereferenced
FAKE_ODD = ctypes.c_void_p(0x100002)   # misaligned


TIMELINE_HEADER = os.path.join(ROOT, "include", "spa_timeline.h")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["spa_build_page_table", "spa_build_metadata", "spa_paged_decode_attention",
              "spa_paged_verify_attention", "spa_verify_workspace_bytes", "spa_split_merge",
              "spa_decode_workspace_bytes", "spa_workspace_reset", "spa_status_string"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", spa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    L = spa.lib()
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(L, n)
    assert L.spa_abi_version() == 3


def _exports(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    return set(l.split()[-1] for l in out.splitlines() if l.strip())


def test_timeline_build_exports_the_library_and_its_own_calls():
    """libspa_timeline.so (the diagnostics build) exports every function of
    spa.h and of spa_timeline.h; libspa.so exports none of the latter."""
    from split_paged_attention_amd import build as spa_build
    tl = _exports(spa_build.TIMELINE_LIB)
    own = declared_functions(TIMELINE_HEADER)
    assert own == ["spa_timeline_clear", "spa_timeline_read"]
    for n in declared_functions() + own:
        assert n in tl, n
    lib_exports = _exports(spa.LIB_PATH)
    assert not any(n in lib_exports for n in own)


def test_status_strings():
    assert spa.status_string(0) == "SPA_OK"
    assert spa.status_string(3) == "SPA_ERR_WORKSPACE_TOO_SMALL"
    assert spa.status_string(99) == "SPA_ERR_UNKNOWN"


def _attn(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=None, vs=None, pt=FAKE, pts=128, sl=FAKE, B=1, Hq=32,
             Hkv=8, D=128, P=64, npg=16, S=4, scale=0.088, kvd=0, flags=0, ws=FAKE,
             wsb=1 << 30, out=FAKE, lse=FAKE)
    a.update(kw)
    return spa.lib().spa_paged_decode_attention(
        a["q"], a["k"], a["v"], a["ks"], a["vs"], a["pt"], a["pts"], a["sl"], a["B"], a["Hq"],
        a["Hkv"], a["D"], a["P"], a["npg"], a["S"], a["scale"], a["kvd"], a["flags"], a["ws"],
        a["wsb"], a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(Hq=30), spa.SPA_ERR_INVALID_ARGUMENT),            # Hq % Hkv != 0
    (dict(S=0), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(kvd=7), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(flags=16), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(flags=3), spa.SPA_ERR_INVALID_ARGUMENT),            # both merge placements
    (dict(flags=12), spa.SPA_ERR_INVALID_ARGUMENT),           # both producer shapes
    (dict(Hq=12, Hkv=3, flags=4), spa.SPA_ERR_UNSUPPORTED),   # head-grouped needs even Hkv
    (dict(B=0, flags=2 | 4), spa.SPA_OK),
    (dict(scale=math.nan), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(scale=math.inf), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(pts=0), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(q=None), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(out=None), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(ws=None), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(kvd=1), spa.SPA_ERR_INVALID_ARGUMENT),            # int8 without scales
    (dict(kvd=2), spa.SPA_ERR_INVALID_ARGUMENT),            # fp8 without scales
    (dict(kvd=2, ks=FAKE, vs=FAKE, B=0), spa.SPA_OK),
    (dict(kvd=3), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(q=FAKE_ODD), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(k=FAKE_ODD), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(D=64), spa.SPA_ERR_UNSUPPORTED),
    (dict(P=32), spa.SPA_ERR_UNSUPPORTED),
    (dict(Hq=64), spa.SPA_ERR_UNSUPPORTED),                 # group 8
    (dict(Hq=8, Hkv=8), spa.SPA_ERR_UNSUPPORTED),           # group 1
    (dict(S=1025), spa.SPA_ERR_UNSUPPORTED),
    (dict(wsb=1024), spa.SPA_ERR_WORKSPACE_TOO_SMALL),
    (dict(B=0), spa.SPA_OK),                                # no launch
    (dict(B=0, q=None, out=None), spa.SPA_OK),
])
def test_attention_argument_checks(kw, code):
    assert _attn(**kw) == code


def test_workspace_bytes():
    f = spa.decode_workspace_bytes
    assert f(0, 32, 8, 128, 16) > 0
    n = f(32, 32, 8, 128, 16)
    rows = 32 * 32 * 16
    assert n >= rows * 128 * 4 + 2 * rows * 4 + 32 * 8 * 4
    assert n % 256 == 0
    assert f(-1, 32, 8, 128, 4) == 0 and f(1, 32, 8, 128, 0) == 0 and f(1, 0, 8, 128, 4) == 0
    assert _attn(wsb=n - 1, B=32, S=16) == spa.SPA_ERR_WORKSPACE_TOO_SMALL


def _noalloc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=None, vs=None, pt=FAKE, pts=128, sl=FAKE, B=1, Hq=32,
             Hkv=8, D=128, P=64, npg=16, S=4, scale=0.088, kvd=0, flags=0, out=FAKE, lse=FAKE)
    a.update(kw)
    return spa.lib().spa_paged_decode_attention_noalloc(
        a["q"], a["k"], a["v"], a["ks"], a["vs"], a["pt"], a["pts"], a["sl"], a["B"], a["Hq"],
        a["Hkv"], a["D"], a["P"], a["npg"], a["S"], a["scale"], a["kvd"], a["flags"], a["out"],
        a["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=64, S=64), spa.SPA_ERR_WORKSPACE_TOO_SMALL),   # needs 68 MB > the 32 MiB scratch
    (dict(D=64), spa.SPA_ERR_UNSUPPORTED),
    (dict(out=None), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(flags=3), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(B=0), spa.SPA_OK),                                 # no launch
])
def test_noalloc_argument_checks(kw, code):
    assert _noalloc(**kw) == code


def test_workspace_reset_checks():
    L = spa.lib()
    assert L.spa_workspace_reset(None, 0, None) == spa.SPA_OK
    assert L.spa_workspace_reset(None, 16, None) == spa.SPA_ERR_INVALID_ARGUMENT
    assert L.spa_workspace_reset(FAKE, 6, None) == spa.SPA_ERR_INVALID_ARGUMENT


def _partials(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=None, vs=None, pt=FAKE, pts=128, sl=FAKE, B=1, Hq=32,
             Hkv=8, D=128, P=64, npg=16, S=4, scale=0.088, kvd=0, flags=0, acc=FAKE, mx=FAKE,
             sm=FAKE)
    a.update(kw)
    return spa.lib().spa_paged_decode_partials(
        a["q"], a["k"], a["v"], a["ks"], a["vs"], a["pt"], a["pts"], a["sl"], a["B"], a["Hq"],
        a["Hkv"], a["D"], a["P"], a["npg"], a["S"], a["scale"], a["kvd"], a["flags"], a["acc"],
        a["mx"], a["sm"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(flags=spa.SPA_DECODE_SEPARATE_MERGE), spa.SPA_ERR_INVALID_ARGUMENT),   # merge flags
    (dict(flags=spa.SPA_DECODE_FUSED_MERGE), spa.SPA_ERR_INVALID_ARGUMENT),      # are the caller's
    (dict(flags=12), spa.SPA_ERR_INVALID_ARGUMENT),           # both producer shapes
    (dict(flags=16), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(acc=None), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(mx=None), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(sm=None), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(acc=ctypes.c_void_p(0x100004)), spa.SPA_ERR_INVALID_ARGUMENT),   # acc needs 16 B
    (dict(mx=FAKE_ODD), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(kvd=1), spa.SPA_ERR_INVALID_ARGUMENT),              # int8 without scales
    (dict(scale=math.inf), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(D=64), spa.SPA_ERR_UNSUPPORTED),
    (dict(Hq=12, Hkv=3, flags=spa.SPA_DECODE_HEAD_GROUPED), spa.SPA_ERR_UNSUPPORTED),
    (dict(S=1025), spa.SPA_ERR_UNSUPPORTED),
    (dict(B=0), spa.SPA_OK),                                  # no launch
    (dict(B=0, acc=None, q=None), spa.SPA_OK),
])
def test_partials_argument_checks(kw, code):
    assert _partials(**kw) == code


def test_default_flags():
    f = spa.decode_default_flags
    HG, PS = spa.SPA_DECODE_HEAD_GROUPED, spa.SPA_DECODE_PAGE_SPLIT
    SEP, FUS = spa.SPA_DECODE_SEPARATE_MERGE, spa.SPA_DECODE_FUSED_MERGE
    assert f(32, 8, 16, "bf16", 128) == HG | SEP        # batch 32 / 8K: 4096 triples
    assert f(1, 8, 4, "bf16", 16) == PS | FUS           # batch 1 / 1K, 4 splits
    assert f(1, 8, 16, "bf16", 128) == PS | SEP         # more than 8 splits: second launch
    assert f(8, 8, 4, "bf16", 16) == HG | FUS           # 256 triples, 4-page splits
    assert f(8, 8, 4, "bf16", 128) == PS | FUS          # 256 triples, 32-page splits
    assert f(8, 8, 8, "bf16", 128) == PS | FUS          # 512 triples, 16-page splits
    assert f(1, 8, 16, "bf16", 16) == HG | SEP          # 128 triples, 1-page splits
    assert f(1, 8, 8, "bf16", 32) == PS | FUS           # 64 triples, 4-page splits
    assert f(16, 8, 4, "bf16", 16) == HG | FUS          # 512 triples, 4 splits
    assert f(16, 8, 8, "bf16", 16) == HG | SEP          # 1024 triples, 8 splits
    assert f(32, 8, 16, "int8", 128) == HG | SEP        # 4096 triples
    assert f(8, 8, 16, "fp8", 128) == HG | SEP          # 1024 triples, 8-page splits
    assert f(4, 8, 16, "int8", 16) == PS | SEP          # 512 triples: 1-byte page split
    assert f(4, 8, 16, "bf16", 16) == HG | SEP          # 512 triples: bf16 head grouped
    assert f(32, 8, 4, "fp8", 128) == HG | FUS          # 1024 triples, 4 splits
    assert f(8, 8, 4, "fp8", 128) == PS | FUS           # 256 triples
    assert f(2, 8, 16, "int8", 16) == PS | SEP          # 256 triples, 16 splits
    assert f(32, 3, 16, "bf16", 128) == PS | SEP        # odd kv heads: page split only
    # the producer rule at its edges (triples = batch x kv heads x splits;
    # split pages = ceil(page-table stride / splits))
    prod = lambda *a: f(*a) & (HG | PS)
    assert prod(16, 8, 1, "bf16", 2) == HG              # 128 triples, 2-page splits
    assert prod(15, 8, 1, "bf16", 2) == PS              # 120 triples
    assert prod(16, 8, 1, "bf16", 3) == PS              # 128 triples, 3-page splits
    assert prod(4, 8, 8, "bf16", 64) == HG              # 256 triples, 8-page splits
    assert prod(4, 8, 8, "bf16", 65) == PS              # 256 triples, 9-page splits
    assert prod(31, 8, 1, "bf16", 8) == PS              # 248 triples
    assert prod(128, 8, 1, "bf16", 4096) == HG          # 1024 triples, any split length
    assert prod(127, 8, 1, "bf16", 4096) == PS          # 1016 triples, long splits
    assert prod(128, 8, 1, "int8", 4096) == HG          # 1-byte codes: 1024 triples only
    assert prod(127, 8, 1, "fp8", 1) == PS              # 1016 triples, even 1-page splits
    # every result is exactly one producer and one merge flag
    for args in [(1, 8, 1, "bf16", 1), (64, 8, 8, "int8", 32), (4, 2, 1024, "fp8", 128)]:
        v = f(*args)
        assert bin(v & (HG | PS)).count("1") == 1 and bin(v & (SEP | FUS)).count("1") == 1
    assert f(-1, 8, 4, "bf16", 16) == 0 and f(1, 8, 0, "bf16", 16) == 0
    assert f(1, 8, 1025, "bf16", 16) == 0 and f(1, 8, 4, "bf16", 0) == 0


def _meta(**kw):
    a = dict(r2t=FAKE, r2ts=8192, pool=64, rpi=FAKE, sl=FAKE, bs=4, off=0, P=64, msp=128,
             pt=FAKE, pts=128, cache=FAKE, cu=FAKE)
    a.update(kw)
    return spa.lib().spa_build_page_table(a["r2t"], a["r2ts"], a["pool"], a["rpi"], a["sl"],
                                          a["bs"], a["off"], a["P"], a["msp"], a["pt"], a["pts"],
                                          a["cache"], a["cu"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(bs=-1), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(P=0), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(msp=-1), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(pts=100), spa.SPA_ERR_INVALID_ARGUMENT),          # stride < max_seq_pages
    (dict(r2ts=127 * 64), spa.SPA_ERR_INVALID_ARGUMENT),    # last column past the row
    (dict(pool=0), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(r2t=None), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(cu=None), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(bs=2**31 - 1), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(bs=0), spa.SPA_OK),
    (dict(bs=0, r2t=None, cu=None), spa.SPA_OK),
])
def test_page_table_argument_checks(kw, code):
    assert _meta(**kw) == code


def _full(**kw):
    a = dict(r2t=FAKE, r2ts=8192, pool=64, rpi=FAKE, sl=FAKE, bs=4, off=0, P=64, msp=128,
             pt=FAKE, pts=128, cache=FAKE, cu=FAKE, qm=0, ql=None, qs=0, cuq=None, swa=None,
             swal=1 << 20, spt=None, spts=0, ocl=None, nocl=0, sout=None, soutl=0)
    a.update(kw)
    return spa.lib().spa_build_metadata(
        a["r2t"], a["r2ts"], a["pool"], a["rpi"], a["sl"], a["bs"], a["off"], a["P"], a["msp"],
        a["pt"], a["pts"], a["cache"], a["cu"], a["qm"], a["ql"], a["qs"], a["cuq"], a["swa"],
        a["swal"], a["spt"], a["spts"], a["ocl"], a["nocl"], a["sout"], a["soutl"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(qm=3), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(qm=-1), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(qm=1, cuq=FAKE), spa.SPA_ERR_INVALID_ARGUMENT),         # cumsum needs qlens
    (dict(qm=1, ql=FAKE), spa.SPA_ERR_INVALID_ARGUMENT),          # ... and cu_seqlens_q
    (dict(qm=2), spa.SPA_ERR_INVALID_ARGUMENT),                   # strided needs cu_seqlens_q
    (dict(spt=FAKE, spts=128), spa.SPA_ERR_INVALID_ARGUMENT),     # swa table needs the map
    (dict(spt=FAKE, spts=100, swa=FAKE), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(sout=FAKE, soutl=8, ocl=FAKE, nocl=4), spa.SPA_ERR_INVALID_ARGUMENT),  # needs the map
    (dict(sout=FAKE, soutl=-1), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(sout=FAKE, soutl=8, ocl=FAKE, nocl=-1, swa=FAKE), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(sout=FAKE, soutl=2**62, swa=FAKE), spa.SPA_ERR_INVALID_ARGUMENT),   # grid too large
    (dict(sout=FAKE_ODD, soutl=8, swa=FAKE), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(swa=FAKE_ODD, spt=FAKE, spts=128), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(swa=FAKE, swal=-1, spt=FAKE, spts=128), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(pts=100), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(bs=2**31 - 1), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(bs=0, qm=1, sout=FAKE, soutl=8, ocl=FAKE, nocl=8), spa.SPA_OK),   # no launch
])
def test_full_metadata_argument_checks(kw, code):
    assert _full(**kw) == code


def _verify(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=None, vs=None, pt=FAKE, pts=128, sl=FAKE, cu=FAKE, B=2,
             T=8, mq=4, Hq=32, Hkv=8, D=128, P=64, npg=16, S=4, scale=0.088, kvd=0, ws=FAKE,
             wsb=1 << 30, out=FAKE, lse=FAKE)
    a.update(kw)
    return spa.lib().spa_paged_verify_attention(
        a["q"], a["k"], a["v"], a["ks"], a["vs"], a["pt"], a["pts"], a["sl"], a["cu"], a["B"],
        a["T"], a["mq"], a["Hq"], a["Hkv"], a["D"], a["P"], a["npg"], a["S"], a["scale"], a["kvd"],
        a["ws"], a["wsb"], a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(mq=0), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(mq=65), spa.SPA_ERR_UNSUPPORTED),
    (dict(T=-1), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(cu=None), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(Hq=12, Hkv=3), spa.SPA_ERR_UNSUPPORTED),            # odd kv heads
    (dict(kvd=1), spa.SPA_ERR_INVALID_ARGUMENT),              # int8 without scales
    (dict(kvd=2, ks=FAKE, vs=FAKE, T=0), spa.SPA_OK),
    (dict(out=FAKE_ODD), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(wsb=1024), spa.SPA_ERR_WORKSPACE_TOO_SMALL),
    (dict(scale=math.nan), spa.SPA_ERR_INVALID_ARGUMENT),
    (dict(D=64), spa.SPA_ERR_UNSUPPORTED),
    (dict(B=0), spa.SPA_OK),
])
def test_verify_argument_checks(kw, code):
    assert _verify(**kw) == code


def test_verify_workspace_bytes():
    f = spa.verify_workspace_bytes
    n = f(128, 32, 8, 128, 16)
    rows = 128 * 32 * 16
    assert n >= rows * 128 * 4 + 2 * rows * 4 and n % 256 == 0
    assert f(-1, 32, 8, 128, 4) == 0
    assert _verify(wsb=n - 1, T=128, S=16) == spa.SPA_ERR_WORKSPACE_TOO_SMALL


@pytest.mark.parametrize("args,code", [
    ((FAKE, FAKE, FAKE, 1, 32, 128, 0, FAKE, FAKE), spa.SPA_ERR_INVALID_ARGUMENT),
    ((FAKE, FAKE, FAKE, 1, 32, 0, 4, FAKE, FAKE), spa.SPA_ERR_INVALID_ARGUMENT),
    ((FAKE, FAKE, FAKE, 1, 32, 5000, 4, FAKE, FAKE), spa.SPA_ERR_INVALID_ARGUMENT),
    ((FAKE, FAKE, FAKE, -1, 32, 128, 4, FAKE, FAKE), spa.SPA_ERR_INVALID_ARGUMENT),
    ((None, FAKE, FAKE, 1, 32, 128, 4, FAKE, FAKE), spa.SPA_ERR_INVALID_ARGUMENT),
    ((FAKE, FAKE, FAKE, 1, 32, 128, 4, None, FAKE), spa.SPA_ERR_INVALID_ARGUMENT),
    ((None, None, None, 0, 32, 128, 4, None, None), spa.SPA_OK),
])
def test_split_merge_argument_checks(args, code):
    assert spa.lib().spa_split_merge(*args, None) == code


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(spa, "_lib", None)
    monkeypatch.setattr(spa, "LIB_PATH", "/nonexistent/libspa.so")
    with pytest.raises(RuntimeError, match="missing"):
        spa.lib()

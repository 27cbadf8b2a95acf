"""The C ABI library loads, exports what include/attn.h declares, and validates
arguments on the host (CPU only: every call here fails validation or is an
empty problem, so no HIP call is made)."""
import ctypes
import os
import re
import subprocess

import pytest

import compressed_latent_causal_amd as attn
from compressed_latent_causal_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, ENULL, ESHAPE, EUNSUP, EALIGN, EWS, EHIP, ESCRATCH = range(8)
F32, BF16 = 0, 1
FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_library_exports_every_declared_symbol(L):
    declared = _declared()
    assert declared == sorted(_lib.SIGNATURES), declared
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (attn_\w+)", out))
    assert set(declared) <= exported
    # nothing else leaks out under the attn_ prefix, and no C++ symbols are exported
    assert exported == set(declared)
    assert not re.search(r" T _Z", out)


def test_status_strings(L):
    for s in range(8):
        assert L.attn_status_string(s).decode()
    assert L.attn_status_string(99) == b"unknown status"


def test_enum_values_match_header():
    text = open(HEADER).read()
    for name, val in [("ATTN_F32", 0), ("ATTN_BF16", 1), ("ATTN_OK", 0), ("ATTN_ERR_NULL", 1),
                      ("ATTN_ERR_SHAPE", 2), ("ATTN_ERR_UNSUPPORTED", 3), ("ATTN_ERR_ALIGN", 4),
                      ("ATTN_ERR_WORKSPACE", 5), ("ATTN_ERR_HIP", 6), ("ATTN_ERR_SCRATCH", 7)]:
        assert re.search(rf"\b{name}\s*=\s*{val}\b", text), name
        if name.startswith("ATTN_ERR") or name == "ATTN_OK":
            assert _lib.STATUS[val] == name


# ---------------------------------------------------------------- rope
@pytest.mark.parametrize("name", ["attn_rope", "attn_rope_backward"])
def test_rope_validation(L, name):
    r = lambda *a: getattr(L, name)(*a)
    assert r(FAKE, FAKE, BF16, -1, 8, 16, 128, None, 0, 1e4, None) == ESHAPE
    assert r(FAKE, FAKE, BF16, 1, 0, 16, 128, None, 0, 1e4, None) == ESHAPE
    assert r(FAKE, FAKE, BF16, 1, 8, -2, 128, None, 0, 1e4, None) == ESHAPE
    assert r(FAKE, FAKE, BF16, 1, 8, 16, 96, None, 0, 1e4, None) == EUNSUP
    assert r(FAKE, FAKE, 7, 1, 8, 16, 128, None, 0, 1e4, None) == EUNSUP
    assert r(FAKE, FAKE, BF16, 1, 8, 16, 128, None, 0, 0.0, None) == EUNSUP
    assert r(FAKE, FAKE, BF16, 1, 8, 16, 128, None, 0, float("nan"), None) == EUNSUP
    assert r(None, FAKE, BF16, 1, 8, 16, 128, None, 0, 1e4, None) == ENULL
    assert r(FAKE, None, BF16, 1, 8, 16, 128, None, 0, 1e4, None) == ENULL
    assert r(FAKE + 8, FAKE, BF16, 1, 8, 16, 128, None, 0, 1e4, None) == EALIGN
    assert r(FAKE, FAKE, BF16, 1, 8, 16, 128, FAKE + 2, 0, 1e4, None) == EALIGN
    assert r(FAKE, FAKE, BF16, 70000, 8, 16, 128, None, 0, 1e4, None) == ESHAPE
    # empty problems succeed without touching the (NULL) pointers
    assert r(None, None, BF16, 0, 8, 16, 128, None, 0, 1e4, None) == OK
    assert r(None, None, F32, 3, 8, 0, 64, None, 0, 1e4, None) == OK


# ---------------------------------------------------------------- prefill
def test_prefill_validation(L):
    p = lambda *a: L.attn_prefill(*a)
    args = lambda **kw: [kw.get("o", FAKE), kw.get("q", FAKE), kw.get("k", FAKE), kw.get("v", FAKE),
                         kw.get("dt", BF16), kw.get("B", 1), kw.get("Hq", 8), kw.get("Hkv", 2),
                         kw.get("S", 16), kw.get("D", 64), kw.get("scale", 0.125),
                         kw.get("theta", 0.0), None]
    assert p(*args(Hkv=3)) == ESHAPE
    assert p(*args(Hkv=0)) == ESHAPE
    assert p(*args(Hq=0)) == ESHAPE
    assert p(*args(B=-1)) == ESHAPE
    assert p(*args(S=-5)) == ESHAPE
    assert p(*args(D=32)) == EUNSUP
    assert p(*args(dt=2)) == EUNSUP
    assert p(*args(scale=0.0)) == EUNSUP
    assert p(*args(scale=-0.1)) == EUNSUP
    assert p(*args(scale=float("inf"))) == EUNSUP
    assert p(*args(theta=-1.0)) == EUNSUP
    assert p(*args(theta=float("nan"))) == EUNSUP
    assert p(*args(theta=float("inf"))) == EUNSUP
    for name in "oqkv":
        assert p(*args(**{name: None})) == ENULL
        assert p(*args(**{name: FAKE + 4})) == EALIGN
    assert p(*args(B=1 << 20, S=1 << 20)) == ESHAPE  # grid would overflow 32 bits
    assert p(*args(B=1, Hq=1, Hkv=1, S=1 << 23, D=128)) == ESHAPE  # one head's K spans 2 GiB
    assert p(*args(B=1, Hq=1, Hkv=1, S=1 << 23, D=128, dt=F32)) == ESHAPE
    assert p(*args(o=None, q=None, k=None, v=None, B=0)) == OK
    assert p(*args(o=None, q=None, k=None, v=None, S=0)) == OK


def test_prefill_lse_validation(L):
    p = lambda *a: L.attn_prefill_lse(*a)
    args = lambda **kw: [kw.get("o", FAKE), kw.get("lse", FAKE), kw.get("q", FAKE),
                         kw.get("k", FAKE), kw.get("v", FAKE), kw.get("dt", BF16), kw.get("B", 1),
                         kw.get("Hq", 8), kw.get("Hkv", 2), kw.get("S", 16), kw.get("D", 64),
                         kw.get("scale", 0.125), kw.get("theta", 0.0), None]
    assert p(*args(Hkv=3)) == ESHAPE
    assert p(*args(dt=F32)) == EUNSUP  # bf16 only
    assert p(*args(D=96)) == EUNSUP
    assert p(*args(scale=0.0)) == EUNSUP
    assert p(*args(theta=-2.0)) == EUNSUP
    for name in ("o", "lse", "q", "k", "v"):
        assert p(*args(**{name: None})) == ENULL
    for name in "oqkv":
        assert p(*args(**{name: FAKE + 4})) == EALIGN
    assert p(*args(lse=FAKE + 2)) == EALIGN  # lse needs 4-byte alignment only
    assert p(*args(B=1, Hq=1, Hkv=1, S=1 << 23, D=128)) == ESHAPE
    assert p(*args(o=None, lse=None, q=None, k=None, v=None, B=0)) == OK


def test_prefill_backward_workspace_and_validation(L):
    ws = L.attn_prefill_backward_workspace_size
    # two fp32 per row, each head padded to whole 64-row tiles plus one (MHA
    # never splits its heads)
    assert ws(2, 8, 8, 100, 64) == 2 * 8 * (128 + 64) * 8
    assert ws(1, 1, 1, 64, 128) == (64 + 64) * 8
    # a launch far too small to fill a device splits the group's 4 heads over
    # 4 workgroups per key block: 4 fp32 partial sums of dk and dv follow the
    # statistics (rounded up to 256 bytes)
    stats = 1 * 8 * (64 + 64) * 8
    assert ws(1, 8, 2, 16, 64) == stats + 4 * 2 * (1 * 2 * 16 * 64) * 4
    # groups of 3 heads have no slicing into 2 or 4: statistics only
    assert ws(1, 6, 2, 16, 128) == 1 * 6 * (64 + 64) * 8
    assert ws(0, 8, 2, 100, 64) == 0 and ws(1, 0, 1, 5, 64) == 0 and ws(1, 1, 1, 0, 64) == 0
    assert ws(1, 8, 3, 16, 64) == 0 and ws(1, 8, 2, 16, 96) == 0 and ws(1, 8, 0, 16, 64) == 0
    need = ws(1, 8, 2, 16, 64)
    p = lambda *a: L.attn_prefill_backward(*a)
    names = ["dq", "dk", "dv", "q", "k", "v", "o", "dout"]
    args = lambda **kw: [kw.get(n, FAKE) for n in names] + [
        kw.get("lse", FAKE), kw.get("dt", BF16), kw.get("B", 1), kw.get("Hq", 8), kw.get("Hkv", 2),
        kw.get("S", 16), kw.get("D", 64), kw.get("scale", 0.125), kw.get("ws", FAKE),
        kw.get("wsb", need), None]
    assert p(*args(Hkv=3)) == ESHAPE
    assert p(*args(Hq=0)) == ESHAPE
    assert p(*args(S=-1)) == ESHAPE
    assert p(*args(dt=F32)) == EUNSUP
    assert p(*args(D=32)) == EUNSUP
    assert p(*args(scale=float("nan"))) == EUNSUP
    for name in names + ["lse"]:
        assert p(*args(**{name: None})) == ENULL
    for name in names:
        assert p(*args(**{name: FAKE + 8})) == EALIGN
    assert p(*args(ws=None)) == EWS
    assert p(*args(wsb=need - 1)) == EWS
    assert p(*args(ws=FAKE + 4)) == EALIGN
    assert p(*args(B=1, Hq=1, Hkv=1, S=1 << 23, D=128)) == ESHAPE
    assert p(*args(**{n: None for n in names}, lse=None, ws=None, B=0)) == OK


# ---------------------------------------------------------------- decode
def test_decode_workspace_size(L):
    ws = L.attn_decode_workspace_size
    assert ws(1, 8, 3, 100, 128) == 0          # Hq % Hkv
    assert ws(1, 8, 2, 100, 96) == 0           # head dim
    assert ws(0, 8, 2, 100, 128) == 0          # empty
    n = ws(32, 32, 8, 8192, 128)
    # 8192 tokens = 256 sub-tiles of 32; a split workgroup takes at least 16
    # of them -> at most 16 partials per group; (D + 2) floats per (sequence,
    # head, partial), an 8-byte tag per (sequence, KV head, partial) and an
    # 8-byte epoch per (sequence, KV head)
    assert n == 32 * 32 * 16 * 130 * 4 + 32 * 8 * 16 * 8 + 32 * 8 * 8
    # partials per (sequence, head, chunk): grows with max_len, never shrinks
    sizes = [ws(1, 64, 8, L_, 128) for L_ in (1, 512, 4096, 131072)]
    assert sizes == sorted(sizes) and sizes[0] > 0
    assert ws(2, 8, 2, 0, 64) > 0              # the merge pass still writes zeros


def test_decode_validation(L):
    d = L.attn_decode
    big = 1 << 40

    def args(**kw):
        return [kw.get("o", FAKE), kw.get("q", FAKE), kw.get("kc", FAKE), kw.get("vc", FAKE),
                kw.get("dt", BF16), kw.get("B", 2), kw.get("Hq", 8), kw.get("Hkv", 2),
                kw.get("S_cap", 64), kw.get("D", 128), kw.get("lens", FAKE),
                kw.get("max_len", 64), kw.get("scale", 0.088), kw.get("theta", 0.0),
                kw.get("ws", FAKE), kw.get("ws_bytes", big), None]

    assert d(*args(Hkv=3)) == ESHAPE
    assert d(*args(max_len=65)) == ESHAPE
    assert d(*args(max_len=-1)) == ESHAPE
    assert d(*args(S_cap=0, max_len=0)) == ESHAPE
    # fp32 caches take the accuracy path, for groups with G * D <= 4096
    assert d(*args(dt=F32, o=None)) == ENULL
    assert d(*args(dt=F32, Hq=64, Hkv=1, D=128)) == EUNSUP
    assert d(*args(dt=F32, Hq=32, Hkv=1, D=128, o=None)) == ENULL
    assert d(*args(dt=F32, B=70000, Hkv=1, Hq=1, S_cap=64)) == ESHAPE
    assert d(*args(dt=2)) == EUNSUP
    assert d(*args(D=80)) == EUNSUP
    assert d(*args(scale=0.0)) == EUNSUP
    assert d(*args(theta=-1.0)) == EUNSUP
    assert d(*args(theta=float("nan"))) == EUNSUP
    for name in ("o", "q", "kc", "vc", "lens"):
        assert d(*args(**{name: None})) == ENULL
    for name in ("o", "q", "kc", "vc"):
        assert d(*args(**{name: FAKE + 8})) == EALIGN
    assert d(*args(lens=FAKE + 2)) == EALIGN
    assert d(*args(ws=None)) == EWS
    need = L.attn_decode_workspace_size(2, 8, 2, 64, 128)
    assert d(*args(ws_bytes=need - 1)) == EWS
    assert d(*args(ws=FAKE + 4)) == EALIGN
    assert d(*args(B=70000)) == ESHAPE
    # one head's max_len keys must span less than 2 GiB
    assert d(*args(S_cap=1 << 23, max_len=1 << 23)) == ESHAPE
    assert d(*args(o=None, q=None, kc=None, vc=None, lens=None, ws=None, B=0)) == OK


def test_decode_paged_validation(L):
    d = L.attn_decode_paged
    big = 1 << 40

    def args(**kw):
        return [kw.get("o", FAKE), kw.get("q", FAKE), kw.get("kp", FAKE), kw.get("vp", FAKE),
                kw.get("dt", BF16), kw.get("B", 2), kw.get("Hq", 8), kw.get("Hkv", 2),
                kw.get("page", 64), kw.get("D", 128), kw.get("npages", 10), kw.get("table", FAKE),
                kw.get("max_pages", 4), kw.get("lens", FAKE), kw.get("max_len", 256),
                kw.get("window", 0), kw.get("scale", 0.088), kw.get("theta", 0.0),
                kw.get("ws", FAKE), kw.get("ws_bytes", big), None]

    assert d(*args(Hkv=3)) == ESHAPE
    for page in (0, 16, 48, -32):
        assert d(*args(page=page)) == ESHAPE            # a positive multiple of 32
    assert d(*args(npages=0)) == ESHAPE
    assert d(*args(max_pages=0)) == ESHAPE
    assert d(*args(max_len=257)) == ESHAPE               # beyond max_pages * page_size
    assert d(*args(max_len=-1)) == ESHAPE
    assert d(*args(page=1 << 16, max_pages=1 << 8, max_len=1 << 23)) == ESHAPE  # keys span 2 GiB
    assert d(*args(dt=F32)) == EUNSUP
    assert d(*args(D=96)) == EUNSUP
    assert d(*args(scale=float("inf"))) == EUNSUP
    assert d(*args(theta=float("inf"))) == EUNSUP
    for name in ("o", "q", "kp", "vp", "table", "lens"):
        assert d(*args(**{name: None})) == ENULL
    for name in ("o", "q", "kp", "vp"):
        assert d(*args(**{name: FAKE + 8})) == EALIGN
    for name in ("table", "lens"):
        assert d(*args(**{name: FAKE + 2})) == EALIGN
    assert d(*args(ws=None)) == EWS
    need = L.attn_decode_workspace_size(2, 8, 2, 256, 128)
    assert d(*args(ws_bytes=need - 1)) == EWS
    assert d(*args(B=0, o=None, q=None, kp=None, vp=None, table=None, lens=None, ws=None)) == OK


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "_HERE", str(tmp_path))
    with pytest.raises(RuntimeError, match="missing"):
        _lib.lib()


def test_attn_error_carries_status():
    e = attn.AttnError(ESHAPE)
    assert e.status == ESHAPE and "ATTN_ERR_SHAPE" in str(e)


def test_package_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "compressed_latent_causal_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "liboracle" not in text, f
                assert "oracle.c" not in text, f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c", ".h")):
            text = open(os.path.join(ROOT, "oracle", f)).read()
            assert not re.search(r"^\s*(import|from)\s+compressed_latent_causal_amd\b", text,
                                 re.M), f
            assert "libattn" not in text, f


def test_decode_noalloc_validation(L):
    """Same checks as attn_decode, minus the workspace; problems whose
    workspace would exceed the static scratch are refused before any HIP call."""
    text = open(HEADER).read()
    m = re.search(r"#define ATTN_DECODE_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.DECODE_SCRATCH_BYTES
    d = lambda *a: L.attn_decode_noalloc(*a)
    args = lambda **kw: [kw.get("o", FAKE), kw.get("q", FAKE), kw.get("k", FAKE), kw.get("v", FAKE),
                         kw.get("dt", BF16), kw.get("B", 2), kw.get("Hq", 8), kw.get("Hkv", 2),
                         kw.get("S_cap", 64), kw.get("D", 128), kw.get("lens", FAKE),
                         kw.get("max_len", 64), kw.get("scale", 0.1), kw.get("theta", 0.0), None]
    assert d(*args(Hkv=3)) == ESHAPE
    assert d(*args(max_len=65)) == ESHAPE
    assert d(*args(dt=F32)) == EUNSUP
    assert d(*args(D=96)) == EUNSUP
    assert d(*args(scale=0.0)) == EUNSUP
    for name in ("o", "q", "k", "v", "lens"):
        assert d(*args(**{name: None})) == ENULL
    assert d(*args(lens=FAKE + 2)) == EALIGN
    assert d(*args(o=None, q=None, k=None, v=None, lens=None, B=0)) == OK
    # the two decode workloads fit the scratch; twice the first does not
    ws = L.attn_decode_workspace_size
    assert ws(32, 32, 8, 8192, 128) <= _lib.DECODE_SCRATCH_BYTES
    assert ws(1, 64, 8, 131072, 128) <= _lib.DECODE_SCRATCH_BYTES
    assert ws(64, 32, 8, 8192, 128) > _lib.DECODE_SCRATCH_BYTES
    assert d(*args(B=64, Hq=32, Hkv=8, S_cap=8192, max_len=8192)) == ESCRATCH


def test_cca_mix_decode_validation(L):
    """The decode step of the CCA pre-attention operations: bf16 only, widths
    1 to 8, the group's convolved rows must fit 64 KiB of LDS, and the rings
    may be NULL only for a width of 1."""
    d = lambda *a: L.attn_cca_mix_decode(*a)
    args = lambda **kw: [kw.get("qo", FAKE), kw.get("ko", FAKE), kw.get("vo", FAKE),
                         kw.get("q", FAKE), kw.get("k", FAKE), kw.get("v", FAKE),
                         kw.get("dt", BF16), kw.get("B", 2), kw.get("Hq", 8), kw.get("Hkv", 2),
                         kw.get("D", 64), kw.get("cq", FAKE), kw.get("ck", FAKE), kw.get("W", 4),
                         kw.get("mq", FAKE), kw.get("mk", FAKE), kw.get("qs", FAKE),
                         kw.get("ks", FAKE), kw.get("vs", FAKE), kw.get("t", FAKE),
                         kw.get("pos", None), kw.get("theta", 1e4), None]
    assert d(*args(Hkv=3)) == ESHAPE
    assert d(*args(B=-1)) == ESHAPE
    assert d(*args(dt=F32)) == EUNSUP
    assert d(*args(D=96)) == EUNSUP
    assert d(*args(W=0)) == EUNSUP
    assert d(*args(W=9)) == EUNSUP
    assert d(*args(theta=-1.0)) == EUNSUP
    assert d(*args(theta=float("inf"))) == EUNSUP
    # (G + 2) D 4 bytes of LDS: G = 126 fits at D = 128, G = 127 does not
    assert d(*args(Hq=126, Hkv=1, D=128, qo=None)) == ENULL
    assert d(*args(Hq=127, Hkv=1, D=128)) == EUNSUP
    for name in ("qo", "ko", "vo", "q", "k", "v", "cq", "ck", "mq", "mk", "qs", "ks", "vs", "t"):
        assert d(*args(**{name: None})) == ENULL, name
    assert d(*args(W=1, qs=None, ks=None, qo=None)) == ENULL  # rings optional at W = 1 only
    assert d(*args(qs=FAKE + 8)) == EALIGN
    assert d(*args(t=FAKE + 2)) == EALIGN
    assert d(*args(pos=FAKE + 1)) == EALIGN
    assert d(*args(B=0, qo=None, ko=None, vo=None, q=None, k=None, v=None, t=None)) == OK


def test_cca_mix_validation(L):
    d = lambda *a: L.attn_cca_mix(*a)
    args = lambda **kw: [kw.get("qo", FAKE), kw.get("ko", FAKE), kw.get("vo", FAKE),
                         kw.get("q", FAKE), kw.get("k", FAKE), kw.get("v", FAKE),
                         kw.get("dt", BF16), kw.get("B", 2), kw.get("Hq", 8), kw.get("Hkv", 2),
                         kw.get("S", 100), kw.get("D", 64), kw.get("cq", FAKE), kw.get("ck", FAKE),
                         kw.get("W", 4), kw.get("mq", FAKE), kw.get("mk", FAKE),
                         kw.get("pos", None), kw.get("theta", 1e4), None]
    assert d(*args(Hkv=3)) == ESHAPE
    assert d(*args(S=-1)) == ESHAPE
    assert d(*args(S=(1 << 24) - 64 + 1, D=64)) == ESHAPE  # (S + 64) D 2 reaches 2^31
    assert d(*args(dt=F32)) == EUNSUP
    assert d(*args(D=32)) == EUNSUP
    assert d(*args(W=0)) == EUNSUP
    assert d(*args(W=9)) == EUNSUP
    assert d(*args(theta=float("nan"))) == EUNSUP
    for name in ("qo", "ko", "vo", "q", "k", "v", "cq", "ck", "mq", "mk"):
        assert d(*args(**{name: None})) == ENULL, name
    assert d(*args(cq=FAKE + 4)) == EALIGN
    assert d(*args(pos=FAKE + 2)) == EALIGN
    assert d(*args(S=0, qo=None, ko=None, vo=None, q=None, k=None, v=None)) == OK
    assert d(*args(B=0, qo=None)) == OK


def test_cca_mix_backward_workspace_and_validation(L):
    ws = L.attn_cca_mix_backward_workspace_size
    # the mean's fp32 gradient, the rotation's (cos, sin) per (sequence, token,
    # pair), then fp32 partial dM (D D) and taps (W D) per (sequence, 256-token
    # chunk, head)
    assert ws(2, 8, 2, 300, 64, 4) == 4 * (2 * 2 * 300 * 64 + 2 * 300 * 64 +
                                           2 * 2 * 10 * (64 * 64 + 4 * 64))
    assert ws(1, 4, 4, 1, 128, 1) == 4 * (4 * 128 + 128 + 1 * 8 * (128 * 128 + 128))
    assert ws(0, 8, 2, 300, 64, 4) == 0 and ws(1, 8, 3, 16, 64, 4) == 0
    assert ws(1, 8, 2, 16, 96, 4) == 0 and ws(1, 8, 2, 16, 64, 9) == 0 and ws(1, 8, 2, 0, 64, 4) == 0
    need = ws(2, 8, 2, 100, 64, 4)
    d = lambda *a: L.attn_cca_mix_backward(*a)
    names = ["dq", "dk", "dv", "dcq", "dck", "dmq", "dmk", "gq", "gk", "gv", "q", "k"]
    args = lambda **kw: [kw.get(n, FAKE) for n in names] + [
        kw.get("dt", BF16), kw.get("B", 2), kw.get("Hq", 8), kw.get("Hkv", 2), kw.get("S", 100),
        kw.get("D", 64), kw.get("cq", FAKE), kw.get("ck", FAKE), kw.get("W", 4), kw.get("mq", FAKE),
        kw.get("mk", FAKE), kw.get("pos", None), kw.get("theta", 1e4), kw.get("ws", FAKE),
        kw.get("wsb", need), None]
    assert d(*args(Hkv=3)) == ESHAPE
    assert d(*args(S=-1)) == ESHAPE
    assert d(*args(dt=F32)) == EUNSUP
    assert d(*args(D=32)) == EUNSUP
    assert d(*args(W=0)) == EUNSUP and d(*args(W=9)) == EUNSUP
    assert d(*args(theta=float("nan"))) == EUNSUP and d(*args(theta=-1.0)) == EUNSUP
    for name in names + ["cq", "ck", "mq", "mk"]:
        assert d(*args(**{name: None})) == ENULL, name
    assert d(*args(dcq=FAKE + 2)) == EALIGN
    assert d(*args(gq=FAKE + 8)) == EALIGN
    assert d(*args(mq=FAKE + 8)) == EALIGN
    assert d(*args(cq=FAKE + 1)) == EALIGN
    assert d(*args(pos=FAKE + 2)) == EALIGN
    assert d(*args(wsb=need - 1)) == EWS
    assert d(*args(ws=None)) == EWS
    assert d(*args(ws=FAKE + 8)) == EALIGN

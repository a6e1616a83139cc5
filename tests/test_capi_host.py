"""Host-only checks of the C ABI: the library loads, exports every symbol the header
declares, and rejects bad arguments with the documented codes before any HIP call.

Every call here fails validation on purpose (fake, never-dereferenced pointers), so
no kernel is ever launched and no GPU is needed.
"""

import ctypes
import math
import os
import re
import subprocess

import pytest

from online_softmax_09_amd import _lib
from parity import split_bounds

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mi355attn.h")

INVALID, UNSUPPORTED, OK = _lib.ERR_INVALID_ARG, _lib.ERR_UNSUPPORTED, _lib.OK

# Fake device addresses: 16-byte aligned, far apart, never dereferenced.
A, Bp, C, D, E = (0x100000000 * (i + 1) for i in range(5))


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libmi355attn.so not built")
    return _lib.load()


def test_header_declares_the_boundary():
    fns = header_functions()
    assert set(fns) == set(_lib.SIGNATURES), fns


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in ("fa_fwd", "fa_fwd_f32", "online_softmax_rows", "fa_strerror"):
        assert name in exported, name
    for name in header_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    # and no other C symbol leaks out of the library
    assert {n for n in exported if not n.startswith("_")} == set(header_functions())


def header_codes():
    """Name -> value of every enumerator in the header's return-code enum."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"enum\s*\{(.*?)\}", text, flags=re.S).group(1)
    codes = {}
    for item in body.split(","):
        name, _, value = (t.strip() for t in item.partition("="))
        codes[name] = codes[value] if value in codes else int(value)
    return codes


def test_return_codes_match_the_boundary():
    # The boundary's error names and values; the MI355ATTN_* names are aliases.
    codes = header_codes()
    assert {k: codes[k] for k in ("FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_HIP")} == {
        "FA_OK": 0, "FA_ERR_INVALID_ARG": -1, "FA_ERR_UNSUPPORTED": -2, "FA_ERR_HIP": -3}
    for suffix in ("OK", "ERR_INVALID_ARG", "ERR_UNSUPPORTED", "ERR_HIP"):
        assert codes["MI355ATTN_" + suffix] == codes["FA_" + suffix]
    assert (_lib.OK, _lib.ERR_INVALID_ARG, _lib.ERR_UNSUPPORTED, _lib.ERR_HIP) == (0, -1, -2, -3)


def test_version_and_strerror(lib):
    assert lib.mi355attn_version() >= 100
    for code in (OK, INVALID, UNSUPPORTED, _lib.ERR_HIP, 12345):
        assert isinstance(_lib.strerror(code), str) and _lib.strerror(code)
        assert lib.fa_strerror(code) == lib.mi355attn_strerror(code)
    assert lib.fa_strerror(OK) == b"success"
    assert b"invalid argument" in lib.fa_strerror(INVALID)
    assert b"unsupported" in lib.fa_strerror(UNSUPPORTED)
    assert b"HIP runtime error" in lib.fa_strerror(_lib.ERR_HIP)
    assert lib.mi355attn_last_hip_error() == 0


def _fa(lib, entry, q=A, k=Bp, v=C, o=D, lse=E, B=1, H=1, N=16, d=64, scale=0.125, causal=0):
    return getattr(lib, entry)(q, k, v, o, lse, B, H, N, d, scale, causal, None)


@pytest.mark.parametrize("entry", ["fa_fwd", "fa_fwd_f16", "fa_fwd_f32"])
def test_attention_argument_checks(lib, entry):
    assert _fa(lib, entry, q=None) == INVALID
    assert _fa(lib, entry, k=None) == INVALID
    assert _fa(lib, entry, v=None) == INVALID
    assert _fa(lib, entry, o=None) == INVALID
    assert _fa(lib, entry, lse=None) == INVALID
    for bad in (dict(B=0), dict(H=0), dict(N=0), dict(B=-1), dict(d=0)):
        assert _fa(lib, entry, **bad) == INVALID, bad
    for s in (math.inf, -math.inf, math.nan):
        assert _fa(lib, entry, scale=s) == INVALID
    assert _fa(lib, entry, causal=2) == INVALID
    assert _fa(lib, entry, q=A + 8) == INVALID          # misaligned
    assert _fa(lib, entry, lse=E + 4) == INVALID
    assert _fa(lib, entry, o=A + 64) == INVALID         # o overlaps q
    assert _fa(lib, entry, lse=Bp + 16) == INVALID      # lse overlaps k
    for d in (32, 96, 256, 65):
        assert _fa(lib, entry, d=d) == UNSUPPORTED, d
    assert _fa(lib, entry, B=1 << 16, H=1 << 16) == UNSUPPORTED


def test_softmax_argument_checks(lib):
    f = lib.online_softmax_rows
    assert f(A, Bp, 0, 16, None) == OK            # no rows: nothing to do, no HIP call
    assert f(None, None, 0, 16, None) == OK
    assert f(A, Bp, -1, 16, None) == INVALID
    assert f(A, Bp, 4, 0, None) == INVALID
    assert f(None, Bp, 4, 16, None) == INVALID
    assert f(A, None, 4, 16, None) == INVALID
    assert f(A + 2, Bp, 4, 16, None) == INVALID   # not even 4-byte aligned
    assert f(A, A + 16, 4, 16, None) == INVALID   # partial overlap
    assert f(A, Bp, 4, (1 << 20) + 1, None) == UNSUPPORTED
    assert f(A, Bp, 1 << 31, 4, None) == UNSUPPORTED


# More fake addresses for the gradient entry point.
F, G, Hp, I, J = (0x100000000 * (i + 6) for i in range(5))


def _bwd(lib, q=A, k=Bp, v=C, o=D, do=F, lse=E, dq=G, dk=Hp, dv=I, ws=J, B=1, H=1, N=16, d=64, scale=0.125,
         causal=0):
    return lib.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, B, H, N, d, scale, causal, None)


def test_backward_argument_checks(lib):
    for name in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "ws"):
        assert _bwd(lib, **{name: None}) == INVALID, name
    for bad in (dict(B=0), dict(H=0), dict(N=0), dict(d=0)):
        assert _bwd(lib, **bad) == INVALID, bad
    for s in (math.inf, math.nan):
        assert _bwd(lib, scale=s) == INVALID
    assert _bwd(lib, causal=-1) == INVALID
    for name, addr in (("do", F), ("dq", G), ("dk", Hp), ("dv", I), ("ws", J)):
        assert _bwd(lib, **{name: addr + 8}) == INVALID, name  # misaligned
    assert _bwd(lib, dq=A + 32) == INVALID    # dq overlaps q
    assert _bwd(lib, dk=F) == INVALID         # dk overlaps dout
    assert _bwd(lib, dv=G + 16) == INVALID    # dv overlaps dq
    assert _bwd(lib, ws=E) == INVALID         # workspace overlaps lse
    for d in (32, 96, 256):
        assert _bwd(lib, d=d) == UNSUPPORTED, d


def test_backward_workspace_size(lib):
    assert lib.fa_bwd_workspace_bytes(2, 32, 8192) == 2 * 32 * 8192 * 8
    assert lib.fa_bwd_workspace_bytes(1, 1, 1) == 8
    assert lib.fa_bwd_workspace_bytes(0, 1, 1) == -1
    assert lib.fa_bwd_workspace_bytes(1, 1, -5) == -1


def _skv(lib, q=A, k=Bp, v=C, o=D, lse=E, ws=F, B=1, H=2, Nq=3, Nk=100, d=128, scale=0.1, causal=1, n=4):
    return lib.fa_fwd_splitkv(q, k, v, o, lse, ws, B, H, Nq, Nk, d, scale, causal, n, None)


def test_splitkv_argument_checks(lib):
    for name in ("q", "k", "v", "o", "lse", "ws"):
        assert _skv(lib, **{name: None}) == INVALID, name
    for bad in (dict(B=0), dict(H=0), dict(Nq=0), dict(Nk=0), dict(d=0), dict(n=0), dict(n=4097),
                dict(causal=2), dict(Nq=101, Nk=100)):
        assert _skv(lib, **bad) == INVALID, bad
    assert _skv(lib, scale=math.nan) == INVALID
    assert _skv(lib, ws=F + 4) == INVALID             # misaligned
    assert _skv(lib, o=A + 16) == INVALID             # o overlaps q
    assert _skv(lib, ws=Bp + 32) == INVALID           # workspace overlaps k
    assert _skv(lib, lse=D + 32) == INVALID           # lse overlaps o
    assert _skv(lib, d=96) == UNSUPPORTED
    assert lib.fa_fwd_splitkv_workspace_bytes(1, 2, 3, 128, 4) == 4 * 6 * 129 * 4
    assert lib.fa_fwd_splitkv_workspace_bytes(1, 2, 3, 128, 0) == -1


def test_split_bounds_contract():
    # The part boundaries the header states for fa_fwd_splitkv (multiples of 64 keys).
    assert split_bounds(1000, 4) == [(0, 256), (256, 512), (512, 768), (768, 1000)]
    assert split_bounds(100, 8) == [(0, 64), (64, 100)] + [(100, 100)] * 6
    assert split_bounds(64, 1) == [(0, 64)]
    b = split_bounds(131072, 256)
    assert b[0] == (0, 512) and b[-1] == (130560, 131072)


def test_merge_argument_checks(lib):
    f = lib.attn_merge_states
    assert f(A, Bp, C, D, 4, 0, 128, None) == OK          # no rows: nothing to do
    assert f(None, Bp, C, D, 4, 8, 128, None) == INVALID
    assert f(A, None, C, D, 4, 8, 128, None) == INVALID
    assert f(A, Bp, None, D, 4, 8, 128, None) == INVALID
    assert f(A, Bp, C, None, 4, 8, 128, None) == INVALID
    assert f(A, Bp, C, D, 0, 8, 128, None) == INVALID
    assert f(A, Bp, C, D, 65537, 8, 128, None) == INVALID
    assert f(A, Bp, C, D, 4, -1, 128, None) == INVALID
    assert f(A + 4, Bp, C, D, 4, 8, 128, None) == INVALID  # o_parts misaligned
    assert f(A, Bp + 2, C, D, 4, 8, 128, None) == INVALID  # lse_parts misaligned
    assert f(A, Bp, A + 64, D, 4, 8, 128, None) == INVALID  # o overlaps o_parts
    assert f(A, Bp, C, Bp, 4, 8, 128, None) == INVALID     # lse overlaps lse_parts
    assert f(A, Bp, C, D, 4, 8, 32, None) == UNSUPPORTED


def test_norm_argument_checks(lib):
    rms, ln = lib.fused_add_rmsnorm, lib.fused_add_layernorm
    assert rms(A, Bp, C, D, E, 0, 64, 1e-5, None) == OK          # no rows: nothing to do
    assert rms(None, Bp, C, D, E, 4, 64, 1e-5, None) == INVALID
    assert rms(A, Bp, None, D, E, 4, 64, 1e-5, None) == INVALID
    assert rms(A, Bp, C, None, E, 4, 64, 1e-5, None) == INVALID
    assert ln(A, Bp, C, None, D, E, 4, 64, 1e-5, None) == INVALID  # LayerNorm needs beta
    assert rms(A, Bp, C, D, E, -1, 64, 1e-5, None) == INVALID
    assert rms(A, Bp, C, D, E, 4, 0, 1e-5, None) == INVALID
    assert rms(A, Bp, C, D, E, 4, 64, -1.0, None) == INVALID
    assert rms(A, Bp, C, D, E, 4, 64, math.nan, None) == INVALID
    assert rms(A + 1, Bp, C, D, E, 4, 64, 1e-5, None) == INVALID  # odd address
    assert rms(A, Bp, C, A + 64, E, 4, 64, 1e-5, None) == INVALID  # y overlaps x partially
    assert rms(A, Bp, C, D, D + 64, 4, 64, 1e-5, None) == INVALID  # y overlaps residual_out
    assert rms(A, Bp, C, C + 2, E, 4, 64, 1e-5, None) == INVALID   # y overlaps gamma
    assert rms(A, Bp, C, D, E, 4, 32769, 1e-5, None) == UNSUPPORTED
    assert rms(A, Bp, C, D, E, 4, 4097, 1e-5, None) == UNSUPPORTED  # not a multiple of 8
    assert rms(A + 2, Bp, C, D, E, 4, 8192, 1e-5, None) == UNSUPPORTED  # 2-byte units only


def _skv_na(lib, q=A, k=Bp, v=C, o=D, lse=E, B=1, H=2, Nq=3, Nk=100, d=128, scale=0.1, causal=1, n=4):
    return lib.fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, n, None)


def test_splitkv_noalloc_argument_checks(lib):
    for name in ("q", "k", "v", "o", "lse"):
        assert _skv_na(lib, **{name: None}) == INVALID, name
    for bad in (dict(B=0), dict(H=0), dict(Nq=0), dict(Nk=0), dict(d=0), dict(n=0), dict(n=4097),
                dict(causal=2), dict(Nq=101, Nk=100)):
        assert _skv_na(lib, **bad) == INVALID, bad
    assert _skv_na(lib, scale=math.inf) == INVALID
    assert _skv_na(lib, o=A + 16) == INVALID            # o overlaps q
    assert _skv_na(lib, lse=D + 32) == INVALID          # lse overlaps o
    assert _skv_na(lib, d=96) == UNSUPPORTED
    # partials beyond the 32 MiB scratch are refused before any HIP call
    limit = _lib.SPLITKV_SCRATCH_BYTES
    assert limit == 32 << 20
    H, Nq, d = 32, 16, 128
    fits = limit // (H * Nq * (d + 1) * 4)                      # 127 parts fit, 128 do not
    assert lib.fa_fwd_splitkv_workspace_bytes(1, H, Nq, d, fits) <= limit
    assert lib.fa_fwd_splitkv_workspace_bytes(1, H, Nq, d, fits + 1) > limit
    assert _skv_na(lib, H=H, Nq=Nq, Nk=32768, n=fits + 1) == UNSUPPORTED
    assert _skv_na(lib, B=4, H=H, Nq=Nq, Nk=32768, n=fits) == UNSUPPORTED

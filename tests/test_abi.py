"""The C ABI on the host: the library loads, exports what include/fmha.h declares, and
rejects bad arguments before anything is launched.  No GPU needed: every call here
returns from host validation (fake, never dereferenced device addresses)."""
import os
import re

import pytest

import head_attention_03_amd as fmha

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fmha.h")
P = 0x10000  # 16-byte aligned stand-in address; validation never dereferences it


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fmha_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = fmha.load()
    names = declared_functions()
    assert names == sorted(fmha.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert fmha.fmha_version() >= 100
    for s in range(7):
        assert fmha.fmha_status_string(s)
    assert fmha.fmha_status_string(0) == "ok"
    assert fmha.fmha_status_string(99) == "unknown status"


def call(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, Sq=16, Sk=16, H=2, H_kv=1, D=64, scale=0.125, mask="none",
             dtype="f16", o_scale=1.0, varlen=None, stream=None)
    a.update(kw)
    return fmha.fmha_fwd(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=0), 1), (dict(v=None), 1), (dict(o=None), 1), (dict(k=None, Sk=0, B=0, v=None), 0),
    (dict(k=None, varlen=fmha.make_varlen(P, P, 16, 5)), 1),
    (dict(varlen=fmha.make_varlen(P, None, 16, 16)), 1),
    (dict(varlen=fmha.make_varlen(None, None, 16, 16)), 1),
    (dict(B=-1), 2), (dict(Sq=-3), 2), (dict(Sk=-1), 2), (dict(H=-2), 2),
    (dict(H=3, H_kv=2), 2), (dict(H_kv=0), 2), (dict(D=48), 2), (dict(D=256), 2), (dict(D=0), 2),
    (dict(varlen=fmha.make_varlen(P, P, -1, 16)), 2),
    (dict(dtype=3), 3), (dict(dtype=-1), 3), (dict(mask=4), 3), (dict(mask=-1), 3),
    (dict(Sq=1 << 22, H=64, H_kv=64, D=128), 3),
    (dict(dtype="f8e4m3", D=32), 3), (dict(H=1 << 16, H_kv=1 << 16, D=128, Sq=1, Sk=1), 3),
    (dict(H=1 << 15, H_kv=1, D=128, Sq=1, Sk=1), 3),
    (dict(q=P + 2), 4), (dict(o=P + 8), 4), (dict(lse=P + 2), 4),
    (dict(scale=0.0), 5), (dict(scale=-0.1), 5), (dict(scale=float("inf")), 5), (dict(scale=float("nan")), 5),
    (dict(o_scale=float("inf")), 5), (dict(o_scale=float("nan")), 5),
])
def test_invalid_arguments_are_rejected(kw, status):
    assert call(**kw) == status


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(Sq=0),
                                dict(varlen=fmha.make_varlen(P, P, 0, 5))])
def test_empty_problems_return_ok_without_launch(kw):
    assert call(**kw) == 0


def test_check_raises_with_status_name():
    with pytest.raises(fmha.FmhaError, match="FMHA_ERR_INVALID_SHAPE"):
        fmha.check(call(D=48))

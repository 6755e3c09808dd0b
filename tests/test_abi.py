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
    for s in range(8):
        assert fmha.fmha_status_string(s) and fmha.fmha_status_string(s) != "unknown status"
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
    (dict(B=1 << 10, Sq=1 << 21, H=64, H_kv=64, D=128), 3),  # 2^31 query rows: past int32 row indices
    (dict(dtype="f8e4m3", D=32, q=P + 2), 4), (dict(H=1 << 16, H_kv=1 << 16, D=128, Sq=1, Sk=1), 3),
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


# ---- split-KV entry point ----------------------------------------------------------------
def call_skv(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, Sq=1, Sk=300, H=4, H_kv=2, D=64, scale=0.125, mask="none",
             dtype="f16", o_scale=1.0, varlen=None, workspace=P, workspace_bytes=1 << 30, stream=None)
    a.update(kw)
    return fmha.fmha_fwd_splitkv(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(v=None), 1), (dict(o=None), 1), (dict(workspace=None), 1),
    (dict(varlen=fmha.make_varlen(P, None, 1, 300)), 1),
    (dict(B=-1), 2), (dict(H=3, H_kv=2), 2), (dict(D=96), 2),
    (dict(dtype="f8e4m3", D=32, workspace_bytes=100), 5), (dict(dtype=7), 3), (dict(mask=9), 3),
    (dict(Sq=1 << 16, H=128, H_kv=128, D=128), 3),  # 2 GiB of Q in one sequence
    (dict(H=1 << 15, H_kv=1 << 15, D=128), 3),  # a K row of 8 MiB: a split would pass 31-bit offsets
    (dict(q=P + 4), 4), (dict(lse=P + 1), 4), (dict(workspace=P + 8), 4),
    (dict(scale=0.0), 5), (dict(o_scale=float("nan")), 5), (dict(workspace_bytes=100), 5),
])
def test_splitkv_invalid_arguments_are_rejected(kw, status):
    assert call_skv(**kw) == status


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(Sq=0), dict(B=0, workspace=None, workspace_bytes=0)])
def test_splitkv_empty_problems_return_ok_without_launch(kw):
    assert call_skv(**kw) == 0


def test_splitkv_workspace_is_rejected_one_byte_short():
    need = fmha.fmha_fwd_splitkv_workspace_size(1, 1, 300, 4, 2, 64)
    assert need > 0
    assert call_skv(workspace_bytes=need - 1) == 5


@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 1, 32), (16, 1, 8192, 32, 8, 128), (2, 4, 1000, 16, 2, 64),
                                   (3, 16, 70000, 8, 8, 128), (64, 1, 300, 8, 1, 64), (1, 300, 5, 4, 4, 32)])
def test_splitkv_workspace_size_holds_whole_splits(shape):
    # n_splits partial rows of D fp32 values and one fp32 LSE per (query row, head), n_splits >= 1,
    # and no split shorter than the 256-key minimum unless there is only one
    B, Sq, Sk, H, H_kv, D = shape
    rows = B * Sq * H
    need = fmha.fmha_fwd_splitkv_workspace_size(B, Sq, Sk, H, H_kv, D)
    assert need % (rows * (D + 1) * 4) == 0
    n_splits = need // (rows * (D + 1) * 4)
    assert 1 <= n_splits <= max(1, -(-Sk // 256))


def test_splitkv_workspace_size_packed_uses_total_rows():
    vl = fmha.make_varlen(P, P, 7, 5000)
    need = fmha.fmha_fwd_splitkv_workspace_size(3, 4, 3000, 8, 2, 64, vl)
    assert need > 0 and need % (7 * 8 * 65 * 4) == 0
    assert fmha.fmha_fwd_splitkv_workspace_size(3, 4, 3000, 6, 4, 64) == 0  # H % H_kv != 0


# ---- allocation-free split-KV entry point: host validation (nothing here reaches the device) ----
def call_noalloc(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, Sq=1, Sk=300, H=4, H_kv=2, D=64, scale=0.125, mask="none",
             dtype="f16", o_scale=1.0, varlen=None, stream=None)
    a.update(kw)
    return fmha.fmha_fwd_splitkv_noalloc(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(v=None), 1), (dict(B=-1), 2), (dict(D=96), 2), (dict(dtype="f8e4m3", D=32, q=P + 4), 4),
    (dict(q=P + 4), 4), (dict(scale=0.0), 5),
    # 64 sequences x 16 new tokens x 64 heads x D 128: the partials need more than the 32 MiB scratch
    (dict(B=64, Sq=16, Sk=8192, H=64, H_kv=8, D=128), 7),
])
def test_noalloc_invalid_arguments_are_rejected(kw, status):
    assert call_noalloc(**kw) == status


def test_noalloc_limit_is_the_workspace_size():
    # the largest shapes are refused exactly when the caller-workspace entry point would need more
    # than 32 MiB of workspace
    big = (64, 16, 8192, 64, 8, 128)
    assert fmha.fmha_fwd_splitkv_workspace_size(*big) > 32 << 20
    assert fmha.fmha_fwd_splitkv_workspace_size(16, 1, 8192, 32, 8, 128) <= 32 << 20


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(Sq=0)])
def test_noalloc_empty_problems_return_ok_without_launch(kw):
    assert call_noalloc(**kw) == 0


def test_splitkv_workspace_size_ignores_kv_bytes():
    # a cache of 2^20 keys x 8 heads x 128 dims (2 GiB of K): both entry points take it (the
    # contiguous kernels place their descriptors at each split); 8 units of work split 128 ways
    # for the 1024-workgroup target, so the workspace holds 128 partials of 32 rows
    need = fmha.fmha_fwd_splitkv_workspace_size(1, 1, 1 << 20, 32, 8, 128)
    assert need == 128 * 32 * (128 + 1) * 4
    assert call_skv(Sk=1 << 20, H=32, H_kv=8, D=128, workspace_bytes=need - 1) == 5  # shapes pass, one byte short
    pk = fmha.make_paged_kv(P, P, 1 << 13, 128, 1 << 13, "bf16")
    assert fmha.fmha_fwd_splitkv_paged(q=P, k_cache=P, v_cache=P, o=P, lse=None, B=1, Sq=1, Sk=1 << 20, H=32, H_kv=8,
                                       D=128, scale=0.125, mask="none", dtype="bf16", paged=pk, workspace=P,
                                       workspace_bytes=need - 1) == 5  # passes the shape checks, one byte short


# ----------------------------------------------------------------------------------------------
# fmha_bwd: host validation and workspace size
# ----------------------------------------------------------------------------------------------
def call_bwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, dout=P, lse=P, dq=P, dk=P, dv=P, B=1, Sq=16, Sk=16, H=2, H_kv=1, D=64, scale=0.125,
             mask="causal_qbegin", dtype="bf16", varlen=None, workspace=P, workspace_bytes=1 << 20, stream=None)
    a.update(kw)
    return fmha.fmha_bwd(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(dout=None), 1), (dict(lse=None), 1), (dict(dq=None), 1),
    (dict(k=None), 1), (dict(v=None), 1), (dict(dk=None), 1), (dict(dv=None), 1), (dict(workspace=None), 1),
    (dict(varlen=fmha.make_varlen(P, None, 16, 16)), 1), (dict(varlen=fmha.make_varlen(None, None, 16, 16)), 1),
    (dict(B=-1), 2), (dict(Sk=-1), 2), (dict(H=3, H_kv=2), 2), (dict(H_kv=0), 2), (dict(D=48), 2),
    (dict(varlen=fmha.make_varlen(P, P, 16, -1)), 2),
    (dict(dtype=3), 3), (dict(mask=4), 3), (dict(mask=-1), 3),
    (dict(H=70000, H_kv=70000, Sq=1, Sk=1), 3), (dict(Sq=1 << 22, H=64, H_kv=64, D=128), 3),
    (dict(q=P + 2), 4), (dict(dq=P + 8), 4), (dict(dk=P + 4), 4), (dict(dout=P + 2), 4), (dict(lse=P + 2), 4),
    (dict(workspace=P + 8), 4),
    (dict(scale=0.0), 5), (dict(scale=float("inf")), 5), (dict(scale=float("nan")), 5), (dict(workspace_bytes=0), 5),
    # e4m3: the statistics alone are not enough (the bf16 copies of the inputs follow them)
    (dict(dtype="f8e4m3", workspace_bytes=2 * 512), 5), (dict(dtype="f8e4m3", q=None), 1),
    (dict(dtype="f8e4m3", o=P + 8), 4),
    # no query rows: the q-side pointers and the workspace are not needed; no keys: the k side
    (dict(B=0, q=None, k=None, workspace=None), 0),
])
def test_bwd_rejects_bad_arguments(kw, status):
    assert call_bwd(**kw) == status


def test_bwd_workspace_size():
    # dense: 512 bytes per 64-row block of every (sequence, head)
    assert fmha.fmha_bwd_workspace_size(4, 2048, 2048, 16, 16, 128, "bf16", None) == 4 * 16 * 32 * 512
    assert fmha.fmha_bwd_workspace_size(2, 65, 10, 3, 1, 64, "f16", None) == 2 * 3 * 2 * 512
    assert fmha.fmha_bwd_workspace_size(1, 0, 10, 3, 1, 64, "bf16", None) == 0
    # packed: per head, floor(total_q / 64) + B + 1 blocks (sequences start on their own block)
    vl = fmha.make_varlen(P, P, 1000, 50)
    assert fmha.fmha_bwd_workspace_size(5, 400, 30, 4, 2, 128, "bf16", vl) == 4 * (1000 // 64 + 5 + 1) * 512
    # e4m3: the statistics, then bf16 copies of q, o, dO (rows_q x H x D) and k, v (rows_k x H_kv x D),
    # each starting on a 256-byte boundary
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    stats = 2 * 3 * 2 * 512
    assert fmha.fmha_bwd_workspace_size(2, 65, 10, 3, 1, 64, "f8e4m3", None) == (
        up(stats) + 3 * up(2 * 2 * 65 * 3 * 64) + 2 * up(2 * 2 * 10 * 1 * 64))
    assert fmha.fmha_bwd_workspace_size(5, 400, 30, 4, 2, 128, "f8e4m3", vl) == (
        up(4 * (1000 // 64 + 5 + 1) * 512) + 3 * up(2 * 1000 * 4 * 128) + 2 * up(2 * 50 * 2 * 128))
    # e4m3 with no query rows still needs the copies of k and v
    assert fmha.fmha_bwd_workspace_size(1, 0, 10, 3, 1, 64, "f8e4m3", None) == 2 * up(2 * 10 * 64)
    # invalid shapes and dtypes
    assert fmha.fmha_bwd_workspace_size(1, 16, 16, 3, 2, 64, "bf16", None) == 0
    assert fmha.fmha_bwd_workspace_size(1, 16, 16, 2, 2, 48, "bf16", None) == 0
    assert fmha.fmha_bwd_workspace_size(1, 16, 16, 2, 2, 64, 7, None) == 0
    # one byte short of the size is rejected
    need = fmha.fmha_bwd_workspace_size(1, 16, 16, 2, 1, 64, "bf16", None)
    assert call_bwd(workspace_bytes=need - 1) == 5
    need8 = fmha.fmha_bwd_workspace_size(1, 16, 16, 2, 1, 64, "f8e4m3", None)
    assert need8 > need
    assert call_bwd(dtype="f8e4m3", workspace_bytes=need8 - 1) == 5
    # e4m3 with keys but no query rows: the workspace is required
    assert call_bwd(dtype="f8e4m3", Sq=0, q=None, workspace=None) == 1


# ----------------------------------------------------------------------------------------------
# fmha_fwd_splitkv_paged: host validation
# ----------------------------------------------------------------------------------------------
def call_paged(**kw):
    pk = kw.pop("paged", fmha.make_paged_kv(P, P, 4, 128, 8, "bf16"))
    a = dict(q=P, k_cache=P, v_cache=P, o=P, lse=None, B=1, Sq=1, Sk=500, H=8, H_kv=2, D=128, scale=0.1,
             mask="none", dtype="bf16", o_scale=1.0, paged=pk, workspace=P, workspace_bytes=1 << 24, stream=None)
    a.update(kw)
    return fmha.fmha_fwd_splitkv_paged(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(paged=None), 1), (dict(k_cache=None), 1), (dict(q=None), 1), (dict(workspace=None), 1),
    (dict(paged=fmha.make_paged_kv(None, P, 4, 128, 8, "bf16")), 1), (dict(paged=fmha.make_paged_kv(P, None, 4, 128, 8, "bf16")), 1),
    (dict(paged=fmha.make_paged_kv(P, P, 4, 96, 8, "bf16")), 2), (dict(paged=fmha.make_paged_kv(P, P, 4, 16, 8, "bf16")), 2),
    (dict(paged=fmha.make_paged_kv(P, P, 3, 128, 8, "bf16")), 2), (dict(paged=fmha.make_paged_kv(P, P, 4, 128, 0, "bf16")), 2),
    (dict(paged=fmha.make_paged_kv(P, P, 4, 1 << 17, 8, "bf16")), 2),
    (dict(paged=fmha.make_paged_kv(P, P, 4, 128, 8, "f16")), 3), (dict(paged=fmha.make_paged_kv(P, P, 4, 128, 8, 7)), 3),
    (dict(paged=fmha.make_paged_kv(P, P, 4, 128, 8, "f8e4m3"), D=32, workspace_bytes=16), 5),
    (dict(dtype="f8e4m3"), 3),  # e4m3 queries over a bf16 cache
    (dict(dtype="f8e4m3", paged=fmha.make_paged_kv(P, P, 4, 128, 8, "f8e4m3"), D=32, workspace_bytes=16), 5),
    (dict(dtype="f8e4m3", paged=fmha.make_paged_kv(P, P, 4, 128, 8, "f8e4m3"), q=P + 4), 4),  # accepted up to alignment
    (dict(H=3), 2), (dict(D=48), 2),
    (dict(k_cache=P + 8), 4), (dict(workspace=P + 8), 4),
    (dict(scale=0.0), 5), (dict(workspace_bytes=16), 5),
    (dict(B=0), 0), (dict(Sk=0, k_cache=None, v_cache=None, paged=fmha.make_paged_kv(None, None, 0, 128, 0, "bf16"), B=0), 0),
])
def test_paged_rejects_bad_arguments(kw, status):
    assert call_paged(**kw) == status


# ----------------------------------------------------------------------------------------------
# fmha_paged_kv_append: host validation (every case returns before any launch)
# ----------------------------------------------------------------------------------------------
def call_append(**kw):
    pk = kw.pop("paged", fmha.make_paged_kv(P, P, 4, 128, 8, "bf16"))
    a = dict(k_cache=P, v_cache=P, k_new=P, v_new=P, B=2, S_new=1, H_kv=2, D=128, paged=pk, stream=None)
    a.update(kw)
    return fmha.fmha_paged_kv_append(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(paged=None), 1), (dict(k_cache=None), 1), (dict(v_cache=None), 1), (dict(k_new=None), 1),
    (dict(v_new=None), 1),
    (dict(paged=fmha.make_paged_kv(None, P, 4, 128, 8, "bf16")), 1), (dict(paged=fmha.make_paged_kv(P, None, 4, 128, 8, "bf16")), 1),
    (dict(B=-1), 2), (dict(S_new=-1), 2), (dict(H_kv=0), 2), (dict(D=48), 2),
    (dict(paged=fmha.make_paged_kv(P, P, 4, 96, 8, "bf16")), 2), (dict(paged=fmha.make_paged_kv(P, P, 4, 16, 8, "bf16")), 2),
    (dict(paged=fmha.make_paged_kv(P, P, 0, 128, 8, "bf16")), 2), (dict(paged=fmha.make_paged_kv(P, P, 4, 128, 0, "bf16")), 2),
    (dict(paged=fmha.make_paged_kv(P, P, 4, 128, 8, 7)), 3),
    (dict(B=1 << 16, S_new=1 << 15), 3), (dict(H_kv=1 << 23), 3),
    (dict(k_cache=P + 8), 4), (dict(v_new=P + 4), 4),
    (dict(B=0), 0), (dict(S_new=0), 0), (dict(B=0, k_cache=None, k_new=None), 0),
])
def test_append_rejects_bad_arguments(kw, status):
    assert call_append(**kw) == status

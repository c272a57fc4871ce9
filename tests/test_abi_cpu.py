"""CPU-side checks of the C ABI: the library loads, exports every function
the header declares, its structs have the layout ctypes assumes, and bad
arguments are refused on the host before anything reaches a GPU.

No test here launches a kernel: every call below fails argument checking,
which happens before any HIP call.
"""
import ctypes
import os
import re
import subprocess

import pytest

from block_sparse_masked_fa_amd import _capi as C
from block_sparse_masked_fa_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flexattn.h")

needs_lib = pytest.mark.skipif(not os.path.exists(C.LIB_PATH),
                               reason="libflexattn.so not built")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S[^\n(]*?\b(fa_[a-z_0-9]+)\s*\(", text,
                                 flags=re.M)))


def test_header_and_binding_agree():
    declared = _declared_functions()
    assert declared == sorted(C.SIGNATURES), declared


@needs_lib
def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", C.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fa_[a-z_0-9]+)$", out, flags=re.M))
    for name in _declared_functions():
        assert name in exported, name
    L = C.lib()
    for name in _declared_functions():
        assert hasattr(L, name)
    assert L.fa_abi_version() == C.ABI_VERSION


@needs_lib
def test_every_kernel_launch_stub_is_defined():
    # a kernel whose host-side stub was not emitted leaves an undefined
    # symbol that only fails when the library is loaded for a launch
    out = subprocess.run(["nm", "-D", C.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    missing = [l for l in out.splitlines()
               if " U " in l and "__device_stub" in l]
    assert not missing, missing


def test_struct_layout_matches_c(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(f"""
#include <stdio.h>
#include <stddef.h>
#include "{HEADER}"
int main(void) {{
  printf("%zu %zu %zu %zu\\n", sizeof(fa_mask_mod), offsetof(fa_mask_mod, doc_id),
         offsetof(fa_mask_mod, doc_len), offsetof(fa_mask_mod, doc_stride));
  printf("%zu %zu\\n", sizeof(fa_score_mod), offsetof(fa_score_mod, softcap));
  printf("%zu %zu %zu %zu %zu\\n", sizeof(fa_block_mask),
         offsetof(fa_block_mask, B), offsetof(fa_block_mask, separate_full_blocks),
         offsetof(fa_block_mask, kv_num_blocks),
         offsetof(fa_block_mask, full_kv_indices));
  return 0;
}}
""")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-o", str(exe), str(src)],
                   check=True)
    lines = subprocess.run([str(exe)], capture_output=True, text=True,
                           check=True).stdout.split("\n")
    got = [list(map(int, l.split())) for l in lines if l.strip()]
    assert got[0] == [ctypes.sizeof(C.fa_mask_mod), C.fa_mask_mod.doc_id.offset,
                      C.fa_mask_mod.doc_len.offset,
                      C.fa_mask_mod.doc_stride.offset]
    assert got[1] == [ctypes.sizeof(C.fa_score_mod),
                      C.fa_score_mod.softcap.offset]
    assert got[2] == [ctypes.sizeof(C.fa_block_mask), C.fa_block_mask.B.offset,
                      C.fa_block_mask.separate_full_blocks.offset,
                      C.fa_block_mask.kv_num_blocks.offset,
                      C.fa_block_mask.full_kv_indices.offset]


def test_header_compiles_as_c_and_cpp(tmp_path):
    for comp, ext in (("gcc", "c"), ("g++", "cpp")):
        src = tmp_path / f"inc.{ext}"
        src.write_text(f'#include "{HEADER}"\nint main(void){{return 0;}}\n')
        subprocess.run([comp, "-Wall", "-Werror", "-o",
                        str(tmp_path / f"inc_{ext}"), str(src)], check=True)


@needs_lib
def test_status_strings():
    L = C.lib()
    names = [L.fa_status_string(s).decode() for s in range(6)]
    assert names == ["FA_OK", "FA_ERR_NULL_POINTER", "FA_ERR_INVALID_VALUE",
                     "FA_ERR_UNSUPPORTED", "FA_ERR_SHAPE_MISMATCH",
                     "FA_ERR_HIP"]
    assert L.fa_status_string(99).decode() == "unknown fa_status"


@needs_lib
def test_block_mask_dims():
    assert api.fa_block_mask_dims(256, 256, 64, 64) == (4, 4)
    assert api.fa_block_mask_dims(300, 129, 128, 64) == (3, 3)
    assert api.fa_block_mask_dims(0, 0, 128, 128) == (0, 0)
    for bad in ((-1, 4, 4, 4), (4, 4, 0, 4), (4, 4, 4, 2000)):
        with pytest.raises(C.FlexAttnError):
            api.fa_block_mask_dims(*bad)
    with pytest.raises(C.FlexAttnError, match="FA_ERR_UNSUPPORTED"):
        api.fa_block_mask_dims(1 << 30, 1 << 30, 1, 1)


FAKE = 1 << 20  # a non-null, 16-byte aligned address that is never touched


def _bm(**kw):
    b = C.fa_block_mask(kv_num_blocks=FAKE, kv_indices=FAKE,
                        full_kv_num_blocks=FAKE, full_kv_indices=FAKE)
    for k, v in kw.items():
        setattr(b, k, v)
    return b


@needs_lib
@pytest.mark.parametrize("mask,B,H,ql,kl,bm_,bn_,status", [
    (C.fa_mask_mod(kind=C.FA_MASK_SLIDING_WINDOW, window=0), 1, 1, 64, 64,
     64, 64, C.FA_ERR_INVALID_VALUE),
    (C.fa_mask_mod(kind=C.FA_MASK_DOCUMENT), 1, 1, 64, 64, 64, 64,
     C.FA_ERR_NULL_POINTER),
    (C.fa_mask_mod(kind=C.FA_MASK_DOCUMENT, doc_id=FAKE, doc_len=63), 1, 1,
     64, 64, 64, 64, C.FA_ERR_SHAPE_MISMATCH),
    (C.fa_mask_mod(kind=C.FA_MASK_DOCUMENT, doc_id=FAKE, doc_len=64,
                   doc_stride=-64), 2, 1, 64, 64, 64, 64,
     C.FA_ERR_INVALID_VALUE),
    (C.fa_mask_mod(kind=C.FA_MASK_LOCAL_WINDOW, window=0), 1, 1, 64, 64,
     64, 64, C.FA_ERR_INVALID_VALUE),
    (C.fa_mask_mod(kind=7), 1, 1, 64, 64, 64, 64, C.FA_ERR_INVALID_VALUE),
    (C.fa_mask_mod(kind=C.FA_MASK_CAUSAL), 0, 1, 64, 64, 64, 64,
     C.FA_ERR_INVALID_VALUE),
    (C.fa_mask_mod(kind=C.FA_MASK_CAUSAL), 1, 1, 64, 64, 0, 64,
     C.FA_ERR_INVALID_VALUE),
    (C.fa_mask_mod(kind=C.FA_MASK_CAUSAL), 1, 1, 64, 64, 64, 4096,
     C.FA_ERR_UNSUPPORTED),
    (C.fa_mask_mod(kind=C.FA_MASK_CAUSAL), 1, 1, -1, 64, 64, 64,
     C.FA_ERR_INVALID_VALUE),
])
def test_create_block_mask_refuses(mask, B, H, ql, kl, bm_, bn_, status):
    b = _bm()
    st = api.fa_create_block_mask(mask, B, H, ql, kl, bm_, bn_, 1, b, None)
    assert st == status, C.lib().fa_last_error()
    assert C.lib().fa_last_error().decode()


@needs_lib
def test_create_block_mask_null_arrays():
    m = C.fa_mask_mod(kind=C.FA_MASK_CAUSAL)
    for field in ("kv_num_blocks", "kv_indices", "full_kv_num_blocks",
                  "full_kv_indices"):
        b = _bm(**{field: None})
        st = api.fa_create_block_mask(m, 1, 1, 64, 64, 64, 64, 1, b, None)
        assert st == C.FA_ERR_NULL_POINTER, field
    st = C.lib().fa_create_block_mask(ctypes.byref(m), 1, 1, 64, 64, 64, 64,
                                      1, None, None)
    assert st == C.FA_ERR_NULL_POINTER
    st = C.lib().fa_create_block_mask(None, 1, 1, 64, 64, 64, 64, 1,
                                      ctypes.byref(_bm()), None)
    assert st == C.FA_ERR_NULL_POINTER


def _good_bm(q_len=256, kv_len=256, block=128, B=1, H=1):
    nq = -(-q_len // block)
    nk = -(-kv_len // block)
    return _bm(mask=C.fa_mask_mod(kind=C.FA_MASK_CAUSAL), B=B, H=H,
               q_len=q_len, kv_len=kv_len, block_m=block, block_n=block,
               num_q_blocks=nq, num_kv_blocks=nk, separate_full_blocks=1)


def _fwd(**over):
    a = dict(dtype=C.FA_BF16, B=2, H=4, H_kv=4, q_len=256, kv_len=256, D=128,
             q=FAKE, q_stride=(4 * 256 * 128, 256 * 128, 128), k=FAKE,
             k_stride=(4 * 256 * 128, 256 * 128, 128), v=FAKE,
             v_stride=(4 * 256 * 128, 256 * 128, 128), scale=0.088,
             bm=_good_bm(), score=C.fa_score_mod(kind=C.FA_SCORE_NONE),
             o=FAKE, lse=FAKE, stream=None, workspace=None, workspace_bytes=0)
    a.update(over)
    return api.fa_flex_attention_fwd(**a)


@needs_lib
@pytest.mark.parametrize("over,status", [
    (dict(dtype=9), C.FA_ERR_INVALID_VALUE),
    (dict(D=96), C.FA_ERR_UNSUPPORTED),
    (dict(D=256), C.FA_ERR_UNSUPPORTED),
    (dict(H_kv=3), C.FA_ERR_INVALID_VALUE),
    (dict(H_kv=0), C.FA_ERR_INVALID_VALUE),
    (dict(scale=0.0), C.FA_ERR_INVALID_VALUE),
    (dict(scale=float("nan")), C.FA_ERR_INVALID_VALUE),
    (dict(scale=float("inf")), C.FA_ERR_INVALID_VALUE),
    (dict(q_len=128), C.FA_ERR_SHAPE_MISMATCH),
    (dict(kv_len=512), C.FA_ERR_SHAPE_MISMATCH),
    (dict(bm=_good_bm(B=3)), C.FA_ERR_SHAPE_MISMATCH),
    (dict(bm=_good_bm(H=2)), C.FA_ERR_SHAPE_MISMATCH),
    (dict(bm=_good_bm(block=32)), C.FA_ERR_UNSUPPORTED),
    (dict(bm=_bm(**{**{f: getattr(_good_bm(), f) for f, _ in
                       C.fa_block_mask._fields_}, "block_n": 256,
                    "num_kv_blocks": 1})), C.FA_ERR_UNSUPPORTED),
    (dict(dtype=C.FA_FP32, D=64, q_stride=(4 * 256 * 64, 256 * 64, 64),
          k_stride=(4 * 256 * 64, 256 * 64, 64),
          v_stride=(4 * 256 * 64, 256 * 64, 64),
          bm=_bm(**{**{f: getattr(_good_bm(), f) for f, _ in
                       C.fa_block_mask._fields_}, "block_n": 64,
                    "num_kv_blocks": 4})), C.FA_ERR_UNSUPPORTED),
    (dict(bm=_bm(**{**{f: getattr(_good_bm(), f) for f, _ in
                       C.fa_block_mask._fields_}, "num_kv_blocks": 5})),
     C.FA_ERR_SHAPE_MISMATCH),
    (dict(score=C.fa_score_mod(kind=C.FA_SCORE_SOFTCAP, softcap=0.0)),
     C.FA_ERR_INVALID_VALUE),
    (dict(score=C.fa_score_mod(kind=C.FA_SCORE_SOFTCAP,
                               softcap=float("inf"))),
     C.FA_ERR_INVALID_VALUE),
    (dict(score=C.fa_score_mod(kind=5)), C.FA_ERR_INVALID_VALUE),
    (dict(q=None), C.FA_ERR_NULL_POINTER),
    (dict(o=None), C.FA_ERR_NULL_POINTER),
    (dict(k=None), C.FA_ERR_NULL_POINTER),
    (dict(bm=None), C.FA_ERR_NULL_POINTER),
    (dict(q=FAKE + 8), C.FA_ERR_UNSUPPORTED),
    (dict(v=FAKE + 2), C.FA_ERR_UNSUPPORTED),
    (dict(q_stride=(4 * 256 * 128, 256 * 128, 100)), C.FA_ERR_UNSUPPORTED),
    (dict(k_stride=(4 * 256 * 128, -128, 128)), C.FA_ERR_INVALID_VALUE),
    (dict(B=-1), C.FA_ERR_INVALID_VALUE),
    (dict(workspace=FAKE + 4, workspace_bytes=256), C.FA_ERR_UNSUPPORTED),
    (dict(workspace=FAKE, workspace_bytes=255), C.FA_ERR_INVALID_VALUE),
])
def test_fwd_refuses(over, status):
    if "bm" in over and over["bm"] is None:
        a = dict(over)
        st = C.lib().fa_flex_attention_fwd(
            C.FA_BF16, 1, 1, 1, 256, 256, 128, FAKE, C.Stride3(1, 1, 128),
            FAKE, C.Stride3(1, 1, 128), FAKE, C.Stride3(1, 1, 128), 0.1,
            None, None, None, 0, FAKE, FAKE, None)
        assert st == status
        return
    st = _fwd(**over)
    assert st == status, C.lib().fa_last_error()


@needs_lib
def test_fwd_refuses_broadcast_of_per_batch_document_mask():
    bm = _good_bm()
    bm.mask = C.fa_mask_mod(kind=C.FA_MASK_DOCUMENT, doc_id=FAKE, doc_len=256,
                            doc_stride=256)
    assert _fwd(bm=bm) == C.FA_ERR_SHAPE_MISMATCH       # bm.B = 1, call B = 2
    bm.mask.doc_stride = 0
    bm2 = _good_bm(B=2)
    bm2.mask = C.fa_mask_mod(kind=C.FA_MASK_DOCUMENT, doc_id=FAKE, doc_len=255,
                             doc_stride=256)
    assert _fwd(bm=bm2) == C.FA_ERR_SHAPE_MISMATCH      # doc_len < q_len


@needs_lib
def test_fwd_empty_problem_is_a_noop():
    # B = 0 or q_len = 0: succeeds without touching any pointer or the GPU
    assert _fwd(B=0, q=None, k=None, v=None, o=None) == C.FA_OK
    bm = _good_bm(q_len=0)
    bm.num_q_blocks = 0
    assert _fwd(q_len=0, bm=bm, q=None, o=None) == C.FA_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(C, "_lib", None)
    monkeypatch.setattr(C, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        C.lib()


@needs_lib
def test_split_workspace_bytes():
    # num_splits * B * H * q_len * (D + 2) * 4: fp32 partial outputs, then the
    # per-row maximum and sum
    assert api.fa_split_workspace_bytes(1, 1, 8192, 64, 8) == 8 * 8192 * 66 * 4
    assert api.fa_split_workspace_bytes(2, 3, 100, 128, 5) == 5 * 6 * 100 * 130 * 4
    assert api.fa_split_workspace_bytes(2, 3, 100, 128, 1) == 0
    assert api.fa_split_workspace_bytes(0, 3, 100, 128, 4) == 0
    for bad in (dict(num_splits=0), dict(num_splits=C.FA_MAX_SPLITS + 1),
                dict(B=-1), dict(q_len=-5)):
        a = dict(B=1, H=1, q_len=64, D=64, num_splits=2)
        a.update(bad)
        with pytest.raises(C.FlexAttnError) as e:
            api.fa_split_workspace_bytes(**a)
        assert e.value.status == C.FA_ERR_INVALID_VALUE, bad
    assert C.lib().fa_split_workspace_bytes(1, 1, 64, 64, 2, None) == \
        C.FA_ERR_NULL_POINTER


def _fwd_split(**over):
    a = dict(dtype=C.FA_BF16, B=2, H=4, H_kv=4, q_len=256, kv_len=256, D=128,
             q=FAKE, q_stride=(4 * 256 * 128, 256 * 128, 128), k=FAKE,
             k_stride=(4 * 256 * 128, 256 * 128, 128), v=FAKE,
             v_stride=(4 * 256 * 128, 256 * 128, 128), scale=0.088,
             bm=_good_bm(), score=C.fa_score_mod(kind=C.FA_SCORE_NONE),
             num_splits=4, workspace=FAKE,
             workspace_bytes=4 * 8 * 256 * 130 * 4, o=FAKE, lse=FAKE,
             stream=None)
    a.update(over)
    return api.fa_flex_attention_fwd_split(**a)


@needs_lib
@pytest.mark.parametrize("over,status", [
    (dict(num_splits=0), C.FA_ERR_INVALID_VALUE),
    (dict(num_splits=C.FA_MAX_SPLITS + 1), C.FA_ERR_INVALID_VALUE),
    (dict(workspace_bytes=4 * 8 * 256 * 130 * 4 - 1), C.FA_ERR_INVALID_VALUE),
    (dict(workspace=None), C.FA_ERR_NULL_POINTER),
    (dict(workspace=FAKE + 4), C.FA_ERR_UNSUPPORTED),
    (dict(dtype=C.FA_FP32, D=64, q_stride=(4 * 256 * 64, 256 * 64, 64),
          k_stride=(4 * 256 * 64, 256 * 64, 64),
          v_stride=(4 * 256 * 64, 256 * 64, 64)), C.FA_ERR_UNSUPPORTED),
    # the forward's own checks come first
    (dict(D=96), C.FA_ERR_UNSUPPORTED),
    (dict(scale=0.0), C.FA_ERR_INVALID_VALUE),
    (dict(bm=_good_bm(B=3)), C.FA_ERR_SHAPE_MISMATCH),
    (dict(q=None), C.FA_ERR_NULL_POINTER),
])
def test_fwd_split_refuses(over, status):
    st = _fwd_split(**over)
    assert st == status, C.lib().fa_last_error()


@needs_lib
def test_fwd_split_empty_problem_is_a_noop():
    assert _fwd_split(B=0, q=None, k=None, v=None, o=None,
                      workspace_bytes=0, workspace=FAKE) == C.FA_OK


def test_auto_num_splits():
    import torch
    # two workgroups per compute unit when the grid is short of one per unit
    assert api.auto_num_splits(torch.bfloat16, 1, 1, 64, 256) == 8
    assert api.auto_num_splits(torch.bfloat16, 1, 1, 3, 256) == \
        min(C.FA_MAX_SPLITS, -(-512 // 3))
    assert api.auto_num_splits(torch.bfloat16, 4, 16, 64, 256) == 1
    assert api.auto_num_splits(torch.bfloat16, 1, 1, 256, 256) == 1
    assert api.auto_num_splits(torch.float32, 1, 1, 4, 256) == 1
    assert api.auto_num_splits(torch.bfloat16, 0, 1, 4, 256) == 1


def _bwd_ws_bytes(B, H, q_len, nq, nk, Bm=1, Hm=1, full=True, H_kv=None,
                  kv_len=0, D=128, splits=1):
    # the documented layout: delta and the row exponent offsets, tile
    # states, then per key block a count and NQB indices (twice with full
    # lists), then with splits the parts' fp32 dQ, dK, dV; each piece
    # rounded to 256
    r = lambda x: -(-x // 256) * 256  # noqa: E731
    n = 2 * r(B * H * q_len * 4) + r(Bm * Hm * nq * nk)
    n += r(Bm * Hm * nk * 4) + r(Bm * Hm * nk * nq * 4)
    if full:
        n += r(Bm * Hm * nk * 4) + r(Bm * Hm * nk * nq * 4)
    if splits > 1:
        n += r(splits * B * H * q_len * D * 4)
        n += 2 * r(splits * B * H_kv * kv_len * D * 4)
    return n


@needs_lib
def test_bwd_workspace_bytes():
    bm = _good_bm(q_len=300, kv_len=200, block=128)       # 3 x 2 blocks
    ws = lambda *a, **k: api.fa_bwd_workspace_bytes(*a, **k)  # noqa: E731
    assert ws(2, 4, 2, 300, 200, 128, bm) == _bwd_ws_bytes(2, 4, 300, 3, 2)
    assert ws(2, 4, 2, 300, 200, 64, bm, 3) == _bwd_ws_bytes(
        2, 4, 300, 3, 2, H_kv=2, kv_len=200, D=64, splits=3)
    bm.separate_full_blocks = 0
    assert ws(2, 4, 2, 300, 200, 128, bm) == \
        _bwd_ws_bytes(2, 4, 300, 3, 2, full=False)
    bm = _good_bm(q_len=8192, kv_len=8192, block=128, B=4, H=16)
    assert ws(4, 16, 16, 8192, 8192, 128, bm) == \
        _bwd_ws_bytes(4, 16, 8192, 64, 64, Bm=4, Hm=16)
    assert ws(4, 16, 16, 8192, 8192, 128, bm, 64) == _bwd_ws_bytes(
        4, 16, 8192, 64, 64, Bm=4, Hm=16, H_kv=16, kv_len=8192, splits=64)
    for bad in ((-1, 4, 4, 300, 200, 128, bm), (1, 4, 4, 300, -2, 128, bm),
                (1, 4, 4, 300, 200, 128, bm, 0), (1, 4, 4, 300, 200, 128, bm, 65)):
        with pytest.raises(C.FlexAttnError) as e:
            ws(*bad)
        assert e.value.status == C.FA_ERR_INVALID_VALUE
    assert C.lib().fa_bwd_workspace_bytes(1, 1, 1, 64, 64, 64, None, 1, None) == \
        C.FA_ERR_NULL_POINTER


def _bwd(**over):
    bm = over.pop("bm", _good_bm())
    a = dict(dtype=C.FA_BF16, B=2, H=4, H_kv=2, q_len=256, kv_len=256, D=128,
             q=FAKE, q_stride=(4 * 256 * 128, 256 * 128, 128), k=FAKE,
             k_stride=(2 * 256 * 128, 256 * 128, 128), v=FAKE,
             v_stride=(2 * 256 * 128, 256 * 128, 128), scale=0.088,
             bm=bm, score=C.fa_score_mod(kind=C.FA_SCORE_NONE),
             dq_kv_order=1, num_splits=1, o=FAKE, lse=FAKE, dout=FAKE,
             workspace=FAKE,
             workspace_bytes=_bwd_ws_bytes(2, 4, 256, 2, 2), dq=FAKE, dk=FAKE,
             dv=FAKE, stream=None)
    a.update(over)
    return api.fa_flex_attention_bwd(**a)


@needs_lib
@pytest.mark.parametrize("over,status", [
    (dict(dtype=C.FA_FP32), C.FA_ERR_UNSUPPORTED),
    (dict(dq_kv_order=2), C.FA_ERR_INVALID_VALUE),
    (dict(dq_kv_order=-1), C.FA_ERR_INVALID_VALUE),
    (dict(bm=_bm(**{**{f: getattr(_good_bm(), f) for f, _ in
                       C.fa_block_mask._fields_}, "block_n": 32,
                    "num_kv_blocks": 8})), C.FA_ERR_UNSUPPORTED),
    (dict(workspace_bytes=_bwd_ws_bytes(2, 4, 256, 2, 2) - 1),
     C.FA_ERR_INVALID_VALUE),
    (dict(num_splits=0), C.FA_ERR_INVALID_VALUE),
    (dict(num_splits=65), C.FA_ERR_INVALID_VALUE),
    # split mode needs room for the parts' sums
    (dict(num_splits=2), C.FA_ERR_INVALID_VALUE),
    (dict(num_splits=2, workspace_bytes=_bwd_ws_bytes(
        2, 4, 256, 2, 2, H_kv=2, kv_len=256, splits=2) - 1),
     C.FA_ERR_INVALID_VALUE),
    (dict(workspace=None), C.FA_ERR_NULL_POINTER),
    (dict(workspace=FAKE + 16), C.FA_ERR_UNSUPPORTED),
    (dict(o=None), C.FA_ERR_NULL_POINTER),
    (dict(lse=None), C.FA_ERR_NULL_POINTER),
    (dict(dout=None), C.FA_ERR_NULL_POINTER),
    (dict(dq=None), C.FA_ERR_NULL_POINTER),
    (dict(dk=None), C.FA_ERR_NULL_POINTER),
    (dict(dv=None), C.FA_ERR_NULL_POINTER),
    (dict(dk=FAKE + 8), C.FA_ERR_UNSUPPORTED),
    (dict(lse=FAKE + 4), C.FA_ERR_UNSUPPORTED),
    # the forward's own checks apply
    (dict(D=96), C.FA_ERR_UNSUPPORTED),
    (dict(H_kv=3), C.FA_ERR_INVALID_VALUE),
    (dict(scale=0.0), C.FA_ERR_INVALID_VALUE),
    (dict(bm=_good_bm(B=3)), C.FA_ERR_SHAPE_MISMATCH),
    (dict(q=None), C.FA_ERR_NULL_POINTER),
    (dict(score=C.fa_score_mod(kind=C.FA_SCORE_SOFTCAP, softcap=-1.0)),
     C.FA_ERR_INVALID_VALUE),
])
def test_bwd_refuses(over, status):
    st = _bwd(**over)
    assert st == status, C.lib().fa_last_error()


@needs_lib
def test_bwd_empty_problem_is_a_noop():
    # B = 0, or no keys and no queries: nothing to do, no pointer touched
    assert _bwd(B=0, q=None, k=None, v=None, o=None, lse=None, dout=None,
                workspace=None, workspace_bytes=0, dq=None, dk=None,
                dv=None) == C.FA_OK
    bm = _good_bm(q_len=0, kv_len=0)
    bm.num_q_blocks = bm.num_kv_blocks = 0
    assert _bwd(q_len=0, kv_len=0, bm=bm, q=None, k=None, v=None, o=None,
                lse=None, dout=None, workspace=None, workspace_bytes=0,
                dq=None, dk=None, dv=None) == C.FA_OK
    # no queries but keys: dK and dV must still be given (they are cleared)
    bm = _good_bm(q_len=0)
    bm.num_q_blocks = 0
    assert _bwd(q_len=0, bm=bm, q=None, o=None, lse=None, dout=None,
                dq=None, dk=None) == C.FA_ERR_NULL_POINTER


def _decode(**over):
    a = dict(B=2, H=8, H_kv=2, D=128, q=FAKE, q_stride=(8 * 128, 128),
             k_pages=FAKE, k_stride=(128 * 2 * 128, 2 * 128, 128),
             v_pages=FAKE, v_stride=(128 * 2 * 128, 2 * 128, 128),
             num_pages=10, page_size=128, page_table=FAKE, max_pages=5,
             seq_lens=FAKE, scale=0.088,
             mask=C.fa_mask_mod(kind=C.FA_MASK_CAUSAL),
             score=C.fa_score_mod(kind=C.FA_SCORE_NONE), num_splits=1,
             workspace=None, workspace_bytes=0, o=FAKE, lse=FAKE, stream=None)
    a.update(over)
    return api.fa_flex_attention_decode_paged(**a)


@needs_lib
@pytest.mark.parametrize("over,status", [
    (dict(D=96), C.FA_ERR_UNSUPPORTED),
    (dict(H_kv=3), C.FA_ERR_INVALID_VALUE),
    (dict(H=66, H_kv=2), C.FA_ERR_UNSUPPORTED),          # 33 heads per key head
    (dict(page_size=96), C.FA_ERR_UNSUPPORTED),
    (dict(page_size=32), C.FA_ERR_UNSUPPORTED),
    (dict(num_pages=0), C.FA_ERR_INVALID_VALUE),
    (dict(max_pages=-1), C.FA_ERR_INVALID_VALUE),
    (dict(scale=0.0), C.FA_ERR_INVALID_VALUE),
    (dict(mask=C.fa_mask_mod(kind=C.FA_MASK_SLIDING_WINDOW, window=0)),
     C.FA_ERR_INVALID_VALUE),
    (dict(mask=C.fa_mask_mod(kind=C.FA_MASK_DOCUMENT, doc_id=FAKE,
                             doc_len=639)), C.FA_ERR_SHAPE_MISMATCH),
    (dict(mask=None), C.FA_ERR_NULL_POINTER),
    (dict(score=C.fa_score_mod(kind=C.FA_SCORE_SOFTCAP, softcap=0.0)),
     C.FA_ERR_INVALID_VALUE),
    (dict(num_splits=0), C.FA_ERR_INVALID_VALUE),
    (dict(num_splits=65), C.FA_ERR_INVALID_VALUE),
    (dict(num_splits=4), C.FA_ERR_NULL_POINTER),         # no workspace
    (dict(num_splits=4, workspace=FAKE, workspace_bytes=4 * 16 * 130 * 4 - 1),
     C.FA_ERR_INVALID_VALUE),
    (dict(q=None), C.FA_ERR_NULL_POINTER),
    (dict(o=None), C.FA_ERR_NULL_POINTER),
    (dict(seq_lens=None), C.FA_ERR_NULL_POINTER),
    (dict(page_table=None), C.FA_ERR_NULL_POINTER),
    (dict(k_pages=None), C.FA_ERR_NULL_POINTER),
    (dict(q=FAKE + 8), C.FA_ERR_UNSUPPORTED),
    (dict(k_stride=(128 * 2 * 128, 2 * 128, 100)), C.FA_ERR_UNSUPPORTED),
    (dict(v_stride=(-1, 2 * 128, 128)), C.FA_ERR_UNSUPPORTED),
])
def test_decode_refuses(over, status):
    if "mask" in over and over["mask"] is None:
        a = dict(over)
        a.pop("mask")
        st = C.lib().fa_flex_attention_decode_paged(
            1, 1, 1, 128, FAKE, C.Stride2(128, 128), FAKE,
            C.Stride3(128 * 128, 128, 128), FAKE, C.Stride3(128 * 128, 128, 128),
            1, 128, FAKE, 1, FAKE, 0.1, None, None, 1, None, 0, FAKE, FAKE,
            None)
        assert st == status
        return
    st = _decode(**over)
    assert st == status, C.lib().fa_last_error()


@needs_lib
def test_decode_empty_problem_is_a_noop():
    assert _decode(B=0, q=None, o=None, seq_lens=None, page_table=None,
                   k_pages=None, v_pages=None) == C.FA_OK


def test_auto_bwd_splits():
    # about two dK / dV workgroups per compute unit once one row per unit
    # is short, at most 16 parts and at most one per key block
    assert api.auto_bwd_splits(1, 1, 64, 256) == 8
    assert api.auto_bwd_splits(1, 1, 8, 256) == 8
    assert api.auto_bwd_splits(1, 1, 2, 256) == 2
    assert api.auto_bwd_splits(1, 4, 16, 256) == 8
    assert api.auto_bwd_splits(1, 1, 128, 256) == 4
    assert api.auto_bwd_splits(1, 1, 255, 256) == 3
    assert api.auto_bwd_splits(1, 1, 256, 256) == 1
    assert api.auto_bwd_splits(4, 16, 64, 256) == 1
    assert api.auto_bwd_splits(0, 16, 64, 256) == 1


def test_auto_decode_splits():
    # about sixteen single-wavefront workgroups per compute unit, never more
    # parts than 64-key stages, at most 64
    assert api.auto_decode_splits(16, 8, 32768, 256) == 32
    assert api.auto_decode_splits(1, 1, 32768, 256) == 64
    assert api.auto_decode_splits(1, 1, 128, 256) == 2
    assert api.auto_decode_splits(256, 8, 32768, 256) == 2
    assert api.auto_decode_splits(512, 8, 32768, 256) == 1
    assert api.auto_decode_splits(0, 8, 32768, 256) == 1


def _softmax(**over):
    a = dict(BH=2, q_len=64, kv_len=256, q_offset=0, scores=FAKE,
             score_stride=(64 * 256, 256),
             mask=C.fa_mask_mod(kind=C.FA_MASK_CAUSAL), probs=FAKE,
             stream=None)
    a.update(over)
    return api.fa_masked_softmax(**a)


@needs_lib
@pytest.mark.parametrize("over,status", [
    (dict(kv_len=250), C.FA_ERR_UNSUPPORTED),
    (dict(q_offset=-1), C.FA_ERR_INVALID_VALUE),
    (dict(BH=-1), C.FA_ERR_INVALID_VALUE),
    (dict(scores=None), C.FA_ERR_NULL_POINTER),
    (dict(probs=None), C.FA_ERR_NULL_POINTER),
    (dict(scores=FAKE + 2), C.FA_ERR_UNSUPPORTED),
    (dict(score_stride=(64 * 256, 250)), C.FA_ERR_UNSUPPORTED),
    (dict(mask=C.fa_mask_mod(kind=C.FA_MASK_SLIDING_WINDOW, window=0)),
     C.FA_ERR_INVALID_VALUE),
    (dict(mask=C.fa_mask_mod(kind=C.FA_MASK_DOCUMENT, doc_id=FAKE,
                             doc_len=255)), C.FA_ERR_SHAPE_MISMATCH),
    (dict(q_offset=300, mask=C.fa_mask_mod(kind=C.FA_MASK_DOCUMENT, doc_id=FAKE,
                                           doc_len=300)), C.FA_ERR_SHAPE_MISMATCH),
    (dict(mask=C.fa_mask_mod(kind=C.FA_MASK_DOCUMENT, doc_id=FAKE,
                             doc_len=256, doc_stride=256)), C.FA_ERR_UNSUPPORTED),
    (dict(mask=C.fa_mask_mod(kind=C.FA_MASK_DOCUMENT, doc_id=FAKE + 4,
                             doc_len=256)), C.FA_ERR_UNSUPPORTED),
])
def test_masked_softmax_refuses(over, status):
    st = _softmax(**over)
    assert st == status, C.lib().fa_last_error()


@needs_lib
def test_masked_softmax_empty_is_a_noop():
    assert _softmax(BH=0, scores=None, probs=None) == C.FA_OK
    assert _softmax(kv_len=0, scores=None, probs=None) == C.FA_OK

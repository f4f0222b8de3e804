"""C-ABI checks that need no GPU: the built library exports every function include/ctxsparse.h
declares, and host-side validation rejects bad arguments before any GPU work (the pointers
passed here are never dereferenced because validation fails first)."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ctxsparse.h")


@pytest.fixture(scope="module")
def lib():
    import long_context_sparse_oracle_amd as m

    return m


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\([^;{]*\)\s*;", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_entry_points():
    names = _declared_functions()
    for n in ("topk_index", "sparse_decode_attn", "dense_decode_attn", "topk_index_workspace_size",
              "sparse_decode_attn_workspace_size", "dense_decode_attn_workspace_size",
              "sparse_decode_step", "sparse_decode_step_workspace_size", "key_sketch_build",
              "topk_index_sketch", "topk_index_sketch_workspace_size", "sparse_decode_step_sketch",
              "sparse_decode_step_sketch_workspace_size", "cs_status_str", "cs_version",
              "sparse_decode_attn_noalloc"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    out = subprocess.run(["nm", "-D", "--defined-only", lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = [n for n in declared if n not in exported]
    assert not missing, missing
    # no undeclared C-linkage function leaks out of the library (C++ symbols are mangled "_Z...")
    extra = sorted(n for n in exported if not n.startswith("_Z") and n not in declared)
    assert not extra, extra
    from long_context_sparse_oracle_amd import _lib

    assert sorted(_lib.EXPORTS) == declared
    for n in declared:
        assert hasattr(lib.LIB, n)


def test_status_strings(lib):
    from long_context_sparse_oracle_amd import _lib

    for code, name in _lib.STATUS_NAMES.items():
        assert lib.LIB.cs_status_str(code).decode() == name
    assert lib.LIB.cs_status_str(99).decode() == "CS_ERR_UNKNOWN"
    assert lib.LIB.cs_version() >= 100


# ------------------------------------------------------------------------------ validation
FAKE = 0x10000  # aligned, never dereferenced
INVALID, UNSUPPORTED, WS_SMALL = 1, 2, 3


def _shape(B=2, T=1, Hq=8, Hkv=2, d=128):
    from long_context_sparse_oracle_amd._lib import DecodeShape

    return DecodeShape(B, T, Hq, Hkv, d)


def _kv(layout=0, max_len=1000, page_size=0, max_pages=0, num_pages=0, page_table=0, k=FAKE,
        v=FAKE, seq_lens=FAKE):
    from long_context_sparse_oracle_amd._lib import KVDesc

    return KVDesc(k, v, layout, max_len, page_size, max_pages, num_pages, page_table, seq_lens)


def _topk(L, shape, kv, k_max=10, scale=0.088, ws=FAKE, ws_bytes=1 << 40, q=FAKE, idx=FAKE):
    shp = ctypes.byref(shape) if shape is not None else None
    kvp = ctypes.byref(kv) if kv is not None else None
    return L.topk_index(shp, q, kvp, scale, None, k_max, idx, ws, ws_bytes, None)


def _sparse(L, shape, kv, k_max=10, splits=0, ws=FAKE, ws_bytes=1 << 40, idx=FAKE, out=FAKE):
    return L.sparse_decode_attn(ctypes.byref(shape), FAKE, ctypes.byref(kv), idx, k_max, 0.088,
                                splits, out, FAKE, ws, ws_bytes, None)


def _dense(L, shape, kv, splits=0, ws=FAKE, ws_bytes=1 << 40, out=FAKE):
    return L.dense_decode_attn(ctypes.byref(shape), FAKE, ctypes.byref(kv), 0.088, splits, out,
                               FAKE, ws, ws_bytes, None)


@pytest.mark.parametrize(
    "shape_kw,expect",
    [
        (dict(B=0), INVALID),
        (dict(T=0), INVALID),
        (dict(Hq=0), INVALID),
        (dict(Hkv=0), INVALID),
        (dict(Hq=6, Hkv=4), INVALID),
        (dict(d=96), UNSUPPORTED),
        (dict(d=256), UNSUPPORTED),
        (dict(Hq=64, Hkv=1, T=2), UNSUPPORTED),  # G*T = 128 > 64
    ],
)
def test_bad_shapes(lib, shape_kw, expect):
    L = lib.LIB
    assert _topk(L, _shape(**shape_kw), _kv()) == expect
    assert _sparse(L, _shape(**shape_kw), _kv()) == expect
    assert _dense(L, _shape(**shape_kw), _kv()) == expect


def test_null_shape_and_kv(lib):
    L = lib.LIB
    assert _topk(L, None, _kv()) == INVALID
    assert _topk(L, _shape(), None) == INVALID


@pytest.mark.parametrize(
    "kv_kw,expect",
    [
        (dict(k=0), INVALID),
        (dict(v=0), INVALID),
        (dict(seq_lens=0), INVALID),
        (dict(k=FAKE + 2), INVALID),  # K must be 16-byte aligned
        (dict(max_len=0), INVALID),
        (dict(layout=7), INVALID),
        (dict(layout=1, page_size=16, max_pages=100, num_pages=10, page_table=0), INVALID),
        (dict(layout=1, page_size=8, max_pages=200, num_pages=10, page_table=FAKE), UNSUPPORTED),
        (dict(layout=1, page_size=24, max_pages=100, num_pages=10, page_table=FAKE), UNSUPPORTED),
        (dict(layout=1, page_size=16, max_pages=10, num_pages=10, page_table=FAKE), INVALID),
        (dict(layout=1, page_size=16, max_pages=100, num_pages=0, page_table=FAKE), INVALID),
    ],
)
def test_bad_kv(lib, kv_kw, expect):
    L = lib.LIB
    assert _topk(L, _shape(), _kv(**kv_kw)) == expect
    assert _sparse(L, _shape(), _kv(**kv_kw)) == expect
    assert _dense(L, _shape(), _kv(**kv_kw)) == expect


def test_max_len_below_q_len(lib):
    assert _topk(lib.LIB, _shape(T=4), _kv(max_len=3)) == INVALID


def test_topk_arguments(lib):
    L = lib.LIB
    assert _topk(L, _shape(), _kv(), k_max=0) == INVALID
    assert _topk(L, _shape(), _kv(max_len=50), k_max=51) == INVALID
    assert _topk(L, _shape(), _kv(), scale=float("nan")) == INVALID
    assert _topk(L, _shape(), _kv(), scale=float("inf")) == INVALID
    assert _topk(L, _shape(), _kv(), q=FAKE + 4) == INVALID
    assert _topk(L, _shape(), _kv(), q=0) == INVALID
    assert _topk(L, _shape(), _kv(), idx=0) == INVALID
    assert _topk(L, _shape(), _kv(max_len=262145), k_max=10) == UNSUPPORTED
    need = L.topk_index_workspace_size(ctypes.byref(_shape()), ctypes.byref(_kv()), 10)
    assert need > 0
    assert _topk(L, _shape(), _kv(), ws_bytes=need - 1) == WS_SMALL
    assert _topk(L, _shape(), _kv(), ws=0) == INVALID


def test_attention_arguments(lib):
    L = lib.LIB
    assert _sparse(L, _shape(), _kv(), k_max=0) == INVALID
    assert _sparse(L, _shape(), _kv(), splits=-1) == INVALID
    assert _sparse(L, _shape(), _kv(), idx=0) == INVALID
    assert _sparse(L, _shape(), _kv(), out=0) == INVALID
    assert _dense(L, _shape(), _kv(), splits=-2) == INVALID
    assert _dense(L, _shape(), _kv(), out=0) == INVALID
    need = L.sparse_decode_attn_workspace_size(ctypes.byref(_shape()), 1000, 4)
    assert need > 0
    assert _sparse(L, _shape(), _kv(), k_max=1000, splits=4, ws_bytes=need - 1) == WS_SMALL
    need = L.dense_decode_attn_workspace_size(ctypes.byref(_shape()), ctypes.byref(_kv()), 4)
    assert need > 0
    assert _dense(L, _shape(), _kv(), splits=4, ws_bytes=need - 1) == WS_SMALL


SCRATCH_LIMIT = 5


def _noalloc(L, shape, kv, k_max=10, splits=0, idx=FAKE, out=FAKE, lse=FAKE, q=FAKE, scale=0.088):
    return L.sparse_decode_attn_noalloc(ctypes.byref(shape), q, ctypes.byref(kv), idx, k_max, scale, splits,
                                        out, lse, None)


def test_noalloc_arguments_and_scratch_limit(lib):
    L = lib.LIB
    assert _noalloc(L, _shape(d=96), _kv()) == UNSUPPORTED
    assert _noalloc(L, _shape(), _kv(k=0)) == INVALID
    assert _noalloc(L, _shape(), _kv(), k_max=0) == INVALID
    assert _noalloc(L, _shape(), _kv(), splits=-1) == INVALID
    assert _noalloc(L, _shape(), _kv(), idx=0) == INVALID
    assert _noalloc(L, _shape(), _kv(), out=0) == INVALID
    assert _noalloc(L, _shape(), _kv(), lse=FAKE + 2) == INVALID
    assert _noalloc(L, _shape(), _kv(), q=FAKE + 4) == INVALID
    assert _noalloc(L, _shape(), _kv(), scale=float("nan")) == INVALID
    # a split plan whose partials exceed the fixed 4 MiB scratch is refused before any GPU work:
    # 16 rows x 1000 splits x (128 + 2) floats = 8.3 MB
    limit = 4 << 20
    need = L.sparse_decode_attn_workspace_size(ctypes.byref(_shape()), 1000, 1000)
    assert need > limit
    assert _noalloc(L, _shape(), _kv(), k_max=1000, splits=1000) == SCRATCH_LIMIT
    assert L.cs_status_str(SCRATCH_LIMIT).decode() == "CS_ERR_SCRATCH_LIMIT"


def _step(L, shape, kv, k_max=10, scale=0.088, ws=FAKE, ws_bytes=1 << 40, q=FAKE, idx=None, out=FAKE,
          lse=FAKE):
    return L.sparse_decode_step(ctypes.byref(shape), q, ctypes.byref(kv), scale, None, k_max, idx, out,
                                lse, ws, ws_bytes, None)


def test_step_arguments(lib):
    L = lib.LIB
    assert _step(L, _shape(d=96), _kv()) == UNSUPPORTED
    assert _step(L, _shape(), _kv(k=0)) == INVALID
    assert _step(L, _shape(), _kv(), k_max=0) == INVALID
    assert _step(L, _shape(), _kv(max_len=50), k_max=51) == INVALID
    assert _step(L, _shape(), _kv(), scale=float("nan")) == INVALID
    assert _step(L, _shape(), _kv(), q=FAKE + 4) == INVALID
    assert _step(L, _shape(), _kv(), out=0) == INVALID
    assert _step(L, _shape(), _kv(), lse=0) == INVALID
    assert _step(L, _shape(), _kv(), idx=FAKE + 2) == INVALID
    assert _step(L, _shape(), _kv(max_len=262145), k_max=10) == UNSUPPORTED
    need = L.sparse_decode_step_workspace_size(ctypes.byref(_shape()), ctypes.byref(_kv()), 10)
    assert need >= L.topk_index_workspace_size(ctypes.byref(_shape()), ctypes.byref(_kv()), 10)
    assert _step(L, _shape(), _kv(), ws_bytes=need - 1) == WS_SMALL
    assert L.sparse_decode_step_workspace_size(ctypes.byref(_shape(d=96)), ctypes.byref(_kv()), 10) == 0


def test_workspace_sizes(lib):
    L = lib.LIB
    sz = lambda B, n: L.topk_index_workspace_size(ctypes.byref(_shape(B=B)),  # noqa: E731
                                                 ctypes.byref(_kv(max_len=n)), 10)
    assert sz(1, 1000) < sz(2, 1000) < sz(2, 2000)
    # at least: fp32 scores of every position of every row (or the filtered indexer's candidate
    # slots, half a (position, score) pair per position of every chunk), a 4096-bin histogram and
    # a threshold per row
    rows = 16
    assert sz(2, 1000) >= rows * 1000 * 4 + rows * 4096 * 4 + rows * 4
    assert sz(2, 1000) % 256 == 0
    # a single split needs no workspace; more splits need more
    s = lambda k, S: L.sparse_decode_attn_workspace_size(ctypes.byref(_shape()), k, S)  # noqa: E731
    assert s(100, 1) == 0
    assert 0 < s(100, 2) < s(100, 4)
    assert s(10, 1000) == s(10, 10)  # never more splits than entries
    d = lambda S: L.dense_decode_attn_workspace_size(ctypes.byref(_shape()),  # noqa: E731
                                                    ctypes.byref(_kv(max_len=4096)), S)
    assert d(1) == 0 and 0 < d(2) < d(8)
    # invalid inputs give 0
    assert L.sparse_decode_attn_workspace_size(ctypes.byref(_shape(d=96)), 100, 2) == 0


def _sketch_desc(codes=FAKE, scales=FAKE):
    from long_context_sparse_oracle_amd._lib import KeySketchDesc

    return KeySketchDesc(codes, scales)


def _sketch_topk(L, shape, kv, sk, k_max=10, m=2, scale=0.088, ws=FAKE, ws_bytes=1 << 40, q=FAKE, idx=FAKE):
    skp = ctypes.byref(sk) if sk is not None else None
    return L.topk_index_sketch(ctypes.byref(shape), q, ctypes.byref(kv), skp, scale, None, k_max, m, idx, ws,
                               ws_bytes, None)


def _sketch_step(L, shape, kv, sk, k_max=10, m=2, ws=FAKE, ws_bytes=1 << 40, out=FAKE, lse=FAKE):
    return L.sparse_decode_step_sketch(ctypes.byref(shape), FAKE, ctypes.byref(kv), ctypes.byref(sk), 0.088,
                                       None, k_max, m, None, out, lse, ws, ws_bytes, None)


def test_sketch_arguments(lib):
    L = lib.LIB
    sk = _sketch_desc()
    # the sketch itself
    assert L.key_sketch_build(ctypes.byref(_shape()), ctypes.byref(_kv()), 0, None, None) == INVALID
    assert L.key_sketch_build(ctypes.byref(_shape()), ctypes.byref(_kv()), 0,
                              ctypes.byref(_sketch_desc(codes=0)), None) == INVALID
    assert L.key_sketch_build(ctypes.byref(_shape()), ctypes.byref(_kv()), 0,
                              ctypes.byref(_sketch_desc(codes=FAKE + 8)), None) == INVALID
    assert L.key_sketch_build(ctypes.byref(_shape()), ctypes.byref(_kv()), 0,
                              ctypes.byref(_sketch_desc(scales=FAKE + 2)), None) == INVALID
    assert L.key_sketch_build(ctypes.byref(_shape()), ctypes.byref(_kv()), -1, ctypes.byref(sk), None) == INVALID
    assert L.key_sketch_build(ctypes.byref(_shape(d=96)), ctypes.byref(_kv()), 0, ctypes.byref(sk), None) == UNSUPPORTED
    # the indexer and the step
    assert _sketch_topk(L, _shape(), _kv(), None) == INVALID
    assert _sketch_topk(L, _shape(), _kv(), sk, m=0) == INVALID
    assert _sketch_topk(L, _shape(), _kv(), sk, m=65) == INVALID
    assert _sketch_topk(L, _shape(), _kv(), sk, k_max=0) == INVALID
    assert _sketch_topk(L, _shape(), _kv(), sk, idx=0) == INVALID
    assert _sketch_topk(L, _shape(), _kv(), sk, scale=float("nan")) == INVALID
    assert _sketch_topk(L, _shape(), _kv(max_len=262145), sk) == UNSUPPORTED
    assert _sketch_step(L, _shape(), _kv(), sk, out=0) == INVALID
    assert _sketch_step(L, _shape(), _kv(), sk, m=0) == INVALID
    need = L.topk_index_sketch_workspace_size(ctypes.byref(_shape()), ctypes.byref(_kv()), 10, 2)
    assert need > 0
    assert _sketch_topk(L, _shape(), _kv(), sk, ws_bytes=need - 1) == WS_SMALL
    need_s = L.sparse_decode_step_sketch_workspace_size(ctypes.byref(_shape()), ctypes.byref(_kv()), 10, 2)
    assert need_s > need
    assert _sketch_step(L, _shape(), _kv(), sk, ws_bytes=need_s - 1) == WS_SMALL
    # more candidates need more list room
    assert need < L.topk_index_sketch_workspace_size(ctypes.byref(_shape()), ctypes.byref(_kv()), 10, 8)
    assert L.topk_index_sketch_workspace_size(ctypes.byref(_shape()), ctypes.byref(_kv()), 10, 0) == 0


C_CLIENT = r"""
#include "ctxsparse.h"
#include <stdio.h>
int main(void) {
  cs_decode_shape s = {2, 1, 8, 2, 128};
  cs_kv_desc kv = {0};
  /* a null K pointer: every entry point refuses before any GPU work */
  cs_status st = topk_index(&s, (const void*)0x10000, &kv, 0.088f, NULL, 10, (int*)0x10000,
                            (void*)0x10000, 1u << 20, NULL);
  size_t w = topk_index_workspace_size(&s, &kv, 10);
  printf("%s %s %d %lu\n", cs_status_str(st), cs_status_str(CS_ERR_SCRATCH_LIMIT), cs_version(),
         (unsigned long)w);
  return st == CS_ERR_INVALID_ARG && w == 0 ? 0 : 1;
}
"""


def test_header_is_c99_and_links_from_c(lib, tmp_path):
    """include/ctxsparse.h compiles as strict C99 and a C program links against the library and
    gets the validation statuses through the plain C ABI (no GPU work)."""
    import shutil

    if shutil.which("gcc") is None:
        pytest.skip("gcc not installed")
    src = tmp_path / "client.c"
    src.write_text(C_CLIENT)
    exe = tmp_path / "client"
    libdir = os.path.dirname(lib.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I",
                    os.path.join(ROOT, "include"), str(src), "-L", libdir, "-lctxsparse",
                    f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=dict(os.environ, HIP_VISIBLE_DEVICES=""))
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.split()[:2] == ["CS_ERR_INVALID_ARG", "CS_ERR_SCRATCH_LIMIT"]

"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/locks.h declares, and rejects bad arguments before
launching anything."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "locks.h")

L = pytest.importorskip("kv_cache_page_int4_amd.locks")


def _lib_or_skip():
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("liblocks.so not built")
    return L.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(locks_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ["locks_build_summaries", "locks_score_select", "locks_sparse_attend",
                 "locks_score_pages", "locks_select_pages", "locks_summary_bytes",
                 "locks_workspace_bytes", "locks_score_workspace_bytes",
                 "locks_attend_workspace_bytes", "locks_status_str"]:
        assert want in names


def test_header_compiles_as_c_and_cpp(tmp_path):
    """The public header is valid C and C++ on its own (a stray comment
    terminator or a C++-only construct would break callers)."""
    import shutil
    import subprocess
    hdr = os.path.join(ROOT, "include", "locks.h")
    for cc, lang in (("gcc", "c"), ("g++", "c++")):
        exe = shutil.which(cc)
        if exe is None:
            pytest.skip(f"{cc} not found")
        src = tmp_path / f"use.{'c' if lang == 'c' else 'cpp'}"
        src.write_text(f'#include "{hdr}"\nint main(void) {{ return (int)sizeof(locks_dims); }}\n')
        r = subprocess.run([exe, "-fsyntax-only", "-Wall", "-Werror", str(src)],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_library_exports_every_declared_symbol():
    lib = _lib_or_skip()
    h = ctypes.CDLL(L.LIB_PATH)
    for name in declared_functions():
        assert hasattr(h, name), name


def test_summary_bytes_and_unsupported_dims():
    _lib_or_skip()
    assert L.summary_bytes(L.dims(32, 8)) == 832
    assert L.summary_bytes(L.dims(32, 8, head_dim=64)) == 0
    assert L.summary_bytes(L.dims(32, 8, rank=4)) == 512
    assert L.summary_bytes(L.dims(32, 8, rank=16)) == 1536
    assert L.summary_bytes(L.dims(32, 8, rank=5)) == 0
    assert L.summary_bytes(L.dims(32, 8, rank=32)) == 0
    # GQA groups of 1, 2, 4 and 8 query heads per KV head; others refused
    for hq, hkv in ((8, 8), (16, 8), (32, 8), (64, 8), (4, 1), (8, 1), (1, 1)):
        assert L.summary_bytes(L.dims(hq, hkv)) == 832, (hq, hkv)
    for hq, hkv in ((24, 8), (12, 4), (128, 8), (6, 4), (4, 8), (3, 1)):
        assert L.summary_bytes(L.dims(hq, hkv)) == 0, (hq, hkv)


def test_workspace_sizes_monotone():
    _lib_or_skip()
    d = L.dims(32, 8)
    a = L.score_workspace_bytes(d, 1, 2048, 128)
    b = L.score_workspace_bytes(d, 1, 65536, 128)
    assert 0 < a < b
    assert L.score_workspace_bytes(d, 0, 2048, 128) == 0
    assert L.attend_workspace_bytes(d, 1, 129) > 0
    assert L.attend_workspace_bytes(d, 8, 129) >= L.attend_workspace_bytes(d, 1, 129)


def test_one_workspace_serves_every_call():
    """locks_workspace_bytes covers the scoring part followed by the
    attention part of a sparse or a dense pass, and grows with the group."""
    _lib_or_skip()
    rnd = lambda x: -(-x // 256) * 256  # noqa: E731
    for hq, hkv, batch, pages, budget in ((32, 8, 1, 65536, 128), (32, 8, 16, 16384, 128),
                                         (8, 8, 2, 2048, 128), (64, 8, 1, 2048, 128),
                                         (4, 1, 1, 256, 32), (32, 8, 1, 64, 512)):
        d = L.dims(hq, hkv)
        n = L.workspace_bytes(d, batch, pages, budget)
        sc = L.score_workspace_bytes(d, batch, pages, budget)
        att_sparse = L.attend_workspace_bytes(d, batch, budget + 1)
        att_dense = L.attend_workspace_bytes(d, batch, pages + 1)
        assert n == rnd(sc) + max(att_sparse, att_dense, L.attend_workspace_bytes(
            d, batch, max(budget, pages) + 1)), (hq, hkv)
        assert n >= sc + att_sparse and n >= att_dense
    d = L.dims(32, 8)
    assert L.workspace_bytes(d, 1, 2048, 0) == 0
    assert L.workspace_bytes(d, 0, 2048, 128) == 0
    assert L.workspace_bytes(L.dims(24, 8), 1, 2048, 128) == 0
    # a group of 8 keeps twice the query-head rows of a group of 4
    assert L.workspace_bytes(L.dims(64, 8), 1, 2048, 128) > L.workspace_bytes(d, 1, 2048, 128)


def test_decode_layer_single_workspace_checks():
    """With attend_ws NULL the one workspace must hold both parts and be
    16-byte aligned; nothing is launched when it does not."""
    lib = _lib_or_skip()
    d = L.dims(32, 8)
    P = ctypes.c_void_p
    lay = L.KVLayout(32768, 4096, 128)
    B, MP, BUD = 1, 2048, 128
    sc = L.score_workspace_bytes(d, B, MP, BUD)
    att = L.attend_workspace_bytes(d, B, BUD + 1)
    need = -(-sc // 256) * 256 + att          # what the call checks: both parts
    assert L.workspace_bytes(d, B, MP, BUD) >= need
    full = need

    def call(ws=P(256), ws_bytes=full, att=None, att_bytes=0):
        return lib.locks_decode_layer(ctypes.byref(d), P(256), P(256), P(256), P(256), lay, 4096,
                                      P(256), MP, P(256), B, BUD, 0.0883, P(256), P(256), P(256),
                                      None, ws, ws_bytes, att, att_bytes, None)

    assert call(ws_bytes=sc) == L.ERR_WORKSPACE            # no room for the attention part
    assert call(ws_bytes=full - 1) == L.ERR_WORKSPACE
    assert call(ws=P(264)) == L.ERR_WORKSPACE              # misaligned single workspace
    assert call(ws=None) == L.ERR_WORKSPACE
    # separate workspaces: each checked against its own part
    assert call(ws_bytes=sc - 1, att=P(256), att_bytes=att) == L.ERR_WORKSPACE
    assert call(ws_bytes=sc, att=P(256), att_bytes=att - 1) == L.ERR_WORKSPACE


def test_stage1_chunks_widen_for_large_grids():
    """Stage-1 selection chunks are 2048 pages, or 4096 once 2048-page chunks
    would need more than 512 workgroups (batch x KV heads x chunks): the
    candidate arrays in the score workspace (key + index, 4 bytes each, per
    (sequence, KV head), chunk and slot) follow that plan."""
    _lib_or_skip()
    d = L.dims(32, 8)

    def cand_bytes(batch, pages, budget):
        lse = batch * 32 * pages * 4
        part = batch * 32 * max(-(-pages // 64), -(-pages // 2048)) * 8
        rnd = lambda x: -(-x // 256) * 256
        return L.score_workspace_bytes(d, batch, pages, budget) - rnd(lse) - rnd(part)

    # 1M context, batch 1: 32 chunks x 8 heads = 256 workgroups -> 2048 pages
    assert cand_bytes(1, 65536, 128) == 2 * 1 * 8 * 32 * 128 * 4
    # 256K, batch 16: 8 x 8 x 16 = 1024 workgroups -> 4096-page chunks
    assert cand_bytes(16, 16384, 128) == 2 * 16 * 8 * 4 * 128 * 4
    # budget above the chunk: a chunk keeps all of its pages
    assert cand_bytes(1, 2048, 4000) == 2 * 1 * 8 * 1 * 2048 * 4


def _raw_score(lib, d, **kw):
    args = dict(q=1, summ=1, num_blocks=1, bt=1, max_pages=1, seq=1, batch=1, lse=1, ws=1,
                ws_bytes=1 << 40)
    args.update(kw)
    P = lambda v: ctypes.c_void_p(v) if v else None  # noqa: E731
    return lib.locks_score_pages(ctypes.byref(d), P(args["q"] and 256), P(args["summ"] and 256),
                                 args["num_blocks"], P(args["bt"] and 256), args["max_pages"],
                                 P(args["seq"] and 256), args["batch"], P(args["lse"] and 256),
                                 P(args["ws"] and 256), args["ws_bytes"], None)


def test_validation_errors_launch_nothing():
    lib = _lib_or_skip()
    d = L.dims(32, 8)
    assert _raw_score(lib, d, q=0) == L.ERR_NULL
    assert _raw_score(lib, d, lse=0) == L.ERR_NULL
    assert _raw_score(lib, d, batch=0) == L.ERR_SHAPE
    assert _raw_score(lib, d, max_pages=0) == L.ERR_SHAPE
    assert _raw_score(lib, d, num_blocks=0) == L.ERR_SHAPE
    assert _raw_score(lib, d, ws=0) == L.ERR_WORKSPACE
    assert _raw_score(lib, d, ws_bytes=16) == L.ERR_WORKSPACE
    assert _raw_score(lib, L.dims(32, 8, page_size=32)) == L.ERR_UNSUPPORTED
    # the pending-newest-page flag is 0 or 1
    bad = L.dims(32, 8)
    bad.newest_page_pending = 2
    assert _raw_score(lib, bad) == L.ERR_SHAPE
    assert L.summary_bytes(bad) == 0 and L.workspace_bytes(bad, 1, 64, 8) == 0
    assert L.dims(32, 8, newest_page_pending=True).newest_page_pending == 1
    assert lib.locks_score_pages(None, None, None, 0, None, 0, None, 0, None, None, 0, None) == L.ERR_NULL
    # misaligned q
    P = ctypes.c_void_p
    assert lib.locks_score_pages(ctypes.byref(d), P(258), P(256), 1, P(256), 1, P(256), 1, P(256),
                                 P(256), 1 << 40, None) == L.ERR_SHAPE


def test_misaligned_buffers_are_refused_before_any_launch():
    """16 bytes for q / K / V / summaries and workspaces, 4 bytes for int32
    and fp32 arrays and the bf16 output; the fake pointers never reach a
    kernel because validation fails first."""
    lib = _lib_or_skip()
    d = L.dims(32, 8)
    P = ctypes.c_void_p
    A, W = P(256), 1 << 40

    def score(q=A, summ=A, bt=A, seq=A, lse=A, ws=A):
        return lib.locks_score_pages(ctypes.byref(d), q, summ, 4, bt, 4, seq, 1, lse, ws, W, None)

    assert score(summ=P(264)) == L.ERR_SHAPE
    assert score(bt=P(258)) == L.ERR_SHAPE
    assert score(seq=P(258)) == L.ERR_SHAPE
    assert score(lse=P(258)) == L.ERR_SHAPE
    assert score(ws=P(264)) == L.ERR_WORKSPACE

    def select(lse=A, seq=A, sel=A, cnt=A, ws=A):
        return lib.locks_select_pages(ctypes.byref(d), lse, 16, seq, 1, 4, sel, cnt, ws, W, None)

    assert select(lse=P(258)) == L.ERR_SHAPE
    assert select(sel=P(258)) == L.ERR_SHAPE
    assert select(cnt=P(258)) == L.ERR_SHAPE
    assert select(ws=P(264)) == L.ERR_WORKSPACE

    def score_select(sel=A, cnt=A, lse=None, ws=A):
        return lib.locks_score_select(ctypes.byref(d), A, A, 4, A, 4, A, 1, 4, sel, cnt, lse, ws,
                                      W, None)

    assert score_select(sel=P(258)) == L.ERR_SHAPE
    assert score_select(lse=P(258)) == L.ERR_SHAPE
    assert score_select(ws=P(264)) == L.ERR_WORKSPACE

    lay = L.KVLayout(16384, 2048, 128)

    def attend(q=A, k=A, v=A, sel=A, cnt=A, out=A, olse=None, ws=A):
        return lib.locks_sparse_attend(ctypes.byref(d), q, k, v, lay, 4, A, 4, A, 1, sel, cnt, 4,
                                       0.1, out, olse, ws, W, None)

    assert attend(v=P(264)) == L.ERR_SHAPE
    assert attend(out=P(258)) == L.ERR_SHAPE
    assert attend(olse=P(258)) == L.ERR_SHAPE
    assert attend(sel=P(258)) == L.ERR_SHAPE
    assert attend(ws=P(264)) == L.ERR_WORKSPACE

    def layer(out=A, ws=A, att=None, att_bytes=0):
        return lib.locks_decode_layer(ctypes.byref(d), A, A, A, A, lay, 4, A, 4, A, 1, 4, 0.1, A,
                                      A, out, None, ws, W, att, att_bytes, None)

    assert layer(out=P(258)) == L.ERR_SHAPE
    assert layer(ws=P(264), att=A, att_bytes=W) == L.ERR_WORKSPACE
    assert layer(att=P(264), att_bytes=W) == L.ERR_WORKSPACE

    assert lib.locks_exact_page_lse(ctypes.byref(d), A, A, lay, 4, A, 4, A, 1, 0.1, P(258),
                                    None) == L.ERR_SHAPE
    assert lib.locks_finalize_pages(ctypes.byref(d), A, lay, 4, A, 4, A, 1, P(264), 1, 0, 0,
                                    None) == L.ERR_SHAPE
    assert lib.locks_build_summaries(ctypes.byref(d), A, lay, P(258), 3, 4, A, None,
                                     None) == L.ERR_SHAPE


def test_attend_and_build_validation():
    lib = _lib_or_skip()
    d = L.dims(4, 1)
    P = ctypes.c_void_p
    lay = L.KVLayout(2048, 2048, 128)
    # sel given without sel_count
    st = lib.locks_sparse_attend(ctypes.byref(d), P(256), P(256), P(256), lay, 4, P(256), 4,
                                 P(256), 1, P(256), None, 4, 0.1, P(256), None, P(256), 1 << 40, None)
    assert st == L.ERR_NULL
    # non-positive softmax scale
    st = lib.locks_sparse_attend(ctypes.byref(d), P(256), P(256), P(256), lay, 4, P(256), 4,
                                 P(256), 1, None, None, 0, -1.0, P(256), None, P(256), 1 << 40, None)
    assert st == L.ERR_SHAPE
    # token stride shorter than a row
    bad = L.KVLayout(2048, 2048, 64)
    st = lib.locks_sparse_attend(ctypes.byref(d), P(256), P(256), P(256), bad, 4, P(256), 4,
                                 P(256), 1, None, None, 0, 0.1, P(256), None, P(256), 1 << 40, None)
    assert st == L.ERR_SHAPE
    # too small workspace
    st = lib.locks_sparse_attend(ctypes.byref(d), P(256), P(256), P(256), lay, 4, P(256), 4,
                                 P(256), 1, None, None, 0, 0.1, P(256), None, P(256), 8, None)
    assert st == L.ERR_WORKSPACE
    # build: empty list is a no-op, null summaries rejected
    assert lib.locks_build_summaries(ctypes.byref(d), P(256), lay, P(256), 0, 4, None, None, None) == L.OK
    assert lib.locks_build_summaries(ctypes.byref(d), P(256), lay, P(256), 3, 4, None, None, None) == L.ERR_NULL
    assert lib.locks_build_summaries(ctypes.byref(d), P(256), lay, P(256), -1, 4, P(256), None, None) == L.ERR_SHAPE
    # select: zero budget rejected
    st = lib.locks_select_pages(ctypes.byref(d), P(256), 16, P(256), 1, 0, P(256), P(256), P(256),
                                1 << 40, None)
    assert st == L.ERR_SHAPE


def test_status_strings():
    _lib_or_skip()
    for st in (L.OK, L.ERR_NULL, L.ERR_SHAPE, L.ERR_UNSUPPORTED, L.ERR_WORKSPACE, L.ERR_LAUNCH):
        assert len(L.status_str(st)) > 0
    # the unsupported-shape message names every accepted rank and group
    msg = L.status_str(L.ERR_UNSUPPORTED)
    assert "4/8/16" in msg and "{1,2,4,8}" in msg
    assert L.status_str(-99) == "unknown status"


def test_exact_page_lse_validation():
    """Bad arguments of the exact scorer are refused on the host (nothing is
    launched, so these run without a GPU)."""
    lib = _lib_or_skip()
    d = L.dims(32, 8)
    P = ctypes.c_void_p
    lay = L.KVLayout(16384, 2048, 128)
    ok = dict(q=P(256), k=P(256), lay=lay, nb=4, bt=P(256), mp=4, seq=P(256), batch=1,
              scale=0.1, lse=P(256))

    def call(**kw):
        a = dict(ok, **kw)
        return lib.locks_exact_page_lse(ctypes.byref(a.pop("d", d)), a["q"], a["k"], a["lay"],
                                        a["nb"], a["bt"], a["mp"], a["seq"], a["batch"],
                                        a["scale"], a["lse"], None)

    assert call(q=None) == L.ERR_NULL
    assert call(lse=None) == L.ERR_NULL
    assert call(batch=0) == L.ERR_SHAPE
    assert call(nb=0) == L.ERR_SHAPE
    assert call(scale=-1.0) == L.ERR_SHAPE
    assert call(scale=float("nan")) == L.ERR_SHAPE
    assert call(lay=L.KVLayout(16384, 2048, 64)) == L.ERR_SHAPE
    assert call(k=P(264)) == L.ERR_SHAPE
    assert call(d=L.dims(32, 8, rank=6)) == L.ERR_UNSUPPORTED


def test_table_count_validation():
    """n_tables must be a positive divisor of the KV-head count; the check
    comes before anything is launched."""
    lib = _lib_or_skip()
    d = L.dims(32, 8)
    P = ctypes.c_void_p
    lay = L.KVLayout(32768, 4096, 128)
    for bad in (0, -1, 3, 16):
        st = lib.locks_select_pages_tables(ctypes.byref(d), P(256), 16, P(256), 1, 4, bad, P(256),
                                           P(256), P(256), 1 << 40, None)
        assert st == L.ERR_SHAPE, bad
        st = lib.locks_sparse_attend_tables(ctypes.byref(d), P(256), P(256), P(256), lay, 4,
                                            P(256), 4, P(256), 1, P(256), P(256), 4, bad, 0.1,
                                            P(256), None, P(256), 1 << 40, None)
        assert st == L.ERR_SHAPE, bad
        st = lib.locks_decode_layer_tables(ctypes.byref(d), P(256), P(256), P(256), P(256), lay, 4,
                                           P(256), 4, P(256), 1, 4, bad, 0.1, P(256), P(256),
                                           P(256), None, P(256), 1 << 40, P(256), 1 << 40, None)
        assert st == L.ERR_SHAPE, bad
    # a valid count still meets the other checks (workspace too small here)
    st = lib.locks_select_pages_tables(ctypes.byref(d), P(256), 16, P(256), 1, 4, 2, P(256),
                                       P(256), P(256), 8, None)
    assert st == L.ERR_WORKSPACE
    assert lib.locks_select_pages_tables(None, P(256), 16, P(256), 1, 4, 1, P(256), P(256),
                                         P(256), 1 << 40, None) == L.ERR_NULL


def test_shared_basis_validation():
    lib = _lib_or_skip()
    d = L.dims(32, 8)
    P = ctypes.c_void_p
    lay = L.KVLayout(32768, 4096, 128)
    need = lib.locks_shared_basis_workspace_bytes(ctypes.byref(d), 1000)
    assert need > 0 and lib.locks_shared_basis_workspace_bytes(ctypes.byref(d), 0) == 0
    assert lib.locks_shared_basis_workspace_bytes(ctypes.byref(L.dims(32, 8, rank=12)), 10) == 0
    call = lambda **kw: lib.locks_shared_basis(
        ctypes.byref(kw.get("d", d)), kw.get("k", P(256)), kw.get("lay", lay), kw.get("ids", P(256)),
        kw.get("n", 1000), 4096, kw.get("basis", P(256)), None, kw.get("ws", P(256)),
        kw.get("wsb", need), None)
    assert call(n=0) == L.ERR_SHAPE
    assert call(basis=None) == L.ERR_NULL
    assert call(k=None) == L.ERR_NULL
    assert call(wsb=need - 1) == L.ERR_WORKSPACE
    assert call(ws=None) == L.ERR_WORKSPACE
    assert call(lay=L.KVLayout(32768, 4096, 64)) == L.ERR_SHAPE
    assert call(d=L.dims(32, 8, head_dim=64)) == L.ERR_UNSUPPORTED
    b = lambda n, basis=P(256), summ=P(256): lib.locks_build_summaries_basis(
        ctypes.byref(d), P(256), lay, P(256), n, 4096, basis, summ, None)
    assert b(0) == L.OK
    assert b(-1) == L.ERR_SHAPE
    assert b(3, basis=None) == L.ERR_NULL
    assert b(3, summ=None) == L.ERR_NULL
    assert b(3, summ=P(264)) == L.ERR_SHAPE

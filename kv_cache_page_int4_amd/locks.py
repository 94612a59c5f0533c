"""Python binding of liblocks.so (argument marshalling only).

Every function forwards to the C entry point of the same name in
include/locks.h.  Tensors supply device pointers and the current torch stream;
no computation happens here.  If the shared library is missing the import of
this module still works but every call raises, so nothing can silently fall
back to a host path.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblocks.so")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_LAUNCH = 0, -1, -2, -3, -4, -5
SUMMARY_BYTES = 832   # record bytes at rank 8; summary_bytes(d) gives any rank


class LocksError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: status {status} ({status_str(status)})")


class Dims(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("newest_page_pending", ctypes.c_int32)]


class KVLayout(ctypes.Structure):
    _fields_ = [("block_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64),
                ("token_stride", ctypes.c_int64)]


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_DP = ctypes.POINTER(Dims)

_SIGS = {
    "locks_summary_bytes": (_SZ, [_DP]),
    "locks_workspace_bytes": (_SZ, [_DP, _I32, _I32, _I32]),
    "locks_score_workspace_bytes": (_SZ, [_DP, _I32, _I32, _I32]),
    "locks_attend_workspace_bytes": (_SZ, [_DP, _I32, _I32]),
    "locks_build_summaries": (_I32, [_DP, _P, KVLayout, _P, _I32, _I32, _P, _P, _P]),
    "locks_score_pages": (_I32, [_DP, _P, _P, _I32, _P, _I32, _P, _I32, _P, _P, _SZ, _P]),
    "locks_select_pages": (_I32, [_DP, _P, _I32, _P, _I32, _I32, _P, _P, _P, _SZ, _P]),
    "locks_score_select": (_I32, [_DP, _P, _P, _I32, _P, _I32, _P, _I32, _I32, _P, _P, _P, _P,
                                  _SZ, _P]),
    "locks_sparse_attend": (_I32, [_DP, _P, _P, _P, KVLayout, _I32, _P, _I32, _P, _I32, _P, _P,
                                   _I32, ctypes.c_float, _P, _P, _P, _SZ, _P]),
    "locks_decode_layer": (_I32, [_DP, _P, _P, _P, _P, KVLayout, _I32, _P, _I32, _P, _I32, _I32,
                                  ctypes.c_float, _P, _P, _P, _P, _P, _SZ, _P, _SZ, _P]),
    "locks_decode_layer_noalloc_bytes": (_SZ, [_DP, _I32, _I32, _I32]),
    "locks_decode_layer_noalloc": (_I32, [_DP, _P, _P, _P, _P, KVLayout, _I32, _P, _I32, _P, _I32,
                                          _I32, ctypes.c_float, _P, _P, _P, _P, _P]),
    "locks_finalize_pages": (_I32, [_DP, _P, KVLayout, _I32, _P, _I32, _P, _I32, _P, _I32,
                                    ctypes.c_int64, ctypes.c_int64, _P]),
    "locks_exact_page_lse": (_I32, [_DP, _P, _P, KVLayout, _I32, _P, _I32, _P, _I32,
                                    ctypes.c_float, _P, _P]),
    "locks_select_pages_tables": (_I32, [_DP, _P, _I32, _P, _I32, _I32, _I32, _P, _P, _P, _SZ,
                                         _P]),
    "locks_sparse_attend_tables": (_I32, [_DP, _P, _P, _P, KVLayout, _I32, _P, _I32, _P, _I32, _P,
                                          _P, _I32, _I32, ctypes.c_float, _P, _P, _P, _SZ, _P]),
    "locks_decode_layer_tables": (_I32, [_DP, _P, _P, _P, _P, KVLayout, _I32, _P, _I32, _P, _I32,
                                         _I32, _I32, ctypes.c_float, _P, _P, _P, _P, _P, _SZ, _P,
                                         _SZ, _P]),
    "locks_shared_basis_workspace_bytes": (_SZ, [_DP, _I32]),
    "locks_shared_basis": (_I32, [_DP, _P, KVLayout, _P, _I32, _I32, _P, _P, _P, _SZ, _P]),
    "locks_build_summaries_basis": (_I32, [_DP, _P, KVLayout, _P, _I32, _I32, _P, _P, _P]),
    "locks_status_str": (ctypes.c_char_p, [_I32]),
}


def lib():
    """Load liblocks.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype, f.argtypes = res, args
        _lib = h
    return _lib


def status_str(status: int) -> str:
    return lib().locks_status_str(int(status)).decode()


def _check(fn, st):
    if st != OK:
        raise LocksError(fn, st)


def dims(num_q_heads, num_kv_heads, head_dim=128, page_size=16, rank=8,
         newest_page_pending=False) -> Dims:
    """newest_page_pending: the page holding each sequence's newest token is
    not summarized yet (attended in full instead), as in a decode step whose
    completed pages are summarized after it."""
    return Dims(num_q_heads, num_kv_heads, head_dim, page_size, rank,
                int(bool(newest_page_pending)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype, numel=None):
    """Type checks; with numel, also that the tensor is dense and holds at
    least the numel elements the library will read or write through its
    pointer (the C ABI itself cannot see buffer sizes)."""
    if t is None:
        return
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None:
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.numel() < numel:
            raise ValueError(f"{name} holds {t.numel()} elements; the call needs {numel}")


def _on_device(**tensors):
    """Every given tensor lives on the GPU (checked after the size checks)."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")


def _rec_bytes(d: Dims) -> int:
    """Record bytes at rank d.rank (84 r + 130 bytes of fields, padded to 64)."""
    return (84 * d.rank + 130 + 63) // 64 * 64


def _kv_heads(d: Dims, cache, name):
    if cache.dim() >= 3 and cache.shape[-3] != d.num_kv_heads:
        raise ValueError(f"{name} has {cache.shape[-3]} KV heads, dims say {d.num_kv_heads}")


def kv_layout(cache: torch.Tensor) -> KVLayout:
    """Strides of a [num_blocks, num_kv_heads, page, head_dim] cache view."""
    if cache.dim() != 4 or cache.stride(3) != 1:
        raise ValueError("cache must be a [blocks, kv_heads, page, dim] view with unit dim stride")
    return KVLayout(cache.stride(0), cache.stride(1), cache.stride(2))


def summary_bytes(d: Dims) -> int:
    return lib().locks_summary_bytes(ctypes.byref(d))


def workspace_bytes(d: Dims, batch, max_pages, budget_pages) -> int:
    """One workspace size that serves every decode-path call with these sizes
    (and decode_layer with attend_ws=None)."""
    return lib().locks_workspace_bytes(ctypes.byref(d), batch, max_pages, budget_pages)


def workspace(d: Dims, batch, max_pages, budget_pages, device="cuda") -> torch.Tensor:
    """A workspace of workspace_bytes(...) bytes."""
    n = workspace_bytes(d, batch, max_pages, budget_pages)
    if n == 0:
        raise ValueError("unsupported dims or sizes for a workspace")
    return torch.empty(n, dtype=torch.uint8, device=device)


def score_workspace_bytes(d: Dims, batch, max_pages, budget_pages=0) -> int:
    return lib().locks_score_workspace_bytes(ctypes.byref(d), batch, max_pages, budget_pages)


def attend_workspace_bytes(d: Dims, batch, max_attended_pages) -> int:
    return lib().locks_attend_workspace_bytes(ctypes.byref(d), batch, max_attended_pages)


def attend_workspace(d: Dims, batch, max_attended_pages, device="cuda") -> torch.Tensor:
    """An attend workspace of the required size."""
    return torch.empty(attend_workspace_bytes(d, batch, max_attended_pages), dtype=torch.uint8,
                       device=device)


def build_summaries(d: Dims, k_cache, block_ids, summaries, raw_debug=None, stream=None):
    """k_cache: bf16 [num_blocks, Hkv, 16, 128] (one layer); block_ids: int32
    [n]; summaries: uint8 [Hkv, num_blocks, summary_bytes(d)]; raw_debug: fp32
    [n, Hkv, 128 + 144 * rank] (1280 at rank 8)."""
    nb, hkv, n = k_cache.shape[0], d.num_kv_heads, block_ids.numel()
    _need(k_cache, "k_cache", torch.bfloat16)
    _kv_heads(d, k_cache, "k_cache")
    _need(block_ids, "block_ids", torch.int32, numel=n)
    _need(summaries, "summaries", torch.uint8, numel=hkv * nb * _rec_bytes(d))
    _need(raw_debug, "raw_debug", torch.float32, numel=n * hkv * (128 + 144 * d.rank))
    _on_device(k_cache=k_cache, block_ids=block_ids, summaries=summaries, raw_debug=raw_debug)
    st = lib().locks_build_summaries(ctypes.byref(d), _ptr(k_cache), kv_layout(k_cache),
                                     _ptr(block_ids), block_ids.numel(), k_cache.shape[0],
                                     _ptr(summaries), _ptr(raw_debug), _stream(stream))
    _check("locks_build_summaries", st)


def score_pages(d: Dims, q, summaries, num_blocks, block_table, seq_lens, page_lse, workspace,
                stream=None):
    B, P, hq = block_table.shape[0], block_table.shape[1], d.num_q_heads
    _need(q, "q", torch.bfloat16, numel=B * hq * d.head_dim)
    _need(summaries, "summaries", torch.uint8, numel=d.num_kv_heads * num_blocks * _rec_bytes(d))
    _need(block_table, "block_table", torch.int32, numel=B * P)
    _need(seq_lens, "seq_lens", torch.int32, numel=B)
    _need(page_lse, "page_lse", torch.float32, numel=B * hq * P)
    _on_device(q=q, summaries=summaries, block_table=block_table, seq_lens=seq_lens,
               page_lse=page_lse, workspace=workspace)
    st = lib().locks_score_pages(ctypes.byref(d), _ptr(q), _ptr(summaries), num_blocks,
                                 _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
                                 block_table.shape[0], _ptr(page_lse), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream))
    _check("locks_score_pages", st)


def select_pages(d: Dims, page_lse, seq_lens, budget_pages, sel, sel_count, workspace, stream=None,
                 n_tables=None):
    """n_tables=None: one table per KV head (sel [batch, Hkv, budget]); else
    n_tables tables per sequence (sel [batch, n_tables, budget])."""
    B, P = page_lse.shape[0], page_lse.shape[-1]
    ntab = d.num_kv_heads if n_tables is None else int(n_tables)
    _need(page_lse, "page_lse", torch.float32, numel=B * d.num_q_heads * P)
    _need(seq_lens, "seq_lens", torch.int32, numel=B)
    _need(sel, "sel", torch.int32, numel=B * ntab * budget_pages)
    _need(sel_count, "sel_count", torch.int32, numel=B * ntab)
    _on_device(page_lse=page_lse, seq_lens=seq_lens, sel=sel, sel_count=sel_count,
               workspace=workspace)
    args = [ctypes.byref(d), _ptr(page_lse), page_lse.shape[-1], _ptr(seq_lens),
            page_lse.shape[0], budget_pages]
    rest = [_ptr(sel), _ptr(sel_count), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream)]
    if n_tables is None:
        _check("locks_select_pages", lib().locks_select_pages(*args, *rest))
    else:
        _check("locks_select_pages_tables",
               lib().locks_select_pages_tables(*args, int(n_tables), *rest))


def score_select(d: Dims, q, summaries, num_blocks, block_table, seq_lens, budget_pages, sel,
                 sel_count, workspace, page_lse=None, stream=None):
    B, P, hq, hkv = block_table.shape[0], block_table.shape[1], d.num_q_heads, d.num_kv_heads
    _need(q, "q", torch.bfloat16, numel=B * hq * d.head_dim)
    _need(summaries, "summaries", torch.uint8, numel=hkv * num_blocks * _rec_bytes(d))
    _need(block_table, "block_table", torch.int32, numel=B * P)
    _need(seq_lens, "seq_lens", torch.int32, numel=B)
    _need(sel, "sel", torch.int32, numel=B * hkv * budget_pages)
    _need(sel_count, "sel_count", torch.int32, numel=B * hkv)
    _need(page_lse, "page_lse", torch.float32, numel=B * hq * P)
    _on_device(q=q, summaries=summaries, block_table=block_table, seq_lens=seq_lens, sel=sel,
               sel_count=sel_count, page_lse=page_lse, workspace=workspace)
    st = lib().locks_score_select(ctypes.byref(d), _ptr(q), _ptr(summaries), num_blocks,
                                  _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
                                  block_table.shape[0], budget_pages, _ptr(sel), _ptr(sel_count),
                                  _ptr(page_lse), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream))
    _check("locks_score_select", st)


def sparse_attend(d: Dims, q, k_cache, v_cache, block_table, seq_lens, sel, sel_count,
                  budget_pages, out, workspace, out_lse=None, softmax_scale=None, stream=None,
                  n_tables=None):
    """sel=None attends every summarized page (dense attention); n_tables as
    for select_pages."""
    B, P, hq = block_table.shape[0], block_table.shape[1], d.num_q_heads
    ntab = d.num_kv_heads if n_tables is None else int(n_tables)
    _need(q, "q", torch.bfloat16, numel=B * hq * d.head_dim)
    _need(k_cache, "k_cache", torch.bfloat16)
    _need(v_cache, "v_cache", torch.bfloat16)
    _kv_heads(d, k_cache, "k_cache")
    _kv_heads(d, v_cache, "v_cache")
    _need(block_table, "block_table", torch.int32, numel=B * P)
    _need(seq_lens, "seq_lens", torch.int32, numel=B)
    if sel is not None:
        _need(sel, "sel", torch.int32, numel=B * ntab * budget_pages)
        _need(sel_count, "sel_count", torch.int32, numel=B * ntab)
    _need(out, "out", torch.bfloat16, numel=B * hq * d.head_dim)
    _need(out_lse, "out_lse", torch.float32, numel=B * hq)
    _on_device(q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table, seq_lens=seq_lens,
               sel=sel, sel_count=sel_count, out=out, out_lse=out_lse, workspace=workspace)
    lay = kv_layout(k_cache)
    lv = kv_layout(v_cache)
    if (lay.block_stride, lay.head_stride, lay.token_stride) != (
            lv.block_stride, lv.head_stride, lv.token_stride):
        raise ValueError("k_cache and v_cache must share one layout")
    if softmax_scale is None:
        softmax_scale = 1.0 / (d.head_dim ** 0.5)
    head = [ctypes.byref(d), _ptr(q), _ptr(k_cache), _ptr(v_cache), lay, k_cache.shape[0],
            _ptr(block_table), block_table.shape[1], _ptr(seq_lens), block_table.shape[0],
            _ptr(sel), _ptr(sel_count), budget_pages if sel is not None else 0]
    tail = [float(softmax_scale), _ptr(out), _ptr(out_lse), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream)]
    if n_tables is None:
        _check("locks_sparse_attend", lib().locks_sparse_attend(*head, *tail))
    else:
        _check("locks_sparse_attend_tables",
               lib().locks_sparse_attend_tables(*head, int(n_tables), *tail))


def exact_page_lse(d: Dims, q, k_cache, block_table, seq_lens, page_lse, softmax_scale=None,
                   stream=None):
    """Exact page LSE from the keys (the read-every-key comparator); page_lse:
    fp32 [batch, Hq, max_pages], the layout of score_pages' output."""
    B, P, hq = block_table.shape[0], block_table.shape[1], d.num_q_heads
    _need(q, "q", torch.bfloat16, numel=B * hq * d.head_dim)
    _need(k_cache, "k_cache", torch.bfloat16)
    _kv_heads(d, k_cache, "k_cache")
    _need(block_table, "block_table", torch.int32, numel=B * P)
    _need(seq_lens, "seq_lens", torch.int32, numel=B)
    _need(page_lse, "page_lse", torch.float32, numel=B * hq * P)
    _on_device(q=q, k_cache=k_cache, block_table=block_table, seq_lens=seq_lens, page_lse=page_lse)
    if softmax_scale is None:
        softmax_scale = 1.0 / (d.head_dim ** 0.5)
    st = lib().locks_exact_page_lse(ctypes.byref(d), _ptr(q), _ptr(k_cache), kv_layout(k_cache),
                                    k_cache.shape[0], _ptr(block_table), block_table.shape[1],
                                    _ptr(seq_lens), block_table.shape[0], float(softmax_scale),
                                    _ptr(page_lse), _stream(stream))
    _check("locks_exact_page_lse", st)


def finalize_pages(d: Dims, k_cache, block_table, seq_lens, summaries, stream=None):
    """Summarize each sequence's last page when its length is a positive
    multiple of 16 (decided on the device; graph-capturable).  k_cache:
    [blocks, Hkv, 16, 128] for one layer or [layers, blocks, Hkv, 16, 128] for
    all layers at once; summaries: [Hkv, blocks, summary_bytes(d)] or
    [layers, Hkv, blocks, summary_bytes(d)] to match."""
    B, P = block_table.shape[0], block_table.shape[1]
    _need(k_cache, "k_cache", torch.bfloat16)
    _kv_heads(d, k_cache, "k_cache")
    _need(block_table, "block_table", torch.int32, numel=B * P)
    _need(seq_lens, "seq_lens", torch.int32, numel=B)
    _on_device(k_cache=k_cache, block_table=block_table, seq_lens=seq_lens, summaries=summaries)
    if k_cache.dim() == 5:
        if summaries.dim() != 4 or summaries.shape[0] != k_cache.shape[0]:
            raise ValueError("summaries must be [layers, Hkv, blocks, record] for a 5-d k_cache")
        n_layers, ks, ss = k_cache.shape[0], k_cache.stride(0), summaries.stride(0)
        k0, s0 = k_cache[0], summaries[0]
    else:
        n_layers, ks, ss, k0, s0 = 1, 0, 0, k_cache, summaries
    per_layer = d.num_kv_heads * k0.shape[0] * _rec_bytes(d)
    _need(s0, "summaries (one layer)", torch.uint8, numel=per_layer)
    if n_layers > 1 and ss < per_layer:
        raise ValueError("summaries layers overlap")
    st = lib().locks_finalize_pages(ctypes.byref(d), _ptr(k0), kv_layout(k0), k0.shape[0],
                                    _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
                                    block_table.shape[0], _ptr(s0), n_layers, ks, ss,
                                    _stream(stream))
    _check("locks_finalize_pages", st)


def decode_layer(d: Dims, q, summaries, k_cache, v_cache, block_table, seq_lens, budget_pages,
                 sel, sel_count, out, score_ws, attend_ws=None, out_lse=None, softmax_scale=None,
                 stream=None, n_tables=None):
    """score_select followed by sparse_attend in one call (identical outputs);
    n_tables as for select_pages.  attend_ws=None: score_ws is one workspace of
    workspace_bytes(...) bytes holding both parts.  softmax_scale (default
    1/sqrt(d)) is the logit scale of both the page estimate and the attention."""
    B, P, hq = block_table.shape[0], block_table.shape[1], d.num_q_heads
    ntab = d.num_kv_heads if n_tables is None else int(n_tables)
    _need(q, "q", torch.bfloat16, numel=B * hq * d.head_dim)
    _need(summaries, "summaries", torch.uint8,
          numel=d.num_kv_heads * k_cache.shape[0] * _rec_bytes(d))
    _need(k_cache, "k_cache", torch.bfloat16)
    _need(v_cache, "v_cache", torch.bfloat16)
    _kv_heads(d, k_cache, "k_cache")
    _kv_heads(d, v_cache, "v_cache")
    _need(block_table, "block_table", torch.int32, numel=B * P)
    _need(seq_lens, "seq_lens", torch.int32, numel=B)
    _need(sel, "sel", torch.int32, numel=B * ntab * budget_pages)
    _need(sel_count, "sel_count", torch.int32, numel=B * ntab)
    _need(out, "out", torch.bfloat16, numel=B * hq * d.head_dim)
    _need(out_lse, "out_lse", torch.float32, numel=B * hq)
    _on_device(q=q, summaries=summaries, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
               seq_lens=seq_lens, sel=sel, sel_count=sel_count, out=out, out_lse=out_lse,
               score_ws=score_ws, attend_ws=attend_ws)
    lay = kv_layout(k_cache)
    lv = kv_layout(v_cache)
    if (lay.block_stride, lay.head_stride, lay.token_stride) != (
            lv.block_stride, lv.head_stride, lv.token_stride):
        raise ValueError("k_cache and v_cache must share one layout")
    if softmax_scale is None:
        softmax_scale = 1.0 / (d.head_dim ** 0.5)
    head = [ctypes.byref(d), _ptr(q), _ptr(summaries), _ptr(k_cache), _ptr(v_cache), lay,
            k_cache.shape[0], _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
            block_table.shape[0], budget_pages]
    tail = [float(softmax_scale), _ptr(sel), _ptr(sel_count), _ptr(out), _ptr(out_lse),
            _ptr(score_ws), score_ws.numel() * score_ws.element_size(), _ptr(attend_ws),
            0 if attend_ws is None else attend_ws.numel() * attend_ws.element_size(),
            _stream(stream)]
    if n_tables is None:
        _check("locks_decode_layer", lib().locks_decode_layer(*head, *tail))
    else:
        _check("locks_decode_layer_tables",
               lib().locks_decode_layer_tables(*head, int(n_tables), *tail))


NOALLOC_SCRATCH_BYTES = 64 << 20


def decode_layer_noalloc_bytes(d: Dims, batch, max_pages, budget_pages) -> int:
    return lib().locks_decode_layer_noalloc_bytes(ctypes.byref(d), batch, max_pages, budget_pages)


def decode_layer_noalloc(d: Dims, q, summaries, k_cache, v_cache, block_table, seq_lens,
                         budget_pages, sel, sel_count, out, out_lse=None, softmax_scale=None,
                         stream=None):
    """decode_layer without workspaces: the library's own device scratch array
    (64 MiB per GPU) stands in for them.  Calls that overlap on one GPU race
    on that array."""
    B, P, hq = block_table.shape[0], block_table.shape[1], d.num_q_heads
    _need(q, "q", torch.bfloat16, numel=B * hq * d.head_dim)
    _need(summaries, "summaries", torch.uint8,
          numel=d.num_kv_heads * k_cache.shape[0] * _rec_bytes(d))
    _need(k_cache, "k_cache", torch.bfloat16)
    _need(v_cache, "v_cache", torch.bfloat16)
    _kv_heads(d, k_cache, "k_cache")
    _kv_heads(d, v_cache, "v_cache")
    _need(block_table, "block_table", torch.int32, numel=B * P)
    _need(seq_lens, "seq_lens", torch.int32, numel=B)
    _need(sel, "sel", torch.int32, numel=B * d.num_kv_heads * budget_pages)
    _need(sel_count, "sel_count", torch.int32, numel=B * d.num_kv_heads)
    _need(out, "out", torch.bfloat16, numel=B * hq * d.head_dim)
    _need(out_lse, "out_lse", torch.float32, numel=B * hq)
    _on_device(q=q, summaries=summaries, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
               seq_lens=seq_lens, sel=sel, sel_count=sel_count, out=out, out_lse=out_lse)
    lay = kv_layout(k_cache)
    lv = kv_layout(v_cache)
    if (lay.block_stride, lay.head_stride, lay.token_stride) != (
            lv.block_stride, lv.head_stride, lv.token_stride):
        raise ValueError("k_cache and v_cache must share one layout")
    if softmax_scale is None:
        softmax_scale = 1.0 / (d.head_dim ** 0.5)
    st = lib().locks_decode_layer_noalloc(
        ctypes.byref(d), _ptr(q), _ptr(summaries), _ptr(k_cache), _ptr(v_cache), lay,
        k_cache.shape[0], _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
        block_table.shape[0], budget_pages, float(softmax_scale), _ptr(sel), _ptr(sel_count),
        _ptr(out), _ptr(out_lse), _stream(stream))
    _check("locks_decode_layer_noalloc", st)


def shared_basis(d: Dims, k_cache, block_ids, basis, eigvals=None, workspace=None, stream=None):
    """Top-rank eigenvectors of the pooled page deviations per KV head.
    basis: fp32 [Hkv, rank, 128]; eigvals: optional fp32 [Hkv, 128]."""
    n, hkv = block_ids.numel(), d.num_kv_heads
    _need(k_cache, "k_cache", torch.bfloat16)
    _kv_heads(d, k_cache, "k_cache")
    _need(block_ids, "block_ids", torch.int32, numel=n)
    _need(basis, "basis", torch.float32, numel=hkv * d.rank * d.head_dim)
    _need(eigvals, "eigvals", torch.float32, numel=hkv * d.head_dim)
    _on_device(k_cache=k_cache, block_ids=block_ids, basis=basis, eigvals=eigvals,
               workspace=workspace)
    if workspace is None:
        nbytes = lib().locks_shared_basis_workspace_bytes(ctypes.byref(d), n)
        workspace = torch.empty(max(1, nbytes), dtype=torch.uint8, device=k_cache.device)
    st = lib().locks_shared_basis(ctypes.byref(d), _ptr(k_cache), kv_layout(k_cache),
                                  _ptr(block_ids), n, k_cache.shape[0], _ptr(basis),
                                  _ptr(eigvals), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream))
    _check("locks_shared_basis", st)


def build_summaries_basis(d: Dims, k_cache, block_ids, basis, summaries, stream=None):
    """Summaries of the listed blocks in a given basis (fp32 [Hkv, rank, 128])."""
    hkv = d.num_kv_heads
    _need(k_cache, "k_cache", torch.bfloat16)
    _kv_heads(d, k_cache, "k_cache")
    _need(block_ids, "block_ids", torch.int32, numel=block_ids.numel())
    _need(basis, "basis", torch.float32, numel=hkv * d.rank * d.head_dim)
    _need(summaries, "summaries", torch.uint8, numel=hkv * k_cache.shape[0] * _rec_bytes(d))
    _on_device(k_cache=k_cache, block_ids=block_ids, basis=basis, summaries=summaries)
    st = lib().locks_build_summaries_basis(ctypes.byref(d), _ptr(k_cache), kv_layout(k_cache),
                                           _ptr(block_ids), block_ids.numel(), k_cache.shape[0],
                                           _ptr(basis), _ptr(summaries), _stream(stream))
    _check("locks_build_summaries_basis", st)

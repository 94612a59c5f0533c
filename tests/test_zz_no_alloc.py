"""The decode layer that allocates nothing (locks_decode_layer_noalloc): its
outputs equal locks_decode_layer's, call after call, with the library's own
device scratch array in place of the workspaces.  The second call is smaller
than the first, so stale scratch contents from the first cannot pass."""

import ctypes

import numpy as np
import pytest
import torch

from kv_cache_page_int4_amd import locks as L
from synth import get_workload
from synth.host import generate


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def test_oversize_request_is_refused_before_any_launch():
    """Host-side: a request above the 64 MiB scratch returns a workspace
    error before the device is touched (the pointers here are never used)."""
    if not __import__("os").path.exists(L.LIB_PATH):
        pytest.skip("liblocks.so not built")
    lib = L.lib()
    d = L.dims(32, 8)
    assert L.decode_layer_noalloc_bytes(d, 1, 65537, 128) < L.NOALLOC_SCRATCH_BYTES
    big = (64, 16385, 128)                       # 64 sequences of 256K tokens
    assert L.decode_layer_noalloc_bytes(d, *big) > L.NOALLOC_SCRATCH_BYTES
    P = ctypes.c_void_p
    lay = L.KVLayout(32768, 4096, 128)
    st = lib.locks_decode_layer_noalloc(ctypes.byref(d), P(256), P(256), P(256), P(256), lay,
                                        1 << 20, P(256), big[1], P(256), big[0], big[2], 0.0883,
                                        P(256), P(256), P(256), None, None)
    assert st == L.ERR_WORKSPACE
    # an invalid shape reports the shape error, also before any launch
    st = lib.locks_decode_layer_noalloc(ctypes.byref(L.dims(24, 8)), P(256), P(256), P(256),
                                        P(256), lay, 4, P(256), 4, P(256), 1, 4, 0.0883, P(256),
                                        P(256), P(256), None, None)
    assert st == L.ERR_UNSUPPORTED


def _layer(name, **kw):
    w = get_workload(name, **kw)
    x = generate(w)
    d = L.dims(w.hq, w.hkv)
    k, v, q = _dev(x.k_cache[0]), _dev(x.v_cache[0]), _dev(x.q[0])
    bt = torch.from_numpy(x.block_table).cuda()
    seq = torch.from_numpy(x.seq_lens).cuda()
    summ = torch.empty((w.hkv, w.num_blocks, L.summary_bytes(d)), dtype=torch.uint8, device="cuda")
    L.build_summaries(d, k, torch.arange(w.num_blocks, dtype=torch.int32, device="cuda"), summ)
    return w, d, k, v, q, bt, seq, summ


@pytest.mark.gpu
def test_noalloc_equals_decode_layer_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cases = [("llama8b-32k", dict(batch=2)),                      # larger first
             ("llama8b-32k", dict(batch=1, ctx=16 * 700 + 9))]    # then smaller, ragged
    for name, kw in cases:
        w, d, k, v, q, bt, seq, summ = _layer(name, **kw)
        budget = w.budget_pages
        P = bt.shape[1]
        need = L.decode_layer_noalloc_bytes(d, w.batch, P, budget)
        assert 0 < need <= L.NOALLOC_SCRATCH_BYTES
        outs = []
        for noalloc in (False, True):
            sel = torch.full((w.batch, w.hkv, budget), -7, dtype=torch.int32, device="cuda")
            cnt = torch.full((w.batch, w.hkv), -7, dtype=torch.int32, device="cuda")
            out = torch.full((w.batch, w.hq, 128), 3.0, dtype=torch.bfloat16, device="cuda")
            olse = torch.full((w.batch, w.hq), 3.0, dtype=torch.float32, device="cuda")
            if noalloc:
                L.decode_layer_noalloc(d, q, summ, k, v, bt, seq, budget, sel, cnt, out,
                                       out_lse=olse)
            else:
                ws = L.workspace(d, w.batch, P, budget)
                L.decode_layer(d, q, summ, k, v, bt, seq, budget, sel, cnt, out, ws,
                               out_lse=olse)
            torch.cuda.synchronize()
            outs.append((sel, cnt, out, olse))
        for a, b, what in zip(outs[0], outs[1], ("sel", "sel_count", "out", "out_lse")):
            assert torch.equal(a, b), f"{what} differs ({name} {kw})"
        print(f"[no-alloc] {name} {kw}: identical to locks_decode_layer "
              f"({need / 2**20:.1f} MiB of scratch)", flush=True)

"""The Python binding refuses buffers that are too small or not dense before
anything reaches the library (the C ABI takes raw pointers and cannot see
buffer sizes).  Runs on the CPU: the checks come before any device work."""

import pytest
import torch

L = pytest.importorskip("kv_cache_page_int4_amd.locks")

D = L.dims(32, 8)
B, P, BUD = 2, 64, 16


def t(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def base():
    return dict(q=t((B, 32, 128), torch.bfloat16), bt=t((B, P), torch.int32),
                seq=t((B,), torch.int32), lse=t((B, 32, P), torch.float32),
                summ=t((8, 100, 832), torch.uint8), ws=t((16,), torch.uint8),
                k=t((100, 8, 16, 128), torch.bfloat16), v=t((100, 8, 16, 128), torch.bfloat16),
                sel=t((B, 8, BUD), torch.int32), cnt=t((B, 8), torch.int32),
                out=t((B, 32, 128), torch.bfloat16), olse=t((B, 32), torch.float32))


def test_select_pages_sizes():
    a = base()
    with pytest.raises(ValueError, match="sel holds"):
        L.select_pages(D, a["lse"], a["seq"], BUD, t((B, 8, BUD - 1), torch.int32), a["cnt"],
                       a["ws"])
    with pytest.raises(ValueError, match="sel_count holds"):
        L.select_pages(D, a["lse"], a["seq"], BUD, a["sel"], t((B, 7), torch.int32), a["ws"])
    # two tables need only [B, 2, budget]; one table per KV head needs [B, 8, budget]
    with pytest.raises(ValueError, match="must be a device tensor"):
        L.select_pages(D, a["lse"], a["seq"], BUD, t((B, 2, BUD), torch.int32),
                       t((B, 2), torch.int32), a["ws"], n_tables=2)
    with pytest.raises(ValueError, match="sel holds"):
        L.select_pages(D, a["lse"], a["seq"], BUD, t((B, 2, BUD), torch.int32),
                       t((B, 2), torch.int32), a["ws"])


def test_score_pages_and_select_sizes():
    a = base()
    with pytest.raises(ValueError, match="page_lse holds"):
        L.score_pages(D, a["q"], a["summ"], 100, a["bt"], a["seq"], t((B, 32, P - 1), torch.float32),
                      a["ws"])
    with pytest.raises(ValueError, match="summaries holds"):
        L.score_pages(D, a["q"], t((8, 99, 832), torch.uint8), 100, a["bt"], a["seq"], a["lse"],
                      a["ws"])
    with pytest.raises(ValueError, match="q holds"):
        L.score_select(D, t((B, 31, 128), torch.bfloat16), a["summ"], 100, a["bt"], a["seq"], BUD,
                       a["sel"], a["cnt"], a["ws"])
    # rank 16 records are 1536 bytes
    with pytest.raises(ValueError, match="summaries holds"):
        L.score_pages(L.dims(32, 8, rank=16), a["q"], a["summ"], 100, a["bt"], a["seq"], a["lse"],
                      a["ws"])


def test_attend_and_layer_sizes():
    a = base()
    with pytest.raises(ValueError, match="out holds"):
        L.sparse_attend(D, a["q"], a["k"], a["v"], a["bt"], a["seq"], a["sel"], a["cnt"], BUD,
                        t((B, 32, 127), torch.bfloat16), a["ws"])
    with pytest.raises(ValueError, match="out_lse holds"):
        L.sparse_attend(D, a["q"], a["k"], a["v"], a["bt"], a["seq"], None, None, 0, a["out"],
                        a["ws"], out_lse=t((B, 31), torch.float32))
    with pytest.raises(ValueError, match="KV heads"):
        L.sparse_attend(D, a["q"], t((100, 4, 16, 128), torch.bfloat16), a["v"], a["bt"],
                        a["seq"], None, None, 0, a["out"], a["ws"])
    with pytest.raises(ValueError, match="sel holds"):
        L.decode_layer(D, a["q"], a["summ"], a["k"], a["v"], a["bt"], a["seq"], BUD + 1, a["sel"],
                       a["cnt"], a["out"], a["ws"], a["ws"])
    with pytest.raises(ValueError, match="must be contiguous"):
        L.sparse_attend(D, a["q"], a["k"], a["v"], a["bt"], a["seq"], None, None, 0,
                        t((B, 128, 32), torch.bfloat16).transpose(1, 2), a["ws"])


def test_build_and_basis_sizes():
    a = base()
    ids = t((10,), torch.int32)
    with pytest.raises(ValueError, match="summaries holds"):
        L.build_summaries(D, a["k"], ids, t((8, 100, 831), torch.uint8))
    with pytest.raises(ValueError, match="raw_debug holds"):
        L.build_summaries(D, a["k"], ids, a["summ"], raw_debug=t((10, 8, 1279), torch.float32))
    with pytest.raises(ValueError, match="basis holds"):
        L.shared_basis(D, a["k"], ids, t((8, 7, 128), torch.float32))
    with pytest.raises(ValueError, match="eigvals holds"):
        L.shared_basis(D, a["k"], ids, t((8, 8, 128), torch.float32),
                       eigvals=t((8, 127), torch.float32))
    with pytest.raises(ValueError, match="summaries holds"):
        L.build_summaries_basis(L.dims(32, 8, rank=4), a["k"], ids, t((8, 4, 128), torch.float32),
                                t((8, 100, 511), torch.uint8))


def test_workspaces_are_checked_to_be_on_the_device(monkeypatch):
    """Every workspace a call hands to the kernels goes through the device
    check, with the call's other buffers (a host workspace would give the
    kernels a host pointer)."""
    a = base()
    seen = []

    def spy(**tensors):
        seen.append(set(k for k, v in tensors.items() if v is not None))
        raise ValueError("stop before any launch")

    monkeypatch.setattr(L, "_on_device", spy)
    calls = [
        (lambda: L.score_pages(D, a["q"], a["summ"], 100, a["bt"], a["seq"], a["lse"], a["ws"]),
         {"workspace"}),
        (lambda: L.select_pages(D, a["lse"], a["seq"], BUD, a["sel"], a["cnt"], a["ws"]),
         {"workspace"}),
        (lambda: L.score_select(D, a["q"], a["summ"], 100, a["bt"], a["seq"], BUD, a["sel"],
                                a["cnt"], a["ws"]), {"workspace"}),
        (lambda: L.sparse_attend(D, a["q"], a["k"], a["v"], a["bt"], a["seq"], a["sel"], a["cnt"],
                                 BUD, a["out"], a["ws"]), {"workspace"}),
        (lambda: L.decode_layer(D, a["q"], a["summ"], a["k"], a["v"], a["bt"], a["seq"], BUD,
                                a["sel"], a["cnt"], a["out"], a["ws"], a["ws"]),
         {"score_ws", "attend_ws"}),
        (lambda: L.decode_layer(D, a["q"], a["summ"], a["k"], a["v"], a["bt"], a["seq"], BUD,
                                a["sel"], a["cnt"], a["out"], a["ws"]), {"score_ws"}),
        (lambda: L.shared_basis(D, a["k"], t((10,), torch.int32), t((8, 8, 128), torch.float32),
                                workspace=a["ws"]), {"workspace"}),
    ]
    for fn, want in calls:
        seen.clear()
        with pytest.raises(ValueError, match="stop before any launch"):
            fn()
        assert seen and want <= seen[-1], (want, seen)


def test_host_workspace_is_refused():
    """A host workspace with otherwise valid shapes raises before the library
    is reached (CPU tensors throughout: the first non-device buffer named)."""
    a = base()
    with pytest.raises(ValueError, match="must be a device tensor"):
        L.score_pages(D, a["q"], a["summ"], 100, a["bt"], a["seq"], a["lse"], a["ws"])
    with pytest.raises(ValueError, match="must be a device tensor"):
        L._on_device(workspace=a["ws"])

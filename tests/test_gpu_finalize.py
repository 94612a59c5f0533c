"""Incremental finalization on the GPU: locks_finalize_pages builds exactly
the records locks_build_summaries builds, only for sequences whose newest
token completed a page, and a captured decode step that includes it keeps
the summaries current while tokens are appended between replays."""

import numpy as np
import pytest
import torch

from kv_cache_page_int4_amd import locks as L
from kv_cache_page_int4_amd.step import DecodeStep
from synth import get_workload
from synth.host import generate

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from tests.gpu_common import log  # noqa: E402


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def test_finalize_builds_only_completed_pages():
    seq = [16 * 37, 16 * 37 + 5, 16 * 200, 0, 16 * 256]
    w = get_workload("tiny-4k", batch=len(seq), shuffled_blocks=True)
    x = generate(w, seq_lens=seq)
    d = L.dims(w.hq, w.hkv)
    k = _dev(x.k_cache[0])
    bt = torch.from_numpy(x.block_table).cuda()
    sl = torch.from_numpy(x.seq_lens).cuda()
    nb = w.num_blocks
    summ = torch.zeros((w.hkv, nb, 832), dtype=torch.uint8, device="cuda")
    L.finalize_pages(d, k, bt, sl, summ)
    ref = torch.zeros_like(summ)
    L.build_summaries(d, k, torch.arange(nb, dtype=torch.int32, device="cuda"), ref)
    torch.cuda.synchronize()
    want = set()
    for b, s in enumerate(seq):
        if s > 0 and s % 16 == 0:
            want.add(int(x.block_table[b, s // 16 - 1]))
    for blk in range(nb):
        if blk in want:
            assert torch.equal(summ[:, blk], ref[:, blk]), f"block {blk} differs from a direct build"
        else:
            assert int(summ[:, blk].abs().sum()) == 0, f"block {blk} should be untouched"
    log(f"[finalize] built {len(want)} pages, others untouched")


def test_decode_graph_with_incremental_finalization():
    """Tokens are appended between replays of one captured step; whenever a
    page fills, the replay summarizes it, and every output equals the eager
    library calls on the same state."""
    w = get_workload("llama8b-32k", batch=2, layers=2, ctx=16 * 512)
    start = [16 * 300 - 3, 16 * 500 - 1]
    x = generate(w, seq_lens=start)
    d = L.dims(w.hq, w.hkv)
    k, v, q = _dev(x.k_cache), _dev(x.v_cache), _dev(x.q)
    bt = torch.from_numpy(x.block_table).cuda()
    seq = torch.from_numpy(x.seq_lens.copy()).cuda()
    nb = w.num_blocks
    summ = torch.zeros((w.layers, w.hkv, nb, 832), dtype=torch.uint8, device="cuda")
    for layer in range(w.layers):   # pages finalized before decoding starts
        for b, s in enumerate(start):
            blocks = torch.from_numpy(x.block_table[b, :s // 16].astype(np.int32)).cuda()
            L.build_summaries(d, k[layer], blocks, summ[layer])
    step = DecodeStep(d, k, v, summ, q, bt, seq, 32, finalize=True)
    step.run()
    torch.cuda.synchronize()
    step.capture()
    gen = torch.Generator(device="cuda").manual_seed(7)
    cur = list(start)
    completed = []
    for t in range(20):
        # append one token per sequence (eager work outside the graph)
        for b in range(w.batch):
            pos = cur[b]
            blk = int(x.block_table[b, pos // 16])
            k[:, blk, :, pos % 16, :] = torch.randn((w.layers, w.hkv, 128), generator=gen,
                                                    device="cuda").to(torch.bfloat16)
            v[:, blk, :, pos % 16, :] = torch.randn((w.layers, w.hkv, 128), generator=gen,
                                                    device="cuda").to(torch.bfloat16)
            cur[b] += 1
            if cur[b] % 16 == 0:
                completed.append((b, cur[b] // 16 - 1, t))
        seq.copy_(torch.tensor(cur, dtype=torch.int32))
        torch.cuda.synchronize()
        step.replay()
        torch.cuda.synchronize()
        if t in (2, 7, 19):
            # eager reference on the same state
            sel_r = torch.empty_like(step.sel[0])
            cnt_r = torch.empty_like(step.cnt[0])
            out_r = torch.empty_like(step.out[0])
            ws = torch.empty_like(step.ws_score)
            wa = torch.empty_like(step.ws_att)
            for layer in range(w.layers):
                L.score_select(d, q[layer], summ[layer], nb, bt, seq, 32, sel_r, cnt_r, ws)
                L.sparse_attend(d, q[layer], k[layer], v[layer], bt, seq, sel_r, cnt_r, 32, out_r,
                                wa)
                torch.cuda.synchronize()
                assert torch.equal(sel_r, step.sel[layer]) and torch.equal(cnt_r, step.cnt[layer])
                assert torch.equal(out_r, step.out[layer]), f"replay {t} layer {layer} output"
    assert len(completed) >= 2, completed
    # every finalized page's record equals a direct build of the final cache
    ref = torch.zeros_like(summ)
    for layer in range(w.layers):
        for b in range(w.batch):
            blocks = torch.from_numpy(x.block_table[b, :cur[b] // 16].astype(np.int32)).cuda()
            L.build_summaries(d, k[layer], blocks, ref[layer])
    torch.cuda.synchronize()
    for layer in range(w.layers):
        for b in range(w.batch):
            for j in range(cur[b] // 16):
                blk = int(x.block_table[b, j])
                assert torch.equal(summ[layer, :, blk], ref[layer, :, blk]), (layer, b, j)
    log(f"[finalize graph] pages completed during decoding: {completed}")

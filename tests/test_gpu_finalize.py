"""Incremental finalization on the GPU: locks_finalize_pages builds exactly
the records locks_build_summaries builds, only for sequences whose newest
token completed a page, and a captured decode step that appends each layer's
newest key and summarizes the page it completes keeps the summaries current
while tokens are appended between replays; its records, selections and
outputs are checked against the oracle.  Both forms of the step are held to
it: the page summarized inside the step before the layer is scored, and
summarized after the step (all layers in one launch) with the newest page
pending during the step, attended in full."""

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

import oracle as O  # noqa: E402
from tests.gpu_common import (LSE_TOL, OUT_TOL, check_selection, compare_build_codes,  # noqa: E402
                              from_dev_bf16, log)


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


@pytest.mark.parametrize("mode", ["layer", "step"])
def test_decode_graph_with_incremental_finalization(mode):
    """A captured step that, per layer, appends the newest token's key and
    value (the model's work, inside the graph) and runs that layer's decode,
    summarizing the page that key completed either before the layer is scored
    (mode "layer") or after the step (mode "step", the newest page pending
    during it).  Tokens are appended between replays; every record finalized
    during the replays is checked against the oracle's build of the same keys,
    the replays in which a page completes (and the last one) against the
    oracle, and two others against the eager library calls."""
    w = get_workload("llama8b-32k", batch=2, layers=2, ctx=16 * 512)
    start = [16 * 300 - 3, 16 * 500 - 1]
    x = generate(w, seq_lens=start)
    d = L.dims(w.hq, w.hkv)
    k, v, q = _dev(x.k_cache), _dev(x.v_cache), _dev(x.q)
    bt = torch.from_numpy(x.block_table).cuda()
    seq = torch.from_numpy(x.seq_lens.copy()).cuda()
    nb = w.num_blocks
    budget = 32
    summ = torch.zeros((w.layers, w.hkv, nb, 832), dtype=torch.uint8, device="cuda")
    for layer in range(w.layers):   # pages finalized before decoding starts
        for b, s in enumerate(start):
            blocks = torch.from_numpy(x.block_table[b, :s // 16].astype(np.int32)).cuda()
            L.build_summaries(d, k[layer], blocks, summ[layer])
    # the newest token's key and value of every layer, written by the step
    # itself at position seq_lens - 1 (staged here between replays)
    new_k = torch.empty((w.layers, w.batch, w.hkv, 128), dtype=torch.bfloat16, device="cuda")
    new_v = torch.empty_like(new_k)
    rows = torch.arange(w.batch, device="cuda")
    for b, s in enumerate(start):   # staged = the current last token: the warm-up rewrites it
        blk = int(x.block_table[b, (s - 1) // 16])
        new_k[:, b] = k[:, blk, :, (s - 1) % 16]
        new_v[:, b] = v[:, blk, :, (s - 1) % 16]

    def append(layer):
        pos = (seq - 1).long()
        blk = bt[rows, pos // 16].long()
        slot = pos % 16
        k[layer][blk, :, slot] = new_k[layer]
        v[layer][blk, :, slot] = new_v[layer]

    step = DecodeStep(d, k, v, summ, q, bt, seq, budget, finalize=mode, before_layer=append)
    assert step.d.newest_page_pending == (mode == "step")
    d = step.d
    step.capture()
    gen = torch.Generator(device="cuda").manual_seed(7)
    cur = list(start)
    completed = []
    oracle_checked = []
    for t in range(20):
        new_k.copy_(torch.randn(new_k.shape, generator=gen, device="cuda").to(torch.bfloat16))
        new_v.copy_(torch.randn(new_v.shape, generator=gen, device="cuda").to(torch.bfloat16))
        done_now = []
        for b in range(w.batch):
            cur[b] += 1
            if cur[b] % 16 == 0:
                done_now.append((b, cur[b] // 16 - 1))
                completed.append((b, cur[b] // 16 - 1, t))
        seq.copy_(torch.tensor(cur, dtype=torch.int32))
        torch.cuda.synchronize()
        for a in (step.sel, step.cnt, step.out, step.out_lse):
            a.fill_(-3)
        step.replay()
        torch.cuda.synchronize()
        for b in range(w.batch):   # the staged token landed at its position in every layer
            blk = int(x.block_table[b, (cur[b] - 1) // 16])
            assert torch.equal(k[:, blk, :, (cur[b] - 1) % 16], new_k[:, b])
        if done_now or t == 19:
            _check_against_oracle(d, k, v, q, summ, bt, seq, step, budget, cur, done_now)
            oracle_checked.append(t)
        if t in (5, 11):
            # eager reference on the same state
            sel_r = torch.empty_like(step.sel[0])
            cnt_r = torch.empty_like(step.cnt[0])
            out_r = torch.empty_like(step.out[0])
            ws = torch.empty_like(step.ws_score)
            wa = torch.empty_like(step.ws_att)
            for layer in range(w.layers):
                L.score_select(d, q[layer], summ[layer], nb, bt, seq, budget, sel_r, cnt_r, ws)
                L.sparse_attend(d, q[layer], k[layer], v[layer], bt, seq, sel_r, cnt_r, budget,
                                out_r, wa)
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
    log(f"[finalize graph, {mode}] pages completed during decoding: {completed}; "
        f"replays checked against the oracle: {oracle_checked}")


def _check_against_oracle(d, k, v, q, summ, bt, seq, step, budget, cur, done_now):
    """The replay's state against the oracle: records of the pages completed
    in this replay (codes against the oracle's build of the keys now in the
    cache), the page LSE of every summarized page on the GPU's codes (with
    the newest page pending, the page just completed is not one of them: it
    was attended in full), the selection from the GPU's scores and the output
    over the GPU's selection."""
    layers, hkv, nb = summ.shape[0], summ.shape[1], summ.shape[2]
    hq = q.shape[2]
    G = hq // hkv
    btn = bt.cpu().numpy()
    P = btn.shape[1]
    kb = from_dev_bf16(k)
    vb = from_dev_bf16(v)
    qb = from_dev_bf16(q)
    recs_all = summ.cpu().numpy()
    lse = torch.empty((len(cur), hq, P), dtype=torch.float32, device="cuda")
    ws = torch.empty(L.score_workspace_bytes(d, len(cur), P, 0), dtype=torch.uint8, device="cuda")
    for layer in range(layers):
        for b, j in done_now:
            blk = int(btn[b, j])
            for g in range(hkv):
                K = O.bf16_to_f64(kb[layer, blk, g])[None]
                compare_build_codes(K, recs_all[layer, g, blk][None],
                                    where=f"finalized layer {layer} b={b} page {j} g={g}")
        L.score_pages(d, q[layer], summ[layer], nb, bt, seq, lse, ws)
        torch.cuda.synchronize()
        pend = d.newest_page_pending
        for b in range(len(cur)):
            n = O.summarized_pages(cur[b], pend)
            assert torch.all(torch.isneginf(lse[b, :, n:P]))
            for g in range(hkv):
                qd = O.bf16_to_f64(qb[layer, b, g * G:(g + 1) * G])
                s_ref = O.score_records(qd, recs_all[layer, g, btn[b, :n]])
                s_gpu = lse[b, g * G:(g + 1) * G, :n].double().cpu().numpy()
                assert np.abs(s_gpu - s_ref).max() <= LSE_TOL
                _, log_m, _ = O.group_mass(s_gpu)
                c = int(step.cnt[layer, b, g])
                got = step.sel[layer, b, g, :c].cpu().numpy()
                check_selection(got, log_m, budget)
                o_ref, l_ref = O.sparse_attention(qd, kb[layer], vb[layer], btn[b], g, got, cur[b],
                                                  pending=pend)
                o_gpu = step.out[layer, b, g * G:(g + 1) * G].float().cpu().numpy()
                assert np.abs(o_gpu - o_ref).max() <= OUT_TOL
                assert np.abs(step.out_lse[layer, b, g * G:(g + 1) * G].cpu().numpy()
                              - l_ref).max() <= LSE_TOL

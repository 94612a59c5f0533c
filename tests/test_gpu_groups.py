"""GQA groups other than 4 query heads per KV head, and the logit scale of the
one-call layer, on the GPU against the fp64 oracle.

The pages average the mass shares of "the query heads of a group" and target
standard GQA models (LOCKS explainer, technical summary sec. 2, group-shared
selection; sec. 4): groups of 1 (multi-head attention), 2, 4 and 8 heads per
KV head are accepted.  Every gate is the one the group-of-4 parity tests use:
page LSE 1e-3 absolute on the GPU's own codes, selected sets identical outside
the 1e-4 relative window, sparse output 2e-2 max-abs, the read-every-key page
LSE 1e-3, and the one-call layer bit-identical to the two calls."""

import math

import numpy as np
import pytest
import torch

import oracle as O
from kv_cache_page_int4_amd import locks as L
from synth import get_workload
from synth.host import generate

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from tests.gpu_common import (LSE_TOL, OUT_TOL, Layer, check_selection, log,  # noqa: E402
                              oracle_scores, scores_of)

# (query heads, KV heads, batch, sequence lengths or None for the full 32K)
GROUPS = [
    (32, 32, 1, None),                     # G = 1
    (16, 8, 1, None),                      # G = 2
    (64, 8, 1, None),                      # G = 8
    (8, 1, 2, [4096 - 5, 16 * 37 + 9]),    # G = 8, ragged, tail pages
    (2, 1, 2, [4096 - 11, 16 * 101]),      # G = 2, ragged
    (1, 1, 1, [4096 - 1]),                 # G = 1, one head
]


def _gen(hq, hkv, batch, seqs):
    if seqs is None:
        w = get_workload("llama8b-32k", hq=hq, hkv=hkv, batch=batch)
    else:
        w = get_workload("tiny-4k", hq=hq, hkv=hkv, batch=batch, shuffled_blocks=True)
    return generate(w, seq_lens=seqs)


@pytest.mark.parametrize("hq,hkv,batch,seqs", GROUPS,
                         ids=[f"{a}q{b}kv-b{c}" for a, b, c, _ in GROUPS])
def test_group_sizes_against_oracle(hq, hkv, batch, seqs):
    x = _gen(hq, hkv, batch, seqs)
    w = x.w
    G = w.group
    budget = w.budget_pages
    log(f"[groups] {hq}q/{hkv}kv (G={G}) batch {batch} ctx {w.ctx}")
    lay = Layer(x, 0)
    lay.gpu_build()
    torch.cuda.synchronize()
    recs = lay.summ.cpu().numpy()
    lse = lay.score()
    sel, cnt, lse2 = lay.score_select(budget)
    out, olse = lay.attend(sel, cnt, budget)
    # one-call layer with a single workspace
    P = lay.bt.shape[1]
    ws = L.workspace(lay.d, batch, P, budget)
    sel1 = torch.full_like(sel, -7)
    cnt1 = torch.full_like(cnt, -7)
    out1 = torch.empty_like(out)
    olse1 = torch.empty_like(olse)
    L.decode_layer(lay.d, lay.q, lay.summ, lay.k, lay.v, lay.bt, lay.seq, budget, sel1, cnt1, out1,
                   ws, out_lse=olse1)
    # read-every-key page LSE
    ex = torch.full((batch, hq, P), float("nan"), dtype=torch.float32, device="cuda")
    L.exact_page_lse(lay.d, lay.q, lay.k, lay.bt, lay.seq, ex)
    torch.cuda.synchronize()
    assert torch.equal(lse, lse2)
    assert torch.equal(sel1, sel) and torch.equal(cnt1, cnt), "one-call layer selection differs"
    assert torch.equal(out1, out) and torch.equal(olse1, olse), "one-call layer output differs"
    worst_lse = worst_out = worst_ex = 0.0
    ties = 0
    for b in range(batch):
        n = int(x.seq_lens[b]) // 16
        for g in range(hkv):
            s_gpu = scores_of(x, 0, b, g, lse)
            s_ref = oracle_scores(x, recs, 0, b, g)
            err = float(np.abs(s_gpu - s_ref).max())
            worst_lse = max(worst_lse, err)
            assert err <= LSE_TOL, f"page LSE off by {err} (b={b}, g={g})"
            assert torch.all(torch.isneginf(lse[b, g * G:(g + 1) * G, n:]))
            _, log_m, _ = O.group_mass(s_gpu)
            c = int(cnt[b, g])
            got = sel[b, g, :c].cpu().numpy()
            ties += check_selection(got, log_m, budget)
            q = O.bf16_to_f64(x.q[0, b, g * G:(g + 1) * G])
            o_ref, l_ref = O.sparse_attention(q, x.k_cache[0], x.v_cache[0], x.block_table[b], g,
                                              got, int(x.seq_lens[b]))
            e = float(np.abs(out[b, g * G:(g + 1) * G].float().cpu().numpy() - o_ref).max())
            worst_out = max(worst_out, e)
            assert e <= OUT_TOL, f"attention output off by {e} (b={b}, g={g})"
            assert np.abs(olse[b, g * G:(g + 1) * G].cpu().numpy() - l_ref).max() <= LSE_TOL
            if g < 4:   # the exact scorer on a few groups (it reads every key)
                K = O.bf16_to_f64(x.k_cache[0][x.block_table[b, :n], g])
                want = O.page_lse_exact(q[None], K)                   # [n, G]
                ee = float(np.abs(ex[b, g * G:(g + 1) * G, :n].double().cpu().numpy()
                                  - want.T).max())
                worst_ex = max(worst_ex, ee)
                assert ee <= LSE_TOL, f"exact page LSE off by {ee} (b={b}, g={g})"
                assert torch.all(torch.isneginf(ex[b, g * G:(g + 1) * G, n:]))
    log(f"[groups {hq}q/{hkv}kv] max|dLSE|={worst_lse:.2e} exact {worst_ex:.2e} "
        f"max|dOut|={worst_out:.2e} tie-window pages={ties}")


def test_group_of_eight_with_layer_wide_table():
    """A group of 8 with one selection table for the whole layer (all 64
    query heads share one page set) against the oracle's table selection."""
    x = _gen(64, 8, 1, None)
    w = x.w
    budget = w.budget_pages
    lay = Layer(x, 0)
    lay.gpu_build()
    lse = lay.score()
    P = lay.bt.shape[1]
    sel = torch.full((1, 1, budget), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((1, 1), -7, dtype=torch.int32, device="cuda")
    ws = L.workspace(lay.d, 1, P, budget)
    L.select_pages(lay.d, lse, lay.seq, budget, sel, cnt, ws, n_tables=1)
    torch.cuda.synchronize()
    n = w.pages
    s_all = lse[0, :, :n].double().cpu().numpy()
    (log_m, _), = O.table_selection(s_all, 1, budget)
    got = sel[0, 0, :int(cnt[0, 0])].cpu().numpy()
    ties = check_selection(got, log_m, budget)
    log(f"[groups 64q/8kv, one table] tie-window pages={ties}")


def test_decode_layer_scores_at_its_softmax_scale():
    """locks_decode_layer scores pages at the logit scale it attends with.
    With scale s the GPU's selection must be the oracle's top-k of the masses
    computed at s on the GPU's codes, up to the error the page-LSE gate
    allows: each page LSE and each head normalizer within 1e-3, so a log mass
    within 2e-3 of the oracle's; pages whose oracle log mass lies within 4e-3
    of the k-th are exempt.  The output must be the oracle's attention at s
    over the GPU's selection."""
    x = _gen(32, 8, 1, None)
    w = x.w
    budget = w.budget_pages
    lay = Layer(x, 0)
    lay.gpu_build()
    torch.cuda.synchronize()
    recs = lay.summ.cpu().numpy()
    P = lay.bt.shape[1]
    ws = L.workspace(lay.d, 1, P, budget)
    scale = 0.5 / math.sqrt(128)
    sel = torch.full((1, w.hkv, budget), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((1, w.hkv), -7, dtype=torch.int32, device="cuda")
    out = torch.empty((1, w.hq, 128), dtype=torch.bfloat16, device="cuda")
    L.decode_layer(lay.d, lay.q, lay.summ, lay.k, lay.v, lay.bt, lay.seq, budget, sel, cnt, out,
                   ws, softmax_scale=scale)
    sel_def, cnt_def, _ = lay.score_select(budget, with_lse=False)
    torch.cuda.synchronize()
    n = w.pages
    G = w.group
    differs = 0
    worst = 0.0
    for g in range(w.hkv):
        q = O.bf16_to_f64(x.q[0, 0, g * G:(g + 1) * G])
        s_ref = O.score_records(q, recs[g, x.block_table[0, :n]], scale=scale)
        _, log_m, _ = O.group_mass(s_ref)
        got = sel[0, g, :int(cnt[0, g])].cpu().numpy()
        want = O.select_top_pages(log_m, budget)
        lm_k = np.sort(log_m)[::-1][budget - 1]
        near = np.abs(log_m - lm_k) <= 4e-3
        bad = [j for j in set(got.tolist()) ^ set(want.tolist()) if not near[j]]
        assert not bad, f"selection at scale {scale} differs outside the window: {bad[:8]}"
        differs += int(set(got.tolist()) != set(sel_def[0, g, :int(cnt_def[0, g])].tolist()))
        o_ref, _ = O.sparse_attention(q, x.k_cache[0], x.v_cache[0], x.block_table[0], g, got,
                                      w.ctx, scale=scale)
        e = float(np.abs(out[0, g * G:(g + 1) * G].float().cpu().numpy() - o_ref).max())
        worst = max(worst, e)
        assert e <= OUT_TOL
    # the scale reaches the scorer: at half the temperature the page sets change
    assert differs > 0
    log(f"[scale {scale:.4f}] {differs}/{w.hkv} page sets differ from the 1/sqrt(d) ones; "
        f"max|dOut|={worst:.2e}")

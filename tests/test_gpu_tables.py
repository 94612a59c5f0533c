"""GPU parity of the selection-table variants through the C ABI: one table
serving several KV heads, down to one table for the whole layer (the wider
reading of the group-shared table).  The GPU's page scores feed the oracle's
table_selection; each KV head's attention is checked against fp64 attention
over its table's pages; the one-call layer must equal the separate calls.

Tolerances as elsewhere: page LSE 1e-3 absolute on the GPU's own codes;
selected sets identical except pages within 1e-4 (relative) of the k-th
mass; attention output 2e-2 max-abs."""

import numpy as np
import pytest
import torch

import oracle as O
from synth import get_workload
from synth.host import generate

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from kv_cache_page_int4_amd import locks as L  # noqa: E402
from kv_cache_page_int4_amd.step import DecodeStep  # noqa: E402
from tests.gpu_common import LSE_TOL, OUT_TOL, Layer, check_selection, log  # noqa: E402

_CACHE = {}


def gen(name, seq_lens=None, **kw):
    key = (name, None if seq_lens is None else tuple(seq_lens), tuple(sorted(kw.items())))
    if key not in _CACHE:
        _CACHE[key] = generate(get_workload(name, **kw), seq_lens=seq_lens)
    return _CACHE[key]


CASES = [
    # (workload, kwargs, seq_lens, n_tables, budget, newest page pending)
    ("llama8b-32k", {"batch": 2}, [32768 - 5, 16 * 700 + 3], 1, 128, False),
    ("llama8b-32k", {"batch": 2}, [32768 - 5, 16 * 700 + 3], 2, 128, False),
    ("llama8b-32k", {}, None, 4, 37, False),
    ("llama8b-32k", {"ctx": 16 * 5000 + 9}, None, 1, 300, False),      # 3 chunks of candidates
    ("llama8b-32k", {"batch": 3}, [16 * 5 + 2, 7, 16 * 64], 1, 128, False),   # budget >= pages
    ("llama8b-32k", {"batch": 2}, [32768, 16 * 700], 1, 128, True),    # full last pages pending
    ("llama8b-32k", {"batch": 3}, [16 * 64, 16, 16 * 9 + 4], 2, 128, True),
]


@pytest.mark.parametrize("name,kw,seq,n_tables,budget,pending", CASES)
def test_tables_against_oracle(name, kw, seq, n_tables, budget, pending):
    x = gen(name, seq_lens=seq, **kw)
    w = x.w
    lay = Layer(x, 0)
    lay.gpu_build()
    lay.d = L.dims(w.hq, w.hkv, newest_page_pending=pending)
    torch.cuda.synchronize()
    recs = lay.summ.cpu().numpy()
    lse = lay.score()
    P = lay.bt.shape[1]
    sel = torch.full((w.batch, n_tables, budget), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((w.batch, n_tables), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(L.score_workspace_bytes(lay.d, w.batch, P, budget), dtype=torch.uint8,
                     device="cuda")
    L.select_pages(lay.d, lse, lay.seq, budget, sel, cnt, ws, n_tables=n_tables)
    out = torch.empty((w.batch, w.hq, 128), dtype=torch.bfloat16, device="cuda")
    olse = torch.empty((w.batch, w.hq), dtype=torch.float32, device="cuda")
    wa = L.attend_workspace(lay.d, w.batch, budget + 1)
    L.sparse_attend(lay.d, lay.q, lay.k, lay.v, lay.bt, lay.seq, sel, cnt, budget, out, wa,
                    out_lse=olse, n_tables=n_tables)
    torch.cuda.synchronize()
    kv_per_tab = w.hkv // n_tables
    G = w.group
    worst_lse = worst_out = 0.0
    ties = 0
    for b in range(w.batch):
        n = O.summarized_pages(int(x.seq_lens[b]), int(pending))
        assert torch.all(torch.isneginf(lse[b, :, n:]))
        s_gpu = lse[b, :, :n].double().cpu().numpy()
        if n:
            for g in range(w.hkv):
                q = O.bf16_to_f64(x.q[0, b, g * G:(g + 1) * G])
                s_ref = O.score_records(q, recs[g, x.block_table[b, :n]])
                err = float(np.abs(s_ref - s_gpu[g * G:(g + 1) * G]).max())
                worst_lse = max(worst_lse, err)
                assert err <= LSE_TOL, f"page LSE off by {err} (b={b}, g={g})"
        tables = O.table_selection(s_gpu, n_tables, budget) if n else [(np.zeros(0), [])] * n_tables
        for t, (log_m, _) in enumerate(tables):
            c = int(cnt[b, t])
            got = sel[b, t, :c].cpu().numpy()
            assert torch.all(sel[b, t, c:] == -1)
            ties += check_selection(got, log_m, budget)
            for g in range(t * kv_per_tab, (t + 1) * kv_per_tab):
                q = O.bf16_to_f64(x.q[0, b, g * G:(g + 1) * G])
                o_ref, l_ref = O.sparse_attention(q, x.k_cache[0], x.v_cache[0], x.block_table[b],
                                                  g, got, int(x.seq_lens[b]), pending=int(pending))
                if not (o_ref.shape[0] and np.isfinite(l_ref).all()):
                    continue
                e = float(np.abs(out[b, g * G:(g + 1) * G].float().cpu().numpy() - o_ref).max())
                worst_out = max(worst_out, e)
                assert e <= OUT_TOL, f"attention output off by {e} (b={b}, g={g}, table {t})"
                assert np.abs(olse[b, g * G:(g + 1) * G].cpu().numpy() - l_ref).max() <= LSE_TOL
    log(f"[tables {name} b={w.batch} n_tables={n_tables} budget={budget} pending={pending}] "
        f"max|dLSE|={worst_lse:.2e} max|dOut|={worst_out:.2e} tie-window pages={ties}")

    # the one-call layer (last selection stage inside attention) is identical
    sel2 = torch.full_like(sel, -7)
    cnt2 = torch.full_like(cnt, -7)
    out2 = torch.empty_like(out)
    olse2 = torch.empty_like(olse)
    L.decode_layer(lay.d, lay.q, lay.summ, lay.k, lay.v, lay.bt, lay.seq, budget, sel2, cnt2,
                   out2, ws, wa, out_lse=olse2, n_tables=n_tables)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel2) and torch.equal(cnt, cnt2), "decode_layer selection differs"
    assert torch.equal(out, out2) and torch.equal(olse, olse2), "decode_layer attention differs"


def test_per_kv_head_tables_equal_default_calls():
    """n_tables = Hkv is the default call, bit for bit."""
    x = gen("llama8b-32k", batch=2, seq_lens=[32768 - 5, 16 * 700 + 3])
    w = x.w
    lay = Layer(x, 0)
    lay.gpu_build()
    lse = lay.score()
    sel_a, cnt_a = lay.select(lse, 128)
    sel_b = torch.full_like(sel_a, -7)
    cnt_b = torch.full_like(cnt_a, -7)
    ws = torch.empty(L.score_workspace_bytes(lay.d, w.batch, lay.bt.shape[1], 128),
                     dtype=torch.uint8, device="cuda")
    L.select_pages(lay.d, lse, lay.seq, 128, sel_b, cnt_b, ws, n_tables=w.hkv)
    out_a, olse_a = lay.attend(sel_a, cnt_a, 128)
    out_b = torch.empty_like(out_a)
    olse_b = torch.empty_like(olse_a)
    L.sparse_attend(lay.d, lay.q, lay.k, lay.v, lay.bt, lay.seq, sel_b, cnt_b, 128, out_b,
                    L.attend_workspace(lay.d, w.batch, 129), out_lse=olse_b, n_tables=w.hkv)
    torch.cuda.synchronize()
    assert torch.equal(sel_a, sel_b) and torch.equal(cnt_a, cnt_b)
    assert torch.equal(out_a, out_b) and torch.equal(olse_a, olse_b)


def test_layer_wide_step_graph_replays():
    """A two-layer step with one table per layer, captured and replayed,
    equals its eager run and the three-call path."""
    w = get_workload("llama8b-32k", layers=2)
    x = generate(w)
    d = L.dims(w.hq, w.hkv)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    k, v, q = dev(x.k_cache), dev(x.v_cache), dev(x.q)
    bt = torch.from_numpy(x.block_table).cuda()
    seq = torch.from_numpy(x.seq_lens).cuda()
    summ = torch.empty((w.layers, w.hkv, w.num_blocks, 832), dtype=torch.uint8, device="cuda")
    for layer in range(w.layers):
        L.build_summaries(d, k[layer], torch.arange(w.num_blocks, dtype=torch.int32,
                                                    device="cuda"), summ[layer])
    three = DecodeStep(d, k, v, summ, q, bt, seq, w.budget_pages, fused=False, n_tables=1)
    three.run()
    step = DecodeStep(d, k, v, summ, q, bt, seq, w.budget_pages, n_tables=1)
    step.run()
    torch.cuda.synchronize()
    assert step.sel.shape == (2, 1, 1, w.budget_pages)
    for a, r in zip((step.sel, step.cnt, step.out, step.out_lse),
                    (three.sel, three.cnt, three.out, three.out_lse)):
        assert torch.equal(a, r), "fused and three-call layer-wide steps differ"
    ref = [t.clone() for t in (step.sel, step.cnt, step.out, step.out_lse)]
    step.capture()
    for rep in range(3):
        for t in (step.sel, step.cnt, step.out, step.out_lse):
            t.zero_()
        torch.cuda.synchronize()
        step.replay()
        torch.cuda.synchronize()
        for a, r in zip((step.sel, step.cnt, step.out, step.out_lse), ref):
            assert torch.equal(a, r), f"replay {rep} differs from the eager step"
        _ = (q.float() * 2).sum().item()
    log("[tables] layer-wide step: fused == three calls; 3 graph replays identical")

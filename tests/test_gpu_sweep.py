"""Seeded sweep over combinations of the path's options on the GPU, against
the fp64 oracle.

The other parity tests vary one option at a time.  Here every case draws, from
a fixed seed, a GQA group (1, 2, 4 or 8 query heads per KV head; LOCKS
explainer, technical summary sec. 2, group-shared selection), a summary rank
(4, 8 or 16), whether the page of the newest token is pending (summarized only
after the step), a batch of ragged lengths (empty, one token, whole pages,
partial tail pages), a shuffled or contiguous block table and a budget from
one page to more pages than a sequence has.  Each case is checked at the
stated gates: page LSE within 1e-3 of fp64 on the GPU's own codes and -inf
past the summarized pages, the selected sets against the oracle's share and
top-k on the GPU's scores (identical outside the 1e-4 relative window),
sparse attention within 2e-2 of fp64 attention over the selected pages plus
the unsummarized tokens, the one-call layer bit-identical to the separate
calls, and the read-every-key page LSE within 1e-3."""

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

from tests.gpu_common import LSE_TOL, OUT_TOL, Layer, check_selection, log  # noqa: E402

N_CASES = 20


def _case(i):
    rng = np.random.default_rng([20261203, i])
    G = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2]))
    rank = int(rng.choice([4, 8, 16]))
    pending = int(rng.integers(0, 2))
    batch = int(rng.integers(1, 4))
    ctx = 16 * int(rng.integers(8, 200)) + int(rng.integers(0, 16))
    kinds = rng.choice(5, size=batch, p=[0.25, 0.25, 0.3, 0.1, 0.1])
    seqs = []
    for kd in kinds:
        if kd == 0:
            seqs.append(ctx)                                    # the longest
        elif kd == 1:
            seqs.append(16 * int(rng.integers(1, ctx // 16 + 1)))   # whole pages
        elif kd == 2:
            seqs.append(int(rng.integers(1, ctx + 1)))           # any length
        elif kd == 3:
            seqs.append(int(rng.integers(0, 2)))                 # empty or one token
        else:
            seqs.append(16)                                      # one full page
    budget = int(rng.choice([1, 2, int(rng.integers(3, 40)), ctx // 16 + 3]))
    shuffled = bool(rng.integers(0, 2))
    return dict(G=G, hkv=hkv, rank=rank, pending=pending, ctx=ctx, seqs=seqs, budget=budget,
                shuffled=shuffled)


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep_against_oracle(i):
    c = _case(i)
    G, hkv, r, pend, budget = c["G"], c["hkv"], c["rank"], c["pending"], c["budget"]
    w = get_workload("tiny-4k", hq=G * hkv, hkv=hkv, batch=len(c["seqs"]), ctx=c["ctx"],
                     budget_tokens=16 * budget, shuffled_blocks=c["shuffled"], seed=100 + i)
    x = generate(w, seq_lens=c["seqs"])
    log(f"[sweep {i}] G={G} hkv={hkv} rank={r} pending={pend} budget={budget} "
        f"shuffled={c['shuffled']} lengths={list(map(int, x.seq_lens))}")
    lay = Layer(x, 0, rank=r)
    lay.gpu_build()
    lay.d = L.dims(w.hq, w.hkv, rank=r, newest_page_pending=bool(pend))
    P = lay.bt.shape[1]

    lse = lay.score()
    sel, cnt, _ = lay.score_select(budget, with_lse=False)
    out, olse = lay.attend(sel, cnt, budget)
    ws = L.workspace(lay.d, w.batch, P, budget)
    sel1, cnt1 = torch.full_like(sel, -7), torch.full_like(cnt, -7)
    out1, olse1 = torch.empty_like(out), torch.empty_like(olse)
    L.decode_layer(lay.d, lay.q, lay.summ, lay.k, lay.v, lay.bt, lay.seq, budget, sel1, cnt1,
                   out1, ws, out_lse=olse1)
    ex = torch.full((w.batch, w.hq, P), float("nan"), dtype=torch.float32, device="cuda")
    L.exact_page_lse(lay.d, lay.q, lay.k, lay.bt, lay.seq, ex)
    torch.cuda.synchronize()
    assert torch.equal(sel1, sel) and torch.equal(cnt1, cnt), "one-call layer selection differs"
    assert torch.equal(out1, out) and torch.equal(olse1, olse), "one-call layer output differs"

    recs = lay.summ.cpu().numpy()
    worst = dict(lse=0.0, out=0.0, exact=0.0)
    for b in range(w.batch):
        s = int(x.seq_lens[b])
        n = O.summarized_pages(s, pend)
        assert torch.all(torch.isneginf(lse[b, :, n:])), f"unsummarized page scored (b={b})"
        assert torch.all(torch.isneginf(ex[b, :, n:])), f"unsummarized page scored exactly (b={b})"
        for g in range(w.hkv):
            q = O.bf16_to_f64(x.q[0, b, g * G:(g + 1) * G])
            k = int(cnt[b, g])
            assert k == min(budget, n), (k, budget, n)
            got = sel[b, g, :k].cpu().numpy()
            if n:
                s_gpu = lse[b, g * G:(g + 1) * G, :n].double().cpu().numpy()
                s_ref = O.score_records(q, recs[g, x.block_table[b, :n]], r=r)
                e = float(np.abs(s_gpu - s_ref).max())
                worst["lse"] = max(worst["lse"], e)
                assert e <= LSE_TOL, f"page LSE off by {e} (b={b}, g={g})"
                _, log_m, _ = O.group_mass(s_gpu)
                check_selection(got, log_m, budget)
                K = O.bf16_to_f64(x.k_cache[0][x.block_table[b, :n], g])
                want = O.page_lse_exact(q[None], K)
                ee = float(np.abs(ex[b, g * G:(g + 1) * G, :n].double().cpu().numpy()
                                  - want.T).max())
                worst["exact"] = max(worst["exact"], ee)
                assert ee <= LSE_TOL, f"exact page LSE off by {ee} (b={b}, g={g})"
            if s == 0:
                continue
            o_ref, l_ref = O.sparse_attention(q, x.k_cache[0], x.v_cache[0], x.block_table[b], g,
                                              got, s, pending=pend)
            e = float(np.abs(out[b, g * G:(g + 1) * G].float().cpu().numpy() - o_ref).max())
            worst["out"] = max(worst["out"], e)
            assert e <= OUT_TOL, f"attention output off by {e} (b={b}, g={g})"
            assert np.abs(olse[b, g * G:(g + 1) * G].cpu().numpy() - l_ref).max() <= LSE_TOL
    log(f"[sweep {i}] max|dLSE|={worst['lse']:.2e} exact {worst['exact']:.2e} "
        f"max|dOut|={worst['out']:.2e}")

"""The newest page pending (locks_dims.newest_page_pending = 1) on the GPU
against the fp64 oracle.

With the flag set, the page that holds a sequence's newest token is not
summarized yet, even when it is full: the summarized pages of n tokens are the
first (n - 1) // 16, and the 1 to 16 tokens after them are attended in full
(the decode step whose completed pages are summarized after it, off its
critical path; LOCKS explainer, technical summary sec. 2, implementation).
Every call that scores, selects or attends must read the flag the same way:

  * page LSE on the GPU's own codes within 1e-3 of fp64, and -inf from the
    pending page on;
  * selected sets against the oracle's share + top-k on the GPU's scores
    (1e-4 relative window), never holding the pending page;
  * sparse and dense attention within 2e-2 of fp64 attention over the same
    pages plus the pending page's tokens;
  * the one-call layer bit-identical to the separate calls;
  * the read-every-key page LSE within 1e-3, -inf from the pending page on;
  * sequences whose length is not a multiple of 16 bit-identical to the
    calls without the flag (the flag changes nothing for them)."""

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

CASES = {
    # ragged, shuffled blocks: full pages, a partial tail, one token, an
    # empty sequence and a full table
    "tiny-ragged": ("tiny-4k", dict(batch=6, shuffled_blocks=True),
                    [16 * 37, 16 * 37 + 5, 16, 1, 0, 16 * 256]),
    # 32K context (a whole number of pages), eight KV heads
    "32k": ("llama8b-32k", {}, None),
}


def _pending_dims(w):
    return L.dims(w.hq, w.hkv, newest_page_pending=True)


@pytest.mark.parametrize("case", list(CASES))
def test_pending_page_against_oracle(case):
    name, over, seqs = CASES[case]
    w = get_workload(name, **over)
    x = generate(w, seq_lens=seqs)
    log(f"[pending {case}] batch {w.batch}, lengths {list(x.seq_lens)[:8]}")
    lay = Layer(x, 0)
    lay.gpu_build()
    d0 = lay.d
    lay.d = _pending_dims(w)
    budget = w.budget_pages
    lse = lay.score()
    sel, cnt, lse2 = lay.score_select(budget)
    out, olse = lay.attend(sel, cnt, budget)
    dout, dolse = lay.attend(None, None, budget, dense=True)
    P = lay.bt.shape[1]
    ws = L.workspace(lay.d, w.batch, P, budget)
    sel1, cnt1 = torch.full_like(sel, -7), torch.full_like(cnt, -7)
    out1, olse1 = torch.empty_like(out), torch.empty_like(olse)
    L.decode_layer(lay.d, lay.q, lay.summ, lay.k, lay.v, lay.bt, lay.seq, budget, sel1, cnt1,
                   out1, ws, out_lse=olse1)
    ex = torch.full((w.batch, w.hq, P), float("nan"), dtype=torch.float32, device="cuda")
    L.exact_page_lse(lay.d, lay.q, lay.k, lay.bt, lay.seq, ex)
    torch.cuda.synchronize()
    assert torch.equal(lse, lse2)
    assert torch.equal(sel1, sel) and torch.equal(cnt1, cnt), "one-call layer selection differs"
    assert torch.equal(out1, out) and torch.equal(olse1, olse), "one-call layer output differs"
    recs = lay.summ.cpu().numpy()
    G = w.group
    worst = dict(lse=0.0, out=0.0, dense=0.0, exact=0.0)
    for b in range(w.batch):
        s = int(x.seq_lens[b])
        n = O.summarized_pages(s, 1)
        assert torch.all(torch.isneginf(lse[b, :, n:])), f"pending page scored (b={b})"
        assert torch.all(torch.isneginf(ex[b, :, n:])), f"pending page scored exactly (b={b})"
        for g in range(w.hkv):
            q = O.bf16_to_f64(x.q[0, b, g * G:(g + 1) * G])
            c = int(cnt[b, g])
            assert c == min(budget, n)
            got = sel[b, g, :c].cpu().numpy()
            if n:
                s_gpu = lse[b, g * G:(g + 1) * G, :n].double().cpu().numpy()
                s_ref = O.score_records(q, recs[g, x.block_table[b, :n]])
                e = float(np.abs(s_gpu - s_ref).max())
                worst["lse"] = max(worst["lse"], e)
                assert e <= LSE_TOL, f"page LSE off by {e} (b={b}, g={g})"
                _, log_m, _ = O.group_mass(s_gpu)
                check_selection(got, log_m, budget)
                if g < 2:
                    K = O.bf16_to_f64(x.k_cache[0][x.block_table[b, :n], g])
                    want = O.page_lse_exact(q[None], K)
                    ee = float(np.abs(ex[b, g * G:(g + 1) * G, :n].double().cpu().numpy()
                                      - want.T).max())
                    worst["exact"] = max(worst["exact"], ee)
                    assert ee <= LSE_TOL, f"exact page LSE off by {ee} (b={b}, g={g})"
            if s == 0:
                continue
            o_ref, l_ref = O.sparse_attention(q, x.k_cache[0], x.v_cache[0], x.block_table[b], g,
                                              got, s, pending=1)
            e = float(np.abs(out[b, g * G:(g + 1) * G].float().cpu().numpy() - o_ref).max())
            worst["out"] = max(worst["out"], e)
            assert e <= OUT_TOL, f"attention output off by {e} (b={b}, g={g})"
            assert np.abs(olse[b, g * G:(g + 1) * G].cpu().numpy() - l_ref).max() <= LSE_TOL
            if g < 2:
                o_d, l_d = O.sparse_attention(q, x.k_cache[0], x.v_cache[0], x.block_table[b], g,
                                              np.arange(n), s, pending=1)
                e = float(np.abs(dout[b, g * G:(g + 1) * G].float().cpu().numpy() - o_d).max())
                worst["dense"] = max(worst["dense"], e)
                assert e <= OUT_TOL, f"dense output off by {e} (b={b}, g={g})"
                assert np.abs(dolse[b, g * G:(g + 1) * G].cpu().numpy() - l_d).max() <= LSE_TOL
    # lengths that are not a multiple of 16: the flag changes nothing
    lay.d = d0
    sel0, cnt0, lse0 = lay.score_select(budget)
    out0, olse0 = lay.attend(sel0, cnt0, budget)
    torch.cuda.synchronize()
    for b in range(w.batch):
        if int(x.seq_lens[b]) % 16:
            assert torch.equal(lse0[b], lse2[b]) and torch.equal(sel0[b], sel[b])
            assert torch.equal(out0[b], out[b]) and torch.equal(olse0[b], olse[b])
    log(f"[pending {case}] max|dLSE|={worst['lse']:.2e} exact {worst['exact']:.2e} "
        f"max|dOut|={worst['out']:.2e} dense {worst['dense']:.2e}")

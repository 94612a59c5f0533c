"""GPU parity of every step of the LOCKS decode path against the fp64 oracle,
through the C ABI, on seeded synthetic inputs.

Tolerances (stated targets): page LSE 1e-3 absolute on the same codes;
selected sets identical except pages within 1e-4 (relative) of the k-th
mass, indices bit-exact when untied; sparse output 2e-2 max-abs; summary
codes within 1 LSB after the sign convention, scales within 1 fp16 ulp,
with near-degenerate eigenpairs exempted (their reconstruction compared
instead)."""

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
from tests.gpu_common import (LSE_TOL, OUT_TOL, Layer, check_selection,  # noqa: E402
                              compare_build_codes, log, oracle_scores, scores_of)

_CACHE = {}


def gen(name, **kw):
    key = (name, tuple(sorted((k, tuple(v) if isinstance(v, list) else v) for k, v in kw.items())))
    if key not in _CACHE:
        seq = kw.pop("seq_lens", None)
        w = get_workload(name, **kw)
        _CACHE[key] = generate(w, seq_lens=seq)
    return _CACHE[key]


def run_and_check(x, budget=None, gpu_records=False, check_build=False):
    w = x.w
    budget = w.budget_pages if budget is None else budget
    lay = Layer(x, 0)
    if gpu_records:
        lay.gpu_build()
        torch.cuda.synchronize()
        recs = lay.summ.cpu().numpy()
    else:
        recs = lay.upload_oracle_records()
    lse = lay.score()
    sel, cnt, lse2 = lay.score_select(budget)
    out, olse = lay.attend(sel, cnt, budget)
    sel_sa, cnt_sa = lay.select(lse, budget)
    torch.cuda.synchronize()
    assert torch.equal(lse, lse2), "score_pages and score_select disagree on page LSE"
    worst_lse, worst_out, ties = 0.0, 0.0, 0
    for b in range(w.batch):
        n = int(x.seq_lens[b]) // 16
        for g in range(w.hkv):
            G = w.group
            if n:
                s_gpu = scores_of(x, 0, b, g, lse)
                s_ref = oracle_scores(x, recs, 0, b, g)
                err = np.abs(s_gpu - s_ref).max()
                worst_lse = max(worst_lse, err)
                assert err <= LSE_TOL, f"page LSE off by {err} (b={b}, g={g})"
                tail = lse[b, g * G:(g + 1) * G, n:]
                assert torch.all(torch.isneginf(tail)), "non-finalized pages must score -inf"
                _, log_m, _ = O.group_mass(s_gpu)
            else:
                log_m = np.zeros(0)
            c = int(cnt[b, g])
            got = sel[b, g, :c].cpu().numpy()
            assert torch.all(sel[b, g, c:] == -1)
            ties += check_selection(got, log_m, budget)
            assert torch.equal(sel[b, g], sel_sa[b, g]) and int(cnt_sa[b, g]) == c
            q = O.bf16_to_f64(x.q[0, b, g * G:(g + 1) * G])
            o_ref, l_ref = O.sparse_attention(q, x.k_cache[0], x.v_cache[0], x.block_table[b], g,
                                              got, int(x.seq_lens[b]))
            o_gpu = out[b, g * G:(g + 1) * G].float().cpu().numpy()
            if o_ref.shape[0] and np.isfinite(l_ref).all():
                e = np.abs(o_gpu - o_ref).max()
                worst_out = max(worst_out, e)
                assert e <= OUT_TOL, f"attention output off by {e}"
                assert np.abs(olse[b, g * G:(g + 1) * G].cpu().numpy() - l_ref).max() <= LSE_TOL
    log(f"[{w.name} b={w.batch} budget={budget}] max|dLSE|={worst_lse:.2e} "
        f"max|dOut|={worst_out:.2e} tie-window pages={ties}")
    return lay, recs


@pytest.mark.parametrize("name", ["tiny-4k", "llama8b-32k"])
def test_pipeline_on_oracle_records(name):
    run_and_check(gen(name))


@pytest.mark.parametrize("name", ["tiny-4k", "llama8b-32k"])
def test_pipeline_on_gpu_records(name):
    run_and_check(gen(name), gpu_records=True)


def test_ragged_batch_tail_pages_and_shuffled_blocks():
    x = gen("tiny-4k", batch=3, shuffled_blocks=True, seq_lens=[4096 - 5, 16 * 37 + 9, 7])
    run_and_check(x, budget=32)


@pytest.mark.parametrize("budget", [1, 3, 255, 256, 1000])
def test_budget_edges(budget):
    run_and_check(gen("tiny-4k"), budget=budget)


def test_dense_attention_matches_oracle():
    x = gen("tiny-4k", seq_lens=[4096 - 3])
    lay = Layer(x, 0)
    out, olse = lay.attend(None, None, 0, dense=True)
    torch.cuda.synchronize()
    q = O.bf16_to_f64(x.q[0, 0])
    o_ref, l_ref = O.sparse_attention(q, x.k_cache[0], x.v_cache[0], x.block_table[0], 0,
                                      list(range((4096 - 3) // 16)), 4096 - 3)
    assert np.abs(out[0].float().cpu().numpy() - o_ref).max() <= OUT_TOL
    assert np.abs(olse[0].cpu().numpy() - l_ref).max() <= 1e-3


def test_dense_attention_long_splits():
    """A block table wide enough that a split spans more than 64 pages (the
    page list is walked in chunks of 64): dense attention over a short
    sequence in such a table still matches the oracle."""
    x = gen("tiny-4k", seq_lens=[16 * 150 + 5])
    lay = Layer(x, 0)
    wide = np.full((1, 2560 * 68), -1, dtype=np.int32)
    wide[0, :x.block_table.shape[1]] = x.block_table[0]
    lay.bt = torch.from_numpy(wide).cuda()
    out, olse = lay.attend(None, None, 0, dense=True)
    torch.cuda.synchronize()
    q = O.bf16_to_f64(x.q[0, 0])
    o_ref, l_ref = O.sparse_attention(q, x.k_cache[0], x.v_cache[0], x.block_table[0], 0,
                                      list(range(150)), 16 * 150 + 5)
    e = np.abs(out[0].float().cpu().numpy() - o_ref).max()
    log(f"[dense, 2560 x 68 table] max|dOut|={e:.2e}")
    assert e <= OUT_TOL
    assert np.abs(olse[0].cpu().numpy() - l_ref).max() <= 1e-3


def test_full_budget_equals_dense_on_gpu():
    x = gen("tiny-4k")
    lay = Layer(x, 0)
    lay.upload_oracle_records()
    sel, cnt, _ = lay.score_select(10 ** 4)
    o1, l1 = lay.attend(sel, cnt, 10 ** 4)
    o2, l2 = lay.attend(None, None, 0, dense=True)
    torch.cuda.synchronize()
    assert int(cnt[0, 0]) == 256
    assert torch.equal(sel[0, 0, :256].cpu(), torch.arange(256, dtype=torch.int32))
    assert (o1.float() - o2.float()).abs().max().item() <= 1e-2
    assert (l1 - l2).abs().max().item() <= 1e-4


def test_invalid_block_ids_are_absent():
    x = gen("tiny-4k")
    lay = Layer(x, 0)
    lay.upload_oracle_records()
    bt = lay.bt.clone()
    bt[0, 5] = -1
    bt[0, 9] = lay.nb + 3
    lay.bt = bt
    lse = lay.score()
    sel, cnt, _ = lay.score_select(32)
    out, _ = lay.attend(sel, cnt, 32)
    torch.cuda.synchronize()
    assert torch.isneginf(lse[0, :, 5]).all() and torch.isneginf(lse[0, :, 9]).all()
    s = set(sel[0, 0, :int(cnt[0, 0])].tolist())
    assert 5 not in s and 9 not in s and int(cnt[0, 0]) == 32
    assert torch.isfinite(out.float()).all()


def test_short_sequences_without_finalized_pages():
    x = gen("tiny-4k", batch=2, seq_lens=[0, 11])
    lay = Layer(x, 0)
    lay.upload_oracle_records()
    sel, cnt, lse = lay.score_select(32)
    out, olse = lay.attend(sel, cnt, 32)
    torch.cuda.synchronize()
    assert int(cnt[0, 0]) == 0 and int(cnt[1, 0]) == 0
    assert torch.isneginf(olse[0]).all() and torch.all(out[0].float() == 0)
    q = O.bf16_to_f64(x.q[0, 1])
    o_ref, l_ref = O.sparse_attention(q, x.k_cache[0], x.v_cache[0], x.block_table[1], 0, [], 11)
    assert np.abs(out[1].float().cpu().numpy() - o_ref).max() <= OUT_TOL


# ---------------------------------------------------------------------------
# summary builder codes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny-4k", "llama8b-32k"])
def test_builder_codes(name):
    x = gen(name)
    w = x.w
    lay = Layer(x, 0)
    raw = lay.gpu_build(raw=True)
    torch.cuda.synchronize()
    recs = lay.summ.cpu().numpy()
    raw = raw.cpu().numpy()
    n_cols = n_ex = 0
    worst_rec = 0.0
    for g in range(w.hkv):
        blk = x.block_table[0, :w.pages]
        K = O.bf16_to_f64(x.k_cache[0][blk, g])
        c, e, r = compare_build_codes(K, recs[g, blk], where=f"{name} g={g}")
        n_cols, n_ex, worst_rec = n_cols + c, n_ex + e, max(worst_rec, r)
        # unquantized debug output reproduces the centroid
        mu = K.mean(axis=1)
        rmu = raw[blk, g, :128]
        assert np.abs(rmu - mu).max() <= 1e-5 * (1 + np.abs(mu).max())
    log(f"[{name}] builder: {n_ex}/{n_cols} columns exempt, worst exempt-page residual excess {worst_rec:.2f} e_q")
    assert n_ex <= 0.02 * n_cols


def test_builder_record_does_not_depend_on_the_call():
    """A page-head's record is the same whatever else the call summarizes:
    the blocks in another order, one block per call, short lists of 2, 3, 5
    and 7 blocks, and a list with duplicates and out-of-range ids (skipped)
    all give the bytes of one call over every block.  The builder solves
    several pages per wave; this holds only if each page's eigensolve stops
    where that page converges, not where its neighbours do."""
    x = gen("llama8b-32k")
    lay = Layer(x, 0)
    lay.gpu_build()
    ref = lay.summ.clone()
    nb = lay.nb
    rng = np.random.default_rng(11)

    def build(ids):
        summ = torch.zeros_like(ref)
        L.build_summaries(lay.d, lay.k, torch.tensor(ids, dtype=torch.int32, device="cuda"), summ)
        return summ

    perm = rng.permutation(nb)
    got = build(perm.tolist())
    assert torch.equal(got, ref), "records differ when the blocks come in another order"
    picks = rng.choice(nb, 24, replace=False).tolist()
    summ = torch.zeros_like(ref)
    for b in picks:
        L.build_summaries(lay.d, lay.k, torch.tensor([b], dtype=torch.int32, device="cuda"), summ)
    for n in (2, 3, 5, 7):
        ids = rng.choice(nb, n, replace=False).tolist()
        picks += ids
        L.build_summaries(lay.d, lay.k, torch.tensor(ids, dtype=torch.int32, device="cuda"), summ)
    mixed = [-1, picks[0], nb, picks[1], picks[1], 10**6, picks[2], -5, picks[0]]
    summ2 = build(mixed)
    torch.cuda.synchronize()
    sel = torch.tensor(sorted(set(picks)), dtype=torch.long, device="cuda")
    assert torch.equal(summ[:, sel], ref[:, sel]), "records differ in calls of 1 to 7 blocks"
    m = torch.tensor(sorted(set(picks[:3])), dtype=torch.long, device="cuda")
    assert torch.equal(summ2[:, m], ref[:, m]), "records differ with duplicates and skipped ids"
    untouched = torch.ones(nb, dtype=torch.bool, device="cuda")
    untouched[m] = False
    assert int(summ2[:, untouched].abs().sum()) == 0, "a skipped id wrote a record"
    log(f"[builder] records identical across {len(set(picks))} blocks in calls of 1-7 blocks, "
        f"a permuted call and a call with duplicates and out-of-range ids")


def test_builder_exact_low_rank_pages():
    """Pages whose keys vary in only 5 coordinates: the GPU's unquantized
    summary reproduces the keys exactly (up to fp32), and the record's
    estimate matches the exact page LSE to quantization accuracy."""
    w = get_workload("tiny-4k")
    x = generate(w)
    rng = np.random.default_rng(3)
    from synth.host import f32_to_bf16_bits
    nb = w.num_blocks
    k = np.zeros((nb, 1, 16, 128))
    for p in range(nb):
        mu = rng.standard_normal(128)
        kk = np.tile(mu, (16, 1))
        coords = rng.choice(128, 5, replace=False)
        kk[:, coords] += rng.standard_normal((16, 5)) * 2
        k[p, 0] = kk
    x.k_cache[0] = f32_to_bf16_bits(k)
    lay = Layer(x, 0)
    raw = lay.gpu_build(raw=True)
    torch.cuda.synchronize()
    raw = raw.cpu().numpy()
    K = O.bf16_to_f64(x.k_cache[0][:, 0])
    mu, V, C = raw[:, 0, :128], raw[:, 0, 128:1152].reshape(-1, 8, 128), raw[:, 0, 1152:].reshape(-1, 16, 8)
    recon = mu[:, None, :] + C @ V
    assert np.abs(recon - K).max() <= 2e-4 * np.abs(K).max()
    assert np.all(np.abs(V[:, 5:]) == 0)


# ---------------------------------------------------------------------------
# exact ties: selection must keep the lowest page indices
# ---------------------------------------------------------------------------

def test_zero_query_all_ties_select_first_pages():
    x = gen("llama8b-32k")
    lay = Layer(x, 0)
    lay.upload_oracle_records()
    lay.q.zero_()
    sel, cnt, lse = lay.score_select(128)
    torch.cuda.synchronize()
    n = x.w.pages
    assert torch.allclose(lse[0, :, :n], torch.full_like(lse[0, :, :n], float(np.log(16.0))), atol=1e-6)
    for g in range(x.w.hkv):
        assert int(cnt[0, g]) == 128
        assert torch.equal(sel[0, g].cpu(), torch.arange(128, dtype=torch.int32))


def test_repeated_pages_exact_ties():
    """Pages repeat with period 7, so scores tie exactly in groups; the GPU must
    pick exactly the oracle's pages (lowest index among equal masses)."""
    x = gen("tiny-4k")
    x2 = generate(x.w)
    blk = x2.block_table[0]
    for j in range(x.w.pages):
        x2.k_cache[0][blk[j]] = x2.k_cache[0][blk[j % 7]]
    lay = Layer(x2, 0)
    lay.upload_oracle_records()
    for budget in (1, 5, 32, 100):
        sel, cnt, lse = lay.score_select(budget)
        torch.cuda.synchronize()
        s_gpu = scores_of(x2, 0, 0, 0, lse)
        _, log_m, _ = O.group_mass(s_gpu)
        want = O.select_top_pages(log_m, budget)
        got = sel[0, 0, :int(cnt[0, 0])].cpu().numpy()
        assert list(got) == list(want), (budget, got[:10], want[:10])


@pytest.mark.parametrize("ctx,budget", [(16 * 8192, 600), (16 * 12000 + 7, 2000),
                                        (16 * 40000 + 3, 2048)])
def test_long_candidate_lists(ctx, budget):
    """Selection merge paths with about 5, 12 and 40 candidates per thread
    (the last one re-reads its candidates from memory in every pass)."""
    x = gen("tiny-4k", ctx=ctx, carriers=8)
    run_and_check(x, budget=budget, gpu_records=True)


# ---------------------------------------------------------------------------
# one-call layer step: identical to score_select + sparse_attend
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,kw,budget", [
    ("tiny-4k", {}, 32),
    ("tiny-4k", {}, 1),
    ("tiny-4k", {"batch": 3, "shuffled_blocks": True,
                 "seq_lens": [4096 - 5, 16 * 37 + 9, 7]}, 32),
    ("llama8b-32k", {}, 128),
    ("tiny-4k", {"ctx": 16 * 8192, "carriers": 8}, 128),     # 4 chunks x 128 candidates
    ("tiny-4k", {"ctx": 16 * 8192, "carriers": 8}, 1000),    # budget near the fused limit
    ("tiny-4k", {"ctx": 16 * 16384, "carriers": 8}, 600),    # 4800 candidates, 1024 selectors
    ("tiny-4k", {"ctx": 16 * 12000 + 7, "carriers": 8}, 2000),   # budget above it: two calls
    ("tiny-4k", {"ctx": 16 * 40000 + 3, "carriers": 8}, 512),    # 40960 candidates: two calls
])
def test_decode_layer_equals_two_calls(name, kw, budget):
    from kv_cache_page_int4_amd import locks as L
    x = gen(name, **kw)
    w = x.w
    lay = Layer(x, 0)
    lay.gpu_build()
    sel_a, cnt_a, _ = lay.score_select(budget, with_lse=False)
    out_a, olse_a = lay.attend(sel_a, cnt_a, budget)
    P = lay.bt.shape[1]
    sel_b = torch.full_like(sel_a, -7)
    cnt_b = torch.full_like(cnt_a, -7)
    out_b = torch.empty_like(out_a)
    olse_b = torch.empty_like(olse_a)
    ws = torch.empty(L.score_workspace_bytes(lay.d, w.batch, P, budget), dtype=torch.uint8,
                     device="cuda")
    wa = L.attend_workspace(lay.d, w.batch, budget + 1)
    L.decode_layer(lay.d, lay.q, lay.summ, lay.k, lay.v, lay.bt, lay.seq, budget, sel_b, cnt_b,
                   out_b, ws, wa, out_lse=olse_b)
    torch.cuda.synchronize()
    assert torch.equal(sel_a, sel_b) and torch.equal(cnt_a, cnt_b), "selection differs"
    assert torch.equal(out_a, out_b), "attention output differs"
    assert torch.equal(olse_a, olse_b), "attention LSE differs"
    log(f"[decode_layer {name} b={w.batch} budget={budget}] identical to the two calls")

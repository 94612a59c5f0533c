"""GPU parity at summary ranks 4 and 16 (the same method at other state
sizes; rank 8 is covered everywhere else), through the C ABI:
  * builder codes against the oracle's rank-r build of the same keys (codes
    within 1 LSB, scales within 1 fp16 ulp, near-degenerate columns compared
    by reconstruction);
  * page LSE against fp64 on the GPU's own records (1e-3), the selected set
    against the oracle's (1e-4 relative window) and the sparse output (2e-2);
  * the one-call layer equal to the separate calls, and incremental
    finalization equal to a direct build;
  * the shared-basis build at rank 4 against the oracle's in the same basis."""

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
                              compare_build_codes, log)

_CACHE = {}


def gen(name, seq_lens=None, **kw):
    key = (name, None if seq_lens is None else tuple(seq_lens), tuple(sorted(kw.items())))
    if key not in _CACHE:
        _CACHE[key] = generate(get_workload(name, **kw), seq_lens=seq_lens)
    return _CACHE[key]


CASES = [("tiny-4k", {}, None, False),
         ("llama8b-32k", {"batch": 2}, [32768 - 5, 16 * 700 + 3], False),
         ("tiny-4k", {}, None, True)]        # the newest (full) page pending


@pytest.mark.parametrize("rank", [4, 16])
@pytest.mark.parametrize("name,kw,seq,pending", CASES)
def test_rank_pipeline(rank, name, kw, seq, pending):
    x = gen(name, seq_lens=seq, **kw)
    w = x.w
    lay = Layer(x, 0, rank=rank)
    assert lay.summ.shape[-1] == L.summary_bytes(lay.d) == O.record_bytes(rank)
    lay.gpu_build()
    torch.cuda.synchronize()
    recs = lay.summ.cpu().numpy()
    # builder codes on sampled page-heads
    rng = np.random.default_rng(rank)
    n0 = int(x.seq_lens[0]) // 16
    pick = np.sort(rng.choice(n0, min(n0, 96), replace=False))
    blk = x.block_table[0, pick]
    n_cols = n_ex = 0
    for g in range(w.hkv):
        K = O.bf16_to_f64(x.k_cache[0][blk, g])
        c, e, _ = compare_build_codes(K, recs[g, blk], where=f"rank {rank} g={g}", r=rank)
        n_cols, n_ex = n_cols + c, n_ex + e
    assert n_ex <= 0.05 * n_cols, (n_ex, n_cols)
    # score, select, attend
    lay.d = L.dims(w.hq, w.hkv, rank=rank, newest_page_pending=pending)
    budget = w.budget_pages
    sel, cnt, lse = lay.score_select(budget)
    out, olse = lay.attend(sel, cnt, budget)
    torch.cuda.synchronize()
    G = w.group
    worst_lse = worst_out = 0.0
    ties = 0
    for b in range(w.batch):
        n = O.summarized_pages(int(x.seq_lens[b]), int(pending))
        assert torch.all(torch.isneginf(lse[b, :, n:]))
        for g in range(w.hkv):
            s_gpu = lse[b, g * G:(g + 1) * G, :n].double().cpu().numpy()
            s_ref = O.score_records(O.bf16_to_f64(x.q[0, b, g * G:(g + 1) * G]),
                                    recs[g, x.block_table[b, :n]], r=rank)
            err = float(np.abs(s_gpu - s_ref).max())
            worst_lse = max(worst_lse, err)
            assert err <= LSE_TOL, f"page LSE off by {err} (rank {rank}, b={b}, g={g})"
            _, log_m, _ = O.group_mass(s_gpu)
            c = int(cnt[b, g])
            got = sel[b, g, :c].cpu().numpy()
            ties += check_selection(got, log_m, budget)
            q = O.bf16_to_f64(x.q[0, b, g * G:(g + 1) * G])
            o_ref, l_ref = O.sparse_attention(q, x.k_cache[0], x.v_cache[0], x.block_table[b], g,
                                              got, int(x.seq_lens[b]), pending=int(pending))
            e = float(np.abs(out[b, g * G:(g + 1) * G].float().cpu().numpy() - o_ref).max())
            worst_out = max(worst_out, e)
            assert e <= OUT_TOL
    # the one-call layer equals the separate calls
    P = lay.bt.shape[1]
    sel2 = torch.full_like(sel, -7)
    cnt2 = torch.full_like(cnt, -7)
    out2 = torch.empty_like(out)
    olse2 = torch.empty_like(olse)
    ws = torch.empty(L.score_workspace_bytes(lay.d, w.batch, P, budget), dtype=torch.uint8,
                     device="cuda")
    L.decode_layer(lay.d, lay.q, lay.summ, lay.k, lay.v, lay.bt, lay.seq, budget, sel2, cnt2,
                   out2, ws, L.attend_workspace(lay.d, w.batch, budget + 1), out_lse=olse2)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel2) and torch.equal(cnt, cnt2) and torch.equal(out, out2)
    log(f"[rank {rank} {name} pending={pending}] codes exempt {n_ex}/{n_cols}; max|dLSE|={worst_lse:.2e} "
        f"max|dOut|={worst_out:.2e} tie-window pages={ties}")


@pytest.mark.parametrize("rank", [4, 16])
def test_rank_finalize_equals_direct_build(rank):
    x = gen("tiny-4k", batch=3, shuffled_blocks=True, seq_lens=[16 * 100, 16 * 37 + 9, 16 * 5])
    w = x.w
    lay = Layer(x, 0, rank=rank)
    lay.gpu_build()
    direct = lay.summ.clone()
    lay.summ.zero_()
    L.finalize_pages(lay.d, lay.k, lay.bt, lay.seq, lay.summ)
    torch.cuda.synchronize()
    for b, sl in enumerate(x.seq_lens):
        sl = int(sl)
        if sl % 16 == 0 and sl > 0:
            blk = int(x.block_table[b, sl // 16 - 1])
            assert torch.equal(lay.summ[:, blk], direct[:, blk]), f"rank {rank}, sequence {b}"
        else:
            assert int(lay.summ[:, int(x.block_table[b, sl // 16 - 1])].abs().sum()) == 0


def test_rank4_shared_basis_records():
    x = gen("llama8b-32k")
    w = x.w
    lay = Layer(x, 0, rank=4)
    n = int(x.seq_lens[0]) // 16
    blocks = x.block_table[0, :n]
    bl = torch.from_numpy(blocks.astype(np.int32)).cuda()
    basis = torch.empty((w.hkv, 4, 128), dtype=torch.float32, device="cuda")
    ev = torch.empty((w.hkv, 128), dtype=torch.float32, device="cuda")
    L.shared_basis(lay.d, lay.k, bl, basis, eigvals=ev)
    L.build_summaries_basis(lay.d, lay.k, bl, basis, lay.summ)
    torch.cuda.synchronize()
    recs = lay.summ.cpu().numpy()
    Vg = basis.double().cpu().numpy()
    evg = ev.double().cpu().numpy()
    pick = np.sort(np.random.default_rng(9).choice(n, 128, replace=False))
    for g in range(w.hkv):
        K = O.bf16_to_f64(x.k_cache[0][blocks, g])
        S = O.pooled_scatter(K)
        B = Vg[g].T
        for k in range(4):
            res = np.linalg.norm(S @ B[:, k] - evg[g, k] * B[:, k]) / evg[g, 0]
            assert res <= 1e-3, res
        want, _ = O.build_records_with_basis(K[pick], B)
        a = O.unpack_records(recs[g, blocks[pick]], r=4)
        b = O.unpack_records(want, r=4)
        for key in ("mu_q", "v_q", "c_q"):
            assert np.abs(a[key].astype(int) - b[key].astype(int)).max() <= 1, key

"""GPU parity of the exact ("read every key") page scorer against the fp64
oracle on the same bf16 keys, and of the exact selection built from it.

Tolerances: page LSE 1e-3 absolute; selected sets identical except pages
within 1e-4 (relative) of the k-th mass, indices bit-exact when untied."""

import numpy as np
import pytest
import torch

import oracle as O
from kv_cache_page_int4_amd import locks as L
from synth import get_workload
from synth.device import generate_device
from synth.host import generate

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from tests.gpu_common import LSE_TOL, Layer, check_selection, log  # noqa: E402


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _exact(lay):
    w = lay.w
    P = lay.bt.shape[1]
    lse = torch.full((w.batch, w.hq, P), 7.0, dtype=torch.float32, device="cuda")
    L.exact_page_lse(lay.d, lay.q, lay.k, lay.bt, lay.seq, lse)
    return lse


@pytest.mark.parametrize("name,kw", [("tiny-4k", {}), ("llama8b-32k", {}),
                                     ("tiny-4k", {"batch": 3, "shuffled_blocks": True,
                                                  "seq_lens": [4096 - 5, 16 * 37 + 9, 7]})])
def test_exact_lse_and_selection(name, kw):
    kw = dict(kw)
    seq = kw.pop("seq_lens", None)
    w = get_workload(name, **kw)
    x = generate(w, seq_lens=seq)
    log(f"[exact {name} b={w.batch}]")
    lay = Layer(x, 0)
    lse = _exact(lay)
    budget = w.budget_pages
    sel, cnt = lay.select(lse, budget)
    torch.cuda.synchronize()
    G = w.group
    worst = 0.0
    ties = 0
    for b in range(w.batch):
        n = int(x.seq_lens[b]) // 16
        for g in range(w.hkv):
            tail = lse[b, g * G:(g + 1) * G, n:]
            assert torch.all(torch.isneginf(tail)), "pages that are not finalized must be -inf"
            if n == 0:
                assert int(cnt[b, g]) == 0
                continue
            q = O.bf16_to_f64(x.q[0, b, g * G:(g + 1) * G])
            K = O.bf16_to_f64(x.k_cache[0][x.block_table[b, :n], g])      # [n, 16, d]
            ref = O.page_lse_exact(q[None], K).T      # [G, n]
            got = lse[b, g * G:(g + 1) * G, :n].double().cpu().numpy()
            err = float(np.abs(got - ref).max())
            worst = max(worst, err)
            assert err <= LSE_TOL, f"exact page LSE off by {err} (b={b}, g={g})"
            _, log_m, _ = O.group_mass(got)
            c = int(cnt[b, g])
            ties += check_selection(sel[b, g, :c].cpu().numpy(), log_m, budget)
    log(f"[exact {name}] max|dLSE|={worst:.2e} tie-window pages={ties}")


def test_exact_lse_invalid_block_ids():
    x = generate(get_workload("tiny-4k"))
    lay = Layer(x, 0)
    bt = lay.bt.clone()
    bt[0, 5] = -1
    bt[0, 9] = lay.nb + 3
    lay.bt = bt
    lse = _exact(lay)
    torch.cuda.synchronize()
    assert torch.isneginf(lse[0, :, 5]).all() and torch.isneginf(lse[0, :, 9]).all()
    assert torch.isfinite(lse[0, :, :5]).all()


def test_exact_lse_full_size_sampled():
    """One layer of the 1M-context workload, sampled pages against the oracle."""
    w = get_workload("llama8b-1m")
    log("[exact llama8b-1m] one layer on the device")
    inp = generate_device(w, layers=1)
    d = L.dims(w.hq, w.hkv)
    P = inp.block_table.shape[1]
    lse = torch.empty((w.batch, w.hq, P), dtype=torch.float32, device="cuda")
    L.exact_page_lse(d, inp.q[0], inp.k[0], inp.block_table, inp.seq_lens, lse)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    bt = inp.block_table.cpu().numpy()
    G = w.group
    worst = 0.0
    for g in (0, w.hkv - 1):
        pages = np.unique(np.concatenate([rng.choice(w.pages, 256, replace=False), [0, w.pages - 1]]))
        blk = torch.from_numpy(bt[0, pages].astype(np.int64)).cuda()
        K = O.bf16_to_f64(_bits(inp.k[0].index_select(0, blk)[:, g]))
        q = O.bf16_to_f64(_bits(inp.q[0, 0, g * G:(g + 1) * G]))
        ref = O.page_lse_exact(q[None], K).T
        got = lse[0, g * G:(g + 1) * G][:, torch.from_numpy(pages).cuda()].double().cpu().numpy()
        err = float(np.abs(got - ref).max())
        worst = max(worst, err)
        assert err <= LSE_TOL, f"exact page LSE off by {err} (g={g})"
    log(f"[exact llama8b-1m] max|dLSE|={worst:.2e}")

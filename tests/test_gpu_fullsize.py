"""GPU parity at the full per-layer sizes of the large configurations, with
the same library calls and launch plans that bench.py times, checked on
sampled outputs the oracle can compute one by one:

  * page LSE of sampled pages against the fp64 oracle on the GPU's own codes;
  * the selected set of sampled (sequence, KV head) groups against the
    oracle's share + top-k on the GPU's scores (1e-4 relative window);
  * the sparse output of those groups against fp64 attention over the
    GPU's selection;
  * summary codes of sampled page-heads against the oracle's build of the
    same keys.

The outputs checked are those of a replay of the captured decode-step graph
(cleared before the replay), so the graph itself is held to the oracle.  The
first group's page LSE is checked on every page, the others' on samples.

Also here: the device input generator's recipe statistics, and the captured
decode-step graph replaying to the eager result."""

import math

import numpy as np
import pytest
import torch

import oracle as O
from kv_cache_page_int4_amd import locks as L
from kv_cache_page_int4_amd.step import DecodeStep
from synth import get_workload
from synth.device import generate_device
from synth.host import generate

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from tests.gpu_common import (LSE_TOL, OUT_TOL, check_selection, compare_build_codes,  # noqa: E402
                              log)


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _groups(w, rng):
    """A few (sequence, KV head) groups: both ends and a random one."""
    picks = {(0, 0), (w.batch - 1, w.hkv - 1),
             (int(rng.integers(w.batch)), int(rng.integers(w.hkv)))}
    return sorted(picks)


@pytest.mark.parametrize("name", ["llama8b-128k-b8", "llama8b-1m", "llama8b-256k-b16"])
def test_full_size_sampled(name):
    w = get_workload(name)
    rng = np.random.default_rng(11)
    log(f"[{name}] one layer on the device: batch {w.batch}, ctx {w.ctx}, "
        f"{w.num_blocks} blocks x {w.hkv} KV heads")
    inp = generate_device(w, layers=1)
    d = L.dims(w.hq, w.hkv)
    nb, budget = w.num_blocks, w.budget_pages
    summ = torch.empty((1, w.hkv, nb, L.summary_bytes(d)), dtype=torch.uint8, device="cuda")
    L.build_summaries(d, inp.k[0], torch.arange(nb, dtype=torch.int32, device="cuda"), summ[0])
    torch.cuda.synchronize()
    log(f"[{name}] summaries built; decode step captured in a graph (bench plans), "
        f"outputs cleared, replayed")

    step = DecodeStep(d, inp.k, inp.v, summ, inp.q, inp.block_table, inp.seq_lens, budget)
    step.capture()
    for t in (step.sel, step.cnt, step.out, step.out_lse):
        t.fill_(-3)
    torch.cuda.synchronize()
    step.replay()
    torch.cuda.synchronize()
    P = inp.block_table.shape[1]
    lse = torch.empty((w.batch, w.hq, P), dtype=torch.float32, device="cuda")
    sel2 = torch.empty_like(step.sel[0])
    cnt2 = torch.empty_like(step.cnt[0])
    L.score_select(d, inp.q[0], summ[0], nb, inp.block_table, inp.seq_lens, budget, sel2, cnt2,
                   step.ws_score, page_lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(sel2, step.sel[0]) and torch.equal(cnt2, step.cnt[0]), \
        "the replayed selection differs from an eager score_select"

    bt = inp.block_table.cpu().numpy()
    G = w.group
    worst_lse = worst_out = 0.0
    ties = n_cols = n_ex = 0
    for gi, (b, g) in enumerate(_groups(w, rng)):
        n = w.ctx // w.page
        log(f"[{name}] group b={b} kvh={g}")
        q = O.bf16_to_f64(_bits(inp.q[0, b, g * G:(g + 1) * G]))
        s_gpu = lse[b, g * G:(g + 1) * G, :n].double().cpu().numpy()
        c = int(step.cnt[0, b, g])
        got = step.sel[0, b, g, :c].cpu().numpy()

        # page LSE: every page of the first group, sampled pages (plus the
        # selected ones) of the others
        if gi == 0:
            pages = np.arange(n)
        else:
            pages = np.unique(np.concatenate([rng.choice(n, 384, replace=False), [0, n - 1],
                                              got[:64]]))
        blk = torch.from_numpy(bt[b, pages].astype(np.int64)).cuda()
        recs = summ[0, g].index_select(0, blk).cpu().numpy()
        s_ref = O.score_records(q, recs)
        err = float(np.abs(s_ref - s_gpu[:, pages]).max())
        worst_lse = max(worst_lse, err)
        assert err <= LSE_TOL, f"page LSE off by {err} (b={b}, g={g})"

        # selection from the GPU's scores
        _, log_m, _ = O.group_mass(s_gpu)
        ties += check_selection(got, log_m, budget)

        # sparse attention over the GPU's selection (ctx is a whole number of pages)
        phys = torch.from_numpy(bt[b, got].astype(np.int64)).cuda()
        ksub = _bits(inp.k[0].index_select(0, phys))
        vsub = _bits(inp.v[0].index_select(0, phys))
        row = np.zeros(bt.shape[1], dtype=np.int64)
        row[got] = np.arange(len(got))
        o_ref, l_ref = O.sparse_attention(q, ksub, vsub, row, g, got, w.ctx)
        o_gpu = step.out[0, b, g * G:(g + 1) * G].float().cpu().numpy()
        e = float(np.abs(o_gpu - o_ref).max())
        worst_out = max(worst_out, e)
        assert e <= OUT_TOL, f"attention output off by {e} (b={b}, g={g})"
        assert np.abs(step.out_lse[0, b, g * G:(g + 1) * G].cpu().numpy() - l_ref).max() <= LSE_TOL

        # summary codes of sampled page-heads
        bpages = rng.choice(n, 48, replace=False)
        bblk = torch.from_numpy(bt[b, bpages].astype(np.int64)).cuda()
        K = O.bf16_to_f64(_bits(inp.k[0].index_select(0, bblk)[:, g]))
        cc, ee, _ = compare_build_codes(K, summ[0, g].index_select(0, bblk).cpu().numpy(),
                                        where=f"{name} b={b} g={g}")
        n_cols, n_ex = n_cols + cc, n_ex + ee
    log(f"[{name}] max|dLSE|={worst_lse:.2e} max|dOut|={worst_out:.2e} "
        f"tie-window pages={ties} builder exempt {n_ex}/{n_cols}")
    assert n_ex <= 0.02 * n_cols


def test_device_generator_recipe():
    """The device generator follows the input recipe: rank-8 energy of the
    key deviations about 0.74 (variance reading), unit-variance centroids,
    values and queries, and carrier keys aligned with their query head."""
    w = get_workload("llama8b-32k")
    log("[device generator] llama8b-32k, one layer")
    inp = generate_device(w, layers=1)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    pick = torch.from_numpy(rng.choice(w.num_blocks, 256, replace=False).astype(np.int64)).cuda()
    K = O.bf16_to_f64(_bits(inp.k[0].index_select(0, pick)[:, 0]))
    lam = O.page_spectrum(K)[2]
    energy = float(O.energy_captured(lam).mean())
    assert 0.70 <= energy <= 0.78, energy
    mu = K.mean(axis=1)
    assert 0.85 <= mu.std() <= 1.15, mu.std()
    v = inp.v[0].float()
    assert abs(v.mean().item()) < 0.01 and abs(v.std().item() - 1.0) < 0.01
    q = inp.q[0].float()
    assert abs(q.std().item() - 1.0) < 0.05
    # carriers: (layer, b, g, page, slot, head)
    bt = inp.block_table.cpu().numpy()
    for (_, b, g, page, slot, head) in inp.carriers[:32]:
        key = O.bf16_to_f64(_bits(inp.k[0, int(bt[b, page]), g, slot]))
        qh = O.bf16_to_f64(_bits(inp.q[0, b, head]))
        proj = float(key @ qh / np.linalg.norm(qh))
        assert 2.0 <= proj <= 4.0, proj
    log(f"[device generator] energy {energy:.3f}, centroid std {mu.std():.3f}")


def test_decode_graph_replays_match_eager():
    """The captured step (all library calls of a layer) replays to exactly
    the eager outputs, with eager work and synchronizations between replays."""
    w = get_workload("llama8b-32k", layers=2)
    log("[graph] llama8b-32k, 2 layers")
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
    step = DecodeStep(d, k, v, summ, q, bt, seq, w.budget_pages)
    step.run()
    torch.cuda.synchronize()
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
        _ = (q.float() * 2).sum().item()   # eager work between replays
    log("[graph] 3 replays identical to the eager step")
    assert math.isfinite(float(step.out_lse.float().sum()))

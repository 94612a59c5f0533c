"""GPU parity of the shared-basis selector (the baseline the pages reject,
Proposition 1) through the C ABI.

The top-8 eigenvectors of the pooled scatter are unique only up to the order
and span of (near-)equal eigenvalues, so the checks compare what is unique and
check that the rest is valid:
  * every eigenvalue of S against the fp64 oracle's (numpy eigvalsh on the
    oracle's pooled scatter), within 2e-4 of the largest;
  * each GPU basis vector is an eigenvector of the fp64 S (residual within
    1e-3 of the largest eigenvalue), the 8 are orthonormal (1e-4), signed by
    the rule, and capture the top-8 energy;
  * records built in the GPU's basis against the oracle's build in that same
    basis: codes within 1 LSB, scales within 1 fp16 ulp;
  * page LSE of those records against the oracle (1e-3)."""

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
from tests.gpu_common import LSE_TOL, Layer, log  # noqa: E402

EIG_TOL = 2e-4      # eigenvalues, relative to the largest
RES_TOL = 1e-3      # |S v - lambda v|, relative to the largest eigenvalue
ORTH_TOL = 1e-4


def _ulp16(x):
    """fp16 spacing at |x| (normal range)."""
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -14)))
    return 2.0 ** (e - 10)


@pytest.mark.parametrize("name,kw", [("tiny-4k", {}), ("llama8b-32k", {"batch": 2}),
                                     ("tiny-4k", {"ctx": 16 * 6000 + 5})])
def test_shared_basis_against_oracle(name, kw):
    x = generate(get_workload(name, **kw))
    w = x.w
    lay = Layer(x, 0)
    # pool the finalized pages of every sequence (a block may appear once)
    blocks = np.unique(np.concatenate([x.block_table[b, :int(x.seq_lens[b]) // 16]
                                       for b in range(w.batch)]))
    bl = torch.from_numpy(blocks.astype(np.int32)).cuda()
    basis = torch.empty((w.hkv, 8, 128), dtype=torch.float32, device="cuda")
    ev = torch.empty((w.hkv, 128), dtype=torch.float32, device="cuda")
    L.shared_basis(lay.d, lay.k, bl, basis, eigvals=ev)
    torch.cuda.synchronize()
    Vg = basis.double().cpu().numpy()
    evg = ev.double().cpu().numpy()
    worst_ev = worst_res = 0.0
    for g in range(w.hkv):
        K = O.bf16_to_f64(x.k_cache[0][blocks, g])
        S = O.pooled_scatter(K)
        ref = np.linalg.eigvalsh(S)[::-1]
        lmax = ref[0]
        e = float(np.abs(evg[g] - ref).max() / lmax)
        worst_ev = max(worst_ev, e)
        assert e <= EIG_TOL, f"eigenvalues off by {e} of the largest (g={g})"
        assert np.all(np.diff(evg[g]) <= 0), "eigenvalues not descending"
        B = Vg[g].T                                            # [128, 8] columns
        assert np.abs(B.T @ B - np.eye(8)).max() <= ORTH_TOL
        for k in range(8):
            v = B[:, k]
            r = float(np.linalg.norm(S @ v - evg[g, k] * v) / lmax)
            worst_res = max(worst_res, r)
            assert r <= RES_TOL, f"basis vector {k} is no eigenvector (residual {r}, g={g})"
            t = int(np.argmax(np.abs(v)))
            assert v[t] > 0 and np.all(np.abs(v[:t]) < abs(v[t]))
        # the basis holds the top-8 energy (sum of the 8 largest eigenvalues)
        np.testing.assert_allclose(np.trace(B.T @ S @ B), ref[:8].sum(), rtol=1e-3)
    log(f"[shared basis {name} {len(blocks)} pages x {w.hkv} heads] "
        f"max|d eig|/lmax={worst_ev:.1e} max residual={worst_res:.1e}")


def test_records_in_shared_basis_against_oracle():
    x = generate(get_workload("llama8b-32k"))
    w = x.w
    lay = Layer(x, 0)
    n = int(x.seq_lens[0]) // 16
    blocks = x.block_table[0, :n]
    bl = torch.from_numpy(blocks.astype(np.int32)).cuda()
    basis = torch.empty((w.hkv, 8, 128), dtype=torch.float32, device="cuda")
    L.shared_basis(lay.d, lay.k, bl, basis)
    L.build_summaries_basis(lay.d, lay.k, bl, basis, lay.summ)
    torch.cuda.synchronize()
    recs = lay.summ.cpu().numpy()
    Vg = basis.double().cpu().numpy()
    rng = np.random.default_rng(3)
    pick = np.sort(rng.choice(n, 256, replace=False))
    for g in range(w.hkv):
        K = O.bf16_to_f64(x.k_cache[0][blocks[pick], g])
        want, _ = O.build_records_with_basis(K, Vg[g].T)
        a = O.unpack_records(recs[g, blocks[pick]])
        b = O.unpack_records(want)
        for key in ("mu_q", "v_q", "c_q"):
            d = np.abs(a[key].astype(np.int32) - b[key].astype(np.int32))
            assert d.max() <= 1, f"{key} codes differ by {d.max()} (g={g})"
        for key in ("s_mu", "s_v", "s_c"):
            assert np.all(np.abs(a[key] - b[key]) <= _ulp16(b[key]) * 1.0001), key
        # every record carries the same basis codes
        assert np.all(a["v_q"] == a["v_q"][:1]) and np.all(a["s_v"] == a["s_v"][:1])
    # the unchanged scorer on these records matches the oracle on the same codes
    lse = lay.score()
    torch.cuda.synchronize()
    G = w.group
    for g in range(w.hkv):
        q = O.bf16_to_f64(x.q[0, 0, g * G:(g + 1) * G])
        s_ref = O.score_records(q, recs[g, blocks])
        s_gpu = lse[0, g * G:(g + 1) * G, :n].double().cpu().numpy()
        assert np.abs(s_ref - s_gpu).max() <= LSE_TOL
    log("[shared basis] records within 1 LSB of the oracle's in the same basis; scores match")

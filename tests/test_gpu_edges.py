"""Branches of the builder and the scorer that ordinary inputs never take,
driven on the GPU with inputs built to take them, against the fp64 oracle:

  * the scorer's max-shifted page LSE, used when a page's 16 deviation
    exponentials sum outside [1e-30, 1e30] (pages whose key deviations are a
    few hundred times the usual size);
  * constant pages: no deviation at all, so no basis; the estimate is the
    closed form q.mu / sqrt(d) + log 16 (LOCKS explainer, technical summary
    sec. 2: the estimate with zero coefficients)."""

import math

import numpy as np
import pytest
import torch

import oracle as O
from synth import get_workload
from synth.host import bf16_bits_to_f32, f32_to_bf16_bits, generate

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from tests.gpu_common import LSE_TOL, Layer, compare_build_codes, fp16_ulp, log  # noqa: E402


def test_scorer_overflow_fallback_matches_oracle():
    w = get_workload("tiny-4k")
    x = generate(w)
    kc = x.k_cache[0]                                    # [nb, 1, 16, 128] bf16 bits
    big = np.arange(0, 256, 3)                           # every third page
    K = bf16_bits_to_f32(kc[x.block_table[0, big], 0]).astype(np.float64)
    K = (K - K.mean(axis=1, keepdims=True)) * 500.0      # centroid 0, huge deviations
    kc[x.block_table[0, big], 0] = f32_to_bf16_bits(K)
    lay = Layer(x, 0)
    lay.gpu_build()
    lse = lay.score()
    torch.cuda.synchronize()
    recs = lay.summ.cpu().numpy()
    q = O.bf16_to_f64(x.q[0, 0])
    rec_rows = recs[0, x.block_table[0, :w.pages]]
    s_ref = O.score_records(q, rec_rows)                 # [4, 256]
    s_gpu = lse[0, :, :w.pages].double().cpu().numpy()
    err = float(np.abs(s_gpu - s_ref).max())
    # the fallback is needed: deviation exponentials of some pages sum past
    # 1e30 (the centroid term is subtracted: it is added outside the sum)
    qz = O.unpack_records(rec_rows)
    mu_hat = qz["mu_q"].astype(np.float64) * qz["s_mu"][:, None]
    dev_lse = s_ref - (q @ mu_hat.T) / math.sqrt(128)
    n_over = int((dev_lse > math.log(1e30)).sum())
    log(f"[fallback] {n_over} (head, page) deviation sums past 1e30; max|dLSE|={err:.2e}; "
        f"largest page LSE {s_ref.max():.1f}")
    assert n_over > 0
    assert err <= LSE_TOL
    # the builder on these pages still meets the code gate
    Kf = O.bf16_to_f64(kc[x.block_table[0, big], 0])
    compare_build_codes(Kf, recs[0, x.block_table[0, big]], where="huge deviations")


def test_constant_pages_closed_form():
    w = get_workload("tiny-4k")
    x = generate(w)
    kc = x.k_cache[0]
    const = np.arange(1, 256, 5)
    for j in const:
        blk = x.block_table[0, j]
        kc[blk, 0, :, :] = kc[blk, 0, 0, :][None, :]       # every token = the first one
    lay = Layer(x, 0)
    lay.gpu_build()
    lse = lay.score()
    torch.cuda.synchronize()
    recs = lay.summ.cpu().numpy()
    blk = x.block_table[0, const]
    qg = O.unpack_records(recs[0, blk])
    # no basis: zero codes and zero scales for every column
    assert np.all(qg["v_q"] == 0) and np.all(qg["c_q"] == 0)
    assert np.all(qg["s_v"] == 0) and np.all(qg["s_c"] == 0)
    # the centroid is the key itself, quantized as the oracle quantizes it
    K = O.bf16_to_f64(kc[blk, 0])
    mu, V, C, lam = O.page_summary(K)
    assert np.all(V == 0) and np.all(C == 0)
    qo = O.quantize_summary(mu, V, C)
    assert np.abs(qg["mu_q"].astype(int) - qo["mu_q"]).max() <= 1
    assert np.all(np.abs(qg["s_mu"] - qo["s_mu"]) <= fp16_ulp(qo["s_mu"]))
    # closed form on the GPU's own codes: q.mu_hat / sqrt(d) + log 16
    q = O.bf16_to_f64(x.q[0, 0])
    mu_hat = qg["mu_q"].astype(np.float64) * qg["s_mu"][:, None]
    want = (q @ mu_hat.T) / math.sqrt(128) + math.log(16)
    got = lse[0, :, const].double().cpu().numpy()
    err = float(np.abs(got - want).max())
    log(f"[constant pages] {len(const)} pages, max|dLSE| against the closed form {err:.2e}")
    assert err <= LSE_TOL

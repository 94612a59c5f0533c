"""Pins of the CPU oracle to facts fixed by the LOCKS pages and by mathematics.

None of these retypes the oracle's formula: each checks a closed form, an
invariant, a special case that reduces to a textbook result, a hand-worked
example, or brute force on a tiny input.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")
rng0 = np.random.default_rng(1234)


def _orthonormal(rng, d, r):
    q, _ = np.linalg.qr(rng.standard_normal((d, r)))
    return q


def _low_rank_pages(rng, n, rho, d=128, B=16, scale=1.0):
    """Pages whose centered keys have rank exactly rho (float64)."""
    pages = []
    for _ in range(n):
        mu = rng.standard_normal(d)
        U = _orthonormal(rng, d, rho)
        A = rng.standard_normal((B, rho)) * scale
        A -= A.mean(axis=0)                 # keep mu the exact centroid
        pages.append(mu + A @ U.T)
    return np.stack(pages)


# --- summary size: about 10% of KV bytes ------------------------------------

def test_summary_bytes_about_a_tenth():
    g = json.load(open(os.path.join(GOLD, "summary_size.json")))
    frac = O.RECORD_BYTES / g["kv_bytes_per_page_head"]
    assert g["fraction_low"] <= frac <= g["fraction_high"]
    codes = sum(g["code_bytes"].values())
    # int4 basis d*r/2, int8 coefficients B*r, int8 centroid d
    assert codes == 128 * 8 // 2 + 16 * 8 + 128
    assert O.OFF_END <= O.RECORD_BYTES and O.RECORD_BYTES % 64 == 0


# --- exactness: rank <= r and no quantization gives the exact page LSE ------

@pytest.mark.parametrize("rho", [1, 3, 8])
def test_estimate_exact_when_rank_le_r(rho):
    rng = np.random.default_rng(rho)
    K = _low_rank_pages(rng, 6, rho)
    mu, V, C, lam = O.page_summary(K)
    q = rng.standard_normal((4, 128)) * 2.0
    est = O.page_lse(q[None], mu, V, C)              # [n, G]
    exact = O.page_lse_exact(q[None], K)
    np.testing.assert_allclose(est, exact, rtol=0, atol=1e-10)
    # reconstruction mu + V c_i is the key itself
    np.testing.assert_allclose(mu[:, None, :] + C @ np.swapaxes(V, 1, 2), K, atol=1e-10)


@pytest.mark.parametrize("r,rho", [(4, 2), (4, 4), (16, 11), (16, 15)])
def test_estimate_exact_when_rank_le_r_other_ranks(r, rho):
    """The rank-4 and rank-16 summaries follow the same rule: a page of
    centered rank rho <= r is reconstructed exactly (16 centered tokens have
    rank <= 15, so rank 16 is exact on every page)."""
    rng = np.random.default_rng(100 + 10 * r + rho)
    K = _low_rank_pages(rng, 5, rho)
    mu, V, C, lam = O.page_summary(K, r)
    assert V.shape == (5, 128, r) and C.shape == (5, 16, r)
    q = rng.standard_normal((4, 128)) * 2.0
    np.testing.assert_allclose(O.page_lse(q[None], mu, V, C), O.page_lse_exact(q[None], K),
                               rtol=0, atol=1e-10)
    if r == 16:
        K2 = rng.standard_normal((3, 16, 128))
        m2, V2, C2, lam2 = O.page_summary(K2, 16)
        np.testing.assert_allclose(O.energy_captured(lam2, 16), 1.0, atol=1e-12)
        np.testing.assert_allclose(O.page_lse(q[None], m2, V2, C2),
                                   O.page_lse_exact(q[None], K2), atol=1e-10)


def test_record_layout_other_ranks():
    """Rank-r records: 84r + 130 bytes of fields padded to a multiple of 64
    (512 / 832 / 1536 bytes, 6.25% / 10.2% / 18.75% of a page-head's 8 KB of
    K and V); rank 8 is the layout above.  Each field sits where the layout
    says: a single nonzero code or scale lands in the byte it names, and a
    pack/unpack round trip is exact."""
    assert [O.record_bytes(r) for r in (4, 8, 16)] == [512, 832, 1536]
    lay8 = O.record_layout(8)
    assert (lay8["c"], lay8["mu"], lay8["sv"], lay8["sc"], lay8["smu"], lay8["end"]) == (
        O.OFF_C, O.OFF_MU, O.OFF_SV, O.OFF_SC, O.OFF_SMU, O.OFF_END)
    rng = np.random.default_rng(61)
    for r in (4, 16):
        lay = O.record_layout(r)
        z = dict(v_q=np.zeros((128, r), np.int8), c_q=np.zeros((16, r), np.int8),
                 mu_q=np.zeros(128, np.int8), s_v=np.zeros(r), s_c=np.zeros(r), s_mu=0.0)
        t, k = 5, r - 1
        one = dict(z, c_q=z["c_q"].copy())
        one["c_q"][t, k] = 3
        rec = O.pack_record(one)
        assert rec.shape == (lay["bytes"],) and np.flatnonzero(rec).tolist() == [64 * r + r * t + k]
        one = dict(z, mu_q=z["mu_q"].copy())
        one["mu_q"][7] = -2
        assert np.flatnonzero(O.pack_record(one)).tolist() == [80 * r + 7]
        one = dict(z, s_c=np.eye(r)[k] * 1.0)      # fp16 1.0 = 0x3C00: high byte only
        assert np.flatnonzero(O.pack_record(one)).tolist() == [82 * r + 128 + 2 * k + 1]
        one = dict(z, s_mu=1.0)
        assert np.flatnonzero(O.pack_record(one)).tolist() == [84 * r + 128 + 1]
        # round trip, single and batched
        K = rng.standard_normal((7, 16, 128)) * 2
        recs, qz, _ = O.build_records(K, r)
        assert recs.shape == (7, lay["bytes"]) and np.all(recs[:, lay["end"]:] == 0)
        for p in range(7):
            assert np.array_equal(O.pack_record({key: np.asarray(qz[key])[p] for key in qz}),
                                  recs[p])
            u = O.unpack_record(recs[p], r=r)
            for key in qz:
                np.testing.assert_array_equal(u[key], np.asarray(qz[key])[p])
        ub = O.unpack_records(recs, r=r)
        for key in qz:
            np.testing.assert_array_equal(ub[key], qz[key])
        # scoring the records is scoring the quantized summary they carry
        q = rng.standard_normal((4, 128))
        mh, Vh, Ch = O.dequantize_summary(qz)
        np.testing.assert_allclose(O.score_records(q, recs, r=r),
                                   O.page_lse(q[None], mh, Vh, Ch).T, atol=1e-12)


def test_estimate_exact_on_bf16_axis_aligned_pages():
    """bf16 pages whose keys differ only in <= 8 coordinates keep rank <= 8
    after rounding, so the unquantized estimate is exact on the stored bytes."""
    rng = np.random.default_rng(7)
    from synth.host import f32_to_bf16_bits
    mu = rng.standard_normal(128)
    coords = rng.choice(128, size=5, replace=False)
    K = np.tile(mu, (16, 1))
    K[:, coords] += rng.standard_normal((16, 5))
    Kb = O.bf16_to_f64(f32_to_bf16_bits(K))
    m, V, C, _ = O.page_summary(Kb[None])
    q = rng.standard_normal((4, 128))
    np.testing.assert_allclose(O.page_lse(q[None], m, V, C), O.page_lse_exact(q[None], Kb[None]),
                               atol=1e-10)


def test_constant_page_closed_form():
    """All keys equal: no deviations, the estimate is q.mu/sqrt(d) + log 16."""
    rng = np.random.default_rng(3)
    mu = rng.standard_normal(128)
    K = np.tile(mu, (16, 1))[None]
    m, V, C, lam = O.page_summary(K)
    assert np.all(V == 0) and np.all(C == 0) and lam.max() < 1e-20
    q = rng.standard_normal((2, 128))
    want = q @ mu / math.sqrt(128) + math.log(16)
    np.testing.assert_allclose(O.page_lse(q[None], m, V, C)[0], want, atol=1e-12)


def test_zero_query_gives_log16_and_index_order_selection():
    rng = np.random.default_rng(5)
    K = rng.standard_normal((10, 16, 128))
    recs, _, _ = O.build_records(K)
    s = O.score_records(np.zeros((4, 128)), recs)
    np.testing.assert_allclose(s, math.log(16), atol=1e-12)
    L, log_m, m = O.group_mass(s)
    np.testing.assert_allclose(m, 0.1, atol=1e-15)
    assert list(O.select_top_pages(log_m, 3)) == [0, 1, 2]


# --- eigen structure: top-r eigenvectors of the deviations -------------------

def test_basis_matches_scatter_eigenvectors():
    """V's columns are eigenvectors of X^T X (checked with a dense symmetric
    eigensolver on the d x d scatter, a different routine on a different
    matrix than the oracle's SVD of X)."""
    rng = np.random.default_rng(11)
    K = rng.standard_normal((3, 16, 128)) + rng.standard_normal((3, 1, 128)) * 4
    mu, V, C, lam = O.page_summary(K)
    for p in range(3):
        X = K[p] - K[p].mean(axis=0)
        S = X.T @ X
        ev = np.linalg.eigvalsh(S)[::-1]
        np.testing.assert_allclose(lam[p][:15], ev[:15], rtol=1e-9, atol=1e-9)
        assert abs(ev[15]) < 1e-9            # centered 16 tokens: rank <= 15
        for k in range(8):
            v = V[p][:, k]
            np.testing.assert_allclose(S @ v, lam[p][k] * v, atol=1e-8 * lam[p][0])
            assert abs(np.linalg.norm(v) - 1) < 1e-12
        np.testing.assert_allclose(V[p].T @ V[p], np.eye(8), atol=1e-12)
        np.testing.assert_allclose(C[p], X @ V[p], atol=1e-12)
        np.testing.assert_allclose(C[p].sum(axis=0), 0, atol=1e-10)   # centered


def test_residual_optimality_eckart_young():
    """The page's own basis leaves the smallest residual of all orthonormal
    rank-r bases, random ones and a shared (pooled) basis included
    ([P1] sec. 3: residual optimality)."""
    rng = np.random.default_rng(17)
    K = O.bf16_to_f64(__import__("synth.host", fromlist=["x"]).f32_to_bf16_bits(
        __import__("synth.host", fromlist=["x"]).page_keys(rng, 8, __import__("synth").get_workload("tiny-4k"))))
    mu, V, C, lam = O.page_summary(K)
    Wsh = O.shared_basis(K)
    for p in range(8):
        X = K[p] - mu[p]
        res_own = np.sum((X - X @ V[p] @ V[p].T) ** 2)
        np.testing.assert_allclose(res_own, lam[p][8:].sum(), rtol=1e-9)
        res_sh = np.sum((X - X @ Wsh @ Wsh.T) ** 2)
        assert res_own <= res_sh + 1e-9
        for _ in range(125):
            W = _orthonormal(rng, 128, 8)
            assert res_own <= np.sum((X - X @ W @ W.T) ** 2) + 1e-9


def test_sign_convention():
    rng = np.random.default_rng(19)
    K = rng.standard_normal((20, 16, 128))
    _, V, C, _ = O.page_summary(K)
    for p in range(20):
        for k in range(8):
            v = V[p][:, k]
            t = int(np.argmax(np.abs(v)))
            assert v[t] > 0
            assert np.all(np.abs(v[:t]) < abs(v[t]))


def test_rank_deficient_columns_are_zero():
    rng = np.random.default_rng(23)
    K = _low_rank_pages(rng, 2, 3)
    _, V, C, lam = O.page_summary(K)
    assert np.all(V[:, :, 3:] == 0) and np.all(C[:, :, 3:] == 0)
    assert np.all(np.linalg.norm(V[:, :, :3], axis=1) > 0.999)


def test_proposition1_shared_projection_content_blind():
    """Two pages that differ only in a direction orthogonal to a shared
    rank-rho basis get identical shared summaries, but different LOCKS
    estimates ([P1] sec. 3, Proposition 1)."""
    rng = np.random.default_rng(29)
    d, rho = 128, 8
    W = _orthonormal(rng, d, rho + 2)
    Wsh, e1, e2 = W[:, :rho], W[:, rho], W[:, rho + 1]
    mu = rng.standard_normal(d)
    a = rng.standard_normal(16) * 5
    a -= a.mean()
    KA = mu + np.outer(a, e1)
    KB = mu + np.outer(a, e2)
    # shared summary: centroid + coefficients in the shared basis
    for K in (KA, KB):
        assert np.allclose((K - K.mean(0)) @ Wsh, 0, atol=1e-12)
    assert np.allclose(KA.mean(0), KB.mean(0))
    q = (e1 * 6.0)[None]
    mA, VA, CA, _ = O.page_summary(KA[None])
    mB, VB, CB, _ = O.page_summary(KB[None])
    sA = O.page_lse(q[None], mA, VA, CA)[0, 0]
    sB = O.page_lse(q[None], mB, VB, CB)[0, 0]
    assert sA - sB > 0.5
    np.testing.assert_allclose(sA, O.page_lse_exact(q[None], KA[None])[0, 0], atol=1e-10)


def test_pooled_scatter_trace_and_subspace():
    """The pooled scatter's trace is the pages' total deviation energy (the
    sum of every page's eigenvalues, from per-page SVDs), and its top
    eigenvectors span the same subspace as the shared basis (an SVD of the
    stacked deviations, another routine on another matrix)."""
    rng = np.random.default_rng(53)
    K = rng.standard_normal((30, 16, 128)) * np.linspace(0.2, 3.0, 128)
    S = O.pooled_scatter(K)
    lam = O.page_spectrum(K)[2]
    np.testing.assert_allclose(np.trace(S), lam.sum(), rtol=1e-12)
    np.testing.assert_allclose(S, S.T, atol=1e-9)
    ev, W = np.linalg.eigh(S)
    top = W[:, ::-1][:, :8]
    Wsh = O.shared_basis(K)
    np.testing.assert_allclose(np.abs(np.linalg.svd(top.T @ Wsh)[1]), 1.0, atol=1e-8)


def test_records_with_own_basis_equal_locks_records():
    """Summarizing a page in its own eigenbasis reproduces the LOCKS record
    bit for bit; a page whose deviations lie in a given orthonormal basis is
    scored exactly by the shared summary (unquantized)."""
    rng = np.random.default_rng(59)
    K = rng.standard_normal((6, 16, 128)) + rng.standard_normal((6, 1, 128)) * 3
    recs, _, _ = O.build_records(K)
    mu, V, _, _ = O.page_summary(K)
    for p in range(6):
        r2, _ = O.build_records_with_basis(K[p:p + 1], V[p])
        assert np.array_equal(r2[0], recs[p])
    Wb = _orthonormal(rng, 128, 8)
    a = rng.standard_normal((3, 16, 8)) * 4
    Kin = rng.standard_normal((3, 1, 128)) + a @ Wb.T
    m2, V2, C2 = O.shared_summary(Kin, Wb)
    q = rng.standard_normal((4, 128))
    np.testing.assert_allclose(O.page_lse(q, m2, V2, C2), O.page_lse_exact(q, Kin), atol=1e-9)


# --- quantization and packing ------------------------------------------------

def test_bf16_decoding_fixed_patterns():
    """bf16 is the upper half of an IEEE-754 binary32: 1 sign bit, 8 exponent
    bits (bias 127), 7 fraction bits.  Values worked by hand from that
    definition, subnormals and infinities included."""
    cases = {
        0x3F80: 1.0,                                   # exponent 127, fraction 0
        0xC040: -3.0,                                  # -(1 + 64/128) * 2^1
        0x4049: 3.140625,                              # (1 + 73/128) * 2^1
        0x3E00: 0.125,                                 # exponent 124
        0x0001: math.ldexp(1.0, -133),                 # smallest subnormal: 2^-126 * 2^-7
        0x0080: math.ldexp(1.0, -126),                 # smallest normal
        0x7F7F: math.ldexp(2.0 - 2.0 ** -7, 127),      # largest finite
        0x8000: -0.0,
        0x7F80: math.inf,
        0xFF80: -math.inf,
    }
    bits = np.array(list(cases), dtype=np.uint16)
    got = O.bf16_to_f64(bits)
    assert got.dtype == np.float64
    for b, g in zip(bits, got):
        want = cases[int(b)]
        assert g == want, (hex(int(b)), g, want)
    assert math.copysign(1.0, float(got[list(cases).index(0x8000)])) == -1.0
    nan = O.bf16_to_f64(np.array([0x7FC0], dtype=np.uint16))
    assert np.isnan(nan).all()


def test_quantization_rounds_half_to_even():
    """Exact half-way quotients x / s go to the even code (the reading of the
    rounding rule), with scales chosen so that fp16(max|x| / qmax) is exact."""
    # basis column: max|x| = 3.5 gives s = 3.5 / 7 = 0.5 exactly in fp16
    V = np.zeros((128, 8))
    V[:8, 0] = [3.5, 1.25, 1.75, -1.25, 0.25, -0.25, 0.75, -3.5]   # x/s = 7, 2.5, 3.5, -2.5, .5, -.5, 1.5, -7
    # coefficient column: max|x| = 31.75 gives s = 0.25 exactly
    C = np.zeros((16, 8))
    C[:6, 0] = [31.75, 0.625, 0.875, -0.625, 0.125, 0.375]        # x/s = 127, 2.5, 3.5, -2.5, .5, 1.5
    # centroid: max|x| = 127 gives s = 1
    mu = np.zeros(128)
    mu[:5] = [127.0, 2.5, -3.5, 4.5, -0.5]
    qz = O.quantize_summary(mu, V, C)
    assert float(qz["s_v"][0]) == 0.5 and float(qz["s_c"][0]) == 0.25 and float(qz["s_mu"]) == 1.0
    assert qz["v_q"][:8, 0].tolist() == [7, 2, 4, -2, 0, 0, 2, -7]
    assert qz["c_q"][:6, 0].tolist() == [127, 2, 4, -2, 0, 2]
    assert qz["mu_q"][:5].tolist() == [127, 2, -4, 4, 0]


def test_quantization_codes_and_scales():
    rng = np.random.default_rng(31)
    K = rng.standard_normal((50, 16, 128)) * 3
    mu, V, C, _ = O.page_summary(K)
    qz = O.quantize_summary(mu, V, C)
    assert qz["v_q"].min() >= -7 and qz["v_q"].max() <= 7
    assert np.abs(qz["c_q"]).max() <= 127 and np.abs(qz["mu_q"]).max() <= 127
    # scales are the fp16 rounding of max|x| / qmax
    np.testing.assert_array_equal(qz["s_v"], np.float16(np.abs(V).max(axis=1) / 7).astype(np.float64))
    np.testing.assert_array_equal(qz["s_mu"], np.float16(np.abs(mu).max(axis=1) / 127).astype(np.float64))
    mh, Vh, Ch = O.dequantize_summary(qz)
    # rounding error is at most half a step, except where clamping at qmax
    # absorbs the fp16 rounding of the scale (at most qmax * 2^-11 steps more)
    assert np.all(np.abs(Vh - V) <= qz["s_v"][:, None, :] * (0.5 + 7 * 2.0 ** -11) + 1e-15)
    assert np.all(np.abs(Ch - C) <= qz["s_c"][:, None, :] * (0.5 + 127 * 2.0 ** -11) + 1e-15)
    assert np.all(np.abs(mh - mu) <= qz["s_mu"][:, None] * (0.5 + 127 * 2.0 ** -11) + 1e-15)
    # the largest magnitude uses (nearly) the full code range
    assert np.all(np.abs(qz["v_q"]).max(axis=1) >= 6)


def test_zero_scale_gives_zero_codes():
    qz = O.quantize_summary(np.zeros(128), np.zeros((128, 8)), np.zeros((16, 8)))
    assert float(qz["s_mu"]) == 0 and np.all(qz["mu_q"] == 0)
    assert np.all(qz["s_v"] == 0) and np.all(qz["v_q"] == 0)
    assert np.all(qz["s_c"] == 0) and np.all(qz["c_q"] == 0)


def test_pack_unpack_roundtrip():
    rng = np.random.default_rng(37)
    qz = dict(v_q=rng.integers(-7, 8, size=(3, 128, 8)).astype(np.int8),
              c_q=rng.integers(-127, 128, size=(3, 16, 8)).astype(np.int8),
              mu_q=rng.integers(-127, 128, size=(3, 128)).astype(np.int8),
              s_v=np.float16(rng.random((3, 8))).astype(np.float64),
              s_c=np.float16(rng.random((3, 8))).astype(np.float64),
              s_mu=np.float16(rng.random(3)).astype(np.float64))
    recs = O.pack_records(qz)
    for i in range(3):
        one = O.pack_record({k: v[i] for k, v in qz.items()})
        np.testing.assert_array_equal(one, recs[i])
        back = O.unpack_record(recs[i])
        for k in qz:
            np.testing.assert_array_equal(np.asarray(back[k]), qz[k][i])
    vec = O.unpack_records(recs)
    for k in qz:
        np.testing.assert_array_equal(vec[k], qz[k])
    assert np.all(recs[:, O.OFF_END:] == 0)
    # layout spot checks: basis 0, d=0 low nibble of byte 0; d=4 high nibble
    assert recs[0, 0] & 0xF == qz["v_q"][0, 0, 0] & 0xF
    assert recs[0, 0] >> 4 == qz["v_q"][0, 4, 0] & 0xF
    assert recs[0, 64 * 2 + 4] & 0xF == qz["v_q"][0, 8, 2] & 0xF


# --- shares and selection ----------------------------------------------------

def test_share_hand_worked_cases():
    g = json.load(open(os.path.join(GOLD, "share_cases.json")))
    for case in g["cases"]:
        s = np.array(case["s_hat"])
        L, log_m, m = O.group_mass(s)
        np.testing.assert_allclose(m, case["m"], atol=1e-12)
        np.testing.assert_allclose(np.exp(log_m), case["m"], atol=1e-12)
        assert list(O.select_top_pages(log_m, case["budget"])) == case["sel"]


def test_topk_against_counting_bruteforce():
    rng = np.random.default_rng(41)
    for trial in range(30):
        n = int(rng.integers(1, 60))
        vals = rng.integers(0, 6, size=n).astype(np.float64)   # many ties
        k = int(rng.integers(0, n + 3))
        sel = set(O.select_top_pages(vals, k).tolist())
        # page j is kept iff fewer than k pages beat it (larger, or equal with lower index)
        want = {j for j in range(n)
                if sum(1 for i in range(n) if vals[i] > vals[j] or (vals[i] == vals[j] and i < j)) < k}
        assert sel == want
        assert list(O.select_top_pages(vals, k)) == sorted(sel)


def test_table_selection_bruteforce():
    """Tables over several KV heads: shares from explicit loops (each head's
    softmax over pages, averaged over the table's heads) and the top-k by
    counting, for 1, 2 and 4 tables over 8 query heads."""
    rng = np.random.default_rng(47)
    for trial in range(12):
        hq, n = 8, int(rng.integers(1, 25))
        s = rng.standard_normal((hq, n)) * 3
        s[:, rng.integers(0, n)] += 4          # a shared heavy page now and then
        for n_tables in (1, 2, 4):
            k = int(rng.integers(1, n + 2))
            got = O.table_selection(s, n_tables, k)
            assert len(got) == n_tables
            hpt = hq // n_tables
            for t, (log_m, sel) in enumerate(got):
                heads = range(t * hpt, (t + 1) * hpt)
                m = []
                for j in range(n):
                    acc = 0.0
                    for h in heads:
                        z = sum(math.exp(s[h, i]) for i in range(n))
                        acc += math.exp(s[h, j]) / z
                    m.append(acc / hpt)
                np.testing.assert_allclose(np.exp(log_m), m, rtol=1e-12)
                want = sorted(j for j in range(n)
                              if sum(1 for i in range(n)
                                     if m[i] > m[j] or (m[i] == m[j] and i < j)) < k)
                assert list(sel) == want


def test_table_selection_layer_wide_differs_from_per_kv_head():
    """Two KV heads of 2 query heads each, 3 pages, k = 1, shares written out.
    Case 1: KV head 0's heads give pages (0.45, 0.40, 0.15), KV head 1's
    (0.15, 0.40, 0.45).  Per KV head: pages {0} and {2}.  One table for the
    layer averages to (0.30, 0.40, 0.30) and keeps page 1, which neither
    per-KV-head table keeps.  Case 2: (0.65, 0.30, 0.05) and (0.05, 0.30,
    0.65) average to (0.35, 0.30, 0.35); the tie goes to the lower index, so
    the layer-wide table keeps page 0 and KV head 1 loses its top page."""
    def logits(shares):
        return np.log(np.array(shares))
    s = np.stack([logits([0.45, 0.40, 0.15])] * 2 + [logits([0.15, 0.40, 0.45])] * 2)
    assert [list(sel) for _, sel in O.table_selection(s, 2, 1)] == [[0], [2]]
    (log_m, sel), = O.table_selection(s, 1, 1)
    np.testing.assert_allclose(np.exp(log_m), [0.30, 0.40, 0.30], atol=1e-12)
    assert list(sel) == [1]
    s2 = np.stack([logits([0.65, 0.30, 0.05])] * 2 + [logits([0.05, 0.30, 0.65])] * 2)
    assert [list(sel) for _, sel in O.table_selection(s2, 2, 1)] == [[0], [2]]
    (log_m2, sel2), = O.table_selection(s2, 1, 1)
    np.testing.assert_allclose(np.exp(log_m2), [0.35, 0.30, 0.35], atol=1e-12)
    assert list(sel2) == [0]


def test_shift_invariance_of_shares():
    rng = np.random.default_rng(43)
    s = rng.standard_normal((4, 30))
    _, lm1, _ = O.group_mass(s)
    _, lm2, _ = O.group_mass(s + rng.standard_normal((4, 1)) * 10)
    np.testing.assert_allclose(lm1, lm2, atol=1e-12)


# --- attention ---------------------------------------------------------------

def _attention_loops(q, K, V, scale):
    out, lse = [], []
    for h in range(len(q)):
        logits = [scale * sum(q[h][t] * K[i][t] for t in range(len(q[h]))) for i in range(len(K))]
        m = max(logits)
        e = [math.exp(x - m) for x in logits]
        z = sum(e)
        out.append([sum(e[i] * V[i][t] for i in range(len(K))) / z for t in range(len(V[0]))])
        lse.append(m + math.log(z))
    return np.array(out), np.array(lse)


def test_attention_bruteforce_loops():
    rng = np.random.default_rng(47)
    q, K, V = rng.standard_normal((2, 8)), rng.standard_normal((5, 8)), rng.standard_normal((5, 8))
    o, l = O.attention(q, K, V, scale=0.3)
    o2, l2 = _attention_loops(q.tolist(), K.tolist(), V.tolist(), 0.3)
    np.testing.assert_allclose(o, o2, atol=1e-13)
    np.testing.assert_allclose(l, l2, atol=1e-13)


@pytest.mark.parametrize("seq_len,pending", [(4096, 0), (4096 - 5, 0), (16 * 7 + 1, 0),
                                             (4096, 1), (16 * 7 + 1, 1), (16, 1), (1, 1)])
def test_full_budget_equals_dense(seq_len, pending):
    """Every page selected is dense attention over all seq_len tokens, with
    the tail page holding exactly the tokens past the summarized pages: the
    partial last page, or with the newest page pending the whole page holding
    the newest token (1 to 16 tokens)."""
    from synth import get_workload
    from synth.host import generate
    w = get_workload("tiny-4k", ctx=4096)
    x = generate(w, seq_lens=[seq_len])
    q = O.bf16_to_f64(x.q[0, 0])
    row = x.block_table[0]
    n_fin = (seq_len - pending) // 16
    assert O.summarized_pages(seq_len, pending) == n_fin
    res = O.decode_group(q, x.k_cache[0], x.v_cache[0], row, 0, seq_len, budget_pages=10 ** 6,
                         pending=pending)
    assert list(res["sel"]) == list(range(n_fin))
    Kall = O.bf16_to_f64(x.k_cache[0][row[:-(-seq_len // 16)], 0].reshape(-1, 128)[:seq_len])
    Vall = O.bf16_to_f64(x.v_cache[0][row[:-(-seq_len // 16)], 0].reshape(-1, 128)[:seq_len])
    o, l = O.attention(q, Kall, Vall)
    np.testing.assert_allclose(res["out"], o, atol=1e-12)
    np.testing.assert_allclose(res["lse"], l, atol=1e-12)


def test_pending_newest_page():
    """The page that holds the newest token, when pending, is not a candidate
    and is attended in full: at 32 tokens only page 0 is summarized and page
    1's 16 tokens are the tail; a length that is not a multiple of 16 gives the
    same page count and the same result either way; and an empty sequence
    has no pages."""
    from synth import get_workload
    from synth.host import generate
    assert [O.summarized_pages(n, 1) for n in (0, 1, 15, 16, 17, 32, 33)] == [0, 0, 0, 0, 1, 1, 2]
    assert [O.summarized_pages(n, 0) for n in (0, 1, 15, 16, 17, 32, 33)] == [0, 0, 0, 1, 1, 2, 2]
    w = get_workload("tiny-4k", ctx=4096)
    x = generate(w, seq_lens=[32])
    q = O.bf16_to_f64(x.q[0, 0])
    row = x.block_table[0]
    res = O.decode_group(q, x.k_cache[0], x.v_cache[0], row, 0, 32, budget_pages=1, pending=1)
    assert res["s_hat"].shape == (4, 1) and list(res["sel"]) == [0]
    K = O.gather_pages(x.k_cache[0], row, 0, [0], 32, pending=1)
    assert K.shape == (32, 128)
    np.testing.assert_array_equal(K[16:], O.bf16_to_f64(x.k_cache[0][row[1], 0]))
    for n in (16 * 40 + 3, 16 * 40 + 15):
        a = O.decode_group(q, x.k_cache[0], x.v_cache[0], row, 0, n, budget_pages=8)
        b = O.decode_group(q, x.k_cache[0], x.v_cache[0], row, 0, n, budget_pages=8, pending=1)
        assert list(a["sel"]) == list(b["sel"])
        np.testing.assert_array_equal(a["out"], b["out"])


def test_sparse_attention_is_dense_over_selected_tokens():
    rng = np.random.default_rng(53)
    from synth import get_workload
    from synth.host import generate
    x = generate(get_workload("tiny-4k"), seq_lens=[16 * 20 + 3])
    q = O.bf16_to_f64(x.q[0, 0])
    pages = [2, 5, 11]
    o, l = O.sparse_attention(q, x.k_cache[0], x.v_cache[0], x.block_table[0], 0, pages, 16 * 20 + 3)
    toks = [(p, i) for p in pages for i in range(16)] + [(20, i) for i in range(3)]
    K = np.array([O.bf16_to_f64(x.k_cache[0][x.block_table[0][p], 0, i]) for p, i in toks])
    V = np.array([O.bf16_to_f64(x.v_cache[0][x.block_table[0][p], 0, i]) for p, i in toks])
    o2, l2 = _attention_loops(q.tolist(), K.tolist(), V.tolist(), 1 / math.sqrt(128))
    np.testing.assert_allclose(o, o2, atol=1e-12)
    np.testing.assert_allclose(l, l2, atol=1e-12)


# --- the generator's recipe ---------------------------------------------------

def test_generator_energy_matches_recipe():
    """Rank-8 energy share of generated pages.  A centered 16-token page spans
    at most 15 directions, so any top-8 share is at least 8/15; the noise
    (variance 0.05 in each of 128 dims) dominates the 8 structured directions
    (variances 1/k) under the variance reading, less so under the std reading."""
    from synth import get_workload
    from synth.host import page_keys
    w = get_workload("tiny-4k")
    e_var = O.energy_captured(O.page_summary(page_keys(np.random.default_rng(0), 400, w))[3]).mean()
    w2 = w.with_(noise_var=0.05 ** 2, coef_var_is_inv_k=False)
    e_std = O.energy_captured(O.page_summary(page_keys(np.random.default_rng(0), 400, w2))[3]).mean()
    assert 8 / 15 < e_var < e_std < 1.0
    assert 0.70 < e_var < 0.78 and 0.88 < e_std < 0.97

"""Helpers for the GPU parity tests: upload seeded inputs, run the library,
compare with the oracle at the stated tolerances."""

import math

import numpy as np
import torch

import oracle as O
from kv_cache_page_int4_amd import locks as L

LSE_TOL = 1e-3        # page LSE, absolute, against fp64 on the same codes
OUT_TOL = 2e-2        # sparse attention output, max-abs
WINDOW = 1e-4         # relative mass window around the k-th page


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def from_dev_bf16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class Layer:
    """Device copies of one layer of a generated workload."""

    def __init__(self, x, layer=0, rank=8):
        w = x.w
        self.x, self.w, self.layer, self.rank = x, w, layer, rank
        self.d = L.dims(w.hq, w.hkv, rank=rank)
        self.k = to_dev_bf16(x.k_cache[layer])      # [nb, hkv, 16, 128]
        self.v = to_dev_bf16(x.v_cache[layer])
        self.q = to_dev_bf16(x.q[layer])            # [b, hq, 128]
        self.bt = torch.from_numpy(x.block_table).cuda()
        self.seq = torch.from_numpy(x.seq_lens).cuda()
        self.nb = w.num_blocks
        self.summ = torch.zeros((w.hkv, self.nb, O.record_bytes(self.d.rank)), dtype=torch.uint8,
                                device="cuda")

    # -- oracle-built records (host), uploaded ---------------------------------
    def upload_oracle_records(self):
        x, w = self.x, self.w
        recs = np.zeros((w.hkv, self.nb, O.record_bytes(self.rank)), dtype=np.uint8)
        for b in range(w.batch):
            n = int(x.seq_lens[b]) // 16
            if n == 0:
                continue
            blk = x.block_table[b, :n]
            for g in range(w.hkv):
                K = O.bf16_to_f64(x.k_cache[self.layer][blk, g])
                r, _, _ = O.build_records(K, self.rank)
                recs[g, blk] = r
        self.summ.copy_(torch.from_numpy(recs))
        return recs

    def gpu_build(self, raw=False):
        blocks = torch.arange(self.nb, dtype=torch.int32, device="cuda")
        rd = (torch.zeros((self.nb, self.w.hkv, 128 + 144 * self.rank), dtype=torch.float32,
                          device="cuda") if raw else None)
        L.build_summaries(self.d, self.k, blocks, self.summ, raw_debug=rd)
        return rd

    def score(self):
        w = self.w
        P = self.bt.shape[1]
        # NaN-filled, so that a page the scorer skips cannot pass as -inf
        lse = torch.full((w.batch, w.hq, P), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.empty(L.score_workspace_bytes(self.d, w.batch, P, 0), dtype=torch.uint8, device="cuda")
        L.score_pages(self.d, self.q, self.summ, self.nb, self.bt, self.seq, lse, ws)
        return lse

    def score_select(self, budget, with_lse=True):
        w = self.w
        P = self.bt.shape[1]
        sel = torch.full((w.batch, w.hkv, budget), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((w.batch, w.hkv), -7, dtype=torch.int32, device="cuda")
        lse = (torch.full((w.batch, w.hq, P), float("nan"), dtype=torch.float32, device="cuda")
               if with_lse else None)
        ws = torch.empty(L.score_workspace_bytes(self.d, w.batch, P, budget), dtype=torch.uint8,
                         device="cuda")
        L.score_select(self.d, self.q, self.summ, self.nb, self.bt, self.seq, budget, sel, cnt, ws,
                       page_lse=lse)
        return sel, cnt, lse

    def select(self, lse, budget):
        w = self.w
        sel = torch.full((w.batch, w.hkv, budget), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((w.batch, w.hkv), -7, dtype=torch.int32, device="cuda")
        ws = torch.empty(L.score_workspace_bytes(self.d, w.batch, lse.shape[-1], budget),
                         dtype=torch.uint8, device="cuda")
        L.select_pages(self.d, lse, self.seq, budget, sel, cnt, ws)
        return sel, cnt

    def attend(self, sel, cnt, budget, dense=False):
        w = self.w
        out = torch.empty((w.batch, w.hq, 128), dtype=torch.bfloat16, device="cuda")
        olse = torch.empty((w.batch, w.hq), dtype=torch.float32, device="cuda")
        n_att = (self.bt.shape[1] if dense else budget) + 1
        ws = L.attend_workspace(self.d, w.batch, n_att)
        L.sparse_attend(self.d, self.q, self.k, self.v, self.bt, self.seq,
                        None if dense else sel, None if dense else cnt, budget, out, ws,
                        out_lse=olse)
        return out, olse


def oracle_scores(x, recs, layer, b, g, r=8):
    """fp64 page LSE of the group's heads from records (host array [hkv, nb, 832])."""
    n = int(x.seq_lens[b]) // 16
    G = x.w.group
    q = O.bf16_to_f64(x.q[layer, b, g * G:(g + 1) * G])
    return O.score_records(q, recs[g, x.block_table[b, :n]], r=r)


def check_selection(gpu_sel, oracle_log_m, budget):
    """Selected set must equal the oracle's except for pages whose mass is
    within WINDOW (relative) of the k-th largest mass.  Returns the number of
    pages inside that window."""
    n = oracle_log_m.shape[0]
    k = min(budget, n)
    want = O.select_top_pages(oracle_log_m, budget)
    got = np.asarray(gpu_sel)
    assert got.shape[0] == k, (got.shape, k)
    assert np.all(np.diff(got) > 0), "selection not strictly ascending"
    if k == 0 or k == n:
        assert list(got) == list(range(n)) if k == n else True
        return 0
    lm_k = np.sort(oracle_log_m)[::-1][k - 1]
    # |m_j - m_k| <= WINDOW * m_k  <=>  |exp(lm_j - lm_k) - 1| <= WINDOW
    near = np.abs(np.expm1(oracle_log_m - lm_k)) <= WINDOW
    g_set, w_set = set(got.tolist()), set(want.tolist())
    diff = g_set ^ w_set
    bad = [j for j in diff if not near[j]]
    assert not bad, f"selection differs outside the tie window at pages {sorted(bad)[:10]}"
    if not (near.sum() > 1):
        assert list(got) == list(want)
    return int(near.sum())


def dequant_recon(qz):
    mu, V, C = O.dequantize_summary(qz)
    return mu[..., None, :] + C @ np.swapaxes(V, -1, -2)


def fp16_ulp(x):
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def scores_of(x, layer, b, g, lse_dev):
    G = x.w.group
    n = int(x.seq_lens[b]) // 16
    return lse_dev[b, g * G:(g + 1) * G, :n].double().cpu().numpy()


def log(msg):
    print(msg, flush=True)


def softmax_scale():
    return 1.0 / math.sqrt(128)


# ---------------------------------------------------------------------------
# summary builder codes against the oracle on the same keys
# ---------------------------------------------------------------------------

def exempt_columns(lam, V):
    """Columns whose codes are not unique under rounding: near-degenerate
    eigenvalues, a near-tie for the sign pivot, or an eigenvalue near the
    rank floor."""
    r = V.shape[-1]
    lam1 = lam[0]
    ex = np.zeros(r, dtype=bool)
    for k in range(r):
        gaps = []
        if k > 0:
            gaps.append(lam[k - 1] - lam[k])
        if k + 1 < len(lam):
            gaps.append(lam[k] - lam[k + 1])
        if min(gaps) < 1e-3 * lam1:
            ex[k] = True
        a = np.sort(np.abs(V[:, k]))[::-1]
        if a[0] > 0 and (a[0] - a[1]) <= 1e-4 * a[0]:
            ex[k] = True
        if 0.5 * O.TAU * lam1 <= lam[k] <= 2 * O.TAU * lam1:
            ex[k] = True
    return ex


def quant_error_rms(qz, r=8):
    """Expected RMS error (Frobenius) that quantization adds to a page's
    reconstruction C V^T, from the record's own scales: rounding to a step s
    leaves an error uniform on [-s/2, s/2], of variance s^2 / 12, in each of
    the 128 entries of basis column k (step s_V[k]) and the 16 entries of
    coefficient column k (step s_c[k]); column k's error term is
    |c_k| |dv_k| + |dc_k| |v_k|, so its expected square is
    |c_k|^2 128 s_V[k]^2 / 12 + |v_k|^2 16 s_c[k]^2 / 12."""
    mu, V, C = O.dequantize_summary(qz)
    sv, sc = np.asarray(qz["s_v"]), np.asarray(qz["s_c"])
    cn2 = (C * C).sum(axis=-2)          # [..., r]
    vn2 = (V * V).sum(axis=-2)
    return np.sqrt((cn2 * 128 * sv ** 2 / 12 + vn2 * 16 * sc ** 2 / 12).sum(axis=-1))


def compare_build_codes(K, recs_gpu, where="", r=8):
    """K: fp64 keys [n, 16, 128]; recs_gpu: the GPU's rank-r records [n, bytes] for
    the same page-heads.  Codes within 1 LSB and scales within 1 fp16 ulp
    outside the exempt columns.  An exempt page (a near-degenerate eigenvalue,
    an ambiguous sign or an eigenvalue at the rank floor) has no unique basis:
    any orthonormal basis of a near-degenerate cluster is an equally valid
    eigenbasis, so its codes cannot be compared.  What is unique is the
    residual: by Eckart-Young a rank-r basis of the top-r eigenspace leaves
    |X - X V V^T|^2 = sum_{k>r} lam_k, swapping an eigenvector across a gap
    below 1e-3 lam_1 (the exemption threshold) adds exactly that gap, and
    quantization adds e_q^2 on average, e_q the expected RMS quantization
    error of the record (quant_error_rms, from its own int4/int8 steps).  The
    GPU record's dequantized reconstruction must leave
        residual^2 <= sum_{k>r} lam_k + n_ex * 1e-3 lam_1 + (1.5 e_q)^2.
    On oracle records sqrt(residual^2 - sum_{k>r} lam_k) / e_q is 0.99-1.07
    for ranks 4, 8 and 16; a random basis gives 6 or more.  Returns (columns,
    exempt columns, worst exempt-page ratio sqrt(residual^2 - optimum) / e_q)."""
    mu, V, C, lam = O.page_summary(K, r)
    qo = O.quantize_summary(mu, V, C)
    qg = O.unpack_records(recs_gpu, r=r)
    assert np.abs(qg["mu_q"].astype(int) - qo["mu_q"]).max() <= 1, where
    assert np.all(np.abs(qg["s_mu"] - qo["s_mu"]) <= fp16_ulp(qo["s_mu"])), where
    n_cols = n_ex = 0
    worst = 0.0
    for i in range(K.shape[0]):
        ex = exempt_columns(lam[i], V[i])
        n_cols += len(ex)
        n_ex += int(ex.sum())
        ok = ~ex
        dv = np.abs(qg["v_q"][i][:, ok].astype(int) - qo["v_q"][i][:, ok])
        dc = np.abs(qg["c_q"][i][:, ok].astype(int) - qo["c_q"][i][:, ok])
        assert dv.max(initial=0) <= 1, f"basis codes off by {dv.max()} ({where}, page {i})"
        assert dc.max(initial=0) <= 1, f"coefficient codes off by {dc.max()} ({where}, page {i})"
        assert np.all(np.abs(qg["s_v"][i][ok] - qo["s_v"][i][ok]) <= fp16_ulp(qo["s_v"][i][ok]))
        assert np.all(np.abs(qg["s_c"][i][ok] - qo["s_c"][i][ok]) <= fp16_ulp(qo["s_c"][i][ok]))
        if ex.any():
            gi = {k: v[i] for k, v in qg.items()}
            _, Vg, Cg = O.dequantize_summary(gi)
            X = K[i] - mu[i]
            res2 = float(np.sum((X - Cg @ Vg.T) ** 2))
            opt2 = max(float(lam[i][r:].sum()), 0.0)
            eq = float(quant_error_rms(gi, r))
            bound = opt2 + ex.sum() * 1e-3 * lam[i][0] + (1.5 * eq) ** 2
            assert res2 <= bound, (
                f"exempt page residual^2 {res2:.4g} above {bound:.4g} ({where}, page {i})")
            worst = max(worst, np.sqrt(max(res2 - opt2, 0.0)) / max(eq, 1e-30))
    return n_cols, n_ex, worst

"""Planted mistakes in the oracle must trip at least one pin.

Each case swaps one oracle function for a subtly wrong copy (a dropped term,
a flipped sign, a wrong tie-break, a transposed operand) on the CPU and
checks that the named pin then fails.  This shows the pins constrain the
oracle rather than merely restating it.
"""

import numpy as np
import pytest

import oracle as O
import oracle.locks_oracle as OL
import tests.test_oracle_pins as P


def _no_centering(K, r=O.RANK, tau=O.TAU):
    K = np.asarray(K, np.float64)
    mu = K.mean(axis=-2)
    _, sig, W = np.linalg.svd(K, full_matrices=False)   # mistake: not centered
    V = np.swapaxes(W[..., :r, :], -1, -2)
    C = (K - mu[..., None, :]) @ V
    return mu, V, C, sig * sig


def _logits_no_mu(q, mu, V, C, scale=None):
    q = np.asarray(q, np.float64)
    scale = 1 / np.sqrt(q.shape[-1]) if scale is None else scale
    w = np.einsum("...gd,...dk->...gk", q, V)
    return np.einsum("...gk,...ik->...gi", w, C) * scale      # mistake: q.mu dropped


def _logits_sign(q, mu, V, C, scale=None):
    q = np.asarray(q, np.float64)
    scale = 1 / np.sqrt(q.shape[-1]) if scale is None else scale
    qmu = np.einsum("...gd,...d->...g", q, mu)
    w = np.einsum("...gd,...dk->...gk", q, V)
    return (qmu[..., None] - np.einsum("...gk,...ik->...gi", w, C)) * scale   # mistake: sign


def _spectrum_transposed(K):
    mu, X, lam, W = _orig_spectrum(K)
    n = W.shape[-1]
    Wt = np.swapaxes(W, -1, -2)[..., : W.shape[-2], :] if W.shape[-2] == n else W[..., ::-1, :]
    return mu, X, lam, Wt                                     # mistake: wrong eigenvector order


_orig_spectrum = OL.page_spectrum


def _select_high_ties(mass, budget_pages):
    mass = np.asarray(mass, np.float64)
    k = min(int(budget_pages), mass.shape[0])
    order = sorted(range(mass.shape[0]), key=lambda j: (-mass[j], -j))  # mistake: ties to higher index
    return np.array(sorted(order[:k]), dtype=np.int64)


def _group_mass_unnormalized(s_hat):
    s = np.asarray(s_hat, np.float64)
    m = np.exp(s).mean(axis=0)                                # mistake: no per-head normalization
    return OL.logsumexp(s, axis=-1), np.log(m), m


def _gather_no_tail(cache_layer, block_row, kvh, pages, seq_len, page=O.PAGE, pending=0):
    parts = [O.bf16_to_f64(cache_layer[block_row[j], kvh]) for j in pages]   # mistake: tail dropped
    return np.concatenate(parts, axis=0) if parts else np.zeros((0, cache_layer.shape[-1]))


def _gather_partial_tail_only(cache_layer, block_row, kvh, pages, seq_len, page=O.PAGE,
                              pending=0):
    n_fin = OL.summarized_pages(seq_len, pending, page)
    tail = seq_len % page                                     # mistake: a full pending page dropped
    parts = [O.bf16_to_f64(cache_layer[block_row[j], kvh]) for j in pages]
    if tail:
        parts.append(O.bf16_to_f64(cache_layer[block_row[n_fin], kvh, :tail]))
    return np.concatenate(parts, axis=0) if parts else np.zeros((0, cache_layer.shape[-1]))


def _summarized_ignores_pending(seq_len, pending=0, page=O.PAGE):
    return seq_len // page if seq_len > 0 else 0              # mistake: pending page summarized


def _tables_strided(s_hat, n_tables, budget_pages):
    s = np.asarray(s_hat, np.float64)
    out = []
    for t in range(n_tables):                                 # mistake: heads t, t + n_tables, ...
        _, log_m, _ = OL.group_mass(s[t::n_tables])
        out.append((log_m, OL.select_top_pages(log_m, budget_pages)))
    return out


def _scale_no_fp16(x):
    return np.asarray(x, np.float64)                          # mistake: scale not rounded to fp16


def _bf16_wrong_shift(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 15   # mistake: shift by 15
    return b.view(np.float32).astype(np.float64)


def _bf16_as_fp16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)  # mistake: fp16


def _quant_half_away(x, qmax, axis):
    m = np.max(np.abs(x), axis=axis, keepdims=True)
    s = OL.fp16_round(m / qmax)
    safe = np.where(s > 0, s, 1.0)
    q = x / safe
    code = np.clip(np.sign(q) * np.floor(np.abs(q) + 0.5), -qmax, qmax)   # mistake: half away from 0
    code = np.where(s > 0, code, 0.0)
    return code.astype(np.int8), np.squeeze(s, axis=axis)


MUTANTS = [
    ("page_summary", _no_centering, lambda: P.test_estimate_exact_when_rank_le_r(8)),
    ("page_summary", _no_centering, P.test_basis_matches_scatter_eigenvectors),
    ("reconstructed_logits", _logits_no_mu, lambda: P.test_estimate_exact_when_rank_le_r(3)),
    ("reconstructed_logits", _logits_sign, lambda: P.test_estimate_exact_when_rank_le_r(8)),
    ("page_spectrum", _spectrum_transposed, P.test_basis_matches_scatter_eigenvectors),
    ("select_top_pages", _select_high_ties, P.test_topk_against_counting_bruteforce),
    ("select_top_pages", _select_high_ties, P.test_share_hand_worked_cases),
    ("group_mass", _group_mass_unnormalized, P.test_share_hand_worked_cases),
    ("table_selection", _tables_strided, P.test_table_selection_layer_wide_differs_from_per_kv_head),
    ("gather_pages", _gather_no_tail, lambda: P.test_full_budget_equals_dense(4096 - 5, 0)),
    ("gather_pages", _gather_partial_tail_only, lambda: P.test_full_budget_equals_dense(4096, 1)),
    ("summarized_pages", _summarized_ignores_pending, P.test_pending_newest_page),
    ("fp16_round", _scale_no_fp16, P.test_quantization_codes_and_scales),
    ("bf16_to_f64", _bf16_wrong_shift, P.test_bf16_decoding_fixed_patterns),
    ("bf16_to_f64", _bf16_as_fp16, P.test_bf16_decoding_fixed_patterns),
    ("_sym_quant", _quant_half_away, P.test_quantization_rounds_half_to_even),
]


@pytest.mark.parametrize("name,fn,pin", MUTANTS, ids=[m[0] + ":" + m[1].__name__ for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, fn, pin):
    monkeypatch.setattr(OL, name, fn)
    monkeypatch.setattr(O, name, fn, raising=False)
    with pytest.raises(AssertionError):
        pin()

"""LOCKS oracle: plain float64 reference for every step of the decode path.

TEST INFRASTRUCTURE.  Nothing in the library imports this module; only the
tests, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg do.

Sources (cited by page and section; no passage is quoted):
  [P1] "LOCKS: Page-Local Compact Key Summaries for Efficient Long-Context
       Decoding", gist.science explainer (technical summary), sec. 2 "Method"
       (core mechanism; reconstruction and selection; group-shared selection),
       sec. 3 "Contributions", sec. 4 "Significance".
  [P2] The same paper's digest page (arXiv 2607.24555v1) and its English
       abstract.

Readings where the pages are silent:
  * The eigendecomposition is of the page's centered keys X = K - 1 mu^T; its
    top-r eigenvectors are those of the scatter X^T X, obtained here as the
    right singular vectors of X.
  * Basis columns whose eigenvalue is not above TAU * lambda_1 are set to zero;
    a page whose top eigenvalue is below EPS_CONST * |K|_F^2 has no basis.
  * Sign: each basis vector is flipped so that its largest-magnitude entry
    (lowest index on ties) is positive.
  * Coefficients are projections on the unquantized basis: c_i = V^T x_i.
  * Quantization is symmetric with round-half-to-even, one fp16 scale per
    centroid and per basis / coefficient column, and the code is computed
    against the fp16-rounded scale.
  * The GQA share of a page is the plain mean over the group's query heads of
    that head's softmax over pages; selection keeps the k largest shares,
    ties to the lower page index, returned in ascending page order.
  * Sparse attention is an ordinary softmax renormalized over the selected
    pages' tokens plus the partial (unsummarized) tail page.
  * When the page holding the newest token is pending (its summary is built
    after the decode step, off the step's critical path: [P1] sec. 2,
    implementation), the summarized pages are the first (n - 1) // 16 of a
    sequence of n tokens, and the 1..16 tokens after them are attended in
    full, as the tail page.
"""

import numpy as np

D_HEAD = 128
PAGE = 16
RANK = 8
TAU = 1e-5            # relative eigenvalue floor for a kept basis column
EPS_CONST = 1e-12     # lam_1 below this fraction of |K|_F^2: constant page
RECORD_BYTES = 832    # packed summary record per (page, KV head)
V_QMAX = 7            # int4 basis codes lie in [-7, 7]
CM_QMAX = 127         # int8 coefficient / centroid codes lie in [-127, 127]
FP16_MAX = 65504.0

# byte offsets inside one record (rank 8)
OFF_V, OFF_C, OFF_MU, OFF_SV, OFF_SC, OFF_SMU, OFF_END = 0, 512, 640, 768, 784, 800, 802
RANKS = (4, 8, 16)    # ranks with a record layout


def record_layout(r=RANK):
    """Byte offsets of a rank-r record, the rank-8 layout with every field
    sized by r: basis codes at 0 (64 bytes per column), coefficient codes at
    64r ([16 tokens][r]), centroid codes at 80r, s_V at 80r + 128, s_c at
    82r + 128, s_mu at 84r + 128; zero padding up to a multiple of 64 bytes
    (512, 832 and 1536 bytes for r = 4, 8, 16)."""
    off_c = 64 * r
    off_mu = off_c + PAGE * r
    off_sv = off_mu + D_HEAD
    off_sc = off_sv + 2 * r
    off_smu = off_sc + 2 * r
    end = off_smu + 2
    return dict(v=0, c=off_c, mu=off_mu, sv=off_sv, sc=off_sc, smu=off_smu, end=end,
                bytes=-(-end // 64) * 64)


def record_bytes(r=RANK):
    return record_layout(r)["bytes"]


# ---------------------------------------------------------------------------
# bf16 decoding
# ---------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Summary build  [P1] sec. 2, core mechanism: page-local spectral decomposition
# ---------------------------------------------------------------------------

def page_spectrum(K):
    """Centroid, centered keys and eigen-decomposition of one or more pages.

    K: [..., B, d] float64 keys of a page.  Returns (mu [..., d], X [..., B, d],
    lam [..., min(B, d)] descending eigenvalues of X^T X, W [..., min(B,d), d]
    the matching unit eigenvectors as rows).  X^T X = W^T diag(lam) W follows
    from the SVD X = U diag(sigma) W with lam = sigma^2.
    """
    K = np.asarray(K, dtype=np.float64)
    mu = K.mean(axis=-2)
    X = K - mu[..., None, :]
    _, sig, W = np.linalg.svd(X, full_matrices=False)
    return mu, X, sig * sig, W


def page_summary(K, r=RANK, tau=TAU):
    """Unquantized LOCKS summary of pages K [..., B, d].

    Returns mu [..., d], V [..., d, r] (basis as columns), C [..., B, r]
    (one coefficient vector per token) and lam [..., min(B,d)].
      * mu is the page centroid and X = K - mu the deviations ([P1] sec. 2).
      * V holds the top-r eigenvectors of the deviations ([P1] sec. 2: the
        summary stores the top-r eigenvectors and per-token coefficients).
      * Columns with lam_k <= tau * lam_1 are zero (reading: rank-deficient
        pages carry no direction there); if lam_1 <= EPS_CONST * |K|_F^2 the
        page counts as constant and every column is zero.
      * Sign: largest-|entry| component positive, lowest index on ties.
      * C = X V, the projections on the unquantized basis.
    """
    mu, X, lam, W = page_spectrum(K)
    V = np.swapaxes(W[..., :r, :], -1, -2).copy()          # [..., d, r]
    lam1 = lam[..., :1]
    keep = lam[..., :r] > tau * lam1                          # [..., r]
    # a page whose deviation energy is rounding noise next to its keys is
    # treated as constant (no basis at all)
    energy = np.sum(np.asarray(K, np.float64) ** 2, axis=(-2, -1))[..., None]
    keep &= lam1 > EPS_CONST * energy
    V = V * keep[..., None, :]
    tstar = np.argmax(np.abs(V), axis=-2)                    # first max wins
    piv = np.take_along_axis(V, tstar[..., None, :], axis=-2)[..., 0, :]
    sgn = np.where(piv < 0, -1.0, 1.0)
    V = V * sgn[..., None, :]
    C = X @ V
    return mu, V, C, lam


def energy_captured(lam, r=RANK):
    """Fraction of the page's key-deviation energy in its top-r directions
    ([P1] sec. 3, locality of structure)."""
    lam = np.asarray(lam, dtype=np.float64)
    tot = lam.sum(axis=-1)
    return np.where(tot > 0, lam[..., :r].sum(axis=-1) / np.where(tot > 0, tot, 1), 1.0)


def shared_basis(K_pages, rho=RANK):
    """Top-rho eigenvectors of the deviations pooled over many pages.

    The 'shared low-rank basis' the pages contrast LOCKS with ([P1] sec. 1 and
    sec. 3, Proposition 1; [P2] abstract).  Returns [d, rho]."""
    K = np.asarray(K_pages, dtype=np.float64)
    X = (K - K.mean(axis=-2, keepdims=True)).reshape(-1, K.shape[-1])
    _, _, W = np.linalg.svd(X, full_matrices=False)
    return W[:rho].T.copy()


def pooled_scatter(K_pages):
    """Sum over pages of X_j^T X_j with X_j = K_j - mu_j, the deviations of
    each page from its own centroid, pooled: the matrix whose top eigenvectors
    are the shared basis above.  K [n, B, d] -> [d, d]."""
    K = np.asarray(K_pages, dtype=np.float64)
    X = (K - K.mean(axis=-2, keepdims=True)).reshape(-1, K.shape[-1])
    return X.T @ X


def shared_summary(K_pages, Vb):
    """Summaries of pages K [n, B, d] in one given basis Vb [d, r] (columns):
    each page keeps its own centroid, its coefficients are C = X Vb, and every
    record carries Vb -- the shared-basis selector the pages contrast LOCKS
    with ([P1] sec. 3, Proposition 1), at the same state size.  Returns
    (mu [n, d], V [n, d, r], C [n, B, r])."""
    K = np.asarray(K_pages, dtype=np.float64)
    Vb = np.asarray(Vb, dtype=np.float64)
    mu = K.mean(axis=-2)
    X = K - mu[..., None, :]
    V = np.broadcast_to(Vb, K.shape[:-2] + Vb.shape).copy()
    return mu, V, X @ Vb


# ---------------------------------------------------------------------------
# Quantization  [P1] sec. 2: int4 basis, int8 coefficients and centroid
# ---------------------------------------------------------------------------

def fp16_round(x):
    """Round to the nearest fp16 value (saturating at the fp16 maximum)."""
    x = np.minimum(np.asarray(x, dtype=np.float64), FP16_MAX)
    return x.astype(np.float16).astype(np.float64)


def _sym_quant(x, qmax, axis):
    """Symmetric quantization of x with one scale per slice along `axis`.

    scale = fp16(max|x| / qmax); code = clamp(rint(x / scale), -qmax, qmax);
    a zero scale gives zero codes."""
    m = np.max(np.abs(x), axis=axis, keepdims=True)
    s = fp16_round(m / qmax)
    safe = np.where(s > 0, s, 1.0)
    code = np.clip(np.rint(x / safe), -qmax, qmax)
    code = np.where(s > 0, code, 0.0)
    return code.astype(np.int8), np.squeeze(s, axis=axis)


def quantize_summary(mu, V, C):
    """Quantize one page-head summary (or a batch of them).

    mu [..., d] -> int8 codes + one fp16 scale; V [..., d, r] -> int4 codes
    (stored in int8) + one fp16 scale per column; C [..., B, r] -> int8 codes
    + one fp16 scale per column."""
    mu_q, s_mu = _sym_quant(mu, CM_QMAX, axis=-1)
    v_q, s_v = _sym_quant(V, V_QMAX, axis=-2)
    c_q, s_c = _sym_quant(C, CM_QMAX, axis=-2)
    return dict(mu_q=mu_q, s_mu=s_mu, v_q=v_q, s_v=s_v, c_q=c_q, s_c=s_c)


def dequantize_summary(qz):
    mu = qz["mu_q"].astype(np.float64) * np.asarray(qz["s_mu"])[..., None]
    V = qz["v_q"].astype(np.float64) * np.asarray(qz["s_v"])[..., None, :]
    C = qz["c_q"].astype(np.float64) * np.asarray(qz["s_c"])[..., None, :]
    return mu, V, C


# ---------------------------------------------------------------------------
# Record packing (832 bytes per page-head; the pages fix only bit widths)
# ---------------------------------------------------------------------------

def _v_byte_index(k, d):
    """Byte holding basis column k, dimension d, and whether it is the high
    nibble.  Column k owns bytes [64k, 64k+64); 32-bit word w covers
    d in [8w, 8w+8); byte m of the word holds d = 8w+m in its low nibble and
    d = 8w+4+m in its high nibble."""
    w, e = d // 8, d % 8
    return OFF_V + 64 * k + 4 * w + (e % 4), e >= 4


def pack_record(qz) -> np.ndarray:
    """Pack one quantized summary into its record (832 bytes at rank 8)."""
    v = np.asarray(qz["v_q"], dtype=np.int64)      # [d, r]
    d, r = v.shape
    lay = record_layout(r)
    rec = np.zeros(lay["bytes"], dtype=np.uint8)
    for k in range(r):
        for t in range(d):
            bi, hi = _v_byte_index(k, t)
            nib = int(v[t, k]) & 0xF
            rec[bi] |= (nib << 4) if hi else nib
    c = np.asarray(qz["c_q"], dtype=np.int8)       # [B, r]
    rec[lay["c"]:lay["c"] + c.size] = c.reshape(-1).view(np.uint8)
    m = np.asarray(qz["mu_q"], dtype=np.int8)
    rec[lay["mu"]:lay["mu"] + m.size] = m.view(np.uint8)
    rec[lay["sv"]:lay["sv"] + 2 * r] = np.asarray(qz["s_v"], dtype=np.float16).view(np.uint8)
    rec[lay["sc"]:lay["sc"] + 2 * r] = np.asarray(qz["s_c"], dtype=np.float16).view(np.uint8)
    rec[lay["smu"]:lay["smu"] + 2] = np.asarray([qz["s_mu"]], dtype=np.float16).view(np.uint8)
    return rec


def unpack_record(rec, d=D_HEAD, B=PAGE, r=RANK):
    """Inverse of pack_record for one record (uint8[record_bytes(r)])."""
    rec = np.asarray(rec, dtype=np.uint8)
    lay = record_layout(r)
    v = np.zeros((d, r), dtype=np.int8)
    for k in range(r):
        for t in range(d):
            bi, hi = _v_byte_index(k, t)
            nib = (int(rec[bi]) >> 4) if hi else (int(rec[bi]) & 0xF)
            v[t, k] = nib - 16 if nib >= 8 else nib
    c = rec[lay["c"]:lay["c"] + B * r].view(np.int8).reshape(B, r).copy()
    mu = rec[lay["mu"]:lay["mu"] + d].view(np.int8).copy()
    s_v = rec[lay["sv"]:lay["sv"] + 2 * r].view(np.float16).astype(np.float64)
    s_c = rec[lay["sc"]:lay["sc"] + 2 * r].view(np.float16).astype(np.float64)
    s_mu = float(rec[lay["smu"]:lay["smu"] + 2].view(np.float16)[0])
    return dict(mu_q=mu, s_mu=s_mu, v_q=v, s_v=s_v, c_q=c, s_c=s_c)


def unpack_records(recs, d=D_HEAD, B=PAGE, r=RANK):
    """Vectorized unpack of records [..., record_bytes(r)] into a dict of
    stacked arrays."""
    recs = np.asarray(recs, dtype=np.uint8)
    lay = record_layout(r)
    lead = recs.shape[:-1]
    kk, tt = np.meshgrid(np.arange(r), np.arange(d), indexing="ij")   # [r, d]
    w, e = tt // 8, tt % 8
    bi = OFF_V + 64 * kk + 4 * w + (e % 4)
    byte = recs[..., bi].astype(np.int16)                               # [..., r, d]
    nib = np.where(e >= 4, byte >> 4, byte & 0xF)
    v = np.where(nib >= 8, nib - 16, nib).astype(np.int8)
    v = np.swapaxes(v, -1, -2)                                          # [..., d, r]
    c = recs[..., lay["c"]:lay["c"] + B * r].copy().view(np.int8).reshape(*lead, B, r)
    mu = recs[..., lay["mu"]:lay["mu"] + d].copy().view(np.int8)
    s_v = recs[..., lay["sv"]:lay["sv"] + 2 * r].copy().view(np.float16).astype(np.float64)
    s_c = recs[..., lay["sc"]:lay["sc"] + 2 * r].copy().view(np.float16).astype(np.float64)
    s_mu = recs[..., lay["smu"]:lay["smu"] + 2].copy().view(np.float16).astype(np.float64)[..., 0]
    return dict(mu_q=mu, s_mu=s_mu, v_q=v, s_v=s_v, c_q=c, s_c=s_c)


def pack_records(qz) -> np.ndarray:
    """Vectorized pack_record over a batch: qz arrays with a leading axis n."""
    v = np.asarray(qz["v_q"], dtype=np.int64)                  # [n, d, r]
    n, d, r = v.shape
    lay = record_layout(r)
    nbytes = lay["bytes"]
    recs = np.zeros((n, nbytes), dtype=np.uint8)
    kk, tt = np.meshgrid(np.arange(r), np.arange(d), indexing="ij")
    w, e = tt // 8, tt % 8
    bi = (OFF_V + 64 * kk + 4 * w + (e % 4)).reshape(-1)
    sh = np.where(e >= 4, 4, 0).reshape(-1)
    nib = (np.swapaxes(v, 1, 2).reshape(n, -1) & 0xF) << sh       # [n, r*d]
    acc = np.zeros((n, nbytes), dtype=np.int64)
    np.add.at(acc, (slice(None), bi), nib)
    oc, om, osv, osc, osm = lay["c"], lay["mu"], lay["sv"], lay["sc"], lay["smu"]
    recs[:, :oc] = acc[:, :oc].astype(np.uint8)
    c = np.asarray(qz["c_q"], dtype=np.int8).reshape(n, -1)
    recs[:, oc:oc + c.shape[1]] = c.view(np.uint8)
    m = np.asarray(qz["mu_q"], dtype=np.int8).reshape(n, -1)
    recs[:, om:om + m.shape[1]] = m.view(np.uint8)
    recs[:, osv:osv + 2 * r] = np.asarray(qz["s_v"], np.float16).reshape(n, r).view(np.uint8)
    recs[:, osc:osc + 2 * r] = np.asarray(qz["s_c"], np.float16).reshape(n, r).view(np.uint8)
    recs[:, osm:osm + 2] = np.asarray(qz["s_mu"], np.float16).reshape(n, 1).view(np.uint8)
    return recs


def build_records(K_pages, r=RANK):
    """Summaries of pages K [n, B, d] (float64) at rank r -> (records
    [n, record_bytes(r)], qz, lam)."""
    mu, V, C, lam = page_summary(K_pages, r)
    qz = quantize_summary(mu, V, C)
    return pack_records(qz), qz, lam


def build_records_with_basis(K_pages, Vb):
    """Records of pages K [n, B, d] summarized in the given basis Vb [d, r]
    (quantized and packed as LOCKS records) -> (records [n, 832], qz)."""
    mu, V, C = shared_summary(K_pages, Vb)
    qz = quantize_summary(mu, V, C)
    return pack_records(qz), qz


# ---------------------------------------------------------------------------
# Scoring  [P1] sec. 2, reconstruction and selection: the equation for
# s_hat_j(q) (log-sum-exp of the reconstructed within-page logits); [P2] abstract
# ---------------------------------------------------------------------------

def logsumexp(x, axis=-1):
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=axis, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    return np.squeeze(m, axis=axis) + np.log(np.sum(np.exp(x - m), axis=axis))


def reconstructed_logits(q, mu, V, C, scale=None):
    """Within-page logits (q.mu + (V^T q).c_i) * scale for every token.

    q [..., G, d]; mu [..., d]; V [..., d, r]; C [..., B, r] -> [..., G, B]."""
    q = np.asarray(q, dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    qmu = np.einsum("...gd,...d->...g", q, mu)
    w = np.einsum("...gd,...dk->...gk", q, V)
    dev = np.einsum("...gk,...ik->...gi", w, C)
    return (qmu[..., None] + dev) * scale


def page_lse(q, mu, V, C, scale=None):
    """Estimated page mass s_hat = LSE over the page's tokens of the
    reconstructed logits ([P1] sec. 2 equation; [P2] abstract)."""
    return logsumexp(reconstructed_logits(q, mu, V, C, scale), axis=-1)


def page_lse_exact(q, K, scale=None):
    """Exact page LSE from the true keys (the 'read every key' quantity the
    pages compare selection against, [P1] sec. 3 empirical results).
    q [..., G, d]; K [..., B, d] -> [..., G]."""
    q = np.asarray(q, dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    return logsumexp(np.einsum("...gd,...id->...gi", q, K) * scale, axis=-1)


def score_records(q, records, scale=None, r=RANK):
    """s_hat for G query heads q [G, d] against rank-r records
    [n, record_bytes(r)] -> [G, n]."""
    qz = unpack_records(records, r=r)
    mu, V, C = dequantize_summary(qz)
    s = page_lse(np.asarray(q, np.float64)[None], mu, V, C, scale)     # [n, G]
    return s.T.copy()


# ---------------------------------------------------------------------------
# GQA shares and selection  [P1] sec. 2, group-shared selection; reconstruction
# and selection (rank pages, attend the top ones); [P2] abstract
# ---------------------------------------------------------------------------

def group_mass(s_hat):
    """s_hat [G, N] -> (L [G], log_m [N], m [N]).

    L_h = LSE_j s_hat_hj normalizes each head's estimated mass over pages;
    m_j = (1/G) sum_h exp(s_hat_hj - L_h) is the group-averaged share."""
    s = np.asarray(s_hat, dtype=np.float64)
    L = logsumexp(s, axis=-1)
    share = np.exp(s - L[:, None])
    m = share.mean(axis=0)
    log_m = logsumexp(s - L[:, None], axis=0) - np.log(s.shape[0])
    return L, log_m, m


def select_top_pages(mass, budget_pages):
    """Indices of the min(budget, N) largest entries of `mass` (ties to the
    lower index), returned in ascending order."""
    mass = np.asarray(mass, dtype=np.float64)
    n = mass.shape[0]
    k = min(int(budget_pages), n)
    order = sorted(range(n), key=lambda j: (-mass[j], j))
    return np.array(sorted(order[:k]), dtype=np.int64)


def table_selection(s_hat, n_tables, budget_pages):
    """Selection with n_tables tables per sequence.  [P1] sec. 2, group-shared
    selection: the heads that share a table average their mass shares and all
    attend the table's pages.  The default reading gives each KV head its own
    table (n_tables = Hkv); n_tables = 1 is the wider reading, one table for
    the whole layer.

    s_hat [Hq, N]: every query head of one sequence, query head h belonging to
    KV head h // (Hq / Hkv).  Table t averages the query heads
    [t*Hq/n_tables, (t+1)*Hq/n_tables).  Returns a list over tables of
    (log_m [N], selected pages ascending)."""
    s = np.asarray(s_hat, dtype=np.float64)
    hq = s.shape[0]
    if n_tables < 1 or hq % n_tables:
        raise ValueError("n_tables must divide the number of query heads")
    hpt = hq // n_tables
    out = []
    for t in range(n_tables):
        _, log_m, _ = group_mass(s[t * hpt:(t + 1) * hpt])
        out.append((log_m, select_top_pages(log_m, budget_pages)))
    return out


# ---------------------------------------------------------------------------
# Sparse attention  [P2] abstract (attend only the top pages); [P1] sec. 2
# ---------------------------------------------------------------------------

def attention(q, K, V, scale=None):
    """Softmax attention of heads q [G, d] over tokens K, V [T, d].
    Returns (out [G, d], lse [G])."""
    q = np.asarray(q, dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    logits = (q @ np.asarray(K, np.float64).T) * scale
    lse = logsumexp(logits, axis=-1)
    p = np.exp(logits - lse[:, None])
    return p @ np.asarray(V, np.float64), lse


def summarized_pages(seq_len, pending=0, page=PAGE):
    """Pages of a sequence of seq_len tokens whose summaries are in use: every
    full page, or, with pending=1, every page before the one holding the
    newest token."""
    return (seq_len - pending) // page if seq_len > 0 else 0


def gather_pages(cache_layer, block_row, kvh, pages, seq_len, page=PAGE, pending=0):
    """Tokens of the given logical pages plus the tail page.

    cache_layer: bf16 bits [num_blocks, hkv, page, d]; returns float64 [T, d].
    The tail page (the tokens past the summarized pages: the partial last
    page, or with pending=1 the whole page holding the newest token) is
    always appended."""
    n_fin = summarized_pages(seq_len, pending, page)
    tail = seq_len - n_fin * page
    parts = [bf16_to_f64(cache_layer[block_row[j], kvh]) for j in pages]
    if tail:
        parts.append(bf16_to_f64(cache_layer[block_row[n_fin], kvh, :tail]))
    if not parts:
        return np.zeros((0, cache_layer.shape[-1]))
    return np.concatenate(parts, axis=0)


def sparse_attention(q, k_layer, v_layer, block_row, kvh, pages, seq_len, scale=None,
                     pending=0):
    """Attention of the group's heads q [G, d] restricted to the selected
    pages' tokens plus the tail page.  Returns (out [G, d], lse [G])."""
    K = gather_pages(k_layer, block_row, kvh, pages, seq_len, pending=pending)
    V = gather_pages(v_layer, block_row, kvh, pages, seq_len, pending=pending)
    return attention(q, K, V, scale)


# ---------------------------------------------------------------------------
# End-to-end reference for one (layer, sequence, KV head)
# ---------------------------------------------------------------------------

def page_keys_f64(k_layer, block_row, kvh, n_pages):
    """Keys of the first n_pages logical pages, float64 [n, B, d]."""
    return bf16_to_f64(k_layer[np.asarray(block_row[:n_pages]), kvh])


def decode_group(q_group, k_layer, v_layer, block_row, kvh, seq_len, budget_pages,
                 records=None, scale=None, pending=0):
    """The whole LOCKS decode step for one KV-head group.

    q_group: float64 [G, d]; returns dict with s_hat [G, N], log_m [N],
    sel (ascending), out [G, d], lse [G]."""
    n_fin = summarized_pages(seq_len, pending)
    if records is None and n_fin:
        records, _, _ = build_records(page_keys_f64(k_layer, block_row, kvh, n_fin))
    s_hat = score_records(q_group, records, scale) if n_fin else np.zeros((q_group.shape[0], 0))
    _, log_m, m = group_mass(s_hat) if n_fin else (None, np.zeros(0), np.zeros(0))
    sel = select_top_pages(log_m, budget_pages)
    out, lse = sparse_attention(q_group, k_layer, v_layer, block_row, kvh, sel, seq_len, scale,
                                pending)
    return dict(s_hat=s_hat, log_m=log_m, m=m, sel=sel, out=out, lse=lse)

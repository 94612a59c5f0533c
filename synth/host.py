"""Host (numpy) generator for small workloads.

Produces bf16 bit patterns (uint16) in the cache layout the library reads:
  k_cache, v_cache : [layers][num_blocks][hkv][page][d]
  q                : [layers][batch][hq][d]
  block_table      : [batch][total_pages] int32, logical page -> physical block
  seq_lens         : [batch] int32
Random streams come from numpy's PCG64 seeded per (seed, layer, sequence,
KV head); the device generator follows the same recipe with Philox, so the two
do not agree bit for bit.  Every consumer (oracle and GPU path) reads the same
bytes, whichever generator made them.
"""

from dataclasses import dataclass, field

import numpy as np

from .workloads import Workload


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest even), return uint16 bits."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((u >> 16) & 1)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class KVInputs:
    w: Workload
    k_cache: np.ndarray
    v_cache: np.ndarray
    q: np.ndarray
    block_table: np.ndarray
    seq_lens: np.ndarray
    carriers: list = field(default_factory=list)  # (layer, b, kvh, page, token, qhead)

    @property
    def layout(self):
        """(block_stride, head_stride, token_stride) in bf16 elements."""
        w = self.w
        return (w.hkv * w.page * w.d, w.page * w.d, w.d)


def _haar_orthonormal(rng, n, d, r):
    """n independent d x r matrices with orthonormal columns, Haar distributed."""
    g = rng.standard_normal((n, d, r))
    qm, rm = np.linalg.qr(g)
    s = np.sign(np.einsum("nii->ni", rm))
    s[s == 0] = 1.0
    return qm * s[:, None, :]


def page_keys(rng, n_pages, w: Workload):
    """Keys of n_pages pages of one KV head, float64 [n, page, d]."""
    d, B, r = w.d, w.page, w.rank
    centroid = rng.standard_normal((n_pages, d))
    u = _haar_orthonormal(rng, n_pages, d, r)
    if w.coef_var_is_inv_k:
        sd = 1.0 / np.sqrt(np.arange(1, r + 1))
    else:
        sd = 1.0 / np.arange(1, r + 1)
    a = rng.standard_normal((n_pages, B, r)) * sd
    noise = rng.standard_normal((n_pages, B, d)) * np.sqrt(w.noise_var)
    return centroid[:, None, :] + np.einsum("nik,ndk->nid", a, u) + noise


def generate(w: Workload, seq_lens=None) -> KVInputs:
    if seq_lens is None:
        seq_lens = [w.ctx] * w.batch
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    assert seq_lens.shape == (w.batch,) and int(seq_lens.max()) <= w.ctx
    P = w.total_pages
    nb = w.num_blocks
    L, b_, hq, hkv, d, B, G = w.layers, w.batch, w.hq, w.hkv, w.d, w.page, w.group

    root = np.random.default_rng([w.seed, 0xB10C])
    block_table = np.full((b_, P), -1, dtype=np.int32)
    phys = np.arange(nb, dtype=np.int32)
    if w.shuffled_blocks:
        phys = root.permutation(nb).astype(np.int32)
    for b in range(b_):
        block_table[b, :] = phys[b * P:(b + 1) * P]

    k_cache = np.zeros((L, nb, hkv, B, d), dtype=np.uint16)
    v_cache = np.zeros((L, nb, hkv, B, d), dtype=np.uint16)
    q = np.zeros((L, b_, hq, d), dtype=np.uint16)
    carriers = []
    for layer in range(L):
        for b in range(b_):
            rq = np.random.default_rng([w.seed, layer, b, 0x9])
            qf = f32_to_bf16_bits(rq.standard_normal((hq, d)))
            q[layer, b] = qf
            qd = bf16_bits_to_f32(qf).astype(np.float64)
            n_tok = int(seq_lens[b])
            n_pages = -(-n_tok // B)
            n_fin = n_tok // B
            for g in range(hkv):
                rng = np.random.default_rng([w.seed, layer, b, g, 0x4B])
                keys = page_keys(rng, n_pages, w)
                vals = rng.standard_normal((n_pages, B, d))
                n_car = min(w.carriers, n_fin)
                if n_car > 0:
                    pages = rng.choice(n_fin, size=n_car, replace=False)
                    slots = rng.integers(0, B, size=n_car)
                    for c in range(n_car):
                        h = g * G + (c % G)
                        qh = qd[h]
                        nz = rng.standard_normal(d) * np.sqrt(w.noise_var)
                        keys[pages[c], slots[c]] = 3.0 * qh / np.linalg.norm(qh) + nz
                        carriers.append((layer, b, g, int(pages[c]), int(slots[c]), h))
                # tokens past the sequence end stay zero
                valid = (np.arange(n_pages * B) < n_tok).reshape(n_pages, B)
                keys = np.where(valid[..., None], keys, 0.0)
                vals = np.where(valid[..., None], vals, 0.0)
                blk = block_table[b, :n_pages]
                k_cache[layer, blk, g] = f32_to_bf16_bits(keys)
                v_cache[layer, blk, g] = f32_to_bf16_bits(vals)
    return KVInputs(w, k_cache, v_cache, q, block_table, seq_lens, carriers)

"""Device generator: the synth recipe drawn on the GPU (for workloads too
large for host memory).  Returns torch tensors in the library's layout:
  k, v : bf16 [layers, num_blocks, hkv, 16, 128]
  q    : bf16 [layers, batch, hq, 128]
  block_table int32 [batch, total_pages], seq_lens int32 [batch]
Carrier positions are drawn on the host (numpy) and planted on the device.
"""

import ctypes
import math
import os

import numpy as np
import torch

from .workloads import Workload

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.path.join(_HERE, "libsynth.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} missing: run __graft_entry__.build()")
        h = ctypes.CDLL(path)
        P, I64, I32, U32, F = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32,
                               ctypes.c_float)
        h.synth_fill_q.argtypes = [P, I64, U32, U32, P]
        h.synth_fill_pages.argtypes = [P, P, I64, I64, I64, P, P, I32, I32, I32, U32, U32, F, I32, P]
        h.synth_plant_carriers.argtypes = [P, I64, I64, I64, P, I32, P, I32, P, I32, U32, U32, F, P]
        h.synth_copy.argtypes = [P, P, I64, P]
        h.synth_read.argtypes = [P, I64, P, I32, P]
        for f in (h.synth_fill_q, h.synth_fill_pages, h.synth_plant_carriers, h.synth_copy,
                  h.synth_read):
            f.restype = I32
        _lib = h
    return _lib


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _s():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class DeviceInputs:
    def __init__(self, w, k, v, q, block_table, seq_lens, carriers):
        self.w, self.k, self.v, self.q = w, k, v, q
        self.block_table, self.seq_lens, self.carriers = block_table, seq_lens, carriers


def generate_device(w: Workload, device="cuda", seq_lens=None, layers=None) -> DeviceInputs:
    L = w.layers if layers is None else layers
    seq = np.full(w.batch, w.ctx, np.int32) if seq_lens is None else np.asarray(seq_lens, np.int32)
    P = w.total_pages
    nb = w.num_blocks
    root = np.random.default_rng([w.seed, 0xB10C])
    phys = np.arange(nb, dtype=np.int32)
    if w.shuffled_blocks:
        phys = root.permutation(nb).astype(np.int32)
    bt = phys.reshape(w.batch, P)
    k = torch.empty((L, nb, w.hkv, w.page, w.d), dtype=torch.bfloat16, device=device)
    v = torch.empty_like(k)
    q = torch.empty((L, w.batch, w.hq, w.d), dtype=torch.bfloat16, device=device)
    bt_d = torch.from_numpy(np.ascontiguousarray(bt)).to(device)
    seq_d = torch.from_numpy(seq).to(device)
    h = lib()
    bs, hs, ts = w.hkv * w.page * w.d, w.page * w.d, w.d
    carriers_all = []
    for layer in range(L):
        st = h.synth_fill_q(_p(q[layer]), q[layer].numel(), w.seed, layer, _s())
        assert st == 0, st
        st = h.synth_fill_pages(_p(k[layer]), _p(v[layer]), bs, hs, ts, _p(bt_d), _p(seq_d),
                                w.batch, w.hkv, P, w.seed, layer, math.sqrt(w.noise_var),
                                1 if w.coef_var_is_inv_k else 0, _s())
        assert st == 0, st
        rng = np.random.default_rng([w.seed, layer, 0xCA])
        car = []
        for b in range(w.batch):
            n_fin = int(seq[b]) // w.page
            for g in range(w.hkv):
                n_car = min(w.carriers, n_fin)
                if n_car == 0:
                    continue
                pages = rng.choice(n_fin, size=n_car, replace=False)
                slots = rng.integers(0, w.page, size=n_car)
                for c in range(n_car):
                    car.append((b, g, int(pages[c]), int(slots[c]), g * w.group + c % w.group))
        if car:
            ca = torch.tensor(car, dtype=torch.int32, device=device)
            st = h.synth_plant_carriers(_p(k[layer]), bs, hs, ts, _p(bt_d), P, _p(q[layer]), w.hq,
                                        _p(ca), len(car), w.seed, layer, math.sqrt(w.noise_var),
                                        _s())
            assert st == 0, st
        carriers_all.extend((layer,) + c for c in car)
    return DeviceInputs(w, k, v, q, bt_d, seq_d, carriers_all)


def device_copy(dst: torch.Tensor, src: torch.Tensor):
    """Plain streaming copy of src into dst (same byte size)."""
    n = src.numel() * src.element_size()
    st = lib().synth_copy(_p(dst), _p(src), n, _s())
    assert st == 0, st


def device_read(src: torch.Tensor, sink: torch.Tensor, blocks: int = 8192):
    """Plain streaming read of src (reduced into sink, >= 4*blocks uint32)."""
    n = src.numel() * src.element_size()
    st = lib().synth_read(_p(src), n, _p(sink), blocks, _s())
    assert st == 0, st

"""Named synthetic workloads (shapes only; no arithmetic of the method).

All share head dim 128, page size 16, rank 8 and bf16 K/V/q.  Sizes follow
the decode settings the LOCKS pages discuss: a Llama-3.1-8B-shaped cache
(32 layers, 32 query heads over 8 KV heads), contexts from 32K to 1M tokens
and a 2048-token attention budget (LOCKS abstract; technical summary sec. 3,
efficiency results).
"""

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    batch: int
    ctx: int            # tokens per sequence
    hq: int             # query heads
    hkv: int            # KV heads
    budget_tokens: int  # attention budget in tokens
    carriers: int       # carrier pages per (layer, sequence, KV head)
    d: int = 128
    page: int = 16
    rank: int = 8
    seed: int = 0
    noise_var: float = 0.05     # variance of the additive key noise
    coef_var_is_inv_k: bool = True  # a_ik ~ N(0, 1/k) as a variance
    shuffled_blocks: bool = False

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def pages(self) -> int:
        """Finalized pages per sequence (a partial tail page is not counted)."""
        return self.ctx // self.page

    @property
    def total_pages(self) -> int:
        """Pages per sequence including a partial tail page."""
        return -(-self.ctx // self.page)

    @property
    def budget_pages(self) -> int:
        return self.budget_tokens // self.page

    @property
    def num_blocks(self) -> int:
        """Physical KV blocks per layer (every sequence owns its own blocks)."""
        return self.batch * self.total_pages

    def kv_bytes_per_layer(self) -> int:
        return 2 * self.num_blocks * self.hkv * self.page * self.d * 2

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # 1 layer, 1 KV head, GQA 4, 4096 tokens = 256 pages, budget 512 tokens.
    "tiny-4k": Workload("tiny-4k", layers=1, batch=1, ctx=4096, hq=4, hkv=1,
                        budget_tokens=512, carriers=4),
    # One Llama-3.1-8B-shaped layer at 32K context.
    "llama8b-32k": Workload("llama8b-32k", layers=1, batch=1, ctx=32768, hq=32,
                            hkv=8, budget_tokens=2048, carriers=16),
    # 32 layers resident, batch 8 at 128K each.
    "llama8b-128k-b8": Workload("llama8b-128k-b8", layers=32, batch=8,
                                ctx=131072, hq=32, hkv=8,
                                budget_tokens=2048, carriers=16),
    # 32 layers, one sequence of 1M tokens (65,536 pages per KV head).
    "llama8b-1m": Workload("llama8b-1m", layers=32, batch=1, ctx=1048576,
                           hq=32, hkv=8, budget_tokens=2048, carriers=16),
    # 8 layers, batch 16 at 256K, doubled carrier density.
    "llama8b-256k-b16": Workload("llama8b-256k-b16", layers=8, batch=16,
                                 ctx=262144, hq=32, hkv=8,
                                 budget_tokens=2048, carriers=32),
}


def get_workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.with_(**overrides) if overrides else w

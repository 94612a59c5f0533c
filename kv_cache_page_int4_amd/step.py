"""A whole LOCKS decode step over all layers, captured in one HIP graph.

The decode step (technical summary sec. 2, implementation paragraph: scoring,
selection and sparse attention run inside one full graph with no Python
dispatch) is, per layer, locks_decode_layer (locks_score_select followed by
locks_sparse_attend, with the last selection stage inside the attention).

Incremental finalization (a page is summarized once, when the token that
fills it arrives, off the decode critical path) comes in two forms:

  * finalize="step" (or True): the page that the step's token completes is
    summarized after the step, for every layer in one launch, and selected
    from the next step on.  During the step the page that holds the newest
    token is not summarized yet, so the step's calls run with
    newest_page_pending = 1: that page is attended in full, as the tail, and
    the build is off the step's critical path.
  * finalize="layer": the page is summarized inside the step, per layer,
    before that layer is scored (newest_page_pending = 0).  In a model the
    newest token's key of layer l is written during layer l, so the build of
    that layer's page sits on the layer's path.

An optional before_layer(l) callback, recorded into the graph too, stands for
the model's work that precedes layer l's attention (appending the token's key
and value, for instance).
This module only allocates the per-layer outputs and the workspaces, issues
the library calls in order on the current stream and records them into a
torch.cuda.CUDAGraph (a hipGraph on ROCm).  Layers run in sequence because in
a model layer l+1's query depends on layer l's output.
"""

import torch

from . import locks as L


class DecodeStep:
    """k, v: bf16 [layers, blocks, hkv, 16, 128]; summaries: uint8
    [layers, hkv, blocks, record bytes]; q: bf16 [layers, batch, hq, 128];
    block_table: int32 [batch, max_pages]; seq_lens: int32 [batch].
    dense=True attends every summarized page instead (no scoring/selection);
    finalize="step" (or True) summarizes the pages the step's token completed
    after the step, all layers in one launch, and runs the step's calls with
    the newest page pending; finalize="layer" summarizes them per layer before
    the layer is scored; before_layer(layer) is called (and captured) at the
    head of every layer;
    fused=True issues each layer as one locks_decode_layer call (the last
    selection stage runs inside the attention kernel), fused=False as
    locks_score_select + locks_sparse_attend.  n_tables sets the number of
    selection tables per sequence (default: one per KV head; 1: one table for
    the whole layer); sel and cnt then hold n_tables rows per sequence."""

    def __init__(self, d, k, v, summaries, q, block_table, seq_lens, budget_pages, dense=False,
                 finalize=False, fused=True, n_tables=None, before_layer=None):
        if finalize is True:
            finalize = "step"
        if finalize not in (False, None, "step", "layer"):
            raise ValueError(f"finalize must be False, True, 'step' or 'layer', not {finalize!r}")
        if finalize == "step":   # the step's newest page is summarized after it
            d = L.dims(d.num_q_heads, d.num_kv_heads, d.head_dim, d.page_size, d.rank,
                       newest_page_pending=True)
        self.d, self.k, self.v, self.summ, self.q = d, k, v, summaries, q
        self.bt, self.seq, self.budget, self.dense = block_table, seq_lens, budget_pages, dense
        self.finalize = finalize or False
        self.before_layer = before_layer
        self.fused = fused
        self.n_tables = n_tables
        ntab = d.num_kv_heads if n_tables is None else n_tables
        n_layers, batch = q.shape[0], q.shape[1]
        P = block_table.shape[1]
        dev = q.device
        self.layers = n_layers
        self.num_blocks = k.shape[1]
        self.sel = torch.full((n_layers, batch, ntab, budget_pages), -1, dtype=torch.int32,
                              device=dev)
        self.cnt = torch.zeros((n_layers, batch, ntab), dtype=torch.int32, device=dev)
        self.out = torch.zeros((n_layers, batch, d.num_q_heads, d.head_dim), dtype=torch.bfloat16,
                               device=dev)
        self.out_lse = torch.zeros((n_layers, batch, d.num_q_heads), dtype=torch.float32, device=dev)
        self.ws_score = torch.empty(max(1, L.score_workspace_bytes(d, batch, P, budget_pages)),
                                    dtype=torch.uint8, device=dev)
        n_att = (P if dense else budget_pages) + 1
        self.ws_att = L.attend_workspace(d, batch, n_att, device=dev)
        # page scores for the three-call path with several KV heads per table
        self.lse = (torch.empty((batch, d.num_q_heads, P), dtype=torch.float32, device=dev)
                    if n_tables is not None and not fused and not dense else None)
        self.graph = None

    def run_layer(self, layer, stream=None):
        d = self.d
        if self.before_layer is not None:
            self.before_layer(layer)
        if self.finalize == "layer":   # the page this layer's newest key completed, if any
            L.finalize_pages(d, self.k[layer], self.bt, self.seq, self.summ[layer], stream=stream)
        if not self.dense and self.fused:
            L.decode_layer(d, self.q[layer], self.summ[layer], self.k[layer], self.v[layer],
                           self.bt, self.seq, self.budget, self.sel[layer], self.cnt[layer],
                           self.out[layer], self.ws_score, self.ws_att,
                           out_lse=self.out_lse[layer], stream=stream, n_tables=self.n_tables)
            return
        if not self.dense and self.n_tables is None:
            L.score_select(d, self.q[layer], self.summ[layer], self.num_blocks, self.bt, self.seq,
                           self.budget, self.sel[layer], self.cnt[layer], self.ws_score,
                           stream=stream)
        elif not self.dense:
            L.score_pages(d, self.q[layer], self.summ[layer], self.num_blocks, self.bt, self.seq,
                          self.lse, self.ws_score, stream=stream)
            L.select_pages(d, self.lse, self.seq, self.budget, self.sel[layer], self.cnt[layer],
                           self.ws_score, stream=stream, n_tables=self.n_tables)
        L.sparse_attend(d, self.q[layer], self.k[layer], self.v[layer], self.bt, self.seq,
                        None if self.dense else self.sel[layer],
                        None if self.dense else self.cnt[layer], self.budget, self.out[layer],
                        self.ws_att, out_lse=self.out_lse[layer], stream=stream,
                        n_tables=self.n_tables)

    def run(self):
        for layer in range(self.layers):
            self.run_layer(layer)
        if self.finalize == "step":    # every layer's completed page, off the step's path
            L.finalize_pages(self.d, self.k, self.bt, self.seq, self.summ)

    def capture(self):
        """Record one full step into a graph (after one eager warm-up run)."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.run()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run()
        torch.cuda.synchronize()
        self.graph = g
        return g

    def replay(self):
        self.graph.replay()


def build_all_layers(d, k, summaries, blocks=None):
    """Summarize the given physical blocks (int32 device tensor; default:
    every block) of every layer (prefill finalization)."""
    n_layers, nb = k.shape[0], k.shape[1]
    if blocks is None:
        blocks = torch.arange(nb, dtype=torch.int32, device=k.device)
    for layer in range(n_layers):
        L.build_summaries(d, k[layer], blocks, summaries[layer])

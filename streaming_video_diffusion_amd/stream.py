"""One streaming chunk's attention through libstreamattn.

A ``ChunkAttention`` owns the persistent packed K/V buffers of one layer and
one denoising-step bank. The static prefix (style-prompt K/V and the session
reference frame) is packed once; every chunk then rebuilds the rotary tables
of its position template, rewrites the dynamic region (history tiers and the
current chunk) in place and runs the forward pass. This is the sequence the
pages describe: prefix K/V computed once per denoising step and reused, only
recent history and the current chunk recomputed, one cache bank per step,
persistent per-layer buffers updated in place (StreamRender-H3 page,
streaming-context and inference-acceleration sections).

Device memory comes from torch; every step of the computation runs in the
library's HIP kernels.
"""

import numpy as np
import torch

from . import binding as B


class ChunkAttention:
    """Persistent context + inputs of one attention call of a workload.

    ``workload`` is an ``inputs.Workload``; ``call`` selects the denoising
    step (its own bank and its own seeded tensors).
    """

    def __init__(self, workload, call=0, device="cuda", out_dtype=None):
        w = workload
        self.w = w
        self.call = call
        self.device = device
        self.dtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.out_dtype = out_dtype or self.dtype
        dev = torch.device(device)

        def up(x):
            return torch.from_numpy(x).to(dev).to(self.dtype)

        self.q = up(w.q(call))
        self.q_pos = torch.from_numpy(w.q_pos).to(dev) if w.q_pos is not None else None
        self.q_table = (torch.empty((w.nq, w.head_dim // 2, 2), dtype=torch.float32, device=dev)
                        if w.q_pos is not None else None)
        self.segs = []
        row = 0
        for i, s in enumerate(w.segments):
            k, v = w.kv(i, call)
            # A dynamic segment at exactly the query positions reuses the query table
            # (built with the dynamic tables; static segments are packed before it).
            shares_q = (s.dynamic and s.pos is not None and w.q_pos is not None
                        and s.pos.shape == w.q_pos.shape and np.array_equal(s.pos, w.q_pos))
            pos = None
            table = None
            if s.pos is not None and not shares_q and s.rows > 0:
                pos = torch.from_numpy(s.pos).to(dev)
                table = torch.empty((s.rows, w.head_dim // 2, 2), dtype=torch.float32, device=dev)
            pool = (s.pool, s.grid[0], s.grid[1]) if s.pool > 1 else None
            self.segs.append(dict(name=s.name, k=up(k), v=up(v), pos=pos, table=table, dst=row,
                                  dynamic=s.dynamic, rotary=s.pos is not None, shares_q=shares_q, pool=pool))
            row += s.rows
        self.q_norm = self.k_norm = None
        weights = w.norm_weights()
        if weights is not None:
            qw, kw = (torch.from_numpy(x).to(dev) for x in weights)
            self.q_norm, self.k_norm = B.Norm(qw, w.norm_eps), B.Norm(kw, w.norm_eps)
        self.ctx = B.PackedContext(w.heads, w.head_dim, self.dtype, w.nk, device=dev)
        self.ctx.rows = w.nk
        self.out = torch.empty((w.nq, w.heads, w.head_dim), dtype=self.out_dtype, device=dev)
        # Workspace that lets the forward balance its last round of workgroups
        # (allocated once; None when the forward would not use it).
        ws = B.sa_forward_workspace_bytes(self.ctx, w.nq)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=dev) if ws else None

    def _tables(self, dynamic, stream):
        w = self.w
        if dynamic and self.q_table is not None:
            B.sa_make_rope_tables(self.q_pos, w.head_dim, w.axis_dims, w.theta, table=self.q_table, stream=stream)
        for s in self.segs:
            if s["dynamic"] == dynamic and s["table"] is not None:
                B.sa_make_rope_tables(s["pos"], w.head_dim, w.axis_dims, w.theta, table=s["table"], stream=stream)

    def _pack(self, dynamic, stream):
        segs = []
        for s in self.segs:
            if s["dynamic"] != dynamic:
                continue
            rope = self.q_table if s["shares_q"] else (s["table"] if s["rotary"] else None)
            segs.append((s["k"], s["v"], s["dst"], rope, self.k_norm, s["pool"]))
        B.sa_pack_context(self.ctx, segs, stream=stream)

    def pack_static(self, stream=None):
        """Build the static prefix's tables and pack it (once per bank)."""
        self._tables(False, stream)
        self._pack(False, stream)

    def step(self, stream=None, rebuild_tables=True):
        """One chunk: rotary tables of the template, dynamic pack, forward."""
        if rebuild_tables:
            self._tables(True, stream)
        self._pack(True, stream)
        return self.forward(stream)

    def forward(self, stream=None):
        B.sa_forward_ws(self.ctx, self.q, self.q_table, self.w.scale, out=self.out, stream=stream,
                        q_norm=self.q_norm, workspace=self.workspace)
        return self.out

    def host_inputs(self):
        """The exact host values fed to the device (for the oracle): queries,
        query positions and ``(k, v, pos)`` per segment; a pooled segment gives
        its full-resolution frames as ``(k, v, pos, (grid_h, grid_w, s))``."""
        w = self.w
        segs = []
        for i, s in enumerate(w.segments):
            k, v = w.kv(i, self.call)
            segs.append((k, v, s.pos, (s.grid[0], s.grid[1], s.pool)) if s.pool > 1 else (k, v, s.pos))
        return w.q(self.call), w.q_pos, segs

    def host_norms(self):
        """QK-norm of queries and keys as ``(weight, eps)`` host pairs, or ``(None, None)``."""
        weights = self.w.norm_weights()
        if weights is None:
            return None, None
        return (weights[0], self.w.norm_eps), (weights[1], self.w.norm_eps)

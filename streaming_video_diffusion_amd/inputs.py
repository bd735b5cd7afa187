"""Seeded synthetic workloads for streaming-chunk attention.

This module holds no arithmetic of the method (no rotary angles, no
attention): only shapes, token positions and seeded random draws. Both the GPU
path's callers and the fp64 oracle's tests take their inputs from here.

Shapes follow the streaming renderer the pages describe: 1344x768 video at
24 fps (StreamRender-H3 page, data section), a video VAE that compresses 16x in
space and 4x in time (MiniMax-H3 deep-dive page, components table, VisualVAE
row), so one latent frame of 1344x768 is an 84x48 token grid, 40 Hz audio
latents (same table, AudioVAE row), head dimension 128 (DiT configuration
table), and a key/value context made of a persistent style prompt, the
session's reference frame, clean history (optionally coarser tiers for older
history) and the current chunk (AlayaRenderer-Flash page, key contributions
and technical details). Real latents, trained weights and the pages' datasets
are not used; every tensor is i.i.d. N(0, 1) (standing in for the unit-RMS
rows that QK-norm produces), rounded to bfloat16 with round-to-nearest-even
for bf16 workloads.

Readings of points the pages leave open (each one is only input data):

* token order inside a latent frame is row-major over the grid (h, then w);
  position (t, h, w) = (latent frame index, grid row, grid column);
* t counts latent frames from the reference frame (t = 0), through the history
  segments oldest first, to the current chunk;
* a spatially pooled history tier keeps its frame index and places each pooled
  cell at the centre of the full-resolution cells it covers:
  ``h = s*i + (s-1)/2`` (likewise w) for pooling factor s;
* audio token a of a segment that starts at latent frame t0 sits at
  ``t = t0 + 0.15*a`` (40 Hz in units of 6 Hz latent frames: 24 fps / 4),
  ``h = w = 0``; audio rows follow the video rows of their segment;
* the style-prompt segment carries no position (no rotary encoding).
"""

from dataclasses import dataclass, field
import math

import numpy as np

# Fixed entropy of every seeded draw (recorded in bench output).
ENTROPY = 0x5EED_A77E

# Rotary base and band split of the head dimension over (t, h, w).
ROPE_THETA = 10000.0
AXIS_DIMS = {64: (16, 24, 24), 128: (32, 48, 48)}


def round_bf16(x):
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16. NaN is
    not expected in synthetic inputs and is not special-cased.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    r = ((u + bias) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32).reshape(x.shape)


def frame_positions(t_values, grid_h, grid_w, pool=1):
    """(t, h, w) of every token of the given latent frames, row-major grid.

    ``pool`` > 1 gives the positions of a ``pool x pool`` spatially pooled
    tier: ``grid_h / pool`` by ``grid_w / pool`` cells, each at the centre of
    the full-resolution cells it covers.
    """
    gh, gw = grid_h // pool, grid_w // pool
    off = (pool - 1) / 2.0
    hh, ww = np.meshgrid(np.arange(gh, dtype=np.float64) * pool + off,
                         np.arange(gw, dtype=np.float64) * pool + off, indexing="ij")
    out = []
    for t in t_values:
        f = np.empty((gh * gw, 3), dtype=np.float64)
        f[:, 0] = t
        f[:, 1] = hh.reshape(-1)
        f[:, 2] = ww.reshape(-1)
        out.append(f)
    return np.concatenate(out, axis=0).astype(np.float32)


def audio_positions(t0, count, step=0.15):
    """Positions of ``count`` 40 Hz audio tokens starting at latent frame t0."""
    p = np.zeros((count, 3), dtype=np.float64)
    p[:, 0] = t0 + step * np.arange(count, dtype=np.float64)
    return p.astype(np.float32)


@dataclass
class Segment:
    """One part of the key/value context, in pack order."""
    name: str
    rows: int
    pos: object          # float32 [rows][3] or None (no rotary encoding)
    dynamic: bool        # re-packed every chunk (False: persistent prefix)
    pool: int = 1        # > 1: rows are s x s spatial means the pack forms from full-resolution frames
    grid: tuple = None   # (grid_h, grid_w) of those full-resolution frames

    @property
    def src_rows(self):
        """Rows of the segment's source tensors (full resolution when pooled)."""
        return self.rows * self.pool * self.pool


@dataclass
class Workload:
    """One attention call's shapes, positions and seeded values."""
    name: str
    cfg_id: int
    dtype: str                  # "bf16" or "f32": Q/K/V element type
    heads: int
    head_dim: int
    q_pos: object               # float32 [Nq][3] or None
    segments: list
    calls: int = 1              # sequential denoise calls (own bank each)
    theta: float = ROPE_THETA
    axis_dims: tuple = None
    scale: float = None
    description: str = ""
    q_rows: int = None          # Nq; taken from q_pos when that is given
    meta: dict = field(default_factory=dict)
    qk_norm: str = None         # None, "shared" ([d] weights) or "per_head" ([H][d] weights)
    norm_eps: float = 1e-6

    def __post_init__(self):
        if self.q_rows is None:
            self.q_rows = 0 if self.q_pos is None else int(self.q_pos.shape[0])
        if self.axis_dims is None:
            self.axis_dims = AXIS_DIMS[self.head_dim]
        if self.scale is None:
            self.scale = 1.0 / math.sqrt(self.head_dim)

    @property
    def nq(self):
        return int(self.q_rows)

    @property
    def nk(self):
        return int(sum(s.rows for s in self.segments))

    def flops_per_call(self):
        """Q.K^T and P.V multiply-adds, 2 flops each: 4*Nq*Nk*d*H."""
        return 4.0 * self.nq * self.nk * self.head_dim * self.heads

    def _draw(self, call, tensor_id, rows):
        ss = np.random.SeedSequence([ENTROPY, self.cfg_id, call, tensor_id])
        rng = np.random.default_rng(ss)
        x = rng.standard_normal((rows, self.heads, self.head_dim), dtype=np.float32)
        return round_bf16(x) if self.dtype == "bf16" else x

    def q(self, call=0):
        """Queries of call ``call``: float32 [Nq][H][d] (bf16-exact for bf16)."""
        return self._draw(call, 0, self.nq)

    def kv(self, seg, call=0):
        """Keys and values of segment index ``seg`` for call ``call`` (the
        full-resolution frames of a pooled segment)."""
        rows = self.segments[seg].src_rows
        return self._draw(call, 1 + 2 * seg, rows), self._draw(call, 2 + 2 * seg, rows)

    def norm_weights(self):
        """QK-norm weights (query, key): float32 [d] or [H][d], drawn as
        1 + 0.2 N(0, 1); ``None`` when the workload has no QK-norm."""
        return _norm_weights(self.cfg_id, self.heads, self.head_dim, self.qk_norm)


def _norm_weights(cfg_id, heads, head_dim, kind):
    if kind is None:
        return None
    shape = (head_dim,) if kind == "shared" else (heads, head_dim)
    out = []
    for tensor_id in (900, 901):
        rng = np.random.default_rng(np.random.SeedSequence([ENTROPY, cfg_id, tensor_id]))
        out.append((1.0 + 0.2 * rng.standard_normal(shape)).astype(np.float32))
    return tuple(out)


def _video_segments(prompt, grid_h, grid_w, ref_t, tiers, cur_t, audio=0, produce=False):
    """Build segments: prompt, ref, history tiers (oldest first), current.
    ``produce``: pooled tiers are formed by the pack from full-resolution
    frames (else they are given at their pooled size)."""
    segs = [Segment("prompt", prompt, None, False),
            Segment("ref", grid_h * grid_w, frame_positions([ref_t], grid_h, grid_w), False)]
    for name, t_values, pool in tiers:
        pos = frame_positions(t_values, grid_h, grid_w, pool)
        if audio and pool == 1:
            pos = np.concatenate([pos, audio_positions(t_values[0], audio)])
        if produce and pool > 1:
            segs.append(Segment(name, int(pos.shape[0]), pos, True, pool=pool, grid=(grid_h, grid_w)))
        else:
            segs.append(Segment(name, int(pos.shape[0]), pos, True))
    cur = frame_positions(cur_t, grid_h, grid_w)
    if audio:
        cur = np.concatenate([cur, audio_positions(cur_t[0], audio)])
    segs.append(Segment("current", int(cur.shape[0]), cur, True))
    return segs, cur


def tiny_f32():
    """Tiny f32 case: 1 head, d 64, one 12x8 latent frame per segment."""
    segs, cur = _video_segments(16, 8, 12, 0, [("history", [1], 1)], [2])
    return Workload("tiny_f32", 1, "f32", 1, 64, cur, segs,
                    description="tiny f32: 96 q x 304 kv, 1 head, d64")


def lowres_bf16():
    """Low-resolution bf16 chunk: 8 heads, d 128, 21x12 grid, 3 latent frames."""
    segs, cur = _video_segments(64, 12, 21, 0, [("history", [1, 2, 3], 1)], [4, 5, 6])
    return Workload("lowres_bf16", 2, "bf16", 8, 128, cur, segs,
                    description="low-res bf16: 756 q x 1828 kv, 8 heads, d128")


def full_1344x768():
    """The 1344x768 chunk of 3 latent frames (84x48 grid), 40 heads, d 128."""
    segs, cur = _video_segments(256, 48, 84, 0, [("history", [1, 2, 3], 1)], [4, 5, 6])
    return Workload("full_1344x768", 3, "bf16", 40, 128, cur, segs,
                    description="1344x768 chunk: 12096 q x 28480 kv, 40 heads, d128")


def hier_1344x768():
    """1344x768 chunk with 4x4- and 2x2-pooled older history tiers."""
    tiers = [("pool4", [1, 2, 3], 4), ("pool2", [4, 5, 6], 2), ("prev", [7, 8, 9], 1)]
    segs, cur = _video_segments(256, 48, 84, 0, tiers, [10, 11, 12])
    return Workload("hier_1344x768", 4, "bf16", 40, 128, cur, segs,
                    description="1344x768 hierarchical history: 12096 q x 32260 kv, 40 heads, d128")


def hier_pooled(name, cfg_id, dtype, heads, head_dim, grid_h, grid_w, prompt, qk_norm=None):
    """Hierarchical history whose pooled tiers the pack produces from
    full-resolution frames: 4x4 tier of frames 1-3, 2x2 tier of frames 4-6,
    full-resolution previous chunk 7-9, current chunk 10-12."""
    tiers = [("pool4", [1, 2, 3], 4), ("pool2", [4, 5, 6], 2), ("prev", [7, 8, 9], 1)]
    segs, cur = _video_segments(prompt, grid_h, grid_w, 0, tiers, [10, 11, 12], produce=True)
    return Workload(name, cfg_id, dtype, heads, head_dim, cur, segs, qk_norm=qk_norm,
                    description=f"hierarchical history, pooled tiers produced from full resolution: "
                                f"{3 * grid_h * grid_w} q, {heads} heads, d{head_dim}")


def hier_pooled_1344x768():
    """The hierarchical 1344x768 context with its 4x4 and 2x2 tiers pooled by
    the pack from full-resolution frames (same attention shape: 12096 q x 32260 kv)."""
    return hier_pooled("hier_pooled_1344x768", 9, "bf16", 40, 128, 48, 84, 256)


def video_audio_1344x768():
    """1 s joint video+audio chunk (6 latent frames + 40 audio tokens), 2 calls."""
    segs, cur = _video_segments(256, 48, 84, 0, [("history", [1, 2, 3, 4, 5, 6], 1)],
                                [7, 8, 9, 10, 11, 12], audio=40)
    return Workload("video_audio_1344x768", 5, "bf16", 40, 128, cur, segs, calls=2,
                    description="1344x768 video+audio 1 s chunk: 24232 q x 52752 kv, 40 heads, d128, 2 calls")


CONFIGS = {w().name: w for w in (tiny_f32, lowres_bf16, full_1344x768, hier_1344x768,
                                 video_audio_1344x768)}


# Query-side variants on the same kernel (StreamRender-H3 page, streaming-context
# section): at inference the recent history is recomputed together with the
# current chunk; the first window, having no earlier context, generates seven
# scheduling units at once; the fixed prefix (conditions, reference, sink)
# attends only to itself when its key/values are computed. One scheduling unit
# is read as one latent frame (the page gives one to two) and the sink as two
# units, as in the deployed model the page describes.

def history_query_1344x768():
    """Recomputed history + current chunk as queries over the 1344x768 context."""
    segs, cur = _video_segments(256, 48, 84, 0, [("history", [1, 2, 3], 1)], [4, 5, 6])
    q_pos = np.concatenate([segs[2].pos, cur])
    return Workload("history_query_1344x768", 6, "bf16", 40, 128, q_pos, segs,
                    description="1344x768 history+current as queries: 24192 q x 28480 kv, 40 heads, d128")


def first_window_1344x768():
    """First window: seven latent frames generated at once over prompt + reference + themselves."""
    segs, cur = _video_segments(256, 48, 84, 0, [], [1, 2, 3, 4, 5, 6, 7])
    return Workload("first_window_1344x768", 7, "bf16", 40, 128, cur, segs,
                    description="1344x768 first window: 28224 q x 32512 kv, 40 heads, d128")


def prefix_self_1344x768():
    """Prefix pass: reference + two sink frames attend to prompt + themselves only."""
    segs = [Segment("prompt", 256, None, False),
            Segment("ref", 4032, frame_positions([0], 48, 84), False),
            Segment("sink", 8064, frame_positions([1, 2], 48, 84), False)]
    q_pos = np.concatenate([segs[1].pos, segs[2].pos])
    return Workload("prefix_self_1344x768", 8, "bf16", 40, 128, q_pos, segs,
                    description="1344x768 prefix self-attention: 12096 q x 12352 kv, 40 heads, d128")


VARIANTS = {w().name: w for w in (history_query_1344x768, first_window_1344x768, prefix_self_1344x768)}


@dataclass
class TierStream:
    """Inputs of a chunk-by-chunk stream whose history ages through coarser
    tiers: a style prompt and a reference frame fixed for the session, and
    every chunk's queries, keys and values (``frames`` latent frames of
    ``grid_h`` x ``grid_w`` tokens), drawn per chunk index. Positions come
    from one fixed template: reference at t = 0, then ``slots`` history slots
    of ``frames`` frames each (oldest first), then the current chunk; a slot
    pooled s x s places each cell at the centre of the cells it covers. Which
    chunk fills which slot is the stream's business, not this class's.
    """
    name: str
    cfg_id: int
    dtype: str
    heads: int
    head_dim: int
    grid_h: int
    grid_w: int
    frames: int
    prompt: int
    slots: int = 3
    theta: float = ROPE_THETA
    axis_dims: tuple = None
    scale: float = None
    description: str = ""
    qk_norm: str = None         # None, "shared" ([d] weights) or "per_head" ([H][d] weights)
    norm_eps: float = 1e-6

    def __post_init__(self):
        if self.axis_dims is None:
            self.axis_dims = AXIS_DIMS[self.head_dim]
        if self.scale is None:
            self.scale = 1.0 / math.sqrt(self.head_dim)

    def norm_weights(self):
        """QK-norm weights (query, key) as for ``Workload``, or ``None``."""
        return _norm_weights(self.cfg_id, self.heads, self.head_dim, self.qk_norm)

    @property
    def chunk_rows(self):
        return self.frames * self.grid_h * self.grid_w

    def _draw(self, chunk, tensor_id, rows):
        # chunk -1 is the session's static part; seed words must be non-negative
        rng = np.random.default_rng(np.random.SeedSequence([ENTROPY, self.cfg_id, chunk + 1, tensor_id]))
        x = rng.standard_normal((rows, self.heads, self.head_dim), dtype=np.float32)
        return round_bf16(x) if self.dtype == "bf16" else x

    def static_kv(self):
        """``[(k, v, pos_or_None)]`` of the prompt (no rotary) and the reference frame (t = 0)."""
        ref_rows = self.grid_h * self.grid_w
        return [(self._draw(-1, 1, self.prompt), self._draw(-1, 2, self.prompt), None),
                (self._draw(-1, 3, ref_rows), self._draw(-1, 4, ref_rows),
                 frame_positions([0], self.grid_h, self.grid_w))]

    def chunk_q(self, c):
        return self._draw(c, 0, self.chunk_rows)

    def chunk_kv(self, c):
        """Full-resolution keys and values of chunk ``c``."""
        return self._draw(c, 1, self.chunk_rows), self._draw(c, 2, self.chunk_rows)

    def slot_t(self, slot):
        """Frame indices of history slot ``slot`` (0 = oldest); ``slot = slots`` is the current chunk."""
        return list(range(1 + slot * self.frames, 1 + (slot + 1) * self.frames))

    def slot_positions(self, slot, pool=1):
        return frame_positions(self.slot_t(slot), self.grid_h, self.grid_w, pool)


def tier_stream_small(dtype="bf16", head_dim=128):
    """A small tiered stream: 16 x 12 grid, 3 frames per chunk, 3 heads."""
    return TierStream(f"tier_stream_small_{dtype}_d{head_dim}", 20 + head_dim // 64 + (dtype == "f32") * 4, dtype, 3,
                      head_dim, 12, 16, 3, 40, description="tiered history stream, 16x12 grid, 3 frames per chunk")


def tier_stream_1344x768():
    """The 1344x768 tiered stream (84 x 48 grid, 3 latent frames per chunk, 40 heads, d 128): at steady state
    12096 queries over 256 + 4032 + 756 + 3024 + 12096 + 12096 = 32260 keys."""
    return TierStream("tier_stream_1344x768", 30, "bf16", 40, 128, 48, 84, 3, 256,
                      description="1344x768 tiered history stream: 12096 q x up to 32260 kv, 40 heads, d128")


def custom(name, cfg_id, dtype, heads, head_dim, seg_rows, nq, rotary=True, prompt_rows=0,
           pos_scale=40.0, axis_dims=None, theta=ROPE_THETA, scale=None, qk_norm=None):
    """Arbitrary-shape workload for tests: random positions, given row counts.

    ``seg_rows``: rows of each rotary segment after an optional prompt
    segment of ``prompt_rows`` rows. Positions are seeded uniform in
    ``[0, pos_scale)`` per axis and stored as float32.
    """
    rng = np.random.default_rng(np.random.SeedSequence([ENTROPY, cfg_id, 99]))

    def pos(n):
        return (rng.random((n, 3)) * pos_scale).astype(np.float32) if rotary else None

    segs = []
    if prompt_rows:
        segs.append(Segment("prompt", prompt_rows, None, False))
    for i, r in enumerate(seg_rows):
        segs.append(Segment(f"seg{i}", int(r), pos(int(r)), True))
    return Workload(name, cfg_id, dtype, heads, head_dim, pos(nq) if rotary else None, segs,
                    axis_dims=axis_dims, theta=theta, scale=scale, q_rows=nq, qk_norm=qk_norm)

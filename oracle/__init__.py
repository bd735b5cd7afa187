"""Independent fp64 CPU oracle for streaming-chunk DiT self-attention.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The product path (``streaming_video_diffusion_amd``) never imports it,
and this package imports nothing from the product path: the two share no
kernels, headers, helpers, tables or constants.

What it computes is the plain definition of the operation, in float64:

* ``rope64``  -- 3D (time, height, width) rotary position encoding: angles from
  positions and the per-pair rotation.
* ``norm64``  -- per-head RMS normalisation of queries and keys (QK-norm),
  applied before the rotation.
* ``pool64``  -- s x s spatial mean pooling of aged history frames into a
  coarser tier (of keys before their normalisation and rotation, and of values).
* ``tiers64`` -- which chunk feeds which history tier as chunks age (full
  resolution -> 2x2 -> 4x4 -> dropped) and the fixed position template.
* ``attn64``  -- dense softmax attention of the current chunk's queries over the
  concatenated key/value context (prompt KV | reference frame | history tiers |
  current chunk), vectorised with numpy per head and query block.
* ``brute``   -- the same definition as scalar Python loops with ``math.fsum``,
  used only on tiny inputs to pin ``attn64``.

Sources: the dense softmax attention with 3D MM-RoPE and QK-norm of the
MiniMax-H3 DiT (MiniMax-H3 deep-dive page, DiT configuration table and the
attention paragraph after it); the bidirectional, unmasked window whose moving
part sees the whole window (StreamRender-H3 page, section on streaming
context); persistent style-prompt key/values in every self-attention layer and
hierarchical history (AlayaRenderer-Flash page, key contributions and
technical details).

Every function here is pinned by ``tests/test_oracle_pins.py`` to closed forms,
invariants, a library routine (SDPA) and brute force; nothing is "parity
unpinned".
"""

from . import rope64, norm64, pool64, attn64, brute, tiers64  # noqa: F401

__all__ = ["rope64", "norm64", "pool64", "attn64", "brute", "tiers64"]

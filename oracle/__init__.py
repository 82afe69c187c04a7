"""fp64 CPU oracle for streaming chunk attention -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct NumPy code for what the GPU path computes:

* ``rope``      -- 3D (t, h, w) rotary position embedding of one head vector
                   per token (RoFormer's rotation, applied per axis segment).
* ``attention`` -- softmax attention of a chunk's queries over an explicit set
                   of visible keys, plus a scalar brute-force twin for tiny inputs.
* ``stream``    -- the stream semantics: a persistent sink chunk, a sliding
                   window of the most recent committed chunks, the current chunk
                   itself, RoPE offsets re-based ("refresh"), and sink updates
                   (StreamDiffusionV2, "Sommario tecnico" 2.A.2; SANA-Streaming,
                   "Transformer a diffusione ibrido"). Two formulations:
                   ``HistoryOracle`` (the definition: keep every committed chunk
                   raw, rotate at use time) and ``RingOracle`` (rotated keys in a
                   bounded ring, re-rotated on refresh, optionally rounding every
                   stored value to bfloat16 the way a bf16 device cache does).
* ``bf16``      -- direct float64 -> bfloat16 round-to-nearest-even.
* ``gdn``       -- the gated delta rule (GDN linear attention) as the plain token loop
                   (published Gated DeltaNet recurrence; the pages name the block only).
* ``fp8``       -- direct float64 -> E4M3 (OCP 8-bit float) round-to-nearest-even,
                   saturating at +-448, for the storage-emulating oracle of the
                   fp8 cache variant.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path (the C-ABI library and
its Python binding) never imports, links or calls anything here, and this
package imports nothing from the product path: the two share no code. The
only shared module is ``synth`` (seeded input generators, no method arithmetic).

Parity status: every function here is pinned by ``-m "not gpu"`` tests against
closed forms, library special cases, brute force and hand-worked expectations.
The conventions the pages leave open (RoPE axis split, base, pairing, the
temporal unit, refresh semantics) are readings, each stated in the module that
applies it; they cannot be pinned against the pages' own systems, which print
no formula or number for this path.
"""
from .bf16 import round_bf16, is_bf16_exact
from .fp8 import round_e4m3, is_e4m3_exact
from .gdn import gdn_recurrent
from .rope import rope_split, token_coords, rope_freqs, rope3d, rotate_temporal
from .attention import attend, attend_bruteforce, attention_probs
from .stream import StreamSpec, HistoryOracle, RingOracle, SHIFT_SINK, fp8_q_scale

__all__ = [
    "round_bf16", "is_bf16_exact", "round_e4m3", "is_e4m3_exact", "gdn_recurrent",
    "rope_split", "token_coords", "rope_freqs", "rope3d", "rotate_temporal",
    "attend", "attend_bruteforce", "attention_probs",
    "StreamSpec", "HistoryOracle", "RingOracle", "SHIFT_SINK", "fp8_q_scale",
]

"""CPU oracle for paged attention over an FP8/fp16 block-paged KV cache.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, float64 statement of
what the paged-attention path computes. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The HIP library never imports, links or calls anything here, and
nothing here imports the HIP library or its Python binding: the two share no
code. The only module both sides use is the seeded input generator
``attention_paged_flashattention_amd.synth``, which holds no attention or FP8
arithmetic.

Sources (cited by page title and section):

* "1Cat-vLLM 1.0.0" README, section "Optional experimental feature: FP8 KV
  cache" -- the KV cache may be stored as ``fp8_e5m2`` or ``fp8_e4m3``.
* "1Cat-vLLM 1.5.0" RELEASE notes, section "Flash-V100 long-context
  improvements" -- paged decode that reuses page ids per page, the grouped
  q8 verifier ("exact grouped q8 verification over FP8 E5M2 KV"), long-prefill
  GQA attention, "useful causal" FLOP accounting.
* "SM70 release profile and acceleration status" -- 2048-token KV pages, a
  4096-token prefill chunk budget, E4M3 KV for the release profile, and the
  statement that block tables use physical page units.

The FP8 formats themselves are not defined on those pages; ``oracle.fp8``
restates them from the OCP 8-bit floating point specification (OFP8, E4M3 and
E5M2 encodings).

Modules:

* ``oracle.fp8``       -- FP8 decode table, RNE+saturating encode, dequant.
* ``oracle.paged``     -- cache layout, write (quantize-on-write), gather.
* ``oracle.attention`` -- naive fp64 causal attention over the paged cache,
  plus a partitioned log-sum-exp variant used only to self-test the combine
  algebra.
"""

from . import fp8, paged, attention  # noqa: F401

"""CPU oracle for the AKV state-restoration path.  TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct reference that the GPU
library is checked against.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does and
shares no code with it (no kernels, helpers, tables or constants).

Everything here is NumPy in float64, written from the text of two pages about
AKV ("Cache Engineering for Agents", arXiv 2610.28577v1):
  [P1] the jaehun.me review "Cache Engineering for Agents";
  [P2] the vibeprogramminglab explainer "KV만 줄이려면: AKV가 캐시 작업 이력을
       기록하는 이유".
Each function cites the section of the page it follows.

Readings where the pages are silent or garbled (the RoPE equation of P1
"what to keep / how to align positions" (§3.3) was lost in extraction):
  * RoPE pairs (x_i, x_{i+d/2}) by default, (x_{2i}, x_{2i+1}) optionally;
    theta_i = base^(-2i/d); moving a key from position p to q multiplies it
    by the rotation R((q-p) theta).  Angles are exact integers times fp64.
  * softmax scale 1/sqrt(d); GQA maps q head h to kv head h // (Hq/Hkv).
  * version keys are rotated once from the raw key: RoPE(k, to_pos).

Parity pins live in tests/test_oracle_pins.py; functions without a pin say
"parity unpinned" in their docstring (none at present).
"""
from .opseq import APPEND, DROP, REPOS, OpSequenceError, canonical_ops  # noqa: F401
from .rope import theta, rope, rotate  # noqa: F401
from .replay import replay_tokens, replay_events  # noqa: F401
from .attention import (attention_replay, segment_attention, visibility_mask,  # noqa: F401
                        decode, decode_after_ops, repos)
from .tables import plan_tables, tile_classes, tile_class_of  # noqa: F401
from .bf16 import f64_to_bf16_bits  # noqa: F401

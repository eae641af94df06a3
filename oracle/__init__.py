"""CPU oracle for compressed-KV decode attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with
the HIP library and never imports it.

What it computes (plain NumPy; float32 where the encoding rule fixes float32
arithmetic, float64 for attention):

* ``quant``     - calibration-free INT4 (group 32 along head_dim, asymmetric,
                  fp16 scale/min) and INT8 (per-token per-head symmetric
                  absmax) encode/decode; nibble packing.
* ``regions``   - which positions are INT8 (16 sink + 128 recent) and which
                  are INT4, and the INT8 ring slot of a position.
* ``policy``    - the per-head scoring MLP and the budgeted top-k keep set
                  (the shadow mask).
* ``attention`` - masked softmax attention over the union of the kept
                  positions (the plain definition), split partials and the
                  exact log-sum-exp merge (used only by invariant tests).
* ``reference`` - the composition for one (sequence, kv head).
* ``dense``     - the uncompressed baseline: bfloat16 rows, every position
                  attended (what the INT4 cache is measured against).

Sources: the KV4-RL review page ("KV4-RL: Unlocking Faster Asynchronous
Rollouts for RLVR with INT4 KV Cache Quantization"), section 3 "Method & Key
Results" and the "Selective Protection" entry of section 1; the KVP promo page
for arXiv 2602.10238, section "Core mechanism"; the Shadow Mask Distillation
page (arXiv 2605.06850), Figure 1 caption. The numeric rules the pages leave
open (group size, scale format, rounding, tie-breaking) follow the readings
listed in each function's docstring.
"""
from . import quant, regions, policy, attention, reference, dense  # noqa: F401

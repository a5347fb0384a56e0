"""CPU oracle for the DFlash + DDTree draft-and-verify chain.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers or table generators); the two meet only
through the seeded arrays of the ``synth`` module.

Each function is the plain definition of one step of the chain, written for a
reader to check against the pages by eye:

* ``logits.topk_logprobs``     per-position log-softmax + top-K
* ``logits.argmax_rows``       the target's greedy token per tree slot
* ``tree.build_tree``          DDTree best-first top-B prefix tree, flattened,
                               with parent/depth arrays and the ancestor mask
* ``attention.masked_attention``  GQA attention over prefix KV + own KV with
                               the ancestor-only (verify) or dense-block
                               (drafter) visibility rule, in float64
* ``accept.accept_compact``    greedy longest-matching-path walk + KV-row
                               compaction

Pages cited (by title and section):
  [DDTree]  "Accelerating Speculative Decoding with Block Diffusion Draft
            Trees" summary, bluediary8.tistory.com/1288
  [DFlash]  "DFlash: Block Diffusion for Flash Speculative Decoding" summary,
            honbul.tistory.com/178
  [DFlash-news]  DFlash article, darkpulse.kr/?p=2484

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
brute force, closed forms, invariants and independent library routines.  The
end-to-end acceptance lengths the DDTree page reports need trained models and
datasets and are "parity unpinned" (not reproduced here).
"""
from . import accept, attention, logits, tree  # noqa: F401

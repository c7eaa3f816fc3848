"""CPU oracle for mixed FP8/TQ3 paged decode attention.

TEST INFRASTRUCTURE, NOT PART OF THE LIBRARY.  Only the test suite, the smoke
check in __graft_entry__ and the CPU-baseline leg of bench.py may import this
package.  The HIP library never calls it and has no CPU fallback through it.

It is a plain, slow, fp64 restatement of what the Minima-KV summaries
(brainszone.ai, pt and fr editions) describe: a paged KV cache whose pages are
stored in different numeric formats (FP8 anchors, packed TQ3 archive), decoded
directly by per-format partial attention plus a globally normalised merge.  It
shares no code with the HIP path.

Modules:
  codecs      FP8 E4M3, fp16/bf16 and TQ3 codecs written from their definitions
  pool_model  CPU model of pages: append with rescale-on-grow, FP8->TQ3 demote,
              page byte records; the dense BF16 control cache
  attention   fp64 softmax attention on the dequantised cache, partial states
              and the merge

Every function here is pinned by tests under tests/ against closed forms,
library routines, hand-derived byte patterns or brute force; none is
"parity unpinned".
"""
from . import attention, codecs, pool_model  # noqa: F401

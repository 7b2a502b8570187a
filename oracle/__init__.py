"""fp64 CPU oracle for causal attention forward, backward, LSE merge and the
saved-tensor pack.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP
library never calls it, and it shares no code with the HIP library: no
kernels, headers, helpers or constant tables.  Only the seeded input
generators in ``workloads`` serve both sides.

What is computed, and where it comes from
-----------------------------------------
The pages (five pull-request pages on context-parallel attention) print no
formulas, so every function here is the plain textbook definition of softmax
attention and its exact gradient, written out in float64:

* forward: S = s*Q K^T over the visible keys, LSE = natural-log logsumexp of
  each row (PR 3527 "cuDNN FROST attention backend for head_dim in (256,
  512]", commit "Add frost_attention.py": the forward LSE is a natural-log
  logsumexp in fp32, which is what makes a ring merge valid), P = exp(S -
  LSE), O = P V.  Keyless rows give O = 0 and LSE = -inf.
* backward: the exact gradient of O with respect to Q, K, V given dO,
  through the softmax Jacobian dS = P * (dP - rowsum(P * dP)), dP = dO V^T
  (PR 3510 "Add head-parallel FA4 backward for cuDNN CP attention", Diagram:
  the backward consumes the saved Q, K, V, O, dO and LSE).  LSE itself is not
  differentiated.
* merge: the exact recombination of partial results over disjoint key sets
  by their LSE (PR 3527, commits on the CP ring: per-step kernel calls
  interleaved with KV exchange and LSE correction).
* pack/unpack: a byte permutation of O and the raw fp32 LSE bits (PR 3510,
  Description: packing preserves the FP32 log-sum-exp values).
* exchange buffers: the byte permutation of any row tensors and LSEs into
  per-peer segments for the head-parallel all-to-alls (PR 3510, Diagram).

Visibility is given by explicit positions: key j is visible to query i iff
it is a real key of the same sequence, (not causal or k_pos[j] <= q_pos[i])
and, with a sliding window (left, right), q_pos[i] - left <= k_pos[j] <=
q_pos[i] + right where -1 leaves that side unbounded (PR 3527, commits on
sliding window).  Top-left causal is q_pos = arange(S_q), k_pos = arange(S_k);
bottom-right adds S_k - S_q to q_pos (PR 3699 "Add cuDNN OSS backward
dispatch for context parallel attention", Implementation and supported
scope; PR 3527 commit on the all_gather path).

Pins (tests/oracle): pure-Python brute force, central finite differences,
torch's own float64 scaled_dot_product_attention and autograd, closed forms
(hand-derived golden cases in tests/golden), softmax rows summing to one,
gradient-sum invariants, merged == unmerged, GQA == repeated MHA, THD ==
per-document dense.
"""
from .attention import (  # noqa: F401
    forward, backward, merge, bshd_forward, bshd_backward, thd_forward,
    thd_backward, positions_from_segments, forward_rows,
)
from .pack import pack_saved, unpack_saved, pack_layout  # noqa: F401
from .xchg import xchg_layout, xchg_pack, xchg_unpack  # noqa: F401

"""CPU float64 oracle for the tiled attention forward and the row-wise online softmax.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import anything from here.  The
GPU library (``online_softmax_09_amd``) never imports, links or calls this package,
and this package imports nothing from it: the two share no kernels, helpers, tables
or constants.  Only the seeded input generators (``workloads.py``, which holds none
of the method's arithmetic) feed both.

Everything is computed in float64 from the exact float64 upcast of the stored
fp32 / bf16 inputs, by the plain definition of the operation:

* ``softmax``   — three-pass safe softmax of rows, plus the scalar online-normaliser
  instruments ``online_state`` / ``merge_state`` / ``online_weighted`` that fix the
  semantics the GPU tree reduction must reproduce.
* ``attention`` — standard attention with the score matrix S materialised,
  softmax by the same three passes, ``O = P V`` and ``LSE = m + ln l``.
* ``attention_bwd`` — the gradients dQ, dK, dV of that definition for an upstream dO,
  by the chain rule with S, P, dP and dS materialised.
* ``attention_split`` — the same definition for N_q queries against N_k keys (causal
  masks bottom-right aligned), and the log-domain merge of partial (O, LSE) results over
  disjoint key sets.
* ``norms`` — residual add followed by LayerNorm or RMSNorm of rows, by the formulas.

Pages cited (titles as they appear on the pages; section numbers are the pages'):

* [SNS] "Softmax numerical stability and IO-aware attention: from online
  normalisation to FlashAttention" (zhouzhq2021.github.io, 2026-07-28), sections 2-9.
* [FAM] lihaoran.work FlashAttention note (auto-20261009-2330), sections "the problem
  starts with the intermediate matrix", "why per-block softmaxes cannot be averaged",
  "checking the result with three scores".
* [WHY] "Why do Flash Attention's results differ slightly from standard attention?
  Lossy but worth it" (guanweilu.cn/article/547), section "the culprit is the rescale
  step of online softmax".
* [INT] "Are Flash Attention and standard attention outputs exactly the same?"
  (agentalpha.top interview basics-tk168), follow-up question 1.

Parity status: every function here is pinned by ``tests/test_oracle_*.py`` against
values the pages print, closed forms, brute force and library routines; none is
"parity unpinned".
"""

from .softmax import (  # noqa: F401
    softmax_rows,
    logsumexp_rows,
    online_state,
    merge_state,
    online_weighted,
    weighted_full,
)
from .attention import attention, attention_rows  # noqa: F401
from .attention_bwd import attention_backward  # noqa: F401
from .attention_split import attention_rect, merge_attention_states  # noqa: F401
from .norms import layer_norm, rms_norm, residual_sum  # noqa: F401

"""CPU oracle for exact attention (forward and backward) -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct reference the GPU library is
checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path (the HIP
library and its Python binding) never imports, calls or links anything here,
and this package imports nothing from the product path.  It shares no code
with the GPU kernels: no helpers, tables or constants.

Sources (web pages, cited by title and section):

* [v1.7]  release page "v1.7 / flash_attn 2.9.2.post1" of the ussoewwin
  flash-attention fork -- section 1.2 "A-1 -- rescale threshold and max
  lagging" (threshold 8.0, max lagging, P <= 256), section 2 (public API
  features: causal, window, ALiBi, softcap, varlen, kv-cache), section 4.6
  (edge probes: LSE shape [B, H, S], window (0,0) gives V), section 4.4
  (backward: dQ, dK, dV checked against an fp32 reference).
* [v1.2]  release page "FA2 2.9.0 Kernel Changes in v1.2" -- section 1
  (softmax_rescale_o: scaled difference of old and new row max in log2
  units, rescale of O and row_sum), section 2 (scale_apply_exp2: exp2 of
  score*scale*log2e minus max*scale*log2e, with a guard that treats a -inf
  row max as 0), section 3 (Is_first on the first KV step).
* [aichaai]  Dao-AILab/flash-attention project page, release notes of
  fa4-v4.0.0.beta30 (a window bound of 0 is a real, zero-width bound) and
  fa4-v4.0.0.beta37 (unused cache entries must not spread NaN).

Modules:

* ``attention``  -- the plain definition (full materialised softmax, fp64).
* ``backward``   -- the gradients (dQ, dK, dV) of that definition, fp64.
* ``tiled``      -- the tiled online-softmax algorithm with RescaleThreshold
  and max lagging, step by step in fp64 (pins the method's semantics).
* ``metrics``    -- rel_Linf, cosine and LSE error as the gates use them.

Parity status of every function is stated in its docstring; all of them are
pinned by tests in ``tests/test_oracle_pins.py``.
"""

from .attention import (  # noqa: F401
    attention_ref,
    attention_varlen_ref,
    attention_kvcache_ref,
    allowed_mask,
    gather_pages,
)
from .backward import attention_bwd_ref, attention_bwd_varlen_ref  # noqa: F401
from .tiled import tiled_ref  # noqa: F401
from .metrics import rel_linf, cosine, lse_max_abs_err, compare  # noqa: F401

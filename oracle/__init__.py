"""CPU oracle for exact attention forward — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it, and this package never imports the
product path: the two share no code.

Everything here is plain numpy in float64, written to be read against the
pages it follows:

* "Flash Attention 3：让 GPU 跑满的注意力计算" (guijiagi.com blog post):
  §1.2 standard attention (S = QK^T, P = softmax(S), O = PV), §2.2 the
  softmax definition and the tiled (online) softmax update equations,
  §5.2 variable-length batches through cu_seqlens prefix sums;
* "FlashAttention-3" (lukebest.github.io wiki page): the claim of exact
  attention (opening paragraph), and "Three techniques" §3 FP8 precision:
  block quantisation with one scale per tile, and incoherent processing
  Q' = QM, K' = KM with M an orthogonal Hadamard times random +-1.

Modules:

* ``exact``: the definition, materialising S (dense and varlen);
* ``tiled``: the online-softmax recurrence on tiles, in both the per-step
  normalised form the blog prints and the deferred-normalisation form;
* ``fp8``: e4m3 rounding from the format definition, the Sylvester Hadamard
  and its fast transform, the rotation, block/per-tensor quantisation, and
  an fp64 emulation of fp8 attention, and both for variable-length batches
  (scale tiles restarting at every sequence);
* ``splitkv``: attention over key chunks and the (O, lse) merge of the
  partial results;
* ``backward``: the gradients dQ, dK, dV of the attention definition (the
  chain rule written out; the pages measure a backward pass but print no
  algorithm for it);
* ``paged``: attention over a paged key/value cache (pages gathered through
  a page table, then the definition);
* ``fp8_backward``: e5m2 rounding from the format definition, block
  quantisation of dO, and an fp64 emulation of the backward pass with its
  products on fp8 operands (E5M2 for the gradient operands).

Pins (the independent checks each function is held to) live in
``tests/test_oracle_*.py``; every function here is pinned, none is "parity
unpinned".
"""

from .exact import attention, attention_varlen, softmax_rows, scores  # noqa: F401
from .tiled import attention_tiled  # noqa: F401
from . import fp8  # noqa: F401
from . import splitkv  # noqa: F401
from . import backward  # noqa: F401
from . import paged  # noqa: F401
from . import fp8_backward  # noqa: F401

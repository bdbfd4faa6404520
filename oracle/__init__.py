"""CPU oracle for the fused multi-query attention step -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything in this package.  The GPU library never calls
it, links it or falls back to it, and this package imports nothing from the GPU
library: the two implementations share no code, table or helper.

Pages cited (by title and section):

* [P-Metal] "How DeepSeek V4 Flash Model Inference Works on Apple Silicon with
  Metal Backend" (instagit.com, antirez/ds4).
* [P-DS4] "DwarfStar 4 (DS4) -- DeepSeek V4 Flash Inference Engine"
  (wikichat.gnat.co, summary of ds4.md), section "Architecture Deep Dive".

Modules:

* ``reference`` -- the plain definition in float64 NumPy: allowed-row sets,
  softmax(QK^T * scale) V per query token, the 32-row padded layout and the
  per-block skip map.
* ``brute`` -- an independent pure-Python formulation over a materialised
  -inf mask (lists and ``math.exp`` only), used to pin ``reference`` on tiny
  inputs.
* ``fp8`` -- the FP8 (E4M3, per-row scale) quantize step and its inverse.
* ``topk`` -- the indexer's top-k selection from given scores.
* ``compress`` -- compressor pooling of raw rows into compressed rows, with the
  rolling state of the incomplete group.

Every function of ``reference``, ``brute``, ``fp8`` and ``topk`` is pinned by at
least one check in ``tests/test_oracle*.py`` (brute force, closed forms,
invariants, library routines) against what the pages and the mathematics fix.

``compress`` is **parity unpinned**: the pages name the compressor's rolling
KV/score state and its ratio boundaries but give no pooling formula, so no value
they print, and no definition they state, can pin it.  Its checks pin the code
to this package's own reading of the pages (a per-element softmax over each
group); a different reading would pass none of them, but nothing shows that the
reading is the engine's.
"""

from . import reference, brute  # noqa: F401

"""CPU oracle for one layer of indexed block-sparse paged-attention decode.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark import this package.  The product path (the
HIP library and its Python binding) never imports, calls or links it, and the
oracle imports nothing from the product path: the two share no code.

Everything is plain numpy in float64, written from the definitions the sources
give (cited per function) and, where they are silent, from the readings listed
in each docstring:

* ``formats``  - exact decoding of bf16, e4m3fn, e2m1, e8m0 and the MXFP4 page;
* ``pools``    - reading tokens out of the paged index and K/V caches;
* ``decode``   - index score, top-k selection, sparse block-table emission and
                 sparse attention, and the four chained as one decode layer;
* ``prefill``  - the same steps for a ragged prefill batch, each query token
                 with its own request id and absolute position;
* ``writer``   - writing a step's new tokens into the caches (optional QK-norm
                 and rope, the fp8 / MXFP4 encodings) and the e4m3 query cast.

Parity status: every function here is pinned by the CPU tests (closed forms,
library routines on special cases, brute force on tiny inputs, invariants),
except for two readings the sources leave open - the block score being the
maximum over the block's tokens, and index heads of one KV group being summed -
whose arithmetic is pinned but whose choice of definition is a reading.
"""

from . import formats, pools, decode, prefill, writer  # noqa: F401

"""CPU oracle for block-sparse tiled video attention (test infrastructure).

A plain, slow, obviously correct numpy implementation of what the GPU path
computes, written from the FastVideo attention-backend pages:
  * geometry.py  -- tile counts, per-tile valid-token counts, token -> slot map
  * tiling.py    -- raster <-> zero-padded tile order
  * select.py    -- per-tile mean pooling, pooled scores, top-k and STA masks,
                    mask -> CSR index map
  * attention.py -- masked softmax attention over the selected tiles, and a
                    brute-force dense attention with an explicit token mask
  * packed.py    -- packed sequences of dense segments and video regions:
                    layout, selection with per-region keep rates, attention
  * prune.py     -- query pruning: kept tokens per tile, the kept queries'
                    means for the selection, attention of the kept rows

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP path and imports nothing
from it.  Floating point is float64 except where a reading fixes another
precision (pooled tile vectors are rounded once to float32).

Pinning: every function is checked by the CPU tests against closed forms,
brute force on tiny inputs, library routines for special cases and
hand-derived fixtures (tests/golden).  No function here is "parity unpinned".
"""

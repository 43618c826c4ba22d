"""Compressed-attention block selection on AMD MI355X (gfx950).

For each layer and each query row, score every compressed block that the
row's admission mask and causal limit let through, and return the best k
blocks (default 512) in order, using three hand-written HIP kernels behind a C
ABI (``include/ds_sel.h``, ``libdssel.so``).  Page "DeepSeek V4.1F Q4 on M3
Ultra with native DSpark MTP (40tps / 800tps)", paragraph "Decode at depth",
describes the chain: score only the admitted blocks, build the admitted index
once per row, keep the top 512 with a radix select of bounded depth.

Importing the package loads nothing native.  ``selector.Selector`` loads the
library on first use and raises if it is missing.
"""

__all__ = ["workloads", "selector"]

"""CPU oracle for FP8 (E4M3) smoothed attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this package; only
the test suite, the smoke check in ``__graft_entry__`` and the CPU-baseline leg
of ``bench.py`` call it.  It shares no code with the HIP path: every step is
written out here from the pages' description, in plain NumPy, float64 unless
the pages fix the precision (FP32 K centring and FP32 softmax exponential, and
the E4M3 format itself).

Modules
-------
e4m3       OCP FP8 E4M3 ("FN") codec from the format definition.
fp4        OCP MX FP4 (E2M1) codec and the MXFP4 (E8M0 per 32 tokens) V quantizer.
smoothing  exact K/V statistics and the per-128-token-block quantizers.
kmeans     integer Lloyd k-means on V, stable label sort, joint K/V gather.
grouping   the static spatiotemporal-cube permutation of a video token grid.
attention  FP64 dense attention, the tiled online-softmax recurrence with the
           rank-one V-mean restore, E4M3 / ExpCast-FP8 probability casts.
pipeline   the whole hot path chained in the pages' order.

Parity status of every function is stated in its docstring; the only parts
whose end result is not pinned beyond the oracle itself are the quantized
pipeline outputs (O, lse2) for which the pages print no worked example
("parity unpinned" in ``pipeline``); their individual steps are pinned.
"""

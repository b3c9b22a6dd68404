"""CPU oracle for the TurboQuant KV-cache hot path.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(the C-ABI library and its Python binding) never imports, calls or links it,
and this package imports nothing from the product.

Everything here is plain numpy/scipy in float64 (parameters that the method
stores in fp32 -- levels, boundaries, rotation, QJL matrix, norms -- are rounded
to fp32 where the method stores them and promoted back to float64 for
arithmetic). Each function cites the passage of the pages it follows:

* "FlashQuant ... KV缓存压缩方案" (zingnex.cn), sections "TurboQuant" (the
  four-step pipeline and the MSE bound), "QJL" (the residual-sign estimator),
  "架构设计" (codebook / quantizer / packing / rotation / paged split-K decode)
  and "性能数据" (bytes per token).
* "TurboQuant : compresser le KV-cache" (patricehuetz.fr), sections
  "Couche 1" (randomized Walsh-Hadamard), "Couche 2" (Lloyd-Max, binary search
  over boundaries), "Couche 3" (packing) and "Couche 4" (fp32 norms).

Modules:
  rng        counter-based SplitMix64 -> uniform -> Box-Muller Gaussians, signs
  codebook   Lloyd-Max fixed point for N(0,1), scaled by 1/sqrt(d)
  rotation   Haar rotation (QR + sign fix), randomized Walsh-Hadamard
  quantize   normalise / rotate / quantize / pack, QJL residual signs
  paged      paged compressed-cache layout (block tables, slots)
  attention  decode attention over the compressed cache (two forms), exact
             attention over uncompressed vectors
"""

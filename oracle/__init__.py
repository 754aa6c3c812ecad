"""CPU oracle for tile-granular rANS weight coding fused into a GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, no
constants generator and no header with ``decode_gemm_tile_amd`` (the HIP
library); the only module both sides read is ``workloads`` (seeded synthetic
inputs, which holds none of the method's arithmetic).

Everything here is plain NumPy / Python on the CPU, in fp64 for floating
point, written from the pages that describe the method:

  [P1] "arXiv'26 | 无损压缩逼近 Shannon 极限：你的 LLM 权重里一半以上的 bit 是白存的"
       (blog write-up of "Approaching Shannon Bound with Lossless LLM Weight
       Compression").  §2.1 per-layer histogram entropy; §2.2 the three design
       principles (decode keeps up with HBM, tile-granular random access,
       decode straight into on-chip memory); §3.1 the execution model (tiles
       cut in the GEMM's tiling geometry, one shared ANS codebook per layer, a
       per-tile start-offset index, R lane sub-streams per tile); §4.1
       finite-precision frequency normalisation.
  [P2] "70%大小，100%准确！完美压缩LLM性能0损失，推理速度最高飙升39倍"
       (DFloat11 news page), section "实验方法": Shannon entropy of a discrete
       variable (formula lost in extraction; read as H = -sum p log2 p).
  [P4] "Approaching Shannon Bound: Lossless LLM Weight Compression" (podcast
       summary): reference list names Duda's asymmetric numeral systems, the
       coder this oracle implements (rANS, Duda 2013, range variant).
  [P5] "突破1.58比特极限：三元LLM如何逼近信息论边界": uniform ternary entropy
       log2(3) ~= 1.585 bits (a pin for the entropy routine).

Module map
  entropy   empirical Shannon entropy of a symbol histogram          (pinned)
  freq      integer frequency quantisation to 2**prob_bits           (pinned)
  order     tile partition and tile-local symbol order               (pinned)
  rans      interleaved R-lane rANS encode / decode                  (pinned)
  blob      compressed-layer byte format writer / reader             (pinned)
  numerics  bf16 / e4m3 casts, int4 dequant, fp8 activation quant    (pinned)
  gemm      fp64 reference GEMM Y = X W^T                            (pinned)

Every function is pinned by a ``-m "not gpu"`` test in ``tests/test_oracle_*``
against closed forms, brute force, library routines or hand-worked golden
examples under ``tests/golden/``.  No function here is "parity unpinned".
"""

__all__ = ["entropy", "freq", "order", "rans", "blob", "numerics", "gemm"]

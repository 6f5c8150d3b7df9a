"""Plain, slow CPU oracle for the QuaRot online-rotation + INT4 hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The product path (``hadamard_rotation_int4_amd``) never imports it
and shares no code with it: the two meet only through the seeded input
generators in ``workloads.py``, which hold none of the method's arithmetic.

What it computes, and where the pages define it (page titles below; "QuaRot
paper" is the paper text "QuaRot: Outlier-Free 4-Bit Inference in Rotated
LLMs", "QuaRot blog" is "QuaRot: Rotating Away the Outliers That Make 4-Bit
LLMs Impossible"):

* ``hadamard``: Sylvester H_{2^n}, the Kronecker construction H_{2^n} (x) H_m
  for widths that are not powers of two, the randomized Hadamard
  H diag(s) / sqrt(d) (QuaRot paper, background on Hadamard matrices), the
  fast Walsh-Hadamard transform (QuaRot blog, "Hadamard matrices: orthogonal
  and fast"), and the incoherence ratio (QuaRot blog, "Computational
  invariance" and its outlier demo).
* ``quant``: per-token symmetric INT4 round-to-nearest (QuaRot paper,
  activation-quantization paragraph; QuaRot blog, "The outlier problem,
  stated precisely") and nibble packing; b-bit codes one per byte (the paper's
  6- and 8-bit RTN results) and one scale per group of G consecutive elements
  (the paper's group-wise quantization ablation).
* ``gemm``: the exact INT4 x INT4 -> INT32 product and the per-token x
  per-channel scale epilogue (QuaRot paper, activation-quantization paragraph);
  the int8 form (W8A8) and the group-wise form, whose per-group scaled
  accumulators are summed in fp32.
* ``kv``: head-wise rotation of keys and queries and asymmetric group-wise
  4-bit KV quantization (QuaRot paper, keys/queries paragraph and the
  implementation paragraph on clipping ratios and group size 128).
* ``attention``: the Decode routine, softmax attention of one query per
  sequence over the dequantized 4-bit cache, with grouped-query heads (QuaRot
  paper, attention paragraph and its attention routines: Init, Append,
  Decode).
* ``block``: the block's other online steps: RMSNorm without its scale in
  front of the QKV/gate/up quantizer, and the Hadamard-heads transform
  Z (H_{n_h} (x) I) in front of the O projection's quantizer (QuaRot paper,
  method section and the attention-block paragraph with Figure 6).

Two modes exist where floating point is involved.  "Math" functions work in
float64 throughout.  "Recipe" functions follow the fp32 step sequence that the
library documents for its kernels (the spec the kernels implement); on inputs
whose rotation is exact in fp32 they give the bit pattern the kernels must
reproduce.

Parity unpinned (pinned only by self-consistency): the particular H_28 and
H_172 chosen (any matrix with H H^T = m I is valid), the RNG streams, and the
fp32 step order of the recipe functions.
"""

"""CPU oracle for RMSNorm + NVFP4 block quantization (test infrastructure only).

This package is the plain, slow, obviously-correct reference that the HIP path
is checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. It shares no code with the
HIP path (no kernels, headers, tables or helpers) and imports nothing from the
package ``rmsnorm_nvfp4_block_amd``.

Every quantizer step is one IEEE binary32 operation rounded to nearest, carried
out on ``numpy.float32`` arrays (numpy does no FMA contraction), because the
method fixes single precision for its scaling and conversions. The RMSNorm
statistics are the one exception: they are evaluated in float64 and the output
is rounded once to bfloat16, which makes the oracle the exact value that any
fp32 reduction order approximates.

Citation keys used in docstrings:
  * "PR" -- the pytorch/ao pull request page "[nvfp4_training] Optimize
    CuteDSL kernels for NVFP4 training" (#4798). Section names are the
    page's own: Optimization (numbered items), Fast math, Grouped allocation
    tail, Config surface and AUTO, Performance, Correctness.
  * "Blog" -- the Perplexity engineering post "CuTeDSL at Perplexity",
    sections "QK Norm", "Blackwell support", "Prefill and decode".

Where the pages leave a step open, the reading taken is stated in the function
that implements it. Readings are:
  R-eps      eps is a float32 value (the ABI passes ``float``).
  R-bias     "weight bias" is both the Blog's scalar added to the weight and
             an optional per-channel additive beta.
  R-y        the quantizer consumes the bfloat16-rounded normalized output.
  R-scale    S_enc = 2688/amax, S_dec = amax/2688 (two fp32 divisions);
             amax == 0 or non-finite S_enc gives S_enc = S_dec = 1.
  R-bscale   block scale = E4M3_rne_sat(RN(RN(bmax/6) * S_enc)).
  R-rcp      encode reciprocal = RN(1/RN(f32(s) * S_dec)); 0 when s == 0;
             clamped to the largest finite float.
  R-e2m1     round-to-nearest-even, saturating to 6, sign kept (-0 -> 0x8).
  R-nibble   even element in the low nibble.
  R-col      "columnwise" = 16 consecutive rows of one column, stored as the
             transposed plane [cols, rows/2].
  R-philox   key = (seed lo32, seed hi32); counter = (blk lo32, blk hi32,
             tag, offset); tag 0 rowwise, 1 columnwise.
  R-blk      blk = linear index of the block's scale byte in a packed
             (unpadded) scale plane.
  R-sr       element j of a block uses byte (j & 3) of Philox word (j >> 2);
             it rounds away from the lower neighbour iff
             r + floor(256 * frac) >= 256.
  R-rht      D = diag(d), d_i = -1 iff bit i of a 16-bit mask is set; FWHT in
             Sylvester order, stages h = 1, 2, 4, 8 of fp32 (a+b, a-b);
             times 0.25; bfloat16 round-through. Same D for every block.
  R-fast     fast math (grouped, with the transform): the transform's fp32
             output RN(0.25 * FWHT(D x)) is quantized and enters the group
             amax without the bf16 round-through; the encode reciprocal stays
             RN(1 / RN(f32(s) * S_dec)) (on this hardware it comes from a
             127-entry table, so an approximate reciprocal would save nothing).
  R-rowcol   grouped rowwise + columnwise: the rowwise plane of x's rows,
             no transform, one amax per group (max|x| over its rows), SR tag
             0 with block index row * (K/16) + k/16 in x's row numbering.
  R-2dblk    "2D" weight scaling: one E4M3 scale per 16 x 16 tile (the tile
             amax through R-bscale), used by every element of the tile in
             both planes; the planes keep the 1D scale layout with the
             tile's code repeated on its 16 rows / 16 columns.
  R-experts  grouped 2D weights: expert e of E stacked [M, K] weights is the
             2D quantization of its own weight under its own amax, SR tags
             2e (rowwise) and 2e + 1 (columnwise); planes stacked by expert.
  R-dtype    fp16 / fp32 inputs: quantizers take the values as given; the
             norms round y in the input's type; the grouped transform's
             output is rounded through the input's type (bf16, fp16) or not
             at all (fp32).
  R-qk       QK norm: the RMSNorm formula above applied to each attention head
             (64, 128 or 256 elements) of q and of k, each tensor with its own
             weight of head_dim entries, output in the input's place.
  R-group    each group is zero-padded to a multiple of 16 rows, groups are
             laid out back to back in one transposed plane; storage past the
             last padded column is never written.
"""
from .formats import (  # noqa: F401
    bf16_to_f32, f32_to_bf16, f64_to_bf16, e4m3_decode, e4m3_encode, e2m1_decode, e2m1_encode,
    pack_nibbles, unpack_nibbles, E2M1_VALUES,
)
from .philox import philox4x32_10  # noqa: F401
from .quantize import (  # noqa: F401
    global_scales, block_scale_codes, encode_reciprocal, quantize_blocks, quantize_rowwise,
    quantize_colwise, quantize_2d, quantize_2d_block, quantize_2d_experts, encode_blocks, dequantize_rowwise, sr_round,
)
from .rmsnorm import rmsnorm_bf16, rmsnorm_quantize, qk_norm  # noqa: F401
from .rht import rht16, rht16_f32  # noqa: F401
from .grouped import padded_offsets, grouped_quantize  # noqa: F401

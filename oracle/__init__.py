"""CPU oracle for lossless BF16 exponent compression and the products over it.

TEST INFRASTRUCTURE ONLY.  Nothing in the library may import, call, link or
run this package: only the tests, the package smoke check and the bench's CPU
baseline leg use it.  It shares no code with the GPU library (no kernels,
headers, tables or helpers); both sides are written independently from the
same written format description.

What it computes, and the passages it follows ("Unweight: how we compressed an
LLM 22% without sacrificing quality"):

  * split of every bf16 into a sign+mantissa byte and an exponent byte
    (paragraph on the anatomy of a BF16 value);
  * exponent histogram, top-K palette (paragraph on exponent redundancy:
    16 exponents cover >99% of a layer, ~2.6 bits of entropy);
  * rows of 64 holding any exponent outside the palette are stored raw
    (paragraph on rare exponents);
  * Huffman coding of the exponent byte only (paragraph on Huffman coding),
    made length-limited by package-merge and canonical per RFC 1951 3.2.2;
  * lossless round trip (results paragraph: 100% bit-exact);
  * the direct-palette form (4-bit palette index + sign+mantissa byte per
    weight, raw groups verbatim) built at load time (section on the four
    execution pipelines), in palette.py;
  * the products y = W x and Y = X W^T over the original weights with fp64
    ground truth and an fp32 reference (paragraph on the reconstructive
    matmul: the kernel multiplies the reconstructed bf16 weights).

Every function is pinned by the CPU tests against values that do not come
from this package: hand-derived streams, the RFC's printed example, brute
force over all length vectors, closed forms, exact rational sums and
invariants.
"""
from . import huffman, blob, palette, products  # noqa: F401

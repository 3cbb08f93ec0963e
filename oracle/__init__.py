"""CPU oracle for MXFP8 block-scaled attention -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 NumPy restatement of what the pages compute, written to
be checked by eye.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the product library never does, and the two
share no code (only the seeded input generator in ``synth``).  ``cpp/mx_oracle.cpp``
states the same MXFP8 point arithmetic in plain C++ (codecs, quantizers, the
forward and backward of one head); the tests check the two against each other.

Pages cited (by title; sections named in each docstring):
  [News]  "Low Precision Flash Attention 4: End-to-End Block-Scaled Attention
          for Blackwell" (aivexanews.com)
  [Blog]  "Low-Precision FlashAttention-4: End-to-End Block-Scaled Attention
          for NVIDIA Blackwell" (explore.n1n.ai)
  [Brief] "FlashAttention-4 Adds Low-Precision Blackwell Support" (setupai.cc)
External specifications used where the pages are silent: the OCP 8-bit
floating point specification (E4M3 encoding) and the OCP Microscaling (MX)
v1.0 specification (E8M0 shared-scale selection).
"""
from . import mx, attention, norm  # noqa: F401

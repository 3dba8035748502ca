"""Plain, slow CPU oracle for the online 4-bit activation path of a quantized DiT linear.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links this
package: only the tests, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code, table or constant generator with the HIP library; the two meet
only through the seeded input generator in ``synth`` (which holds none of the
method's arithmetic).

Everything is computed in float64 with NumPy/SciPy, written from the definitions on
the pages (cited per function):

* KroQuant: Kronecker-Structured Block Transforms for Efficient Post-Training
  Quantization of Diffusion Transformers (iselia-ai.com/papers/2607-21446):
  §01 (the identity Y = (XP)(P^-1 W)), §02 (P = A (x) B on 32-element blocks),
  §03 (MXFP4 target format).
* OrbitQuant: data-independent quantization for image and video DiTs
  (iselia-ai.com/papers/2607-02461): §03 (RPBH(X) = X.P.H.D, W' = R^-1 W,
  one Lloyd-Max codebook).
* CentriQ: Calibration-Free Quantization of DiTs via Exact Mean Centering
  (physicalainews.jp/papers/2610.06260): arXiv abstract (each token is centred
  before the rotation and its mean added back afterwards by a rank-1 term kept in
  high precision; a closed-form per-token scale).
* SVDQuant explainer (aibr.jp/archives/95399): §3 (16-bit low-rank branch L1 L2
  beside the 4-bit residual product, fused in the engine).

The MXFP4 element and scale rules the pages only name ("MXFP4") follow the OCP
Microscaling Formats v1.0 specification (E2M1 elements, E8M0 shared scale, block 32).

Pins (closed forms, invariants, brute force, library routines) live in
``tests/test_oracle_pins.py``.  Parity unpinned: nothing here (every function has
at least one pin); the learned A, B of KroQuant and the pages' quality claims are
out of scope and not computed.
"""

from . import mxfp4, transforms, lloyd_max, pipeline, linear, ties  # noqa: F401

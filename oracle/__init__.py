"""CPU oracle for grouped routed-MoE prefill (fp64).  TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import or call anything here.  The product path (the HIP library and
its Python binding) never does, and this package imports nothing from it: the
two share no kernels, helpers, tables or constants.  The only thing both sides
consume is the seeded input generator, which holds none of the method's
arithmetic.

What is computed, and where the pages state it:

* ``route.route_table`` -- route histogram, prefix and scatter "for up to 256
  experts" ("perf(ds4): batch heterogeneous MoE prefill by expert", Summary),
  stable in route order so the selected-row order is preserved ("perf(ds4):
  extend sparse prefill scheduling to 10K", Summary of the earlier
  description).  Masked routes go to a trailing bin E and are never computed
  ("... by expert", Correctness and validation: unwritten masked lanes).
* ``moe.moe_ref_per_token`` -- the literal per-token loop over selected
  experts: gate/up projection, SwiGLU, down projection, route-weighted sum in
  ascending route order starting from +0.0; masked routes contribute exact
  zeros ("... by expert", Summary: masked owner routes are exact-zero
  contributions).  SwiGLU is silu(gate) * up ("perf(ggml): reuse ROCmFP4
  weights across q=4 columns", DS4 SwiGLU split op).
* ``moe.moe_ref_dense`` -- brute force: every expert applied to every token,
  weighted by a dense gate matrix that is zero off the selected active routes.
* ``moe.moe_ref_blocked`` -- the same fp64 mathematics, expert-major, with the
  products done by BLAS dgemm.  It is the timed CPU baseline.
* ``router.route_topk`` -- top-k expert selection from router logits with
  renormalised gates; the pages keep native top-6 routing and the selected-row
  order ("perf(ds4): extend sparse prefill scheduling to 10K", Summary) and
  leave the arithmetic to the model (reading in the module).
* ``moe.combine_ref`` -- the fused route combine ("perf(ds4): accelerate ROCm
  decode and long-context selection", lucebox8 gfx1151 A/B; "... 10K",
  Historical fused-combine discriminator).
* ``numerics`` -- bf16 round-to-nearest-even, OCP E4M3FN decode/encode
  (round-to-nearest-even, saturating to +-448) and per-row fp8 quantisation
  with an fp32 scale amax/448.  The pages never define their own low-bit
  formats; the fp8 workload uses the OCP 8-bit floating point format.

Precision contract shared with the HIP path (a reading, the pages are silent):
the SwiGLU output h is rounded to bf16 before the down projection; y, the
combine and the output stay fp32 on the GPU and fp64 here.

Pins (tests marked "not gpu"): torch's CPU bf16 and float8_e4m3fn
conversions, the OCP E4M3 landmark values in tests/golden, numpy's bincount /
stable argsort, brute-force dense evaluation, the single-expert case against a
torch CPU SwiGLU MLP, and invariants (zero input, masked routes, power-of-two
gate scaling, token permutation).  Every function above has at least one pin.
"""

from . import numerics, route, moe  # noqa: F401

__all__ = ["numerics", "route", "moe"]

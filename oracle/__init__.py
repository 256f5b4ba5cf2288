"""CPU oracle for the MoE layer hot path. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never imports, calls or links anything here, and this
package imports nothing from the product path: the two share no code. The
only module both sides use is ``workloads`` (seeded input generation, which
holds none of the layer's arithmetic).

Everything here is plain NumPy in float64 (integer work in int64), written
for a reader to check against the pages by eye; it is slow on purpose.

Pages cited (titles as published):
  [R] "Mixture-of-Kittens: a deterministic MoE megakernel for NVL72 racks"
      (hysenlabs.com project review of the MoK README).
  [A] "nemo_automodel.components.moe.mok_experts" (NeMo AutoModel API page
      for the MoK expert backend).
  [B] the moses-y.github.io blog review "mixture-of-kittens".

Modules:
  schedule  -- counts, capacity, padded offsets, stable permutation, inverse
               map, per-minibatch sub-offsets ([R] §"The two API layers and
               the schedule object", §"Tuning the five hyperparameters before
               production").
  mxfp8     -- OCP E4M3 codec, E8M0 block scale, quantize / dequantize along
               a chosen axis in 32-element blocks ([R] §"Tuning the five
               hyperparameters before production", MXFP8 workflow).
  moe       -- forward (routed SwiGLU experts + shared expert + router-weighted
               combine) and backward, in float64; MXFP8-emulated variants.

Parity status: every function here is pinned by a test in
``tests/test_oracle_*.py`` against something other than itself (brute force,
closed forms, a library routine, finite differences, autograd); see each
function's docstring for its pin. The MoK library's own numerics (its exact
schedule layout, padding, drop rule and quantizer rounding) are not given on
the pages; where the pages are silent this oracle takes a stated reading.
"""

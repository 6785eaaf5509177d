"""CPU oracle for the 2-bit sign-symmetric routed-expert MoE forward and the NVFP4 -> 2-bit
re-quantizer.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call, link or execute anything
under this directory; only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it. It shares no code with ``bit_routed_expert_amd`` (no kernels, headers, tables,
helpers or constants) and imports nothing from it.

What it computes is written from the pages that describe the method (vLLM-Moet):

* README (wiki page), bullet "2-bit expert planes - the sign-bias finding": routed experts use the
  sign-symmetric codebook {-4, -1, 1, 4}.
* "The v0.24.0 port" page, section "Our hooks", bullet "modelopt.py (ModelOptNvFp4FusedMoE)":
  NVFP4 experts (e2m1 codes x e4m3 block-16 scales x per-tensor fp32 scale_2) are dequantized to
  f64 exactly and re-quantized to the codebook with UE8M0 block-32 scales that absorb scale_2.
* same page, bullet "Deterministic unpermute": valid sorted ids are a permutation of
  token*top_k+j; per-pair outputs are placed bijectively and summed in a fixed order.
* starlog article "Running 753B MoE Models on Consumer GPUs", section "Technical Insight": the
  illustrative kernel's comment gives the code order {0,1,2,3} -> {-4,-1,1,4}.

Modules:
  formats  - the number formats (codebook, UE8M0, e2m1, e4m3) and the canonical code packing.
  forward  - routing and the f64 forward (definition written out; numpy matmul as the only
             library step).
  requant  - the re-quantizers (NVFP4, FP8 block-128 and MXFP4 inputs): an exact Fraction
             reference for small inputs and a ctypes wrapper around ``requant_exact.c`` (exact
             integer arithmetic) for large ones.
  sweep    - the sign-bias codebook sweep (README bullet "2-bit expert planes - the sign-bias
             finding"): an exact Fraction reference for single blocks and a ctypes wrapper around
             ``codebook_sweep.c`` (float64 in element order) for whole tensors.

Parity status of each function is stated in its docstring; every function here is pinned by a
``-m "not gpu"`` test except where a docstring says "parity unpinned".
"""

"""CPU oracle for paged GQA attention: TEST INFRASTRUCTURE, not part of the product.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
package. It shares no code with the HIP library or its Python binding and imports
neither: it takes plain numpy arrays (values, raw bits or FP8 codes) and computes in
float64, with float32 only where the quantiser fixes float32 arithmetic.

Modules
  fp8    OCP e4m3fn codec written from the format definition (decode table, nearest-
         value encoder with ties to even and saturation) and the per-token-per-head
         absmax/448 quantiser.
  int8   symmetric int8 codec: absmax/127 per-token-per-head quantiser (nearest
         integer, ties to even, clamp to [-127, 127]) and its dequantisation.
  blocks reference block manager (allocation, prefix sharing of full blocks, copy-on-
         write) in plain lists, for the host block manager's index work.
  rope   rotary position embedding (pair i with i + D/2, table-driven, fp32 with every
         operation rounded) and the fused RoPE + KV store built on ref's stores.
  ref    the plain definition: store through slot_mapping, gather the paged KV of each
         sequence through its block table, then dense causal softmax attention; also
         partial (lse, o) over a key subset and their log-sum-exp merge.
  brute  pure-Python loops with math.fsum, per-token block-table lookup and no
         max-subtraction: a second, structurally different implementation used to pin
         `ref` on tiny inputs.

Pins: every function here is checked by the `-m "not gpu"` tests against closed forms,
hand-computed fixtures under tests/golden/, invariants, a library routine (torch's
float8_e4m3fn cast) and the brute force. See the module docstrings for what pins what.
"""

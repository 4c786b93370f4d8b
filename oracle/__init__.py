"""Reference oracle for TurboQuant-style compressed KV attention.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU
baseline leg of the benchmark may import this package.  The product library
(the C-ABI shared object and its Python binding) never calls into it, and this
package imports nothing from the product: the two share no code, no tables and
no constant generators.

Everything here is plain, slow, float64 NumPy (plus pure-Python loops for the
random-number generator), written step by step from the pages it follows:

* "turbo-attn 0.24.0" (PyPI page), sections "How it works" and
  "Configuration": rotate, store the magnitude, quantise each rotated
  coordinate to a shared codebook; rotate the query once and attend in the
  rotated space; split-K paged decode.
* "How 0xsero/turboquant works", sections "Compression Pipeline",
  "Key Storage and Attention Scoring" and "Value Compression": random
  orthogonal rotation, Lloyd-Max scalar codebook and a QJL residual-sign
  projection for keys; per-group scale/zero low-bit values with packed
  payloads.
* "5x Faster LLM Inference? This KV Cache Hack Changes Everything", sections
  "What is TurboQuant-GPU?" and "Example 4: Kernel-Level Operations":
  normalise -> rotate -> Lloyd-Max quantise -> pack; a rotation fixed per head
  applied to both keys and values; fused attention over compressed K/V; 3-bit
  MSE-coded values beside 2-bit keys with QJL (the value mode "mse").
* "tiny-turboquant 0.18.0", sections "Knobs that actually move the needle"
  and "Measured quality": the K4/V4 ... K3/V2 presets, value groups of 32.

Where the pages leave a step open the oracle takes one stated reading; every
reading is listed in the design notes of the repository.

Parity status: every public function is pinned by a CPU test against values
fixed by mathematics (closed forms, textbook Lloyd-Max tables, published
SplitMix64 output, statistical identities) or against brute force.  The one
exception is attention *quality* against uncompressed attention, which the
pages give no number for: it is reported, not pinned (parity unpinned).
"""


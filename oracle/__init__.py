"""CPU oracle for the quantized decode / routed-expert path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product (the HIP library and its Python binding) never calls it, and this
package never imports the product.

Everything here is a plain, slow, obviously correct restatement of what the
path computes, in float64 NumPy:

* ``oracle.formats``  -- the block formats: quantizer, packer, unpacker,
  exact dequantization (Q8_0, Q4_0, MXFP4, Q4_K, Q6_K and the ternary T5).
* ``oracle.moe``      -- dense quantized GEMV, router + softmax top-k,
  expert permutation, expert FFN with SwiGLU, weighted combine, the whole
  routed-expert layer, and the per-element error bounds used for parity.
* ``oracle.mx``       -- MXFP8 (E4M3) activation quantization and the MX GEMM
  reference for MXFP4 weights on block-scaled matrix cores.
* ``oracle.int8``     -- int8 activation quantization and the Q8_0 x int8
  GEMV reference (integer dot products).
* ``oracle.brute``    -- pure-Python scalar loops for tiny cases, used only to
  cross-check the vectorised oracle.

Parity status: every public function is pinned by a CPU test in
``tests/test_oracle_*.py`` against something other than the oracle itself:
closed-form blocks and quantizer error bounds (``formats``, ``mx``,
``int8``), scalar loops over the packed bytes and exhaustive code searches
(``brute``, the MX expert FFN, the int8 GEMV), enumeration of every k-subset
(``topk`` and the selection margin ``topk_gap``), NumPy's stable argsort
(``permute``) and layer invariants (top-1 routing equals the dense FFN, token
reordering, shared-only routing).  The helpers ``router_logits``,
``softmax_over`` and ``silu`` are pinned through ``route`` and the brute-force
layers that call them.
"""

"""CPU oracle for the splash-attention forward path (TEST INFRASTRUCTURE ONLY).

This package is the slow, obviously-correct reference that the GPU path is
checked against. Only the test-suite, the smoke check in the repository entry
module and the CPU-baseline leg of the benchmark may import it; the product
path (the C-ABI library and its Python binding) never does, and this package
imports nothing from the product.

Sources (the pages):
  * "Splash Attention: When the Mask Stops Being Arithmetic and Becomes the
    Loop" (explainers.rudrite.com/splash-attention), FAQ answers "What is
    splash attention...", "What is MaskInfo...", "Does splash attention make
    every sparse mask faster?" and "What does grid shrinking do...".
  * "Flash Attention on a TPU, Line by Line"
    (explainers.rudrite.com/pallas-flash-attention-tpu), FAQ answer "What
    does the TPU flash attention kernel save for the backward pass?".
  * EasyDeL BlockSparseAttn module page, forward_native (default softmax
    scale head_dim ** -0.5, GQA head shapes, logits_soft_cap parameter).

Modules:
  masks      -- the mask definitions, materialised as dense bool arrays.
  mask_info  -- MaskInfo built by the plain any/all definition.
  attention  -- dense fp64 masked softmax attention, (out, lse).

Every function is pinned by tests/test_oracle_*.py against page-printed
counts, closed forms, brute force and library routines.  The fill values of
data_next / mask_next at empty or non-partial grid positions are fixed only by
a convention (next slot, else previous slot, else 0): parity unpinned by the
pages for those entries; the reconstruction invariant pins every entry the
kernel actually reads.
"""

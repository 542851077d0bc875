"""MI355X (gfx950) implementation of the Qwen Sparse Attention hot path.

The computation runs in the HIP library ``libqsa.so`` (built from ``csrc/``);
:mod:`.binding` marshals torch tensors into its C ABI.  Nothing here computes
on the CPU.
"""

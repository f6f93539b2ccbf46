"""mask_only_logits_amd: mask-only LM-head logits on MI355X (gfx950).

The hot path lives in a C-ABI shared library (``libmosaic.so``, declared in
``include/mosaic.h``) built from hand-written HIP kernels under ``csrc/``:
stream compaction of the mask into an ascending index list, a fused gather-GEMM
``logits[M, V] = H[idx, :] . W^T`` that reads the masked rows through the index
list, and a row-chunk driver.  ``mosaic`` is the thin ctypes binding over it;
``inputs`` draws the seeded synthetic workloads.
"""

"""Absorbed Multi-head Latent Attention decode for MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``libmla_latent.so``, declared in ``include/mla_latent.h``); ``binding``
wraps its calls with the same names for torch tensors.  ``inputs`` draws the
seeded synthetic batches.
"""

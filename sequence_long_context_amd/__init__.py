"""Ulysses attention hot path for MI355X (gfx950).

The sequence-shard <-> head-shard layout change of DeepSpeed-Ulysses,
simulated over P virtual ranks in one GPU's HBM, and each rank's local
full-sequence attention, as hand-written HIP kernels behind a C ABI
(``libulysses.so``).  ``ulysses`` is the thin ctypes binding; importing the
package does not load the library, so CPU-only tools can use ``synth``.
"""

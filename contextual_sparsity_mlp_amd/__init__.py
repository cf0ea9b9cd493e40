"""Deja Vu contextual-sparsity decode step for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libdv.so`` built from ``csrc/`` (hand-written
HIP); ``contextual_sparsity_mlp_amd.dv`` is its thin ctypes binding.  Importing this
package loads nothing; the binding loads the library on first use and raises if it
is missing.
"""

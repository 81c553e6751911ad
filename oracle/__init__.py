"""CPU oracle of the affine group-quantized qmv -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  The GPU library and its Python binding never do.
"""

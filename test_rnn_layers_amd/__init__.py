"""libttt: the TTT layer hot path (TTT-Linear / TTT-MLP mini-batch test-time
training in the dual form) as HIP kernels for MI355X (gfx950) behind a C ABI.

``libttt`` is the ctypes binding (functions named as in include/ttt.h);
``synth`` draws the seeded synthetic inputs; ``build_lib`` compiles the
shared library in-tree.
"""
from . import libttt  # noqa: F401

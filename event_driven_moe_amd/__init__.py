"""Event Tensor megakernels for MI355X (gfx950).

The library itself is ``libet.so`` (C ABI in ``include/et.h``); ``et`` is its
Python binding and ``synth`` the seeded input generators.
"""

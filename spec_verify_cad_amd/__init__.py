"""MI355X-native span-commit / verify path: n-gram draft lookup, span forward
(causal-span or block-triangular mask) and acceptance scan, as hand-written HIP
kernels for gfx950 behind a C-ABI library (`libcad.so`).

`spec_verify_cad_amd.cad` is the thin ctypes binding; importing this package does not
load the library, calling into the binding does (and fails loudly if it is missing).
"""
__all__ = ["synth", "configs"]

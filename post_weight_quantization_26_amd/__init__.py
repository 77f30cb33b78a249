"""AWQ per-layer activation-aware scale search on MI355X (gfx950).

The computation lives in the HIP library behind the C ABI of include/awq.h.
Submodules: ``api`` (torch-facing wrappers; the library is loaded on first
use and any call fails loudly if it was not built), ``synth`` (seeded
synthetic layers), ``build_lib`` (hipcc build).
"""

"""PCP-sharded MLA prefill attention with an LSE/sink merge, for MI355X (gfx950).

The work runs in ``libmla_pcp.so`` (hand-written HIP kernels behind the C ABI in
``include/mla_pcp.h``); ``_lib`` is its ctypes binding, ``pipeline`` the device
plumbing for one step, ``synth`` the seeded synthetic inputs and ``build`` the hipcc
build. Importing the package loads nothing; the library is loaded on first use.
"""
__all__ = ["_lib", "pipeline", "synth", "build"]

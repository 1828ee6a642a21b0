"""Cascade attention for the target-verify step of top-k tree speculative decoding,
built for AMD Instinct MI355X (gfx950).

The compute path lives in a C-ABI shared library (``libcascade_attn.so``, sources
under ``csrc/``).  ``binding`` is a thin ctypes layer over it with the same entry
point names; ``workload`` draws the seeded synthetic inputs.  Importing this
package loads nothing: the library is opened on first use and every entry point
raises if it is missing.
"""

__all__ = ["binding", "workload"]

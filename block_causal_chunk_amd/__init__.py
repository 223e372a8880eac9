"""block_causal_chunk_amd: block-causal mixed-noise chunk attention for MI355X (gfx950).

The compute lives in ``libwfattn.so`` (hand-written HIP kernels behind a C ABI declared in
``include/wfattn.h``); ``binding`` is a thin ctypes layer with the same names.  Importing this
package loads nothing; ``binding`` loads the library on first use and raises if it is missing.
"""

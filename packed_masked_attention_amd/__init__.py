"""MI355X-native packed masked attention for the MiniMax-H3 DiT block.

The compute lives in a HIP/C library (``libpma.so``, built from ``csrc/`` for
gfx950) behind the C ABI declared in ``include/pma.h``.  ``binding`` marshals
arguments to it; ``synth`` makes seeded synthetic inputs.  Importing this
package loads nothing: ``binding`` loads the library on first use and raises
if it has not been built.
"""
__all__ = ["binding", "synth"]

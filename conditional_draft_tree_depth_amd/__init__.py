"""MI355X-native construction of conditional draft trees (DARTree-style
depth-wise build over a Domino-corrected drafter).

The compute lives in ``libdtree.so`` (hand-written HIP for gfx950, C ABI in
``include/dtree.h``); ``_lib`` is its thin ctypes binding.  Importing this
package loads nothing; ``_lib.load()`` opens the library and fails loudly if
it has not been built.
"""

"""MI355X-native modality-aware short convolution + Kimi Delta Attention forward.

The package holds three things:

* ``inputs``  -- seeded synthetic token streams (shapes and value distributions
  only; none of the method's arithmetic lives there);
* ``kda``     -- the thin ctypes binding over the C-ABI library ``libkdaconv.so``
  (argument marshalling only: every step of the path runs in the HIP kernels);
* ``csrc/``   -- the HIP kernels for gfx950 and the C-ABI host code.

Nothing is imported eagerly so that ``inputs`` can be used without loading the
HIP library.
"""

__all__ = ["inputs", "kda"]

"""k-Maximum-Inner-Product attention on AMD MI355X (gfx950): libkmip and its
Python binding.  Import of this package does not load the library; the first
call does, and fails loudly if libkmip.so has not been built."""
from . import kmip  # noqa: F401

"""GPipe pipeline-cell training step for AMD Instinct MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``csrc/``, declared in ``include/gpipe.h``); ``gpipe`` is its thin ctypes
binding.  Importing this package loads nothing; ``gpipe.lib()`` loads the
library and raises if it has not been built.
"""

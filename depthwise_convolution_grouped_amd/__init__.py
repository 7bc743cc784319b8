"""MI355X-native grouped / depthwise convolution forward.

The compute path is the C-ABI library ``libgconv.so`` (hand-written HIP for
gfx950, declared in ``include/gconv.h``); ``gconv`` is its thin ctypes
binding.  Importing this package loads nothing: the library is opened on the
first call into ``gconv``, which raises if it has not been built.
"""

__all__ = ["gconv", "inputs", "metrics"]

"""MI355X (gfx950) SVDQuant W4A4 + low-rank linear layer and INT8 KV-cache quantizer.

The compute lives in ``lib/libsvdq.so`` (hand-written HIP behind the C ABI of
``include/svdq.h``); ``binding`` exposes its entry points to Python under the same names and
``layer`` wires them into a linear layer.  Importing this package does not load the library;
``binding.load()`` does, and fails loudly if it has not been built.
"""
from . import binding  # noqa: F401

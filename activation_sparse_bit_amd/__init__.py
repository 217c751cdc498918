"""MI355X-native dynamically sparse int4 GEMV.

The kernels and the C ABI live in ``csrc/`` and are built into
``lib/libsgemv.so`` by ``build.build()``; ``sgemv`` is the Python binding.
Importing the package loads nothing; ``sgemv.lib()`` loads the library and
raises if it is missing (there is no fallback path).
"""

"""MI355X (gfx950) W8A8 INT8 linear layer: HIP kernels behind a C ABI.

``int8_w8a8_quantized_amd.lib`` is the thin ctypes binding of ``libw8a8.so``
(argument marshalling only); ``synth`` draws seeded synthetic inputs.
Importing the package loads nothing: the library is opened on first use and
a missing library is an error, never a fallback.
"""

"""MI355X-native MXFP8 partial amax / combine / scale / cast (distributed master-weight
writeback), as hand-written HIP kernels for gfx950 behind a C ABI.

The Python layer only marshals torch tensors (device memory and streams) into the C ABI;
every step of the path runs in the HIP kernels of ``libmxfp8partial.so``.
"""

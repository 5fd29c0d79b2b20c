"""MI355X (gfx950) tile rasteriser for 3D Gaussian splatting.

The compute path is libgsraster.so (HIP kernels behind the C ABI in include/gs_raster.h);
``raster`` is its ctypes binding and ``scenes`` draws seeded synthetic inputs.
"""

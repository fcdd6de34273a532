"""MI355X (gfx950) hot path of RaBiT-style 2-path residual binarization.

librabit.so (HIP kernels + C ABI, include/rabit.h) does the work; `rabit` is
its ctypes binding. Build with `python -m bit_residual_binarized_amd.build`.
"""

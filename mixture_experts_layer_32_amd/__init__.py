"""MI355X-native fused MoE layer (forward and backward) behind a C ABI (include/moe.h).

The compute path is the HIP library libmoe.so, built for gfx950. This package holds only two
things:
 * its ctypes binding (argument marshalling);
 * the seeded input generator.
"""

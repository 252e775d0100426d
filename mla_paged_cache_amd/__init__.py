"""MI355X-native splice / evict path for a paged MLA KV cache.

The work happens in libleyline.so (HIP kernels for gfx950 and a C++ host
planner behind the C ABI of include/leyline.h); `leyline` is its Python
binding."""

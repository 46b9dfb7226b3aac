"""MI355X-native HSTU block forward over jagged per-user sequences with a paged
KV cache.  The compute lives in libhstu.so (HIP kernels for gfx950 behind the C
ABI in include/hstu.h); `hstu` is its ctypes binding, `runtime` drives a
request through it with torch device memory, and `workloads` draws seeded
synthetic inputs."""

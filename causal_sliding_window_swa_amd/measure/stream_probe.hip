// stream_probe.hip -- measurement support, not part of the attention library:
// the HBM read bandwidth a plain streaming kernel reaches on this GPU, the
// practical ceiling beside the 8 TB/s specification for the memory-bound
// decode step.  Each thread reads 16-byte pieces in a grid-stride loop, four
// loads in flight, and folds them into one value per block so that no load
// can be dropped.  Built into libswa_measure.so (C ABI below).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *p, size_t n16,
                                                          uint32_t *out) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(p + i);
        const u32x4 b = __builtin_nontemporal_load(p + i + stride);
        const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3];
        acc ^= c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
    }
    for (; i < n16; i += stride) {
        const u32x4 a = p[i];
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
    __shared__ uint32_t red[256];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int t = 0; t < 256; t++) r ^= red[t];
        out[blockIdx.x] = r;
    }
}

}  // namespace

// Reads `bytes` (a multiple of 16) at device pointer `buf` once; `out` is
// device memory for `blocks` uint32 values.  Returns 0, or a HIP error code.
extern "C" int swa_measure_stream_read(const void *buf, size_t bytes, uint32_t *out, int blocks,
                                       void *stream) {
    if (!buf || !out || blocks < 1 || bytes % 16) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4 *)buf, bytes / 16, out);
    return (int)hipGetLastError();
}

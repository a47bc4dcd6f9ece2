// stream_read.hip -- calibration kernel for the benchmark's measured ceilings
// (not part of the attention path): a read-only stream over a device buffer, to
// give the HBM read rate this GPU reaches in the same session.  Every 16-byte
// piece is loaded once (grid-stride, 8 loads in flight per thread) and folded
// into an XOR that each thread stores, so no load can be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *__restrict__ p, size_t n16,
                                                          uint32_t *__restrict__ out) {
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 7 * stride < n16; i += 8 * stride) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            v[u] = p[i + u * stride];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

// Read `bytes` (a multiple of 16) from device buffer p with `blocks` workgroups of
// 256 threads; out receives blocks * 256 uint32 values.  Returns a hipError_t.
extern "C" int calib_stream_read(const void *p, size_t bytes, uint32_t *out, int blocks,
                                 void *stream) {
    if (!p || !out || blocks <= 0 || bytes % 16 != 0)
        return (int)hipErrorInvalidValue;
    stream_read_kernel<<<dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream>>>(
        (const uint4 *)p, bytes / 16, out);
    return (int)hipGetLastError();
}

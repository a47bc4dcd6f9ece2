// stream_read.hip -- calibration kernel for the benchmark's measured ceilings
// (not part of the attention path): a read-only stream over a device buffer, to
// give the HBM read rate this GPU reaches in the same session.  Each workgroup
// reads one contiguous chunk (8 loads in flight per thread) with non-temporal
// loads -- the fastest streaming form measured on MI355X (4 GiB: ~7.0 TB/s,
// against ~5.6-5.8 TB/s with plain loads) -- and folds every 16-byte piece into
// an XOR that each thread stores, so no load can be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *__restrict__ p, size_t n16,
                                                          uint32_t *__restrict__ out) {
    // chunk of this workgroup: [c0, c1)
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t c0 = (size_t)blockIdx.x * per;
    const size_t c1 = c0 + per < n16 ? c0 + per : n16;
    size_t i = c0 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 7 * 256 < c1; i += 8 * 256) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            v[u] = __builtin_nontemporal_load((const u32x4 *)(p + i + u * 256));
#pragma unroll
        for (int u = 0; u < 8; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < c1; i += 256) {
        const u32x4 v = __builtin_nontemporal_load((const u32x4 *)(p + i));
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

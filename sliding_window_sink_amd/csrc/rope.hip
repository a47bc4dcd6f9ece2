// rope.hip -- partial rotary position embedding, in place (gfx950).
//
// MiMo-V2-Flash Technical Report, Section 2.1: RoPE is applied only to the
// first 64 of the 192 query/key dims; Section 3.2 gives the bases (1e4 for SWA
// layers; 6.4e5, later 5e6, for global layers).  Pair c (c < rope_dim/2) is
// rotated by angle pos * base^(-2c/rope_dim) (RoFormer).
//
// The angle is formed in fp64: in fp32, pos * theta loses ~1e-3 of a radian
// near position 1e5, which is visible at fp32 tolerance.  Each workgroup
// handles kTokens tokens: it first evaluates cos/sin once per (token, pair) in
// fp64 into LDS, then every (token, head, pair) rotation reads them, so the
// fp64 work does not scale with the head count.  Dims >= rope_dim are never
// touched.  Traffic is one read and one write of the rotated dims.
#include "common.h"

namespace sinkattn {
namespace {

constexpr int kThreads = 256;
constexpr int kTokens = 8;
constexpr int kMaxPairs = 128;  // rope_dim <= 256

template <typename T>
__device__ __forceinline__ float load_f(const T *p);
template <>
__device__ __forceinline__ float load_f<float>(const float *p) { return *p; }
template <>
__device__ __forceinline__ float load_f<uint16_t>(const uint16_t *p) { return bf16_bits_to_f32(*p); }

__device__ __forceinline__ void store_f(float *p, float v) { *p = v; }
__device__ __forceinline__ void store_f(uint16_t *p, float v) { *p = f32_to_bf16_bits(v); }

template <typename T>
__global__ __launch_bounds__(kThreads) void rope_kernel(T *x, int64_t n_tok, int n_heads,
                                                        int head_dim, int rope_dim,
                                                        const int32_t *pos, double base, int style) {
    __shared__ float cs[kTokens][kMaxPairs][2];
    const int half = rope_dim / 2;
    const int64_t tok0 = (int64_t)blockIdx.x * kTokens;
    const int ntok = (int)min<int64_t>(kTokens, n_tok - tok0);
    for (int idx = threadIdx.x; idx < ntok * half; idx += kThreads) {
        const int tt = idx / half, c = idx % half;
        const float2 v = rope_cos_sin(pos[tok0 + tt], rope_inv_freq(base, c, rope_dim));
        cs[tt][c][0] = v.x;
        cs[tt][c][1] = v.y;
    }
    __syncthreads();
    const int per_tok = n_heads * half;
    for (int idx = threadIdx.x; idx < ntok * per_tok; idx += kThreads) {
        const int tt = idx / per_tok;
        const int rem = idx % per_tok;
        const int h = rem / half, c = rem % half;
        T *row = x + ((tok0 + tt) * n_heads + h) * (int64_t)head_dim;
        const int i0 = style == 0 ? 2 * c : c;
        const int i1 = style == 0 ? 2 * c + 1 : c + half;
        const float x0 = load_f(row + i0), x1 = load_f(row + i1);
        float y0, y1;
        rope_pair(x0, x1, make_float2(cs[tt][c][0], cs[tt][c][1]), y0, y1);
        store_f(row + i0, y0);
        store_f(row + i1, y1);
    }
}

// The common case -- bf16 rows, interleaved pairs, rope_dim 64, head_dim a
// multiple of 8, 16-byte aligned rows -- with 16-byte accesses: one thread per
// 8-dim chunk of the rotated dims (four pairs), the same cos/sin and rounding as
// rope_kernel.  (rope_kernel moves 2-byte elements, which leaves the memory
// system mostly idle.)
__global__ __launch_bounds__(kThreads) void rope_vec_kernel(uint16_t *x, int64_t n_tok, int n_heads,
                                                            int head_dim, const int32_t *pos,
                                                            double base) {
    __shared__ float2 cs[kTokens * 32];
    const int64_t tok0 = (int64_t)blockIdx.x * kTokens;
    const int ntok = (int)min<int64_t>(kTokens, n_tok - tok0);
    for (int idx = threadIdx.x; idx < ntok * 32; idx += kThreads)
        cs[idx] = rope_cos_sin(pos[tok0 + (idx >> 5)], rope_inv_freq(base, idx & 31, 64));
    __syncthreads();
    const int per_tok = n_heads * 8;  // 8 chunks of 8 dims = the 64 rotated dims
    for (int idx = threadIdx.x; idx < ntok * per_tok; idx += kThreads) {
        const int tt = idx / per_tok, rem = idx % per_tok;
        const int h = rem >> 3, ci = rem & 7;
        uint4 *p = (uint4 *)(x + ((tok0 + tt) * n_heads + h) * (int64_t)head_dim) + ci;
        *p = rope_chunk_bf16(*p, cs + tt * 32 + 4 * ci);
    }
}

// Out-of-place variant for bf16 rows of 192 dims at positions 0..T-1 of each
// sequence (the keys of a prefill with the RoPE fused): one thread per 16-byte
// chunk; chunks 0..7 (dims 0..63, interleaved pairs) are rotated with the same
// cos/sin and rounding as rope_kernel, the rest are copied.
__global__ __launch_bounds__(kThreads) void rope_rows_kernel(const uint4 *src, uint4 *dst,
                                                             int64_t n_tok, int T, int n_heads,
                                                             double base) {
    __shared__ float2 cs[kTokens * 32];
    const int64_t tok0 = (int64_t)blockIdx.x * kTokens;
    const int ntok = (int)min<int64_t>(kTokens, n_tok - tok0);
    for (int idx = threadIdx.x; idx < ntok * 32; idx += kThreads)
        cs[idx] = rope_cos_sin((int)((tok0 + (idx >> 5)) % T), rope_inv_freq(base, idx & 31, 64));
    __syncthreads();
    constexpr int kChunks = kDqk / 8;
    const int per_tok = n_heads * kChunks;
    for (int idx = threadIdx.x; idx < ntok * per_tok; idx += kThreads) {
        const int tt = idx / per_tok, ci = (idx % per_tok) % kChunks;
        const int64_t at = tok0 * per_tok + idx;
        uint4 x = src[at];
        if (ci < 8)
            x = rope_chunk_bf16(x, cs + tt * 32 + 4 * ci);
        dst[at] = x;
    }
}

}  // namespace

hipError_t launch_rope_rows(const void *src, void *dst, int B, int T, int n_heads, double base,
                            hipStream_t s) {
    const int64_t n_tok = (int64_t)B * T;
    if (n_tok == 0 || n_heads == 0)
        return hipSuccess;
    const unsigned blocks = (unsigned)((n_tok + kTokens - 1) / kTokens);
    rope_rows_kernel<<<dim3(blocks), dim3(kThreads), 0, s>>>((const uint4 *)src, (uint4 *)dst,
                                                             n_tok, T, n_heads, base);
    return hipGetLastError();
}

hipError_t launch_rope(void *x, int bf16, int64_t n_tok, int n_heads, int head_dim, int rope_dim,
                       const int32_t *pos, double base, int style, hipStream_t s) {
    if (n_tok == 0 || n_heads == 0 || rope_dim == 0)
        return hipSuccess;
    const unsigned blocks = (unsigned)((n_tok + kTokens - 1) / kTokens);
    if (bf16 && style == 0 && rope_dim == 64 && head_dim % 8 == 0 &&
        reinterpret_cast<uintptr_t>(x) % 16 == 0)
        rope_vec_kernel<<<dim3(blocks), dim3(kThreads), 0, s>>>((uint16_t *)x, n_tok, n_heads,
                                                                head_dim, pos, base);
    else if (bf16)
        rope_kernel<uint16_t><<<dim3(blocks), dim3(kThreads), 0, s>>>(
            (uint16_t *)x, n_tok, n_heads, head_dim, rope_dim, pos, base, style);
    else
        rope_kernel<float><<<dim3(blocks), dim3(kThreads), 0, s>>>(
            (float *)x, n_tok, n_heads, head_dim, rope_dim, pos, base, style);
    return hipGetLastError();
}

}  // namespace sinkattn

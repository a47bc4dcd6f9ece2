// common.h -- device helpers shared by the gfx950 sink-attention kernels.
//
// MFMA lane layouts used throughout (v_mfma_f32_32x32x16_bf16, one wave64):
//   A (32 x 16):  lane l holds row l%32, k = (l/32)*8 + e for its 8 bf16 e.
//   B (16 x 32):  lane l holds col l%32, k = (l/32)*8 + e.
//   C (32 x 32):  lane l, register i holds row (i/4)*8 + (l/32)*4 + i%4, col l%32.
// The contraction index of A and B only has to agree between the two operands,
// so every kernel is free to map (k-step, lane half, element) to any head-dim
// or key index it likes; the comments at each use say which mapping it takes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace sinkattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kDqk = 192;
constexpr int kDv = 128;

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ uint4 as_uint4(const bf16x8 &b) { return __builtin_bit_cast(uint4, b); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
    return __builtin_bit_cast(float, (uint32_t)h << 16);
}
// Two floats -> one dword holding (lo, hi) bf16, round to nearest even.  Built as
// a two-element vector so the pair becomes one v_cvt_pk_bf16_f32 (packing two
// separate conversions costs a shift and an or on top of two conversions).
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2v v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- buffer (descriptor) memory access ----
// A raw buffer descriptor covers [base, base + bytes); the hardware returns 0
// for loads and drops stores whose offset falls outside it, so ragged tails
// need no branches, and addresses are a wave-uniform descriptor plus a 32-bit
// per-lane byte offset.  Word 3 (0x00020000) is the raw-buffer format of gfx9.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ BufRsrc make_buf(const void *base, uint64_t bytes) {
    const uint32_t n = bytes > 0x7FFFFFF0ull ? 0x7FFFFFF0u : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n,
                                             0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(BufRsrc r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint2 buf_load8(BufRsrc r, uint32_t off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store16(BufRsrc r, uint32_t off, uint4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
}
__device__ __forceinline__ void buf_store8(BufRsrc r, uint32_t off, uint2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, 0);
}
// Streaming variants with the non-temporal cache policy (the "nt" bit of the
// gfx950 buffer instructions), for data read or written exactly once: a
// decode's or verify's KV cache, a prefill's q and o.  Measured on MI355X: a
// plain 4 GiB read stream 5.6-5.8 TB/s, the same stream with nt loads 6.9-7.0
// TB/s.
constexpr int kCacheNt = 2;
__device__ __forceinline__ uint4 buf_load16_nt(BufRsrc r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCacheNt));
}
__device__ __forceinline__ uint2 buf_load8_nt(BufRsrc r, uint32_t off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCacheNt));
}
__device__ __forceinline__ void buf_store16_nt(BufRsrc r, uint32_t off, uint4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCacheNt);
}

// Online-softmax rescale threshold (log2 units): the running max is only
// raised when a block's max exceeds it by more than this, so exp2(x - m) stays
// <= 2^8 and the accumulator rescale is rare.  Any m works (it cancels in
// acc / l); this only trades a bounded growth of p for fewer rescales.
constexpr float kRescaleSlack = 8.0f;

// Cross-lane exchanges on the VALU (gfx950's v_permlane32_swap / v_permlane16_swap)
// instead of a ds_bpermute round trip through the LDS unit, which sat on the
// softmax's critical path once per key block.  permlane32_swap(a, b) swaps rows
// 2-3 of a with rows 0-1 of b (a row is 16 lanes); with a = b = x the two results
// hold, in every lane l, x of lane l % 32 and of lane l % 32 + 32.
// permlane16_swap(a, b) swaps the odd rows of a with the even rows of b: the
// results hold x of rows (0, 1) in rows 0-1 and of rows (2, 3) in rows 2-3.
__device__ __forceinline__ float2 lanes_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float2 lanes_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Max / sum over the two 32-lane halves of a wave (lanes l and l^32 hold the same
// column); the sum adds the lower half's value first in both lanes (the same bits
// as x + x(l^32) in either lane: addition commutes).
__device__ __forceinline__ float max_across_halves(float x) {
    const float2 h = lanes_xor32(x);
    return fmaxf(h.x, h.y);
}
__device__ __forceinline__ float sum_across_halves(float x) {
    const float2 h = lanes_xor32(x);
    return h.x + h.y;
}
// Over the four 16-lane rows (lanes l, l^16, l^32, l^48 hold the same column).
__device__ __forceinline__ float max_across_rows(float x) {
    const float2 h = lanes_xor16(x);
    return max_across_halves(fmaxf(h.x, h.y));
}
__device__ __forceinline__ float sum_across_rows(float x) {
    const float2 h = lanes_xor16(x);
    return sum_across_halves(h.x + h.y);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        x += __shfl_xor(x, o, 64);
    return x;
}

// Row of the 32x32 C tile held by register i of a lane in half `hh` (= lane/32).
__device__ __forceinline__ int c_row(int i, int hh) { return (i >> 2) * 8 + hh * 4 + (i & 3); }

// Key order inside a 32-key block: the A-operand row r that must hold key kk so
// that register i of lane half hh ends up holding key 16*hh + i.
__host__ __device__ __forceinline__ int row_of_key(int kk) {
    const int hh = kk >> 4, a = (kk >> 2) & 3, b = kk & 3;
    return a * 8 + hh * 4 + b;
}
__host__ __device__ __forceinline__ int key_of_row(int r) {
    return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
}

// Which (key, 8-dim chunk) of a 32-key x 128-dim V block thread tid (of 512)
// stages.  Each wave takes 16 keys x 4 chunks, the chunks chosen so that the
// scattered 2-byte writes into the transposed V^T tile (rows pv_row_of_dim,
// 80-byte pitch) land in 32 distinct LDS banks; the plain 4-keys x 16-chunks
// order aliased them 4-way.
__device__ __forceinline__ void v_stage_coords(int tid, int &kk, int &dc) {
    const int wave = tid >> 6, lane = tid & 63, s = wave >> 1, idx = lane >> 4;
    kk = (lane & 15) + 16 * (wave & 1);
    dc = (s & 1) * 2 + (s >> 1) * 8 + (idx & 1) + (idx >> 1) * 4;
}

// ---- partial RoPE (shared by the standalone kernel and the fused prefill) ----
// theta_c = base^(-2c/rope_dim), angle = pos * theta_c, both in fp64 (an fp32
// angle is off by ~1e-3 rad near position 1e5); cos/sin rounded to fp32.
__device__ __forceinline__ double rope_inv_freq(double base, int c, int rope_dim) {
    return pow(base, -2.0 * (double)c / (double)rope_dim);
}
// cos/sin of the fp64 angle p * inv_freq.  The angle is reduced modulo 2*pi
// first (Cody-Waite, two-part constant) so sincos only ever sees |r| <= pi:
// large angles (position 1e5 at theta_0 = 1) otherwise take the slow
// wide-argument path.
__device__ __forceinline__ double2 rope_sincos64(int p, double inv_freq) {
    const double two_pi_hi = 6.283185307179586232e+00;
    const double two_pi_lo = 2.449293598294706414e-16;
    const double inv_two_pi = 1.591549430918953358e-01;
    const double phi = (double)p * inv_freq;
    const double kq = rint(phi * inv_two_pi);
    double red = fma(-kq, two_pi_hi, phi);
    red = fma(-kq, two_pi_lo, red);
    double sn, cn;
    sincos(red, &sn, &cn);
    return make_double2(cn, sn);
}
// A position is split as p = hi + lo with hi = 32*floor(p/32), lo = p mod 32; the
// two rotations compose in fp64 and the result is rounded once to fp32.  Every
// kernel (the standalone RoPE and the fused prefill, which tabulates the lo part
// once and the hi part once per 32 tokens) evaluates exactly this expression, so
// their results agree bit for bit.
__device__ __forceinline__ float2 rope_compose(double2 hi, double2 lo) {
    const double c = __fma_rn(hi.x, lo.x, -__dmul_rn(hi.y, lo.y));
    const double s = __fma_rn(hi.y, lo.x, __dmul_rn(hi.x, lo.y));
    return make_float2((float)c, (float)s);
}
__device__ __forceinline__ float2 rope_cos_sin(int pos, double inv_freq) {
    return rope_compose(rope_sincos64(pos & ~31, inv_freq), rope_sincos64(pos & 31, inv_freq));
}
// Rotate the pair (x0, x1) by the angle whose (cos, sin) is cs, in fp32, with an
// explicit operation order so every kernel rounds identically.
__device__ __forceinline__ void rope_pair(float x0, float x1, float2 cs, float &y0, float &y1) {
    y0 = __fmaf_rn(x0, cs.x, -__fmul_rn(x1, cs.y));
    y1 = __fmaf_rn(x0, cs.y, __fmul_rn(x1, cs.x));
}
// (cos, sin) of the 32 pairs of a 64-dim rotation for positions pos0 .. pos0+n-1,
// tab[t * 32 + c], filled cooperatively by the workgroup (the caller syncs).
__device__ __forceinline__ void rope_fill_table64(float2 *tab, int pos0, int n, double base,
                                                  int tid, int nthreads) {
    for (int i = tid; i < n * 32; i += nthreads)
        tab[i] = rope_cos_sin(pos0 + (i >> 5), rope_inv_freq(base, i & 31, 64));
}
// The same table from a frequency the thread computed beforehand, inv_freq =
// rope_inv_freq(base, tid % 32, 64) (nthreads a multiple of 32, so every entry the
// thread fills has pair tid % 32): the fp64 pow can then run before the position
// is known.
__device__ __forceinline__ void rope_fill_table64_inv(float2 *tab, int pos0, int n, double inv_freq,
                                                      int tid, int nthreads) {
    for (int i = tid; i < n * 32; i += nthreads)
        tab[i] = rope_cos_sin(pos0 + (i >> 5), inv_freq);
}
// Rotate the 4 interleaved pairs held in 8 bf16 (one 16-byte chunk); cs[p] is the
// (cos, sin) of pair p of the chunk.
__device__ __forceinline__ uint4 rope_chunk_bf16(uint4 x, const float2 *cs) {
    uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float x0 = bf16_bits_to_f32((uint16_t)(w[p] & 0xffffu));
        const float x1 = bf16_bits_to_f32((uint16_t)(w[p] >> 16));
        float y0, y1;
        rope_pair(x0, x1, cs[p], y0, y1);
        w[p] = pack_bf16x2(y0, y1);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// ---- FP8 (OCP E4M3) cache codes ----
// Two E4M3 codes (bytes 0,1, or 2,3 with kHi, of w) to two bf16, exactly (every E4M3 value
// is a bf16 value; the gfx950 conversion follows the OCP definition, scale 1).
template <bool kHi>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi);
    return __builtin_bit_cast(uint32_t, r);
}
// 8 codes (one uint2) -> 8 bf16 (one uint4), element order kept.
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint2 c) {
    return make_uint4(e4m3x2_to_bf16x2<false>(c.x), e4m3x2_to_bf16x2<true>(c.x),
                      e4m3x2_to_bf16x2<false>(c.y), e4m3x2_to_bf16x2<true>(c.y));
}
// Nearest E4M3 code of a finite fp32 value, ties to the even code, magnitudes
// past 448 saturate (never the NaN code).  Integer rounding of the fp32 fields.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
    const uint32_t bits = __builtin_bit_cast(uint32_t, v);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const float a = __builtin_fabsf(v);
    uint32_t code;
    if (!(a < 448.0f)) {
        code = 0x7Eu;
    } else if (a < 0x1p-6f) {  // E4M3 subnormals: multiples of 2^-9 (8 -> code 0x08)
        code = (uint32_t)__builtin_rintf(a * 512.0f);
    } else {
        const uint32_t ab = bits & 0x7fffffffu;
        int e = (int)(ab >> 23) - 127;           // -6 .. 8
        const uint32_t m = ab & 0x7fffffu;
        uint32_t q = (m + 0x7ffffu + ((m >> 20) & 1u)) >> 20;  // RNE to 3 bits
        if (q == 8u) {
            q = 0u;
            ++e;
        }
        code = ((uint32_t)(e + 7) << 3) | q;
        code = code > 0x7Eu ? 0x7Eu : code;
    }
    return code | sign;
}
// 8 bf16 (one uint4) -> 8 codes of (x / scale), the quotient rounded once to fp32.
__device__ __forceinline__ uint2 bf16x8_to_e4m3x8(uint4 x, float scale) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint16_t h = (uint16_t)((w[i >> 1] >> ((i & 1) * 16)) & 0xffffu);
        const uint32_t c = f32_to_e4m3(__fdiv_rn(bf16_bits_to_f32(h), scale));
        out[i >> 2] |= c << ((i & 3) * 8);
    }
    return make_uint2(out[0], out[1]);
}

// New-token side effects of a decode / verify launch, done by one workgroup per
// (sequence, KV head): decode stores token 0 into the cache at position P (its
// k rotated when kRope); with kRope a k_rot output receives every new token's
// rotated k.  tab holds the (cos, sin) of positions P .. P+nq-1 when kRope.  Nothing in
// the launch reads the rows written here.
// store_cache = false leaves the cache store to the caller (which holds the rows).
template <bool kRope, bool kFp8 = false>
__device__ __forceinline__ void cached_store_new(const CachedArgs &a, size_t crow0, size_t nrow0,
                                                 int P, const float2 *tab, int tid,
                                                 int nthreads, bool store_cache = true) {
    const uint16_t *ks = (const uint16_t *)a.k_new;
    if (store_cache && a.write_new && (a.ring || P < a.cap)) {
        const int slot = a.ring ? (P % a.cap) : P;
        const uint16_t *vs = (const uint16_t *)a.v_new + nrow0 * kDv;
        for (int i = tid; i < (kDqk + kDv) / 8; i += nthreads) {
            const bool is_k = i < kDqk / 8;
            const int ci = is_k ? i : i - kDqk / 8;
            uint4 x = is_k ? *(const uint4 *)(ks + nrow0 * kDqk + ci * 8)
                           : *(const uint4 *)(vs + ci * 8);
            if (kRope && is_k && ci < 8)
                x = rope_chunk_bf16(x, tab + 4 * ci);
            const size_t row = (crow0 + slot) * (is_k ? kDqk : kDv) + ci * 8;
            if constexpr (kFp8) {
                uint8_t *dst = (uint8_t *)(is_k ? a.k_cache : a.v_cache) + row;
                *(uint2 *)dst = bf16x8_to_e4m3x8(x, is_k ? a.k_scale : a.v_scale);
            } else {
                uint16_t *dst = (uint16_t *)(is_k ? a.k_cache : a.v_cache) + row;
                *(uint4 *)dst = x;
            }
        }
    }
    if (kRope && a.k_rot) {
        for (int i = tid; i < a.nq * (kDqk / 8); i += nthreads) {
            const int t = i / (kDqk / 8), ci = i % (kDqk / 8);
            const size_t row = nrow0 + (size_t)t * a.Hkv;
            uint4 x = *(const uint4 *)(ks + row * kDqk + ci * 8);
            if (ci < 8)
                x = rope_chunk_bf16(x, tab + t * 32 + 4 * ci);
            *(uint4 *)((uint16_t *)a.k_rot + row * kDqk + ci * 8) = x;
        }
    }
}

}  // namespace sinkattn

// backward.hip -- gradients of causal sink attention (gfx950, bf16 in, fp32 out).
//
// For the forward of prefill.hip / prefill_swa.hip (MiMo-V2-Flash Technical
// Report, Section 2.2: s_ij = e^(a_ij) / (e^(sink) + sum_j' e^(a_ij')),
// o_i = sum_j s_ij v_j, a_ij = scale q_i . k_j) and an upstream gradient dO,
// the chain rule gives, with the forward's log-normaliser lse_i = ln Z_i
// (so s_ij = e^(a_ij - lse_i) and the sink's share p_i = e^(sink - lse_i)):
//   D_i    = dO_i . o_i
//   dP_ij  = dO_i . v_j,      dS_ij = s_ij (dP_ij - D_i)
//   dq_i   = scale sum_j dS_ij k_j
//   dk_j   = scale sum_i dS_ij q_i,   dv_j = sum_i s_ij dO_i   (summed over the
//            query heads that share the KV head)
//   dsink_h = - sum_i p_i D_i          (the sink is a softmax column with no value)
// The sink's learnable logit gets its gradient here; it is absent from the
// flash-attention backward it otherwise follows.
//
// Kernels:
//   bwd_dq_kernel    per (KV group, head half, 32-query tile), 8 waves = 8 heads:
//                    first D_i = dO_i . o_i and -p_i D_i of the tile's rows (o is
//                    read here, beside dO, instead of in a pass of its own), then
//                    dQ in the forward's layout -- S^T = K Q^T with each lane owning a
//                    query column, K rows permuted so C-register i of half hh is
//                    key 16hh + i; dP^T = V dO^T with V rows permuted the same
//                    way; dQ^T += K^T dS^T with the K^T operand read from the
//                    same K rows by gfx950's transposing LDS loads.  The tile's
//                    Q / dO rows come in and its fp32 dQ rows go out in whole
//                    128-byte lines per instruction, regrouped through LDS.
//   bwd_dsink_kernel dsink_h = fixed-order sum over tokens (deterministic)
//   bwd_dkdv_kernel  (windowed layers) per (KV group, 64-key block), 4 waves of 16 keys each, every
//                    query head of the group: 16x16x32 products, S = Q K^T with
//                    each lane owning a key column and Q rows permuted so the C
//                    registers of a lane hold 8 consecutive queries, so P and dS
//                    are directly the B operands of dV^T += dO^T P and
//                    dK^T += Q^T dS; the step's Q and dO tile is shared by the
//                    4 waves, put into LDS two steps ahead by global->LDS loads
//                    in MFMA operand order (the Q^T / dO^T operands come from
//                    the same pieces through transposing reads); dK / dV rows
//                    leave in whole 128-byte lines, regrouped through LDS.
//   bwd_dkdv32_kernel (global layers) the same with 32x32x16 products: per (KV
//                    group, 128-key block), 4 waves of 32 keys each, one wave per
//                    SIMD; every LDS operand read feeds twice the pairs.
// Whole-line stores matter here: the fp32 gradient rows are the largest stream
// of the SWA backward, and stores that cover a quarter of a line per instruction
// ran the dQ kernel ~25% slower (0.99 vs 0.75 ms at T 32768, W 128).
// Every output element is written once (no atomics): results are deterministic.
#include "common.h"
#include "lds_tr.h"

namespace sinkattn {
namespace {

constexpr int kKb = 32;   // keys per block
constexpr int kTq = 32;   // queries per tile
constexpr uint32_t kOob = 0x80000000u;

// ------------------------------------------------------------------ D, dsink

// sum over the 8 bf16 pairs of two 16-byte chunks, in element order (fma chain)
__device__ __forceinline__ float dot8_bf16(const uint4 &x, const uint4 &y) {
    const uint32_t xw[4] = {x.x, x.y, x.z, x.w}, yw[4] = {y.x, y.y, y.z, y.w};
    float d = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        d = __fmaf_rn(bf16_bits_to_f32((uint16_t)(xw[i >> 1] >> (16 * (i & 1)))),
                      bf16_bits_to_f32((uint16_t)(yw[i >> 1] >> (16 * (i & 1)))), d);
    return d;
}

// dsink_h = -sum over (b, t) of e^(sink_h - lse) D: one workgroup per head, fixed
// order (D from the workspace the dQ kernel filled).
constexpr int kSinkThreads = 1024;
__global__ __launch_bounds__(kSinkThreads) void bwd_dsink_kernel(BwdArgs a) {
    __shared__ float red[kSinkThreads];
    const int h = blockIdx.x;
    const float sink = a.sink[h];
    float s = 0.f;
    if (sink != -INFINITY) {
        for (int b = 0; b < a.B; ++b) {
            const size_t row = ((size_t)b * a.Hq + h) * a.T;
            for (int t = threadIdx.x; t < a.T; t += kSinkThreads)
                s += -__expf(sink - a.lse[row + t]) * a.D[row + t];
        }
    }
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = kSinkThreads / 2; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w)
            red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0)
        a.dsink[h] = red[0];
}

// ------------------------------------------------------------------ dQ

constexpr int kQWaves = 8;
constexpr int kQThreads = kQWaves * 64;
constexpr int kKPitch = kDqk + 8;   // K rows in LDS (bf16)
constexpr int kVPitch = kDv + 8;    // V rows in LDS (bf16)
constexpr int kKChunks = kKb * kDqk / 8;  // 768 16-byte pieces of a K block

struct DqSmem {
    uint16_t k[2][kKb * kKPitch];
    uint16_t v[2][kKb * kVPitch];
};

struct DqStaged {
    uint4 k[2];
    uint4 v;
};

template <bool kWindowed>
__global__ __launch_bounds__(kQThreads) void bwd_dq_kernel(BwdArgs a, int n_units, int n_tiles,
                                                           float scale_log2) {
    __shared__ DqSmem sm;
    __shared__ float xch[kQWaves][kTq * 36];  // per-wave row exchange: 32 rows x (128 + 16) bytes
    const int T = a.T, Hq = a.Hq, Hkv = a.Hkv, window = a.window;
    const int group = Hq / Hkv, parts = group / kQWaves;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 31, hh = lane >> 5;
    const int unit = blockIdx.x % n_units;
    const int tix = blockIdx.x / n_units;
    const int tile = kWindowed ? tix : (n_tiles - 1 - tix);  // longest first (global)
    const int part = unit % parts;
    const int g = (unit / parts) % Hkv;
    const int b = unit / (parts * Hkv);
    const int h = g * group + part * kQWaves + wave;
    const int t0 = tile * kTq;
    const int query = t0 + r;

    const size_t row0 = (size_t)b * T;
    const uint32_t qrow = (uint32_t)Hq * kDqk * 2, orow = (uint32_t)Hq * kDv * 2;
    const uint32_t krow = (uint32_t)Hkv * kDqk * 2, vrow = (uint32_t)Hkv * kDv * 2;
    const BufRsrc qbuf = make_buf((const uint16_t *)a.q + row0 * Hq * kDqk, (uint64_t)T * qrow);
    const BufRsrc gbuf = make_buf((const uint16_t *)a.dout + row0 * Hq * kDv, (uint64_t)T * orow);
    const BufRsrc obuf = make_buf((const uint16_t *)a.o + row0 * Hq * kDv, (uint64_t)T * orow);
    const BufRsrc kbuf = make_buf((const uint16_t *)a.k + row0 * Hkv * kDqk, (uint64_t)T * krow);
    const BufRsrc vbuf = make_buf((const uint16_t *)a.v + row0 * Hkv * kDv, (uint64_t)T * vrow);
    const uint32_t kcol = (uint32_t)g * kDqk * 2, vcol = (uint32_t)g * kDv * 2;

    // B operands held for the whole tile: Q^T (k-step s: dims (2s+hh)*8 ..) and dO^T.
    // The rows are fetched in whole 128-byte lines (8 lanes x 16 bytes of one row per
    // line; rows 8i + lane/8 in instruction i) and regrouped into the operand layout
    // through a per-wave LDS area, one line column (32 rows x 128 bytes) at a time.
    uint4 qf[kDqk / 16], gf[kDv / 16];
    {
        const int lr8 = lane >> 3, c8 = lane & 7;
        uint4 rq[kDqk / 16], rg[kDv / 16], ro[kDv / 16];
#pragma unroll
        for (int li = 0; li < kDqk / 64; ++li)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                rq[4 * li + i] = buf_load16(qbuf, (uint32_t)(t0 + 8 * i + lr8) * qrow + (uint32_t)h * kDqk * 2 +
                                                      128 * li + 16 * c8);
#pragma unroll
        for (int li = 0; li < kDv / 64; ++li)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                rg[4 * li + i] = buf_load16(gbuf, (uint32_t)(t0 + 8 * i + lr8) * orow + (uint32_t)h * kDv * 2 +
                                                      128 * li + 16 * c8);
#pragma unroll
        for (int li = 0; li < kDv / 64; ++li)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ro[4 * li + i] = buf_load16(obuf, (uint32_t)(t0 + 8 * i + lr8) * orow + (uint32_t)h * kDv * 2 +
                                                      128 * li + 16 * c8);
        uint4 *xs = (uint4 *)xch[wave];  // row pitch 9 pieces (128 + 16 bytes)
        auto regroup = [&](const uint4 *raw, uint4 *dst) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xs[(8 * i + lr8) * 9 + c8] = raw[i];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
                dst[s4] = xs[r * 9 + 2 * s4 + hh];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        };
#pragma unroll
        for (int li = 0; li < kDqk / 64; ++li)
            regroup(rq + 4 * li, qf + 4 * li);
#pragma unroll
        for (int li = 0; li < kDv / 64; ++li)
            regroup(rg + 4 * li, gf + 4 * li);
        // D of rows 8i + lane/8: 8-dim partial dot products, the two line columns
        // added, then summed over the row's 8 lanes
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float d = dot8_bf16(ro[i], rg[i]) + dot8_bf16(ro[4 + i], rg[4 + i]);
#pragma unroll
            for (int m = 4; m >= 1; m >>= 1)
                d += __shfl_xor(d, m, 64);
            if (c8 == 0)
                xch[wave][8 * i + lr8] = d;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    const bool qok = query < T;
    const size_t lidx = ((size_t)b * Hq + h) * T + (qok ? query : 0);
    const float lse = qok ? a.lse[lidx] : 0.f;
    const float lse2 = lse * kLog2e;
    const float Dq = qok ? xch[wave][r] : 0.f;
    if (qok && hh == 0) {  // D and lse in log2 units for the dK/dV kernels
        a.D[lidx] = Dq;
        a.L2[lidx] = lse2;
    }

    const int kstart = kWindowed ? max(0, t0 - window + 1) : 0;
    const int kend = min(T, t0 + kTq);
    const int kb0 = kstart & ~(kKb - 1);
    const int nblk = (kend - kb0 + kKb - 1) / kKb;

    // staging: K pieces c = tid, tid + 512 (key c/24, dims (c%24)*8 ..); V piece tid
    const bool k2 = tid + kQThreads < kKChunks;  // wave-uniform
    auto load_block = [&](int kb, DqStaged &st) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = min(tid + u * kQThreads, kKChunks - 1);
            if (u == 0 || k2)
                st.k[u] = buf_load16(kbuf, (uint32_t)(kb + c / 24) * krow + kcol +
                                               (uint32_t)(c % 24) * 16);
        }
        st.v = buf_load16(vbuf, (uint32_t)(kb + tid / 16) * vrow + vcol + (uint32_t)(tid % 16) * 16);
    };
    auto store_block = [&](int buf, const DqStaged &st) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (u == 1 && !k2)
                continue;
            const int c = tid + u * kQThreads;
            const int key = c / 24, d0 = (c % 24) * 8;
            *(uint4 *)&sm.k[buf][row_of_key(key) * kKPitch + d0] = st.k[u];
        }
        *(uint4 *)&sm.v[buf][row_of_key(tid / 16) * kVPitch + (tid % 16) * 8] = st.v;
    };

    f32x16 acc[kDqk / 32];
#pragma unroll
    for (int db = 0; db < kDqk / 32; ++db)
        acc[db] = f32x16{};

    // K^T operand of dQ^T += K^T dS^T through transposing reads of the K rows: in
    // lane group G = lane/16, source lane 4e'+q points at key 16hh + 8t + 4L + e'
    // (row row_of_key of the staged tile) and dims 32d + 16(G%2) + 4q .. +3, so
    // A-row r holds dim 32d + r and element 4L + e' holds key 16hh + 8t + 4L + e'.
    int kt_off[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int L = 0; L < 2; ++L)
            kt_off[t][L] = row_of_key(16 * hh + 8 * t + 4 * L + ((lane & 15) >> 2)) * kKPitch +
                           16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    DqStaged st;
    load_block(kb0, st);
    store_block(0, st);
    if (nblk > 1)
        load_block(kb0 + kKb, st);
    __syncthreads();

    for (int j = 0; j < nblk; ++j) {
        const int kb = kb0 + j * kKb;
        const uint16_t *ks = sm.k[j & 1], *vs = sm.v[j & 1];
        f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int s = 0; s < kDqk / 16; ++s) {
            const bf16x8 ka = as_bf16x8(*(const uint4 *)(ks + r * kKPitch + (2 * s + hh) * 8));
            sc = mfma32x32x16(ka, as_bf16x8(qf[s]), sc);
        }
#pragma unroll
        for (int s = 0; s < kDv / 16; ++s) {
            const bf16x8 va = as_bf16x8(*(const uint4 *)(vs + r * kVPitch + (2 * s + hh) * 8));
            dp = mfma32x32x16(va, as_bf16x8(gf[s]), dp);
        }
        // register i holds key kb + 16hh + i of query column `query`.  Only blocks on
        // the diagonal or the window edge need the mask (a uniform test); masked
        // scores become -inf, so P = 0 there without a branch per element.  Query
        // columns past the end need none: their q and dO rows, lse and D are zero,
        // so their dS is zero.
        const bool full = (kb + kKb - 1 <= t0) && (!kWindowed || t0 + kTq - 1 - kb < window);
        if (!full) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = kb + 16 * hh + i;
                sc[i] = (key <= query && (!kWindowed || query - key < window)) ? sc[i] : -INFINITY;
            }
        }
        bf16x8 db_[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p = fast_exp2(__fmaf_rn(sc[i], scale_log2, -lse2));
            db_[i >> 3][i & 7] = (__bf16)(p * (dp[i] - Dq));
        }
        // dQ^T += K^T dS^T: A = K^T rows (dims), keys 16hh + 8t .. +7 of step t
#pragma unroll
        for (int d = 0; d < kDqk / 32; ++d)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const uint2 lo = lds_tr16(ks + kt_off[t][0] + 32 * d);
                const uint2 hi = lds_tr16(ks + kt_off[t][1] + 32 * d);
                acc[d] = mfma32x32x16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), db_[t], acc[d]);
            }
        if (j + 1 < nblk)
            store_block((j + 1) & 1, st);
        __syncthreads();
        if (j + 2 < nblk)
            load_block(kb + 2 * kKb, st);
    }

    // dq[query][h][dim] = scale * acc (C row (i/4)*8 + 4hh + i%4 of tile d = dim
    // 32d + 8(i/4) + 4hh + i%4).  The rows leave through LDS so that every store
    // instruction writes whole 128-byte lines: 8 lanes x 16 bytes of one
    // (query, head) row's 32 dims of tile d.
    {
        float *stage = xch[wave];  // 32 rows x (32 + 4) floats
        const int nq = min(kTq, T - t0);
        const BufRsrc dqbuf = make_buf(a.dq + ((row0 + t0) * Hq) * kDqk, (uint64_t)nq * Hq * kDqk * 4);
#pragma unroll
        for (int d = 0; d < kDqk / 32; ++d) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                *(float4 *)(stage + r * 36 + 8 * q4 + 4 * hh) =
                    make_float4(acc[d][4 * q4] * a.scale, acc[d][4 * q4 + 1] * a.scale,
                                acc[d][4 * q4 + 2] * a.scale, acc[d][4 * q4 + 3] * a.scale);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int row = 8 * it + (lane >> 3), c = lane & 7;
                const uint4 w = *(const uint4 *)(stage + row * 36 + 4 * c);
                buf_store16(dqbuf, (uint32_t)(row * Hq + h) * (kDqk * 4) + 128 * d + 16 * c, w);
            }
        }
    }
}

// ------------------------------------------------------------------ dK, dV

typedef float f32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4v mfma16x16x32(const bf16x8 &a, const bf16x8 &b, const f32x4v &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

constexpr int kKWaves = 4;
constexpr int kKThreads = kKWaves * 64;
constexpr int kKPerWave = 16;                     // keys per wave (16x16x32 tiles)
constexpr int kKBlk = kKWaves * kKPerWave;        // keys per workgroup
constexpr int kQPieces = 2 * (kDqk / 32);         // 12 pieces of 1 KB: Q tile
constexpr int kGPieces = 2 * (kDv / 32);          // 8: dO tile
constexpr int kTilePieces = kQPieces + kGPieces;  // 20
constexpr int kStepBytes = kTilePieces * 1024;
constexpr int kStepLoads = kTilePieces / kKWaves + 2;  // global->LDS loads per thread per step
static_assert(kQPieces % kKWaves == 0 && kGPieces % kKWaves == 0, "uniform piece split");

// One global->LDS load per wave: lane l's 16 (4) bytes at r + off land at
// lds + 16 l (4 l).
__device__ __forceinline__ void lds_load16(BufRsrc r, uint8_t *lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16,
                                             off, 0, 0, 0);
}
__device__ __forceinline__ void lds_load4(BufRsrc r, uint8_t *lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 4,
                                             off, 0, 0, 0);
}
// Wait until at most N vector memory operations of this thread are outstanding
// (kLds: and none of its LDS operations).
template <int N, bool kLds = false>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | ((kLds ? 0 : 0xF) << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wg_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// dK, dV of one 64-key block of KV group g.  Wave w owns keys kb + 16w .. +15 and
// keeps their dK^T / dV^T (80 accumulators per lane) over every query head of
// the group and every 32-query tile that sees the block; the four waves share
// each step's Q and dO tile, which global->LDS loads (no registers held) put
// into a ring of three LDS slots two steps ahead, so a wave fits in ~200
// registers and two waves share a SIMD.  Lane l: lr = l % 16, lg = l / 16.
//   Tile layout: 1 KB pieces in 16x16x32 A-operand order -- Q piece 6mt + s,
//   lane l holds query pq(mt, l%16) = 8((l%16)/4) + 4mt + (l%16)%4 of the tile,
//   dims 32s + 8(l/16) .. +7 (dO likewise, 4 pieces per half) -- so the A
//   operands of S = Q K^T and dP = dO V^T are conflict-free 16-byte reads and
//   their C registers hold queries 8lg .. 8lg+7 (register i of half mt: query
//   8lg + 4mt + i) of key lr: exactly the B operand (k = queries) of
//   dV^T += dO^T P and dK^T += Q^T dS.  The dO^T / Q^T operands (row = dim, k =
//   queries 8lg ..) are read from the same pieces by gfx950's transposing loads
//   (each 16-lane group touches 512 contiguous bytes: no bank conflicts).
//   K and V of the wave's 16 keys stay in registers as the B operands.
// Every thread issues exactly 7 global->LDS loads per step (5 tile pieces; its
// wave's own copy of the tile's lse and D), so "at most 7 outstanding" before a
// step's barrier means its part of that step has landed.  The slots are separate LDS arrays named statically
// in a loop unrolled by three (the compiler's wait counts can then tell them
// apart), and steps past the last load past-the-end offsets (zeros, no memory
// access).
template <bool kWindowed>
__global__ __launch_bounds__(kKThreads, 2) void bwd_dkdv_kernel(BwdArgs a, int n_units, int n_blk,
                                                                float scale_log2) {
    __shared__ __attribute__((aligned(1024))) uint8_t st0[kStepBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t st1[kStepBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t st2[kStepBytes];
    // per slot, the tile's lse (floats 0..31) and D (64..95), one copy per wave
    __shared__ __attribute__((aligned(16))) float ls0[kKWaves][128];
    __shared__ __attribute__((aligned(16))) float ls1[kKWaves][128];
    __shared__ __attribute__((aligned(16))) float ls2[kKWaves][128];
    const int T = a.T, Hq = a.Hq, Hkv = a.Hkv, window = a.window;
    const int group = Hq / Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int unit = blockIdx.x % n_units;
    const int blk = blockIdx.x / n_units;  // ascending: key block 0 sees the most queries
    const int g = unit % Hkv, b = unit / Hkv;
    const int kb = blk * kKBlk;
    const int kw = kb + kKPerWave * wave;  // this wave's first key
    const int key = kw + lr;               // this lane's key column
    if (kb >= T)
        return;  // uniform

    // queries that can see some key of the block: [kb, last]
    const int last = kWindowed ? min(T - 1, kb + kKBlk - 1 + window - 1) : T - 1;
    const int n_tiles = (last - kb) / kTq + 1;
    const int n_steps = group * n_tiles;  // step = (head of the group, query tile)

    const size_t row0 = (size_t)b * T;
    const uint32_t qrow = (uint32_t)Hq * kDqk * 2, orow = (uint32_t)Hq * kDv * 2;
    const uint32_t krow = (uint32_t)Hkv * kDqk * 2, vrow = (uint32_t)Hkv * kDv * 2;
    const BufRsrc qbuf = make_buf((const uint16_t *)a.q + row0 * Hq * kDqk, (uint64_t)T * qrow);
    const BufRsrc gbuf = make_buf((const uint16_t *)a.dout + row0 * Hq * kDv, (uint64_t)T * orow);
    const BufRsrc lbuf = make_buf(a.L2 + (size_t)b * Hq * T, (uint64_t)Hq * T * 4);
    const BufRsrc dbuf = make_buf(a.D + (size_t)b * Hq * T, (uint64_t)Hq * T * 4);

    // B operands: K (k-step s: dims 32s + 8lg .. +7 of key lr) and V, for the whole kernel
    uint4 kr[kDqk / 32], vr[kDv / 32];
    {
        const BufRsrc kbuf = make_buf((const uint16_t *)a.k + row0 * Hkv * kDqk, (uint64_t)T * krow);
        const BufRsrc vbuf = make_buf((const uint16_t *)a.v + row0 * Hkv * kDv, (uint64_t)T * vrow);
        const uint32_t ko = key < T ? (uint32_t)key * krow + (uint32_t)g * kDqk * 2 + (uint32_t)lg * 16 : kOob;
        const uint32_t vo = key < T ? (uint32_t)key * vrow + (uint32_t)g * kDv * 2 + (uint32_t)lg * 16 : kOob;
#pragma unroll
        for (int s = 0; s < kDqk / 32; ++s)
            kr[s] = buf_load16(kbuf, ko + (uint32_t)s * 64);
#pragma unroll
        for (int s = 0; s < kDv / 32; ++s)
            vr[s] = buf_load16(vbuf, vo + (uint32_t)s * 64);
    }

    // Step k -> (query head, first query of the tile).  Windowed layers: heads
    // outer, tiles ascending (a neighbouring block reads the same tile two steps
    // later, while it is still in L2).  Global layers: tiles descending from the
    // last one, heads inner: every block of the group walks the same (head,
    // tile) sequence from the top and only stops at a different place, so the
    // workgroups resident at one time read the same tile at about the same time
    // (one fetch from memory, L2 hits for the rest).
    auto step_head = [&](int k) {
        return g * group + (kWindowed ? k / n_tiles : k % group);
    };
    auto step_q0 = [&](int k) {
        return kb + (kWindowed ? k % n_tiles : n_tiles - 1 - k / group) * kTq;
    };
    // This thread's 7 loads of step k into a slot (offsets with bit 31 set read
    // nothing; every real offset is below 2^31).
    const int pq_lane = 8 * (lr >> 2) + (lr & 3);  // + 4mt: query of A row lr
    auto load_step = [&](uint8_t *slot, int k) {
        const uint32_t step_oob = k < n_steps ? 0u : kOob;
        const int kk = k < n_steps ? k : 0;
        const int h = step_head(kk);
        const int q0 = step_q0(kk);
#pragma unroll
        for (int u = 0; u < kQPieces / kKWaves; ++u) {
            const int pc = wave + kKWaves * u;
            const int mt = pc / 6, s = pc % 6;
            const int q = q0 + pq_lane + 4 * mt;
            const uint32_t off = ((uint32_t)q * qrow + (uint32_t)h * kDqk * 2 + (uint32_t)(32 * s + 8 * lg) * 2) |
                                 step_oob | (q < T ? 0u : kOob);
            lds_load16(qbuf, slot + pc * 1024, off);
        }
#pragma unroll
        for (int u = 0; u < kGPieces / kKWaves; ++u) {
            const int pc = wave + kKWaves * u;
            const int mt = pc / 4, s = pc % 4;
            const int q = q0 + pq_lane + 4 * mt;
            const uint32_t off = ((uint32_t)q * orow + (uint32_t)h * kDv * 2 + (uint32_t)(32 * s + 8 * lg) * 2) |
                                 step_oob | (q < T ? 0u : kOob);
            lds_load16(gbuf, slot + (kQPieces + pc) * 1024, off);
        }
    };
    // the tile's lse and D of step k into this wave's copy in a slot
    auto load_ld = [&](float (*ls)[128], int k) {
        const uint32_t step_oob = k < n_steps ? 0u : kOob;
        const int kk = k < n_steps ? k : 0;
        const int h = step_head(kk);
        const int q = step_q0(kk) + lane;  // lanes 0..31: the tile's queries
        const uint32_t off = ((uint32_t)h * T + (uint32_t)q) * 4 | step_oob |
                             (lane < kTq && q < T ? 0u : kOob);
        lds_load4(lbuf, (uint8_t *)ls[wave], off);
        lds_load4(dbuf, (uint8_t *)&ls[wave][64], off);
    };

    f32x4v dk[kDqk / 16], dv[kDv / 16];  // C tiles: rows dims 16dt + 4lg + i, column key lr
#pragma unroll
    for (int d = 0; d < kDqk / 16; ++d)
        dk[d] = f32x4v{};
#pragma unroll
    for (int d = 0; d < kDv / 16; ++d)
        dv[d] = f32x4v{};

    // transposing-read source of this lane inside a half's pieces: tile row
    // (query) 8lg + lr/4 (+4 in half 1), dims 16dt + 4(lr%4) .. +3
    const int tr_off = 16 * (4 * lg + (lr >> 2) + 16 * ((lr & 3) >> 1)) + 8 * (lr & 1);

    auto compute = [&](const uint8_t *slot, const float (*ls)[128], int k) {
        const int q0 = step_q0(k);
        // does any (query, key) pair of the tile and this wave's keys count?
        const bool act = q0 + kTq - 1 >= kw && (!kWindowed || q0 <= kw + kKPerWave - 1 + window - 1);
        if (!act)
            return;  // wave-uniform
        const uint8_t *qs = slot, *gs = slot + kQPieces * 1024;
        f32x4v sc[2] = {f32x4v{}, f32x4v{}}, dp[2] = {f32x4v{}, f32x4v{}};
#pragma unroll
        for (int s = 0; s < kDqk / 32; ++s)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                sc[mt] = mfma16x16x32(as_bf16x8(*(const uint4 *)(qs + (6 * mt + s) * 1024 + lane * 16)),
                                      as_bf16x8(kr[s]), sc[mt]);
#pragma unroll
        for (int s = 0; s < kDv / 32; ++s)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                dp[mt] = mfma16x16x32(as_bf16x8(*(const uint4 *)(gs + (4 * mt + s) * 1024 + lane * 16)),
                                      as_bf16x8(vr[s]), dp[mt]);
        // P and dS of this lane's 8 queries (element j = query q0 + 8lg + j)
        const float *ld = ls[wave];
        const float4 l0 = *(const float4 *)(ld + 8 * lg), l1 = *(const float4 *)(ld + 8 * lg + 4);
        const float4 d0 = *(const float4 *)(ld + 64 + 8 * lg), d1 = *(const float4 *)(ld + 64 + 8 * lg + 4);
        const float lw[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        const float dw[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
        bf16x8 pb, sb;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int q = q0 + 8 * lg + j;
            const bool vis = q < T && key <= q && (!kWindowed || q - key < window);
            const float sv = sc[j >> 2][j & 3], dpv = dp[j >> 2][j & 3];
            const float p = vis ? fast_exp2(__fmaf_rn(sv, scale_log2, -lw[j])) : 0.f;
            pb[j] = (__bf16)p;
            sb[j] = (__bf16)(p * (dpv - dw[j]));
        }
        // dV^T += dO^T P (tile dt: dims 16dt ..; k-step = the tile's 32 queries)
#pragma unroll
        for (int dt = 0; dt < kDv / 16; ++dt) {
            const uint8_t *src = gs + (dt >> 1) * 1024 + (dt & 1) * 512 + tr_off;
            const uint2 x0 = lds_tr16((const uint16_t *)src);
            const uint2 x1 = lds_tr16((const uint16_t *)(src + 4 * 1024));
            dv[dt] = mfma16x16x32(as_bf16x8(make_uint4(x0.x, x0.y, x1.x, x1.y)), pb, dv[dt]);
        }
        // dK^T += Q^T dS
#pragma unroll
        for (int dt = 0; dt < kDqk / 16; ++dt) {
            const uint8_t *src = qs + (dt >> 1) * 1024 + (dt & 1) * 512 + tr_off;
            const uint2 x0 = lds_tr16((const uint16_t *)src);
            const uint2 x1 = lds_tr16((const uint16_t *)(src + 6 * 1024));
            dk[dt] = mfma16x16x32(as_bf16x8(make_uint4(x0.x, x0.y, x1.x, x1.y)), sb, dk[dt]);
        }
    };

    // Step k: wait for this thread's loads of step k (step k+1's seven may still
    // be in flight), barrier (every thread's part of step k is in, and every
    // wave is done with step k-1, whose slot receives step k+2), compute.
    load_step(st0, 0);
    load_ld(ls0, 0);
    load_step(st1, 1);
    load_ld(ls1, 1);
    auto step = [&](int k, const uint8_t *cur, const float (*lcur)[128], uint8_t *next2,
                    float (*lnext2)[128]) {
        wait_vmem<kStepLoads>();
        wg_barrier();
        load_step(next2, k + 2);
        load_ld(lnext2, k + 2);
        if (k < n_steps)
            compute(cur, lcur, k);
    };
    for (int k = 0; k < n_steps; k += 3) {
        step(k, st0, ls0, st2, ls2);
        step(k + 1, st1, ls1, st0, ls0);
        step(k + 2, st2, ls2, st1, ls1);
    }
    wait_vmem<0>();  // no load into LDS outlives the workgroup
    wg_barrier();    // every wave is done with the slots: st0 is reused below

    // dK / dV rows leave through LDS, one 32-dim column (128 bytes of each key's row)
    // at a time, so that every store instruction writes whole 128-byte lines
    // (8 lanes x 16 bytes of one key's row; keys kw + 8it + lane/8).
    {
        uint8_t *xs = st0 + wave * (kKPerWave * 144);  // 16 rows x (128 + 16) bytes
        const int nk = max(0, min(kKPerWave, T - kw));
        const BufRsrc dkbuf = make_buf(a.dk + ((row0 + kw) * Hkv) * kDqk, (uint64_t)nk * Hkv * kDqk * 4);
        const BufRsrc dvbuf = make_buf(a.dv + ((row0 + kw) * Hkv) * kDv, (uint64_t)nk * Hkv * kDv * 4);
        const int lr8 = lane >> 3, c8 = lane & 7;
        auto emit = [&](const f32x4v &x0, const f32x4v &x1, const BufRsrc &dst, uint32_t rowbytes, int c) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            *(f32x4v *)(xs + lr * 144 + 16 * lg) = x0;
            *(f32x4v *)(xs + lr * 144 + 64 + 16 * lg) = x1;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int row = 8 * it + lr8;
                const uint4 w = *(const uint4 *)(xs + row * 144 + 16 * c8);
                buf_store16(dst, (uint32_t)(row * Hkv + g) * rowbytes + 128 * c + 16 * c8, w);
            }
        };
#pragma unroll
        for (int c = 0; c < kDqk / 32; ++c)
            emit(dk[2 * c] * a.scale, dk[2 * c + 1] * a.scale, dkbuf, kDqk * 4, c);
#pragma unroll
        for (int c = 0; c < kDv / 32; ++c)
            emit(dv[2 * c], dv[2 * c + 1], dvbuf, kDv * 4, c);
    }
}

// ------------------------------------------------------------------ dK, dV (global layers)

// dK, dV of one 128-key block of KV group g for global (unwindowed) layers, with
// 32x32x16 products.  Wave w owns keys kb + 32w .. +31 and keeps their dK^T / dV^T
// (160 accumulators per lane) over every (query head, 32-query tile) step at or
// after the block; one wave per SIMD.  Against the 16-key kernel above, every
// operand read from LDS feeds twice the pairs (32 keys), and the 32x32x16 product
// issues ~20% more FLOP per cycle than 16x16x32 (2.33 vs 1.94 PFLOP/s in a
// throughput probe on MI355X): at 16x16x32 with one LDS operand per product the
// products would need ~120 TB/s of LDS reads against the ~107 TB/s that
// conflict-free 16-byte reads deliver.  Lane l: col = l % 32 (key), hh = l / 32.
//   Tile layout: the step's Q rows and dO rows in query order with row pitches of
//   400 and 304 bytes (100 and 76 dwords: 36 and 12 modulo the 64 banks), so the
//   16-byte operand reads of S = Q K^T and dP = dO V^T (16 consecutive rows per
//   bank pass) and the transposing reads of the Q^T / dO^T operands (4 rows x 16
//   dims per 16 lanes) are free of bank conflicts, and every operand address is
//   one per-lane base plus an immediate offset (XOR-swizzled rows instead made
//   the compiler's wait counts lose track of which slot a read touches).  S and
//   dP come out with C rows 8a + 4hh + e = query
//   q0 + 8a + 4hh + e of key col; their elements 8ks .. 8ks+7 are directly the B
//   operand (k = queries 16ks + 8t + 4hh + e, element 4t + e) of k-step ks of
//   dV^T += dO^T P and dK^T += Q^T dS, whose A operands the transposing reads
//   take in the same query order.
//   K and V of the wave's 32 keys stay in registers as the B operands of S and dP.
// The global->LDS loads of a step (six 1 KB pieces per thread, plus the tile's
// lse and D), the three slots and the barrier follow the 16-key kernel.
constexpr int kK32Waves = 4;
constexpr int kK32Threads = kK32Waves * 64;
constexpr int kK32PerWave = 32;
constexpr int kK32Blk = kK32Waves * kK32PerWave;  // 128 keys per workgroup
constexpr int kK32QPitch = kDqk * 2 + 16;  // 400 bytes: 24 data chunks + 1 pad
constexpr int kK32GPitch = kDv * 2 + 48;   // 304 bytes: 16 data chunks + 3 pad
constexpr int kK32QPieces = (kTq * kK32QPitch + 1023) / 1024;  // 13 pieces of 1 KB
constexpr int kK32GPieces = (kTq * kK32GPitch + 1023) / 1024;  // 10
constexpr int kK32Pieces = 24;  // 13 + 10 + 1 that loads nothing: 6 per thread
constexpr int kK32StepBytes = kK32Pieces * 1024;
constexpr int kK32QBytes = kK32QPieces * 1024;
constexpr int kK32StepLoads = kK32Pieces / kK32Waves + 2;  // 8
static_assert(kK32QPieces + kK32GPieces < kK32Pieces && kK32Pieces % kK32Waves == 0, "uniform pieces");

__global__ __launch_bounds__(kK32Threads, 1) void bwd_dkdv32_kernel(BwdArgs a, int n_units, int n_blk,
                                                                   float scale_log2) {
    __shared__ __attribute__((aligned(1024))) uint8_t st0[kK32StepBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t st1[kK32StepBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t st2[kK32StepBytes];
    __shared__ __attribute__((aligned(16))) float ls0[kK32Waves][128];
    __shared__ __attribute__((aligned(16))) float ls1[kK32Waves][128];
    __shared__ __attribute__((aligned(16))) float ls2[kK32Waves][128];
    const int T = a.T, Hq = a.Hq, Hkv = a.Hkv;
    const int group = Hq / Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, hh = lane >> 5;
    const int unit = blockIdx.x % n_units;
    const int blk = blockIdx.x / n_units;  // ascending: key block 0 sees the most queries
    const int g = unit % Hkv, b = unit / Hkv;
    const int kb = blk * kK32Blk;
    const int kw = kb + kK32PerWave * wave;  // this wave's first key
    const int key = kw + col;                // this lane's key column
    if (kb >= T)
        return;  // uniform

    const int n_tiles = (T - 1 - kb) / kTq + 1;  // queries kb .. T-1
    const int n_steps = group * n_tiles;         // step = (head of the group, query tile)

    const size_t row0 = (size_t)b * T;
    const uint32_t qrow = (uint32_t)Hq * kDqk * 2, orow = (uint32_t)Hq * kDv * 2;
    const uint32_t krow = (uint32_t)Hkv * kDqk * 2, vrow = (uint32_t)Hkv * kDv * 2;
    const BufRsrc qbuf = make_buf((const uint16_t *)a.q + row0 * Hq * kDqk, (uint64_t)T * qrow);
    const BufRsrc gbuf = make_buf((const uint16_t *)a.dout + row0 * Hq * kDv, (uint64_t)T * orow);
    const BufRsrc lbuf = make_buf(a.L2 + (size_t)b * Hq * T, (uint64_t)Hq * T * 4);
    const BufRsrc dbuf = make_buf(a.D + (size_t)b * Hq * T, (uint64_t)Hq * T * 4);

    // B operands: K (k-step s: dims 16s + 8hh .. +7 of key col) and V
    uint4 kr[kDqk / 16], vr[kDv / 16];
    {
        const BufRsrc kbuf = make_buf((const uint16_t *)a.k + row0 * Hkv * kDqk, (uint64_t)T * krow);
        const BufRsrc vbuf = make_buf((const uint16_t *)a.v + row0 * Hkv * kDv, (uint64_t)T * vrow);
        const uint32_t ko = key < T ? (uint32_t)key * krow + (uint32_t)g * kDqk * 2 + (uint32_t)hh * 16 : kOob;
        const uint32_t vo = key < T ? (uint32_t)key * vrow + (uint32_t)g * kDv * 2 + (uint32_t)hh * 16 : kOob;
#pragma unroll
        for (int s = 0; s < kDqk / 16; ++s)
            kr[s] = buf_load16(kbuf, ko + (uint32_t)s * 32);
#pragma unroll
        for (int s = 0; s < kDv / 16; ++s)
            vr[s] = buf_load16(vbuf, vo + (uint32_t)s * 32);
    }

    // Step k -> (query head, first query of the tile): tiles descending from the last
    // one, heads inner (every block of the group walks the same sequence from the top).
    auto step_head = [&](int k) { return g * group + k % group; };
    auto step_q0 = [&](int k) { return kb + (n_tiles - 1 - k / group) * kTq; };
    // This thread's 7 loads of step k into a slot: pieces wave + 4u (u < 5) of the
    // 20 KB tile (pieces 0..11 Q rows, 12..19 dO rows), then lse and D.  Offsets with
    // bit 31 set read nothing; every real offset is below 2^31.
    // Piece pc = wave + 4u of a slot: 16-byte chunk 64 pc' + lane of the padded Q rows
    // (pc' = pc < 13) or dO rows (pc' = pc - 13 < 10); chunks in the padding, past row
    // 31 or in the last piece read nothing.  Per thread: row r_u, byte column cb_u.
    int ld_row[kK32Pieces / kK32Waves];
    uint32_t ld_col[kK32Pieces / kK32Waves];
#pragma unroll
    for (int u = 0; u < kK32Pieces / kK32Waves; ++u) {
        const int pc = wave + kK32Waves * u;
        if (pc < kK32QPieces) {
            const int ci = 64 * pc + lane, r = ci / (kK32QPitch / 16), c = ci % (kK32QPitch / 16);
            const bool ok = r < kTq && c < kDqk / 8;
            ld_row[u] = ok ? r : 0;
            ld_col[u] = ok ? (uint32_t)c * 16 : kOob;
        } else if (pc < kK32QPieces + kK32GPieces) {
            const int ci = 64 * (pc - kK32QPieces) + lane, r = ci / (kK32GPitch / 16), c = ci % (kK32GPitch / 16);
            const bool ok = r < kTq && c < kDv / 8;
            ld_row[u] = ok ? r : 0;
            ld_col[u] = ok ? (uint32_t)c * 16 : kOob;
        } else {
            ld_row[u] = 0;
            ld_col[u] = kOob;
        }
    }
    auto load_step = [&](uint8_t *slot, int k) {
        const uint32_t step_oob = k < n_steps ? 0u : kOob;
        const int kk = k < n_steps ? k : 0;
        const int h = step_head(kk);
        const int q0 = step_q0(kk);
#pragma unroll
        for (int u = 0; u < kK32Pieces / kK32Waves; ++u) {
            const int pc = wave + kK32Waves * u;
            const int q = q0 + ld_row[u];
            const uint32_t oob = step_oob | (q < T ? 0u : kOob);
            // pc < 13: Q rows; else dO rows (the last piece reads nothing either way)
            const bool isq = pc < kK32QPieces;  // wave-uniform
            const uint32_t off = isq ? (uint32_t)q * qrow + (uint32_t)h * kDqk * 2
                                     : (uint32_t)q * orow + (uint32_t)h * kDv * 2;
            lds_load16(isq ? qbuf : gbuf, slot + pc * 1024, (off + ld_col[u]) | oob);
        }
    };
    auto load_ld = [&](float (*ls)[128], int k) {
        const uint32_t step_oob = k < n_steps ? 0u : kOob;
        const int kk = k < n_steps ? k : 0;
        const int h = step_head(kk);
        const int q = step_q0(kk) + lane;  // lanes 0..31: the tile's queries
        const uint32_t off = ((uint32_t)h * T + (uint32_t)q) * 4 | step_oob |
                             (lane < kTq && q < T ? 0u : kOob);
        lds_load4(lbuf, (uint8_t *)ls[wave], off);
        lds_load4(dbuf, (uint8_t *)&ls[wave][64], off);
    };

    f32x16 dk[kDqk / 32], dv[kDv / 32];  // C tiles: rows dims 32dt + 8a + 4hh + e, column key col
#pragma unroll
    for (int d = 0; d < kDqk / 32; ++d)
        dk[d] = f32x16{};
#pragma unroll
    for (int d = 0; d < kDv / 32; ++d)
        dv[d] = f32x16{};

    // Transposing-read sources of this lane (lane i = 4e + m of its 16-lane group G):
    // query row 16ks + 8t + 4hh + e, dims 32dt + 16(G%2) + 4m .. +3.
    const int tr_row = 4 * hh + ((lane & 15) >> 2), tr_dim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int q_tr_base = tr_row * kK32QPitch + 2 * tr_dim, g_tr_base = tr_row * kK32GPitch + 2 * tr_dim;
    const int q_rd_base = col * kK32QPitch + 16 * hh, g_rd_base = col * kK32GPitch + 16 * hh;
    auto q_tr = [&](const uint8_t *qs, int dt, int ks, int t) {
        return lds_tr16((const uint16_t *)(qs + q_tr_base + (16 * ks + 8 * t) * kK32QPitch + 64 * dt));
    };
    auto g_tr = [&](const uint8_t *gs, int dt, int ks, int t) {
        return lds_tr16((const uint16_t *)(gs + g_tr_base + (16 * ks + 8 * t) * kK32GPitch + 64 * dt));
    };

    auto compute = [&](const uint8_t *slot, const float (*ls)[128], int k) {
        const int q0 = step_q0(k);
        if (q0 + kTq - 1 < kw)
            return;  // wave-uniform: every query of the tile precedes this wave's keys
        const uint8_t *qs = slot, *gs = slot + kK32QBytes;
        // A operands of S and dP: row = query col, k-step s: dims 16s + 8hh .. +7
        uint4 qa[kDqk / 16], ga[kDv / 16];
#pragma unroll
        for (int s = 0; s < kDqk / 16; ++s) {
            qa[s] = *(const uint4 *)(qs + q_rd_base + 32 * s);
            if (s < kDv / 16)
                ga[s] = *(const uint4 *)(gs + g_rd_base + 32 * s);
        }
        f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int s = 0; s < kDqk / 16; ++s) {
            sc = mfma32x32x16(as_bf16x8(qa[s]), as_bf16x8(kr[s]), sc);
            if (s < kDv / 16)
                dp = mfma32x32x16(as_bf16x8(ga[s]), as_bf16x8(vr[s]), dp);
        }
        // P and dS: C register i = 4a + e holds query q0 + 8a + 4hh + e
        const float *ld = ls[wave];
        float lw[16], dw[16];
#pragma unroll
        for (int aa = 0; aa < 4; ++aa) {
            const float4 l4 = *(const float4 *)(ld + 8 * aa + 4 * hh);
            const float4 d4 = *(const float4 *)(ld + 64 + 8 * aa + 4 * hh);
            lw[4 * aa] = l4.x; lw[4 * aa + 1] = l4.y; lw[4 * aa + 2] = l4.z; lw[4 * aa + 3] = l4.w;
            dw[4 * aa] = d4.x; dw[4 * aa + 1] = d4.y; dw[4 * aa + 2] = d4.z; dw[4 * aa + 3] = d4.w;
        }
        // only tiles on the diagonal or past the end need the mask (uniform test)
        if (!(q0 >= kw + kK32PerWave - 1 && q0 + kTq - 1 < T)) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int q = q0 + 8 * (i >> 2) + 4 * hh + (i & 3);
                sc[i] = (q < T && key <= q) ? sc[i] : -INFINITY;
            }
        }
        bf16x8 pb[2], sb[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p = fast_exp2(__fmaf_rn(sc[i], scale_log2, -lw[i]));
            pb[i >> 3][i & 7] = (__bf16)p;
            sb[i >> 3][i & 7] = (__bf16)(p * (dp[i] - dw[i]));
        }
        // dV^T += dO^T P, dK^T += Q^T dS: k-step ks = queries 16ks .. 16ks+15
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int dt = 0; dt < kDv / 32; ++dt) {
                const uint2 x0 = g_tr(gs, dt, ks, 0), x1 = g_tr(gs, dt, ks, 1);
                dv[dt] = mfma32x32x16(as_bf16x8(make_uint4(x0.x, x0.y, x1.x, x1.y)), pb[ks], dv[dt]);
            }
#pragma unroll
            for (int dt = 0; dt < kDqk / 32; ++dt) {
                const uint2 x0 = q_tr(qs, dt, ks, 0), x1 = q_tr(qs, dt, ks, 1);
                dk[dt] = mfma32x32x16(as_bf16x8(make_uint4(x0.x, x0.y, x1.x, x1.y)), sb[ks], dk[dt]);
            }
        }
    };

    load_step(st0, 0);
    load_ld(ls0, 0);
    load_step(st1, 1);
    load_ld(ls1, 1);
    auto step = [&](int k, const uint8_t *cur, const float (*lcur)[128], uint8_t *next2,
                    float (*lnext2)[128]) {
        wait_vmem<kK32StepLoads>();
        wg_barrier();
        load_step(next2, k + 2);
        load_ld(lnext2, k + 2);
        if (k < n_steps)
            compute(cur, lcur, k);
    };
    for (int k = 0; k < n_steps; k += 3) {
        step(k, st0, ls0, st2, ls2);
        step(k + 1, st1, ls1, st0, ls0);
        step(k + 2, st2, ls2, st1, ls1);
    }
    wait_vmem<0>();  // no load into LDS outlives the workgroup
    wg_barrier();    // every wave is done with the slots: st0 is reused below

    // dK / dV rows leave through LDS, one 32-dim tile (128 bytes of each key's row) at
    // a time: every store instruction writes whole 128-byte lines (keys kw + 8it + lane/8).
    {
        uint8_t *xs = st0 + wave * (kK32PerWave * 144);  // 32 rows x (128 + 16) bytes
        const int nk = max(0, min(kK32PerWave, T - kw));
        const BufRsrc dkbuf = make_buf(a.dk + ((row0 + kw) * Hkv) * kDqk, (uint64_t)nk * Hkv * kDqk * 4);
        const BufRsrc dvbuf = make_buf(a.dv + ((row0 + kw) * Hkv) * kDv, (uint64_t)nk * Hkv * kDv * 4);
        const int lr8 = lane >> 3, c8 = lane & 7;
        auto emit = [&](const f32x16 &x, float mul, const BufRsrc &dst, uint32_t rowbytes, int dt) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int aa = 0; aa < 4; ++aa)
                *(float4 *)(xs + col * 144 + 32 * aa + 16 * hh) =
                    make_float4(x[4 * aa] * mul, x[4 * aa + 1] * mul, x[4 * aa + 2] * mul, x[4 * aa + 3] * mul);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int row = 8 * it + lr8;
                const uint4 w = *(const uint4 *)(xs + row * 144 + 16 * c8);
                buf_store16(dst, (uint32_t)(row * Hkv + g) * rowbytes + 128 * dt + 16 * c8, w);
            }
        };
#pragma unroll
        for (int dt = 0; dt < kDqk / 32; ++dt)
            emit(dk[dt], a.scale, dkbuf, kDqk * 4, dt);
#pragma unroll
        for (int dt = 0; dt < kDv / 32; ++dt)
            emit(dv[dt], 1.f, dvbuf, kDv * 4, dt);
    }
}

}  // namespace

hipError_t launch_backward(const BwdArgs &a, hipStream_t s) {
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    hipError_t e;
    const int group = a.Hq / a.Hkv;
    const int parts = group / kQWaves;
    const int q_units = a.B * a.Hkv * parts;
    const int n_tiles = (a.T + kTq - 1) / kTq;
    const dim3 qgrid((unsigned)(q_units * n_tiles));
    if (a.window > 0)
        bwd_dq_kernel<true><<<qgrid, dim3(kQThreads), 0, s>>>(a, q_units, n_tiles, scale_log2);
    else
        bwd_dq_kernel<false><<<qgrid, dim3(kQThreads), 0, s>>>(a, q_units, n_tiles, scale_log2);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    bwd_dsink_kernel<<<dim3((unsigned)a.Hq), dim3(kSinkThreads), 0, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    const int k_units = a.B * a.Hkv;
    if (a.window > 0) {
        const int n_blk = (a.T + kKBlk - 1) / kKBlk;
        bwd_dkdv_kernel<true><<<dim3((unsigned)(k_units * n_blk)), dim3(kKThreads), 0, s>>>(
            a, k_units, n_blk, scale_log2);
    } else {
        const int n_blk = (a.T + kK32Blk - 1) / kK32Blk;
        bwd_dkdv32_kernel<<<dim3((unsigned)(k_units * n_blk)), dim3(kK32Threads), 0, s>>>(
            a, k_units, n_blk, scale_log2);
    }
    return hipGetLastError();
}

}  // namespace sinkattn

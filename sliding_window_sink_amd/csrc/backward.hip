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
//   bwd_pre_kernel   D and -p_i D_i per (token, head)  (one 16-lane group per row)
//   bwd_dsink_kernel dsink_h = fixed-order sum over tokens (deterministic)
//   bwd_dq_kernel    per (KV group, head half, 32-query tile), 8 waves = 8 heads:
//                    the forward's layout -- S^T = K Q^T with each lane owning a
//                    query column, K rows permuted so C-register i of half hh is
//                    key 16hh + i; dP^T = V dO^T with V rows permuted the same
//                    way; dQ^T += K^T dS^T with the K^T operand read from the
//                    same K rows by gfx950's transposing LDS loads.
//   bwd_dkdv_kernel  per (KV group, 32-key block), 4 waves: S = Q K^T with each
//                    lane owning a key column and Q rows permuted so C-register i
//                    of half hh is query 16hh + i, so P and dS are directly the
//                    B operands of dV^T += dO^T P and dK^T += Q^T dS; Q and dO
//                    rows go to a per-wave row-major LDS tile whose transposing
//                    reads give the Q^T / dO^T operands; the 4 waves (disjoint
//                    heads) are summed through LDS in a fixed order at the end.
// Every output element is written once (no atomics): results are deterministic.
#include "common.h"
#include "lds_tr.h"

namespace sinkattn {
namespace {

constexpr int kKb = 32;   // keys per block
constexpr int kTq = 32;   // queries per tile
constexpr uint32_t kOob = 0x80000000u;

// ------------------------------------------------------------------ preprocess

__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 4, li = lane & 15;
    const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + grp;  // (b*T+t)*Hq + h
    const int64_t n_rows = (int64_t)a.B * a.T * a.Hq;
    float d = 0.f;
    if (row < n_rows) {
        const uint4 o = *(const uint4 *)((const uint16_t *)a.o + row * kDv + li * 8);
        const uint4 g = *(const uint4 *)((const uint16_t *)a.dout + row * kDv + li * 8);
        const uint32_t ow[4] = {o.x, o.y, o.z, o.w}, gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x = bf16_bits_to_f32((uint16_t)(ow[i >> 1] >> (16 * (i & 1))));
            const float y = bf16_bits_to_f32((uint16_t)(gw[i >> 1] >> (16 * (i & 1))));
            d = __fmaf_rn(x, y, d);
        }
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1)
        d += __shfl_xor(d, o, 64);
    if (row < n_rows && li == 0) {
        const int h = (int)(row % a.Hq);
        const int64_t bt = row / a.Hq;
        const int t = (int)(bt % a.T), b = (int)(bt / a.T);
        const size_t idx = ((size_t)b * a.Hq + h) * a.T + t;
        a.D[idx] = d;
        const float lse = a.lse[idx], sink = a.sink[h];
        const float ps = (sink == -INFINITY) ? 0.f : __expf(sink - lse);
        a.PS[idx] = -ps * d;
    }
}

// dsink_h = sum over (b, t) of PS[b][h][t]: one workgroup per head, fixed order.
constexpr int kSinkThreads = 1024;
__global__ __launch_bounds__(kSinkThreads) void bwd_dsink_kernel(BwdArgs a) {
    __shared__ float red[kSinkThreads];
    const int h = blockIdx.x;
    float s = 0.f;
    for (int b = 0; b < a.B; ++b) {
        const float *p = a.PS + ((size_t)b * a.Hq + h) * a.T;
        for (int t = threadIdx.x; t < a.T; t += kSinkThreads)
            s += p[t];
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
    const BufRsrc kbuf = make_buf((const uint16_t *)a.k + row0 * Hkv * kDqk, (uint64_t)T * krow);
    const BufRsrc vbuf = make_buf((const uint16_t *)a.v + row0 * Hkv * kDv, (uint64_t)T * vrow);
    const uint32_t kcol = (uint32_t)g * kDqk * 2, vcol = (uint32_t)g * kDv * 2;

    // B operands held for the whole tile: Q^T (k-step s: dims (2s+hh)*8 ..) and dO^T.
    uint4 qf[kDqk / 16], gf[kDv / 16];
    {
        const uint32_t qo = (uint32_t)query * qrow + (uint32_t)h * kDqk * 2 + (uint32_t)hh * 16;
        const uint32_t go = (uint32_t)query * orow + (uint32_t)h * kDv * 2 + (uint32_t)hh * 16;
#pragma unroll
        for (int s = 0; s < kDqk / 16; ++s)
            qf[s] = buf_load16(qbuf, qo + (uint32_t)s * 32);
#pragma unroll
        for (int s = 0; s < kDv / 16; ++s)
            gf[s] = buf_load16(gbuf, go + (uint32_t)s * 32);
    }
    const bool qok = query < T;
    const size_t lidx = ((size_t)b * Hq + h) * T + (qok ? query : 0);
    const float lse2 = qok ? a.lse[lidx] * kLog2e : 0.f;
    const float Dq = qok ? a.D[lidx] : 0.f;

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
        // register i holds key kb + 16hh + i of query column `query`
        bf16x8 db_[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = kb + 16 * hh + i;
            const bool vis = qok && key <= query && (!kWindowed || query - key < window);
            const float p = vis ? fast_exp2(__fmaf_rn(sc[i], scale_log2, -lse2)) : 0.f;
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

    // dq[query][h][dim] = scale * acc; C row (i/4)*8 + 4hh + i%4 of tile d = dim 32d + ...
    if (qok) {
        float *dst = a.dq + ((row0 + query) * Hq + h) * kDqk;
#pragma unroll
        for (int d = 0; d < kDqk / 32; ++d)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int dim = 32 * d + 8 * q4 + 4 * hh;
                *(float4 *)(dst + dim) =
                    make_float4(acc[d][4 * q4] * a.scale, acc[d][4 * q4 + 1] * a.scale,
                                acc[d][4 * q4 + 2] * a.scale, acc[d][4 * q4 + 3] * a.scale);
            }
    }
}

// ------------------------------------------------------------------ dK, dV

constexpr int kKWaves = 4;
constexpr int kKThreads = kKWaves * 64;
constexpr int kQRPitch = kDqk + 8;  // per-wave Q rows (bf16): 400 bytes
constexpr int kGRPitch = kDv + 8;   // per-wave dO rows (bf16): 272 bytes
constexpr int kRedPitch = kKb + 1;  // fp32 reduction rows

struct DkvSmem {
    union {
        struct {
            uint16_t qr[kKWaves][kTq * kQRPitch];
            uint16_t gr[kKWaves][kTq * kGRPitch];
        } w;
        float red[2][(kDqk + kDv) * kRedPitch];
    };
};

template <bool kWindowed>
__global__ __launch_bounds__(kKThreads) void bwd_dkdv_kernel(BwdArgs a, int n_units, int n_blk,
                                                             float scale_log2) {
    __shared__ DkvSmem sm;
    const int T = a.T, Hq = a.Hq, Hkv = a.Hkv, window = a.window;
    const int group = Hq / Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 31, hh = lane >> 5;
    const int unit = blockIdx.x % n_units;
    const int blk = blockIdx.x / n_units;  // ascending: key block 0 sees the most queries
    const int g = unit % Hkv, b = unit / Hkv;
    const int kb = blk * kKb;
    const int key = kb + r;  // this lane's key column

    const size_t row0 = (size_t)b * T;
    const uint32_t qrow = (uint32_t)Hq * kDqk * 2, orow = (uint32_t)Hq * kDv * 2;
    const uint32_t krow = (uint32_t)Hkv * kDqk * 2, vrow = (uint32_t)Hkv * kDv * 2;
    const BufRsrc qbuf = make_buf((const uint16_t *)a.q + row0 * Hq * kDqk, (uint64_t)T * qrow);
    const BufRsrc gbuf = make_buf((const uint16_t *)a.dout + row0 * Hq * kDv, (uint64_t)T * orow);
    const BufRsrc kbuf = make_buf((const uint16_t *)a.k + row0 * Hkv * kDqk, (uint64_t)T * krow);
    const BufRsrc vbuf = make_buf((const uint16_t *)a.v + row0 * Hkv * kDv, (uint64_t)T * vrow);

    // B operands for the whole block: K^T and V^T columns = this lane's key.
    uint4 kf[kDqk / 16], vf[kDv / 16];
    {
        const uint32_t ko = (uint32_t)key * krow + (uint32_t)g * kDqk * 2 + (uint32_t)hh * 16;
        const uint32_t vo = (uint32_t)key * vrow + (uint32_t)g * kDv * 2 + (uint32_t)hh * 16;
#pragma unroll
        for (int s = 0; s < kDqk / 16; ++s)
            kf[s] = buf_load16(kbuf, ko + (uint32_t)s * 32);
#pragma unroll
        for (int s = 0; s < kDv / 16; ++s)
            vf[s] = buf_load16(vbuf, vo + (uint32_t)s * 32);
    }

    f32x16 dk[kDqk / 32], dv[kDv / 32];
#pragma unroll
    for (int d = 0; d < kDqk / 32; ++d)
        dk[d] = f32x16{};
#pragma unroll
    for (int d = 0; d < kDv / 32; ++d)
        dv[d] = f32x16{};

    // queries that can see some key of the block: [kb, last]
    const int last = kWindowed ? min(T - 1, kb + kKb - 1 + window - 1) : T - 1;
    const int n_tiles = kb < T ? (last - kb) / kTq + 1 : 0;
    const int qrow_r = key_of_row(r);  // A-row r of a tile holds query q0 + key_of_row(r)
    uint16_t *qt = sm.w.qr[wave], *gt = sm.w.gr[wave];
    // Q^T / dO^T operands through transposing reads of the row-major tiles: source
    // lane 4e'+q of group G points at query 16hh + 8t + 4L + e' and dims
    // 32d + 16(G%2) + 4q .. +3 (A-row r = dim 32d + r)
    int qt_off[2][2], gt_off[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int L = 0; L < 2; ++L) {
            const int qq = 16 * hh + 8 * t + 4 * L + ((lane & 15) >> 2);
            const int dd = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
            qt_off[t][L] = qq * kQRPitch + dd;
            gt_off[t][L] = qq * kGRPitch + dd;
        }

    for (int hi = wave; hi < group; hi += kKWaves) {
        const int h = g * group + hi;
        const float *lse_h = a.lse + ((size_t)b * Hq + h) * T;
        const float *D_h = a.D + ((size_t)b * Hq + h) * T;
        const BufRsrc lbuf = make_buf(lse_h, (uint64_t)T * 4);
        const BufRsrc dbuf = make_buf(D_h, (uint64_t)T * 4);
        for (int it = 0; it < n_tiles; ++it) {
            const int q0 = kb + it * kTq;
            const int qa_row = q0 + qrow_r;
            uint4 qa[kDqk / 16], ga[kDv / 16];
            {
                const uint32_t qo = qa_row < T ? (uint32_t)qa_row * qrow + (uint32_t)h * kDqk * 2 +
                                                     (uint32_t)hh * 16
                                               : kOob;
                const uint32_t go = qa_row < T ? (uint32_t)qa_row * orow + (uint32_t)h * kDv * 2 +
                                                     (uint32_t)hh * 16
                                               : kOob;
#pragma unroll
                for (int s = 0; s < kDqk / 16; ++s)
                    qa[s] = buf_load16(qbuf, qo + (uint32_t)s * 32);
#pragma unroll
                for (int s = 0; s < kDv / 16; ++s)
                    ga[s] = buf_load16(gbuf, go + (uint32_t)s * 32);
            }
            // lse and D of the 16 queries q0 + 16hh + i this lane's registers hold
            float ls[16], dd[16];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t off = (uint32_t)(q0 + 16 * hh + 4 * c) * 4;
                const uint4 l4 = buf_load16(lbuf, off), d4 = buf_load16(dbuf, off);
                ls[4 * c + 0] = __builtin_bit_cast(float, l4.x);
                ls[4 * c + 1] = __builtin_bit_cast(float, l4.y);
                ls[4 * c + 2] = __builtin_bit_cast(float, l4.z);
                ls[4 * c + 3] = __builtin_bit_cast(float, l4.w);
                dd[4 * c + 0] = __builtin_bit_cast(float, d4.x);
                dd[4 * c + 1] = __builtin_bit_cast(float, d4.y);
                dd[4 * c + 2] = __builtin_bit_cast(float, d4.z);
                dd[4 * c + 3] = __builtin_bit_cast(float, d4.w);
            }
            // Q and dO rows of the tile into this wave's LDS, queries in natural order
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int s = 0; s < kDqk / 16; ++s)
                *(uint4 *)&qt[qrow_r * kQRPitch + (2 * s + hh) * 8] = qa[s];
#pragma unroll
            for (int s = 0; s < kDv / 16; ++s)
                *(uint4 *)&gt[qrow_r * kGRPitch + (2 * s + hh) * 8] = ga[s];
            // S = Q K^T and dP = dO V^T: column = key, register i = query q0 + 16hh + i
            f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int s = 0; s < kDqk / 16; ++s)
                sc = mfma32x32x16(as_bf16x8(qa[s]), as_bf16x8(kf[s]), sc);
#pragma unroll
            for (int s = 0; s < kDv / 16; ++s)
                dp = mfma32x32x16(as_bf16x8(ga[s]), as_bf16x8(vf[s]), dp);
            bf16x8 pb[2], sb[2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int q = q0 + 16 * hh + i;
                const bool vis = q < T && key <= q && (!kWindowed || q - key < window);
                const float p = vis ? fast_exp2(__fmaf_rn(sc[i], scale_log2, -ls[i] * kLog2e)) : 0.f;
                pb[i >> 3][i & 7] = (__bf16)p;
                sb[i >> 3][i & 7] = (__bf16)(p * (dp[i] - dd[i]));
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // dV^T += dO^T P, dK^T += Q^T dS: A rows = dims, step t = queries 16hh + 8t ..
#pragma unroll
            for (int d = 0; d < kDv / 32; ++d)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const uint2 lo = lds_tr16(gt + gt_off[t][0] + 32 * d);
                    const uint2 hi = lds_tr16(gt + gt_off[t][1] + 32 * d);
                    dv[d] = mfma32x32x16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pb[t], dv[d]);
                }
#pragma unroll
            for (int d = 0; d < kDqk / 32; ++d)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const uint2 lo = lds_tr16(qt + qt_off[t][0] + 32 * d);
                    const uint2 hi = lds_tr16(qt + qt_off[t][1] + 32 * d);
                    dk[d] = mfma32x32x16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), sb[t], dk[d]);
                }
        }
    }

    // Sum the 4 waves' partials in the fixed order (w0 + w2) + (w1 + w3) through two
    // LDS regions: waves 0 and 1 store theirs, waves 2 and 3 then add theirs into
    // region wave & 1 (every read of a lane issued before its writes, so the wave
    // pays one LDS latency rather than one per element), and the row writer adds
    // the two regions.
    float *red = sm.red[wave & 1];
    auto red_at = [&](int row) -> float & { return red[row * kRedPitch + r]; };
    __syncthreads();
    if (wave < 2) {
#pragma unroll
        for (int d = 0; d < kDqk / 32; ++d)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                red_at(32 * d + c_row(i, hh)) = dk[d][i];
#pragma unroll
        for (int d = 0; d < kDv / 32; ++d)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                red_at(kDqk + 32 * d + c_row(i, hh)) = dv[d][i];
    }
    __syncthreads();
    if (wave >= 2) {
        float pk[kDqk / 32][16], pv[kDv / 32][16];
#pragma unroll
        for (int d = 0; d < kDqk / 32; ++d)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                pk[d][i] = red_at(32 * d + c_row(i, hh));
#pragma unroll
        for (int d = 0; d < kDv / 32; ++d)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                pv[d][i] = red_at(kDqk + 32 * d + c_row(i, hh));
#pragma unroll
        for (int d = 0; d < kDqk / 32; ++d)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                red_at(32 * d + c_row(i, hh)) = pk[d][i] + dk[d][i];
#pragma unroll
        for (int d = 0; d < kDv / 32; ++d)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                red_at(kDqk + 32 * d + c_row(i, hh)) = pv[d][i] + dv[d][i];
    }
    __syncthreads();
    for (int idx = tid; idx < kKb * (kDqk + kDv); idx += kKThreads) {
        const int kk = idx / (kDqk + kDv), dim = idx % (kDqk + kDv);
        if (kb + kk >= T)
            continue;
        const float x = sm.red[0][dim * kRedPitch + kk] + sm.red[1][dim * kRedPitch + kk];
        const size_t trow = (row0 + kb + kk) * Hkv + g;
        if (dim < kDqk)
            a.dk[trow * kDqk + dim] = x * a.scale;
        else
            a.dv[trow * kDv + dim - kDqk] = x;
    }
}

}  // namespace

hipError_t launch_backward(const BwdArgs &a, hipStream_t s) {
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    const int64_t n_rows = (int64_t)a.B * a.T * a.Hq;
    const unsigned pre_blocks = (unsigned)((n_rows + 15) / 16);
    bwd_pre_kernel<<<dim3(pre_blocks), dim3(256), 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    bwd_dsink_kernel<<<dim3((unsigned)a.Hq), dim3(kSinkThreads), 0, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
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
    const int k_units = a.B * a.Hkv;
    const int n_blk = (a.T + kKb - 1) / kKb;
    const dim3 kgrid((unsigned)(k_units * n_blk));
    if (a.window > 0)
        bwd_dkdv_kernel<true><<<kgrid, dim3(kKThreads), 0, s>>>(a, k_units, n_blk, scale_log2);
    else
        bwd_dkdv_kernel<false><<<kgrid, dim3(kKThreads), 0, s>>>(a, k_units, n_blk, scale_log2);
    return hipGetLastError();
}

}  // namespace sinkattn

// verify_lds.hip -- sink attention of up to 64 (token, head) columns per KV group
// over a long contiguous bf16 cache, with the K/V blocks staged in LDS by
// gfx950's global->LDS loads.
//
// The operation is that of cached.hip (MiMo-V2-Flash Technical Report, Section
// 2.2 sink softmax; Section 2.3.1: the main model checks the draft tokens in one
// pass over the per-request cache, so verifying 1 + 3 tokens should cost about
// one decode step's cache read).  With 4 tokens x 16 query heads = 64 columns
// per KV head, keeping the columns' state in registers (cached.hip's 32x32 tiles:
// 128 accumulators per lane) leaves no room for cache blocks in flight, and
// giving each 16-column wave its own stream of the cache (decode16.hip's token
// waves) reads every block four times through L2.  Here a workgroup of four
// waves -- wave w owns columns 16w .. 16w+15, with decode16.hip's 16x16x32
// operand layouts -- shares one stream of 32-key blocks that global->LDS loads
// (buffer_load ... lds) put into a ring of three LDS slots.  Those loads hold no
// registers while in flight, so two blocks stay in flight per workgroup and two
// workgroups share a compute unit (62 KB of LDS, ~150 registers each).
//
// LDS slot of one block (20 KB):
//   K, 12 KB: 1 KB pieces in MFMA operand order -- piece 6kt + s, lane l holds
//     key 16kt + l%16, dims 32s + 8(l/16) .. +7 -- so each A operand of the score
//     product is one conflict-free 16-byte read per lane;
//   V, 8 KB: row-major, 256 bytes per key, the 16-byte chunk c of key row R
//     stored at position c ^ (R % 16), so the transposing reads (ds_read_b64_tr_b16)
//     that build the V^T operands spread over the banks.
// Order inside a block: the score tile's C registers hold keys 16kt + 4(l/16) + i
// of column l%16, and the PV product's k index runs over the keys in the same
// order (its V^T operand rows are read in that order), so P^T feeds the MFMA
// straight from those registers.
// Waiting for the loads: a thread's LDS loads of a block are followed by those of
// exactly one more block before it waits, so "at most 5 loads outstanding" means
// its pieces of the block have landed; the barrier after the wait makes every
// thread's pieces visible.  Each slot is its own LDS array named statically in a
// loop unrolled by three, so the compiler can tell the slots apart and adds no
// wait of its own for loads into the other slots; slots past the last block
// receive loads of past-the-end offsets (zeros, no memory access) to keep the
// count exact.  The new tokens' keys (read from k_new / v_new, rotated when RoPE
// is fused) go through a slot as ordinary LDS stores after the cache blocks.
#include "common.h"
#include "lds_tr.h"

namespace sinkattn {
namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kKb = 32;
constexpr int kCols = 16;
constexpr int kMaxNq = 8;
constexpr int kKBytes = kKb * kDqk * 2;      // 12288
constexpr int kVBytes = kKb * kDv * 2;       // 8192
constexpr int kSlotBytes = kKBytes + kVBytes;
constexpr int kKPieces = kKBytes / 1024;     // 12 (one 1 KB load per wave each)
constexpr int kPieces = kSlotBytes / 1024;   // 20
constexpr int kLoadsPerBlock = kPieces / kWaves;  // 5 per thread
static_assert(kPieces % kWaves == 0 && kKPieces % kWaves == 0, "uniform piece split");
constexpr uint32_t kOob = 0x80000000u;  // past every descriptor: reads 0, touches nothing

__device__ __forceinline__ f32x4v mfma16x16x32(const bf16x8 &a, const bf16x8 &b, const f32x4v &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One 1 KB global->LDS load: lane l's 16 bytes at r + off land at lds + 16 l.
// kNt: the non-temporal cache policy, for the V pieces, whose load instructions
// read whole rows once (on the K pieces, 64-byte halves of 128-byte lines, it
// measured slower: the other half is then fetched again).
template <bool kNt>
__device__ __forceinline__ void lds_load16(BufRsrc r, uint8_t *lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16,
                                             off, 0, 0, kNt ? kCacheNt : 0);
}

// Wait until at most N vector memory operations of this thread are outstanding
// (s_waitcnt with the other counters left open).
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}
// Wait for this thread's LDS operations.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier that is also a compiler barrier for memory operations but
// adds no wait of its own (the waits are explicit around it).
__device__ __forceinline__ void wg_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(kThreads, 2) void verify_lds_kernel(CachedArgs a, float scale_log2) {
    __shared__ __attribute__((aligned(1024))) uint8_t kv0[kSlotBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t kv1[kSlotBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t kv2[kSlotBytes];
    __shared__ float2 rope_tab[kMaxNq * 32];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, kg = lane >> 4;
    const int split = blockIdx.x % a.n_splits;
    const int bg = blockIdx.x / a.n_splits;
    const int Hkv = a.Hkv, nq = a.nq, Hq = a.Hq;
    const int g = bg % Hkv, b = bg / Hkv;
    const int group = Hq / Hkv;
    const int n_cols = nq * group;
    const int P = clamp_len(a.cache_len[b], a.max_len);
    const int hi = P + nq;
    int rlo = 0, rhi = hi;
    if (a.n_splits > 1) {
        rlo = split * a.chunk;
        rhi = min(hi, (split + 1) * a.chunk);
    }
    if (rlo >= rhi)
        return;  // uniform: this chunk holds no visible key

    const size_t crow0 = ((size_t)b * Hkv + g) * a.cap;
    const size_t nrow0 = (size_t)b * nq * Hkv + g;  // row of new token t: nrow0 + t*Hkv
    const BufRsrc kc = make_buf((const uint16_t *)a.k_cache + crow0 * kDqk, (uint64_t)P * kDqk * 2);
    const BufRsrc vc = make_buf((const uint16_t *)a.v_cache + crow0 * kDv, (uint64_t)P * kDv * 2);

    // Q^T operand (B of the score product): column col = (token, head) = divmod(col, group),
    // k-step s: dims 32s + 8kg .. +7.
    const int col = kCols * wave + lr;
    const bool col_ok = col < n_cols;
    const int qpos = col_ok ? P + col / group : -1;
    uint4 qr[kDqk / 32];
    {
        const BufRsrc qb = make_buf((const uint16_t *)a.q + (size_t)b * nq * Hq * kDqk,
                                    (uint64_t)nq * Hq * kDqk * 2);
        const uint32_t off =
            col_ok ? (uint32_t)((col / group) * Hq + g * group + col % group) * kDqk * 2 : kOob;
#pragma unroll
        for (int s = 0; s < kDqk / 32; ++s)
            qr[s] = buf_load16(qb, off + (uint32_t)(32 * s + 8 * kg) * 2);
    }

    const int ce = min(rhi, P);  // cache keys of this chunk: [rlo, ce)
    const int n_cache_blk = ce > rlo ? (ce - rlo + kKb - 1) / kKb : 0;
    const int new_lo = max(rlo, P);

    // This thread's 5 loads of cache block j into a slot: pieces wave + 4u, the
    // first three K pieces, the last two V pieces (4 key rows each).  Blocks past
    // the last read nothing.
    auto load_block = [&](uint8_t *slot, int j) {
        const int kb = rlo + j * kKb;
        // past-the-end offsets set bit 31 (every real offset is below 2^31): kept
        // as plain bit operations so that no load sits under a branch
        const uint32_t blk_oob = j < n_cache_blk ? 0u : kOob;
#pragma unroll
        for (int u = 0; u < kKPieces / kWaves; ++u) {
            const int pc = wave + kWaves * u;
            const int kt = pc / 6, s = pc % 6;
            const int p = kb + 16 * kt + lr;
            const uint32_t off = ((uint32_t)p * (kDqk * 2) + (uint32_t)(32 * s + 8 * kg) * 2) |
                                 blk_oob | (p < ce ? 0u : kOob);
            lds_load16<false>(kc, slot + pc * 1024, off);
        }
#pragma unroll
        for (int u = 0; u < (kPieces - kKPieces) / kWaves; ++u) {
            const int pv = wave + kWaves * u;  // V piece: key rows 4pv .. 4pv+3
            const int row = 4 * pv + kg;
            const int p = kb + row;
            const int chunk = lr ^ (row & 15);
            const uint32_t off = ((uint32_t)p * (kDv * 2) + (uint32_t)chunk * 16) | blk_oob |
                                 (p < ce ? 0u : kOob);
            lds_load16<true>(vc, slot + kKBytes + pv * 1024, off);
        }
    };
    load_block(kv0, 0);
    load_block(kv1, 1);

    // RoPE (when fused): (cos, sin) of positions P .. P+nq-1 for q and the new keys.
    if (a.rope) {
        rope_fill_table64(rope_tab, P, nq, a.rope_base, tid, kThreads);
        wait_lds();
        wg_barrier();
    }
    // The chunk holding position P stores the new token (decode) / rotated keys.
    if (P >= rlo && P < rhi) {
        if (a.rope)
            cached_store_new<true, false>(a, crow0, nrow0, P, rope_tab, tid, kThreads);
        else
            cached_store_new<false, false>(a, crow0, nrow0, P, rope_tab, tid, kThreads);
    }

    bf16x8 qf[kDqk / 32];
    if (a.rope && col_ok) {  // k-steps 0, 1 hold dims < 64
        const float2 *cs = rope_tab + (col / group) * 32;
#pragma unroll
        for (int s = 0; s < 2; ++s)
            qr[s] = rope_chunk_bf16(qr[s], cs + (32 * s + 8 * kg) / 2);
    }
#pragma unroll
    for (int s = 0; s < kDqk / 32; ++s)
        qf[s] = as_bf16x8(qr[s]);

    float m = -INFINITY, l = 0.f;
    f32x4v acc[kDv / 16];  // O^T tile dt: rows (dims) 16dt + 4kg + i, column lr
#pragma unroll
    for (int dt = 0; dt < kDv / 16; ++dt)
        acc[dt] = f32x4v{};

    // transposing-read source of this lane: key row 16h + 4kg + lr/4 of the V
    // tile (h = 0, 1), dims 16dt + 4(lr%4) .. +3 -> chunk 2dt + (lr%4)/2
    const int vrow = 4 * kg + (lr >> 2);  // row for h = 0; row & 15 is the same for h = 1
    const int vhalf8 = 8 * (lr & 1);

    // Scores, softmax and PV of the block in a slot: keys kb .. kb+31, visible below
    // kend (and at most the column's position).
    auto compute = [&](const uint8_t *slot, int kb, int kend, bool full) {
        f32x4v sc[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            sc[kt] = f32x4v{};
#pragma unroll
            for (int s = 0; s < kDqk / 32; ++s) {
                const uint4 kx = *(const uint4 *)(slot + (6 * kt + s) * 1024 + lane * 16);
                sc[kt] = mfma16x16x32(as_bf16x8(kx), qf[s], sc[kt]);
            }
        }
        // element e: key kb + (e/4)*16 + 4kg + e%4, column lr
        float xs[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = sc[e >> 2][e & 3];
            if (!full) {
                const int p = kb + (e >> 2) * 16 + 4 * kg + (e & 3);
                v = (p < kend && p <= qpos) ? v : -INFINITY;
            }
            xs[e] = col_ok ? v : -INFINITY;
        }
        float bm = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            bm = fmaxf(bm, xs[e]);
        bm = max_across_rows(bm);
        bm *= scale_log2;
        const bool up = bm > m + kRescaleSlack || (m == -INFINITY && bm > -INFINITY);
        const float mn = up ? bm : m;
        const float alpha = up ? fast_exp2(m - mn) : 1.f;
        m = mn;
        const float mu = (mn == -INFINITY) ? 0.f : mn;
        float ps = 0.f;
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float pr = fast_exp2(__fmaf_rn(xs[e], scale_log2, -mu));
            ps += pr;
            pb[e] = (__bf16)pr;
        }
        l = __fmaf_rn(l, alpha, ps);
        if (__builtin_amdgcn_ballot_w64(up) != 0) {
#pragma unroll
            for (int dt = 0; dt < kDv / 16; ++dt)
                acc[dt] *= alpha;
        }
        const uint8_t *vt = slot + kKBytes;
#pragma unroll
        for (int dt = 0; dt < kDv / 16; ++dt) {
            const int pos = ((2 * dt + ((lr & 3) >> 1)) ^ (vrow & 15)) * 16 + vhalf8;
            const uint2 x0 = lds_tr16((const uint16_t *)(vt + vrow * 256 + pos));
            const uint2 x1 = lds_tr16((const uint16_t *)(vt + (vrow + 16) * 256 + pos));
            acc[dt] = mfma16x16x32(as_bf16x8(make_uint4(x0.x, x0.y, x1.x, x1.y)), pb, acc[dt]);
        }
    };

    // Step j: wait for this thread's loads of block j (block j+1's five may still
    // be in flight), barrier (every thread's pieces of block j are in, and every
    // wave is done with block j-1, whose slot receives block j+2), compute.
    // The step count is rounded up to a multiple of three so the slots stay
    // static; the extra steps compute nothing.
    auto step = [&](int j, const uint8_t *cur, uint8_t *next2) {
        wait_vmem<kLoadsPerBlock>();
        wg_barrier();
        load_block(next2, j + 2);
        if (j < n_cache_blk) {
            const int kb = rlo + j * kKb;
            compute(cur, kb, ce, kb + kKb <= ce);
        }
    };
    for (int j = 0; j < n_cache_blk; j += 3) {
        step(j, kv0, kv2);
        step(j + 1, kv1, kv0);
        step(j + 2, kv2, kv1);
    }
    wait_vmem<0>();  // no load into LDS outlives the workgroup

    // The new tokens' block (keys new_lo .. rhi-1 from k_new / v_new) through slot
    // kv0 with ordinary LDS stores, once every load has landed and every wave is
    // done with the cache blocks.
    if (rhi > new_lo) {
        wg_barrier();
        const uint16_t *kn = (const uint16_t *)a.k_new;
        const uint16_t *vn = (const uint16_t *)a.v_new;
        for (int i = tid; i < kKPieces * 64; i += kThreads) {
            const int pc = i >> 6, ln = i & 63;
            const int kt = pc / 6, s = pc % 6;
            const int p = new_lo + 16 * kt + (ln & 15);
            const int d0 = 32 * s + 8 * (ln >> 4);
            uint4 x = make_uint4(0u, 0u, 0u, 0u);
            if (p < rhi) {
                x = *(const uint4 *)(kn + (nrow0 + (size_t)(p - P) * Hkv) * kDqk + d0);
                if (a.rope && d0 < 64)
                    x = rope_chunk_bf16(x, rope_tab + (p - P) * 32 + d0 / 2);
            }
            *(uint4 *)(kv0 + pc * 1024 + ln * 16) = x;
        }
        for (int i = tid; i < (kPieces - kKPieces) * 64; i += kThreads) {
            const int pv = i >> 6, ln = i & 63;
            const int row = 4 * pv + (ln >> 4);
            const int p = new_lo + row;
            const int chunk = (ln & 15) ^ (row & 15);
            uint4 x = make_uint4(0u, 0u, 0u, 0u);
            if (p < rhi)
                x = *(const uint4 *)(vn + (nrow0 + (size_t)(p - P) * Hkv) * kDv + chunk * 8);
            *(uint4 *)(kv0 + kKBytes + pv * 1024 + ln * 16) = x;
        }
        wait_lds();
        wg_barrier();
        compute(kv0, new_lo, rhi, false);
    }

    // l is per lane group (16 lanes) -> total over the 4 groups of the column
    const float lt = sum_across_rows(l);
    if (!col_ok)
        return;
    const bool write_final = a.n_splits == 1;
    const size_t rows_total = (size_t)a.B * nq * Hq;
    const int t = col / group;
    const int h = g * group + col % group;
    const size_t row = ((size_t)b * nq + t) * Hq + h;
    float M = m, zs = 0.f;
    if (write_final) {
        const float sink2 = a.sink[h] * kLog2e;
        M = fmaxf(m, sink2);
        zs = (sink2 == -INFINITY || M == -INFINITY) ? 0.f : fast_exp2(sink2 - M);
    }
    const float f0 = (m == -INFINITY) ? 0.f : fast_exp2(m - M);
    const float z = zs + lt * f0;
    const float so = write_final ? (z > 0.f ? f0 / z : 0.f) : f0;
#pragma unroll
    for (int dt = 0; dt < kDv / 16; ++dt) {
        const int d0 = 16 * dt + 4 * kg;
        if (write_final) {
            uint2 u;
            u.x = pack_bf16x2(acc[dt][0] * so, acc[dt][1] * so);
            u.y = pack_bf16x2(acc[dt][2] * so, acc[dt][3] * so);
            *(uint2 *)((uint16_t *)a.o + row * kDv + d0) = u;
        } else {
            float *dst = &a.ws[2 * rows_total * a.n_splits + (row * a.n_splits + split) * kDv + d0];
            *(float4 *)dst = make_float4(acc[dt][0] * so, acc[dt][1] * so, acc[dt][2] * so,
                                         acc[dt][3] * so);
        }
    }
    if (!write_final && kg == 0) {
        const size_t slot = row * a.n_splits + split;
        a.ws[slot] = M;
        a.ws[rows_total * a.n_splits + slot] = (M == -INFINITY) ? 0.f : z;
    }
}

}  // namespace

hipError_t launch_verify_lds(const CachedArgs &a, hipStream_t s) {
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    const dim3 grid((unsigned)(a.B * a.Hkv * a.n_splits)), block(kThreads);
    verify_lds_kernel<<<grid, block, 0, s>>>(a, scale_log2);
    return hipGetLastError();
}

}  // namespace sinkattn

// decode16.hip -- decode sink attention with 16-column MFMA tiles (gfx950, bf16).
//
// Same operation as cached.hip (MiMo-V2-Flash Technical Report, Section 2.2
// sink softmax; Section 2.3.1 one new token per step over a per-request
// cache), for the case where the (token, head) columns of one KV group number
// at most 16: a decode step of a global layer (16 query heads per KV head,
// Table 1) or of an SWA layer (8), or a 2-token verify of an SWA layer.  A
// second mode ("token waves") serves up to 64 columns over a short window
// (verify of 1 + 3 tokens on an SWA layer): each wave takes 16 columns and
// reads the whole key range, which for a 128-key window is only a few blocks.
//
// Why a second kernel: decode is HBM bound (16 FLOP per byte), and with only
// 16 columns the 32x32 MFMA tile of cached.hip wastes half its columns and,
// more importantly, its 64-column accumulators force one wave per SIMD.  With
// v_mfma_f32_16x16x32_bf16 the per-wave state halves (Q^T 24 registers, O^T 32)
// so two waves per SIMD fit, and the operand layouts give better HBM access:
//   - A = K (16 keys x 32 dims per MFMA): lane l owns key l%16 and reads 16
//     bytes at dims 32s + 8(l/16): four lanes cover 64 contiguous bytes;
//   - A = V^T (16 output dims x 32 keys): the output-dim order is chosen as
//     dim = 8*row + tile, so lane (row, group) loads 16 contiguous bytes (8
//     dims) of each of its 8 keys -- every load instruction reads 4 whole
//     256-byte V rows -- and an 8x8 register transpose builds the 8 operands;
//   - C = S^T (16 keys x 16 columns): lane l owns column l%16, keys 4(l/16)+i;
//     the P^T operand is taken straight from those registers.
// Everything else follows cached.hip: a workgroup of 4 waves per (sequence, KV
// group, context chunk), blocks of 32 keys taken by the waves in turn, online
// softmax without the sink per wave, an LDS merge that adds the sink (one
// chunk) or writes unnormalised partials for the split-K combine; decode stores
// the new token into the cache in the same launch (the attention reads
// positions >= P from k_new).  Chunks that hold no key return at once: the
// combine only reads the chunks that intersect the visible range.
// A one-token decode over a 128-slot ring (kSlots) reads the ring in slot order,
// one 32-slot block per wave, before the sequence length arrives; the length then
// tells each slot's position, which slots are visible, and which slot the new
// token replaces (that wave computes and stores it from registers).
#include <type_traits>

#include "common.h"

namespace sinkattn {
namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kKb = 32;
constexpr int kCols = 16;
constexpr int kMaxNq = kCols / 8;  // at least 8 query heads per KV head
constexpr int kMaxNqTok = 4 * kCols / 8;
constexpr int kMergeStride = kDv + 4;
constexpr uint32_t kOob = 0x80000000u;  // an offset past every descriptor: reads 0

__device__ __forceinline__ f32x4v mfma16x16x32(const bf16x8 &a, const bf16x8 &b, const f32x4v &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One block of 32 keys in operand layout.  bf16 rows (the cache, or the new
// tokens):
struct KV16 {
    uint4 k[2][kDqk / 32];  // key tile kt (keys 16kt + l%16), k-step s: dims kdim0(s) .. +7
    uint4 v[8];             // key (e/4)*16 + 4(l/16) + e%4, dims 8(l%16) .. +7
};
// E4M3 cache rows: K as 16-byte runs (dims 64u + 16(l/16) .. +15 serve k-steps
// 2u and 2u+1), V as 8-byte runs (dims 8(l%16) .. +7); converted to bf16 in
// registers just before the MFMAs.
struct KV8 {
    uint4 k[2][kDqk / 64];
    uint2 v[8];
};

// First head dim of k-step s for lane group kg.  Any order of the 192 dims
// works if q and k use the same one; the E4M3 layout pairs k-steps so that one
// 16-byte load of a 192-byte row feeds two of them.
template <bool kFp8>
__device__ __forceinline__ int kdim0(int s, int kg) {
    return kFp8 ? 64 * (s >> 1) + 16 * kg + 8 * (s & 1) : 32 * s + 8 * kg;
}

__device__ __forceinline__ bf16x8 k_operand(const KV16 &x, int kt, int s) {
    return as_bf16x8(x.k[kt][s]);
}
__device__ __forceinline__ bf16x8 k_operand(const KV8 &x, int kt, int s) {
    const uint4 r = x.k[kt][s >> 1];
    const uint32_t w0 = (s & 1) ? r.z : r.x, w1 = (s & 1) ? r.w : r.y;
    return as_bf16x8(make_uint4(e4m3x2_to_bf16x2<false>(w0), e4m3x2_to_bf16x2<true>(w0),
                                e4m3x2_to_bf16x2<false>(w1), e4m3x2_to_bf16x2<true>(w1)));
}
__device__ __forceinline__ uint4 v_rows(const KV16 &x, int e) { return x.v[e]; }
__device__ __forceinline__ uint4 v_rows(const KV8 &x, int e) { return e4m3x8_to_bf16x8(x.v[e]); }

template <bool kTok, bool kFp8, bool kSlots>
__global__ __launch_bounds__(kThreads, 2) void decode16_kernel(CachedArgs a, float scale_log2) {
    using KVc = typename std::conditional<kFp8, KV8, KV16>::type;  // cache block registers
    constexpr uint32_t kEs = kFp8 ? 1 : 2;  // bytes per cached element
    // kTok = false: <= 16 columns, the waves split the key blocks and merge.
    // kTok = true: <= 64 columns in n_cg groups of 16; wave w owns column group
    // w % n_cg and, when fewer than 4 groups leave waves over, takes every n_kh-th
    // key block (phase w / n_cg); the phases of a group merge like the waves of
    // the other mode (the waves stream the same rows: one HBM read, L2 hits).
    constexpr int kMerge = kWaves - 1;  // parked states at most
    __shared__ __attribute__((aligned(16))) float merge[kTok ? kMerge : kWaves][kCols][kMergeStride];
    __shared__ float2 rope_tab[(kTok ? kMaxNqTok : kMaxNq) * 32];
    __shared__ uint4 new_row[(kDqk + kDv) / 8];  // one new token's k, v rows (merged block)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, kg = lane >> 4;
    const int split = blockIdx.x % a.n_splits;
    const int bg = blockIdx.x / a.n_splits;
    const int Hkv = a.Hkv, nq = a.nq, Hq = a.Hq;
    const int g = bg % Hkv, b = bg / Hkv;
    const int group = Hq / Hkv;
    const int n_cols = nq * group;
    const size_t crow0 = ((size_t)b * Hkv + g) * a.cap;
    const size_t nrow0 = (size_t)b * nq * Hkv + g;  // row of new token t: nrow0 + t*Hkv

    // Q^T operand (B of the QK MFMA): column col = (token t, head) = divmod(col, group).
    // Issued before the cache blocks, rotated once the RoPE table is ready (requested
    // once the chunk is known to hold keys, or, in slot mode, at once).
    const int n_cg = kTok ? min(kWaves, (n_cols + kCols - 1) / kCols) : 1;  // column groups
    const int n_kh = kTok ? kWaves / n_cg : kWaves;  // key phases per column group
    const int cw = kTok ? wave % n_cg : 0, kh = kTok ? wave / n_cg : wave;
    const bool active = kh < n_kh;  // wave-uniform (3 column groups leave wave 3 idle)
    const int col = kTok ? kCols * cw + lr : lr;
    const bool col_ok = col < n_cols;
    uint4 qr[kDqk / 32];
    auto load_q = [&]() {
        const BufRsrc qb = make_buf((const uint16_t *)a.q + (size_t)b * nq * Hq * kDqk,
                                    (uint64_t)nq * Hq * kDqk * 2);
        const uint32_t off =
            col_ok ? (uint32_t)((col / group) * Hq + g * group + col % group) * kDqk * 2 : kOob;
#pragma unroll
        for (int s = 0; s < kDqk / 32; ++s)
            qr[s] = buf_load16(qb, off + (uint32_t)kdim0<kFp8>(s, kg) * 2);
    };
    if constexpr (kSlots)
        load_q();

    // A one-token decode over a ring of exactly kWaves blocks (128 slots): wave w
    // reads slots 32w .. 32w+31 in slot order, requested before the sequence
    // length is known (every slot is in bounds).  Which position a slot holds,
    // whether it is visible and which slot the new token replaces follow from the
    // length once it arrives, so the cache loads do not wait for it.
    // (kSlots: the launcher checked ring, nq == 1, cap == 128 and one split.)
    constexpr bool slot_mode = kSlots;
    static_assert(!kSlots || (!kTok && !kFp8), "slot order: one-token bf16 decode");
    KVc x;
    uint4 nk = make_uint4(0u, 0u, 0u, 0u), nv = nk;  // lane l: piece l of the new k / v row
    // Slot mode reads the length through a vector load issued ahead of the cache
    // blocks (a scalar load would be waited for together with the kernel's other
    // scalar loads), so the fp64 RoPE frequency below runs while it is on its way.
    uint32_t len_v = 0;
    if constexpr (kSlots) {
        len_v = __builtin_amdgcn_raw_buffer_load_b32(make_buf(a.cache_len + b, 4), 0u, 0, 0);
        const BufRsrc kn0 = make_buf((const uint16_t *)a.k_new + nrow0 * kDqk, kDqk * 2);
        const BufRsrc vn0 = make_buf((const uint16_t *)a.v_new + nrow0 * kDv, kDv * 2);
        nk = buf_load16(kn0, lane < kDqk / 8 ? (uint32_t)lane * 16 : kOob);
        nv = buf_load16(vn0, lane < kDv / 8 ? (uint32_t)lane * 16 : kOob);
        const BufRsrc kc0 = make_buf((const uint8_t *)a.k_cache + crow0 * kDqk * kEs,
                                     (uint64_t)a.cap * kDqk * kEs);
        const BufRsrc vc0 = make_buf((const uint8_t *)a.v_cache + crow0 * kDv * kEs,
                                     (uint64_t)a.cap * kDv * kEs);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const uint32_t off = (uint32_t)(kKb * wave + 16 * kt + lr) * kDqk * 2;
#pragma unroll
            for (int s = 0; s < kDqk / 32; ++s)
                x.k[kt][s] = buf_load16(kc0, off + (uint32_t)kdim0<false>(s, kg) * 2);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int sl = kKb * wave + (e >> 2) * 16 + 4 * kg + (e & 3);
            x.v[e] = buf_load16_nt(vc0, ((uint32_t)sl * kDv + (uint32_t)lr * 8) * 2);
        }
    }
    const double inv_freq = kSlots && a.rope ? rope_inv_freq(a.rope_base, tid & 31, 64) : 0.0;
    const int P = clamp_len(kSlots ? (int)__builtin_amdgcn_readfirstlane(len_v) : a.cache_len[b],
                            a.max_len);
    const int lo = a.window > 0 ? max(0, P - a.window + 1) : 0;
    const int hi = P + nq;
    int rlo = lo, rhi = hi;
    if (a.n_splits > 1) {
        rlo = max(lo, split * a.chunk);
        rhi = min(hi, (split + 1) * a.chunk);
    }

    if (rlo >= rhi)
        return;  // uniform: this chunk holds no visible key

    const uint64_t cache_rows = a.ring ? (uint64_t)a.cap : (uint64_t)P;
    const BufRsrc kc = make_buf((const uint8_t *)a.k_cache + crow0 * kDqk * kEs,
                                cache_rows * kDqk * kEs);
    const BufRsrc vc = make_buf((const uint8_t *)a.v_cache + crow0 * kDv * kEs,
                                cache_rows * kDv * kEs);
    const BufRsrc kn = make_buf((const uint16_t *)a.k_new + nrow0 * kDqk,
                                ((uint64_t)(nq - 1) * Hkv + 1) * kDqk * 2);
    const BufRsrc vn = make_buf((const uint16_t *)a.v_new + nrow0 * kDv,
                                ((uint64_t)(nq - 1) * Hkv + 1) * kDv * 2);

    const int qpos = col_ok ? P + col / group : -1;
    if constexpr (!kSlots)
        load_q();
    const int ce = min(rhi, P);
    const int n_cache_blk = ce > rlo ? (ce - rlo + kKb - 1) / kKb : 0;
    const int new_lo = max(rlo, P);
    // One new token whose position falls inside the last cache block's 32-key span
    // (a ring layer's window of 128 keys: 127 cached + the new one) is computed as
    // part of that block instead of as a block of its own: the wave that takes
    // the block stages the token's k (rotated when RoPE is fused) and v rows in
    // LDS, and the lanes holding key P take their operands from there (the cache
    // loads of position P read nothing).  bf16 caches, waves splitting the blocks.
    const bool merge_new = !kTok && !kFp8 && nq == 1 && n_cache_blk > 0 && rhi > new_lo &&
                           P < rlo + n_cache_blk * kKb;
    const int nblk = n_cache_blk + (rhi > new_lo && !merge_new ? 1 : 0);
    const int slot_new = P & (kWaves * kKb - 1);  // slot mode: the slot of position P
    const int window = a.window;
    const uint32_t krow = (uint32_t)Hkv * kDqk * 2, vrow = (uint32_t)Hkv * kDv * 2;

    auto block_base = [&](int j) { return j < n_cache_blk ? rlo + j * kKb : new_lo; };
    // K and V of block j are loaded separately: the K registers are reloaded
    // for the wave's next block as soon as QK has consumed them, the V registers
    // after PV, so one register set keeps loads in flight through the compute.
    // Cache blocks and the new-token block use separate functions so that every
    // load names one descriptor.
    auto load_k = [&](int j, KVc &x) {
        const int kb = rlo + j * kKb;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const int p = kb + 16 * kt + lr;
            const int slot = a.ring ? p % a.cap : p;
            if constexpr (kFp8) {
                const uint32_t off = p < ce ? (uint32_t)slot * kDqk + (uint32_t)kg * 16 : kOob;
#pragma unroll
                for (int u = 0; u < kDqk / 64; ++u)
                    x.k[kt][u] = buf_load16(kc, off + (uint32_t)u * 64);
            } else {
                const uint32_t off = p < ce ? (uint32_t)slot * kDqk * 2 : kOob;
#pragma unroll
                for (int s = 0; s < kDqk / 32; ++s)
                    x.k[kt][s] = buf_load16(kc, off + (uint32_t)kdim0<false>(s, kg) * 2);
            }
        }
    };
    auto load_v = [&](int j, KVc &x) {
        const int kb = rlo + j * kKb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int p = kb + (e >> 2) * 16 + 4 * kg + (e & 3);
            const int slot = a.ring ? p % a.cap : p;
            const uint32_t off =
                p < ce ? ((uint32_t)slot * kDv + (uint32_t)lr * 8) * kEs : kOob;
            // a load instruction reads whole V rows: non-temporal when each row is
            // read once (token waves read every row once per wave: keep them in L2)
            if constexpr (kFp8)
                x.v[e] = kTok ? buf_load8(vc, off) : buf_load8_nt(vc, off);
            else
                x.v[e] = kTok ? buf_load16(vc, off) : buf_load16_nt(vc, off);
        }
    };
    auto load_new = [&](KV16 &x) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const int p = new_lo + 16 * kt + lr;
            const uint32_t off = p < rhi ? (uint32_t)(p - P) * krow : kOob;
#pragma unroll
            for (int s = 0; s < kDqk / 32; ++s)
                x.k[kt][s] = buf_load16(kn, off + (uint32_t)kdim0<kFp8>(s, kg) * 2);
            if (a.rope && p < rhi) {
                const float2 *cs = rope_tab + (p - P) * 32;
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    x.k[kt][s] = rope_chunk_bf16(x.k[kt][s], cs + 4 * (kdim0<kFp8>(s, kg) / 8));
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int p = new_lo + (e >> 2) * 16 + 4 * kg + (e & 3);
            const uint32_t off = p < rhi ? (uint32_t)(p - P) * vrow + (uint32_t)lr * 16 : kOob;
            x.v[e] = buf_load16(vn, off);
        }
    };
    // The wave's first cache block is requested before the RoPE table and the
    // new-token store, so its memory latency overlaps that work (the store
    // writes position P, which no cache block reads).
    const bool merge_wave = slot_mode ? slot_new / kKb == wave
                                      : merge_new && (n_cache_blk - 1) % kWaves == wave;  // wave-uniform
    if (merge_wave && !slot_mode) {
        nk = buf_load16(kn, lane < kDqk / 8 ? (uint32_t)lane * 16 : kOob);
        nv = buf_load16(vn, lane < kDv / 8 ? (uint32_t)lane * 16 : kOob);
    }
    if constexpr (kTok) {
        if (active && kh < n_cache_blk) {
            load_k(kh, x);
            load_v(kh, x);
        }
    } else {
        if (!slot_mode && wave < n_cache_blk) {
            load_k(wave, x);
            load_v(wave, x);
        }
    }

    // RoPE (when fused): (cos, sin) of positions P .. P+nq-1 for q and the new keys.
    if (a.rope) {
        if constexpr (kSlots)
            rope_fill_table64_inv(rope_tab, P, nq, inv_freq, tid, kThreads);
        else
            rope_fill_table64(rope_tab, P, nq, a.rope_base, tid, kThreads);
        __syncthreads();
    }
    // The chunk holding position P stores the new token (decode) / rotated keys.
    if (P >= rlo && P < rhi) {
        if (a.rope)
            cached_store_new<true, kFp8>(a, crow0, nrow0, P, rope_tab, tid, kThreads, !kSlots);
        else
            cached_store_new<false, kFp8>(a, crow0, nrow0, P, rope_tab, tid, kThreads, !kSlots);
    }

    if (merge_wave) {  // wave-private: the same wave reads the rows back (LDS keeps its order)
        // slot mode: this wave also stores the token into the cache from these
        // registers (slot P mod 128), instead of the workgroup reading k_new / v_new
        // again for the store
        const bool store = kSlots && a.write_new;
        if (lane < kDqk / 8) {
            uint4 v = nk;
            if (a.rope && lane < 8)
                v = rope_chunk_bf16(v, rope_tab + 4 * lane);
            new_row[lane] = v;
            if (store)
                *(uint4 *)((uint16_t *)a.k_cache + (crow0 + slot_new) * kDqk + lane * 8) = v;
        }
        if (lane < kDv / 8) {
            new_row[kDqk / 8 + lane] = nv;
            if (store)
                *(uint4 *)((uint16_t *)a.v_cache + (crow0 + slot_new) * kDv + lane * 8) = nv;
        }
    }

    bf16x8 qf[kDqk / 32];
    if (a.rope && col_ok) {  // k-steps 0, 1 hold dims < 64: 8-dim chunk kdim0/8
        const float2 *cs = rope_tab + (col / group) * 32;
#pragma unroll
        for (int s = 0; s < 2; ++s)
            qr[s] = rope_chunk_bf16(qr[s], cs + 4 * (kdim0<kFp8>(s, kg) / 8));
    }
#pragma unroll
    for (int s = 0; s < kDqk / 32; ++s)
        qf[s] = as_bf16x8(qr[s]);

    float m = -INFINITY, l = 0.f;
    f32x4v acc[8];
#pragma unroll
    for (int db = 0; db < 8; ++db)
        acc[db] = f32x4v{};

    // x is a cache block (KVc, prefetching the wave's next block jn) or the
    // new-token block (KV16 read from k_new / v_new, bf16 even with E4M3 caches).
    auto compute = [&](int j, int jn, auto &x) {
        constexpr bool kCacheRegs = std::is_same<std::decay_t<decltype(x)>, KVc>::value;
        constexpr bool kScaled = kFp8 && kCacheRegs;  // E4M3 codes: fold the scales in
        const int kb = block_base(j);
        const bool merged = kCacheRegs && (slot_mode ? merge_wave : merge_new && j == n_cache_blk - 1);
        const int kend = j < n_cache_blk && !merged && !slot_mode ? ce : rhi;
        // position of key i of the block (slot mode: the slot's newest position <= P,
        // negative for a slot not written yet) and whether it is the new token
        auto key_pos = [&](int i) {
            return slot_mode ? P - ((P - (kKb * wave + i)) & (kWaves * kKb - 1)) : kb + i;
        };
        if constexpr (kCacheRegs && !kFp8) {
            if (merged) {  // lanes holding key P take its operands from the staged rows
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
                    if (key_pos(16 * kt + lr) == P) {
#pragma unroll
                        for (int s = 0; s < kDqk / 32; ++s)
                            x.k[kt][s] = new_row[kdim0<false>(s, kg) / 8];
                    }
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (key_pos((e >> 2) * 16 + 4 * kg + (e & 3)) == P)
                        x.v[e] = new_row[kDqk / 8 + lr];
            }
        }
        const float sl2 = kScaled ? scale_log2 * a.k_scale : scale_log2;
        f32x4v sc[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            sc[kt] = f32x4v{};
#pragma unroll
            for (int s = 0; s < kDqk / 32; ++s)
                sc[kt] = mfma16x16x32(k_operand(x, kt, s), qf[s], sc[kt]);
        }
        if constexpr (kCacheRegs) {
            if (jn < n_cache_blk)
                load_k(jn, x);
        }
        // element e of this lane: key kb + (e/4)*16 + 4*kg + e%4, column lr
        const bool full = slot_mode ? P >= kWaves * kKb - 1 && (window <= 0 || window >= kWaves * kKb)
                                    : j < n_cache_blk && !merged && kb + kKb <= ce &&
                                          (window <= 0 || kb >= P + nq - window);
        float xs[8];
        uint32_t hidden = 0;  // slot mode: elements whose V rows must stay out of PV
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = sc[e >> 2][e & 3];
            if (!full) {
                const int p = key_pos((e >> 2) * 16 + 4 * kg + (e & 3));
                const bool vis = p >= 0 && p < kend && p <= qpos && (window <= 0 || qpos - p < window);
                v = vis ? v : -INFINITY;
                // by key, whatever the lane's column: a slot not written yet, or one
                // behind a window narrower than the ring (stale rows of any value)
                hidden |= (p < 0 || (window > 0 && P - p >= window)) ? 1u << e : 0u;
            }
            xs[e] = col_ok ? v : -INFINITY;
        }
        float bm = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            bm = fmaxf(bm, xs[e]);
        bm = max_across_rows(bm);
        bm *= sl2;
        const bool up = bm > m + kRescaleSlack || (m == -INFINITY && bm > -INFINITY);
        const float mn = up ? bm : m;
        const float alpha = up ? fast_exp2(m - mn) : 1.f;
        m = mn;
        const float mu = (mn == -INFINITY) ? 0.f : mn;
        float ps = 0.f;
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float pr = fast_exp2(__fmaf_rn(xs[e], sl2, -mu));
            ps += pr;
            pb[e] = (__bf16)(kScaled ? pr * a.v_scale : pr);  // P^T feeds V codes * v_scale
        }
        l = __fmaf_rn(l, alpha, ps);
        if (__builtin_amdgcn_ballot_w64(up) != 0) {
#pragma unroll
            for (int db = 0; db < 8; ++db)
                acc[db] *= alpha;
        }
        // V^T operand of tile db: element e = V[key(e)][8*lr + db]; vr[e] holds dims
        // 8lr..8lr+7 of key(e), so each operand word pairs one 16-bit half of two loads.
        uint4 vr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            vr[e] = v_rows(x, e);
        if (slot_mode && !full) {  // a slot not written yet may hold anything (NaN): zero it
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (hidden & (1u << e))
                    vr[e] = make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            uint32_t w[4];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const uint4 va0 = vr[2 * e2], va1 = vr[2 * e2 + 1];
                const uint32_t wa = (db >> 1) == 0 ? va0.x : (db >> 1) == 1 ? va0.y : (db >> 1) == 2 ? va0.z : va0.w;
                const uint32_t wb = (db >> 1) == 0 ? va1.x : (db >> 1) == 1 ? va1.y : (db >> 1) == 2 ? va1.z : va1.w;
                w[e2] = (db & 1) ? __builtin_amdgcn_perm(wb, wa, 0x07060302u)
                                 : __builtin_amdgcn_perm(wb, wa, 0x05040100u);
            }
            acc[db] = mfma16x16x32(as_bf16x8(make_uint4(w[0], w[1], w[2], w[3])), pb, acc[db]);
        }
        if constexpr (kCacheRegs) {
            if (jn < n_cache_blk)
                load_v(jn, x);
        }
    };

    // Cache blocks j = wave, wave+4, ..., then the new-token block (index
    // n_cache_blk) on the wave it falls to.  At about 200 registers two waves
    // share each SIMD (a second register set per wave measured slower: one wave
    // per SIMD).
    if constexpr (kTok) {
        if (active) {  // wave-uniform
            for (int j = kh; j < n_cache_blk; j += n_kh)
                compute(j, j + n_kh, x);
            if (nblk > n_cache_blk && n_cache_blk % n_kh == kh) {
                KV16 xn;
                load_new(xn);
                compute(n_cache_blk, nblk, xn);
            }
        }
    } else if (slot_mode) {
        compute(wave, 1 << 30, x);  // the wave's 32 slots, the new token merged in
    } else {
        for (int j = wave; j < n_cache_blk; j += kWaves)
            compute(j, j + kWaves, x);
        if (nblk > n_cache_blk && n_cache_blk % kWaves == wave) {
            KV16 xn;
            load_new(xn);
            compute(n_cache_blk, nblk, xn);
        }
    }

    // l is per lane group (16 lanes) -> total over the 4 groups of the column
    const float lt = sum_across_rows(l);

    if constexpr (!kTok) {
        // merge: every wave parks (acc, m, l) in LDS slot `wave`; after one barrier
        // wave w finalizes dims 8*(4kg + w) .. +7 of each column (lane (lr, kg)) from
        // the four slots in wave order, so the merge and the output stores are
        // spread over the four waves.  acc[db][i] holds dim 8*(4kg + i) + db of
        // column lr.
        if (col_ok) {
            float *e = &merge[wave][lr][0];
            if (kg == 0) {
                e[kDv] = m;
                e[kDv + 1] = lt;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 8 * (4 * kg + i);
                *(float4 *)&e[d0] = make_float4(acc[0][i], acc[1][i], acc[2][i], acc[3][i]);
                *(float4 *)&e[d0 + 4] = make_float4(acc[4][i], acc[5][i], acc[6][i], acc[7][i]);
            }
        }
        __syncthreads();
        if (!col_ok)
            return;
        const bool write_final = a.n_splits == 1;
        const size_t rows_total = (size_t)a.B * nq * Hq;
        const int h = g * group + col % group;
        const size_t row = ((size_t)b * nq + col / group) * Hq + h;
        float mw[kWaves], fw[kWaves];
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            mw[w] = merge[w][lr][kDv];
            mx = fmaxf(mx, mw[w]);
        }
        float M = mx, z = 0.f;
        if (write_final) {
            const float sink2 = a.sink[h] * kLog2e;
            M = fmaxf(mx, sink2);
            z = (sink2 == -INFINITY || M == -INFINITY) ? 0.f : fast_exp2(sink2 - M);
        }
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            fw[w] = (mw[w] == -INFINITY) ? 0.f : fast_exp2(mw[w] - M);
            z += merge[w][lr][kDv + 1] * fw[w];
        }
        const float so = write_final ? (z > 0.f ? 1.f / z : 0.f) : 1.f;
        const int d0 = 8 * (4 * kg + wave);
        float vals[8];
        {
            const float4 p0 = *(const float4 *)&merge[0][lr][d0];
            const float4 p1 = *(const float4 *)&merge[0][lr][d0 + 4];
            vals[0] = p0.x * fw[0];
            vals[1] = p0.y * fw[0];
            vals[2] = p0.z * fw[0];
            vals[3] = p0.w * fw[0];
            vals[4] = p1.x * fw[0];
            vals[5] = p1.y * fw[0];
            vals[6] = p1.z * fw[0];
            vals[7] = p1.w * fw[0];
        }
#pragma unroll
        for (int w = 1; w < kWaves; ++w) {
            const float4 p0 = *(const float4 *)&merge[w][lr][d0];
            const float4 p1 = *(const float4 *)&merge[w][lr][d0 + 4];
            vals[0] += p0.x * fw[w];
            vals[1] += p0.y * fw[w];
            vals[2] += p0.z * fw[w];
            vals[3] += p0.w * fw[w];
            vals[4] += p1.x * fw[w];
            vals[5] += p1.y * fw[w];
            vals[6] += p1.z * fw[w];
            vals[7] += p1.w * fw[w];
        }
        if (write_final) {
            uint4 u;
            u.x = pack_bf16x2(vals[0] * so, vals[1] * so);
            u.y = pack_bf16x2(vals[2] * so, vals[3] * so);
            u.z = pack_bf16x2(vals[4] * so, vals[5] * so);
            u.w = pack_bf16x2(vals[6] * so, vals[7] * so);
            *(uint4 *)((uint16_t *)a.o + row * kDv + d0) = u;
        } else {
            float *dst = &a.ws[2 * rows_total * a.n_splits + (row * a.n_splits + split) * kDv + d0];
            *(float4 *)dst = make_float4(vals[0], vals[1], vals[2], vals[3]);
            *(float4 *)(dst + 4) = make_float4(vals[4], vals[5], vals[6], vals[7]);
            if (kg == 0 && wave == 0) {
                const size_t slot = row * a.n_splits + split;
                a.ws[slot] = M;
                a.ws[rows_total * a.n_splits + slot] = (M == -INFINITY) ? 0.f : z;
            }
        }
    } else {
        // merge: the waves of phases 1 .. n_kh-1 of a column group park (acc, m, l) in
        // LDS (slot (phase-1) * n_cg + group); phase 0 folds them in, in phase order,
        // and writes.  acc[db][i] holds dim 8*(4kg + i) + db of column lr.
        const int n_park = n_kh - 1;
        if (active && kh > 0 && col_ok) {
            float *e = &merge[(kh - 1) * n_cg + cw][lr][0];
            if (kg == 0) {
                e[kDv] = m;
                e[kDv + 1] = lt;
            }
    #pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 8 * (4 * kg + i);
                *(float4 *)&e[d0] = make_float4(acc[0][i], acc[1][i], acc[2][i], acc[3][i]);
                *(float4 *)&e[d0 + 4] = make_float4(acc[4][i], acc[5][i], acc[6][i], acc[7][i]);
            }
        }
        if (n_park > 0)  // uniform
            __syncthreads();
        if (active && kh == 0 && col_ok) {
            const bool write_final = a.n_splits == 1;
            const size_t rows_total = (size_t)a.B * nq * Hq;
            const int t = col / group;
            const int h = g * group + col % group;
            const size_t row = ((size_t)b * nq + t) * Hq + h;
            float mx = m;
    #pragma unroll
            for (int w = 0; w < kMerge; ++w)
                if (w < n_park)
                    mx = fmaxf(mx, merge[w * n_cg + cw][lr][kDv]);
            float M = mx, zs = 0.f;
            if (write_final) {
                const float sink2 = a.sink[h] * kLog2e;
                M = fmaxf(mx, sink2);
                zs = (sink2 == -INFINITY || M == -INFINITY) ? 0.f : fast_exp2(sink2 - M);
            }
            const float f0 = (m == -INFINITY) ? 0.f : fast_exp2(m - M);
            float fw[kMerge];
            float z = zs + lt * f0;
    #pragma unroll
            for (int w = 0; w < kMerge; ++w) {
                fw[w] = 0.f;
                if (w < n_park) {
                    const float mw = merge[w * n_cg + cw][lr][kDv];
                    fw[w] = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
                    z += merge[w * n_cg + cw][lr][kDv + 1] * fw[w];
                }
            }
            const float so = write_final ? (z > 0.f ? 1.f / z : 0.f) : 1.f;
    #pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 8 * (4 * kg + i);
                float vals[8];
    #pragma unroll
                for (int db = 0; db < 8; ++db)
                    vals[db] = acc[db][i] * f0;
    #pragma unroll
                for (int w = 0; w < kMerge; ++w) {
                    if (w >= n_park)
                        break;
                    const float4 p0 = *(const float4 *)&merge[w * n_cg + cw][lr][d0];
                    const float4 p1 = *(const float4 *)&merge[w * n_cg + cw][lr][d0 + 4];
                    vals[0] += p0.x * fw[w];
                    vals[1] += p0.y * fw[w];
                    vals[2] += p0.z * fw[w];
                    vals[3] += p0.w * fw[w];
                    vals[4] += p1.x * fw[w];
                    vals[5] += p1.y * fw[w];
                    vals[6] += p1.z * fw[w];
                    vals[7] += p1.w * fw[w];
                }
                if (write_final) {
                    uint4 u;
                    u.x = pack_bf16x2(vals[0] * so, vals[1] * so);
                    u.y = pack_bf16x2(vals[2] * so, vals[3] * so);
                    u.z = pack_bf16x2(vals[4] * so, vals[5] * so);
                    u.w = pack_bf16x2(vals[6] * so, vals[7] * so);
                    *(uint4 *)((uint16_t *)a.o + row * kDv + d0) = u;
                } else {
                    float *dst = &a.ws[2 * rows_total * a.n_splits + (row * a.n_splits + split) * kDv + d0];
                    *(float4 *)dst = make_float4(vals[0], vals[1], vals[2], vals[3]);
                    *(float4 *)(dst + 4) = make_float4(vals[4], vals[5], vals[6], vals[7]);
                }
            }
            if (!write_final && kg == 0) {
                const size_t slot = row * a.n_splits + split;
                a.ws[slot] = M;
                a.ws[rows_total * a.n_splits + slot] = (M == -INFINITY) ? 0.f : z;
            }
        }
    }
}

}  // namespace

hipError_t launch_decode16(const CachedArgs &a, hipStream_t s) {
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    const dim3 grid((unsigned)(a.B * a.Hkv * a.n_splits)), block(kThreads);
    const bool tok = a.nq * (a.Hq / a.Hkv) > kCols;
    const bool slots = a.ring && a.nq == 1 && a.cap == kWaves * kKb && a.n_splits == 1;
    if (a.fp8) {
        if (tok)
            decode16_kernel<true, true, false><<<grid, block, 0, s>>>(a, scale_log2);
        else
            decode16_kernel<false, true, false><<<grid, block, 0, s>>>(a, scale_log2);
    } else {
        if (tok)
            decode16_kernel<true, false, false><<<grid, block, 0, s>>>(a, scale_log2);
        else if (slots)
            decode16_kernel<false, false, true><<<grid, block, 0, s>>>(a, scale_log2);
        else
            decode16_kernel<false, false, false><<<grid, block, 0, s>>>(a, scale_log2);
    }
    return hipGetLastError();
}

}  // namespace sinkattn

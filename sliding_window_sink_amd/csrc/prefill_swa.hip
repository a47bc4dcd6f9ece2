// prefill_swa.hip -- persistent sliding-window sink-attention prefill (gfx950, bf16).
//
// The operation is that of the MiMo-V2-Flash Technical Report, Section 2.2
// (sink softmax, equations 1-4) restricted to a window of W <= 129 keys
// (Table 1: W = 128): query i sees keys i-W+1 .. i.  With the rope option it
// also applies the partial RoPE of Section 2.1 (first 64 dims, interleaved
// pairs, base from Section 3.2) to q and k as they are loaded, giving the same
// bits as rotating q and k first with the standalone RoPE kernel.
//
// Why a persistent kernel: a sliding-window layer is HBM bound (about 114
// FLOP per byte, below the MI355X ridge), and its traffic is dominated by
// reading Q and writing O once.  Each workgroup therefore walks a contiguous
// run of 32-token tiles of one KV group and overlaps everything it can:
//   - the last 5 key blocks (32 keys each) of the window live in a 6-slot LDS
//     ring, so every K/V row is fetched from memory once per run, not once per
//     tile (a 32-token tile sees 159 keys);
//   - while tile i is computed, the next tile's Q (into registers) and its new
//     key block (into registers, then into the free ring slot) are in flight;
//   - the next tile's Q is requested in two halves, at the start of the tile
//     and after its third key block, so the loads reach HBM over most of the
//     tile rather than in one burst at its start (the memory otherwise idled
//     while the tile's last blocks were computed);
//   - one barrier per tile publishes the new key block;
//   - with RoPE, the fp32 (cos, sin) of a tile's 32 tokens are composed once per
//     tile into an LDS table (two entries per thread) that the Q of all 8 heads
//     and the tile's key block read, instead of each wave composing them in
//     fp64 for its own head.
// All global traffic goes through raw buffer descriptors (a wave-uniform base
// for the run plus a 32-bit lane offset): rows past the end of the sequence
// read as zero and their stores are dropped by the hardware, so there are no
// per-lane branches around loads and no 64-bit address registers to spill.
//
// Inside a tile: wave w owns query head 8*part + w; the 32 tokens are the MFMA
// columns; S^T = K Q^T with K rows permuted so register i of lane half hh holds
// key 16*hh + i; the online softmax is seeded with the sink; O^T += V^T P^T
// reads V^T from LDS.  The V^T rows are laid out so that each lane ends up
// holding runs of 8 consecutive output dims (16-byte stores).
//
// Grid: (batch, KV group, head part) units x runs, unit = blockIdx % units, so
// each XCD keeps whole runs of one KV group in its L2.  One workgroup per CU
// (8 waves, 2 per SIMD, ~151 KB of LDS).
#include <algorithm>

#include "common.h"

namespace sinkattn {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kTq = 32;
constexpr int kKb = 32;
constexpr int kSlots = 6;
constexpr int kKPitch = kDqk + 8;   // 400-byte LDS rows for K
constexpr int kVPitch = kKb + 8;    // 80-byte LDS rows for V^T
constexpr int kKChunks = kKb * kDqk / 8;  // 768 16-byte pieces per key block
constexpr int kVChunks = kKb * kDv / 8;   // 512
constexpr int kPairs = 32;          // rope_dim / 2 with rope_dim = 64
constexpr int kMaxWinBlocks = kSlots - 1;  // key blocks a tile's window spans (W <= 129)
constexpr int kQSplit = 3;  // key blocks after which the second half of the next Q is requested
static_assert(kVChunks == kThreads, "one V piece per thread");

// RoPE.  A position splits as p = 32*floor(p/32) + (p mod 32); its (cos, sin)
// is the fp64 composition of the rotations by the two parts, rounded to fp32
// (rope_compose).  Tiles and key blocks are both 32 tokens, so one table of
// fp32 (cos, sin) per tile serves the tile's Q (all 8 heads) and its key block.
struct SwaSmem {
    uint16_t k[kSlots][kKb * kKPitch];
    uint16_t vt[kSlots][kDv * kVPitch];
    // tables of tiles t (buffer t & 1), pair major, so the 32 lanes of a wave --
    // one token each -- read consecutive entries
    float2 cs[2][kPairs][kTq];
    double2 hi_rot[2][kPairs];                 // by the bases of tiles (buffer t & 1)
    double2 hi_pro[kMaxWinBlocks][kPairs];     // by the bases of the prologue's blocks
    double inv_freq[kPairs];
};

struct SwaRope {
    double base;
    uint16_t *k_rot;  // optional copy of rotated k [B,T,Hkv,192]
};

// rope_sincos64 as a real call, for the refill inside the tile loop: inlined,
// the compiler keeps the fp64 sincos's polynomial constants in VGPR pairs
// across the whole loop (16 registers the score loop can use instead).
__device__ __attribute__((noinline)) double2 rope_sincos64_call(int p, double inv_freq) {
    return rope_sincos64(p, inv_freq);
}

// V^T LDS row holding output dim d.  Block db, C-row rho = 8a + 4hh + e of the PV
// accumulators holds dim 32a + 16(db/2) + 8hh + 4(db%2) + e, so for each (a, db/2)
// a lane owns 8 consecutive dims and the two lane halves are adjacent.
__device__ __forceinline__ int pv_row_of_dim(int d) {
    const int a = d >> 5, j = (d >> 4) & 1, hh = (d >> 3) & 1, dbl = (d >> 2) & 1, e = d & 3;
    return 32 * (2 * j + dbl) + 8 * a + 4 * hh + e;
}

template <bool kRope>
__global__ __launch_bounds__(kThreads) void prefill_swa_kernel(PrefillArgs a, SwaRope rp,
                                                                int n_units, int n_tiles,
                                                                int tiles_per_run,
                                                                float scale_log2) {
    __shared__ SwaSmem sm;
    const int T = a.T, Hq = a.Hq, Hkv = a.Hkv, window = a.window;
    const int group = Hq / Hkv;
    const int parts = group / kWaves;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 31, hh = lane >> 5;
    const int unit = blockIdx.x % n_units;
    const int run = blockIdx.x / n_units;
    const int part = unit % parts;
    const int g = (unit / parts) % Hkv;
    const int b = unit / (parts * Hkv);
    const int h = g * group + part * kWaves + wave;
    const int tile_begin = run * tiles_per_run;
    const int tile_end = min(n_tiles, tile_begin + tiles_per_run);
    if (tile_begin >= tile_end)
        return;

    auto first_block = [&](int t0) { return max(0, t0 - window + 1) / kKb; };

    // Descriptors for this run: every token it touches is >= tbase.
    const int tbase = first_block(tile_begin * kTq) * kKb;
    const size_t row0 = (size_t)b * T + tbase;
    const uint64_t nrows = (uint64_t)(T - tbase);
    const uint32_t qrow = (uint32_t)Hq * kDqk * 2, orow = (uint32_t)Hq * kDv * 2;
    const uint32_t krow = (uint32_t)Hkv * kDqk * 2, vrow = (uint32_t)Hkv * kDv * 2;
    const BufRsrc qbuf = make_buf((const uint16_t *)a.q + row0 * Hq * kDqk, nrows * qrow);
    const BufRsrc kbuf = make_buf((const uint16_t *)a.k + row0 * Hkv * kDqk, nrows * krow);
    const BufRsrc vbuf = make_buf((const uint16_t *)a.v + row0 * Hkv * kDv, nrows * vrow);
    const BufRsrc obuf = make_buf((uint16_t *)a.o + row0 * Hq * kDv, nrows * orow);
    const bool write_krot = kRope && rp.k_rot != nullptr && part == 0;
    const BufRsrc krbuf = make_buf(write_krot ? rp.k_rot + row0 * Hkv * kDqk : (uint16_t *)a.k,
                                   write_krot ? nrows * krow : 0);
    const uint32_t qcol = (uint32_t)h * kDqk * 2, kcol = (uint32_t)g * kDqk * 2,
                   vcol = (uint32_t)g * kDv * 2, ocol = (uint32_t)h * kDv * 2;

    // Each thread builds table entries (pair c_lo, token j) and (c_lo + 16, j) of
    // every tile; it keeps the rotations of those two entries by j * theta_c in
    // registers for the whole run.
    const int c_lo = tid / kTq, j_lo = tid % kTq;
    double2 lo_a = make_double2(1.0, 0.0), lo_b = lo_a;
    if (kRope) {
        if (tid < kPairs)
            sm.inv_freq[tid] = rope_inv_freq(rp.base, tid, 2 * kPairs);
        __syncthreads();
        lo_a = rope_sincos64(j_lo, sm.inv_freq[c_lo]);
        lo_b = rope_sincos64(j_lo, sm.inv_freq[c_lo + kPairs / 2]);
    }
    // hi_rot[t & 1] <- rotation by the base of tile t, threads 0..31.
    auto fill_hi = [&](int t) {
        if (tid < kPairs)
            sm.hi_rot[t & 1][tid] = rope_sincos64_call(t * kTq, sm.inv_freq[tid]);
    };
    // cs[buf] <- the table of the block whose base rotation is hi[]: two entries
    // per thread (the entry indices are recomputed from an opaque copy of tid,
    // not held in registers across the loop)
    auto fill_table = [&](const double2 *hi, int buf) {
        int t = tid;
        asm volatile("" : "+v"(t));
        const int c = t / kTq, j = t % kTq;
        sm.cs[buf][c][j] = rope_compose(hi[c], lo_a);
        sm.cs[buf][c + kPairs / 2][j] = rope_compose(hi[c + kPairs / 2], lo_b);
    };
    // (cos, sin) of pairs c0..c0+3 of the token at offset j, from table buf
    auto rot4 = [&](int buf, int j, int c0, float2 (&cs)[4]) {
#pragma unroll
        for (int p = 0; p < 4; ++p)
            cs[p] = sm.cs[buf][c0 + p][j];
    };

    // ---- key blocks: global -> registers -> (rotate) -> LDS ring slot ----
    // Per-thread offsets, computed once: K pieces c = tid, tid + 512 (key c/24, dims
    // (c%24)*8..+7); V piece of v_stage_coords.  Output dim
    // 8*dc + j sits in V^T row vrow0 + 32*(j/4) + j%4 (see pv_row_of_dim).
    // These per-thread coordinates are recomputed from an opaque copy of tid
    // where a block is loaded or stored (a few integer operations per tile)
    // instead of being held in ~10 registers across the score loop.
    const bool k2 = tid + kThreads < kKChunks;  // wave-uniform
    struct Piece {
        int k_key[2], k_d[2], v_kk, v_dc;
    };
    auto piece = [&]() {
        int t = tid;
        asm volatile("" : "+v"(t));
        Piece pc;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = min(t + u * kThreads, kKChunks - 1);
            pc.k_key[u] = c / (kDqk / 8);
            pc.k_d[u] = c % (kDqk / 8);
        }
        v_stage_coords(t, pc.v_kk, pc.v_dc);
        return pc;
    };
    auto kg_off = [&](const Piece &pc, int u) {
        return (uint32_t)pc.k_key[u] * krow + kcol + (uint32_t)pc.k_d[u] * 16;
    };

    auto load_block = [&](int jb, uint4 (&kreg)[2], uint4 &vreg) {
        const Piece pc = piece();
        const uint32_t rel = (uint32_t)(jb * kKb - tbase);
        kreg[0] = buf_load16(kbuf, rel * krow + kg_off(pc, 0));
        if (k2)
            kreg[1] = buf_load16(kbuf, rel * krow + kg_off(pc, 1));
        vreg = buf_load16(vbuf, (rel + (uint32_t)pc.v_kk) * vrow + vcol + (uint32_t)pc.v_dc * 16);
    };
    // tab: table of the block's tokens (rope only); own: this run writes k_rot
    auto store_block = [&](int jb, const uint4 (&kreg)[2], const uint4 &vreg, int tab, bool own) {
        const Piece pc = piece();
        const int slot = jb % kSlots;
        const uint32_t rel = (uint32_t)(jb * kKb - tbase);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (u == 0 || k2) {
                uint4 x = kreg[u];
                if (kRope && pc.k_d[u] < 8) {
                    float2 cs[4];
                    rot4(tab, pc.k_key[u], 4 * pc.k_d[u], cs);
                    x = rope_chunk_bf16(x, cs);
                }
                *(uint4 *)&sm.k[slot][row_of_key(pc.k_key[u]) * kKPitch + pc.k_d[u] * 8] = x;
                if (kRope && write_krot && own)
                    buf_store16(krbuf, rel * krow + kg_off(pc, u), x);
            }
        }
        const uint32_t w[4] = {vreg.x, vreg.y, vreg.z, vreg.w};
        uint16_t *vt = &sm.vt[slot][pv_row_of_dim(pc.v_dc * 8) * kVPitch + pc.v_kk];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            vt[(32 * (j >> 2) + (j & 3)) * kVPitch] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
    };
    // Q^T operand of one tile: k-step s, half hh -> dims (2s+hh)*8 .. +7 of token t0+r.
    // k-steps [s_lo, s_hi) of it
    auto load_q = [&](int t0, uint4 (&qr)[kDqk / 16], int s_lo, int s_hi) {
        const uint32_t off = (uint32_t)(t0 + r - tbase) * qrow + qcol + (uint32_t)hh * 16;
#pragma unroll
        for (int s = 0; s < kDqk / 16; ++s)
            if (s >= s_lo && s < s_hi)
                qr[s] = buf_load16(qbuf, off + (uint32_t)s * 32);
    };
    auto rotate_q = [&](uint4 (&qr)[kDqk / 16], int tab) {
        if (kRope) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {  // dims < 64: chunks 2s+hh < 8
                float2 cs[4];
                rot4(tab, r, 4 * (2 * s + hh), cs);
                qr[s] = rope_chunk_bf16(qr[s], cs);
            }
        }
    };

    // ---- prologue: the first tile's window and Q ----
    // Rotation schedule of the loop (tile i, all before its closing barrier): the
    // new key block and the next Q are rotated with tile i+1's table; then every
    // thread builds its entries of tile i+2's table from hi_rot of tile i+2, and
    // threads 0..31 compute hi_rot of tile i+3.  The barrier publishes both, and
    // the buffers written are the ones last read before the previous barrier.
    uint4 qcur[kDqk / 16];
    {
        // All of the first tile's window blocks are requested at once (one memory
        // latency rather than one per block), their base rotations computed side
        // by side into hi_pro, those of the next two tiles into hi_rot.
        const int t0 = tile_begin * kTq;
        const int jlo = first_block(t0), jhi = t0 / kKb;
        const int nb = jhi - jlo + 1;  // 1 .. kMaxWinBlocks
        const int cb = tile_begin & 1;
        uint4 kr[kMaxWinBlocks][2], vr[kMaxWinBlocks];
#pragma unroll
        for (int i = 0; i < kMaxWinBlocks; ++i)
            if (i < nb)
                load_block(jlo + i, kr[i], vr[i]);
        load_q(t0, qcur, 0, kDqk / 16);
        if (kRope) {
            const int i = tid / kPairs, c = tid % kPairs;
            if (i < nb)
                sm.hi_pro[i][c] = rope_sincos64((jlo + i) * kKb, sm.inv_freq[c]);
            else if (i >= kMaxWinBlocks && i < kMaxWinBlocks + 2) {
                const int t = tile_begin + 1 + (i - kMaxWinBlocks);
                if (t < tile_end)
                    sm.hi_rot[t & 1][c] = rope_sincos64(t * kTq, sm.inv_freq[c]);
            }
            __syncthreads();
            if (tile_begin + 1 < tile_end)
                fill_table(sm.hi_rot[cb ^ 1], cb ^ 1);
        }
        // window blocks one at a time through table cb (with RoPE): build, sync,
        // rotate and store, sync
#pragma unroll
        for (int i = 0; i < kMaxWinBlocks; ++i)
            if (i < nb) {
                if (kRope) {
                    fill_table(sm.hi_pro[i], cb);
                    __syncthreads();
                }
                store_block(jlo + i, kr[i], vr[i], cb, i == nb - 1);
                if (i == nb - 1)
                    rotate_q(qcur, cb);
                if (kRope)
                    __syncthreads();
            }
        __syncthreads();
    }

    const float sink2 = a.sink[h] * kLog2e;

    for (int tile = tile_begin; tile < tile_end; ++tile) {
        const int t0 = tile * kTq;
        const int query = t0 + r;
        const int jlo = first_block(t0), jhi = t0 / kKb;
        const bool has_next = tile + 1 < tile_end;

        // The next tile's Q is requested in two halves, the second after the
        // first kQSplit key blocks (see the header).
        uint4 kreg[2], vreg, qnext[kDqk / 16];
        if (has_next) {
            load_block(jhi + 1, kreg, vreg);
            load_q(t0 + kTq, qnext, 0, kDqk / 32);
        }

        float m = sink2;
        float l = (hh == 0 && sink2 != -INFINITY) ? 1.f : 0.f;
        f32x16 acc[4];
#pragma unroll
        for (int db = 0; db < 4; ++db)
            acc[db] = f32x16{};

        for (int jb = jlo; jb <= jhi; ++jb) {
            const int kb = jb * kKb;
            const uint16_t *ks = sm.k[jb % kSlots];
            const uint16_t *vs = sm.vt[jb % kSlots];
            if (has_next && jb == jlo + kQSplit)
                load_q(t0 + kTq, qnext, kDqk / 32, kDqk / 16);
            f32x16 sc = f32x16{};
            // K operands are read from LDS 4 k-steps at a time: the fence keeps the
            // scheduler from hoisting all 12 reads (48 registers) above the MFMAs.
#pragma unroll
            for (int s0 = 0; s0 < kDqk / 16; s0 += 4) {
#pragma unroll
                for (int s = s0; s < s0 + 4; ++s) {
                    const bf16x8 ka =
                        as_bf16x8(*(const uint4 *)(ks + r * kKPitch + (2 * s + hh) * 8));
                    sc = mfma32x32x16(ka, as_bf16x8(qcur[s]), sc);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // raw scores; masked ones -> -inf.  scale_log2 > 0, so the max of the raw
            // scores times the scale is the max of the scaled logits.
            // only the window-edge and diagonal blocks need the per-element mask;
            // the test is uniform, so the mask sits behind a scalar branch
            const bool full = (kb + kKb - 1 <= t0) && (t0 + kTq - 1 - kb < window);
            if (!full) {
                // key kb + 16hh + i is visible iff 0 <= query - key < window: one
                // unsigned compare of d - i per element
                const uint32_t d = (uint32_t)(query - kb - 16 * hh);
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    sc[i] = (d - (uint32_t)i < (uint32_t)window) ? sc[i] : -INFINITY;
            }
            float bm = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                bm = fmaxf(bm, sc[i]);
            bm = max_across_halves(bm) * scale_log2;
            // raise m only when the block max passes it by more than the slack
            const bool up = bm > m + kRescaleSlack || (m == -INFINITY && bm > -INFINITY);
            const float mn = up ? bm : m;
            const float alpha = up ? fast_exp2(m - mn) : 1.f;
            m = mn;
            const float mu = (mn == -INFINITY) ? 0.f : mn;
            float ps = 0.f;
            bf16x8 pb[2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = fast_exp2(__fmaf_rn(sc[i], scale_log2, -mu));
                ps += p;
                pb[i >> 3][i & 7] = (__bf16)p;
            }
            l = __fmaf_rn(l, alpha, ps);
            if (__builtin_amdgcn_ballot_w64(up) != 0) {  // wave-uniform rescale
#pragma unroll
                for (int db = 0; db < 4; ++db)
                    acc[db] *= alpha;
            }
            // Raised wave priority while issuing the PV products, so the SIMD's
            // other wave (in its softmax) does not delay their issue: 0.5-2%
            // faster (the same around the score products gave nothing).
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int db = 0; db < 4; ++db) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const bf16x8 va =
                        as_bf16x8(*(const uint4 *)(vs + (32 * db + r) * kVPitch + 16 * hh + 8 * t));
                    acc[db] = mfma32x32x16(va, pb[t], acc[db]);
                }
                if (db & 1)
                    __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_s_setprio(0);
        }

        if (has_next && jhi < jlo + kQSplit)  // windows of fewer blocks
            load_q(t0 + kTq, qnext, kDqk / 32, kDqk / 16);
        // The prefetched key block and Q are consumed before O is stored, so no
        // wait on the prefetch can also end up waiting on the stores.
        if (has_next) {
            const int nb = (tile + 1) & 1;  // table of the next tile's tokens
            store_block(jhi + 1, kreg, vreg, nb, true);
            rotate_q(qnext, nb);
        }

        // epilogue: o = acc / l, 16-byte stores of 8 consecutive dims
        const float lt = sum_across_halves(l);
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const uint32_t obase = (uint32_t)(query - tbase) * orow + ocol + (uint32_t)hh * 16;
#pragma unroll
        for (int aa = 0; aa < 4; ++aa)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const f32x16 &lo = acc[2 * j], &hi = acc[2 * j + 1];
                uint4 w;
                w.x = pack_bf16x2(lo[4 * aa + 0] * inv, lo[4 * aa + 1] * inv);
                w.y = pack_bf16x2(lo[4 * aa + 2] * inv, lo[4 * aa + 3] * inv);
                w.z = pack_bf16x2(hi[4 * aa + 0] * inv, hi[4 * aa + 1] * inv);
                w.w = pack_bf16x2(hi[4 * aa + 2] * inv, hi[4 * aa + 3] * inv);
                buf_store16(obuf, obase + (uint32_t)(64 * aa + 32 * j), w);
            }
        if (a.lse && hh == 0 && query < T) {
            const float mu = (m == -INFINITY) ? 0.f : m;
            a.lse[((size_t)b * Hq + h) * T + query] = lt > 0.f ? (mu + log2f(lt)) * kLn2 : -INFINITY;
        }

        if (has_next) {
#pragma unroll
            for (int s = 0; s < kDqk / 16; ++s)
                qcur[s] = qnext[s];
        }
        if (kRope) {
            if (tile + 2 < tile_end)
                fill_table(sm.hi_rot[tile & 1], tile & 1);
            if (tile + 3 < tile_end)
                fill_hi(tile + 3);
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_prefill_swa_persistent(const PrefillArgs &a, double rope_base, void *k_rot,
                                         bool rope, hipStream_t s) {
    const int group = a.Hq / a.Hkv;
    const int n_units = a.B * a.Hkv * (group / kWaves);
    const int n_tiles = (a.T + kTq - 1) / kTq;
    const int cus = device_cu_count();
    // one run per CU: enough runs to cover every CU once, each a contiguous range;
    // a run's byte span (its tiles plus the window before them) must stay below
    // 2^31 for the 32-bit offsets
    int runs_per_unit = std::max(1, std::min(n_tiles, (cus + n_units - 1) / n_units));
    const int64_t row_bytes = (int64_t)a.Hq * kDqk * 2;
    const int64_t max_tiles =
        std::max<int64_t>(1, ((1ll << 31) / row_bytes - 2 * kKb - kSwaMaxWindow) / kTq);
    runs_per_unit = (int)std::max<int64_t>(runs_per_unit, (n_tiles + max_tiles - 1) / max_tiles);
    const int tiles_per_run = (n_tiles + runs_per_unit - 1) / runs_per_unit;
    const int runs = (n_tiles + tiles_per_run - 1) / tiles_per_run;
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    const dim3 grid((unsigned)(n_units * runs)), block(kThreads);
    SwaRope rp{rope_base, (uint16_t *)k_rot};
    if (rope)
        prefill_swa_kernel<true><<<grid, block, 0, s>>>(a, rp, n_units, n_tiles, tiles_per_run,
                                                         scale_log2);
    else
        prefill_swa_kernel<false><<<grid, block, 0, s>>>(a, rp, n_units, n_tiles, tiles_per_run,
                                                          scale_log2);
    return hipGetLastError();
}

}  // namespace sinkattn

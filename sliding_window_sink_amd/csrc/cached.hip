// cached.hip -- decode / speculative-verify sink attention over a KV cache (gfx950, bf16).
//
// Queries at positions P + t (P = cache_len[b], t < nq) attend to the cached
// keys of their window plus the new tokens 0..t (MiMo-V2-Flash Technical
// Report, Section 2.2 for the sink softmax; Section 2.3.1 for decoding one
// token, or verifying 1 + K draft tokens in one pass, over a per-request cache).
//
// Caches are head-major [B, Hkv, cap, d].  A sliding-window layer keeps a ring
// of cap >= W slots (position p in slot p % cap); a global layer keeps a
// contiguous cache (position p at index p).  Positions >= P are always read
// from k_new / v_new, never from the cache: decode may therefore store its new
// token into the cache in the same launch without racing the readers, and
// verify never writes the cache at all.
//
// Which kernel serves a bf16 launch: decode16.hip for at most 16 columns, short
// windows and E4M3 caches; verify_lds.hip for more columns over a whole
// contiguous cache; the kernel below for the rest (windows past 4096 keys).
//
// Decomposition: one workgroup (4 waves) per (sequence, KV group, context
// chunk).  Columns of the 32x32 MFMA tile are (token, head) pairs of the KV
// group: nq*group <= 64, so one or two column blocks.  The chunk's cached keys
// are cut into blocks of 32 that the 4 waves take in turn (the <= 8 new tokens
// form one extra block at the end); each wave keeps its own online-softmax
// state (no sink), then the 4 states are merged through LDS.  With one chunk
// the merge adds the sink and writes o; with several it writes the
// unnormalised (m, l, acc) of the chunk to the workspace and a combine kernel
// adds the sink exactly once:
//   M = max(sink, max_c m_c),  Z = e^(sink-M) + sum_c l_c e^(m_c-M),
//   o = sum_c acc_c e^(m_c-M) / Z.
//
// Memory access: decode is HBM bound (16 FLOP per byte at 16 heads per KV
// head), so K and V go straight from HBM into MFMA operand registers (every
// byte read once, no LDS round trip) through raw buffer descriptors (keys past
// the valid range read as zero without a branch).  Each wave double-buffers:
// the loads of its next block are in flight while it computes the current one.
// For K the lane that owns A-row r reads 32 contiguous bytes of that key per
// k-step.  For V the output-dim order is chosen as dim = 4*row + block, so each
// lane reads 8 contiguous bytes (4 dims) of 16 keys and two lanes cover a
// 256-byte row; a register shuffle then builds the V^T operands.
#include "common.h"

namespace sinkattn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kKb = 32;
constexpr int kMaxNq = 8;
constexpr int kMergeStride = kDv + 4;  // floats per (wave, column): acc[128], m, l, pad
constexpr uint32_t kOob = 0x80000000u;  // an offset past every descriptor: reads 0

struct CachedGeom {
    int b, g, group, P, lo, hi, rlo, rhi;
};

__device__ __forceinline__ CachedGeom cached_geom(const CachedArgs &a, int split, int bg) {
    CachedGeom c;
    c.g = bg % a.Hkv;
    c.b = bg / a.Hkv;
    c.group = a.Hq / a.Hkv;
    c.P = clamp_len(a.cache_len[c.b], a.max_len);
    c.lo = a.window > 0 ? max(0, c.P - a.window + 1) : 0;
    c.hi = c.P + a.nq;
    c.rlo = c.lo;
    c.rhi = c.hi;
    if (a.n_splits > 1) {
        c.rlo = max(c.lo, split * a.chunk);
        c.rhi = min(c.hi, (split + 1) * a.chunk);
    }
    return c;
}

// One block of 32 keys in MFMA operand layout.
struct KVRegs {
    uint4 k[kDqk / 16];  // A-row r = key key_of_row(r); k-step s: dims (2s+hh)*8 .. +7
    uint2 v[16];         // keys 16*hh + i, dims 4r .. 4r+3
};

template <int NCB, bool kRope>
__global__ __launch_bounds__(kThreads) void cached_bf16_kernel(CachedArgs a, float scale_log2) {
    __shared__ __attribute__((aligned(16))) float merge[kWaves - 1][32][kMergeStride];
    __shared__ float2 rope_tab[kRope ? kMaxNq * 32 : 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 31, hh = lane >> 5;
    const int split = blockIdx.x % a.n_splits;
    const CachedGeom c = cached_geom(a, split, blockIdx.x / a.n_splits);
    const int group = c.group;
    const int n_cols = a.nq * group;
    const int Hkv = a.Hkv, nq = a.nq;

    // Descriptors: this (sequence, KV head)'s cache rows, and the new tokens.
    const size_t crow0 = ((size_t)c.b * Hkv + c.g) * a.cap;
    const uint64_t cache_rows = a.ring ? (uint64_t)a.cap : (uint64_t)c.P;
    const BufRsrc kc = make_buf((const uint16_t *)a.k_cache + crow0 * kDqk, cache_rows * kDqk * 2);
    const BufRsrc vc = make_buf((const uint16_t *)a.v_cache + crow0 * kDv, cache_rows * kDv * 2);
    const size_t nrow0 = (size_t)c.b * nq * Hkv + c.g;  // row of token t: nrow0 + t*Hkv
    const uint64_t new_bytes_k = ((uint64_t)(nq - 1) * Hkv + 1) * kDqk * 2;
    const uint64_t new_bytes_v = ((uint64_t)(nq - 1) * Hkv + 1) * kDv * 2;
    const BufRsrc kn = make_buf((const uint16_t *)a.k_new + nrow0 * kDqk, new_bytes_k);
    const BufRsrc vn = make_buf((const uint16_t *)a.v_new + nrow0 * kDv, new_bytes_v);

    // RoPE (when fused): (cos, sin) of positions P .. P+nq-1 for q and the new keys.
    if constexpr (kRope) {
        rope_fill_table64(rope_tab, c.P, nq, a.rope_base, tid, kThreads);
        __syncthreads();
    }
    // Decode: store the new token into the cache (slot / index P); verify with
    // fused RoPE: write the rotated new keys out.  Nothing in this launch reads
    // those rows.
    if (split == 0) {
        if constexpr (kRope) {
            cached_store_new<true>(a, crow0, nrow0, c.P, rope_tab, tid, kThreads);
        } else if (a.write_new && (a.ring || c.P < a.cap)) {
            const int slot = a.ring ? (c.P % a.cap) : c.P;
            uint16_t *kd = (uint16_t *)a.k_cache + (crow0 + slot) * kDqk;
            uint16_t *vd = (uint16_t *)a.v_cache + (crow0 + slot) * kDv;
            const uint16_t *ks = (const uint16_t *)a.k_new + nrow0 * kDqk;
            const uint16_t *vs = (const uint16_t *)a.v_new + nrow0 * kDv;
            if (tid < kDqk / 8)
                *(uint4 *)(kd + tid * 8) = *(const uint4 *)(ks + tid * 8);
            else if (tid < kDqk / 8 + kDv / 8)
                *(uint4 *)(vd + (tid - kDqk / 8) * 8) = *(const uint4 *)(vs + (tid - kDqk / 8) * 8);
        }
    }

    // Q^T operands; column cb*32 + r is (token t, head) = divmod(column, group).
    bf16x8 qf[NCB][kDqk / 16];
    int qpos[NCB];
    {
        const BufRsrc qb = make_buf((const uint16_t *)a.q + (size_t)c.b * nq * a.Hq * kDqk,
                                    (uint64_t)nq * a.Hq * kDqk * 2);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int col = cb * 32 + r;
            const bool ok = col < n_cols;
            const int t = col / group;
            qpos[cb] = ok ? c.P + t : -1;
            const uint32_t off = ok ? ((uint32_t)(t * a.Hq + c.g * group + col % group) * kDqk +
                                       (uint32_t)hh * 8) * 2
                                    : kOob;
#pragma unroll
            for (int s = 0; s < kDqk / 16; ++s)
                qf[cb][s] = as_bf16x8(buf_load16(qb, off + (uint32_t)s * 32));
            if (kRope && ok) {  // dims 16s + 8hh .. +7 (s < 4): pairs 8s + 4hh ..
                const float2 *cs = rope_tab + t * 32 + 4 * hh;
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    qf[cb][s] = as_bf16x8(rope_chunk_bf16(as_uint4(qf[cb][s]), cs + 8 * s));
            }
        }
    }

    float m[NCB], l[NCB];
    f32x16 acc[NCB][4];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        m[cb] = -INFINITY;
        l[cb] = 0.f;
#pragma unroll
        for (int db = 0; db < 4; ++db)
            acc[cb][db] = f32x16{};
    }

    // Blocks: cached keys [rlo, ce) in blocks of 32, then (if this chunk holds
    // them) the new tokens [max(rlo, P), rhi) as one more block.
    const int ce = min(c.rhi, c.P);
    const int n_cache_blk = ce > c.rlo ? (ce - c.rlo + kKb - 1) / kKb : 0;
    const int new_lo = max(c.rlo, c.P);
    const int nblk = n_cache_blk + (c.rhi > new_lo ? 1 : 0);
    const int window = a.window;
    const uint32_t krow = (uint32_t)Hkv * kDqk * 2, vrow = (uint32_t)Hkv * kDv * 2;
    const int kr_key = key_of_row(r);

    auto block_base = [&](int j) { return j < n_cache_blk ? c.rlo + j * kKb : new_lo; };
    auto load_kv = [&](int j, KVRegs &x) {
        const int kb = block_base(j);
        if (j < n_cache_blk) {  // wave-uniform
            const int p = kb + kr_key;
            const int slot = a.ring ? p % a.cap : p;
            const uint32_t off = p < ce ? (uint32_t)slot * kDqk * 2 + (uint32_t)hh * 16 : kOob;
#pragma unroll
            for (int s = 0; s < kDqk / 16; ++s)
                x.k[s] = buf_load16(kc, off + (uint32_t)s * 32);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int pv = kb + 16 * hh + i;
                const int sv = a.ring ? pv % a.cap : pv;
                const uint32_t ov = pv < ce ? (uint32_t)sv * kDv * 2 + (uint32_t)r * 8 : kOob;
                x.v[i] = buf_load8(vc, ov);
            }
        } else {
            const int p = kb + kr_key;
            const uint32_t off = p < c.rhi ? (uint32_t)(p - c.P) * krow + (uint32_t)hh * 16 : kOob;
#pragma unroll
            for (int s = 0; s < kDqk / 16; ++s)
                x.k[s] = buf_load16(kn, off + (uint32_t)s * 32);
            if (kRope && p < c.rhi) {
                const float2 *cs = rope_tab + (p - c.P) * 32 + 4 * hh;
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    x.k[s] = rope_chunk_bf16(x.k[s], cs + 8 * s);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int pv = kb + 16 * hh + i;
                const uint32_t ov = pv < c.rhi ? (uint32_t)(pv - c.P) * vrow + (uint32_t)r * 8 : kOob;
                x.v[i] = buf_load8(vn, ov);
            }
        }
    };
    auto compute = [&](int j, const KVRegs &x) {
        const int kb = block_base(j);
        const int kend = j < n_cache_blk ? ce : c.rhi;
        f32x16 sc[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
            sc[cb] = f32x16{};
#pragma unroll
        for (int s = 0; s < kDqk / 16; ++s)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
                sc[cb] = mfma32x32x16(as_bf16x8(x.k[s]), qf[cb][s], sc[cb]);

        // V^T operands: block db (dims 4*row + db), k-step t (keys 16hh + 8t + e).
        bf16x8 va[4][2];
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                uint32_t w[4];
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const uint2 lo = x.v[8 * t + 2 * e2], hi = x.v[8 * t + 2 * e2 + 1];
                    const uint32_t wl = (db < 2) ? lo.x : lo.y;
                    const uint32_t wh = (db < 2) ? hi.x : hi.y;
                    w[e2] = (db & 1) ? __builtin_amdgcn_perm(wh, wl, 0x07060302u)
                                     : __builtin_amdgcn_perm(wh, wl, 0x05040100u);
                }
                va[db][t] = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
            }

        // Cached blocks are fully visible unless they cut the range end or the
        // window start of a later query; the new-token block is causal.
        const bool full = j < n_cache_blk && kb + kKb <= ce &&
                          (window <= 0 || kb >= c.P + nq - window);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int qp = qpos[cb];
            if (!full) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int p = kb + 16 * hh + i;
                    const bool vis = p < kend && p <= qp && (window <= 0 || qp - p < window);
                    sc[cb][i] = vis ? sc[cb][i] : -INFINITY;
                }
            }
            if (qp < 0) {  // padding column (only in the last column block)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    sc[cb][i] = -INFINITY;
            }
            float bm = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                bm = fmaxf(bm, sc[cb][i]);
            bm = max_across_halves(bm) * scale_log2;
            const bool up = bm > m[cb] + kRescaleSlack || (m[cb] == -INFINITY && bm > -INFINITY);
            const float mn = up ? bm : m[cb];
            const float alpha = up ? fast_exp2(m[cb] - mn) : 1.f;
            m[cb] = mn;
            const float mu = (mn == -INFINITY) ? 0.f : mn;
            float ps = 0.f;
            bf16x8 pb[2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float pr = fast_exp2(__fmaf_rn(sc[cb][i], scale_log2, -mu));
                ps += pr;
                pb[i >> 3][i & 7] = (__bf16)pr;
            }
            l[cb] = __fmaf_rn(l[cb], alpha, ps);
            if (__builtin_amdgcn_ballot_w64(up) != 0) {
#pragma unroll
                for (int db = 0; db < 4; ++db)
                    acc[cb][db] *= alpha;
            }
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    acc[cb][db] = mfma32x32x16(va[db][t], pb[t], acc[cb][db]);
        }
    };

    // Blocks j = wave, wave+4, ...  With one column block, two register sets keep
    // the loads of a wave's next block in flight while it computes the current
    // one; with two column blocks the registers only hold one set.
    if constexpr (NCB == 1) {
        KVRegs x0, x1;
        int j = wave;
        if (j < nblk)
            load_kv(j, x0);
        for (; j < nblk; j += 2 * kWaves) {
            if (j + kWaves < nblk)
                load_kv(j + kWaves, x1);
            compute(j, x0);
            if (j + kWaves < nblk) {
                if (j + 2 * kWaves < nblk)
                    load_kv(j + 2 * kWaves, x0);
                compute(j + kWaves, x1);
            }
        }
    } else {
        for (int j = wave; j < nblk; j += kWaves) {
            KVRegs x;
            load_kv(j, x);
            compute(j, x);
        }
    }

    // Merge the 4 waves' states, one column block at a time: waves 1..3 park
    // (acc, m, l) in LDS, wave 0 folds them into its registers and writes.
    const bool write_final = a.n_splits == 1;
    const size_t rows_total = (size_t)a.B * nq * a.Hq;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int ncol = min(32, n_cols - cb * 32);
        if (ncol <= 0)
            break;
        const float lt = sum_across_halves(l[cb]);
        if (wave > 0 && r < ncol) {
            float *e = &merge[wave - 1][r][0];
            if (hh == 0) {
                e[kDv] = m[cb];
                e[kDv + 1] = lt;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float4 v4 = make_float4(acc[cb][0][i], acc[cb][1][i], acc[cb][2][i],
                                              acc[cb][3][i]);
                *(float4 *)&e[4 * c_row(i, hh)] = v4;
            }
        }
        __syncthreads();
        if (wave == 0 && r < ncol) {
            const int col = cb * 32 + r;
            const int t = col / group;
            const int h = c.g * group + col % group;
            const size_t row = ((size_t)c.b * nq + t) * a.Hq + h;
            float mx = m[cb];
#pragma unroll
            for (int w = 0; w < kWaves - 1; ++w)
                mx = fmaxf(mx, merge[w][r][kDv]);
            float M = mx, zs = 0.f;
            if (write_final) {
                const float sink2 = a.sink[h] * kLog2e;
                M = fmaxf(mx, sink2);
                zs = (sink2 == -INFINITY || M == -INFINITY) ? 0.f : fast_exp2(sink2 - M);
            }
            const float f0 = (m[cb] == -INFINITY) ? 0.f : fast_exp2(m[cb] - M);
            float fw[kWaves - 1];
            float z = zs + lt * f0;
#pragma unroll
            for (int w = 0; w < kWaves - 1; ++w) {
                const float mw = merge[w][r][kDv];
                fw[w] = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
                z += merge[w][r][kDv + 1] * fw[w];
            }
            const float scale_out = write_final ? (z > 0.f ? 1.f / z : 0.f) : 1.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int d0 = 4 * c_row(i, hh);  // dims d0 .. d0+3 (blocks 0..3)
                float vals[4];
#pragma unroll
                for (int db = 0; db < 4; ++db)
                    vals[db] = acc[cb][db][i] * f0;
#pragma unroll
                for (int w = 0; w < kWaves - 1; ++w) {
                    const float4 p4 = *(const float4 *)&merge[w][r][d0];
                    vals[0] += p4.x * fw[w];
                    vals[1] += p4.y * fw[w];
                    vals[2] += p4.z * fw[w];
                    vals[3] += p4.w * fw[w];
                }
                if (write_final) {
                    uint2 u;
                    u.x = pack_bf16x2(vals[0] * scale_out, vals[1] * scale_out);
                    u.y = pack_bf16x2(vals[2] * scale_out, vals[3] * scale_out);
                    *(uint2 *)((uint16_t *)a.o + row * kDv + d0) = u;
                } else {
                    const size_t slot = row * a.n_splits + split;
                    *(float4 *)&a.ws[2 * rows_total * a.n_splits + slot * kDv + d0] =
                        make_float4(vals[0], vals[1], vals[2], vals[3]);
                }
            }
            if (!write_final && hh == 0) {
                const size_t slot = row * a.n_splits + split;
                a.ws[slot] = M;
                a.ws[rows_total * a.n_splits + slot] = (M == -INFINITY) ? 0.f : z;
            }
        }
        __syncthreads();
    }
}

// Split-K combine: one wave per (b, t, h) row; adds the sink exactly once.
__global__ __launch_bounds__(64) void combine_kernel(CachedArgs a, int out_bf16) {
    const int row = blockIdx.x;  // ((b * nq) + t) * Hq + h
    const int lane = threadIdx.x;
    const int h = row % a.Hq;
    const int b = row / (a.nq * a.Hq);
    const int S = a.n_splits;
    const size_t rows_total = (size_t)a.B * a.nq * a.Hq;
    const float *wm = a.ws + (size_t)row * S;
    const float *wl = a.ws + rows_total * S + (size_t)row * S;
    const float *wa = a.ws + 2 * rows_total * S + (size_t)row * S * kDv;
    const int P = clamp_len(a.cache_len[b], a.max_len);
    const int lo = a.window > 0 ? max(0, P - a.window + 1) : 0;
    const int hi = P + a.nq;
    const int s0 = lo / a.chunk;
    const int s1 = min(S, (hi + a.chunk - 1) / a.chunk);

    const float sink2 = a.sink[h] * kLog2e;
    float mx = sink2;
    for (int s = s0 + lane; s < s1; s += 64)
        mx = fmaxf(mx, wm[s]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    float z = 0.f, acc0 = 0.f, acc1 = 0.f;
    if (mx != -INFINITY) {
        z = (sink2 == -INFINITY) ? 0.f : fast_exp2(sink2 - mx);
        // Splits in groups of kGroup: all loads of a group are issued before
        // any is used (indices past the last split repeat it and get weight
        // 0), so a row waits for one memory latency per group, not per split.
        constexpr int kGroup = 8;
        for (int s = s0; s < s1; s += kGroup) {
            float ms[kGroup], ls[kGroup], a0[kGroup], a1[kGroup];
#pragma unroll
            for (int j = 0; j < kGroup; ++j) {
                const int sj = min(s + j, s1 - 1);
                ms[j] = wm[sj];
                ls[j] = wl[sj];
                a0[j] = wa[(size_t)sj * kDv + lane];
                a1[j] = wa[(size_t)sj * kDv + 64 + lane];
            }
#pragma unroll
            for (int j = 0; j < kGroup; ++j) {
                const float f =
                    (s + j >= s1 || ms[j] == -INFINITY) ? 0.f : fast_exp2(ms[j] - mx);
                z += ls[j] * f;
                acc0 += a0[j] * f;
                acc1 += a1[j] * f;
            }
        }
    }
    const float inv = z > 0.f ? 1.f / z : 0.f;
    if (out_bf16) {
        uint16_t *o = (uint16_t *)a.o + (size_t)row * kDv;
        o[lane] = f32_to_bf16_bits(acc0 * inv);
        o[64 + lane] = f32_to_bf16_bits(acc1 * inv);
    } else {
        float *o = (float *)a.o + (size_t)row * kDv;
        o[lane] = acc0 * inv;
        o[64 + lane] = acc1 * inv;
    }
}

// After a commit: cache_len[b] += the number of tokens kv_append stored for b.
__global__ void advance_len_kernel(int32_t *cache_len, const int32_t *n_accept, int B, int n) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B)
        cache_len[b] += n_accept ? min(n, max(0, n_accept[b])) : n;
}

// Commit accepted tokens: one thread per 16-byte piece of a K or V row.
__global__ void append_kernel(AppendArgs a, int row_bytes_k, int row_bytes_v) {
    const int pk = row_bytes_k / 16, pv = row_bytes_v / 16;
    const int per_tok = (pk + pv) * a.Hkv;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)a.B * a.n * per_tok;
    if (idx >= total)
        return;
    const int b = (int)(idx / ((size_t)a.n * per_tok));
    const int rem = (int)(idx % ((size_t)a.n * per_tok));
    const int t = rem / per_tok;
    const int rr = rem % per_tok;
    const int g = rr / (pk + pv);
    const int piece = rr % (pk + pv);
    const int nacc = a.n_accept ? min(a.n, max(0, a.n_accept[b])) : a.n;
    if (t >= nacc)
        return;
    const int p = max(0, a.cache_len[b]) + t;
    int slot;
    if (a.ring) {
        if (t < nacc - a.cap)  // a later token of this call takes the same slot
            return;
        slot = p % a.cap;
    } else {
        if (p >= a.cap)
            return;
        slot = p;
    }
    const size_t crow = ((size_t)b * a.Hkv + g) * a.cap + slot;
    const size_t nrow = ((size_t)b * a.n + t) * a.Hkv + g;
    const bool is_k = piece < pk;
    const int pc = is_k ? piece : piece - pk;
    const int rb = is_k ? row_bytes_k : row_bytes_v;
    const uint4 x = *(const uint4 *)((const char *)(is_k ? a.k_new : a.v_new) + nrow * rb + pc * 16);
    if (a.fp8) {  // 8 bf16 -> 8 E4M3 codes of x / scale; cache rows are 1 byte per dim
        char *dst = (char *)(is_k ? a.k_cache : a.v_cache) + crow * (rb / 2) + pc * 8;
        *(uint2 *)dst = bf16x8_to_e4m3x8(x, is_k ? a.k_scale : a.v_scale);
    } else {
        char *dst = (char *)(is_k ? a.k_cache : a.v_cache) + crow * rb + pc * 16;
        *(uint4 *)dst = x;
    }
}

}  // namespace

hipError_t launch_cached_bf16(const CachedArgs &a, hipStream_t s) {
    const int n_cols = a.nq * (a.Hq / a.Hkv);
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    const dim3 grid((unsigned)(a.B * a.Hkv * a.n_splits)), block(kThreads);
    // <= 16 columns, or a short window (each workgroup's key range is a few
    // blocks, so streaming it once per 16-column wave costs little), or E4M3
    // caches: the 16-column kernel; more columns over a whole contiguous cache:
    // the kernel that stages the K/V blocks in LDS for four 16-column waves
    // (measured 16% faster than the 32x32 kernel at 64 columns, 2.5% at 32);
    // otherwise (windows past 4096 keys) the 32-column kernel, whose waves split
    // the key blocks.
    if (a.fp8 || n_cols <= 16 || (a.window > 0 && a.window <= 4096)) {
        const hipError_t e16 = launch_decode16(a, s);
        if (e16 != hipSuccess)
            return e16;
    } else if (!a.ring && a.window <= 0) {
        const hipError_t el = launch_verify_lds(a, s);
        if (el != hipSuccess)
            return el;
    } else if (n_cols <= 32) {
        if (a.rope)
            cached_bf16_kernel<1, true><<<grid, block, 0, s>>>(a, scale_log2);
        else
            cached_bf16_kernel<1, false><<<grid, block, 0, s>>>(a, scale_log2);
    } else {
        if (a.rope)
            cached_bf16_kernel<2, true><<<grid, block, 0, s>>>(a, scale_log2);
        else
            cached_bf16_kernel<2, false><<<grid, block, 0, s>>>(a, scale_log2);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_splits == 1)
        return e;
    combine_kernel<<<dim3((unsigned)(a.B * a.nq * a.Hq)), dim3(64), 0, s>>>(a, 1);
    return hipGetLastError();
}

hipError_t launch_append(const AppendArgs &a, int bf16, hipStream_t s) {
    const int esz = bf16 ? 2 : 4;
    const int rbk = kDqk * esz, rbv = kDv * esz;
    const size_t total = (size_t)a.B * a.n * a.Hkv * ((rbk + rbv) / 16);
    if (total == 0)
        return hipSuccess;
    const unsigned blocks = (unsigned)((total + 255) / 256);
    append_kernel<<<dim3(blocks), dim3(256), 0, s>>>(a, rbk, rbv);
    return hipGetLastError();
}

hipError_t launch_advance_len(int32_t *cache_len, const int32_t *n_accept, int B, int n,
                              hipStream_t s) {
    if (B == 0)
        return hipSuccess;
    advance_len_kernel<<<dim3((unsigned)((B + 255) / 256)), dim3(256), 0, s>>>(cache_len,
                                                                              n_accept, B, n);
    return hipGetLastError();
}

}  // namespace sinkattn

// prefill.hip -- causal sink-attention prefill on gfx950 (bf16 in, fp32 accumulate):
// global-attention layers, and sliding windows wider than the persistent SWA
// kernel holds (W > 129).
//
// Computes, for every query token i of a sequence and every query head h
// (MiMo-V2-Flash Technical Report, Section 2.2, equations 1-4):
//   a_ij = q_i . k_j * scale,  m_i = max(max_j a_ij, sink_h),
//   o_i  = sum_j exp(a_ij - m_i) v_j / (exp(sink_h - m_i) + sum_j exp(a_ij - m_i))
// over the visible keys j <= i (and i - j < W for a windowed layer).
//
// The softmax is evaluated online, flash style, with the running state seeded
// by the sink: m <- sink, l <- 1 (l <- 0 when sink = -inf), acc <- 0.  That makes
// the sink term exact and counted once, with no extra pass.
//
// Work decomposition (one workgroup = 8 waves):
//   - a workgroup owns one KV group g (Table 1: 16 query heads per KV head for
//     global layers, handled as two workgroups of 8) and a tile of 32
//     consecutive query tokens; wave w owns query head 8*part + w;
//   - the 32 tokens are the 32 MFMA columns; Q stays in registers for the
//     whole tile (12 k-steps of 16 dims);
//   - keys stream in blocks of 32 through two LDS stages; every block is
//     fetched once per workgroup and read by all 8 heads; the global loads of
//     block j+2 are issued while block j is computed (two register sets), so
//     about two blocks of compute cover the memory latency;
//   - scores are computed transposed, S^T = K Q^T (rows = keys, columns =
//     queries), so each lane owns one query column and the row max / sum are
//     per-lane register reductions plus one exchange between wave halves;
//   - K rows are written into LDS in the order that makes C-register i of lane
//     half hh hold key 16*hh + i, so P^T feeds the PV MFMA directly as its B
//     operand; V rows stay row-major in LDS (one 16-byte write per piece) and
//     the V^T A operand is read with gfx950's transposing LDS loads (two
//     ds_read_b64_tr_b16 per MFMA); this replaced a transposed V^T tile built
//     with 8 scattered 2-byte writes per piece (3-5% of the kernel).
// Global memory is read through raw buffer descriptors (rows past the end of
// the sequence read as zero; stores past it are dropped).
// Workgroup order: blockIdx % units picks (batch, KV group, head half), so on
// the 8 XCDs of MI355X each XCD sees tiles of the same KV group and the shared
// K/V blocks hit in its L2.  Global layers run the longest (last) tiles first.
#include "common.h"
#include "lds_tr.h"

namespace sinkattn {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kTq = 32;             // query tokens per tile (MFMA columns)
constexpr int kKb = 32;             // keys per block (MFMA rows)
constexpr int kKPitch = kDqk + 8;   // LDS row pitch of K, bf16 elements (400 bytes)
constexpr int kVPitch = kDv + 8;    // LDS row pitch of V rows, bf16 elements (272 bytes)
constexpr int kKChunks = kKb * kDqk / 8;   // 16-byte pieces of one K block (768)
constexpr int kVChunks = kKb * kDv / 8;    // 16-byte pieces of one V block (512)
static_assert(kVChunks == kThreads, "one V piece per thread");

struct PrefillSmem {
    uint16_t k[2][kKb * kKPitch];
    uint16_t v[2][kKb * kVPitch];
};

// PV accumulator block db, C-row rho = 8a + 4hh + e holds output dim
// 32a + 16(db/2) + 8hh + 4(db%2) + e, so a lane owns runs of 8 consecutive output
// dims (16-byte stores); the transposing V reads below pick their dims to match.

struct Staged {
    uint4 k[2];
    uint4 v;
};

template <bool kWindowed, bool kRopeQ>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(PrefillArgs a, int n_units,
                                                                 int n_tiles, float scale_log2) {
    __shared__ PrefillSmem sm;
    __shared__ float2 rope_tab[kRopeQ ? kTq * 32 : 1];
    const int T = a.T, Hq = a.Hq, Hkv = a.Hkv, window = a.window;
    const int group = Hq / Hkv;
    const int parts = group / kWaves;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 31, hh = lane >> 5;

    const int unit = blockIdx.x % n_units;
    const int tix = blockIdx.x / n_units;
    const int tile = kWindowed ? tix : (n_tiles - 1 - tix);
    const int part = unit % parts;
    const int g = (unit / parts) % Hkv;
    const int b = unit / (parts * Hkv);
    const int h = g * group + part * kWaves + wave;
    const int t0 = tile * kTq;
    const int query = t0 + r;  // this lane's query column

    const size_t row0 = (size_t)b * T;
    const uint32_t qrow = (uint32_t)Hq * kDqk * 2, orow = (uint32_t)Hq * kDv * 2;
    const uint32_t krow = (uint32_t)Hkv * kDqk * 2, vrow = (uint32_t)Hkv * kDv * 2;
    const BufRsrc qbuf = make_buf((const uint16_t *)a.q + row0 * Hq * kDqk, (uint64_t)T * qrow);
    const BufRsrc kbuf = make_buf((const uint16_t *)a.k + row0 * Hkv * kDqk, (uint64_t)T * krow);
    const BufRsrc vbuf = make_buf((const uint16_t *)a.v + row0 * Hkv * kDv, (uint64_t)T * vrow);
    const BufRsrc obuf = make_buf((uint16_t *)a.o + row0 * Hq * kDv, (uint64_t)T * orow);
    const uint32_t kcol = (uint32_t)g * kDqk * 2, vcol = (uint32_t)g * kDv * 2;

    // Partial RoPE of q on load (fused variant): (cos, sin) of the tile's 32
    // positions, computed once per workgroup.
    if constexpr (kRopeQ) {
        rope_fill_table64(rope_tab, t0, kTq, a.rope_base, tid, kThreads);
        __syncthreads();
    }

    // Q^T as the B operand: k-step s, lane half hh -> head dims (2s+hh)*8 .. +7.
    uint4 qf[kDqk / 16];
    {
        const uint32_t off = (uint32_t)query * qrow + (uint32_t)h * kDqk * 2 + (uint32_t)hh * 16;
#pragma unroll
        for (int s = 0; s < kDqk / 16; ++s)
            qf[s] = buf_load16(qbuf, off + (uint32_t)s * 32);
        if constexpr (kRopeQ) {  // dims 16s + 8hh .. +7 (s < 4): pairs 8s + 4hh ..
            const float2 *cs = rope_tab + r * 32 + 4 * hh;
#pragma unroll
            for (int s = 0; s < 4; ++s)
                qf[s] = rope_chunk_bf16(qf[s], cs + 8 * s);
        }
    }

    const int kstart = kWindowed ? max(0, t0 - window + 1) : 0;
    const int kend = min(T, t0 + kTq);
    const int kb0 = kstart & ~(kKb - 1);
    const int nblk = (kend - kb0 + kKb - 1) / kKb;

    // Per-thread staging offsets, computed once: K pieces c = tid, tid + 512 (key c/24,
    // dims (c%24)*8..+7); V piece tid (key tid/16, dims (tid%16)*8..+7).
    const bool k2 = tid + kThreads < kKChunks;  // wave-uniform
    uint32_t kg_off[2];
    int kl_off[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int c = min(tid + u * kThreads, kKChunks - 1);
        kg_off[u] = (uint32_t)(c / (kDqk / 8)) * krow + kcol + (uint32_t)(c % (kDqk / 8)) * 16;
        kl_off[u] = row_of_key(c / (kDqk / 8)) * kKPitch + (c % (kDqk / 8)) * 8;
    }
    const int v_kk = tid >> 4, v_dc = tid & 15;  // V rows stay row-major in LDS
    const uint32_t vg_off = (uint32_t)v_kk * vrow + vcol + (uint32_t)v_dc * 16;
    const int vl_off = v_kk * kVPitch + v_dc * 8;
    // V^T operand of the PV product read from the row-major V tile with transposing
    // loads: in group G = lane/16, source lane 4e'+q points at key 16hh + 8t + 4L + e'
    // and dims d0 = 64(G%2) + 32(q/2) + 16(db/2) + 8(q%2) + 4(db%2), so A-row r holds
    // dim pv_dim(r) (runs of 8 consecutive output dims per lane, as before).
    const int vt_lane = (16 * hh + ((lane & 15) >> 2)) * kVPitch + 64 * ((lane >> 4) & 1) +
                        32 * ((lane & 3) >> 1) + 8 * (lane & 1);

    auto load_block = [&](int kb, Staged &st) {
        st.k[0] = buf_load16(kbuf, (uint32_t)kb * krow + kg_off[0]);
        if (k2)
            st.k[1] = buf_load16(kbuf, (uint32_t)kb * krow + kg_off[1]);
        st.v = buf_load16(vbuf, (uint32_t)kb * vrow + vg_off);
    };
    auto store_block = [&](int buf, const Staged &st) {
        *(uint4 *)&sm.k[buf][kl_off[0]] = st.k[0];
        if (k2)
            *(uint4 *)&sm.k[buf][kl_off[1]] = st.k[1];
        *(uint4 *)&sm.v[buf][vl_off] = st.v;
    };

    // Online-softmax state in log2 units, seeded with the sink.
    const float sink2 = a.sink[h] * kLog2e;
    float m = sink2;
    float l = (hh == 0 && sink2 != -INFINITY) ? 1.f : 0.f;  // the sink counted once per column
    f32x16 acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
        acc[db] = f32x16{};

    // pipeline: block j computed from LDS stage j&1; block j+1 stored at the end of
    // block j from register set (j+1)&1; block j+2 loaded at the start of block j.
    // The loop is unrolled by two so the two register sets are named statically
    // (a runtime-indexed register array would live in scratch memory).
    Staged st0, st1;
    load_block(kb0, st0);
    if (nblk > 1)
        load_block(kb0 + kKb, st1);
    store_block(0, st0);
    __syncthreads();

    auto step = [&](int j, Staged &cur_next2, Staged &next1) {
        // cur_next2: the set that held block j, refilled with block j+2;
        // next1: the set holding block j+1, stored into LDS at the end.
        const int kb = kb0 + j * kKb;
        if (j + 2 < nblk)
            load_block(kb + 2 * kKb, cur_next2);
        const uint16_t *ks = sm.k[j & 1];
        const uint16_t *vs = sm.v[j & 1];

        // S^T = K Q^T: rows = keys (permuted so register i <-> key 16*hh + i).  The K
        // operands are read in two groups of six, the second group's reads issued
        // before the first group's products (one LDS latency per group).
        f32x16 sc = f32x16{};
        {
            uint4 ka[kDqk / 16];
#pragma unroll
            for (int s = 0; s < 6; ++s)
                ka[s] = *(const uint4 *)(ks + r * kKPitch + (2 * s + hh) * 8);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 6; s < 12; ++s)
                ka[s] = *(const uint4 *)(ks + r * kKPitch + (2 * s + hh) * 8);
#pragma unroll
            for (int s = 0; s < 6; ++s)
                sc = mfma32x32x16(as_bf16x8(ka[s]), as_bf16x8(qf[s]), sc);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 6; s < 12; ++s)
                sc = mfma32x32x16(as_bf16x8(ka[s]), as_bf16x8(qf[s]), sc);
        }

        // The V^T operand reads of the PV product are issued here, ahead of the
        // softmax, so their LDS latency overlaps its VALU work (3% faster than
        // issuing them with the products).
        uint4 vpre[4][2];
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const uint16_t *vp = vs + vt_lane + 8 * t * kVPitch + 16 * (db >> 1) + 4 * (db & 1);
                const uint2 lo = lds_tr16(vp), hi = lds_tr16(vp + 4 * kVPitch);
                vpre[db][t] = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }
        // Only blocks on the causal diagonal or the window edge need the per-element
        // mask; the test is uniform, so the mask sits behind a scalar branch.
        const bool full = (kb + kKb - 1 <= t0) && (!kWindowed || (t0 + kTq - 1 - kb < window));
        if (!full) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = kb + 16 * hh + i;
                const bool vis = key <= query && (!kWindowed || query - key < window);
                sc[i] = vis ? sc[i] : -INFINITY;
            }
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

        // O^T += V^T P^T: A = V^T rows (dims) from LDS, B = P^T from registers.
        {
            uint4(&va)[4][2] = vpre;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    acc[db] = mfma32x32x16(as_bf16x8(va[db][t]), pb[t], acc[db]);
        }

        if (j + 1 < nblk)
            store_block((j + 1) & 1, next1);
        __syncthreads();
    };
    for (int j = 0; j < nblk; j += 2) {
        step(j, st0, st1);
        if (j + 1 < nblk)
            step(j + 1, st1, st0);
    }

    // Epilogue: o = acc / l, with l summed over both wave halves.
    const float lt = sum_across_halves(l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const uint32_t obase = (uint32_t)query * orow + (uint32_t)h * kDv * 2 + (uint32_t)hh * 16;
#pragma unroll
    for (int aa = 0; aa < 4; ++aa)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const f32x16 &lo = acc[2 * jj], &hi = acc[2 * jj + 1];
            uint4 w;
            w.x = pack_bf16x2(lo[4 * aa + 0] * inv, lo[4 * aa + 1] * inv);
            w.y = pack_bf16x2(lo[4 * aa + 2] * inv, lo[4 * aa + 3] * inv);
            w.z = pack_bf16x2(hi[4 * aa + 0] * inv, hi[4 * aa + 1] * inv);
            w.w = pack_bf16x2(hi[4 * aa + 2] * inv, hi[4 * aa + 3] * inv);
            buf_store16(obuf, obase + (uint32_t)(64 * aa + 32 * jj), w);
        }
    if (a.lse && hh == 0 && query < T) {
        const float mu = (m == -INFINITY) ? 0.f : m;
        a.lse[((size_t)b * Hq + h) * T + query] = lt > 0.f ? (mu + log2f(lt)) * kLn2 : -INFINITY;
    }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs &a, hipStream_t s) {
    const int group = a.Hq / a.Hkv;
    const int parts = group / kWaves;
    const int n_units = a.B * a.Hkv * parts;
    const int n_tiles = (a.T + kTq - 1) / kTq;
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    const dim3 grid((unsigned)(n_units * n_tiles)), block(kThreads);
    if (a.window > 0)
        prefill_bf16_kernel<true, false><<<grid, block, 0, s>>>(a, n_units, n_tiles, scale_log2);
    else if (a.rope_q)
        prefill_bf16_kernel<false, true><<<grid, block, 0, s>>>(a, n_units, n_tiles, scale_log2);
    else
        prefill_bf16_kernel<false, false><<<grid, block, 0, s>>>(a, n_units, n_tiles, scale_log2);
    return hipGetLastError();
}

}  // namespace sinkattn

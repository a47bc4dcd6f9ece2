// prefill.hip -- causal sink-attention prefill on gfx950 (bf16 in, fp32 accumulate).
//
// Computes, for every query token i of a sequence and every query head h
// (MiMo-V2-Flash Technical Report, Section 2.2, equations 1-4):
//   a_ij = q_i . k_j * scale,  m_i = max(max_j a_ij, sink_h),
//   o_i  = sum_j exp(a_ij - m_i) v_j / (exp(sink_h - m_i) + sum_j exp(a_ij - m_i))
// over the visible keys j <= i (and i - j < W for a sliding-window layer).
//
// The softmax is evaluated online, flash style, with the running state seeded
// by the sink: m <- sink, l <- 1 (l <- 0 when sink = -inf), acc <- 0.  That makes
// the sink term exact and counted once, with no extra pass.
//
// Work decomposition (one workgroup = 8 waves):
//   - a workgroup owns one KV group g (Table 1: 8 query heads per KV head for
//     SWA layers, 16 for global layers, handled as two workgroups of 8) and a
//     tile of 32 consecutive query tokens; wave w owns query head 8*part + w;
//   - the 32 tokens are the 32 MFMA columns; Q stays in registers for the
//     whole tile (12 k-steps of 16 dims);
//   - keys stream through LDS in blocks of 32, double buffered: every K/V
//     block is fetched from memory once per workgroup and read by all 8 heads;
//   - scores are computed transposed, S^T = K Q^T (rows = keys, columns =
//     queries), so each lane owns one query column and the row max / sum are
//     per-lane register reductions plus one exchange between wave halves;
//   - K rows are written into LDS in the order that makes C-register i of lane
//     half hh hold key 16*hh + i, so P^T feeds the PV MFMA directly as its B
//     operand and V is stored transposed ([dim][key]) so its A operand is one
//     16-byte LDS read per lane.
// Workgroup order: blockIdx % units picks (batch, KV group, head half), so on
// the 8 XCDs of MI355X each XCD sees consecutive tiles of the same KV group and
// the overlapping K/V windows hit in its L2.  Global layers run the longest
// (last) tiles first.
#include "common.h"

namespace sinkattn {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kTq = 32;             // query tokens per tile (MFMA columns)
constexpr int kKb = 32;             // keys per block (MFMA rows)
constexpr int kKPitch = kDqk + 8;   // LDS row pitch of K, bf16 elements (400 bytes)
constexpr int kVPitch = kKb + 8;    // LDS row pitch of V^T, bf16 elements (80 bytes)
constexpr int kKChunks = kKb * kDqk / 8;   // 16-byte pieces of one K block (768)
constexpr int kVChunks = kKb * kDv / 8;    // 16-byte pieces of one V block (512)
static_assert(kVChunks == kThreads, "one V piece per thread");

struct PrefillSmem {
    uint16_t k[2][kKb * kKPitch];
    uint16_t vt[2][kDv * kVPitch];
};

template <bool kWindowed>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(PrefillArgs a, int n_units,
                                                                 int n_tiles, float scale_log2) {
    __shared__ PrefillSmem sm;
    const uint16_t *__restrict__ q = (const uint16_t *)a.q;
    const uint16_t *__restrict__ k = (const uint16_t *)a.k;
    const uint16_t *__restrict__ v = (const uint16_t *)a.v;
    uint16_t *__restrict__ o = (uint16_t *)a.o;
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

    // Q^T as the B operand: k-step s, lane half hh -> head dims (2s+hh)*8 .. +7.
    bf16x8 qf[kDqk / 16];
    {
        const bool ok = query < T;
        const uint16_t *qrow = q + ((size_t)(b * T + (ok ? query : 0)) * Hq + h) * kDqk;
#pragma unroll
        for (int s = 0; s < kDqk / 16; ++s) {
            uint4 u = ok ? *(const uint4 *)(qrow + (2 * s + hh) * 8) : make_uint4(0, 0, 0, 0);
            qf[s] = as_bf16x8(u);
        }
    }

    const int kstart = kWindowed ? max(0, t0 - window + 1) : 0;
    const int kend = min(T, t0 + kTq);
    const int kb0 = kstart & ~(kKb - 1);
    const int nblk = (kend - kb0 + kKb - 1) / kKb;

    const size_t krow_stride = (size_t)Hkv * kDqk;
    const size_t vrow_stride = (size_t)Hkv * kDv;
    const uint16_t *kbase = k + (size_t)b * T * krow_stride + (size_t)g * kDqk;
    const uint16_t *vbase = v + (size_t)b * T * vrow_stride + (size_t)g * kDv;

    auto load_block = [&](int kb, uint4 (&kreg)[2], uint4 &vreg) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = tid + u * kThreads;
            kreg[u] = make_uint4(0, 0, 0, 0);
            if (c < kKChunks) {
                const int kk = c / (kDqk / 8), d = c % (kDqk / 8);
                const int key = kb + kk;
                if (key < T)
                    kreg[u] = *(const uint4 *)(kbase + (size_t)key * krow_stride + d * 8);
            }
        }
        const int kk = tid / (kDv / 8), dc = tid % (kDv / 8);
        const int key = kb + kk;
        vreg = key < T ? *(const uint4 *)(vbase + (size_t)key * vrow_stride + dc * 8)
                       : make_uint4(0, 0, 0, 0);
    };
    auto store_block = [&](int buf, const uint4 (&kreg)[2], const uint4 &vreg) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = tid + u * kThreads;
            if (c < kKChunks) {
                const int kk = c / (kDqk / 8), d = c % (kDqk / 8);
                *(uint4 *)&sm.k[buf][row_of_key(kk) * kKPitch + d * 8] = kreg[u];
            }
        }
        const int kk = tid / (kDv / 8), dc = tid % (kDv / 8);
        const uint32_t w[4] = {vreg.x, vreg.y, vreg.z, vreg.w};
#pragma unroll
        for (int j = 0; j < 8; ++j)
            sm.vt[buf][(dc * 8 + j) * kVPitch + kk] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
    };

    // Online-softmax state in log2 units, seeded with the sink.
    const float sink2 = a.sink[h] * kLog2e;
    float m = sink2;
    float l = (hh == 0 && sink2 != -INFINITY) ? 1.f : 0.f;  // the sink counted once per column
    f32x16 acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
        acc[db] = f32x16{};

    {
        uint4 kreg[2], vreg;
        load_block(kb0, kreg, vreg);
        store_block(0, kreg, vreg);
    }
    __syncthreads();

    for (int j = 0; j < nblk; ++j) {
        const int kb = kb0 + j * kKb;
        const bool more = j + 1 < nblk;
        uint4 kreg[2], vreg;
        if (more)
            load_block(kb + kKb, kreg, vreg);
        const uint16_t *ks = sm.k[j & 1];
        const uint16_t *vs = sm.vt[j & 1];

        // S^T = K Q^T: rows = keys (permuted so register i <-> key 16*hh + i).
        f32x16 sc = f32x16{};
#pragma unroll
        for (int s = 0; s < kDqk / 16; ++s) {
            const uint4 ka = *(const uint4 *)(ks + r * kKPitch + (2 * s + hh) * 8);
            sc = mfma32x32x16(as_bf16x8(ka), qf[s], sc);
        }

        const bool full = (kb + kKb - 1 <= t0) && (!kWindowed || (t0 + kTq - 1 - kb < window));
        float x[16];
        float bm = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float val = sc[i] * scale_log2;
            if (!full) {
                const int key = kb + 16 * hh + i;
                const bool vis = key <= query && (!kWindowed || query - key < window);
                val = vis ? val : -INFINITY;
            }
            x[i] = val;
            bm = fmaxf(bm, val);
        }
        bm = max_across_halves(bm);
        const float mn = fmaxf(m, bm);
        const float mu = (mn == -INFINITY) ? 0.f : mn;
        const float alpha = fast_exp2(m - mu);
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            x[i] = fast_exp2(x[i] - mu);
            ps += x[i];
        }
        l = l * alpha + ps;
        m = mn;
#pragma unroll
        for (int db = 0; db < 4; ++db)
            acc[db] *= alpha;

        bf16x8 pb[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                pb[t][e] = (__bf16)x[8 * t + e];

        // O^T += V^T P^T: A = V^T rows (dims) from LDS, B = P^T from registers.
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const uint4 va = *(const uint4 *)(vs + (32 * db + r) * kVPitch + 16 * hh + 8 * t);
                acc[db] = mfma32x32x16(as_bf16x8(va), pb[t], acc[db]);
            }

        if (more)
            store_block((j + 1) & 1, kreg, vreg);
        __syncthreads();
    }

    // Epilogue: o = acc / l, with l summed over both wave halves.
    const float lt = sum_across_halves(l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (query < T) {
        uint16_t *orow = o + ((size_t)(b * T + query) * Hq + h) * kDv;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                uint2 w;
                w.x = pack_bf16x2(acc[db][4 * i4 + 0] * inv, acc[db][4 * i4 + 1] * inv);
                w.y = pack_bf16x2(acc[db][4 * i4 + 2] * inv, acc[db][4 * i4 + 3] * inv);
                *(uint2 *)(orow + 32 * db + 8 * i4 + 4 * hh) = w;
            }
        if (a.lse && hh == 0) {
            const float mu = (m == -INFINITY) ? 0.f : m;
            a.lse[((size_t)b * Hq + h) * T + query] = lt > 0.f ? (mu + log2f(lt)) * kLn2 : -INFINITY;
        }
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
        prefill_bf16_kernel<true><<<grid, block, 0, s>>>(a, n_units, n_tiles, scale_log2);
    else
        prefill_bf16_kernel<false><<<grid, block, 0, s>>>(a, n_units, n_tiles, scale_log2);
    return hipGetLastError();
}

}  // namespace sinkattn

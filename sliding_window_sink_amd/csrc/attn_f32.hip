// attn_f32.hip -- fp32 sink attention (prefill, decode, verify) with fp32 arithmetic.
//
// Same operation as the bf16 MFMA kernels (MiMo-V2-Flash Technical Report,
// Section 2.2, equations 1-4), for fp32 inputs, where the product must not be
// rounded through bf16: one wave per (sequence, query token, query head) row,
// lanes split the head dims (3 of the 192 QK dims, 2 of the 128 V dims per
// lane), and the online softmax is seeded with the sink (m <- sink, l <- 1).
// It is a straightforward kernel meant for exactness on small fp32 problems,
// not for throughput.
#include "common.h"

namespace sinkattn {
namespace {

struct RowState {
    float m, l, a0, a1;
};

__device__ __forceinline__ void row_step(RowState &st, float logit2, float v0, float v1) {
    // logit2 is the scaled logit in log2 units; st.m starts at the sink.
    const float mn = fmaxf(st.m, logit2);
    const float mu = (mn == -INFINITY) ? 0.f : mn;
    const float alpha = exp2f(st.m - mu);
    const float p = exp2f(logit2 - mu);
    st.l = st.l * alpha + p;
    st.a0 = st.a0 * alpha + p * v0;
    st.a1 = st.a1 * alpha + p * v1;
    st.m = mn;
}

__device__ __forceinline__ float dot192(const float *q, const float *k, int lane) {
    float s = q[lane] * k[lane] + q[lane + 64] * k[lane + 64] + q[lane + 128] * k[lane + 128];
    return wave_sum(s);
}

// Prefill: row = (b*T + i)*Hq + h.
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillArgs a, float scale_log2) {
    const int lane = threadIdx.x;
    const size_t row = blockIdx.x;
    const int h = (int)(row % a.Hq);
    const int i = (int)((row / a.Hq) % a.T);
    const int b = (int)(row / ((size_t)a.Hq * a.T));
    const int g = h / (a.Hq / a.Hkv);
    const float *q = (const float *)a.q + row * kDqk;
    const float *k = (const float *)a.k + ((size_t)b * a.T * a.Hkv + g) * kDqk;
    const float *v = (const float *)a.v + ((size_t)b * a.T * a.Hkv + g) * kDv;
    const size_t ks = (size_t)a.Hkv * kDqk, vs = (size_t)a.Hkv * kDv;
    const float sink2 = a.sink[h] * kLog2e;
    RowState st{sink2, sink2 == -INFINITY ? 0.f : 1.f, 0.f, 0.f};
    const int lo = a.window > 0 ? max(0, i - a.window + 1) : 0;
    for (int j = lo; j <= i; ++j) {
        const float logit2 = dot192(q, k + j * ks, lane) * scale_log2;
        row_step(st, logit2, v[j * vs + lane], v[j * vs + 64 + lane]);
    }
    const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
    float *o = (float *)a.o + row * kDv;
    o[lane] = st.a0 * inv;
    o[64 + lane] = st.a1 * inv;
    if (a.lse && lane == 0) {
        const float mu = (st.m == -INFINITY) ? 0.f : st.m;
        a.lse[((size_t)b * a.Hq + h) * a.T + i] = st.l > 0.f ? (mu + log2f(st.l)) * kLn2 : -INFINITY;
    }
}

// Decode / verify: row = (b*nq + t)*Hq + h; query position P + t.
__global__ __launch_bounds__(64) void cached_f32_kernel(CachedArgs a, float scale_log2) {
    const int lane = threadIdx.x;
    const size_t row = blockIdx.x;
    const int h = (int)(row % a.Hq);
    const int t = (int)((row / a.Hq) % a.nq);
    const int b = (int)(row / ((size_t)a.Hq * a.nq));
    const int group = a.Hq / a.Hkv;
    const int g = h / group;
    const int P = clamp_len(a.cache_len[b], a.max_len);
    const float *kc = (const float *)a.k_cache + ((size_t)b * a.Hkv + g) * a.cap * kDqk;
    const float *vc = (const float *)a.v_cache + ((size_t)b * a.Hkv + g) * a.cap * kDv;
    const float *kn = (const float *)a.k_new + ((size_t)b * a.nq * a.Hkv + g) * kDqk;
    const float *vn = (const float *)a.v_new + ((size_t)b * a.nq * a.Hkv + g) * kDv;
    const size_t kns = (size_t)a.Hkv * kDqk, vns = (size_t)a.Hkv * kDv;

    // Decode: the first head of each group stores the new token at position P.
    if (a.write_new && t == 0 && h % group == 0 && (a.ring || P < a.cap)) {
        const int slot = a.ring ? P % a.cap : P;
        float *kd = (float *)a.k_cache + (((size_t)b * a.Hkv + g) * a.cap + slot) * kDqk;
        float *vd = (float *)a.v_cache + (((size_t)b * a.Hkv + g) * a.cap + slot) * kDv;
        for (int d = lane; d < kDqk; d += 64)
            kd[d] = kn[d];
        for (int d = lane; d < kDv; d += 64)
            vd[d] = vn[d];
    }

    const float *q = (const float *)a.q + row * kDqk;
    const float sink2 = a.sink[h] * kLog2e;
    RowState st{sink2, sink2 == -INFINITY ? 0.f : 1.f, 0.f, 0.f};
    const int qp = P + t;
    const int lo = a.window > 0 ? max(0, qp - a.window + 1) : 0;
    for (int p = lo; p <= qp; ++p) {
        const float *kr, *vr;
        if (p < P) {
            const int slot = a.ring ? p % a.cap : p;
            kr = kc + (size_t)slot * kDqk;
            vr = vc + (size_t)slot * kDv;
        } else {
            kr = kn + (size_t)(p - P) * kns;
            vr = vn + (size_t)(p - P) * vns;
        }
        const float logit2 = dot192(q, kr, lane) * scale_log2;
        row_step(st, logit2, vr[lane], vr[64 + lane]);
    }
    const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
    float *o = (float *)a.o + row * kDv;
    o[lane] = st.a0 * inv;
    o[64 + lane] = st.a1 * inv;
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs &a, hipStream_t s) {
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    const size_t rows = (size_t)a.B * a.T * a.Hq;
    prefill_f32_kernel<<<dim3((unsigned)rows), dim3(64), 0, s>>>(a, scale_log2);
    return hipGetLastError();
}

hipError_t launch_cached_f32(const CachedArgs &a, hipStream_t s) {
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    const size_t rows = (size_t)a.B * a.nq * a.Hq;
    cached_f32_kernel<<<dim3((unsigned)rows), dim3(64), 0, s>>>(a, scale_log2);
    return hipGetLastError();
}

}  // namespace sinkattn

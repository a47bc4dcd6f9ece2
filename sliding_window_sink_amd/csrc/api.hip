// api.hip -- the C ABI of include/sinkattn.h: argument validation and dispatch.
//
// Every entry point validates its arguments on the host and returns a
// SINKATTN_ERR_* code before touching the HIP runtime; only then does it
// enqueue kernels on the caller's stream.  No device memory is allocated or
// freed here; the only global state is the per-device compute-unit count used
// by the split-K heuristic and the per-device address of the fixed scratch
// array of sinkattn_decode_noalloc.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/sinkattn.h"
#include "launch.h"

namespace sinkattn {

int device_cu_count() {
    static std::mutex mu;
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Split-K scratch of sinkattn_decode_noalloc: a fixed device array, so that
// entry point allocates nothing.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address (one copy per GPU) is looked
// up once per device with hipGetSymbolAddress and only that address is used.
static __device__ __align__(256) unsigned char scratch[SINKATTN_STATIC_SCRATCH_BYTES];

hipError_t static_scratch_address(void **out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {nullptr};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (p == nullptr)
            return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

}  // namespace sinkattn

using namespace sinkattn;

namespace {

constexpr int kDqk = 192, kDv = 128;

int esize(int dtype) { return dtype == SINKATTN_BF16 ? 2 : 4; }

bool overlaps(const void *a, size_t an, const void *b, size_t bn) {
    if (!a || !b || an == 0 || bn == 0)
        return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + bn && y < x + an;
}

int status_from_hip(hipError_t e) { return e == hipSuccess ? SINKATTN_OK : SINKATTN_ERR_HIP; }

// Shared checks of the attention entry points.
int check_heads(int Hq, int Hkv, int dqk, int dv, int dtype) {
    if (dtype != SINKATTN_F32 && dtype != SINKATTN_BF16)
        return SINKATTN_ERR_DTYPE;
    if (Hq <= 0 || Hkv <= 0 || dqk <= 0 || dv <= 0 || Hq % Hkv != 0)
        return SINKATTN_ERR_SHAPE;
    if (dqk != kDqk || dv != kDv)
        return SINKATTN_ERR_UNSUPPORTED;
    if (dtype == SINKATTN_BF16 && (Hq / Hkv) % 8 != 0)
        return SINKATTN_ERR_UNSUPPORTED;
    return SINKATTN_OK;
}

int prefill_common(const void *q, const void *k, const void *v, const float *sink, void *o,
                   float *lse, int B, int T, int Hq, int Hkv, int dqk, int dv, int window,
                   float scale, int dtype, void *stream) {
    int st = check_heads(Hq, Hkv, dqk, dv, dtype);
    if (st)
        return st;
    if ((int64_t)B * T != 0 && (!q || !k || !v || !sink || !o))  // empty: may be NULL
        return SINKATTN_ERR_NULL_PTR;
    if (B < 0 || T < 0)
        return SINKATTN_ERR_SHAPE;
    const size_t es = esize(dtype);
    // One sequence's q rows are addressed with 32-bit byte offsets, except by the
    // persistent sliding-window kernel, which re-bases every run of tiles.
    const bool rebased = dtype == SINKATTN_BF16 && window > 0 && window <= kSwaMaxWindow;
    if ((int64_t)B * T * Hq > INT_MAX || (int64_t)B * T > INT_MAX / kDqk ||
        (!rebased && (int64_t)T * Hq * kDqk * (int64_t)es > INT_MAX))
        return SINKATTN_ERR_SHAPE;
    const size_t qn = (size_t)B * T * Hq * kDqk * es, kn = (size_t)B * T * Hkv * kDqk * es;
    const size_t vn = (size_t)B * T * Hkv * kDv * es, on = (size_t)B * T * Hq * kDv * es;
    const size_t ln = lse ? (size_t)B * Hq * T * 4 : 0;
    if (overlaps(o, on, q, qn) || overlaps(o, on, k, kn) || overlaps(o, on, v, vn) ||
        overlaps(lse, ln, q, qn) || overlaps(lse, ln, k, kn) || overlaps(lse, ln, v, vn) ||
        overlaps(lse, ln, o, on))
        return SINKATTN_ERR_ALIAS;
    if ((size_t)B * T == 0)
        return SINKATTN_OK;
    PrefillArgs a{q, k, v, sink, o, lse, B, T, Hq, Hkv, window,
                  scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)dqk))};
    hipStream_t s = (hipStream_t)stream;
    if (dtype != SINKATTN_BF16)
        return status_from_hip(launch_prefill_f32(a, s));
    if (window > 0 && window <= kSwaMaxWindow)
        return status_from_hip(launch_prefill_swa_persistent(a, 0.0, nullptr, false, s));
    return status_from_hip(launch_prefill_bf16(a, s));
}

size_t ws_bytes_for(int B, int Hq, int dv, int nq, int splits) {
    if (splits <= 1 || B <= 0 || Hq <= 0 || dv <= 0 || nq <= 0)
        return 0;
    return (size_t)B * nq * Hq * splits * (dv + 2) * sizeof(float);
}

int cached_common(const void *q, const void *k_new, const void *v_new, void *k_cache,
                  void *v_cache, int kind, int cap, const int32_t *cache_len, int max_len_hint,
                  const float *sink, void *o, int B, int nq, int Hq, int Hkv, int dqk, int dv,
                  int window, float scale, int num_splits, void *workspace, size_t ws_bytes,
                  int dtype, void *stream, int write_new, int rope = 0, int rope_dim = 0,
                  double rope_base = 0.0, void *k_rot = nullptr, int fp8 = 0,
                  float k_scale = 1.f, float v_scale = 1.f, bool static_ws = false) {
    // static_ws: the split-K scratch is the library's fixed device array; its
    // address is looked up only after validation, when a split is taken
    if (static_ws) {
        workspace = nullptr;
        ws_bytes = SINKATTN_STATIC_SCRATCH_BYTES;
    }
    int st = check_heads(Hq, Hkv, dqk, dv, dtype);
    if (st)
        return st;
    if (fp8) {
        if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) ||
            !std::isfinite(v_scale))
            return SINKATTN_ERR_SHAPE;
        if (dtype != SINKATTN_BF16)
            return SINKATTN_ERR_UNSUPPORTED;
    }
    if (rope) {
        if (!(rope_base > 0.0) || !std::isfinite(rope_base) || rope_dim < 0 ||
            rope_dim % 2 != 0 || rope_dim > dqk)
            return SINKATTN_ERR_SHAPE;
        if (dtype != SINKATTN_BF16 || rope_dim != 64)
            return SINKATTN_ERR_UNSUPPORTED;
    }
    if (kind != SINKATTN_CACHE_RING && kind != SINKATTN_CACHE_CONTIG)
        return SINKATTN_ERR_UNSUPPORTED;
    if (B != 0 && (!q || !k_new || !v_new || !k_cache || !v_cache || !cache_len || !sink || !o))
        return SINKATTN_ERR_NULL_PTR;
    if (B < 0 || nq < 1 || nq > 8 || cap < 1 || max_len_hint < 0 || num_splits < 0)
        return SINKATTN_ERR_SHAPE;
    if (dtype == SINKATTN_BF16 && nq * (Hq / Hkv) > 64)
        return SINKATTN_ERR_UNSUPPORTED;
    // a (sequence, KV head)'s cache rows are addressed with 32-bit byte offsets
    if ((int64_t)max_len_hint + nq > INT_MAX / 2 || (int64_t)B * nq * Hq > INT_MAX ||
        (int64_t)B * Hkv * cap > (int64_t)INT_MAX * 8 ||
        (int64_t)cap * kDqk * (fp8 ? 1 : (int64_t)esize(dtype)) > INT_MAX)
        return SINKATTN_ERR_SHAPE;
    if (kind == SINKATTN_CACHE_RING) {
        if (window < 1)
            return SINKATTN_ERR_SHAPE;
        if (cap < window)
            return SINKATTN_ERR_CAPACITY;
    } else {
        // decode stores the new token at index max_len; verify only reads < max_len
        if (write_new ? max_len_hint >= cap : max_len_hint > cap)
            return SINKATTN_ERR_CAPACITY;
    }
    const size_t es = esize(dtype);
    const size_t on = (size_t)B * nq * Hq * kDv * es;
    const size_t ces = fp8 ? 1 : es;  // bytes per cached element
    const size_t kcn = (size_t)B * Hkv * cap * kDqk * ces, vcn = (size_t)B * Hkv * cap * kDv * ces;
    const size_t qn = (size_t)B * nq * Hq * kDqk * es;
    const size_t knn = (size_t)B * nq * Hkv * kDqk * es, vnn = (size_t)B * nq * Hkv * kDv * es;
    if (k_rot && (overlaps(k_rot, knn, q, qn) || overlaps(k_rot, knn, k_new, knn) ||
                  overlaps(k_rot, knn, v_new, vnn) || overlaps(k_rot, knn, k_cache, kcn) ||
                  overlaps(k_rot, knn, v_cache, vcn) || overlaps(k_rot, knn, o, on)))
        return SINKATTN_ERR_ALIAS;
    if (overlaps(o, on, q, qn) || overlaps(o, on, k_cache, kcn) || overlaps(o, on, v_cache, vcn) ||
        overlaps(o, on, k_new, knn) || overlaps(o, on, v_new, vnn) ||
        overlaps(k_cache, kcn, v_cache, vcn) ||
        (write_new && (overlaps(k_cache, kcn, k_new, knn) || overlaps(k_cache, kcn, v_new, vnn) ||
                       overlaps(v_cache, vcn, k_new, knn) || overlaps(v_cache, vcn, v_new, vnn))))
        return SINKATTN_ERR_ALIAS;

    // Split-K over the context (contiguous cache, bf16 path).
    int splits = 1, chunk = INT_MAX;
    const int64_t span = (int64_t)max_len_hint + nq;  // keys of the longest sequence
    if (kind == SINKATTN_CACHE_CONTIG && dtype == SINKATTN_BF16 && num_splits != 1 && B > 0) {
        const int n_cols = nq * (Hq / Hkv);
        const size_t per_split = ws_bytes_for(B, Hq, dv, nq, 2) / 2;
        const bool have_ws = workspace != nullptr || static_ws;
        if (num_splits > 1) {
            if (!have_ws || ws_bytes < per_split * (size_t)num_splits)
                return SINKATTN_ERR_WORKSPACE;
            int64_t c = (span + num_splits - 1) / num_splits;
            chunk = (int)((c + 127) / 128 * 128);
        } else {
            // automatic: ~24 workgroups per compute unit over the longest sequence
            // (sequences of unequal length need the finer pieces to even out the
            // work per compute unit), but chunks of at least 176 keys per (token,
            // head) column, so that a workgroup's fixed costs (its q, the merge,
            // 520 B of partial state per column) stay small next to the K/V bytes
            // it streams (640 B per key).  Measured at batch 64 x 16K: decode
            // 0.527 -> 0.488 ms (10 -> 6 splits) against a floor of 112 keys per
            // column; unchanged at batch 32 over 16K-128K contexts (47 splits of
            // 2816 keys, where 24 or 12 longer splits ran 6-10% slower).
            const int64_t cus = device_cu_count();
            int64_t c = ((int64_t)B * Hkv * span + 24 * cus - 1) / (24 * cus);
            c = std::max<int64_t>(c, 176 * (int64_t)n_cols);
            c = (c + 127) / 128 * 128;
            const int64_t want = (span + c - 1) / c;
            const int64_t room = have_ws ? (int64_t)(ws_bytes / per_split) : 0;
            const int64_t s_eff = std::min<int64_t>(want, room);
            if (s_eff >= 2) {
                c = (span + s_eff - 1) / s_eff;
                c = (c + 127) / 128 * 128;
                // A power-of-two chunk puts the start of every chunk of a sequence
                // at the same offset modulo a large power of two, so the chunks
                // read in step hit the same HBM channels: measured 8% slower than
                // a neighbouring size.  Step to the next multiple of 128 keys.
                if (((c / 128) & (c / 128 - 1)) == 0)
                    c += 128;
                chunk = (int)c;
            }
        }
        if (chunk != INT_MAX) {
            splits = (int)((span + chunk - 1) / chunk);
            if (splits < 2) {
                splits = 1;
                chunk = INT_MAX;
            }
        }
        if (splits > 1 && (overlaps(workspace, per_split * splits, o, on) ||
                           overlaps(workspace, per_split * splits, k_rot, k_rot ? knn : 0)))
            return SINKATTN_ERR_ALIAS;
    }
    if (B == 0)
        return SINKATTN_OK;
    if (static_ws && splits > 1) {
        if (hipError_t e = static_scratch_address(&workspace); e != hipSuccess)
            return SINKATTN_ERR_HIP;
    }

    CachedArgs a{};
    a.q = q;
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.cache_len = cache_len;
    a.sink = sink;
    a.o = o;
    a.ws = splits > 1 ? (float *)workspace : nullptr;
    a.B = B;
    a.nq = nq;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.cap = cap;
    a.window = kind == SINKATTN_CACHE_RING ? window : (window > 0 ? window : 0);
    a.ring = kind == SINKATTN_CACHE_RING;
    a.write_new = write_new;
    a.max_len = max_len_hint;
    a.n_splits = splits;
    a.chunk = chunk;
    a.scale = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)dqk));
    a.rope = rope;
    a.rope_base = rope_base;
    a.k_rot = k_rot;
    a.fp8 = fp8;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    hipStream_t s = (hipStream_t)stream;
    return status_from_hip(dtype == SINKATTN_BF16 ? launch_cached_bf16(a, s)
                                                  : launch_cached_f32(a, s));
}

}  // namespace

extern "C" {

int sinkattn_abi_version(void) { return SINKATTN_ABI_VERSION; }

const char *sinkattn_status_string(int status) {
    switch (status) {
    case SINKATTN_OK: return "ok";
    case SINKATTN_ERR_NULL_PTR: return "a required pointer is NULL";
    case SINKATTN_ERR_SHAPE: return "a size is out of range or inconsistent";
    case SINKATTN_ERR_DTYPE: return "unknown dtype code";
    case SINKATTN_ERR_UNSUPPORTED: return "valid but unsupported configuration";
    case SINKATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case SINKATTN_ERR_CAPACITY: return "cache capacity too small for the request";
    case SINKATTN_ERR_ALIAS: return "an output overlaps an input";
    case SINKATTN_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
    }
}

int sinkattn_rope_partial(void *x, int dtype, int64_t n_tok, int n_heads, int head_dim,
                          int rope_dim, const int32_t *pos, double base, int style,
                          void *stream) {
    if (dtype != SINKATTN_F32 && dtype != SINKATTN_BF16)
        return SINKATTN_ERR_DTYPE;
    if (n_tok != 0 && (!x || !pos))
        return SINKATTN_ERR_NULL_PTR;
    if (n_tok < 0 || n_heads < 0 || head_dim <= 0 || rope_dim < 0 || rope_dim % 2 != 0 ||
        rope_dim > head_dim || !(base > 0.0) || !std::isfinite(base) ||
        (style != SINKATTN_ROPE_INTERLEAVED && style != SINKATTN_ROPE_HALF))
        return SINKATTN_ERR_SHAPE;
    if (rope_dim > 256)
        return SINKATTN_ERR_UNSUPPORTED;
    if (n_tok > (int64_t)INT_MAX * 8 || (int64_t)n_heads * head_dim > INT_MAX)
        return SINKATTN_ERR_SHAPE;
    return status_from_hip(launch_rope(x, dtype == SINKATTN_BF16, n_tok, n_heads, head_dim,
                                       rope_dim, pos, base, style, (hipStream_t)stream));
}

int sinkattn_prefill_swa(const void *q, const void *k, const void *v, const float *sink,
                         void *o, float *lse, int B, int T, int Hq, int Hkv, int dqk, int dv,
                         int window, float scale, int dtype, void *stream) {
    if (window < 1) {
        int st = check_heads(Hq, Hkv, dqk, dv, dtype);
        return st ? st : SINKATTN_ERR_SHAPE;
    }
    return prefill_common(q, k, v, sink, o, lse, B, T, Hq, Hkv, dqk, dv, window, scale, dtype,
                          stream);
}

int sinkattn_prefill_swa_rope(const void *q, const void *k, const void *v, const float *sink,
                              void *o, float *lse, void *k_rot, int B, int T, int Hq, int Hkv,
                              int dqk, int dv, int window, float scale, int rope_dim,
                              double rope_base, int dtype, void *stream) {
    int st = check_heads(Hq, Hkv, dqk, dv, dtype);
    if (st)
        return st;
    if ((int64_t)B * T != 0 && (!q || !k || !v || !sink || !o))
        return SINKATTN_ERR_NULL_PTR;
    if (B < 0 || T < 0 || window < 1 || !(rope_base > 0.0) || !std::isfinite(rope_base) ||
        rope_dim < 0 || rope_dim % 2 != 0 || rope_dim > dqk)
        return SINKATTN_ERR_SHAPE;
    if (dtype != SINKATTN_BF16 || rope_dim != 64 || window > kSwaMaxWindow)
        return SINKATTN_ERR_UNSUPPORTED;
    if ((int64_t)B * T * Hq > INT_MAX || (int64_t)B * T > INT_MAX / kDqk)
        return SINKATTN_ERR_SHAPE;
    const size_t es = esize(dtype);
    const size_t qn = (size_t)B * T * Hq * kDqk * es, kn = (size_t)B * T * Hkv * kDqk * es;
    const size_t vn = (size_t)B * T * Hkv * kDv * es, on = (size_t)B * T * Hq * kDv * es;
    const size_t ln = lse ? (size_t)B * Hq * T * 4 : 0;
    const void *ins[3] = {q, k, v};
    const size_t insz[3] = {qn, kn, vn};
    for (int i = 0; i < 3; ++i)
        if (overlaps(o, on, ins[i], insz[i]) || overlaps(lse, ln, ins[i], insz[i]) ||
            overlaps(k_rot, kn, ins[i], insz[i]))
            return SINKATTN_ERR_ALIAS;
    if (overlaps(lse, ln, o, on) || overlaps(k_rot, kn, o, on) || overlaps(k_rot, kn, lse, ln))
        return SINKATTN_ERR_ALIAS;
    if ((size_t)B * T == 0)
        return SINKATTN_OK;
    PrefillArgs a{q, k, v, sink, o, lse, B, T, Hq, Hkv, window,
                  scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)dqk))};
    return status_from_hip(
        launch_prefill_swa_persistent(a, rope_base, k_rot, true, (hipStream_t)stream));
}

int sinkattn_prefill_global(const void *q, const void *k, const void *v, const float *sink,
                            void *o, float *lse, int B, int T, int Hq, int Hkv, int dqk,
                            int dv, float scale, int dtype, void *stream) {
    return prefill_common(q, k, v, sink, o, lse, B, T, Hq, Hkv, dqk, dv, 0, scale, dtype,
                          stream);
}

int sinkattn_prefill_global_rope(const void *q, const void *k, const void *v, const float *sink,
                                 void *o, float *lse, void *k_rot, int B, int T, int Hq,
                                 int Hkv, int dqk, int dv, float scale, int rope_dim,
                                 double rope_base, int dtype, void *stream) {
    int st = check_heads(Hq, Hkv, dqk, dv, dtype);
    if (st)
        return st;
    if ((int64_t)B * T != 0 && (!q || !k || !v || !sink || !o || !k_rot))
        return SINKATTN_ERR_NULL_PTR;
    if (B < 0 || T < 0 || !(rope_base > 0.0) || !std::isfinite(rope_base) || rope_dim < 0 ||
        rope_dim % 2 != 0 || rope_dim > dqk)
        return SINKATTN_ERR_SHAPE;
    if (dtype != SINKATTN_BF16 || rope_dim != 64)
        return SINKATTN_ERR_UNSUPPORTED;
    const size_t es = esize(dtype);
    // one sequence's q rows are addressed with 32-bit byte offsets
    if ((int64_t)B * T * Hq > INT_MAX || (int64_t)B * T > INT_MAX / kDqk ||
        (int64_t)T * Hq * kDqk * (int64_t)es > INT_MAX)
        return SINKATTN_ERR_SHAPE;
    const size_t qn = (size_t)B * T * Hq * kDqk * es, kn = (size_t)B * T * Hkv * kDqk * es;
    const size_t vn = (size_t)B * T * Hkv * kDv * es, on = (size_t)B * T * Hq * kDv * es;
    const size_t ln = lse ? (size_t)B * Hq * T * 4 : 0;
    const void *ins[3] = {q, k, v};
    const size_t insz[3] = {qn, kn, vn};
    for (int i = 0; i < 3; ++i)
        if (overlaps(o, on, ins[i], insz[i]) || overlaps(lse, ln, ins[i], insz[i]) ||
            overlaps(k_rot, kn, ins[i], insz[i]))
            return SINKATTN_ERR_ALIAS;
    if (overlaps(lse, ln, o, on) || overlaps(k_rot, kn, o, on) || overlaps(k_rot, kn, lse, ln))
        return SINKATTN_ERR_ALIAS;
    if ((size_t)B * T == 0)
        return SINKATTN_OK;
    hipStream_t s = (hipStream_t)stream;
    // The keys are rotated once (T x Hkv rows, written to k_rot, read back by
    // every query tile); q is rotated on load inside the attention kernel.
    hipError_t e = launch_rope_rows(k, k_rot, B, T, Hkv, rope_base, s);
    if (e != hipSuccess)
        return SINKATTN_ERR_HIP;
    PrefillArgs a{q, k_rot, v, sink, o, lse, B, T, Hq, Hkv, 0,
                  scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)dqk))};
    a.rope_q = 1;
    a.rope_base = rope_base;
    return status_from_hip(launch_prefill_bf16(a, s));
}

size_t sinkattn_backward_workspace_bytes(int B, int T, int Hq) {
    if (B <= 0 || T <= 0 || Hq <= 0)
        return 0;
    return 2 * (size_t)B * T * Hq * sizeof(float);
}

int sinkattn_backward(const void *q, const void *k, const void *v, const void *o,
                      const void *dout, const float *lse, const float *sink, float *dq,
                      float *dk, float *dv, float *dsink, int B, int T, int Hq, int Hkv, int dqk,
                      int dv_dim, int window, float scale, void *workspace, size_t ws_bytes,
                      int dtype, void *stream) {
    int st = check_heads(Hq, Hkv, dqk, dv_dim, dtype);
    if (st)
        return st;
    if (dtype != SINKATTN_BF16)
        return SINKATTN_ERR_UNSUPPORTED;
    if ((int64_t)B * T != 0 &&
        (!q || !k || !v || !o || !dout || !lse || !sink || !dq || !dk || !dv || !dsink))
        return SINKATTN_ERR_NULL_PTR;
    if (B < 0 || T < 0 || window < 0)
        return SINKATTN_ERR_SHAPE;
    if ((int64_t)B * T * Hq > INT_MAX || (int64_t)B * T > INT_MAX / kDqk ||
        (int64_t)T * Hq * kDqk * 4 > INT_MAX)
        return SINKATTN_ERR_SHAPE;
    const size_t need = sinkattn_backward_workspace_bytes(B, T, Hq);
    if (need > 0 && (!workspace || ws_bytes < need))
        return SINKATTN_ERR_WORKSPACE;
    const size_t n = (size_t)B * T;
    const size_t qn = n * Hq * kDqk * 2, kn = n * Hkv * kDqk * 2, vn = n * Hkv * kDv * 2;
    const size_t on = n * Hq * kDv * 2, ln = n * Hq * 4;
    const size_t dqn = n * Hq * kDqk * 4, dkn = n * Hkv * kDqk * 4, dvn = n * Hkv * kDv * 4;
    const void *ins[7] = {q, k, v, o, dout, lse, sink};
    const size_t insz[7] = {qn, kn, vn, on, on, ln, (size_t)Hq * 4};
    const void *outs[5] = {dq, dk, dv, dsink, workspace};
    const size_t outsz[5] = {dqn, dkn, dvn, (size_t)Hq * 4, need};
    for (int i = 0; i < 5; ++i) {
        for (int j = 0; j < 7; ++j)
            if (overlaps(outs[i], outsz[i], ins[j], insz[j]))
                return SINKATTN_ERR_ALIAS;
        for (int j = i + 1; j < 5; ++j)
            if (overlaps(outs[i], outsz[i], outs[j], outsz[j]))
                return SINKATTN_ERR_ALIAS;
    }
    if (n == 0)
        return SINKATTN_OK;
    BwdArgs a{q, k, v, o, dout, lse, sink, dq, dk, dv, dsink, (float *)workspace,
              (float *)workspace + n * Hq, B, T, Hq, Hkv, window,
              scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)dqk))};
    return status_from_hip(launch_backward(a, (hipStream_t)stream));
}

size_t sinkattn_decode_workspace_bytes(int B, int Hq, int dv, int n_q, int max_splits) {
    return ws_bytes_for(B, Hq, dv, n_q, max_splits);
}

int sinkattn_decode(const void *q, const void *k_new, const void *v_new, void *k_cache,
                    void *v_cache, int kind, int cap, const int32_t *cache_len,
                    int max_len_hint, const float *sink, void *o, int B, int Hq, int Hkv,
                    int dqk, int dv, int window, float scale, int num_splits, void *workspace,
                    size_t ws_bytes, int dtype, void *stream) {
    return cached_common(q, k_new, v_new, k_cache, v_cache, kind, cap, cache_len, max_len_hint,
                         sink, o, B, 1, Hq, Hkv, dqk, dv, window, scale, num_splits, workspace,
                         ws_bytes, dtype, stream, 1);
}

int sinkattn_decode_noalloc(const void *q, const void *k_new, const void *v_new, void *k_cache,
                            void *v_cache, int kind, int cap, const int32_t *cache_len,
                            int max_len_hint, const float *sink, void *o, int B, int Hq,
                            int Hkv, int dqk, int dv, int window, float scale, int num_splits,
                            int dtype, void *stream) {
    return cached_common(q, k_new, v_new, k_cache, v_cache, kind, cap, cache_len, max_len_hint,
                         sink, o, B, 1, Hq, Hkv, dqk, dv, window, scale, num_splits, nullptr, 0,
                         dtype, stream, 1, 0, 0, 0.0, nullptr, 0, 1.f, 1.f, true);
}

int sinkattn_verify(const void *q, const void *k_new, const void *v_new, const void *k_cache,
                    const void *v_cache, int kind, int cap, const int32_t *cache_len,
                    int max_len_hint, const float *sink, void *o, int B, int nq, int Hq,
                    int Hkv, int dqk, int dv, int window, float scale, int num_splits,
                    void *workspace, size_t ws_bytes, int dtype, void *stream) {
    return cached_common(q, k_new, v_new, (void *)k_cache, (void *)v_cache, kind, cap,
                         cache_len, max_len_hint, sink, o, B, nq, Hq, Hkv, dqk, dv, window,
                         scale, num_splits, workspace, ws_bytes, dtype, stream, 0);
}

int sinkattn_decode_rope(const void *q, const void *k_new, const void *v_new, void *k_cache,
                         void *v_cache, int kind, int cap, const int32_t *cache_len,
                         int max_len_hint, const float *sink, void *o, int B, int Hq, int Hkv,
                         int dqk, int dv, int window, float scale, int rope_dim,
                         double rope_base, int num_splits, void *workspace, size_t ws_bytes,
                         int dtype, void *stream) {
    return cached_common(q, k_new, v_new, k_cache, v_cache, kind, cap, cache_len, max_len_hint,
                         sink, o, B, 1, Hq, Hkv, dqk, dv, window, scale, num_splits, workspace,
                         ws_bytes, dtype, stream, 1, 1, rope_dim, rope_base, nullptr);
}

int sinkattn_verify_rope(const void *q, const void *k_new, const void *v_new,
                         const void *k_cache, const void *v_cache, int kind, int cap,
                         const int32_t *cache_len, int max_len_hint, const float *sink, void *o,
                         void *k_rot, int B, int nq, int Hq, int Hkv, int dqk, int dv,
                         int window, float scale, int rope_dim, double rope_base,
                         int num_splits, void *workspace, size_t ws_bytes, int dtype,
                         void *stream) {
    return cached_common(q, k_new, v_new, (void *)k_cache, (void *)v_cache, kind, cap,
                         cache_len, max_len_hint, sink, o, B, nq, Hq, Hkv, dqk, dv, window,
                         scale, num_splits, workspace, ws_bytes, dtype, stream, 0, 1, rope_dim,
                         rope_base, k_rot);
}

int sinkattn_kv_append(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                       int kind, int cap, const int32_t *cache_len, const int32_t *n_accept,
                       int B, int n, int Hkv, int dqk, int dv, int dtype, void *stream) {
    if (dtype != SINKATTN_F32 && dtype != SINKATTN_BF16)
        return SINKATTN_ERR_DTYPE;
    if (kind != SINKATTN_CACHE_RING && kind != SINKATTN_CACHE_CONTIG)
        return SINKATTN_ERR_UNSUPPORTED;
    if ((int64_t)B * n != 0 && (!k_new || !v_new || !k_cache || !v_cache || !cache_len))
        return SINKATTN_ERR_NULL_PTR;
    if (B < 0 || n < 0 || Hkv <= 0 || cap < 1 || dqk <= 0 || dv <= 0)
        return SINKATTN_ERR_SHAPE;
    if (dqk != kDqk || dv != kDv)
        return SINKATTN_ERR_UNSUPPORTED;
    if ((int64_t)B * n * Hkv > INT_MAX / 64)
        return SINKATTN_ERR_SHAPE;
    const size_t es = esize(dtype);
    const size_t kcn = (size_t)B * Hkv * cap * kDqk * es, vcn = (size_t)B * Hkv * cap * kDv * es;
    const size_t knn = (size_t)B * n * Hkv * kDqk * es, vnn = (size_t)B * n * Hkv * kDv * es;
    if (overlaps(k_cache, kcn, v_cache, vcn) || overlaps(k_cache, kcn, k_new, knn) ||
        overlaps(k_cache, kcn, v_new, vnn) || overlaps(v_cache, vcn, k_new, knn) ||
        overlaps(v_cache, vcn, v_new, vnn))
        return SINKATTN_ERR_ALIAS;
    if (B == 0 || n == 0)
        return SINKATTN_OK;
    AppendArgs a{k_new, v_new, k_cache, v_cache, cache_len, n_accept, B, n, Hkv, cap,
                 kind == SINKATTN_CACHE_RING};
    return status_from_hip(launch_append(a, dtype == SINKATTN_BF16, (hipStream_t)stream));
}

int sinkattn_decode_fp8(const void *q, const void *k_new, const void *v_new, void *k_cache,
                        void *v_cache, int kind, int cap, const int32_t *cache_len,
                        int max_len_hint, const float *sink, void *o, int B, int Hq, int Hkv,
                        int dqk, int dv, int window, float scale, float k_scale, float v_scale,
                        int rope_dim, double rope_base, int num_splits, void *workspace,
                        size_t ws_bytes, void *stream) {
    return cached_common(q, k_new, v_new, k_cache, v_cache, kind, cap, cache_len, max_len_hint,
                         sink, o, B, 1, Hq, Hkv, dqk, dv, window, scale, num_splits, workspace,
                         ws_bytes, SINKATTN_BF16, stream, 1, rope_dim != 0, rope_dim, rope_base,
                         nullptr, 1, k_scale, v_scale);
}

int sinkattn_verify_fp8(const void *q, const void *k_new, const void *v_new, const void *k_cache,
                        const void *v_cache, int kind, int cap, const int32_t *cache_len,
                        int max_len_hint, const float *sink, void *o, void *k_rot, int B,
                        int nq, int Hq, int Hkv, int dqk, int dv, int window, float scale,
                        float k_scale, float v_scale, int rope_dim, double rope_base,
                        int num_splits, void *workspace, size_t ws_bytes, void *stream) {
    if (k_rot && rope_dim == 0)
        return SINKATTN_ERR_SHAPE;  // rotated keys exist only with the RoPE fused
    return cached_common(q, k_new, v_new, (void *)k_cache, (void *)v_cache, kind, cap,
                         cache_len, max_len_hint, sink, o, B, nq, Hq, Hkv, dqk, dv, window,
                         scale, num_splits, workspace, ws_bytes, SINKATTN_BF16, stream, 0,
                         rope_dim != 0, rope_dim, rope_base, k_rot, 1, k_scale, v_scale);
}

int sinkattn_kv_append_fp8(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                           int kind, int cap, const int32_t *cache_len, const int32_t *n_accept,
                           int B, int n, int Hkv, int dqk, int dv, float k_scale, float v_scale,
                           void *stream) {
    if (kind != SINKATTN_CACHE_RING && kind != SINKATTN_CACHE_CONTIG)
        return SINKATTN_ERR_UNSUPPORTED;
    if ((int64_t)B * n != 0 && (!k_new || !v_new || !k_cache || !v_cache || !cache_len))
        return SINKATTN_ERR_NULL_PTR;
    if (B < 0 || n < 0 || Hkv <= 0 || cap < 1 || dqk <= 0 || dv <= 0 || !(k_scale > 0.f) ||
        !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
        return SINKATTN_ERR_SHAPE;
    if (dqk != kDqk || dv != kDv)
        return SINKATTN_ERR_UNSUPPORTED;
    if ((int64_t)B * n * Hkv > INT_MAX / 64)
        return SINKATTN_ERR_SHAPE;
    const size_t kcn = (size_t)B * Hkv * cap * kDqk, vcn = (size_t)B * Hkv * cap * kDv;
    const size_t knn = (size_t)B * n * Hkv * kDqk * 2, vnn = (size_t)B * n * Hkv * kDv * 2;
    if (overlaps(k_cache, kcn, v_cache, vcn) || overlaps(k_cache, kcn, k_new, knn) ||
        overlaps(k_cache, kcn, v_new, vnn) || overlaps(v_cache, vcn, k_new, knn) ||
        overlaps(v_cache, vcn, v_new, vnn))
        return SINKATTN_ERR_ALIAS;
    if (B == 0 || n == 0)
        return SINKATTN_OK;
    AppendArgs a{k_new, v_new, k_cache, v_cache, cache_len, n_accept, B, n, Hkv, cap,
                 kind == SINKATTN_CACHE_RING};
    a.fp8 = 1;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    return status_from_hip(launch_append(a, 1, (hipStream_t)stream));
}

int sinkattn_advance_len(int32_t *cache_len, const int32_t *n_accept, int B, int n,
                         void *stream) {
    if (B != 0 && !cache_len)
        return SINKATTN_ERR_NULL_PTR;
    if (B < 0 || n < 0)
        return SINKATTN_ERR_SHAPE;
    if (overlaps(cache_len, (size_t)B * 4, n_accept, n_accept ? (size_t)B * 4 : 0))
        return SINKATTN_ERR_ALIAS;
    return status_from_hip(launch_advance_len(cache_len, n_accept, B, n, (hipStream_t)stream));
}

}  // extern "C"

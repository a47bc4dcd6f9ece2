// launch.h -- internal parameter blocks and launchers (host <-> kernels).
// Nothing here crosses the public C ABI; the host entry points in api.hip
// validate arguments and then call these launchers on the caller's stream.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sinkattn {

// Causal prefill over positions 0..T-1 of B sequences (window <= 0: global).
struct PrefillArgs {
    const void *q, *k, *v;  // [B,T,Hq,192], [B,T,Hkv,192], [B,T,Hkv,128]
    const float *sink;      // [Hq]
    void *o;                // [B,T,Hq,128]
    float *lse;             // [B,Hq,T] or nullptr
    int B, T, Hq, Hkv, window;
    float scale;            // softmax scale (natural units)
    int rope_q = 0;         // global bf16 kernel: rotate q (64 dims, interleaved) on load
    double rope_base = 0.0;
};

// Queries at positions cache_len[b] + t (t < nq) over a ring or contiguous
// cache plus nq new tokens.
struct CachedArgs {
    const void *q;              // [B,nq,Hq,192]
    const void *k_new, *v_new;  // [B,nq,Hkv,192], [B,nq,Hkv,128]
    void *k_cache, *v_cache;    // [B,Hkv,cap,192], [B,Hkv,cap,128]
    const int32_t *cache_len;   // [B] device
    const float *sink;          // [Hq]
    void *o;                    // [B,nq,Hq,128]
    float *ws;                  // split workspace (fp32) or nullptr
    int B, nq, Hq, Hkv, cap, window, ring, write_new;
    int max_len;                // cache_len values are clamped to [0, max_len]
    int n_splits, chunk;        // context chunks (chunk keys each) when n_splits > 1
    float scale;
    int rope;                   // rotate q and k_new (64 dims, interleaved) at P + t
    double rope_base;
    void *k_rot;                // [B,nq,Hkv,192]: rotated k_new out, or nullptr
    int fp8;                    // caches hold E4M3 codes: value = code * k_scale / v_scale
    float k_scale, v_scale;
};

struct AppendArgs {
    const void *k_new, *v_new;  // [B,n,Hkv,192], [B,n,Hkv,128]
    void *k_cache, *v_cache;
    const int32_t *cache_len, *n_accept;
    int B, n, Hkv, cap, ring;
    int fp8 = 0;                // bf16 rows quantized into E4M3 caches
    float k_scale = 1.f, v_scale = 1.f;
};

// Gradients of a causal prefill (positions 0..T-1, window <= 0: global).
struct BwdArgs {
    const void *q, *k, *v, *o, *dout;  // bf16, layouts as the prefill's
    const float *lse, *sink;           // forward lse [B,Hq,T] (natural log), sinks [Hq]
    float *dq, *dk, *dv, *dsink;       // fp32 outputs
    float *D, *L2;                     // workspace, [B,Hq,T] each: D_i and lse_i * log2(e)
    int B, T, Hq, Hkv, window;
    float scale;
};

// Clamp a device-side cached length into the range the host validated.
__device__ __forceinline__ int clamp_len(int len, int max_len) {
    return len < 0 ? 0 : (len > max_len ? max_len : len);
}

// Out-of-place partial RoPE of bf16 rows [B,T,H,192] at positions 0..T-1 of
// each sequence (64 dims, interleaved pairs; dims 64.. copied).
hipError_t launch_rope_rows(const void *src, void *dst, int B, int T, int n_heads, double base,
                            hipStream_t s);
hipError_t launch_rope(void *x, int bf16, int64_t n_tok, int n_heads, int head_dim, int rope_dim,
                       const int32_t *pos, double base, int style, hipStream_t s);
hipError_t launch_prefill_bf16(const PrefillArgs &a, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs &a, hipStream_t s);
// Sliding-window prefill for window <= kSwaMaxWindow (bf16), optionally applying
// partial RoPE (64 dims, interleaved, base rope_base) to q and k on load and
// writing the rotated k to k_rot (may be null).
constexpr int kSwaMaxWindow = 129;
hipError_t launch_prefill_swa_persistent(const PrefillArgs &a, double rope_base, void *k_rot,
                                         bool rope, hipStream_t s);
hipError_t launch_cached_bf16(const CachedArgs &a, hipStream_t s);
// Attention part of launch_cached_bf16 for at most 16 columns per KV group
// (no split-K combine).
hipError_t launch_decode16(const CachedArgs &a, hipStream_t s);
// Attention part of launch_cached_bf16 for 17..64 columns per KV group over a
// contiguous bf16 cache without a window (K/V staged in LDS; no combine).
hipError_t launch_verify_lds(const CachedArgs &a, hipStream_t s);
hipError_t launch_cached_f32(const CachedArgs &a, hipStream_t s);
hipError_t launch_append(const AppendArgs &a, int bf16, hipStream_t s);
hipError_t launch_advance_len(int32_t *cache_len, const int32_t *n_accept, int B, int n,
                              hipStream_t s);

hipError_t launch_backward(const BwdArgs &a, hipStream_t s);

// Number of compute units of the current device (cached per device).
int device_cu_count();

}  // namespace sinkattn

/*
 * sinkattn.h -- C ABI of the MI355X (gfx950) sink-attention library.
 *
 * The operation is the attention layer of the MiMo-V2-Flash Technical Report
 * (full translation, garden.houmin.site/digest/mimo-v2-flash):
 *
 *   Section 2.2, equations 1-4: for one head, a_ij = q_i . k_j / sqrt(d);
 *   s_ij = exp(a_ij - m_i) / (exp(sink - m_i) + sum_j' exp(a_ij' - m_i)),
 *   m_i = max(max_j a_ij, sink); o_i = sum_j s_ij v_j.  One learnable sink
 *   logit per head sits in the denominator only (it has no value vector).
 *
 *   Section 2.1 and Table 1: grouped-query attention, sliding-window (W = 128,
 *   64 query / 8 KV heads) or global (64 query / 4 KV heads) layers; QK head
 *   dim 192, V head dim 128; RoPE only on the first 64 dims of q and k.
 *
 *   Section 2.3.1: decoding is memory-bound because every request keeps its
 *   own KV cache; draft tokens are verified by the main model in one pass
 *   without extra KV-cache traffic (the verify entry point below).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates or frees device memory and keeps no pointer after return.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *    is enqueued asynchronously; results are valid once the caller has
 *    synchronised the stream.  Host-side argument errors are returned before
 *    anything is enqueued; a device fault surfaces at the caller's sync.
 *  - Every function returns 0 (SINKATTN_OK) or a negative SINKATTN_ERR_* code;
 *    sinkattn_status_string() names it.
 *  - dtype is SINKATTN_F32 or SINKATTN_BF16 and applies to q, k, v, o, the
 *    caches and the new-token tensors alike.  `sink` is always fp32 [Hq] in
 *    logit units (not divided by sqrt(d)); -INFINITY disables a head's sink.
 *    `lse` (when requested) is always fp32.
 *  - Layouts are dense row-major:
 *        q [B,T,Hq,dqk]   k [B,T,Hkv,dqk]   v [B,T,Hkv,dv]   o [B,T,Hq,dv]
 *        lse [B,Hq,T]
 *        caches, head-major: k_cache [B,Hkv,cap,dqk], v_cache [B,Hkv,cap,dv]
 *    Query head h reads KV head h / (Hq/Hkv).
 *  - scale <= 0 selects 1/sqrt(dqk) (the report's d is the QK head dim).
 *  - A sliding window of W holds W keys including the query itself: a key at
 *    position p is visible to a query at position P iff P - W < p <= P.
 *  - Supported in this version: dqk == 192, dv == 128 (SINKATTN_ERR_UNSUPPORTED
 *    otherwise); Hq % Hkv == 0.  The bf16 paths need (Hq/Hkv) % 8 == 0.
 *  - Size limits (SINKATTN_ERR_SHAPE beyond them): B*T*Hq and B*T*dqk below
 *    2^31; the global prefills, windows over 129 and all fp32 prefills address
 *    one sequence's q with 32-bit byte offsets, so T*Hq*dqk*(element size) must
 *    stay below 2^31 (bf16, 64 query heads: T <= 87381); the sliding-window
 *    bf16 prefills (W <= 129) have no per-sequence limit.  A cache's rows of
 *    one (sequence, KV head) likewise: cap*dqk*(cache element size) below 2^31
 *    (bf16: cap <= 5592405).
 *  - A call with nothing to do (B*T == 0 for a prefill or backward; B == 0 for
 *    decode, verify and advance_len; B*n == 0 for kv_append; n_tok == 0 for
 *    RoPE) returns SINKATTN_OK with no HIP call; its data pointers may be NULL.
 *  - Calls on different streams that write the same buffers race; nothing else
 *    is shared between calls.
 */
#ifndef SINKATTN_H
#define SINKATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SINKATTN_ABI_VERSION 1

enum {
    SINKATTN_OK = 0,
    SINKATTN_ERR_NULL_PTR = -1,    /* a required pointer is NULL */
    SINKATTN_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
    SINKATTN_ERR_DTYPE = -3,       /* unknown dtype code */
    SINKATTN_ERR_UNSUPPORTED = -4, /* valid but not implemented (head dims, group) */
    SINKATTN_ERR_WORKSPACE = -5,   /* workspace missing or too small */
    SINKATTN_ERR_CAPACITY = -6,    /* cache capacity too small for the request */
    SINKATTN_ERR_ALIAS = -7,       /* an output overlaps an input it must not */
    SINKATTN_ERR_HIP = -8          /* the HIP runtime reported an error at launch */
};

enum { SINKATTN_F32 = 0, SINKATTN_BF16 = 1 };
enum { SINKATTN_CACHE_RING = 0, SINKATTN_CACHE_CONTIG = 1 };
enum { SINKATTN_ROPE_INTERLEAVED = 0, SINKATTN_ROPE_HALF = 1 };

/* Version of this ABI (SINKATTN_ABI_VERSION of the built library). */
int sinkattn_abi_version(void);

/* Static, never-NULL description of a status code. */
const char *sinkattn_status_string(int status);

/*
 * Partial rotary position embedding, in place (Section 2.1: RoPE on the first
 * 64 dims of q and k; RoFormer; bases from Section 3.2: 1e4 for SWA layers,
 * 6.4e5 then 5e6 for global layers).
 *   x    [n_tok, n_heads, head_dim] (dtype), rotated in place
 *   pos  device int32 [n_tok]: absolute position of each token (>= 0)
 *   rope_dim: even, <= head_dim; dims >= rope_dim are left bit-identical
 *   style: SINKATTN_ROPE_INTERLEAVED pairs (2c, 2c+1);
 *          SINKATTN_ROPE_HALF pairs (c, c + rope_dim/2)
 *   angle = pos * base^(-2c/rope_dim) is formed in fp64; the rotation is done
 *   in fp32 and rounded once to dtype (round to nearest even).
 */
int sinkattn_rope_partial(void *x, int dtype, int64_t n_tok, int n_heads, int head_dim,
                          int rope_dim, const int32_t *pos, double base, int style,
                          void *stream);

/*
 * Causal sliding-window prefill (Section 2.2; window from Table 1).
 *   q, k, v, o as in the conventions, positions 0..T-1 in every sequence;
 *   window >= 1 (W); lse may be NULL.  o must not overlap q, k or v.
 */
int sinkattn_prefill_swa(const void *q, const void *k, const void *v, const float *sink,
                         void *o, float *lse, int B, int T, int Hq, int Hkv, int dqk, int dv,
                         int window, float scale, int dtype, void *stream);

/*
 * Sliding-window prefill with the partial RoPE fused into the loads: the result
 * equals sinkattn_rope_partial(q, positions 0..T-1), the same for k, then
 * sinkattn_prefill_swa -- bit for bit -- without writing the rotated q.
 * q and k are read-only (un-rotated); if k_rot is non-NULL the rotated k is
 * written there ([B,T,Hkv,192], e.g. straight into a KV cache; it must not
 * overlap any input).  Supported: bf16, rope_dim == 64 (interleaved pairs,
 * Section 2.1), 1 <= window <= 129 (SINKATTN_ERR_UNSUPPORTED otherwise).
 */
int sinkattn_prefill_swa_rope(const void *q, const void *k, const void *v, const float *sink,
                              void *o, float *lse, void *k_rot, int B, int T, int Hq, int Hkv,
                              int dqk, int dv, int window, float scale, int rope_dim,
                              double rope_base, int dtype, void *stream);

/* Causal prefill over the full context (global-attention layers, Table 1). */
int sinkattn_prefill_global(const void *q, const void *k, const void *v, const float *sink,
                            void *o, float *lse, int B, int T, int Hq, int Hkv, int dqk,
                            int dv, float scale, int dtype, void *stream);

/*
 * Global prefill with the partial RoPE fused (Section 2.1: 64 rotated dims;
 * Section 3.2: global layers use base 6.4e5, later 5e6).  The result equals
 * sinkattn_rope_partial(q, positions 0..T-1), the same for k, then
 * sinkattn_prefill_global -- bit for bit.  q and k are read-only (un-rotated).
 * k_rot [B,T,Hkv,192] is REQUIRED: the rotated keys are written there first
 * (each key is read by every later query tile, so it is rotated once) and the
 * attention reads them back; q is rotated on load and never written.  k_rot
 * must not overlap any input or output.  Supported: bf16, rope_dim == 64
 * (interleaved pairs); SINKATTN_ERR_UNSUPPORTED otherwise.
 */
int sinkattn_prefill_global_rope(const void *q, const void *k, const void *v, const float *sink,
                                 void *o, float *lse, void *k_rot, int B, int T, int Hq,
                                 int Hkv, int dqk, int dv, float scale, int rope_dim,
                                 double rope_base, int dtype, void *stream);

/*
 * Backward of a causal prefill (sinkattn_prefill_swa with window >= 1, or
 * sinkattn_prefill_global with window = 0): gradients of the loss with respect
 * to q, k, v and the sink logits, given the upstream gradient dout of o.
 * From Section 2.2 by the chain rule, with lse_i the forward log-normaliser
 * (ln of e^sink + sum_j e^(a_ij)), s_ij = e^(a_ij - lse_i), D_i = dout_i . o_i:
 *   dS_ij = s_ij (dout_i . v_j - D_i),  dq_i = scale sum_j dS_ij k_j,
 *   dk_j = scale sum_i dS_ij q_i,  dv_j = sum_i s_ij dout_i  (dk, dv summed over
 *   the query heads of the KV head),  dsink_h = -sum_i e^(sink_h - lse_i) D_i
 *   (summed over every token of every sequence).
 *   q, k, v, o, dout: bf16, layouts of the prefill (o, lse: the forward's outputs
 *   for these inputs; pass lse from the forward call with return of lse).
 *   dq [B,T,Hq,192], dk [B,T,Hkv,192], dv [B,T,Hkv,128], dsink [Hq]: fp32,
 *   overwritten.  Gradients are with respect to the q and k the attention saw
 *   (after RoPE).  workspace: sinkattn_backward_workspace_bytes(B, T, Hq)
 *   bytes.  Deterministic (no atomics).  Supported: bf16 (UNSUPPORTED
 *   otherwise); outputs and workspace must not overlap each other or inputs.
 *   B*T == 0: returns at once with no HIP call; no output is written (the
 *   caller owns the zero dsink of an empty batch).
 */
size_t sinkattn_backward_workspace_bytes(int B, int T, int Hq);

int sinkattn_backward(const void *q, const void *k, const void *v, const void *o,
                      const void *dout, const float *lse, const float *sink, float *dq,
                      float *dk, float *dv, float *dsink, int B, int T, int Hq, int Hkv, int dqk,
                      int dv_dim, int window, float scale, void *workspace, size_t ws_bytes,
                      int dtype, void *stream);

/*
 * Bytes of fp32 workspace that sinkattn_decode / sinkattn_verify need for a
 * split-K pass over a contiguous cache with at most `max_splits` splits:
 * B * n_q * Hq * max_splits * (dv + 2) * 4.  Zero if max_splits <= 1.
 */
size_t sinkattn_decode_workspace_bytes(int B, int Hq, int dv, int n_q, int max_splits);

/*
 * One decode step (Section 2.3.1: one new token per sequence).
 *   q      [B,Hq,dqk]   k_new [B,Hkv,dqk]   v_new [B,Hkv,dv]   o [B,Hq,dv]
 *   cache_len: device int32 [B], the number of tokens already cached; the new
 *          token sits at position P = cache_len[b].  Not modified.
 *   kind = SINKATTN_CACHE_RING: a W-slot ring per (sequence, KV head); position
 *          p lives in slot p % cap; requires window >= 1 and cap >= window.
 *          The query sees positions max(0, P-W+1) .. P.
 *   kind = SINKATTN_CACHE_CONTIG: position p lives at index p; requires
 *          max_len_hint < cap.  window <= 0 is global (positions 0..P),
 *          window >= 1 restricts to the last W positions.
 *   The step also stores k_new/v_new into the cache at position P (ring slot
 *   P % cap, or index P).  The attention itself reads the new token from
 *   k_new/v_new, never from the cache, so that store does not race with it.
 *   max_len_hint: host bound on max(cache_len); sizes the split grid.
 *   num_splits: CONTIG only: 0 = choose automatically, 1 = no split, S > 1 = at
 *          most S context chunks merged by an exact log-sum-exp combine that
 *          adds the sink once.  RING ignores it (at most W keys).
 *   workspace / ws_bytes: fp32 scratch of sinkattn_decode_workspace_bytes(B,
 *          Hq, dv, 1, S) bytes for the chosen S > 1 (may be NULL when no split
 *          is taken; the automatic choice never exceeds what ws_bytes holds).
 */
int sinkattn_decode(const void *q, const void *k_new, const void *v_new, void *k_cache,
                    void *v_cache, int kind, int cap, const int32_t *cache_len,
                    int max_len_hint, const float *sink, void *o, int B, int Hq, int Hkv,
                    int dqk, int dv, int window, float scale, int num_splits,
                    void *workspace, size_t ws_bytes, int dtype, void *stream);

/*
 * sinkattn_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments and results as sinkattn_decode, bit for bit, except that the
 * split-K scratch is not passed in: it is a fixed array of
 * SINKATTN_STATIC_SCRATCH_BYTES bytes of device memory inside the library,
 * which every GPU the library runs on holds from the library's load until the
 * process ends.  The call allocates nothing (no hipMalloc, no library
 * allocator).  The first call on a device looks the array's address up once
 * (hipGetSymbolAddress) and keeps it for that device.
 *   num_splits: 0 = automatic, limited to what the scratch holds (each split
 *   takes B * Hq * (dv + 2) * 4 bytes); an explicit S > 1 whose
 *   sinkattn_decode_workspace_bytes(B, Hq, dv, 1, S) exceeds the scratch is
 *   rejected with SINKATTN_ERR_WORKSPACE before anything is enqueued.
 *   Nothing in the scratch has to start at zero: every split that the combine
 *   step reads is written by the same call first.
 *   All calls on one GPU share that GPU's scratch, so calls that overlap in
 *   time on one GPU (different streams, or host threads on one stream without
 *   ordering) race; calls ordered on one stream do not.
 */
#define SINKATTN_STATIC_SCRATCH_BYTES (32u << 20)

int sinkattn_decode_noalloc(const void *q, const void *k_new, const void *v_new, void *k_cache,
                            void *v_cache, int kind, int cap, const int32_t *cache_len,
                            int max_len_hint, const float *sink, void *o, int B, int Hq,
                            int Hkv, int dqk, int dv, int window, float scale, int num_splits,
                            int dtype, void *stream);

/*
 * Multi-query speculative verification (Section 2.3.1 and Section 5: the main
 * model scores 1 + K draft tokens in one pass; Table 10 uses 3 draft heads).
 *   q [B,nq,Hq,dqk]; k_new/v_new [B,nq,Hkv,d]; o [B,nq,Hq,dv]; 1 <= nq <= 8.
 *   Query t sits at position P + t (P = cache_len[b]) and sees the visible
 *   cached positions plus new tokens 0..t.  THE CACHES ARE READ-ONLY: drafts
 *   are taken from k_new/v_new and committed later with sinkattn_kv_append
 *   (writing them into a W-slot ring first would overwrite keys still inside
 *   query 0's window).  Other arguments as in sinkattn_decode.
 *   Supported: nq * (Hq/Hkv) <= 64 on the bf16 path.
 */
int sinkattn_verify(const void *q, const void *k_new, const void *v_new,
                    const void *k_cache, const void *v_cache, int kind, int cap,
                    const int32_t *cache_len, int max_len_hint, const float *sink, void *o,
                    int B, int nq, int Hq, int Hkv, int dqk, int dv, int window, float scale,
                    int num_splits, void *workspace, size_t ws_bytes, int dtype,
                    void *stream);

/*
 * Decode and verify with the partial RoPE fused (Section 2.1): q and k_new are
 * given un-rotated and read-only; token t is rotated at position P + t
 * (P = cache_len[b]) inside the attention kernel, 64 dims, interleaved pairs,
 * base rope_base.  Results equal sinkattn_rope_partial on q and k_new at those
 * positions followed by sinkattn_decode / sinkattn_verify -- bit for bit:
 *   sinkattn_decode_rope stores the ROTATED k_new (and v_new) into the cache;
 *   sinkattn_verify_rope leaves the caches untouched and, if k_rot is non-NULL,
 *   writes the rotated k_new there ([B,nq,Hkv,192], the input of a later
 *   sinkattn_kv_append; it must not overlap any other argument).
 * Other arguments as in sinkattn_decode / sinkattn_verify.  Supported: bf16,
 * rope_dim == 64 (SINKATTN_ERR_UNSUPPORTED otherwise).
 */
int sinkattn_decode_rope(const void *q, const void *k_new, const void *v_new, void *k_cache,
                         void *v_cache, int kind, int cap, const int32_t *cache_len,
                         int max_len_hint, const float *sink, void *o, int B, int Hq, int Hkv,
                         int dqk, int dv, int window, float scale, int rope_dim,
                         double rope_base, int num_splits, void *workspace, size_t ws_bytes,
                         int dtype, void *stream);

int sinkattn_verify_rope(const void *q, const void *k_new, const void *v_new,
                         const void *k_cache, const void *v_cache, int kind, int cap,
                         const int32_t *cache_len, int max_len_hint, const float *sink, void *o,
                         void *k_rot, int B, int nq, int Hq, int Hkv, int dqk, int dv,
                         int window, float scale, int rope_dim, double rope_base,
                         int num_splits, void *workspace, size_t ws_bytes, int dtype,
                         void *stream);

/*
 * Commit accepted tokens into a cache (Section 2.3.1: the main model verifies
 * the draft tokens in one pass and the accepted ones join the context; this is
 * the step after verification that stores them).
 *   k_new [B,n,Hkv,dqk], v_new [B,n,Hkv,dv]: tokens at positions
 *   cache_len[b] .. cache_len[b]+n-1.  n_accept: device int32 [B] (NULL = n):
 *   only tokens t < min(n_accept[b], n) are written.  RING: position p goes to
 *   slot p % cap, and when more than cap tokens are written only the last cap
 *   of them are stored (so one call can lay a whole prefill into a ring).
 *   CONTIG: index p; positions >= cap are dropped (callers size cap).
 *   cache_len is not modified.
 */
int sinkattn_kv_append(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                       int kind, int cap, const int32_t *cache_len, const int32_t *n_accept,
                       int B, int n, int Hkv, int dqk, int dv, int dtype, void *stream);

/*
 * FP8 KV caches.  The report runs training and inference in FP8 (Section 4.6)
 * without defining the attention cache format; these entry points keep the
 * caches as OCP E4M3 codes (1 byte per element: sign, 4 exponent bits with
 * bias 7, 3 mantissa bits; no infinities; largest finite 448) with one scale
 * per tensor: cached value = code value * k_scale (keys) or * v_scale (values).
 * Activations (q, k_new, v_new, o, k_rot) are bf16.  A value x is stored as
 * the nearest E4M3 value of fl32(x / scale), ties to the even code, saturating
 * at +-448 (never NaN).  The new tokens of a step attend at bf16 precision
 * (read from k_new / v_new, as in sinkattn_decode) and are stored quantized.
 *   sinkattn_decode_fp8 / sinkattn_verify_fp8: as sinkattn_decode /
 *     sinkattn_verify (k_cache, v_cache: [B,Hkv,cap,192] / [B,Hkv,cap,128]
 *     uint8 codes); rope_dim = 0 takes q and k_new as already rotated,
 *     rope_dim = 64 fuses the RoPE as sinkattn_decode_rope / verify_rope do
 *     (k_rot, verify only, requires rope_dim = 64: bf16 rotated keys out).
 *   sinkattn_kv_append_fp8: as sinkattn_kv_append, quantizing bf16 rows.
 * Errors: k_scale or v_scale not finite and > 0 -> SINKATTN_ERR_SHAPE; other
 * codes as for the bf16 entry points.
 */
int sinkattn_decode_fp8(const void *q, const void *k_new, const void *v_new, void *k_cache,
                        void *v_cache, int kind, int cap, const int32_t *cache_len,
                        int max_len_hint, const float *sink, void *o, int B, int Hq, int Hkv,
                        int dqk, int dv, int window, float scale, float k_scale, float v_scale,
                        int rope_dim, double rope_base, int num_splits, void *workspace,
                        size_t ws_bytes, void *stream);

int sinkattn_verify_fp8(const void *q, const void *k_new, const void *v_new, const void *k_cache,
                        const void *v_cache, int kind, int cap, const int32_t *cache_len,
                        int max_len_hint, const float *sink, void *o, void *k_rot, int B,
                        int nq, int Hq, int Hkv, int dqk, int dv, int window, float scale,
                        float k_scale, float v_scale, int rope_dim, double rope_base,
                        int num_splits, void *workspace, size_t ws_bytes, void *stream);

int sinkattn_kv_append_fp8(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                           int kind, int cap, const int32_t *cache_len, const int32_t *n_accept,
                           int B, int n, int Hkv, int dqk, int dv, float k_scale, float v_scale,
                           void *stream);

/*
 * Advance the cached lengths after a commit (Section 2.3.1: accepted draft
 * tokens join the context): cache_len[b] += min(max(n_accept[b], 0), n), or
 * += n when n_accept is NULL -- exactly the tokens sinkattn_kv_append stored
 * with the same n_accept and n.  cache_len and n_accept are device int32 [B];
 * the update is stream-ordered, so a draft -> verify -> kv_append -> advance
 * loop runs without any host round trip (the host keeps max_len_hint an upper
 * bound by adding n per step).  Errors: NULL cache_len -> NULL_PTR; B < 0 or
 * n < 0 -> SHAPE; cache_len overlapping n_accept -> ALIAS.
 */
int sinkattn_advance_len(int32_t *cache_len, const int32_t *n_accept, int B, int n,
                         void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SINKATTN_H */

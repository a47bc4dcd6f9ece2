// Host-only stand-ins for the kernel launchers of launch.h, for building the C
// ABI's validation layer (api.hip) without device code under AddressSanitizer
// and UndefinedBehaviorSanitizer.  Each stub records its call and returns
// hipSuccess; nothing touches the pointers it is given.
#include "../../sliding_window_sink_amd/csrc/launch.h"

#include "stub_record.h"

namespace sinkattn {

StubRecord g_last;

static hipError_t rec(const char *name) {
    g_last = StubRecord{};
    g_last.name = name;
    ++g_last.calls;
    return hipSuccess;
}

hipError_t launch_rope_rows(const void *, void *, int B, int T, int n_heads, double,
                            hipStream_t) {
    (void)rec("rope_rows");
    g_last.B = B;
    g_last.T = T;
    g_last.H = n_heads;
    return hipSuccess;
}
hipError_t launch_rope(void *, int, int64_t n_tok, int n_heads, int, int, const int32_t *, double,
                       int, hipStream_t) {
    (void)rec("rope");
    g_last.T = (int)n_tok;
    g_last.H = n_heads;
    return hipSuccess;
}
hipError_t launch_prefill_bf16(const PrefillArgs &a, hipStream_t) {
    (void)rec("prefill_bf16");
    g_last.B = a.B;
    g_last.T = a.T;
    g_last.window = a.window;
    g_last.rope = a.rope_q;
    return hipSuccess;
}
hipError_t launch_prefill_f32(const PrefillArgs &a, hipStream_t) {
    (void)rec("prefill_f32");
    g_last.B = a.B;
    g_last.T = a.T;
    g_last.window = a.window;
    return hipSuccess;
}
hipError_t launch_prefill_swa_persistent(const PrefillArgs &a, double, void *, bool rope,
                                         hipStream_t) {
    (void)rec("prefill_swa");
    g_last.B = a.B;
    g_last.T = a.T;
    g_last.window = a.window;
    g_last.rope = rope;
    return hipSuccess;
}
static hipError_t cached(const char *name, const CachedArgs &a) {
    (void)rec(name);
    g_last.B = a.B;
    g_last.nq = a.nq;
    g_last.splits = a.n_splits;
    g_last.chunk = a.chunk;
    g_last.ws = a.ws;
    g_last.window = a.window;
    g_last.rope = a.rope;
    g_last.fp8 = a.fp8;
    return hipSuccess;
}
hipError_t launch_cached_bf16(const CachedArgs &a, hipStream_t) { return cached("cached_bf16", a); }
hipError_t launch_decode16(const CachedArgs &a, hipStream_t) { return cached("decode16", a); }
hipError_t launch_cached_f32(const CachedArgs &a, hipStream_t) { return cached("cached_f32", a); }
hipError_t launch_append(const AppendArgs &a, int, hipStream_t) {
    (void)rec("append");
    g_last.B = a.B;
    g_last.nq = a.n;
    g_last.fp8 = a.fp8;
    return hipSuccess;
}
hipError_t launch_advance_len(int32_t *, const int32_t *, int B, int n, hipStream_t) {
    (void)rec("advance_len");
    g_last.B = B;
    g_last.nq = n;
    return hipSuccess;
}
hipError_t launch_backward(const BwdArgs &a, hipStream_t) {
    (void)rec("backward");
    g_last.B = a.B;
    g_last.T = a.T;
    g_last.window = a.window;
    return hipSuccess;
}

}  // namespace sinkattn

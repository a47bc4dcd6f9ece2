// What the last stub launcher call saw (host-only sanitizer build of the C ABI).
#pragma once
#include <cstddef>

namespace sinkattn {
struct StubRecord {
    const char *name = nullptr;
    int calls = 0;
    int B = -1, T = -1, H = -1, nq = -1, window = -1, splits = -1, chunk = -1, rope = -1,
        fp8 = -1;
    const float *ws = nullptr;
};
extern StubRecord g_last;
}  // namespace sinkattn

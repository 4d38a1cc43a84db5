// What the stand-in launchers saw last (tests/sanitize only).
#pragma once
#include <cstdint>
struct StubRecord {
    int calls = 0;
    const char *last = "";
    int64_t sizes[4] = {0, 0, 0, 0};
};
extern StubRecord g_stub;

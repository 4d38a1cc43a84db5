// What the stand-in launchers saw last (tests/sanitize only).
#pragma once
#include <cstdint>
struct StubRecord {
    int calls = 0;
    const char *last = "";
    int64_t sizes[4] = {0, 0, 0, 0};
    int64_t layout = 0;  // pieces flag of a layout launch; rows per piece of an attention launch
};
extern StubRecord g_stub;

// What the host stand-ins of the GPU side record (tests/sanitize).
#pragma once
#include <cstdint>

struct StubState {
    const uint8_t* lo = nullptr;   // the container standing in for its device copy
    const uint8_t* hi = nullptr;
    uint64_t launches = 0;
    uint64_t dot_launches = 0;
    int64_t live_allocs = 0;       // "device" allocations not yet freed
    uint32_t last_no_long = 0;     // the last launch's no_long and one_code flags
    uint32_t last_one_code = 0;
    const uint32_t* last_status = nullptr;   // the last launch's debug status word
};
extern StubState g_stub;

// The stand-in launchers' registry of device allocations (fake addresses that
// the host code only does arithmetic on).
#pragma once
#include <cstdint>

void stub_register(const void *p, int64_t bytes);
void stub_reset();
long stub_launches();

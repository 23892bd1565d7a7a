// Shared by the stubs and the driver of the sanitizer build (tests/hostcheck).
#pragma once
#include <stddef.h>

namespace hostcheck {
// Registers [p, p + bytes) as a buffer that launches may touch.
void register_range(const void* p, size_t bytes, const char* name);
void clear_ranges();
// Launches that reached a (stub) launcher so far, and stream synchronisations.
long launches();
long syncs();
// The no-allocation entry point's workspace stand-in (64 MiB, registered by the driver).
void* scratch_range();
}  // namespace hostcheck

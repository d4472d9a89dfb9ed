// The library's static device scratch, for the entry points that allocate nothing.
#pragma once

#include <stddef.h>

namespace pkv {

// Bytes of the static scratch array (the same on every device).
constexpr size_t kScratchBytes = size_t(32) << 20;

// Device address of the current device's copy of the scratch array, looked up once per
// device with that device current; nullptr if the lookup fails or the device id is beyond
// the table of kScratchDevices devices.
void* scratch_region();

constexpr int kScratchDevices = 64;

}  // namespace pkv

// Fixed device scratch of the allocation-free entry point (la_decode_noalloc):
// one array per device, holding the lean exchange that a per-stream workspace
// holds otherwise.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kernels.h"

namespace la {

// Layout of the scratch array, in bytes from its start:
//   [0, 4 kCtlWords)      control block (kCtl* words, per-CU counters included)
//   [kScratchFlagsOff, + 4 G_max)  flags, one per workgroup
//   [kScratchPartOff, +kScratchPartBytes)  partial records
constexpr int kScratchMaxGrid = 2048;
constexpr size_t kScratchFlagsOff = sizeof(uint32_t) * kCtlWords;
constexpr size_t kScratchPartOff = kScratchFlagsOff + sizeof(uint32_t) * kScratchMaxGrid;
constexpr size_t kScratchPartBytes = size_t(8) << 20;
constexpr size_t kScratchBytes = kScratchPartOff + kScratchPartBytes;
static_assert(kScratchPartOff % 256 == 0, "records start on a 256-byte boundary");

constexpr int kMaxDevices = 64;

// The device address of `dev`'s scratch array. The first call for a device
// (which must be the current one) looks the address up and clears the control
// block and flags with a fill kernel on `stream`; later calls return the
// stored address. Thread-safe.
hipError_t scratch_setup(int dev, hipStream_t stream, void** base);

// The address scratch_setup stored for `dev`, or null if it has not run.
void* scratch_base(int dev);

}  // namespace la

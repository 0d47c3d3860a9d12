// A 64-bit value as two 32-bit halves and back: the form in which a
// wave-uniform 64-bit value (an address, a tile index) passes through the
// 32-bit wave broadcast (readfirstlane), which takes and returns a signed int.
// Each half is taken as uint32_t before widening: a low half with bit 31 set
// widened as a signed int would fill the high word with ones. Plain C++ (no
// HIP types), so that the host test suite compiles and checks it as is.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define DCP_HOST_DEVICE __host__ __device__
#else
#define DCP_HOST_DEVICE
#endif

namespace dcp {

DCP_HOST_DEVICE inline constexpr int low_half(uint64_t v) { return static_cast<int>(static_cast<uint32_t>(v)); }
DCP_HOST_DEVICE inline constexpr int high_half(uint64_t v) { return static_cast<int>(static_cast<uint32_t>(v >> 32)); }
DCP_HOST_DEVICE inline constexpr uint64_t join_halves(int lo, int hi) {
  return static_cast<uint64_t>(static_cast<uint32_t>(lo)) | (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32);
}

}  // namespace dcp

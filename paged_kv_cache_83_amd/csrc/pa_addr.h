// Address arithmetic shared by host and device code (plain constexpr C++, so
// the host compiler builds it too and the CPU tests check it directly).
#pragma once

#include <cstdint>

namespace pa_detail {

// A 64-bit address from its two 32-bit words, as readfirstlane returns them
// when a wave-uniform address is pinned to scalar registers. Both words are
// widened as unsigned: a low word with bit 31 set must not be sign-extended
// into the high word (which would point 4 GiB below the address, or far
// outside the allocation).
constexpr uint64_t join_address_words(uint32_t hi, uint32_t lo) {
  return (static_cast<uint64_t>(hi) << 32) | static_cast<uint64_t>(lo);
}

}  // namespace pa_detail

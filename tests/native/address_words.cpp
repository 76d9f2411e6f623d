// CPU check of the scalar-base composition the prefill tile kernel uses for its
// global-to-LDS loads (pa_addr.h): every address survives the split into two
// 32-bit words and the join, including low words with bit 31 set; the
// composition that sign-extends the low word (the faulty form) is shown to fail
// on exactly those, so this check would have caught it.
#include <cstdint>
#include <cstdio>

#include "../../paged_kv_cache_83_amd/csrc/pa_addr.h"

using pa_detail::join_address_words;

static uint64_t join_sign_extended(uint32_t hi, uint32_t lo) {
  return (static_cast<uint64_t>(hi) << 32) | static_cast<uint64_t>(static_cast<int64_t>(static_cast<int32_t>(lo)));
}

int main() {
  static_assert(join_address_words(0x7f12u, 0x80000000u) == 0x00007f1280000000ull, "bit 31");
  static_assert(join_address_words(0u, 0xffffffffu) == 0x00000000ffffffffull, "all ones");
  const uint64_t bases[] = {0x00007f0000000000ull, 0x00007fa2c0000000ull, 0x0000700012345000ull,
                            0x00007ffe7fff0000ull};
  long checked = 0, bad = 0, sign_ext_wrong = 0, bit31 = 0;
  for (uint64_t base : bases) {
    // 4 KiB tiles across 16 GiB: every low-word pattern class, both halves of the 32-bit range
    for (uint64_t off = 0; off < (16ull << 30); off += 4096 * 997) {
      const uint64_t a = base + off;
      const uint32_t hi = static_cast<uint32_t>(a >> 32), lo = static_cast<uint32_t>(a);
      ++checked;
      if (join_address_words(hi, lo) != a) ++bad;
      const bool high_bit = (lo >> 31) != 0;
      bit31 += high_bit;
      if ((join_sign_extended(hi, lo) != a) != high_bit) ++bad;   // fails exactly when bit 31 is set
      sign_ext_wrong += join_sign_extended(hi, lo) != a;
    }
  }
  std::printf("checked %ld addresses, %ld with bit 31 of the low word set, sign-extending join wrong on %ld, failures %ld\n",
              checked, bit31, sign_ext_wrong, bad);
  return (bad == 0 && bit31 > 0 && sign_ext_wrong == bit31) ? 0 : 1;
}

// Host check of the plane -> code rebuild against a bit-by-bit reference.
// Built with hipcc as a host program; needs no GPU.
#include <stdio.h>
#include <stdlib.h>

#include "bitplane.hpp"

static uint32_t lcg(uint64_t& s) {
  s = s * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(s >> 33);
}

int main() {
  uint64_t seed = 12345;
  long checked = 0;
  for (int trial = 0; trial < 20000; ++trial) {
    uint8_t code[32];
    for (int c = 0; c < 32; ++c) code[c] = (uint8_t)lcg(seed);
    // Pack the word exactly as the store defines it: column 4m + j at bit 8j + m of plane p (code bit 7 - p).
    uint32_t w[8] = {0};
    for (int p = 0; p < 8; ++p)
      for (int c = 0; c < 32; ++c) {
        const int m = c / 4, j = c % 4;
        if ((code[c] >> (7 - p)) & 1) w[p] |= 1u << (8 * j + m);
      }
    for (int b = 0; b <= 8; ++b) {
      uint32_t wb[8];
      for (int p = 0; p < 8; ++p) wb[p] = p < b ? w[p] : 0u;   // planes a reader did not fetch are 0
      uint32_t d[8];
      grinqh::planes_to_codes_rt(b, wb, d);
      uint32_t d8[8];
      grinqh::planes_to_codes<8>(wb, d8);                      // the generic network agrees
      // the VMM's choice: the 2-plane network for b <= 2, the 3-plane one for
      // b = 3 and the full one above, always with the missing planes zero
      uint32_t dv[8];
      if (b <= 2) grinqh::planes_to_codes<2>(wb, dv);
      else if (b == 3) grinqh::planes_to_codes<3>(wb, dv);
      else grinqh::planes_to_codes<8>(wb, dv);
      const unsigned mask = b == 0 ? 0u : (0xFFu << (8 - b)) & 0xFFu;
      for (int c = 0; c < 32; ++c) {
        const int m = c / 4, j = c % 4;
        const unsigned got = (d[m] >> (8 * j)) & 0xFFu;
        const unsigned got8 = (d8[m] >> (8 * j)) & 0xFFu;
        const unsigned gotv = (dv[m] >> (8 * j)) & 0xFFu;
        const unsigned want = code[c] & mask;
        if (got != want || got8 != want || gotv != want) {
          printf("FAIL trial %d b %d col %d: got %02x/%02x/%02x want %02x\n", trial, b, c, got, got8, gotv, want);
          return 1;
        }
        ++checked;
      }
    }
  }
  printf("bitplane rebuild ok (%ld codes)\n", checked);
  return 0;
}

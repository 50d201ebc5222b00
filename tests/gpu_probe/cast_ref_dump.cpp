// Host build of cast_ref.hpp (test infrastructure): reads fp32 bit patterns as
// little-endian uint32 from stdin, writes one E4M3 code byte and one bf16 uint16
// per input to stdout.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "cast_ref.hpp"

int main() {
  std::vector<uint32_t> in;
  uint32_t u;
  while (fread(&u, 4, 1, stdin) == 1) in.push_back(u);
  for (uint32_t v : in) {
    const uint8_t c = (uint8_t)castref::e4m3_code(v);
    fwrite(&c, 1, 1, stdout);
  }
  for (uint32_t v : in) {
    const uint16_t b = (uint16_t)castref::bf16_bits(v);
    fwrite(&b, 2, 1, stdout);
  }
  return 0;
}

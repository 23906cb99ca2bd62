// Host build of the kernels' scalar helpers, driven by tests/test_host_helpers.py.
// Reads commands from stdin:  "r <double-hex-bits> <up>"  -> bf16 bits
//                             "t <u64-hex>"                -> transpose8
//                             "h <u64-hex>"                -> transpose8_halves
//                             "p <a> <b> <sel>"            -> perm_bytes
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "bitops.h"

int main() {
  char op;
  while (std::scanf(" %c", &op) == 1) {
    if (op == 'r') {
      unsigned long long bits;
      int up;
      if (std::scanf("%llx %d", &bits, &up) != 2) return 1;
      double v;
      std::memcpy(&v, &bits, 8);
      std::printf("%x\n", readkv::bf16_round_dir(v, up != 0));
    } else if (op == 'h') {
      unsigned long long x;
      if (std::scanf("%llx", &x) != 1) return 1;
      uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
      readkv::transpose8_halves(lo, hi);
      std::printf("%llx\n", ((unsigned long long)hi << 32) | lo);
    } else if (op == 'p') {
      unsigned a, b, sel;
      if (std::scanf("%x %x %x", &a, &b, &sel) != 3) return 1;
      std::printf("%x\n", readkv::perm_bytes(a, b, sel));
    } else if (op == 't') {
      unsigned long long x;
      if (std::scanf("%llx", &x) != 1) return 1;
      std::printf("%llx\n", (unsigned long long)readkv::transpose8(x));
    }
  }
  return 0;
}

// Host check of the address split/join helpers (addr_words.h), built with g++ by
// tests/test_addr_words.py: every address comes back whole, also when its words pass through
// an int (what the lane-broadcast builtin returns) on the way, and joining a sign-extended low
// word the naive way would corrupt the high word for every low word >= 2^31.
#include <cstdio>

#include "addr_words.h"

using namespace dm;

int main() {
  const unsigned long long highs[] = {0ull, 1ull, 0x7full, 0x7fffull, 0xffffull, 0x7fffffffull};
  const unsigned lows[] = {0u, 1u, 0x1000u, 0x7fffffffu, 0x80000000u, 0x80000001u, 0x9abcdef0u, 0xfffff000u, 0xffffffffu};
  int fails = 0, naive_broken = 0, high_low = 0;
  for (unsigned long long h : highs)
    for (unsigned l : lows) {
      const unsigned long long a = (h << 32) | l;
      if (addr_join(addr_lo(a), addr_hi(a)) != a) ++fails;
      const int li = (int)addr_lo(a), hi = (int)addr_hi(a);  // as readfirstlane hands them back
      if (addr_join((unsigned)li, (unsigned)hi) != a) ++fails;
      const unsigned long long naive = ((unsigned long long)(unsigned)hi << 32) | (unsigned long long)(long long)li;
      if (l >= 0x80000000u) {
        ++high_low;
        if (naive != a) ++naive_broken;
      } else if (naive != a) {
        ++fails;
      }
    }
  printf("%d round-trip failures; the naive join breaks %d of %d addresses with a low word >= 2^31\n", fails,
         naive_broken, high_low);
  return (fails == 0 && naive_broken == high_low && high_low > 0) ? 0 : 1;
}

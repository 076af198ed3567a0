// Host check of the 8-bit AdamW kernel's code search: for every float a in
// [0, 1 + 4 ulp] the direct search (octave table, linear estimate within a
// decade, a three-entry window) returns the same code as a plain bisection of
// the same book followed by the nearer-neighbour rule (ties to the smaller
// magnitude).  Built with hipcc from the kernel's own source; the search is a
// host-callable function there.  Prints one line per book and exits non-zero
// on any mismatch.
#include "gq_adamw8bit.hip"

#include <cmath>
#include <cstdio>
#include <cstring>

using namespace gq::adamw8;

template <int N>
static int bisect_nearest(const float* book, float a) {
  int lo = 0;  // largest k with book[k] <= a
  for (int step = N / 2; step > 0; step >>= 1)
    if (lo + step < N && book[lo + step] <= a) lo += step;
  if (lo + 1 < N && book[lo + 1] - a < a - book[lo]) return lo + 1;
  return lo;
}

template <int BITS>
static long check(uint32_t last) {
  constexpr int N = 1 << BITS;
  constexpr CodeBook cb = make_book(BITS);
  constexpr DecadeTable dt = make_decades(BITS);
  constexpr OctaveTable ot = make_octaves(BITS);
  float book[N + PAD];
  for (int i = 0; i < N; ++i) book[i] = cb.v[i];
  for (int i = 0; i < PAD; ++i) book[N + i] = INFINITY;
  long bad = 0;
  for (uint32_t u = 0;; ++u) {
    float a;
    std::memcpy(&a, &u, 4);
    const int x = nearest_code<BITS>(book, ot.o, dt.d, a), y = bisect_nearest<N>(book, a);
    if (x != y && bad++ < 5) std::printf("  %d-bit book: a = %.9g direct %d bisection %d\n", BITS, a, x, y);
    if (u == last) break;
  }
  std::printf("%d-bit book: %ld mismatches over %u floats\n", BITS, bad, last + 1);
  return bad;
}

int main() {
  const uint32_t last = 0x3f800004u;  // 1.0f plus four ulps
  const long bad = check<7>(last) + check<8>(last);
  return bad ? 1 : 0;
}

// Host check of the library's fp64 exponential (exp2_neg in sv_device.hpp)
// against long-double exp2l.  Built and run by test_device_math.py; prints
// "max_rel <value> zero_ok <0|1> count <n>".
#include <cmath>
#include <cstdio>

#include "sv_device.hpp"

int main() {
  long double worst = 0.0L;
  long count = 0;
  auto check = [&](double t) {
    const double got = sv::exp2_neg(t);
    const long double ref = exp2l(static_cast<long double>(t));
    if (ref < 0x1p-1022L) return;  // the final scaling rounds denormal results
    const long double rel = fabsl((static_cast<long double>(got) - ref) / ref);
    if (rel > worst) worst = rel;
    ++count;
  };
  // a dense sweep of [-64, 0], then the whole range down to the normal limit,
  // and points next to every integer and half-integer (|f| largest there)
  for (long i = 0; i <= 4000000; ++i) check(-64.0 * static_cast<double>(i) / 4000000.0);
  for (long i = 0; i <= 1000000; ++i) check(-1021.0 * static_cast<double>(i) / 1000000.0);
  for (int k = 0; k <= 1021; ++k)
    for (double d : {-1e-12, 0.0, 1e-12})
      for (double h : {0.0, 0.5}) check(-static_cast<double>(k) - h + d);
  const bool zero_ok = sv::exp2_neg(-INFINITY) == 0.0 && sv::exp2_neg(-5000.0) == 0.0 && sv::exp2_neg(0.0) == 1.0;
  std::printf("max_rel %.6Le zero_ok %d count %ld\n", worst, zero_ok ? 1 : 0, count);
  return 0;
}

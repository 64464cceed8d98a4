// Host check of the library's table-based fp64 exponential (exp2_tab in
// sv_device.hpp) against long-double exp2l.  Built and run by
// test_device_math.py; prints "max_rel <value> zero_ok <0|1> count <n>".
#include <cmath>
#include <cstdio>

#include "sv_device.hpp"

int main() {
  sv::Exp2Table tab;
  for (int j = 0; j < 64; ++j) tab.v[j] = sv::exp2_table_entry(j);
  long double worst = 0.0L;
  long count = 0;
  auto check = [&](double t) {
    const double got = sv::exp2_tab(t, tab);
    const long double ref = exp2l(static_cast<long double>(t));
    if (ref < 0x1p-1022L) return;  // the final scaling rounds denormal results
    const long double rel = fabsl((static_cast<long double>(got) - ref) / ref);
    if (rel > worst) worst = rel;
    ++count;
  };
  // a dense sweep of [-64, 0], then the whole range down to the normal limit,
  // and points next to every table knot and half-knot
  for (long i = 0; i <= 4000000; ++i) check(-64.0 * static_cast<double>(i) / 4000000.0);
  for (long i = 0; i <= 1000000; ++i) check(-1021.0 * static_cast<double>(i) / 1000000.0);
  for (int k = 0; k <= 64 * 40; ++k)
    for (double d : {-1e-12, 0.0, 1e-12})
      for (double h : {0.0, 1.0 / 128.0}) check(-(k / 64.0) - h + d);
  const bool zero_ok = sv::exp2_tab(-INFINITY, tab) == 0.0 && sv::exp2_tab(-5000.0, tab) == 0.0 &&
                       sv::exp2_tab(0.0, tab) == 1.0;
  std::printf("max_rel %.6Le zero_ok %d count %ld\n", worst, zero_ok ? 1 : 0, count);
  return 0;
}

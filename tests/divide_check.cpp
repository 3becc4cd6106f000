// Host harness for the library's float32 divide-by-scale helper (pa_divide.h):
// reads (x, s) float32 pairs from stdin, writes div_rn(x, s) as float32 to
// stdout. Built and driven by tests/test_divide_host.py.
#include <cstdio>
#include <vector>

#include "pa_divide.h"

int main() {
  std::vector<float> buf(2 * 4096);
  size_t n;
  while ((n = fread(buf.data(), sizeof(float), buf.size(), stdin)) > 0) {
    std::vector<float> out(n / 2);
    for (size_t i = 0; i + 1 < n; i += 2) {
      const pa::Divisor d = pa::make_divisor(buf[i + 1]);
      out[i / 2] = pa::div_rn(buf[i], d);
    }
    fwrite(out.data(), sizeof(float), out.size(), stdout);
  }
  return 0;
}

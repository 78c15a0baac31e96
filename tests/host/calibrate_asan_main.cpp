// Host-only driver for the calibration code under AddressSanitizer and
// UndefinedBehaviorSanitizer: random keys with a known per-axis variance,
// several sizes (including D = 1 and n = 2), and the argument checks.
// Exit status 0 when every call behaved.
#include <cmath>
#include <cstdio>
#include <random>
#include <vector>

#include "loki.h"

int main() {
  std::mt19937_64 gen(7);
  std::normal_distribution<double> nd(0.0, 1.0);
  const int dims[] = {1, 2, 7, 64, 128};
  for (int D : dims) {
    for (int64_t n : {int64_t(2), int64_t(3), int64_t(500)}) {
      std::vector<float> keys(static_cast<size_t>(n) * D);
      for (int64_t i = 0; i < n; ++i)
        for (int m = 0; m < D; ++m) keys[i * D + m] = static_cast<float>(nd(gen) * std::exp(-m / 8.0));
      std::vector<float> P(static_cast<size_t>(D) * D, -1.f);
      std::vector<double> ev(D, -1.0);
      if (loki_calibrate(keys.data(), n, D, P.data(), ev.data()) != LOKI_OK) return 1;
      for (int i = 1; i < D; ++i)
        if (ev[i] > ev[i - 1] + 1e-12) return 2;
      // columns of P are unit vectors
      for (int c = 0; c < D; ++c) {
        double s = 0.0;
        for (int m = 0; m < D; ++m) s += static_cast<double>(P[m * D + c]) * P[m * D + c];
        if (std::fabs(s - 1.0) > 1e-5) return 3;
      }
      if (loki_calibrate(keys.data(), n, D, P.data(), nullptr) != LOKI_OK) return 4;
    }
  }
  std::vector<float> k(8, 1.f), P(4);
  if (loki_calibrate(nullptr, 4, 2, P.data(), nullptr) != LOKI_EINVAL) return 5;
  if (loki_calibrate(k.data(), 1, 2, P.data(), nullptr) != LOKI_EINVAL) return 6;
  if (loki_calibrate(k.data(), 4, 0, P.data(), nullptr) != LOKI_EINVAL) return 7;
  if (loki_calibrate(k.data(), 4, 2, nullptr, nullptr) != LOKI_EINVAL) return 8;
  std::puts("ok");
  return 0;
}

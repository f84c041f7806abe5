// Host-only check of the multiply-high divider the kernels use to split a flat
// index into (row, column): for each divisor, FastDiv::make's constants must
// give floor(n / d) for every n < 2^31 (the kernels' indices stay below 2^30
// by their launch splits). __umulhi(n, m) is the high 32 bits of the 64-bit
// product, evaluated here on the host. Prints the number of mismatches.
#include <cstdio>
#include <cstdint>
#include "../microscaling_block_scaled_amd/csrc/mx_common.hpp"

static uint32_t host_div(const mx::FastDiv& f, uint32_t n) {
  return f.m ? (uint32_t)(((uint64_t)n * f.m) >> 32) >> f.s : n >> f.s;
}

int main() {
  uint64_t bad = 0, checked = 0, lcg = 0x9E3779B97F4A7C15ull;
  auto rnd = [&]() { lcg = lcg * 6364136223846793005ull + 1442695040888963407ull; return (uint32_t)(lcg >> 33); };
  auto check_d = [&](uint32_t d) {
    const mx::FastDiv f = mx::FastDiv::make(d);
    auto one = [&](uint32_t n) {
      if (n >= (1u << 31)) return;
      ++checked;
      if (host_div(f, n) != n / d) {
        if (bad < 10) printf("d=%u n=%u got %u want %u\n", d, n, host_div(f, n), n / d);
        ++bad;
      }
    };
    const uint32_t top = (1u << 31) - 1;
    for (uint32_t n : {0u, 1u, d - 1, d, d + 1, 2 * d - 1, top, top - 1, top - d}) one(n);
    const uint32_t kmax = top / d;
    for (uint32_t k : {kmax, kmax - 1, kmax / 2, kmax / 3}) { one(k * d); one(k * d - 1); one(k * d + d - 1); }
    for (int i = 0; i < 2000; ++i) one(rnd());
    for (int i = 0; i < 200; ++i) { const uint32_t k = rnd() % (kmax + 1); one(k * d); one(k * d - 1); }
  };
  for (uint32_t d = 1; d <= 8192; ++d) check_d(d);
  for (int l = 13; l <= 30; ++l)
    for (int64_t e = -3; e <= 3; ++e) check_d((uint32_t)((1ll << l) + e));
  for (int i = 0; i < 20000; ++i) check_d(1 + rnd() % (1u << 30));
  printf("checked %llu quotients, %llu wrong\n", (unsigned long long)checked, (unsigned long long)bad);
  return bad ? 1 : 0;
}

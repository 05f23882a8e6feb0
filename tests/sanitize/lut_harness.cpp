// Runs the library's lookup-table parser and matcher (host code, built on its
// own with AddressSanitizer and UndefinedBehaviorSanitizer) over the packaged
// table, the built-in text, and truncated and mutated tables.
#include <cstdio>
#include <cstdlib>
#include <fstream>
#include <sstream>
#include <string>

#include "bsa_lut.h"

namespace bsa {
static thread_local std::string g_err;
bsa_status fail(bsa_status s, const std::string &msg) {
  g_err = msg;
  return s;
}
}  // namespace bsa

static uint64_t rng = 0x2545f4914f6cdd1dull;
static uint32_t next_u32() {
  rng ^= rng << 13, rng ^= rng >> 7, rng ^= rng << 17;
  return (uint32_t)(rng >> 16);
}

int main(int argc, char **argv) {
  if (argc < 2) return 2;
  std::ifstream f(argv[1]);
  std::stringstream ss;
  ss << f.rdbuf();
  const std::string packaged = ss.str();
  int failures = 0;
  bsa::LutTable t;
  if (bsa::parse_lut(packaged.c_str(), &t) != BSA_OK || t.rules.empty()) ++failures;
  bsa::LutTable t2;
  if (bsa::parse_lut(bsa::kDefaultLutText, &t2) != BSA_OK || t2.rules.size() != t.rules.size()) ++failures;
  // every rule set answers some random queries
  for (int i = 0; i < 2000; ++i) {
    const int64_t key[4] = {next_u32() % 2 ? 64 : 128, next_u32() % 2, next_u32() % 2, next_u32() % 2};
    const int64_t val[5] = {16 << (next_u32() % 6), 16 << (next_u32() % 6), next_u32() % 1001,
                            next_u32() % 100000, next_u32() % 200000};
    bsa::Regime r;
    if (!bsa::lut_match(t, key, val, &r)) ++failures;  // the packaged table ends in a catch-all
  }
  // truncations and mutations: OK or BSA_ERR_LUT, never anything else
  std::string buf;
  for (size_t cut = 0; cut <= packaged.size(); cut += 7) {
    buf = packaged.substr(0, cut);
    bsa::LutTable x;
    const bsa_status s = bsa::parse_lut(buf.c_str(), &x);
    if (s != BSA_OK && s != BSA_ERR_LUT) ++failures;
  }
  const char alphabet[] = " \n#*->0123456789abcdefghijklmnopqrstuvwxyz-+9999999999999999999999";
  for (int it = 0; it < 3000; ++it) {
    buf = packaged;
    const int nmut = 1 + next_u32() % 4;
    for (int m = 0; m < nmut; ++m) {
      const size_t at = next_u32() % buf.size();
      switch (next_u32() % 3) {
        case 0: buf[at] = alphabet[next_u32() % (sizeof alphabet - 1)]; break;
        case 1: buf.erase(at, 1 + next_u32() % 8); break;
        default: buf.insert(at, std::string(1 + next_u32() % 30, alphabet[next_u32() % (sizeof alphabet - 1)]));
      }
      if (buf.empty()) buf = "x";
    }
    bsa::LutTable x;
    const bsa_status s = bsa::parse_lut(buf.c_str(), &x);
    if (s != BSA_OK && s != BSA_ERR_LUT) ++failures;
    const int64_t key[4] = {128, 0, 0, 0}, val[5] = {64, 64, 100, 16, 1000};
    bsa::Regime r;
    (void)bsa::lut_match(x, key, val, &r);
  }
  if (failures) {
    std::fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  std::printf("lut harness ok\n");
  return 0;
}

// Regime lookup table: text parser and rule matching (host code only, no
// HIP; also built on its own, with sanitizers, by the CPU tests).
//
// Tessera (abstract): plan selection by profile-guided regime choice through
// a lookup table built from offline profiling. A rule matches the problem's
// key (head dim, dtype, union, paged) and ranges over mask-shape features;
// the first matching rule gives the regime (Tq, Tk, schedule, split, pack).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "bsa.h"

namespace bsa {

struct Regime {
  int tq = 128, tk = 64, sched = 0, split = 0, pack = 1;
};

struct LutRule {
  int64_t key[4];        // D, dtype, union, paged (-1 = any)
  int64_t lo[5], hi[5];  // min bq, min bk, density per mille, imbalance x16, Sq (version 2)
  Regime r;
};

struct LutTable {
  std::vector<LutRule> rules;
};

// Records msg as the calling thread's last error and returns s.
bsa_status fail(bsa_status s, const std::string &msg);

// Parses the text format of bsa.h into *out (rules appended). BSA_ERR_LUT
// with a message on malformed text.
bsa_status parse_lut(const char *text, LutTable *out);

// First rule of t matching key = {D, dtype, union, paged} and
// val = {min bq, min bk, density per mille, imbalance x16, Sq}; false if none.
bool lut_match(const LutTable &t, const int64_t key[4], const int64_t val[5], Regime *out);

// Text of the packaged table, compiled into the library (the built-in
// default of bsa_lut_load).
extern const char *const kDefaultLutText;

}  // namespace bsa

// The opaque table handle of the C ABI.
struct bsa_lut_s : public bsa::LutTable {};

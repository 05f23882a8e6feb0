// Regime lookup table: text parser and first-match lookup (host code only).
// Format and semantics are stated at bsa_lut_load in bsa.h.
#include "bsa_lut.h"

#include <cerrno>
#include <climits>
#include <cstdlib>
#include <sstream>

namespace bsa {

#include "bsa_lut_default.inc"

static bool parse_i64(const std::string &t, int64_t *out) {
  if (t.empty()) return false;
  char *end = nullptr;
  errno = 0;
  const long long v = std::strtoll(t.c_str(), &end, 10);
  if (*end || errno == ERANGE) return false;
  *out = v;
  return true;
}

bsa_status parse_lut(const char *text, LutTable *lut) {
  // Tokenise, dropping '#' comments.
  std::vector<std::string> tok;
  std::istringstream lines(text);
  std::string line;
  while (std::getline(lines, line)) {
    const size_t hash = line.find('#');
    if (hash != std::string::npos) line.resize(hash);
    std::istringstream ws(line);
    std::string t;
    while (ws >> t) tok.push_back(t);
  }
  size_t i = 0;
  auto next = [&](std::string &t) {
    if (i >= tok.size()) return false;
    t = tok[i++];
    return true;
  };
  std::string t;
  int64_t x;
  if (!next(t) || t != "bsa-lut" || !next(t) || !parse_i64(t, &x) || (x != 1 && x != 2))
    return fail(BSA_ERR_LUT, "lookup table must start with 'bsa-lut 1' or 'bsa-lut 2'");
  const int nranges = x == 2 ? 5 : 4;  // version 2 adds a range on the query length
  while (next(t)) {
    if (t != "rule") return fail(BSA_ERR_LUT, "expected 'rule', got '" + t + "'");
    LutRule r{};
    for (int f = 0; f < 4; ++f) {
      if (!next(t)) return fail(BSA_ERR_LUT, "truncated rule");
      if (t == "*") r.key[f] = -1;
      else if (f == 1 && t == "bf16") r.key[f] = BSA_BF16;
      else if (f == 1 && t == "f32") r.key[f] = BSA_F32;
      else if (f != 1 && parse_i64(t, &x) && x >= 0) r.key[f] = x;
      else return fail(BSA_ERR_LUT, "bad rule key '" + t + "'");
    }
    r.lo[4] = 0, r.hi[4] = INT64_MAX;
    for (int f = 0; f < nranges; ++f) {
      if (!next(t) || !parse_i64(t, &r.lo[f]) || !next(t) || !parse_i64(t, &r.hi[f]))
        return fail(BSA_ERR_LUT, "bad rule range");
    }
    if (!next(t) || t != "->") return fail(BSA_ERR_LUT, "expected '->' in rule");
    int64_t v[5];
    for (int f = 0; f < 5; ++f) {
      if (!next(t)) return fail(BSA_ERR_LUT, "truncated rule");
      if (f == 2 && t == "local") v[f] = 0;
      else if (f == 2 && t == "lpt") v[f] = 1;
      else if (f == 2 && t == "dealt") v[f] = 2;
      else if (f == 2 || !parse_i64(t, &v[f])) return fail(BSA_ERR_LUT, "bad regime value '" + t + "'");
    }
    if ((v[0] != 128 && v[0] != 256) || (v[1] != 64 && v[1] != 128) || v[3] < 0 ||
        v[3] > (1 << 30) || v[4] < 0 || v[4] > 2)
      return fail(BSA_ERR_LUT, "regime out of range (Tq 128|256, Tk 64|128, split >= 0, pack 0|1|2)");
    r.r = Regime{(int)v[0], (int)v[1], (int)v[2], (int)v[3], (int)v[4]};
    lut->rules.push_back(r);
  }
  return BSA_OK;
}

bool lut_match(const LutTable &t, const int64_t key[4], const int64_t val[5], Regime *out) {
  for (const LutRule &r : t.rules) {
    bool ok = true;
    for (int f = 0; f < 4; ++f)
      if (r.key[f] >= 0 && r.key[f] != key[f]) ok = false;
    for (int f = 0; f < 5; ++f)
      if (val[f] < r.lo[f] || val[f] > r.hi[f]) ok = false;
    if (ok) {
      *out = r.r;
      return true;
    }
  }
  return false;
}

}  // namespace bsa

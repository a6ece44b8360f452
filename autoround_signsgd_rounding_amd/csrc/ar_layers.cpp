// Per-layer quantization config resolution (host code): the rules of the
// SGLang AutoRound page, "2. 레이어별 개별 설정", "3. 정규식 기반 레이어 매칭" and
// "4. FusedMoE와 Fused QKV 처리".
//   - no rules: the defaults, or (bits 16, group -1, sym 1) for a layer outside
//     the quantized set (16 bits = leave unquantized);
//   - a rule whose key equals the layer name: its fields, unset ones from the
//     defaults (from (16, -1, 1) outside the quantized set);
//   - else the first rule whose key contains a regular-expression special
//     character and matches the whole name: its fields, unset ones from the
//     defaults; keys that do not compile are skipped;
//   - else as with no rules.
// A fused layer's sub-layers must all resolve to the same config.
// Patterns use the ECMAScript grammar of std::regex; the pages' Python `re`
// agrees with it on the constructs layer-name patterns use (literals, '.',
// escapes, classes, groups, alternation, repetition, anchors).
#include <algorithm>
#include <cstring>
#include <regex>
#include <string>

#include "../../include/autoround_hip.h"

namespace {

// A key is a pattern when it holds a regular-expression special character.
bool has_special(const char* key) { return std::strpbrk(key, "*+?^$()[]{}|\\") != nullptr; }

// True when key is a pattern that compiles and matches all of name.
bool whole_name_match(const char* key, const char* name) {
  if (!has_special(key)) return false;
  try {
    return std::regex_match(name, std::regex(key, std::regex::ECMAScript));
  } catch (const std::regex_error&) {
    return false;
  }
}

ar_layer_qconfig unquantized() {
  ar_layer_qconfig c;
  c.bits = 16;
  c.group_size = -1;
  c.sym = 1;
  return c;
}

ar_layer_qconfig fill(const ar_layer_rule& r, const ar_layer_qconfig& base) {
  ar_layer_qconfig c;
  c.bits = r.bits >= 0 ? r.bits : base.bits;
  c.group_size = r.group_size != 0 ? r.group_size : base.group_size;
  c.sym = r.sym >= 0 ? (r.sym != 0) : base.sym;
  return c;
}

ar_layer_qconfig resolve(const ar_layer_rule* rules, int32_t n, const ar_layer_qconfig& d,
                         bool quantized, const char* name) {
  const ar_layer_qconfig fallback = quantized ? d : unquantized();
  const ar_layer_rule* end = rules + n;
  const ar_layer_rule* exact = std::find_if(
      rules, end, [&](const ar_layer_rule& r) { return std::strcmp(r.key, name) == 0; });
  if (exact != end) return fill(*exact, fallback);
  const ar_layer_rule* pattern = std::find_if(
      rules, end, [&](const ar_layer_rule& r) { return whole_name_match(r.key, name); });
  return pattern != end ? fill(*pattern, d) : fallback;
}

bool same(const ar_layer_qconfig& a, const ar_layer_qconfig& b) {
  return a.bits == b.bits && a.group_size == b.group_size && a.sym == b.sym;
}

bool rules_ok(const ar_layer_rule* rules, int32_t n) {
  if (n < 0 || (n > 0 && !rules)) return false;
  for (int32_t i = 0; i < n; ++i)
    if (!rules[i].key) return false;
  return true;
}

}  // namespace

extern "C" {

ar_status ar_resolve_layer_config(const ar_layer_rule* rules, int32_t nrules,
                                  const ar_layer_qconfig* defaults, int32_t quantized,
                                  const char* name, ar_layer_qconfig* out) {
  if (!rules_ok(rules, nrules) || !defaults || !name || !out) return AR_ERR_INVALID_ARG;
  try {
    *out = resolve(rules, nrules, *defaults, quantized != 0, name);
  } catch (...) {
    return AR_ERR_INVALID_ARG;
  }
  return AR_OK;
}

ar_status ar_resolve_fused_config(const ar_layer_rule* rules, int32_t nrules,
                                  const ar_layer_qconfig* defaults, int32_t quantized,
                                  const char* layer_name, const char* const* sub_names,
                                  int32_t nsub, ar_layer_qconfig* out) {
  // sub_names given with no entries is an empty sub-layer set: nothing to agree on
  if (!rules_ok(rules, nrules) || !defaults || !layer_name || !out || nsub < 0 ||
      (nsub > 0) != (sub_names != nullptr))
    return AR_ERR_INVALID_ARG;
  try {
    const bool q = quantized != 0;
    bool any = false;
    ar_layer_qconfig first{};
    auto take = [&](const char* nm) {
      const ar_layer_qconfig c = resolve(rules, nrules, *defaults, q, nm);
      if (!any) {
        first = c;
        any = true;
        return true;
      }
      return same(first, c);
    };
    if (nsub > 0) {
      for (int32_t i = 0; i < nsub; ++i) {
        if (!sub_names[i]) return AR_ERR_INVALID_ARG;
        if (!take(sub_names[i])) return AR_ERR_INVALID_ARG;
      }
    } else {
      const std::string prefix(layer_name);
      for (int32_t i = 0; i < nrules; ++i) {
        if (std::string(rules[i].key).compare(0, prefix.size(), prefix) != 0) continue;
        if (!take(rules[i].key)) return AR_ERR_INVALID_ARG;
      }
      if (!any) first = resolve(rules, nrules, *defaults, q, layer_name);
    }
    *out = first;
  } catch (...) {
    return AR_ERR_INVALID_ARG;
  }
  return AR_OK;
}

}  // extern "C"

// Command-line driver of the per-layer config resolvers (csrc/ar_layers.cpp),
// for a host build under AddressSanitizer / UndefinedBehaviorSanitizer.
// Reads tab-separated lines on stdin:
//   R <key> <bits> <group_size> <sym>         append a rule (-1 / 0 / -1 = unset)
//   D <bits> <group_size> <sym>               set the defaults
//   L <quantized> <name>                      ar_resolve_layer_config
//   F <quantized> <layer> <nsub> [<sub>...]   ar_resolve_fused_config
//                                             (nsub -1: sub_names NULL)
// and prints one line per L / F query: "<bits> <group_size> <sym>", or
// "ERR <status>".
#include <cstdio>
#include <iostream>
#include <string>
#include <vector>

#include "../include/autoround_hip.h"

// Fields between tabs, empty ones included (an empty name is a valid query).
static std::vector<std::string> split_tabs(const std::string& line) {
  std::vector<std::string> out;
  size_t start = 0;
  for (;;) {
    const size_t tab = line.find('\t', start);
    out.push_back(line.substr(start, tab == std::string::npos ? std::string::npos : tab - start));
    if (tab == std::string::npos) break;
    start = tab + 1;
  }
  return out;
}

static void print(ar_status s, const ar_layer_qconfig& c) {
  if (s != AR_OK)
    std::printf("ERR %d\n", (int)s);
  else
    std::printf("%d %d %d\n", c.bits, c.group_size, c.sym);
}

int main() {
  std::vector<std::string> keys;   // owns the key strings of the rules
  std::vector<ar_layer_rule> rules;
  std::vector<int> fields;
  ar_layer_qconfig defaults{4, 128, 0};
  std::string line;
  while (std::getline(std::cin, line)) {
    const std::vector<std::string> f = split_tabs(line);
    if (f.empty()) continue;
    if (f[0] == "R" && f.size() == 5) {
      keys.push_back(f[1]);
      fields.push_back(std::stoi(f[2]));
      fields.push_back(std::stoi(f[3]));
      fields.push_back(std::stoi(f[4]));
      rules.clear();
      for (size_t i = 0; i < keys.size(); ++i)
        rules.push_back(ar_layer_rule{keys[i].c_str(), fields[3 * i], fields[3 * i + 1],
                                      fields[3 * i + 2]});
    } else if (f[0] == "D" && f.size() == 4) {
      defaults = ar_layer_qconfig{std::stoi(f[1]), std::stoi(f[2]), std::stoi(f[3])};
    } else if (f[0] == "L" && f.size() == 3) {
      ar_layer_qconfig out{};
      print(ar_resolve_layer_config(rules.data(), (int32_t)rules.size(), &defaults,
                                    std::stoi(f[1]), f[2].c_str(), &out),
            out);
    } else if (f[0] == "F" && f.size() >= 4) {
      const int nsub = std::stoi(f[3]);
      std::vector<const char*> subs;
      for (size_t i = 4; i < f.size(); ++i) subs.push_back(f[i].c_str());
      // an empty list still passes a non-NULL array, as a caller with a vector would
      const char* none[1] = {nullptr};
      const char* const* names = nsub < 0 ? nullptr : (subs.empty() ? none : subs.data());
      ar_layer_qconfig out{};
      print(ar_resolve_fused_config(rules.data(), (int32_t)rules.size(), &defaults,
                                    std::stoi(f[1]), f[2].c_str(), names, nsub < 0 ? 0 : nsub,
                                    &out),
            out);
    } else {
      std::fprintf(stderr, "bad line: %s\n", line.c_str());
      return 2;
    }
  }
  return 0;
}

// Host-code driver for the sanitizer tests: builds the planner and the C ABI's
// argument validation (kda_plan.cpp, kda_validate.cpp) with a host compiler
// and -fsanitize=address,undefined, and runs the cases it reads from stdin,
// one per line:
//   plan N S c_0 .. c_N [b_0 .. b_S]   -> "status w_0 w_1 ..." (the plan blob)
//   check N S c_0 .. c_N H sizes... fmt bound -> "summaries compose carry" statuses
// `check` builds the balanced plan and calls the three validation functions
// with fake, never dereferenced, 16-byte-aligned addresses and the given byte
// counts (in the order of kda_forward's buffers: plan_dev q k v g beta
// initial_state transitions updates carry_in o final_state workspace, then
// o_format and the safe gate's lower bound); nothing is launched.
#include <cstdint>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "kda.h"
#include "kda_internal.h"
#include "kda_validate.h"

namespace {

const void* fake(int i) { return reinterpret_cast<const void*>(static_cast<uintptr_t>(1 << 20) + 256 * i); }

void run_plan(std::istringstream& in) {
  int32_t N, S;
  in >> N >> S;
  std::vector<int32_t> cu(N + 1);
  for (auto& c : cu) in >> c;
  std::vector<int32_t> bounds;
  int32_t b;
  while (in >> b) bounds.push_back(b);
  kda_plan* plan = nullptr;
  const int st = kda_plan_segments(cu.data(), N, S, bounds.empty() ? nullptr : bounds.data(), &plan);
  std::cout << st;
  if (st == KDA_OK) {
    const int32_t* blob = nullptr;
    size_t n = 0;
    kda_plan_blob(plan, &blob, &n);
    for (size_t i = 0; i < n; ++i) std::cout << ' ' << blob[i];
    kda_plan_destroy(plan);
  }
  std::cout << '\n';
}

void run_check(std::istringstream& in) {
  int32_t N, S, H;
  in >> N >> S;
  std::vector<int32_t> cu(N + 1);
  for (auto& c : cu) in >> c;
  in >> H;
  size_t z[13];
  for (auto& x : z) in >> x;
  int32_t fmt;
  in >> fmt;
  std::string bound_text;
  in >> bound_text;
  const float bound = std::stof(bound_text);
  kda_plan* plan = nullptr;
  if (kda_plan_segments(cu.data(), N, S, nullptr, &plan) != KDA_OK) {
    std::cout << "noplan\n";
    return;
  }
  auto u16 = [](int i) { return static_cast<const uint16_t*>(fake(i)); };
  auto f32 = [](int i) { return static_cast<const float*>(fake(i)); };
  const int32_t* pd = static_cast<const int32_t*>(fake(0));
  const int s1 = kda::check_summaries(plan, pd, z[0], u16(2), z[2], u16(3), z[3], u16(4), z[4], u16(5), z[5],
                                      bound, f32(6), z[6], H, 128, 128, 0, H, f32(7), z[7], f32(8), z[8], fake(12), z[12]);
  const int s2 = kda::check_compose(plan, pd, z[0], f32(7), z[7], f32(8), z[8], H, 128, 128, 0, H, f32(9), z[9]);
  const int s3 = kda::check_carry(plan, pd, z[0], u16(1), z[1], u16(2), z[2], u16(3), z[3], u16(4), z[4], u16(5),
                                  z[5], bound, f32(6), z[6], H, 128, 128, 0, H, f32(9), z[9], fake(10), z[10], fmt,
                                  f32(11), z[11], fake(12), z[12]);
  std::cout << s1 << ' ' << s2 << ' ' << s3 << '\n';
  kda_plan_destroy(plan);
}

}  // namespace

int main() {
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string kind;
    in >> kind;
    if (kind == "plan") run_plan(in);
    else if (kind == "check") run_check(in);
  }
  return 0;
}

// Record of the stand-in kernel launchers (see stub_launchers.cpp).
#pragma once

#include <string>
#include <vector>

#include "internal.hpp"

namespace sv {

struct StubLog {
  std::vector<std::string> calls;
  int B = -1, Tq = -1, N = -1;
  AttnArgs attn{};
  AcceptRule rule{};
  CommitArgs commit{};
  void clear() { *this = StubLog{}; }
};

extern StubLog g_stub;

}  // namespace sv

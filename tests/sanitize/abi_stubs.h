// Recorded launches of the stand-in kernel launchers (abi_stubs.cpp) used by the
// host-only, sanitizer-instrumented build of the C ABI. Test infrastructure only.
#pragma once

#include <vector>

#include "fa_kernels.hpp"

namespace stub {

struct Calls {
  std::vector<fa::FwdArgs> fwd;
  std::vector<fa::BwdArgs> pre, dkdv, dq;
  std::vector<fa::SoftmaxArgs> softmax;
  std::vector<fa::DecodeArgs> decode;
  std::vector<fa::KvOuterArgs> kv_outer;
  size_t total() const {
    return fwd.size() + pre.size() + dkdv.size() + dq.size() + softmax.size() + decode.size() +
           kv_outer.size();
  }
  void clear() { *this = Calls{}; }
};

extern Calls calls;

}  // namespace stub

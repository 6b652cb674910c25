// Stand-ins for the kernel launchers of libfa.so, linked with the C ABI (fa_api.hip)
// in a host-only build under AddressSanitizer and UndefinedBehaviorSanitizer: each
// records the arguments the C ABI hands it and launches nothing, so the build needs
// no GPU and no device code. Test infrastructure only.
#include "abi_stubs.h"

namespace stub {
Calls calls;
}

namespace fa {

hipError_t launch_fwd(const FwdArgs& a, hipStream_t) {
  stub::calls.fwd.push_back(a);
  return hipSuccess;
}
hipError_t launch_bwd_preprocess(const BwdArgs& a, hipStream_t) {
  stub::calls.pre.push_back(a);
  return hipSuccess;
}
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t) {
  stub::calls.dkdv.push_back(a);
  return hipSuccess;
}
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t) {
  stub::calls.dq.push_back(a);
  return hipSuccess;
}
hipError_t launch_softmax_rows(const SoftmaxArgs& a, hipStream_t) {
  stub::calls.softmax.push_back(a);
  return hipSuccess;
}
hipError_t launch_decode(const DecodeArgs& a, hipStream_t) {
  stub::calls.decode.push_back(a);
  return hipSuccess;
}
hipError_t launch_fwd_kv_outer(const KvOuterArgs& a, hipStream_t) {
  stub::calls.kv_outer.push_back(a);
  return hipSuccess;
}

}  // namespace fa

// Host-only stand-ins for the kernel launchers of libcsa.so, so that the C
// ABI's validation and launch-planning code (csa_abi.cpp) can be built and
// run on a CPU under AddressSanitizer / UndefinedBehaviorSanitizer.  Each
// stub records the parameter block it was given and launches nothing.
#include "launch_stubs.h"

namespace csa {

StubLog g_stub;

hipError_t launch_index_scores(const IndexParams& p, hipStream_t) {
  g_stub.index = p;
  ++g_stub.n_index;
  return hipSuccess;
}
hipError_t launch_topk(const TopkParams& p, hipStream_t) {
  g_stub.topk = p;
  ++g_stub.n_topk;
  return hipSuccess;
}
hipError_t launch_topk_merge(const TopkParams& p, hipStream_t) {
  g_stub.topk = p;
  ++g_stub.n_topk;
  return hipSuccess;
}
hipError_t launch_index_topk(const IndexParams& ip, const TopkParams& tp, hipStream_t) {
  g_stub.index = ip;
  g_stub.topk = tp;
  ++g_stub.n_index_topk;
  return hipSuccess;
}
hipError_t launch_index_topk_prefill(const IndexParams& ip, const TopkParams& tp, hipStream_t) {
  g_stub.index = ip;
  g_stub.topk = tp;
  ++g_stub.n_index_topk;
  ++g_stub.n_index_topk_prefill;
  return hipSuccess;
}
hipError_t launch_attn(const AttnParams& p, hipStream_t) {
  g_stub.attn = p;
  ++g_stub.n_attn;
  return hipSuccess;
}
hipError_t attn_scratch_address(void** ptr) {
  // a 256-byte-aligned stand-in address, never dereferenced on the host
  *ptr = reinterpret_cast<void*>(uintptr_t(1) << 40);
  return hipSuccess;
}

}  // namespace csa

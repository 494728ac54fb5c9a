// Stand-ins for the kernel launchers, for a host-only build of the C-ABI layer
// (api.hip) under AddressSanitizer / UndefinedBehaviorSanitizer: each records
// its arguments and returns success, so the driver can check both the
// argument validation and what a valid call would enqueue, without a GPU.
#include "stub_launchers.hpp"

namespace sv {

StubLog g_stub;

hipError_t launch_build_mask(const int32_t*, const uint8_t*, const int32_t*, int B, int Tq, uint32_t*, uint32_t*,
                             hipStream_t) {
  g_stub.calls.push_back("build_mask");
  g_stub.B = B;
  g_stub.Tq = Tq;
  return hipSuccess;
}
hipError_t launch_build_msa_mask(const int32_t*, const int32_t*, int B, int, int, int Tq, uint32_t*, uint32_t*,
                                 int32_t*, hipStream_t) {
  g_stub.calls.push_back("build_msa_mask");
  g_stub.B = B;
  g_stub.Tq = Tq;
  return hipSuccess;
}
hipError_t launch_draft_tree(const void*, int, int, int, int, const int32_t*, const int32_t*, const int32_t*, int,
                             const int32_t*, int, int, int N, int32_t*, int32_t*, int32_t*, int32_t*, hipStream_t) {
  g_stub.calls.push_back("draft_tree");
  g_stub.N = N;
  return hipSuccess;
}
hipError_t launch_attn_valu(const AttnArgs& a, int, hipStream_t) {
  g_stub.calls.push_back("attn_valu");
  g_stub.attn = a;
  return hipSuccess;
}
hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t) {
  g_stub.calls.push_back("attn_mfma");
  g_stub.attn = a;
  return hipSuccess;
}
hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t) {
  g_stub.calls.push_back("attn_combine");
  g_stub.attn = a;
  return hipSuccess;
}
hipError_t launch_argmax(const void*, int, int, int, int, const int32_t*, int32_t*, hipStream_t) {
  g_stub.calls.push_back("argmax");
  return hipSuccess;
}
hipError_t launch_argmax_lse(const void*, int, int, int, int, const int32_t*, int32_t*, float*, hipStream_t) {
  g_stub.calls.push_back("argmax_lse");
  return hipSuccess;
}
hipError_t launch_accept(int, int, const int32_t*, const int32_t*, const int32_t*, const int32_t*, const int32_t*,
                         int, int32_t*, int32_t*, int32_t*, const AcceptRule& rule, const CommitArgs& commit,
                         hipStream_t) {
  g_stub.calls.push_back("accept");
  g_stub.rule = rule;
  g_stub.commit = commit;
  return hipSuccess;
}
hipError_t launch_commit(int, int, int, int, int, int64_t, int64_t, int64_t, int64_t, int v_tiled, void*, void*,
                         const int32_t*, int32_t*, const void*, const void*, const int32_t*, const int32_t*, int,
                         hipStream_t) {
  g_stub.calls.push_back("commit");
  g_stub.commit.v_tiled = v_tiled;
  return hipSuccess;
}

}  // namespace sv

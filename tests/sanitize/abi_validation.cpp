// Host-side checks of the C ABI built under AddressSanitizer and
// UndefinedBehaviorSanitizer (api.hip compiled for the host only, the kernel
// launchers replaced by recording stubs; no GPU needed).  Every entry point
// is called with arguments it must refuse -- the status and a message must
// come back and nothing may be launched -- and with valid ones, whose resolved
// launch arguments are checked: workspace partitions inside the caller's
// buffer, rows per kv-head, mask words, the log2-domain scale, the V layout
// and the acceptance rule.  Exit status = number of failed checks.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "spec_verify.h"
#include "stub_launchers.hpp"

namespace {

int g_fail = 0;

void check(bool ok, const char* what, int line) {
  if (!ok) {
    ++g_fail;
    fprintf(stderr, "FAILED line %d: %s (last error: %s)\n", line, what, spec_last_error());
  }
}
#define CHECK(cond) check((cond), #cond, __LINE__)

// A device address that the host code must never dereference.
void* const F = reinterpret_cast<void*>(uintptr_t(1) << 20);
template <typename T>
T* fake() { return reinterpret_cast<T*>(F); }

spec_attn_desc desc(int B = 2, int Tq = 60, int Hq = 32, int Hkv = 8, int D = 128, int S = 16, int lmax = 4160) {
  spec_attn_desc d{};
  d.B = B;
  d.Tq = Tq;
  d.Hq = Hq;
  d.Hkv = Hkv;
  d.D = D;
  d.S = S;
  d.dtype = SPEC_BF16;
  d.scale = 0.f;
  d.lmax = lmax;
  d.kv_stride_b = (int64_t)lmax * Hkv * D;   // token-major [B, lmax, Hkv, D]
  d.kv_stride_l = (int64_t)Hkv * D;
  d.kv_stride_h = D;
  d.kv_splits = 0;
  d.v_layout = SPEC_V_ROWS;
  return d;
}

int attn(const spec_attn_desc& d, void* ws = nullptr, size_t wsb = 0, const void* q = F, const void* soft = F) {
  return spec_verify_attn(&d, q, F, F, fake<int32_t>(), F, F, d.S ? soft : nullptr, d.S ? soft : nullptr,
                          fake<uint32_t>(), fake<uint32_t>(), fake<int32_t>(), fake<float>(), nullptr, ws, wsb,
                          nullptr);
}

// A refused call: the status, a message, and nothing launched.
void refused(int status, int want, int line) {
  char msg[160];
  snprintf(msg, sizeof msg, "status %d, expected %d, nothing launched, message set", status, want);
  check(status == want && sv::g_stub.calls.empty() && spec_last_error()[0] != '\0', msg, line);
}
#define REFUSED(call, want) \
  do {                      \
    sv::g_stub.clear();     \
    refused((call), (want), __LINE__); \
  } while (0)

void descriptor_refusals() {
  REFUSED(spec_verify_attn(nullptr, F, F, F, fake<int32_t>(), F, F, nullptr, nullptr, fake<uint32_t>(),
                           fake<uint32_t>(), fake<int32_t>(), fake<float>(), nullptr, nullptr, 0, nullptr),
          SPEC_EINVAL);
  struct Case {
    void (*edit)(spec_attn_desc&);
    int want;
  };
  const Case cases[] = {
      {[](spec_attn_desc& d) { d.B = -1; }, SPEC_EINVAL},
      {[](spec_attn_desc& d) { d.Tq = 0; }, SPEC_EINVAL},
      {[](spec_attn_desc& d) { d.Tq = SPEC_MAX_TQ + 1; }, SPEC_EINVAL},
      {[](spec_attn_desc& d) { d.Hq = 30; }, SPEC_EINVAL},
      {[](spec_attn_desc& d) { d.Hkv = 0; }, SPEC_EINVAL},
      {[](spec_attn_desc& d) { d.dtype = 7; }, SPEC_EINVAL},
      {[](spec_attn_desc& d) { d.D = 96; }, SPEC_EUNSUPPORTED},
      {[](spec_attn_desc& d) { d.S = SPEC_MAX_SOFT + 1; }, SPEC_EINVAL},
      {[](spec_attn_desc& d) { d.lmax = -1; }, SPEC_EINVAL},
      {[](spec_attn_desc& d) { d.kv_stride_l = 0; }, SPEC_EINVAL},
      {[](spec_attn_desc& d) { d.kv_stride_l = d.Hkv * d.D + 1; }, SPEC_EINVAL},      // not 16-byte multiples
      {[](spec_attn_desc& d) { d.kv_stride_h = 64; }, SPEC_EINVAL},                   // heads overlap
      {[](spec_attn_desc& d) { d.kv_splits = 65; }, SPEC_EINVAL},
      {[](spec_attn_desc& d) { d.v_layout = 2; }, SPEC_EINVAL},
      {[](spec_attn_desc& d) { d.v_layout = SPEC_V_TILE32; }, SPEC_EINVAL},           // token-major cache
      {[](spec_attn_desc& d) { d.dtype = SPEC_F32; d.v_layout = SPEC_V_TILE32; }, SPEC_EUNSUPPORTED},
      {[](spec_attn_desc& d) {
         d.v_layout = SPEC_V_TILE32; d.lmax = 4150; d.kv_stride_l = d.D; d.kv_stride_h = 4160 * d.D;
       }, SPEC_EINVAL},                                                                 // lmax % 32
      {[](spec_attn_desc& d) { d.out_dtype = 5; }, SPEC_EINVAL},
      {[](spec_attn_desc& d) { d.dtype = SPEC_F32; d.out_dtype = SPEC_BF16; }, SPEC_EUNSUPPORTED},
      {[](spec_attn_desc& d) { d.scale = NAN; }, SPEC_EINVAL},
      {[](spec_attn_desc& d) { d.scale = -1.f; }, SPEC_EINVAL},
      {[](spec_attn_desc& d) { d.B = 70000; d.Hkv = 1; d.Hq = 1; }, SPEC_EUNSUPPORTED},  // B * Hkv > 65535
  };
  for (const Case& c : cases) {
    spec_attn_desc d = desc();
    c.edit(d);
    CHECK(spec_verify_attn_workspace(&d) == 0);
    REFUSED(attn(d), c.want);
    REFUSED(spec_commit_kv(&d, F, F, fake<int32_t>(), fake<int32_t>(), F, F, fake<int32_t>(), fake<int32_t>(), 8,
                           nullptr),
            c.want);
  }
}

void attention_calls() {
  spec_attn_desc d = desc();
  // array arguments: NULL, soft with S == 0, misaligned
  REFUSED(attn(d, nullptr, 0, nullptr), SPEC_EINVAL);
  REFUSED(attn(d, nullptr, 0, reinterpret_cast<char*>(F) + 4), SPEC_EINVAL);
  REFUSED(attn(d, nullptr, 0, F, nullptr), SPEC_EINVAL);
  spec_attn_desc d0 = desc(2, 60, 32, 8, 128, 0);
  REFUSED(spec_verify_attn(&d0, F, F, F, fake<int32_t>(), F, F, F, F, fake<uint32_t>(), fake<uint32_t>(),
                           fake<int32_t>(), fake<float>(), nullptr, nullptr, 0, nullptr),
          SPEC_EINVAL);
  // two requests x 8 kv-heads x 2 row chunks: the planner splits the keys and needs a workspace
  const size_t need = spec_verify_attn_workspace(&d);
  CHECK(need > 0);
  REFUSED(attn(d), SPEC_EWORKSPACE);
  std::vector<char> host_ws(need + 64);
  char* ws = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(host_ws.data()) + 15) & ~uintptr_t(15));
  REFUSED(attn(d, ws, need - 1), SPEC_EWORKSPACE);
  REFUSED(attn(d, ws + 4, need), SPEC_EINVAL);
  sv::g_stub.clear();
  CHECK(attn(d, ws, need) == SPEC_OK);
  CHECK(sv::g_stub.calls.size() == 2 && sv::g_stub.calls[0] == "attn_mfma" && sv::g_stub.calls[1] == "attn_combine");
  const sv::AttnArgs& a = sv::g_stub.attn;
  CHECK(a.G == 4 && a.R == 240 && a.W == 2 && a.n_split > 1 && a.rows_per_wg == 128 && a.row_chunks == 2);
  CHECK(fabsf(a.c - 1.4426950408889634f / sqrtf(128.f)) < 1e-7f);
  // both partial arrays lie inside the caller's workspace
  const size_t rows = (size_t)a.n_split * d.B * d.Hkv * a.R;
  const char* o_end = reinterpret_cast<const char*>(a.part_o + rows * d.D);
  const char* ml_end = reinterpret_cast<const char*>(a.part_ml + rows * 2);
  CHECK(reinterpret_cast<const char*>(a.part_o) == ws && o_end <= reinterpret_cast<const char*>(a.part_ml));
  CHECK(ml_end <= ws + need);
  // one split: no workspace, no combine
  d.kv_splits = 1;
  CHECK(spec_verify_attn_workspace(&d) == 0);
  sv::g_stub.clear();
  CHECK(attn(d) == SPEC_OK && sv::g_stub.calls.size() == 1 && sv::g_stub.attn.n_split == 1);
  // fp32 goes to the vector kernel; a custom scale is used as given
  spec_attn_desc f = desc(1, 4, 2, 2, 64, 0, 132);
  f.dtype = SPEC_F32;
  f.scale = 0.25f;
  sv::g_stub.clear();
  const size_t fneed = spec_verify_attn_workspace(&f);
  std::vector<char> fws(fneed + 16);
  char* fw = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(fws.data()) + 15) & ~uintptr_t(15));
  CHECK(spec_verify_attn(&f, F, F, F, fake<int32_t>(), F, F, nullptr, nullptr, fake<uint32_t>(), nullptr,
                         fake<int32_t>(), fake<float>(), nullptr, fw, fneed, nullptr) == SPEC_OK);
  CHECK(!sv::g_stub.calls.empty() && sv::g_stub.calls[0] == "attn_valu");
  CHECK(fabsf(sv::g_stub.attn.c - 0.25f * 1.4426950408889634f) < 1e-7f);
  // transposed V tiles: a head-major cache with lmax % 32 == 0
  spec_attn_desc t = desc(16, 60, 32, 8, 128, 16, 4160);
  t.kv_stride_b = (int64_t)8 * 4160 * 128;
  t.kv_stride_l = 128;
  t.kv_stride_h = (int64_t)4160 * 128;
  t.v_layout = SPEC_V_TILE32;
  sv::g_stub.clear();
  CHECK(attn(t) == SPEC_OK && sv::g_stub.attn.v_tiled == 1 && sv::g_stub.attn.n_split == 1);
  sv::g_stub.clear();
  CHECK(spec_commit_kv(&t, F, F, fake<int32_t>(), fake<int32_t>(), F, F, fake<int32_t>(), fake<int32_t>(), 6,
                       nullptr) == SPEC_OK);
  CHECK(sv::g_stub.calls.size() == 1 && sv::g_stub.commit.v_tiled == 1);
  // B == 0 is a no-op
  spec_attn_desc e = desc(0);
  sv::g_stub.clear();
  CHECK(spec_verify_attn(&e, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                         nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) == SPEC_OK);
  CHECK(spec_verify_attn_noalloc(&e, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                 nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == SPEC_OK);
  CHECK(sv::g_stub.calls.empty());
  // the allocation-free entry: more scratch than it holds is refused before any HIP call
  spec_attn_desc big = desc(64, 256, 64, 8, 128, 0, 16384);
  big.kv_splits = 8;
  CHECK(spec_verify_attn_workspace(&big) > (size_t)SPEC_NOALLOC_SCRATCH_BYTES);
  REFUSED(spec_verify_attn_noalloc(&big, F, F, F, fake<int32_t>(), F, F, nullptr, nullptr, fake<uint32_t>(),
                                   fake<uint32_t>(), fake<int32_t>(), fake<float>(), nullptr, nullptr),
          SPEC_EWORKSPACE);
  // without a split it needs no scratch and launches like spec_verify_attn
  sv::g_stub.clear();
  CHECK(spec_verify_attn_noalloc(&t, F, F, F, fake<int32_t>(), F, F, F, F, fake<uint32_t>(), fake<uint32_t>(),
                                 fake<int32_t>(), fake<float>(), nullptr, nullptr) == SPEC_OK);
  CHECK(sv::g_stub.calls.size() == 1 && sv::g_stub.calls[0] == "attn_mfma");
}

void mask_and_acceptance_calls() {
  REFUSED(spec_build_mask(fake<int32_t>(), nullptr, fake<int32_t>(), -1, 60, fake<uint32_t>(), fake<uint32_t>(),
                          nullptr),
          SPEC_EINVAL);
  REFUSED(spec_build_mask(fake<int32_t>(), nullptr, fake<int32_t>(), 2, 0, fake<uint32_t>(), fake<uint32_t>(),
                          nullptr),
          SPEC_EINVAL);
  REFUSED(spec_build_mask(nullptr, nullptr, fake<int32_t>(), 2, 60, fake<uint32_t>(), fake<uint32_t>(), nullptr),
          SPEC_EINVAL);
  REFUSED(spec_build_mask(reinterpret_cast<int32_t*>(reinterpret_cast<char*>(F) + 2), nullptr, fake<int32_t>(), 2,
                          60, fake<uint32_t>(), fake<uint32_t>(), nullptr),
          SPEC_EINVAL);
  sv::g_stub.clear();
  CHECK(spec_build_mask(fake<int32_t>(), fake<uint8_t>(), fake<int32_t>(), 3, 60, fake<uint32_t>(), fake<uint32_t>(),
                        nullptr) == SPEC_OK);
  CHECK(sv::g_stub.calls.size() == 1 && sv::g_stub.B == 3 && sv::g_stub.Tq == 60);
  // multi-stream rows: N * (1 + gamma) must fit the block
  REFUSED(spec_build_msa_mask(fake<int32_t>(), fake<int32_t>(), 2, 40, 3, 159, fake<uint32_t>(), fake<uint32_t>(),
                              fake<int32_t>(), nullptr),
          SPEC_EINVAL);
  sv::g_stub.clear();
  CHECK(spec_build_msa_mask(fake<int32_t>(), fake<int32_t>(), 2, 40, 3, 160, fake<uint32_t>(), fake<uint32_t>(),
                            fake<int32_t>(), nullptr) == SPEC_OK);
  // greedy acceptance
  REFUSED(spec_argmax_accept(F, SPEC_BF16, 2, 0, 100, fake<int32_t>(), fake<int32_t>(), fake<int32_t>(), 8,
                             fake<int32_t>(), fake<int32_t>(), fake<int32_t>(), nullptr),
          SPEC_EINVAL);
  REFUSED(spec_argmax_accept(F, SPEC_BF16, 2, 30, 100, fake<int32_t>(), fake<int32_t>(), fake<int32_t>(),
                             SPEC_MAX_DEPTH + 1, fake<int32_t>(), fake<int32_t>(), fake<int32_t>(), nullptr),
          SPEC_EINVAL);
  REFUSED(spec_argmax_accept(reinterpret_cast<char*>(F) + 1, SPEC_BF16, 2, 30, 100, fake<int32_t>(), fake<int32_t>(),
                             fake<int32_t>(), 8, fake<int32_t>(), fake<int32_t>(), fake<int32_t>(), nullptr),
          SPEC_EINVAL);
  sv::g_stub.clear();
  CHECK(spec_argmax_accept_rows(F, SPEC_BF16, 2, 30, 100, fake<int32_t>(), fake<int32_t>(), fake<int32_t>(),
                                fake<int32_t>(), 8, fake<int32_t>(), fake<int32_t>(), fake<int32_t>(),
                                fake<int32_t>(), nullptr) == SPEC_OK);
  CHECK(sv::g_stub.calls.size() == 2 && sv::g_stub.calls[0] == "argmax" && sv::g_stub.rule.mode == 0 &&
        sv::g_stub.commit.enabled == 0);
  // probability rules
  REFUSED(spec_prob_accept(F, SPEC_BF16, 2, 30, 100, fake<int32_t>(), fake<int32_t>(), fake<int32_t>(), nullptr, 8,
                           SPEC_ACCEPT_SOFT, 0.f, nullptr, nullptr, fake<int32_t>(), fake<float>(), fake<int32_t>(),
                           fake<int32_t>(), nullptr, nullptr),
          SPEC_EINVAL);
  REFUSED(spec_prob_accept(F, SPEC_BF16, 2, 30, 100, fake<int32_t>(), fake<int32_t>(), fake<int32_t>(), nullptr, 8,
                           SPEC_ACCEPT_THRESHOLD, NAN, nullptr, nullptr, fake<int32_t>(), fake<float>(),
                           fake<int32_t>(), fake<int32_t>(), nullptr, nullptr),
          SPEC_EINVAL);
  sv::g_stub.clear();
  CHECK(spec_prob_accept(F, SPEC_BF16, 2, 30, 100, fake<int32_t>(), fake<int32_t>(), fake<int32_t>(), nullptr, 8,
                         SPEC_ACCEPT_SOFT, 0.f, fake<float>(), fake<float>(), fake<int32_t>(), fake<float>(),
                         fake<int32_t>(), fake<int32_t>(), nullptr, nullptr) == SPEC_OK);
  CHECK(sv::g_stub.calls.size() == 2 && sv::g_stub.calls[0] == "argmax_lse" && sv::g_stub.rule.mode == 2 &&
        sv::g_stub.rule.V == 100 && sv::g_stub.rule.logits_bf16 == 1);
  // fused argmax + acceptance + commit: T may not exceed the block, the commit is enabled
  spec_attn_desc d = desc(2, 60);
  REFUSED(spec_argmax_accept_commit(F, SPEC_BF16, 61, 100, fake<int32_t>(), fake<int32_t>(), fake<int32_t>(),
                                    nullptr, 8, fake<int32_t>(), fake<int32_t>(), fake<int32_t>(), nullptr, &d, F, F,
                                    fake<int32_t>(), fake<int32_t>(), F, F, nullptr),
            SPEC_EINVAL);
  sv::g_stub.clear();
  CHECK(spec_argmax_accept_commit(F, SPEC_BF16, 30, 100, fake<int32_t>(), fake<int32_t>(), fake<int32_t>(), nullptr,
                                  8, fake<int32_t>(), fake<int32_t>(), fake<int32_t>(), nullptr, &d, F, F,
                                  fake<int32_t>(), fake<int32_t>(), F, F, nullptr) == SPEC_OK);
  CHECK(sv::g_stub.calls.size() == 2 && sv::g_stub.commit.enabled == 1 && sv::g_stub.commit.Tq == 60 &&
        sv::g_stub.commit.esize == 2);
  // the next draft: a k-ary tree of depth gamma must fit the block limit
  REFUSED(spec_draft_tree(F, SPEC_BF16, 2, 160, 100, fake<int32_t>(), fake<int32_t>(), fake<int32_t>(), 8,
                          fake<int32_t>(), 8, 3, fake<int32_t>(), fake<int32_t>(), fake<int32_t>(), fake<int32_t>(),
                          nullptr),
          SPEC_EINVAL);
  sv::g_stub.clear();
  CHECK(spec_draft_tree(F, SPEC_BF16, 2, 160, 100, fake<int32_t>(), fake<int32_t>(), fake<int32_t>(), 8,
                        fake<int32_t>(), 3, 3, fake<int32_t>(), fake<int32_t>(), fake<int32_t>(), fake<int32_t>(),
                        nullptr) == SPEC_OK);
  CHECK(sv::g_stub.calls.size() == 1 && sv::g_stub.N == 40);
}

}  // namespace

int main() {
  CHECK(strcmp(spec_strerror(SPEC_OK), "success") == 0);
  CHECK(strcmp(spec_strerror(12345), "unknown status") == 0);
  CHECK(spec_version()[0] != '\0');
  descriptor_refusals();
  attention_calls();
  mask_and_acceptance_calls();
  if (g_fail == 0) printf("host validation under sanitizers: all checks passed\n");
  return g_fail;
}

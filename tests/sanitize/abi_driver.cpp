// Host-only driver for the sanitizer test: calls every entry point of
// include/gdn.h with arguments that fail validation (and the empty calls that
// return before any launch), so AddressSanitizer and UndefinedBehaviorSanitizer
// watch the whole argument-checking layer.  No call reaches a kernel.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "gdn.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    std::fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

int main() {
  alignas(16) static unsigned char buf[4096];
  void* A = buf;
  void* U = buf + 4;  // misaligned
  const float* F = reinterpret_cast<const float*>(buf);
  float* Fw = reinterpret_cast<float*>(buf);

  for (int s = -2; s < 12; ++s)
    if (!gdn_status_str(s) || !std::strlen(gdn_status_str(s))) ++failures;

  // gdn_chunk_fwd
  expect("fwd dtype", gdn_chunk_fwd(A, A, A, F, F, nullptr, 64, A, A, 1, 64, 1, 64, 64, 9, nullptr, 0, nullptr),
         GDN_ERR_DTYPE);
  expect("fwd shape", gdn_chunk_fwd(A, A, A, F, F, nullptr, 64, A, A, -1, 64, 1, 64, 64, GDN_BF16, nullptr, 0, nullptr),
         GDN_ERR_SHAPE);
  expect("fwd huge", gdn_chunk_fwd(A, A, A, F, F, nullptr, 64, A, A, 1 << 20, 1 << 20, 1 << 10, 64, 64, GDN_BF16,
                                   nullptr, 0, nullptr),
         GDN_ERR_SHAPE);
  expect("fwd chunk", gdn_chunk_fwd(A, A, A, F, F, nullptr, 32, A, A, 1, 64, 1, 64, 64, GDN_BF16, nullptr, 0, nullptr),
         GDN_ERR_UNSUPPORTED);
  expect("fwd dims", gdn_chunk_fwd(A, A, A, F, F, nullptr, 64, A, A, 1, 64, 1, 96, 96, GDN_BF16, nullptr, 0, nullptr),
         GDN_ERR_UNSUPPORTED);
  expect("fwd null", gdn_chunk_fwd(nullptr, A, A, F, F, nullptr, 64, A, A, 1, 64, 1, 64, 64, GDN_F32, nullptr, 0,
                                   nullptr),
         GDN_ERR_NULL);
  expect("fwd align", gdn_chunk_fwd(U, A, A, F, F, nullptr, 64, A, A, 1, 64, 1, 64, 64, GDN_F32, nullptr, 0, nullptr),
         GDN_ERR_ALIGN);
  expect("fwd workspace", gdn_chunk_fwd(A, A, A, F, F, nullptr, 64, A, A, 2, 256, 3, 128, 128, GDN_BF16, nullptr, 0,
                                        nullptr),
         GDN_ERR_WORKSPACE);
  expect("fwd empty", gdn_chunk_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 64, nullptr, nullptr, 0, 64, 1,
                                    64, 64, GDN_F32, nullptr, 0, nullptr),
         GDN_OK);
  for (int dt : {GDN_F32, GDN_BF16, GDN_C64})
    for (int d : {32, 64, 128})
      for (int T : {0, 1, 64, 65, 100000}) (void)gdn_chunk_fwd_workspace_bytes(3, T, 7, d, d, 64, dt);
  (void)gdn_chunk_fwd_workspace_bytes(-1, 1, 1, 64, 64, 64, GDN_BF16);
  (void)gdn_chunk_fwd_workspace_bytes(1, 1, 1, 64, 64, 32, GDN_BF16);
  expect("noalloc huge", gdn_chunk_fwd_noalloc(A, A, A, F, F, nullptr, 64, A, A, 512, 65536, 16, 128, 128, GDN_BF16,
                                               nullptr),
         GDN_ERR_WORKSPACE);

  // gdn_chunk_fwd_prologue
  expect("pro scale", gdn_chunk_fwd_prologue(A, A, A, F, F, 3.f, nullptr, 64, A, A, 1, 64, 1, 64, 64, GDN_BF16, nullptr,
                                             0, nullptr),
         GDN_ERR_SHAPE);
  expect("pro null", gdn_chunk_fwd_prologue(A, nullptr, A, F, F, 1.f, nullptr, 64, A, A, 1, 64, 1, 64, 64, GDN_BF16,
                                            nullptr, 0, nullptr),
         GDN_ERR_NULL);
  expect("pro workspace", gdn_chunk_fwd_prologue(A, A, A, F, F, 1.f, nullptr, 64, A, A, 1, 64, 1, 32, 32, GDN_C64,
                                                 A, 64, nullptr),
         GDN_ERR_WORKSPACE);
  expect("pro f32 d128", gdn_chunk_fwd_prologue(A, A, A, F, F, 1.f, nullptr, 64, A, A, 1, 64, 1, 128, 128, GDN_F32,
                                                nullptr, 0, nullptr),
         GDN_ERR_UNSUPPORTED);
  for (int dt : {GDN_F32, GDN_BF16, GDN_C64})
    for (int d : {32, 64, 128})
      for (int T : {0, 1, 64, 65, 100000}) (void)gdn_chunk_fwd_prologue_workspace_bytes(3, T, 7, d, d, 64, dt);

  // gdn_chunk_bwd
  expect("bwd dtype", gdn_chunk_bwd(A, A, A, F, F, nullptr, A, nullptr, Fw, Fw, Fw, Fw, Fw, Fw, 1, 64, 1, 64, 64, 7,
                                    A, 1 << 20, nullptr),
         GDN_ERR_DTYPE);
  expect("bwd c64 d64", gdn_chunk_bwd(A, A, A, F, F, nullptr, A, nullptr, Fw, Fw, Fw, Fw, Fw, Fw, 1, 64, 1, 64, 64,
                                      GDN_C64, A, 1 << 20, nullptr),
         GDN_ERR_UNSUPPORTED);
  expect("bwd c64 workspace", gdn_chunk_bwd(A, A, A, F, F, nullptr, A, nullptr, Fw, Fw, Fw, Fw, Fw, Fw, 1, 64, 1, 32,
                                            32, GDN_C64, A, 16, nullptr),
         GDN_ERR_WORKSPACE);
  expect("bwd null", gdn_chunk_bwd(A, A, A, F, F, nullptr, nullptr, nullptr, Fw, Fw, Fw, Fw, Fw, Fw, 1, 64, 1, 64, 64,
                                   GDN_F32, A, 1 << 20, nullptr),
         GDN_ERR_NULL);
  expect("bwd workspace", gdn_chunk_bwd(A, A, A, F, F, nullptr, A, nullptr, Fw, Fw, Fw, Fw, Fw, Fw, 2, 640, 3, 128, 128,
                                        GDN_BF16, A, 16, nullptr),
         GDN_ERR_WORKSPACE);
  for (int dt : {GDN_F32, GDN_BF16, GDN_C64})
    for (int d : {32, 64, 128})
      for (int T : {0, 1, 64, 65, 100000}) (void)gdn_chunk_bwd_workspace_bytes(3, T, 7, d, d, dt);

  // gdn_fwd_channel_decay
  expect("chd dims", gdn_fwd_channel_decay(A, A, A, F, F, nullptr, A, Fw, 1, 16, 1, 32, 32, GDN_BF16, nullptr),
         GDN_ERR_UNSUPPORTED);
  expect("chd align", gdn_fwd_channel_decay(A, A, A, reinterpret_cast<const float*>(U), F, nullptr, A, Fw, 1, 16, 1, 64,
                                            64, GDN_F32, nullptr),
         GDN_ERR_ALIGN);

  // gdn_recurrent_step
  expect("step shape", gdn_recurrent_step(A, A, A, F, F, A, A, -5, 64, 64, GDN_BF16, nullptr), GDN_ERR_SHAPE);
  expect("step dims", gdn_recurrent_step(A, A, A, F, F, A, A, 4, 64, 32, GDN_BF16, nullptr), GDN_ERR_UNSUPPORTED);
  expect("step empty", gdn_recurrent_step(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 64, 64,
                                          GDN_F32, nullptr),
         GDN_OK);

  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("abi driver: all checks passed\n");
  return 0;
}

// Drives the library's host-side validation through the C ABI, for a build
// of the launcher (gla_api.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_sanitizers.py).  Every call here
// fails on the host; without a device, a call with valid arguments fails at
// the first HIP call.  Exit status 0: every status was the expected one.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "gla.h"

static int failures = 0;
static void expect(gla_status got, gla_status want, const char *what) {
  if (got != want) {
    std::fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, (int)got, (int)want,
                 gla_last_error());
    ++failures;
  }
  (void)gla_status_string(got);
}

int main(int argc, char **argv) {
  const bool no_device = argc > 1 && std::strcmp(argv[1], "--no-device") == 0;
  char *base = reinterpret_cast<char *>(uintptr_t(1) << 40);
  void *t[9];
  for (int i = 0; i < 9; ++i) t[i] = base + (uintptr_t(i) << 32);  // 4 GiB apart, never read
  const gla_status bad = GLA_ERR_INVALID_ARG;

  expect(gla_forward(nullptr, t[1], t[2], t[3], t[4], 1, 2, 2, 4, 4, 32, 1e4f, 1e-6f, GLA_BF16,
                     nullptr), bad, "null q");
  expect(gla_forward(t[0], t[1], t[2], t[3], t[4], 1, 2, 2, 4, 4, 24, 1e4f, 1e-6f, GLA_BF16,
                     nullptr), bad, "d = 24");
  expect(gla_forward(t[0], t[1], t[2], t[3], t[4], 0, 2, 2, 4, 4, 32, 1e4f, 1e-6f, GLA_BF16,
                     nullptr), bad, "B = 0");
  expect(gla_forward(t[0], t[1], t[2], t[3], t[0], 1, 2, 2, 4, 4, 32, 1e4f, 1e-6f, GLA_BF16,
                     nullptr), bad, "out aliases q");
  expect(gla_forward(t[0], t[1], t[2], t[3], t[4], 1, 2, 2, 4, 4, 32, 1e4f, -1.f, GLA_BF16,
                     nullptr), bad, "eps < 0");
  expect(gla_forward(t[0], t[1], t[2], t[3], t[4], INT64_MAX / 2, 2, 2, 4, 4, 32, 1e4f, 1e-6f,
                     GLA_BF16, nullptr), bad, "size overflow");
  expect(gla_block_causal_forward(t[0], t[1], t[2], t[3], t[4], 1, 2, 6, 4, 4, 32, 4, 1e4f,
                                  1e-6f, GLA_BF16, nullptr), bad, "F does not divide T");
  expect(gla_forward_ws(t[0], t[1], t[2], t[3], t[4], 1, 2, 2, 4, 4, 32, 0, 1e4f, 1e-6f,
                        GLA_BF16, base + 8, 1 << 20, nullptr), bad, "misaligned workspace");
  size_t bytes = 0;
  expect(gla_workspace_bytes(1, 0, 2, 4, 4, 32, 0, GLA_BF16, &bytes), bad, "workspace H = 0");
  expect(gla_workspace_bytes(1, 2, 2, 4, 4, 32, 0, GLA_BF16, nullptr), bad, "null bytes");
  expect(gla_state(t[1], t[2], nullptr, nullptr, 1, 2, 2, 4, 4, 32, 0, 1e4f, GLA_BF16, nullptr),
         bad, "state null outputs");
  expect(gla_block_step(t[0], t[1], t[2], t[3], nullptr, static_cast<float *>(t[5]),
                        static_cast<float *>(t[6]), 1, 2, 2, 4, 4, 32, 0, 0,
                        1e4f, 1e-6f, GLA_BF16, nullptr, 0, nullptr), bad, "step: no out, no update");
  expect(gla_gated_forward(t[0], t[1], t[2], t[3], t[5], t[6], t[4], 1, 2, 2, 4, 4, 32, 0, 1e4f,
                           1e-6f, -1.f, GLA_BF16, nullptr, 0, nullptr), bad, "rms_eps < 0");
  expect(gla_backward(t[0], t[1], t[2], t[3], t[4], t[5], t[6], t[7], t[0], 1, 2, 2, 4, 4, 32, 0,
                      1e4f, 1e-6f, GLA_BF16, nullptr, 0, nullptr), bad, "dg aliases q");
  expect(gla_token_causal_forward(t[0], t[1], t[2], t[3], t[4], 1, 2, 2, 4, 4, 40, 1e4f, 1e-6f,
                                  GLA_BF16, nullptr, 0, nullptr), bad, "token causal d = 40");
  expect(gla_profile_enable(1), GLA_OK, "profile on");
  expect(gla_profile_enable(0), GLA_OK, "profile off");
  if (no_device)
    expect(gla_forward(t[0], t[1], t[2], t[3], t[4], 1, 2, 2, 4, 4, 32, 1e4f, 1e-6f, GLA_BF16,
                       nullptr), GLA_ERR_HIP, "valid call without a device");
  if (failures) std::fprintf(stderr, "%d unexpected status(es)\n", failures);
  return failures ? 1 : 0;
}

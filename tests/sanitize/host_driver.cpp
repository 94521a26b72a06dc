// A driver for the host side of libspecverify under AddressSanitizer and
// UndefinedBehaviorSanitizer (built by tests/test_sanitizers.py with hipcc,
// each -fsanitize= after -Xarch_host): the argument checks, size limits and
// workspace layout of every entry point, and the host digests of the commit
// step.  No call here reaches a kernel launch or any device call, so it runs
// without a GPU.  Exits 0 when every call returns the expected code.
#include <stdio.h>
#include <string.h>

#include "specverify.h"

static int fails = 0;
static bool sv_launch_reached();
#define EXPECT(c)                                              \
  do {                                                         \
    if (!(c)) {                                                \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #c); \
      ++fails;                                                 \
    }                                                          \
  } while (0)

int main() {
  char fake_buf[64];
  void* f = fake_buf;  // never dereferenced on these paths
  const int32_t* fi = (const int32_t*)f;
  int32_t* fo = (int32_t*)f;
  const sv_sampling* fs = (const sv_sampling*)f;
  // workspace sizes
  EXPECT(sv_workspace_bytes(1, 1, 1) > 0);
  EXPECT(sv_workspace_bytes(0, 4, 100) == 0);
  EXPECT(sv_workspace_bytes(4, 65, 100) == 0);
  EXPECT(sv_workspace_bytes(4, 4, (1 << 24) + 1) == 0);
  EXPECT(sv_workspace_bytes(1 << 21, 1, 10) > 0);
  EXPECT(sv_workspace_bytes((1 << 21) + 1, 1, 10) == 0);
  EXPECT(sv_workspace_bytes(1 << 19, 32, 10) == 0);
  for (int B = 1; B < 3000; B += 97)
    for (int M = 1; M <= 64; M += 9)
      for (int V = 1; V < 300000; V = V * 3 + 1) EXPECT(sv_workspace_bytes(B, M, V) % 256 == 0);
  const size_t ws = sv_workspace_bytes(4, 4, 100);
  // call-level argument errors: nothing is enqueued
  EXPECT(sv_verify(nullptr, f, SV_BF16, fi, fi, fi, fs, 4, 4, 100, 0, 1, fo, fo, f, ws, nullptr,
                   nullptr) == SV_ERR_ARG);
  EXPECT(sv_verify(f, f, 7, fi, fi, fi, fs, 4, 4, 100, 0, 1, fo, fo, f, ws, nullptr, nullptr) ==
         SV_ERR_ARG);
  EXPECT(sv_verify(f, f, SV_BF16, fi, fi, fi, fs, 4, 0, 100, 0, 1, fo, fo, f, ws, nullptr,
                   nullptr) == SV_ERR_ARG);
  EXPECT(sv_verify(f, f, SV_BF16, fi, fi, fi, fs, 4, 4, 100, 0, 1, fo, fo, f, ws - 1, nullptr,
                   nullptr) == SV_ERR_WORKSPACE);
  EXPECT(sv_verify_sdcp(f, f, SV_BF16, fi, fi, fi, fs, nullptr, 4, 4, 100, fo, fo, f, ws, nullptr,
                        nullptr) == SV_ERR_ARG);
  EXPECT(sv_verify_qrows(f, SV_FP32, (const float*)f, fi, fi, fi, fs, nullptr, 4, 4, 0, 0, 1, fo,
                         fo, f, ws, nullptr, nullptr) == SV_ERR_ARG);
  EXPECT(sv_verify_early(f, f, (const float*)f, SV_BF16, fi, fi, fi, fs, nullptr, 4, 4, 100, 0, 1,
                         2, fo, fo, f, ws, nullptr, nullptr) == SV_ERR_ARG);
  EXPECT(sv_verify_early(f, f, nullptr, SV_BF16, fi, fi, fi, fs, nullptr, 4, 4, 100, 0, 1, 0, fo,
                         fo, f, ws, nullptr, nullptr) == SV_ERR_ARG);
  EXPECT(sv_verify_early(f, f, nullptr, SV_BF16, fi, fi, fi, fs, nullptr, 4, 4, 100, 0, 1, 66, fo,
                         fo, f, ws, nullptr, nullptr) == SV_ERR_ARG);
  EXPECT(sv_verify_noalloc(f, f, SV_BF16, fi, fi, fi, fs, 1 << 20, 8, 1 << 20, 0, 1, fo, fo,
                           nullptr, nullptr) == SV_ERR_WORKSPACE);
  EXPECT(sv_verify_noalloc(f, f, 9, fi, fi, fi, fs, 4, 4, 100, 0, 1, fo, fo, nullptr, nullptr) ==
         SV_ERR_ARG);
  {
    sv_commit_io io = {(const sv_contract*)f, (sv_session_state*)f, nullptr, fo, fo};
    EXPECT(sv_verify_commit(f, f, SV_BF16, fi, fi, fi, fs, nullptr, 4, 4, 100, 0, 1, fo, fo,
                            nullptr, f, ws, nullptr, nullptr) == SV_ERR_ARG);
    EXPECT(sv_verify_commit(f, f, SV_BF16, fi, fi, fi, fs, nullptr, 0, 4, 100, 0, 1, fo, fo, &io,
                            f, ws, nullptr, nullptr) == SV_ERR_ARG);
    EXPECT(sv_verify_commit(f, f, SV_BF16, fi, fi, fi, fs, nullptr, 4, 4, 100, 0, 1, fo, fo, &io,
                            f, 16, nullptr, nullptr) == SV_ERR_WORKSPACE);
    io.action = nullptr;
    EXPECT(sv_verify_commit(f, f, SV_BF16, fi, fi, fi, fs, nullptr, 4, 4, 100, 0, 1, fo, fo, &io,
                            f, ws, nullptr, nullptr) == SV_ERR_ARG);
  }
  EXPECT(sv_commit(nullptr, nullptr, fi, fi, fo, nullptr, 4, 4, fo, fo, nullptr) == SV_ERR_ARG);
  EXPECT(sv_commit((const sv_contract*)f, (sv_session_state*)f, fi, fi, fo, nullptr, 4, 65, fo, fo,
                   nullptr) == SV_ERR_ARG);
  // host digests (SDCP Sec. 4.1, 4.2)
  uint8_t cd[32], d0[32];
  const uint8_t cbor[3] = {0xa1, 0x01, 0x02};
  EXPECT(sv_contract_digest(cbor, sizeof cbor, cd) == SV_OK);
  int32_t prompt[300];
  for (int i = 0; i < 300; ++i) prompt[i] = i * 7919;
  for (uint32_t P = 0; P < 300; P += 13) EXPECT(sv_prefix_digest(cd, prompt, P, d0) == SV_OK);
  EXPECT(sv_prefix_digest(nullptr, prompt, 3, d0) == SV_ERR_ARG);
  EXPECT(sv_contract_digest(nullptr, 3, cd) == SV_ERR_ARG);
  for (int c = -5; c <= 1; ++c) EXPECT(sv_strerror(c) && strlen(sv_strerror(c)) > 0);
  for (int c = -6; c <= 1; ++c) EXPECT(sv_status_str(c) != nullptr);
  EXPECT(sv_version() == SV_VERSION);
  EXPECT(!sv_launch_reached());
  printf("host driver done, %d failures\n", fails);
  return fails != 0;
}

// The row and per-session kernels' launchers: this driver builds the host
// entry points (sv_api.hip) and the commit step (sv_commit.hip) only, and no
// call above reaches a launch.
#include "sv_kernels.hpp"
namespace sv {
bool launch_reached = false;
void launch_rows_stream(const LaunchArgs&, hipStream_t) { launch_reached = true; }
void launch_rows_dense32(const LaunchArgs&, hipStream_t) { launch_reached = true; }
void launch_finalize(const LaunchArgs&, hipStream_t) { launch_reached = true; }
void launch_advance(const LaunchArgs&, hipStream_t, int) { launch_reached = true; }
}  // namespace sv

static bool sv_launch_reached() { return sv::launch_reached; }

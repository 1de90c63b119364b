// Host-only check of the C ABI's argument handling, built with
// -fsanitize=address,undefined by tests/test_abi_sanitized.py.  TEST
// INFRASTRUCTURE.
//
// api.cpp is compiled unchanged; the kernel launchers and the two HIP
// runtime calls it makes are replaced by the stubs below, so nothing here
// needs a GPU.  The program calls every entry point with valid arguments
// (the launcher must be reached once, with the arguments passed through
// unchanged), with each kind of invalid argument (the launcher must not be
// reached), with a launcher that fails (ATTN_ERR_HIP and its text), and
// with OSFA_SYNC_CHECK=1 (the stream is synchronized once per call).  Any
// out-of-bounds access, use of uninitialized stack, overflow or other
// undefined behaviour in the validation code stops the run.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>

#include "launch.h"
#include "osfa.h"

namespace {
int g_launches = 0;
int g_syncs = 0;
hipError_t g_result = hipSuccess;
osfa::FwdArgs g_fwd{};
osfa::DecodeArgs g_dec{};
osfa::BwdArgs g_bwd{};
int g_fails = 0;

void expect(bool ok, const char* what, int line) {
  if (!ok) {
    std::fprintf(stderr, "FAILED line %d: %s (last error: %s)\n", line, what, attn_last_error());
    ++g_fails;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)
}  // namespace

// --- stubs of what api.cpp calls -------------------------------------------
extern "C" const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "stub launch error"; }
extern "C" hipError_t hipStreamSynchronize(hipStream_t) {
  ++g_syncs;
  return hipSuccess;
}
namespace osfa {
hipError_t launch_attn_fwd_bf16(const FwdArgs& a, hipStream_t) { ++g_launches; g_fwd = a; return g_result; }
hipError_t launch_attn_fwd_f32(const FwdArgs& a, hipStream_t) { ++g_launches; g_fwd = a; return g_result; }
hipError_t launch_attn_fwd_bf16_exp2_offload(const FwdArgs& a, int, hipStream_t) { ++g_launches; g_fwd = a; return g_result; }
hipError_t launch_attn_fwd_fp8(const FwdArgs& a, float, float, hipStream_t) { ++g_launches; g_fwd = a; return g_result; }
hipError_t launch_attn_bwd_bf16(const BwdArgs& a, hipStream_t) { ++g_launches; g_bwd = a; return g_result; }
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t) { ++g_launches; g_dec = a; return g_result; }
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t) { ++g_launches; g_dec = a; return g_result; }
hipError_t launch_decode_noalloc(const DecodeArgs& a, bool, hipStream_t) { ++g_launches; g_dec = a; return g_result; }
hipError_t launch_softmax_rows(const float*, float*, int, int, hipStream_t) { ++g_launches; return g_result; }
hipError_t launch_softmax_topk(const float*, float*, float*, int32_t*, int, int, int, hipStream_t) { ++g_launches; return g_result; }
}  // namespace osfa

int main() {
  // Fake, suitably aligned device addresses: never dereferenced.
  char* const P = reinterpret_cast<char*>(uintptr_t(1) << 20);
  const int32_t* KV = reinterpret_cast<const int32_t*>(P + 64);
  float* F = reinterpret_cast<float*>(P);

  // attn_fwd: valid call reaches the launcher once with the same arguments.
  g_launches = 0;
  EXPECT(attn_fwd(ATTN_BF16, P, P, P, P, F, 2, 3, 77, 128, 0.125f, 1, 16, KV, nullptr) == ATTN_OK);
  EXPECT(g_launches == 1);
  EXPECT(g_fwd.B == 2 && g_fwd.H == 3 && g_fwd.N == 77 && g_fwd.d == 128 && g_fwd.scale == 0.125f &&
         g_fwd.causal == 1 && g_fwd.window == 16 && g_fwd.kv_len == KV);
  EXPECT(attn_fwd(ATTN_F32, P, P, P, P, F, 1, 1, 1000, 64, 0.125f, 0, 0, nullptr, nullptr) == ATTN_OK);
  EXPECT(g_launches == 2);
  // invalid arguments: nothing is launched, text names the problem.
  const int before = g_launches;
  EXPECT(attn_fwd(ATTN_BF16, nullptr, P, P, P, F, 1, 1, 16, 128, 0.1f, 0, 0, nullptr, nullptr) == ATTN_ERR_INVALID_ARG);
  EXPECT(std::strstr(attn_last_error(), "null") != nullptr);
  EXPECT(attn_fwd(ATTN_BF16, P, P, P, P, F, 1, 1, 16, 96, 0.1f, 0, 0, nullptr, nullptr) == ATTN_ERR_UNSUPPORTED);
  EXPECT(attn_fwd(ATTN_BF16, P, P, P, P, F, 1, 1, 16, 128, NAN, 0, 0, nullptr, nullptr) == ATTN_ERR_INVALID_ARG);
  EXPECT(attn_fwd(ATTN_BF16, P, P, P, P, F + 0, 1, 1, 16, 128, 0.1f, 0, 0, KV + 0, nullptr) == ATTN_OK);
  EXPECT(attn_fwd(ATTN_BF16, P, P, P, P, reinterpret_cast<float*>(P + 2), 1, 1, 16, 128, 0.1f, 0, 0, nullptr,
                  nullptr) == ATTN_ERR_INVALID_ARG);
  EXPECT(attn_fwd(ATTN_BF16, P, P, P, P, F, 1, 1, 16, 128, 0.1f, 0, 0, reinterpret_cast<const int32_t*>(P + 1),
                  nullptr) == ATTN_ERR_INVALID_ARG);
  EXPECT(attn_fwd(ATTN_BF16, P, P, P, P, F, 1 << 12, 1 << 12, 1 << 12, 128, 0.1f, 0, 0, nullptr, nullptr) ==
         ATTN_ERR_INVALID_ARG);
  EXPECT(attn_fwd(static_cast<attn_dtype_t>(9), P, P, P, P, F, 1, 1, 16, 128, 0.1f, 0, 0, nullptr, nullptr) ==
         ATTN_ERR_INVALID_ARG);
  EXPECT(g_launches == before + 1);  // only the valid call in the middle launched

  // The variants.
  EXPECT(attn_fwd_exp2_offload(P, P, P, P, F, 1, 2, 300, 128, 0.1f, 1, 64, KV, 4, nullptr) == ATTN_OK);
  EXPECT(attn_fwd_exp2_offload(P, P, P, P, F, 1, 2, 300, 128, 0.1f, 1, 64, KV, 3, nullptr) == ATTN_ERR_UNSUPPORTED);
  EXPECT(attn_fwd_fp8(P, P, P, P, F, 1, 2, 300, 128, 0.1f, 0.5f, 0.25f, 2.0f, 1, 0, nullptr, nullptr) == ATTN_OK);
  EXPECT(attn_fwd_fp8(P, P, P, P, F, 1, 2, 300, 128, 0.1f, 1e30f, 1e30f, 2.0f, 1, 0, nullptr, nullptr) ==
         ATTN_ERR_INVALID_ARG);
  EXPECT(attn_bwd(ATTN_BF16, P, P, P, P, P, F, P, P, P, 1, 2, 300, 128, 0.1f, 1, 0, nullptr, P,
                  attn_bwd_workspace_bytes(1, 2, 300), nullptr) == ATTN_OK);
  EXPECT(attn_bwd(ATTN_BF16, P, P, P, P, P, F, P, P, P, 1, 2, 300, 128, 0.1f, 1, 0, nullptr, P,
                  attn_bwd_workspace_bytes(1, 2, 300) - 1, nullptr) == ATTN_ERR_INVALID_ARG);
  // The stored-dS way: chosen by the workspace size, tiles after the D / LSE part rounded up to 256 bytes.
  const size_t bmin = attn_bwd_workspace_bytes(1, 2, 300), bst = attn_bwd_stored_ds_workspace_bytes(1, 2, 300, 1, 0);
  EXPECT(bst == 4864 + size_t(2) * 10 * 10 * 2048);  // 2*300*4*2 = 4800 -> 4864; 10 query blocks x 10 key blocks
  EXPECT(attn_bwd(ATTN_BF16, P, P, P, P, P, F, P, P, P, 1, 2, 300, 128, 0.1f, 1, 0, nullptr, P, bmin, nullptr) == ATTN_OK);
  EXPECT(g_bwd.ds == nullptr);
  EXPECT(attn_bwd(ATTN_BF16, P, P, P, P, P, F, P, P, P, 1, 2, 300, 128, 0.1f, 1, 0, nullptr, P, bst, nullptr) == ATTN_OK);
  EXPECT(g_bwd.ds == static_cast<char*>(P) + 4864);
  EXPECT(attn_bwd(ATTN_BF16, P, P, P, P, P, F, P, P, P, 1, 2, 300, 128, 0.1f, 1, 0, nullptr, P, bst - 1, nullptr) ==
         ATTN_OK);
  EXPECT(g_bwd.ds == nullptr);
  EXPECT(attn_bwd_stored_ds_workspace_bytes(1, 1, 8192, 1, 1024) == 65536 + size_t(256) * 33 * 2048);
  EXPECT(attn_bwd_stored_ds_workspace_bytes(1, 1, 8192, 0, 1024) == 65536 + size_t(256) * 66 * 2048);
  EXPECT(attn_bwd_stored_ds_workspace_bytes(1, 1, 100, 1, 5000) == 1024 + size_t(4) * 4 * 2048);  // window > N: clamped
  EXPECT(attn_bwd_stored_ds_workspace_bytes(1, 1, 1 << 20, 0, 0) == 0);  // one head's tiles > 2^31 bytes
  EXPECT(attn_bwd_stored_ds_workspace_bytes(0, 1, 8, 0, 0) == 0);
  EXPECT(attn_bwd_stored_ds_workspace_bytes(1, 1, 8, 2, 0) == 0);

  // Decode.
  const size_t ws = attn_decode_splitkv_workspace_bytes(1, 32, 128, 64);
  EXPECT(ws == size_t(32) * 64 * 130 * 4);
  EXPECT(attn_decode_splitkv(ATTN_BF16, P, P, P, F, 1, 32, 131072, 128, 64, P, ws, nullptr) == ATTN_OK);
  EXPECT(g_dec.Nkv == 131072 && g_dec.nsplit == 64 && g_dec.d == 128);
  EXPECT(attn_decode_splitkv(ATTN_BF16, P, P, P, F, 1, 32, 131072, 128, 64, P, ws - 4, nullptr) == ATTN_ERR_INVALID_ARG);
  EXPECT(attn_decode_splitkv(ATTN_F32, P, P, P, F, 1, 1, 10, 64, 11, P, ws, nullptr) == ATTN_ERR_INVALID_ARG);
  // The allocation-free variant: same checks, and the partials must fit in its scratch.
  g_launches = 0;
  EXPECT(attn_decode_splitkv_noalloc(ATTN_BF16, P, P, P, F, 1, 32, 131072, 128, 64, nullptr) == ATTN_OK);
  EXPECT(g_launches == 1 && g_dec.ws == nullptr && g_dec.nsplit == 64);
  EXPECT(attn_decode_splitkv_noalloc(ATTN_BF16, P, P, P, F, 8, 32, 131072, 128, 64, nullptr) == ATTN_ERR_INVALID_ARG);
  EXPECT(std::strstr(attn_last_error(), "scratch") != nullptr);
  EXPECT(attn_decode_splitkv_noalloc(ATTN_BF16, P, P, P, F, 1, 32, 131072, 96, 64, nullptr) == ATTN_ERR_UNSUPPORTED);
  EXPECT(attn_decode_splitkv_noalloc(ATTN_BF16, P + 8, P, P, F, 1, 32, 131072, 128, 64, nullptr) ==
         ATTN_ERR_INVALID_ARG);
  EXPECT(g_launches == 1);

  // Softmax and top-k (x == y allowed, partial overlap refused).
  EXPECT(online_softmax_rows(F, F, 4, 100, nullptr) == ATTN_OK);
  EXPECT(online_softmax_rows(F, F + 3, 4, 100, nullptr) == ATTN_ERR_INVALID_ARG);
  EXPECT(online_softmax_topk_rows(F, nullptr, F + 4096, reinterpret_cast<int32_t*>(P + 65536), 4, 100, 5, nullptr) ==
         ATTN_OK);
  EXPECT(online_softmax_topk_rows(F, nullptr, F + 4096, reinterpret_cast<int32_t*>(P + 65536), 4, 100, 17, nullptr) ==
         ATTN_ERR_UNSUPPORTED);

  // A failing launcher: ATTN_ERR_HIP with the runtime's text.
  g_result = hipErrorInvalidValue;
  EXPECT(online_softmax_rows(F, F, 4, 100, nullptr) == ATTN_ERR_HIP);
  EXPECT(std::strstr(attn_last_error(), "stub launch error") != nullptr);
  g_result = hipSuccess;

  // OSFA_SYNC_CHECK=1: one synchronization per successful call, none otherwise.
  setenv("OSFA_SYNC_CHECK", "1", 1);
  g_syncs = 0;
  EXPECT(online_softmax_rows(F, F, 4, 100, nullptr) == ATTN_OK);
  EXPECT(attn_fwd(ATTN_BF16, P, P, P, P, F, 1, 1, 16, 128, 0.1f, 0, 0, nullptr, nullptr) == ATTN_OK);
  EXPECT(attn_fwd(ATTN_BF16, P, P, P, P, F, 1, 1, 16, 96, 0.1f, 0, 0, nullptr, nullptr) == ATTN_ERR_UNSUPPORTED);
  EXPECT(g_syncs == 2);
  setenv("OSFA_SYNC_CHECK", "0", 1);
  EXPECT(online_softmax_rows(F, F, 4, 100, nullptr) == ATTN_OK);
  EXPECT(g_syncs == 2);

  // Error text is per thread and long messages are truncated safely.
  EXPECT(attn_fwd(ATTN_BF16, P, P, P, P, F, 1, 1, 16, 96, 0.1f, 0, 0, nullptr, nullptr) == ATTN_ERR_UNSUPPORTED);
  std::string other = "unset";
  std::thread t([&] { other = attn_last_error(); });
  t.join();
  EXPECT(other.empty());
  EXPECT(std::strstr(attn_last_error(), "head dim") != nullptr);
  EXPECT(std::strstr(osfa_version(), "gfx950") != nullptr);

  if (g_fails == 0) std::printf("abi host check ok\n");
  return g_fails == 0 ? 0 : 1;
}

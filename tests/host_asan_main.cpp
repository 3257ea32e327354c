// Host-side check of the C ABI's argument validation and failure reporting,
// built with AddressSanitizer on the host code only (the test that builds it
// instruments the driver's host code; device code is not instrumented).
//
// Every call here either fails validation (before any HIP call) or, on a host
// without a GPU, fails at its first HIP runtime call.  No pointer passed is
// ever dereferenced on these paths; they are aligned stand-ins.  Prints one
// line per case and "ALL OK" at the end; exits non-zero on a wrong status.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "ringattn.h"

namespace {

int g_fail = 0;

void expect(const char* what, int got, int want, const char* needle) {
  const char* msg = ringattn_last_error();
  const bool ok = got == want && (needle == nullptr || std::strstr(msg, needle) != nullptr);
  std::printf("%s %s: status %d (want %d) \"%s\"\n", ok ? "ok  " : "FAIL", what, got, want, msg);
  if (!ok) g_fail = 1;
}

}  // namespace

int main(int argc, char** argv) {
  const bool no_gpu = argc > 1 && std::strcmp(argv[1], "--no-gpu") == 0;
  void* F = reinterpret_cast<void*>(uintptr_t{0x10000});
  void* M = reinterpret_cast<void*>(uintptr_t{0x10008});
  float* Ff = static_cast<float*>(F);
  float* Mf = static_cast<float*>(M);

  // forward: bad arguments (both dtypes).
  for (int f32 = 0; f32 < 2; ++f32) {
    auto fwd = [&](void* q, void* k, void* out, float* lse, int64_t N, int P, int rank, int Hq, int Hkv, int d,
                   int causal, int layout) {
      return f32 ? ringattn_forward_f32(static_cast<float*>(q), static_cast<float*>(k), Ff, static_cast<float*>(out),
                                        lse, N, P, rank, Hq, Hkv, d, causal, layout, nullptr)
                 : ringattn_forward(q, k, F, out, lse, N, P, rank, Hq, Hkv, d, causal, layout, nullptr);
    };
    expect("forward null q", fwd(nullptr, F, F, nullptr, 1024, 4, 0, 4, 2, 128, 1, 0), RINGATTN_EINVAL, "non-null");
    expect("forward misaligned k", fwd(F, M, F, nullptr, 1024, 4, 0, 4, 2, 128, 1, 0), RINGATTN_EINVAL, "aligned");
    expect("forward misaligned lse", fwd(F, F, F, Mf, 1024, 4, 0, 4, 2, 128, 1, 0), RINGATTN_EINVAL, "aligned");
    expect("forward P=0", fwd(F, F, F, nullptr, 1024, 0, 0, 4, 2, 128, 1, 0), RINGATTN_EINVAL, "P must be");
    expect("forward N%P", fwd(F, F, F, nullptr, 1023, 4, 0, 4, 2, 128, 1, 0), RINGATTN_EINVAL, "multiple of P");
    expect("forward rank", fwd(F, F, F, nullptr, 1024, 4, 4, 4, 2, 128, 1, 0), RINGATTN_EINVAL, "rank");
    expect("forward Hq%Hkv", fwd(F, F, F, nullptr, 1024, 4, 0, 3, 2, 128, 1, 0), RINGATTN_EINVAL, "Hq");
    expect("forward causal", fwd(F, F, F, nullptr, 1024, 4, 0, 4, 2, 128, 2, 0), RINGATTN_EINVAL, "causal");
    expect("forward layout", fwd(F, F, F, nullptr, 1024, 4, 0, 4, 2, 128, 1, 7), RINGATTN_EINVAL, "layout");
    expect("forward zigzag N%2P", fwd(F, F, F, nullptr, 1028, 4, 0, 4, 2, 128, 1, 2), RINGATTN_EINVAL, "2P");
    expect("forward d_h", fwd(F, F, F, nullptr, 1024, 4, 0, 4, 2, 96, 1, 0), RINGATTN_EUNSUPPORTED, "d_h");
    expect("forward too large", fwd(F, F, F, nullptr, int64_t{1} << 31, 4, 0, 4, 2, 128, 1, 0),
           RINGATTN_EUNSUPPORTED, "too large");
  }

  // backward, merge, decode: bad arguments.
  expect("backward null dout",
         ringattn_backward(F, F, F, F, Ff, nullptr, Ff, Ff, Ff, 1024, 4, 0, 4, 2, 128, 1, 0, nullptr),
         RINGATTN_EINVAL, "non-null");
  expect("backward misaligned dq",
         ringattn_backward(F, F, F, F, Ff, F, Mf, Ff, Ff, 1024, 4, 0, 4, 2, 128, 1, 0, nullptr), RINGATTN_EINVAL,
         "aligned");
  expect("merge nparts", ringattn_merge(Ff, Ff, Ff, 0, 10, 4, 128, F, 0, nullptr, nullptr), RINGATTN_EINVAL,
         "nparts");
  expect("merge d_h", ringattn_merge(Ff, Ff, Ff, 2, 10, 4, 32, F, 0, nullptr, nullptr), RINGATTN_EUNSUPPORTED,
         "d_h");
  expect("merge zero rows", ringattn_merge(Ff, Ff, Ff, 2, 0, 4, 128, F, 0, nullptr, nullptr), RINGATTN_OK, nullptr);
  expect("decode n_q", ringattn_decode_partial(F, F, F, 0, 10, 4, 1, 128, Ff, Ff, Ff, nullptr), RINGATTN_EINVAL,
         "n_q");
  expect("decode too large", ringattn_decode_partial(F, F, F, 1 << 20, 10, 1, 1, 128, Ff, Ff, Ff, nullptr),
         RINGATTN_EUNSUPPORTED, "too large");
  expect("status string", std::strcmp(ringattn_status_string(RINGATTN_EHIP), "HIP runtime error"), 0, nullptr);

  // Valid arguments on a host without a GPU: the first HIP call fails and the
  // error comes back as a status and a message, not an abort.
  if (no_gpu) {
    expect("forward, no GPU", ringattn_forward(F, F, F, F, Ff, 1024, 4, 3, 4, 2, 128, 1, 0, nullptr),
           RINGATTN_EHIP, "failed");
    expect("forward_f32, no GPU", ringattn_forward_f32(Ff, Ff, Ff, Ff, Ff, 1024, 4, 0, 4, 2, 64, 0, 1, nullptr),
           RINGATTN_EHIP, "failed");
    expect("backward, no GPU",
           ringattn_backward(F, F, F, F, Ff, F, Ff, Ff, Ff, 1024, 4, 1, 4, 2, 128, 1, 2, nullptr), RINGATTN_EHIP,
           "failed");
    expect("merge, no GPU", ringattn_merge(Ff, Ff, Ff, 2, 10, 4, 128, F, 0, Ff, nullptr), RINGATTN_EHIP, "failed");
    expect("decode, no GPU", ringattn_decode_partial(F, F, F, 1, 1000, 8, 2, 128, Ff, Ff, Ff, nullptr),
           RINGATTN_EHIP, "failed");
    int64_t a = -1, b = -1;
    expect("redo count, no GPU", ringattn_redo_count(&a, &b), RINGATTN_EHIP, nullptr);
  }
  std::printf(g_fail ? "SOME FAILED\n" : "ALL OK\n");
  return g_fail;
}

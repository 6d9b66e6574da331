// Sweeps the C ABI (include/vsel.h) over shapes and arguments in a host build
// of csrc/api.cpp linked with the checking launch stand-ins
// (api_launch_stubs.cpp), under AddressSanitizer and UndefinedBehaviorSanitizer.
// The sweep covers argument validation, workspace sizing and layout, and the
// segment plans of every entry point: each call's workspace is sized by
// vsel_workspace_bytes and declared to the stand-ins, which check every array
// the kernels would address.  Device pointers are placeholders (nothing is
// dereferenced: no kernel runs).
#include <cstdint>
#include <cstdio>
#include <initializer_list>

#include "../../include/vsel.h"

namespace stub {
extern uintptr_t ws_lo, ws_hi;
extern long launches, failures;
}  // namespace stub

namespace {

int errors = 0;
// placeholders: 256-byte aligned, far apart, never dereferenced
char* const kIn = reinterpret_cast<char*>(uintptr_t(1) << 40);
char* const kOut = reinterpret_cast<char*>(uintptr_t(1) << 41);
char* const kWs = reinterpret_cast<char*>(uintptr_t(1) << 42);

size_t declare(int op, int dt, int64_t rows, int64_t V, int32_t k) {
  const size_t n = vsel_workspace_bytes(op, dt, rows, V, k);
  stub::ws_lo = reinterpret_cast<uintptr_t>(kWs);
  stub::ws_hi = stub::ws_lo + n;
  return n;
}

void expect(int got, int want, const char* what, int64_t rows, int64_t V, int64_t k) {
  if (got != want) {
    ++errors;
    std::fprintf(stderr, "%s rows %lld V %lld k %lld: status %d, expected %d\n", what, (long long)rows,
                 (long long)V, (long long)k, got, want);
  }
}

template <class T>
T* out(size_t off = 0) {
  return reinterpret_cast<T*>(kOut + off);
}

void selection(int dt, int64_t rows, int64_t V, int64_t ld) {
  const void* x = kIn + (ld % 2 ? 2 : 0) * (dt == VSEL_F32 ? 2 : 1);  // element-aligned, not always 16-byte
  size_t n = declare(VSEL_OP_ARGMAX, dt, rows, V, 0);
  expect(vsel_argmax(x, dt, rows, V, ld, out<uint32_t>(), out<float>(1 << 20), kWs, n, nullptr), VSEL_OK, "argmax",
         rows, V, 0);
  expect(vsel_argmax_excluding(x, dt, rows, V, ld, out<uint32_t>(2 << 20), 17, out<uint32_t>(), out<uint32_t>(4096),
                               kWs, n, nullptr),
         VSEL_OK, "argmax_excluding", rows, V, 0);
  for (int32_t k : {1, 20, 64, 84, 128, 129, 500, 1024}) {
    if (k > V) continue;
    n = declare(VSEL_OP_TOPK, dt, rows, V, k);
    expect(vsel_topk(x, dt, rows, V, ld, k, out<float>(), out<uint32_t>(8 << 20), out<uint32_t>(16 << 20),
                     out<float>(17 << 20), kWs, n, nullptr),
           VSEL_OK, "topk", rows, V, k);
    expect(vsel_topk(x, dt, rows, V, ld, k, out<float>(), out<uint32_t>(8 << 20), nullptr, nullptr, kWs, n / 2,
                     nullptr),
           n / 2 >= vsel_workspace_bytes(VSEL_OP_TOPK, dt, rows, V, k) ? VSEL_OK : VSEL_EWORKSPACE, "topk (half ws)",
           rows, V, k);
  }
  for (int32_t k : {0, 1, 2, 20, 128, 1024}) {
    n = declare(VSEL_OP_SAMPLE, dt, rows, V, k);
    for (float T : {0.0f, 0.7f})
      for (float tp : {1.0f, 0.9f})
        expect(vsel_sample(x, dt, rows, V, ld, T, k, tp, out<float>(), out<uint32_t>(4096), out<float>(8192), kWs, n,
                           nullptr),
               VSEL_OK, "sample", rows, V, k);
    n = declare(VSEL_OP_SAMPLE_CHAIN, dt, rows, V, k);
    struct Chain { float sig, typ, tp, mp; };
    for (const Chain& c : {Chain{0, 1, 1, 0}, Chain{1, 1, 1, 0.05f}, Chain{0, 0.9f, 1, 0}, Chain{1, 0.9f, 0.8f, 0.1f},
                           Chain{0, 1, 0.95f, 0}, Chain{2, 0.5f, 1, 0}}) {
      expect(vsel_sample_chain(x, dt, rows, V, ld, 0.8f, c.sig, k, c.typ, c.tp, c.mp, out<float>(), out<uint32_t>(4096),
                               out<float>(8192), kWs, n, nullptr),
             VSEL_OK, "sample_chain", rows, V, k);
    }
  }
}

void speculative(int64_t B, int32_t G, int64_t V, int64_t ld) {
  const float* t = reinterpret_cast<const float*>(kIn);
  const float* d = reinterpret_cast<const float*>(kIn + (uintptr_t(1) << 36));
  size_t n = declare(VSEL_OP_SPEC_ACCEPT, VSEL_F32, B, V, G);
  for (float T : {0.0f, 1.0f})
    expect(vsel_spec_accept(t, ld, d, ld, B, G, V, T, out<uint32_t>(), out<float>(4096), out<float>(8192),
                            out<float>(12288), out<int32_t>(16384), out<uint32_t>(20480), out<int32_t>(24576),
                            out<uint32_t>(28672), out<float>(1 << 20), out<float>(2 << 20), kWs, n, nullptr),
           VSEL_OK, "spec_accept", B, V, G);
  expect(vsel_spec_match(t, ld, d, ld, B, G, V, 0.7f, out<uint32_t>(), out<float>(4096), out<int32_t>(16384),
                         out<uint32_t>(20480), out<float>(1 << 20), kWs, n, nullptr),
         VSEL_OK, "spec_match", B, V, G);
  n = declare(VSEL_OP_SPEC_FILTERED, VSEL_F32, B, V, G);
  struct Filt { int32_t k; float tp, mp; };
  for (const Filt& f : {Filt{0, 1, 0}, Filt{1, 1, 0}, Filt{50, 0.95f, 0}, Filt{0, 0.9f, 0}, Filt{0, 1, 0.05f},
                        Filt{200, 0.8f, 0.1f}, Filt{1024, 1, 0}}) {
    if (f.k > V) continue;
    expect(vsel_spec_accept_filtered(t, ld, d, ld, B, G, V, 0.9f, f.k, f.tp, f.mp, out<uint32_t>(), out<float>(4096),
                                     out<float>(8192), out<float>(12288), out<int32_t>(16384), out<uint32_t>(20480),
                                     nullptr, nullptr, out<float>(1 << 20), nullptr, kWs, n, nullptr),
           VSEL_OK, "spec_accept_filtered", B, V, G);
    expect(vsel_spec_match_filtered(t, ld, d, ld, B, G, V, 0.9f, f.k, f.tp, f.mp, out<uint32_t>(), out<float>(4096),
                                    out<int32_t>(16384), out<uint32_t>(20480), nullptr, kWs, n, nullptr),
           VSEL_OK, "spec_match_filtered", B, V, G);
  }
}

void bad_arguments() {
  // sizes the ABI rejects size to 0 and are refused before any launch
  for (int op = 0; op <= 5; ++op) {
    for (int64_t rows : {int64_t(0), int64_t(-3), int64_t(1) << 40})
      if (vsel_workspace_bytes(op, VSEL_F32, rows, 1000, 8) != 0) ++errors;
    for (int64_t V : {int64_t(0), int64_t(1) << 31, int64_t(1) << 62})
      if (vsel_workspace_bytes(op, VSEL_F32, 4, V, 8) != 0) ++errors;
  }
  const long before = stub::launches;
  stub::ws_lo = stub::ws_hi = 0;
  expect(vsel_topk(kIn, VSEL_F32, INT64_MAX / 2, 1000, 1000, 8, out<float>(), out<uint32_t>(), nullptr, nullptr, kWs,
                   SIZE_MAX, nullptr),
         VSEL_EINVAL, "topk huge rows", INT64_MAX / 2, 1000, 8);
  expect(vsel_sample(kIn, VSEL_F32, 4, int64_t(1) << 30, int64_t(1) << 30, 0.7f, 0, 1.0f, out<float>(),
                     out<uint32_t>(), nullptr, kWs, SIZE_MAX, nullptr),
         VSEL_EINVAL, "sample whole row past the draw limit", 4, int64_t(1) << 30, 0);
  expect(vsel_spec_accept(reinterpret_cast<const float*>(kIn), 100, reinterpret_cast<const float*>(kIn), 100,
                          int64_t(1) << 40, 8, 100, 1.0f, out<uint32_t>(), out<float>(), out<float>(), out<float>(),
                          out<int32_t>(), out<uint32_t>(), nullptr, nullptr, nullptr, nullptr, kWs, SIZE_MAX, nullptr),
         VSEL_EINVAL, "spec huge batch", int64_t(1) << 40, 100, 8);
  if (stub::launches != before) ++errors;
}

}  // namespace

int main() {
  for (int dt : {VSEL_F32, VSEL_BF16})
    for (int64_t rows : {1, 3, 49, 64, 1024, 4100})
      for (int64_t V : {1, 7, 1000, 20011, 202048, 248320})
        for (int64_t pad : {0, 3, 64}) {
          if (rows * V > (int64_t)300e6 && pad == 3) continue;
          selection(dt, rows, V, V + pad);
        }
  selection(VSEL_F32, 2, 67108864, 67108864);  // the largest whole-row draw
  for (int64_t B : {1, 5, 32, 128})
    for (int32_t G : {1, 3, 8, 16})
      for (int64_t V : {2, 7, 1000, 202048}) speculative(B, G, V, V + (B % 2));
  bad_arguments();
  std::printf("api driver: %ld launches checked, %ld launch failures, %d call failures\n", stub::launches,
              stub::failures, errors);
  return (errors == 0 && stub::failures == 0 && stub::launches > 1000) ? 0 : 1;
}

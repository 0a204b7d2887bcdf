// Host-side checks of the C ABI (include/switch_moe.h), meant to be built
// with AddressSanitizer and UndefinedBehaviorSanitizer on the host code of
// every library source.  It drives argument validation, the capacity
// arithmetic, every workspace-size function, the launch-name list, the error
// text and the debug-sync path over shapes from empty to the largest
// supported, and checks each return code.  Calls that pass validation are
// made only where no GPU is visible: their kernel launches then fail with a
// HIP error (the buffers here are host stand-ins that no kernel may touch).
// Prints "abi_check ok" and exits 0 when every check holds; any sanitizer
// report aborts the run.

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "../include/switch_moe.h"

namespace {

int g_failures = 0;
int g_checks = 0;
bool g_launch = false;  // no GPU visible: calls that pass validation may be made

#define CHECK(cond, ...)                                        \
  do {                                                          \
    ++g_checks;                                                 \
    if (!(cond)) {                                              \
      std::fprintf(stderr, "FAIL line %d: ", __LINE__);         \
      std::fprintf(stderr, __VA_ARGS__);                        \
      std::fputc('\n', stderr);                                 \
      ++g_failures;                                             \
    }                                                           \
  } while (0)

// A failed call leaves a non-empty, terminated message of bounded length.
void expect_rc(int rc, int want, int line) {
  ++g_checks;
  if (rc != want) {
    std::fprintf(stderr, "FAIL line %d: rc %d, expected %d (%s)\n", line, rc, want, switch_last_error());
    ++g_failures;
    return;
  }
  if (rc != SWITCH_OK) {
    const char *e = switch_last_error();
    const size_t n = e ? std::strlen(e) : 0;
    CHECK(e && n > 0 && n < 512, "error text of rc %d: length %zu", rc, n);
  }
}
#define EXPECT(call, want) expect_rc((call), (want), __LINE__)

// A call that passes validation launches a kernel; without device code the
// launch fails, so the result is SWITCH_E_HIP (or SWITCH_OK where the call
// launches nothing).
void expect_launch(int rc, int line) {
  ++g_checks;
  if (rc != SWITCH_E_HIP && rc != SWITCH_OK) {
    std::fprintf(stderr, "FAIL line %d: rc %d after validation (%s)\n", line, rc, switch_last_error());
    ++g_failures;
  }
}
#define EXPECT_LAUNCH(call)                     \
  do {                                          \
    if (g_launch) expect_launch((call), __LINE__); \
  } while (0)

switch_shape shape(int64_t T, int d, int f, int N, int C, int dtype) {
  switch_shape s;
  s.tokens = T;
  s.d_model = d;
  s.d_ff = f;
  s.num_experts = N;
  s.capacity = C;
  s.dtype = dtype;
  return s;
}

// Stand-ins for device buffers: 256-byte aligned host blocks.  Host code only
// checks their alignment; nothing dereferences them on the host, and no
// kernel can run without device code.
struct Buf {
  void *p;
  explicit Buf(size_t bytes = 4096) : p(std::aligned_alloc(256, bytes)) {}
  ~Buf() { std::free(p); }
  Buf(const Buf &) = delete;
  Buf &operator=(const Buf &) = delete;
  template <typename T>
  T *as(size_t offset = 0) const {
    return reinterpret_cast<T *>(static_cast<char *>(p) + offset);
  }
};

void capacity_checks() {
  int32_t c = -1;
  EXPECT(switch_capacity(16384, 128, 1.25, &c), SWITCH_OK);
  CHECK(c == 160, "capacity(16384, 128, 1.25) = %d", c);
  EXPECT(switch_capacity(0, 8, 1.0, &c), SWITCH_OK);
  CHECK(c == 0, "capacity(0, 8, 1) = %d", c);
  EXPECT(switch_capacity(10, 3, 1.0, &c), SWITCH_OK);
  CHECK(c == 4, "capacity(10, 3, 1) = %d", c);
  EXPECT(switch_capacity(-1, 8, 1.0, &c), SWITCH_E_INVALID);
  EXPECT(switch_capacity(16, 0, 1.0, &c), SWITCH_E_INVALID);
  EXPECT(switch_capacity(16, 8, 0.0, &c), SWITCH_E_INVALID);
  EXPECT(switch_capacity(16, 8, -1.0, &c), SWITCH_E_INVALID);
  EXPECT(switch_capacity(16, 8, std::nan(""), &c), SWITCH_E_INVALID);
  EXPECT(switch_capacity(16, 8, std::numeric_limits<double>::infinity(), &c), SWITCH_E_INVALID);
  EXPECT(switch_capacity(16, 8, 1.0, nullptr), SWITCH_E_INVALID);
  EXPECT(switch_capacity(std::numeric_limits<int64_t>::max(), 1, 1.0, &c), SWITCH_E_UNSUPPORTED);
  EXPECT(switch_capacity(1 << 30, 1, 1e300, &c), SWITCH_E_UNSUPPORTED);
  EXPECT(switch_capacity(1, 1, 5e-324, &c), SWITCH_OK);
  CHECK(c == 1, "capacity(1, 1, denormal) = %d", c);
}

void size_checks() {
  size_t b = 0;
  const switch_shape shapes[] = {
      shape(0, 64, 64, 1, 0, SWITCH_F32),        shape(512, 64, 256, 8, 64, SWITCH_F32),
      shape(16384, 768, 3072, 128, 160, SWITCH_BF16), shape(16384, 1024, 2816, 128, 128, SWITCH_BF16),
      shape(8192, 4096, 10240, 64, 160, SWITCH_BF16), shape(32768, 2048, 6144, 2048, 16, SWITCH_BF16),
      shape(7, 64, 128, 3, 0, SWITCH_BF16),      shape(1, 64, 64, 4096, 1, SWITCH_BF16),
  };
  for (const auto &s : shapes) {
    EXPECT(switch_workspace_bytes(&s, &b), SWITCH_OK);
    CHECK(b % 256 == 0, "workspace bytes %zu not a multiple of 256", b);
    size_t bb = 0;
    EXPECT(switch_backward_workspace_bytes(&s, &bb), SWITCH_OK);
    for (int k = 1; k <= 2 && k <= s.num_experts; ++k) {
      size_t kb = 0;
      EXPECT(switch_topk_workspace_bytes(&s, k, &kb), SWITCH_OK);
      if (k == 1) CHECK(kb == b, "top-1 workspace %zu differs from the layer's %zu", kb, b);
    }
    const char *names[8] = {};
    int32_t n = -1;
    EXPECT(switch_launch_names(&s, names, 8, &n), SWITCH_OK);
    CHECK(n >= 3 && n <= 5, "launch names: %d", n);
    for (int i = 0; i < n; ++i) CHECK(names[i] && names[i][0], "launch name %d empty", i);
    EXPECT(switch_launch_names(&s, names, 1, &n), SWITCH_OK);
    EXPECT(switch_launch_names(&s, nullptr, 0, &n), SWITCH_OK);
    EXPECT(switch_launch_names(&s, nullptr, 3, &n), SWITCH_E_INVALID);
  }
  switch_shape s = shape(16384, 768, 3072, 128, 160, SWITCH_BF16);
  EXPECT(switch_workspace_bytes(nullptr, &b), SWITCH_E_INVALID);
  EXPECT(switch_workspace_bytes(&s, nullptr), SWITCH_E_INVALID);
  switch_shape bad = s;
  bad.d_model = 96;
  EXPECT(switch_workspace_bytes(&bad, &b), SWITCH_E_UNSUPPORTED);
  bad = s;
  bad.tokens = (int64_t)1 << 31;
  EXPECT(switch_workspace_bytes(&bad, &b), SWITCH_E_UNSUPPORTED);
  bad = s;
  bad.tokens = -5;
  EXPECT(switch_workspace_bytes(&bad, &b), SWITCH_E_INVALID);
  bad = s;
  bad.dtype = 7;
  EXPECT(switch_workspace_bytes(&bad, &b), SWITCH_E_INVALID);
  bad = s;
  bad.capacity = -1;
  EXPECT(switch_workspace_bytes(&bad, &b), SWITCH_E_INVALID);
  bad = s;
  bad.num_experts = 0;
  EXPECT(switch_workspace_bytes(&bad, &b), SWITCH_E_INVALID);
  // sizes whose products pass 2^62
  bad = shape((1LL << 31) - 1, 1 << 24, 1 << 24, 1 << 20, 1 << 30, SWITCH_F32);
  EXPECT(switch_workspace_bytes(&bad, &b), SWITCH_E_UNSUPPORTED);
  EXPECT(switch_backward_workspace_bytes(&bad, &b), SWITCH_E_UNSUPPORTED);
  EXPECT(switch_topk_workspace_bytes(&s, 0, &b), SWITCH_E_INVALID);
  EXPECT(switch_topk_workspace_bytes(&s, 129, &b), SWITCH_E_INVALID);
  size_t nb = 0;
  EXPECT(switch_noalloc_scratch_bytes(&nb), SWITCH_OK);
  CHECK(nb > 0 && nb % 256 == 0, "no-allocation scratch %zu", nb);
  EXPECT(switch_noalloc_scratch_bytes(nullptr), SWITCH_E_INVALID);
}

void layer_checks() {
  const switch_shape s = shape(1024, 256, 512, 16, 80, SWITCH_BF16);
  size_t wsb = 0;
  EXPECT(switch_workspace_bytes(&s, &wsb), SWITCH_OK);
  Buf x, wr, w_in, w_out, y, idx, gate, slot, drop, cnt, aux, ws;
  auto fwd = [&](const switch_shape *sh, const void *xp, void *wsp, size_t wsbytes) {
    return switch_layer_forward(sh, xp, wr.as<float>(), nullptr, w_in.p, w_out.p, 0, y.p, idx.as<int32_t>(),
                                gate.as<float>(), slot.as<int32_t>(), drop.as<uint8_t>(), cnt.as<int32_t>(),
                                aux.as<float>(), wsp, wsbytes, nullptr);
  };
  EXPECT(fwd(nullptr, x.p, ws.p, wsb), SWITCH_E_INVALID);
  EXPECT(fwd(&s, nullptr, ws.p, wsb), SWITCH_E_INVALID);
  EXPECT(fwd(&s, x.as<char>(4), ws.p, wsb), SWITCH_E_INVALID);
  EXPECT(fwd(&s, x.p, nullptr, wsb), SWITCH_E_INVALID);
  EXPECT(fwd(&s, x.p, ws.as<char>(16), wsb), SWITCH_E_INVALID);
  EXPECT(fwd(&s, x.p, ws.p, wsb - 1), SWITCH_E_WORKSPACE);
  EXPECT_LAUNCH(fwd(&s, x.p, ws.p, wsb));
  switch_shape empty = s;
  empty.tokens = 0;
  size_t wse = 0;
  EXPECT(switch_workspace_bytes(&empty, &wse), SWITCH_OK);
  EXPECT_LAUNCH(fwd(&empty, nullptr, ws.p, wse));

  // measurement variant: kernel range and repeat count are validated first
  auto prof = [&](int first, int last, int times) {
    return switch_layer_forward_profiled(&s, x.p, wr.as<float>(), nullptr, w_in.p, w_out.p, 0, y.p,
                                         idx.as<int32_t>(), gate.as<float>(), slot.as<int32_t>(),
                                         drop.as<uint8_t>(), cnt.as<int32_t>(), aux.as<float>(), ws.p, wsb,
                                         nullptr, first, last, times);
  };
  EXPECT(prof(0, 3, 0), SWITCH_E_INVALID);
  EXPECT(prof(-1, 3, 1), SWITCH_E_INVALID);
  EXPECT(prof(3, 2, 1), SWITCH_E_INVALID);
  EXPECT_LAUNCH(prof(0, 3, 2));

  // top-k
  auto topk = [&](int k) {
    size_t kb = 0;
    if (switch_topk_workspace_bytes(&s, k, &kb) != SWITCH_OK) kb = wsb;
    return switch_topk_layer_forward(&s, k, x.p, wr.as<float>(), nullptr, w_in.p, w_out.p, 1, y.p,
                                     idx.as<int32_t>(), gate.as<float>(), slot.as<int32_t>(), drop.as<uint8_t>(),
                                     cnt.as<int32_t>(), aux.as<float>(), ws.p, kb, nullptr);
  };
  EXPECT(topk(0), SWITCH_E_INVALID);
  EXPECT(topk(17), SWITCH_E_INVALID);
  EXPECT_LAUNCH(topk(2));

  // no-allocation variant: a shape beyond its workspace is refused before
  // anything else; a fitting one reaches the device lookup or the launch
  switch_shape big = shape(16384, 4096, 10240, 64, 320, SWITCH_BF16);
  EXPECT(switch_layer_forward_noalloc(&big, x.p, wr.as<float>(), nullptr, w_in.p, w_out.p, 0, y.p,
                                      idx.as<int32_t>(), gate.as<float>(), slot.as<int32_t>(), drop.as<uint8_t>(),
                                      cnt.as<int32_t>(), aux.as<float>(), nullptr),
         SWITCH_E_WORKSPACE);
  EXPECT_LAUNCH(switch_layer_forward_noalloc(&s, x.p, wr.as<float>(), nullptr, w_in.p, w_out.p, 0, y.p,
                                             idx.as<int32_t>(), gate.as<float>(), slot.as<int32_t>(),
                                             drop.as<uint8_t>(), cnt.as<int32_t>(), aux.as<float>(), nullptr));
}

void stage_checks() {
  const switch_shape s = shape(1024, 256, 512, 16, 80, SWITCH_BF16);
  size_t wsb = 0;
  EXPECT(switch_workspace_bytes(&s, &wsb), SWITCH_OK);
  Buf x, wr, bias, w_in, w_out, y, idx, gate, slot, drop, cnt, aux, ws, disp, eo, gamma, beta, out;
  auto route = [&](const float *b, void *wsp, size_t n) {
    return switch_route(&s, x.p, wr.as<float>(), b, idx.as<int32_t>(), gate.as<float>(), slot.as<int32_t>(),
                        drop.as<uint8_t>(), cnt.as<int32_t>(), aux.as<float>(), wsp, n, nullptr);
  };
  EXPECT(route(bias.as<float>(2), ws.p, wsb), SWITCH_E_INVALID);
  EXPECT(route(nullptr, ws.p, 0), SWITCH_E_WORKSPACE);
  EXPECT_LAUNCH(route(bias.as<float>(), ws.p, wsb));

  auto rd = [&](const switch_shape *sh, void *d) {
    return switch_route_dispatch(sh, x.p, wr.as<float>(), nullptr, idx.as<int32_t>(), gate.as<float>(),
                                 slot.as<int32_t>(), drop.as<uint8_t>(), cnt.as<int32_t>(), aux.as<float>(), d,
                                 ws.p, wsb, nullptr);
  };
  switch_shape many = s;
  many.num_experts = 4096;
  EXPECT(rd(&many, disp.p), SWITCH_E_UNSUPPORTED);
  EXPECT(rd(&s, nullptr), SWITCH_E_INVALID);
  EXPECT_LAUNCH(rd(&s, disp.p));

  EXPECT(switch_dispatch(&s, x.p, idx.as<int32_t>(), slot.as<int32_t>(), nullptr, disp.p, nullptr),
         SWITCH_E_INVALID);
  EXPECT_LAUNCH(switch_dispatch(&s, x.p, idx.as<int32_t>(), slot.as<int32_t>(), drop.as<uint8_t>(), disp.p,
                                nullptr));
  EXPECT(switch_expert_ffn(&s, disp.p, cnt.as<int32_t>(), w_in.p, w_out.p, eo.p, ws.p, 16, nullptr),
         SWITCH_E_WORKSPACE);
  EXPECT_LAUNCH(switch_expert_ffn(&s, disp.p, cnt.as<int32_t>(), w_in.p, w_out.p, eo.p, ws.p, wsb, nullptr));
  EXPECT(switch_combine(&s, eo.p, idx.as<int32_t>(), slot.as<int32_t>(), drop.as<uint8_t>(), gate.as<float>(),
                        x.as<char>(8), y.p, nullptr),
         SWITCH_E_INVALID);
  EXPECT_LAUNCH(switch_combine(&s, eo.p, idx.as<int32_t>(), slot.as<int32_t>(), drop.as<uint8_t>(),
                               gate.as<float>(), x.p, y.p, nullptr));
  EXPECT(switch_add_norm(&s, x.p, y.p, gamma.as<float>(), beta.as<float>(), std::nanf(""), out.p, nullptr),
         SWITCH_E_INVALID);
  EXPECT(switch_add_norm(&s, x.p, y.p, gamma.as<float>(), beta.as<float>(), -1.f, out.p, nullptr),
         SWITCH_E_INVALID);
  switch_shape wide = s;
  wide.d_model = 1 << 20;
  EXPECT(switch_add_norm(&wide, x.p, y.p, gamma.as<float>(), beta.as<float>(), 1e-6f, out.p, nullptr),
         SWITCH_E_UNSUPPORTED);
  EXPECT_LAUNCH(switch_add_norm(&s, x.p, y.p, gamma.as<float>(), beta.as<float>(), 1e-6f, out.p, nullptr));
  EXPECT(switch_combine_add_norm(&s, eo.p, idx.as<int32_t>(), slot.as<int32_t>(), drop.as<uint8_t>(),
                                 gate.as<float>(), nullptr, gamma.as<float>(), beta.as<float>(), 1e-6f, out.p,
                                 nullptr),
         SWITCH_E_INVALID);
  EXPECT_LAUNCH(switch_combine_add_norm(&s, eo.p, idx.as<int32_t>(), slot.as<int32_t>(), drop.as<uint8_t>(),
                                        gate.as<float>(), x.p, gamma.as<float>(), beta.as<float>(), 1e-6f, out.p,
                                        nullptr));
}

void backward_checks() {
  const switch_shape s = shape(1024, 256, 512, 16, 80, SWITCH_BF16);
  size_t wsb = 0, bwb = 0;
  EXPECT(switch_workspace_bytes(&s, &wsb), SWITCH_OK);
  EXPECT(switch_backward_workspace_bytes(&s, &bwb), SWITCH_OK);
  Buf x, wr, w_in, w_out, idx, drop, cnt, fws, dy, dx, dwr, db, dwi, dwo, ws;
  auto bwd = [&](const void *fw, size_t fwb, float d_aux, size_t n) {
    return switch_layer_backward(&s, x.p, wr.as<float>(), nullptr, w_in.p, w_out.p, 0, idx.as<int32_t>(),
                                 drop.as<uint8_t>(), cnt.as<int32_t>(), fw, fwb, dy.p, d_aux, dx.p,
                                 dwr.as<float>(), db.as<float>(), dwi.p, dwo.p, ws.p, n, nullptr);
  };
  EXPECT(bwd(fws.p, wsb, std::nanf(""), bwb), SWITCH_E_INVALID);
  EXPECT(bwd(nullptr, wsb, 0.01f, bwb), SWITCH_E_INVALID);
  EXPECT(bwd(fws.p, wsb - 256, 0.01f, bwb), SWITCH_E_WORKSPACE);
  EXPECT(bwd(fws.p, wsb, 0.01f, bwb - 1), SWITCH_E_WORKSPACE);
  EXPECT_LAUNCH(bwd(fws.p, wsb, 0.01f, bwb));
  EXPECT(switch_layer_backward_profiled(&s, x.p, wr.as<float>(), nullptr, w_in.p, w_out.p, 0, idx.as<int32_t>(),
                                        drop.as<uint8_t>(), cnt.as<int32_t>(), fws.p, wsb, dy.p, 0.01f, dx.p,
                                        dwr.as<float>(), db.as<float>(), dwi.p, dwo.p, ws.p, bwb, nullptr, 2, 1, 1),
         SWITCH_E_INVALID);
}

}  // namespace

int main(int argc, char **argv) {
  // with "debug" the library's debug-sync mode is on for every call
  if (argc > 1 && std::strcmp(argv[1], "debug") == 0) setenv("SMX_DEBUG_SYNC", "1", 1);
  int devices = 0;
  if (hipGetDeviceCount(&devices) != hipSuccess) devices = 0;
  g_launch = devices == 0;
  if (!g_launch) std::printf("abi_check: %d GPU(s) visible: calls that would launch kernels are skipped\n", devices);
  capacity_checks();
  size_checks();
  layer_checks();
  stage_checks();
  backward_checks();
  if (g_failures) {
    std::fprintf(stderr, "abi_check: %d of %d checks failed\n", g_failures, g_checks);
    return 1;
  }
  std::printf("abi_check ok (%d checks)\n", g_checks);
  return 0;
}

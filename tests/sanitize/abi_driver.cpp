// abi_driver.cpp -- the host side of libgdn's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer, on the CPU: every call below is rejected by the
// argument checks (fake device pointers, never dereferenced), and the workspace
// queries run over many shapes.  Linked with launch stubs that fail loudly, so
// a call that got past validation would be reported rather than launched.
// Prints "ok <n>" with the number of checked calls; any sanitizer report or a
// wrong status ends the program with a non-zero exit code.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/gdn.h"

static int n_checked = 0;
static const char* g_case = "";

// CASE(name) names the call that follows (a stub that aborts prints it)
#define CASE(name) (g_case = (name))

extern "C" const char* abi_driver_case(void) { return g_case; }

static void expect(gdn_status got, gdn_status want, const char* what) {
  ++n_checked;
  if (got != want) {
    std::fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, (int)got, (int)want, gdn_last_error_message());
    std::exit(2);
  }
}

// dt as an int: an out-of-range value is written as the integer a C caller
// would store (the library reads it as such)
static gdn_problem problem(int64_t T, int64_t H, int64_t dk, int64_t dv, int dt) {
  gdn_problem p;
  std::memset(&p, 0, sizeof(p));
  p.batch = 1;
  p.seqlen = T;
  p.heads = H;
  p.dk = dk;
  p.dv = dv;
  p.chunk = 64;
  p.scale = 1.f;
  std::memcpy(&p.dtype, &dt, sizeof(dt));
  return p;
}

int main() {
  const uintptr_t F = (uintptr_t)0x7f0000000000ull;
  auto P = [&](uintptr_t off) { return reinterpret_cast<void*>(F + off); };
  const uintptr_t G = (uintptr_t)1 << 34;   // 16 GiB between fake tensors

  // workspace queries over shapes, dtypes, varlen tables, strides and normalisation
  for (int dt = 0; dt < 2; ++dt)
    for (int64_t dk : {64, 128, 96})
      for (int64_t dv : {64, 128})
        for (int64_t T : {0, 1, 63, 64, 65, 4096})
          for (int64_t H : {1, 3, 16})
            for (int l2 = 0; l2 < 2; ++l2) {
              gdn_problem p = problem(T, H, dk, dv, dt);
              p.qk_l2norm = l2;
              const size_t f = gdn_fwd_workspace_bytes(&p), b = gdn_bwd_workspace_bytes(&p);
              ++n_checked;
              if ((dk == 96) != (f == 0) || (f == 0) != (b == 0) || f % 256 || b % 256) {
                std::fprintf(stderr, "workspace sizes %zu %zu for dk %lld dv %lld T %lld\n", f, b, (long long)dk,
                             (long long)dv, (long long)T);
                return 3;
              }
            }
  // varlen tables: valid, decreasing, wrong end; the host copy is read N+1 entries far
  {
    std::vector<int32_t> cu = {0, 5, 5, 70, 200};
    gdn_problem p = problem(200, 2, 64, 128, GDN_BF16);
    p.num_seqs = 4;
    p.cu_seqlens_host = cu.data();
    p.cu_seqlens_dev = reinterpret_cast<const int32_t*>(P(0));
    ++n_checked;
    if (gdn_fwd_workspace_bytes(&p) == 0) return 4;
    cu[2] = 4;
    CASE("decreasing cu_seqlens");
    expect(gdn_fwd(&p, P(G), P(2 * G), P(3 * G), (const float*)P(4 * G), (const float*)P(5 * G), nullptr, P(6 * G),
                   nullptr, P(7 * G), (size_t)1 << 40, nullptr),
           GDN_ERR_INVALID_ARGUMENT, "decreasing cu_seqlens");
    cu[2] = 5;
    cu[4] = 199;
    CASE("cu_seqlens end");
    expect(gdn_fwd(&p, P(G), P(2 * G), P(3 * G), (const float*)P(4 * G), (const float*)P(5 * G), nullptr, P(6 * G),
                   nullptr, P(7 * G), (size_t)1 << 40, nullptr),
           GDN_ERR_INVALID_ARGUMENT, "cu_seqlens end");
  }
  // pointer checks: NULLs, misalignment, overlaps (also strided, interleaved rows)
  {
    gdn_problem p = problem(256, 2, 64, 64, GDN_BF16);
    const size_t need = gdn_fwd_workspace_bytes(&p);
    CASE("null q");
    expect(gdn_fwd(&p, nullptr, P(2 * G), P(3 * G), (const float*)P(4 * G), (const float*)P(5 * G), nullptr, P(6 * G),
                   nullptr, P(7 * G), need, nullptr),
           GDN_ERR_INVALID_ARGUMENT, "null q");
    CASE("misaligned q");
    expect(gdn_fwd(&p, P(G + 8), P(2 * G), P(3 * G), (const float*)P(4 * G), (const float*)P(5 * G), nullptr,
                   P(6 * G), nullptr, P(7 * G), need, nullptr),
           GDN_ERR_INVALID_ARGUMENT, "misaligned q");
    CASE("o overlaps q");
    expect(gdn_fwd(&p, P(G), P(2 * G), P(3 * G), (const float*)P(4 * G), (const float*)P(5 * G), nullptr, P(G + 64),
                   nullptr, P(7 * G), need, nullptr),
           GDN_ERR_INVALID_ARGUMENT, "o overlaps q");
    CASE("small workspace");
    expect(gdn_fwd(&p, P(G), P(2 * G), P(3 * G), (const float*)P(4 * G), (const float*)P(5 * G), nullptr, P(6 * G),
                   nullptr, P(7 * G), need - 256, nullptr),
           GDN_ERR_WORKSPACE_TOO_SMALL, "small workspace");
    // strided q, k, v in one buffer: rows interleave without sharing a byte (accepted by the
    // checks, so the forward would launch: only its validation-stage twin is called here)
    p.qkv_token_stride = 3 * 2 * 64;
    const size_t e = 2;
    CASE("o inside the strided buffer");
    expect(gdn_fwd(&p, P(G), P(G + 2 * 64 * e), P(G + 4 * 64 * e), (const float*)P(4 * G), (const float*)P(5 * G),
                   nullptr, P(G + 64), nullptr, P(7 * G), need, nullptr),
           GDN_ERR_INVALID_ARGUMENT, "o inside the strided buffer");
    // (inputs may alias each other; outputs may not touch inputs or each other)
    p.qkv_token_stride = 0;
    {
      // backward with q, k, v and dq, dk, dv interleaved in two [tokens][3*H*d] buffers: the
      // strided-overlap arithmetic runs over every pair; first the layouts are disjoint and
      // dg aliasing g is what rejects the call, then dk is shifted onto dq's rows
      gdn_problem ps = problem(256, 2, 64, 64, GDN_BF16);
      ps.qkv_token_stride = 3 * 2 * 64;
      const size_t nb = gdn_bwd_workspace_bytes(&ps);
      const uintptr_t X = G, Y = 20 * G, row = 2 * 64 * e;
      CASE("strided, disjoint; dg aliases g");
      expect(gdn_bwd(&ps, P(X), P(X + row), P(X + 2 * row), (const float*)P(4 * G), (const float*)P(5 * G), nullptr,
                     P(6 * G), nullptr, P(Y), P(Y + row), P(Y + 2 * row), (float*)P(4 * G), (float*)P(11 * G),
                     nullptr, nullptr, P(12 * G), nb, nullptr),
             GDN_ERR_INVALID_ARGUMENT, "strided, disjoint; dg aliases g");
      CASE("strided dk onto dq");
      expect(gdn_bwd(&ps, P(X), P(X + row), P(X + 2 * row), (const float*)P(4 * G), (const float*)P(5 * G), nullptr,
                     P(6 * G), nullptr, P(Y), P(Y + row - 16), P(Y + 2 * row), (float*)P(10 * G), (float*)P(11 * G),
                     nullptr, nullptr, P(12 * G), nb, nullptr),
             GDN_ERR_INVALID_ARGUMENT, "strided dk onto dq");
      CASE("strided dv onto the next token's q");
      expect(gdn_bwd(&ps, P(X), P(X + row), P(X + 2 * row), (const float*)P(4 * G), (const float*)P(5 * G), nullptr,
                     P(6 * G), nullptr, P(Y), P(Y + row), P(X + 3 * row - 16), (float*)P(10 * G), (float*)P(11 * G),
                     nullptr, nullptr, P(12 * G), nb, nullptr),
             GDN_ERR_INVALID_ARGUMENT, "strided dv onto the next token's q");
    }
    // backward: dq aliasing do, missing workspace
    const size_t needb = gdn_bwd_workspace_bytes(&p);
    CASE("dq aliases do");
    expect(gdn_bwd(&p, P(G), P(2 * G), P(3 * G), (const float*)P(4 * G), (const float*)P(5 * G), nullptr, P(6 * G),
                   nullptr, P(6 * G), P(8 * G), P(9 * G), (float*)P(10 * G), (float*)P(11 * G), nullptr, nullptr,
                   P(12 * G), needb, nullptr),
           GDN_ERR_INVALID_ARGUMENT, "dq aliases do");
    CASE("null workspace");
    expect(gdn_bwd(&p, P(G), P(2 * G), P(3 * G), (const float*)P(4 * G), (const float*)P(5 * G), nullptr, P(6 * G),
                   nullptr, P(7 * G), P(8 * G), P(9 * G), (float*)P(10 * G), (float*)P(11 * G), nullptr, nullptr,
                   nullptr, needb, nullptr),
           GDN_ERR_INVALID_ARGUMENT, "null workspace");
    // the allocation-free forward: beyond the static scratch
    gdn_problem big = problem(16384, 16, 64, 64, GDN_BF16);
    CASE("no-alloc limit");
    expect(gdn_fwd_noalloc(&big, P(G), P(2 * G), P(3 * G), (const float*)P(4 * G), (const float*)P(5 * G), nullptr,
                           P(6 * G), nullptr, nullptr),
           GDN_ERR_UNSUPPORTED, "no-alloc limit");
  }
  // problem fields
  {
    gdn_problem p = problem(256, 2, 64, 64, GDN_BF16);
    p.chunk = 32;
    CASE("chunk 32");
    expect(gdn_fwd(&p, P(G), P(2 * G), P(3 * G), nullptr, nullptr, nullptr, P(6 * G), nullptr, P(7 * G), 0, nullptr),
           GDN_ERR_UNSUPPORTED, "chunk 32");
    p = problem(256, 2, 64, 64, 7);
    CASE("dtype");
    expect(gdn_fwd(&p, P(G), P(2 * G), P(3 * G), nullptr, nullptr, nullptr, P(6 * G), nullptr, P(7 * G), 0, nullptr),
           GDN_ERR_UNSUPPORTED, "dtype");
    p = problem(256, 2, 64, 64, GDN_BF16);
    p.scale = 0.f / 0.f;
    CASE("scale nan");
    expect(gdn_fwd(&p, P(G), P(2 * G), P(3 * G), nullptr, nullptr, nullptr, P(6 * G), nullptr, P(7 * G), 0, nullptr),
           GDN_ERR_INVALID_ARGUMENT, "scale nan");
    CASE("null problem");
    expect(gdn_fwd(nullptr, P(G), P(2 * G), P(3 * G), nullptr, nullptr, nullptr, P(6 * G), nullptr, P(7 * G), 0,
                   nullptr),
           GDN_ERR_INVALID_ARGUMENT, "null problem");
  }
  // the layer's other entry points
  {
    gdn_gated_norm_problem g;
    std::memset(&g, 0, sizeof(g));
    g.rows = 100;
    g.dim = 96;
    g.dtype = GDN_BF16;
    CASE("gnorm dim");
    expect(gdn_gated_rmsnorm_fwd(&g, P(G), P(2 * G), (const float*)P(3 * G), P(4 * G), nullptr), GDN_ERR_UNSUPPORTED,
           "gnorm dim");
    gdn_conv_problem c;
    std::memset(&c, 0, sizeof(c));
    c.batch = 1;
    c.seqlen = 10;
    c.channels = 6;
    c.kernel_size = 4;
    c.dtype = GDN_BF16;
    CASE("conv channels");
    expect(gdn_causal_conv1d_fwd(&c, P(G), (const float*)P(2 * G), nullptr, P(3 * G), nullptr), GDN_ERR_UNSUPPORTED,
           "conv channels");
  }
  std::printf("ok %d\n", n_checked);
  return 0;
}

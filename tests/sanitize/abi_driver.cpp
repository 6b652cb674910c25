// Host-only exercise of the C ABI (fa_api.hip) linked with the stand-in launchers of
// abi_stubs.cpp, built with AddressSanitizer and UndefinedBehaviorSanitizer. Every
// entry point is called with valid and invalid arguments; the placeholder "device"
// buffers are host allocations the library never dereferences. Checks: the returned
// status, that failed validation enqueues nothing, and that the arguments handed to
// the launchers stay inside the buffers the caller passed (workspace split, decoding
// split, row-softmax launch chunks). Prints "all checks passed" and exits 0 on
// success. Test infrastructure only.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "abi_stubs.h"
#include "fa.h"

namespace {

int failures = 0;

#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      ++failures;                                                        \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
    }                                                                    \
  } while (0)

// A 256-byte aligned host buffer standing in for a device allocation.
struct Buf {
  std::vector<unsigned char> mem;
  unsigned char* p;
  size_t n;
  explicit Buf(size_t bytes) : mem(bytes + 256), n(bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(mem.data());
    p = mem.data() + ((256 - (a & 255)) & 255);
  }
  unsigned char* at(size_t off) { return p + off; }
};

bool inside(const void* lo, size_t bytes, const void* base, size_t base_bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(lo), b = reinterpret_cast<uintptr_t>(base);
  return a >= b && a + bytes <= b + base_bytes;
}

// Every error return must leave the launch log empty.
void expect_status(int got, int want, int line) {
  if (got != want) {
    ++failures;
    fprintf(stderr, "line %d: status %d (%s), expected %d\n", line, got, fa_strerror(got), want);
  }
  if (want != FA_OK && stub::calls.total() != 0) {
    ++failures;
    fprintf(stderr, "line %d: a failed call enqueued %zu launches\n", line, stub::calls.total());
  }
  stub::calls.clear();
}
#define EXPECT(call, want)    \
  do {                        \
    stub::calls.clear();      \
    const int rc_ = (call);   \
    expect_status(rc_, want, __LINE__); \
  } while (0)

void forward_checks() {
  const int B = 2, H = 3, N = 200, d = 64;
  const size_t tb = (size_t)B * H * N * d * 2;
  Buf q(tb), k(tb), v(tb), o(tb), lse((size_t)B * H * N * 4);
  const float sc = 0.125f;

  stub::calls.clear();
  CHECK(fa_fwd(q.p, k.p, v.p, o.p, (float*)lse.p, B, H, N, d, sc, nullptr, nullptr) == FA_OK);
  CHECK(stub::calls.fwd.size() == 1);
  if (stub::calls.fwd.size() == 1) {
    const fa::FwdArgs& a = stub::calls.fwd[0];
    CHECK(a.BH == B * H && a.N == N && a.d == d && a.scale == sc);
    CHECK(!a.mask.causal && a.mask.blocks == nullptr && a.mask.nb == 2);
    CHECK(a.q == q.p && a.o == o.p && a.lse == (float*)lse.p);
  }

  Buf grid(4);
  fa_mask_t m{FA_MASK_CAUSAL | FA_MASK_BLOCK, 128, grid.p, 0};
  stub::calls.clear();
  CHECK(fa_fwd(q.p, k.p, v.p, o.p, (float*)lse.p, B, H, N, d, sc, &m, nullptr) == FA_OK);
  CHECK(stub::calls.fwd.size() == 1 && stub::calls.fwd[0].mask.causal &&
        stub::calls.fwd[0].mask.blocks == grid.p);

  // zero extents: no launch
  EXPECT(fa_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 0, H, N, d, sc, nullptr, nullptr),
         FA_OK);
  CHECK(stub::calls.total() == 0);
  EXPECT(fa_fwd(q.p, k.p, v.p, o.p, (float*)lse.p, B, H, 0, d, sc, nullptr, nullptr), FA_OK);

  // validation failures
  EXPECT(fa_fwd(nullptr, k.p, v.p, o.p, (float*)lse.p, B, H, N, d, sc, nullptr, nullptr),
         FA_ERR_NULL);
  EXPECT(fa_fwd(q.p, k.p, v.p, o.p, nullptr, B, H, N, d, sc, nullptr, nullptr), FA_ERR_NULL);
  EXPECT(fa_fwd(q.p + 8, k.p, v.p, o.p, (float*)lse.p, B, H, N, d, sc, nullptr, nullptr),
         FA_ERR_ALIGN);
  EXPECT(fa_fwd(q.p, k.p, v.p, o.p, (float*)(lse.p + 2), B, H, N, d, sc, nullptr, nullptr),
         FA_ERR_ALIGN);
  for (int bad_d : {0, 32, 96, 256, -64})
    EXPECT(fa_fwd(q.p, k.p, v.p, o.p, (float*)lse.p, B, H, N, bad_d, sc, nullptr, nullptr),
           FA_ERR_SHAPE);
  EXPECT(fa_fwd(q.p, k.p, v.p, o.p, (float*)lse.p, -1, H, N, d, sc, nullptr, nullptr),
         FA_ERR_SHAPE);
  for (float bad : {0.f, -1.f, INFINITY, NAN})
    EXPECT(fa_fwd(q.p, k.p, v.p, o.p, (float*)lse.p, B, H, N, d, bad, nullptr, nullptr),
           FA_ERR_SCALE);
  fa_mask_t bad_kind{4, 128, nullptr, 0}, bad_block{FA_MASK_BLOCK, 64, grid.p, 0},
      no_grid{FA_MASK_BLOCK, 128, nullptr, 0}, neg_stride{FA_MASK_BLOCK, 128, grid.p, -1};
  for (const fa_mask_t* bm : {&bad_kind, &bad_block, &no_grid, &neg_stride})
    EXPECT(fa_fwd(q.p, k.p, v.p, o.p, (float*)lse.p, B, H, N, d, sc, bm, nullptr), FA_ERR_MASK);
  // a block mask needs ceil(N / 128) <= 16384
  EXPECT(fa_fwd(q.p, k.p, v.p, o.p, (float*)lse.p, 1, 1, 16384 * 128 + 1, d, sc, &m, nullptr),
         FA_ERR_MASK);
  // aliasing
  EXPECT(fa_fwd(q.p, k.p, v.p, q.p, (float*)lse.p, B, H, N, d, sc, nullptr, nullptr),
         FA_ERR_ALIAS);
  EXPECT(fa_fwd(q.p, k.p, v.p, o.p, (float*)(k.p + 64), B, H, N, d, sc, nullptr, nullptr),
         FA_ERR_ALIAS);
  EXPECT(fa_fwd(q.p, k.p, v.p, o.p, (float*)(o.p + 16), B, H, N, d, sc, nullptr, nullptr),
         FA_ERR_ALIAS);

  // sizes at and past the limits: no overflow in the checks
  EXPECT(fa_fwd(q.p, k.p, v.p, o.p, (float*)lse.p, 65536, 32768, 1, d, sc, nullptr, nullptr),
         FA_ERR_SHAPE);   // B*H > 2^31 - 1
  EXPECT(fa_fwd(q.p, k.p, v.p, o.p, (float*)lse.p, 46340, 46340, 0x7fffffff, 128, sc, nullptr,
                nullptr),
         FA_ERR_SHAPE);   // B*H*N*d far past 2^63
  EXPECT(fa_fwd(q.p, k.p, v.p, o.p, (float*)lse.p, 1, 1, 0x7fffffff, 128, sc, nullptr, nullptr),
         FA_ERR_SHAPE);   // N past 2^31 - 1025
  EXPECT(fa_fwd(q.p, k.p, v.p, o.p, (float*)lse.p, 1, 1, 0x7fffffff - 1024, 128, sc, nullptr,
                nullptr),
         FA_ERR_SHAPE);   // under 2^40 elements, but a launch would need 2^33 work-items
  EXPECT(fa_fwd(q.p, k.p, v.p, o.p, (float*)lse.p, 1, 1, (1 << 30) - 255, 128, sc, nullptr,
                nullptr),
         FA_ERR_SHAPE);   // 4 * 2^30 work-items: one past the limit
  EXPECT(fa_fwd(q.p, k.p, v.p, o.p, (float*)lse.p, 1, 1, (1 << 30) - 256, 128, sc, nullptr,
                nullptr),
         FA_ERR_ALIAS);   // the largest legal N for one head, but then these buffers overlap
}

void backward_checks() {
  const int B = 1, H = 2, N = 333, d = 128;
  const int Np = 384;
  const size_t tb = (size_t)B * H * N * d * 2;
  Buf q(tb), k(tb), v(tb), o(tb), dout(tb), dq(tb), dk(tb), dv(tb), lse((size_t)B * H * N * 4);
  size_t wsb = 0;
  CHECK(fa_bwd_workspace_size(B, H, N, d, &wsb) == FA_OK);
  CHECK(wsb == 2 * (((size_t)B * H * Np * 4 + 255) / 256 * 256));
  CHECK(fa_bwd_workspace_size(B, H, N, d, nullptr) == FA_ERR_NULL);
  CHECK(fa_bwd_workspace_size(B, H, N, 48, &wsb) == FA_ERR_SHAPE);
  CHECK(fa_bwd_workspace_size(B, H, N, d, &wsb) == FA_OK);
  Buf ws(wsb);
  const float sc = 0.088f;

  stub::calls.clear();
  CHECK(fa_bwd(q.p, k.p, v.p, o.p, dout.p, (float*)lse.p, dq.p, dk.p, dv.p, B, H, N, d, sc,
               nullptr, ws.p, wsb, nullptr) == FA_OK);
  CHECK(stub::calls.pre.size() == 1 && stub::calls.dkdv.size() == 1 &&
        stub::calls.dq.size() == 1);
  for (const auto* log : {&stub::calls.pre, &stub::calls.dkdv, &stub::calls.dq}) {
    if (log->size() != 1) continue;
    const fa::BwdArgs& a = (*log)[0];
    CHECK(a.Np == Np && a.BH == B * H && a.N == N && a.d == d);
    CHECK(inside(a.dvec, (size_t)a.BH * a.Np * 4, ws.p, wsb));
    CHECK(inside(a.l2, (size_t)a.BH * a.Np * 4, ws.p, wsb));
    CHECK(reinterpret_cast<uintptr_t>(a.l2) % 256 == 0);
    CHECK((const unsigned char*)a.dvec + (size_t)a.BH * a.Np * 4 <= (const unsigned char*)a.l2);
  }
  CHECK(stub::calls.dkdv.size() == 1 && stub::calls.dkdv[0].dk == dk.p &&
        stub::calls.dkdv[0].dv == dv.p);
  CHECK(stub::calls.dq.size() == 1 && stub::calls.dq[0].dq == dq.p);

  EXPECT(fa_bwd(q.p, k.p, v.p, o.p, dout.p, (float*)lse.p, dq.p, dk.p, dv.p, B, H, N, d, sc,
                nullptr, ws.p, wsb - 1, nullptr),
         FA_ERR_WORKSPACE);
  EXPECT(fa_bwd(q.p, k.p, v.p, o.p, dout.p, (float*)lse.p, dq.p, dk.p, dv.p, B, H, N, d, sc,
                nullptr, nullptr, wsb, nullptr),
         FA_ERR_WORKSPACE);
  EXPECT(fa_bwd(q.p, k.p, v.p, o.p, dout.p, (float*)lse.p, dq.p, dk.p, dv.p, B, H, N, d, sc,
                nullptr, ws.p + 4, wsb, nullptr),
         FA_ERR_ALIGN);
  EXPECT(fa_bwd(q.p, k.p, v.p, o.p, dout.p, (float*)lse.p, dq.p, dk.p, dq.p, B, H, N, d, sc,
                nullptr, ws.p, wsb, nullptr),
         FA_ERR_ALIAS);
  EXPECT(fa_bwd(q.p, k.p, v.p, o.p, dout.p, (float*)lse.p, dq.p, dk.p, dv.p, B, H, N, d, sc,
                nullptr, dq.p, wsb, nullptr),
         FA_ERR_ALIAS);
  EXPECT(fa_bwd(q.p, k.p, v.p, o.p, dout.p, nullptr, dq.p, dk.p, dv.p, B, H, N, d, sc, nullptr,
                ws.p, wsb, nullptr),
         FA_ERR_NULL);
  // the stages one by one
  EXPECT(fa_bwd_preprocess(o.p, dout.p, (float*)lse.p, B, H, N, d, ws.p, wsb, nullptr), FA_OK);
  EXPECT(fa_bwd_preprocess(o.p, dout.p, (float*)lse.p, B, H, N, d, o.p, wsb, nullptr),
         FA_ERR_ALIAS);
  EXPECT(fa_bwd_dkdv(q.p, k.p, v.p, dout.p, dk.p, dv.p, B, H, N, d, sc, nullptr, ws.p, wsb,
                     nullptr),
         FA_OK);
  EXPECT(fa_bwd_dkdv(q.p, k.p, v.p, dout.p, dk.p, k.p, B, H, N, d, sc, nullptr, ws.p, wsb,
                     nullptr),
         FA_ERR_ALIAS);
  EXPECT(fa_bwd_dq(q.p, k.p, v.p, dout.p, dq.p, B, H, N, d, sc, nullptr, ws.p, wsb, nullptr),
         FA_OK);
  EXPECT(fa_bwd_dq(q.p, k.p, v.p, dout.p, dq.p, B, H, N, d, -sc, nullptr, ws.p, wsb, nullptr),
         FA_ERR_SCALE);
  EXPECT(fa_bwd_workspace_size(46340, 46340, 0x7fffffff, 128, &wsb), FA_ERR_SHAPE);
}

void decode_checks() {
  const int B = 2, H = 4, Nq = 16, Nk = 5000, d = 128;
  Buf q((size_t)B * H * Nq * d * 2), o((size_t)B * H * Nq * d * 2),
      lse((size_t)B * H * Nq * 4), k((size_t)B * H * Nk * d * 2), v((size_t)B * H * Nk * d * 2);
  size_t wsb = 0;
  CHECK(fa_decode_workspace_size(B, H, Nq, Nk, d, &wsb) == FA_OK);
  Buf ws(wsb);
  stub::calls.clear();
  CHECK(fa_decode(q.p, k.p, v.p, o.p, (float*)lse.p, B, H, Nq, Nk, d, 0.088f, 1, ws.p, wsb,
                  nullptr) == FA_OK);
  CHECK(stub::calls.decode.size() == 1);
  if (stub::calls.decode.size() == 1) {
    const fa::DecodeArgs& a = stub::calls.decode[0];
    CHECK(a.chunk % 32 == 0 && a.nsplit >= 1);
    CHECK((int64_t)a.nsplit * a.chunk >= Nk && (int64_t)(a.nsplit - 1) * a.chunk < Nk);
    CHECK(inside(a.part_o, (size_t)a.BH * a.nsplit * Nq * d * 4, ws.p, wsb));
    CHECK(inside(a.part_ml, (size_t)a.BH * a.nsplit * Nq * 2 * 4, ws.p, wsb));
    CHECK(a.causal);
  }
  EXPECT(fa_decode(q.p, k.p, v.p, o.p, (float*)lse.p, B, H, 33, Nk, d, 0.088f, 1, ws.p, wsb,
                   nullptr),
         FA_ERR_SHAPE);
  EXPECT(fa_decode(q.p, k.p, v.p, o.p, (float*)lse.p, B, H, Nq, Nk, d, 0.088f, 2, ws.p, wsb,
                   nullptr),
         FA_ERR_MASK);
  EXPECT(fa_decode(q.p, k.p, v.p, o.p, (float*)lse.p, B, H, Nq, Nk, d, 0.088f, 0, ws.p, wsb - 4,
                   nullptr),
         FA_ERR_WORKSPACE);
  EXPECT(fa_decode(q.p, k.p, v.p, k.p, (float*)lse.p, B, H, Nq, Nk, d, 0.088f, 0, ws.p, wsb,
                   nullptr),
         FA_ERR_ALIAS);
  EXPECT(fa_decode_workspace_size(46340, 46340, 32, 0x7fffffff, 128, &wsb), FA_ERR_SHAPE);
  // every split of a range of cache lengths covers the keys exactly
  for (int nk : {1, 31, 32, 33, 255, 256, 257, 4096, 100000, 1 << 20}) {
    for (int bh : {1, 7, 64, 2048, 5000}) {
      int ns = 0, ch = 0;
      fa::decode_split(bh, nk, &ns, &ch);
      CHECK(ch % 32 == 0 && ns >= 1 && (int64_t)ns * ch >= nk && (int64_t)(ns - 1) * ch < nk);
    }
  }
}

void kv_outer_checks() {
  const int B = 1, H = 2, N = 130, d = 64;
  const size_t tb = (size_t)B * H * N * d * 2;
  Buf q(tb), k(tb), v(tb), o(tb), lse((size_t)B * H * N * 4);
  size_t wsb = 0;
  CHECK(fa_fwd_kv_outer_workspace_size(B, H, N, d, &wsb) == FA_OK);
  Buf ws(wsb);
  stub::calls.clear();
  CHECK(fa_fwd_kv_outer(q.p, k.p, v.p, o.p, (float*)lse.p, B, H, N, d, 0.125f, 1, ws.p, wsb,
                        nullptr) == FA_OK);
  CHECK(stub::calls.kv_outer.size() == 1);
  if (stub::calls.kv_outer.size() == 1) {
    const fa::KvOuterArgs& a = stub::calls.kv_outer[0];
    CHECK(inside(a.ow, (size_t)a.BH * N * d * 4, ws.p, wsb));
    CHECK(inside(a.mw, (size_t)a.BH * N * 4, ws.p, wsb));
    CHECK(inside(a.lw, (size_t)a.BH * N * 4, ws.p, wsb));
  }
  EXPECT(fa_fwd_kv_outer(q.p, k.p, v.p, o.p, (float*)lse.p, B, H, N, d, 0.125f, 0, ws.p, wsb / 2,
                         nullptr),
         FA_ERR_WORKSPACE);
  EXPECT(fa_fwd_kv_outer(q.p, k.p, v.p, o.p, (float*)lse.p, B, H, N, d, 0.125f, 0, q.p, wsb,
                         nullptr),
         FA_ERR_ALIAS);
}

void softmax_checks() {
  // Placeholder device addresses 16 TiB apart (never dereferenced), so that the
  // ranges of large matrices do not overlap.
  struct Fake {
    unsigned char* p;
  } x{reinterpret_cast<unsigned char*>(uintptr_t(1) << 44)},
      y{reinterpret_cast<unsigned char*>(uintptr_t(2) << 44)};
  // 2^27 rows of 4 columns (2 GiB): split into launches of at most 2^21 rows that
  // cover every row once, in order
  const int64_t rows = int64_t(1) << 27, cols = 4;
  stub::calls.clear();
  CHECK(fa_softmax_rows((const float*)x.p, (float*)y.p, rows, cols, nullptr) == FA_OK);
  int64_t next = 0;
  bool ok = true;
  for (const fa::SoftmaxArgs& a : stub::calls.softmax) {
    ok = ok && a.rows >= 1 && a.rows <= fa::kSoftmaxRowsPerLaunch && a.cols == cols;
    ok = ok && a.x == (const float*)x.p + next * cols && a.y == (float*)y.p + next * cols;
    next += a.rows;
  }
  CHECK(ok && next == rows && stub::calls.softmax.size() == 64);
  // rows not a multiple of the launch size
  stub::calls.clear();
  CHECK(fa_softmax_rows((const float*)x.p, (float*)y.p, 5000001, 3, nullptr) == FA_OK);
  CHECK(stub::calls.softmax.size() == 3 && stub::calls.softmax.back().rows == 5000001 - 2 * 2097152);
  EXPECT(fa_softmax_rows((const float*)x.p, (float*)x.p, 7, 5, nullptr), FA_OK);   // in place
  EXPECT(fa_softmax_rows((const float*)x.p, (float*)(x.p + 4), 7, 5, nullptr), FA_ERR_ALIAS);
  EXPECT(fa_softmax_rows((const float*)x.p, (float*)y.p, 0x7fffffff, 0x7fffffff, nullptr),
         FA_ERR_SHAPE);
  EXPECT(fa_softmax_rows((const float*)x.p, (float*)y.p, int64_t(1) << 31, 1, nullptr),
         FA_ERR_SHAPE);
  EXPECT(fa_softmax_rows((const float*)x.p, (float*)y.p, -1, 4, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_softmax_rows(nullptr, (float*)y.p, 2, 4, nullptr), FA_ERR_NULL);
  EXPECT(fa_softmax_rows((const float*)(x.p + 2), (float*)y.p, 2, 4, nullptr), FA_ERR_ALIGN);
  EXPECT(fa_softmax_rows(nullptr, nullptr, 0, 4, nullptr), FA_OK);
}

void strerror_checks() {
  for (int s = 1; s >= -9; --s) CHECK(fa_strerror(s) != nullptr);
  CHECK(fa_strerror(12345) != nullptr);
}

}  // namespace

int main() {
  forward_checks();
  backward_checks();
  decode_checks();
  kv_outer_checks();
  softmax_checks();
  strerror_checks();
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("all checks passed\n");
  return 0;
}

// C ABI of the attention library (declared in include/fa.h): host-side argument
// checks, workspace layout, and kernel dispatch on the caller's stream.
#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 40;
// A dispatch counts its work-items in 32 bits: every launch stays below 2^32.
constexpr int64_t kMaxWorkItems = (int64_t(1) << 32) - 1;
// Sequence lengths stay this far below 2^31 so that rounding N up to any tile
// (at most 256 rows) stays inside int.
constexpr int kMaxSeq = INT32_MAX - 1024;

struct Shape {
  int B, H, N, d;
  int64_t bh() const { return (int64_t)B * H; }
  int64_t elems() const { return bh() * N * d; }
  bool empty() const { return B == 0 || H == 0 || N == 0; }
};

int check_shape(const Shape& s) {
  if (s.B < 0 || s.H < 0 || s.N < 0 || s.N > kMaxSeq) return FA_ERR_SHAPE;
  if (s.d != 64 && s.d != 128) return FA_ERR_SHAPE;
  if (s.bh() > INT32_MAX) return FA_ERR_SHAPE;
  // B*H*N*d can exceed 2^63 before the limit check (B*H and N up to 2^31 - 1 each)
  if ((unsigned __int128)s.bh() * (unsigned)s.N * (unsigned)s.d >= (unsigned __int128)kMaxElems)
    return FA_ERR_SHAPE;
  // The widest launches (the backward preprocess, dK/dV at d = 128) run four
  // work-items per row of every head, rows rounded up to the 256-row blocks of
  // the forward; the other attention launches run at most two per row, and the
  // K/V-outer forward 256 per head. B*H*N < 2^34 here, so this cannot overflow.
  if (4 * s.bh() * (((int64_t)s.N + 255) / 256 * 256) > kMaxWorkItems) return FA_ERR_SHAPE;
  return FA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int check_scale(float scale) {
  return (isfinite(scale) && scale > 0.f) ? FA_OK : FA_ERR_SCALE;
}

// Mask check. On success fills the kernel-side description.
int check_mask(const fa_mask_t* m, const Shape& s, fa::MaskArgs* out) {
  out->causal = false;
  out->blocks = nullptr;
  out->bh_stride = 0;
  out->nb = (s.N + 127) / 128;
  if (m == nullptr) return FA_OK;
  if (m->kind & ~(FA_MASK_CAUSAL | FA_MASK_BLOCK)) return FA_ERR_MASK;
  out->causal = (m->kind & FA_MASK_CAUSAL) != 0;
  if (m->kind & FA_MASK_BLOCK) {
    if (m->block != 128 || m->blocks == nullptr || m->bh_stride < 0) return FA_ERR_MASK;
    if (out->nb > fa::kMaxMaskBlocks) return FA_ERR_MASK;
    out->blocks = m->blocks;
    out->bh_stride = m->bh_stride;
  }
  return FA_OK;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range range(const void* p, int64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + (uintptr_t)bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool any_overlap(const Range* outs, int n_out, const Range* ins, int n_in) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlap(outs[i], ins[j])) return true;
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(outs[i], outs[j])) return true;
  }
  return false;
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

int padded_rows(int N) {
  const int r = fa::kBwdRowPad;
  return (N + r - 1) / r * r;
}

// Workspace layout, each part starting on a 256-byte boundary
// (Np = N rounded up to the row padding):
//   D_i             float32 [BH][Np]
//   LSE_i log2(e)   float32 [BH][Np]
size_t ws_part(const Shape& s) {
  return round256((size_t)s.bh() * padded_rows(s.N) * sizeof(float));
}
size_t workspace_bytes(const Shape& s) { return 2 * ws_part(s); }

int check_workspace(const void* ws, size_t bytes, const Shape& s) {
  if (ws == nullptr) return FA_ERR_WORKSPACE;
  if (!aligned16(ws)) return FA_ERR_ALIGN;
  if (bytes < workspace_bytes(s)) return FA_ERR_WORKSPACE;
  return FA_OK;
}

void split_workspace(void* ws, const Shape& s, fa::BwdArgs* a) {
  char* base = static_cast<char*>(ws);
  a->dvec = reinterpret_cast<float*>(base);
  a->l2 = reinterpret_cast<float*>(base + ws_part(s));
  a->Np = padded_rows(s.N);
}

int launched(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

#define FA_TRY(expr)          \
  do {                        \
    const int rc_ = (expr);   \
    if (rc_ != FA_OK) return rc_; \
  } while (0)

// Checks shared by the two gradient stages (dK/dV and dQ); outs are the stage's
// bf16 outputs (n_out of them). On success fills *a; *empty reports a zero extent.
int check_grad_stage(const void* q, const void* k, const void* v, const void* dout,
                     void* const* outs, int n_out, int B, int H, int N, int d,
                     float scale, const fa_mask_t* mask, void* workspace, size_t ws_bytes,
                     fa::BwdArgs* a, bool* empty) {
  const Shape s{B, H, N, d};
  FA_TRY(check_shape(s));
  FA_TRY(check_scale(scale));
  fa::MaskArgs m;
  FA_TRY(check_mask(mask, s, &m));
  *empty = s.empty();
  if (*empty) return FA_OK;
  if (!q || !k || !v || !dout) return FA_ERR_NULL;
  for (int i = 0; i < n_out; ++i)
    if (!outs[i]) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout)) return FA_ERR_ALIGN;
  for (int i = 0; i < n_out; ++i)
    if (!aligned16(outs[i])) return FA_ERR_ALIGN;
  FA_TRY(check_workspace(workspace, ws_bytes, s));
  const int64_t tb = s.elems() * 2;
  const Range ins[5] = {range(q, tb), range(k, tb), range(v, tb), range(dout, tb),
                        range(workspace, (int64_t)workspace_bytes(s))};
  Range out_r[2];
  for (int i = 0; i < n_out; ++i) out_r[i] = range(outs[i], tb);
  if (any_overlap(out_r, n_out, ins, 5)) return FA_ERR_ALIAS;
  *a = fa::BwdArgs{};
  a->q = q;
  a->k = k;
  a->v = v;
  a->dout = dout;
  a->BH = (int)s.bh();
  a->N = N;
  a->d = d;
  a->scale = scale;
  a->mask = m;
  split_workspace(workspace, s, a);
  return FA_OK;
}

// Decoding: shape checks and the workspace of the key split.
int decode_shape(int B, int H, int Nq, int Nk, int d) {
  if (B < 0 || H < 0 || Nq < 0 || Nq > 32 || Nk < 0 || Nk > kMaxSeq) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_SHAPE;
  if ((int64_t)B * H > INT32_MAX) return FA_ERR_SHAPE;
  if ((unsigned __int128)((int64_t)B * H) * (uint64_t)((int64_t)Nk + Nq) * (unsigned)d >=
      (unsigned __int128)kMaxElems)
    return FA_ERR_SHAPE;
  // Work-items of the two launches: the merge runs d per query row of every
  // head, the key split 64 per chunk, with at most B*H + 1024 chunks in all.
  const int64_t bh = (int64_t)B * H;
  if (bh * Nq * d > kMaxWorkItems || 64 * (bh + 1024) > kMaxWorkItems) return FA_ERR_SHAPE;
  return FA_OK;
}
size_t decode_ws_o(int64_t BH, int Nq, int Nk, int d) {
  int ns = 1, ch = 32;
  fa::decode_split((int)BH, Nk, &ns, &ch);
  return round256((size_t)BH * ns * Nq * d * sizeof(float));
}
size_t decode_ws_ml(int64_t BH, int Nq, int Nk) {
  int ns = 1, ch = 32;
  fa::decode_split((int)BH, Nk, &ns, &ch);
  return round256((size_t)BH * ns * Nq * 2 * sizeof(float));
}

// Workspace of the K/V-outer forward: O float32 [BH][N][d], then m and l [BH][N].
size_t kvo_ws_o(const Shape& s) { return round256((size_t)s.bh() * s.N * s.d * sizeof(float)); }
size_t kvo_ws_v(const Shape& s) { return round256((size_t)s.bh() * s.N * sizeof(float)); }
size_t kvo_workspace_bytes(const Shape& s) { return kvo_ws_o(s) + 2 * kvo_ws_v(s); }

}  // namespace

extern "C" {

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE:
      return "unsupported shape: need B, H, N >= 0, d in {64, 128}, B*H*N*d < 2^40, and at most "
             "2^32 - 1 work-items per launch";
    case FA_ERR_MASK: return "invalid mask: unknown kind, block != 128, or missing block grid";
    case FA_ERR_ALIGN: return "a data pointer is not 16-byte aligned";
    case FA_ERR_WORKSPACE: return "backward workspace missing or smaller than fa_bwd_workspace_size()";
    case FA_ERR_HIP: return "HIP runtime error at kernel launch";
    case FA_ERR_SCALE: return "scale must be finite and > 0";
    case FA_ERR_ALIAS: return "an output buffer overlaps another argument buffer";
    case FA_ERR_SCRATCH:
      return "too large for fa_bwd_noalloc's fixed 16 MiB scratch (B*H*ceil(N/128)*128 > 2^21)";
    default: return "unknown status";
  }
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, float scale, const fa_mask_t* mask, void* stream) {
  const Shape s{B, H, N, d};
  FA_TRY(check_shape(s));
  FA_TRY(check_scale(scale));
  fa::MaskArgs m;
  FA_TRY(check_mask(mask, s, &m));
  if (s.empty()) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
    return FA_ERR_ALIGN;
  const int64_t tb = s.elems() * 2;
  const Range ins[3] = {range(q, tb), range(k, tb), range(v, tb)};
  const Range outs[2] = {range(o, tb), range(lse, s.bh() * N * 4)};
  if (any_overlap(outs, 2, ins, 3)) return FA_ERR_ALIAS;
  fa::FwdArgs a{q, k, v, o, lse, (int)s.bh(), N, d, scale, m};
  return launched(fa::launch_fwd(a, static_cast<hipStream_t>(stream)));
}

int fa_bwd_workspace_size(int B, int H, int N, int d, size_t* bytes) {
  if (bytes == nullptr) return FA_ERR_NULL;
  const Shape s{B, H, N, d};
  FA_TRY(check_shape(s));
  *bytes = workspace_bytes(s);
  return FA_OK;
}

int fa_bwd_preprocess(const void* o, const void* dout, const float* lse, int B, int H, int N,
                      int d, void* workspace, size_t ws_bytes, void* stream) {
  const Shape s{B, H, N, d};
  FA_TRY(check_shape(s));
  if (s.empty()) return FA_OK;
  if (!o || !dout || !lse) return FA_ERR_NULL;
  if (!aligned16(o) || !aligned16(dout) || !aligned4(lse)) return FA_ERR_ALIGN;
  FA_TRY(check_workspace(workspace, ws_bytes, s));
  const int64_t tb = s.elems() * 2;
  const Range ins[3] = {range(o, tb), range(dout, tb), range(lse, s.bh() * N * 4)};
  const Range outs[1] = {range(workspace, (int64_t)workspace_bytes(s))};
  if (any_overlap(outs, 1, ins, 3)) return FA_ERR_ALIAS;
  fa::BwdArgs a{};
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.BH = (int)s.bh();
  a.N = N;
  a.d = d;
  split_workspace(workspace, s, &a);
  return launched(fa::launch_bwd_preprocess(a, static_cast<hipStream_t>(stream)));
}

int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv, int B, int H, int N, int d, float scale,
                const fa_mask_t* mask, void* workspace, size_t ws_bytes, void* stream) {
  void* const outs[2] = {dk, dv};
  fa::BwdArgs a;
  bool empty = false;
  FA_TRY(check_grad_stage(q, k, v, dout, outs, 2, B, H, N, d, scale, mask, workspace,
                          ws_bytes, &a, &empty));
  if (empty) return FA_OK;
  a.dk = dk;
  a.dv = dv;
  return launched(fa::launch_bwd_dkdv(a, static_cast<hipStream_t>(stream)));
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout, void* dq, int B, int H, int N, int d, float scale, const fa_mask_t* mask,
              void* workspace, size_t ws_bytes, void* stream) {
  void* const outs[1] = {dq};
  fa::BwdArgs a;
  bool empty = false;
  FA_TRY(check_grad_stage(q, k, v, dout, outs, 1, B, H, N, d, scale, mask, workspace,
                          ws_bytes, &a, &empty));
  if (empty) return FA_OK;
  a.dq = dq;
  return launched(fa::launch_bwd_dq(a, static_cast<hipStream_t>(stream)));
}

int fa_decode_workspace_size(int B, int H, int Nq, int Nk, int d, size_t* bytes) {
  if (bytes == nullptr) return FA_ERR_NULL;
  FA_TRY(decode_shape(B, H, Nq, Nk, d));
  const int64_t BH = (int64_t)B * H;
  *bytes = decode_ws_o(BH, Nq, Nk, d) + decode_ws_ml(BH, Nq, Nk);
  return FA_OK;
}

int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
              int Nq, int Nk, int d, float scale, int causal, void* workspace, size_t ws_bytes,
              void* stream) {
  FA_TRY(decode_shape(B, H, Nq, Nk, d));
  FA_TRY(check_scale(scale));
  if (causal != 0 && causal != 1) return FA_ERR_MASK;
  const int64_t BH = (int64_t)B * H;
  if (BH == 0 || Nq == 0) return FA_OK;
  if (!q || !o || !lse || (Nk > 0 && (!k || !v))) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(o) || !aligned4(lse) || !aligned16(k) || !aligned16(v))
    return FA_ERR_ALIGN;
  const size_t need = decode_ws_o(BH, Nq, Nk, d) + decode_ws_ml(BH, Nq, Nk);
  if (workspace == nullptr || ws_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  const int64_t qb = BH * Nq * d * 2, kb = BH * (int64_t)Nk * d * 2;
  const Range ins[3] = {range(q, qb), range(k, kb), range(v, kb)};
  const Range outs[3] = {range(o, qb), range(lse, BH * Nq * 4), range(workspace, (int64_t)need)};
  if (any_overlap(outs, 3, ins, 3)) return FA_ERR_ALIAS;
  fa::DecodeArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.BH = (int)BH;
  a.Nq = Nq;
  a.Nk = Nk;
  a.d = d;
  a.scale = scale;
  a.causal = causal != 0;
  fa::decode_split(a.BH, Nk, &a.nsplit, &a.chunk);
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + decode_ws_o(BH, Nq, Nk, d));
  return launched(fa::launch_decode(a, static_cast<hipStream_t>(stream)));
}

int fa_fwd_kv_outer_workspace_size(int B, int H, int N, int d, size_t* bytes) {
  if (bytes == nullptr) return FA_ERR_NULL;
  const Shape s{B, H, N, d};
  FA_TRY(check_shape(s));
  *bytes = kvo_workspace_bytes(s);
  return FA_OK;
}

int fa_fwd_kv_outer(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                    int H, int N, int d, float scale, int causal, void* workspace,
                    size_t ws_bytes, void* stream) {
  const Shape s{B, H, N, d};
  FA_TRY(check_shape(s));
  FA_TRY(check_scale(scale));
  if (causal != 0 && causal != 1) return FA_ERR_MASK;
  if (s.empty()) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
    return FA_ERR_ALIGN;
  if (workspace == nullptr || ws_bytes < kvo_workspace_bytes(s)) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  const int64_t tb = s.elems() * 2;
  const Range ins[3] = {range(q, tb), range(k, tb), range(v, tb)};
  const Range outs[3] = {range(o, tb), range(lse, s.bh() * N * 4),
                         range(workspace, (int64_t)kvo_workspace_bytes(s))};
  if (any_overlap(outs, 3, ins, 3)) return FA_ERR_ALIAS;
  fa::KvOuterArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.BH = (int)s.bh();
  a.N = N;
  a.d = d;
  a.scale = scale;
  a.causal = causal != 0;
  char* w = static_cast<char*>(workspace);
  a.ow = reinterpret_cast<float*>(w);
  a.mw = reinterpret_cast<float*>(w + kvo_ws_o(s));
  a.lw = reinterpret_cast<float*>(w + kvo_ws_o(s) + kvo_ws_v(s));
  return launched(fa::launch_fwd_kv_outer(a, static_cast<hipStream_t>(stream)));
}

int fa_softmax_rows(const float* x, float* y, int64_t rows, int64_t cols, void* stream) {
  if (rows < 0 || cols < 0 || rows > 0x7fffffff || cols > 0x7fffffff) return FA_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FA_OK;
  if (rows * cols >= (int64_t(1) << 40)) return FA_ERR_SHAPE;
  if (!x || !y) return FA_ERR_NULL;
  if (!aligned4(x) || !aligned4(y)) return FA_ERR_ALIGN;
  const int64_t bytes = rows * cols * 4;
  // y == x (in place) is allowed; any other overlap is not
  if (x != y) {
    const Range in[1] = {range(x, bytes)};
    const Range out[1] = {range(y, bytes)};
    if (any_overlap(out, 1, in, 1)) return FA_ERR_ALIAS;
  }
  // Launches of at most kSoftmaxRowsPerLaunch rows each, in row order.
  for (int64_t r0 = 0; r0 < rows; r0 += fa::kSoftmaxRowsPerLaunch) {
    const int64_t n = rows - r0 < fa::kSoftmaxRowsPerLaunch ? rows - r0 : fa::kSoftmaxRowsPerLaunch;
    const fa::SoftmaxArgs a{x + r0 * cols, y + r0 * cols, n, cols};
    FA_TRY(launched(fa::launch_softmax_rows(a, static_cast<hipStream_t>(stream))));
  }
  return FA_OK;
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
           float scale, const fa_mask_t* mask, void* workspace, size_t ws_bytes, void* stream) {
  const Shape s{B, H, N, d};
  FA_TRY(check_shape(s));
  FA_TRY(check_scale(scale));
  fa::MaskArgs m;
  FA_TRY(check_mask(mask, s, &m));
  if (s.empty()) return FA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned4(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_ALIGN;
  FA_TRY(check_workspace(workspace, ws_bytes, s));
  const int64_t tb = s.elems() * 2;
  const Range ins[6] = {range(q, tb), range(k, tb), range(v, tb), range(o, tb), range(dout, tb),
                        range(lse, s.bh() * N * 4)};
  const Range outs[4] = {range(dq, tb), range(dk, tb), range(dv, tb),
                         range(workspace, (int64_t)workspace_bytes(s))};
  if (any_overlap(outs, 4, ins, 6)) return FA_ERR_ALIAS;
  FA_TRY(fa_bwd_preprocess(o, dout, lse, B, H, N, d, workspace, ws_bytes, stream));
  FA_TRY(fa_bwd_dkdv(q, k, v, dout, dk, dv, B, H, N, d, scale, mask, workspace, ws_bytes, stream));
  return fa_bwd_dq(q, k, v, dout, dq, B, H, N, d, scale, mask, workspace, ws_bytes, stream);
}

}  // extern "C"

// Kernel launch interface between the C ABI (fa_api.hip) and the kernel files.
// Arguments here are already validated; launchers only pick an instantiation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct MaskArgs {
  bool causal;
  const uint8_t* blocks;  // nullptr = no block mask; else [nb][nb] per (b, h)
  int64_t bh_stride;      // elements between (b, h) grids (0 = shared)
  int nb;                 // ceil(N / 128)
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int BH, N, d;
  float scale;
  MaskArgs mask;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int BH, N, d;
  float scale;
  MaskArgs mask;
  float* dvec;   // workspace: D_i = dO_i . O_i, [BH][Np] (0 past N)
  float* l2;     // workspace: LSE_i log2(e), [BH][Np] (+inf past N and for empty rows)
  int Np;        // N rounded up to kBwdRowPad
};

struct SoftmaxArgs {
  const float* x;
  float* y;
  int64_t rows;   // 1 .. kSoftmaxRowsPerLaunch
  int64_t cols;   // 1 .. 2^31 - 1
};

struct DecodeArgs {
  const void* q;    // [BH][Nq][d]
  const void* k;    // [BH][Nk][d]
  const void* v;
  void* o;          // [BH][Nq][d]
  float* lse;       // [BH][Nq]
  int BH, Nq, Nk, d;
  float scale;
  bool causal;
  float* part_o;    // workspace: [BH][nsplit][Nq][d]
  float* part_ml;   // workspace: [BH][nsplit][Nq][2]
  int nsplit;       // from decode_split
  int chunk;
};

// Key split of the decoding kernels: nsplit chunks of `chunk` keys (a multiple
// of 32) cover Nk. About 1024 chunk waves in all (four per CU: measured faster
// than 2048 to 8192 on every decode shape tried, the merge reading fewer
// partial states), chunks of at least eight 32-key tiles.
inline void decode_split(int BH, int Nk, int* nsplit, int* chunk) {
  const int target = (1024 + BH - 1) / BH;
  const int max_split = Nk > 0 ? (Nk + 255) / 256 : 1;
  int ns = target < max_split ? target : max_split;
  if (ns < 1) ns = 1;
  int ch = Nk > 0 ? (Nk + ns - 1) / ns : 32;
  ch = (ch + 31) / 32 * 32;
  *chunk = ch;
  *nsplit = Nk > 0 ? (Nk + ch - 1) / ch : 1;
}

struct KvOuterArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int BH, N, d;
  float scale;
  bool causal;
  float* ow;   // workspace: O float32 [BH][N][d]
  float* mw;   // workspace: m [BH][N]
  float* lw;   // workspace: l [BH][N]
};

// Row padding of the per-row arrays in the backward workspace.
constexpr int kBwdRowPad = 128;

// Rows of one row-softmax launch: the C ABI splits larger matrices into
// launches of at most this many rows, so that no launch asks for more than
// 2^31 work-items (the streaming kernel runs 1024 threads per row).
constexpr int64_t kSoftmaxRowsPerLaunch = int64_t(1) << 21;

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_preprocess(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream);
hipError_t launch_softmax_rows(const SoftmaxArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_fwd_kv_outer(const KvOuterArgs& a, hipStream_t stream);

}  // namespace fa

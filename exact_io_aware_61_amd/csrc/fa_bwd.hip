// Backward attention for gfx950: dQ, dK, dV with P recomputed from the saved LSE.
//
// Recomputation (lecture summary on FlashAttention v1, part 4.2): no N x N matrix
// is read back; each tile of S and P is rebuilt on chip from Q, K and the row
// logsumexp, the only statistic kept (FlashAttention-2 overview, backward pass).
// Partitioning (same overview): one workgroup per block of key columns of one
// (batch, head); it sweeps the query row blocks, keeps its dK and dV on chip,
// and merges dQ, the only quantity shared between column blocks, by atomic
// addition into a float32 accumulator.
//
// Per key block (4 waves x 32 keys) and query row block (64 rows), per wave:
//   S  = Q K_w^T       MFMA, Q rows read from LDS, K_w^T held in VGPRs. The
//                      accumulator puts one key column in each lane.
//   P  = 2^(S scale log2e - LSE_i log2e)       (masked pairs -> 0)
//   dP = dO V_w^T      MFMA, as S
//   dS = P o (dP - D_i),  D_i = dO_i . O_i (preprocess kernel)
//   dV_w^T += dO^T P   MFMA, P straight from registers as the B operand,
//                      dO^T via the transposing LDS read
//   dK_w^T += Q^T dS   likewise (scale applied once at the end)
//   dS^T -> LDS; then the workgroup computes dQ_rows = dS K for all 128 keys
//   (A = dS via transposing reads of dS^T, B = K via transposing reads) and adds
//   it atomically to the float32 accumulator.
// The formulas are the chain rule through the softmax; the pages only name it.
#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {
namespace {

// ------------------------------------------------------------------------------------------------
// Preprocess: D_i = sum_c dO_ic O_ic (float32), and zero the dQ accumulator rows.

template <int D>
__global__ __launch_bounds__(256) void fa_bwd_pre_kernel(const bf16* __restrict__ o,
                                                         const bf16* __restrict__ dout,
                                                         float* __restrict__ dvec,
                                                         float* __restrict__ dqacc,
                                                         int64_t rows) {
  constexpr int LPR = D / 8;                 // lanes per row, 8 elements each
  constexpr int RPB = 256 / LPR;             // rows per block
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(o + row * D + 8 * part);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(dout + row * D + 8 * part);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)b[e];
    f32x4* z = reinterpret_cast<f32x4*>(dqacc + row * D + 8 * part);
    z[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    z[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) dvec[row] = acc;
}

// ------------------------------------------------------------------------------------------------
// Finish: dq = bf16(scale * dQ accumulator).

__global__ __launch_bounds__(256) void fa_bwd_finish_kernel(const float* __restrict__ dqacc,
                                                            bf16* __restrict__ dq, float scale,
                                                            int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = reinterpret_cast<const f32x4*>(dqacc)[2 * i];
  const f32x4 b = reinterpret_cast<const f32x4*>(dqacc)[2 * i + 1];
  reinterpret_cast<bf16x8*>(dq)[i] = to_bf16x8(a[0] * scale, a[1] * scale, a[2] * scale,
                                               a[3] * scale, b[0] * scale, b[1] * scale,
                                               b[2] * scale, b[3] * scale);
}

// ------------------------------------------------------------------------------------------------
// Main backward kernel.

template <int D>
struct BwdCfg {
  static constexpr int WAVES = 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BN = 32 * WAVES;     // keys per workgroup (128)
  static constexpr int BM = 64;             // query rows per iteration
  static constexpr int STR = D == 128 ? 152 : 72;  // LDS row stride (elements) for K, Q, dO
  static constexpr int SSTR = BM + 8;              // LDS row stride of dS^T (72 = 36 dwords)
  static constexpr int KS = D / 16;
  static constexpr int CT = D / 32;
  static constexpr int IT = BM / 32;        // 32-row sub-tiles per row block
  static constexpr int QCHUNKS = BM * D / 8;
  static constexpr int QCPT = QCHUNKS / THREADS;
  static constexpr int KCHUNKS = BN * D / 8;
  static constexpr int KCPT = KCHUNKS / THREADS;
  static constexpr int DQT = IT * CT / WAVES;  // dQ output tiles per wave
  static_assert(QCHUNKS % THREADS == 0 && KCHUNKS % THREADS == 0, "even split");
  static_assert((IT * CT) % WAVES == 0, "dQ tiles split evenly over waves");
};

struct BwdParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* dout;
  const float* lse;
  const float* dvec;
  float* dqacc;
  bf16* dk;
  bf16* dv;
  int BH;
  int N;
  float sl2;    // scale * log2(e)
  float scale;
  const uint8_t* blocks;
  int64_t blocks_bh_stride;
  int nb;
};

template <int D, bool CAUSAL, bool BLOCK>
__global__ __launch_bounds__(256) void fa_bwd_main_kernel(BwdParams p) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) bf16 Ks[C::BN * C::STR];
  __shared__ __attribute__((aligned(16))) bf16 Qs[C::BM * C::STR];
  __shared__ __attribute__((aligned(16))) bf16 dOs[C::BM * C::STR];
  __shared__ __attribute__((aligned(16))) bf16 dSt[C::BN * C::SSTR];
  __shared__ __attribute__((aligned(16))) float Ls[C::BM];   // LSE * log2e (+inf = no row)
  __shared__ __attribute__((aligned(16))) float Ds[C::BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int g16 = lane >> 4;
  const int i16 = lane & 15;

  const int bh = blockIdx.x % p.BH;
  const int kb = blockIdx.x / p.BH;   // key block; block 0 carries the most rows under causal
  const int N = p.N;
  const int64_t head = (int64_t)bh * N * D;
  const bf16* __restrict__ Qh = p.q + head;
  const bf16* __restrict__ Kh = p.k + head;
  const bf16* __restrict__ Vh = p.v + head;
  const bf16* __restrict__ dOh = p.dout + head;
  const float* __restrict__ Lh = p.lse + (int64_t)bh * N;
  const float* __restrict__ Dh = p.dvec + (int64_t)bh * N;
  float* __restrict__ dQh = p.dqacc + head;

  const int key0 = kb * C::BN;
  const int wkey0 = key0 + 32 * wave;
  const int mykey = wkey0 + l32;   // this lane's key column

  // K block -> LDS (for dQ), K_w and V_w operands -> VGPRs.
#pragma unroll
  for (int c = 0; c < C::KCPT; ++c) {
    const int id = tid + c * C::THREADS;
    const int r = id / (D / 8);
    const int col = (id % (D / 8)) * 8;
    u32x4 x = {0, 0, 0, 0};
    if (key0 + r < N) x = *reinterpret_cast<const u32x4*>(Kh + (int64_t)(key0 + r) * D + col);
    *reinterpret_cast<u32x4*>(Ks + r * C::STR + col) = x;
  }
  bf16x8 kf[C::KS], vf[C::KS];
#pragma unroll
  for (int kk = 0; kk < C::KS; ++kk) {
    if (mykey < N) {
      kf[kk] = *reinterpret_cast<const bf16x8*>(Kh + (int64_t)mykey * D + 16 * kk + 8 * hh);
      vf[kk] = *reinterpret_cast<const bf16x8*>(Vh + (int64_t)mykey * D + 16 * kk + 8 * hh);
    } else {
      kf[kk] = bf16x8{};
      vf[kk] = bf16x8{};
    }
  }

  f32x16 dk[C::CT], dv[C::CT];
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) {
    dk[ct] = f32x16{};
    dv[ct] = f32x16{};
  }

  // Row-block range: under causal, rows before key0 see none of these keys.
  const int n_rb = (N + C::BM - 1) / C::BM;
  const int rb_begin = CAUSAL ? key0 / C::BM : 0;
  auto kept = [&](int rb) -> bool {
    if (!BLOCK) return true;
    return p.blocks[bh * p.blocks_bh_stride + (int64_t)((rb * C::BM) / 128) * p.nb + kb] != 0;
  };

  for (int rb = rb_begin; rb < n_rb; ++rb) {
    if (!kept(rb)) continue;
    const int row0 = rb * C::BM;
    // Q, dO row block -> LDS; LSE (log2 domain) and D -> LDS.
#pragma unroll
    for (int c = 0; c < C::QCPT; ++c) {
      const int id = tid + c * C::THREADS;
      const int r = id / (D / 8);
      const int col = (id % (D / 8)) * 8;
      u32x4 xq = {0, 0, 0, 0}, xo = {0, 0, 0, 0};
      if (row0 + r < N) {
        xq = *reinterpret_cast<const u32x4*>(Qh + (int64_t)(row0 + r) * D + col);
        xo = *reinterpret_cast<const u32x4*>(dOh + (int64_t)(row0 + r) * D + col);
      }
      *reinterpret_cast<u32x4*>(Qs + r * C::STR + col) = xq;
      *reinterpret_cast<u32x4*>(dOs + r * C::STR + col) = xo;
    }
    if (tid < C::BM) {
      const int row = row0 + tid;
      float l2 = INFINITY, dd = 0.f;
      if (row < N) {
        const float lse = Lh[row];
        // A row with no visible key has LSE = -inf and contributes nothing.
        l2 = lse == -INFINITY ? INFINITY : lse * kLog2e;
        dd = Dh[row];
      }
      Ls[tid] = l2;
      Ds[tid] = dd;
    }
    __syncthreads();

    // S and dP for this wave's 32 keys and the 64 rows (two 32-row sub-tiles).
    f32x16 s[C::IT], dp[C::IT];
#pragma unroll
    for (int it = 0; it < C::IT; ++it) {
      s[it] = f32x16{};
      dp[it] = f32x16{};
    }
#pragma unroll
    for (int kk = 0; kk < C::KS; ++kk) {
#pragma unroll
      for (int it = 0; it < C::IT; ++it) {
        const bf16x8 a = lds_b128(Qs + (32 * it + l32) * C::STR + 16 * kk + 8 * hh);
        s[it] = mfma32(a, kf[kk], s[it]);
        const bf16x8 b = lds_b128(dOs + (32 * it + l32) * C::STR + 16 * kk + 8 * hh);
        dp[it] = mfma32(b, vf[kk], dp[it]);
      }
    }
    // s[it][v]: row row0 + 32*it + 8*(v/4) + 4*hh + v%4, key mykey.
    const bool edge = (CAUSAL && row0 < wkey0 + 31) || (key0 + C::BN > N);
    bf16x8 pk[2 * C::IT], dsk[2 * C::IT];
#pragma unroll
    for (int it = 0; it < C::IT; ++it) {
      float pv[16], dsv[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int rl = 32 * it + 8 * g + 4 * hh;   // local row of v = 4g
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(Ls + rl);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(Ds + rl);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int v = 4 * g + r;
          float pe = fast_exp2(__builtin_fmaf(s[it][v], p.sl2, -l4[r]));
          if (edge) {
            const int row = row0 + rl + r;
            if ((CAUSAL && mykey > row) || mykey >= N) pe = 0.f;
          }
          pv[v] = pe;
          dsv[v] = pe * (dp[it][v] - d4[r]);
        }
      }
      pk[2 * it] = to_bf16x8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
      pk[2 * it + 1] = to_bf16x8(pv[8], pv[9], pv[10], pv[11], pv[12], pv[13], pv[14], pv[15]);
      dsk[2 * it] = to_bf16x8(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
      dsk[2 * it + 1] =
          to_bf16x8(dsv[8], dsv[9], dsv[10], dsv[11], dsv[12], dsv[13], dsv[14], dsv[15]);
      // dS^T row (key) of this lane, four consecutive query rows per store.
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        *reinterpret_cast<bf16x4*>(dSt + (32 * wave + l32) * C::SSTR + 32 * it + 8 * g + 4 * hh) =
            to_bf16x4(dsv[4 * g], dsv[4 * g + 1], dsv[4 * g + 2], dsv[4 * g + 3]);
      }
    }

    // dV^T += dO^T P and dK^T += Q^T dS. MFMA k-slots (query rows) follow the
    // accumulator layout: lane half hh holds rows 4hh..4hh+3 and 8+4hh..8+4hh+3 of
    // each 16, so the transposed operand is read as those two groups of four rows.
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
      const int n0 = 32 * ct + 16 * (g16 & 1) + 4 * (i16 & 3);
#pragma unroll
      for (int ks = 0; ks < 2 * C::IT; ++ks) {
        const int r0 = 16 * ks + 4 * hh + (i16 >> 2);
        const bf16x8 ot = cat(lds_tr(dOs + r0 * C::STR + n0), lds_tr(dOs + (r0 + 8) * C::STR + n0));
        dv[ct] = mfma32(ot, pk[ks], dv[ct]);
        const bf16x8 qt = cat(lds_tr(Qs + r0 * C::STR + n0), lds_tr(Qs + (r0 + 8) * C::STR + n0));
        dk[ct] = mfma32(qt, dsk[ks], dk[ct]);
      }
    }
    __syncthreads();   // dS^T complete; Q/dO no longer read in this iteration

    // dQ[rows][c] += sum over the 128 keys of dS[row][key] K[key][c].
#pragma unroll
    for (int t = 0; t < C::DQT; ++t) {
      const int tile = wave + C::WAVES * t;
      const int it = tile % C::IT;
      const int ct = tile / C::IT;
      f32x16 acc = f32x16{};
      const int na = 32 * it + 16 * (g16 & 1) + 4 * (i16 & 3);
      const int nb = 32 * ct + 16 * (g16 & 1) + 4 * (i16 & 3);
#pragma unroll
      for (int ks = 0; ks < C::BN / 16; ++ks) {
        const int r0 = 16 * ks + 4 * hh + (i16 >> 2);
        const bf16x8 a = cat(lds_tr(dSt + r0 * C::SSTR + na), lds_tr(dSt + (r0 + 8) * C::SSTR + na));
        const bf16x8 b = cat(lds_tr(Ks + r0 * C::STR + nb), lds_tr(Ks + (r0 + 8) * C::STR + nb));
        acc = mfma32(a, b, acc);
      }
      // acc[v]: row row0 + 32*it + 8*(v/4) + 4*hh + v%4, column 32*ct + l32.
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = row0 + 32 * it + 8 * (v / 4) + 4 * hh + (v % 4);
        if (row < N) unsafeAtomicAdd(dQh + (int64_t)row * D + 32 * ct + l32, acc[v]);
      }
    }
    __syncthreads();   // all dS^T / Q / dO reads done before the next row block overwrites them
  }

  // dK^T / dV^T accumulators: lane holds key mykey, columns 32*ct + 8*g + 4*hh + r.
  if (mykey < N) {
    bf16* dkrow = p.dk + head + (int64_t)mykey * D;
    bf16* dvrow = p.dv + head + (int64_t)mykey * D;
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = 32 * ct + 8 * g + 4 * hh;
        *reinterpret_cast<bf16x4*>(dkrow + c) =
            to_bf16x4(dk[ct][4 * g] * p.scale, dk[ct][4 * g + 1] * p.scale,
                      dk[ct][4 * g + 2] * p.scale, dk[ct][4 * g + 3] * p.scale);
        *reinterpret_cast<bf16x4*>(dvrow + c) =
            to_bf16x4(dv[ct][4 * g], dv[ct][4 * g + 1], dv[ct][4 * g + 2], dv[ct][4 * g + 3]);
      }
    }
  }
}

template <int D>
hipError_t launch_main_d(const BwdArgs& a, hipStream_t stream) {
  using C = BwdCfg<D>;
  BwdParams p;
  p.q = static_cast<const bf16*>(a.q);
  p.k = static_cast<const bf16*>(a.k);
  p.v = static_cast<const bf16*>(a.v);
  p.dout = static_cast<const bf16*>(a.dout);
  p.lse = a.lse;
  p.dvec = a.dvec;
  p.dqacc = a.dqacc;
  p.dk = static_cast<bf16*>(a.dk);
  p.dv = static_cast<bf16*>(a.dv);
  p.BH = a.BH;
  p.N = a.N;
  p.sl2 = a.scale * kLog2e;
  p.scale = a.scale;
  p.blocks = a.mask.blocks;
  p.blocks_bh_stride = a.mask.bh_stride;
  p.nb = a.mask.nb;
  const int n_kb = (a.N + C::BN - 1) / C::BN;
  const dim3 grid((unsigned)n_kb * (unsigned)a.BH);
  const dim3 block(C::THREADS);
  const bool blk = a.mask.blocks != nullptr;
  if (a.mask.causal) {
    if (blk)
      hipLaunchKernelGGL((fa_bwd_main_kernel<D, true, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((fa_bwd_main_kernel<D, true, false>), grid, block, 0, stream, p);
  } else {
    if (blk)
      hipLaunchKernelGGL((fa_bwd_main_kernel<D, false, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((fa_bwd_main_kernel<D, false, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_preprocess(const BwdArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.BH * a.N;
  const int lpr = a.d / 8;
  const int rpb = 256 / lpr;
  const dim3 grid((unsigned)((rows + rpb - 1) / rpb));
  const bf16* o = static_cast<const bf16*>(a.o);
  const bf16* dout = static_cast<const bf16*>(a.dout);
  if (a.d == 128)
    hipLaunchKernelGGL((fa_bwd_pre_kernel<128>), grid, dim3(256), 0, stream, o, dout, a.dvec,
                       a.dqacc, rows);
  else
    hipLaunchKernelGGL((fa_bwd_pre_kernel<64>), grid, dim3(256), 0, stream, o, dout, a.dvec,
                       a.dqacc, rows);
  return hipGetLastError();
}

hipError_t launch_bwd_main(const BwdArgs& a, hipStream_t stream) {
  return a.d == 128 ? launch_main_d<128>(a, stream) : launch_main_d<64>(a, stream);
}

hipError_t launch_bwd_finish(const BwdArgs& a, hipStream_t stream) {
  const int64_t n8 = (int64_t)a.BH * a.N * a.d / 8;
  const dim3 grid((unsigned)((n8 + 255) / 256));
  hipLaunchKernelGGL(fa_bwd_finish_kernel, grid, dim3(256), 0, stream, a.dqacc,
                     static_cast<bf16*>(a.dq), a.scale, n8);
  return hipGetLastError();
}

}  // namespace fa

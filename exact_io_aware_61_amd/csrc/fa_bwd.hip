// Backward attention for gfx950, dK/dV part, with P recomputed from the saved LSE.
//
// Recomputation (lecture summary on FlashAttention v1, part 4.2): no N x N matrix
// is read back; each tile of S and P is rebuilt on chip from Q, K and the row
// logsumexp, the only statistic kept (FlashAttention-2 overview, backward pass).
// Partitioning (same overview): one workgroup per block of key columns of one
// (batch, head); it sweeps the query row blocks and keeps its dK and dV on chip.
// dQ, the one quantity the key blocks share, is computed by its own pass
// (fa_bwd_dq.hip) instead of being merged by atomics here.
//
// The gradients are the chain rule through the softmax (the pages only name
// it): dP = dO V^T, D_i = sum_j P_ij dP_ij = dO_i . O_i, dS = P o (dP - D),
// dV = P^T dO, dK = scale dS^T Q, dQ = scale dS K.
//
// Layout work done once per call (preprocess kernel): D_i and transposed copies
// Q^T and dO^T ([d][rows], rows padded to a multiple of 64). In the transposed
// copies the rows of every 16-row group are stored in the order 0-3, 8-11,
// 4-7, 12-15: eight consecutive positions then hold exactly the rows that one
// half of a wave holds in an MFMA accumulator (rows 4h..4h+3 and 8+4h..8+4h+3),
// so the dK/dV products read their Q^T/dO^T operand with plain 16-byte LDS
// reads instead of transposing 8-byte reads.
//
// dK/dV kernel, per workgroup of 4 waves = 128 keys; wave w owns keys
// key0 + 32w .. +31. Per block of BM query rows, per wave:
//   S  = Q K_w^T, dP = dO V_w^T   MFMA 32x32x16; Q/dO rows from LDS, K_w/V_w in
//                                 VGPRs. Each lane holds one key column.
//   P  = 2^(S scale log2e - LSE_i log2e)  (masked pairs -> 0)
//   dS = P o (dP - D_i)
//   dV_w^T += dO^T P, dK_w^T += Q^T dS    P, dS straight from registers as the
//                                 B operand, dO^T/Q^T by 16-byte LDS reads
#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {
namespace {

// Position <-> row inside a 16-row group of the transposed copies: positions
// 4..7 and 8..11 are exchanged (the map is its own inverse).
__device__ __forceinline__ int perm16(int pos) {
  const int s = pos & 15;
  return (pos & ~15) | ((s >= 4 && s < 12) ? (s ^ 12) : s);
}

// ------------------------------------------------------------------------------------------------
// Preprocess: D_i = sum_c dO_ic O_ic, and the transposed copies Q^T and dO^T.

constexpr int kPreRows = 64;   // rows per preprocess workgroup
constexpr int kRowPad = 128;   // Q^T / dO^T rows are padded to a multiple of this (>= any BM)

struct PreParams {
  const bf16* q;
  const bf16* o;
  const bf16* dout;
  float* dvec;
  bf16* qt;
  bf16* dot;
  int BH;
  int N;
  int Np;   // padded row count of Q^T / dO^T (multiple of kRowPad)
};

template <int D>
__global__ __launch_bounds__(256) void fa_bwd_pre_kernel(PreParams p) {
  constexpr int R = kPreRows;
  constexpr int STR = D + 8;
  constexpr int LPR = D / 8;            // 16-byte chunks (lanes) per row
  constexpr int CH = R * LPR / 256;     // chunks per thread
  constexpr int TI = D * (R / 8) / 256; // transposed 16-byte outputs per thread per tensor
  __shared__ __attribute__((aligned(16))) bf16 Qs[R * STR];
  __shared__ __attribute__((aligned(16))) bf16 Gs[R * STR];

  const int nrb = p.Np / R;
  const int bh = blockIdx.x / nrb;
  const int row0 = (blockIdx.x % nrb) * R;
  const int N = p.N;
  const int tid = threadIdx.x;
  const int64_t head = (int64_t)bh * N * D;

#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int id = tid + 256 * c;
    const int r = id / LPR;
    const int part = id % LPR;
    const int row = row0 + r;
    u32x4 xq = {0, 0, 0, 0}, xg = {0, 0, 0, 0};
    float acc = 0.f;
    if (row < N) {
      const int64_t off = head + (int64_t)row * D + 8 * part;
      xq = *reinterpret_cast<const u32x4*>(p.q + off);
      xg = *reinterpret_cast<const u32x4*>(p.dout + off);
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(p.o + off);
      const bf16x8 b = __builtin_bit_cast(bf16x8, xg);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)b[e];
    }
    // The LPR lanes of one row are consecutive: reduce across them.
#pragma unroll
    for (int sh = LPR / 2; sh > 0; sh >>= 1) acc += __shfl_xor(acc, sh);
    if (row < N && part == 0) p.dvec[(int64_t)bh * N + row] = acc;
    *reinterpret_cast<u32x4*>(Qs + r * STR + 8 * part) = xq;
    *reinterpret_cast<u32x4*>(Gs + r * STR + 8 * part) = xg;
  }
  __syncthreads();

  // Transposed, row-permuted copies: output chunk (column c, positions 8j..8j+7);
  // positions past N (up to the padding) are written as zeros.
#pragma unroll
  for (int t = 0; t < TI; ++t) {
    const int id = tid + 256 * t;
    const int col = id / (R / 8);
    const int j = id % (R / 8);
    bf16x8 vq, vg;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = perm16(8 * j + e);
      vq[e] = Qs[r * STR + col];
      vg[e] = Gs[r * STR + col];
    }
    const int64_t off = ((int64_t)bh * D + col) * p.Np + row0 + 8 * j;
    *reinterpret_cast<bf16x8*>(p.qt + off) = vq;
    *reinterpret_cast<bf16x8*>(p.dot + off) = vg;
  }
}

// ------------------------------------------------------------------------------------------------
// dK/dV kernel.

template <int D>
struct BwdCfg {
  static constexpr int WAVES = 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BN = 32 * WAVES;           // keys per workgroup (= block-mask granularity)
  static constexpr int BM = D == 128 ? 64 : 128;  // query rows per iteration
  static constexpr int IT = BM / 32;              // 32-row sub-tiles
  static constexpr int RS = BM / 16;              // 16-row MFMA k-steps
  static constexpr int KS = D / 16;               // 16-column MFMA k-steps over the head dim
  static constexpr int CT = D / 32;               // 32-column sub-tiles of the head dim
  // LDS row strides (bf16 elements): 16-byte row reads of 32 rows are free of
  // bank conflicts at a stride of 4 (mod 64) dwords (Q, dO: 136 / 72 elements,
  // Q^T, dO^T: 72 / 136 elements).
  static constexpr int STRQ = D + 8;              // Q, dO tiles     [BM][STRQ]
  static constexpr int STRT = BM + 8;             // Q^T, dO^T tiles [D][STRT]
  static constexpr int QTILE = BM * STRQ;
  static constexpr int TTILE = D * STRT;
  static constexpr int STAGE = 2 * QTILE + 2 * TTILE;
  static constexpr int CH = BM * D / 8;           // 16-byte chunks per tile (all four tiles)
  static constexpr int CPT = CH / THREADS;
  static_assert(CH % THREADS == 0, "tiles split evenly over threads");
  static_assert(kRowPad % BM == 0, "row padding of the transposed copies covers whole row blocks");
};

struct BwdParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* dout;
  const bf16* qt;
  const bf16* dot;
  const float* lse;
  const float* dvec;
  bf16* dk;
  bf16* dv;
  int BH;
  int N;
  int Np;
  float sl2;    // scale * log2(e)
  float scale;
  const uint8_t* blocks;
  int64_t blocks_bh_stride;
  int nb;
};

template <int D, bool CAUSAL, bool BLOCK>
__global__ __launch_bounds__(256) void fa_bwd_dkdv_kernel(BwdParams p) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) bf16 tiles[2 * C::STAGE];  // [stage][Q, dO, Q^T, dO^T]
  __shared__ __attribute__((aligned(16))) float rowstat[2][2][C::BM]; // [stage][LSE*log2e, D][row]

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
  const bf16* __restrict__ QTh = p.qt + (int64_t)bh * D * p.Np;
  const bf16* __restrict__ dOTh = p.dot + (int64_t)bh * D * p.Np;
  const float* __restrict__ Lh = p.lse + (int64_t)bh * N;
  const float* __restrict__ Dh = p.dvec + (int64_t)bh * N;

  const int key0 = kb * C::BN;
  const int wkey0 = key0 + 32 * wave;
  const int mykey = wkey0 + l32;   // this lane's key column
  // S / dP B operands: K and V rows of this lane's key, k = head-dim chunks.
  bf16x8 kf[C::KS], vf[C::KS];
  {
    const int key = min(mykey, N - 1);
#pragma unroll
    for (int kk = 0; kk < C::KS; ++kk) {
      kf[kk] = *reinterpret_cast<const bf16x8*>(Kh + (int64_t)key * D + 16 * kk + 8 * hh);
      vf[kk] = *reinterpret_cast<const bf16x8*>(Vh + (int64_t)key * D + 16 * kk + 8 * hh);
    }
  }

  f32x16 dk[C::CT], dv[C::CT];
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) {
    dk[ct] = f32x16{};
    dv[ct] = f32x16{};
  }

  // Row blocks: under causal, rows before key0 see none of these keys.
  const int n_rb = (N + C::BM - 1) / C::BM;
  const int rb_begin = CAUSAL ? key0 / C::BM : 0;
  auto kept = [&](int rb) -> bool {
    if (!BLOCK) return true;
    return p.blocks[bh * p.blocks_bh_stride + (int64_t)((rb * C::BM) / 128) * p.nb + kb] != 0;
  };
  auto next_kept = [&](int rb) -> int {
    ++rb;
    while (rb < n_rb && !kept(rb)) ++rb;
    return rb;
  };

  u32x4 sq[C::CPT], sdo[C::CPT], sqt[C::CPT], sdot[C::CPT];
  float s_l = 0.f, s_d = 0.f;
  int row_next = 0;   // first row of the staged block
  auto load_rb = [&](int rb) {
    const int row0 = rb * C::BM;
    row_next = row0;
#pragma unroll
    for (int c = 0; c < C::CPT; ++c) {
      const int id = tid + c * C::THREADS;
      const int r = id / (D / 8);
      const int col = (id % (D / 8)) * 8;
      const int64_t off = (int64_t)min(row0 + r, N - 1) * D + col;  // rows past N get P = 0
      sq[c] = *reinterpret_cast<const u32x4*>(Qh + off);
      sdo[c] = *reinterpret_cast<const u32x4*>(dOh + off);
      const int dd = id / (C::BM / 8);
      const int j = id % (C::BM / 8);
      const int64_t toff = (int64_t)dd * p.Np + row0 + 8 * j;
      sqt[c] = *reinterpret_cast<const u32x4*>(QTh + toff);
      sdot[c] = *reinterpret_cast<const u32x4*>(dOTh + toff);
    }
    // Raw values only: they are first used after the compute phase, so the
    // loads stay in flight across it (using them here would wait for every
    // load issued above).
    if (tid < C::BM) {
      const int row = min(row0 + tid, N - 1);
      s_l = Lh[row];
      s_d = Dh[row];
    }
  };
  auto store_rb = [&](int buf) {
    bf16* Qs = tiles + buf * C::STAGE;
    bf16* dOs = Qs + C::QTILE;
    bf16* QTs = dOs + C::QTILE;
    bf16* dOTs = QTs + C::TTILE;
#pragma unroll
    for (int c = 0; c < C::CPT; ++c) {
      const int id = tid + c * C::THREADS;
      const int r = id / (D / 8);
      const int col = (id % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(Qs + r * C::STRQ + col) = sq[c];
      *reinterpret_cast<u32x4*>(dOs + r * C::STRQ + col) = sdo[c];
      const int dd = id / (C::BM / 8);
      const int j = id % (C::BM / 8);
      *reinterpret_cast<u32x4*>(QTs + dd * C::STRT + 8 * j) = sqt[c];
      *reinterpret_cast<u32x4*>(dOTs + dd * C::STRT + 8 * j) = sdot[c];
    }
    if (tid < C::BM) {
      // +inf: the row contributes nothing (past N, or no visible key at all).
      const bool live = row_next + tid < N && s_l != -INFINITY;
      rowstat[buf][0][tid] = live ? s_l * kLog2e : INFINITY;
      rowstat[buf][1][tid] = live ? s_d : 0.f;
    }
  };

  auto compute = [&](int rb, int buf) {
    const bf16* Qs = tiles + buf * C::STAGE;
    const bf16* dOs = Qs + C::QTILE;
    const bf16* QTs = dOs + C::QTILE;
    const bf16* dOTs = QTs + C::TTILE;
    const float* Ls = rowstat[buf][0];
    const float* Ds = rowstat[buf][1];
    const int row0 = rb * C::BM;

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
        const bf16x8 a = lds_b128(Qs + (32 * it + l32) * C::STRQ + 16 * kk + 8 * hh);
        s[it] = mfma32(a, kf[kk], s[it]);
        const bf16x8 b = lds_b128(dOs + (32 * it + l32) * C::STRQ + 16 * kk + 8 * hh);
        dp[it] = mfma32(b, vf[kk], dp[it]);
      }
    }
    // s[it][v]: row row0 + 32*it + 8*(v/4) + 4*hh + v%4, key mykey.
    const bool edge = (CAUSAL && row0 < wkey0 + 31) || (key0 + C::BN > N);
    bf16x8 pk[C::RS], dsk[C::RS];
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
    }

    // dV^T += dO^T P and dK^T += Q^T dS; the permuted row order of the transposed
    // tiles makes positions 16ks + 8hh .. +7 the rows this lane half holds in P, dS.
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
#pragma unroll
      for (int ks = 0; ks < C::RS; ++ks) {
        const bf16x8 ot = lds_b128(dOTs + (32 * ct + l32) * C::STRT + 16 * ks + 8 * hh);
        dv[ct] = mfma32(ot, pk[ks], dv[ct]);
        const bf16x8 qt = lds_b128(QTs + (32 * ct + l32) * C::STRT + 16 * ks + 8 * hh);
        dk[ct] = mfma32(qt, dsk[ks], dk[ct]);
      }
    }
  };

  int rb = rb_begin;
  if (rb < n_rb && !kept(rb)) rb = next_kept(rb);
  if (rb < n_rb) {
    load_rb(rb);
    store_rb(0);
    __syncthreads();
    int buf = 0;
    while (rb < n_rb) {
      const int rn = next_kept(rb);
      if (rn < n_rb) load_rb(rn);
      compute(rb, buf);
      if (rn < n_rb) store_rb(buf ^ 1);
      __syncthreads();   // next block staged; this block's buffers free
      buf ^= 1;
      rb = rn;
    }
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
hipError_t launch_dkdv_d(const BwdArgs& a, hipStream_t stream) {
  using C = BwdCfg<D>;
  BwdParams p;
  p.q = static_cast<const bf16*>(a.q);
  p.k = static_cast<const bf16*>(a.k);
  p.v = static_cast<const bf16*>(a.v);
  p.dout = static_cast<const bf16*>(a.dout);
  p.qt = static_cast<const bf16*>(a.qt);
  p.dot = static_cast<const bf16*>(a.dot);
  p.lse = a.lse;
  p.dvec = a.dvec;
  p.dk = static_cast<bf16*>(a.dk);
  p.dv = static_cast<bf16*>(a.dv);
  p.BH = a.BH;
  p.N = a.N;
  p.Np = a.Np;
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
      hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, true, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, true, false>), grid, block, 0, stream, p);
  } else {
    if (blk)
      hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, false, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, false, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

int bwd_row_padding() { return kRowPad; }

hipError_t launch_bwd_preprocess(const BwdArgs& a, hipStream_t stream) {
  PreParams p;
  p.q = static_cast<const bf16*>(a.q);
  p.o = static_cast<const bf16*>(a.o);
  p.dout = static_cast<const bf16*>(a.dout);
  p.dvec = a.dvec;
  p.qt = static_cast<bf16*>(a.qt);
  p.dot = static_cast<bf16*>(a.dot);
  p.BH = a.BH;
  p.N = a.N;
  p.Np = a.Np;
  const dim3 grid((unsigned)(a.BH * (a.Np / kPreRows)));
  if (a.d == 128)
    hipLaunchKernelGGL((fa_bwd_pre_kernel<128>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((fa_bwd_pre_kernel<64>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream) {
  return a.d == 128 ? launch_dkdv_d<128>(a, stream) : launch_dkdv_d<64>(a, stream);
}

}  // namespace fa

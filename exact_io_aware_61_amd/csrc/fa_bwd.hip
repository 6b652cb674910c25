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
#include <type_traits>

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
  // Four tiles per row block, swizzled and unpadded (fa_common.hpp), filled by
  // direct global->LDS loads: Q, dO [BM][D] (rows of CQ chunks) and Q^T, dO^T
  // [D][BM] (rows of CT_ chunks).
  static constexpr int CQ = D / 8;
  static constexpr int CTR = BM / 8;
  static constexpr int TILE = BM * D;             // elements per tile (all four)
  static constexpr int STAGE = 4 * TILE;
  static constexpr int SLOTS = TILE / 512;        // 1 KiB slots per tile
  static constexpr int SPW = SLOTS / WAVES;
  static_assert(SLOTS % WAVES == 0, "tile slots split evenly over waves");
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
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa_bwd_dkdv_kernel(BwdParams p) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) bf16 tiles[2 * C::STAGE];  // [stage][Q, dO, Q^T, dO^T]
  static_assert(2 * C::STAGE * 2 + 2 * 2 * C::BM * 4 <= 160 * 1024, "LDS budget");
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
  // Complete these before the loop: a wait for them inside it would also wait
  // for the row block in flight.
  wait_vmcnt<0>();

  // Lane offsets of the 16-byte row reads inside the tiles; the 32-row (Q, dO)
  // or 32-column (Q^T, dO^T) sub-tile steps add compile-time constants.
  int qoff[C::KS], toff_r[C::RS];
#pragma unroll
  for (int kk = 0; kk < C::KS; ++kk) qoff[kk] = toff<C::CQ>(l32, 16 * kk + 8 * hh);
#pragma unroll
  for (int ks = 0; ks < C::RS; ++ks) toff_r[ks] = toff<C::CTR>(l32, 16 * ks + 8 * hh);

  f32x16 dk[C::CT], dv[C::CT];
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) {
    dk[ct] = f32x16{};
    dv[ct] = f32x16{};
  }

  // Row blocks: under causal, rows before key0 see none of these keys.
  const int n_rb = (N + C::BM - 1) / C::BM;
  const int rb_begin = CAUSAL ? key0 / C::BM : 0;
  // Block mask: this workgroup's key block is one mask column; its bits go to
  // LDS once, so the row-block loop reads no global memory besides its tiles.
  __shared__ uint32_t mbits[BLOCK ? kMaskWords : 1];
  if (BLOCK) {
    const int nw = (p.nb + 63) / 64;
    const uint8_t* grid = p.blocks + bh * p.blocks_bh_stride;
    for (int j = wave; j < nw; j += C::WAVES) {
      const int b = j * 64 + lane;
      const bool keep = b < p.nb && grid[(int64_t)b * p.nb + kb] != 0;
      const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
      if (lane == 0) {
        mbits[2 * j] = (uint32_t)bal;
        mbits[2 * j + 1] = (uint32_t)(bal >> 32);
      }
    }
    wait_vmcnt<0>();
    __syncthreads();
  }
  auto kept = [&](int rb) -> bool {
    if (!BLOCK) return true;
    const int b = (rb * C::BM) / 128;
    return (mbits[b >> 5] >> (b & 31)) & 1u;
  };
  auto next_kept = [&](int rb) -> int {
    ++rb;
    while (rb < n_rb && !kept(rb)) ++rb;
    return rb;
  };

  // Direct global->LDS loads of one row block's four tiles into a stage, and
  // the row statistics into registers (their raw values: they are first used
  // after the compute phase, so the loads stay in flight across it).
  float s_l = 0.f, s_d = 0.f;
  int row_next = 0;   // first row of the staged block
  auto issue = [&](int rb, int buf) {
    const int row0 = rb * C::BM;
    row_next = row0;
    bf16* Qs = tiles + buf * C::STAGE;
    bf16* dOs = Qs + C::TILE;
    bf16* QTs = dOs + C::TILE;
    bf16* dOTs = QTs + C::TILE;
#pragma unroll
    for (int i = 0; i < C::SPW; ++i) {
      const int slot = wave + i * C::WAVES;
      // rows past N are clamped: their P is 0 (LSE = +inf below)
      dma_slot<C::CQ>(Qs, slot, lane,
                      [&](int r) { return Qh + (int64_t)min(row0 + r, N - 1) * D; });
      dma_slot<C::CQ>(dOs, slot, lane,
                      [&](int r) { return dOh + (int64_t)min(row0 + r, N - 1) * D; });
      dma_slot<C::CTR>(QTs, slot, lane, [&](int r) { return QTh + (int64_t)r * p.Np + row0; });
      dma_slot<C::CTR>(dOTs, slot, lane, [&](int r) { return dOTh + (int64_t)r * p.Np + row0; });
    }
    if (tid < C::BM) {
      const int row = min(row0 + tid, N - 1);
      s_l = Lh[row];
      s_d = Dh[row];
    }
  };
  auto store_stats = [&](int buf) {
    if (tid < C::BM) {
      // +inf: the row contributes nothing (past N, or no visible key at all).
      const bool live = row_next + tid < N && s_l != -INFINITY;
      rowstat[buf][0][tid] = live ? s_l * kLog2e : INFINITY;
      rowstat[buf][1][tid] = live ? s_d : 0.f;
    }
  };

  // EDGE: the block has pairs to mask (causal diagonal, keys past N); interior
  // blocks are compiled without any masking code.
  auto compute = [&](int rb, int buf, auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const bf16* Qs = tiles + buf * C::STAGE;
    const bf16* dOs = Qs + C::TILE;
    const bf16* QTs = dOs + C::TILE;
    const bf16* dOTs = QTs + C::TILE;
    const float* Ls = rowstat[buf][0];
    const float* Ds = rowstat[buf][1];
    const int row0 = rb * C::BM;

    // One 32-row sub-tile at a time (S, dP, softmax, then its share of dV/dK):
    // the same LDS reads as a whole-block pass, with half the live registers.
#pragma unroll
    for (int it = 0; it < C::IT; ++it) {
      // All operand reads of the sub-tile are issued before its MFMAs (the
      // scheduling barriers keep the compiler from pairing each read with its
      // MFMA, which would expose the LDS latency once per MFMA).
      bf16x8 qa[C::KS], ga[C::KS];
#pragma unroll
      for (int kk = 0; kk < C::KS; ++kk) {
        qa[kk] = lds_b128(Qs + qoff[kk] + 32 * it * D);
        ga[kk] = lds_b128(dOs + qoff[kk] + 32 * it * D);
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < C::KS; ++kk) {
        s = mfma32(qa[kk], kf[kk], s);
        dp = mfma32(ga[kk], vf[kk], dp);
      }
      // Operands of this sub-tile's dV/dK products: read now, consumed after
      // the softmax below.
      bf16x8 ota[C::CT][2], qta[C::CT][2];
#pragma unroll
      for (int ct = 0; ct < C::CT; ++ct) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          ota[ct][h] = lds_b128(dOTs + toff_r[2 * it + h] + 32 * ct * C::BM);
          qta[ct][h] = lds_b128(QTs + toff_r[2 * it + h] + 32 * ct * C::BM);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // s[v]: row row0 + 32*it + 8*(v/4) + 4*hh + v%4, key mykey.
      float pv[16], dsv[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int rl = 32 * it + 8 * g + 4 * hh;   // local row of v = 4g
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(Ls + rl);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(Ds + rl);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int v = 4 * g + r;
          float pe = fast_exp2(__builtin_fmaf(s[v], p.sl2, -l4[r]));
          if (EDGE) {
            const int row = row0 + rl + r;
            if ((CAUSAL && mykey > row) || mykey >= N) pe = 0.f;
          }
          pv[v] = pe;
          dsv[v] = pe * (dp[v] - d4[r]);
        }
      }
      bf16x8 pk[2], dsk[2];
      pk[0] = to_bf16x8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
      pk[1] = to_bf16x8(pv[8], pv[9], pv[10], pv[11], pv[12], pv[13], pv[14], pv[15]);
      dsk[0] = to_bf16x8(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
      dsk[1] = to_bf16x8(dsv[8], dsv[9], dsv[10], dsv[11], dsv[12], dsv[13], dsv[14], dsv[15]);

      // dV^T += dO^T P and dK^T += Q^T dS over this sub-tile's rows; the permuted
      // row order of the transposed tiles makes positions 16ks + 8hh .. +7 the
      // rows this lane half holds in P and dS.
#pragma unroll
      for (int ct = 0; ct < C::CT; ++ct) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          dv[ct] = mfma32(ota[ct][h], pk[h], dv[ct]);
          dk[ct] = mfma32(qta[ct][h], dsk[h], dk[ct]);
        }
      }
    }
  };

  // One step: stage the next kept row block, compute this one, publish.
  auto step = [&](int& rb, int& buf, auto edge_tag) {
    const int rn = next_kept(rb);
    if (rn < n_rb) issue(rn, buf ^ 1);
    compute(rb, buf, edge_tag);
    if (rn < n_rb) {
      wait_vmcnt<0>();
      store_stats(buf ^ 1);
    }
    __syncthreads();   // next block landed; this block's buffers free
    buf ^= 1;
    rb = rn;
  };
  // Blocks that need masking come first (the causal diagonal: rows below
  // key0 + BN - 1) or are all of them (the last key block when N is ragged);
  // the rest run a copy of the body without any masking code.
  auto edge_block = [&](int rb) {
    return (CAUSAL && rb * C::BM < key0 + C::BN - 1) || key0 + C::BN > N;
  };
  int rb = rb_begin;
  if (rb < n_rb && !kept(rb)) rb = next_kept(rb);
  if (rb < n_rb) {
    issue(rb, 0);
    wait_vmcnt<0>();
    store_stats(0);
    __syncthreads();
    int buf = 0;
    while (rb < n_rb && edge_block(rb)) step(rb, buf, std::true_type{});
    while (rb < n_rb) step(rb, buf, std::false_type{});
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

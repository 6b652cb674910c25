// Backward, dQ part, for gfx950: dQ = scale * dS K with dS recomputed per tile.
//
// The FlashAttention-2 overview (backward pass) merges dQ across the workers
// of different key blocks by atomic addition. On MI355X those float32 atomics
// resolve beyond the per-XCD L2 caches and cost more than the products they
// merge, so dQ has its own pass instead (the alternative the same passage
// leaves open: dQ is the only quantity the key blocks share): one workgroup
// per block of query rows sweeps the key/value tiles exactly like the forward
// pass, recomputes S and dP (lecture summary on FlashAttention v1, part 4.2:
// recompute from the saved statistics) and accumulates dQ on chip. Nothing is
// exchanged between workgroups, and dQ is bitwise reproducible.
//
// Tiles reach LDS exactly as in the forward kernel: direct global->LDS loads
// into the swizzled layout of fa_common.hpp, up to three tiles in flight.
//
// Per wave (32 query rows) and K/V tile (BN keys):
//   S^T  = K_tile Q_w^T        MFMA 32x32x16: K rows from LDS, Q^T in VGPRs;
//   dP^T = V_tile dO_w^T       likewise. Each lane holds one query row, so the
//                              row's LSE and D_i = dO_i . O_i are lane scalars.
//   P  = 2^(S scale log2e - L2_i)    L2_i = LSE_i log2e from the preprocess
//                                    (+inf for rows that see no key); masked
//                                    pairs -> 0
//   dS = P o (dP - D_i)
//   dQ^T += K_tile^T dS^T      dS^T straight from registers as the B operand
//                              (keys in the accumulator's order), K^T by the
//                              transposing LDS read.
// dQ = scale * dQ^T^T is written as bf16 once at the end.
#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {
namespace {

template <int D, bool BLOCK>
struct DqCfg {
  // A block mask works on 128-row blocks: masked launches use 128-row
  // workgroups so that every wave of a workgroup keeps the same tiles. At d=64
  // every launch does: the kernel fits in 168 registers and a 48 KiB ring, so
  // three 4-wave workgroups share a CU (three waves per SIMD), where 8-wave
  // workgroups would leave it at two. Unmasked at d=64 the tiles are 32 keys
  // in a two-stage ring, which brings the kernel to 128 registers: four
  // workgroups and four waves per SIMD. (With a block mask the sweeps are short
  // and the per-tile costs of 32-key tiles outweigh the occupancy.)
  static constexpr bool SMALL = D == 64 && !BLOCK;
  static constexpr int WAVES = (BLOCK || D == 64) ? 4 : 8;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BM = 32 * WAVES;           // query rows per workgroup
  static constexpr int BN = SMALL ? 32 : 64;      // keys per K/V tile
  static constexpr int C = D / 8;                 // 16-byte chunks per tile row
  static constexpr int KS = D / 16;
  static constexpr int NT = BN / 32;
  static constexpr int CT = D / 32;
  static constexpr int TILE = BN * D;             // elements per K or V tile (swizzled, unpadded)
  static constexpr int STAGE = 2 * TILE;
  static constexpr int NSTAGE = (SMALL || (BLOCK && D == 128)) ? 2 : 3;
  static constexpr int SLOTS = BN * C / 64;
  static constexpr int SPW = SLOTS / WAVES;
  static constexpr int LPT = 2 * SPW;
  static constexpr int NMR = BM / 128;            // block-mask rows per workgroup
  static_assert(SLOTS % WAVES == 0, "tile slots split evenly over waves");
};

struct DqParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* dout;
  const float* l2;     // [BH][Np]
  const float* dvec;   // [BH][Np]
  bf16* dq;
  int BH;
  int N;
  int Np;
  int n_row_blocks;
  float sl2;    // scale * log2(e)
  float scale;
  const uint8_t* blocks;
  int64_t blocks_bh_stride;
  int nb;
};

template <int D, bool CAUSAL, bool BLOCK>
__global__ __launch_bounds__((DqCfg<D, BLOCK>::THREADS))
__attribute__((amdgpu_waves_per_eu(DqCfg<D, BLOCK>::SMALL ? 4 : 2)))
void fa_bwd_dq_kernel(DqParams p) {
  using C = DqCfg<D, BLOCK>;
  __shared__ __attribute__((aligned(16))) bf16 smem[C::NSTAGE * C::STAGE];  // [stage][K, V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int g16 = lane >> 4;
  const int i16 = lane & 15;

  // Largest causal row blocks first.
  const WgCoord wc = wg_coord<BLOCK>(blockIdx.x, p.BH, p.n_row_blocks);
  const int bh = wc.bh;
  const int rb = p.n_row_blocks - 1 - wc.blk;
  const int N = p.N;
  const int64_t head = (int64_t)bh * N * D;
  const bf16* __restrict__ Kh = p.k + head;
  const bf16* __restrict__ Vh = p.v + head;
  const int row0 = rb * C::BM;
  const int wrow0 = row0 + 32 * wave;
  const int qrow = wrow0 + l32;

  int kt_end = (N + C::BN - 1) / C::BN;
  if (CAUSAL) kt_end = min(kt_end, (row0 + C::BM - 1) / C::BN + 1);

  // Block mask: the workgroup's rows span two 128-row mask rows; their bits go
  // to LDS once. A tile is loaded if either row keeps it; a wave skips tiles
  // its own row drops.
  __shared__ uint32_t mbits[BLOCK ? C::NMR * kMaskWords : 1];
  const int mr0 = row0 / 128;
  const int my_mr = wrow0 / 128 - mr0;
  if (BLOCK) {
    const int nw = (p.nb + 63) / 64;
    const uint8_t* grid = p.blocks + bh * p.blocks_bh_stride;
    for (int j = wave; j < C::NMR * nw; j += C::WAVES) {
      const int rr = j / nw;
      const int b = (j % nw) * 64 + lane;
      const bool keep = mr0 + rr < p.nb && b < p.nb && grid[(int64_t)(mr0 + rr) * p.nb + b] != 0;
      const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
      if (lane == 0) {
        mbits[rr * kMaskWords + 2 * (j % nw)] = (uint32_t)bal;
        mbits[rr * kMaskWords + 2 * (j % nw) + 1] = (uint32_t)(bal >> 32);
      }
    }
    wait_vmcnt<0>();
    __syncthreads();
  }
  auto mbit = [&](int rr, int kt) -> bool {
    const int b = (kt * C::BN) / 128;
    return (mbits[rr * kMaskWords + (b >> 5)] >> (b & 31)) & 1u;
  };
  auto kept = [&](int kt) -> bool { return !BLOCK || mbit(0, kt) || (C::NMR > 1 && mbit(1, kt)); };
  auto next_kept = [&](int kt) -> int {
    ++kt;
    while (kt < kt_end && !kept(kt)) ++kt;
    return kt;
  };

  // B operands of S^T and dP^T: this lane's Q and dO row, 8 head-dim values per k-step.
  bf16x8 qf[C::KS], gf[C::KS];
  float lrow = INFINITY, drow = 0.f;   // +inf: the row contributes nothing
  {
    const int r = min(qrow, N - 1);
#pragma unroll
    for (int kk = 0; kk < C::KS; ++kk) {
      qf[kk] = *reinterpret_cast<const bf16x8*>(p.q + head + (int64_t)r * D + 16 * kk + 8 * hh);
      gf[kk] = *reinterpret_cast<const bf16x8*>(p.dout + head + (int64_t)r * D + 16 * kk + 8 * hh);
    }
    if (qrow < N) {
      lrow = p.l2[(int64_t)bh * p.Np + r];
      drow = p.dvec[(int64_t)bh * p.Np + r];
    }
  }

  // Direct global->LDS loads of one K/V tile into a stage (keys past N clamped).
  // Byte offsets of this lane's chunks in its slots, the same for every tile.
  const int uwave = __builtin_amdgcn_readfirstlane(wave);   // uniform: scalar address math
  const uint32_t lds0 = lds_byte_addr(smem);
  uint32_t soff[C::SPW];
#pragma unroll
  for (int i = 0; i < C::SPW; ++i) soff[i] = slot_offset<C::C>(wave + i * C::WAVES, lane, 2 * D);
  auto issue = [&](int kt, int stage) {
    bf16* Ks = smem + stage * C::STAGE;
    bf16* Vs = Ks + C::TILE;
    const int key0 = kt * C::BN;
    if (key0 + C::BN <= N) {
      // whole tile inside the sequence: scalar base, fixed lane offsets
      const bf16* kb = Kh + (int64_t)key0 * D;
      const bf16* vb = Vh + (int64_t)key0 * D;
      const uint32_t kdst = lds0 + 2u * (uint32_t)(stage * C::STAGE);
#pragma unroll
      for (int i = 0; i < C::SPW; ++i) {
        const uint32_t o = 2u * 512u * (uint32_t)(uwave + i * C::WAVES);
        dma16_s(soff[i], kb, kdst + o);
        dma16_s(soff[i], vb, kdst + 2u * C::TILE + o);
      }
    } else {
      // the ragged last tile: keys past N clamped to the last key
#pragma unroll
      for (int i = 0; i < C::SPW; ++i) {
        const int slot = wave + i * C::WAVES;
        dma_slot<C::C>(Ks, slot, lane,
                       [&](int r) { return Kh + (int64_t)min(key0 + r, N - 1) * D; });
        dma_slot<C::C>(Vs, slot, lane,
                       [&](int r) { return Vh + (int64_t)min(key0 + r, N - 1) * D; });
      }
    }
  };

  // Lane offsets inside a tile: row reads of K and V (same layout), and the
  // transposing reads of K; sub-tile steps add compile-time constants.
  int roff[C::KS], toff_t[C::CT][2];
#pragma unroll
  for (int kk = 0; kk < C::KS; ++kk) roff[kk] = toff<C::C>(l32, 16 * kk + 8 * hh);
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) {
    const int n0 = 32 * ct + 16 * (g16 & 1) + 4 * (i16 & 3);
    toff_t[ct][0] = toff<C::C>(4 * hh + (i16 >> 2), n0);
    toff_t[ct][1] = toff<C::C>(8 + 4 * hh + (i16 >> 2), n0);
  }

  f32x16 acc[C::CT];
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) acc[ct] = f32x16{};

  auto compute = [&](int kt, int stage) {
    const bf16* Ks = smem + stage * C::STAGE;
    const bf16* Vs = Ks + C::TILE;
    const int kbase = kt * C::BN;
    if (CAUSAL && kbase > wrow0 + 31) return;   // this wave's rows see none of the tile
    if (BLOCK && !mbit(my_mr, kt)) return;     // nor of a tile its mask row drops

    f32x16 s[C::NT], dp[C::NT];
#pragma unroll
    for (int st = 0; st < C::NT; ++st) {
      s[st] = f32x16{};
      dp[st] = f32x16{};
    }
#pragma unroll
    for (int kk = 0; kk < C::KS; ++kk) {
#pragma unroll
      for (int st = 0; st < C::NT; ++st) {
        const bf16x8 a = lds_b128(Ks + roff[kk] + 32 * st * D);
        s[st] = mfma32(a, qf[kk], s[st]);
        const bf16x8 b = lds_b128(Vs + roff[kk] + 32 * st * D);
        dp[st] = mfma32(b, gf[kk], dp[st]);
      }
    }
    // s[st][v]: key kbase + 32*st + 8*(v/4) + 4*hh + v%4, query row qrow. Masked
    // scores become -inf (one uniform branch per tile), so P and dS are 0 there.
    const bool edge = (CAUSAL && kbase + C::BN - 1 > wrow0) || (kbase + C::BN > N);
    if (edge) {
#pragma unroll
      for (int st = 0; st < C::NT; ++st) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kbase + 32 * st + 8 * (v / 4) + 4 * hh + (v % 4);
          if ((CAUSAL && key > qrow) || key >= N) s[st][v] = -INFINITY;
        }
      }
    }
    bf16x8 dsk[2 * C::NT];
#pragma unroll
    for (int st = 0; st < C::NT; ++st) {
      float ds[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float pe = fast_exp2(__builtin_fmaf(s[st][v], p.sl2, -lrow));
        ds[v] = pe * (dp[st][v] - drow);
      }
      dsk[2 * st] = to_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
      dsk[2 * st + 1] = to_bf16x8(ds[8], ds[9], ds[10], ds[11], ds[12], ds[13], ds[14], ds[15]);
    }
    // dQ^T[c][i] += sum_j K[j][c] dS^T[j][i]; k-slots follow the accumulator's key
    // order (lane half hh: keys 4hh..4hh+3 and 8+4hh..8+4hh+3 of each 16).
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
#pragma unroll
      for (int ks = 0; ks < 2 * C::NT; ++ks) {
        const i16x4 lo = lds_tr(Ks + toff_t[ct][0] + 16 * ks * D);
        const i16x4 hi = lds_tr(Ks + toff_t[ct][1] + 16 * ks * D);
        acc[ct] = mfma32(cat(lo, hi), dsk[ks], acc[ct]);
      }
    }
  };

  // Ring of NSTAGE stages, as in the forward kernel.
  int kt = 0;
  if (BLOCK && kt < kt_end && !kept(kt)) kt = next_kept(kt);
  int kn = kt < kt_end ? next_kept(kt) : kt_end;
  if (kt < kt_end) issue(kt, 0);
  // The row operand loads above must be complete before the loop: a wait for
  // them inside the loop would also wait for the tiles in flight.
  wait_vmcnt<0>();
  if (C::NSTAGE == 3 && kn < kt_end) issue(kn, 1);
  int stage = 0;
  // At d=64 three workgroups share a CU: keep them at one pace.
  const int kt_first = kt;
  int prio_set = -1;
  while (kt < kt_end) {
    const int knn = kn < kt_end ? next_kept(kn) : kt_end;
    if (D == 64) prio_by_progress(kt - kt_first, kt_end - kt_first, prio_set);
    if (C::NSTAGE == 3 && kn < kt_end)
      wait_vmcnt<C::LPT>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    if (C::NSTAGE == 3) {
      if (knn < kt_end) issue(knn, stage == 0 ? 2 : stage - 1);
    } else {
      if (kn < kt_end) issue(kn, stage ^ 1);
    }
    compute(kt, stage);
    stage = stage == C::NSTAGE - 1 ? 0 : stage + 1;
    kt = kn;
    kn = knn;
  }

  // acc[ct][v] = dQ[qrow][32*ct + 8*(v/4) + 4*hh + v%4] / scale.
  if (qrow < N) {
    bf16* drow_out = p.dq + head + (int64_t)qrow * D;
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = 32 * ct + 8 * g + 4 * hh;
        *reinterpret_cast<bf16x4*>(drow_out + c) =
            to_bf16x4(acc[ct][4 * g] * p.scale, acc[ct][4 * g + 1] * p.scale,
                      acc[ct][4 * g + 2] * p.scale, acc[ct][4 * g + 3] * p.scale);
      }
    }
  }
}

template <int D, bool CAUSAL, bool BLOCK>
hipError_t launch_one(const BwdArgs& a, hipStream_t stream) {
  using C = DqCfg<D, BLOCK>;
  DqParams p;
  p.q = static_cast<const bf16*>(a.q);
  p.k = static_cast<const bf16*>(a.k);
  p.v = static_cast<const bf16*>(a.v);
  p.dout = static_cast<const bf16*>(a.dout);
  p.l2 = a.l2;
  p.dvec = a.dvec;
  p.dq = static_cast<bf16*>(a.dq);
  p.BH = a.BH;
  p.N = a.N;
  p.Np = a.Np;
  p.n_row_blocks = (a.N + C::BM - 1) / C::BM;
  p.sl2 = a.scale * kLog2e;
  p.scale = a.scale;
  p.blocks = a.mask.blocks;
  p.blocks_bh_stride = a.mask.bh_stride;
  p.nb = a.mask.nb;
  const dim3 grid((unsigned)p.n_row_blocks * (unsigned)a.BH);
  hipLaunchKernelGGL((fa_bwd_dq_kernel<D, CAUSAL, BLOCK>), grid, dim3(C::THREADS), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dq_d(const BwdArgs& a, hipStream_t stream) {
  const bool blk = a.mask.blocks != nullptr;
  if (a.mask.causal)
    return blk ? launch_one<D, true, true>(a, stream) : launch_one<D, true, false>(a, stream);
  return blk ? launch_one<D, false, true>(a, stream) : launch_one<D, false, false>(a, stream);
}

}  // namespace

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream) {
  return a.d == 128 ? launch_dq_d<128>(a, stream) : launch_dq_d<64>(a, stream);
}

}  // namespace fa

// Forward attention for gfx950: O = softmax(scale Q K^T, masked) V and LSE.
//
// Follows the tiled forward with the online softmax (lecture summary on
// FlashAttention v1, sections 3.1-3.3) in the FlashAttention-2 loop order
// (FlashAttention-2 overview, forward pass): each workgroup owns one block of
// query rows of one (batch, head) and sweeps the key/value tiles, so no
// workgroup talks to another. Inside the workgroup every wave owns 32 query
// rows (the "split-Q" partition of the same overview): K/V tiles are shared
// through LDS, and no partial results are exchanged between waves. Tiles reach
// LDS by direct global->LDS loads (no staging registers), up to three tiles
// in flight, in the swizzled layout of fa_common.hpp.
//
// Per wave and K/V tile (BN keys):
//   S^T = K_tile Q_wave^T       MFMA 32x32x16, K read from LDS, Q^T held in VGPRs.
//                               The transposed product puts one query row in each
//                               lane (the same row in lanes l and l+32), so a row
//                               max is a lane-local max plus one cross-half swap.
//   P^T = 2^(S^T * scale*log2e - m)                 (m: the row's reference max)
//   l  += rowsum(P^T)           fp32, before P is rounded to bf16: gives the LSE
//   lb += rowsum(bf16(P^T))     bf16 dot products: the sum of exactly the
//                               probabilities the next product consumes, used to
//                               normalise O (then O is a convex combination of V
//                               rows even when one probability dominates)
//   O^T += V_tile^T P^T         MFMA, P^T straight from registers as the B
//                               operand; V^T via the transposing LDS read.
// The reference max m only moves when a tile's row max exceeds it by more than
// 2^8 (in probability terms); then O^T and l are rescaled by 2^(m_old - m_new).
// Between moves P stays below 2^8, far inside fp32/bf16 range, and because O
// and l always share the same m the final O / l is the same exact quantity as
// the per-tile rescaled recurrence of the lecture (section 3.2), with the
// rescale of O skipped on almost every tile. Normalisation by l happens once
// at the end (the reading of the FlashAttention-2 "fewer non-matmul
// operations" change), and LSE = ln2 * (m + log2 l) is written instead of
// (m, l).
#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {
namespace {

template <int D, bool BLOCK>
struct FwdCfg {
  // A block mask works on 128-row blocks: masked launches use 128-row
  // workgroups so that every wave of a workgroup keeps the same tiles. At d=64
  // every launch does, with a two-stage ring: the kernel then fits in 128
  // registers and 32 KiB, so four workgroups share a CU (four waves per SIMD)
  // and each tile barrier waits for four waves instead of eight.
  static constexpr int WAVES = (BLOCK || D == 64) ? 4 : 8;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BM = 32 * WAVES;           // query rows per workgroup
  static constexpr int BN = 64;                   // keys per K/V tile
  static constexpr int C = D / 8;                 // 16-byte chunks per tile row
  static constexpr int KS = D / 16;               // MFMA k-steps over the head dim
  static constexpr int NT = BN / 32;              // 32-key sub-tiles of S^T
  static constexpr int CT = D / 32;               // 32-column sub-tiles of O^T
  static constexpr int TILE = BN * D;             // elements per K or V tile (swizzled, unpadded)
  static constexpr int STAGE = 2 * TILE;          // K tile, V tile
  // Tiles in flight: three (two loading while one is used) for the 8-wave
  // workgroups; two for the 4-wave ones, whose LDS must hold several
  // workgroups per CU.
  static constexpr int NSTAGE = (BLOCK || D == 64) ? 2 : 3;
  static constexpr int SLOTS = BN * C / 64;       // 1 KiB direct-load slots per tile
  static constexpr int SPW = SLOTS / WAVES;       // ... per wave
  static constexpr int LPT = 2 * SPW;             // direct loads per thread per K+V tile
  static constexpr int NMR = BM / 128;            // block-mask rows per workgroup
  // K operands are read this many k-steps ahead of their products. At d=64 a
  // deeper lead would push the register count past 128 and halve occupancy.
  static constexpr int KPRE = D == 128 ? 4 : 1;
  static_assert(SLOTS % WAVES == 0, "tile slots split evenly over waves");
};

// Reference-max moves happen only when a row max exceeds it by more than this
// (log2 units): probabilities stay <= 2^8 between moves.
constexpr float kRescaleThreshold = 8.0f;

struct FwdParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  int BH;
  int N;
  int n_row_blocks;
  float sl2;  // scale * log2(e)
  const uint8_t* blocks;
  int64_t blocks_bh_stride;
  int nb;
};

template <int D, bool CAUSAL, bool BLOCK>
__global__ __launch_bounds__((FwdCfg<D, BLOCK>::THREADS)) __attribute__((amdgpu_waves_per_eu(2)))
void fa_fwd_kernel(FwdParams p) {
  using C = FwdCfg<D, BLOCK>;
  __shared__ __attribute__((aligned(16))) bf16 smem[C::NSTAGE * C::STAGE];  // [stage][K, V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;     // which half of the wave
  const int g16 = lane >> 4;    // 16-lane group (transposing reads)
  const int i16 = lane & 15;

  // Largest row blocks first: under a causal mask they carry the most tiles.
  const WgCoord wc = wg_coord<BLOCK>(blockIdx.x, p.BH, p.n_row_blocks);
  const int bh = wc.bh;
  const int rb = p.n_row_blocks - 1 - wc.blk;   // largest causal row blocks first
  const int N = p.N;
  const int64_t head = (int64_t)bh * N * D;
  const bf16* __restrict__ Qh = p.q + head;
  const bf16* __restrict__ Kh = p.k + head;
  const bf16* __restrict__ Vh = p.v + head;
  const int row0 = rb * C::BM;
  const int wrow0 = row0 + 32 * wave;   // first row of this wave
  const int qrow = wrow0 + l32;         // this lane's query row

  int kt_end = (N + C::BN - 1) / C::BN;
  if (CAUSAL) kt_end = min(kt_end, (row0 + C::BM - 1) / C::BN + 1);

  // Block mask: the workgroup's rows span two 128-row mask rows; their bits go
  // to LDS once (so the tile loop reads no global memory besides the tiles). A
  // tile is loaded if either row keeps it; a wave skips tiles its row drops.
  __shared__ uint32_t mbits[BLOCK ? C::NMR * kMaskWords : 1];
  const int mr0 = row0 / 128;
  const int my_mr = wrow0 / 128 - mr0;   // this wave's mask row: 0 or 1
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

  // Q^T operand: lane holds Q[qrow][16*kk + 8*hh .. +7] for every k-step.
  bf16x8 qf[C::KS];
#pragma unroll
  for (int kk = 0; kk < C::KS; ++kk) {
    if (qrow < N)
      qf[kk] = *reinterpret_cast<const bf16x8*>(Qh + (int64_t)qrow * D + 16 * kk + 8 * hh);
    else
      qf[kk] = bf16x8{};
  }

  // Direct global->LDS loads of one K/V tile into a stage; keys past N are
  // clamped to N-1 (they are masked, any valid row will do).
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
      // the ragged last tile: rows past N clamped to the last row
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

  // Lane offsets inside a K / V tile. The swizzle term depends only on the lane
  // and on the k-step (K) or column sub-tile (V); the remaining steps (32-key
  // sub-tile of K, 16-key step of V) add compile-time constants.
  int koff[C::KS], voff[C::CT][2];
#pragma unroll
  for (int kk = 0; kk < C::KS; ++kk) koff[kk] = toff<C::C>(l32, 16 * kk + 8 * hh);
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) {
    const int n0 = 32 * ct + 16 * (g16 & 1) + 4 * (i16 & 3);
    voff[ct][0] = toff<C::C>(4 * hh + (i16 >> 2), n0);
    voff[ct][1] = toff<C::C>(8 + 4 * hh + (i16 >> 2), n0);
  }

  f32x16 oacc[C::CT];
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) oacc[ct] = f32x16{};
  float m_run = -INFINITY;  // reference max of scaled scores, log2 domain
  float l_run = 0.f;        // denominator relative to m_run, this lane half's keys only
  float lb_run = 0.f;       // the same sum over the bf16-rounded probabilities
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};

  auto compute = [&](int kt, int stage) {
    const bf16* Ks = smem + stage * C::STAGE;
    const bf16* Vs = Ks + C::TILE;
    const int kbase = kt * C::BN;
    // Under the causal mask a wave whose rows all precede this tile sees none of
    // it; under the block mask a wave skips the tiles its mask row drops.
    if (CAUSAL && kbase > wrow0 + 31) return;
    if (BLOCK && !mbit(my_mr, kt)) return;

    f32x16 s[C::NT];
#pragma unroll
    for (int st = 0; st < C::NT; ++st) s[st] = f32x16{};
    // The reads of k-step kk + KPRE are issued behind the products of k-step kk
    // (a rotating set of KPRE + 1 operand registers), so every product finds
    // its operand loaded instead of waiting out an LDS round trip.
    constexpr int KPRE = C::KPRE;
    bf16x8 ka[KPRE + 1][C::NT];
#pragma unroll
    for (int kk = 0; kk < KPRE; ++kk)
#pragma unroll
      for (int st = 0; st < C::NT; ++st) ka[kk][st] = lds_b128(Ks + koff[kk] + 32 * st * D);
    if (KPRE > 1) __builtin_amdgcn_sched_group_barrier(0x100, C::NT * KPRE, 0);   // DS reads
#pragma unroll
    for (int kk = 0; kk < C::KS; ++kk) {
#pragma unroll
      for (int st = 0; st < C::NT; ++st) s[st] = mfma32(ka[kk % (KPRE + 1)][st], qf[kk], s[st]);
      if (kk + KPRE < C::KS) {
#pragma unroll
        for (int st = 0; st < C::NT; ++st)
          ka[(kk + KPRE) % (KPRE + 1)][st] = lds_b128(Ks + koff[kk + KPRE] + 32 * st * D);
      }
      if (KPRE > 1) {
        __builtin_amdgcn_sched_group_barrier(0x008, C::NT, 0);                   // MFMA
        if (kk + KPRE < C::KS) __builtin_amdgcn_sched_group_barrier(0x100, C::NT, 0);
      }
    }
    // s[st][v] is the score of query qrow and key kbase + 32*st + 8*(v/4) + 4*hh + v%4.
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
    // Row max as two chains of three-input maxima (v_max3_f32: two scores per step).
    float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
    for (int st = 0; st < C::NT; ++st) {
#pragma unroll
      for (int v = 0; v < 16; v += 4) {
        m0 = fmaxf(fmaxf(m0, s[st][v]), s[st][v + 1]);
        m1 = fmaxf(fmaxf(m1, s[st][v + 2]), s[st][v + 3]);
      }
    }
    float mx = fmaxf(m0, m1);
    mx = fmaxf(mx, swap_halves(mx)) * p.sl2;
    // Move the reference max only if some row of this wave outgrew it by > 2^8.
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleThreshold) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
      lb_run *= alpha;
#pragma unroll
      for (int ct = 0; ct < C::CT; ++ct) oacc[ct] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;  // nothing visible yet: all P are 0

    bf16x8 pk[2 * C::NT];
    float rs = 0.f;
#pragma unroll
    for (int st = 0; st < C::NT; ++st) {
      float e[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        e[v] = fast_exp2(__builtin_fmaf(s[st][v], p.sl2, -m_use));
        rs += e[v];
      }
      pk[2 * st] = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
      pk[2 * st + 1] = to_bf16x8(e[8], e[9], e[10], e[11], e[12], e[13], e[14], e[15]);
    }
    l_run += rs;
#pragma unroll
    for (int j = 0; j < 2 * C::NT; ++j) {
#pragma unroll
      for (int h = 0; h < 4; ++h)
        lb_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pk[j][2 * h], pk[j][2 * h + 1]}, ones,
                                                 lb_run, false);
    }

    // O^T[c][i] += sum_j V[j][c] P^T[j][i]. MFMA k-slot order within each 16 keys
    // follows the accumulator layout of S^T: lane half hh holds keys 4hh..4hh+3 and
    // 8+4hh..8+4hh+3, so the V^T operand is read as those two groups of four rows.
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
#pragma unroll
      for (int ks = 0; ks < 2 * C::NT; ++ks) {
        const i16x4 lo = lds_tr(Vs + voff[ct][0] + 16 * ks * D);
        const i16x4 hi = lds_tr(Vs + voff[ct][1] + 16 * ks * D);
        oacc[ct] = mfma32(cat(lo, hi), pk[ks], oacc[ct]);
      }
    }
  };

  // Ring of NSTAGE stages: while tile i is computed, tiles i+1 (and i+2 with
  // three stages) are loading. At the top of each step a thread waits for its
  // own loads of tile i; the barrier then publishes every thread's loads and
  // guarantees that no wave still reads the stage the next load overwrites.
  int kt = 0;
  if (BLOCK && kt < kt_end && !kept(kt)) kt = next_kept(kt);
  int kn = kt < kt_end ? next_kept(kt) : kt_end;
  if (kt < kt_end) issue(kt, 0);
  // The row operand loads above must be complete before the loop: a wait for
  // them inside the loop would also wait for the tiles in flight.
  wait_vmcnt<0>();
  if (C::NSTAGE == 3 && kn < kt_end) issue(kn, 1);
  int stage = 0;
  // At d=64 four workgroups share a CU: keep them at one pace.
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

  // Epilogue: combine the two lane halves' denominators, normalise once.
  const float l_tot = l_run + swap_halves(l_run);
  const float lb_tot = lb_run + swap_halves(lb_run);
  const float inv = lb_tot > 0.f ? fast_rcp(lb_tot) : 0.f;
  if (qrow < N) {
    bf16* orow = p.o + head + (int64_t)qrow * D;
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = 32 * ct + 8 * g + 4 * hh;
        *reinterpret_cast<bf16x4*>(orow + c) =
            to_bf16x4(oacc[ct][4 * g] * inv, oacc[ct][4 * g + 1] * inv,
                      oacc[ct][4 * g + 2] * inv, oacc[ct][4 * g + 3] * inv);
      }
    }
    if (hh == 0)
      p.lse[(int64_t)bh * N + qrow] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL, bool BLOCK>
hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
  using C = FwdCfg<D, BLOCK>;
  FwdParams p;
  p.q = static_cast<const bf16*>(a.q);
  p.k = static_cast<const bf16*>(a.k);
  p.v = static_cast<const bf16*>(a.v);
  p.o = static_cast<bf16*>(a.o);
  p.lse = a.lse;
  p.BH = a.BH;
  p.N = a.N;
  p.n_row_blocks = (a.N + C::BM - 1) / C::BM;
  p.sl2 = a.scale * kLog2e;
  p.blocks = a.mask.blocks;
  p.blocks_bh_stride = a.mask.bh_stride;
  p.nb = a.mask.nb;
  const dim3 grid((unsigned)p.n_row_blocks * (unsigned)a.BH);
  hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, BLOCK>), grid, dim3(C::THREADS), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  const bool blk = a.mask.blocks != nullptr;
  if (a.mask.causal)
    return blk ? launch_one<D, true, true>(a, stream) : launch_one<D, true, false>(a, stream);
  return blk ? launch_one<D, false, true>(a, stream) : launch_one<D, false, false>(a, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  return a.d == 128 ? launch_d<128>(a, stream) : launch_d<64>(a, stream);
}

}  // namespace fa

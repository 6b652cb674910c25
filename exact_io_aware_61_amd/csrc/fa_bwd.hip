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
// Preprocess kernel (once per call): D_i and L2_i = LSE_i log2(e) for every row,
// into arrays padded per head to Np rows (Np = N rounded up to 128). Rows past
// N, and rows with no visible key (LSE = -inf), get L2 = +inf and D = 0: their
// probabilities recompute to exactly 0 with no test in the kernels.
//
// Two dK/dV kernels share the arithmetic below and differ in where K and V sit.
// At d = 64 (fa_bwd_dkdv_kernel), a workgroup of 4 waves = 128 keys; wave w
// owns keys key0 + 32w .. +31, keeps their K and V rows in VGPRs and their
// dK^T, dV^T accumulators on chip; two workgroups share a CU. At d = 128
// (fa_bwd_dkdv8_kernel, further down) those registers would leave room for one
// wave per SIMD only, so K and V are read from LDS and 8 waves split the work
// (two per SIMD). Per block of 64 query rows (the Q and dO tiles and the rows'
// L2 and D reach LDS by direct global->LDS loads), per wave and 32-row sub-tile:
//   S  = Q K_w^T, dP = dO V_w^T   MFMA 32x32x16, Q/dO rows by 16-byte LDS reads;
//                                 each lane holds one key column.
//   P  = 2^(S scale log2e - L2_i), dS = P o (dP - D_i)
//   dV_w^T += dO^T P, dK_w^T += Q^T dS
//                                 P and dS straight from registers as the B
//                                 operand; dO^T and Q^T by transposing LDS reads
//                                 of the same tiles, taking in each 16 rows the
//                                 order (4h..4h+3, 8+4h..8+4h+3) in which lane
//                                 half h holds P.
#include <type_traits>

#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {
namespace {

// ------------------------------------------------------------------------------------------------
// Preprocess: D_i = sum_c dO_ic O_ic and L2_i = LSE_i log2(e), padded as above.

constexpr int kPreRows = 64;   // rows per preprocess workgroup

struct PreParams {
  const bf16* o;
  const bf16* dout;
  const float* lse;
  float* dvec;   // [BH][Np]
  float* l2;     // [BH][Np]
  int N;
  int Np;
};

template <int D>
__global__ __launch_bounds__(256) void fa_bwd_pre_kernel(PreParams p) {
  constexpr int LPR = D / 8;                  // 16-byte chunks (lanes) per row
  constexpr int CH = kPreRows * LPR / 256;    // chunks per thread
  const int nrb = p.Np / kPreRows;
  const int bh = blockIdx.x / nrb;
  const int row0 = (blockIdx.x % nrb) * kPreRows;
  const int N = p.N;
  const int tid = threadIdx.x;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int id = tid + 256 * c;
    const int r = id / LPR;
    const int part = id % LPR;
    const int row = row0 + r;
    float acc = 0.f;
    if (row < N) {
      const int64_t off = ((int64_t)bh * N + row) * D + 8 * part;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(p.o + off);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(p.dout + off);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)b[e];
    }
    // The LPR lanes of one row are consecutive: reduce across them.
#pragma unroll
    for (int sh = LPR / 2; sh > 0; sh >>= 1) acc += __shfl_xor(acc, sh);
    if (part == 0) {
      const float lse = row < N ? p.lse[(int64_t)bh * N + row] : -INFINITY;
      const bool live = lse != -INFINITY;
      p.dvec[(int64_t)bh * p.Np + row] = live ? acc : 0.f;
      p.l2[(int64_t)bh * p.Np + row] = live ? lse * kLog2e : INFINITY;
    }
  }
}

// ------------------------------------------------------------------------------------------------
// dK/dV kernel.

template <int D>
struct BwdCfg {
  static constexpr int WAVES = 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BN = 32 * WAVES;           // keys per workgroup (= block-mask granularity)
  // Query rows per block: 64 keeps the four-stage ring at 68 KiB at d=64, so
  // two workgroups share a CU and each SIMD runs two waves (one wave's softmax
  // under the other's products).
  static constexpr int BM = 64;
  static constexpr int IT = BM / 32;              // 32-row sub-tiles
  static constexpr int KS = D / 16;               // 16-column MFMA k-steps over the head dim
  static constexpr int CT = D / 32;               // 32-column sub-tiles of the head dim
  static constexpr int C = D / 8;                 // 16-byte chunks per tile row
  static constexpr int TILE = BM * D;             // elements of a Q or dO tile (swizzled)
  static constexpr int STAGE = 2 * TILE + 2 * BM * 2;  // + the L2 and D rows (floats)
  static constexpr int NSTAGE = 4;                // one block in use, three loading
  static constexpr int SLOTS = TILE / 512;        // 1 KiB slots per tile
  static constexpr int SPW = SLOTS / WAVES;
  static constexpr int SROWS = BM / 64;           // 256-byte loads per row array
  static_assert(SLOTS % WAVES == 0, "tile slots split evenly over waves");
  static_assert(kBwdRowPad % BM == 0, "row padding covers whole row blocks");
  static_assert(2 * SROWS <= WAVES, "at most one row-array load per wave");
};

struct BwdParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* dout;
  const float* l2;
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

// dK/dV kernel at d = 64 (fa_bwd_dkdv8_kernel below serves d = 128).
template <int D, bool CAUSAL, bool BLOCK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dkdv_kernel(BwdParams p) {
  static_assert(D == 64, "d = 128 runs fa_bwd_dkdv8_kernel");
  using C = BwdCfg<D>;
  // [stage][Q tile, dO tile, L2 rows, D rows]
  __shared__ __attribute__((aligned(16))) bf16 smem[C::NSTAGE * C::STAGE];
  __shared__ uint32_t mbits[BLOCK ? kMaskWords : 1];
  static_assert(C::NSTAGE * C::STAGE * 2 + (BLOCK ? kMaskWords * 4 : 4) <= 160 * 1024,
                "LDS budget");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int g16 = lane >> 4;
  const int i16 = lane & 15;

  const WgCoord wc = wg_coord<BLOCK>(blockIdx.x, p.BH, (p.N + C::BN - 1) / C::BN);
  const int bh = wc.bh;
  const int kb = wc.blk;   // key block; block 0 carries the most rows under causal
  const int N = p.N;
  const int64_t head = (int64_t)bh * N * D;
  const bf16* __restrict__ Qh = p.q + head;
  const bf16* __restrict__ Kh = p.k + head;
  const bf16* __restrict__ Vh = p.v + head;
  const bf16* __restrict__ dOh = p.dout + head;
  const float* __restrict__ L2h = p.l2 + (int64_t)bh * p.Np;
  const float* __restrict__ Dh = p.dvec + (int64_t)bh * p.Np;

  const int key0 = kb * C::BN;
  const int mykey = key0 + 32 * wave + l32;   // this lane's key column

  // Block mask: this workgroup's key block is one mask column; its bits go to
  // LDS once, so the row-block loop reads no global memory besides its tiles.
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
  }

  // S / dP B operands: K and V rows of this lane's key, k = head-dim chunks.
  // Keys past N are clamped (masked below).
  bf16x8 kf[C::KS], vf[C::KS];
  {
    const int key = min(mykey, N - 1);
#pragma unroll
    for (int kk = 0; kk < C::KS; ++kk) {
      kf[kk] = *reinterpret_cast<const bf16x8*>(Kh + (int64_t)key * D + 16 * kk + 8 * hh);
      vf[kk] = *reinterpret_cast<const bf16x8*>(Vh + (int64_t)key * D + 16 * kk + 8 * hh);
    }
  }
  // These loads (and the mask reads) complete before the loop: a wait for them
  // inside it would also wait for the row blocks in flight.
  wait_vmcnt<0>();
  if (BLOCK) __syncthreads();

  // Lane offsets inside a tile: 16-byte row reads (S, dP operands) and the
  // transposing reads (dV, dK operands); sub-tile steps add constants.
  int qoff[C::KS], troff[C::CT][2];
#pragma unroll
  for (int kk = 0; kk < C::KS; ++kk) qoff[kk] = toff<C::C>(l32, 16 * kk + 8 * hh);
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) {
    const int n0 = 32 * ct + 16 * (g16 & 1) + 4 * (i16 & 3);
    troff[ct][0] = toff<C::C>(4 * hh + (i16 >> 2), n0);
    troff[ct][1] = toff<C::C>(8 + 4 * hh + (i16 >> 2), n0);
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
    const int b = (rb * C::BM) / 128;
    return (mbits[b >> 5] >> (b & 31)) & 1u;
  };
  auto next_kept = [&](int rb) -> int {
    ++rb;
    while (rb < n_rb && !kept(rb)) ++rb;
    return rb;
  };

  // Direct global->LDS loads of one row block into a stage: the Q and dO tiles
  // (rows past N clamped; their L2 is +inf) and the block's L2 and D rows, one
  // 256-byte load each by the first 2*SROWS waves.
  const bool row_loader = wave < 2 * C::SROWS;
  const int uwave = __builtin_amdgcn_readfirstlane(wave);   // uniform: scalar address math
  const uint32_t lds0 = lds_byte_addr(smem);
  uint32_t soff[C::SPW];   // byte offsets of this lane's chunks, the same for every block
#pragma unroll
  for (int i = 0; i < C::SPW; ++i) soff[i] = slot_offset<C::C>(wave + i * C::WAVES, lane, 2 * D);
  auto issue = [&](int rb, int stage) {
    const int row0 = rb * C::BM;
    bf16* Qs = smem + stage * C::STAGE;
    bf16* dOs = Qs + C::TILE;
    float* Rs = reinterpret_cast<float*>(dOs + C::TILE);
    if (row0 + C::BM <= N) {
      // whole block inside the sequence: scalar base, fixed lane offsets
      const bf16* qb = Qh + (int64_t)row0 * D;
      const bf16* gb = dOh + (int64_t)row0 * D;
      const uint32_t qdst = lds0 + 2u * (uint32_t)(stage * C::STAGE);
#pragma unroll
      for (int i = 0; i < C::SPW; ++i) {
        const uint32_t o = 2u * 512u * (uint32_t)(uwave + i * C::WAVES);
        dma16_s(soff[i], qb, qdst + o);
        dma16_s(soff[i], gb, qdst + 2u * C::TILE + o);
      }
    } else {
      // the ragged last block: rows past N clamped to the last row
#pragma unroll
      for (int i = 0; i < C::SPW; ++i) {
        const int slot = wave + i * C::WAVES;
        dma_slot<C::C>(Qs, slot, lane,
                       [&](int r) { return Qh + (int64_t)min(row0 + r, N - 1) * D; });
        dma_slot<C::C>(dOs, slot, lane,
                       [&](int r) { return dOh + (int64_t)min(row0 + r, N - 1) * D; });
      }
    }
    if (row_loader) {
      const int arr = wave / C::SROWS;   // 0: L2, 1: D
      const int part = wave % C::SROWS;
      const float* src = (arr == 0 ? L2h : Dh) + row0 + 64 * part + lane;
      dma4(src, Rs + arr * C::BM + 64 * part);
    }
  };

  // Software pipeline over 32-row sub-tiles (a second workgroup's wave shares
  // each SIMD and fills in while this one waits). At the start of a sub-tile
  // its Q/dO row operands are already in registers (read during the previous
  // sub-tile's dV/dK products); its transposed operands and row statistics
  // are read between its S/dP products, two reads per product; after the
  // softmax, the dV/dK products run with one read of the next sub-tile's rows
  // after each. Scheduling-group barriers pin that interleave (left alone, the
  // compiler pairs each read with the product that uses it, or bunches all the
  // reads, which overfills the LDS request queue of the four waves).
  bf16x8 qa[C::KS], ga[C::KS];
  auto read_rows = [&](int stage, int it) {
    const bf16* Qs = smem + stage * C::STAGE;
    const bf16* dOs = Qs + C::TILE;
#pragma unroll
    for (int kk = 0; kk < C::KS; ++kk) {
      qa[kk] = lds_b128(Qs + qoff[kk] + 32 * it * D);
      ga[kk] = lds_b128(dOs + qoff[kk] + 32 * it * D);
    }
  };

  // Ring of four stages. Loads run two to three blocks ahead: after the softmax
  // of the last sub-tile of block j each thread waits for its own loads of
  // block j+1 (loads complete in issue order, so it waits until no more than
  // the loads of the block after that are outstanding); the barrier then
  // publishes every thread's loads of block j+1 and guarantees that every wave
  // has finished block j-1, whose stage the loads of block j+3 then take.
  auto wait_block = [&](int later) {   // later: blocks issued after the awaited one (0 or 1)
    constexpr int A = 2 * C::SPW;       // loads per block, tile-only waves
    constexpr int B = 2 * C::SPW + 1;   // loads per block, row-array loaders
    if (row_loader) {
      if (later == 1) wait_vmcnt<B>();
      else wait_vmcnt<0>();
    } else {
      if (later == 1) wait_vmcnt<A>();
      else wait_vmcnt<0>();
    }
  };
  int rb = rb_begin;
  if (rb < n_rb && !kept(rb)) rb = next_kept(rb);
  int r1 = rb < n_rb ? next_kept(rb) : n_rb;
  int r2 = r1 < n_rb ? next_kept(r1) : n_rb;
  if (rb < n_rb) issue(rb, 0);
  if (r1 < n_rb) issue(r1, 1);
  if (r2 < n_rb) issue(r2, 2);
  int stage = 0;
  if (rb < n_rb) {
    // block rb: wait until only the loads of r1 and r2 are outstanding
    const int later = (r1 < n_rb ? 1 : 0) + (r2 < n_rb ? 1 : 0);
    constexpr int A = 2 * C::SPW, B = 2 * C::SPW + 1;
    if (row_loader) {
      if (later == 2) wait_vmcnt<2 * B>();
      else if (later == 1) wait_vmcnt<B>();
      else wait_vmcnt<0>();
    } else {
      if (later == 2) wait_vmcnt<2 * A>();
      else if (later == 1) wait_vmcnt<A>();
      else wait_vmcnt<0>();
    }
    __syncthreads();
    read_rows(0, 0);
  }

  // One row block. EDGE: the block has pairs to mask (causal diagonal, keys
  // past N); interior blocks are compiled without any masking code.
  auto block = [&](auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const bf16* Qs = smem + stage * C::STAGE;
    const bf16* dOs = Qs + C::TILE;
    const float* Ls = reinterpret_cast<const float*>(dOs + C::TILE);
    const float* Ds = Ls + C::BM;
    const int row0 = rb * C::BM;
#pragma unroll
    for (int it = 0; it < C::IT; ++it) {
      // Region A: this sub-tile's transposed operands and row statistics are
      // read while its S/dP products run (two reads per product).
      bf16x8 ota[C::CT][2], qta[C::CT][2];
      f32x4 l4[4], d4[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int rl = 32 * it + 8 * g + 4 * hh;
        l4[g] = *reinterpret_cast<const f32x4*>(Ls + rl);
        d4[g] = *reinterpret_cast<const f32x4*>(Ds + rl);
      }
#pragma unroll
      for (int ct = 0; ct < C::CT; ++ct) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int ro = (32 * it + 16 * h) * D;
          ota[ct][h] = cat(lds_tr(dOs + troff[ct][0] + ro), lds_tr(dOs + troff[ct][1] + ro));
          qta[ct][h] = cat(lds_tr(Qs + troff[ct][0] + ro), lds_tr(Qs + troff[ct][1] + ro));
        }
      }
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < C::KS; ++kk) {
        s = mfma32(qa[kk], kf[kk], s);
        dp = mfma32(ga[kk], vf[kk], dp);
      }
      {
        // 8 reads first, then the rest two by two between the products
        constexpr int NR = 8 * C::CT + 8;          // reads in this region
        constexpr int NM = 2 * C::KS;              // products in this region
        constexpr int PER = (NR - 8 + NM - 1) / NM;
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // 0x100: LDS reads
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 0x008: MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, PER, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // Region B: softmax.
      float pv[16], dsv[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int v = 4 * g + r;
          float pe = fast_exp2(__builtin_fmaf(s[v], p.sl2, -l4[g][r]));
          if (EDGE) {
            const int row = row0 + 32 * it + 8 * g + 4 * hh + r;
            if ((CAUSAL && mykey > row) || mykey >= N) pe = 0.f;
          }
          pv[v] = pe;
          dsv[v] = pe * (dp[v] - d4[g][r]);
        }
      }
      bf16x8 pk[2], dsk[2];
      pk[0] = to_bf16x8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
      pk[1] = to_bf16x8(pv[8], pv[9], pv[10], pv[11], pv[12], pv[13], pv[14], pv[15]);
      dsk[0] = to_bf16x8(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
      dsk[1] = to_bf16x8(dsv[8], dsv[9], dsv[10], dsv[11], dsv[12], dsv[13], dsv[14], dsv[15]);
      // Block boundary: publish the next block before its rows are read.
      bool more = true;
      int nstage = stage;
      if (it + 1 == C::IT) {
        const int r3 = r2 < n_rb ? next_kept(r2) : n_rb;
        more = r1 < n_rb;
        if (more) {
          wait_block(r2 < n_rb ? 1 : 0);
          __syncthreads();
          if (r3 < n_rb) issue(r3, (stage + 3) & 3);
        }
        nstage = (stage + 1) & 3;
        r1 = r2;
        r2 = r3;
      }
      __builtin_amdgcn_sched_barrier(0);
      // Region C: dV/dK products, interleaved with the next sub-tile's row reads.
#pragma unroll
      for (int ct = 0; ct < C::CT; ++ct) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          dv[ct] = mfma32(ota[ct][h], pk[h], dv[ct]);
          dk[ct] = mfma32(qta[ct][h], dsk[h], dk[ct]);
        }
      }
      read_rows(nstage, it + 1 < C::IT ? it + 1 : 0);   // after the last block: unused
      {
        // one read of the next sub-tile's rows after each product
        constexpr int NR = 2 * C::KS;
        constexpr int NM = 4 * C::CT;
        constexpr int PER = (NR + NM - 1) / NM;
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, PER, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    stage = (stage + 1) & 3;
  };
  // Blocks that need masking come first (the causal diagonal: rows below
  // key0 + BN - 1) or are all of them (the last key block when N is ragged);
  // the rest run a copy of the body without any masking code. rb advances to
  // the r1 the block leaves behind (r1 is shifted inside the block, so the
  // value to advance to is saved first).
  auto edge_block = [&](int b) {
    return (CAUSAL && b * C::BM < key0 + C::BN - 1) || key0 + C::BN > N;
  };
  // Two workgroups share a CU: keep them at one pace.
  int prio_set = -1;
  while (rb < n_rb && edge_block(rb)) {
    prio_by_progress(rb - rb_begin, n_rb - rb_begin, prio_set);
    const int nxt = r1;
    block(std::true_type{});
    rb = nxt;
  }
  while (rb < n_rb) {
    prio_by_progress(rb - rb_begin, n_rb - rb_begin, prio_set);
    const int nxt = r1;
    block(std::false_type{});
    rb = nxt;
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

// ------------------------------------------------------------------------------------------------
// dK/dV kernel at d = 128 with two waves per SIMD.
//
// A wave that keeps 32 keys' K and V rows and their fp32 dK/dV accumulators in
// registers needs more than half the register file at d = 128, so only one such
// wave fits per SIMD and every stall of its in-order instruction stream (the
// softmax, the burst of global->LDS loads at a block boundary, waits on LDS)
// leaves the matrix unit idle. Here the workgroup's K and V tiles (128 keys)
// sit in LDS instead, read as MFMA operands like the Q and dO rows, and the
// workgroup has 8 waves: wave w owns keys 32 (w mod 4) .. +31 for the 32-row
// sub-tile w / 4 of every 64-row block, so each key group has two waves, each
// summing half of the row sub-tiles into its own accumulators. The two halves
// are added through LDS at the end, in a fixed order (bitwise reproducible).
// Q/dO tiles and row statistics arrive by direct global->LDS loads into a
// two-stage ring (one block ahead).
struct Dkdv8Cfg {
  static constexpr int D = 128;
  static constexpr int WAVES = 8;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BN = 128;                  // keys per workgroup
  static constexpr int BM = 64;                   // query rows per block
  static constexpr int KS = D / 16;
  static constexpr int CT = D / 32;
  static constexpr int C = D / 8;                 // 16-byte chunks per row
  static constexpr int KVROW = D + 8;             // K/V tile row pitch (elements): 272 bytes
  static constexpr int KVT = BN * KVROW;          // elements of the K or V tile
  static constexpr int TILE = BM * D;             // elements of a Q or dO tile
  static constexpr int STAGE = 2 * TILE + 2 * BM * 2;   // + L2 and D rows (floats)
  static constexpr int NSTAGE = 2;
  static constexpr int SLOTS = TILE / 512;        // 1 KiB slots per Q/dO tile
  static constexpr int LOADERS = 4;              // waves 4..7 issue the ring's loads
  static constexpr int SPW = SLOTS / LOADERS;
  static constexpr int KVCH = BN * C / THREADS;   // 16-byte K (and V) chunks per thread
  static_assert(SLOTS % LOADERS == 0 && (BN * C) % THREADS == 0, "loads split evenly");
  static_assert(kBwdRowPad % BM == 0, "row padding covers whole row blocks");
};

template <bool CAUSAL, bool BLOCK>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dkdv8_kernel(BwdParams p) {
  using C = Dkdv8Cfg;
  constexpr int D = C::D;
  // [K tile][V tile][stage 0][stage 1]; a stage is [Q tile, dO tile, L2 rows, D rows]
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * C::KVT + C::NSTAGE * C::STAGE];
  __shared__ uint32_t mbits[BLOCK ? kMaskWords : 1];
  static_assert((2 * C::KVT + C::NSTAGE * C::STAGE) * 2 + (BLOCK ? kMaskWords * 4 : 4) <=
                    160 * 1024,
                "LDS budget");
  static_assert(2 * C::KVT + C::NSTAGE * C::STAGE >= 4 * 64 * 128 * 2,
                "the accumulator exchange fits in the tile area");
  static_assert((C::KVROW * 2) % 16 == 0, "16-byte aligned K/V rows");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kq = wave & 3;     // key group: keys 32 kq .. +31 of the block
  const int par = wave >> 2;   // row sub-tile of every block this wave takes
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int g16 = lane >> 4;
  const int i16 = lane & 15;

  const WgCoord wc = wg_coord<BLOCK>(blockIdx.x, p.BH, (p.N + C::BN - 1) / C::BN);
  const int bh = wc.bh;
  const int kb = wc.blk;
  const int N = p.N;
  const int64_t head = (int64_t)bh * N * D;
  const bf16* __restrict__ Qh = p.q + head;
  const bf16* __restrict__ Kh = p.k + head;
  const bf16* __restrict__ Vh = p.v + head;
  const bf16* __restrict__ dOh = p.dout + head;
  const float* __restrict__ L2h = p.l2 + (int64_t)bh * p.Np;
  const float* __restrict__ Dh = p.dvec + (int64_t)bh * p.Np;

  const int key0 = kb * C::BN;
  const int mykey = key0 + 32 * kq + l32;

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
  }

  if (BLOCK) __syncthreads();   // the mask bits, before any wave reads them
  bf16* const Ks = smem;
  bf16* const Vs = smem + C::KVT;
  bf16* const ring = smem + 2 * C::KVT;

  // K and V tiles of the block's 128 keys (keys past N clamped; masked below),
  // loaded once through registers into rows padded to 272 bytes: the rows of a
  // 16-byte operand read then start 4 banks apart, which keeps the reads free
  // of bank conflicts with one base address and immediate offsets per lane
  // (the swizzle the direct loads need would cost a register per k-step).
#pragma unroll
  for (int i = 0; i < C::KVCH; ++i) {
    const int idx = tid + i * C::THREADS;
    const int r = idx / C::C, ch = idx % C::C;
    const int64_t src = (int64_t)min(key0 + r, N - 1) * D + 8 * ch;
    *reinterpret_cast<bf16x8*>(Ks + r * C::KVROW + 8 * ch) =
        *reinterpret_cast<const bf16x8*>(Kh + src);
    *reinterpret_cast<bf16x8*>(Vs + r * C::KVROW + 8 * ch) =
        *reinterpret_cast<const bf16x8*>(Vh + src);
  }

  // Lane offsets: B operands (this lane's key row of K and V), A operands (rows
  // of the wave's Q/dO sub-tile), transposing reads of the same sub-tile.
  const int kbase = (32 * kq + l32) * C::KVROW + 8 * hh;
  int qoff[C::KS], troff[C::CT][2];
#pragma unroll
  for (int kk = 0; kk < C::KS; ++kk) qoff[kk] = toff<C::C>(32 * par + l32, 16 * kk + 8 * hh);
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) {
    const int n0 = 32 * ct + 16 * (g16 & 1) + 4 * (i16 & 3);
    troff[ct][0] = toff<C::C>(32 * par + 4 * hh + (i16 >> 2), n0);
    troff[ct][1] = toff<C::C>(32 * par + 8 + 4 * hh + (i16 >> 2), n0);
  }

  f32x16 dk[C::CT], dv[C::CT];
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) {
    dk[ct] = f32x16{};
    dv[ct] = f32x16{};
  }

  const int n_rb = (N + C::BM - 1) / C::BM;
  const int rb_begin = CAUSAL ? key0 / C::BM : 0;
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

  // Only the waves of the second row sub-tile (4..7) issue the ring's loads:
  // while they wait on the load path after a barrier, the waves of the first
  // sub-tile on the same SIMDs already compute, so the two waves of a SIMD
  // leave the barrier a phase apart.
  const bool loader = __builtin_amdgcn_readfirstlane(wave) >= 4;   // uniform branch
  const int lw = wave - 4;
  const bool row_loader = lw == 0 || lw == 1;   // waves 4 and 5 load the L2 and D rows
  const int uwave = __builtin_amdgcn_readfirstlane(lw);
  const uint32_t ring0 = lds_byte_addr(ring);
  uint32_t soff[C::SPW];
#pragma unroll
  for (int i = 0; i < C::SPW; ++i) soff[i] = slot_offset<C::C>(lw + i * C::LOADERS, lane, 2 * D);
  auto issue = [&](int rb, int stage) {
    if (!loader) return;
    const int row0 = rb * C::BM;
    bf16* Qs = ring + stage * C::STAGE;
    bf16* dOs = Qs + C::TILE;
    float* Rs = reinterpret_cast<float*>(dOs + C::TILE);
    if (row0 + C::BM <= N) {
      const bf16* qb = Qh + (int64_t)row0 * D;
      const bf16* gb = dOh + (int64_t)row0 * D;
      const uint32_t qdst = ring0 + 2u * (uint32_t)(stage * C::STAGE);
#pragma unroll
      for (int i = 0; i < C::SPW; ++i) {
        const uint32_t o = 2u * 512u * (uint32_t)(uwave + i * C::LOADERS);
        dma16_s(soff[i], qb, qdst + o);
        dma16_s(soff[i], gb, qdst + 2u * C::TILE + o);
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::SPW; ++i) {
        const int slot = lw + i * C::LOADERS;
        dma_slot<C::C>(Qs, slot, lane,
                       [&](int r) { return Qh + (int64_t)min(row0 + r, N - 1) * D; });
        dma_slot<C::C>(dOs, slot, lane,
                       [&](int r) { return dOh + (int64_t)min(row0 + r, N - 1) * D; });
      }
    }
    if (row_loader) {
      const float* src = (lw == 0 ? L2h : Dh) + row0 + lane;
      dma4(src, Rs + lw * C::BM);
    }
  };

  // Double-buffered ring: at the top of block j every thread waits for all its
  // loads (block j's; block j+1 is not issued yet), the barrier publishes them
  // and guarantees every wave has finished block j-1, whose stage the loads of
  // block j+1 then take while block j is computed.
  int rb = rb_begin;
  if (rb < n_rb && !kept(rb)) rb = next_kept(rb);
  if (rb < n_rb) issue(rb, 0);
  int stage = 0;

  auto block = [&](auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const int nxt = next_kept(rb);
    wait_vmcnt<0>();
    __syncthreads();
    if (nxt < n_rb) issue(nxt, stage ^ 1);
    const bf16* Qs = ring + stage * C::STAGE;
    const bf16* dOs = Qs + C::TILE;
    const float* Ls = reinterpret_cast<const float*>(dOs + C::TILE);
    const float* Ds = Ls + C::BM;
    const int row0 = rb * C::BM + 32 * par;   // the wave's sub-tile
    // S = Q K^T and dP = dO V^T for the wave's 32 rows x 32 keys.
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < C::KS; ++kk) {
      s = mfma32(lds_b128(Qs + qoff[kk]), lds_b128(Ks + kbase + 16 * kk), s);
      dp = mfma32(lds_b128(dOs + qoff[kk]), lds_b128(Vs + kbase + 16 * kk), dp);
    }
    float pv[16], dsv[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int rl = 32 * par + 8 * g + 4 * hh;
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(Ls + rl);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(Ds + rl);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = 4 * g + r;
        float pe = fast_exp2(__builtin_fmaf(s[v], p.sl2, -l4[r]));
        if (EDGE) {
          const int row = row0 + 8 * g + 4 * hh + r;
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
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ro = 16 * h * D;
        const bf16x8 ota = cat(lds_tr(dOs + troff[ct][0] + ro), lds_tr(dOs + troff[ct][1] + ro));
        const bf16x8 qta = cat(lds_tr(Qs + troff[ct][0] + ro), lds_tr(Qs + troff[ct][1] + ro));
        dv[ct] = mfma32(ota, pk[h], dv[ct]);
        dk[ct] = mfma32(qta, dsk[h], dk[ct]);
      }
    }
    stage ^= 1;
    rb = nxt;
  };
  auto edge_block = [&](int b) {
    return (CAUSAL && b * C::BM < key0 + C::BN - 1) || key0 + C::BN > N;
  };
  // The first block's barrier also publishes the K/V tiles.
  while (rb < n_rb && edge_block(rb)) block(std::true_type{});
  while (rb < n_rb) block(std::false_type{});

  // Sum the two waves' halves of each key group: waves 4..7 hand their
  // accumulators over through LDS (the tile area, free once every wave is past
  // its last block), waves 0..3 add them to their own and write dK, dV.
  wait_vmcnt<0>();
  __syncthreads();
  float* xch = reinterpret_cast<float*>(smem) + (size_t)kq * 64 * 128;
  if (par == 1) {
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        *reinterpret_cast<f32x4*>(xch + ((2 * ct) * 4 + q4) * 256 + lane * 4) =
            f32x4{dk[ct][4 * q4], dk[ct][4 * q4 + 1], dk[ct][4 * q4 + 2], dk[ct][4 * q4 + 3]};
        *reinterpret_cast<f32x4*>(xch + ((2 * ct + 1) * 4 + q4) * 256 + lane * 4) =
            f32x4{dv[ct][4 * q4], dv[ct][4 * q4 + 1], dv[ct][4 * q4 + 2], dv[ct][4 * q4 + 3]};
      }
    }
  }
  __syncthreads();
  if (par == 0) {
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(xch + ((2 * ct) * 4 + q4) * 256 + lane * 4);
        const f32x4 b = *reinterpret_cast<const f32x4*>(xch + ((2 * ct + 1) * 4 + q4) * 256 + lane * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dk[ct][4 * q4 + e] += a[e];
          dv[ct][4 * q4 + e] += b[e];
        }
      }
    }
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
}

template <int D, bool CAUSAL, bool BLOCK>
hipError_t launch_dkdv_one(const BwdArgs& a, hipStream_t stream) {
  using C = BwdCfg<D>;
  BwdParams p;
  p.q = static_cast<const bf16*>(a.q);
  p.k = static_cast<const bf16*>(a.k);
  p.v = static_cast<const bf16*>(a.v);
  p.dout = static_cast<const bf16*>(a.dout);
  p.l2 = a.l2;
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
  if constexpr (D == 128)
    hipLaunchKernelGGL((fa_bwd_dkdv8_kernel<CAUSAL, BLOCK>), grid, dim3(Dkdv8Cfg::THREADS), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, CAUSAL, BLOCK>), grid, dim3(C::THREADS), 0, stream,
                       p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dkdv_d(const BwdArgs& a, hipStream_t stream) {
  const bool blk = a.mask.blocks != nullptr;
  if (a.mask.causal)
    return blk ? launch_dkdv_one<D, true, true>(a, stream)
               : launch_dkdv_one<D, true, false>(a, stream);
  return blk ? launch_dkdv_one<D, false, true>(a, stream)
             : launch_dkdv_one<D, false, false>(a, stream);
}

}  // namespace

hipError_t launch_bwd_preprocess(const BwdArgs& a, hipStream_t stream) {
  PreParams p;
  p.o = static_cast<const bf16*>(a.o);
  p.dout = static_cast<const bf16*>(a.dout);
  p.lse = a.lse;
  p.dvec = a.dvec;
  p.l2 = a.l2;
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

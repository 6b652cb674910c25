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
// Per wave (32 query rows) and K/V tile (BN keys):
//   S^T  = K_tile Q_w^T        MFMA 32x32x16: K rows from LDS, Q^T in VGPRs;
//   dP^T = V_tile dO_w^T       likewise. Each lane holds one query row, so the
//                              row's LSE and D_i = dO_i . O_i are lane scalars.
//   P  = 2^(S scale log2e - LSE_i log2e)      (masked pairs -> 0)
//   dS = P o (dP - D_i)
//   dQ^T += K_tile^T dS^T      dS^T straight from registers as the B operand
//                              (keys in the accumulator's order), K^T by the
//                              transposing LDS read.
// dQ = scale * dQ^T^T is written as bf16 once at the end.
#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {
namespace {

template <int D>
struct DqCfg {
  static constexpr int WAVES = 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BM = 32 * WAVES;           // query rows per workgroup
  static constexpr int BN = 64;                   // keys per K/V tile
  // K is read by 16-byte row reads (S^T) and by transposing reads (dQ^T):
  // a stride of 12 (mod 64) dwords serves both without 2-way conflicts on the
  // row reads; V is read by row reads only.
  static constexpr int STRK = D + 24;             // 152 / 88
  static constexpr int STRV = D + 8;              // 136 / 72
  static constexpr int KS = D / 16;
  static constexpr int NT = BN / 32;
  static constexpr int CT = D / 32;
  static constexpr int CHUNKS = BN * D / 8;
  static constexpr int CPT = CHUNKS / THREADS;
  static constexpr int KTILE = BN * STRK;
  static constexpr int VTILE = BN * STRV;
  static constexpr int STAGE = KTILE + VTILE;
  static_assert(CHUNKS % THREADS == 0, "tile must split evenly over threads");
};

struct DqParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* dout;
  const float* lse;
  const float* dvec;
  bf16* dq;
  int BH;
  int N;
  int n_row_blocks;
  float sl2;    // scale * log2(e)
  float scale;
  const uint8_t* blocks;
  int64_t blocks_bh_stride;
  int nb;
};

template <int D, bool CAUSAL, bool BLOCK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void fa_bwd_dq_kernel(DqParams p) {
  using C = DqCfg<D>;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * C::STAGE];  // [buffer][K tile, V tile]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int g16 = lane >> 4;
  const int i16 = lane & 15;

  // Largest causal row blocks first; every block of one head on one XCD when
  // B*H is a multiple of 8 (consecutive workgroups go to different XCDs).
  const int bh = blockIdx.x % p.BH;
  const int rb = p.n_row_blocks - 1 - blockIdx.x / p.BH;
  const int N = p.N;
  const int64_t head = (int64_t)bh * N * D;
  const bf16* __restrict__ Kh = p.k + head;
  const bf16* __restrict__ Vh = p.v + head;
  const int row0 = rb * C::BM;
  const int wrow0 = row0 + 32 * wave;
  const int qrow = wrow0 + l32;

  int kt_end = (N + C::BN - 1) / C::BN;
  if (CAUSAL) kt_end = min(kt_end, (row0 + C::BM - 1) / C::BN + 1);
  const uint8_t* mrow = nullptr;
  if (BLOCK) mrow = p.blocks + bh * p.blocks_bh_stride + (int64_t)(row0 / 128) * p.nb;
  auto kept = [&](int kt) -> bool { return !BLOCK || mrow[(kt * C::BN) / 128] != 0; };
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
    const float lse = p.lse[(int64_t)bh * N + r];
    if (qrow < N && lse != -INFINITY) {
      lrow = lse * kLog2e;
      drow = p.dvec[(int64_t)bh * N + r];
    }
  }

  u32x4 kst[C::CPT], vst[C::CPT];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int c = 0; c < C::CPT; ++c) {
      const int id = tid + c * C::THREADS;
      const int r = id / (D / 8);
      const int col = (id % (D / 8)) * 8;
      const int key = min(kt * C::BN + r, N - 1);  // keys past N are masked
      kst[c] = *reinterpret_cast<const u32x4*>(Kh + (int64_t)key * D + col);
      vst[c] = *reinterpret_cast<const u32x4*>(Vh + (int64_t)key * D + col);
    }
  };
  auto store_tile = [&](int buf) {
    bf16* Ks = smem + buf * C::STAGE;
    bf16* Vs = Ks + C::KTILE;
#pragma unroll
    for (int c = 0; c < C::CPT; ++c) {
      const int id = tid + c * C::THREADS;
      const int r = id / (D / 8);
      const int col = (id % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(Ks + r * C::STRK + col) = kst[c];
      *reinterpret_cast<u32x4*>(Vs + r * C::STRV + col) = vst[c];
    }
  };

  f32x16 acc[C::CT];
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) acc[ct] = f32x16{};

  auto compute = [&](int kt, int buf) {
    const bf16* Ks = smem + buf * C::STAGE;
    const bf16* Vs = Ks + C::KTILE;
    const int kbase = kt * C::BN;
    if (CAUSAL && kbase > wrow0 + 31) return;   // this wave's rows see none of the tile

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
        const bf16x8 a = lds_b128(Ks + (32 * st + l32) * C::STRK + 16 * kk + 8 * hh);
        s[st] = mfma32(a, qf[kk], s[st]);
        const bf16x8 b = lds_b128(Vs + (32 * st + l32) * C::STRV + 16 * kk + 8 * hh);
        dp[st] = mfma32(b, gf[kk], dp[st]);
      }
    }
    // s[st][v]: key kbase + 32*st + 8*(v/4) + 4*hh + v%4, query row qrow.
    const bool edge = (CAUSAL && kbase + C::BN - 1 > wrow0) || (kbase + C::BN > N);
    bf16x8 dsk[2 * C::NT];
#pragma unroll
    for (int st = 0; st < C::NT; ++st) {
      float ds[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float pe = fast_exp2(__builtin_fmaf(s[st][v], p.sl2, -lrow));
        if (edge) {
          const int key = kbase + 32 * st + 8 * (v / 4) + 4 * hh + (v % 4);
          if ((CAUSAL && key > qrow) || key >= N) pe = 0.f;
        }
        ds[v] = pe * (dp[st][v] - drow);
      }
      dsk[2 * st] = to_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
      dsk[2 * st + 1] = to_bf16x8(ds[8], ds[9], ds[10], ds[11], ds[12], ds[13], ds[14], ds[15]);
    }
    // dQ^T[c][i] += sum_j K[j][c] dS^T[j][i]; k-slots follow the accumulator's key
    // order (lane half hh: keys 4hh..4hh+3 and 8+4hh..8+4hh+3 of each 16).
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
      const int n0 = 32 * ct + 16 * (g16 & 1) + 4 * (i16 & 3);
#pragma unroll
      for (int ks = 0; ks < 2 * C::NT; ++ks) {
        const int r0 = 16 * ks + 4 * hh + (i16 >> 2);
        const i16x4 lo = lds_tr(Ks + r0 * C::STRK + n0);
        const i16x4 hi = lds_tr(Ks + (r0 + 8) * C::STRK + n0);
        acc[ct] = mfma32(cat(lo, hi), dsk[ks], acc[ct]);
      }
    }
  };

  int kt = 0;
  if (BLOCK && kt < kt_end && !kept(kt)) kt = next_kept(kt);
  if (kt < kt_end) {
    load_tile(kt);
    store_tile(0);
    __syncthreads();
    int buf = 0;
    while (kt < kt_end) {
      const int kn = next_kept(kt);
      if (kn < kt_end) load_tile(kn);
      compute(kt, buf);
      if (kn < kt_end) store_tile(buf ^ 1);
      __syncthreads();
      buf ^= 1;
      kt = kn;
    }
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

template <int D>
hipError_t launch_dq_d(const BwdArgs& a, hipStream_t stream) {
  using C = DqCfg<D>;
  DqParams p;
  p.q = static_cast<const bf16*>(a.q);
  p.k = static_cast<const bf16*>(a.k);
  p.v = static_cast<const bf16*>(a.v);
  p.dout = static_cast<const bf16*>(a.dout);
  p.lse = a.lse;
  p.dvec = a.dvec;
  p.dq = static_cast<bf16*>(a.dq);
  p.BH = a.BH;
  p.N = a.N;
  p.n_row_blocks = (a.N + C::BM - 1) / C::BM;
  p.sl2 = a.scale * kLog2e;
  p.scale = a.scale;
  p.blocks = a.mask.blocks;
  p.blocks_bh_stride = a.mask.bh_stride;
  p.nb = a.mask.nb;
  const dim3 grid((unsigned)p.n_row_blocks * (unsigned)a.BH);
  const dim3 block(C::THREADS);
  const bool blk = a.mask.blocks != nullptr;
  if (a.mask.causal) {
    if (blk)
      hipLaunchKernelGGL((fa_bwd_dq_kernel<D, true, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((fa_bwd_dq_kernel<D, true, false>), grid, block, 0, stream, p);
  } else {
    if (blk)
      hipLaunchKernelGGL((fa_bwd_dq_kernel<D, false, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((fa_bwd_dq_kernel<D, false, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream) {
  return a.d == 128 ? launch_dq_d<128>(a, stream) : launch_dq_d<64>(a, stream);
}

}  // namespace fa

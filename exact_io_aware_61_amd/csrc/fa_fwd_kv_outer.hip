// The forward in the loop order of the lecture summary's algorithm overview
// (section 3.3, the FlashAttention v1 order), kept to measure its IO against
// the FlashAttention-2 order of fa_fwd.hip.
//
// Order: O, l, m live in device memory (a float32 workspace). The outer loop
// walks the K/V blocks (Tc = N / BN of them), each loaded on chip once; the
// inner loop walks every Q block (Tr = N / BM), reading Q_i, O_i, l_i, m_i,
// updating them with the online-softmax recurrence of section 3.2 (O kept
// normalised at every step) and writing O_i, l_i, m_i back. Parallelism is over
// (batch, head) only: one workgroup runs both loops for its head, as the
// FlashAttention-2 overview describes the first version. The device traffic
// per head is therefore K, V once, Q and the O/l/m round trip Tc times, against
// Q, O once and K, V Tr times in fa_fwd.
//
// Inside a workgroup the four waves split each Q block by rows (32 each); a
// wave always owns the same rows, so its read-modify-writes of O, l, m need no
// synchronisation with the other waves (it waits for its own stores). At the
// first K/V block the initial values (O = 0, l = 0, m = -inf) are used instead
// of being read. A last sweep writes O as bf16 and LSE = m + ln l.
#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {
namespace {

template <int D>
struct KvoCfg {
  static constexpr int WAVES = 4;
  static constexpr int BM = 32 * WAVES;   // Q block rows
  static constexpr int BN = 64;           // K/V block keys
  static constexpr int NT = BN / 32;
  static constexpr int C = D / 8;
  static constexpr int KS = D / 16;
  static constexpr int CT = D / 32;
  static constexpr int TILE = BN * D;
  static constexpr int SPW = TILE / 512 / WAVES;   // direct-load slots per wave per tile
};

struct KvoParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  float* ow;     // workspace O, float32 [BH][N][D]
  float* mw;     // workspace m (log2 units of scaled scores), [BH][N]
  float* lw;     // workspace l, [BH][N]
  int N;
  float sl2;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fa_fwd_kv_outer_kernel(KvoParams p) {
  using C = KvoCfg<D>;
  __shared__ __attribute__((aligned(16))) bf16 kv[2 * C::TILE];   // K tile, V tile

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int g16 = lane >> 4;
  const int i16 = lane & 15;
  const int bh = blockIdx.x;
  const int N = p.N;
  const int64_t head = (int64_t)bh * N * D;
  const bf16* __restrict__ Qh = p.q + head;
  const bf16* __restrict__ Kh = p.k + head;
  const bf16* __restrict__ Vh = p.v + head;
  float* __restrict__ Ow = p.ow + head;
  float* __restrict__ Mw = p.mw + (int64_t)bh * N;
  float* __restrict__ Lw = p.lw + (int64_t)bh * N;
  const int Tc = (N + C::BN - 1) / C::BN;
  const int Tr = (N + C::BM - 1) / C::BM;

  int koff[C::KS], voff[C::CT][2];
#pragma unroll
  for (int kk = 0; kk < C::KS; ++kk) koff[kk] = toff<C::C>(l32, 16 * kk + 8 * hh);
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) {
    const int n0 = 32 * ct + 16 * (g16 & 1) + 4 * (i16 & 3);
    voff[ct][0] = toff<C::C>(4 * hh + (i16 >> 2), n0);
    voff[ct][1] = toff<C::C>(8 + 4 * hh + (i16 >> 2), n0);
  }

  for (int j = 0; j < Tc; ++j) {
    const int key0 = j * C::BN;
    __syncthreads();   // every wave is done with the previous K/V block
#pragma unroll
    for (int i = 0; i < C::SPW; ++i) {
      const int slot = wave + i * C::WAVES;
      dma_slot<C::C>(kv, slot, lane, [&](int r) { return Kh + (int64_t)min(key0 + r, N - 1) * D; });
      dma_slot<C::C>(kv + C::TILE, slot, lane,
                     [&](int r) { return Vh + (int64_t)min(key0 + r, N - 1) * D; });
    }
    wait_vmcnt<0>();
    __syncthreads();
    const bf16* Ks = kv;
    const bf16* Vs = kv + C::TILE;

    // Under the causal mask Q blocks that end before key0 see none of this block.
    const int i0 = CAUSAL ? key0 / C::BM : 0;
    for (int i = i0; i < Tr; ++i) {
      const int r0 = i * C::BM + 32 * wave;
      if (r0 >= N) continue;
      if (CAUSAL && key0 > r0 + 31) continue;
      const int qrow = r0 + l32;
      const int qr = min(qrow, N - 1);
      bf16x8 qf[C::KS];
#pragma unroll
      for (int kk = 0; kk < C::KS; ++kk)
        qf[kk] = *reinterpret_cast<const bf16x8*>(Qh + (int64_t)qr * D + 16 * kk + 8 * hh);
      // O_i, l_i, m_i from device memory (initial values at the first block)
      f32x16 oacc[C::CT];
      float m = -INFINITY, l = 0.f;
      float* orow = Ow + (int64_t)qr * D;
      if (j == 0) {
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct) oacc[ct] = f32x16{};
      } else {
        m = Mw[qr];
        l = Lw[qr];
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(orow + 32 * ct + 8 * g + 4 * hh);
#pragma unroll
            for (int r = 0; r < 4; ++r) oacc[ct][4 * g + r] = t[r];
          }
        }
      }
      // S_ij^T = K_j Q_i^T; s[st][v]: key key0 + 32 st + 8 (v/4) + 4 hh + v%4, row qrow
      f32x16 s[C::NT];
#pragma unroll
      for (int st = 0; st < C::NT; ++st) s[st] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < C::KS; ++kk)
#pragma unroll
        for (int st = 0; st < C::NT; ++st)
          s[st] = mfma32(lds_b128(Ks + koff[kk] + 32 * st * D), qf[kk], s[st]);
      if ((CAUSAL && key0 + C::BN - 1 > r0) || key0 + C::BN > N) {
#pragma unroll
        for (int st = 0; st < C::NT; ++st)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = key0 + 32 * st + 8 * (v / 4) + 4 * hh + (v % 4);
            if ((CAUSAL && key > qrow) || key >= N) s[st][v] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < C::NT; ++st)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[st][v]);
      mx = fmaxf(mx, swap_halves(mx)) * p.sl2;
      // Every row sees key 0, so m is finite from the first block on.
      const float m_new = fmaxf(m, mx);
      const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - m_new);
      float rs = 0.f;
      bf16x8 pk[2 * C::NT];
#pragma unroll
      for (int st = 0; st < C::NT; ++st) {
        float e[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          e[v] = fast_exp2(__builtin_fmaf(s[st][v], p.sl2, -m_new));
          rs += e[v];
        }
        pk[2 * st] = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
        pk[2 * st + 1] = to_bf16x8(e[8], e[9], e[10], e[11], e[12], e[13], e[14], e[15]);
      }
      rs += swap_halves(rs);
      const float l_new = l * alpha + rs;
      // O_i <- (l_i alpha O_i + P V_j) / l_new, the normalised recurrence
      const float keep = l * alpha;
#pragma unroll
      for (int ct = 0; ct < C::CT; ++ct) oacc[ct] *= keep;
#pragma unroll
      for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
        for (int ks = 0; ks < 2 * C::NT; ++ks)
          oacc[ct] = mfma32(cat(lds_tr(Vs + voff[ct][0] + 16 * ks * D),
                                lds_tr(Vs + voff[ct][1] + 16 * ks * D)),
                            pk[ks], oacc[ct]);
      const float inv = fast_rcp(l_new);
#pragma unroll
      for (int ct = 0; ct < C::CT; ++ct) oacc[ct] *= inv;
      if (qrow < N) {
#pragma unroll
        for (int ct = 0; ct < C::CT; ++ct)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<f32x4*>(orow + 32 * ct + 8 * g + 4 * hh) =
                f32x4{oacc[ct][4 * g], oacc[ct][4 * g + 1], oacc[ct][4 * g + 2],
                      oacc[ct][4 * g + 3]};
        if (hh == 0) {
          Mw[qrow] = m_new;
          Lw[qrow] = l_new;
        }
      }
      wait_vmcnt<0>();   // this wave reads these rows back at the next K/V block
    }
  }

  // Outputs: O as bf16, LSE = (m + log2 l) ln 2.
  for (int i = 0; i < Tr; ++i) {
    const int r0 = i * C::BM + 32 * wave;
    const int qrow = r0 + l32;
    if (qrow >= N) continue;
    const float* orow = Ow + (int64_t)qrow * D;
    bf16* out = p.o + head + (int64_t)qrow * D;
#pragma unroll
    for (int c = 8 * hh; c < D; c += 16) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(orow + c);
      const f32x4 b = *reinterpret_cast<const f32x4*>(orow + c + 4);
      *reinterpret_cast<bf16x8*>(out + c) = to_bf16x8(a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]);
    }
    if (hh == 0) p.lse[(int64_t)bh * N + qrow] = (Mw[qrow] + fast_log2(Lw[qrow])) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_one(const KvOuterArgs& a, hipStream_t stream) {
  KvoParams p;
  p.q = static_cast<const bf16*>(a.q);
  p.k = static_cast<const bf16*>(a.k);
  p.v = static_cast<const bf16*>(a.v);
  p.o = static_cast<bf16*>(a.o);
  p.lse = a.lse;
  p.ow = a.ow;
  p.mw = a.mw;
  p.lw = a.lw;
  p.N = a.N;
  p.sl2 = a.scale * kLog2e;
  hipLaunchKernelGGL((fa_fwd_kv_outer_kernel<D, CAUSAL>), dim3((unsigned)a.BH), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_kv_outer(const KvOuterArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch_one<128, true>(a, stream) : launch_one<128, false>(a, stream);
  return a.causal ? launch_one<64, true>(a, stream) : launch_one<64, false>(a, stream);
}

}  // namespace fa

// Decoding against a key/value cache on gfx950: the newest Nq (<= 32) queries of
// each (batch, head) attend its Nk cached keys, split over many workgroups.
//
// The pages only name inference with a KV cache and FlashDecoding (lecture
// summary, remark after section 3.1 and the conclusion). With Nq this small a
// head has no query blocks to spread over the chip, so the keys are split
// instead: each workgroup runs the tiled online softmax of the forward pass
// (lecture summary, section 3.2) over one chunk of the keys and leaves its
// unnormalised output and its (max, denominator) pair; a second kernel merges
// the chunks with the same rescale that merges tiles, which is the merge of two
// online-softmax states (m, l, O) -> (M, l e^(m - M) + l' e^(m' - M), ...).
// Query i sits at position Nk - Nq + i; under the causal mask it sees key j iff
// j <= Nk - Nq + i.
//
// Split kernel: one wave per (b, h, chunk). The wave holds Q^T of its (padded to
// 32) query rows in VGPRs; per tile of 32 keys it loads the K rows straight into
// VGPRs (the A operand of S^T = K Q^T, one key per lane row) and the V tile into
// LDS by direct global->LDS loads (the transposing LDS read then gives V^T for
// O^T += V^T P^T). Both are fetched one tile ahead. The work is bound by the
// K/V stream from HBM: 4 d bytes per key.
#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {
namespace {

template <int D>
struct DecCfg {
  static constexpr int BN = 32;         // keys per tile
  static constexpr int C = D / 8;       // 16-byte chunks per row
  static constexpr int KS = D / 16;     // MFMA k-steps over the head dim
  static constexpr int CT = D / 32;     // 32-column sub-tiles of the head dim
  static constexpr int TILE = BN * D;   // elements of a V tile
  static constexpr int SLOTS = TILE / 512;   // 1 KiB direct-load slots per tile
};

struct DecParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  float* part_o;    // [BH][nsplit][Nq][D] unnormalised outputs
  float* part_ml;   // [BH][nsplit][Nq][2]: running max (log2 units of scaled scores), denominator
  int BH;
  int Nq;
  int Nk;
  int nsplit;
  int chunk;        // keys per split (multiple of 32)
  float sl2;        // scale * log2(e)
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
void fa_decode_split_kernel(DecParams p) {
  using C = DecCfg<D>;
  __shared__ __attribute__((aligned(16))) bf16 vs[2 * C::TILE];

  const int lane = threadIdx.x;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int g16 = lane >> 4;
  const int i16 = lane & 15;

  const int bh = blockIdx.x / p.nsplit;
  const int sp = blockIdx.x % p.nsplit;
  const int Nq = p.Nq, Nk = p.Nk;
  const bf16* __restrict__ Kh = p.k + (int64_t)bh * Nk * D;
  const bf16* __restrict__ Vh = p.v + (int64_t)bh * Nk * D;
  const int kbeg = sp * p.chunk;
  const int kend = min(Nk, kbeg + p.chunk);
  const int qrow = l32;                       // this lane's query row (rows >= Nq are padding)
  const int limit = CAUSAL ? Nk - Nq + qrow : Nk - 1;   // last key this row may see

  // Q^T: B operand of S^T = K Q^T, zeros for padding rows.
  bf16x8 qf[C::KS];
#pragma unroll
  for (int kk = 0; kk < C::KS; ++kk) qf[kk] = bf16x8{};
  if (qrow < Nq) {
    const bf16* qr = p.q + ((int64_t)bh * Nq + qrow) * D;
#pragma unroll
    for (int kk = 0; kk < C::KS; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qr + 16 * kk + 8 * hh);
  }

  int voff[C::CT][2];
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) {
    const int n0 = 32 * ct + 16 * (g16 & 1) + 4 * (i16 & 3);
    voff[ct][0] = toff<C::C>(4 * hh + (i16 >> 2), n0);
    voff[ct][1] = toff<C::C>(8 + 4 * hh + (i16 >> 2), n0);
  }

  // Loads of one tile: K rows into registers, V rows into an LDS stage. Keys
  // past the chunk are clamped to its last key and masked below.
  auto load_k = [&](int t0, bf16x8 (&ka)[C::KS]) {
    const int key = min(t0 + l32, kend - 1);
#pragma unroll
    for (int kk = 0; kk < C::KS; ++kk)
      ka[kk] = *reinterpret_cast<const bf16x8*>(Kh + (int64_t)key * D + 16 * kk + 8 * hh);
  };
  auto load_v = [&](int t0, int stage) {
#pragma unroll
    for (int slot = 0; slot < C::SLOTS; ++slot)
      dma_slot<C::C>(vs + stage * C::TILE, slot, lane,
                     [&](int r) { return Vh + (int64_t)min(t0 + r, kend - 1) * D; });
  };

  f32x16 oacc[C::CT];
#pragma unroll
  for (int ct = 0; ct < C::CT; ++ct) oacc[ct] = f32x16{};
  float m_run = -INFINITY;   // running max of scaled scores, log2 units
  float l_run = 0.f;         // this lane half's share of the denominator

  // One tile: S^T from the K registers, then (once the products have read
  // them) the next tile's K rows are loaded into the same registers, then the
  // softmax and O^T += V^T P^T from the tile's V stage.
  bf16x8 ka[C::KS];
  auto compute = [&](int t0, int stage, int t_next) {
    f32x16 s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < C::KS; ++kk) s = mfma32(ka[kk], qf[kk], s);
    if (t_next < kend) load_k(t_next, ka);
    // s[v]: key t0 + 8*(v/4) + 4*hh + v%4, query qrow
    if (t0 + C::BN > kend || (CAUSAL && t0 + C::BN - 1 > Nk - Nq)) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = t0 + 8 * (v / 4) + 4 * hh + (v % 4);
        if (key >= kend || key > limit) s[v] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[v]);
    mx = fmaxf(mx, swap_halves(mx)) * p.sl2;
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;   // nothing visible yet: all P are 0
    const float alpha = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) oacc[ct] *= alpha;
    float e[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      e[v] = fast_exp2(__builtin_fmaf(s[v], p.sl2, -m_use));
      l_run += e[v];
    }
    const bf16x8 pk0 = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
    const bf16x8 pk1 = to_bf16x8(e[8], e[9], e[10], e[11], e[12], e[13], e[14], e[15]);
    const bf16* V = vs + stage * C::TILE;
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
      oacc[ct] = mfma32(cat(lds_tr(V + voff[ct][0]), lds_tr(V + voff[ct][1])), pk0, oacc[ct]);
      oacc[ct] = mfma32(cat(lds_tr(V + voff[ct][0] + 16 * D), lds_tr(V + voff[ct][1] + 16 * D)),
                        pk1, oacc[ct]);
    }
  };

  // Tiles of the chunk, loads one tile ahead (V into the other LDS stage, K
  // into the registers as soon as the current tile's S^T has read them).
  int t0 = kbeg;
  int stage = 0;
  if (t0 < kend) {
    load_k(t0, ka);
    load_v(t0, 0);
  }
  while (t0 < kend) {
    const int t1 = t0 + C::BN;
    wait_vmcnt<0>();
    __syncthreads();
    if (t1 < kend) load_v(t1, stage ^ 1);
    compute(t0, stage, t1);
    stage ^= 1;
    t0 = t1;
  }

  // Partial state of this chunk: unnormalised O^T (lane: row qrow, columns
  // 32ct + 8g + 4hh + r), running max and the denominator of both halves.
  const float l_tot = l_run + swap_halves(l_run);
  if (qrow < Nq) {
    const int64_t base = ((int64_t)bh * p.nsplit + sp) * Nq + qrow;
    float* orow = p.part_o + base * D;
#pragma unroll
    for (int ct = 0; ct < C::CT; ++ct) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = 32 * ct + 8 * g + 4 * hh;
        *reinterpret_cast<f32x4*>(orow + c) =
            f32x4{oacc[ct][4 * g], oacc[ct][4 * g + 1], oacc[ct][4 * g + 2], oacc[ct][4 * g + 3]};
      }
    }
    if (hh == 0) {
      p.part_ml[2 * base] = m_run;
      p.part_ml[2 * base + 1] = l_tot;
    }
  }
}

// Merge of the chunks: one workgroup of D threads per (b, h, query row), one
// output column per thread. One pass over the chunks with the online-softmax
// merge (the running max M moves to the larger of M and the chunks' maxima,
// rescaling the sums by 2^(M_old - M_new)), reading eight chunks' partial
// states per step so that their loads are in flight together.
template <int D>
__global__ __launch_bounds__(D) void fa_decode_combine_kernel(const float* part_o,
                                                             const float* part_ml, bf16* o,
                                                             float* lse, int nsplit, int Nq) {
  constexpr int U = 8;
  const int row = blockIdx.x;             // (bh, q) flattened
  const int bh = row / Nq, q = row % Nq;
  const int c = threadIdx.x;
  const int64_t first = (int64_t)bh * nsplit * Nq + q;   // chunk s sits at first + s * Nq
  float M = -INFINITY, L = 0.f, acc = 0.f;
  auto merge = [&](const float* mm, const float* ll, const float* oo, int n) {
    float mx = M;
    for (int j = 0; j < n; ++j) mx = fmaxf(mx, mm[j]);
    if (mx == -INFINITY) return;            // nothing visible in any chunk so far
    const float a = M == -INFINITY ? 0.f : fast_exp2(M - mx);
    L *= a;
    acc *= a;
    for (int j = 0; j < n; ++j) {
      const float w = fast_exp2(mm[j] - mx);   // 0 for a chunk that saw nothing
      L += w * ll[j];
      acc += w * oo[j];
    }
    M = mx;
  };
  int s = 0;
  for (; s + U <= nsplit; s += U) {
    float mm[U], ll[U], oo[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t base = first + (int64_t)(s + j) * Nq;
      mm[j] = part_ml[2 * base];
      ll[j] = part_ml[2 * base + 1];
      oo[j] = part_o[base * D + c];
    }
    merge(mm, ll, oo, U);
  }
  for (; s < nsplit; ++s) {
    const int64_t base = first + (int64_t)s * Nq;
    const float mm = part_ml[2 * base], ll = part_ml[2 * base + 1], oo = part_o[base * D + c];
    merge(&mm, &ll, &oo, 1);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  o[(int64_t)row * D + c] = (bf16)(acc * inv);
  if (c == 0) lse[row] = L > 0.f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
}

template <int D, bool CAUSAL>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  DecParams p;
  p.q = static_cast<const bf16*>(a.q);
  p.k = static_cast<const bf16*>(a.k);
  p.v = static_cast<const bf16*>(a.v);
  p.part_o = a.part_o;
  p.part_ml = a.part_ml;
  p.BH = a.BH;
  p.Nq = a.Nq;
  p.Nk = a.Nk;
  p.nsplit = a.nsplit;
  p.chunk = a.chunk;
  p.sl2 = a.scale * kLog2e;
  hipLaunchKernelGGL((fa_decode_split_kernel<D, CAUSAL>), dim3((unsigned)(a.BH * a.nsplit)),
                     dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fa_decode_combine_kernel<D>), dim3((unsigned)(a.BH * a.Nq)), dim3(D), 0,
                     stream, a.part_o, a.part_ml, static_cast<bf16*>(a.o), a.lse, a.nsplit, a.Nq);
  return hipGetLastError();
}

}  // namespace


hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.d == 128)
    return a.causal ? launch_d<128, true>(a, stream) : launch_d<128, false>(a, stream);
  return a.causal ? launch_d<64, true>(a, stream) : launch_d<64, false>(a, stream);
}

}  // namespace fa

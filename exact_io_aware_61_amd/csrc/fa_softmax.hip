// Row softmax for gfx950 with the online normalizer, as a kernel of its own.
//
// The normalizer ("why attention is slow" page, section on the online
// normalizer): while scanning x, keep the running maximum m and the denominator
// d relative to it, d_i = d_(i-1) e^(m_(i-1) - m_i) + e^(x_i - m_i); the second
// pass writes e^(x_i - m_N) / d_N. Two (m, d) pairs of disjoint parts of a row
// merge by the same rescale, (m, d) + (m', d') = (M, d e^(m - M) + d' e^(m' - M))
// with M = max(m, m'), which is what lets lanes and waves scan in parallel.
//
// Two launch shapes, both memory-bound:
//   short rows (cols <= 4096, 16-byte aligned rows): one wave per row. The row is
//     read once into registers, each lane forms (m, d) of its part and keeps its
//     exponentials, the wave merges the pairs by butterfly exchanges, and each
//     lane rescales its exponentials by e^(m_lane - M) / D and writes them. One
//     read and one write per element (8 bytes of HBM traffic).
//   any other row: one workgroup of 1024 threads per row, two streaming passes
//     (the online normalizer element by element, then the output), the pairs
//     of the 16 waves merged through LDS. 12 bytes per element at most; the
//     second read usually hits in cache.
// -inf entries get probability 0; a row without a finite entry is all zeros.
#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {
namespace {

struct MD {
  float m;   // running maximum
  float d;   // sum of e^(x - m) over the elements seen
};

__device__ __forceinline__ float exp_rel(float x, float m) {
  return fast_exp2((x - m) * kLog2e);
}

__device__ __forceinline__ MD md_merge(MD a, MD b) {
  const float M = fmaxf(a.m, b.m);
  if (M == -INFINITY) return {-INFINITY, 0.f};
  return {M, a.d * exp_rel(a.m, M) + b.d * exp_rel(b.m, M)};
}

__device__ __forceinline__ MD wave_merge(MD md) {
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) {
    const MD o{__shfl_xor(md.m, sh), __shfl_xor(md.d, sh)};
    md = md_merge(md, o);
  }
  return md;
}

// ---- short rows: one wave per row, the row held in registers --------------------------------

constexpr int kRowsPerBlock = 4;   // waves (rows) per 256-thread workgroup

template <int CPL>   // 16-byte chunks per lane: cols <= 256 * CPL
__global__ __launch_bounds__(256) void softmax_rows_reg(const float* x, float* y, int64_t rows,
                                                       int cols) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;   // whole wave; no barrier below
  const f32x4* xr = reinterpret_cast<const f32x4*>(x + row * cols);
  f32x4* yr = reinterpret_cast<f32x4*>(y + row * cols);
  const int n4 = cols >> 2;
  // Every element is read once and written once: non-temporal accesses keep
  // the input and output streams from evicting each other in the L2.
  f32x4 v[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int i = lane + 64 * c;
    v[c] = i < n4 ? __builtin_nontemporal_load(&xr[i]) : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  }
  float m = -INFINITY;
#pragma unroll
  for (int c = 0; c < CPL; ++c) m = fmaxf(fmaxf(m, fmaxf(v[c][0], v[c][1])), fmaxf(v[c][2], v[c][3]));
  // Exponentials relative to this lane's maximum; a lane without a finite
  // entry holds zeros (its -inf entries must not reach the final product).
  const float mu = m == -INFINITY ? 0.f : m;
  float d = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[c][e] = exp_rel(v[c][e], mu);
      d += v[c][e];
    }
  }
  const MD all = wave_merge(MD{m, d});
  // this lane's exponentials are relative to its own m: rescale to the row's
  const float f = (m == -INFINITY || all.d == 0.f) ? 0.f : exp_rel(m, all.m) / all.d;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int i = lane + 64 * c;
    if (i < n4) __builtin_nontemporal_store(v[c] * f, &yr[i]);
  }
}

// ---- any row: one workgroup per row, two streaming passes -----------------------------------

constexpr int kStreamThreads = 1024;

template <bool VEC>   // VEC: rows are 16-byte aligned (cols % 4 == 0, aligned x and y)
__global__ __launch_bounds__(kStreamThreads) void softmax_rows_stream(const float* x, float* y,
                                                                     int64_t cols) {
  __shared__ float sm[kStreamThreads / 64], sd[kStreamThreads / 64];
  const int tid = threadIdx.x;
  const float* xr = x + (int64_t)blockIdx.x * cols;
  float* yr = y + (int64_t)blockIdx.x * cols;
  auto step = [](MD& md, float xi) {
    if (xi == -INFINITY) return;
    if (xi > md.m) {
      md.d = md.d * exp_rel(md.m, xi) + 1.f;   // e^(m_old - m_new); 0 while d is 0
      md.m = xi;
    } else {
      md.d += exp_rel(xi, md.m);
    }
  };
  MD md{-INFINITY, 0.f};
  if (VEC) {
    // four 16-byte loads in flight per thread, then their elements in order
    const f32x4* x4 = reinterpret_cast<const f32x4*>(xr);
    const int64_t n4 = cols >> 2;
    int64_t i = tid;
    for (; i + 3 * kStreamThreads < n4; i += 4 * kStreamThreads) {
      f32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = x4[i + u * kStreamThreads];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) step(md, v[u][e]);
    }
    for (; i < n4; i += kStreamThreads) {
      const f32x4 v = x4[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) step(md, v[e]);
    }
  } else {
    for (int64_t i = tid; i < cols; i += kStreamThreads) step(md, xr[i]);
  }
  md = wave_merge(md);
  if ((tid & 63) == 0) {
    sm[tid >> 6] = md.m;
    sd[tid >> 6] = md.d;
  }
  __syncthreads();
  MD all{-INFINITY, 0.f};
#pragma unroll
  for (int w = 0; w < kStreamThreads / 64; ++w) all = md_merge(all, MD{sm[w], sd[w]});
  const float M = all.m;
  const float inv = all.d > 0.f ? 1.f / all.d : 0.f;   // no finite entry: all zeros
  const float Mu = M == -INFINITY ? 0.f : M;
  if (VEC) {
    const f32x4* x4 = reinterpret_cast<const f32x4*>(xr);
    f32x4* y4 = reinterpret_cast<f32x4*>(yr);
    const int64_t n4 = cols >> 2;
    auto out = [&](f32x4 v) {
      return f32x4{exp_rel(v[0], Mu), exp_rel(v[1], Mu), exp_rel(v[2], Mu), exp_rel(v[3], Mu)} * inv;
    };
    // The row's last read and its only write: non-temporal (see softmax_rows_reg).
    int64_t i = tid;
    for (; i + 3 * kStreamThreads < n4; i += 4 * kStreamThreads) {
      f32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(&x4[i + u * kStreamThreads]);
#pragma unroll
      for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(out(v[u]), &y4[i + u * kStreamThreads]);
    }
    for (; i < n4; i += kStreamThreads) __builtin_nontemporal_store(out(__builtin_nontemporal_load(&x4[i])), &y4[i]);
  } else {
    for (int64_t i = tid; i < cols; i += kStreamThreads) yr[i] = exp_rel(xr[i], Mu) * inv;
  }
}

template <int CPL>
hipError_t launch_reg(const SoftmaxArgs& a, hipStream_t stream) {
  const int64_t blocks = (a.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL((softmax_rows_reg<CPL>), dim3((unsigned)blocks), dim3(256), 0, stream, a.x,
                     a.y, a.rows, (int)a.cols);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_softmax_rows(const SoftmaxArgs& a, hipStream_t stream) {
  // At most 2^21 rows: 2^31 work-items for the streaming kernel, 2^27 for the other.
  if (a.rows < 1 || a.rows > kSoftmaxRowsPerLaunch) return hipErrorInvalidValue;
  const bool vec = (a.cols % 4) == 0 && (reinterpret_cast<uintptr_t>(a.x) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.y) & 15) == 0;
  if (vec && a.cols <= 4096) {
    if (a.cols <= 256) return launch_reg<1>(a, stream);
    if (a.cols <= 512) return launch_reg<2>(a, stream);
    if (a.cols <= 1024) return launch_reg<4>(a, stream);
    if (a.cols <= 2048) return launch_reg<8>(a, stream);
    return launch_reg<16>(a, stream);
  }
  const dim3 grid((unsigned)a.rows);
  if (vec)
    hipLaunchKernelGGL((softmax_rows_stream<true>), grid, dim3(kStreamThreads), 0, stream, a.x,
                       a.y, a.cols);
  else
    hipLaunchKernelGGL((softmax_rows_stream<false>), grid, dim3(kStreamThreads), 0, stream, a.x,
                       a.y, a.cols);
  return hipGetLastError();
}

}  // namespace fa

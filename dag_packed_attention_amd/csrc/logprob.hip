// Compact-to-semantic log-probabilities and the gradient of reused logit rows
// (HARTS: Hybrid-Attention RL over Tree Structures, Sec. 3.5 Eq. 17 and 19-20).
//
//   lambda_s = z[m(s), y_s] - lse(z[m(s)]),   lse(r) = log sum_v exp r_v
//   dz[c, v] = sum_{s: m(s)=c, y_s=v} g_s - (sum_{s: m(s)=c} g_s) softmax(z[c])_v
//
// Vocabulary-wide work runs once per compact row c: one block of 256 threads
// streams the row, keeps a running (max, sum of exponentials) per thread and
// combines them in a fixed tree; the positions that map to c are read from the
// row-grouped map (row_first / row_pos).  No S x V array is ever formed.  Both
// kernels are bound by HBM: the forward reads each row once, the backward reads
// it once and writes its gradient once.
//
// Layout: z and dz are [C][V] row-major.  The fast path takes 16-byte loads and
// needs V to be a multiple of 16 / sizeof(element) and z (and dz) 16-byte
// aligned; any other shape runs the element-wise path.  Rows with no position
// are not read: the forward writes lse = 0 for them, the backward writes a zero
// gradient row.  A target outside [0, V) gives lambda = NaN and adds no target
// term to dz.  Results do not depend on launch timing: every sum has a fixed order.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "logprob.hpp"

namespace dagattn {
namespace {

constexpr int kThreads = 256;
constexpr float kL2e = 1.4426950408889634f;
constexpr float kLn2f = 0.6931471805599453f;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float ld1(const uint16_t* p) { return __uint_as_float(((uint32_t)*p) << 16); }
__device__ __forceinline__ float ld1(const float* p) { return *p; }
__device__ __forceinline__ uint16_t to_bf(float x) {
  __bf16 b = (__bf16)x;
  return *reinterpret_cast<uint16_t*>(&b);
}
__device__ __forceinline__ void st1(uint16_t* p, float x) { *p = to_bf(x); }
__device__ __forceinline__ void st1(float* p, float x) { *p = x; }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Rows are touched once: stream them past the caches both ways.
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4 v = {a, b, c, d};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// elements of one 16-byte load
template <typename T> struct Vec;
template <> struct Vec<uint16_t> { static constexpr int n = 8; };
template <> struct Vec<float> { static constexpr int n = 4; };

template <typename T>
__device__ __forceinline__ void unpack(const uint4& w, float* x);
template <>
__device__ __forceinline__ void unpack<uint16_t>(const uint4& w, float* x) {
  x[0] = bf_lo(w.x); x[1] = bf_hi(w.x); x[2] = bf_lo(w.y); x[3] = bf_hi(w.y);
  x[4] = bf_lo(w.z); x[5] = bf_hi(w.z); x[6] = bf_lo(w.w); x[7] = bf_hi(w.w);
}
template <>
__device__ __forceinline__ void unpack<float>(const uint4& w, float* x) {
  x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
  x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
}

// store n = Vec<T>::n gradient values (T = dz element type) at p, 16-byte aligned
template <typename TG, int n>
__device__ __forceinline__ void store_vec(TG* p, const float* d);
template <>
__device__ __forceinline__ void store_vec<uint16_t, 8>(uint16_t* p, const float* d) {
  st_stream(p, (uint32_t)to_bf(d[0]) | ((uint32_t)to_bf(d[1]) << 16),
            (uint32_t)to_bf(d[2]) | ((uint32_t)to_bf(d[3]) << 16),
            (uint32_t)to_bf(d[4]) | ((uint32_t)to_bf(d[5]) << 16),
            (uint32_t)to_bf(d[6]) | ((uint32_t)to_bf(d[7]) << 16));
}
template <>
__device__ __forceinline__ void store_vec<uint16_t, 4>(uint16_t* p, const float* d) {
  uint2 w;
  w.x = (uint32_t)to_bf(d[0]) | ((uint32_t)to_bf(d[1]) << 16);
  w.y = (uint32_t)to_bf(d[2]) | ((uint32_t)to_bf(d[3]) << 16);
  *reinterpret_cast<uint2*>(p) = w;
}
template <>
__device__ __forceinline__ void store_vec<float, 8>(float* p, const float* d) {
  st_stream(p, __float_as_uint(d[0]), __float_as_uint(d[1]), __float_as_uint(d[2]), __float_as_uint(d[3]));
  st_stream(p + 4, __float_as_uint(d[4]), __float_as_uint(d[5]), __float_as_uint(d[6]), __float_as_uint(d[7]));
}
template <>
__device__ __forceinline__ void store_vec<float, 4>(float* p, const float* d) {
  st_stream(p, __float_as_uint(d[0]), __float_as_uint(d[1]), __float_as_uint(d[2]), __float_as_uint(d[3]));
}

// Running (max m, sum s of exp(x - m)).  m = -inf with s = 0 is the empty state.
struct MS {
  float m, s;
};

__device__ __forceinline__ MS ms_merge(MS a, MS b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return {m, 0.f};
  const float sa = a.s == 0.f ? 0.f : a.s * __builtin_amdgcn_exp2f((a.m - m) * kL2e);
  const float sb = b.s == 0.f ? 0.f : b.s * __builtin_amdgcn_exp2f((b.m - m) * kL2e);
  return {m, sa + sb};
}

// Fold n values into the running state: rescale once if the batch raises the max.
template <int n>
__device__ __forceinline__ void ms_add(MS& r, const float* x) {
  float mx = x[0];
#pragma unroll
  for (int i = 1; i < n; ++i) mx = fmaxf(mx, x[i]);
  if (mx > r.m) {
    r.s = r.s == 0.f ? 0.f : r.s * __builtin_amdgcn_exp2f((r.m - mx) * kL2e);
    r.m = mx;
  }
  if (r.m == -INFINITY) return;
  const float ml = -r.m * kL2e;
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < n; ++i) acc += __builtin_amdgcn_exp2f(fmaf(x[i], kL2e, ml));
  r.s += acc;
}

// Fixed-order combination over the block: butterfly within each wave, then the
// four wave results in wave order.  Every thread returns the same state.
__device__ __forceinline__ MS block_ms(MS r, MS* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    MS o{__shfl_xor(r.m, off), __shfl_xor(r.s, off)};
    r = (threadIdx.x & off) ? ms_merge(o, r) : ms_merge(r, o);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = r;
  __syncthreads();
  MS t = ms_merge(ms_merge(red[0], red[1]), ms_merge(red[2], red[3]));
  __syncthreads();
  return t;
}

__device__ __forceinline__ float block_sum(float x, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float o = __shfl_xor(x, off);
    x = (threadIdx.x & off) ? o + x : x + o;
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  const float t = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return t;
}

__device__ __forceinline__ void row_range(const int32_t* row_first, int64_t c, int64_t n_pos, int64_t& b,
                                          int64_t& e) {
  b = row_first[c];
  e = row_first[c + 1];
  b = b < 0 ? 0 : (b > n_pos ? n_pos : b);
  e = e < b ? b : (e > n_pos ? n_pos : e);
}

// kVec: 16-byte path (V a multiple of Vec<T>::n, z 16-byte aligned).
template <typename T, bool kVec>
__global__ __launch_bounds__(kThreads) void lp_fwd_kernel(const T* __restrict__ z, int64_t C, int V,
                                                          const int32_t* __restrict__ row_first,
                                                          const int32_t* __restrict__ row_pos,
                                                          const int32_t* __restrict__ pos_target, int64_t n_pos,
                                                          float* __restrict__ lse, float* __restrict__ lam) {
  __shared__ MS red[4];
  const int t = threadIdx.x;
  for (int64_t c = blockIdx.x; c < C; c += gridDim.x) {
    int64_t b, e;
    row_range(row_first, c, n_pos, b, e);
    if (b == e) {
      if (t == 0) lse[c] = 0.f;
      continue;
    }
    const T* row = z + c * (int64_t)V;
    MS r{-INFINITY, 0.f};
    if constexpr (kVec) {
      constexpr int n = Vec<T>::n;
      constexpr int U = 4;  // loads in flight per thread
      const uint4* rv = reinterpret_cast<const uint4*>(row);
      const int nv = V / n;
      int i = t;
      for (; i + (U - 1) * kThreads < nv; i += U * kThreads) {
        uint4 w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) w[u] = ld_stream(rv + i + u * kThreads);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float x[n];
          unpack<T>(w[u], x);
          ms_add<n>(r, x);
        }
      }
      for (; i < nv; i += kThreads) {
        float x[n];
        unpack<T>(rv[i], x);
        ms_add<n>(r, x);
      }
    } else {
      for (int i = t; i < V; i += kThreads) {
        float x = ld1(row + i);
        ms_add<1>(r, &x);
      }
    }
    const MS tot = block_ms(r, red);
    const float l = tot.m + __builtin_amdgcn_logf(tot.s) * kLn2f;
    if (t == 0) lse[c] = l;
    for (int64_t i = b + t; i < e; i += kThreads) {
      const int32_t s = row_pos[i];
      if (s < 0 || s >= n_pos) continue;
      const int32_t y = pos_target[s];
      lam[s] = (y >= 0 && y < V) ? ld1(row + y) - l : __builtin_nanf("");
    }
  }
}

template <typename T, bool kVec>
__device__ __forceinline__ int owner_of(int v) {
  if constexpr (kVec) return (v / Vec<T>::n) % kThreads;
  return v % kThreads;
}

// Positions of one row staged in LDS for the backward: target and g per position,
// in map order (up to kStage of them; longer rows read the map from global memory).
constexpr int kStage = 1024;

template <typename T, typename TG, bool kVec>
__global__ __launch_bounds__(kThreads) void lp_bwd_kernel(const T* __restrict__ z, const float* __restrict__ lse,
                                                          int64_t C, int V, const int32_t* __restrict__ row_first,
                                                          const int32_t* __restrict__ row_pos,
                                                          const int32_t* __restrict__ pos_target,
                                                          const float* __restrict__ g, int64_t n_pos,
                                                          TG* __restrict__ dz) {
  __shared__ float red[4];
  __shared__ int32_t s_tg[kStage];
  __shared__ float s_g[kStage];
  const int t = threadIdx.x;
  constexpr int n = Vec<T>::n;
  for (int64_t c = blockIdx.x; c < C; c += gridDim.x) {
    int64_t b, e;
    row_range(row_first, c, n_pos, b, e);
    TG* out = dz + c * (int64_t)V;
    if (b == e) {
      if constexpr (kVec) {
        const float zero[n] = {};
        for (int i = t; i < V / n; i += kThreads) store_vec<TG, n>(out + (int64_t)i * n, zero);
      } else {
        for (int i = t; i < V; i += kThreads) st1(out + i, 0.f);
      }
      continue;
    }
    const int64_t cnt = e - b;
    const bool staged = cnt <= kStage;
    // target and g of position i of the row (an invalid map entry: no target, g = 0)
    auto fetch = [&](int64_t i, int32_t& y, float& gv) {
      const int32_t s = row_pos[b + i];
      const bool ok = s >= 0 && s < n_pos;
      y = ok ? pos_target[s] : -1;
      gv = ok ? g[s] : 0.f;
    };
    float gp = 0.f;
    for (int64_t i = t; i < cnt; i += kThreads) {
      int32_t y;
      float gv;
      fetch(i, y, gv);
      if (staged) {
        s_tg[i] = y;
        s_g[i] = gv;
      }
      gp += gv;
    }
    // G = sum of the row's upstream gradients, in a fixed order (also publishes the stage)
    const float nG = -block_sum(gp, red);
    const float ll = -lse[c] * kL2e;
    const T* row = z + c * (int64_t)V;
    if constexpr (kVec) {
      constexpr int U = 4;
      const uint4* rv = reinterpret_cast<const uint4*>(row);
      const int nv = V / n;
      int i = t;
      for (; i + (U - 1) * kThreads < nv; i += U * kThreads) {
        uint4 w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) w[u] = ld_stream(rv + i + u * kThreads);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float x[n];
          unpack<T>(w[u], x);
#pragma unroll
          for (int k = 0; k < n; ++k) x[k] = nG * __builtin_amdgcn_exp2f(fmaf(x[k], kL2e, ll));
          store_vec<TG, n>(out + (int64_t)(i + u * kThreads) * n, x);
        }
      }
      for (; i < nv; i += kThreads) {
        float x[n];
        unpack<T>(rv[i], x);
#pragma unroll
        for (int k = 0; k < n; ++k) x[k] = nG * __builtin_amdgcn_exp2f(fmaf(x[k], kL2e, ll));
        store_vec<TG, n>(out + (int64_t)i * n, x);
      }
    } else {
      for (int i = t; i < V; i += kThreads) st1(out + i, nG * __builtin_amdgcn_exp2f(fmaf(ld1(row + i), kL2e, ll)));
    }
    // Target terms: the thread that wrote element y rewrites it once, with the
    // sum of g over the row's positions that target y (in map order) added
    // before the single rounding.  Same thread, same address: the rewrite lands last.
    for (int64_t i = 0; i < cnt; ++i) {
      int32_t y;
      float gi;
      if (staged) {
        y = s_tg[i];
        gi = s_g[i];
      } else {
        fetch(i, y, gi);
      }
      if (y < 0 || y >= V || owner_of<T, kVec>(y) != t) continue;
      bool first = true;
      for (int64_t j = 0; j < i && first; ++j) {
        int32_t yj;
        float gj;
        if (staged) {
          yj = s_tg[j];
        } else {
          fetch(j, yj, gj);
        }
        first = yj != y;
      }
      if (!first) continue;
      float acc = gi;
      for (int64_t j = i + 1; j < cnt; ++j) {
        int32_t yj;
        float gj;
        if (staged) {
          yj = s_tg[j];
          gj = s_g[j];
        } else {
          fetch(j, yj, gj);
        }
        if (yj == y) acc += gj;
      }
      st1(out + y, acc + nG * __builtin_amdgcn_exp2f(fmaf(ld1(row + y), kL2e, ll)));
    }
    __syncthreads();  // the stage is rewritten by the next row
  }
}

int grid_for(int64_t C) { return (int)(C < 1048576 ? C : 1048576); }

template <typename T>
bool vec_ok(const void* p, int V) {
  return (V % Vec<T>::n) == 0 && (reinterpret_cast<uintptr_t>(p) & 15) == 0;
}

}  // namespace

template <typename T>
void launch_lp_fwd(const T* z, int64_t C, int V, const int32_t* row_first, const int32_t* row_pos,
                   const int32_t* pos_target, int64_t n_pos, float* lse, float* lam, hipStream_t st) {
  if (C <= 0) return;
  const dim3 grid(grid_for(C)), block(kThreads);
  if (vec_ok<T>(z, V))
    hipLaunchKernelGGL((lp_fwd_kernel<T, true>), grid, block, 0, st, z, C, V, row_first, row_pos, pos_target,
                       n_pos, lse, lam);
  else
    hipLaunchKernelGGL((lp_fwd_kernel<T, false>), grid, block, 0, st, z, C, V, row_first, row_pos, pos_target,
                       n_pos, lse, lam);
}

template <typename T, typename TG>
void launch_lp_bwd(const T* z, const float* lse, int64_t C, int V, const int32_t* row_first, const int32_t* row_pos,
                   const int32_t* pos_target, const float* g, int64_t n_pos, TG* dz, hipStream_t st) {
  if (C <= 0) return;
  const dim3 grid(grid_for(C)), block(kThreads);
  if (vec_ok<T>(z, V) && (reinterpret_cast<uintptr_t>(dz) & 15) == 0)
    hipLaunchKernelGGL((lp_bwd_kernel<T, TG, true>), grid, block, 0, st, z, lse, C, V, row_first, row_pos,
                       pos_target, g, n_pos, dz);
  else
    hipLaunchKernelGGL((lp_bwd_kernel<T, TG, false>), grid, block, 0, st, z, lse, C, V, row_first, row_pos,
                       pos_target, g, n_pos, dz);
}

template void launch_lp_fwd<uint16_t>(const uint16_t*, int64_t, int, const int32_t*, const int32_t*, const int32_t*,
                                      int64_t, float*, float*, hipStream_t);
template void launch_lp_fwd<float>(const float*, int64_t, int, const int32_t*, const int32_t*, const int32_t*,
                                   int64_t, float*, float*, hipStream_t);
template void launch_lp_bwd<uint16_t, uint16_t>(const uint16_t*, const float*, int64_t, int, const int32_t*,
                                                const int32_t*, const int32_t*, const float*, int64_t, uint16_t*,
                                                hipStream_t);
template void launch_lp_bwd<uint16_t, float>(const uint16_t*, const float*, int64_t, int, const int32_t*,
                                             const int32_t*, const int32_t*, const float*, int64_t, float*,
                                             hipStream_t);
template void launch_lp_bwd<float, uint16_t>(const float*, const float*, int64_t, int, const int32_t*,
                                             const int32_t*, const int32_t*, const float*, int64_t, uint16_t*,
                                             hipStream_t);
template void launch_lp_bwd<float, float>(const float*, const float*, int64_t, int, const int32_t*, const int32_t*,
                                          const int32_t*, const float*, int64_t, float*, hipStream_t);

}  // namespace dagattn

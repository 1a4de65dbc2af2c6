// Short causal convolution of a linear-attention block over a rollout tree
// (HARTS: Hybrid-Attention RL over Tree Structures, Sec. 4.2; Octopus App. C).
//
// Per channel c, with taps W[c, 0..w-1] (w <= 4; the last multiplies the current
// token) along each token's own root-to-node path (mounted spans skipped):
//   pre_t = sum_k W[c, w-1-k] x_{t-k},   y_t = act(pre_t),   act = identity or SiLU.
// A token's window is the same on every trajectory that holds it, so each
// compact row is computed once.  Backward: dpre_t = dy_t act'(pre_t);
// dx_t = sum over every output s whose window holds t (itself, the next rows of
// its node, and the first rows of every branch below it) of W[c, w-1-d(s,t)] dpre_s;
// dW[c, w-1-k] = sum_t dpre_t x_{t-k}.
//
// Work split: one 64-row page per block (and 1,024 channels, 4 per thread, 8-byte
// loads).  The forward walks the page's rows with the previous three inputs in
// registers, starting from the three path predecessors of the page's first token
// (conv_prev).  The backward walks the rows downwards with the window of inputs
// and the next three dpre values in registers; successors outside the page come
// from the host's list (conv_ext: each with its own three predecessors, so its
// dpre is recomputed here).  dW is summed per block over its pages and then over
// blocks in a fixed order: no atomics, bitwise reproducible.  HBM-bound: the
// forward reads x and writes y once; the backward reads x and dy and writes dx
// once, plus the few successor rows per page.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "conv.hpp"

namespace dagattn {
namespace {

constexpr int kThreads = 256;
constexpr int kNV = 4;                   // channels per thread (8-byte bf16 loads)
constexpr int kChan = kNV * kThreads;    // channels per block
constexpr float kL2e = 1.4426950408889634f;

// kNV channels of one row: bf16 bits as loaded (B) and as fp32 values (F)
struct B {
  uint32_t w[kNV / 2];
};
struct F {
  float v[kNV];
};

__device__ __forceinline__ F zeroF() {
  F r;
#pragma unroll
  for (int i = 0; i < kNV; ++i) r.v[i] = 0.f;
  return r;
}
__device__ __forceinline__ B zeroB() {
  B r;
#pragma unroll
  for (int i = 0; i < kNV / 2; ++i) r.w[i] = 0;
  return r;
}

__device__ __forceinline__ F unpack(const B& b) {
  F r;
#pragma unroll
  for (int i = 0; i < kNV / 2; ++i) {
    r.v[2 * i] = __uint_as_float(b.w[i] << 16);
    r.v[2 * i + 1] = __uint_as_float(b.w[i] & 0xffff0000u);
  }
  return r;
}

__device__ __forceinline__ uint32_t bf16_bits(float x) {
  __bf16 b = (__bf16)x;
  return (uint32_t)(*reinterpret_cast<uint16_t*>(&b));
}

__device__ __forceinline__ B loadB(const uint16_t* p) {
  B r;
  if constexpr (kNV == 8) {
    const uint4 q = *reinterpret_cast<const uint4*>(p);
    r.w[0] = q.x; r.w[1] = q.y; r.w[2] = q.z; r.w[3] = q.w;
  } else {
    const uint2 q = *reinterpret_cast<const uint2*>(p);
    r.w[0] = q.x; r.w[1] = q.y;
  }
  return r;
}

__device__ __forceinline__ void storeV(uint16_t* p, const F& d) {
  uint32_t w[kNV / 2];
#pragma unroll
  for (int i = 0; i < kNV / 2; ++i) w[i] = bf16_bits(d.v[2 * i]) | (bf16_bits(d.v[2 * i + 1]) << 16);
  if constexpr (kNV == 8)
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  else
    *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
}
__device__ __forceinline__ void storeV(float* p, const F& d) {
#pragma unroll
  for (int i = 0; i < kNV / 4; ++i)
    reinterpret_cast<float4*>(p)[i] = make_float4(d.v[4 * i], d.v[4 * i + 1], d.v[4 * i + 2], d.v[4 * i + 3]);
}

// 1 / (1 + e^-p)
__device__ __forceinline__ float sigm(float p) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-p * kL2e));
}

template <int kAct>
__device__ __forceinline__ float act(float p) {
  if constexpr (kAct == 1) return p * sigm(p);
  return p;
}

template <int kAct>
__device__ __forceinline__ float act_grad(float p) {
  if constexpr (kAct == 1) {
    const float s = sigm(p);
    return s * (1.f + p * (1.f - s));
  }
  return 1.f;
}

// Taps of this thread's channels, left-padded to 4: T[m] multiplies the input
// 3 - m steps back (T[3] the current one).
struct Taps {
  float t[4][kNV];
};

__device__ __forceinline__ Taps load_taps(const float* W, int w, int c0) {
  Taps T;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < kNV; ++i) {
      const int j = m - (4 - w);
      T.t[m][i] = j >= 0 ? W[(int64_t)(c0 + i) * w + j] : 0.f;
    }
  return T;
}

// pre = sum_k T[3-k] x_{t-k} for the window x0 (current) .. x3 (3 back)
__device__ __forceinline__ float tap4(const Taps& T, int i, float x0, float x1, float x2, float x3) {
  return fmaf(T.t[0][i], x3, fmaf(T.t[1][i], x2, fmaf(T.t[2][i], x1, T.t[3][i] * x0)));
}

template <int kAct>
__global__ __launch_bounds__(kThreads) void conv_fwd_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ W, int Ch, int w,
                                                            const int32_t* __restrict__ page_nrows,
                                                            const int32_t* __restrict__ prev, int64_t pages,
                                                            uint16_t* __restrict__ y) {
  const int c0 = (blockIdx.y * kThreads + threadIdx.x) * kNV;
  if (c0 >= Ch) return;
  const Taps T = load_taps(W, w, c0);
  for (int64_t p = blockIdx.x; p < pages; p += gridDim.x) {
    const int n = page_nrows[p];
    F h[3];  // inputs 1, 2, 3 steps back
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int32_t r = prev[4 * p + k];
      h[k] = r >= 0 ? unpack(loadB(x + (int64_t)r * Ch + c0)) : zeroF();
    }
    const uint16_t* xp = x + p * 64 * (int64_t)Ch + c0;
    uint16_t* yp = y + p * 64 * (int64_t)Ch + c0;
    for (int r0 = 0; r0 < 64; r0 += 8) {
      B raw[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) raw[q] = r0 + q < n ? loadB(xp + (int64_t)(r0 + q) * Ch) : zeroB();
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const F cur = unpack(raw[q]);
        F out;
#pragma unroll
        for (int i = 0; i < kNV; ++i) out.v[i] = act<kAct>(tap4(T, i, cur.v[i], h[0].v[i], h[1].v[i], h[2].v[i]));
        storeV(yp + (int64_t)(r0 + q) * Ch, r0 + q < n ? out : zeroF());
        h[2] = h[1];
        h[1] = h[0];
        h[0] = cur;
      }
    }
  }
}

template <int kAct, typename TG>
__global__ __launch_bounds__(kThreads) void conv_bwd_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ dy,
                                                            const float* __restrict__ W, int Ch, int w,
                                                            const int32_t* __restrict__ page_nrows,
                                                            const int32_t* __restrict__ prev,
                                                            const int64_t* __restrict__ ext_off,
                                                            const ConvExt* __restrict__ ext, int64_t pages,
                                                            TG* __restrict__ dx, float* __restrict__ part) {
  const int c0 = (blockIdx.y * kThreads + threadIdx.x) * kNV;
  if (c0 >= Ch) return;
  const Taps T = load_taps(W, w, c0);
  float dW[4][kNV];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < kNV; ++i) dW[m][i] = 0.f;
  auto xrow = [&](int32_t r) { return r >= 0 ? loadB(x + (int64_t)r * Ch + c0) : zeroB(); };
  for (int64_t p = blockIdx.x; p < pages; p += gridDim.x) {
    const int n = page_nrows[p];
    const int64_t base = p * 64;
    TG* dxp = dx + base * Ch + c0;
    for (int r = n; r < 64; ++r) storeV(dxp + (int64_t)r * Ch, zeroF());
    if (n == 0) continue;
    // successors outside the page: their taps on this page's last three rows
    F tail[3];  // tail[q] belongs to row n - 1 - q
#pragma unroll
    for (int q = 0; q < 3; ++q) tail[q] = zeroF();
    for (int64_t e = ext_off[p]; e < ext_off[p + 1]; ++e) {
      const ConvExt E = ext[e];
      const F x0 = unpack(xrow(E.s)), x1 = unpack(xrow(E.p1)), x2 = unpack(xrow(E.p2)), x3 = unpack(xrow(E.p3));
      const F g = unpack(loadB(dy + (int64_t)E.s * Ch + c0));
      F dp;
#pragma unroll
      for (int i = 0; i < kNV; ++i)
        dp.v[i] = g.v[i] * act_grad<kAct>(tap4(T, i, x0.v[i], x1.v[i], x2.v[i], x3.v[i]));
      const int32_t pk[3] = {E.p1, E.p2, E.p3};
#pragma unroll
      for (int k = 1; k <= 3; ++k) {
        const int64_t q = base + n - 1 - pk[k - 1];
        if (pk[k - 1] < 0 || q < 0 || q > 2) continue;
#pragma unroll
        for (int qq = 0; qq < 3; ++qq)
          if (qq == q)
#pragma unroll
            for (int i = 0; i < kNV; ++i) tail[qq].v[i] = fmaf(T.t[3 - k][i], dp.v[i], tail[qq].v[i]);
      }
    }
    // rows n-1 .. 0: X[j] = input at row r - j (as loaded); dn[k] = dpre at row r + 1 + k (0 past the page)
    const uint16_t* xp = x + base * Ch + c0;
    const uint16_t* gp = dy + base * Ch + c0;
    auto xin = [&](int rr) -> B {
      if (rr >= 0) return loadB(xp + (int64_t)rr * Ch);
      return -rr <= 3 ? xrow(prev[4 * p + (-rr - 1)]) : zeroB();
    };
    B X[8];
    F dn[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) dn[k] = zeroF();
#pragma unroll
    for (int j = 0; j < 4; ++j) X[j] = xin(n - 1 - j);
    for (int r = n - 1; r >= 0; r -= 4) {
      B g[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        X[4 + j] = xin(r - 4 - j);
        g[j] = r - j >= 0 ? loadB(gp + (int64_t)(r - j) * Ch) : zeroB();
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rr = r - q;
        if (rr < 0) break;
        const F x0 = unpack(X[q]), x1 = unpack(X[q + 1]), x2 = unpack(X[q + 2]), x3 = unpack(X[q + 3]);
        const F gq = unpack(g[q]);
        F dp, out;
#pragma unroll
        for (int i = 0; i < kNV; ++i) {
          dp.v[i] = gq.v[i] * act_grad<kAct>(tap4(T, i, x0.v[i], x1.v[i], x2.v[i], x3.v[i]));
          dW[3][i] = fmaf(dp.v[i], x0.v[i], dW[3][i]);
          dW[2][i] = fmaf(dp.v[i], x1.v[i], dW[2][i]);
          dW[1][i] = fmaf(dp.v[i], x2.v[i], dW[1][i]);
          dW[0][i] = fmaf(dp.v[i], x3.v[i], dW[0][i]);
          out.v[i] = fmaf(T.t[0][i], dn[2].v[i], fmaf(T.t[1][i], dn[1].v[i], fmaf(T.t[2][i], dn[0].v[i],
                                                                                T.t[3][i] * dp.v[i])));
        }
        const int qt = n - 1 - rr;
        if (qt < 3)
#pragma unroll
          for (int qq = 0; qq < 3; ++qq)
            if (qq == qt)
#pragma unroll
              for (int i = 0; i < kNV; ++i) out.v[i] += tail[qq].v[i];
        storeV(dxp + (int64_t)rr * Ch, out);
        dn[2] = dn[1];
        dn[1] = dn[0];
        dn[0] = dp;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) X[j] = X[4 + j];
    }
  }
  float* pp = part + (int64_t)blockIdx.x * Ch * 4;
#pragma unroll
  for (int i = 0; i < kNV; ++i)
    *reinterpret_cast<float4*>(pp + (int64_t)(c0 + i) * 4) = make_float4(dW[0][i], dW[1][i], dW[2][i], dW[3][i]);
}

// dW[c][j] = sum over blocks b (in order) of part[b][c][4 - w + j]
__global__ __launch_bounds__(kThreads) void conv_dw_reduce_kernel(const float* __restrict__ part, int nb, int Ch,
                                                                  int w, float* __restrict__ dW) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= (int64_t)Ch * w) return;
  const int c = (int)(t / w), j = (int)(t % w);
  float acc = 0.f;
  for (int b = 0; b < nb; ++b) acc += part[((int64_t)b * Ch + c) * 4 + 4 - w + j];
  dW[t] = acc;
}

}  // namespace

int conv_bwd_blocks(int64_t pages) { return (int)(pages < 2048 ? pages : 2048); }

void launch_conv_fwd(const uint16_t* x, const float* W, int Ch, int w, int act, const int32_t* page_nrows,
                     const int32_t* prev, int64_t pages, uint16_t* y, hipStream_t st) {
  if (pages <= 0) return;
  const dim3 grid((unsigned)(pages < 1048576 ? pages : 1048576), (Ch + kChan - 1) / kChan), block(kThreads);
  if (act == 1)
    hipLaunchKernelGGL((conv_fwd_kernel<1>), grid, block, 0, st, x, W, Ch, w, page_nrows, prev, pages, y);
  else
    hipLaunchKernelGGL((conv_fwd_kernel<0>), grid, block, 0, st, x, W, Ch, w, page_nrows, prev, pages, y);
}

template <typename TG>
void launch_conv_bwd(const uint16_t* x, const uint16_t* dy, const float* W, int Ch, int w, int act,
                     const int32_t* page_nrows, const int32_t* prev, const int64_t* ext_off, const ConvExt* ext,
                     int64_t pages, TG* dx, float* dW, float* part, hipStream_t st) {
  if (pages <= 0) return;
  const int nb = conv_bwd_blocks(pages);
  const dim3 grid(nb, (Ch + kChan - 1) / kChan), block(kThreads);
  if (act == 1)
    hipLaunchKernelGGL((conv_bwd_kernel<1, TG>), grid, block, 0, st, x, dy, W, Ch, w, page_nrows, prev, ext_off, ext,
                       pages, dx, part);
  else
    hipLaunchKernelGGL((conv_bwd_kernel<0, TG>), grid, block, 0, st, x, dy, W, Ch, w, page_nrows, prev, ext_off, ext,
                       pages, dx, part);
  const int64_t nt = (int64_t)Ch * w;
  hipLaunchKernelGGL(conv_dw_reduce_kernel, dim3((unsigned)((nt + kThreads - 1) / kThreads)), dim3(kThreads), 0, st,
                     part, nb, Ch, w, dW);
}

template void launch_conv_bwd<uint16_t>(const uint16_t*, const uint16_t*, const float*, int, int, int, const int32_t*,
                                        const int32_t*, const int64_t*, const ConvExt*, int64_t, uint16_t*, float*,
                                        float*, hipStream_t);
template void launch_conv_bwd<float>(const uint16_t*, const uint16_t*, const float*, int, int, int, const int32_t*,
                                     const int32_t*, const int64_t*, const ConvExt*, int64_t, float*, float*, float*,
                                     hipStream_t);

}  // namespace dagattn

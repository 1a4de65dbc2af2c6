// HIP kernels for packed attention over a rollout DAG, written for gfx950.
//
// Data layout in HBM (C compact rows = pages * 64):
//   user tensors   q, o, dO  [C][Hq][D] bf16/fp32   k, v [C][Hkv][D]   lse [C][Hq] fp32
//                  dq [C][Hq][D], dk, dv [C][Hkv][D] in the gradient type (bf16 or fp32)
//   workspace      cs  [C][D/2] float2          cos/sin of the Eq. 1 rotation per row
//                  xn  [page][H][64][D] fp16    rotated (q, k) or copied (v, dO), page-major
//                  xt  [page][H][D][64] fp16    the same, transposed; the rows of every 16-group
//                                               are stored with bits 2 and 3 of the row index
//                                               swapped (the order in which an MFMA accumulator
//                                               lane holds them, see below)
//                  ld  [page][Hq][64] float2    the S and dP offsets of every row for the backward
//                  amax[4]                      largest |q|, |k|, |v|, |dO| (float bits)
//
// MFMA path (D = 128, Hq = 4 Hkv).  Operands are fp16: each of q, k, v, dO is scaled by a
// power of two from its largest |x| (amax), so no finite bf16 input overflows fp16; q and
// k land in [2^14, 2^15), which leaves 28 binades of normal fp16 range below the largest
// element, v and dO in [1, 2), which keeps the backward's fp16 dS operand in range.  The
// scales are folded into the softmax's exponent factor and the output multipliers, exactly.  The
// rotated q/k and the probabilities P and dS keep three more mantissa bits than bf16.
// A work-group serves one 64-row block and one KV head; its four
// waves are the four query heads of that GQA group, so every K/V tile staged
// in LDS is read by four heads.  Products are taken in the transposed
// orientation S^T = K Q^T and O^T = V^T P^T with v_mfma_f32_32x32x16_f16: a
// 32x32 accumulator lane then holds one query row (column n = lane % 32) and
// 16 keys, so the online-softmax state is per lane and only the max crosses
// lanes (lane ^ 32).  Accumulator element r of lane l is row
// m = 8 (r / 4) + 4 (l / 32) + r % 4.  Feeding it straight back as the B
// operand of the next product makes the contraction index of the two operands
// follow that same order, hence the bit-swapped rows of the transposed layouts.
//
// The backward is two kernels.  dK/dV: one work-group per KV page and KV head
// walks the page's reader list (every query block that sees the page, in a
// fixed order), keeps dK and dV in registers, sums the four heads through LDS
// in a fixed order and writes once: deterministic, no atomics.  dQ: one
// work-group per query block, like the forward.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"
#include "plan.hpp"

namespace dagattn {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef _Float16 f16_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf2f(bf16_t x) { return __uint_as_float(((uint32_t)x) << 16); }
__device__ __forceinline__ bf16_t f2bf(float x) {
  __bf16 b = (__bf16)x;
  return *reinterpret_cast<bf16_t*>(&b);
}
template <typename T> __device__ __forceinline__ float ld_f(const T* p);
template <> __device__ __forceinline__ float ld_f<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld_f<bf16_t>(const bf16_t* p) { return bf2f(*p); }
template <> __device__ __forceinline__ float ld_f<f16_t>(const f16_t* p) { return (float)*p; }
template <typename T> __device__ __forceinline__ void st_f(T* p, float x);
template <> __device__ __forceinline__ void st_f<float>(float* p, float x) { *p = x; }
template <> __device__ __forceinline__ void st_f<bf16_t>(bf16_t* p, float x) { *p = f2bf(x); }
template <> __device__ __forceinline__ void st_f<f16_t>(f16_t* p, float x) { *p = (f16_t)x; }

// Where the operand copies put their tensor's largest magnitude: q and k in [2^14, 2^15)
// (a rotated pair then stays below 2^15.5, inside fp16), v and dO in [1, 2): with P <= 1
// the backward's dS in those units is bounded by |dO.v| + |D| <= 4 D, far inside fp16.
constexpr int kTopQK = 14, kTopVO = 0;

// 2^(top - e) for the largest |x| = m 2^e (m in [1, 2)), from the float bits of that
// maximum: a power-of-two factor that maps a tensor's largest magnitude into
// [2^top, 2^(top+1)), exactly reversible.  e is taken as at least -24, so a tensor of
// tiny values is scaled up by at most 2^(top+24) and the products of factors the kernels
// form stay well inside fp32's normal range.
__device__ __forceinline__ float pow2_scale(uint32_t maxbits, int top) {
  const float m = __uint_as_float(maxbits);
  if (!(m > 0.f) || !isfinite(m)) return 1.f;
  return ldexpf(1.f, top - max(ilogbf(m), -24));
}

// ---------------------------------------------------------------------------
// Plan-table checks (device debug builds).  Built with DAG_DEBUG, the attention
// kernels check every query page, tile range, page id, mask id, visible interval and
// reader step they read from the plan tables against the plan's sizes (set by the
// host before each call).  A failed check records (code, value) once and counts
// every failure in g_dbg_err, and the kernel goes on with a safe value (page 0, an
// empty interval, no mask, the table's first entry), so no access leaves its buffer.
// Without DAG_DEBUG every check compiles to nothing.
// ---------------------------------------------------------------------------
#ifdef DAG_DEBUG
__device__ DbgLimits g_dbg_lim;
__device__ uint32_t g_dbg_err[4];  // first code, its value, number of failures
__device__ __noinline__ void dbg_fail(uint32_t code, int64_t value) {
  atomicAdd(&g_dbg_err[2], 1u);
  if (atomicCAS(&g_dbg_err[0], 0u, code) == 0u) atomicExch(&g_dbg_err[1], (uint32_t)value);
}
#endif
__device__ __forceinline__ int dbg_index(int i, int64_t n, uint32_t code) {  // 0 <= i < n
#ifdef DAG_DEBUG
  if (i < 0 || i >= n) {
    dbg_fail(code, i);
    return 0;
  }
#endif
  return i;
}
__device__ __forceinline__ int dbg_page(int page, uint32_t code) {
#ifdef DAG_DEBUG
  return dbg_index(page, g_dbg_lim.pages, code);
#else
  return page;
#endif
}
__device__ __forceinline__ int dbg_lohi(int lohi) {  // lo | hi << 8, lo <= hi <= 64
#ifdef DAG_DEBUG
  const int lo = lohi & 0xff, hi = (lohi >> 8) & 0xff;
  if (lohi < 0 || lo > hi || hi > 64) {
    dbg_fail(kDbgInterval, lohi);
    return 0;
  }
#endif
  return lohi;
}
__device__ __forceinline__ int dbg_mask(int mi) {  // -1 (no mask) or a mask id
#ifdef DAG_DEBUG
  if (mi < -1 || mi >= g_dbg_lim.masks) {
    dbg_fail(kDbgMask, mi);
    return -1;
  }
#endif
  return mi;
}
// a query page: its page and a tile list inside the table (at least one tile)
__device__ __forceinline__ QPage dbg_qpage(QPage qp) {
#ifdef DAG_DEBUG
  if (qp.tile_begin < 0 || qp.tile_count < 1 || (int64_t)qp.tile_begin + qp.tile_count > g_dbg_lim.tiles) {
    dbg_fail(kDbgTileRange, qp.tile_begin);
    qp.tile_begin = 0;
    qp.tile_count = 1;
  }
  qp.phys = dbg_page(qp.phys, kDbgQPage);
#endif
  return qp;
}
// a merged reader step: its query page and the two sides' intervals
__device__ __forceinline__ KStep dbg_step(KStep d) {
#ifdef DAG_DEBUG
  d.qph = dbg_page(d.qph, kDbgStepPage);
  bool ok = true;
  for (int side = 0; side < 2; ++side) {
    const uint32_t inf = ((uint32_t)d.info >> (16 * side)) & 0xffffu;
    const int lo = (inf >> 1) & 0x7f, hi = (inf >> 8) & 0x7f;
    ok = ok && lo <= hi && hi <= 64;
  }
  if (!ok) {
    dbg_fail(kDbgInterval, d.info);
    d.info &= 1;  // both sides empty
  }
#endif
  return d;
}

// a four-page group's reader step: its query page, its 32-row half and the pages' intervals
__device__ __forceinline__ GStep dbg_gstep(GStep d) {
#ifdef DAG_DEBUG
  d.qph = dbg_page(d.qph, kDbgStepPage);
  bool ok = d.rb == 0 || d.rb == 1;
  for (int i = 0; i < kGroup; ++i) {
    const uint32_t v = gvis_of(d, i);
    ok = ok && gvis_lo(v) <= gvis_hi(v) && gvis_hi(v) <= 64;
  }
  if (!ok) {
    dbg_fail(kDbgInterval, (int64_t)d.vis[0]);
    d.rb = 0;
    d.vis[0] = d.vis[1] = 0;  // no page read
  }
#endif
  return d;
}

// position of row r inside its transposed 16-group (bits 2 and 3 swapped)
__device__ __forceinline__ int tperm(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// ---------------------------------------------------------------------------
// prologue
// ---------------------------------------------------------------------------

// cos/sin of the rotary angle pos * base^(-2i/D) for every row and frequency,
// formed in double precision and rounded to float.
__global__ void cs_kernel(const int32_t* __restrict__ pos_of_row, float2* __restrict__ cs,
                          int64_t C, int half, double log2_base, int D) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= C * half) return;
  const int64_t row = idx / half;
  const int i = (int)(idx % half);
  const int p = pos_of_row[row];
  float2 r = make_float2(1.f, 0.f);
  if (p >= 0) {
    const double theta = exp2(-2.0 * (double)i / (double)D * log2_base);
    double s, c;
    sincos((double)p * theta, &s, &c);
    r = make_float2((float)c, (float)s);
  }
  cs[idx] = r;
}

// Rotate (optional) and relayout one page x head of a [C][H][D] tensor into
// page-major natural and/or transposed layouts.  Padding rows become zeros.
// One block of 256 threads per (page, head); D <= 128.
template <typename Tin, typename Tout>
__global__ __launch_bounds__(256) void relayout_kernel(
    const Tin* __restrict__ x, const float2* __restrict__ cs, const int32_t* __restrict__ page_nrows,
    Tout* __restrict__ out_n, Tout* __restrict__ out_t, int H, int D) {
  extern __shared__ float tile[];  // [64][D + 1]
  const int page = blockIdx.x / H, h = blockIdx.x % H;
  const int nrows = page_nrows[page];
  const int half = D / 2, ld = D + 1;
  for (int idx = threadIdx.x; idx < 64 * half; idx += blockDim.x) {
    const int r = idx / half, i = idx % half;
    float a = 0.f, b = 0.f;
    if (r < nrows) {
      const int64_t row = (int64_t)page * 64 + r;
      const Tin* src = x + (row * H + h) * D;
      a = ld_f(src + i);
      b = ld_f(src + i + half);
      if (cs) {
        const float2 t = cs[row * half + i];
        const float a2 = a * t.x - b * t.y;
        b = b * t.x + a * t.y;
        a = a2;
      }
    }
    tile[r * ld + i] = a;
    tile[r * ld + i + half] = b;
  }
  __syncthreads();
  const int64_t base = ((int64_t)page * H + h) * 64 * D;
  if (out_n)
    for (int idx = threadIdx.x; idx < 64 * D; idx += blockDim.x) {
      const int r = idx / D, d = idx % D;
      st_f(out_n + base + idx, tile[r * ld + d]);
    }
  if (out_t)
    for (int idx = threadIdx.x; idx < 64 * D; idx += blockDim.x) {
      const int d = idx / 64, p = idx % 64;
      const int r = tperm(p);
      st_f(out_t + base + (int64_t)d * 64 + p, tile[r * ld + d]);
    }
}

// ld[page][h][r] = (-lse / scale, -sum_d dO * O) for the backward; zero on padding rows.
// These are the offsets a row's raw score s = q.k and dP = dO.v take in the backward:
// P = exp(scale (s - lse / scale)) and dS = P (dP - D), so the MFMA kernels start their
// S and dP accumulators from them.
template <typename T>
__global__ void rowdot_kernel(const T* __restrict__ o, const T* __restrict__ o_lo, const T* __restrict__ dO,
                              const float* __restrict__ lse, const int32_t* __restrict__ page_nrows,
                              float2* __restrict__ ldout, int64_t n_pages, int Hq, int D, float inv_scale) {
  const int64_t idx = (int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;  // one wave per (row, h)
  const int lane = threadIdx.x % 64;
  if (idx >= n_pages * 64 * Hq) return;
  const int64_t row = idx / Hq;
  const int h = (int)(idx % Hq);
  const int64_t page = row / 64;
  const int r = (int)(row % 64);
  float acc = 0.f;
  const bool valid = r < page_nrows[page];
  if (valid)
    for (int d = lane; d < D; d += 64) {
      const int64_t e = (row * Hq + h) * D + d;
      const float ov = o_lo ? ld_f(o + e) + ld_f(o_lo + e) : ld_f(o + e);
      acc += ov * ld_f(dO + e);
    }
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) {
    float2 v = make_float2(0.f, 0.f);
    if (valid) v = make_float2(-lse[row * Hq + h] * inv_scale, -acc);
    ldout[(page * Hq + h) * 64 + r] = v;
  }
}

// out[0 .. n) = 0 (before kernels that take integer maxima into them)
__global__ void zero_u32_kernel(uint32_t* out, int n) {
  if ((int)threadIdx.x < n) out[threadIdx.x] = 0u;
}

// ---------------------------------------------------------------------------
// MFMA kernels: D = 128, four query heads per KV head, fp16 operands
// ---------------------------------------------------------------------------

constexpr int kD = 128;

constexpr int kRun = 8;  // consecutive units of one head that go to one XCD

typedef __attribute__((ext_vector_type(8))) uint16_t u16x8;

// amax[t] = max |x| over the valid rows of tensor t (t = blockIdx.y: q and dO
// [C][Hq][128], k and v [C][Hkv][128], bf16; order q, k, v, dO), as float bits: an integer
// maximum of non-negative floats is exact and order-free, so the result does not depend on
// the schedule.  Padding rows are skipped (callers may leave anything there).  16-byte
// loads, grid-stride over 16-byte pieces; amax must be 0 first.
__global__ __launch_bounds__(256) void absmax_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                     const bf16_t* __restrict__ v, const bf16_t* __restrict__ dO,
                                                     const int32_t* __restrict__ page_nrows, int64_t C, int Hq, int Hkv,
                                                     uint32_t* __restrict__ amax) {
  __shared__ float red[4];
  const int t = blockIdx.y;
  const bf16_t* x = t == 0 ? q : (t == 1 ? k : (t == 2 ? v : dO));
  const int64_t per_row = (int64_t)((t == 0 || t == 3) ? Hq : Hkv) * (kD / 8);
  const int64_t n = C * per_row;
  float m = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t row = i / per_row;
    if ((int)(row & 63) >= page_nrows[row >> 6]) continue;
    const u16x8 u = *reinterpret_cast<const u16x8*>(x + i * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(bf2f(u[e])));
  }
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(amax + t, __float_as_uint(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))));
}

// Prologue of the MFMA path (D = 128, bf16 in, fp16 out).  One block of 512
// threads per 64-row page walks the page's heads; thread (r, j) owns row r's
// columns 8 j .. 8 j + 7 and 64 + 8 j .. 64 + 8 j + 7 (rotation pairs), read and
// written as 16-byte pieces, so every global access is a full 128-byte run per
// eight threads.  Optional: rotation by R(pos) (kRot), the page-major natural
// copy [page][H][64][128] (kNat), the transposed copy [page][H][128][64] with
// rows in MFMA order (kTrans, through LDS) and a power-of-two scale from smax.
// Padding rows become zeros.
template <bool kRot, bool kNat, bool kTrans>
__global__ __launch_bounds__(512) void prep16_kernel(const bf16_t* __restrict__ x, const float2* __restrict__ cs,
                                                     const int32_t* __restrict__ page_nrows,
                                                     const uint32_t* __restrict__ smax, int top,
                                                     f16_t* __restrict__ out_n, f16_t* __restrict__ out_t, int H) {
  constexpr int kTs = 72;  // padded row of the transposed tile (elements)
  __shared__ __attribute__((aligned(16))) f16_t tt[kTrans ? 128 * kTs : 8];
  const int page = blockIdx.x, t = threadIdx.x, r = t >> 3, j = t & 7;
  const bool valid = r < page_nrows[page];
  const int64_t row = (int64_t)page * 64 + r;
  float c[8], sn[8];
  if (kRot) {
    const float4* cp = reinterpret_cast<const float4*>(cs + row * 64 + 8 * j);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float4 v = valid ? cp[e] : make_float4(1.f, 0.f, 1.f, 0.f);
      c[2 * e] = v.x, sn[2 * e] = v.y, c[2 * e + 1] = v.z, sn[2 * e + 1] = v.w;
    }
  }
  const float sc = smax ? pow2_scale(*smax, top) : 1.f;
  for (int h = 0; h < H; ++h) {
    const bf16_t* src = x + (row * H + h) * kD + 8 * j;
    u16x8 ua = {}, ub = {};
    if (valid) {
      ua = *reinterpret_cast<const u16x8*>(src);
      ub = *reinterpret_cast<const u16x8*>(src + 64);
    }
    f16x8 fa, fb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = bf2f(ua[e]), b = bf2f(ub[e]);
      if (kRot) {
        const float a2 = a * c[e] - b * sn[e];
        b = b * c[e] + a * sn[e];
        a = a2;
      }
      fa[e] = (f16_t)(a * sc);
      fb[e] = (f16_t)(b * sc);
    }
    if (kNat) {
      f16_t* dst = out_n + (((int64_t)page * H + h) * 64 + r) * kD + 8 * j;
      *reinterpret_cast<f16x8*>(dst) = fa;
      *reinterpret_cast<f16x8*>(dst + 64) = fb;
    }
    if (kTrans) {
      const int p = tperm(r);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        tt[(8 * j + e) * kTs + p] = fa[e];
        tt[(64 + 8 * j + e) * kTs + p] = fb[e];
      }
      __syncthreads();
      f16_t* dst = out_t + ((int64_t)page * H + h) * kD * 64;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int q = t + 512 * k, d = q >> 3, p0 = (q & 7) * 8;
        *reinterpret_cast<f16x8*>(dst + d * 64 + p0) = *reinterpret_cast<const f16x8*>(&tt[d * kTs + p0]);
      }
      __syncthreads();
    }
  }
}

// ld[page][h][r] = (-sq sk lse / scale, -sv sum_d dO' O) with O = o (+ o_lo), zero on
// padding rows: the offsets that S and dP take in the backward, in the units of the scaled
// fp16 operands (sq, sk, sv, sdo: the power-of-two scales of q, k, v, dO from amax[0..3]).
// dO' = fp16(sdo dO) is exactly the value the dP products read, so D cancels against dP
// wherever the exact values do (a dO element below fp16's range is zero in both), which
// matters where a row's attention sits on one key and |k| is large.  Sixteen lanes per
// (row, head), eight elements each (16-byte loads), summed in a fixed order; grid-stride
// over (row, head).
__global__ __launch_bounds__(256) void rowdot16_kernel(const bf16_t* __restrict__ o, const bf16_t* __restrict__ o_lo,
                                                       const bf16_t* __restrict__ dO, const float* __restrict__ lse,
                                                       const int32_t* __restrict__ page_nrows,
                                                       float2* __restrict__ ldout, const uint32_t* __restrict__ amax,
                                                       int64_t n_pages, int Hq, float inv_scale) {
  const int sub = threadIdx.x & 15;
  const float sqk = pow2_scale(amax[0], kTopQK) * pow2_scale(amax[1], kTopQK);
  const float sv = pow2_scale(amax[2], kTopVO), sdo = pow2_scale(amax[3], kTopVO);
  const int64_t total = n_pages * 64 * Hq;
  for (int64_t it = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4); it < total; it += (int64_t)gridDim.x * 16) {
    const int64_t row = it / Hq;
    const int h = (int)(it % Hq);
    const int64_t page = row >> 6;
    const int r = (int)(row & 63);
    const bool valid = r < page_nrows[page];
    float acc = 0.f;
    if (valid) {
      const int64_t e = (row * Hq + h) * kD + 8 * sub;
      const u16x8 uo = *reinterpret_cast<const u16x8*>(o + e);
      const u16x8 ud = *reinterpret_cast<const u16x8*>(dO + e);
      u16x8 ul = {};
      if (o_lo) ul = *reinterpret_cast<const u16x8*>(o_lo + e);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc += (bf2f(uo[k]) + bf2f(ul[k])) * (float)(f16_t)(bf2f(ud[k]) * sdo);
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (sub == 0)
      ldout[(page * Hq + h) * 64 + r] =
          valid ? make_float2(-lse[row * Hq + h] * inv_scale * sqk, -acc * sv) : make_float2(0.f, 0.f);
  }
}


__device__ __forceinline__ f32x16 mfma(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}
__device__ __forceinline__ f16x8 ld8(const f16_t* p) { return *reinterpret_cast<const f16x8*>(p); }
__device__ __forceinline__ f16x8 pack8(const f32x16& s, int base) {
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (f16_t)s[base + e];
  return r;
}
// key (or row) index within a 32-block held by accumulator element r of a lane in half `hi`
__device__ __forceinline__ int acc_row(int r, int hi) { return 8 * (r >> 2) + 4 * hi + (r & 3); }

// Work-group -> (unit, head).  The dispatcher deals work-groups round-robin over the
// eight XCDs, each with its own L2.  Work-group b is the (b / 8)-th one of XCD b % 8;
// giving every XCD runs of kRun consecutive units of one head lets units that share
// tiles (one node's pages) meet in one L2, while the runs, in launch order, still
// interleave over the XCDs so that the heaviest units start first everywhere.  The
// grid is padded to a multiple of 8 * kRun; padding work-groups return at once.
__device__ __forceinline__ bool map_item(int n_units, int H, int& unit, int& head) {
  const int b = blockIdx.x;
  const int x = b & 7, k = b >> 3;
  const int L = (((k / kRun) << 3) + x) * kRun + (k % kRun);
  const int R = L / kRun;
  head = R % H;
  unit = (R / H) * kRun + (L % kRun);
  return unit < n_units;
}

typedef __attribute__((address_space(3))) void lds_void;

// LDS on gfx950 serves 256 bytes (64 banks) per cycle: a 16-byte read takes 16
// lanes per cycle, an 8-byte read 32.  Staged tiles are laid out so that those
// lane groups never meet in a bank, and so that every fragment address is a
// per-lane base plus a compile-time offset (the k-step or d block).
//
// [rows][128] f16 tiles (K, V, Q, dO) sit in bricks of four rows: brick b (rows
// 4 b .. 4 b + 3) takes 1040 bytes, 1024 of data and 16 of padding, and inside it
// element (rr, col) sits at (col / 32) * 128 + rr * 32 + col % 32: per 32
// columns, the four rows' 64-byte pieces side by side.  Sixteen consecutive rows
// at one 16-byte chunk fall in sixteen different 16-byte bank groups (64 B apart
// inside a brick, one group further per brick), and a transpose read's 32 lanes
// (four rows x 64 bytes) cover one contiguous 256-byte span.  One direct-load
// instruction fills one brick from a contiguous 1 KiB of global memory.
constexpr int kBrick = 520;           // elements per 4-row brick, padding included
constexpr int kStepB = 8 * kBrick;    // a staged [32][128] tile
constexpr int kPageB = 16 * kBrick;   // a staged [64][128] tile

__device__ __forceinline__ int brick_off(int r, int col) {
  return (r >> 2) * kBrick + (col >> 5) * 128 + (r & 3) * 32 + (col & 31);
}
// Stage rows 4 b0 .. 4 (b0 + N) - 1 of a row-major [.][128] f16 block: instruction i
// fills brick b0 + i; lane l brings the 16-byte piece that belongs in slot l.
// Tiles are staged with buffer loads that write LDS directly (buffer_load ... lds):
// each wave instruction writes 64 x 16 B (or 64 x 4 B) contiguously at the LDS
// address held in M0, and the lane that fills a slot fetches the global piece that
// belongs there.  The tile's base is a buffer descriptor in SGPRs sized to the
// tile, so the hardware range-checks every access (reads past it return zero);
// the instruction's place in the tile is a scalar offset and the lane's a 32-bit
// VGPR offset that is computed once and never rewritten.  The loads are issued
// from inline assembly: the compiler cannot tell a load into one LDS buffer from
// a read of the other and would wait for the whole prefetch before the first
// read of the current step.  Every kernel that issues them waits for all of them
// (s_waitcnt 0) and then synchronises before the staged data is read.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 tile_rsrc(const void* p, int bytes) {
  const uint64_t a = (uint64_t)p;
  i32x4 r;
  r.x = (int)(uint32_t)a;
  r.y = (int)((uint32_t)(a >> 32) & 0xffffu);  // stride 0: raw byte offsets
  r.z = bytes;                                  // range limit
  r.w = 0x00020000;                             // 32-bit data format
  return r;
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void*)p;
}
__device__ __forceinline__ void dma16(const void* lds, uint32_t voff, i32x4 rsrc, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr(lds)), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* lds, uint32_t voff, i32x4 rsrc, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(lds_addr(lds)), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}
__device__ __forceinline__ uint32_t brick_lane_off(int lane) {
  return (uint32_t)((((lane >> 2) & 3) * kD + 32 * (lane >> 4) + 8 * (lane & 3)) * 2);
}
// Stage rows 4 b0 .. 4 (b0 + N) - 1 of a row-major [.][128] f16 block: instruction i
// fills brick b0 + i; lane l brings the 16-byte piece that belongs in slot l.
template <int N>
__device__ __forceinline__ void stage_bricks(f16_t* lds, i32x4 src, int b0, uint32_t loff) {
#pragma unroll
  for (int i = 0; i < N; ++i) dma16(lds + (b0 + i) * kBrick, loff, src, (b0 + i) * 4 * kD * 2);
}
// 16-byte row fragments: lane base for row r in half hi, plus kstep(ks) for column
// chunk 2 ks + hi
__device__ __forceinline__ int frag_base(int r, int hi) { return brick_off(r, 8 * hi); }
__device__ __forceinline__ constexpr int kstep(int ks) { return (ks >> 1) * 128 + (ks & 1) * 16; }

// [128][64] f16 tiles (a page's V^T or K^T, 128-byte rows) sit in bricks of eight
// rows, 1152 bytes each (128 of padding), inside which element (rr, col) sits at
// (col / 8) * 64 + rr * 8 + col % 8: the eight rows' 16-byte chunks of one column
// chunk side by side.  Eight consecutive rows at one chunk fill 128 contiguous
// bytes, and the padding puts the next eight rows in the other half of the
// 256-byte bank span.
constexpr int kCBrick = 576;
constexpr int kPageC = 16 * kCBrick;  // a staged [128][64] tile
__device__ __forceinline__ int cbrick_off(int r, int col) {
  return (r >> 3) * kCBrick + (col >> 3) * 64 + (r & 7) * 8 + (col & 7);
}
__device__ __forceinline__ uint32_t cbrick_lane_off(int lane) { return (uint32_t)(((lane & 7) * 64 + 8 * (lane >> 3)) * 2); }
template <int N>
__device__ __forceinline__ void stage_cbricks(f16_t* lds, i32x4 src, int b0, uint32_t loff) {
#pragma unroll
  for (int i = 0; i < N; ++i) dma16(lds + (b0 + i) * kCBrick, loff, src, (b0 + i) * 8 * 64 * 2);
}
// lane's base for 16-byte fragments of row r of a column-brick tile (chunk c is base + 64 c)
__device__ __forceinline__ int cfrag_base(int r, int hi) { return cbrick_off(r, 8 * hi); }

// all of this thread's global->LDS loads (and everything else) have landed
__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0); }
// An empty statement that takes x in registers: the compiler waits for x's load
// here.  Used on values loaded before a loop and read inside it, so that the
// compiler's own waits for them (which it counts without the loads issued from
// inline assembly, and so sets too tight) stay out of the loop instead of draining
// the staging loads in flight there.
__device__ __forceinline__ void pin(const f16x8& x) { asm volatile("" : : "v"(x)); }

constexpr int kTile = 64 * kD;  // elements of a page's 64 x 128 (or 128 x 64) block in global memory

// Lane pair l, l ^ 32: v_permlane32_swap with both operands one value leaves {value of the
// pair's lower lane, of its upper lane} in both lanes (no LDS crossbar, unlike a shuffle).
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Forward for one 64-row query block x one KV head.  Eight waves: wave (hh, nb)
// serves query head 4 g + hh and rows 32 nb .. 32 nb + 31 (two waves per SIMD,
// so one wave's softmax overlaps the other's products).  K/V tiles are
// double-buffered in LDS and fetched straight from global memory while the
// previous tile is multiplied, all by waves 0 and 1 (measured faster than four or
// eight issuing waves: the others' products run without load issue in between);
// each 64-key tile is taken as two 32-key halves.
//
// kMasked (packed page layouts): a tile may carry a mask id; the lane then reads its query
// row's 64-bit key mask and the mask alone decides which keys it sees (the causal rule of
// a page's last tile applies to unmasked tiles only).  Rows of one wave may then have seen
// no key yet when another row raises the running max; their rescale factor is 1.
//
// kForm, the exponent's form: |s sl2| <= D max|q| max|k| |scale log2 e| (rotation keeps
// norms), and only beyond 2^20 does the fused s sl2 - m lose m's rounding.  Unmasked
// plans launch two kernels, kForm 0 (fused) and 1 (unfused), each returning at once
// unless the bound is on its side, so neither carries the other's code in its loop;
// the masked variant (more registers) takes kForm 2, a check of the running max per
// half-tile.
template <bool kMasked, int kForm>
__global__ __launch_bounds__(512, 1) void fwd_mfma_kernel(
    const f16_t* __restrict__ qn, const f16_t* __restrict__ kn, const f16_t* __restrict__ vt,
    const QPage* __restrict__ qpages, const int32_t* __restrict__ order, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ tile_mask, const uint64_t* __restrict__ masks,
    bf16_t* __restrict__ o, float* __restrict__ lse, bf16_t* __restrict__ o_lo, const uint32_t* __restrict__ amax,
    int n_qp, int Hq, int Hkv, float sl2_raw) {
  __shared__ __attribute__((aligned(1024))) f16_t lk[2][kPageB];
  __shared__ __attribute__((aligned(1024))) f16_t lv[2][kPageC];
  int unit, g;
  if (!map_item(n_qp, Hkv, unit, g)) return;
  if constexpr (kForm != 2) {  // the exponent's form (see above): one of the two kernels works
    const float bound = (float)kD * __uint_as_float(amax[0]) * __uint_as_float(amax[1]) * fabsf(sl2_raw);
    if ((kForm == 1) == (bound <= 0x1p20f)) return;
  }
  // the fp16 copies hold sq q, sk k, sv v (powers of two): the scores come out as
  // sq sk q.k and the output as sv O, so the exponent factor and 1 / l absorb them exactly
  const float sl2 = sl2_raw / pow2_scale(amax[0], kTopQK) / pow2_scale(amax[1], kTopQK);
  const float inv_sv = 1.f / pow2_scale(amax[2], kTopVO);
  const QPage qp = dbg_qpage(qpages[dbg_index(order[unit], n_qp, kDbgQPage)]);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave index: uniform
  const int l32 = lane & 31, hi = lane >> 5;
  const int hh = wave & 3, nb = wave >> 2;
  const int h = g * 4 + hh;
  const int row = nb * 32 + l32;
  const int kb0 = frag_base(l32, hi), vb0 = cfrag_base(l32, hi);
  const uint32_t rlo = brick_lane_off(lane), clo = cbrick_lane_off(lane);

  f16x8 qf[8];
  const f16_t* qb = qn + ((int64_t)qp.phys * Hq + h) * 64 * kD;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qf[ks] = ld8(qb + row * kD + ks * 16 + hi * 8);

  f32x16 oacc[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) oacc[a] = zero16();
  float mrow = -INFINITY, lrow = 0.f;

  const int T = qp.tile_count;
  if (wave < 2) {
    const int64_t base = ((int64_t)dbg_page(tiles[qp.tile_begin].page, kDbgTilePage) * Hkv + g) * kTile;
    stage_bricks<8>(lk[0], tile_rsrc(kn + base, kTile * 2), 8 * wave, rlo);
    stage_cbricks<8>(lv[0], tile_rsrc(vt + base, kTile * 2), 8 * wave, clo);
  }
  wait_all_loads();
  __syncthreads();

  for (int t = 0; t < T; ++t) {
    const int buf = t & 1;
    if (t + 1 < T && wave < 2) {
      const int64_t base = ((int64_t)dbg_page(tiles[qp.tile_begin + t + 1].page, kDbgTilePage) * Hkv + g) * kTile;
      stage_bricks<8>(lk[buf ^ 1], tile_rsrc(kn + base, kTile * 2), 8 * wave, rlo);
      stage_cbricks<8>(lv[buf ^ 1], tile_rsrc(vt + base, kTile * 2), 8 * wave, clo);
    }
    const int lohi = dbg_lohi(tiles[qp.tile_begin + t].lohi);
    const int lo = lohi & 0xff, hi_t = (lohi >> 8) & 0xff;
    int mi = -1;
    uint64_t rmask = 0;
    if constexpr (kMasked) {
      mi = dbg_mask(tile_mask[qp.tile_begin + t]);
      if (mi >= 0) rmask = masks[(int64_t)mi * 128 + row];
    }
    const bool diag = (t == T - 1) && mi < 0;
    const bool full = lo == 0 && hi_t == 64 && !diag && mi < 0;
    const f16_t* K = lk[buf];
    const f16_t* V = lv[buf];

#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {  // 32-key halves
      // a half with no key visible to this wave's rows (outside the range, above the
      // diagonal, or rows that are all padding) would add exact zeros: skipped
      if (hi_t <= mb * 32 || lo >= mb * 32 + 32 || (diag && mb * 32 > nb * 32 + 31) || nb * 32 >= qp.nrows)
        continue;
      // all eight K fragments are read first, so the products wait only for the first;
      // the V fragments of this half go out before the softmax and arrive under it
      f16x8 kfr[8], vfr[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) kfr[ks] = ld8(K + kb0 + mb * 8 * kBrick + kstep(ks));
      f32x16 s = zero16();
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) s = mfma(kfr[ks], qf[ks], s);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) vfr[a * 2 + kk] = ld8(V + vb0 + a * 4 * kCBrick + (mb * 2 + kk) * 128);
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      // Online softmax in the log2 domain.  The running max m is raised only when
      // a row's new maximum exceeds it by more than kLazy (any lane of the wave),
      // so the accumulator rescale is rare; in between, probabilities reach at most
      // 2^kLazy, well inside fp16, and the final division by l removes the offset.
      constexpr float kLazy = 8.f;
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = mb * 32 + acc_row(r, hi);
          bool ok = key >= lo && key < hi_t && (!diag || key <= row);
          if constexpr (kMasked) ok = ok && (mi < 0 || ((rmask >> key) & 1ull));
          s[r] = ok ? s[r] : -INFINITY;
        }
      }
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = max_xor32(mx) * sl2;
      if (__any(mx > mrow + kLazy)) {
        const float mnew = fmaxf(mrow, mx);
        float alpha = __builtin_amdgcn_exp2f(mrow - mnew);
        if constexpr (kMasked) alpha = mnew == -INFINITY ? 1.f : alpha;
        mrow = mnew;
        lrow *= alpha;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[a][r] *= alpha;
      }
      // a half-tile can be fully masked before a row has seen any key (a mounted
      // span starting past key 32); then m is still -inf and every score is -inf
      const float mneg = mrow == -INFINITY ? 0.f : -mrow;
      if (kForm == 0 || (kForm == 2 && !__any(fabsf(mrow) > 0x1p20f))) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, mneg));
      } else {
        // logits beyond 2^20 in the log2 domain: the fused s * sl2 - m keeps m's rounding
        // error (over 2^-4 there, over 8 beyond 2^27), so each score is rounded to the log2
        // domain first and the max subtracted after; m is the rounded product of the largest
        // score, so the exponent stays <= kLazy whatever the logits' size
#pragma clang fp contract(off)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(s[r] * sl2 + mneg);
      }
      // The row sum adds the fp16-rounded weights that the PV product multiplies, so the
      // weights O is formed with sum to 1 exactly (a row on one key reproduces that key's
      // value exactly, and rowsum(dO O) in the backward cancels against its dP); summed as
      // fp16 pairs with fp32 accumulation.
      const f16x8 pf0 = pack8(s, 0), pf1 = pack8(s, 8);
      {
        typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
        const f16x2 one2 = {(f16_t)1.f, (f16_t)1.f};
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sum = __builtin_amdgcn_fdot2(f16x2{pf0[2 * i], pf0[2 * i + 1]}, one2, sum, false);
          sum = __builtin_amdgcn_fdot2(f16x2{pf1[2 * i], pf1[2 * i + 1]}, one2, sum, false);
        }
        lrow += sum;
      }
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        oacc[a] = mfma(vfr[a * 2], pf0, oacc[a]);
        oacc[a] = mfma(vfr[a * 2 + 1], pf1, oacc[a]);
      }
    }
    wait_all_loads();
    __syncthreads();
  }

  const float l = sum_xor32(lrow);
  const bool valid = row < qp.nrows;
  const float inv = valid ? inv_sv / l : 0.f;
  const int64_t grow = (int64_t)qp.phys * 64 + row;
  bf16_t* orow = o + (grow * Hq + h) * kD;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = a * 32 + 8 * j + 4 * hi;
      bf16_t hv[4], lv4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = oacc[a][4 * j + i] * inv;
        hv[i] = f2bf(x);
        lv4[i] = f2bf(x - bf2f(hv[i]));
      }
      uint2 w;
      w.x = (uint32_t)hv[0] | ((uint32_t)hv[1] << 16);
      w.y = (uint32_t)hv[2] | ((uint32_t)hv[3] << 16);
      *reinterpret_cast<uint2*>(orow + d) = w;
      if (o_lo) {
        w.x = (uint32_t)lv4[0] | ((uint32_t)lv4[1] << 16);
        w.y = (uint32_t)lv4[2] | ((uint32_t)lv4[3] << 16);
        *reinterpret_cast<uint2*>(o_lo + (grow * Hq + h) * kD + d) = w;
      }
    }
  if (hi == 0) lse[grow * Hq + h] = valid ? (mrow + __log2f(l)) * kLn2 : 0.f;
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i receives element i % 4 of the 8-byte pieces fetched by lanes
// 4 j + i / 4 (j = 0..3).  So if source lane 4 j + q reads row (r0 + j) at
// columns (c0 + 4 q .. + 3), lane i gets column c0 + i of rows r0 .. r0 + 3: a
// column of the tile, as an MFMA operand wants it when the contraction runs
// over rows.
typedef __fp16 v4fp16 __attribute__((__vector_size__(8)));
typedef __attribute__((address_space(3))) v4fp16 lds_v4fp16;

// 8 contraction elements for the lane's column d of a staged tile, rows
// 16 kk + {4 hi .. 4 hi + 3, 8 + 4 hi .. 8 + 4 hi + 3}: the order in which a 32x32
// accumulator lane of half `hi` holds rows 16 kk .. 16 kk + 15.  Source lane
// 16 G + a addresses row 16 kk + 8 half + 4 (G >> 1) + a / 4 at columns
// 32 dblk + 16 (G & 1) + 4 (a & 3) ..: its per-lane part is tr_base(lane), the
// rest (kk, half, dblk) is an immediate.
__device__ __forceinline__ int tr_base(int lane) {
  const int G = lane >> 4, a = lane & 15;
  return (G >> 1) * kBrick + (a >> 2) * 32 + (G & 1) * 16 + 4 * (a & 3);
}
__device__ __forceinline__ f16x8 frag_tr(const f16_t* tb, int kk, int dblk) {
  f16x8 out;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const f16_t* p = tb + (4 * kk + 2 * half) * kBrick + dblk * 128;
    const v4fp16 v = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_v4fp16*)p);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[half * 4 + j] = (f16_t)v[j];
  }
  return out;
}

// dQ for one query block (64 rows) x one KV head.  Eight waves, wave (hh, nb) =
// query head 4 g + hh and rows 32 nb ..; the K and V tiles are double-buffered in
// LDS like the forward's, and the dQ products read K's columns with transpose reads
// (no transposed copy of K is staged).
// kMasked: the forward's tile masks, read the same way.
template <typename TG, bool kMasked>
__global__ __launch_bounds__(512, 1) void dq_mfma_kernel(
    const f16_t* __restrict__ qn, const f16_t* __restrict__ kn, const f16_t* __restrict__ vn, const f16_t* __restrict__ dOn, const float2* __restrict__ ldd,
    const float2* __restrict__ cs, const uint32_t* __restrict__ dmax, const QPage* __restrict__ qpages,
    const int32_t* __restrict__ order, const Tile* __restrict__ tiles, const int32_t* __restrict__ tile_mask,
    const uint64_t* __restrict__ masks, TG* __restrict__ dq,
    const uint32_t* __restrict__ amax, int n_qp, int Hq, int Hkv, float sl2_raw, float scale) {
  __shared__ __attribute__((aligned(1024))) f16_t lk[2][kPageB];
  __shared__ __attribute__((aligned(1024))) f16_t lvv[2][kPageB];
  int unit, g;
  if (!map_item(n_qp, Hkv, unit, g)) return;
  // fp16 copies: sq q, sk k, sv v, sdo dO (powers of two); the S and dP offsets in ldd are
  // in the same scaled units, so dS comes out as sdo sv dS and the sum over keys of dS k
  // as sdo sv sk dQ / scale
  const float sq = pow2_scale(amax[0], kTopQK), sk = pow2_scale(amax[1], kTopQK), sv = pow2_scale(amax[2], kTopVO);
  const float sl2 = sl2_raw / sq / sk;
  const QPage qp = dbg_qpage(qpages[dbg_index(order[unit], n_qp, kDbgQPage)]);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave index: uniform
  const int l32 = lane & 31, hi = lane >> 5;
  const int hh = wave & 3, nb = wave >> 2;
  const int h = g * 4 + hh;
  const int row = nb * 32 + l32;
  const int kb0 = frag_base(l32, hi), tb = tr_base(lane);
  const uint32_t rlo = brick_lane_off(lane);

  f16x8 qf[8], df[8];
  const f16_t* qb = qn + ((int64_t)qp.phys * Hq + h) * 64 * kD;
  const f16_t* db = dOn + ((int64_t)qp.phys * Hq + h) * 64 * kD;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    qf[ks] = ld8(qb + row * kD + ks * 16 + hi * 8);
    df[ks] = ld8(db + row * kD + ks * 16 + hi * 8);
  }
  const float2 lt = ldd[((int64_t)qp.phys * Hq + h) * 64 + row];
  const float nl = lt.x * sl2, nD = lt.y;  // exponent offset (log2 domain) and -D
  f32x16 acc[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) acc[a] = zero16();

  const int T = qp.tile_count;
  if (wave < 4) {
    const int64_t base = ((int64_t)dbg_page(tiles[qp.tile_begin].page, kDbgTilePage) * Hkv + g) * kTile;
    stage_bricks<4>(lk[0], tile_rsrc(kn + base, kTile * 2), 4 * wave, rlo);
    stage_bricks<4>(lvv[0], tile_rsrc(vn + base, kTile * 2), 4 * wave, rlo);
  }
  wait_all_loads();
  __syncthreads();

  for (int t = 0; t < T; ++t) {
    const int buf = t & 1;
    if (t + 1 < T && wave < 4) {
      const int64_t base = ((int64_t)dbg_page(tiles[qp.tile_begin + t + 1].page, kDbgTilePage) * Hkv + g) * kTile;
      stage_bricks<4>(lk[buf ^ 1], tile_rsrc(kn + base, kTile * 2), 4 * wave, rlo);
      stage_bricks<4>(lvv[buf ^ 1], tile_rsrc(vn + base, kTile * 2), 4 * wave, rlo);
    }
    const int lohi = dbg_lohi(tiles[qp.tile_begin + t].lohi);
    const int lo = lohi & 0xff, hi_t = (lohi >> 8) & 0xff;
    int mi = -1;
    uint64_t rmask = 0;
    if constexpr (kMasked) {
      mi = dbg_mask(tile_mask[qp.tile_begin + t]);
      if (mi >= 0) rmask = masks[(int64_t)mi * 128 + row];
    }
    const bool diag = (t == T - 1) && mi < 0;
    const bool full = lo == 0 && hi_t == 64 && !diag && qp.nrows == 64 && mi < 0;
    const f16_t* K = lk[buf];
    const f16_t* V = lvv[buf];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      // a half with no key visible to this wave's rows adds exact zeros: skipped
      if (hi_t <= mb * 32 || lo >= mb * 32 + 32 || (diag && mb * 32 > nb * 32 + 31) || nb * 32 >= qp.nrows)
        continue;
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        s = mfma(ld8(K + kb0 + mb * 8 * kBrick + kstep(ks)), qf[ks], s);
        dp = mfma(ld8(V + kb0 + mb * 8 * kBrick + kstep(ks)), df[ks], dp);
      }
      if (full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, nl)) * (dp[r] + nD);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = mb * 32 + acc_row(r, hi);
          bool ok = key >= lo && key < hi_t && (!diag || key <= row) && row < qp.nrows;
          if constexpr (kMasked) ok = ok && (mi < 0 || ((rmask >> key) & 1ull));
          const float p = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, nl));
          s[r] = ok ? p * (dp[r] + nD) : 0.f;  // padding may hold NaN
        }
      }
      const f16x8 d0 = pack8(s, 0), d1 = pack8(s, 8);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        acc[a] = mfma(frag_tr(K + tb, mb * 2 + 0, a), d0, acc[a]);
        acc[a] = mfma(frag_tr(K + tb, mb * 2 + 1, a), d1, acc[a]);
      }
    }
    wait_all_loads();
    __syncthreads();
  }

  const float gscale = scale / pow2_scale(*dmax, kTopVO) / sv / sk;  // undo the operand scalings
  const bool valid = row < qp.nrows;
  const int64_t grow = (int64_t)qp.phys * 64 + row;
  TG* out = dq + (grow * Hq + h) * kD;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = a * 32 + 8 * j + 4 * hi + i;  // d < 64 pairs with d + 64 (block a + 2)
        const float g1 = acc[a][4 * j + i] * gscale, g2 = acc[a + 2][4 * j + i] * gscale;
        float r1 = 0.f, r2 = 0.f;
        if (valid) {
          const float2 c = cs ? cs[grow * (kD / 2) + d] : make_float2(1.f, 0.f);
          r1 = g1 * c.x + g2 * c.y;
          r2 = g2 * c.x - g1 * c.y;
        }
        st_f(out + d, r1);
        st_f(out + d + 64, r2);
      }
}

// Sum the two head-parity waves' dK (or dV) accumulators of every 32-key tile
// through LDS (parity 0 first, then 1: a fixed order), then scale, rotate dK back
// by R(pos)^T and write the pair's rows once.  Wave (kt, j) holds keys
// 32 kt .. 32 kt + 31 of the pair's 128 (page A: kt = 0, 1; page B: kt = 2, 3).
template <bool kRotate, typename TG>
__device__ __forceinline__ void dkdv_reduce_store(const f32x16 (&acc)[4], float* red, int kt, int j, bool active,
                                                  int hi, int l32, int tid, int physA, int physB, int rowsA,
                                                  int rowsB, int g, int Hkv, float mul,
                                                  const float2* __restrict__ cs, TG* __restrict__ out) {
  for (int jj = 0; jj < 2; ++jj) {
    __syncthreads();
    if (j == jj && active) {
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float* slot = red + (kt * 32 + acc_row(r, hi)) * (kD + 1) + b * 32 + l32;
          *slot = (jj == 0) ? acc[b][r] : *slot + acc[b][r];
        }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < 128 * 64; idx += 512) {
    const int k2 = idx / 64, i = idx % 64;  // key of the pair, column pair (i, i + 64)
    const int side = k2 >> 6, row = k2 & 63;
    const int page = side ? physB : physA;
    if (page < 0) continue;
    const int64_t grow = (int64_t)page * 64 + row;
    float a = red[k2 * (kD + 1) + i] * mul, b = red[k2 * (kD + 1) + i + 64] * mul;
    if (row >= (side ? rowsB : rowsA)) {
      a = b = 0.f;
    } else if (kRotate && cs) {
      const float2 c = cs[grow * (kD / 2) + i];
      const float a2 = a * c.x + b * c.y;
      b = b * c.x - a * c.y;
      a = a2;
    }
    TG* o = out + (grow * Hkv + g) * kD;
    st_f(o + i, a);
    st_f(o + i + 64, b);
  }
}

// dK, dV for a pair of KV pages (a node of one or two pages, or consecutive pages of a
// packed plan; or a lone page) and one KV head; nodes of three pages or more run in
// four-page groups (dkdv_group_kernel below).  Each 32-row reader step of the pair's merged reader list
// is taken as two half-steps, query heads 4 g + 2 hp + {0, 1} (hp = 0, 1).  Eight
// waves: wave (kt, j) serves keys 32 (kt % 2) .. of page kt / 2 and the query heads
// 4 g + j and 4 g + 2 + j, keeping its dK and dV (32 x 128 each) in accumulation
// registers and its K fragments in registers; the two waves of a SIMD share the
// key tile.  A half-step stages two heads' Q and dO rows (32 KiB) in LDS with
// direct loads issued by waves 0..3, double buffered: every staged byte now feeds 128 keys, so a pair
// moves half the staging bytes per product that one page would.  Within a
// half-step the products run as four MFMA chains S, dP, dV, dK (exponentials
// between the dP products, dS between the dV products); hidden keys get a
// per-lane -inf offset.  At the end the two head parities are summed through LDS in
// a fixed order and each page is written once: deterministic, no atomics.
//
// kMasked (packed page layouts): each step carries the two pages' mask ids (fetched with the
// step descriptors); a lane of a masked side reads its key's 64-bit query-row mask and
// zeroes P for the rows it hides (packed steps carry no causal rule).
template <typename TG, bool kMasked>
__global__ __launch_bounds__(512, 1) void dkdv_mfma_kernel(
    const f16_t* __restrict__ qn, const f16_t* __restrict__ kn, const f16_t* __restrict__ vn,
    const f16_t* __restrict__ dOn, const float2* __restrict__ ldd, const float2* __restrict__ cs,
    const uint32_t* __restrict__ dmax, const int32_t* __restrict__ pair_order, const int32_t* __restrict__ pairs,
    const int64_t* __restrict__ pair_off, const KStep* __restrict__ psteps, const KMask* __restrict__ pmasks,
    const uint64_t* __restrict__ masks, const int32_t* __restrict__ page_nrows,
    TG* __restrict__ dk, TG* __restrict__ dv, const uint32_t* __restrict__ amax, int n_pairs, int Hq, int Hkv,
    float sl2_raw, float scale) {
  // [buffer][head of the half-step][Q, dO][32 x 128] f16 (the first 65 KiB are reused
  // for the head-parity sum at the end), the V tiles of pages A and B, and
  // [buffer][head] the 32 rows' offsets: -lse / scale for S, then -D for dP
  __shared__ __attribute__((aligned(1024))) f16_t qd[2][2][2][kStepB];
  __shared__ __attribute__((aligned(1024))) f16_t lvp[2][kPageB];
  __shared__ __attribute__((aligned(16))) float lds_ld[2][2][64];
  int unit, g;
  if (!map_item(n_pairs, Hkv, unit, g)) return;
  // fp16 copies: sq q, sk k, sv v, sdo dO (powers of two), offsets in ldd in the same
  // units: P is exact, dS comes out as sdo sv dS, the sums as sdo dV and sdo sv sq dK / scale
  const float sq = pow2_scale(amax[0], kTopQK), sk = pow2_scale(amax[1], kTopQK), sv = pow2_scale(amax[2], kTopVO);
  const float sl2 = sl2_raw / sq / sk;
  const int pr = dbg_index(pair_order[unit], n_pairs, kDbgPair);
  const int physA = dbg_page(pairs[2 * pr], kDbgPair);
  int physB = pairs[2 * pr + 1];
  if (physB != -1) physB = dbg_page(physB, kDbgPair);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave index: uniform
  const int l32 = lane & 31, hi = lane >> 5;
  const int kt = wave & 3, j = wave >> 2;  // key tile of the pair, head parity
  const int side = kt >> 1, kb = kt & 1;
  const int page = side ? physB : physA;
  const bool active = page >= 0;  // page B of a lone page: this wave only stages

  f16x8 kf[8];
  {
    const int64_t base = ((int64_t)(active ? page : physA) * Hkv + g) * 64 * kD;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kf[ks] = ld8(kn + base + (kb * 32 + l32) * kD + ks * 16 + hi * 8);
    // wave w stages bricks 4 (w % 4) .. of page w / 4's V tile
    const int vp = (wave >> 2) ? physB : physA;
    if (vp >= 0)
      stage_bricks<4>(lvp[wave >> 2], tile_rsrc(vn + ((int64_t)vp * Hkv + g) * kTile, kTile * 2), 4 * (wave & 3),
                      brick_lane_off(lane));
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) pin(kf[ks]);
  }
  f32x16 adk[4], adv[4];  // [d block]
#pragma unroll
  for (int b = 0; b < 4; ++b) adk[b] = adv[b] = zero16();

  // Step descriptors are uniform and come through the scalar cache ahead of their
  // use (no vector-memory wait for them, which would also wait for the staging loads).
  int64_t s_begin = pair_off[pr];
  int n_steps = (int)(pair_off[pr + 1] - s_begin);
#ifdef DAG_DEBUG
  if (s_begin < 0 || n_steps < 1 || s_begin + n_steps > g_dbg_lim.steps) {
    dbg_fail(kDbgStepRange, s_begin);
    s_begin = 0;
    n_steps = 1;
  }
#endif
  const int n_units = 2 * n_steps;
  const KStep* kst = psteps + s_begin;
  KStep cur = dbg_step(kst[0]);
  KStep nxt = dbg_step(kst[min(1, n_steps - 1)]);
  KStep n2 = dbg_step(kst[min(2, n_steps - 1)]);
  KMask cur_m{-1, -1}, nxt_m{-1, -1}, n2_m{-1, -1};
  if constexpr (kMasked) {
    cur_m = pmasks[s_begin];
    nxt_m = pmasks[s_begin + min(1, n_steps - 1)];
    n2_m = pmasks[s_begin + min(2, n_steps - 1)];
    cur_m.a = dbg_mask(cur_m.a), cur_m.b = dbg_mask(cur_m.b);
    nxt_m.a = dbg_mask(nxt_m.a), nxt_m.b = dbg_mask(nxt_m.b);
    n2_m.a = dbg_mask(n2_m.a), n2_m.b = dbg_mask(n2_m.b);
  }
  // staging by waves 0..3 (one per SIMD; measured faster than all eight): head sj of the
  // half-step, tensor ts (0: Q, 1: dO), all eight bricks
  const bool stager = wave < 4;
  const int sj = wave & 1, ts = (wave >> 1) & 1;
  const uint32_t rlo = brick_lane_off(lane);
  const uint32_t llo = (uint32_t)((2 * (lane & 31) + (lane >> 5)) * 4);
  const f16_t* stsrc = ts == 0 ? qn : dOn;
  auto head_row0 = [&](const KStep& d, int hp, int jj) -> int64_t {  // first staged row of head jj
    return ((int64_t)d.qph * Hq + g * 4 + 2 * hp + jj) * 64 + (d.info & 1) * 32;
  };
  {
    const int64_t r0 = head_row0(cur, 0, sj);
    if (stager) {
      stage_bricks<8>(qd[0][sj][ts], tile_rsrc(stsrc + r0 * kD, 32 * kD * 2), 0, rlo);
      if (ts == 0) dma4(&lds_ld[0][sj][0], llo, tile_rsrc(ldd + r0, 256), 0);
    }
  }
  wait_all_loads();
  __syncthreads();

  const int key = kb * 32 + l32;
  const int qb = frag_base(l32, hi), vb = frag_base(key, hi), tb = tr_base(lane);
  for (int u = 0; u < n_units; ++u) {
    const int buf = u & 1, hp = u & 1;
    // staging of unit u + 1 (the same step's second half, or the next step's first);
    // on the last unit it repeats this one into the idle buffer (harmless)
    const KStep& sd = hp ? nxt : cur;
    const int64_t nr0 = head_row0(sd, hp ^ 1, sj);
    const i32x4 nrs = tile_rsrc(stsrc + nr0 * kD, 32 * kD * 2);
    f16_t* ndst = qd[buf ^ 1][sj][ts];
    const bool offs = stager && ts == 0;

    const uint32_t inf = ((uint32_t)cur.info >> (16 * side)) & 0xffffu;
    uint64_t kmask = 0;
    int mi = -1;
    if constexpr (kMasked) {
      mi = side ? cur_m.b : cur_m.a;
      if (mi >= 0 && active) kmask = masks[(int64_t)mi * 128 + 64 + kb * 32 + l32];
    }
    const int rb = cur.info & 1, lo = (inf >> 1) & 0x7f, hi_t = (inf >> 8) & 0x7f;
    const bool diag = (inf >> 15) & 1;
    if (!active || lo >= hi_t) {
      // this wave's page is not read by this step: stage only
      if (stager) {
#pragma unroll
        for (int i = 0; i < 8; ++i) dma16(ndst + i * kBrick, rlo, nrs, i * 4 * kD * 2);
      }
      if (offs) dma4(&lds_ld[buf ^ 1][sj][0], llo, tile_rsrc(ldd + nr0, 256), 0);
    } else {
      const f16_t* Qt = qd[buf][j][0];
      const f16_t* Dt = qd[buf][j][1];
      const f16_t* Vp = lvp[side];
      // S = Q K^T - lse / scale, dP = dO V^T - D: 32 rows (M) x this wave's 32 keys (N);
      // lane holds key kb*32 + l32 and rows rb*32 + acc_row(r, hi), so the offsets of
      // its rows come as four runs of four consecutive floats straight into the
      // accumulators
      f32x16 s, dp;
      {
        const float* L = lds_ld[buf][j];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 a = *reinterpret_cast<const float4*>(L + 8 * q4 + 4 * hi);
          const float4 b = *reinterpret_cast<const float4*>(L + 32 + 8 * q4 + 4 * hi);
          s[4 * q4] = a.x, s[4 * q4 + 1] = a.y, s[4 * q4 + 2] = a.z, s[4 * q4 + 3] = a.w;
          dp[4 * q4] = b.x, dp[4 * q4 + 1] = b.y, dp[4 * q4 + 2] = b.z, dp[4 * q4 + 3] = b.w;
        }
      }
      // The four products run as four chains of eight MFMAs, S, dP, dV, dK, and each
      // chain carries the vector work of the previous one: the exponentials of S run
      // between the dP products, dS = P (dP - D) between the dV products.  A key
      // outside the step's visible range gets -inf added before the exponential.
      const float koff = (key >= lo && key < hi_t) ? 0.f : -INFINITY;
      {
        // S: Q fragments read one k-step ahead; the next unit's staging goes out one
        // load per k-step (waves 0..3)
        f16x8 qa[2];
        qa[0] = ld8(Qt + qb);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          if (ks < 7) qa[(ks + 1) & 1] = ld8(Qt + qb + kstep(ks + 1));
          s = mfma(qa[ks & 1], kf[ks], s);
          if (stager) dma16(ndst + ks * kBrick, rlo, nrs, ks * 4 * kD * 2);
        }
        if (offs) dma4(&lds_ld[buf ^ 1][sj][0], llo, tile_rsrc(ldd + nr0, 256), 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
        for (int ks = 0; ks < 7; ++ks) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      {
        // dP, with P = 2^(S scale log2 e) computed in between
        f16x8 da[2], va[2];
        da[0] = ld8(Dt + qb);
        va[0] = ld8(Vp + vb);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          if (ks < 7) {
            da[(ks + 1) & 1] = ld8(Dt + qb + kstep(ks + 1));
            va[(ks + 1) & 1] = ld8(Vp + vb + kstep(ks + 1));
          }
          dp = mfma(da[ks & 1], va[ks & 1], dp);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, koff));
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          if (ks < 7) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (diag) {
        // the reader's own page: key <= row (a hidden score may have overflowed: select)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = key <= rb * 32 + acc_row(r, hi) ? s[r] : 0.f;
      }
      if constexpr (kMasked) {
        // packed: the rows of the step that see this lane's key
        if (mi >= 0) {
          const uint32_t rows = (uint32_t)(kmask >> (32 * (cur.info & 1)));
#pragma unroll
          for (int r = 0; r < 16; ++r) s[r] = ((rows >> acc_row(r, hi)) & 1u) ? s[r] : 0.f;
        }
      }
      // Padding rows need no mask: their Q and dO rows and offsets are zero, so they add
      // exact zeros to dV and dK.
      const f16x8 pf0 = pack8(s, 0), pf1 = pack8(s, 8);
      // dV += P^T dO, then dK += dS^T Q: keys (M) x d (N), the 32 rows contracted; d
      // block b + 1's fragments (transpose reads) are read while block b's products run
      const f16_t* Dtb = Dt + tb;
      const f16_t* Qtb = Qt + tb;
      f16x8 sf0, sf1;
      f16x8 frq[2];
      {
        f16x8 fr[2][2];
        fr[0][0] = frag_tr(Dtb, 0, 0);
        fr[0][1] = frag_tr(Dtb, 1, 0);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (b < 3) {
            fr[(b + 1) & 1][0] = frag_tr(Dtb, 0, b + 1);
            fr[(b + 1) & 1][1] = frag_tr(Dtb, 1, b + 1);
          }
          adv[b] = mfma(pf0, fr[b & 1][0], adv[b]);
          adv[b] = mfma(pf1, fr[b & 1][1], adv[b]);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] *= s[r];
        sf0 = pack8(dp, 0);
        sf1 = pack8(dp, 8);
        frq[0] = frag_tr(Qtb, 0, 0);
        frq[1] = frag_tr(Qtb, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      {
        f16x8 fr[2][2];
        fr[0][0] = frq[0];
        fr[0][1] = frq[1];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (b < 3) {
            fr[(b + 1) & 1][0] = frag_tr(Qtb, 0, b + 1);
            fr[(b + 1) & 1][1] = frag_tr(Qtb, 1, b + 1);
          }
          adk[b] = mfma(sf0, fr[b & 1][0], adk[b]);
          adk[b] = mfma(sf1, fr[b & 1][1], adk[b]);
        }
#pragma unroll
        for (int b = 0; b < 3; ++b) {
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
    }
    // the descriptor three steps ahead: issued here, where the closing wait covers it
    __builtin_amdgcn_sched_barrier(0);
    const KStep n3 = dbg_step(kst[min((u >> 1) + 3, n_steps - 1)]);
    KMask n3_m{-1, -1};
    if constexpr (kMasked) {
      n3_m = pmasks[s_begin + min((u >> 1) + 3, n_steps - 1)];
      n3_m.a = dbg_mask(n3_m.a), n3_m.b = dbg_mask(n3_m.b);
    }
    wait_all_loads();
    __syncthreads();
    if (hp) {
      cur = nxt;
      nxt = n2;
      n2 = n3;
      if constexpr (kMasked) {
        cur_m = nxt_m;
        nxt_m = n2_m;
        n2_m = n3_m;
      }
    }
  }

  const float inv_sdo = 1.f / pow2_scale(*dmax, kTopVO);  // undo the operand scalings
  float* red = reinterpret_cast<float*>(&qd[0][0][0][0]);  // [128][129] fp32
  const int rowsA = page_nrows[physA], rowsB = physB >= 0 ? page_nrows[physB] : 0;
  // sum the two head parities in order 0, 1 through LDS, then write dk (scaled,
  // un-rotated) and dv for both pages
  dkdv_reduce_store<true>(adk, red, kt, j, active, hi, l32, tid, physA, physB, rowsA, rowsB, g, Hkv,
                          inv_sdo * scale / sv / sq, cs, dk);
  dkdv_reduce_store<false>(adv, red, kt, j, active, hi, l32, tid, physA, physB, rowsA, rowsB, g, Hkv, inv_sdo,
                           cs, dv);
}

// Write the accumulated dK (or dV) of two of the group's pages (slots 2 hf, 2 hf + 1)
// through LDS, so that every row goes out as whole 256-byte runs: the four waves of
// those pages park their 32 x 128 blocks, then all threads scale, rotate dK back by
// R(pos)^T and store.  Each key has one accumulating wave: no sums, no atomics.
template <bool kRotate, typename TG>
__device__ __forceinline__ void dkdv_store_half(const f32x16 (&acc)[4], float* red, int hf, int ps, int kb,
                                                bool active, int hi, int l32, int tid, const int (&phys)[kGroup],
                                                const int (&nrows)[kGroup], int g, int Hkv, float mul,
                                                const float2* __restrict__ cs, TG* __restrict__ out) {
  __syncthreads();
  if ((ps >> 1) == hf && active) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[((ps & 1) * 64 + kb * 32 + acc_row(r, hi)) * (kD + 1) + b * 32 + l32] = acc[b][r];
  }
  __syncthreads();
  for (int idx = tid; idx < 128 * 64; idx += 512) {
    const int k2 = idx / 64, i = idx % 64;  // key of the two pages, column pair (i, i + 64)
    const bool second = k2 >= 64;
    const int row = k2 & 63;
    // selects rather than an index: an indexed private array would live in LDS
    const int page = second ? phys[2 * hf + 1] : phys[2 * hf];
    if (page < 0) continue;
    const int64_t grow = (int64_t)page * 64 + row;
    float a = red[k2 * (kD + 1) + i] * mul, b = red[k2 * (kD + 1) + i + 64] * mul;
    if (row >= (second ? nrows[2 * hf + 1] : nrows[2 * hf])) {
      a = b = 0.f;
    } else if (kRotate && cs) {
      const float2 c = cs[grow * (kD / 2) + i];
      const float a2 = a * c.x + b * c.y;
      b = b * c.x - a * c.y;
      a = a2;
    }
    TG* o = out + (grow * Hkv + g) * kD;
    st_f(o + i, a);
    st_f(o + i + 64, b);
  }
}

// dK, dV for a group of up to four KV pages (consecutive pages of one node, or of the
// packed page sequence) and one KV head.  Eight waves: wave (ps, kb) owns keys
// 32 kb .. 32 kb + 31 of the group's page ps and keeps their dK and dV (32 x 128 each)
// in accumulation registers and their K fragments in registers; the V tiles of the
// four pages sit in LDS.  Each 32-row reader step of the group's merged reader list is
// taken as two half-steps of two query heads (4 g + 2 hp + {0, 1}): a half-step stages
// those heads' Q and dO rows (32 KiB) in LDS with direct loads, double buffered, and
// every wave runs both heads through it, so each staged byte feeds 256 keys.  Per head
// the products run as four MFMA chains S, dP, dV, dK (exponentials between the dP
// products, dS between the dV products); hidden keys get a per-lane -inf offset.  A
// wave whose page the step does not read only stages.  Every key has one owner wave,
// so the pages are written once at the end: deterministic, no atomics.  Plans with one
// node per page only (packed plans run every page in pairs).
template <typename TG>
__global__ __launch_bounds__(512, 1) void dkdv_group_kernel(
    const f16_t* __restrict__ qn, const f16_t* __restrict__ kn, const f16_t* __restrict__ vn,
    const f16_t* __restrict__ dOn, const float2* __restrict__ ldd, const float2* __restrict__ cs,
    const uint32_t* __restrict__ dmax, const int32_t* __restrict__ group_order, const int32_t* __restrict__ groups,
    const int64_t* __restrict__ group_off, const GStep* __restrict__ gsteps, const int32_t* __restrict__ page_nrows,
    TG* __restrict__ dk, TG* __restrict__ dv, const uint32_t* __restrict__ amax, int n_groups, int Hq, int Hkv,
    float sl2_raw, float scale) {
  // [buffer][head of the half-step][Q, dO][32 x 128] f16 (the first 65 KiB are reused
  // for the output staging at the end), the V tiles of the four pages, and
  // [buffer][head] the 32 rows' offsets: -lse / scale for S, then -D for dP
  __shared__ __attribute__((aligned(1024))) f16_t qd[2][2][2][kStepB];
  __shared__ __attribute__((aligned(1024))) f16_t lvp[kGroup][kPageB];
  __shared__ __attribute__((aligned(16))) float lds_ld[2][2][64];
  int unit, g;
  if (!map_item(n_groups, Hkv, unit, g)) return;
  // fp16 copies: sq q, sk k, sv v, sdo dO (powers of two), offsets in ldd in the same
  // units: P is exact, dS comes out as sdo sv dS, the sums as sdo dV and sdo sv sq dK / scale
  const float sq = pow2_scale(amax[0], kTopQK), sk = pow2_scale(amax[1], kTopQK), sv = pow2_scale(amax[2], kTopVO);
  const float sl2 = sl2_raw / sq / sk;
  const int gr = dbg_index(group_order[unit], n_groups, kDbgGroup);
  int phys[kGroup];
#pragma unroll
  for (int i = 0; i < kGroup; ++i) {
    phys[i] = groups[kGroup * gr + i];
    if (phys[i] != -1) phys[i] = dbg_page(phys[i], kDbgGroup);
  }
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave index: uniform
  const int l32 = lane & 31, hi = lane >> 5;
  const int ps = wave >> 1, kb = wave & 1;  // page slot of the group, key half of the page
  // uniform selects rather than an index (an indexed private array would live in LDS)
  const int page = ps == 0 ? phys[0] : ps == 1 ? phys[1] : ps == 2 ? phys[2] : phys[3];
  const bool active = page >= 0;  // a group with fewer pages: this wave only stages

  f16x8 kf[8];
  {
    const int64_t base = ((int64_t)(active ? page : phys[0]) * Hkv + g) * 64 * kD;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kf[ks] = ld8(kn + base + (kb * 32 + l32) * kD + ks * 16 + hi * 8);
    // the two waves of page ps stage its V tile, eight bricks each
    if (active)
      stage_bricks<8>(lvp[ps], tile_rsrc(vn + ((int64_t)page * Hkv + g) * kTile, kTile * 2), 8 * kb,
                      brick_lane_off(lane));
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) pin(kf[ks]);
  }
  f32x16 adk[4], adv[4];  // [d block]
#pragma unroll
  for (int b = 0; b < 4; ++b) adk[b] = adv[b] = zero16();

  // Step descriptors are uniform and come through the scalar cache ahead of their
  // use (no vector-memory wait for them, which would also wait for the staging loads).
  int64_t s_begin = group_off[gr];
  int n_steps = (int)(group_off[gr + 1] - s_begin);
#ifdef DAG_DEBUG
  if (s_begin < 0 || n_steps < 1 || s_begin + n_steps > g_dbg_lim.gsteps) {
    dbg_fail(kDbgStepRange, s_begin);
    s_begin = 0;
    n_steps = 1;
  }
#endif
  const int n_units = 2 * n_steps;
  const GStep* kst = gsteps + s_begin;
  GStep cur = dbg_gstep(kst[0]);
  GStep nxt = dbg_gstep(kst[min(1, n_steps - 1)]);
  // staging by all eight waves (measured faster than by four or two here, where every
  // wave runs two heads per half-step): head sj of the half-step, tensor ts (0: Q,
  // 1: dO), bricks sb0 .. sb0 + 3
  const int sj = wave & 1, ts = (wave >> 1) & 1, sb0 = 4 * (wave >> 2);
  const uint32_t rlo = brick_lane_off(lane);
  const uint32_t llo = (uint32_t)((2 * (lane & 31) + (lane >> 5)) * 4);
  const f16_t* stsrc = ts == 0 ? qn : dOn;
  auto head_row0 = [&](const GStep& d, int hp, int jj) -> int64_t {  // first staged row of head jj
    return ((int64_t)d.qph * Hq + g * 4 + 2 * hp + jj) * 64 + d.rb * 32;
  };
  {
    const int64_t r0 = head_row0(cur, 0, sj);
    stage_bricks<4>(qd[0][sj][ts], tile_rsrc(stsrc + r0 * kD, 32 * kD * 2), sb0, rlo);
    if (ts == 0 && sb0 == 0) dma4(&lds_ld[0][sj][0], llo, tile_rsrc(ldd + r0, 256), 0);
  }
  wait_all_loads();
  __syncthreads();

  const int key = kb * 32 + l32;
  const int qb = frag_base(l32, hi), vb = frag_base(key, hi), tb = tr_base(lane);
  const f16_t* Vp = lvp[ps];
  for (int u = 0; u < n_units; ++u) {
    const int buf = u & 1, hp = u & 1;
    // staging of unit u + 1 (the same step's second half, or the next step's first);
    // on the last unit it repeats this one into the idle buffer (harmless)
    const GStep& sd = hp ? nxt : cur;
    const int64_t nr0 = head_row0(sd, hp ^ 1, sj);
    const i32x4 nrs = tile_rsrc(stsrc + nr0 * kD, 32 * kD * 2);
    f16_t* ndst = qd[buf ^ 1][sj][ts];
    const bool offs = ts == 0 && sb0 == 0;

    const uint32_t vw = (ps & 2) ? cur.vis[1] : cur.vis[0];  // uniform select, see above
    const uint32_t inf = ((ps & 1) ? vw >> 16 : vw) & 0xffffu;
    const int lo = gvis_lo(inf), hi_t = gvis_hi(inf);
    const bool diag = gvis_diag(inf);
    if (!active || lo >= hi_t) {
      // this wave's page is not read by this step: stage only
#pragma unroll
      for (int i = 0; i < 4; ++i) dma16(ndst + (sb0 + i) * kBrick, rlo, nrs, (sb0 + i) * 4 * kD * 2);
      if (offs) dma4(&lds_ld[buf ^ 1][sj][0], llo, tile_rsrc(ldd + nr0, 256), 0);
    } else {
      // A key outside the step's visible range gets -inf added before the exponential.
      const float koff = (key >= lo && key < hi_t) ? 0.f : -INFINITY;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const f16_t* Qt = qd[buf][jj][0];
        const f16_t* Dt = qd[buf][jj][1];
        // S = Q K^T - lse / scale, dP = dO V^T - D: 32 rows (M) x this wave's 32 keys (N);
        // lane holds key kb*32 + l32 and rows rb*32 + acc_row(r, hi), so the offsets of
        // its rows come as four runs of four consecutive floats straight into the
        // accumulators
        f32x16 s, dp;
        {
          const float* L = lds_ld[buf][jj];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const float4 a = *reinterpret_cast<const float4*>(L + 8 * q4 + 4 * hi);
            const float4 b = *reinterpret_cast<const float4*>(L + 32 + 8 * q4 + 4 * hi);
            s[4 * q4] = a.x, s[4 * q4 + 1] = a.y, s[4 * q4 + 2] = a.z, s[4 * q4 + 3] = a.w;
            dp[4 * q4] = b.x, dp[4 * q4 + 1] = b.y, dp[4 * q4 + 2] = b.z, dp[4 * q4 + 3] = b.w;
          }
        }
        // The four products run as four chains of eight MFMAs, S, dP, dV, dK, and each
        // chain carries the vector work of the previous one: the exponentials of S run
        // between the dP products, dS = P (dP - D) between the dV products.
        {
          // S: Q fragments read one k-step ahead; with the first head, the next unit's
          // staging goes out one load per two k-steps
          f16x8 qa[2];
          qa[0] = ld8(Qt + qb);
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) {
            if (ks < 7) qa[(ks + 1) & 1] = ld8(Qt + qb + kstep(ks + 1));
            s = mfma(qa[ks & 1], kf[ks], s);
            if (jj == 0 && (ks & 1) == 0)
              dma16(ndst + (sb0 + ks / 2) * kBrick, rlo, nrs, (sb0 + ks / 2) * 4 * kD * 2);
          }
          if (jj == 0 && offs) dma4(&lds_ld[buf ^ 1][sj][0], llo, tile_rsrc(ldd + nr0, 256), 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
          for (int ks = 0; ks < 7; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        {
          // dP, with P = 2^(S scale log2 e) computed in between
          f16x8 da[2], va[2];
          da[0] = ld8(Dt + qb);
          va[0] = ld8(Vp + vb);
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) {
            if (ks < 7) {
              da[(ks + 1) & 1] = ld8(Dt + qb + kstep(ks + 1));
              va[(ks + 1) & 1] = ld8(Vp + vb + kstep(ks + 1));
            }
            dp = mfma(da[ks & 1], va[ks & 1], dp);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, koff));
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) {
            if (ks < 7) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (diag) {
          // the reader's own page: key <= row (a hidden score may have overflowed: select);
          // compared as key - row0 <= acc_row(r, 0), a constant per element
          const int t = key - cur.rb * 32 - 4 * hi;
#pragma unroll
          for (int r = 0; r < 16; ++r) s[r] = t <= acc_row(r, 0) ? s[r] : 0.f;
        }
        // Padding rows need no mask: their Q and dO rows and offsets are zero, so they add
        // exact zeros to dV and dK.
        const f16x8 pf0 = pack8(s, 0), pf1 = pack8(s, 8);
        // dV += P^T dO, then dK += dS^T Q: keys (M) x d (N), the 32 rows contracted; d
        // block b + 1's fragments (transpose reads) are read while block b's products run
        const f16_t* Dtb = Dt + tb;
        const f16_t* Qtb = Qt + tb;
        f16x8 sf0, sf1;
        f16x8 frq[2];
        {
          f16x8 fr[2][2];
          fr[0][0] = frag_tr(Dtb, 0, 0);
          fr[0][1] = frag_tr(Dtb, 1, 0);
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            if (b < 3) {
              fr[(b + 1) & 1][0] = frag_tr(Dtb, 0, b + 1);
              fr[(b + 1) & 1][1] = frag_tr(Dtb, 1, b + 1);
            }
            adv[b] = mfma(pf0, fr[b & 1][0], adv[b]);
            adv[b] = mfma(pf1, fr[b & 1][1], adv[b]);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) dp[r] *= s[r];
          sf0 = pack8(dp, 0);
          sf1 = pack8(dp, 8);
          frq[0] = frag_tr(Qtb, 0, 0);
          frq[1] = frag_tr(Qtb, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        {
          f16x8 fr[2][2];
          fr[0][0] = frq[0];
          fr[0][1] = frq[1];
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            if (b < 3) {
              fr[(b + 1) & 1][0] = frag_tr(Qtb, 0, b + 1);
              fr[(b + 1) & 1][1] = frag_tr(Qtb, 1, b + 1);
            }
            adk[b] = mfma(sf0, fr[b & 1][0], adk[b]);
            adk[b] = mfma(sf1, fr[b & 1][1], adk[b]);
          }
#pragma unroll
          for (int b = 0; b < 3; ++b) {
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // after a step's second half, the descriptor two steps ahead: first needed by the
    // staging one unit later, so a whole unit covers the scalar load
    __builtin_amdgcn_sched_barrier(0);
    if (hp) {
      cur = nxt;
      nxt = dbg_gstep(kst[min((u >> 1) + 2, n_steps - 1)]);
    }
    wait_all_loads();
    __syncthreads();
  }

  const float inv_sdo = 1.f / pow2_scale(*dmax, kTopVO);  // undo the operand scalings
  float* red = reinterpret_cast<float*>(&qd[0][0][0][0]);  // [128][129] fp32
  int nrows[kGroup];
#pragma unroll
  for (int i = 0; i < kGroup; ++i) nrows[i] = phys[i] >= 0 ? page_nrows[phys[i]] : 0;
  // dk (scaled, un-rotated) and dv, two pages at a time
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    dkdv_store_half<true>(adk, red, hf, ps, kb, active, hi, l32, tid, phys, nrows, g, Hkv, inv_sdo * scale / sv / sq,
                          cs, dk);
    dkdv_store_half<false>(adv, red, hf, ps, kb, active, hi, l32, tid, phys, nrows, g, Hkv, inv_sdo, cs, dv);
  }
}

// ---------------------------------------------------------------------------
// Generic kernels (any even head dim <= 128, any GQA ratio, bf16 or fp32 tensors).
// One thread per query row (forward, dQ) or key row (dK/dV); fp32 throughout.
// ---------------------------------------------------------------------------

constexpr int kMaxD = 128;

template <typename T>
__global__ __launch_bounds__(64) void fwd_simple_kernel(
    const float* __restrict__ qn, const float* __restrict__ kn, const T* __restrict__ v,
    const QPage* __restrict__ qpages, const int32_t* __restrict__ order, const Tile* __restrict__ tiles,
    T* __restrict__ o, float* __restrict__ lse, T* __restrict__ o_lo, int Hq, int Hkv, int D, float scale) {
  const int item = blockIdx.x;
  const QPage qp = qpages[order[item / Hq]];
  const int h = item % Hq, g = h / (Hq / Hkv);
  const int row = threadIdx.x;
  float q[kMaxD], acc[kMaxD];
  const float* qrow = qn + (((int64_t)qp.phys * Hq + h) * 64 + row) * D;
  for (int d = 0; d < D; ++d) {
    q[d] = qrow[d];
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int t = 0; t < qp.tile_count; ++t) {
    const Tile tl = tiles[qp.tile_begin + t];
    const int lo = tl.lohi & 0xff, hi_t = (tl.lohi >> 8) & 0xff;
    const bool diag = (t == qp.tile_count - 1);
    for (int key = lo; key < hi_t; ++key) {
      if (diag && key > row) break;
      const float* krow = kn + (((int64_t)tl.page * Hkv + g) * 64 + key) * D;
      float s = 0.f;
      for (int d = 0; d < D; ++d) s = fmaf(q[d], krow[d], s);
      s *= scale;
      const float mn = fmaxf(m, s);
      const float alpha = expf(m - mn), p = expf(s - mn);
      l = l * alpha + p;
      m = mn;
      const T* vrow = v + (((int64_t)tl.page * 64 + key) * Hkv + g) * D;
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, ld_f(vrow + d), acc[d] * alpha);
    }
  }
  const bool valid = row < qp.nrows;
  const int64_t grow = (int64_t)qp.phys * 64 + row;
  for (int d = 0; d < D; ++d) {
    const float x = valid ? acc[d] / l : 0.f;
    st_f(o + (grow * Hq + h) * D + d, x);
    if (o_lo) st_f(o_lo + (grow * Hq + h) * D + d, x - ld_f(o + (grow * Hq + h) * D + d));
  }
  lse[grow * Hq + h] = valid ? m + logf(l) : 0.f;
}

template <typename T, typename TG>
__global__ __launch_bounds__(64) void dq_simple_kernel(
    const float* __restrict__ qn, const float* __restrict__ kn, const T* __restrict__ v,
    const T* __restrict__ dO, const float2* __restrict__ ldd, const float2* __restrict__ cs,
    const QPage* __restrict__ qpages, const int32_t* __restrict__ order, const Tile* __restrict__ tiles,
    TG* __restrict__ dq, int Hq, int Hkv, int D, float scale) {
  const int item = blockIdx.x;
  const QPage qp = qpages[order[item / Hq]];
  const int h = item % Hq, g = h / (Hq / Hkv);
  const int row = threadIdx.x;
  const int64_t grow = (int64_t)qp.phys * 64 + row;
  float q[kMaxD], gd[kMaxD], acc[kMaxD];
  const float* qrow = qn + (((int64_t)qp.phys * Hq + h) * 64 + row) * D;
  for (int d = 0; d < D; ++d) {
    q[d] = qrow[d];
    gd[d] = ld_f(dO + (grow * Hq + h) * D + d);
    acc[d] = 0.f;
  }
  const float2 lD = ldd[((int64_t)qp.phys * Hq + h) * 64 + row];
  const float lse_n = -lD.x * scale;
  const bool valid = row < qp.nrows;
  if (valid)
    for (int t = 0; t < qp.tile_count; ++t) {
      const Tile tl = tiles[qp.tile_begin + t];
      const int lo = tl.lohi & 0xff, hi_t = (tl.lohi >> 8) & 0xff;
      const bool diag = (t == qp.tile_count - 1);
      for (int key = lo; key < hi_t; ++key) {
        if (diag && key > row) break;
        const float* krow = kn + (((int64_t)tl.page * Hkv + g) * 64 + key) * D;
        const T* vrow = v + (((int64_t)tl.page * 64 + key) * Hkv + g) * D;
        float s = 0.f, dp = 0.f;
        for (int d = 0; d < D; ++d) {
          s = fmaf(q[d], krow[d], s);
          dp = fmaf(gd[d], ld_f(vrow + d), dp);
        }
        const float p = expf(s * scale - lse_n);
        const float ds = p * (dp + lD.y) * scale;
        for (int d = 0; d < D; ++d) acc[d] = fmaf(ds, krow[d], acc[d]);
      }
    }
  const int half = D / 2;
  for (int i = 0; i < half; ++i) {
    float a = acc[i], b = acc[i + half];
    if (cs && valid) {
      const float2 c = cs[grow * half + i];
      const float a2 = a * c.x + b * c.y;
      b = b * c.x - a * c.y;
      a = a2;
    }
    st_f(dq + (grow * Hq + h) * D + i, valid ? a : 0.f);
    st_f(dq + (grow * Hq + h) * D + i + half, valid ? b : 0.f);
  }
}

template <typename T, typename TG>
__global__ __launch_bounds__(64) void dkdv_simple_kernel(
    const float* __restrict__ qn, const float* __restrict__ kn, const T* __restrict__ v,
    const T* __restrict__ dO, const float2* __restrict__ ldd, const float2* __restrict__ cs,
    const int32_t* __restrict__ order, const int32_t* __restrict__ kv_off,
    const KEntry* __restrict__ ents, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ page_nrows, TG* __restrict__ dk, TG* __restrict__ dv, int Hq, int Hkv,
    int D, float scale) {
  const int item = blockIdx.x;
  const int page = order[item / Hkv];
  const int g = item % Hkv;
  const int key = threadIdx.x;
  const int64_t grow = (int64_t)page * 64 + key;
  const bool valid = key < page_nrows[page];
  float k[kMaxD], vv[kMaxD], ak[kMaxD], av[kMaxD];
  const float* krow = kn + (((int64_t)page * Hkv + g) * 64 + key) * D;
  for (int d = 0; d < D; ++d) {
    k[d] = krow[d];
    vv[d] = ld_f(v + (grow * Hkv + g) * D + d);
    ak[d] = av[d] = 0.f;
  }
  const int rep = Hq / Hkv;
  if (valid)
    for (int e = kv_off[page]; e < kv_off[page + 1]; ++e) {
      const KEntry ent = ents[e];
      const int lo = ent.lohi_diag & 0xff, hi_t = (ent.lohi_diag >> 8) & 0xff;
      const bool diag = (ent.lohi_diag >> 16) & 1;
      if (key < lo || key >= hi_t) continue;
      for (int lq = ent.lq0; lq < ent.lq1; ++lq) {
        const int qph = page_table[ent.slot_base + lq];
        const int nrows = page_nrows[qph];
        for (int r = diag ? key : 0; r < nrows; ++r) {
          for (int hh = 0; hh < rep; ++hh) {
            const int h = g * rep + hh;
            const float* qrow = qn + (((int64_t)qph * Hq + h) * 64 + r) * D;
            const T* drow = dO + (((int64_t)qph * 64 + r) * Hq + h) * D;
            const float2 lD = ldd[((int64_t)qph * Hq + h) * 64 + r];
            float s = 0.f, dp = 0.f;
            for (int d = 0; d < D; ++d) {
              s = fmaf(qrow[d], k[d], s);
              dp = fmaf(ld_f(drow + d), vv[d], dp);
            }
            const float p = expf(s * scale + lD.x * scale);
            const float ds = p * (dp + lD.y) * scale;
            for (int d = 0; d < D; ++d) {
              av[d] = fmaf(p, ld_f(drow + d), av[d]);
              ak[d] = fmaf(ds, qrow[d], ak[d]);
            }
          }
        }
      }
    }
  const int half = D / 2;
  for (int i = 0; i < half; ++i) {
    float a = ak[i], b = ak[i + half];
    if (cs && valid) {
      const float2 c = cs[grow * half + i];
      const float a2 = a * c.x + b * c.y;
      b = b * c.x - a * c.y;
      a = a2;
    }
    st_f(dk + (grow * Hkv + g) * D + i, valid ? a : 0.f);
    st_f(dk + (grow * Hkv + g) * D + i + half, valid ? b : 0.f);
  }
  for (int d = 0; d < D; ++d) st_f(dv + (grow * Hkv + g) * D + d, valid ? av[d] : 0.f);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

static inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

void launch_cs(const LaunchShape& s, const int32_t* pos_of_row, float2* cs, hipStream_t st) {
  const int half = s.D / 2;
  cs_kernel<<<blocks_for(s.C * half, 256), 256, 0, st>>>(pos_of_row, cs, s.C, half, s.log2_base, s.D);
}

template <typename Tin, typename Tout>
void launch_relayout(const LaunchShape& s, const Tin* x, const float2* cs, const int32_t* page_nrows,
                     Tout* out_n, Tout* out_t, int H, hipStream_t st) {
  const size_t lds = (size_t)64 * (s.D + 1) * sizeof(float);
  relayout_kernel<Tin, Tout><<<(unsigned)(s.pages * H), 256, lds, st>>>(x, cs, page_nrows, out_n, out_t, H, s.D);
}

template <typename T>
void launch_rowdot(const LaunchShape& s, const T* o, const T* o_lo, const T* dO, const float* lse,
                   const int32_t* page_nrows, float2* ld, hipStream_t st) {
  rowdot_kernel<T><<<blocks_for(s.pages * 64 * s.Hq, 4), 256, 0, st>>>(o, o_lo, dO, lse, page_nrows, ld, s.pages,
                                                                       s.Hq, s.D, 1.f / s.scale);
}

void launch_absmax(const LaunchShape& s, const bf16_t* q, const bf16_t* k, const bf16_t* v, const bf16_t* dO,
                   const int32_t* page_nrows, uint32_t* amax, hipStream_t st) {
  const int64_t pieces = s.C * s.Hq * (kD / 8);
  const int64_t blocks = (pieces + 255) / 256;
  const dim3 grid((unsigned)(blocks < 2048 ? (blocks > 0 ? blocks : 1) : 2048), dO ? 4 : 3);
  absmax_kernel<<<grid, 256, 0, st>>>(q, k, v, dO, page_nrows, s.C, s.Hq, s.Hkv, amax);
}

void launch_zero_u32(uint32_t* out, int n, hipStream_t st) { zero_u32_kernel<<<1, 64, 0, st>>>(out, n); }

#ifdef DAG_DEBUG
bool dbg_enabled() { return true; }
bool dbg_set_limits(const DbgLimits& lim, hipStream_t st) {
  return hipMemcpyToSymbolAsync(HIP_SYMBOL(g_dbg_lim), &lim, sizeof(lim), 0, hipMemcpyHostToDevice, st) == hipSuccess;
}
bool dbg_take(uint32_t out[3], hipStream_t st) {
  uint32_t e[4] = {0, 0, 0, 0};
  const uint32_t zero[4] = {0, 0, 0, 0};
  if (hipMemcpyFromSymbolAsync(e, HIP_SYMBOL(g_dbg_err), sizeof(e), 0, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipMemcpyToSymbolAsync(HIP_SYMBOL(g_dbg_err), zero, sizeof(zero), 0, hipMemcpyHostToDevice, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return false;
  out[0] = e[0], out[1] = e[1], out[2] = e[2];
  return true;
}
#else
bool dbg_enabled() { return false; }
bool dbg_set_limits(const DbgLimits&, hipStream_t) { return true; }
bool dbg_take(uint32_t out[3], hipStream_t) {
  out[0] = out[1] = out[2] = 0;
  return true;
}
#endif

void launch_prep16(const LaunchShape& s, const bf16_t* x, const float2* cs, const int32_t* page_nrows,
                   const uint32_t* smax, bool qk, f16_t* out_n, f16_t* out_t, int H, hipStream_t st) {
  const int top = qk ? kTopQK : kTopVO;
  const unsigned grid = (unsigned)s.pages;
  if (cs) {
    if (out_n && out_t)
      prep16_kernel<true, true, true><<<grid, 512, 0, st>>>(x, cs, page_nrows, smax, top, out_n, out_t, H);
    else
      prep16_kernel<true, true, false><<<grid, 512, 0, st>>>(x, cs, page_nrows, smax, top, out_n, out_t, H);
  } else if (out_n && out_t) {
    prep16_kernel<false, true, true><<<grid, 512, 0, st>>>(x, cs, page_nrows, smax, top, out_n, out_t, H);
  } else if (out_t) {
    prep16_kernel<false, false, true><<<grid, 512, 0, st>>>(x, cs, page_nrows, smax, top, out_n, out_t, H);
  } else {
    prep16_kernel<false, true, false><<<grid, 512, 0, st>>>(x, cs, page_nrows, smax, top, out_n, out_t, H);
  }
}

void launch_rowdot16(const LaunchShape& s, const bf16_t* o, const bf16_t* o_lo, const bf16_t* dO, const float* lse,
                     const int32_t* page_nrows, float2* ld, const uint32_t* amax, hipStream_t st) {
  const int64_t items = s.pages * 64 * s.Hq;
  const int64_t blocks = (items + 15) / 16;
  rowdot16_kernel<<<(unsigned)(blocks < 8192 ? (blocks > 0 ? blocks : 1) : 8192), 256, 0, st>>>(
      o, o_lo, dO, lse, page_nrows, ld, amax, s.pages, s.Hq, 1.f / s.scale);
}

template void launch_relayout<bf16_t, f16_t>(const LaunchShape&, const bf16_t*, const float2*, const int32_t*, f16_t*, f16_t*, int, hipStream_t);
template void launch_relayout<bf16_t, float>(const LaunchShape&, const bf16_t*, const float2*, const int32_t*, float*, float*, int, hipStream_t);
template void launch_relayout<float, float>(const LaunchShape&, const float*, const float2*, const int32_t*, float*, float*, int, hipStream_t);
template void launch_rowdot<bf16_t>(const LaunchShape&, const bf16_t*, const bf16_t*, const bf16_t*, const float*, const int32_t*, float2*, hipStream_t);
template void launch_rowdot<float>(const LaunchShape&, const float*, const float*, const float*, const float*, const int32_t*, float2*, hipStream_t);

// Grid for map_item: whole runs of kRun units per head, padded to a multiple of 8 runs.
static unsigned run_grid(int64_t n_units, int H) {
  const int64_t runs = (n_units + kRun - 1) / kRun;
  const int64_t quantum = 8 * kRun;
  return (unsigned)((runs * H * kRun + quantum - 1) / quantum * quantum);
}

void launch_fwd_mfma(const LaunchShape& s, int64_t n_qp, const f16_t* qn, const f16_t* kn, const f16_t* vt,
                     const QPage* qpages, const int32_t* order, const Tile* tiles, const int32_t* tile_mask,
                     const uint64_t* masks, bf16_t* o, float* lse, bf16_t* o_lo, const uint32_t* amax,
                     hipStream_t st) {
  if (tile_mask) {
    fwd_mfma_kernel<true, 2><<<run_grid(n_qp, s.Hkv), 512, 0, st>>>(
        qn, kn, vt, qpages, order, tiles, tile_mask, masks, o, lse, o_lo, amax, (int)n_qp, s.Hq, s.Hkv,
        s.scale * kLog2e);
  } else {
    // both forms; the one the operand maxima do not select returns at once
    fwd_mfma_kernel<false, 0><<<run_grid(n_qp, s.Hkv), 512, 0, st>>>(
        qn, kn, vt, qpages, order, tiles, nullptr, nullptr, o, lse, o_lo, amax, (int)n_qp, s.Hq, s.Hkv,
        s.scale * kLog2e);
    fwd_mfma_kernel<false, 1><<<run_grid(n_qp, s.Hkv), 512, 0, st>>>(
        qn, kn, vt, qpages, order, tiles, nullptr, nullptr, o, lse, o_lo, amax, (int)n_qp, s.Hq, s.Hkv,
        s.scale * kLog2e);
  }
}

template <typename TG>
void launch_dq_mfma(const LaunchShape& s, int64_t n_qp, const f16_t* qn, const f16_t* kn, const f16_t* vn,
                    const f16_t* dOn, const float2* ld, const float2* cs, const uint32_t* dmax,
                    const QPage* qpages, const int32_t* order, const Tile* tiles, const int32_t* tile_mask,
                    const uint64_t* masks, TG* dq, const uint32_t* amax, hipStream_t st) {
  if (tile_mask)
    dq_mfma_kernel<TG, true><<<run_grid(n_qp, s.Hkv), 512, 0, st>>>(qn, kn, vn, dOn, ld, cs, dmax, qpages, order,
                                                                    tiles, tile_mask, masks, dq, amax, (int)n_qp,
                                                                    s.Hq, s.Hkv, s.scale * kLog2e, s.scale);
  else
    dq_mfma_kernel<TG, false><<<run_grid(n_qp, s.Hkv), 512, 0, st>>>(qn, kn, vn, dOn, ld, cs, dmax, qpages,
                                                                     order, tiles, nullptr, nullptr, dq, amax,
                                                                     (int)n_qp, s.Hq, s.Hkv, s.scale * kLog2e,
                                                                     s.scale);
}

template <typename TG>
void launch_dkdv_mfma(const LaunchShape& s, int64_t n_pairs, const f16_t* qn, const f16_t* kn, const f16_t* vn,
                      const f16_t* dOn, const float2* ld, const float2* cs, const uint32_t* dmax,
                      const int32_t* pair_order, const int32_t* pairs, const int64_t* pair_off, const KStep* psteps,
                      const KMask* pmasks, const uint64_t* masks, const int32_t* page_nrows, TG* dk, TG* dv,
                      const uint32_t* amax, hipStream_t st) {
  if (n_pairs <= 0) return;  // every page in a four-page group
  if (pmasks)
    dkdv_mfma_kernel<TG, true><<<run_grid(n_pairs, s.Hkv), 512, 0, st>>>(
        qn, kn, vn, dOn, ld, cs, dmax, pair_order, pairs, pair_off, psteps, pmasks, masks, page_nrows, dk, dv, amax,
        (int)n_pairs, s.Hq, s.Hkv, s.scale * kLog2e, s.scale);
  else
    dkdv_mfma_kernel<TG, false><<<run_grid(n_pairs, s.Hkv), 512, 0, st>>>(
        qn, kn, vn, dOn, ld, cs, dmax, pair_order, pairs, pair_off, psteps, nullptr, nullptr, page_nrows, dk, dv,
        amax, (int)n_pairs, s.Hq, s.Hkv, s.scale * kLog2e, s.scale);
}

template <typename TG>
void launch_dkdv_group(const LaunchShape& s, int64_t n_groups, const f16_t* qn, const f16_t* kn, const f16_t* vn,
                       const f16_t* dOn, const float2* ld, const float2* cs, const uint32_t* dmax,
                       const int32_t* group_order, const int32_t* groups, const int64_t* group_off,
                       const GStep* gsteps, const int32_t* page_nrows, TG* dk, TG* dv, const uint32_t* amax,
                       hipStream_t st) {
  if (n_groups <= 0) return;
  dkdv_group_kernel<TG><<<run_grid(n_groups, s.Hkv), 512, 0, st>>>(
      qn, kn, vn, dOn, ld, cs, dmax, group_order, groups, group_off, gsteps, page_nrows, dk, dv, amax, (int)n_groups,
      s.Hq, s.Hkv, s.scale * kLog2e, s.scale);
}

#define INST_MFMA_BWD(TG)                                                                                      \
  template void launch_dq_mfma<TG>(const LaunchShape&, int64_t, const f16_t*, const f16_t*, const f16_t*,      \
                                   const f16_t*, const float2*, const float2*, const uint32_t*,                \
                                   const QPage*, const int32_t*, const Tile*, const int32_t*,                  \
                                   const uint64_t*, TG*, const uint32_t*, hipStream_t);                        \
  template void launch_dkdv_mfma<TG>(const LaunchShape&, int64_t, const f16_t*, const f16_t*, const f16_t*,    \
                                     const f16_t*, const float2*, const float2*, const uint32_t*,              \
                                     const int32_t*, const int32_t*, const int64_t*, const KStep*,             \
                                     const KMask*, const uint64_t*, const int32_t*, TG*, TG*,                  \
                                     const uint32_t*, hipStream_t);                                            \
  template void launch_dkdv_group<TG>(const LaunchShape&, int64_t, const f16_t*, const f16_t*, const f16_t*,   \
                                      const f16_t*, const float2*, const float2*, const uint32_t*,             \
                                      const int32_t*, const int32_t*, const int64_t*, const GStep*,            \
                                      const int32_t*, TG*, TG*, const uint32_t*, hipStream_t);
INST_MFMA_BWD(bf16_t)
INST_MFMA_BWD(float)

template <typename T>
void launch_fwd_simple(const LaunchShape& s, int64_t n_qp, const float* qn, const float* kn, const T* v,
                       const QPage* qpages, const int32_t* order, const Tile* tiles, T* o, float* lse, T* o_lo,
                       hipStream_t st) {
  fwd_simple_kernel<T><<<(unsigned)(n_qp * s.Hq), 64, 0, st>>>(qn, kn, v, qpages, order, tiles, o, lse, o_lo, s.Hq,
                                                              s.Hkv, s.D, s.scale);
}

template <typename T, typename TG>
void launch_bwd_simple(const LaunchShape& s, int64_t n_qp, int64_t n_kvp, const float* qn, const float* kn,
                       const T* v, const T* dO, const float2* ld, const float2* cs, const QPage* qpages,
                       const int32_t* fwd_order, const Tile* tiles, const int32_t* bwd_order,
                       const int32_t* kv_off, const KEntry* ents, const int32_t* page_table,
                       const int32_t* page_nrows, TG* dq, TG* dk, TG* dv, hipStream_t st) {
  dq_simple_kernel<T, TG><<<(unsigned)(n_qp * s.Hq), 64, 0, st>>>(qn, kn, v, dO, ld, cs, qpages, fwd_order, tiles,
                                                                  dq, s.Hq, s.Hkv, s.D, s.scale);
  dkdv_simple_kernel<T, TG><<<(unsigned)(n_kvp * s.Hkv), 64, 0, st>>>(qn, kn, v, dO, ld, cs, bwd_order, kv_off,
                                                                      ents, page_table, page_nrows, dk, dv, s.Hq,
                                                                      s.Hkv, s.D, s.scale);
}

template void launch_fwd_simple<bf16_t>(const LaunchShape&, int64_t, const float*, const float*, const bf16_t*, const QPage*, const int32_t*, const Tile*, bf16_t*, float*, bf16_t*, hipStream_t);
template void launch_fwd_simple<float>(const LaunchShape&, int64_t, const float*, const float*, const float*, const QPage*, const int32_t*, const Tile*, float*, float*, float*, hipStream_t);
#define INST_BWD_SIMPLE(T, TG)                                                                                 \
  template void launch_bwd_simple<T, TG>(const LaunchShape&, int64_t, int64_t, const float*, const float*,     \
                                         const T*, const T*, const float2*, const float2*, const QPage*,        \
                                         const int32_t*, const Tile*, const int32_t*, const int32_t*,           \
                                         const KEntry*, const int32_t*, const int32_t*, TG*, TG*, TG*,          \
                                         hipStream_t);
INST_BWD_SIMPLE(bf16_t, bf16_t)
INST_BWD_SIMPLE(bf16_t, float)
INST_BWD_SIMPLE(float, float)

}  // namespace dagattn

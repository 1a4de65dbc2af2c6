// Chunked gated delta rule over a rollout tree (MI355X, gfx950).
//
// What is computed (per head, state S of shape [dv, dk], fp32):
//   S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = scale S_t q_t
// along every token's own root-to-node path (mounted spans are not part of a
// recurrent layer's history, Octopus Sec. 3).  The pages name this layer but
// print no recurrence for it; this is the textbook gated delta rule.
//
// How it is executed (HARTS: Hybrid-Attention RL over Tree Structures):
//   * chunks of B = 64 tokens on the recurrent index (Sec. 2.2 Eq. 2); a
//     branch forking at p starts from the state at a(p) = 64 floor(p / 64) and
//     re-runs the ancestor tokens [a(p), p) without outputs ("replay");
//   * the host schedule (gdn_plan.cpp, Sec. 3.3 Algorithm 1) packs the
//     sequences of each round into one launch; a sequence exports the boundary
//     states its side branches start from, and in the backward the gradient of
//     each exported state is the sum of its consumers' initial-state gradients
//     (Sec. 3.4 Eq. 16), added in a fixed order;
//   * within a chunk (t, i = 0..63 token indices, g_t = sum_{s<=t} log alpha_s,
//     gamma_t = exp(g_t), E_ti = exp(g_t - g_i)), with S0 the state at the
//     chunk's start (the unrolled recurrence written blockwise):
//         A   = strict_lower(beta_t E_ti k_t.k_i)        (unit-lower system I + A)
//         R   = diag(beta) (V - diag(gamma) K S0^T)
//         U   = (I + A)^{-1} R                            (u_t = beta_t (v_t - alpha_t S_{t-1} k_t))
//         O   = scale (diag(gamma) Q S0^T + lower(E o Q K^T) U)
//         S64 = gamma_63 S0 + (diag(E_63,.) U)^T K
//     and the backward is the exact derivative of these lines.
//
// Only the state carry is serial.  Per round, every chunk of every sequence is an
// independent work item for the state-independent part: A, P = scale lower(E o QK^T)
// and T = (I + A)^{-1} (gdn_tinv_kernel, one work-group per chunk and head: forward
// substitution on the identity).  The serial kernels, one work-group (256 threads,
// 4 waves) per (sequence, head), then walk the chunks with products only: the
// solves become U = T R and dR = T^T dU on the matrix cores, with T as an fp16
// high part plus an fp16 low part (T - high), so the product keeps about 22 bits of
// T.  The backward's serial kernel carries only the state gradient and leaves each
// chunk's end-state gradient behind; the rest of the backward (every input gradient)
// is again one work-group per chunk and head (gdn_bpar_kernel).  Dense products run
// on v_mfma_f32_32x32x16_f16 with fp16 operands staged in LDS (transposed operands
// through ds_read_b64_tr_b16) and fp32 accumulation.
#include <hip/hip_runtime.h>

#include "gdn.hpp"

namespace dagattn {
namespace gdn {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __fp16 v4fp16 __attribute__((__vector_size__(8)));
typedef __attribute__((address_space(3))) v4fp16 lds_v4fp16;

constexpr int kB = 64;    // chunk length
constexpr int kD = 128;   // dk = dv
constexpr int LDK = 136;  // halfs per row of an fp16 tile with 128 columns (16-byte pad)
constexpr int LDP = 72;   // halfs per row of an fp16 tile with 64 columns
constexpr int LDA = 68;   // floats per row of an fp32 [64][64] tile
constexpr int LDR = 132;  // floats per row of an fp32 [64][128] tile
constexpr int kRep = 2 * kD + 2;  // replay-gradient record: dk[128], dv[128], dbeta, dalpha

__device__ __forceinline__ float bf2f(bf16_t x) { return __uint_as_float(((uint32_t)x) << 16); }
__device__ __forceinline__ bf16_t f2bf(float x) {
  __bf16 b = (__bf16)x;
  return *reinterpret_cast<bf16_t*>(&b);
}
template <typename T> __device__ __forceinline__ void st_g(T* p, float x);
template <> __device__ __forceinline__ void st_g<float>(float* p, float x) { *p = x; }
template <> __device__ __forceinline__ void st_g<bf16_t>(bf16_t* p, float x) { *p = f2bf(x); }
// Two consecutive elements (p even-aligned).
template <typename T> __device__ __forceinline__ void st2_g(T* p, float x0, float x1);
template <> __device__ __forceinline__ void st2_g<float>(float* p, float x0, float x1) {
  *reinterpret_cast<float2*>(p) = make_float2(x0, x1);
}
template <> __device__ __forceinline__ void st2_g<bf16_t>(bf16_t* p, float x0, float x1) {
  *reinterpret_cast<uint32_t*>(p) = (uint32_t)f2bf(x0) | ((uint32_t)f2bf(x1) << 16);
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
// Row of element r of a 32x32 accumulator in lane half `hi` (column = lane % 32).
__device__ __forceinline__ int acc_row(int r, int hi) { return 8 * (r >> 2) + 4 * hi + (r & 3); }

// Global stores of a 32 x 32 accumulator block two columns per lane: the lanes of each
// even/odd pair (columns c, c + 1) trade one value of every row pair (2 i, 2 i + 1) with a
// DPP swap, so the even lane holds row 2 i and the odd lane row 2 i + 1, each at both
// columns; put(t, x0, x1) stores row t's pair at the pair's even column.  Half the store
// instructions of one element per lane.
__device__ __forceinline__ float swap_adjacent_lanes(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
}
template <typename F>
__device__ __forceinline__ void put_pairs(const f32x16& a, int row0, int lane, F&& put) {
  const int odd = lane & 1, hi = lane >> 5;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float got = swap_adjacent_lanes(odd ? a[2 * i] : a[2 * i + 1]);
    const float x0 = odd ? got : a[2 * i], x1 = odd ? a[2 * i + 1] : got;
    put(row0 + 8 * (i >> 1) + 4 * hi + 2 * (i & 1) + odd, x0, x1);  // acc_row(2 i + odd, hi)
  }
}
typedef __attribute__((ext_vector_type(2))) f16_t f16x2_t;
// fp16 copy of a 32 x 32 accumulator block (column col = col0 + lane % 32) into an LDS tile
// of row stride ld halfs, two columns per lane: one 4-byte write per element pair.
__device__ __forceinline__ void lds_put_f16(const f32x16& a, f16_t* tile, int ld, int row0, int col, int lane) {
  put_pairs(a, row0, lane, [&](int t, float x0, float x1) {
    *reinterpret_cast<f16x2_t*>(tile + t * ld + (col & ~1)) = f16x2_t{(f16_t)x0, (f16_t)x1};
  });
}

// MFMA operand with the contraction index contiguous: rows mn0 + lane % 32 of
// X[.][ld], elements k0 + 8 (lane / 32) .. + 7.
__device__ __forceinline__ f16x8 frag_n(const f16_t* X, int ld, int mn0, int k0, int lane) {
  return *reinterpret_cast<const f16x8*>(X + (mn0 + (lane & 31)) * ld + k0 + 8 * (lane >> 5));
}
// MFMA operand with the contraction index along rows of an LDS tile X[k][mn]:
// lane gets X[k0 + 8 (lane / 32) + j][mn0 + lane % 32], j = 0..7.  Within a
// group of 16 lanes, a transpose read gives lane i element i % 4 of the 8 bytes
// fetched by lane 4 j + i / 4; so lane s fetches row (s / 4) at columns 4 (s % 4) ...
__device__ __forceinline__ f16x8 frag_t(const f16_t* X, int ld, int k0, int mn0, int lane) {
  const int G = lane >> 4, a = lane & 15;
  const int row = k0 + 8 * (G >> 1) + (a >> 2);
  const int col = mn0 + 16 * (G & 1) + 4 * (a & 3);
  const v4fp16 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_v4fp16*)(X + row * ld + col));
  const v4fp16 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_v4fp16*)(X + (row + 4) * ld + col));
  f16x8 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o[j] = (f16_t)v0[j];
    o[4 + j] = (f16_t)v1[j];
  }
  return o;
}
// The values of an LDS tile X[.][ld] at an accumulator lane's 16 rows row0 + acc_row(r, hi)
// and its column col0 + lane % 32, as fp32: four transpose reads of four rows each (in each
// group of 16 lanes, lane s fetches row s / 4 of the group's four at columns 4 (s % 4) ..).
__device__ __forceinline__ void acc_col_f16(const f16_t* X, int ld, int row0, int col0, int lane, float (&v)[16]) {
  const int G = lane >> 4, a = lane & 15;
  const f16_t* p = X + (row0 + 4 * (G >> 1) + (a >> 2)) * ld + col0 + 16 * (G & 1) + 4 * (a & 3);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const v4fp16 w = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_v4fp16*)(p + 8 * q * ld));
#pragma unroll
    for (int j = 0; j < 4; ++j) v[4 * q + j] = (float)(f16_t)w[j];
  }
}
// Same operand layout as frag_n, read from global memory.
__device__ __forceinline__ f16x8 frag_g(const f16_t* __restrict__ X, int mn0, int k0, int lane) {
  return *reinterpret_cast<const f16x8*>(X + (mn0 + (lane & 31)) * kD + k0 + 8 * (lane >> 5));
}
__device__ __forceinline__ f16x8 scale8(f16x8 a, const float (&s)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = (f16_t)((float)a[j] * s[j]);
  return a;
}

// 8 bf16 (16 bytes) -> 8 fp16.
__device__ __forceinline__ f16x8 bf8_to_h8(uint4 u) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  f16x8 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = (f16_t)__uint_as_float(w[i] << 16);
    o[2 * i + 1] = (f16_t)__uint_as_float(w[i] & 0xffff0000u);
  }
  return o;
}

// Lane exchanges inside rows of 16 lanes (DPP): the value of lane i ^ 1, of lane i ^ 2,
// and of the lanes 4 and 8 places away in the lane's row.
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float from_xor1(float x) { return dpp_mov<0xB1>(x); }  // quad_perm 1,0,3,2
__device__ __forceinline__ float from_xor2(float x) { return dpp_mov<0x4E>(x); }  // quad_perm 2,3,0,1
__device__ __forceinline__ float from_ror4(float x) { return dpp_mov<0x124>(x); }  // row_ror 4
__device__ __forceinline__ float from_ror8(float x) { return dpp_mov<0x128>(x); }  // row_ror 8 (lane i ^ 8)

// Sum of the 16 accumulator values of each row over the 32 lanes of one lane half, in a
// fixed order: four halving steps inside each row of 16 lanes, the lane keeping the half
// of its values that one bit of its index selects and adding the partner's partial sums
// of that half (partners: lane ^ 1, lane ^ 2, then the lanes 4 and 8 places away in the
// row, which differ in bits 2 and 3 and agree in the bits already used), then the sum of
// the half's two rows.  Afterwards lanes l and l ^ 16 hold the sum for element
// rowsum16_elem(l) (row acc_row(., hi)); rowsum16_writer(l) picks one of the two.
__device__ __forceinline__ float rowsum16(const float (&x)[16], int lane) {
  float a8[8], a4[4], a2[2], a1;
  const bool b0 = lane & 1, b1 = lane & 2, b2 = lane & 4, b3 = lane & 8;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float send = b0 ? x[j] : x[8 + j];
    const float keep = b0 ? x[8 + j] : x[j];
    a8[j] = keep + from_xor1(send);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float send = b1 ? a8[j] : a8[4 + j];
    const float keep = b1 ? a8[4 + j] : a8[j];
    a4[j] = keep + from_xor2(send);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float send = b2 ? a4[j] : a4[2 + j];
    const float keep = b2 ? a4[2 + j] : a4[j];
    a2[j] = keep + from_ror4(send);
  }
  {
    const float send = b3 ? a2[0] : a2[1];
    const float keep = b3 ? a2[1] : a2[0];
    a1 = keep + from_ror8(send);
  }
  return a1 + __shfl_xor(a1, 16);
}
// Element index of the row whose sum rowsum16 leaves in this lane.
__device__ __forceinline__ int rowsum16_elem(int lane) {
  return 8 * (lane & 1) + 4 * ((lane >> 1) & 1) + 2 * ((lane >> 2) & 1) + ((lane >> 3) & 1);
}
__device__ __forceinline__ bool rowsum16_writer(int lane) { return !(lane & 16); }

// The per-row values v[r] = a[32 rb + acc_row(r, hi)] of an accumulator lane's 16 rows:
// four runs of four consecutive floats (a 16-byte aligned), one 16-byte LDS read each.
__device__ __forceinline__ void rows16(const float* a, int rb, int hi, float (&v)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 x = *reinterpret_cast<const float4*>(a + 32 * rb + 8 * q + 4 * hi);
    v[4 * q] = x.x, v[4 * q + 1] = x.y, v[4 * q + 2] = x.z, v[4 * q + 3] = x.w;
  }
}
// Sum over the 32 rows of one accumulator column (both lane halves).
__device__ __forceinline__ float colsum16(const float (&x)[16]) {
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += x[r];
  return s + __shfl_xor(s, 32);
}

// ---------------------------------------------------------------------------------
// LDS tiles shared by both kernels
// ---------------------------------------------------------------------------------
struct ChunkIn {
  const int32_t* rows;  // sequence token -> compact row
  int n_tok, n_replay;
};

// Eight-wave state layout: wave (rb, cb) holds dv rows 32 cb .. and dk blocks 2 rb and
// 2 rb + 1 (accumulator element r of S[b] is row 32 cb + acc_row(r, hi), column
// 32 (2 rb + b) + lane % 32).
__device__ __forceinline__ void state_to_lds8(const f32x16 (&S)[2], f16_t* Sh, int cb, int rb, int lane) {
  const int hi = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) Sh[(32 * cb + acc_row(r, hi)) * LDK + 32 * (2 * rb + b) + l32] = (f16_t)S[b][r];
}
__device__ __forceinline__ void state_save8(const f32x16 (&S)[2], f16_t* __restrict__ dst, int cb, int rb, int lane) {
  const int hi = lane >> 5, l32 = lane & 31;
  f16_t* nat = dst;
  f16_t* tr = dst + kD * kD;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int nb = 2 * rb + b;
#pragma unroll
    for (int r = 0; r < 16; ++r) nat[(32 * cb + acc_row(r, hi)) * kD + 32 * nb + l32] = (f16_t)S[b][r];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
      f16x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = (f16_t)S[b][4 * r4 + j];
      *reinterpret_cast<f16x4*>(tr + (32 * nb + l32) * kD + 32 * cb + 8 * r4 + 4 * hi) = w;
    }
  }
}
// fp32 [dv][dk] state in global memory <-> the eight-wave accumulators
__device__ __forceinline__ void state_load8(f32x16 (&S)[2], const float* __restrict__ src, int cb, int rb, int lane) {
  const int hi = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) S[b][r] = src[(32 * cb + acc_row(r, hi)) * kD + 32 * (2 * rb + b) + l32];
}
__device__ __forceinline__ void state_store8(const f32x16 (&S)[2], float* __restrict__ dst, int cb, int rb, int lane) {
  const int hi = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) dst[(32 * cb + acc_row(r, hi)) * kD + 32 * (2 * rb + b) + l32] = S[b][r];
}

// The next chunk's inputs, fetched into registers while the current chunk
// computes (one work-group per CU leaves nothing else to hide their latency).
struct ChunkRegs {
  uint4 k4[4], q4[4], v4[4];  // 16-byte pieces: rows (tid >> 4) + 16 m, columns 8 (tid & 15) ..
  int row;                    // tid < 64: the chunk's token tid (-1 past the end)
  float b, a;          //           and its beta, alpha
};

// Rows and gates of the chunk starting at token j0 (threads < 64).
__device__ __forceinline__ void fetch_rows(const ChunkIn& ci, int j0, const float* __restrict__ beta,
                                           const float* __restrict__ alpha, int H, int head, int tid,
                                           ChunkRegs& nx) {
  if (tid < kB) {
    const int j = j0 + tid;
    nx.row = -1;
    nx.b = 0.f;
    nx.a = 1.f;
    if (j < ci.n_tok) {
      nx.row = ci.rows[j];
      nx.b = beta[(int64_t)nx.row * H + head];
      nx.a = alpha[(int64_t)nx.row * H + head];
    }
  }
}

// K, Q and V rows of that chunk, given its rows in LDS (rwn): whole 16-byte pieces of
// each row, so one load instruction covers sixteen rows' 256 contiguous bytes.
__device__ __forceinline__ void fetch_kqv(const int* rwn, const bf16_t* __restrict__ k, const bf16_t* __restrict__ q,
                                          const bf16_t* __restrict__ v, int H, int head, int tid, ChunkRegs& nx) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int row = rwn[(tid >> 4) + 16 * m];
    nx.k4[m] = nx.q4[m] = nx.v4[m] = make_uint4(0, 0, 0, 0);
    if (row >= 0) {
      const int64_t base = ((int64_t)row * H + head) * kD + (tid & 15) * 8;
      nx.k4[m] = *reinterpret_cast<const uint4*>(k + base);
      nx.q4[m] = *reinterpret_cast<const uint4*>(q + base);
      nx.v4[m] = *reinterpret_cast<const uint4*>(v + base);
    }
  }
}

// Make the fetched chunk current: K, Q rows (fp16) into LDS, V rows (fp32, exact) into
// the R tile that the next R computation overwrites in place, row numbers, beta and the
// cumulative log decay.
__device__ __forceinline__ void commit_chunk(const ChunkRegs& nx, f16_t* Kr, f16_t* Qr, float* Rr, int* rw,
                                             float* gs, float* bs, int tid) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int t = (tid >> 4) + 16 * m, c8 = (tid & 15) * 8;
    *reinterpret_cast<f16x8*>(Kr + t * LDK + c8) = bf8_to_h8(nx.k4[m]);
    *reinterpret_cast<f16x8*>(Qr + t * LDK + c8) = bf8_to_h8(nx.q4[m]);
    const uint32_t w[4] = {nx.v4[m].x, nx.v4[m].y, nx.v4[m].z, nx.v4[m].w};
    float4* rv = reinterpret_cast<float4*>(Rr + t * LDR + c8);
    rv[0] = make_float4(__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                        __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u));
    rv[1] = make_float4(__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xffff0000u),
                        __uint_as_float(w[3] << 16), __uint_as_float(w[3] & 0xffff0000u));
  }
  if (tid < kB) {
    rw[tid] = nx.row;
    bs[tid] = nx.b;
    float la = logf(nx.a);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(la, off, 64);
      if (tid >= off) la += y;
    }
    gs[tid] = la;
  }
}

// The backward's next chunk (the one before the current), fetched into registers in
// two steps while the current chunk computes: its row numbers first, then the K, Q,
// dO, V pieces and the gates once the row numbers have arrived.
struct BwdRegs {
  uint4 k4[4], q4[4], d4[4], v4[4];  // rows (tid >> 4) + 16 m, columns 8 (tid & 15) ..
  int r4[4];                         // those rows' compact row (-1 past the sequence)
  int row;                           // tid < 64: token tid's compact row (-1 past the end)
  float b, a;                        //           and its beta, alpha
};

__device__ __forceinline__ void bwd_fetch_rows(const ChunkIn& ci, int j0, int tid, BwdRegs& nx) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int j = j0 + (tid >> 4) + 16 * m;
    nx.r4[m] = j < ci.n_tok ? ci.rows[j] : -1;
  }
  if (tid < kB) nx.row = j0 + tid < ci.n_tok ? ci.rows[j0 + tid] : -1;
}

template <bool kV>
__device__ __forceinline__ void bwd_fetch_data(const ChunkIn& ci, int j0, const bf16_t* __restrict__ k,
                                               const bf16_t* __restrict__ q, const bf16_t* __restrict__ dO,
                                               const bf16_t* __restrict__ v, const float* __restrict__ beta,
                                               const float* __restrict__ alpha, int H, int head, int tid,
                                               BwdRegs& nx) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int j = j0 + (tid >> 4) + 16 * m;
    nx.k4[m] = nx.q4[m] = nx.d4[m] = nx.v4[m] = make_uint4(0, 0, 0, 0);
    if (nx.r4[m] >= 0) {
      const int64_t base = ((int64_t)nx.r4[m] * H + head) * kD + (tid & 15) * 8;
      nx.k4[m] = *reinterpret_cast<const uint4*>(k + base);
      nx.q4[m] = *reinterpret_cast<const uint4*>(q + base);
      if (kV) nx.v4[m] = *reinterpret_cast<const uint4*>(v + base);
      if (j >= ci.n_replay) nx.d4[m] = *reinterpret_cast<const uint4*>(dO + base);
    }
  }
  if (tid < kB) {
    nx.b = 0.f;
    nx.a = 1.f;
    if (nx.row >= 0) {
      nx.b = beta[(int64_t)nx.row * H + head];
      nx.a = alpha[(int64_t)nx.row * H + head];
    }
  }
}

// Make the fetched chunk current: K, Q, dO (and V if kV) rows as fp16 in LDS, row
// numbers, beta, alpha and the cumulative log decay.  Tokens past the sequence's end are
// zero (beta = 0, log alpha = 0), which makes them inert in every product.
template <bool kV>
__device__ __forceinline__ void bwd_commit(const BwdRegs& nx, f16_t* Kr, f16_t* Qr, f16_t* dOr, f16_t* Vr, int* rw,
                                           float* gs, float* bs, float* al, int tid) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int t = (tid >> 4) + 16 * m, c8 = (tid & 15) * 8;
    *reinterpret_cast<f16x8*>(Kr + t * LDK + c8) = bf8_to_h8(nx.k4[m]);
    *reinterpret_cast<f16x8*>(Qr + t * LDK + c8) = bf8_to_h8(nx.q4[m]);
    *reinterpret_cast<f16x8*>(dOr + t * LDK + c8) = bf8_to_h8(nx.d4[m]);
    if (kV) *reinterpret_cast<f16x8*>(Vr + t * LDK + c8) = bf8_to_h8(nx.v4[m]);
  }
  if (tid < kB) {
    rw[tid] = nx.row;
    bs[tid] = nx.b;
    al[tid] = nx.a;
    float la = logf(nx.a);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(la, off, 64);
      if (tid >= off) la += y;
    }
    gs[tid] = la;
  }
}

// Triangular solve with the unit-lower matrix I + A (A strictly lower), for
// the 128 columns of an [64][.] tile, by all 256 threads (or its first 64 columns by
// the first 128): lanes l and l ^ 32 of
// wave w share column c = 32 w + (l & 31), and lane half h = l >> 5 takes target
// rows 8 h .. 8 h + 7 of each 16-row block in the updates from the solved blocks
// (a runtime loop over their rows).  The two halves then swap their partial sums
// and both run the block's own 16-row substitution in registers and store all 16
// solved rows (the same values to the same addresses), so every lane later reads
// only rows it wrote itself.  Each element sees its additions in the same order as
// with one thread per column.  A is kept transposed in LDS (At[i][t] = A[t][i], row
// stride LDA).

// n consecutive entries At[row][col0 .. col0 + n - 1] (broadcast LDS reads).
template <int n>
__device__ __forceinline__ void at_row(const float* At, int row, int col0, float (&a)[n]) {
  const float4* p = reinterpret_cast<const float4*>(At + row * LDA + col0);
#pragma unroll
  for (int q = 0; q < n / 4; ++q) {
    const float4 v = p[q];
    a[4 * q] = v.x;
    a[4 * q + 1] = v.y;
    a[4 * q + 2] = v.z;
    a[4 * q + 3] = v.w;
  }
}

// Both halves' 8 partial sums as the block's 16 (lane half h holds rows 8 h ..).
__device__ __forceinline__ void join_halves(const float (&part)[8], int h, float (&full)[16]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float o = __shfl_xor(part[j], 32, 64);
    full[j] = h ? o : part[j];
    full[8 + j] = h ? part[j] : o;
  }
}

// (I + A) X = R, right-looking: once x_i is final, every later row t takes
// -A[t][i] x_i, and A[t][i] for t in a block is a contiguous run of row i of At.
// X overwrites R in `x` (row stride ldx); the solved rows also go to `out` as
// fp16 if kOut.  The solved rows' contributions are taken four rows at a time
// with all their LDS reads issued first, and row m + 1's coefficients are read
// while row m is finished.  The order of the additions is fixed (row by row,
// ascending).
template <typename TX, bool kOut>
__device__ __forceinline__ void solve_lower(const float* __restrict__ At, TX* __restrict__ x, int ldx,
                                            f16_t* __restrict__ out, int tid) {
  const int c = 32 * (tid >> 6) + (tid & 31), h = (tid >> 5) & 1;
  for (int b = 0; b < 4; ++b) {
    float part[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) part[j] = (float)x[(16 * b + 8 * h + j) * ldx + c];
    for (int i = 0; i < 16 * b; i += 4) {
      float xi[4], a[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        xi[u] = (float)x[(i + u) * ldx + c];
        at_row<8>(At, i + u, 16 * b + 8 * h, a[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) part[j] = fmaf(-a[u][j], xi[u], part[j]);
    }
    float acc[16];
    join_halves(part, h, acc);
    float a[2][16];
    at_row<16>(At, 16 * b, 16 * b, a[0]);
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      if (m < 15) at_row<16>(At, 16 * b + m + 1, 16 * b, a[(m + 1) & 1]);
#pragma unroll
      for (int j = m + 1; j < 16; ++j) acc[j] = fmaf(-a[m & 1][j], acc[m], acc[j]);
      x[(16 * b + m) * ldx + c] = (TX)acc[m];
      if (kOut) out[(16 * b + m) * LDK + c] = (f16_t)acc[m];
    }
  }
}

// ---------------------------------------------------------------------------------
// (I + A)^{-1} and P of every chunk of one round.  Grid: (round's chunk items) x H.
// Per (item, head), kGdnTinvHalfs fp16 values: T's high part, T's low part (T minus the
// high part, rounded) and P, each [64][64] row-major ([t][i]).
// ---------------------------------------------------------------------------------
constexpr int kTinv = 3 * kB * kB;  // halfs per (item, head)

__global__ __launch_bounds__(256) void gdn_tinv_kernel(const GSeq* __restrict__ seqs,
                                                       const int32_t* __restrict__ items,
                                                       const int32_t* __restrict__ grows,
                                                       const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                       const float* __restrict__ beta,
                                                       const float* __restrict__ alpha, f16_t* __restrict__ tinv,
                                                       int H, float scale) {
  __shared__ __attribute__((aligned(16))) f16_t Kr[kB * LDK];
  __shared__ __attribute__((aligned(16))) f16_t Qr[kB * LDK];
  __shared__ __attribute__((aligned(16))) float Ar[kB * LDA];  // A^T
  __shared__ __attribute__((aligned(16))) float gs[kB];
  __shared__ __attribute__((aligned(16))) float bs[kB];
  float* Xr = reinterpret_cast<float*>(Kr);  // after the products: the identity, then T ([t][j])
  static_assert(kB * LDA * 4 <= kB * LDK * 2, "the solve tile fits the K tile");
  __shared__ int rw[kB];
  const int head = blockIdx.x % H;
  const int item = blockIdx.x / H;
  const GSeq sq = seqs[items[2 * item]];
  const int j0 = items[2 * item + 1] * kB;
  const int tid = threadIdx.x, lane = tid & 63, hi = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  if (tid < kB) {
    const int j = j0 + tid;
    int row = -1;
    float b = 0.f, a = 1.f;
    if (j < sq.n_tok) {
      row = grows[sq.tok_off + j];
      b = beta[(int64_t)row * H + head];
      a = alpha[(int64_t)row * H + head];
    }
    rw[tid] = row;
    bs[tid] = b;
    float la = logf(a);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(la, off, 64);
      if (tid >= off) la += y;
    }
    gs[tid] = la;
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int t = (tid >> 4) + 16 * m, c8 = (tid & 15) * 8;
    const int row = rw[t];
    uint4 k4 = make_uint4(0, 0, 0, 0), q4 = make_uint4(0, 0, 0, 0);
    if (row >= 0) {
      const int64_t base = ((int64_t)row * H + head) * kD + c8;
      k4 = *reinterpret_cast<const uint4*>(k + base);
      q4 = *reinterpret_cast<const uint4*>(q + base);
    }
    *reinterpret_cast<f16x8*>(Kr + t * LDK + c8) = bf8_to_h8(k4);
    *reinterpret_cast<f16x8*>(Qr + t * LDK + c8) = bf8_to_h8(q4);
  }
  __syncthreads();
  f16_t* dst = tinv + ((int64_t)item * H + head) * kTinv;
  {
    // A = strict_lower(diag(beta) E o KK^T) (kept transposed) and P = scale lower(E o QK^T)
    const int bm = wave >> 1, bn = wave & 1;
    f32x16 kk = zero16(), qk = zero16();
    if (bm >= bn) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const f16x8 b = frag_n(Kr, LDK, 32 * bn, 16 * s, lane);
        kk = mfma(frag_n(Kr, LDK, 32 * bm, 16 * s, lane), b, kk);
        qk = mfma(frag_n(Qr, LDK, 32 * bm, 16 * s, lane), b, qk);
      }
    }
    const int i = 32 * bn + l32;
    const float gi = gs[i];
    float gt[16], b16[16];
    rows16(gs, bm, hi, gt);
    rows16(bs, bm, hi, b16);
    f32x16 pq;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = 32 * bm + acc_row(r, hi);
      // E_ti = exp(g_t - g_i) on and below the diagonal; exp(-inf) = 0 above it (no branch)
      const float e = __expf(i <= t ? gt[r] - gi : -INFINITY);
      Ar[i * LDA + t] = i < t ? b16[r] * e * kk[r] : 0.f;
      pq[r] = scale * e * qk[r];
    }
    put_pairs(pq, 32 * bm, lane, [&](int t, float x0, float x1) {
      *reinterpret_cast<f16x2_t*>(dst + 2 * kB * kB + t * kB + (i & ~1)) = f16x2_t{(f16_t)x0, (f16_t)x1};
    });
  }
  __syncthreads();
  for (int idx = tid; idx < kB * kB; idx += 256) Xr[(idx >> 6) * LDA + (idx & 63)] = (idx >> 6) == (idx & 63) ? 1.f : 0.f;
  __syncthreads();
  // T = (I + A)^{-1}: the solve on the identity, 64 columns (two waves, two lanes a column)
  if (tid < 128) solve_lower<float, false>(Ar, Xr, LDA, nullptr, tid);
  __syncthreads();
  for (int idx = 2 * tid; idx < kB * kB; idx += 512) {  // two consecutive elements per thread
    const float2 x = *reinterpret_cast<const float2*>(Xr + (idx >> 6) * LDA + (idx & 63));
    const f16_t h0 = (f16_t)x.x, h1 = (f16_t)x.y;
    *reinterpret_cast<f16x2_t*>(dst + idx) = f16x2_t{h0, h1};
    *reinterpret_cast<f16x2_t*>(dst + kB * kB + idx) = f16x2_t{(f16_t)(x.x - (float)h0), (f16_t)(x.y - (float)h1)};
  }
}

// The chunk's T high / low parts and P, fetched into registers one chunk ahead
// (two 16-byte pieces of each tile a thread) and committed to LDS tiles [64][LDP].
struct TinvRegs {
  uint4 h0, h1, l0, l1, p0, p1;
};
__device__ __forceinline__ void fetch_tinv(const f16_t* __restrict__ src, int tid, TinvRegs& nx) {
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
  nx.h0 = s4[tid];
  nx.h1 = s4[tid + 256];
  nx.l0 = s4[512 + tid];
  nx.l1 = s4[512 + tid + 256];
  nx.p0 = s4[1024 + tid];
  nx.p1 = s4[1024 + tid + 256];
}
__device__ __forceinline__ void commit_tinv(const TinvRegs& nx, f16_t* Th, f16_t* Tl, f16_t* Pr, int tid) {
  // piece tid (+ 256) of a [64][64] tile: row (tid >> 3) (+ 32), columns 8 (tid & 7) ..
  const int o0 = (tid >> 3) * LDP + 8 * (tid & 7), o1 = o0 + 32 * LDP;
  *reinterpret_cast<uint4*>(Th + o0) = nx.h0;
  *reinterpret_cast<uint4*>(Th + o1) = nx.h1;
  *reinterpret_cast<uint4*>(Tl + o0) = nx.l0;
  *reinterpret_cast<uint4*>(Tl + o1) = nx.l1;
  *reinterpret_cast<uint4*>(Pr + o0) = nx.p0;
  *reinterpret_cast<uint4*>(Pr + o1) = nx.p1;
}

// The same with 512 threads: one 16-byte piece of each tile a thread (plain vector
// types, which the compiler keeps in registers).
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
struct TinvRegs8 {
  u32x4 h, l, p;
};
__device__ __forceinline__ void fetch_tinv8(const f16_t* __restrict__ src, int tid, TinvRegs8& nx) {
  const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
  nx.h = s4[tid];
  nx.l = s4[512 + tid];
  nx.p = s4[1024 + tid];
}
__device__ __forceinline__ void commit_tinv8(const TinvRegs8& nx, f16_t* Th, f16_t* Tl, f16_t* Pr, int tid) {
  const int o = (tid >> 3) * LDP + 8 * (tid & 7);  // row tid / 8, columns 8 (tid % 8) ..
  *reinterpret_cast<u32x4*>(Th + o) = nx.h;
  *reinterpret_cast<u32x4*>(Tl + o) = nx.l;
  *reinterpret_cast<u32x4*>(Pr + o) = nx.p;
}

// ---------------------------------------------------------------------------------
// Forward.  kOut: the outputs; kSave: every chunk's starting state, saved for the
// backward.  Outputs alone are the plain forward, states alone the backward's
// recomputation, both a forward that keeps its states.  All export boundary states.
// ---------------------------------------------------------------------------------
template <bool kOut, bool kSave>
__global__ __launch_bounds__(512, 1) void gdn_fwd_kernel(
    const GSeq* __restrict__ seqs, const int32_t* __restrict__ order, const int32_t* __restrict__ grows,
    const GExport* __restrict__ exports, const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
    const bf16_t* __restrict__ v, const float* __restrict__ beta, const float* __restrict__ alpha,
    const f16_t* __restrict__ tinv, bf16_t* __restrict__ o, float* __restrict__ slots, f16_t* __restrict__ states,
    int H, float scale) {
  __shared__ __attribute__((aligned(16))) f16_t Kr[kB * LDK];
  __shared__ __attribute__((aligned(16))) f16_t Qr[kB * LDK];
  __shared__ __attribute__((aligned(16))) f16_t Sh[kD * LDK];
  __shared__ __attribute__((aligned(16))) f16_t Pr[kB * LDP];
  __shared__ __attribute__((aligned(16))) f16_t Ur[kB * LDK];
  __shared__ __attribute__((aligned(16))) f16_t Th[kB * LDP];
  __shared__ __attribute__((aligned(16))) f16_t Tl[kB * LDP];
  // V rows (fp32, exact) in; then R as fp16 high and low parts, two [64][LDK] tiles
  __shared__ __attribute__((aligned(16))) float Rr[(2 * kB * LDK) / 2];
  __shared__ float gs[kB], bs[kB], gam[kB], egam[kB];
  __shared__ int rw[kB], rwn[kB];
  static_assert(kB * LDR <= 2 * kB * LDK / 2, "the V rows fit the R tiles");
  f16_t* Rh = reinterpret_cast<f16_t*>(Rr);
  f16_t* Rl = Rh + kB * LDK;

  const int head = blockIdx.x % H;
  const GSeq sq = seqs[order[blockIdx.x / H]];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hi = lane >> 5, l32 = lane & 31;
  const int rb = wave >> 2, cb = wave & 3;
  const bool stager = tid < 256;  // the first four waves fetch and commit the chunk inputs
  const int nch = (sq.n_tok + kB - 1) / kB;
  const ChunkIn ci{grows + sq.tok_off, sq.n_tok, sq.n_replay};
  const f16_t* tinv_seq = tinv + (int64_t)sq.item0 * H * kTinv + (int64_t)head * kTinv;
  const int64_t tinv_step = (int64_t)H * kTinv;

  f32x16 S[2];
  if (sq.init_slot >= 0) {
    state_load8(S, slots + ((int64_t)sq.init_slot * H + head) * kD * kD, cb, rb, lane);
  } else {
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) S[b2] = zero16();
  }
  state_to_lds8(S, Sh, cb, rb, lane);
  if (kSave) state_save8(S, states + ((int64_t)sq.chunk_off * H + head) * 2 * kD * kD, cb, rb, lane);
  int ex = sq.exp_off;
  const int ex_end = sq.exp_off + sq.exp_cnt;

  // chunk 0 is fetched up front; chunk c + 1's inputs are fetched during chunk c
  ChunkRegs nx;
  if (nch > 0) {
    TinvRegs8 t0;
    fetch_tinv8(tinv_seq, tid, t0);
    commit_tinv8(t0, Th, Tl, Pr, tid);
  }
  if (stager) {
    fetch_rows(ci, 0, beta, alpha, H, head, tid, nx);
    if (tid < kB) rwn[tid] = nx.row;
  }
  __syncthreads();
  if (stager) {
    fetch_kqv(rwn, k, q, v, H, head, tid, nx);
    commit_chunk(nx, Kr, Qr, Rr, rw, gs, bs, tid);
  }
  __syncthreads();

  for (int c = 0; c < nch; ++c) {
    // opaque thread indices inside the chunk loop (see the backward kernels)
    int tid_o = threadIdx.x;
    asm volatile("" : "+v"(tid_o));
    const int tid = tid_o, wave = tid >> 6, lane = tid & 63, hi = lane >> 5, l32 = lane & 31;
    const int rb = wave >> 2, cb = wave & 3;
    const int j0 = c * kB;
    const bool has_next = c + 1 < nch;
    if (has_next && stager) fetch_rows(ci, j0 + kB, beta, alpha, H, head, tid, nx);
    if (tid < kB) {
      gam[tid] = __expf(gs[tid]);
      egam[tid] = __expf(gs[kB - 1] - gs[tid]);
    }
    const int cc = 32 * cb + l32;
    TinvRegs8 tx;

    // -- R = diag(beta) (V - diag(gamma) K S0^T), split into fp16 high and low parts ------
    {
      f32x16 ks = zero16();
#pragma unroll
      for (int s = 0; s < 8; ++s)
        ks = mfma(frag_n(Kr, LDK, 32 * rb, 16 * s, lane), frag_n(Sh, LDK, 32 * cb, 16 * s, lane), ks);
      if (tid < kB) rwn[tid] = has_next ? nx.row : -1;
      __syncthreads();  // the decay factors are in place
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = 32 * rb + acc_row(r, hi);
        ks[r] = bs[t] * (Rr[t * LDR + cc] - gam[t] * ks[r]);  // V in, R out
      }
      __syncthreads();  // every V row read: the R tiles overwrite them
      // R as an fp16 high part and the fp16 rounding of the rest, two columns per lane
      put_pairs(ks, 32 * rb, lane, [&](int t, float x0, float x1) {
        const f16_t h0 = (f16_t)x0, h1 = (f16_t)x1;
        *reinterpret_cast<f16x2_t*>(Rh + t * LDK + (cc & ~1)) = f16x2_t{h0, h1};
        *reinterpret_cast<f16x2_t*>(Rl + t * LDK + (cc & ~1)) = f16x2_t{(f16_t)(x0 - (float)h0), (f16_t)(x1 - (float)h1)};
      });
    }
    if (has_next && stager) fetch_kqv(rwn, k, q, v, H, head, tid, nx);
    __syncthreads();

    // -- U = (I + A)^{-1} R = T R: T_hi R_hi + T_hi R_lo + T_lo R_hi ---------------------------
    {
      f32x16 u = zero16();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const f16x8 bh = frag_t(Rh, LDK, 16 * s, 32 * cb, lane);
        const f16x8 bl = frag_t(Rl, LDK, 16 * s, 32 * cb, lane);
        const f16x8 ah = frag_n(Th, LDP, 32 * rb, 16 * s, lane);
        u = mfma(ah, bh, u);
        u = mfma(ah, bl, u);
        u = mfma(frag_n(Tl, LDP, 32 * rb, 16 * s, lane), bh, u);
      }
      lds_put_f16(u, Ur, LDK, 32 * rb, cc, lane);
    }
    // the next chunk's T and P (issued here, where the R and U registers are free; the
    // last chunk fetches its own again)
    fetch_tinv8(tinv_seq + (has_next ? c + 1 : c) * tinv_step, tid, tx);
    __syncthreads();

    // -- outputs: O = scale diag(gamma) Q S0^T + (scale E o QK) U -------------------------
    if (kOut) {
      f32x16 acc_o = zero16();
#pragma unroll
      for (int s = 0; s < 8; ++s)
        acc_o = mfma(frag_n(Qr, LDK, 32 * rb, 16 * s, lane), frag_n(Sh, LDK, 32 * cb, 16 * s, lane), acc_o);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[r] *= scale * gam[32 * rb + acc_row(r, hi)];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc_o = mfma(frag_n(Pr, LDP, 32 * rb, 16 * s, lane), frag_t(Ur, LDK, 16 * s, 32 * cb, lane), acc_o);
      put_pairs(acc_o, 32 * rb, lane, [&](int t, float x0, float x1) {
        const int j = j0 + t;
        if (j >= sq.n_replay && j < sq.n_tok) st2_g<bf16_t>(o + ((int64_t)rw[t] * H + head) * kD + (cc & ~1), x0, x1);
      });
    }
    __syncthreads();  // T and P of this chunk are read: the next chunk's replace them
    commit_tinv8(tx, Th, Tl, Pr, tid);

    // -- state update: S <- gamma_63 S + (diag(E_63,.) U)^T K ------------------------------
    {
      const float gn = gam[kB - 1];
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int r = 0; r < 16; ++r) S[b2][r] *= gn;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = egam[16 * s + 8 * hi + j];
        const f16x8 a = scale8(frag_t(Ur, LDK, 16 * s, 32 * cb, lane), e);
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2) S[b2] = mfma(a, frag_t(Kr, LDK, 16 * s, 32 * (2 * rb + b2), lane), S[b2]);
      }
    }
    if (ex < ex_end && exports[ex].chunk == c + 1) {
      state_store8(S, slots + ((int64_t)exports[ex].slot * H + head) * kD * kD, cb, rb, lane);
      ++ex;
    }
    __syncthreads();
    if (has_next) {
      if (stager) commit_chunk(nx, Kr, Qr, Rr, rw, gs, bs, tid);
      state_to_lds8(S, Sh, cb, rb, lane);
      if (kSave) state_save8(S, states + ((int64_t)(sq.chunk_off + c + 1) * H + head) * 2 * kD * kD, cb, rb, lane);
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------------
// Backward, serial part: one round, sequences in any order, chunks in reverse.  Carries
// only the state gradient dS (fp32, registers): at chunk c it is the gradient of the
// chunk's end state (consumers' initial-state gradients added at exported boundaries),
// saved as fp16 [dv][dk] for the per-chunk kernel; then
//   dU = diag(E_63,.) K dS^T + P^T dO,   dR = T^T dU,
//   dS <- gamma_63 dS + scale (diag(gamma) dO)^T Q - (diag(beta gamma) dR)^T K.
// At the sequence's start dS is its initial-state gradient.
// ---------------------------------------------------------------------------------
__global__ __launch_bounds__(512, 1) void gdn_bscan_kernel(
    const GSeq* __restrict__ seqs, const int32_t* __restrict__ order, const int32_t* __restrict__ grows,
    const GExport* __restrict__ exports, const int32_t* __restrict__ slot_off, const int32_t* __restrict__ slot_cons,
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const float* __restrict__ beta,
    const float* __restrict__ alpha, const bf16_t* __restrict__ dO, const f16_t* __restrict__ tinv,
    float* __restrict__ cgrad, f16_t* __restrict__ dsend, int round_item0, int H, float scale) {
  __shared__ __attribute__((aligned(16))) f16_t dSh[kD * LDK];
  __shared__ __attribute__((aligned(16))) f16_t Kr[kB * LDK];
  __shared__ __attribute__((aligned(16))) f16_t Qr[kB * LDK];
  __shared__ __attribute__((aligned(16))) f16_t dOr[kB * LDK];
  __shared__ __attribute__((aligned(16))) f16_t dRr[kB * LDK];  // dU, then dR
  __shared__ __attribute__((aligned(16))) f16_t Pr[kB * LDP];
  __shared__ __attribute__((aligned(16))) f16_t Th[kB * LDP];
  __shared__ __attribute__((aligned(16))) f16_t Tl[kB * LDP];
  __shared__ float gs[kB], bs[kB], al[kB], gam[kB], egam[kB];
  __shared__ int rw[kB];

  const int head = blockIdx.x % H;
  const GSeq sq = seqs[order[blockIdx.x / H]];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rb = wave >> 2, cb = wave & 3;
  const bool stager = tid < 256;  // the first four waves fetch and commit the chunk inputs
  const int nch = (sq.n_tok + kB - 1) / kB;
  const ChunkIn ci{grows + sq.tok_off, sq.n_tok, sq.n_replay};
  const f16_t* tinv_seq = tinv + (int64_t)sq.item0 * H * kTinv + (int64_t)head * kTinv;
  const int64_t tinv_step = (int64_t)H * kTinv;

  f32x16 D[2];  // dS, eight-wave state layout
#pragma unroll
  for (int b2 = 0; b2 < 2; ++b2) D[b2] = zero16();
  int ex = sq.exp_off + sq.exp_cnt - 1;
  BwdRegs nx;
  TinvRegs8 tx;
  if (nch > 0) {
    if (stager) {
      bwd_fetch_rows(ci, (nch - 1) * kB, tid, nx);
      bwd_fetch_data<false>(ci, (nch - 1) * kB, k, q, dO, nullptr, beta, alpha, H, head, tid, nx);
    }
    fetch_tinv8(tinv_seq + (nch - 1) * tinv_step, tid, tx);
  }

  for (int c = nch - 1; c >= 0; --c) {
    int tid_o = threadIdx.x;
    asm volatile("" : "+v"(tid_o));
    const int tid = tid_o, wave = tid >> 6, lane = tid & 63, hi = lane >> 5, l32 = lane & 31;
    const int rb = wave >> 2, cb = wave & 3;
    const int j0 = c * kB;
    // -- consumers' initial-state gradients enter at exported boundaries ----------------
    if (ex >= sq.exp_off && exports[ex].chunk == c + 1) {
      const int slot = exports[ex].slot;
      for (int e = slot_off[slot]; e < slot_off[slot + 1]; ++e) {
        f32x16 G[2];
        state_load8(G, cgrad + ((int64_t)slot_cons[e] * H + head) * kD * kD, cb, rb, lane);
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
          for (int r = 0; r < 16; ++r) D[b2][r] += G[b2][r];
      }
      --ex;
    }
    {
      f16_t* dst = dsend + ((int64_t)(sq.item0 - round_item0 + c) * H + head) * kD * kD;
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          dst[(32 * cb + acc_row(r, hi)) * kD + 32 * (2 * rb + b2) + l32] = (f16_t)D[b2][r];
    }
    state_to_lds8(D, dSh, cb, rb, lane);
    if (stager) bwd_commit<false>(nx, Kr, Qr, dOr, nullptr, rw, gs, bs, al, tid);
    commit_tinv8(tx, Th, Tl, Pr, tid);
    if (c > 0 && stager) bwd_fetch_rows(ci, j0 - kB, tid, nx);
    fetch_tinv8(tinv_seq + (c > 0 ? c - 1 : c) * tinv_step, tid, tx);
    __syncthreads();
    if (c > 0 && stager) bwd_fetch_data<false>(ci, j0 - kB, k, q, dO, nullptr, beta, alpha, H, head, tid, nx);
    if (tid < kB) {
      gam[tid] = __expf(gs[tid]);
      egam[tid] = __expf(gs[kB - 1] - gs[tid]);
    }
    const int cc = 32 * cb + l32;
    __syncthreads();

    // -- dU = diag(E_63,.) K dS^T + P^T dO ----------------------------------------------------
    {
      f32x16 du = zero16();
#pragma unroll
      for (int s = 0; s < 8; ++s)
        du = mfma(frag_n(Kr, LDK, 32 * rb, 16 * s, lane), frag_n(dSh, LDK, 32 * cb, 16 * s, lane), du);
#pragma unroll
      for (int r = 0; r < 16; ++r) du[r] *= egam[32 * rb + acc_row(r, hi)];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        du = mfma(frag_t(Pr, LDP, 16 * s, 32 * rb, lane), frag_t(dOr, LDK, 16 * s, 32 * cb, lane), du);
      lds_put_f16(du, dRr, LDK, 32 * rb, cc, lane);
    }
    __syncthreads();
    // -- dR = (I + A)^{-T} dU = T^T dU: T_hi^T dU + T_lo^T dU -----------------------------------
    {
      f32x16 dr = zero16();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const f16x8 b = frag_t(dRr, LDK, 16 * s, 32 * cb, lane);
        dr = mfma(frag_t(Th, LDP, 16 * s, 32 * rb, lane), b, dr);
        dr = mfma(frag_t(Tl, LDP, 16 * s, 32 * rb, lane), b, dr);
      }
      __syncthreads();  // every wave has read dU
      lds_put_f16(dr, dRr, LDK, 32 * rb, cc, lane);
    }
    __syncthreads();
    // -- dS_prev = gamma_63 dS + scale (diag(gamma) dO)^T Q - (diag(beta gamma) dR)^T K -----------
    {
      const float gn = gam[kB - 1];
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int r = 0; r < 16; ++r) D[b2][r] *= gn;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float e1[8], e2[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int t = 16 * s + 8 * hi + j;
          e1[j] = scale * gam[t];
          e2[j] = -bs[t] * gam[t];
        }
        const f16x8 a1 = scale8(frag_t(dOr, LDK, 16 * s, 32 * cb, lane), e1);
        const f16x8 a2 = scale8(frag_t(dRr, LDK, 16 * s, 32 * cb, lane), e2);
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2) {
          D[b2] = mfma(a1, frag_t(Qr, LDK, 16 * s, 32 * (2 * rb + b2), lane), D[b2]);
          D[b2] = mfma(a2, frag_t(Kr, LDK, 16 * s, 32 * (2 * rb + b2), lane), D[b2]);
        }
      }
    }
    __syncthreads();
  }
  if (sq.cgrad >= 0) state_store8(D, cgrad + ((int64_t)sq.cgrad * H + head) * kD * kD, cb, rb, lane);
}

// ---------------------------------------------------------------------------------
// Backward, parallel part: every input gradient of one chunk and head, given the
// chunk's start state S0 (saved by the forward's state pass), its end-state gradient
// dS (saved by the serial scan), T and P.  Grid: (round's chunk items) x H.  Eight
// waves, two per SIMD: wave (rb, cb) owns rows 32 rb .. and columns 32 cb .. of every
// [64][128] product; the [64][64] products run on waves 0..3 (block (bm, bn)).
// ---------------------------------------------------------------------------------
template <typename TG>
__global__ __launch_bounds__(512, 1) void gdn_bpar_kernel(
    const GSeq* __restrict__ seqs, const int32_t* __restrict__ items, int round_item0,
    const int32_t* __restrict__ grows, const int32_t* __restrict__ rep_slot, const bf16_t* __restrict__ q,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const float* __restrict__ beta,
    const float* __restrict__ alpha, const bf16_t* __restrict__ dO, const f16_t* __restrict__ states,
    const f16_t* __restrict__ tinv, const f16_t* __restrict__ dsend, TG* __restrict__ dq, TG* __restrict__ dk,
    TG* __restrict__ dv, float* __restrict__ dbeta, float* __restrict__ dalpha, float* __restrict__ rside,
    float* __restrict__ rbuf, int H, float scale) {
  constexpr int kW = 8;
  __shared__ __attribute__((aligned(16))) f16_t dSh[kD * LDK];
  __shared__ __attribute__((aligned(16))) f16_t Kr[kB * LDK];
  __shared__ __attribute__((aligned(16))) f16_t Qr[kB * LDK];
  __shared__ __attribute__((aligned(16))) f16_t dOr[kB * LDK];
  __shared__ __attribute__((aligned(16))) f16_t Ur[kB * LDK];   // R, then U
  __shared__ __attribute__((aligned(16))) f16_t dRr[kB * LDK];  // V rows, then dU, then dR
  __shared__ __attribute__((aligned(16))) f16_t Pr[kB * LDP];   // P, then dP~
  __shared__ __attribute__((aligned(16))) f16_t Th[kB * LDP];   // T high part, then dKk
  __shared__ __attribute__((aligned(16))) f16_t Tl[kB * LDP];
  // per-row values; 16-byte aligned for the accumulator lanes' float4 reads (rows16)
  __shared__ __attribute__((aligned(16))) float gs[kB];
  __shared__ __attribute__((aligned(16))) float bs[kB];
  __shared__ __attribute__((aligned(16))) float al[kB];
  __shared__ __attribute__((aligned(16))) float gam[kB];
  __shared__ __attribute__((aligned(16))) float egam[kB];
  __shared__ int rw[kB];
  // where row t's gradients go: 0 nowhere (past the sequence), 1 the replay buffer,
  // 2 the side buffer of a replayed row, 3 its own dk / dv row; with the base offset
  __shared__ int dst_kind[kB];
  __shared__ int64_t dst_off[kB];
  __shared__ float red_dg[kW][kB], red_g[kW][kB], red_b[kW][kB], red_e[kW][kB], red_s[kW], red_v[kB];

  const int head = blockIdx.x % H;
  const int ritem = blockIdx.x / H;      // within the round (its end-state gradient)
  const int item = round_item0 + ritem;  // among all items (its T and P)
  const GSeq sq = seqs[items[2 * item]];
  const int c = items[2 * item + 1];
  const int tid = threadIdx.x, lane = tid & 63, hi = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: wave-level branches stay scalar
  const int rb = wave >> 2, cb = wave & 3;  // this wave's 32-row, 32-column block
  const int j0 = c * kB;
  const ChunkIn ci{grows + sq.tok_off, sq.n_tok, sq.n_replay};
  f16_t* Kk = Th;
  const int cc = 32 * cb + l32;
  // The start state's fragments go out first, beside the chunk's rows: S0 (for K S0^T)
  // and its transposed copy (contraction over dv: dk rows 32 cb .., read once for
  // <dS, S0>, dQ and dK).  Neither depends on the rows, so their latency overlaps.
  const f16_t* S0n = states + ((int64_t)(sq.chunk_off + c) * H + head) * 2 * kD * kD;
  const f16_t* S0t = S0n + kD * kD;
  f16x8 s0f[8], s0n[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    s0n[s] = frag_g(S0n, 32 * cb, 16 * s, lane);
    s0f[s] = frag_g(S0t, 32 * cb, 16 * s, lane);
  }

  if (tid < 256) {
    BwdRegs nx;
    TinvRegs tx;
    fetch_tinv(tinv + ((int64_t)item * H + head) * kTinv, tid, tx);
    bwd_fetch_rows(ci, j0, tid, nx);
    bwd_fetch_data<true>(ci, j0, k, q, dO, v, beta, alpha, H, head, tid, nx);
    // the end-state gradient: thread tid takes dv rows tid / 2, columns 64 (tid & 1) ..
    const f16_t* src = dsend + ((int64_t)ritem * H + head) * kD * kD + (tid >> 1) * kD + 64 * (tid & 1);
#pragma unroll
    for (int m = 0; m < 8; ++m)
      *reinterpret_cast<uint4*>(dSh + (tid >> 1) * LDK + 64 * (tid & 1) + 8 * m) =
          reinterpret_cast<const uint4*>(src)[m];
    bwd_commit<true>(nx, Kr, Qr, dOr, dRr, rw, gs, bs, al, tid);
    commit_tinv(tx, Th, Tl, Pr, tid);
    if (tid < kB) {  // each row's destination, looked up once; the decay factors
      const int t = tid, row = rw[t], j = j0 + t;
      const int rs = row >= 0 ? rep_slot[row] : -1;
      int kind;
      int64_t off;
      if (j >= sq.n_tok) {
        kind = 0;
        off = 0;
      } else if (j < sq.n_replay) {
        kind = 1;
        off = ((int64_t)(sq.rep_off + j) * H + head) * kRep;
      } else if (rs >= 0) {
        kind = 2;
        off = ((int64_t)rs * H + head) * 2 * kD;
      } else {
        kind = 3;
        off = ((int64_t)row * H + head) * kD;
      }
      dst_kind[t] = kind;
      dst_off[t] = off;
    }
  }
  red_dg[wave][lane] = 0.f;
  red_g[wave][lane] = 0.f;
  red_b[wave][lane] = 0.f;
  red_e[wave][lane] = 0.f;
  __syncthreads();
  if (tid < kB) {
    gam[tid] = __expf(gs[tid]);
    egam[tid] = __expf(gs[kB - 1] - gs[tid]);
  }
  __syncthreads();

  // -- R = diag(beta) (V - diag(gamma) K S0^T) (fp16), then U = T R --------------------------
  f32x16 ks = zero16();  // K S0^T: used for R here and for R's beta/gamma derivatives below
  {
#pragma unroll
    for (int s = 0; s < 8; ++s)
      ks = mfma(frag_n(Kr, LDK, 32 * rb, 16 * s, lane), s0n[s], ks);
    float b16[16], g16[16];
    rows16(bs, rb, hi, b16);
    rows16(gam, rb, hi, g16);
    float v16[16];
    acc_col_f16(dRr, LDK, 32 * rb, 32 * cb, lane, v16);  // V rows, staged by bwd_commit
    f32x16 rr;
#pragma unroll
    for (int r = 0; r < 16; ++r) rr[r] = b16[r] * (v16[r] - g16[r] * ks[r]);
    lds_put_f16(rr, Ur, LDK, 32 * rb, cc, lane);
  }
  __syncthreads();
  {
    f32x16 u = zero16();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f16x8 b = frag_t(Ur, LDK, 16 * s, 32 * cb, lane);
      u = mfma(frag_n(Th, LDP, 32 * rb, 16 * s, lane), b, u);
      u = mfma(frag_n(Tl, LDP, 32 * rb, 16 * s, lane), b, u);
    }
    __syncthreads();  // every wave has read R
    lds_put_f16(u, Ur, LDK, 32 * rb, cc, lane);
  }

  // -- dU = scale P^T dO + diag(E_63,.) K dS^T --------------------------------------------
  {
    f32x16 du = zero16();
#pragma unroll
    for (int s = 0; s < 8; ++s)
      du = mfma(frag_n(Kr, LDK, 32 * rb, 16 * s, lane), frag_n(dSh, LDK, 32 * cb, 16 * s, lane), du);
    {
      float e16[16];
      rows16(egam, rb, hi, e16);
#pragma unroll
      for (int r = 0; r < 16; ++r) du[r] *= e16[r];
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
      du = mfma(frag_t(Pr, LDP, 16 * s, 32 * rb, lane), frag_t(dOr, LDK, 16 * s, 32 * cb, lane), du);
    lds_put_f16(du, dRr, LDK, 32 * rb, cc, lane);
  }
  __syncthreads();

  // -- dR = (I + A)^{-T} dU = T^T dU; dV = diag(beta) dR ---------------------------------------
  f16_t drh[16];  // this lane's dR elements as stored (fp16), reused below
  {
    f32x16 dr = zero16();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f16x8 b = frag_t(dRr, LDK, 16 * s, 32 * cb, lane);
      dr = mfma(frag_t(Th, LDP, 16 * s, 32 * rb, lane), b, dr);
      dr = mfma(frag_t(Tl, LDP, 16 * s, 32 * rb, lane), b, dr);
    }
    __syncthreads();  // every wave has read dU and T
#pragma unroll
    for (int r = 0; r < 16; ++r) drh[r] = (f16_t)dr[r];
    lds_put_f16(dr, dRr, LDK, 32 * rb, cc, lane);
    put_pairs(dr, 32 * rb, lane, [&](int t, float x0, float x1) {
      const int kind = dst_kind[t];
      const int64_t off = dst_off[t] + kD + (cc & ~1);
      const float b = bs[t];
      if (kind == 1) st2_g<float>(rbuf + off, b * x0, b * x1);
      else if (kind == 2) st2_g<float>(rside + off, b * x0, b * x1);
      else if (kind == 3) st2_g<TG>(dv + off - kD, b * x0, b * x1);
    });
  }
  __syncthreads();

  // -- <dS, S0> for the decay of the whole chunk: this wave's dk columns, dv rows 64 rb .. --
  {
    // lane holds S0[16 s + 8 hi + j][32 cb + l32] in s0f[s][j]
    // and dS[16 (4 rb + sb) + 8 hi + j][32 cb + l32] in frag_t(dSh, ..)[j]
    float s = 0.f;
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      const f16x8 ds8 = frag_t(dSh, LDK, 16 * (4 * rb + sb), 32 * cb, lane);
#pragma unroll
      for (int j = 0; j < 8; ++j) s += (float)ds8[j] * (float)(rb ? s0f[4 + sb][j] : s0f[sb][j]);
    }
#pragma unroll
    for (int off = 32; off >= 16; off >>= 1) s += __shfl_xor(s, off);
    s += from_xor1(s);
    s += from_xor2(s);
    s += from_ror4(s);
    s += from_ror8(s);  // every lane: the sum over the row's 16 lanes of the cross-row sums
    if (lane == 0) red_s[wave] = s;
  }
  // -- dP = dO U^T, dA = -dR U^T on block (bm, bn), waves 0..3 ---------------------------------
  if (wave < 4) {
    const int bm = wave >> 1, bn = wave & 1;
    f32x16 dp = zero16(), da = zero16(), kk = zero16(), qk = zero16();
    if (bm >= bn) {  // blocks on or below the diagonal: dA, KK and QK as well
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const f16x8 b = frag_n(Ur, LDK, 32 * bn, 16 * s, lane);
        const f16x8 bk = frag_n(Kr, LDK, 32 * bn, 16 * s, lane);
        dp = mfma(frag_n(dOr, LDK, 32 * bm, 16 * s, lane), b, dp);
        da = mfma(frag_n(dRr, LDK, 32 * bm, 16 * s, lane), b, da);
        kk = mfma(frag_n(Kr, LDK, 32 * bm, 16 * s, lane), bk, kk);
        qk = mfma(frag_n(Qr, LDK, 32 * bm, 16 * s, lane), bk, qk);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s)
        dp = mfma(frag_n(dOr, LDK, 32 * bm, 16 * s, lane), frag_n(Ur, LDK, 32 * bn, 16 * s, lane), dp);
    }
    const int i = 32 * bn + l32;
    const float gi = gs[i];
    float gt[16], b16[16];
    rows16(gs, bm, hi, gt);
    rows16(bs, bm, hi, b16);
    float xy[16], z[16];
    f32x16 dpt16, dkk16;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = 32 * bm + acc_row(r, hi);
      // E_ti = exp(g_t - g_i) on and below the diagonal; exp(-inf) = 0 above it (no branch)
      const float e = __expf(i <= t ? gt[r] - gi : -INFINITY);
      const float dpt = scale * e * dp[r];          // dP~ = d(QK) (scale and decay folded)
      const float dat = i < t ? -da[r] : 0.f;       // dA
      const float dkk = dat * b16[r] * e;           // d(KK)
      dpt16[r] = dpt;
      dkk16[r] = dkk;
      xy[r] = dpt * qk[r] + dkk * kk[r];            // dg from E_ti inside P and A
      z[r] = dat * e * kk[r];                       // dbeta through A
    }
    lds_put_f16(dpt16, Pr, LDP, 32 * bm, i, lane);
    lds_put_f16(dkk16, Kk, LDP, 32 * bm, i, lane);
    const float rs = rowsum16(xy, lane);
    const float rz = rowsum16(z, lane);
    const float cs = colsum16(xy);
    if (rowsum16_writer(lane)) {
      const int t = 32 * bm + acc_row(rowsum16_elem(lane), hi);
      red_dg[wave][t] += rs;
      red_b[wave][t] += rz;
    }
    if (hi == 0) red_dg[wave][i] -= cs;
  } else {
    // sum_c dR[t][c] V[t][c] (beta's derivative through R), on the waves the block above
    // leaves idle: thread (t, part) takes row t's columns 32 part .. 32 part + 31
    const int t = (tid - 256) >> 2, part = tid & 3;
    const int row = rw[t];
    uint4 vrow[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
      vrow[m] = row >= 0 ? *reinterpret_cast<const uint4*>(v + ((int64_t)row * H + head) * kD + 32 * part + 8 * m)
                         : make_uint4(0, 0, 0, 0);
    float acc = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const f16x8 d8 = *reinterpret_cast<const f16x8*>(dRr + t * LDK + 32 * part + 8 * m);
      const uint32_t w[4] = {vrow[m].x, vrow[m].y, vrow[m].z, vrow[m].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf((float)d8[2 * e], __uint_as_float(w[e] << 16), acc);
        acc = fmaf((float)d8[2 * e + 1], __uint_as_float(w[e] & 0xffff0000u), acc);
      }
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    if (part == 0) red_v[t] = acc;
  }
  // -- R's dependence on beta and gamma ------------------------------------------------------
  {
    float xb[16], xg[16], b16[16], g16[16];
    rows16(bs, rb, hi, b16);
    rows16(gam, rb, hi, g16);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float dr = (float)drh[r];
      xb[r] = -dr * g16[r] * ks[r];  // the dR V part is red_v
      xg[r] = -b16[r] * dr * ks[r];
    }
    const float sb = rowsum16(xb, lane);
    const float sg = rowsum16(xg, lane);
    if (rowsum16_writer(lane)) {
      const int t = 32 * rb + acc_row(rowsum16_elem(lane), hi);
      red_b[wave][t] += sb;
      red_g[wave][t] += sg;
    }
  }
  __syncthreads();  // dP~ and dKk (waves 0..3) are read by every wave below

  // -- dQ = scale diag(gamma) dO S0 + dP~ K ----------------------------------------------------
  {
    f32x16 aq = zero16();
#pragma unroll
    for (int s = 0; s < 8; ++s) aq = mfma(frag_n(dOr, LDK, 32 * rb, 16 * s, lane), s0f[s], aq);
    {
      float xg[16], g16[16], q16[16];
      rows16(gam, rb, hi, g16);
      acc_col_f16(Qr, LDK, 32 * rb, 32 * cb, lane, q16);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        xg[r] = scale * aq[r] * q16[r];
        aq[r] *= scale * g16[r];
      }
      const float sg = rowsum16(xg, lane);
      if (rowsum16_writer(lane)) red_g[wave][32 * rb + acc_row(rowsum16_elem(lane), hi)] += sg;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
      aq = mfma(frag_n(Pr, LDP, 32 * rb, 16 * s, lane), frag_t(Kr, LDK, 16 * s, 32 * cb, lane), aq);
    put_pairs(aq, 32 * rb, lane, [&](int t, float x0, float x1) {
      const int j = j0 + t;
      if (j >= sq.n_replay && j < sq.n_tok) st2_g<TG>(dq + ((int64_t)rw[t] * H + head) * kD + (cc & ~1), x0, x1);
    });
  }
  // -- dK = dP~^T Q + dKk K + dKk^T K + diag(E_63,.) U dS - diag(beta gamma) dR S0 -----------
  {
    f32x16 ak = zero16();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f16x8 bq = frag_t(Qr, LDK, 16 * s, 32 * cb, lane);
      const f16x8 bk = frag_t(Kr, LDK, 16 * s, 32 * cb, lane);
      ak = mfma(frag_t(Pr, LDP, 16 * s, 32 * rb, lane), bq, ak);
      ak = mfma(frag_n(Kk, LDP, 32 * rb, 16 * s, lane), bk, ak);
      ak = mfma(frag_t(Kk, LDP, 16 * s, 32 * rb, lane), bk, ak);
    }
    {
      f32x16 ud = zero16();
#pragma unroll
      for (int s = 0; s < 8; ++s)
        ud = mfma(frag_n(Ur, LDK, 32 * rb, 16 * s, lane), frag_t(dSh, LDK, 16 * s, 32 * cb, lane), ud);
      float xe[16], e16[16], k16[16];
      rows16(egam, rb, hi, e16);
      acc_col_f16(Kr, LDK, 32 * rb, 32 * cb, lane, k16);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        xe[r] = ud[r] * k16[r];
        ak[r] = fmaf(e16[r], ud[r], ak[r]);
      }
      const float se = rowsum16(xe, lane);
      if (rowsum16_writer(lane)) red_e[wave][32 * rb + acc_row(rowsum16_elem(lane), hi)] += se;
    }
    {
      f32x16 rs0 = zero16();
#pragma unroll
      for (int s = 0; s < 8; ++s) rs0 = mfma(frag_n(dRr, LDK, 32 * rb, 16 * s, lane), s0f[s], rs0);
      float b16[16], g16[16];
      rows16(bs, rb, hi, b16);
      rows16(gam, rb, hi, g16);
#pragma unroll
      for (int r = 0; r < 16; ++r) ak[r] = fmaf(-b16[r] * g16[r], rs0[r], ak[r]);
    }
    put_pairs(ak, 32 * rb, lane, [&](int t, float x0, float x1) {
      const int kind = dst_kind[t];
      const int64_t off = dst_off[t] + (cc & ~1);
      if (kind == 1) st2_g<float>(rbuf + off, x0, x1);
      else if (kind == 2) st2_g<float>(rside + off, x0, x1);
      else if (kind == 3) st2_g<TG>(dk + off, x0, x1);
    });
  }
  __syncthreads();

  // -- per-token dbeta, dalpha (reverse cumulative sum of dg) --------------------------------
  if (tid < kB) {
    const int t = tid;
    const float en = egam[t];
    float e_t = 0.f, dgp = 0.f, dgam = 0.f, db = 0.f, ss = 0.f;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      dgp += red_dg[w][t];
      dgam += red_g[w][t];
      db += red_b[w][t];
      e_t += red_e[w][t];
      ss += red_s[w];
    }
    db += red_v[t];
    float dg = dgp + gam[t] * dgam - e_t * en;
    float tot = e_t * en;  // sum over the chunk of dEn_i E_63,i goes to g_63
#pragma unroll
    for (int off = 32; off >= 16; off >>= 1) tot += __shfl_xor(tot, off);
    tot += from_xor1(tot);
    tot += from_xor2(tot);
    tot += from_ror4(tot);
    tot += from_ror8(tot);  // every lane: the wave's sum
    if (t == kB - 1) dg += tot + gam[kB - 1] * ss;
    // reverse inclusive scan: dlogalpha_t = sum_{s >= t} dg_s
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_down(dg, off, 64);
      if (t + off < 64) dg += y;
    }
    const int j = j0 + t;
    if (j < sq.n_tok) {
      const float da = dg / al[t];
      if (j < sq.n_replay) {
        float* rb_ = rbuf + ((int64_t)(sq.rep_off + j) * H + head) * kRep;
        rb_[2 * kD] = db;
        rb_[2 * kD + 1] = da;
      } else {
        dbeta[(int64_t)rw[t] * H + head] = db;
        dalpha[(int64_t)rw[t] * H + head] = da;
      }
    }
  }
}

// Rows that are replayed somewhere: own contribution (kept in fp32) plus every
// replayed occurrence's, in schedule order.  Grid: (rows with replays) x H;
// kFixThreads >= kRep threads, one per record element.
constexpr int kFixThreads = 320;
template <typename TG>
__global__ __launch_bounds__(kFixThreads) void gdn_fixup_kernel(const int32_t* __restrict__ rep_rows,
                                                        const int32_t* __restrict__ rep_off,
                                                        const int32_t* __restrict__ rep_tok,
                                                        const float* __restrict__ rside,
                                                        const float* __restrict__ rbuf, TG* __restrict__ dk,
                                                        TG* __restrict__ dv, float* __restrict__ dbeta,
                                                        float* __restrict__ dalpha, int H) {
  const int head = blockIdx.x % H;
  const int rs = blockIdx.x / H;
  const int row = rep_rows[rs];
  const int tid = threadIdx.x;
  const int e0 = rep_off[rs], e1 = rep_off[rs + 1];
  float acc = tid < 2 * kD ? rside[((int64_t)rs * H + head) * 2 * kD + tid] : 0.f;
  if (tid == 2 * kD) acc = dbeta[(int64_t)row * H + head];
  if (tid == 2 * kD + 1) acc = dalpha[(int64_t)row * H + head];
  if (tid < kRep)
    for (int e = e0; e < e1; ++e) acc += rbuf[((int64_t)rep_tok[e] * H + head) * kRep + tid];
  if (tid < kD) st_g<TG>(dk + ((int64_t)row * H + head) * kD + tid, acc);
  else if (tid < 2 * kD) st_g<TG>(dv + ((int64_t)row * H + head) * kD + tid - kD, acc);
  else if (tid == 2 * kD) dbeta[(int64_t)row * H + head] = acc;
  else if (tid == 2 * kD + 1) dalpha[(int64_t)row * H + head] = acc;
}

// Zero the padding rows of a [C, H, W] tensor.  Grid: pages x H.
template <typename T>
__global__ __launch_bounds__(256) void gdn_pad_kernel(T* __restrict__ x, const int32_t* __restrict__ page_nrows,
                                                      int H, int W) {
  const int head = blockIdx.x % H;
  const int64_t page = blockIdx.x / H;
  const int n = page_nrows[page];
  for (int i = threadIdx.x; i < (kB - n) * W; i += 256) {
    const int64_t row = page * kB + n + i / W;
    x[(row * H + head) * W + i % W] = T(0);
  }
}

}  // namespace gdn

// ---------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------
void launch_gdn_tinv(const GdnShape& s, int n_items, const int32_t* items, const bf16_t* q, const bf16_t* k,
                     const float* beta, const float* alpha, f16_t* tinv, hipStream_t st) {
  if (n_items <= 0) return;
  static_assert(gdn::kTinv == kGdnTinvHalfs, "chunk-inverse record size");
  gdn::gdn_tinv_kernel<<<dim3((unsigned)(n_items * s.H)), 256, 0, st>>>(s.seqs, items, s.rows, q, k, beta, alpha,
                                                                        tinv, s.H, s.scale);
}

void launch_gdn_fwd(const GdnShape& s, int n_seq, const int32_t* order, const bf16_t* q,
                    const bf16_t* k, const bf16_t* v, const float* beta, const float* alpha, const f16_t* tinv,
                    bf16_t* o, float* slots, f16_t* states, hipStream_t st) {
  if (n_seq <= 0) return;
  const dim3 grid((unsigned)(n_seq * s.H));
  if (o && states)
    gdn::gdn_fwd_kernel<true, true><<<grid, 512, 0, st>>>(s.seqs, order, s.rows, s.exports, q, k, v, beta, alpha,
                                                          tinv, o, slots, states, s.H, s.scale);
  else if (states)
    gdn::gdn_fwd_kernel<false, true><<<grid, 512, 0, st>>>(s.seqs, order, s.rows, s.exports, q, k, v, beta, alpha,
                                                           tinv, o, slots, states, s.H, s.scale);
  else
    gdn::gdn_fwd_kernel<true, false><<<grid, 512, 0, st>>>(s.seqs, order, s.rows, s.exports, q, k, v, beta, alpha,
                                                           tinv, o, slots, states, s.H, s.scale);
}

void launch_gdn_bscan(const GdnShape& s, int n_seq, const int32_t* order, int item0, const bf16_t* q,
                      const bf16_t* k, const float* beta, const float* alpha, const bf16_t* dO, const f16_t* tinv,
                      float* cgrad, f16_t* dsend, hipStream_t st) {
  if (n_seq <= 0) return;
  gdn::gdn_bscan_kernel<<<dim3((unsigned)(n_seq * s.H)), 512, 0, st>>>(
      s.seqs, order, s.rows, s.exports, s.slot_off, s.slot_cons, q, k, beta, alpha, dO, tinv, cgrad, dsend, item0,
      s.H, s.scale);
}

template <typename TG>
void launch_gdn_bpar(const GdnShape& s, int item0, int n_items, const bf16_t* q, const bf16_t* k,
                     const bf16_t* v, const float* beta, const float* alpha, const bf16_t* dO, const f16_t* states,
                     const f16_t* tinv, const f16_t* dsend, TG* dq, TG* dk, TG* dv, float* dbeta, float* dalpha,
                     float* rside, float* rbuf, hipStream_t st) {
  if (n_items <= 0) return;
  gdn::gdn_bpar_kernel<TG><<<dim3((unsigned)(n_items * s.H)), 512, 0, st>>>(
      s.seqs, s.items, item0, s.rows, s.rep_slot, q, k, v, beta, alpha, dO, states, tinv, dsend, dq, dk, dv, dbeta,
      dalpha, rside, rbuf, s.H, s.scale);
}

template <typename TG>
void launch_gdn_fixup(const GdnShape& s, int n_rows, const float* rside, const float* rbuf, TG* dk, TG* dv,
                      float* dbeta, float* dalpha, hipStream_t st) {
  if (n_rows <= 0) return;
  static_assert(gdn::kFixThreads >= gdn::kRep, "one thread per replay-record element");
  gdn::gdn_fixup_kernel<TG><<<dim3((unsigned)(n_rows * s.H)), gdn::kFixThreads, 0, st>>>(s.rep_rows, s.rep_off, s.rep_tok, rside,
                                                                           rbuf, dk, dv, dbeta, dalpha, s.H);
}

template <typename T>
void launch_gdn_pad(int64_t pages, const int32_t* page_nrows, T* x, int H, int W, hipStream_t st) {
  if (pages <= 0) return;
  gdn::gdn_pad_kernel<T><<<dim3((unsigned)(pages * H)), 256, 0, st>>>(x, page_nrows, H, W);
}

template void launch_gdn_bpar<bf16_t>(const GdnShape&, int, int, const bf16_t*, const bf16_t*,
                                      const bf16_t*, const float*, const float*, const bf16_t*, const f16_t*,
                                      const f16_t*, const f16_t*, bf16_t*, bf16_t*, bf16_t*, float*, float*, float*,
                                      float*, hipStream_t);
template void launch_gdn_bpar<float>(const GdnShape&, int, int, const bf16_t*, const bf16_t*,
                                     const bf16_t*, const float*, const float*, const bf16_t*, const f16_t*,
                                     const f16_t*, const f16_t*, float*, float*, float*, float*, float*, float*,
                                     float*, hipStream_t);
template void launch_gdn_fixup<bf16_t>(const GdnShape&, int, const float*, const float*, bf16_t*, bf16_t*, float*,
                                       float*, hipStream_t);
template void launch_gdn_fixup<float>(const GdnShape&, int, const float*, const float*, float*, float*, float*,
                                      float*, hipStream_t);
template void launch_gdn_pad<bf16_t>(int64_t, const int32_t*, bf16_t*, int, int, hipStream_t);
template void launch_gdn_pad<float>(int64_t, const int32_t*, float*, int, int, hipStream_t);

}  // namespace dagattn

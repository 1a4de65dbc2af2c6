// Launchers of the HIP kernels (defined in kernels.hip, called by abi.cpp).
#pragma once

#include <hip/hip_runtime.h>

#include "plan.hpp"

namespace dagattn {

typedef uint16_t bf16_t;  // bf16 bits

// Plan-table checks of device debug builds (compiled with DAG_DEBUG): the sizes the
// kernels check table entries against, the failure codes they record, and the host
// side.  In other builds dbg_enabled() is false and the other two do nothing.
struct DbgLimits {
  int32_t pages, masks;
  int64_t tiles, steps, qpages, pairs, groups, gsteps;
};
enum : uint32_t {
  kDbgQPage = 1,      // query page id or its launch-order index
  kDbgTileRange = 2,  // a query page's tile list outside the tile table
  kDbgTilePage = 3,   // a tile's KV page
  kDbgInterval = 4,   // a visible interval [lo, hi) not within [0, 64]
  kDbgMask = 5,       // a mask id outside the mask table
  kDbgPair = 6,       // a KV page pair (index or page)
  kDbgStepRange = 7,  // a pair's reader steps outside the step table
  kDbgStepPage = 8,   // a reader step's query page
  kDbgGroup = 9,      // a KV page group (index or page)
};
bool dbg_enabled();
bool dbg_set_limits(const DbgLimits& lim, hipStream_t st);
// the first recorded failure (code, value) and the failure count, cleared; waits for st
bool dbg_take(uint32_t out[3], hipStream_t st);
typedef _Float16 f16_t;

struct LaunchShape {
  int64_t C, pages;
  int Hq, Hkv, D;
  float scale;
  double log2_base;  // log2 of the rotary base; 0 => no rotation
};

void launch_cs(const LaunchShape& s, const int32_t* pos_of_row, float2* cs, hipStream_t st);
template <typename Tin, typename Tout>
void launch_relayout(const LaunchShape& s, const Tin* x, const float2* cs, const int32_t* page_nrows,
                     Tout* out_n, Tout* out_t, int H, hipStream_t st);
template <typename T>
void launch_rowdot(const LaunchShape& s, const T* o, const T* o_lo, const T* dO, const float* lse,
                   const int32_t* page_nrows, float2* ld, hipStream_t st);
// out[0 .. n) = 0, n <= 64 (integer maxima start from it)
void launch_zero_u32(uint32_t* out, int n, hipStream_t st);
// amax[0..3) = max |q|, |k|, |v| (and amax[3] = max |dO| when dO is given) over valid
// rows, as float bits; amax must be 0 first.
void launch_absmax(const LaunchShape& s, const bf16_t* q, const bf16_t* k, const bf16_t* v, const bf16_t* dO,
                   const int32_t* page_nrows, uint32_t* amax, hipStream_t st);
// MFMA-path prologue (D = 128, bf16 in): rotate / scale / relayout one tensor into its fp16
// page-major copy (out_n) and/or transposed copy (out_t), scaled by the power of two that
// maps the maximum *smax into [2^14, 2^15) for q and k (qk), into [1, 2) for v and dO.
void launch_prep16(const LaunchShape& s, const bf16_t* x, const float2* cs, const int32_t* page_nrows,
                   const uint32_t* smax, bool qk, f16_t* out_n, f16_t* out_t, int H, hipStream_t st);
// ld = (-sq sk lse / scale, -sv rowsum(fp16(sdo dO) (o + o_lo))) per (page, head, row), the
// scales from amax[0..3].
void launch_rowdot16(const LaunchShape& s, const bf16_t* o, const bf16_t* o_lo, const bf16_t* dO, const float* lse,
                     const int32_t* page_nrows, float2* ld, const uint32_t* amax, hipStream_t st);
// amax: the q, k, v maxima whose power-of-two scales the fp16 copies carry.  tile_mask /
// masks (packed plans; nullptr otherwise) select the kernels that read per-tile masks.
void launch_fwd_mfma(const LaunchShape& s, int64_t n_qp, const f16_t* qn, const f16_t* kn, const f16_t* vt,
                     const QPage* qpages, const int32_t* order, const Tile* tiles, const int32_t* tile_mask,
                     const uint64_t* masks, bf16_t* o, float* lse, bf16_t* o_lo, const uint32_t* amax,
                     hipStream_t st);
template <typename TG>
void launch_dq_mfma(const LaunchShape& s, int64_t n_qp, const f16_t* qn, const f16_t* kn, const f16_t* vn,
                    const f16_t* dOn, const float2* ld, const float2* cs, const uint32_t* dmax,
                    const QPage* qpages, const int32_t* order, const Tile* tiles, const int32_t* tile_mask,
                    const uint64_t* masks, TG* dq, const uint32_t* amax, hipStream_t st);
template <typename TG>
void launch_dkdv_mfma(const LaunchShape& s, int64_t n_pairs, const f16_t* qn, const f16_t* kn, const f16_t* vn,
                      const f16_t* dOn, const float2* ld, const float2* cs, const uint32_t* dmax,
                      const int32_t* pair_order, const int32_t* pairs, const int64_t* pair_off, const KStep* psteps,
                      const KMask* pmasks, const uint64_t* masks, const int32_t* page_nrows, TG* dk, TG* dv,
                      const uint32_t* amax, hipStream_t st);
template <typename TG>
void launch_dkdv_group(const LaunchShape& s, int64_t n_groups, const f16_t* qn, const f16_t* kn, const f16_t* vn,
                       const f16_t* dOn, const float2* ld, const float2* cs, const uint32_t* dmax,
                       const int32_t* group_order, const int32_t* groups, const int64_t* group_off,
                       const GStep* gsteps, const int32_t* page_nrows, TG* dk, TG* dv, const uint32_t* amax,
                       hipStream_t st);
template <typename T>
void launch_fwd_simple(const LaunchShape& s, int64_t n_qp, const float* qn, const float* kn, const T* v,
                       const QPage* qpages, const int32_t* order, const Tile* tiles, T* o, float* lse, T* o_lo,
                       hipStream_t st);
template <typename T, typename TG>
void launch_bwd_simple(const LaunchShape& s, int64_t n_qp, int64_t n_kvp, const float* qn, const float* kn,
                       const T* v, const T* dO, const float2* ld, const float2* cs, const QPage* qpages,
                       const int32_t* fwd_order, const Tile* tiles, const int32_t* bwd_order,
                       const int32_t* kv_off, const KEntry* ents, const int32_t* page_table,
                       const int32_t* page_nrows, TG* dq, TG* dk, TG* dv, hipStream_t st);

}  // namespace dagattn

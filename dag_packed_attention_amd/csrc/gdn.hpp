// Launchers of the gated-delta-rule kernels (defined in gdn.hip, called by abi.cpp).
#pragma once

#include <hip/hip_runtime.h>

#include "launch.hpp"

namespace dagattn {

// Halfs per (chunk item, head) of the chunk-inverse buffer: (I + A)^{-1} as fp16 high and
// low parts and P = scale E o QK^T (lower), three [64][64] tiles.
constexpr size_t kGdnTinvHalfs = 3 * 64 * 64;

// Device copies of the plan's linear-attention schedule and the layer's shape.
struct GdnShape {
  const GSeq* seqs;
  const int32_t* rows;        // sequence token -> compact row
  const GExport* exports;
  const int32_t* slot_off;    // slot -> consumers (initial-state gradient ids)
  const int32_t* slot_cons;
  const int32_t* rep_slot;    // row -> index among replayed rows, or -1
  const int32_t* rep_rows;    // replayed rows
  const int32_t* rep_off;     // replayed row -> its replay indices
  const int32_t* rep_tok;
  const int32_t* items;       // chunk items (sequence, chunk) of every round, round after round
  int H;
  float scale;
};

// The chunk items items[0 .. n_items) ((sequence, chunk) pairs; item i's record is i):
// T = (I + A)^{-1} (fp16 high and low parts) and P per item and head, into `tinv`.
void launch_gdn_tinv(const GdnShape& s, int n_items, const int32_t* items, const bf16_t* q, const bf16_t* k,
                     const float* beta, const float* alpha, f16_t* tinv, hipStream_t st);
// One round of the forward, after launch_gdn_tinv of every chunk item.  o non-null: write the
// outputs; states non-null: save every chunk's starting state (fp16, [dv][dk] then
// [dk][dv]) into `states` (the backward's recomputation passes only states; a forward
// that keeps its states for the backward passes both).  Every variant exports boundary
// states into `slots` (fp32).
void launch_gdn_fwd(const GdnShape& s, int n_seq, const int32_t* order, const bf16_t* q,
                    const bf16_t* k, const bf16_t* v, const float* beta, const float* alpha, const f16_t* tinv,
                    bf16_t* o, float* slots, f16_t* states, hipStream_t st);
// One round of the backward's state-gradient scan (the round's chunk items start at
// item0): every chunk's end-state gradient into `dsend` (fp16 [dv][dk] per item of the
// round and head), and each sequence's initial-state gradient into cgrad.
void launch_gdn_bscan(const GdnShape& s, int n_seq, const int32_t* order, int item0, const bf16_t* q,
                      const bf16_t* k, const float* beta, const float* alpha, const bf16_t* dO, const f16_t* tinv,
                      float* cgrad, f16_t* dsend, hipStream_t st);
// One round of the backward's per-chunk gradients (chunk items item0 .. item0 + n_items),
// after launch_gdn_bscan of the round.
template <typename TG>
void launch_gdn_bpar(const GdnShape& s, int item0, int n_items, const bf16_t* q, const bf16_t* k,
                     const bf16_t* v, const float* beta, const float* alpha, const bf16_t* dO, const f16_t* states,
                     const f16_t* tinv, const f16_t* dsend, TG* dq, TG* dk, TG* dv, float* dbeta, float* dalpha,
                     float* rside, float* rbuf, hipStream_t st);
// Replayed rows: own plus replayed contributions, in schedule order.
template <typename TG>
void launch_gdn_fixup(const GdnShape& s, int n_rows, const float* rside, const float* rbuf, TG* dk, TG* dv,
                      float* dbeta, float* dalpha, hipStream_t st);
// Zero the padding rows of a [C, H, W] tensor.
template <typename T>
void launch_gdn_pad(int64_t pages, const int32_t* page_nrows, T* x, int H, int W, hipStream_t st);

}  // namespace dagattn

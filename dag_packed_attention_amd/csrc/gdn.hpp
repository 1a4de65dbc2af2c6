// Launchers of the gated-delta-rule kernels (defined in gdn.hip, called by abi.cpp).
#pragma once

#include <hip/hip_runtime.h>

#include "launch.hpp"

namespace dagattn {

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
  int H;
  float scale;
};

// One round of the forward.  o non-null: write the outputs; states non-null: save
// every chunk's starting state (fp16, [dv][dk] then [dk][dv]) into `states` (the
// backward's recomputation passes only states; a forward that keeps its states for
// the backward passes both).  Every variant exports boundary states into `slots`
// (fp32).
void launch_gdn_fwd(const GdnShape& s, int n_seq, const int32_t* order, const bf16_t* q,
                    const bf16_t* k, const bf16_t* v, const float* beta, const float* alpha, bf16_t* o,
                    float* slots, f16_t* states, hipStream_t st);
// One round of the backward.
template <typename TG>
void launch_gdn_bwd(const GdnShape& s, int n_seq, const int32_t* order, const bf16_t* q, const bf16_t* k,
                    const bf16_t* v, const float* beta, const float* alpha, const bf16_t* dO, const f16_t* states,
                    float* cgrad, TG* dq, TG* dk, TG* dv, float* dbeta, float* dalpha, float* rside, float* rbuf,
                    hipStream_t st);
// Replayed rows: own plus replayed contributions, in schedule order.
template <typename TG>
void launch_gdn_fixup(const GdnShape& s, int n_rows, const float* rside, const float* rbuf, TG* dk, TG* dv,
                      float* dbeta, float* dalpha, hipStream_t st);
// Zero the padding rows of a [C, H, W] tensor.
template <typename T>
void launch_gdn_pad(int64_t pages, const int32_t* page_nrows, T* x, int H, int W, hipStream_t st);

}  // namespace dagattn

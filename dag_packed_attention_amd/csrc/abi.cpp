// C ABI of libdag_attn: plan management, workspace sizing and kernel launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <stdexcept>
#include <type_traits>
#include <string>
#include <vector>

#include "abi_internal.hpp"
#include "conv.hpp"
#include "gdn.hpp"
#include "harts_plan.hpp"
#include "launch.hpp"
#include "logprob.hpp"
#include "plan.hpp"

namespace dagattn {

struct DeviceTables {
  int device = -1;
  void* block = nullptr;
  int32_t* pos_of_row = nullptr;
  Tile* tiles = nullptr;
  QPage* qpages = nullptr;
  int32_t* fwd_order = nullptr;
  KEntry* kentries = nullptr;
  int32_t* kv_off = nullptr;
  int32_t* bwd_order = nullptr;
  int32_t* kgroups = nullptr;
  int64_t* kgroup_off = nullptr;
  GStep* kgsteps = nullptr;
  int32_t* group_order = nullptr;
  int32_t* kpairs = nullptr;
  int64_t* kpair_off = nullptr;
  KStep* kpsteps = nullptr;
  int32_t* pair_order = nullptr;
  int32_t* tile_mask = nullptr;   // packed plans only
  uint64_t* masks = nullptr;
  KMask* kstep_mask = nullptr;
  int32_t* page_table = nullptr;
  int32_t* page_nrows = nullptr;
  // linear-attention schedule
  GSeq* gseqs = nullptr;
  int32_t* grows = nullptr;
  GExport* gexports = nullptr;
  int32_t* gslot_off = nullptr;
  int32_t* gslot_cons = nullptr;
  int32_t* ground_seq = nullptr;
  int32_t* gitems = nullptr;
  int32_t* grep_rows = nullptr;
  int32_t* grep_off = nullptr;
  int32_t* grep_tok = nullptr;
  int32_t* grep_slot = nullptr;
  // short convolution
  int32_t* conv_prev = nullptr;
  int64_t* conv_ext_off = nullptr;
  ConvExt* conv_ext = nullptr;
};

struct Timing {
  std::vector<hipEvent_t> ev;     // 2 * capacity events
  std::vector<int> kernel;        // kernel id of each recorded pair
  int used = 0;
};

}  // namespace dagattn

using namespace dagattn;

namespace {

thread_local std::string g_err;

dag_status set_err(dag_status code, const std::string& msg) {
  g_err = msg;
  return code;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// A bump allocator over the caller's workspace.
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base((char*)b) {}
  template <typename T> T* take(size_t count) {
    T* p = base ? (T*)(base + off) : nullptr;
    off += align256(count * sizeof(T));
    return p;
  }
};

bool mfma_path(const dag_attn_params* p) {
  return p->dtype == DAG_DTYPE_BF16 && p->head_dim == 128 && p->n_q_heads == 4 * p->n_kv_heads;
}

dag_status check_params(const dag_attn_params* p) {
  if (!p) return set_err(DAG_E_INVALID, "null params");
  if (p->n_q_heads <= 0 || p->n_kv_heads <= 0 || p->n_q_heads % p->n_kv_heads)
    return set_err(DAG_E_UNSUPPORTED, "n_q_heads must be a positive multiple of n_kv_heads");
  if (p->head_dim < 2 || p->head_dim > 128 || (p->head_dim & 1))
    return set_err(DAG_E_UNSUPPORTED, "head_dim must be even and in [2, 128]");
  if (p->dtype != DAG_DTYPE_BF16 && p->dtype != DAG_DTYPE_FP32)
    return set_err(DAG_E_UNSUPPORTED, "dtype must be DAG_DTYPE_BF16 or DAG_DTYPE_FP32");
  if (p->grad_dtype != DAG_DTYPE_BF16 && p->grad_dtype != DAG_DTYPE_FP32)
    return set_err(DAG_E_UNSUPPORTED, "grad_dtype must be DAG_DTYPE_BF16 or DAG_DTYPE_FP32");
  if (p->dtype == DAG_DTYPE_FP32 && p->grad_dtype != DAG_DTYPE_FP32)
    return set_err(DAG_E_UNSUPPORTED, "fp32 inputs need fp32 gradients");
  if (!(p->rope_base >= 0.f) || std::isinf(p->rope_base) || (p->rope_base > 0.f && p->rope_base <= 1.f))
    return set_err(DAG_E_INVALID, "rope_base must be 0 (off) or > 1");
  // the kernels hide a score by sending it to -inf before the scale multiplies it, so
  // the scale must be positive (a negative one is the positive one with k negated)
  if (!std::isfinite(p->scale) || p->scale < 0.f)
    return set_err(DAG_E_INVALID, "scale must be finite and >= 0 (0 selects 1/sqrt(head_dim))");
  return DAG_OK;
}

LaunchShape shape_of(const Plan& P, const dag_attn_params* p) {
  LaunchShape s;
  s.C = P.info.rows;
  s.pages = P.info.pages;
  s.Hq = p->n_q_heads;
  s.Hkv = p->n_kv_heads;
  s.D = p->head_dim;
  s.scale = p->scale != 0.f ? p->scale : (float)(1.0 / std::sqrt((double)p->head_dim));
  s.log2_base = p->rope_base > 0.f ? std::log2((double)p->rope_base) : 0.0;
  return s;
}

// Workspace regions.  The same function sizes and carves them.
struct FwdWs {
  float2* cs;
  void* qn;
  void* kn;
  void* vt;
  uint32_t* amax;  // max |q|, |k|, |v| (float bits; MFMA path)
};
struct BwdWs {
  float2* cs;
  void* qn;
  void* kn;
  void* vn;
  void* dOn;
  float2* ld;
  uint32_t* amax;  // max |q|, |k|, |v|, |dO| (float bits)
};

size_t carve_fwd(const LaunchShape& s, bool mfma, void* base, FwdWs* w) {
  Carve c(base);
  const size_t C = (size_t)s.C;
  w->cs = s.log2_base > 0 ? c.take<float2>(C * (s.D / 2)) : nullptr;
  if (mfma) {
    w->qn = c.take<f16_t>(C * s.Hq * s.D);
    w->kn = c.take<f16_t>(C * s.Hkv * s.D);
    w->vt = c.take<f16_t>(C * s.Hkv * s.D);
    w->amax = c.take<uint32_t>(3);
  } else {
    w->qn = c.take<float>(C * s.Hq * s.D);
    w->kn = c.take<float>(C * s.Hkv * s.D);
    w->vt = nullptr;
    w->amax = nullptr;
  }
  return c.off;
}

size_t carve_bwd(const LaunchShape& s, bool mfma, void* base, BwdWs* w) {
  Carve c(base);
  const size_t C = (size_t)s.C;
  w->cs = s.log2_base > 0 ? c.take<float2>(C * (s.D / 2)) : nullptr;
  w->ld = c.take<float2>(C * s.Hq);
  w->amax = c.take<uint32_t>(4);
  if (mfma) {
    w->qn = c.take<f16_t>(C * s.Hq * s.D);
    w->dOn = c.take<f16_t>(C * s.Hq * s.D);
    w->kn = c.take<f16_t>(C * s.Hkv * s.D);
    w->vn = c.take<f16_t>(C * s.Hkv * s.D);
  } else {
    w->qn = c.take<float>(C * s.Hq * s.D);
    w->kn = c.take<float>(C * s.Hkv * s.D);
    w->vn = w->dOn = nullptr;
  }
  return c.off;
}

template <typename T> T* dev_take(char* block, size_t& off, size_t count) {
  T* p = (T*)(block + off);
  off += align256(count * sizeof(T));
  return p;
}

dag_status ensure_uploaded(Plan& P, hipStream_t st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return set_err(DAG_E_DEVICE, "hipGetDevice failed");
  if (P.dev) {
    if (P.dev->device != dev)
      return set_err(DAG_E_DEVICE, "plan was uploaded to device " + std::to_string(P.dev->device) +
                                       ", current device is " + std::to_string(dev));
    return DAG_OK;
  }
  size_t bytes = 0;
  bytes += align256(P.pos_of_row.size() * 4) + align256(P.tiles.size() * sizeof(Tile)) +
           align256(P.qpages.size() * sizeof(QPage)) + align256(P.fwd_order.size() * 4) +
           align256(P.kentries.size() * sizeof(KEntry)) + align256(P.kv_off.size() * 4) +
           align256(P.bwd_order.size() * 4) + align256(P.kgroups.size() * 4) +
           align256(P.kgroup_off.size() * 8) + align256(P.kgsteps.size() * sizeof(GStep)) +
           align256(P.group_order.size() * 4) + align256(P.kpairs.size() * 4) + align256(P.kpair_off.size() * 8) +
           align256(P.kpsteps.size() * sizeof(KStep)) + align256(P.pair_order.size() * 4) +
           align256(P.tile_mask.size() * 4) + align256(P.masks.size() * 8) +
           align256(P.kstep_mask.size() * sizeof(KMask)) +
           align256(P.page_table.size() * 4) +
           align256(P.page_nrows.size() * 4) + align256(P.gseqs.size() * sizeof(GSeq)) +
           align256(P.grows.size() * 4) + align256(P.gexports.size() * sizeof(GExport)) +
           align256(P.gslot_off.size() * 4) + align256(P.gslot_cons.size() * 4) + align256(P.ground_seq.size() * 4) +
           align256(P.gitems.size() * 4) + align256(P.grep_rows.size() * 4) + align256(P.grep_off.size() * 4) + align256(P.grep_tok.size() * 4) +
           align256(P.grep_slot.size() * 4) + align256(P.conv_prev.size() * 4) +
           align256(P.conv_ext_off.size() * 8) + align256(P.conv_ext.size() * sizeof(ConvExt)) + 256;
  DeviceTables* D = new (std::nothrow) DeviceTables();
  if (!D) return set_err(DAG_E_DEVICE, "out of host memory");
  D->device = dev;
  if (hipMalloc(&D->block, bytes) != hipSuccess) {
    delete D;
    (void)hipGetLastError();
    return set_err(DAG_E_DEVICE, "hipMalloc of " + std::to_string(bytes) + " plan bytes failed");
  }
  char* b = (char*)D->block;
  size_t off = 0;
  D->pos_of_row = dev_take<int32_t>(b, off, P.pos_of_row.size());
  D->tiles = dev_take<Tile>(b, off, P.tiles.size());
  D->qpages = dev_take<QPage>(b, off, P.qpages.size());
  D->fwd_order = dev_take<int32_t>(b, off, P.fwd_order.size());
  D->kentries = dev_take<KEntry>(b, off, P.kentries.size());
  D->kv_off = dev_take<int32_t>(b, off, P.kv_off.size());
  D->bwd_order = dev_take<int32_t>(b, off, P.bwd_order.size());
  D->kgroups = dev_take<int32_t>(b, off, P.kgroups.size());
  D->kgroup_off = dev_take<int64_t>(b, off, P.kgroup_off.size());
  D->kgsteps = dev_take<GStep>(b, off, P.kgsteps.size());
  D->group_order = dev_take<int32_t>(b, off, P.group_order.size());
  D->kpairs = dev_take<int32_t>(b, off, P.kpairs.size());
  D->kpair_off = dev_take<int64_t>(b, off, P.kpair_off.size());
  D->kpsteps = dev_take<KStep>(b, off, P.kpsteps.size());
  D->pair_order = dev_take<int32_t>(b, off, P.pair_order.size());
  D->tile_mask = P.packed ? dev_take<int32_t>(b, off, P.tile_mask.size()) : nullptr;
  D->masks = P.packed ? dev_take<uint64_t>(b, off, P.masks.size()) : nullptr;
  D->kstep_mask = P.packed ? dev_take<KMask>(b, off, P.kstep_mask.size()) : nullptr;
  D->page_table = dev_take<int32_t>(b, off, P.page_table.size());
  D->page_nrows = dev_take<int32_t>(b, off, P.page_nrows.size());
  D->gseqs = dev_take<GSeq>(b, off, P.gseqs.size());
  D->grows = dev_take<int32_t>(b, off, P.grows.size());
  D->gexports = dev_take<GExport>(b, off, P.gexports.size());
  D->gslot_off = dev_take<int32_t>(b, off, P.gslot_off.size());
  D->gslot_cons = dev_take<int32_t>(b, off, P.gslot_cons.size());
  D->ground_seq = dev_take<int32_t>(b, off, P.ground_seq.size());
  D->gitems = dev_take<int32_t>(b, off, P.gitems.size());
  D->grep_rows = dev_take<int32_t>(b, off, P.grep_rows.size());
  D->grep_off = dev_take<int32_t>(b, off, P.grep_off.size());
  D->grep_tok = dev_take<int32_t>(b, off, P.grep_tok.size());
  D->grep_slot = dev_take<int32_t>(b, off, P.grep_slot.size());
  D->conv_prev = dev_take<int32_t>(b, off, P.conv_prev.size());
  D->conv_ext_off = dev_take<int64_t>(b, off, P.conv_ext_off.size());
  D->conv_ext = dev_take<ConvExt>(b, off, P.conv_ext.size());
  auto put = [&](void* dst, const void* src, size_t n) {
    return n == 0 || hipMemcpyAsync(dst, src, n, hipMemcpyHostToDevice, st) == hipSuccess;
  };
  bool ok = put(D->pos_of_row, P.pos_of_row.data(), P.pos_of_row.size() * 4) &&
            put(D->tiles, P.tiles.data(), P.tiles.size() * sizeof(Tile)) &&
            put(D->qpages, P.qpages.data(), P.qpages.size() * sizeof(QPage)) &&
            put(D->fwd_order, P.fwd_order.data(), P.fwd_order.size() * 4) &&
            put(D->kentries, P.kentries.data(), P.kentries.size() * sizeof(KEntry)) &&
            put(D->kv_off, P.kv_off.data(), P.kv_off.size() * 4) &&
            put(D->bwd_order, P.bwd_order.data(), P.bwd_order.size() * 4) &&
            put(D->kgroups, P.kgroups.data(), P.kgroups.size() * 4) &&
            put(D->kgroup_off, P.kgroup_off.data(), P.kgroup_off.size() * 8) &&
            put(D->kgsteps, P.kgsteps.data(), P.kgsteps.size() * sizeof(GStep)) &&
            put(D->group_order, P.group_order.data(), P.group_order.size() * 4) &&
            put(D->kpairs, P.kpairs.data(), P.kpairs.size() * 4) &&
            put(D->kpair_off, P.kpair_off.data(), P.kpair_off.size() * 8) &&
            put(D->kpsteps, P.kpsteps.data(), P.kpsteps.size() * sizeof(KStep)) &&
            put(D->pair_order, P.pair_order.data(), P.pair_order.size() * 4) &&
            (!P.packed || (put(D->tile_mask, P.tile_mask.data(), P.tile_mask.size() * 4) &&
                           put(D->masks, P.masks.data(), P.masks.size() * 8) &&
                           put(D->kstep_mask, P.kstep_mask.data(), P.kstep_mask.size() * sizeof(KMask)))) &&
            put(D->page_table, P.page_table.data(), P.page_table.size() * 4) &&
            put(D->page_nrows, P.page_nrows.data(), P.page_nrows.size() * 4) &&
            put(D->gseqs, P.gseqs.data(), P.gseqs.size() * sizeof(GSeq)) &&
            put(D->grows, P.grows.data(), P.grows.size() * 4) &&
            put(D->gexports, P.gexports.data(), P.gexports.size() * sizeof(GExport)) &&
            put(D->gslot_off, P.gslot_off.data(), P.gslot_off.size() * 4) &&
            put(D->gslot_cons, P.gslot_cons.data(), P.gslot_cons.size() * 4) &&
            put(D->ground_seq, P.ground_seq.data(), P.ground_seq.size() * 4) &&
            put(D->gitems, P.gitems.data(), P.gitems.size() * 4) &&
            put(D->grep_rows, P.grep_rows.data(), P.grep_rows.size() * 4) &&
            put(D->grep_off, P.grep_off.data(), P.grep_off.size() * 4) &&
            put(D->grep_tok, P.grep_tok.data(), P.grep_tok.size() * 4) &&
            put(D->grep_slot, P.grep_slot.data(), P.grep_slot.size() * 4) &&
            put(D->conv_prev, P.conv_prev.data(), P.conv_prev.size() * 4) &&
            put(D->conv_ext_off, P.conv_ext_off.data(), P.conv_ext_off.size() * 8) &&
            put(D->conv_ext, P.conv_ext.data(), P.conv_ext.size() * sizeof(ConvExt));
  // the host vectors are pageable: finish the copies before returning
  ok = ok && hipStreamSynchronize(st) == hipSuccess;
  if (!ok) {
    (void)hipFree(D->block);
    delete D;
    (void)hipGetLastError();
    return set_err(DAG_E_DEVICE, "plan upload failed");
  }
  P.dev = D;
  return DAG_OK;
}

// Event pair around one kernel launch while timing is enabled.
struct Span {
  Timing* t;
  int slot = -1;
  hipStream_t st;
  Span(Plan& P, int kernel, hipStream_t s) : t(P.timing), st(s) {
    if (t && t->used < (int)t->kernel.size()) {
      slot = t->used++;
      t->kernel[slot] = kernel;
      (void)hipEventRecord(t->ev[2 * slot], st);
    }
  }
  ~Span() {
    if (slot >= 0) (void)hipEventRecord(t->ev[2 * slot + 1], st);
  }
};

void destroy_timing(Plan& P) {
  if (!P.timing) return;
  for (hipEvent_t e : P.timing->ev) (void)hipEventDestroy(e);
  delete P.timing;
  P.timing = nullptr;
}

dag_status launched(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_err(DAG_E_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
  return DAG_OK;
}

// Device debug builds: the plan's table sizes for the kernels' checks before an attention
// call, and the first recorded failure after it (which waits for the stream).
int32_t g_dbg_page_limit = 0;  // test override: page ids from this one on fail the checks
dag_status dbg_begin(const Plan& P, hipStream_t st) {
  if (!dbg_enabled()) return DAG_OK;
  DbgLimits lim;
  lim.pages = (int32_t)P.info.pages;
  if (g_dbg_page_limit > 0 && g_dbg_page_limit < lim.pages) lim.pages = g_dbg_page_limit;
  lim.masks = (int32_t)(P.masks.size() / 128);
  lim.tiles = (int64_t)P.tiles.size();
  lim.steps = (int64_t)P.kpsteps.size();
  lim.qpages = (int64_t)P.qpages.size();
  lim.pairs = (int64_t)P.kpairs.size() / 2;
  lim.groups = (int64_t)P.kgroups.size() / kGroup;
  lim.gsteps = (int64_t)P.kgsteps.size();
  if (!dbg_set_limits(lim, st)) return set_err(DAG_E_DEVICE, "upload of the debug check limits failed");
  return DAG_OK;
}
dag_status dbg_end(dag_status st, const char* what, hipStream_t stream) {
  if (st != DAG_OK || !dbg_enabled()) return st;
  uint32_t e[3];
  if (!dbg_take(e, stream)) return set_err(DAG_E_DEVICE, std::string(what) + ": reading the debug check record failed");
  if (e[0])
    return set_err(DAG_E_INVALID, std::string(what) + ": device check of the plan tables failed (code " +
                                      std::to_string(e[0]) + ", value " + std::to_string((int32_t)e[1]) + ", " +
                                      std::to_string(e[2]) + " failures)");
  return DAG_OK;
}


// ---- gated delta rule -------------------------------------------------------------
dag_status check_gdn(const Plan& P, const dag_gdn_params* p) {
  if (!p) return set_err(DAG_E_INVALID, "null params");
  if (P.info.gdn_chunk != 64)
    return set_err(DAG_E_UNSUPPORTED, "the plan needs a linear-attention schedule with gdn_chunk = 64");
  if (p->n_heads <= 0) return set_err(DAG_E_UNSUPPORTED, "n_heads must be positive");
  if (p->head_dim != 128) return set_err(DAG_E_UNSUPPORTED, "head_dim must be 128");
  if (p->dtype != DAG_DTYPE_BF16) return set_err(DAG_E_UNSUPPORTED, "dtype must be DAG_DTYPE_BF16");
  if (p->grad_dtype != DAG_DTYPE_BF16 && p->grad_dtype != DAG_DTYPE_FP32)
    return set_err(DAG_E_UNSUPPORTED, "grad_dtype must be DAG_DTYPE_BF16 or DAG_DTYPE_FP32");
  if (!std::isfinite(p->scale)) return set_err(DAG_E_INVALID, "scale must be finite");
  if (p->keep_states != 0 && p->keep_states != 1) return set_err(DAG_E_INVALID, "keep_states must be 0 or 1");
  return DAG_OK;
}

struct GdnWs {
  float* slots;
  f16_t* states;
  float* cgrad;
  float* rside;
  float* rbuf;
  f16_t* tinv;   // per chunk item: (I + A)^{-1} as fp16 high and low parts, and P
  f16_t* dsend;  // backward, per chunk item of one round: the state gradient at the chunk's end
};

size_t carve_gdn(const Plan& P, int H, bool bwd, void* base, GdnWs* w) {
  Carve c(base);
  const size_t st = (size_t)H * 128 * 128;
  const size_t items = (size_t)P.gdn_round_chunks_max * H;
  w->slots = c.take<float>((size_t)P.info.gdn_slots * st);
  w->tinv = c.take<f16_t>((size_t)P.info.gdn_chunks * H * kGdnTinvHalfs);
  w->states = bwd ? c.take<f16_t>((size_t)P.info.gdn_chunks * 2 * st) : nullptr;
  w->dsend = bwd ? c.take<f16_t>(items * 128 * 128) : nullptr;
  w->cgrad = bwd ? c.take<float>((size_t)P.gdn_ncgrad * st) : nullptr;
  w->rside = bwd ? c.take<float>(P.grep_rows.size() * H * 256) : nullptr;
  w->rbuf = bwd ? c.take<float>((size_t)P.info.gdn_replay * H * 258) : nullptr;
  return c.off;
}

GdnShape gdn_shape(const Plan& P, const dag_gdn_params* p) {
  const DeviceTables& D = *P.dev;
  GdnShape g;
  g.seqs = D.gseqs;
  g.rows = D.grows;
  g.exports = D.gexports;
  g.slot_off = D.gslot_off;
  g.slot_cons = D.gslot_cons;
  g.rep_slot = D.grep_slot;
  g.rep_rows = D.grep_rows;
  g.rep_off = D.grep_off;
  g.rep_tok = D.grep_tok;
  g.items = D.gitems;
  g.H = p->n_heads;
  g.scale = p->scale != 0.f ? p->scale : 1.f;
  return g;
}

}  // namespace

dag_status dagattn::set_error(dag_status code, const std::string& msg) { return set_err(code, msg); }

dag_status dagattn::attn_fwd_impl(dag_plan* plan, const dag_attn_params* p, const void* q, const void* k,
                                  const void* v, void* o, float* lse, void* o_lo, void* ws, size_t ws_bytes,
                                  void* hip_stream, bool allow_upload) {
  if (!plan) return set_err(DAG_E_INVALID, "null plan");
  dag_status st = check_params(p);
  if (st != DAG_OK) return st;
  Plan& P = plan->p;
  if (P.info.rows == 0) return DAG_OK;
  if (!q || !k || !v || !o || !lse) return set_err(DAG_E_INVALID, "null tensor pointer");
  if (o_lo && p->dtype != DAG_DTYPE_BF16) return set_err(DAG_E_INVALID, "o_lo is for bf16 tensors only");
  const LaunchShape s = shape_of(P, p);
  const bool mfma = mfma_path(p);
  if (P.packed && !mfma)
    return set_err(DAG_E_UNSUPPORTED, "packed page layouts run on the MFMA path only (bf16, head_dim 128, Hq = 4 Hkv)");
  FwdWs w;
  const size_t need = carve_fwd(s, mfma, nullptr, &w);
  if (!ws || ws_bytes < need)
    return set_err(DAG_E_WORKSPACE, "forward workspace needs " + std::to_string(need) + " bytes");
  hipStream_t stream = (hipStream_t)hip_stream;
  if (allow_upload) {
    if ((st = ensure_uploaded(P, stream)) != DAG_OK) return st;
  } else {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return set_err(DAG_E_DEVICE, "hipGetDevice failed");
    if (!P.dev) return set_err(DAG_E_INVALID, "the plan is not on the device yet: call dag_plan_upload first");
    if (P.dev->device != dev)
      return set_err(DAG_E_DEVICE, "plan was uploaded to device " + std::to_string(P.dev->device) +
                                       ", current device is " + std::to_string(dev));
  }
  carve_fwd(s, mfma, ws, &w);
  const DeviceTables& D = *P.dev;
  const int64_t n_qp = (int64_t)P.qpages.size();
  if ((st = dbg_begin(P, stream)) != DAG_OK) return st;
  {
    Span sp(P, DAG_K_PROLOGUE_FWD, stream);
    if (w.cs) launch_cs(s, D.pos_of_row, w.cs, stream);
    const int32_t* nr = D.page_nrows;
    if (mfma) {
      // each fp16 copy is scaled by the power of two that maps its tensor's maximum into
      // [2^14, 2^15) (q, k) or [1, 2) (v), so no finite bf16 input overflows fp16; the
      // kernels undo the scales exactly
      const bf16_t *q16 = (const bf16_t*)q, *k16 = (const bf16_t*)k, *v16 = (const bf16_t*)v;
      launch_zero_u32(w.amax, 3, stream);
      launch_absmax(s, q16, k16, v16, nullptr, nr, w.amax, stream);
      launch_prep16(s, q16, w.cs, nr, w.amax + 0, true, (f16_t*)w.qn, nullptr, s.Hq, stream);
      launch_prep16(s, k16, w.cs, nr, w.amax + 1, true, (f16_t*)w.kn, nullptr, s.Hkv, stream);
      launch_prep16(s, v16, nullptr, nr, w.amax + 2, false, nullptr, (f16_t*)w.vt, s.Hkv, stream);
    } else if (p->dtype == DAG_DTYPE_BF16) {
      launch_relayout<bf16_t, float>(s, (const bf16_t*)q, w.cs, nr, (float*)w.qn, nullptr, s.Hq, stream);
      launch_relayout<bf16_t, float>(s, (const bf16_t*)k, w.cs, nr, (float*)w.kn, nullptr, s.Hkv, stream);
    } else {
      launch_relayout<float, float>(s, (const float*)q, w.cs, nr, (float*)w.qn, nullptr, s.Hq, stream);
      launch_relayout<float, float>(s, (const float*)k, w.cs, nr, (float*)w.kn, nullptr, s.Hkv, stream);
    }
  }
  {
    Span sp(P, DAG_K_FWD, stream);
    if (mfma)
      launch_fwd_mfma(s, n_qp, (const f16_t*)w.qn, (const f16_t*)w.kn, (const f16_t*)w.vt, D.qpages, D.fwd_order,
                      D.tiles, D.tile_mask, D.masks, (bf16_t*)o, lse, (bf16_t*)o_lo, w.amax, stream);
    else if (p->dtype == DAG_DTYPE_BF16)
      launch_fwd_simple<bf16_t>(s, n_qp, (const float*)w.qn, (const float*)w.kn, (const bf16_t*)v, D.qpages,
                                D.fwd_order, D.tiles, (bf16_t*)o, lse, (bf16_t*)o_lo, stream);
    else
      launch_fwd_simple<float>(s, n_qp, (const float*)w.qn, (const float*)w.kn, (const float*)v, D.qpages,
                               D.fwd_order, D.tiles, (float*)o, lse, nullptr, stream);
  }
  return dbg_end(launched("dag_attn_fwd"), "dag_attn_fwd", stream);
}

extern "C" {

const char* dag_last_error(void) { return g_err.c_str(); }

dag_status dag_build(const dag_node* nodes, int32_t n_nodes, const dag_mount* mounts, int32_t n_mounts,
                     const dag_build_opts* opts, dag_plan** out) {
  if (!out) return set_err(DAG_E_INVALID, "null output pointer");
  *out = nullptr;
  dag_plan* plan = new (std::nothrow) dag_plan();
  if (!plan) return set_err(DAG_E_INVALID, "out of host memory");
  std::string err;
  dag_status st;
  try {
    st = build_plan(nodes, n_nodes, mounts, n_mounts, opts, &plan->p, &err);
  } catch (const std::bad_alloc&) {
    st = DAG_E_OVERFLOW;
    err = "out of host memory while building the plan";
  } catch (const std::length_error&) {
    st = DAG_E_OVERFLOW;
    err = "a table of the plan exceeds the host's size limits";
  } catch (const std::exception& e) {
    st = DAG_E_INVALID;
    err = std::string("building the plan failed: ") + e.what();
  }
  if (st != DAG_OK) {
    delete plan;
    return set_err(st, err);
  }
  *out = plan;
  g_err.clear();
  return DAG_OK;
}

void dag_plan_destroy(dag_plan* plan) {
  if (!plan) return;
  destroy_timing(plan->p);
  if (plan->p.dev) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != plan->p.dev->device) (void)hipSetDevice(plan->p.dev->device);
    (void)hipFree(plan->p.dev->block);
    if (cur >= 0 && cur != plan->p.dev->device) (void)hipSetDevice(cur);
    delete plan->p.dev;
  }
  delete plan;
}

dag_status dag_plan_info_get(const dag_plan* plan, dag_plan_info* out) {
  if (!plan || !out) return set_err(DAG_E_INVALID, "null argument");
  *out = plan->p.info;
  return DAG_OK;
}

dag_status dag_plan_stats_get(const dag_plan* plan, dag_plan_stats* out) {
  if (!plan || !out) return set_err(DAG_E_INVALID, "null argument");
  const Plan& P = plan->p;
  constexpr int64_t kTileBytes = 64 * 128 * 2;        // one fp16 64 x 128 tile
  constexpr int64_t kUnitBytes = 2 * 2 * 32 * 128 * 2 + 2 * 256;  // two heads' Q, dO rows + offsets
  dag_plan_stats st{};
  for (const QPage& q : P.qpages) st.fwd_tiles += q.tile_count;  // visits: a node's pages share its list
  st.dkdv_groups = (int64_t)P.kgroups.size() / kGroup;
  st.dkdv_group_steps = (int64_t)P.kgsteps.size();
  st.dkdv_pairs = (int64_t)P.kpairs.size() / 2;
  st.dkdv_pair_steps = (int64_t)P.kpsteps.size();
  st.fwd_staged_bytes = st.fwd_tiles * 2 * kTileBytes;
  st.dq_staged_bytes = st.fwd_staged_bytes;
  int64_t own_pages = 0;  // pages whose K and V tiles a group or pair loads once
  for (int32_t ph : P.kgroups) own_pages += ph >= 0;
  for (int32_t ph : P.kpairs) own_pages += ph >= 0;
  st.dkdv_staged_bytes = (st.dkdv_group_steps + st.dkdv_pair_steps) * 2 * kUnitBytes + own_pages * 2 * kTileBytes;
  *out = st;
  return DAG_OK;
}

dag_status dag_plan_rows(const dag_plan* plan, int32_t* row_of_token, int32_t* pos_of_row) {
  if (!plan) return set_err(DAG_E_INVALID, "null plan");
  if (row_of_token && !plan->p.row_of_token.empty())
    std::memcpy(row_of_token, plan->p.row_of_token.data(), plan->p.row_of_token.size() * 4);
  if (pos_of_row && !plan->p.pos_of_row.empty())
    std::memcpy(pos_of_row, plan->p.pos_of_row.data(), plan->p.pos_of_row.size() * 4);
  return DAG_OK;
}

namespace {
// Write the sorted values into out (up to cap) and their count into *n.
dag_status emit_rows(std::vector<int32_t>& v, int32_t* out, int32_t cap, int32_t* n) {
  std::sort(v.begin(), v.end());
  if (n) *n = (int32_t)v.size();
  if (out)
    for (int32_t i = 0; i < (int32_t)v.size() && i < cap; ++i) out[i] = v[i];
  return DAG_OK;
}
}  // namespace

dag_status dag_plan_visibility(const dag_plan* plan, int32_t row, int32_t* key_rows, int32_t cap, int32_t* n) {
  if (!plan || !n || cap < 0) return set_err(DAG_E_INVALID, "null argument");
  const Plan& P = plan->p;
  if (row < 0 || row >= P.info.rows) return set_err(DAG_E_INVALID, "row out of range");
  const int32_t Q = row / kPage, r = row % kPage;
  std::vector<int32_t> v;
  if (r < P.page_nrows[Q]) {
    for (const QPage& qp : P.qpages) {
      if (qp.phys != Q) continue;
      for (int32_t t = 0; t < qp.tile_count; ++t) {
        const Tile& tl = P.tiles[qp.tile_begin + t];
        const int32_t lo = tl.lohi & 0xff, hi = (tl.lohi >> 8) & 0xff;
        const int32_t mi = P.packed ? P.tile_mask[qp.tile_begin + t] : -1;
        const bool diag = t == qp.tile_count - 1;
        for (int32_t c = lo; c < hi; ++c) {
          if (mi < 0 && diag && c > r) continue;  // a masked tile's mask is exact by itself
          if (mi >= 0 && !((P.masks[(size_t)mi * 2 * kPage + r] >> c) & 1ull)) continue;
          v.push_back(tl.page * kPage + c);
        }
      }
    }
  }
  return emit_rows(v, key_rows, cap, n);
}

dag_status dag_plan_readers(const dag_plan* plan, int32_t row, int32_t* query_rows, int32_t cap, int32_t* n) {
  if (!plan || !n || cap < 0) return set_err(DAG_E_INVALID, "null argument");
  const Plan& P = plan->p;
  if (row < 0 || row >= P.info.rows) return set_err(DAG_E_INVALID, "row out of range");
  const int32_t K = row / kPage, c = row % kPage;
  std::vector<int32_t> v;
  const int64_t ngroups = (int64_t)P.kgroups.size() / kGroup;
  for (int64_t gr = 0; gr < ngroups && c < P.page_nrows[K]; ++gr) {
    for (int side = 0; side < kGroup; ++side) {
      if (P.kgroups[kGroup * gr + side] != K) continue;
      for (int64_t i = P.kgroup_off[gr]; i < P.kgroup_off[gr + 1]; ++i) {
        const GStep& st = P.kgsteps[i];
        const uint32_t inf = gvis_of(st, side);
        const int32_t lo = gvis_lo(inf), hi = gvis_hi(inf);
        const bool diag = gvis_diag(inf);
        if (c < lo || c >= hi) continue;
        for (int32_t rr = 0; rr < 32; ++rr) {
          const int32_t r = st.rb * 32 + rr;
          if (r >= P.page_nrows[st.qph] || (diag && c > r)) continue;
          v.push_back(st.qph * kPage + r);
        }
      }
    }
  }
  const int64_t npairs = (int64_t)P.kpairs.size() / 2;
  for (int64_t pr = 0; pr < npairs && c < P.page_nrows[K]; ++pr) {
    for (int side = 0; side < 2; ++side) {
      if (P.kpairs[2 * pr + side] != K) continue;
      for (int64_t i = P.kpair_off[pr]; i < P.kpair_off[pr + 1]; ++i) {
        const KStep& st = P.kpsteps[i];
        const uint32_t inf = ((uint32_t)st.info >> (16 * side)) & 0xffffu;
        const int32_t rb = st.info & 1, lo = (inf >> 1) & 0x7f, hi = (inf >> 8) & 0x7f;
        const bool diag = (inf >> 15) & 1;
        if (c < lo || c >= hi) continue;
        const int32_t mi = P.packed ? (side ? P.kstep_mask[i].b : P.kstep_mask[i].a) : -1;
        for (int32_t rr = 0; rr < 32; ++rr) {
          const int32_t r = rb * 32 + rr;
          if (r >= P.page_nrows[st.qph] || (diag && c > r)) continue;
          if (mi >= 0 && !((P.masks[(size_t)mi * 2 * kPage + kPage + c] >> r) & 1ull)) continue;
          v.push_back(st.qph * kPage + r);
        }
      }
    }
  }
  return emit_rows(v, query_rows, cap, n);
}

dag_status dag_plan_multiplicity(const dag_plan* plan, int32_t* mult) {
  if (!plan || !mult) return set_err(DAG_E_INVALID, "null argument");
  const Plan& P = plan->p;
  for (int32_t u = 0; u < P.n_nodes; ++u)
    for (int32_t i = 0; i < P.length[u]; ++i) mult[P.tok_off[u] + i] = P.leaves_below[u];
  return DAG_OK;
}

int32_t dag_debug_build(void) { return dbg_enabled() ? 1 : 0; }

dag_status dag_debug_limit_pages(int32_t max_pages) {
  if (!dbg_enabled()) return set_err(DAG_E_UNSUPPORTED, "dag_debug_limit_pages needs a device debug build");
  if (max_pages < 0) return set_err(DAG_E_INVALID, "max_pages must be >= 0");
  g_dbg_page_limit = max_pages;
  return DAG_OK;
}

dag_status dag_plan_starts(const dag_plan* plan, int32_t* start) {
  if (!plan || !start) return set_err(DAG_E_INVALID, "null argument");
  std::memcpy(start, plan->p.start.data(), plan->p.start.size() * 4);
  return DAG_OK;
}

dag_status dag_plan_node_ranges(const dag_plan* plan, int32_t u, int32_t* out, int32_t cap, int32_t* n) {
  if (!plan || !n) return set_err(DAG_E_INVALID, "null argument");
  const Plan& P = plan->p;
  if (u < 0 || u >= P.n_nodes) return set_err(DAG_E_INVALID, "node index out of range");
  const int64_t b = P.range_off[u], e = P.range_off[u + 1];
  *n = (int32_t)(e - b);
  for (int64_t i = b; i < e && i - b < cap && out; ++i)
    for (int j = 0; j < 3; ++j) out[3 * (i - b) + j] = P.ranges[3 * i + j];
  return DAG_OK;
}

dag_status dag_plan_gdn_seqs(const dag_plan* plan, dag_gdn_seq* out, int32_t cap, int32_t* n) {
  if (!plan || !n) return set_err(DAG_E_INVALID, "null argument");
  const Plan& P = plan->p;
  if (P.info.gdn_chunk <= 0) return set_err(DAG_E_INVALID, "plan was built without a linear-attention schedule");
  *n = (int32_t)P.gseq_info.size();
  for (int32_t i = 0; out && i < *n && i < cap; ++i) out[i] = P.gseq_info[i];
  return DAG_OK;
}

dag_status dag_attn_timing_enable(dag_plan* plan, int32_t enable, int32_t capacity) {
  if (!plan) return set_err(DAG_E_INVALID, "null plan");
  destroy_timing(plan->p);
  if (!enable) return DAG_OK;
  if (capacity <= 0 || capacity > (1 << 20)) return set_err(DAG_E_INVALID, "capacity out of range");
  Timing* t = new (std::nothrow) Timing();
  if (!t) return set_err(DAG_E_DEVICE, "out of host memory");
  t->ev.assign(2 * (size_t)capacity, nullptr);
  t->kernel.assign(capacity, -1);
  for (auto& e : t->ev)
    if (hipEventCreate(&e) != hipSuccess) {
      plan->p.timing = t;
      destroy_timing(plan->p);
      return set_err(DAG_E_DEVICE, "hipEventCreate failed");
    }
  plan->p.timing = t;
  return DAG_OK;
}

dag_status dag_attn_timing_read(dag_plan* plan, double* ms, int64_t* counts) {
  if (!plan || !ms || !counts) return set_err(DAG_E_INVALID, "null argument");
  for (int k = 0; k < DAG_K_COUNT; ++k) {
    ms[k] = 0;
    counts[k] = 0;
  }
  Timing* t = plan->p.timing;
  if (!t) return set_err(DAG_E_INVALID, "timing is not enabled");
  for (int i = 0; i < t->used; ++i) {
    float e = 0.f;
    if (hipEventSynchronize(t->ev[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&e, t->ev[2 * i], t->ev[2 * i + 1]) != hipSuccess)
      return set_err(DAG_E_DEVICE, "reading timing events failed");
    ms[t->kernel[i]] += e;
    counts[t->kernel[i]] += 1;
  }
  t->used = 0;
  return DAG_OK;
}

dag_status dag_plan_upload(dag_plan* plan, void* hip_stream) {
  if (!plan) return set_err(DAG_E_INVALID, "null plan");
  return ensure_uploaded(plan->p, (hipStream_t)hip_stream);
}

dag_status dag_attn_workspace(const dag_plan* plan, const dag_attn_params* p, size_t* fwd_bytes,
                              size_t* bwd_bytes) {
  if (!plan) return set_err(DAG_E_INVALID, "null plan");
  dag_status st = check_params(p);
  if (st != DAG_OK) return st;
  const LaunchShape s = shape_of(plan->p, p);
  FwdWs fw;
  BwdWs bw;
  if (fwd_bytes) *fwd_bytes = carve_fwd(s, mfma_path(p), nullptr, &fw);
  if (bwd_bytes) *bwd_bytes = carve_bwd(s, mfma_path(p), nullptr, &bw);
  return DAG_OK;
}

dag_status dag_attn_fwd(dag_plan* plan, const dag_attn_params* p, const void* q, const void* k, const void* v,
                        void* o, float* lse, void* o_lo, void* ws, size_t ws_bytes, void* hip_stream) {
  return attn_fwd_impl(plan, p, q, k, v, o, lse, o_lo, ws, ws_bytes, hip_stream, /*allow_upload=*/true);
}

dag_status dag_attn_bwd(dag_plan* plan, const dag_attn_params* p, const void* q, const void* k, const void* v,
                        const void* o, const float* lse, const void* o_lo, const void* dO, void* dq, void* dk,
                        void* dv, void* ws, size_t ws_bytes, void* hip_stream) {
  if (!plan) return set_err(DAG_E_INVALID, "null plan");
  dag_status st = check_params(p);
  if (st != DAG_OK) return st;
  Plan& P = plan->p;
  if (P.info.rows == 0) return DAG_OK;
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv)
    return set_err(DAG_E_INVALID, "null tensor pointer");
  if (o_lo && p->dtype != DAG_DTYPE_BF16) return set_err(DAG_E_INVALID, "o_lo is for bf16 tensors only");
  if (!o_lo && p->dtype == DAG_DTYPE_BF16)
    return set_err(DAG_E_INVALID, "the bf16 backward needs o_lo, the forward's rounding residual of o");
  const LaunchShape s = shape_of(P, p);
  const bool mfma = mfma_path(p);
  if (P.packed && !mfma)
    return set_err(DAG_E_UNSUPPORTED, "packed page layouts run on the MFMA path only (bf16, head_dim 128, Hq = 4 Hkv)");
  BwdWs w;
  const size_t need = carve_bwd(s, mfma, nullptr, &w);
  if (!ws || ws_bytes < need)
    return set_err(DAG_E_WORKSPACE, "backward workspace needs " + std::to_string(need) + " bytes");
  hipStream_t stream = (hipStream_t)hip_stream;
  if ((st = ensure_uploaded(P, stream)) != DAG_OK) return st;
  carve_bwd(s, mfma, ws, &w);
  if ((st = dbg_begin(P, stream)) != DAG_OK) return st;
  const DeviceTables& D = *P.dev;
  const int64_t n_qp = (int64_t)P.qpages.size(), n_kvp = (int64_t)P.bwd_order.size();
  if (mfma) {
    const bf16_t *q16 = (const bf16_t*)q, *k16 = (const bf16_t*)k, *v16 = (const bf16_t*)v;
    const bf16_t *o16 = (const bf16_t*)o, *d16 = (const bf16_t*)dO;
    {
      const int32_t* nr = D.page_nrows;
      Span sp(P, DAG_K_PROLOGUE_BWD, stream);
      if (w.cs) launch_cs(s, D.pos_of_row, w.cs, stream);
      // power-of-two scales for the fp16 copies of q, k, v (amax[0..2]) and dO (amax[3]); the
      // S and dP offsets in ld are formed in the scaled units
      launch_zero_u32(w.amax, 4, stream);
      launch_absmax(s, q16, k16, v16, d16, nr, w.amax, stream);
      launch_rowdot16(s, o16, (const bf16_t*)o_lo, d16, lse, nr, w.ld, w.amax, stream);
      launch_prep16(s, q16, w.cs, nr, w.amax + 0, true, (f16_t*)w.qn, nullptr, s.Hq, stream);
      launch_prep16(s, k16, w.cs, nr, w.amax + 1, true, (f16_t*)w.kn, nullptr, s.Hkv, stream);
      launch_prep16(s, v16, nullptr, nr, w.amax + 2, false, (f16_t*)w.vn, nullptr, s.Hkv, stream);
      launch_prep16(s, d16, nullptr, nr, w.amax + 3, false, (f16_t*)w.dOn, nullptr, s.Hq, stream);
    }
    auto grads = [&](auto* tag) {
      using TG = std::remove_pointer_t<decltype(tag)>;
      {
        Span sp(P, DAG_K_DKDV, stream);
        launch_dkdv_group<TG>(s, (int64_t)P.group_order.size(), (const f16_t*)w.qn, (const f16_t*)w.kn,
                              (const f16_t*)w.vn, (const f16_t*)w.dOn, w.ld, w.cs, w.amax + 3, D.group_order,
                              D.kgroups, D.kgroup_off, D.kgsteps, D.page_nrows, (TG*)dk, (TG*)dv, w.amax, stream);
        launch_dkdv_mfma<TG>(s, (int64_t)P.pair_order.size(), (const f16_t*)w.qn, (const f16_t*)w.kn,
                             (const f16_t*)w.vn, (const f16_t*)w.dOn, w.ld, w.cs, w.amax + 3, D.pair_order,
                             D.kpairs, D.kpair_off, D.kpsteps, D.kstep_mask, D.masks, D.page_nrows, (TG*)dk,
                             (TG*)dv, w.amax, stream);
      }
      {
        Span sp(P, DAG_K_DQ, stream);
        launch_dq_mfma<TG>(s, n_qp, (const f16_t*)w.qn, (const f16_t*)w.kn,
                           (const f16_t*)w.vn, (const f16_t*)w.dOn, w.ld, w.cs, w.amax + 3, D.qpages,
                           D.fwd_order, D.tiles, D.tile_mask, D.masks, (TG*)dq, w.amax, stream);
      }
    };
    if (p->grad_dtype == DAG_DTYPE_FP32)
      grads((float*)nullptr);
    else
      grads((bf16_t*)nullptr);
  } else if (p->dtype == DAG_DTYPE_BF16) {
    {
      Span sp(P, DAG_K_PROLOGUE_BWD, stream);
      if (w.cs) launch_cs(s, D.pos_of_row, w.cs, stream);
      launch_rowdot<bf16_t>(s, (const bf16_t*)o, (const bf16_t*)o_lo, (const bf16_t*)dO, lse, D.page_nrows, w.ld,
                            stream);
      launch_relayout<bf16_t, float>(s, (const bf16_t*)q, w.cs, D.page_nrows, (float*)w.qn, nullptr, s.Hq,
                                     stream);
      launch_relayout<bf16_t, float>(s, (const bf16_t*)k, w.cs, D.page_nrows, (float*)w.kn, nullptr, s.Hkv,
                                     stream);
    }
    Span sp(P, DAG_K_DKDV, stream);
    if (p->grad_dtype == DAG_DTYPE_FP32)
      launch_bwd_simple<bf16_t, float>(s, n_qp, n_kvp, (const float*)w.qn, (const float*)w.kn, (const bf16_t*)v,
                                       (const bf16_t*)dO, w.ld, w.cs, D.qpages, D.fwd_order, D.tiles, D.bwd_order,
                                       D.kv_off, D.kentries, D.page_table, D.page_nrows, (float*)dq, (float*)dk,
                                       (float*)dv, stream);
    else
      launch_bwd_simple<bf16_t, bf16_t>(s, n_qp, n_kvp, (const float*)w.qn, (const float*)w.kn, (const bf16_t*)v,
                                        (const bf16_t*)dO, w.ld, w.cs, D.qpages, D.fwd_order, D.tiles, D.bwd_order,
                                        D.kv_off, D.kentries, D.page_table, D.page_nrows, (bf16_t*)dq, (bf16_t*)dk,
                                        (bf16_t*)dv, stream);
  } else {
    {
      Span sp(P, DAG_K_PROLOGUE_BWD, stream);
      if (w.cs) launch_cs(s, D.pos_of_row, w.cs, stream);
      launch_rowdot<float>(s, (const float*)o, nullptr, (const float*)dO, lse, D.page_nrows, w.ld, stream);
      launch_relayout<float, float>(s, (const float*)q, w.cs, D.page_nrows, (float*)w.qn, nullptr, s.Hq,
                                    stream);
      launch_relayout<float, float>(s, (const float*)k, w.cs, D.page_nrows, (float*)w.kn, nullptr, s.Hkv,
                                    stream);
    }
    Span sp(P, DAG_K_DKDV, stream);
    launch_bwd_simple<float, float>(s, n_qp, n_kvp, (const float*)w.qn, (const float*)w.kn, (const float*)v,
                             (const float*)dO, w.ld, w.cs, D.qpages, D.fwd_order, D.tiles, D.bwd_order, D.kv_off,
                             D.kentries, D.page_table, D.page_nrows, (float*)dq, (float*)dk, (float*)dv, stream);
  }
  return dbg_end(launched("dag_attn_bwd"), "dag_attn_bwd", stream);
}

dag_status dag_gdn_workspace(const dag_plan* plan, const dag_gdn_params* p, size_t* fwd_bytes, size_t* bwd_bytes) {
  if (!plan) return set_err(DAG_E_INVALID, "null plan");
  dag_status st = check_gdn(plan->p, p);
  if (st != DAG_OK) return st;
  GdnWs w;
  if (fwd_bytes) *fwd_bytes = carve_gdn(plan->p, p->n_heads, p->keep_states != 0, nullptr, &w);
  if (bwd_bytes) *bwd_bytes = carve_gdn(plan->p, p->n_heads, true, nullptr, &w);
  return DAG_OK;
}

dag_status dag_gdn_fwd(dag_plan* plan, const dag_gdn_params* p, const void* q, const void* k, const void* v,
                       const float* beta, const float* alpha, void* o, void* ws, size_t ws_bytes, void* hip_stream) {
  if (!plan) return set_err(DAG_E_INVALID, "null plan");
  Plan& P = plan->p;
  dag_status st = check_gdn(P, p);
  if (st != DAG_OK) return st;
  if (P.info.rows == 0) return DAG_OK;
  if (!q || !k || !v || !beta || !alpha || !o) return set_err(DAG_E_INVALID, "null tensor pointer");
  GdnWs w;
  const bool keep = p->keep_states != 0;
  const size_t need = carve_gdn(P, p->n_heads, keep, nullptr, &w);
  if (need && (!ws || ws_bytes < need))
    return set_err(DAG_E_WORKSPACE, "linear-attention forward workspace needs " + std::to_string(need) + " bytes");
  hipStream_t stream = (hipStream_t)hip_stream;
  if ((st = ensure_uploaded(P, stream)) != DAG_OK) return st;
  carve_gdn(P, p->n_heads, keep, ws, &w);
  const GdnShape g = gdn_shape(P, p);
  const DeviceTables& D = *P.dev;
  {
    Span sp(P, DAG_K_GDN_FWD, stream);
    // every chunk's T and P at once (a forward that keeps its states keeps these too)
    launch_gdn_tinv(g, (int)P.info.gdn_chunks, D.gitems, (const bf16_t*)q, (const bf16_t*)k, beta, alpha, w.tinv,
                    stream);
    for (int r = 0; r < P.info.gdn_rounds; ++r)
      launch_gdn_fwd(g, P.ground_off[r + 1] - P.ground_off[r], D.ground_seq + P.ground_off[r], (const bf16_t*)q,
                     (const bf16_t*)k, (const bf16_t*)v, beta, alpha, w.tinv, (bf16_t*)o, w.slots,
                     keep ? w.states : nullptr, stream);
    launch_gdn_pad<bf16_t>(P.info.pages, D.page_nrows, (bf16_t*)o, p->n_heads, 128, stream);
  }
  return launched("dag_gdn_fwd");
}

dag_status dag_gdn_bwd(dag_plan* plan, const dag_gdn_params* p, const void* q, const void* k, const void* v,
                       const float* beta, const float* alpha, const void* dO, void* dq, void* dk, void* dv,
                       float* dbeta, float* dalpha, void* ws, size_t ws_bytes, void* hip_stream) {
  if (!plan) return set_err(DAG_E_INVALID, "null plan");
  Plan& P = plan->p;
  dag_status st = check_gdn(P, p);
  if (st != DAG_OK) return st;
  if (P.info.rows == 0) return DAG_OK;
  if (!q || !k || !v || !beta || !alpha || !dO || !dq || !dk || !dv || !dbeta || !dalpha)
    return set_err(DAG_E_INVALID, "null tensor pointer");
  GdnWs w;
  const size_t need = carve_gdn(P, p->n_heads, true, nullptr, &w);
  if (need && (!ws || ws_bytes < need))
    return set_err(DAG_E_WORKSPACE, "linear-attention backward workspace needs " + std::to_string(need) + " bytes");
  hipStream_t stream = (hipStream_t)hip_stream;
  if ((st = ensure_uploaded(P, stream)) != DAG_OK) return st;
  carve_gdn(P, p->n_heads, true, ws, &w);
  const GdnShape g = gdn_shape(P, p);
  const DeviceTables& D = *P.dev;
  const int H = p->n_heads;
  const bf16_t *q16 = (const bf16_t*)q, *k16 = (const bf16_t*)k, *v16 = (const bf16_t*)v, *d16 = (const bf16_t*)dO;
  if (!p->keep_states) {  // otherwise the forward left every chunk's state, T and P in ws
    Span sp(P, DAG_K_GDN_STATES, stream);
    launch_gdn_tinv(g, (int)P.info.gdn_chunks, D.gitems, q16, k16, beta, alpha, w.tinv, stream);
    for (int r = 0; r < P.info.gdn_rounds; ++r)
      launch_gdn_fwd(g, P.ground_off[r + 1] - P.ground_off[r], D.ground_seq + P.ground_off[r], q16, k16, v16, beta,
                     alpha, w.tinv, nullptr, w.slots, w.states, stream);
  }
  auto run = [&](auto* tag) {
    using TG = std::remove_pointer_t<decltype(tag)>;
    Span sp(P, DAG_K_GDN_BWD, stream);
    for (int r = P.info.gdn_rounds - 1; r >= 0; --r) {
      const int item0 = P.gitem_off[r], n_items = P.gitem_off[r + 1] - item0;
      launch_gdn_bscan(g, P.ground_off[r + 1] - P.ground_off[r], D.ground_seq + P.ground_off[r], item0, q16, k16,
                       beta, alpha, d16, w.tinv, w.cgrad, w.dsend, stream);
      launch_gdn_bpar<TG>(g, item0, n_items, q16, k16, v16, beta, alpha, d16, w.states, w.tinv, w.dsend, (TG*)dq,
                          (TG*)dk, (TG*)dv, dbeta, dalpha, w.rside, w.rbuf, stream);
    }
    launch_gdn_fixup<TG>(g, (int)P.grep_rows.size(), w.rside, w.rbuf, (TG*)dk, (TG*)dv, dbeta, dalpha, stream);
    launch_gdn_pad<TG>(P.info.pages, D.page_nrows, (TG*)dq, H, 128, stream);
    launch_gdn_pad<TG>(P.info.pages, D.page_nrows, (TG*)dk, H, 128, stream);
    launch_gdn_pad<TG>(P.info.pages, D.page_nrows, (TG*)dv, H, 128, stream);
    launch_gdn_pad<float>(P.info.pages, D.page_nrows, dbeta, H, 1, stream);
    launch_gdn_pad<float>(P.info.pages, D.page_nrows, dalpha, H, 1, stream);
  };
  if (p->grad_dtype == DAG_DTYPE_FP32)
    run((float*)nullptr);
  else
    run((bf16_t*)nullptr);
  return launched("dag_gdn_bwd");
}

// ---- compact-to-semantic log-probabilities -----------------------------------------
dag_status dag_plan_logprob_map(const dag_plan* plan, const int32_t* labels, int64_t cap, int32_t* pos_row,
                                int32_t* pos_target, int32_t* row_first, int32_t* row_pos, int64_t* n_pos) {
  if (!plan || !labels || !n_pos) return set_err(DAG_E_INVALID, "null argument");
  const Plan& P = plan->p;
  std::vector<int32_t> rows, targets;
  std::string err;
  dag_status st;
  try {
    st = build_logprob_map(P, labels, &rows, &targets, &err);
  } catch (const std::bad_alloc&) {
    return set_err(DAG_E_OVERFLOW, "out of host memory building the position map");
  } catch (const std::length_error&) {
    return set_err(DAG_E_OVERFLOW, "sizes beyond the host's limits building the position map");
  } catch (const std::exception& e) {
    return set_err(DAG_E_INVALID, std::string("building the position map failed: ") + e.what());
  }
  if (st != DAG_OK) return set_err(st, err);
  const int64_t n = (int64_t)rows.size();
  *n_pos = n;
  if (cap < n || !pos_row || !pos_target || !row_first || !row_pos) return DAG_OK;
  const int64_t C = P.info.rows;
  if (n) {
    std::memcpy(pos_row, rows.data(), n * 4);
    std::memcpy(pos_target, targets.data(), n * 4);
  }
  // counting sort by row, stable: batch order within a row
  std::vector<int32_t> cnt(C + 1, 0);
  for (int32_t r : rows) ++cnt[r + 1];
  for (int64_t c = 0; c < C; ++c) cnt[c + 1] += cnt[c];
  std::memcpy(row_first, cnt.data(), (C + 1) * 4);
  for (int64_t s = 0; s < n; ++s) row_pos[cnt[rows[s]]++] = (int32_t)s;
  return DAG_OK;
}

namespace {
dag_status check_lp(const dag_logprob_params* p) {
  if (!p) return set_err(DAG_E_INVALID, "null params");
  if (p->rows < 0 || p->n_pos < 0 || p->vocab < 1) return set_err(DAG_E_INVALID, "negative size or vocab < 1");
  if (p->n_pos > INT32_MAX) return set_err(DAG_E_OVERFLOW, "more than 2^31 - 1 positions");
  if ((p->dtype != DAG_DTYPE_BF16 && p->dtype != DAG_DTYPE_FP32) ||
      (p->grad_dtype != DAG_DTYPE_BF16 && p->grad_dtype != DAG_DTYPE_FP32))
    return set_err(DAG_E_UNSUPPORTED, "dtype must be DAG_DTYPE_BF16 or DAG_DTYPE_FP32");
  if (p->rows > INT64_MAX / 4 / p->vocab) return set_err(DAG_E_OVERFLOW, "rows * vocab overflows");
  return DAG_OK;
}

bool aligned_to(const void* x, size_t a) { return (reinterpret_cast<uintptr_t>(x) % a) == 0; }
}  // namespace

dag_status dag_logprob_fwd(const dag_logprob_params* p, const void* z, const int32_t* row_first,
                           const int32_t* row_pos, const int32_t* pos_target, float* lse, float* lambda,
                           void* hip_stream) {
  dag_status st = check_lp(p);
  if (st != DAG_OK) return st;
  if (p->rows == 0) return DAG_OK;
  if (!z || !row_first || !lse || (p->n_pos > 0 && (!row_pos || !pos_target || !lambda)))
    return set_err(DAG_E_INVALID, "null tensor pointer");
  const size_t ez = p->dtype == DAG_DTYPE_BF16 ? 2 : 4;
  if (!aligned_to(z, ez)) return set_err(DAG_E_INVALID, "z is not aligned to its element size");
  hipStream_t stream = (hipStream_t)hip_stream;
  if (p->dtype == DAG_DTYPE_BF16)
    launch_lp_fwd<uint16_t>((const uint16_t*)z, p->rows, p->vocab, row_first, row_pos, pos_target, p->n_pos, lse,
                            lambda, stream);
  else
    launch_lp_fwd<float>((const float*)z, p->rows, p->vocab, row_first, row_pos, pos_target, p->n_pos, lse, lambda,
                         stream);
  return launched("dag_logprob_fwd");
}

dag_status dag_logprob_bwd(const dag_logprob_params* p, const void* z, const float* lse, const int32_t* row_first,
                           const int32_t* row_pos, const int32_t* pos_target, const float* g, void* dz,
                           void* hip_stream) {
  dag_status st = check_lp(p);
  if (st != DAG_OK) return st;
  if (p->rows == 0) return DAG_OK;
  if (!z || !lse || !row_first || !dz || (p->n_pos > 0 && (!row_pos || !pos_target || !g)))
    return set_err(DAG_E_INVALID, "null tensor pointer");
  const size_t ez = p->dtype == DAG_DTYPE_BF16 ? 2 : 4, eg = p->grad_dtype == DAG_DTYPE_BF16 ? 2 : 4;
  if (!aligned_to(z, ez) || !aligned_to(dz, eg))
    return set_err(DAG_E_INVALID, "z or dz is not aligned to its element size");
  hipStream_t stream = (hipStream_t)hip_stream;
  const int64_t C = p->rows, n = p->n_pos;
  const int V = p->vocab;
  if (p->dtype == DAG_DTYPE_BF16) {
    if (p->grad_dtype == DAG_DTYPE_BF16)
      launch_lp_bwd<uint16_t, uint16_t>((const uint16_t*)z, lse, C, V, row_first, row_pos, pos_target, g, n,
                                        (uint16_t*)dz, stream);
    else
      launch_lp_bwd<uint16_t, float>((const uint16_t*)z, lse, C, V, row_first, row_pos, pos_target, g, n, (float*)dz,
                                     stream);
  } else {
    if (p->grad_dtype == DAG_DTYPE_BF16)
      launch_lp_bwd<float, uint16_t>((const float*)z, lse, C, V, row_first, row_pos, pos_target, g, n,
                                     (uint16_t*)dz, stream);
    else
      launch_lp_bwd<float, float>((const float*)z, lse, C, V, row_first, row_pos, pos_target, g, n, (float*)dz,
                                  stream);
  }
  return launched("dag_logprob_bwd");
}

// ---- short causal convolution ------------------------------------------------------
namespace {
dag_status check_conv(const dag_conv_params* p) {
  if (!p) return set_err(DAG_E_INVALID, "null params");
  if (p->channels < 8 || p->channels % 8) return set_err(DAG_E_UNSUPPORTED, "channels must be a positive multiple of 8");
  if (p->width < 1 || p->width > 4) return set_err(DAG_E_UNSUPPORTED, "width must be 1..4");
  if (p->activation != DAG_ACT_NONE && p->activation != DAG_ACT_SILU)
    return set_err(DAG_E_UNSUPPORTED, "activation must be DAG_ACT_NONE or DAG_ACT_SILU");
  if (p->grad_dtype != DAG_DTYPE_BF16 && p->grad_dtype != DAG_DTYPE_FP32)
    return set_err(DAG_E_UNSUPPORTED, "grad_dtype must be DAG_DTYPE_BF16 or DAG_DTYPE_FP32");
  return DAG_OK;
}
size_t conv_ws_bytes(const Plan& P, const dag_conv_params* p) {
  return P.info.pages ? (size_t)conv_bwd_blocks(P.info.pages) * p->channels * 4 * sizeof(float) : 0;
}
bool aligned16(const void* x) { return (reinterpret_cast<uintptr_t>(x) & 15) == 0; }
}  // namespace

dag_status dag_conv_workspace(const dag_plan* plan, const dag_conv_params* p, size_t* bwd_bytes) {
  if (!plan || !bwd_bytes) return set_err(DAG_E_INVALID, "null argument");
  dag_status st = check_conv(p);
  if (st != DAG_OK) return st;
  if (plan->p.packed) return set_err(DAG_E_UNSUPPORTED, "the convolution needs a plan with one node per page");
  *bwd_bytes = conv_ws_bytes(plan->p, p);
  return DAG_OK;
}

dag_status dag_conv_fwd(dag_plan* plan, const dag_conv_params* p, const void* x, const float* weight, void* y,
                        void* hip_stream) {
  if (!plan) return set_err(DAG_E_INVALID, "null plan");
  Plan& P = plan->p;
  dag_status st = check_conv(p);
  if (st != DAG_OK) return st;
  if (plan->p.packed) return set_err(DAG_E_UNSUPPORTED, "the convolution needs a plan with one node per page");
  if (P.info.rows == 0) return DAG_OK;
  if (!x || !weight || !y) return set_err(DAG_E_INVALID, "null tensor pointer");
  if (!aligned16(x) || !aligned16(y)) return set_err(DAG_E_INVALID, "x and y must be 16-byte aligned");
  hipStream_t stream = (hipStream_t)hip_stream;
  if ((st = ensure_uploaded(P, stream)) != DAG_OK) return st;
  {
    Span sp(P, DAG_K_CONV_FWD, stream);
    launch_conv_fwd((const uint16_t*)x, weight, p->channels, p->width, p->activation, P.dev->page_nrows,
                    P.dev->conv_prev, P.info.pages, (uint16_t*)y, stream);
  }
  return launched("dag_conv_fwd");
}

dag_status dag_conv_bwd(dag_plan* plan, const dag_conv_params* p, const void* x, const float* weight,
                        const void* dy, void* dx, float* dweight, void* ws, size_t ws_bytes, void* hip_stream) {
  if (!plan) return set_err(DAG_E_INVALID, "null plan");
  Plan& P = plan->p;
  dag_status st = check_conv(p);
  if (st != DAG_OK) return st;
  if (plan->p.packed) return set_err(DAG_E_UNSUPPORTED, "the convolution needs a plan with one node per page");
  if (P.info.rows == 0) return DAG_OK;
  if (!x || !weight || !dy || !dx || !dweight) return set_err(DAG_E_INVALID, "null tensor pointer");
  if (!aligned16(x) || !aligned16(dy) || !aligned16(dx) || !aligned16(ws))
    return set_err(DAG_E_INVALID, "x, dy, dx and the workspace must be 16-byte aligned");
  const size_t need = conv_ws_bytes(P, p);
  if (!ws || ws_bytes < need)
    return set_err(DAG_E_WORKSPACE, "convolution backward workspace needs " + std::to_string(need) + " bytes");
  hipStream_t stream = (hipStream_t)hip_stream;
  if ((st = ensure_uploaded(P, stream)) != DAG_OK) return st;
  const DeviceTables& D = *P.dev;
  {
    Span sp(P, DAG_K_CONV_BWD, stream);
    if (p->grad_dtype == DAG_DTYPE_FP32)
      launch_conv_bwd<float>((const uint16_t*)x, (const uint16_t*)dy, weight, p->channels, p->width, p->activation,
                             D.page_nrows, D.conv_prev, D.conv_ext_off, D.conv_ext, P.info.pages, (float*)dx, dweight,
                             (float*)ws, stream);
    else
      launch_conv_bwd<uint16_t>((const uint16_t*)x, (const uint16_t*)dy, weight, p->channels, p->width,
                                p->activation, D.page_nrows, D.conv_prev, D.conv_ext_off, D.conv_ext, P.info.pages,
                                (uint16_t*)dx, dweight, (float*)ws, stream);
  }
  return launched("dag_conv_bwd");
}

// ---- trajectory ingestion and microbatch planning ------------------------------------
dag_status dag_trie_build(const int32_t* tokens, const int64_t* traj_off, int32_t n_traj, int32_t cap_nodes,
                          dag_node* nodes, int64_t* node_tok_off, int64_t cap_tokens, int32_t* node_tokens,
                          int32_t* leaf_of_traj, int32_t* n_nodes, int64_t* n_tokens) {
  if (!n_nodes || !n_tokens) return set_err(DAG_E_INVALID, "null argument");
  TrieOut t;
  std::string err;
  dag_status st;
  try {
    st = trie_build(tokens, traj_off, n_traj, &t, &err);
  } catch (const std::bad_alloc&) {
    return set_err(DAG_E_OVERFLOW, "out of host memory building the trie");
  } catch (const std::length_error&) {
    return set_err(DAG_E_OVERFLOW, "sizes beyond the host's limits building the trie");
  } catch (const std::exception& e) {
    return set_err(DAG_E_INVALID, std::string("building the trie failed: ") + e.what());
  }
  if (st != DAG_OK) return set_err(st, err);
  *n_nodes = (int32_t)t.nodes.size();
  *n_tokens = (int64_t)t.tokens.size();
  if (cap_nodes < *n_nodes || cap_tokens < *n_tokens || !nodes || !node_tok_off || !leaf_of_traj ||
      (*n_tokens > 0 && !node_tokens))
    return DAG_OK;
  std::memcpy(nodes, t.nodes.data(), t.nodes.size() * sizeof(dag_node));
  std::memcpy(node_tok_off, t.tok_off.data(), t.tok_off.size() * 8);
  if (*n_tokens) std::memcpy(node_tokens, t.tokens.data(), t.tokens.size() * 4);
  std::memcpy(leaf_of_traj, t.leaf_of_traj.data(), t.leaf_of_traj.size() * 4);
  return DAG_OK;
}

dag_status dag_microbatch_plan(const int32_t* tokens, const int64_t* traj_off, int32_t n_traj,
                               const dag_mb_opts* opts, int32_t* mb_of_traj, int32_t cap_mb,
                               int32_t* replica_of_mb, int32_t* slot_of_mb, int64_t* work_of_mb,
                               dag_mb_info* info) {
  if (!info) return set_err(DAG_E_INVALID, "null argument");
  MbOut m;
  std::string err;
  dag_status st;
  try {
    st = microbatch_plan(tokens, traj_off, n_traj, opts, &m, &err);
  } catch (const std::bad_alloc&) {
    return set_err(DAG_E_OVERFLOW, "out of host memory planning microbatches");
  } catch (const std::length_error&) {
    return set_err(DAG_E_OVERFLOW, "sizes beyond the host's limits planning microbatches");
  } catch (const std::exception& e) {
    return set_err(DAG_E_INVALID, std::string("planning microbatches failed: ") + e.what());
  }
  if (st != DAG_OK) return set_err(st, err);
  *info = m.info;
  const int32_t K = m.info.microbatches;
  if (cap_mb < K || !mb_of_traj || !replica_of_mb || !slot_of_mb || !work_of_mb) return DAG_OK;
  std::memcpy(mb_of_traj, m.mb_of_traj.data(), m.mb_of_traj.size() * 4);
  std::memcpy(replica_of_mb, m.replica.data(), K * 4);
  std::memcpy(slot_of_mb, m.slot.data(), K * 4);
  std::memcpy(work_of_mb, m.work.data(), K * 8);
  return DAG_OK;
}

}  // extern "C"

/*
 * dag_attn.h -- packed attention over a rollout DAG on AMD MI355X (gfx950).
 *
 * A rollout DAG has tree edges (continuation, fork, rewind) and read_thread
 * mount edges (Octopus: One Brain, Many Branches for Latent-KV Multi-Agent RL,
 * Sec. 3 and Table 2).  Every shared prefix is stored once, as compact token
 * rows grouped into 64-row KV pages; each query token attends to its tree
 * ancestors, to the spans mounted along its chain and to its own earlier
 * tokens (Octopus Sec. 3.3 Eq. 4; HARTS: Hybrid-Attention RL over Tree
 * Structures, Sec. 4.2 Eq. 21-22).  Mounted keys keep their native positions
 * and a reader's later tokens jump past them (Octopus Sec. 3.2 Eq. 2).  The
 * backward pass sends every reader's dK/dV into the producer's rows, summed
 * over readers in a fixed order, with no floating-point atomics (Octopus
 * Sec. 3.4 Eq. 8; HARTS Sec. 3.4).
 *
 * Two kinds of calls:
 *   - dag_build & co. run on the host only: they validate the DAG and compile
 *     it into an immutable plan (positions, page table, per-query-page
 *     visibility tile lists, per-KV-page reader lists, launch orders).
 *   - dag_attn_fwd / dag_attn_bwd enqueue HIP kernels on the caller's stream.
 *     They neither allocate (once the plan is uploaded) nor synchronise.
 *
 * Conventions for every call:
 *   - Return value: DAG_OK or an error code; nothing aborts, throws or prints.
 *     dag_last_error() returns a thread-local description of the last error.
 *   - Tensor arguments are device pointers owned by the caller.  Layout is
 *     row-major [C, H, D]: C compact rows (dag_plan_info.rows), H heads, D the
 *     head dimension, contiguous.  Callers place token (node u, own offset i)
 *     at the row dag_plan_rows reports.  Padding rows are ignored on input and
 *     written as zero on output.
 *   - Gradients are written, not accumulated.
 *   - Kernel launch failures return DAG_E_DEVICE; faults during execution
 *     surface at the caller's next synchronisation.
 */
#ifndef DAG_ATTN_H
#define DAG_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DAG_OK = 0,
  DAG_E_INVALID = 1,             /* bad argument, malformed table, no nodes          */
  DAG_E_NOT_TOPO = 2,            /* a node's parent index is not smaller than its own */
  DAG_E_MOUNT_CYCLE = 3,         /* tree and mount edges together form a cycle        */
  DAG_E_MOUNT_RANGE = 4,         /* mounted span outside the source's own tokens      */
  DAG_E_SELF_ANCESTOR_MOUNT = 5, /* a node mounts itself or one of its ancestors      */
  DAG_E_OVERFLOW = 6,            /* a row, page or pair count exceeds its integer type */
  DAG_E_WORKSPACE = 7,           /* workspace pointer missing or too small            */
  DAG_E_UNSUPPORTED = 8,         /* parameters outside what the kernels implement     */
  DAG_E_DEVICE = 9               /* a HIP runtime call or kernel launch failed        */
} dag_status;

/* One node of the DAG: a maximal run of tokens between fork / rewind /
 * read_thread boundaries (Octopus Sec. 3.3 item 1).  Nodes must be listed so
 * that parent < own index.  The node's mounts are mounts[mount_first ..
 * mount_first + mount_count) and are active from the node's first token; they
 * stay active for all descendants. */
typedef struct {
  int32_t parent;       /* -1 for a root                                  */
  int32_t length;       /* own tokens, >= 0                               */
  int32_t mount_first;  /* first entry in the mount table                 */
  int32_t mount_count;  /* number of entries, >= 0                        */
} dag_node;

/* A read_thread mount: the reader sees src's own tokens [begin, end) at their
 * native positions (Octopus Table 2 and Sec. 3.2).  begin == end is a legal
 * no-op (any source, any offset within 0..length(src)). */
typedef struct {
  int32_t src_node;
  int32_t begin;
  int32_t end;
} dag_mount;

typedef struct {
  int32_t page_size;    /* must be 64 (0 selects 64)                                    */
  int32_t q_block;      /* must be 64 (0 selects 64): one query block per KV page.  The    */
                        /*    MFMA kernels take a 64-row query page and all four query     */
                        /*    heads of a GQA group per work-group, so every staged K/V     */
                        /*    tile already feeds 256 query rows (256 flop per byte from    */
                        /*    LDS), and the pages of one node, launched side by side, share */
                        /*    their tiles in L2; a 128-row block would halve the number of  */
                        /*    work-groups without raising the intensity HBM sees.  Other    */
                        /*    values return DAG_E_UNSUPPORTED.                              */
  int32_t transitive;   /* 1: a reader also sees what its mounted sources see (Octopus   */
                        /*    Sec. 3.3 item 1, "including transitive mounts"); 0: direct */
  int32_t page_shuffle; /* 0: pages in node order; otherwise a seed for a random physical */
                        /*    page assignment (the page table stays exact)               */
  int32_t gdn_chunk;    /* 0: no linear-attention schedule; B > 0: also plan the chunked  */
                        /*    gated-delta-rule execution with chunk length B (HARTS Sec.  */
                        /*    3.3; the GDN kernels take B = 64 only)                      */
  int32_t view;         /* which layers' view of the tables the plan serves:               */
                        /*  DAG_VIEW_MOUNTED (0): mounted spans visible, positions by Eq. 2; */
                        /*  DAG_VIEW_MOUNT_FREE (1): the layers that do not mount (Octopus   */
                        /*    App. C: a dense model mounts in a subset of its layers): Eq. 2 */
                        /*    positions, mounted spans not visible;                          */
                        /*  DAG_VIEW_UNSHIFTED (2): mounted spans visible, every node        */
                        /*    continuing from its parent without the jump (Octopus Table 5's */
                        /*    unshifted regime).  Row layout and page table are the same in  */
                        /*    every view, so one set of tensors serves plans of all views.   */
  int32_t pack_pages;   /* 0: every node starts on a fresh page (pages hold one node);       */
                        /* 1: nodes in depth-first order share pages: a node that fits in    */
                        /*    the rest of the open page goes there, a longer one starts a     */
                        /*    page (its last page stays open).  For trees of short segments   */
                        /*    (HARTS App. A's 1-15-token turns) this removes most padding     */
                        /*    rows; a (query page, KV page) tile whose rows see the page      */
                        /*    differently carries a 64 x 64 visibility mask.  Packed plans    */
                        /*    run attention on the MFMA path (bf16, head_dim 128, Hq = 4 Hkv), */
                        /*    the gated delta rule and log-probabilities; the generic          */
                        /*    attention kernels and the convolution return DAG_E_UNSUPPORTED. */
                        /*    Not combinable with page_shuffle.                                */
} dag_build_opts;

enum { DAG_VIEW_MOUNTED = 0, DAG_VIEW_MOUNT_FREE = 1, DAG_VIEW_UNSHIFTED = 2 };

typedef struct dag_plan dag_plan; /* opaque and immutable after dag_build */

typedef struct {
  int64_t rows;            /* C: compact rows including page padding (pages * 64)    */
  int64_t tokens;          /* U: unique tokens = sum of node lengths                  */
  int64_t pages;           /* physical KV pages                                       */
  int64_t query_pages;     /* pages holding at least one row (one query block each)   */
  int64_t visible_pairs;   /* P: visible (query, key) pairs over compact queries      */
  int64_t flat_rows;       /* rows of the per-trajectory expansion incl. spliced spans */
  int64_t flat_pairs;      /* causal pairs of that expansion over every trajectory row */
  int64_t n_trajectories;  /* leaves                                                  */
  int64_t fwd_tiles;       /* sum over query pages of visited KV tiles                 */
  int64_t bwd_entries;     /* reader-list entries over all KV pages                    */
  int32_t max_position;    /* largest Eq. 2 position                                  */
  int32_t transitive;
  /* linear-attention schedule (zero when gdn_chunk == 0) */
  int32_t gdn_chunk;       /* B                                                       */
  int32_t gdn_rounds;      /* sequential packed calls (HARTS T_pre of the roots)      */
  int64_t gdn_sequences;   /* packed input sequences over all rounds                  */
  int64_t gdn_replay;      /* R: replayed state-update positions (HARTS Eq. 15)       */
  int64_t gdn_slots;       /* exported boundary states                                */
  int64_t gdn_chunks;      /* execution chunks over all sequences, replay included    */
  int64_t gdn_segments;    /* fork-free segments of the (mount-free) tree             */
  int32_t view;            /* the build option                                        */
  int64_t semantic_tokens; /* S = sum over tokens of their multiplicity (HARTS Sec. 3.5): */
                           /* own-token rows of the flat per-trajectory batch           */
  int32_t pack_pages;      /* the build option                                        */
} dag_plan_info;

/* Validate the node/mount tables and compile them into a plan.  Host only;
 * does not touch the GPU.  On error *out is left NULL and the code names the
 * first violated rule (checked in this order: table shape, parents, lengths,
 * mount slices and sources (INVALID / NOT_TOPO), span ranges (MOUNT_RANGE),
 * reads of the reader's own chain (SELF_ANCESTOR_MOUNT), cycles
 * (MOUNT_CYCLE), integer overflow (OVERFLOW)).  Zero-length mounts are
 * checked for range only and otherwise ignored. */
dag_status dag_build(const dag_node* nodes, int32_t n_nodes, const dag_mount* mounts,
                     int32_t n_mounts, const dag_build_opts* opts, dag_plan** out);

void dag_plan_destroy(dag_plan* plan);

dag_status dag_plan_info_get(const dag_plan* plan, dag_plan_info* out);

/* What the attention kernels walk for this plan, and the bytes they stage from global
 * memory per KV head on the matrix-core path (head_dim 128, fp16 operand copies) before
 * any cache reuse: a launch stages n_kv_heads times these.  Host only.
 *   forward and dQ: one 64 x 128 K tile and one V tile (32 KiB) per visited tile;
 *   dK/dV: per 32-row reader step two half-steps, each the Q and dO rows of two query
 *   heads (32 KiB) and their two 256-byte row-offset runs, plus each group's or pair's
 *   own K and V tiles once.
 * Comparing these with the kernels' measured HBM reads gives the share the caches absorb
 * (the merged reader lists order steps so that side-by-side groups share rows). */
typedef struct {
  int64_t fwd_tiles;         /* (query page, KV page) tiles of the forward and of dQ  */
  int64_t dkdv_groups;       /* four-page groups                                       */
  int64_t dkdv_group_steps;  /* their 32-row reader steps                              */
  int64_t dkdv_pairs;        /* page pairs (packed plans, small nodes)                 */
  int64_t dkdv_pair_steps;   /* their 32-row reader steps                              */
  int64_t fwd_staged_bytes;  /* per KV head                                            */
  int64_t dq_staged_bytes;   /* per KV head                                            */
  int64_t dkdv_staged_bytes; /* per KV head                                            */
} dag_plan_stats;
dag_status dag_plan_stats_get(const dag_plan* plan, dag_plan_stats* out);

/* Row of every token in node-major order (token (u, i) has index
 * sum_{w<u} length(w) + i) -> row_of_token[U]; Eq. 2 position of every row
 * -> pos_of_row[C] (-1 on padding rows).  Either pointer may be NULL. */
dag_status dag_plan_rows(const dag_plan* plan, int32_t* row_of_token, int32_t* pos_of_row);

/* The compact rows that query row `row` sees, decoded from the plan's forward tables the
 * way the forward and dQ kernels read them (tile ranges, masks, the causal rule on a query
 * page's last unmasked tile), sorted -> key_rows[min(n, cap)], count -> *n (padding rows see
 * nothing).  And the query rows whose contributions the dK/dV kernel sums into key row
 * `row`, decoded from its reader steps.  Both equal Octopus Eq. 4's visible sets mapped to
 * rows; they exist to check the tables on the host.  (The causal rule applies to a query
 * page's last tile only when that tile carries no mask.) */
dag_status dag_plan_visibility(const dag_plan* plan, int32_t row, int32_t* key_rows, int32_t cap, int32_t* n);
dag_status dag_plan_readers(const dag_plan* plan, int32_t row, int32_t* query_rows, int32_t cap, int32_t* n);

/* Multiplicity of every token in node-major order -> mult[U] (HARTS Sec. 3.5: the
 * number of root-to-leaf trajectories that hold the token as one of their own tokens,
 * i.e. the leaves below its node, the node itself if it has no children; mounted spans
 * do not count, since a spliced copy carries no training target).  The multiplicities
 * sum to dag_plan_info.semantic_tokens. */
dag_status dag_plan_multiplicity(const dag_plan* plan, int32_t* mult);

/* Device debug build.  libdag_attn_debug.so is this library compiled with DAG_DEBUG (the
 * Python binding loads it when DAG_ATTN_DEBUG=1): its attention kernels check every
 * query page, tile range, page id, mask id, visible interval and reader step they read
 * from the plan tables against the plan's sizes, record the first failure and go on
 * with a safe in-bounds value, and dag_attn_fwd / dag_attn_bwd then wait for the stream
 * and return DAG_E_INVALID naming the check (codes: 1 query page, 2 tile range, 3 tile
 * page, 4 interval, 5 mask id, 6 page pair, 7 step range, 8 step page, 9 page group).
 * Results of a passing call are bitwise those of the release build.
 * dag_debug_build: 1 in the debug build, 0 otherwise. */
int32_t dag_debug_build(void);
/* Debug build only (DAG_E_UNSUPPORTED otherwise): page ids >= max_pages fail the checks
 * from the next call on (0: the plan's page count), so the checks can be exercised on
 * valid tables without any access leaving its buffer.  Process-wide, not thread-safe. */
dag_status dag_debug_limit_pages(int32_t max_pages);

/* Start position s(u) of every node (Octopus Sec. 3.2 Eq. 2) -> start[n_nodes]. */
dag_status dag_plan_starts(const dag_plan* plan, int32_t* start);

/* Non-self part of what node u's tokens see, as disjoint [lo, hi) ranges of
 * source nodes' own offsets, ordered as the kernels visit them: mounted spans
 * first, then ancestors root to parent (Octopus Eq. 4).  Writes up to cap
 * triples (src, lo, hi) into out[3 * cap] and the total count into *n. */
dag_status dag_plan_node_ranges(const dag_plan* plan, int32_t u, int32_t* out, int32_t cap,
                                int32_t* n);

/* Copy the plan's device tables to the current HIP device, on `hip_stream`,
 * and wait for the copy.  Called implicitly by the first fwd/bwd; call it
 * yourself before capturing fwd/bwd in a graph, since it allocates and
 * synchronises.  A plan serves one device: using it from another returns
 * DAG_E_DEVICE. */
dag_status dag_plan_upload(dag_plan* plan, void* hip_stream);

enum { DAG_DTYPE_BF16 = 0, DAG_DTYPE_FP32 = 1 };

typedef struct {
  int32_t n_q_heads;   /* Hq                                                            */
  int32_t n_kv_heads;  /* Hkv; Hq % Hkv == 0, query head h reads KV head h / (Hq / Hkv) */
  int32_t head_dim;    /* even, 2..128                                                  */
  int32_t dtype;       /* DAG_DTYPE_BF16: bf16 tensors, fp32 accumulation.  When           */
                       /* head_dim == 128 and Hq == 4 Hkv the products run on MFMA with     */
                       /* fp16 operands: q, k, v and dO are each first scaled by the power  */
                       /* of two that puts their tensor's largest |x| (over valid rows) in  */
                       /* [2^14, 2^15) for q and k, [1, 2) for v and dO, undone exactly in  */
                       /* the outputs, so no finite bf16 input overflows.  An element       */
                       /* below 2^-28 (q, k) or 2^-14 (v, dO) of its tensor's maximum keeps */
                       /* fp16's subnormal spacing (2^-38 or 2^-24 of that maximum)          */
                       /* DAG_DTYPE_FP32: fp32 throughout                                   */
  int32_t grad_dtype;  /* element type of dq, dk, dv: DAG_DTYPE_BF16 or DAG_DTYPE_FP32;    */
                       /* must be FP32 when dtype is FP32.  Large shared-row gradients     */
                       /* keep their precision in FP32                                      */
  float scale;         /* softmax scale, finite and >= 0; 0 selects 1/sqrt(head_dim)     */
  float rope_base;     /* rotary base (Octopus Eq. 1, pairs (i, i + D/2),                */
                       /* theta_i = base^(-2i/D), angles in fp64); 0 disables rotation    */
} dag_attn_params;

/* Workspace bytes the forward and the backward need for this plan and shape. */
dag_status dag_attn_workspace(const dag_plan* plan, const dag_attn_params* p, size_t* fwd_bytes,
                              size_t* bwd_bytes);

/* Forward (Octopus Eq. 4 with Eq. 1-2 positions; HARTS Eq. 22):
 *   o[t,h]   = sum_{j in V(t)} softmax_j(scale <R(pos_t) q[t,h], R(pos_j) k[j,g]>) v[j,g]
 *   lse[t,h] = log sum_{j in V(t)} exp(scale <R(pos_t) q[t,h], R(pos_j) k[j,g]>)
 * q, o: [C, Hq, D]; k, v: [C, Hkv, D] (dtype); lse: [C, Hq] fp32.
 * o_lo (bf16 only; NULL for a forward that no backward follows): [C, Hq, D] bf16
 * receiving the rounding residual o_exact - o.  The bf16 backward needs it: it forms
 * rowsum(dO * O) from O = o + o_lo, accurate to ~2^-17 instead of bf16's 2^-9; with O
 * rounded to bf16 alone, attention concentrated on few keys moves dq and dk by more than
 * 2e-2 (measured on logits of standard deviation 16).
 * ws: device workspace of at least fwd_bytes.
 * A plan without rows (every node of length 0) returns DAG_OK after checking p, reading
 * no pointer; the backward and the gated-delta-rule calls do the same. */
dag_status dag_attn_fwd(dag_plan* plan, const dag_attn_params* p, const void* q, const void* k,
                        const void* v, void* o, float* lse, void* o_lo, void* ws, size_t ws_bytes,
                        void* hip_stream);

/* dag_attn_fwd without allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments and results as dag_attn_fwd, minus the workspace: it runs in a static
 * 64 MiB device array that the library holds on every device it runs on until the
 * process ends (forward workspace: about 6.6 KB per compact row at Hq = 16, Hkv = 4,
 * D = 128, i.e. plans up to roughly 10,000 rows).  A plan needing more returns
 * DAG_E_WORKSPACE.  The plan must already be on the current device (dag_plan_upload,
 * which allocates); otherwise DAG_E_INVALID.  Calls on one device share the array:
 * calls that overlap on one device (other streams or threads) race; calls in order on
 * one stream do not. */
dag_status dag_attn_fwd_noalloc(dag_plan* plan, const dag_attn_params* p, const void* q, const void* k,
                                const void* v, void* o, float* lse, void* o_lo, void* hip_stream);

/* Backward of dag_attn_fwd given the upstream gradient dO [C, Hq, D] (dtype):
 * dq [C, Hq, D]; dk, dv [C, Hkv, D] (grad_dtype), where every key row's gradient is the sum
 * over all readers (own branch, descendants, mount readers) taken in a fixed
 * order, so results are bitwise reproducible (Octopus Sec. 3.4 Eq. 8, HARTS
 * Sec. 3.4).  o, lse and o_lo are the forward's outputs; o_lo is required for
 * DAG_DTYPE_BF16 (DAG_E_INVALID when NULL) and must be NULL for DAG_DTYPE_FP32.
 * ws: at least bwd_bytes. */
dag_status dag_attn_bwd(dag_plan* plan, const dag_attn_params* p, const void* q, const void* k,
                        const void* v, const void* o, const float* lse, const void* o_lo,
                        const void* dO, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                        void* hip_stream);

/* ---- Gated delta rule over the same tree (HARTS Sec. 2.2 and 3.3-3.4) ----------
 *
 * A recurrent layer follows each token's own root-to-node path; mounted spans
 * are not part of it (Octopus Sec. 3: read_thread only changes what attention
 * sees).  Per head, with state S of shape [dv, dk], S = 0 at every root:
 *   S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = scale S_t q_t.
 * The pages name the layer but print no recurrence; this is the textbook gated
 * delta rule.  Execution is chunked (B = 64 tokens per chunk, chunk boundaries
 * on the recurrent index, HARTS Eq. 2): the plan contracts the tree into
 * fork-free segments, picks each fork's direct continuation so that the number
 * of sequential rounds is minimal (HARTS Eq. 12-14, Algorithm 1), and starts
 * every other branch from the state at the chunk boundary a(fork) = B floor(fork / B),
 * re-running the ancestor tokens [a(fork), fork) state-only ("replay", HARTS
 * Eq. 15).  All sequences of a round run in one launch; boundary states pass
 * between rounds through the workspace and their gradients flow back into the
 * producing sequence (HARTS Sec. 3.4 Eq. 16). */

/* One packed input sequence of the schedule.  Its own tokens are the path from
 * first_node to last_node (a chain of direct continuations); before them it
 * replays the ancestor positions [start, fork). */
typedef struct {
  int32_t round;         /* 1-based round (packed call) it runs in                      */
  int32_t first_node;    /* DAG node where its own tokens begin                         */
  int32_t last_node;     /* DAG node where they end (a leaf)                            */
  int32_t start;         /* recurrent index of its first (replayed) token, a multiple of B */
  int32_t fork;          /* recurrent index of its first own token                      */
  int32_t own_tokens;
  int32_t init_seq;      /* sequence whose exported state it starts from; -1: zero state */
  int32_t init_boundary; /* recurrent index of that state (a multiple of B), -1 if none  */
} dag_gdn_seq;

/* The schedule's sequences in creation order (trees in table order; within a
 * tree, the recovery's depth-first order).  Writes min(cap, count) entries and
 * the count into *n.  DAG_E_INVALID if the plan was built with gdn_chunk == 0. */
dag_status dag_plan_gdn_seqs(const dag_plan* plan, dag_gdn_seq* out, int32_t cap, int32_t* n);

typedef struct {
  int32_t n_heads;     /* H                                                      */
  int32_t head_dim;    /* dk = dv; must be 128                                   */
  int32_t dtype;       /* q, k, v, o, dO element type; must be DAG_DTYPE_BF16    */
  int32_t grad_dtype;  /* dq, dk, dv: DAG_DTYPE_BF16 or DAG_DTYPE_FP32           */
  float scale;         /* output scale; 0 selects 1                              */
  int32_t keep_states; /* 0: the backward recomputes every chunk's starting state
                          (and its chunk inverse) from the inputs; 1: the
                          forward saves them (fp16) into its workspace and the
                          backward reads them there: pass the same ws to both
                          calls and leave it untouched in between.  Trades a
                          recomputation pass for keeping (2 * 128 * 128 + 3 * 64
                          * 64) * 2 bytes per head and execution chunk alive from
                          the forward to the backward                           */
} dag_gdn_params;

/* Workspace bytes for dag_gdn_fwd and dag_gdn_bwd (with keep_states the two are
 * equal: the forward fills the part of the backward's workspace that holds the
 * states).  Both hold every execution chunk's (I + A)^{-1} and P (3 * 64 * 64
 * fp16 per head and chunk, computed for all chunks at once); the backward adds the
 * chunk states and one round's end-state gradients (128 * 128 fp16 per head and
 * chunk of the largest round). */
dag_status dag_gdn_workspace(const dag_plan* plan, const dag_gdn_params* p, size_t* fwd_bytes,
                             size_t* bwd_bytes);

/* Forward: q, k [C, H, dk] (each head's vector already L2-normalised by the
 * caller), v [C, H, dv] (dtype); beta, alpha [C, H] fp32 (beta in [0, 1], alpha in (0, 1]);
 * o [C, H, dv] (dtype) receives every token's output once.  One launch per
 * round; products on MFMA with fp16 operands and fp32 accumulation, state in
 * fp32.  ws: at least fwd_bytes; with keep_states the call also leaves every
 * chunk's starting state in ws for dag_gdn_bwd. */
dag_status dag_gdn_fwd(dag_plan* plan, const dag_gdn_params* p, const void* q, const void* k,
                       const void* v, const float* beta, const float* alpha, void* o, void* ws,
                       size_t ws_bytes, void* hip_stream);

/* Backward given dO [C, H, dv]: dq, dk [C, H, dk], dv [C, H, dv] (grad_dtype),
 * dbeta, dalpha [C, H] fp32.  Rounds run in reverse; the gradient of each
 * exported boundary state is the sum over its consumers in a fixed order, and a
 * replayed token's contributions are added to its own row after its own
 * sequence's, in a fixed order: results are bitwise reproducible.  Recomputes
 * the forward's states, or with keep_states reads them from ws as the forward
 * left it (same plan, same params, same inputs); ws: at least bwd_bytes. */
dag_status dag_gdn_bwd(dag_plan* plan, const dag_gdn_params* p, const void* q, const void* k,
                       const void* v, const float* beta, const float* alpha, const void* dO,
                       void* dq, void* dk, void* dv, float* dbeta, float* dalpha, void* ws,
                       size_t ws_bytes, void* hip_stream);

/* ---- compact-to-semantic log-probabilities ------------------------------------
 *
 * HARTS Sec. 3.5 Eq. 17: for every nonterminal semantic position s of the
 * original batch, lambda_s = z[m(s), y_s] - log sum_v exp z[m(s), v], where
 * m(s) is the compact logit row of s and y_s the vocabulary id of the next
 * token of s's trajectory.  Eq. 19-20: the gradient of a compact row is the sum
 * over the positions that map to it, dz[c, v] = sum_{m(s)=c, y_s=v} g_s -
 * (sum_{m(s)=c} g_s) softmax(z[c])_v with g_s = dL/dlambda_s.  Vocabulary-wide
 * work runs once per compact row; no [positions x V] array is formed.
 *
 * The original batch: every root-to-leaf trajectory, leaves in depth-first
 * order (roots and children in table order), each the flat sequence that visits
 * node by node the mounted tokens that become visible there (not spliced
 * before, in token order) and then the node's own tokens.  Its positions are
 * its own tokens that have a next token, in sequence order; the target of an
 * own token followed by a splice is the splice's first token.  Spliced tokens
 * hold no position (Octopus Sec. 3.4: mounted spans carry a zero loss mask; their
 * compact rows hold the producer's logits, not the reader's). */

/* Build the map, host only.  labels[C]: vocabulary id of the token on each
 * compact row (padding rows ignored; a negative id on a row that is some
 * position's target is DAG_E_INVALID).  Writes *n_pos = the number of
 * positions n and, when cap >= n and every output is non-NULL:
 *   pos_row[n]      m(s), in batch order
 *   pos_target[n]   y_s
 *   row_first[C+1]  positions of row c are row_pos[row_first[c] .. row_first[c+1])
 *   row_pos[n]      position indices grouped by row, batch order within a row.
 * Otherwise only *n_pos is written.  DAG_E_OVERFLOW beyond 2^31 - 1 positions. */
dag_status dag_plan_logprob_map(const dag_plan* plan, const int32_t* labels, int64_t cap, int32_t* pos_row,
                                int32_t* pos_target, int32_t* row_first, int32_t* row_pos, int64_t* n_pos);

typedef struct {
  int64_t rows;        /* C: rows of z and dz                                       */
  int64_t n_pos;       /* n: entries of pos_target, lambda and g (< 2^31)           */
  int32_t vocab;       /* V >= 1; z and dz are [C, V] row-major                     */
  int32_t dtype;       /* z: DAG_DTYPE_BF16 or DAG_DTYPE_FP32                       */
  int32_t grad_dtype;  /* dz: DAG_DTYPE_BF16 or DAG_DTYPE_FP32                      */
} dag_logprob_params;

/* Forward.  Device pointers: z [C, V] (dtype, element-aligned), the map of
 * dag_plan_logprob_map (or any row-grouped map: row_first[C+1] non-decreasing,
 * row_pos a permutation of 0..n-1, pos_target[n]); lse [C] fp32 receives
 * log sum_v exp z[c, v] for every row that holds a position and 0 for the
 * others, whose z is not read; lambda [n] fp32.  A target outside [0, V) gives
 * lambda = NaN; out-of-range map entries are skipped, never dereferenced.
 * Sums over the vocabulary run in fp32 in a fixed order (bitwise reproducible).
 * Enqueued on hip_stream; no allocation, no synchronisation. */
dag_status dag_logprob_fwd(const dag_logprob_params* p, const void* z, const int32_t* row_first,
                           const int32_t* row_pos, const int32_t* pos_target, float* lse, float* lambda,
                           void* hip_stream);

/* Backward given g [n] fp32 and the forward's lse: dz [C, V] (grad_dtype) is
 * written for every row (zero on rows with no position).  Each target term is
 * added to the softmax term in fp32 before the single rounding; positions of a
 * row that share a target are summed in map order. */
dag_status dag_logprob_bwd(const dag_logprob_params* p, const void* z, const float* lse, const int32_t* row_first,
                           const int32_t* row_pos, const int32_t* pos_target, const float* g, void* dz,
                           void* hip_stream);

/* ---- short causal convolution of a linear-attention block -------------------
 *
 * HARTS Sec. 4.2 and Octopus App. C: the depthwise causal convolution in front of
 * a gated-delta-rule layer takes its history only from a token's true
 * ancestors, i.e. its own root-to-node path with mounted spans skipped; one
 * result is kept per compact token, and the input gradient of a token sums the
 * contributions of every output that reads it, on every branch below it.  Per
 * channel c with taps W[c, 0..w-1] (the last one multiplies the current token):
 *   pre_t = sum_{k<w} W[c, w-1-k] x_{t-k}   (x = 0 before a root),
 *   y_t = act(pre_t),   act = identity or SiLU(p) = p / (1 + e^-p).
 * The pages name the operator but print neither its activation nor its tap
 * order; both are this textbook form. */
enum { DAG_ACT_NONE = 0, DAG_ACT_SILU = 1 };

typedef struct {
  int32_t channels;    /* Ch: a multiple of 8 (e.g. the q, k and v projections side by side) */
  int32_t width;       /* w, 1..4                                                          */
  int32_t activation;  /* DAG_ACT_NONE or DAG_ACT_SILU                                     */
  int32_t grad_dtype;  /* dx: DAG_DTYPE_BF16 or DAG_DTYPE_FP32                             */
} dag_conv_params;

/* Workspace bytes of dag_conv_bwd (per-block dW partials). */
dag_status dag_conv_workspace(const dag_plan* plan, const dag_conv_params* p, size_t* bwd_bytes);

/* Forward: x [C, Ch] bf16 (row layout), weight [Ch, w] fp32 -> y [C, Ch] bf16
 * (padding rows zero).  fp32 arithmetic, one rounding per output. */
dag_status dag_conv_fwd(dag_plan* plan, const dag_conv_params* p, const void* x, const float* weight, void* y,
                        void* hip_stream);

/* Backward given dy [C, Ch] bf16: dx [C, Ch] (grad_dtype; padding rows zero) and
 * dweight [Ch, w] fp32 (written, not accumulated).  The forward's pre-activation
 * is recomputed; every sum has a fixed order (bitwise reproducible, no atomics).
 * ws: at least the bytes dag_conv_workspace reports. */
dag_status dag_conv_bwd(dag_plan* plan, const dag_conv_params* p, const void* x, const float* weight,
                        const void* dy, void* dx, float* dweight, void* ws, size_t ws_bytes, void* hip_stream);

/* ---- trajectory ingestion and prefix-aware microbatch planning (host only) ----
 *
 * HARTS Sec. 3.1-3.2.  Input: N raw root-to-leaf trajectories as token ids,
 * tokens[traj_off[i] .. traj_off[i+1]) for trajectory i (traj_off[0] = 0,
 * non-decreasing).  Neither call touches the GPU. */

/* The trie of the trajectories' shared prefixes as a DAG node table for dag_build
 * (no mounts): nodes are the trie's maximal unbranched runs, numbered depth-first
 * with children in token order (so parent < child and the leaves come in the
 * trajectories' lexicographic order); a trajectory that is a prefix or a repeat of
 * another gets a zero-length leaf of its own, so every trajectory ends at its own
 * leaf.  The compact work C(X) of Eq. 5 is the number of tokens.  Writes *n_nodes
 * and *n_tokens and, when cap_nodes >= *n_nodes, cap_tokens >= *n_tokens and every
 * output is non-NULL: nodes[n_nodes], node_tok_off[n_nodes + 1] (node u's tokens are
 * node_tokens[node_tok_off[u] .. node_tok_off[u+1])), node_tokens[n_tokens] and
 * leaf_of_traj[N].  Otherwise only the counts. */
dag_status dag_trie_build(const int32_t* tokens, const int64_t* traj_off, int32_t n_traj, int32_t cap_nodes,
                          dag_node* nodes, int64_t* node_tok_off, int64_t cap_tokens, int32_t* node_tokens,
                          int32_t* leaf_of_traj, int32_t* n_nodes, int64_t* n_tokens);

typedef struct {
  int32_t replicas;   /* D >= 1: data-parallel replicas                                     */
  int32_t exact_max;  /* N0: exact search up to this many trajectories; 0 selects 512          */
  int64_t capacity;   /* T >= 1: compact tokens per microbatch                                 */
} dag_mb_opts;

typedef struct {
  int32_t microbatches;          /* K, a multiple of D                                        */
  int32_t exact;                 /* 1: exact DP over contiguous partitions (N <= N0)          */
  int32_t natural_microbatches;  /* K0 of the natural partition                               */
  int32_t candidates;            /* fully assigned candidate plans compared                   */
  int64_t total_work;            /* J (Eq. 4): sum of microbatch compact work,                 */
  int64_t slot_critical_work;    /*   sum over slots of the heaviest microbatch,               */
  int64_t max_replica_work;      /*   largest work on one replica                              */
  int64_t trie_work;             /* C(X): all trajectories in one trie                         */
} dag_mb_info;

/* Prefix-aware microbatch plan: membership, DP replica and slot of every
 * microbatch (Eq. 4-10; the search is exact over contiguous partitions of the
 * lexicographic order for N <= N0 and heuristic otherwise, with one trie-aware
 * greedy candidate in every case; ties are broken deterministically).
 * Guarantees: every trajectory in exactly one microbatch, no microbatch empty or
 * above capacity, K mod D = 0 and exactly K / D microbatches per replica, one
 * per slot.  Writes info and, when cap_mb >= K and the outputs are non-NULL,
 * mb_of_traj[N], replica_of_mb[K], slot_of_mb[K], work_of_mb[K].  DAG_E_INVALID
 * when a trajectory is longer than the capacity, N < D, or no feasible plan exists. */
dag_status dag_microbatch_plan(const int32_t* tokens, const int64_t* traj_off, int32_t n_traj,
                               const dag_mb_opts* opts, int32_t* mb_of_traj, int32_t cap_mb,
                               int32_t* replica_of_mb, int32_t* slot_of_mb, int64_t* work_of_mb,
                               dag_mb_info* info);

/* Per-kernel timing, for profiling.  While enabled, dag_attn_fwd/bwd record a
 * HIP event pair on their stream around each of their kernels (at most
 * `capacity` pairs, created here; later launches go unrecorded).
 * The same holds for dag_gdn_fwd/bwd and dag_conv_fwd/bwd.
 * dag_attn_timing_read waits for the recorded events, writes for each kernel
 * k in dag_kernel_id the summed duration ms[k] (milliseconds) and the number of
 * launches counts[k] since the last read, and resets.  Disabling (enable = 0)
 * destroys the events.  The plan must not be in use on another thread. */
enum {
  DAG_K_PROLOGUE_FWD = 0, /* rotary table and operand relayouts of the forward   */
  DAG_K_FWD = 1,          /* attention forward                                    */
  DAG_K_PROLOGUE_BWD = 2, /* rotary table, rowsum(dO * O) and relayouts          */
  DAG_K_DKDV = 3,         /* per-KV-page dK/dV reduction                          */
  DAG_K_DQ = 4,           /* per-query-block dQ                                   */
  DAG_K_GDN_FWD = 5,      /* gated delta rule forward, all rounds                  */
  DAG_K_GDN_STATES = 6,   /* backward's recomputation of chunk and boundary states */
  DAG_K_GDN_BWD = 7,      /* gated delta rule backward, all rounds, and replay fix-up */
  DAG_K_CONV_FWD = 8,     /* short convolution forward                             */
  DAG_K_CONV_BWD = 9,     /* short convolution backward and its dW reduction       */
  DAG_K_COUNT = 10
};
dag_status dag_attn_timing_enable(dag_plan* plan, int32_t enable, int32_t capacity);
dag_status dag_attn_timing_read(dag_plan* plan, double* ms, int64_t* counts);

/* Thread-local description of the last error ("" if none). */
const char* dag_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DAG_ATTN_H */

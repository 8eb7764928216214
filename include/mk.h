/* mk.h -- C ABI of the persistent fused MoE decode-layer step for AMD MI355X (gfx950).
 *
 * One call of mk_layer_step() enqueues ONE kernel launch that runs a whole decoder layer
 * for a batch-one speculative verify step, as the LMSYS / SGLang "Muse Spark Open"
 * megakernel pages draw the fusion boundary (orcarouter.ai write-up, section "where the
 * kernel boundary sits"; alphasignal.ai, "Launch boundaries leave hardware idle"): the
 * launch starts with attention of layer L over the KV cache and ends with layer L+1's
 * query/key/value projection and KV-cache write.  In between: output projection, pooler,
 * top-k-of-E router, routed experts stored as NVFP4 (gate/up GEMM with SwiGLU, an fp4
 * intermediate, down GEMM, combine), unpooler.
 *
 * Conventions (all entry points):
 *  - Every pointer is a caller-owned DEVICE pointer unless marked [host].  The library
 *    never allocates, frees or retains device memory; it keeps no pointer after a call.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls only
 *    enqueue work; they return before it runs.
 *  - Return value: MK_OK (0) or a negative mk_status.  Every argument, shape and alignment
 *    check happens on the host BEFORE any HIP call, so a rejected call enqueues nothing.
 *    Errors found while the kernel runs (a malformed tree, a bounded wait that expired) are
 *    written to the status word in the workspace; read them with mk_read_status().
 *  - Tensors are row-major; weight matrices use the PyTorch Linear layout [out][in].
 *  - bf16 tensors are passed as void* (16-bit patterns).  Device pointers must be 16-byte
 *    aligned unless stated otherwise.
 *  - Thread safety: calls on distinct streams with distinct workspaces may run
 *    concurrently from several host threads.  A mk_layer_step launch needs every CU of
 *    the device (one workgroup per CU); a concurrent kernel on another stream delays it,
 *    and if CUs stay occupied its bounded waits expire with MK_ETIMEOUT instead of hanging.
 */
#ifndef MK_H_
#define MK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MK_OK = 0,
  MK_EINVAL = -1,     /* NULL pointer where one is required, or a bad enum value          */
  MK_ESHAPE = -2,     /* shape outside what the kernels support (see mk_layer_cfg)         */
  MK_EALIGN = -3,     /* pointer not 16-byte aligned                                       */
  MK_ECAPACITY = -4,  /* KV cache or workspace too small                                   */
  MK_EHIP = -5,       /* a HIP runtime call failed (launch, copy, device query)            */
  MK_ETIMEOUT = -6,   /* a bounded in-kernel wait expired (CUs not all available)          */
  MK_EBADTREE = -7,   /* tree_parent malformed: parent[0] != -1 or parent[i] not in [0,i)  */
  MK_ESCRATCH = -8    /* mk_layer_step_noalloc: the configuration's workspace exceeds the
                         static scratch (MK_NOALLOC_SCRATCH_BYTES)                          */
} mk_status;

typedef enum { MK_W_BF16 = 0, MK_W_NVFP4 = 1 } mk_wfmt;

/* Shapes of one GPU's share of a layer [host].  Supported: hidden a multiple of 128 and
 * <= 4096; pooled a multiple of 128 and <= 2048; head_dim 64 or 128; n_q_heads a multiple
 * of n_kv_heads with n_q_heads*head_dim <= 1024 and T*(n_q_heads/n_kv_heads) <= 128;
 * n_experts <= 256 (multiple of 16); 1 <= top_k <= 8; expert_inter a multiple of 32 and
 * <= 256; window 0 (global attention) or >= 1; T <= 16; MK_W_NVFP4 experts also need
 * pooled a multiple of 128. */
typedef struct {
  int hidden, n_q_heads, n_kv_heads, head_dim;   /* H, Hq, Hkv, d                          */
  int pooled, n_experts, top_k, expert_inter;    /* P, E, k, I (this GPU's share of I)     */
  int window;                                    /* sliding window length, 0 = global      */
  int expert_fmt;                                /* mk_wfmt of the routed experts           */
  int kv_capacity;                               /* rows of each KV cache                   */
} mk_layer_cfg;

/* Weights of one layer [host struct of device pointers]. */
typedef struct {
  const void *w_o;         /* bf16 [H][Hq*d]          output projection                     */
  const void *w_pool;      /* bf16 [P][H]             pooler                                */
  const void *w_router;    /* bf16 [E][P]             router                                */
  const void *w_unpool;    /* bf16 [H][P]             unpooler                              */
  const void *w_qkv_next;  /* bf16 [(Hq+2Hkv)*d][H]   next layer's q, k, v rows, in that order;
                              NULL for the last layer of the stack: the launch then ends after
                              the unpooler and q_next / k_cache_next / v_cache_next may be
                              NULL (first and last layers differ: orcarouter.ai write-up,
                              "where the kernel boundary sits")                              */
  const void *w1, *w2;     /* MK_W_BF16:  bf16 [E][2I][P] (rows [0,I) gate, [I,2I) up), [E][P][I] */
  const uint8_t *w1_codes, *w1_scales;  /* MK_W_NVFP4: W1 in GEMM1's operand order, from
                                           mk_nvfp4_pack then mk_nvfp4_tile_w1 */
  const uint8_t *w2_codes, *w2_scales;  /*             [E][P][I/2],  [E][P][I/16]                  */
  const float *w1_tscale, *w2_tscale;   /*             fp32 [E] tensor scales                      */
} mk_layer_weights;

/* Inputs and outputs of one step [host struct; pointers are device pointers]. */
typedef struct {
  int T;                       /* [host] tree nodes, 1..16                                  */
  int ctx_len;                 /* [host] KV rows before the tree; ctx_len + T <= kv_capacity */
  const int32_t *tree_parent;  /* [T]; parent[0] = -1, parent[i] in [0, i).  Node i sits at
                                  position ctx_len + depth(i) and in KV slot ctx_len + i      */
  const void *q_in;            /* bf16 [T][Hq*d]   this layer's queries (previous launch)     */
  const void *h_in;            /* bf16 [T][H]      residual stream entering the layer         */
  const void *k_cache, *v_cache;      /* bf16 [cap][Hkv][d]; rows [0, ctx_len+T) valid        */
  void *k_cache_next, *v_cache_next;  /* bf16 [cap][Hkv][d]; rows ctx_len..ctx_len+T-1 written,
                                         every other row left untouched (NULL: last layer)    */
  void *h_out;                 /* bf16 [T][H]      residual stream leaving the layer          */
  void *q_next;                /* bf16 [T][Hq*d]   next layer's queries (NULL: last layer)    */
  int32_t *topk_idx;           /* [T][k] or NULL   experts per token, best first              */
  float *topk_gate;            /* [T][k] or NULL   softmax over the k selected logits         */
  float *router_logits;        /* [T][E] or NULL   fp32 logits (bias included)                */
  float *attn_stats;           /* [T][Hq][2] or NULL: row max m of the scaled scores and
                                  l = sum exp(score - m), natural-log units                   */
  int32_t *expert_hist;        /* [E] or NULL      += number of (token, slot) pairs per expert */
  const int32_t *prefetch_experts; /* [n_prefetch] or NULL: expert ids to pull into the
                                  device-side cache at launch start (speculative prefetch)    */
  int n_prefetch;              /* [host] 0..16                                              */
  int32_t *prefetch_next;      /* [n_prefetch_next] or NULL: receives this step's most-used
                                  experts by (pair count desc, index asc), -1 after the last
                                  used one -- the next step's prefetch_experts (the pages'
                                  expert prefetch from the previous step's usage: alphasignal.ai
                                  "Four mechanisms keep work moving")                         */
  int n_prefetch_next;         /* [host] 0..16                                              */
  const float *router_bias;    /* [T][E] or NULL   added to the logits before top-k           */
  void *workspace;             /* >= mk_workspace_bytes(); initialised once by
                                  mk_workspace_init(); holds the status word, the
                                  cross-workgroup flags and the stage hand-off buffers        */
  size_t workspace_bytes;      /* [host]                                                    */
  uint64_t *timestamps;        /* NULL, or [n_cu][MK_TS_EVENTS] wall-clock ticks (100 MHz)
                                  written by lane 0 of every workgroup at phase boundaries;
                                  when NULL the launched kernel contains no timing code       */
  int spin_limit;              /* [host] 0 = default; else max polls of each in-kernel wait  */
  int debug_skip_signal_wg;    /* [host] -1 normally; test hook: this workgroup never signals,
                                  so the others' bounded waits must end in MK_ETIMEOUT        */
  int batch;                   /* [host] 0 or 1: one sequence.  2: two sequences verified in
                                  one launch (the pages name batch one as the present limit:
                                  alphasignal.ai, "Batch one defines the current limit"), each
                                  a tree of T = 16 over its own KV cache at the same ctx_len;
                                  every weight is read once for both.  Then tree_parent is
                                  [2][16]; q_in, h_in, h_out, q_next, topk_idx, topk_gate,
                                  router_logits, attn_stats and router_bias hold 32 rows,
                                  sequence b on rows 16b..16b+15; the four KV caches are
                                  [2][cap][Hkv][d] (sequence b at b*cap rows).  Needs NVFP4
                                  experts with expert_inter a multiple of 64 in [128, 192];
                                  not with mk_layer_step_nshard.  Else MK_ESHAPE.            */
} mk_step_io;

#define MK_TS_EVENTS 64

/* Stage hand-off buffers inside the workspace (byte offsets), for stage-local checks.
 * The bf16 activations (attn, h1, xp, y) hold 16 rows (T padded; rows >= T undefined) of K
 * columns in MFMA fragment order: element (t, c) is at index
 *     ((c / 32) * 64 + ((c / 8) % 4) * 16 + t) * 8 + c % 8,
 * so that one 64-lane operand fetch of 32 columns reads 1 KB contiguously.
 * The stage buffers exist twice: a launch uses copy (e & 1) of its epoch e, the copy at
 * offset + (e & 1) * stage_copy, and resets the other copy for the next launch.  After a
 * launch, the uint32 at offset `epoch` holds e + 1. */
typedef struct {
  size_t status;       /* uint32 status word (decode with mk_read_status)         */
  size_t attn;         /* bf16 [16][Hq*d]  attention output (fragment order)     */
  size_t h1;           /* bf16 [16][H]     residual after the output projection  */
  size_t xp;           /* bf16 [16][P]     pooler output (fragment order)        */
  size_t logits;       /* fp32 [T][E]      router logits (bias included)         */
  size_t y;            /* bf16 [16][P]     combined expert output (fragment order) */
  size_t total;        /* bytes needed                                           */
  int n_wg;            /* workgroups per launch (= CUs of the current device)    */
  int attn_items;      /* attention work items (KV chunks)                       */
  size_t stage_copy;   /* bytes from copy 0 to copy 1 of the stage buffers       */
  size_t epoch;        /* uint32 epoch slot of workgroup 0                       */
} mk_workspace_layout;

/* Workspace bytes for this config on the current device (0 on an unsupported config); for
 * T = 16 the size also covers launches of two sequences (mk_step_io.batch = 2).  The stage
 * buffers hold one 16-row tile per sequence: sequence b's tile of a buffer at offset
 * + b * 16 * K * 2 bytes (K its column count). */
size_t mk_workspace_bytes(const mk_layer_cfg *cfg, int T);
/* Offsets of the hand-off buffers; returns MK_OK or an mk_status. */
int mk_workspace_query(const mk_layer_cfg *cfg, int T, mk_workspace_layout *out /* [host] */);
/* Initialise a workspace (fill kernels, no hipMemset): its counters to zero, the rest to the
 * all-ones pattern that marks hand-off data not yet written.  bytes % 16 == 0.  Call once
 * before the workspace's first use.  Launches on a workspace need no re-initialisation afterwards, also not after an
 * in-kernel error: the status word carries the launch's epoch, and the per-launch counters
 * are cleared by the launch that uses them. */
int mk_workspace_init(void *workspace, size_t bytes, void *stream);

/* One fused decoder-layer step (see the file comment).  Enqueues one kernel. */
int mk_layer_step(const mk_layer_cfg *cfg /* [host] */, const mk_layer_weights *w /* [host] */,
                  const mk_step_io *io /* [host] */, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): mk_layer_step with no caller workspace.  The
 * launch uses a static device array of the library, MK_NOALLOC_SCRATCH_BYTES on every GPU it
 * runs on, held until the process ends; io->workspace and io->workspace_bytes are ignored.
 * Same arguments, checks, kernel and results as mk_layer_step; a launch whose workspace
 * exceeds the array is rejected with MK_ESCRATCH before anything is enqueued (at the shard
 * shape: a global-attention context above about 83K tokens, or batch two).  The first call on
 * a device also enqueues the fill kernels of mk_workspace_init on the array (counters to zero,
 * the rest to the all-ones sentinel).  No call allocates or frees memory.  Every call on a GPU shares that GPU's array, which keeps the last call's contents:
 * calls that overlap on one GPU (concurrent streams, host threads) race and must not be
 * issued.  mk_read_status(NULL, stream) returns the in-kernel status of the last call on the
 * current device. */
#define MK_NOALLOC_SCRATCH_BYTES ((size_t)24 << 20)
int mk_layer_step_noalloc(const mk_layer_cfg *cfg /* [host] */, const mk_layer_weights *w /* [host] */,
                          const mk_step_io *io /* [host] */, void *stream);

/* One rank's share of the N-sharded expert layout.  The pages shard both expert GEMMs on
 * their output dimension across the R tensor-parallel ranks, with an fp4 all-gather of the
 * intermediate after the first and a bf16 all-gather of the expert output after the second,
 * a layout bitwise-consistent with expert parallelism (orcarouter.ai write-up, "where the
 * kernel boundary sits"); receivers poll the payload against a sentinel that no result can
 * take, instead of a flag (alphasignal.ai, "Four mechanisms keep work moving").  On one GPU
 * this is rank `rank`'s part of the step, with the two gathered buffers supplied by the caller
 * (the other ranks' parts arrive there as data):
 *  - GEMM1 computes this rank's I = cfg.expert_inter intermediate channels (w1_* as in
 *    mk_layer_step: the full expert's gate and up rows of those channels) and writes them as
 *    records r I/16 .. (r+1) I/16 - 1 of each pair's row of act_recv;
 *  - GEMM2 multiplies the gathered rows (K2 = n_ranks I) by this rank's rows of the full down
 *    projection -- w2_codes uint8 [E][P/R][K2/2], w2_scales uint8 [E][P/R][K2/16] (row-major,
 *    mk_nvfp4_pack layout, whole-matrix tensor scales in w2_tscale) -- for output columns
 *    [r P/R, (r+1) P/R), combines the top-k slots locally and writes those columns of y_recv;
 *  - the unpooler reads all of y_recv.
 * act_recv: [T*top_k][K2/16] records of 16 bytes, pair p = t*top_k + slot; record q holds
 *   elements 16q..16q+15 of the pair's intermediate: uint32 codes of elements 0-7 (element j in
 *   bits 4j..4j+3, E2M1), uint32 E4M3 scale byte (bits 0-7, other bits 0), uint32 codes of
 *   elements 8-15, the scale again; the tensor scale is 1.  A record not yet delivered holds
 *   all ones (a real record never does: its scale word is at most 0x7E).
 * y_recv: bf16 [16][P] in fragment order (as mk_workspace_layout describes), rows >= T
 *   unused; columns not yet delivered hold 0xFFFF (a bf16 result never does).
 * Before the launch the caller sets this rank's records and this rank's y_recv columns to all
 * ones; the other ranks' records and columns hold their data or all ones (the kernel then
 * waits for them, bounded by spin_limit: a slot that never arrives ends in MK_ETIMEOUT).  The
 * launch writes this rank's records and columns and reads everything else.  Both buffers are
 * DEVICE, caller-owned, 16-byte aligned (else MK_EALIGN), NULL -> MK_EINVAL.
 * Shapes: everything mk_layer_step needs, expert_fmt MK_W_NVFP4 (else MK_EINVAL),
 * 2 <= n_ranks <= 8 and 0 <= rank < n_ranks, pooled % (8 n_ranks) == 0 and
 * (n_ranks expert_inter) % 256 == 0, else MK_ESHAPE.  Enqueues one kernel. */
typedef struct {
  int rank;            /* this rank r                                                  */
  int n_ranks;         /* R                                                            */
  void *act_recv;      /* gathered intermediate records (DEVICE)                       */
  void *y_recv;        /* gathered expert output, bf16 fragment order (DEVICE)         */
} mk_nshard;
int mk_layer_step_nshard(const mk_layer_cfg *cfg /* [host] */, const mk_layer_weights *w /* [host] */,
                         const mk_step_io *io /* [host] */, const mk_nshard *ns /* [host] */, void *stream);

/* KV-cache write: copy n new rows into a KV cache pair at rows pos..pos+n-1, bit for bit,
 * every other row untouched.  The pages' launch ends with the next layer's KV write, and the
 * KV history a layer attends over was written by earlier steps (orcarouter.ai write-up,
 * "where the kernel boundary sits"); this call places rows that no fused launch produced
 * (a layer's tree rows supplied by the caller, a commit of accepted tokens).
 * k_cache, v_cache: bf16 [capacity][n_kv_heads][head_dim] (DEVICE, caller-owned, written);
 * k_new, v_new: bf16 [n][n_kv_heads][head_dim] (DEVICE, read).  n >= 0 (0 enqueues nothing);
 * n_kv_heads * head_dim % 8 == 0 else MK_ESHAPE; pos < 0 or pos + n > capacity -> MK_ECAPACITY;
 * any pointer not 16-byte aligned -> MK_EALIGN.  Enqueues one kernel. */
int mk_kv_append(void *k_cache, void *v_cache, int capacity, int n_kv_heads, int head_dim, int pos,
                 const void *k_new, const void *v_new, int n, void *stream);

/* First-layer prologue.  The pages' first and last launches differ from the others
 * (alphasignal.ai, "Draft and verify share one graph"; orcarouter.ai, "where the kernel
 * boundary sits"): no launch before layer 0 produces its queries and tree K/V rows, so this
 * call computes them from the tokens' embeddings.  [q; k; v] = h . w_qkv^T with one bf16
 * rounding (fp32 accumulation): q -> q_out, k and v -> rows pos..pos+T-1 of layer 0's cache
 * (every other row untouched).
 * h bf16 [T][hidden]; w_qkv bf16 [(n_q_heads + 2 n_kv_heads) head_dim][hidden] (query rows,
 * then key rows, then value rows); q_out bf16 [T][n_q_heads head_dim]; k_cache, v_cache bf16
 * [capacity][n_kv_heads][head_dim].  1 <= T <= 16, hidden % 32 == 0, the output width a
 * multiple of 16, n_kv_heads dividing n_q_heads; pos + T > capacity -> MK_ECAPACITY.
 * Enqueues one kernel. */
int mk_qkv_prologue(const void *h, const void *w_qkv, int T, int hidden, int n_q_heads, int n_kv_heads,
                    int head_dim, void *q_out, void *k_cache, void *v_cache, int capacity, int pos,
                    void *stream);

/* Greedy acceptance after a verify step (the pages decode greedily and keep the accepted part
 * of a 16-token tree: orcarouter.ai, "what the number is and isn't"; the rule itself is not
 * printed, the plain greedy one is taken).  From the root (node 0), repeatedly follow the
 * lowest-index child whose drafted token equals the target's greedy token at the current
 * node; stop when no child does.
 * parent int32 [T] (as in mk_step_io: parent[0] = -1, parent[i] < i); draft int32 [T] (each
 * node's token; node 0's is the last accepted token); target int32 [T] (the target model's
 * greedy token after each node).  Outputs: path int32 [T] (accepted nodes root-first, then -1),
 * n_path int32 [1] (>= 1), bonus int32 [1] (the target token after the last accepted node).
 * A malformed tree gives n_path = 0, bonus = -1 and path all -1.  1 <= T <= 64.  Enqueues one
 * kernel; nothing is read back, so the call can sit in a captured step graph. */
int mk_tree_accept(const int32_t *parent, const int32_t *draft, const int32_t *target, int T, int32_t *path,
                   int32_t *n_path, int32_t *bonus, void *stream);

/* KV commit of an accepted path in one layer's cache pair: row ctx + path[j] moves to row
 * ctx + j for j < *n_path (read on the device; values above T are clamped to T), every other
 * row untouched.  All source rows are read before any is written.  k_cache, v_cache bf16
 * [capacity][n_kv_heads][head_dim]; path, n_path as written by mk_tree_accept.  1 <= T <= 64,
 * 2 T n_kv_heads head_dim <= 16384, ctx + T <= capacity.  Enqueues one kernel per call (one
 * call per layer). */
int mk_kv_commit(void *k_cache, void *v_cache, int capacity, int n_kv_heads, int head_dim, int ctx,
                 const int32_t *path, const int32_t *n_path, int T, void *stream);

/* mk_kv_commit for n_layers layers in one launch (one workgroup per layer): k_caches and
 * v_caches are DEVICE arrays of n_layers cache pointers (8-byte aligned; every cache 16-byte
 * aligned, all with the same shape).  Same rules and results as n_layers mk_kv_commit calls. */
int mk_kv_commit_layers(void *const *k_caches, void *const *v_caches, int n_layers, int capacity, int n_kv_heads,
                        int head_dim, int ctx, const int32_t *path, const int32_t *n_path, int T, void *stream);

/* Router on its own: the layer's router sends each token to 8 of 256 experts (orcarouter.ai
 * write-up, "where the kernel boundary sits"; the selection rule and the gates are not
 * printed: top-k by (logit desc, index asc), softmax over the k selected logits).
 * logits = x . w_router^T (+ bias) in fp32 with fp32 accumulation, then the top-k experts per
 * token ordered by (logit desc, index asc) and softmax gates over the k selected logits --
 * the same selection the fused launch makes.
 * x bf16 [T][P]; w_router bf16 [E][P]; bias fp32 [T][E] or NULL; idx int32 [T][k] (written);
 * gate fp32 [T][k] (written); logits fp32 [T][E] or NULL (written); all DEVICE, caller-owned.
 * 1 <= T <= 64, E <= 256, 1 <= k <= min(8, E), P % 8 == 0, else MK_ESHAPE; x and w_router
 * 16-byte aligned, else MK_EALIGN.  Enqueues one kernel. */
int mk_route_topk(const void *x, const void *w_router, const float *bias, int T, int P, int E, int k,
                  int32_t *idx, float *gate, float *logits, void *stream);

/* NVFP4 weight packing: the routed experts are stored as 4-bit NVFP4 (orcarouter.ai write-up,
 * "where the kernel boundary sits"); the format's details are its public definition (E2M1
 * codes, an E4M3 scale per 16 elements, an fp32 tensor scale).
 * Quantisation of `batch` matrices w [batch][N][K] (bf16 when w_is_fp32 == 0, else
 * fp32), K % 16 == 0.  Per matrix: tensor scale ts = fp32(amax) / 2688 (1 when amax = 0);
 * per 16-element block: E4M3 scale s = RNE(amax_block / (6 ts)) saturating at 448;
 * per element: E2M1 code = RNE(x / (s ts)) saturating at +-6, ties to the even code, a zero
 * result stored as +0, all codes 0 when s = 0.  Rounding decisions are exact comparisons with
 * grid midpoints.  Outputs: codes uint8 [batch][N][K/2] (element 2j in the low nibble),
 * scales uint8 [batch][N][K/16], tensor_scale fp32 [batch]. */
int mk_nvfp4_pack(const void *w, int w_is_fp32, int batch, int N, int K, uint8_t *codes,
                  uint8_t *scales, float *tensor_scale, void *stream);

/* Rearranges W1's NVFP4 codes and scales (as mk_nvfp4_pack writes them: codes [batch][N][K/2],
 * scales [batch][N][K/16]) into the order GEMM1 reads them, so that every 64-lane weight fetch
 * is 1 KB contiguous.  N % 16 == 0, K % 128 == 0.  With L = K/128 k-steps per row,
 * p = (L > 8 ? 2 : 1) pieces per row and S = 8 * ceil(L / p) scale bytes per piece and row:
 *   codes_t  [batch][N/16][L][64][16]: codes_t[b][t][s][l][i] = codes[b][16t + l%16][64s + 16(l/16) + i]
 *   scales_t [batch][N/16][p][16][S]:  scales_t[b][t][q][r][i] = scales[b][16t + r][qS + i], 0 past K/16
 * scales_t takes mk_nvfp4_w1_scales_bytes(batch, N, K) bytes (batch * N * K/16 when L is even or
 * at most 8).  Pure byte permutation; codes, codes_t and scales_t 16-byte aligned. */
int mk_nvfp4_tile_w1(const uint8_t *codes, const uint8_t *scales, int batch, int N, int K,
                     uint8_t *codes_t, uint8_t *scales_t, void *stream);
/* Bytes of mk_nvfp4_tile_w1's scales_t, or 0 for an unsupported shape. */
size_t mk_nvfp4_w1_scales_bytes(int batch, int N, int K);

/* Synchronise `stream` and return the in-kernel status of the last mk_layer_step on this
 * workspace (MK_OK, MK_EBADTREE or MK_ETIMEOUT), or MK_EHIP if a copy failed.  An error of an
 * earlier launch is not reported once a later launch has run.  workspace NULL: the status of
 * the last mk_layer_step_noalloc on the current device (MK_EINVAL if there was none). */
int mk_read_status(const void *workspace, void *stream);

/* Streaming-read probe: reads `bytes` bytes of src once, in coalesced 16-byte non-temporal
 * loads with 8 per thread in flight, over n_blocks workgroups of 256 threads (0 = 8 per CU),
 * and computes nothing else.  The time it takes gives the HBM read rate that a plain stream
 * reaches on this device, the practical ceiling for the weight streams of mk_layer_step (the
 * pages price a decode layer by the bytes it must bring from HBM: alphasignal.ai, "Launch
 * boundaries leave hardware idle").  src DEVICE, 16-byte aligned, bytes % 16 == 0, else
 * MK_EALIGN; sink DEVICE uint32 [1], 4-byte aligned: the XOR of every 32-bit word read is
 * XORed into it atomically (a checksum: zero it first to obtain the data's XOR).  n_blocks in
 * [0, 2^20], else MK_ESHAPE.  Enqueues one kernel. */
int mk_stream_read(const void *src, size_t bytes, int n_blocks, uint32_t *sink, void *stream);

/* Human-readable name of a status code. */
const char *mk_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* MK_H_ */

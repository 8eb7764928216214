// C ABI (include/mk.h): argument validation on the host, workspace layout, launches.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/mk.h"
#include "mk_internal.h"

// The static scratch of mk_layer_step_noalloc (see scratch_ptr): a file-scope device array, one
// copy on every GPU the library runs on.
constexpr size_t kScratchBytes = (size_t)24 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
constexpr int kDefaultSpin = 1 << 20;      // polls per wait before MK_ETIMEOUT

std::mutex g_mu;
int g_cu[kMaxDevices];                     // CU count per device (0 = not queried)
bool g_attr[kMaxDevices];

int device_cus(int* n_cu) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MK_EHIP;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_cu[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return MK_EHIP;
    g_cu[dev] = n < 256 ? n : 256;   // the kernel's flag polling covers at most 256 workgroups
  }
  if (!g_attr[dev]) {
    if (mk::set_layer_kernel_attrs(mk::layer_lds_bytes())) return MK_EHIP;
    g_attr[dev] = true;
  }
  *n_cu = g_cu[dev];
  return MK_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

int check_cfg(const mk_layer_cfg* c, int T) {
  if (!c) return MK_EINVAL;
  if (c->expert_fmt != MK_W_BF16 && c->expert_fmt != MK_W_NVFP4) return MK_EINVAL;
  if (T < 1 || T > 16) return MK_ESHAPE;
  if (c->hidden <= 0 || c->hidden % 128 || c->hidden > 4096) return MK_ESHAPE;
  if (c->pooled <= 0 || c->pooled % 128 || c->pooled > 2048) return MK_ESHAPE;
  if (c->head_dim != 64 && c->head_dim != 128) return MK_ESHAPE;
  if (c->n_kv_heads <= 0 || c->n_q_heads <= 0 || c->n_q_heads % c->n_kv_heads) return MK_ESHAPE;
  if (T * (c->n_q_heads / c->n_kv_heads) > 128) return MK_ESHAPE;
  if (c->n_q_heads * c->head_dim > 1024) return MK_ESHAPE;
  if (c->n_experts <= 0 || c->n_experts > 256 || c->n_experts % 16) return MK_ESHAPE;
  if (c->top_k < 1 || c->top_k > 8 || c->top_k > c->n_experts) return MK_ESHAPE;
  if (c->expert_inter <= 0 || c->expert_inter % 32 || c->expert_inter > 256) return MK_ESHAPE;
  if (c->window < 0) return MK_ESHAPE;
  if (c->kv_capacity <= 0) return MK_ESHAPE;
  return MK_OK;
}

struct Layout {
  size_t status, epoch, flags, qkv_cnt, zero_end, stage, qkv_part, part_ml, part_o, total;
  int n_wg, items, chunks_per_head, attn_lo, ck, rw, nrb, part_slots;
};

// The counters at the start of every workspace (status word, epoch slots, flags, qkv arrival
// counters) start at zero; everything after them starts as the all-ones sentinel.
size_t zero_bytes(int n_wg) {
  size_t o = up256(4);                 // status word (mk::kStatusOffset)
  o = up256(o + (size_t)n_wg * 64);    // epoch slots (mk::kEpochOffset)
  o = up256(o + (size_t)n_wg * 64);    // flags
  return up256(o + (size_t)n_wg * 64); // split-K qkv arrival counters
}

constexpr int kChunkMax = 256;     // keys per attention chunk held in LDS

// Attention work split.  The visible context rows [attn_lo, ctx) of each kv head are cut into
// chunks of ck keys, plus one chunk holding the tree's own slots; each chunk's (token, q head)
// rows are cut into row blocks of rw tiles of 16 rows.  An item is one (kv head, chunk, row
// block); its 8 waves split it as rw row tiles x 8/rw key groups.  Among rw = 1, 2, 4, 8 the
// split taken is the one that moves the fewest bytes through one workgroup: the K/V it stages
// and the partials it stores per round of items, plus what one merge unit reads back.
void attn_split(const mk_layer_cfg* c, int T, int ctx, int n_wg, Layout* L) {
  const int l = c->window > 0 ? (ctx - c->window + 1 > 0 ? ctx - c->window + 1 : 0) : 0;
  const int keys = ctx - l, d = c->head_dim, Hkv = c->n_kv_heads;
  const int RT = (T * (c->n_q_heads / Hkv) + 15) / 16;    // row tiles, <= 8
  double best = -1.0;
  for (int rw = 1; rw <= 8; rw *= 2) {
    if (rw > 1 && rw / 2 >= RT) break;                     // whole row tiles of nothing
    const int nrb = (RT + rw - 1) / rw, nkw = 8 / rw, gran = 16 * nkw;
    const int slots = n_wg / (Hkv * nrb) - 1;              // context chunks per round
    int ck = slots > 0 ? (keys + slots - 1) / slots : kChunkMax;
    ck = (ck + gran - 1) / gran * gran;
    if (ck < gran) ck = gran;
    if (ck > kChunkMax) ck = kChunkMax;                    // gran divides kChunkMax
    const int chunks = (keys + ck - 1) / ck + 1;
    const long items = (long)Hkv * nrb * chunks;
    const long rounds = (items + n_wg - 1) / n_wg;
    const double cost = (double)rounds * ((double)ck * 4 * d + (double)rw * 16 * d * 4) + (double)chunks * (d * 4 + 8);
    if (best < 0 || cost < best) {
      best = cost;
      L->attn_lo = l; L->chunks_per_head = chunks; L->ck = ck; L->rw = rw; L->nrb = nrb;
      L->items = (int)items;
    }
  }
}

// `B` sequences of T tokens share the launch: each sequence's attention is split exactly as in
// a launch of its own (so that a sequence's results do not depend on the batch it is in), and
// its items follow the previous sequence's.  The attention partials and the split-K qkv
// partials take B times the room; every offset before them does not depend on B.
Layout layout(const mk_layer_cfg* c, int T, int ctx, int n_wg, int B = 1) {
  Layout L;
  memset(&L, 0, sizeof(L));
  L.n_wg = n_wg;
  attn_split(c, T, ctx, n_wg, &L);
  L.items *= B;
  // partial slots [sequence][kv head][chunk]: a split within one round has at most n_wg of
  // them; beyond, chunks are kChunkMax keys and their count grows with the context
  {
    const int keys_max = ctx - (c->window > 0 && ctx - c->window + 1 > 0 ? ctx - c->window + 1 : 0);
    const int big = c->n_kv_heads * ((keys_max + kChunkMax - 1) / kChunkMax + 1);
    L.part_slots = B * (big > n_wg ? big : n_wg);
  }
  const int d = c->head_dim;
  size_t o = 0;
  L.status = o; o = up256(o + 4);               // mk::kStatusOffset
  L.epoch = o; o = up256(o + (size_t)n_wg * 64); // mk::kEpochOffset
  L.flags = o; o = up256(o + (size_t)n_wg * 64);
  L.qkv_cnt = o; o = up256(o + (size_t)n_wg * 64);
  L.zero_end = o;                                // == zero_bytes(n_wg)
  // the stage buffers, two copies at fixed offsets (mk::kStage*)
  L.stage = o; o = up256(o + 2 * (size_t)mk::kStageBytes);
  // split-K qkv: at most one (tile, part) per workgroup, one partial per sequence
  L.qkv_part = o; o = up256(o + (size_t)n_wg * B * 64 * 4 * 4);
  // attention partials [slot][128 rows]: (m, l), then o
  L.part_ml = o; o = up256(o + (size_t)L.part_slots * 128 * 2 * 4);
  L.part_o = o; o = up256(o + (size_t)L.part_slots * 128 * d * 4);
  L.total = o;
  return L;
}

// Counters to zero, the rest to the sentinel (fill kernels).
int init_workspace(char* ws, size_t bytes, int n_wg, hipStream_t stream) {
  const size_t z = zero_bytes(n_wg) < bytes ? zero_bytes(n_wg) : bytes;
  if (mk::launch_fill(ws, z, 0u, stream)) return MK_EHIP;
  if (bytes > z && mk::launch_fill(ws + z, bytes - z, 0xFFFFFFFFu, stream)) return MK_EHIP;
  return MK_OK;
}

// Every argument, shape and capacity check of a layer launch, and its kernel arguments apart
// from the workspace (bind_workspace).  `need_ws`: io->workspace is the workspace (else the
// caller supplies one of `ws_bytes`).  `*Lout` is the workspace layout once the shape checks
// have passed.  No HIP call enqueues anything here.
int build_args(const mk_layer_cfg* c, const mk_layer_weights* w, const mk_step_io* io, bool need_ws,
               size_t ws_bytes, mk::KArgs* out, Layout* Lout) {
  memset(Lout, 0, sizeof(*Lout));
  if (!c || !w || !io) return MK_EINVAL;
  int rc = check_cfg(c, io->T);
  if (rc) return rc;
  const int T = io->T, ctx = io->ctx_len;
  const int B = io->batch <= 1 ? 1 : io->batch;
  if (io->batch < 0 || B > 2) return MK_ESHAPE;
  if (B > 1 && (T != 16 || c->expert_fmt != MK_W_NVFP4 || c->expert_inter % 64 || c->expert_inter < 128 ||
                c->expert_inter > 192))
    return MK_ESHAPE;
  if (ctx < 0 || ctx + T > c->kv_capacity) return MK_ECAPACITY;
  if (need_ws && !io->workspace) return MK_EINVAL;
  const void* req[] = {io->tree_parent, io->q_in, io->h_in, io->k_cache, io->v_cache, io->h_out,
                       w->w_o, w->w_pool, w->w_router, w->w_unpool};
  for (const void* p : req) if (!p) return MK_EINVAL;
  // the next layer's q/k/v are produced unless this is the stack's last layer (w_qkv_next NULL)
  if (w->w_qkv_next && (!io->q_next || !io->k_cache_next || !io->v_cache_next)) return MK_EINVAL;
  if (c->expert_fmt == MK_W_BF16) {
    if (!w->w1 || !w->w2) return MK_EINVAL;
  } else {
    if (!w->w1_codes || !w->w1_scales || !w->w2_codes || !w->w2_scales || !w->w1_tscale || !w->w2_tscale)
      return MK_EINVAL;
    if (c->pooled % 128) return MK_ESHAPE;
  }
  if (io->n_prefetch < 0 || io->n_prefetch > 16) return MK_ESHAPE;
  if (io->n_prefetch > 0 && !io->prefetch_experts) return MK_EINVAL;
  if (io->n_prefetch_next < 0 || io->n_prefetch_next > 16) return MK_ESHAPE;
  if (io->n_prefetch_next > 0 && !io->prefetch_next) return MK_EINVAL;
  if (io->spin_limit < 0) return MK_EINVAL;
  const void* al[] = {io->q_in, io->h_in, io->k_cache, io->v_cache, io->k_cache_next, io->v_cache_next,
                      io->h_out, io->q_next, need_ws ? io->workspace : nullptr, io->topk_idx, io->topk_gate,
                      io->router_logits, io->attn_stats, io->router_bias, w->w_o, w->w_pool,
                      w->w_router, w->w_unpool, w->w_qkv_next, w->w1, w->w2, w->w1_codes,
                      w->w1_scales, w->w2_codes, w->w2_scales};
  for (const void* p : al) if (p && !aligned16(p)) return MK_EALIGN;
  int n_wg = 0;
  rc = device_cus(&n_wg);
  if (rc) return rc;
  // the workspace must cover the largest context this cache allows, so one workspace serves
  // every step of a layer
  Layout L = layout(c, T, c->kv_capacity - T, n_wg, B);
  Layout Lc = layout(c, T, ctx, n_wg, B);
  *Lout = L;
  if (ws_bytes < L.total) return MK_ECAPACITY;
  if (B * c->n_kv_heads * Lc.chunks_per_head > L.part_slots) return MK_ECAPACITY;

  mk::KArgs& a = *out;
  memset(&a, 0, sizeof(a));
  a.H = c->hidden; a.Hq = c->n_q_heads; a.Hkv = c->n_kv_heads; a.d = c->head_dim; a.P = c->pooled;
  a.E = c->n_experts; a.topk = c->top_k; a.I = c->expert_inter; a.window = c->window;
  a.fmt = c->expert_fmt; a.cap = c->kv_capacity; a.T = T * B; a.ctx = ctx; a.B = B; a.Ts = T;
  a.n_wg = n_wg; a.attn_items = Lc.items; a.attn_chunks_per_head = Lc.chunks_per_head;
  a.attn_lo = Lc.attn_lo; a.ck = Lc.ck; a.attn_rw = Lc.rw; a.attn_nrb = Lc.nrb;
  a.spin_limit = io->spin_limit > 0 ? io->spin_limit : kDefaultSpin;
  a.skip_wg = io->debug_skip_signal_wg;
  a.parent = io->tree_parent;
  a.q_in = (const uint16_t*)io->q_in; a.h_in = (const uint16_t*)io->h_in;
  a.kc = (const uint16_t*)io->k_cache; a.vc = (const uint16_t*)io->v_cache;
  a.kn = (uint16_t*)io->k_cache_next; a.vn = (uint16_t*)io->v_cache_next;
  a.h_out = (uint16_t*)io->h_out; a.q_next = (uint16_t*)io->q_next;
  a.topk_idx = io->topk_idx; a.topk_gate = io->topk_gate; a.router_logits = io->router_logits;
  a.attn_stats = io->attn_stats; a.hist = io->expert_hist;
  a.prefetch = io->prefetch_experts; a.n_prefetch = io->n_prefetch; a.bias = io->router_bias;
  a.prefetch_next = io->prefetch_next; a.n_prefetch_next = io->n_prefetch_next;
  a.w_o = (const uint16_t*)w->w_o; a.w_pool = (const uint16_t*)w->w_pool;
  a.w_router = (const uint16_t*)w->w_router; a.w_unpool = (const uint16_t*)w->w_unpool;
  a.w_qkv = (const uint16_t*)w->w_qkv_next;
  a.w1 = (const uint16_t*)w->w1; a.w2 = (const uint16_t*)w->w2;
  a.w1_codes = w->w1_codes; a.w1_scales = w->w1_scales; a.w2_codes = w->w2_codes; a.w2_scales = w->w2_scales;
  a.w1_ts = w->w1_tscale; a.w2_ts = w->w2_tscale;
  a.timestamps = io->timestamps;
  return MK_OK;
}

// The kernel's workspace regions at `ws` (layout L).
void bind_workspace(mk::KArgs* ap, const Layout& L, char* ws) {
  mk::KArgs& a = *ap;
  a.status = (uint32_t*)(ws + L.status);
  a.epoch = (uint32_t*)(ws + L.epoch);
  a.flags = (uint32_t*)(ws + L.flags);
  a.stage = ws + L.stage;
  a.part_o = (float*)(ws + L.part_o);
  a.part_ml = (float*)(ws + L.part_ml);
  a.qkv_part = (float*)(ws + L.qkv_part);
  a.qkv_cnt = (uint32_t*)(ws + L.qkv_cnt);
}

// ---- static scratch of mk_layer_step_noalloc
// The workspace of the allocation-free entry point: one file-scope device array per GPU that
// the library runs on, held until the process ends.  Its device address is taken once per
// device with hipGetSymbolAddress (the array's name is only a host-side stand-in) and the
// array is initialised then as mk_workspace_init does (the status word, epoch slots, flags and
// counters to zero, the stage buffers to the sentinel); every later call on that device reuses
// it as it was left.
char* g_scratch[kMaxDevices];   // per device: the device address of `scratch`, once set up

int scratch_ptr(hipStream_t stream, int n_wg, char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MK_EHIP;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MK_EHIP;
    if (init_workspace((char*)p, kScratchBytes, n_wg, stream)) return MK_EHIP;
    g_scratch[dev] = (char*)p;
  }
  *out = g_scratch[dev];
  return MK_OK;
}

char* scratch_if_set() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  return g_scratch[dev];
}

}  // namespace

extern "C" {

const char* mk_strerror(int s) {
  switch (s) {
    case MK_OK: return "ok";
    case MK_EINVAL: return "invalid argument";
    case MK_ESHAPE: return "unsupported shape";
    case MK_EALIGN: return "pointer not 16-byte aligned";
    case MK_ECAPACITY: return "KV cache or workspace too small";
    case MK_EHIP: return "HIP runtime error";
    case MK_ETIMEOUT: return "in-kernel wait timed out";
    case MK_EBADTREE: return "malformed tree_parent";
    case MK_ESCRATCH: return "configuration needs a larger workspace than the 24 MiB static scratch of mk_layer_step_noalloc";
    default: return "unknown status";
  }
}

int mk_workspace_query(const mk_layer_cfg* cfg, int T, mk_workspace_layout* out) {
  // the layout depends on ctx through the attention split; the query assumes the largest
  // context the cache allows
  int rc = check_cfg(cfg, T);
  if (rc) return rc;
  if (!out) return MK_EINVAL;
  int n_wg = 0;
  rc = device_cus(&n_wg);
  if (rc) return rc;
  // T = 16 may also run two sequences (mk_step_io.batch = 2): the size covers that
  const int B = T == 16 ? 2 : 1;
  Layout L = layout(cfg, T, cfg->kv_capacity - T > 0 ? cfg->kv_capacity - T : 0, n_wg, B);
  out->status = L.status;
  out->attn = L.stage + mk::kStageAttn;
  out->h1 = L.stage + mk::kStageH1;
  out->xp = L.stage + mk::kStageXp;
  out->logits = L.stage + mk::kStageLogits;
  out->y = L.stage + mk::kStageY;
  out->total = L.total;
  out->n_wg = L.n_wg;
  out->attn_items = L.items;
  out->stage_copy = mk::kStageBytes;
  out->epoch = L.epoch;
  return MK_OK;
}

size_t mk_workspace_bytes(const mk_layer_cfg* cfg, int T) {
  mk_workspace_layout l;
  if (mk_workspace_query(cfg, T, &l)) return 0;
  return l.total;
}

int mk_workspace_init(void* ws, size_t bytes, void* stream) {
  if (!ws || bytes == 0) return MK_EINVAL;
  if (!aligned16(ws) || bytes % 16) return MK_EALIGN;
  int n_wg = 0;
  const int rc = device_cus(&n_wg);
  if (rc) return rc;
  return init_workspace((char*)ws, bytes, n_wg, (hipStream_t)stream);
}

int mk_layer_step(const mk_layer_cfg* c, const mk_layer_weights* w, const mk_step_io* io, void* stream) {
  mk::KArgs a;
  Layout L;
  int rc = build_args(c, w, io, true, io ? io->workspace_bytes : 0, &a, &L);
  if (rc) return rc;
  bind_workspace(&a, L, (char*)io->workspace);
  return mk::launch_layer(a, mk::layer_lds_bytes(), (hipStream_t)stream) ? MK_EHIP : MK_OK;
}

int mk_layer_step_noalloc(const mk_layer_cfg* c, const mk_layer_weights* w, const mk_step_io* io, void* stream) {
  mk::KArgs a;
  Layout L;
  int rc = build_args(c, w, io, false, kScratchBytes, &a, &L);
  if (rc) return rc == MK_ECAPACITY && L.total > kScratchBytes ? MK_ESCRATCH : rc;
  char* ws = nullptr;
  rc = scratch_ptr((hipStream_t)stream, L.n_wg, &ws);
  if (rc) return rc;
  bind_workspace(&a, L, ws);
  return mk::launch_layer(a, mk::layer_lds_bytes(), (hipStream_t)stream) ? MK_EHIP : MK_OK;
}

int mk_layer_step_nshard(const mk_layer_cfg* c, const mk_layer_weights* w, const mk_step_io* io, const mk_nshard* ns,
                         void* stream) {
  if (!ns || !c) return MK_EINVAL;
  if (c->expert_fmt != MK_W_NVFP4) return MK_EINVAL;
  if (ns->n_ranks < 2 || ns->n_ranks > 8 || ns->rank < 0 || ns->rank >= ns->n_ranks) return MK_ESHAPE;
  if (c->pooled % (8 * ns->n_ranks) || (ns->n_ranks * c->expert_inter) % 256) return MK_ESHAPE;
  if (!ns->act_recv || !ns->y_recv) return MK_EINVAL;
  if (!aligned16(ns->act_recv) || !aligned16(ns->y_recv)) return MK_EALIGN;
  if (io && io->batch > 1) return MK_ESHAPE;
  mk::KArgs a;
  Layout L;
  int rc = build_args(c, w, io, true, io ? io->workspace_bytes : 0, &a, &L);
  if (rc) return rc;
  // a workgroup's GEMM2 tasks must span at most two units: the grid covers the column blocks
  // and the units (at most T k / 2)
  if (c->pooled / (8 * ns->n_ranks) > a.n_wg || (io->T * c->top_k + 1) / 2 > a.n_wg) return MK_ESHAPE;
  a.ns_r = ns->rank;
  a.ns_R = ns->n_ranks;
  a.act_recv = (uint32_t*)ns->act_recv;
  a.y_recv = (uint16_t*)ns->y_recv;
  bind_workspace(&a, L, (char*)io->workspace);
  return mk::launch_layer(a, mk::layer_lds_bytes(), (hipStream_t)stream) ? MK_EHIP : MK_OK;
}

int mk_kv_append(void* k_cache, void* v_cache, int capacity, int n_kv_heads, int head_dim, int pos,
                 const void* k_new, const void* v_new, int n, void* stream) {
  if (!k_cache || !v_cache || !k_new || !v_new) return MK_EINVAL;
  if (n_kv_heads <= 0 || head_dim <= 0 || (n_kv_heads * head_dim) % 8 || n < 0 || capacity <= 0) return MK_ESHAPE;
  if (pos < 0 || pos + n > capacity) return MK_ECAPACITY;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new)) return MK_EALIGN;
  if (n == 0) return MK_OK;
  return mk::launch_kv_append((uint16_t*)k_cache, (uint16_t*)v_cache, n_kv_heads * head_dim, pos,
                              (const uint16_t*)k_new, (const uint16_t*)v_new, n, (hipStream_t)stream)
             ? MK_EHIP : MK_OK;
}

int mk_qkv_prologue(const void* h, const void* w_qkv, int T, int hidden, int n_q_heads, int n_kv_heads,
                    int head_dim, void* q_out, void* k_cache, void* v_cache, int capacity, int pos, void* stream) {
  if (!h || !w_qkv || !q_out || !k_cache || !v_cache) return MK_EINVAL;
  if (T < 1 || T > 16 || hidden <= 0 || hidden % 32 || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 ||
      n_q_heads % n_kv_heads || ((n_q_heads + 2 * n_kv_heads) * head_dim) % 16 || capacity <= 0)
    return MK_ESHAPE;
  if (pos < 0 || pos + T > capacity) return MK_ECAPACITY;
  if (!aligned16(h) || !aligned16(w_qkv) || !aligned16(q_out) || !aligned16(k_cache) || !aligned16(v_cache))
    return MK_EALIGN;
  return mk::launch_qkv_prologue((const uint16_t*)h, (const uint16_t*)w_qkv, T, hidden, n_q_heads * head_dim,
                                 n_kv_heads * head_dim, (uint16_t*)q_out, (uint16_t*)k_cache, (uint16_t*)v_cache,
                                 pos, (hipStream_t)stream)
             ? MK_EHIP : MK_OK;
}

int mk_tree_accept(const int32_t* parent, const int32_t* draft, const int32_t* target, int T, int32_t* path,
                   int32_t* n_path, int32_t* bonus, void* stream) {
  if (!parent || !draft || !target || !path || !n_path || !bonus) return MK_EINVAL;
  if (T < 1 || T > 64) return MK_ESHAPE;
  return mk::launch_tree_accept(parent, draft, target, T, path, n_path, bonus, (hipStream_t)stream) ? MK_EHIP : MK_OK;
}

int mk_kv_commit(void* k_cache, void* v_cache, int capacity, int n_kv_heads, int head_dim, int ctx,
                 const int32_t* path, const int32_t* n_path, int T, void* stream) {
  if (!k_cache || !v_cache || !path || !n_path) return MK_EINVAL;
  if (n_kv_heads <= 0 || head_dim <= 0 || (n_kv_heads * head_dim) % 8 || T < 1 || T > 64 ||
      (size_t)2 * T * n_kv_heads * head_dim * 2 > 65536 || capacity <= 0)
    return MK_ESHAPE;
  if (ctx < 0 || ctx + T > capacity) return MK_ECAPACITY;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return MK_EALIGN;
  return mk::launch_kv_commit((uint16_t*)k_cache, (uint16_t*)v_cache, nullptr, nullptr, 1, n_kv_heads * head_dim, ctx,
                              path, n_path, T, (hipStream_t)stream)
             ? MK_EHIP : MK_OK;
}

int mk_kv_commit_layers(void* const* k_caches, void* const* v_caches, int n_layers, int capacity, int n_kv_heads,
                        int head_dim, int ctx, const int32_t* path, const int32_t* n_path, int T, void* stream) {
  if (!k_caches || !v_caches || !path || !n_path) return MK_EINVAL;
  if (n_layers < 1 || n_layers > 65535 || n_kv_heads <= 0 || head_dim <= 0 || (n_kv_heads * head_dim) % 8 || T < 1 ||
      T > 64 || (size_t)2 * T * n_kv_heads * head_dim * 2 > 65536 || capacity <= 0)
    return MK_ESHAPE;
  if (ctx < 0 || ctx + T > capacity) return MK_ECAPACITY;
  if (((uintptr_t)k_caches & 7u) || ((uintptr_t)v_caches & 7u)) return MK_EALIGN;
  return mk::launch_kv_commit(nullptr, nullptr, (uint16_t* const*)k_caches, (uint16_t* const*)v_caches, n_layers,
                              n_kv_heads * head_dim, ctx, path, n_path, T, (hipStream_t)stream)
             ? MK_EHIP : MK_OK;
}

int mk_route_topk(const void* x, const void* w_router, const float* bias, int T, int P, int E, int k,
                  int32_t* idx, float* gate, float* logits, void* stream) {
  if (!x || !w_router || !idx || !gate) return MK_EINVAL;
  if (T < 1 || T > 64 || P <= 0 || P % 8 || E <= 0 || E > 256 || k < 1 || k > 8 || k > E) return MK_ESHAPE;
  if (!aligned16(x) || !aligned16(w_router)) return MK_EALIGN;
  return mk::launch_route_topk((const uint16_t*)x, (const uint16_t*)w_router, bias, T, P, E, k, idx, gate,
                               logits, (hipStream_t)stream) ? MK_EHIP : MK_OK;
}

int mk_nvfp4_pack(const void* w, int w_is_fp32, int batch, int N, int K, uint8_t* codes, uint8_t* scales,
                  float* tensor_scale, void* stream) {
  if (!w || !codes || !scales || !tensor_scale) return MK_EINVAL;
  if (w_is_fp32 != 0 && w_is_fp32 != 1) return MK_EINVAL;
  if (batch < 1 || batch > 65535 || N < 1 || K < 16 || K % 16) return MK_ESHAPE;
  if (!aligned16(w) || !aligned16(codes) || !aligned16(scales) || !aligned16(tensor_scale)) return MK_EALIGN;
  return mk::launch_nvfp4_pack(w, w_is_fp32, batch, N, K, codes, scales, tensor_scale, (hipStream_t)stream)
             ? MK_EHIP : MK_OK;
}

int mk_nvfp4_tile_w1(const uint8_t* codes, const uint8_t* scales, int batch, int N, int K, uint8_t* codes_t,
                     uint8_t* scales_t, void* stream) {
  if (!codes || !scales || !codes_t || !scales_t) return MK_EINVAL;
  if (batch < 1 || batch > 65535 || N < 16 || N % 16 || K < 128 || K % 128) return MK_ESHAPE;
  if (!aligned16(codes) || !aligned16(codes_t) || !aligned16(scales_t)) return MK_EALIGN;
  return mk::launch_nvfp4_tile_w1(codes, scales, batch, N, K, codes_t, scales_t, (hipStream_t)stream) ? MK_EHIP
                                                                                                     : MK_OK;
}

size_t mk_nvfp4_w1_scales_bytes(int batch, int N, int K) {
  if (batch < 1 || N < 16 || N % 16 || K < 128 || K % 128) return 0;
  return (size_t)batch * N * mk::g1_scale_row_bytes(K);
}

int mk_stream_read(const void* src, size_t bytes, int n_blocks, uint32_t* sink, void* stream) {
  if (!src || !sink) return MK_EINVAL;
  if (n_blocks < 0 || n_blocks > (1 << 20)) return MK_ESHAPE;
  if (bytes % 16 != 0 || ((uintptr_t)src & 15) != 0 || ((uintptr_t)sink & 3) != 0) return MK_EALIGN;
  if (bytes == 0) return MK_OK;
  if (n_blocks == 0) {
    int cus = 0;
    if (device_cus(&cus) != 0) return MK_EHIP;
    n_blocks = 8 * cus;
  }
  return mk::launch_stream_read(src, bytes, n_blocks, sink, (hipStream_t)stream) == 0 ? MK_OK : MK_EHIP;
}

int mk_read_status(const void* workspace, void* stream) {
  if (!workspace) workspace = scratch_if_set();   // mk_layer_step_noalloc's status
  if (!workspace) return MK_EINVAL;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return MK_EHIP;
  // the status word and workgroup 0's epoch slot, which the last launch left one past its own
  uint32_t st = 0, ep = 0;
  if (hipMemcpy(&st, (const char*)workspace + mk::kStatusOffset, 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(&ep, (const char*)workspace + mk::kEpochOffset, 4, hipMemcpyDeviceToHost) != hipSuccess)
    return MK_EHIP;
  return mk::status_is_error_of(st, ep - 1u) ? mk::status_code(st) : MK_OK;
}

}  // extern "C"

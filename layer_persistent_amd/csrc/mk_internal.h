// Internal interface between the C ABI (mk_api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define MK_TS_EVENTS_DEV 64
#define MK_ETIMEOUT_DEV (-6)
#define MK_EBADTREE_DEV (-7)

namespace mk {

// The workspace starts with the status word (offset 0) and the per-workgroup epoch slots
// (offset 256, 64 bytes apart), at these offsets for every configuration.
constexpr size_t kStatusOffset = 0;
constexpr size_t kEpochOffset = 256;

// Status word of a launch: the low 24 bits of the launch's epoch above an 8-bit status code
// (0 = ok).  A code is only acted on (waits abort, mk_read_status reports it) when its epoch
// is the current launch's, so an error never outlives the launch that raised it.
__host__ __device__ inline uint32_t status_word(uint32_t epoch, int code) {
  return ((epoch & 0xFFFFFFu) << 8) | ((uint32_t)code & 0xFFu);
}
__host__ __device__ inline bool status_is_error_of(uint32_t word, uint32_t epoch) {
  return (word & 0xFFu) != 0 && (word >> 8) == (epoch & 0xFFFFFFu);
}
__host__ __device__ inline int status_code(uint32_t word) { return (int)(int8_t)(word & 0xFFu); }

// Stage (hand-off) buffers between the phases of a launch.  There are two copies; a launch
// uses copy (epoch & 1) and, at its start, resets the other one to the sentinel for the next
// launch.  Each buffer sits at a fixed offset inside a copy, sized for the largest supported
// shapes (32 rows -- two sequences of 16 --, Hq*d 1024, H 4096, P 2048, E 256, top-k 8, I 256),
// so that one workspace serves every configuration.  Row-tiled activations hold one 16-row
// MFMA fragment tile per sequence, tile b at b * 16 K elements.  A consumer reads them as they
// arrive: see arrived16().
constexpr int kMaxRowTiles = 2;
constexpr uint32_t kStageAttn = 0;                                         // bf16 [tiles][16][Hq*d], fragment order
constexpr uint32_t kStageH1 = kStageAttn + kMaxRowTiles * 16 * 1024 * 2;   // bf16 [tiles][16][H], fragment order
constexpr uint32_t kStageHf = kStageH1 + kMaxRowTiles * 16 * 4096 * 2;     // bf16 h_out, fragment order
constexpr uint32_t kStageXp = kStageHf + kMaxRowTiles * 16 * 4096 * 2;     // bf16 [tiles][16][P], fragment order
constexpr uint32_t kStageLogits = kStageXp + kMaxRowTiles * 16 * 2048 * 2; // fp32 [rows][E]
constexpr uint32_t kStageAct = kStageLogits + kMaxRowTiles * 16 * 256 * 4; // intermediate records / bf16 rows
constexpr uint32_t kStageY = kStageAct + kMaxRowTiles * 16 * 8 * 256 * 2;  // bf16 [tiles][16][P], fragment order
// the N-sharded layout's GEMM2 products before gates, fp32 [T*k][P/R], P/R <= 1024 (reset with
// the rest of the idle copy by every launch, so that the two layouts may share a workspace)
constexpr uint32_t kStagePart = kStageY + kMaxRowTiles * 16 * 2048 * 2;
// each row's routing, published once by one workgroup: 8 slots of (expert int32, gate fp32),
// slots past top-k zero
constexpr uint32_t kStageRoute = kStagePart + 16 * 8 * 1024 * 4;
constexpr uint32_t kStageBytes = kStageRoute + kMaxRowTiles * 16 * 8 * 8;

// Kernel arguments of one fused layer launch (passed by value).
struct KArgs {
  // shapes
  // T: rows of the launch (every token of every sequence); B sequences of Ts tokens each
  // (B > 1: Ts = 16, sequence b on rows 16 b .. 16 b + 15)
  int H, Hq, Hkv, d, P, E, topk, I, window, fmt, cap, T, ctx, B, Ts;
  // launch geometry
  int n_wg, attn_items, attn_chunks_per_head, attn_lo, ck;
  int attn_rw, attn_nrb;     // row tiles per attention item, row blocks per chunk
  int spin_limit, skip_wg;
  // step inputs / outputs
  const int32_t* parent;
  const uint16_t *q_in, *h_in, *kc, *vc;
  uint16_t *kn, *vn, *h_out, *q_next;
  int32_t* topk_idx;
  float *topk_gate, *router_logits, *attn_stats;
  int32_t* hist;
  const int32_t* prefetch;
  int n_prefetch;
  int32_t* prefetch_next;
  int n_prefetch_next;
  const float* bias;
  // weights
  const uint16_t *w_o, *w_pool, *w_router, *w_unpool, *w_qkv, *w1, *w2;
  const uint8_t *w1_codes, *w1_scales, *w2_codes, *w2_scales;
  const float *w1_ts, *w2_ts;
  // workspace
  uint32_t* status;           // status word (status_word)
  uint32_t *epoch, *flags;
  char* stage;                // stage buffers, copy 0 (copy 1 follows at kStageBytes)
  float *part_o, *part_ml;
  // this launch's copy of the stage buffers (set in the kernel from `stage` and the epoch's
  // parity); the buffers at the kStage* offsets: attn, h1, xp, y hand-off activations ([16][K]
  // bf16 tiles in MFMA fragment order), h_out in fragment order (the qkv phase's x), logits,
  // the NVFP4 intermediate records [T*k][I/16][4 dwords] (codes of elements 0-7, scale byte,
  // codes of elements 8-15, scale byte) or bf16 rows [T*k][I], GEMM2 partials, the routing
  char* cur;
  // N-sharded expert layout (rank ns_r of ns_R; ns_R == 0: the ordinary layout): the gathered
  // intermediate records [T*k][ns_R*I/16][4 dwords], the gathered y (bf16 [16][P], fragment
  // order), and GEMM2's products before gates (stage, [T*k][P/ns_R] fp32)
  int ns_r, ns_R;
  uint32_t* act_recv;
  uint16_t* y_recv;
  float* qkv_part;            // split-K qkv partials [tile][part][64 lanes][4]
  uint32_t* qkv_cnt;          // split-K qkv arrival counters, one per tile, 64 bytes apart
  uint64_t* timestamps;
};

// GEMM1's W1 operand order (NVFP4).  A row of K codes is cut into k-steps of 128 elements
// (64 code bytes, 8 scale bytes); a piece is half of a 16-row tile's k-steps when there are
// more than 8, else all of them.  Codes: [N/16][K/128][64 lanes][16 B], lane l holding row
// 16t + l % 16, code bytes 64 ls + 16 (l / 16) .. + 16.  Scales: [N/16][pieces][16 rows]
// [g1_sb(K) B], the piece's scale bytes of each row, zero past the row's end.
__host__ __device__ inline int g1_lsteps(int K) { return K / 128; }
__host__ __device__ inline int g1_pieces(int K) { return g1_lsteps(K) > 8 ? 2 : 1; }
__host__ __device__ inline int g1_hsteps(int K) { return (g1_lsteps(K) + g1_pieces(K) - 1) / g1_pieces(K); }
__host__ __device__ inline int g1_sb(int K) { return g1_hsteps(K) * 8; }
// scale bytes per W1 row in that order (>= K / 16)
__host__ __device__ inline size_t g1_scale_row_bytes(int K) { return (size_t)g1_pieces(K) * g1_sb(K); }

int launch_layer(const KArgs& a, int lds_bytes, hipStream_t stream);
int layer_lds_bytes();
int set_layer_kernel_attrs(int lds_bytes);

int launch_fill_zero(void* p, size_t bytes, hipStream_t stream);
int launch_stream_read(const void* src, size_t bytes, int n_blocks, uint32_t* sink, hipStream_t stream);
// Fill `bytes` bytes (a multiple of 4) with a 32-bit pattern.
int launch_fill(void* p, size_t bytes, uint32_t pattern, hipStream_t stream);
int launch_kv_append(uint16_t* kc, uint16_t* vc, int row_elems, int pos, const uint16_t* kn,
                     const uint16_t* vn, int n, hipStream_t stream);
int launch_qkv_prologue(const uint16_t* h, const uint16_t* w, int T, int H, int qd, int kd, uint16_t* q_out,
                        uint16_t* kc, uint16_t* vc, int pos, hipStream_t stream);
int launch_tree_accept(const int32_t* parent, const int32_t* draft, const int32_t* target, int T, int32_t* path,
                       int32_t* n_path, int32_t* bonus, hipStream_t stream);
int launch_kv_commit(uint16_t* kc, uint16_t* vc, uint16_t* const* kcs, uint16_t* const* vcs, int n_layers,
                     int row_elems, int ctx, const int32_t* path, const int32_t* n_path, int T, hipStream_t stream);
int launch_route_topk(const uint16_t* x, const uint16_t* w, const float* bias, int T, int P, int E,
                      int k, int32_t* idx, float* gate, float* logits, hipStream_t stream);
int launch_nvfp4_pack(const void* w, int is_fp32, int batch, int N, int K, uint8_t* codes,
                      uint8_t* scales, float* ts, hipStream_t stream);
int launch_nvfp4_tile_w1(const uint8_t* codes, const uint8_t* scales, int batch, int N, int K,
                         uint8_t* codes_t, uint8_t* scales_t, hipStream_t stream);

}  // namespace mk

// Persistent fused decoder-layer kernel for gfx950 (MI355X).
//
// One launch = one decoder layer of the batch-one verify step, from attention of layer L to
// the next layer's q/k/v projection and KV write -- the fusion boundary of the LMSYS / SGLang
// "Muse Spark Open" megakernel (orcarouter.ai write-up, "where the kernel boundary sits").
// The grid is one workgroup per CU (the dynamic LDS request keeps a second one off any CU);
// the workgroups stay resident for the whole layer and hand work between phases through
// device-side flags, the role the pages give to device-side counters (alphasignal.ai, "A
// 12-warp pipeline takes over scheduling").
//
// Phases (each ends in a grid-wide hand-off):
//   ATTN   tree-masked GQA attention over KV chunks -> per-chunk partial (m, l, o)
//   MERGE  merge partials per (token, head) -> attn (bf16), stats (m, l)
//   OPROJ  h1 = bf16(h_in + attn Wo^T)
//   POOL   xp = bf16(h1 Wp^T)
//   ROUTER logits = xp Wr^T (+ bias), fp32
//   GEMM1  every workgroup: top-k, gates and dispatch from the logits (identical everywhere);
//          then (expert, 16-column block) tasks: u = xp W1^T ts1, a = silu(u_gate) u_up,
//          NVFP4 requantisation of a (bf16 for bf16 experts)
//   GEMM2  per 8-column slice of P: every active expert's down projection, then the combine
//          y = bf16(sum over the token's slots, in slot order, of gate * out)
//   UNPOOL h_out = bf16(h1 + y Wu^T)
//   QKV    [q; k; v] = h_out Wqkv^T -> q_next, KV rows of the next layer
//
// Cross-workgroup hand-off: a workgroup writes its outputs with device-coherent stores, waits
// for them to complete, then stores its per-phase flag; consumers poll all flags with
// coherent loads and read the data with ordinary loads.  Hand-off buffers are written once
// per launch, before any workgroup of that launch reads them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_device.h"
#include "mk_internal.h"

namespace mk {

// ------------------------------------------------------------------ sync

struct Sync {
  uint32_t* flags;     // [n_wg] x 16 dwords
  int32_t* status;
  uint32_t base;       // epoch * 64
  int spin_limit;
  int skip_wg;
  bool dead;           // a wait expired or the launch aborted: skip the remaining work
};

// Grid-wide hand-off after `phase` (1-based).  Every thread of every workgroup must call it.
__device__ __noinline__ void grid_sync(Sync& s, int phase) {
  // each thread's coherent stores must be complete before its workgroup signals
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const uint32_t target = s.base + (uint32_t)phase;
  if (threadIdx.x == 0 && (int)blockIdx.x != s.skip_wg) st_coh_u32(s.flags + blockIdx.x * 16, target);
  __shared__ int dead_flag;
  if (threadIdx.x < kWave) {
    bool dead = s.dead;
    int polls = 0;
    while (!dead) {
      bool ok = true;
      for (uint32_t w = threadIdx.x; w < gridDim.x; w += kWave) ok &= (int32_t)(ld_coh_u32(s.flags + w * 16) - target) >= 0;
      if (__all(ok)) break;
      if (++polls >= s.spin_limit) {
        if (threadIdx.x == 0) {
          __hip_atomic_store(s.status, (int32_t)MK_ETIMEOUT_DEV, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        dead = true;
      } else if ((polls & 63) == 0) {
        dead = __hip_atomic_load(s.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
      }
    }
    if (threadIdx.x == 0) dead_flag = dead;
  }
  __syncthreads();
  s.dead = dead_flag;
}

template <bool TS>
__device__ __forceinline__ void stamp(uint64_t* ts, int ev) {
  if constexpr (TS) {
    if (threadIdx.x == 0) ts[blockIdx.x * MK_TS_EVENTS_DEV + ev] = wall_clock64();
  }
}

// ------------------------------------------------------------------ shared layout

struct Route {            // routing tables, identical in every workgroup
  int32_t idx[16 * 8];    // [T][k]
  float gate[16 * 8];
  int32_t n_active;
  int32_t act_expert[128];
  int32_t act_off[128];
  int32_t act_cnt[128];
  int32_t pair_list[128]; // pair id t*k + slot, grouped by expert (ascending), then by pair id
  int32_t expert_cnt[256];
  int32_t expert_first[256];
};

struct Tree {
  uint32_t anc[16];
  int32_t lo[16];         // first visible context row per token
  int32_t bad;
};

constexpr int kRedBytes = 8 * 16 * 17 * 4 * 2;   // two 16x16 fp32 tiles per wave, padded
constexpr int kScratchOff = 0;

// ------------------------------------------------------------------ dense tiles

// Partial tile of C[16][16] = x[rows][K] . W[n0 .. n0+16][K]^T over this wave's k-steps.
// Rows m >= T are zero.  K multiple of 32; the WG's 8 waves take k-steps round-robin.
__device__ __forceinline__ f32x4 dense_partial(const uint16_t* __restrict__ x, int T, int K,
                                               const uint16_t* __restrict__ W, int n0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const uint16_t* wrow = W + (size_t)(n0 + nl) * K + g * 8;
  const uint16_t* xrow = x + (size_t)nl * K + g * 8;
  const bool xv = nl < T;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int ksteps = K >> 5;
  int s = wave;
  for (; s + 24 < ksteps; s += 32) {
    u32x4 b[4], a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = ld16(wrow + (s + 8 * j) * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = xv ? ld16(xrow + (s + 8 * j) * 32) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = mfma_bf16(a[j], b[j], acc);
  }
  for (; s < ksteps; s += 8) {
    u32x4 b = ld16(wrow + s * 32);
    u32x4 a = xv ? ld16(xrow + s * 32) : u32x4{0, 0, 0, 0};
    acc = mfma_bf16(a, b, acc);
  }
  return acc;
}

// Store a wave's partial tile into LDS red[wave][row][col] (row stride 17 floats).
__device__ __forceinline__ void red_store(float* red, f32x4 acc) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  float* p = red + wave * (16 * 17);
#pragma unroll
  for (int r = 0; r < 4; ++r) p[(4 * g + r) * 17 + nl] = acc[r];
}
// Sum over the 8 waves, fixed order.
__device__ __forceinline__ float red_sum(const float* red, int row, int col) {
  float v = 0.f;
#pragma unroll
  for (int w = 0; w < 8; ++w) v += red[w * (16 * 17) + row * 17 + col];
  return v;
}

// out_bf16[t][n0..n0+16) = bf16(residual + x W^T), written with coherent stores (4 columns
// per thread, 8-byte stores).
__device__ void dense_tile_bf16(const uint16_t* x, int T, int K, const uint16_t* W, int N, int n0,
                                const uint16_t* residual, uint16_t* out, bool coherent, float* red) {
  f32x4 acc = dense_partial(x, T, K, W, n0);
  red_store(red, acc);
  __syncthreads();
  if (threadIdx.x < 64) {
    const int row = threadIdx.x >> 2, c0 = (threadIdx.x & 3) * 4;
    if (row < T) {
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = red_sum(red, row, c0 + j);
      if (residual) {
        u32x2 r = *(const u32x2*)(residual + (size_t)row * N + n0 + c0);
        v[0] += bf2f(r[0] & 0xFFFF); v[1] += bf2f(r[0] >> 16);
        v[2] += bf2f(r[1] & 0xFFFF); v[3] += bf2f(r[1] >> 16);
      }
      uint64_t packed = (uint64_t)pack_bf2(v[0], v[1]) | ((uint64_t)pack_bf2(v[2], v[3]) << 32);
      uint16_t* dst = out + (size_t)row * N + n0 + c0;
      if (coherent) st_coh_u64(dst, packed);
      else *(uint64_t*)dst = packed;
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------------ attention

// One work item: kv head `g`, keys [kb, kb + nk) (context rows) or the tree slots.
// Rows are (token, q head of this kv head) pairs, row = t * G + (h - g*G), R = T*G <= 128;
// wave w owns rows [16w, 16w + 16).  S^T = K Q^T puts keys on the MFMA M axis so that the
// probabilities land in exactly the B-operand layout the P.V product needs.
__device__ void attention_item(const KArgs& a, const Tree& tr, int item, char* smem) {
  const int d = a.d, G = a.Hq / a.Hkv, R = a.T * G;
  const int g_kv = item / a.attn_chunks_per_head;
  const int chunk = item % a.attn_chunks_per_head;
  const bool tree_chunk = chunk == a.attn_chunks_per_head - 1;
  const int kb = tree_chunk ? a.ctx : a.attn_lo + chunk * a.ck;
  const int nk = tree_chunk ? a.T : min(a.ck, a.ctx - kb);
  const int CK = 128;                           // LDS chunk capacity
  const int ks_stride = d + 8;                  // bf16 elements per K row in LDS
  const int vt_stride = CK + 8;                 // bf16 elements per V^T row in LDS
  uint16_t* Ks = (uint16_t*)smem;               // [CK][ks_stride]
  uint16_t* VT = Ks + CK * ks_stride;           // [d][vt_stride]

  // stage K (row-major) and V (transposed) for keys kb..kb+nk, zero beyond nk
  const int per_row = d / 8;                    // 16-byte pieces per key row
  for (int i = threadIdx.x; i < CK * per_row; i += blockDim.x) {
    const int key = i / per_row, c = (i % per_row) * 8;
    u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
    if (key < nk) {
      const size_t off = ((size_t)(kb + key) * a.Hkv + g_kv) * d + c;
      kv = ld16(a.kc + off);
      vv = ld16(a.vc + off);
    }
    *(u32x4*)(Ks + key * ks_stride + c) = kv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      VT[(c + 2 * j) * vt_stride + key] = (uint16_t)(vv[j] & 0xFFFF);
      VT[(c + 2 * j + 1) * vt_stride + key] = (uint16_t)(vv[j] >> 16);
    }
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, grp = lane >> 4;
  const int row = wave * 16 + nl;               // this lane's query row (MFMA column)
  if (wave * 16 < R) {
    const bool rv = row < R;
    const int tok = rv ? row / G : 0;
    const int head = g_kv * G + (rv ? row % G : 0);
    const int dsteps = d / 32;
    u32x4 qf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qf[s] = (s < dsteps && rv) ? ld16(a.q_in + (size_t)tok * a.Hq * d + head * d + s * 32 + grp * 8)
                                 : u32x4{0, 0, 0, 0};
    }
    const float scale = 1.0f / sqrtf((float)d);
    const int ktiles = (nk + 15) / 16;
    f32x4 sc[8];
    float mrow = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      sc[kt] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (kt < ktiles) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if (s < dsteps) {
            u32x4 kf = *(const u32x4*)(Ks + (kt * 16 + nl) * ks_stride + s * 32 + grp * 8);
            acc = mfma_bf16(kf, qf[s], acc);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kl = kt * 16 + 4 * grp + r;   // key index within the chunk
          bool vis = rv && kl < nk;
          if (vis) {
            if (tree_chunk) vis = (tr.anc[tok] >> kl) & 1u;
            else vis = kb + kl >= tr.lo[tok];
          }
          sc[kt][r] = vis ? acc[r] * scale : -INFINITY;
          mrow = fmaxf(mrow, sc[kt][r]);
        }
      }
    }
    mrow = xgroup_max(mrow);
    float lsum = 0.f;
    uint32_t pb[8][2];
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = (mrow == -INFINITY || sc[kt][r] == -INFINITY) ? 0.f : __expf(sc[kt][r] - mrow);
        lsum += p[r];
      }
      pb[kt][0] = pack_bf2(p[0], p[1]);
      pb[kt][1] = pack_bf2(p[2], p[3]);
    }
    lsum = xgroup_sum(lsum);
    // O^T[dd][row] = sum_keys V^T[dd][key] P^T[key][row]; a 32-key step pairs key tiles
    // (2q, 2q+1): lane group grp supplies keys 4grp..4grp+3 of both tiles.
    f32x4 o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int dtiles = d / 16;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (2 * q < ktiles) {
        u32x4 bfrag = {pb[2 * q][0], pb[2 * q][1], pb[2 * q + 1][0], pb[2 * q + 1][1]};
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          if (dt < dtiles) {
            const uint16_t* vrow = VT + (dt * 16 + nl) * vt_stride;
            u32x2 v0 = *(const u32x2*)(vrow + (2 * q) * 16 + 4 * grp);
            u32x2 v1 = *(const u32x2*)(vrow + (2 * q + 1) * 16 + 4 * grp);
            u32x4 afrag = {v0[0], v0[1], v1[0], v1[1]};
            o[dt] = mfma_bf16(afrag, bfrag, o[dt]);
          }
        }
      }
    }
    if (rv) {
      float* po = a.part_o + ((size_t)item * 128 + row) * d;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        if (dt < dtiles) {
          u32x4 v = {__float_as_uint(o[dt][0]), __float_as_uint(o[dt][1]), __float_as_uint(o[dt][2]),
                     __float_as_uint(o[dt][3])};
          st_coh_u128(po + dt * 16 + 4 * grp, v);
        }
      }
      if (grp == 0) {
        st_coh_u64(a.part_ml + ((size_t)item * 128 + row) * 2,
                   (uint64_t)__float_as_uint(mrow) | ((uint64_t)__float_as_uint(lsum) << 32));
      }
    }
  }
  __syncthreads();
}

// Merge of the per-chunk partials of one (kv head, row): flash-decoding style rescale.
__device__ void merge_unit(const KArgs& a, int unit, float* scratch) {
  const int d = a.d, G = a.Hq / a.Hkv, R = a.T * G;
  const int g_kv = unit / R, row = unit % R;
  const int tok = row / G, head = g_kv * G + row % G;
  const int nchunks = a.attn_chunks_per_head;
  const int quads = d / 4;                      // threads per chunk-group
  const int ngroups = blockDim.x / 32;          // 16 chunk groups of 32 threads
  const int tq = threadIdx.x % 32, cg = threadIdx.x / 32;
  float M = -INFINITY, L = 0.f, O[4] = {0.f, 0.f, 0.f, 0.f};
  if (tq < quads) {
    for (int c = cg; c < nchunks; c += ngroups) {
      const int item = g_kv * nchunks + c;
      const float* ml = a.part_ml + ((size_t)item * 128 + row) * 2;
      const float m = ml[0], l = ml[1];
      if (l <= 0.f) continue;
      const f32x4 o = *(const f32x4*)(a.part_o + ((size_t)item * 128 + row) * d + tq * 4);
      const float Mn = fmaxf(M, m);
      const float s_old = (M == -INFINITY) ? 0.f : __expf(M - Mn);
      const float s_new = __expf(m - Mn);
      L = L * s_old + l * s_new;
#pragma unroll
      for (int j = 0; j < 4; ++j) O[j] = O[j] * s_old + o[j] * s_new;
      M = Mn;
    }
  }
  float* sm = scratch;                          // [ngroups][32][6]
  float* me = sm + (cg * 32 + tq) * 6;
  me[0] = M; me[1] = L; me[2] = O[0]; me[3] = O[1]; me[4] = O[2]; me[5] = O[3];
  __syncthreads();
  if (threadIdx.x < quads) {
    float Mt = -INFINITY;
    for (int q = 0; q < ngroups; ++q) Mt = fmaxf(Mt, sm[(q * 32 + threadIdx.x) * 6]);
    float Lt = 0.f, Ot[4] = {0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < ngroups; ++q) {
      const float* e = sm + (q * 32 + threadIdx.x) * 6;
      if (e[0] == -INFINITY) continue;
      const float s = __expf(e[0] - Mt);
      Lt += e[1] * s;
#pragma unroll
      for (int j = 0; j < 4; ++j) Ot[j] += e[2 + j] * s;
    }
    const float inv = 1.0f / Lt;
    uint64_t packed = (uint64_t)pack_bf2(Ot[0] * inv, Ot[1] * inv) | ((uint64_t)pack_bf2(Ot[2] * inv, Ot[3] * inv) << 32);
    st_coh_u64(a.attn + (size_t)tok * a.Hq * d + head * d + threadIdx.x * 4, packed);
    if (threadIdx.x == 0 && a.attn_stats) {
      a.attn_stats[((size_t)tok * a.Hq + head) * 2 + 0] = Mt;
      a.attn_stats[((size_t)tok * a.Hq + head) * 2 + 1] = Lt;
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------------ routing

// Top-k per token from the logits (value desc, index asc), softmax gates over the selected,
// and the dispatch tables.  Every workgroup computes the same tables.
__device__ void route_tables(const KArgs& a, Route& rt, float* lg) {
  const int T = a.T, E = a.E, K = a.topk;
  for (int i = threadIdx.x; i < T * E; i += blockDim.x) lg[i] = a.logits[i];
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int t = wave; t < T; t += 8) {
    float v[4];
    int e_[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      e_[q] = lane + 64 * q;
      v[q] = e_[q] < E ? lg[t * E + e_[q]] : -INFINITY;
    }
    bool taken[4] = {e_[0] >= E, e_[1] >= E, e_[2] >= E, e_[3] >= E};
    float zsel[8];
    for (int j = 0; j < K; ++j) {
      // lane-local best
      float bv = -INFINITY; int be = 0x7FFFFFFF;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (!taken[q] && (v[q] > bv || (v[q] == bv && e_[q] < be))) { bv = v[q]; be = e_[q]; }
      // wave argmax, ties to the lower index
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        float ov = __shfl_xor(bv, off);
        int oe = __shfl_xor(be, off);
        if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) if (e_[q] == be) taken[q] = true;
      zsel[j] = bv;
      if (lane == 0) rt.idx[t * K + j] = be;
    }
    if (lane == 0) {
      float s = 0.f, ex[8];
      for (int j = 0; j < K; ++j) { ex[j] = __expf(zsel[j] - zsel[0]); s += ex[j]; }
      for (int j = 0; j < K; ++j) rt.gate[t * K + j] = ex[j] / s;
    }
  }
  __syncthreads();
  const int npairs = T * K;
  // per-expert counts and first-pair ranks
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int c = 0;
    for (int p = 0; p < npairs; ++p) c += rt.idx[p] == e;
    rt.expert_cnt[e] = c;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    // serial-in-wave prefix over experts: lane handles 4 consecutive experts
    int base = 0;
    int n_act = 0;
    for (int chunk = 0; chunk < E; chunk += 256) {
      int cnt[4], act[4];
      int sumc = 0, suma = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = chunk + threadIdx.x * 4 + q;
        cnt[q] = e < E ? rt.expert_cnt[e] : 0;
        act[q] = cnt[q] > 0;
        sumc += cnt[q]; suma += act[q];
      }
      // exclusive scan across the wave
      int sc = sumc, sa = suma;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        int oc = __shfl_up(sc, off), oa = __shfl_up(sa, off);
        if ((int)threadIdx.x >= off) { sc += oc; sa += oa; }
      }
      int pc = base + sc - sumc, pa = n_act + sa - suma;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = chunk + threadIdx.x * 4 + q;
        if (e < E) rt.expert_first[e] = pc;
        if (act[q]) {
          rt.act_expert[pa] = e;
          rt.act_off[pa] = pc;
          rt.act_cnt[pa] = cnt[q];
          ++pa;
        }
        pc += cnt[q];
      }
      base += __shfl(sc, 63);
      n_act += __shfl(sa, 63);
    }
    if (threadIdx.x == 0) rt.n_active = n_act;
  }
  __syncthreads();
  for (int p = threadIdx.x; p < npairs; p += blockDim.x) {
    const int e = rt.idx[p];
    int r = 0;
    for (int q = 0; q < p; ++q) r += rt.idx[q] == e;
    rt.pair_list[rt.expert_first[e] + r] = p;
  }
  __syncthreads();
}

// ------------------------------------------------------------------ experts

// GEMM1 task: expert act slot `ai`, intermediate columns [j0, j0+16).  Each wave covers a
// share of K = P; the partial gate and up tiles are reduced across waves in LDS.
__device__ void gemm1_task(const KArgs& a, const Route& rt, int ai, int j0, float* red, float* abuf) {
  const int e = rt.act_expert[ai], cnt = rt.act_cnt[ai], off = rt.act_off[ai];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, grp = lane >> 4;
  const int P = a.P, I = a.I, K = a.topk;
  const int m = nl;                                   // A-operand row = token slot of this expert
  const bool mv = m < cnt;
  const int tok = mv ? rt.pair_list[off + m] / K : 0;
  const uint16_t* xrow = a.xp + (size_t)tok * P;
  f32x4 accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  if (a.fmt == 1) {
    const size_t rows = 2 * (size_t)I;
    const uint8_t* cg = a.w1_codes + ((size_t)e * rows + j0 + nl) * (P / 2);
    const uint8_t* cu = a.w1_codes + ((size_t)e * rows + I + j0 + nl) * (P / 2);
    const uint8_t* sg = a.w1_scales + ((size_t)e * rows + j0 + nl) * (P / 16);
    const uint8_t* su = a.w1_scales + ((size_t)e * rows + I + j0 + nl) * (P / 16);
    const int lsteps = P / 128;                       // 128 k per load step (16 B per lane)
    for (int ls = wave; ls < lsteps; ls += 8) {
      const u32x4 wg = ld16(cg + ls * 64 + grp * 16);
      const u32x4 wu = ld16(cu + ls * 64 + grp * 16);
      const uint32_t scg = *(const uint16_t*)(sg + ls * 8 + grp * 2);
      const uint32_t scu = *(const uint16_t*)(su + ls * 8 + grp * 2);
      const float sg0 = e4m3_to_f32(scg & 0xFF), sg1 = e4m3_to_f32(scg >> 8);
      const float su0 = e4m3_to_f32(scu & 0xFF), su1 = e4m3_to_f32(scu >> 8);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int k = ls * 128 + grp * 32 + s * 8;
        const u32x4 xa = mv ? ld16(xrow + k) : u32x4{0, 0, 0, 0};
        accg = mfma_bf16(xa, fp4x8_to_bf16(wg[s], s < 2 ? sg0 : sg1), accg);
        accu = mfma_bf16(xa, fp4x8_to_bf16(wu[s], s < 2 ? su0 : su1), accu);
      }
    }
  } else {
    const uint16_t* wgr = a.w1 + ((size_t)e * 2 * I + j0 + nl) * P;
    const uint16_t* wur = a.w1 + ((size_t)e * 2 * I + I + j0 + nl) * P;
    for (int s = wave; s < P / 32; s += 8) {
      const int k = s * 32 + grp * 8;
      const u32x4 xa = mv ? ld16(xrow + k) : u32x4{0, 0, 0, 0};
      accg = mfma_bf16(xa, ld16(wgr + k), accg);
      accu = mfma_bf16(xa, ld16(wur + k), accu);
    }
  }
  float* pg = red + wave * (16 * 17);
  float* pu = red + 8 * 16 * 17 + wave * (16 * 17);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    pg[(4 * grp + r) * 17 + nl] = accg[r];
    pu[(4 * grp + r) * 17 + nl] = accu[r];
  }
  __syncthreads();
  if (threadIdx.x < 256) {
    const int mm = threadIdx.x >> 4, j = threadIdx.x & 15;
    float ug = red_sum(red, mm, j), uu = red_sum(red + 8 * 16 * 17, mm, j);
    if (a.fmt == 1) { ug *= a.w1_ts[e]; uu *= a.w1_ts[e]; }
    const float act = ug / (1.0f + __expf(-ug)) * uu;
    abuf[mm * 17 + j] = act;
  }
  __syncthreads();
  if (threadIdx.x < cnt) {
    const int pair = rt.pair_list[off + threadIdx.x];
    const float* v = abuf + threadIdx.x * 17;
    if (a.fmt == 1) {
      float amax = 0.f;
      for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
      const uint32_t sc = e4m3_code_of_amax_over6(amax);
      const float s = e4m3_to_f32(sc);
      uint32_t w0 = 0, w1 = 0;
      if (s > 0.f) {
        for (int j = 0; j < 8; ++j) w0 |= e2m1_code(v[j], s) << (4 * j);
        for (int j = 0; j < 8; ++j) w1 |= e2m1_code(v[8 + j], s) << (4 * j);
      }
      st_coh_u128(a.act_q + ((size_t)pair * (I / 16) + j0 / 16) * 4, u32x4{w0, w1, sc, 0u});
    } else {
      uint16_t* dst = a.act_bf + (size_t)pair * I + j0;
      for (int q = 0; q < 4; ++q) {
        uint64_t packed = (uint64_t)pack_bf2(v[4 * q], v[4 * q + 1]) | ((uint64_t)pack_bf2(v[4 * q + 2], v[4 * q + 3]) << 32);
        st_coh_u64(dst + 4 * q, packed);
      }
    }
  }
  __syncthreads();
}

// GEMM2 + combine for output columns [c0, c0+8) of P: every active expert's down projection
// for those columns (waves take experts round-robin), then per token the gate-weighted sum
// over its slots in slot order.
__device__ void gemm2_slice(const KArgs& a, const Route& rt, int c0, float* outp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, grp = lane >> 4;
  const int P = a.P, I = a.I, K = a.topk;
  const bool nv = nl < 8;
  for (int ai = wave; ai < rt.n_active; ai += 8) {
    const int e = rt.act_expert[ai], cnt = rt.act_cnt[ai], off = rt.act_off[ai];
    const int m = nl;
    const bool mv = m < cnt;
    const int pair = mv ? rt.pair_list[off + m] : 0;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (a.fmt == 1) {
      const uint8_t* cw = a.w2_codes + ((size_t)e * P + c0 + (nv ? nl : 0)) * (I / 2);
      const uint8_t* sw = a.w2_scales + ((size_t)e * P + c0 + (nv ? nl : 0)) * (I / 16);
      const uint32_t* arec = a.act_q + (size_t)pair * (I / 16) * 4;
      for (int s = 0; s < I / 32; ++s) {
        // k = 32 s + 8 grp .. +8  -> block 2s + grp/2, half grp&1 of the block
        const int blk = 2 * s + (grp >> 1);
        uint32_t wc = nv ? *(const uint32_t*)(cw + 16 * s + 4 * grp) : 0u;
        const float ws = nv ? e4m3_to_f32(sw[blk]) : 0.f;
        uint32_t ac = 0u; float as = 0.f;
        if (mv) {
          ac = arec[blk * 4 + (grp & 1)];
          as = e4m3_to_f32(arec[blk * 4 + 2]);
        }
        acc = mfma_bf16(fp4x8_to_bf16(ac, as), fp4x8_to_bf16(wc, ws), acc);
      }
    } else {
      const uint16_t* wr = a.w2 + ((size_t)e * P + c0 + (nv ? nl : 0)) * I;
      const uint16_t* ar = a.act_bf + (size_t)pair * I;
      for (int s = 0; s < I / 32; ++s) {
        const int k = s * 32 + grp * 8;
        u32x4 b = nv ? ld16(wr + k) : u32x4{0, 0, 0, 0};
        u32x4 x = mv ? ld16(ar + k) : u32x4{0, 0, 0, 0};
        acc = mfma_bf16(x, b, acc);
      }
    }
    const float ts = a.fmt == 1 ? a.w2_ts[e] : 1.0f;
    // C lane: col nl (output column), rows 4 grp + r (token slot of this expert)
    if (nv) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int mm = 4 * grp + r;
        if (mm < cnt) outp[rt.pair_list[off + mm] * 8 + nl] = acc[r] * ts;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < a.T) {
    const int t = threadIdx.x;
    float y[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) y[c] = 0.f;
    for (int j = 0; j < K; ++j) {
      const float gt = rt.gate[t * K + j];
      const float* o = outp + (t * K + j) * 8;
#pragma unroll
      for (int c = 0; c < 8; ++c) y[c] += gt * o[c];
    }
    uint16_t* dst = a.y + (size_t)t * P + c0;
    st_coh_u64(dst, (uint64_t)pack_bf2(y[0], y[1]) | ((uint64_t)pack_bf2(y[2], y[3]) << 32));
    st_coh_u64(dst + 4, (uint64_t)pack_bf2(y[4], y[5]) | ((uint64_t)pack_bf2(y[6], y[7]) << 32));
  }
  __syncthreads();
}

// ------------------------------------------------------------------ kernel

template <bool TS>
__global__ void __launch_bounds__(512) layer_kernel(KArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ Route rt;
  __shared__ Tree tr;
  uint64_t* ts = a.timestamps;
  stamp<TS>(ts, 0);

  Sync s;
  s.flags = a.flags;
  s.status = a.status;
  s.spin_limit = a.spin_limit;
  s.skip_wg = a.skip_wg;
  s.dead = false;
  __shared__ uint32_t epoch_sh;
  if (threadIdx.x == 0) epoch_sh = ld_coh_u32(a.epoch + blockIdx.x * 16);
  // tree: ancestor masks, depths, first visible context row per token
  if (threadIdx.x == 0) {
    int bad = 0;
    int depth[16];
    for (int i = 0; i < a.T; ++i) {
      const int p = a.parent[i];
      if (i == 0) {
        bad |= p != -1;
        tr.anc[0] = 1u;
        depth[0] = 0;
      } else if (p < 0 || p >= i) {
        bad = 1;
        tr.anc[i] = 1u << i;
        depth[i] = 0;
      } else {
        tr.anc[i] = tr.anc[p] | (1u << i);
        depth[i] = depth[p] + 1;
      }
      const int pos = a.ctx + depth[i];
      tr.lo[i] = a.window > 0 ? max(0, pos - a.window + 1) : 0;
    }
    tr.bad = bad;
    if (bad && blockIdx.x == 0)
      __hip_atomic_store(a.status, (int32_t)MK_EBADTREE_DEV, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const uint32_t epoch = epoch_sh;
  s.base = epoch * 64u;
  const int nwg = gridDim.x;
  if (!tr.bad) {
    float* red = (float*)smem;                       // dense reductions
    // ---- ATTN
    for (int it = blockIdx.x; it < a.attn_items; it += nwg) attention_item(a, tr, it, smem);
    stamp<TS>(ts, 1);
    grid_sync(s, 1);
    // ---- MERGE
    if (!s.dead) {
      const int units = a.Hkv * a.T * (a.Hq / a.Hkv);
      for (int u = blockIdx.x; u < units; u += nwg) merge_unit(a, u, (float*)smem);
    }
    stamp<TS>(ts, 2);
    grid_sync(s, 2);
    // ---- OPROJ
    if (!s.dead)
      for (int t = blockIdx.x; t < a.H / 16; t += nwg)
        dense_tile_bf16(a.attn, a.T, a.Hq * a.d, a.w_o, a.H, t * 16, a.h_in, a.h1, true, red);
    stamp<TS>(ts, 3);
    grid_sync(s, 3);
    // ---- POOL
    if (!s.dead)
      for (int t = blockIdx.x; t < a.P / 16; t += nwg)
        dense_tile_bf16(a.h1, a.T, a.H, a.w_pool, a.P, t * 16, nullptr, a.xp, true, red);
    stamp<TS>(ts, 4);
    grid_sync(s, 4);
    // ---- ROUTER
    if (!s.dead) {
      for (int t = blockIdx.x; t < a.E / 16; t += nwg) {
        f32x4 acc = dense_partial(a.xp, a.T, a.P, a.w_router, t * 16);
        red_store(red, acc);
        __syncthreads();
        if (threadIdx.x < 64) {
          const int row = threadIdx.x >> 2, c0 = (threadIdx.x & 3) * 4;
          if (row < a.T) {
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              v[j] = red_sum(red, row, c0 + j);
              if (a.bias) v[j] += a.bias[(size_t)row * a.E + t * 16 + c0 + j];
            }
            float* dst = a.logits + (size_t)row * a.E + t * 16 + c0;
            st_coh_u128(dst, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
            if (a.router_logits) *(f32x4*)(a.router_logits + (size_t)row * a.E + t * 16 + c0) = f32x4{v[0], v[1], v[2], v[3]};
          }
        }
        __syncthreads();
      }
    }
    stamp<TS>(ts, 5);
    grid_sync(s, 5);
    // ---- ROUTE + GEMM1
    if (!s.dead) {
      route_tables(a, rt, (float*)smem);
      if (blockIdx.x == 0) {
        for (int p = threadIdx.x; p < a.T * a.topk; p += blockDim.x) {
          if (a.topk_idx) a.topk_idx[p] = rt.idx[p];
          if (a.topk_gate) a.topk_gate[p] = rt.gate[p];
        }
        if (a.hist)
          for (int e = threadIdx.x; e < a.E; e += blockDim.x) a.hist[e] += rt.expert_cnt[e];
      }
      stamp<TS>(ts, 6);
      const int jblocks = a.I / 16;
      const int ntasks = rt.n_active * jblocks;
      float* abuf = red + 2 * 8 * 16 * 17;
      for (int t = blockIdx.x; t < ntasks; t += nwg) gemm1_task(a, rt, t / jblocks, (t % jblocks) * 16, red, abuf);
    }
    stamp<TS>(ts, 7);
    grid_sync(s, 6);
    // ---- GEMM2 + combine
    if (!s.dead)
      for (int c = blockIdx.x; c < a.P / 8; c += nwg) gemm2_slice(a, rt, c * 8, (float*)smem);
    stamp<TS>(ts, 8);
    grid_sync(s, 7);
    // ---- UNPOOL
    if (!s.dead)
      for (int t = blockIdx.x; t < a.H / 16; t += nwg)
        dense_tile_bf16(a.y, a.T, a.P, a.w_unpool, a.H, t * 16, a.h1, a.h_out, true, red);
    stamp<TS>(ts, 9);
    grid_sync(s, 8);
    // ---- QKV + KV write
    if (!s.dead) {
      const int qd = a.Hq * a.d, kd = a.Hkv * a.d, N = qd + 2 * kd;
      for (int t = blockIdx.x; t < N / 16; t += nwg) {
        const int n0 = t * 16;
        f32x4 acc = dense_partial(a.h_out, a.T, a.H, a.w_qkv, n0);
        red_store(red, acc);
        __syncthreads();
        if (threadIdx.x < 64) {
          const int row = threadIdx.x >> 2, c0 = (threadIdx.x & 3) * 4;
          if (row < a.T) {
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = red_sum(red, row, c0 + j);
            const uint64_t packed = (uint64_t)pack_bf2(v[0], v[1]) | ((uint64_t)pack_bf2(v[2], v[3]) << 32);
            const int n = n0 + c0;
            uint16_t* dst;
            if (n < qd) dst = a.q_next + (size_t)row * qd + n;
            else if (n < qd + kd) dst = a.kn + (size_t)(a.ctx + row) * kd + (n - qd);
            else dst = a.vn + (size_t)(a.ctx + row) * kd + (n - qd - kd);
            *(uint64_t*)dst = packed;
          }
        }
        __syncthreads();
      }
    }
    stamp<TS>(ts, 10);
  }
  // next launch on this workspace uses the next epoch
  if (threadIdx.x == 0) st_coh_u32(a.epoch + blockIdx.x * 16, epoch + 1);
}

template __global__ void layer_kernel<false>(KArgs);
template __global__ void layer_kernel<true>(KArgs);

int launch_layer(const KArgs& a, int lds_bytes, hipStream_t stream) {
  if (a.timestamps) {
    hipLaunchKernelGGL(layer_kernel<true>, dim3(a.n_wg), dim3(512), lds_bytes, stream, a);
  } else {
    hipLaunchKernelGGL(layer_kernel<false>, dim3(a.n_wg), dim3(512), lds_bytes, stream, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int set_layer_kernel_attrs(int lds_bytes) {
  if (hipFuncSetAttribute((const void*)layer_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes) != hipSuccess) return -5;
  if (hipFuncSetAttribute((const void*)layer_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes) != hipSuccess) return -5;
  return 0;
}

}  // namespace mk

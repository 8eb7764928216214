// Small kernels behind the C ABI: workspace fill, KV-cache append, stand-alone router top-k,
// and NVFP4 packing of weight matrices.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_device.h"
#include "mk_internal.h"

namespace mk {

// ------------------------------------------------------------------ fill

// bytes [0, 16 n16) as 16-byte words of `pattern`, then ntail more bytes of it
__global__ void fill_kernel(u32x4* p, size_t n16, uint8_t* tail, size_t ntail, uint32_t pattern) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = u32x4{pattern, pattern, pattern, pattern};
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = (uint8_t)(pattern >> (8 * (threadIdx.x & 3)));
}

int launch_fill(void* p, size_t bytes, uint32_t pattern, hipStream_t stream) {
  const size_t n16 = bytes / 16, ntail = bytes % 16;
  int grid = (int)((n16 + 255) / 256);
  if (grid < 1) grid = 1;
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(fill_kernel, dim3(grid), dim3(256), 0, stream, (u32x4*)p, n16, (uint8_t*)p + n16 * 16,
                     ntail, pattern);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int launch_fill_zero(void* p, size_t bytes, hipStream_t stream) { return launch_fill(p, bytes, 0u, stream); }

// ------------------------------------------------------------------ streaming read

// Reads bytes [0, 16 n16) of src once, 16 bytes per load, U loads in flight per thread: each
// workgroup takes consecutive 256 * 16 * U-byte blocks, one contiguous 16-byte piece per thread
// and load (coalesced).  The XOR of every 32-bit word read is folded per wave and XORed into
// sink[0] by one atomic per wave: a checksum that keeps the loads alive and lets a test see
// that every piece was read exactly once.
template <int U>
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4* __restrict__ src, size_t n16, uint32_t* sink) {
  constexpr size_t kBlock = (size_t)256 * U;
  uint32_t acc = 0;
  for (size_t b = (size_t)blockIdx.x * kBlock; b < n16; b += (size_t)gridDim.x * kBlock) {
    u32x4 v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const size_t i = b + (size_t)j * 256 + threadIdx.x;
      v[j] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < U; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m);
  if ((threadIdx.x & 63) == 0 && acc != 0) atomicXor(sink, acc);
}

int launch_stream_read(const void* src, size_t bytes, int n_blocks, uint32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel<8>, dim3(n_blocks), dim3(256), 0, stream, (const u32x4*)src, bytes / 16,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// ------------------------------------------------------------------ KV append

// rows pos..pos+n-1 of both caches <- k_new / v_new; row_elems = n_kv_heads * head_dim (bf16)
__global__ void kv_append_kernel(uint16_t* kc, uint16_t* vc, int row_elems, int pos, const uint16_t* kn,
                                 const uint16_t* vn, int n) {
  const int per_row = row_elems / 8;  // 16-byte pieces
  const int total = n * per_row;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
    const int r = i / per_row, c = (i % per_row) * 8;
    *(u32x4*)(kc + (size_t)(pos + r) * row_elems + c) = *(const u32x4*)(kn + (size_t)r * row_elems + c);
    *(u32x4*)(vc + (size_t)(pos + r) * row_elems + c) = *(const u32x4*)(vn + (size_t)r * row_elems + c);
  }
}

int launch_kv_append(uint16_t* kc, uint16_t* vc, int row_elems, int pos, const uint16_t* kn,
                     const uint16_t* vn, int n, hipStream_t stream) {
  const int total = n * (row_elems / 8);
  int grid = (total + 255) / 256;
  if (grid < 1) grid = 1;
  if (grid > 1024) grid = 1024;
  hipLaunchKernelGGL(kv_append_kernel, dim3(grid), dim3(256), 0, stream, kc, vc, row_elems, pos, kn, vn, n);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// ------------------------------------------------------------------ first-layer prologue

// [q; k; v] = h W^T for the step's T <= 16 tokens: h bf16 [T][H] (the tokens' embeddings),
// W bf16 [N][H] with N = qd + 2 kd (layer 0's query, key and value projections stacked); q
// goes to q_out [T][qd], k and v to the cache rows pos..pos+T-1 ([capacity][kd]).  One
// workgroup of 16 waves per 16 output columns: the 16 token rows are one MFMA tile, wave w
// takes the 32-element k-steps w, w+16, ..., eight of them loaded together, and the 16 partial
// tiles are summed in LDS in wave order before the single bf16 rounding.  Rows past T are zero.
constexpr int kPrologueWaves = 16;
__global__ void __launch_bounds__(64 * kPrologueWaves) qkv_prologue_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ w, int T, int H, int qd, int kd,
    uint16_t* __restrict__ q_out, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, int pos) {
  __shared__ float red[kPrologueWaves][16][17];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nl = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16, ksteps = H / 32;
  const bool xv = nl < T;
  const uint16_t* xrow = h + (size_t)(xv ? nl : 0) * H + 8 * g;
  const uint16_t* wrow = w + (size_t)(n0 + nl) * H + 8 * g;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = wave; s0 < ksteps; s0 += 8 * kPrologueWaves) {
    u32x4 xa[8], wb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int s = s0 + kPrologueWaves * j;
      const bool ok = s < ksteps;
      xa[j] = (ok && xv) ? *(const u32x4*)(xrow + 32 * s) : u32x4{0, 0, 0, 0};
      wb[j] = ok ? *(const u32x4*)(wrow + 32 * s) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + kPrologueWaves * j < ksteps) acc = mfma_bf16(xa[j], wb[j], acc);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][4 * g + r][nl] = acc[r];
  __syncthreads();
  if (threadIdx.x < 256) {
    const int t = threadIdx.x >> 4, c = threadIdx.x & 15;
    if (t < T) {
      float v = 0.f;
#pragma unroll
      for (int q = 0; q < kPrologueWaves; ++q) v += red[q][t][c];
      const uint16_t b = (uint16_t)f2bf(v);
      const int n = n0 + c;
      if (n < qd) q_out[(size_t)t * qd + n] = b;
      else if (n < qd + kd) kc[(size_t)(pos + t) * kd + (n - qd)] = b;
      else vc[(size_t)(pos + t) * kd + (n - qd - kd)] = b;
    }
  }
}

int launch_qkv_prologue(const uint16_t* h, const uint16_t* w, int T, int H, int qd, int kd, uint16_t* q_out,
                        uint16_t* kc, uint16_t* vc, int pos, hipStream_t stream) {
  hipLaunchKernelGGL(qkv_prologue_kernel, dim3((qd + 2 * kd) / 16), dim3(64 * kPrologueWaves), 0, stream, h, w, T,
                     H, qd, kd,
                     q_out, kc, vc, pos);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// ------------------------------------------------------------------ acceptance and KV commit

// Greedy acceptance along the verified tree, one wave: lane i holds node i's parent, drafted
// token and target token.  From the root, each round takes the lowest-index child of the
// current node whose drafted token equals the target token at the current node (a ballot);
// the walk stops when none does.  path[0..n) = accepted nodes root-first, the rest -1;
// bonus = the target token at the last accepted node.  A malformed tree accepts nothing
// (n = 0, bonus = -1).
__global__ void __launch_bounds__(64) tree_accept_kernel(const int32_t* __restrict__ parent,
                                                         const int32_t* __restrict__ draft,
                                                         const int32_t* __restrict__ target, int T,
                                                         int32_t* __restrict__ path, int32_t* __restrict__ n_path,
                                                         int32_t* __restrict__ bonus) {
  const int lane = threadIdx.x;
  const bool in = lane < T;
  const int32_t p = in ? parent[lane] : -2;
  const int32_t dr = in ? draft[lane] : 0;
  const int32_t tg = in ? target[lane] : 0;
  const bool ok = !in || (lane == 0 ? p == -1 : (p >= 0 && p < lane));
  const bool bad = __ballot(!ok) != 0;
  int cur = 0, n = 1;
  int32_t mine = lane == 0 ? 0 : -1;             // lane j keeps path[j]
  if (!bad) {
    for (int r = 1; r < T; ++r) {
      const int32_t want = __shfl(tg, cur);
      const uint64_t hit = __ballot(in && lane > 0 && p == cur && dr == want);
      if (hit == 0) break;
      cur = __ffsll((unsigned long long)hit) - 1;
      mine = lane == n ? cur : mine;
      ++n;
    }
  }
  const int32_t last = __shfl(tg, cur);           // every lane takes part in the shuffle
  if (in) path[lane] = bad ? -1 : mine;
  if (lane == 0) {
    *n_path = bad ? 0 : n;
    *bonus = bad ? -1 : last;
  }
}

// KV commit of an accepted path in one layer's cache pair: row ctx + path[j] -> row ctx + j for
// j < n (n read on the device).  Every source row is read into LDS before any row is written,
// so the moves may overlap.  One workgroup; rows are row_elems bf16 (a multiple of 8).
// Workgroup y commits layer y of n_layers: its cache pair is kcs[y], vcs[y] when the pointer
// arrays are given (device memory), else kc, vc.
__global__ void __launch_bounds__(256) kv_commit_kernel(uint16_t* __restrict__ kc, uint16_t* __restrict__ vc,
                                                        uint16_t* const* __restrict__ kcs,
                                                        uint16_t* const* __restrict__ vcs,
                                                        int row_elems, int ctx, const int32_t* __restrict__ path,
                                                        const int32_t* __restrict__ n_path, int T) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  if (kcs) {
    kc = kcs[blockIdx.x];
    vc = vcs[blockIdx.x];
  }
  u32x4* buf = (u32x4*)lds;                       // [2][T][row_elems / 8]
  const int n = min(max(*n_path, 0), T);
  const int per = row_elems / 8, total = n * per;
  // a path entry outside [0, T) (not one mk_tree_accept writes) moves nothing
  for (int i = threadIdx.x; i < total; i += blockDim.x) {
    const int j = i / per, c = i % per, pj = path[j];
    if (pj < 0 || pj >= T) continue;
    const size_t src = (size_t)(ctx + pj) * row_elems + 8 * c;
    buf[i] = *(const u32x4*)(kc + src);
    buf[T * per + i] = *(const u32x4*)(vc + src);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < total; i += blockDim.x) {
    const int j = i / per, c = i % per, pj = path[j];
    if (pj < 0 || pj >= T) continue;
    const size_t dst = (size_t)(ctx + j) * row_elems + 8 * c;
    *(u32x4*)(kc + dst) = buf[i];
    *(u32x4*)(vc + dst) = buf[T * per + i];
  }
}

int launch_tree_accept(const int32_t* parent, const int32_t* draft, const int32_t* target, int T, int32_t* path,
                       int32_t* n_path, int32_t* bonus, hipStream_t stream) {
  hipLaunchKernelGGL(tree_accept_kernel, dim3(1), dim3(64), 0, stream, parent, draft, target, T, path, n_path, bonus);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int launch_kv_commit(uint16_t* kc, uint16_t* vc, uint16_t* const* kcs, uint16_t* const* vcs, int n_layers,
                     int row_elems, int ctx, const int32_t* path, const int32_t* n_path, int T, hipStream_t stream) {
  const size_t lds = (size_t)2 * T * row_elems * 2;
  hipLaunchKernelGGL(kv_commit_kernel, dim3(n_layers), dim3(256), lds, stream, kc, vc, kcs, vcs, row_elems, ctx, path,
                     n_path, T);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// ------------------------------------------------------------------ router top-k

// One workgroup (256 threads) per token: fp32 logits by per-expert dot products, then the
// top-k by (value desc, index asc) in wave 0, softmax gates over the selected logits.
__global__ void __launch_bounds__(256) route_topk_kernel(const uint16_t* x, const uint16_t* w,
                                                         const float* bias, int P, int E, int k,
                                                         int32_t* idx, float* gate, float* logits) {
  __shared__ float lg[256];
  const int t = blockIdx.x;
  const uint16_t* xr = x + (size_t)t * P;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const uint16_t* wr = w + (size_t)e * P;
    float acc = 0.f;
    for (int c = 0; c < P; c += 8) {
      const u32x4 xv = *(const u32x4*)(xr + c), wv = *(const u32x4*)(wr + c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc = fmaf(bf2f(xv[j] & 0xFFFF), bf2f(wv[j] & 0xFFFF), acc);
        acc = fmaf(bf2f(xv[j] >> 16), bf2f(wv[j] >> 16), acc);
      }
    }
    if (bias) acc += bias[(size_t)t * E + e];
    lg[e] = acc;
    if (logits) logits[(size_t)t * E + e] = acc;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    float v[4];
    int ee[4];
    bool taken[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ee[q] = lane + 64 * q;
      taken[q] = ee[q] >= E;
      v[q] = taken[q] ? -INFINITY : lg[ee[q]];
    }
    float zsel[8];
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int be = 0x7FFFFFFF;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (!taken[q] && (v[q] > bv || (v[q] == bv && ee[q] < be))) { bv = v[q]; be = ee[q]; }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oe = __shfl_xor(be, off);
        if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) if (ee[q] == be) taken[q] = true;
      zsel[j] = bv;
      if (lane == 0) idx[(size_t)t * k + j] = be;
    }
    if (lane == 0) {
      float s = 0.f, ex[8];
      for (int j = 0; j < k; ++j) { ex[j] = __expf(zsel[j] - zsel[0]); s += ex[j]; }
      for (int j = 0; j < k; ++j) gate[(size_t)t * k + j] = ex[j] / s;
    }
  }
}

int launch_route_topk(const uint16_t* x, const uint16_t* w, const float* bias, int T, int P, int E,
                      int k, int32_t* idx, float* gate, float* logits, hipStream_t stream) {
  hipLaunchKernelGGL(route_topk_kernel, dim3(T), dim3(256), 0, stream, x, w, bias, P, E, k, idx, gate, logits);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// ------------------------------------------------------------------ NVFP4 packing

__device__ __forceinline__ float load_w(const void* w, int is_fp32, size_t i) {
  return is_fp32 ? ((const float*)w)[i] : bf2f(((const uint16_t*)w)[i]);
}

// pass 1: amax of each matrix, as the bit pattern of a non-negative float (monotone as uint)
__global__ void amax_kernel(const void* w, int is_fp32, size_t per_mat, uint32_t* amax_bits) {
  const int b = blockIdx.y;
  float m = 0.f;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < per_mat; i += (size_t)gridDim.x * blockDim.x)
    m = fmaxf(m, fabsf(load_w(w, is_fp32, (size_t)b * per_mat + i)));
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) atomicMax(amax_bits + b, __float_as_uint(m));
}

// pass 2: ts = fp32(amax) / 2688 (correctly rounded fp32 division), 1 when amax = 0
__global__ void tscale_kernel(float* ts, int batch) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch) {
    const float amax = __uint_as_float(((const uint32_t*)ts)[b]);
    ts[b] = amax > 0.f ? amax / 2688.0f : 1.0f;
  }
}

// E4M3 byte -> value in fp64 (non-negative codes 0..126)
__device__ __forceinline__ double e4m3_pos_f64(int c) {
  const int E = c >> 3, M = c & 7;
  return E == 0 ? (double)M * 0x1p-9 : (1.0 + M / 8.0) * ldexp(1.0, E - 7);
}

// pass 3: one thread per 16-element block.  Scale and code decisions are exact fp64
// comparisons of the input with midpoint * 6 * ts and midpoint * s * ts (<= 31 significant bits).
__global__ void pack_kernel(const void* w, int is_fp32, int N, int K, int batch, const float* ts,
                            uint8_t* codes, uint8_t* scales) {
  const size_t nblk_row = K / 16;
  const size_t nblocks = (size_t)batch * N * nblk_row;
  for (size_t blk = (size_t)blockIdx.x * blockDim.x + threadIdx.x; blk < nblocks;
       blk += (size_t)gridDim.x * blockDim.x) {
    const size_t b = blk / ((size_t)N * nblk_row);
    const double t = (double)ts[b];
    float x[16];
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      x[j] = load_w(w, is_fp32, blk * 16 + j);
      amax = fmaxf(amax, fabsf(x[j]));
    }
    // scale: number of midpoints passed, ties to the even code
    int lo = 0, hi = 126;
    while (lo < hi) {
      const int c = (lo + hi) >> 1;
      const double thr = 6.0 * t * (0.5 * (e4m3_pos_f64(c) + e4m3_pos_f64(c + 1)));
      const bool passed = (double)amax > thr || ((double)amax == thr && (c & 1));
      if (passed) lo = c + 1; else hi = c;
    }
    const int sc = lo;
    const double unit = e4m3_pos_f64(sc) * t;
    uint32_t w0 = 0, w1 = 0;
    if (unit > 0.0) {
      const double mids[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const double ax = fabs((double)x[j]);
        uint32_t c = 0;
#pragma unroll
        for (int i = 0; i < 7; ++i) {
          const double thr = mids[i] * unit;
          c += (ax > thr || (ax == thr && (i & 1))) ? 1u : 0u;
        }
        if (x[j] < 0.f && c) c |= 8u;
        if (j < 8) w0 |= c << (4 * j); else w1 |= c << (4 * (j - 8));
      }
    }
    *(u32x2*)(codes + blk * 8) = u32x2{w0, w1};
    scales[blk] = (uint8_t)sc;
  }
}

int launch_nvfp4_pack(const void* w, int is_fp32, int batch, int N, int K, uint8_t* codes,
                      uint8_t* scales, float* ts, hipStream_t stream) {
  if (launch_fill_zero(ts, (size_t)batch * 4, stream)) return -5;
  const size_t per_mat = (size_t)N * K;
  int gx = (int)((per_mat + 255) / 256);
  if (gx > 256) gx = 256;
  if (gx < 1) gx = 1;
  hipLaunchKernelGGL(amax_kernel, dim3(gx, batch), dim3(256), 0, stream, w, is_fp32, per_mat, (uint32_t*)ts);
  if (hipGetLastError() != hipSuccess) return -5;
  hipLaunchKernelGGL(tscale_kernel, dim3((batch + 255) / 256), dim3(256), 0, stream, ts, batch);
  if (hipGetLastError() != hipSuccess) return -5;
  const size_t nblocks = (size_t)batch * N * (K / 16);
  size_t g = (nblocks + 255) / 256;
  if (g > 65536) g = 65536;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)g), dim3(256), 0, stream, w, is_fp32, N, K, batch, ts, codes, scales);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// W1 codes and scales from row-major into GEMM1's operand order (g1_* in mk_internal.h): one
// thread per 16-byte chunk of tiled codes, then one per (tile, piece, row) of tiled scales.
__global__ void tile_w1_codes_kernel(const uint8_t* codes, int N, int K, size_t nchunks, uint8_t* codes_t) {
  const int ls_n = g1_lsteps(K);
  for (size_t o = (size_t)blockIdx.x * blockDim.x + threadIdx.x; o < nchunks; o += (size_t)gridDim.x * blockDim.x) {
    const int l = (int)(o % 64);
    const size_t tl = o / 64;                   // (matrix, tile, k-step)
    const int ls = (int)(tl % ls_n);
    const size_t row = (tl / ls_n) * 16 + (l & 15);   // row over the whole batch (N % 16 == 0)
    const u32x4 v = *(const u32x4*)(codes + row * (K / 2) + ls * 64 + (l >> 4) * 16);
    *(u32x4*)(codes_t + o * 16) = v;
  }
}
__global__ void tile_w1_scales_kernel(const uint8_t* scales, int N, int K, size_t nrows, uint8_t* scales_t) {
  const int np = g1_pieces(K), sb = g1_sb(K), rb = K / 16;
  for (size_t o = (size_t)blockIdx.x * blockDim.x + threadIdx.x; o < nrows; o += (size_t)gridDim.x * blockDim.x) {
    const int r = (int)(o % 16);
    const size_t tp = o / 16;                   // (matrix, tile, piece)
    const int p = (int)(tp % np);
    const size_t row = (tp / np) * 16 + r;
    uint8_t* dst = scales_t + o * sb;
    for (int i = 0; i < sb; ++i) {
      const int c = p * sb + i;
      dst[i] = c < rb ? scales[row * rb + c] : (uint8_t)0;
    }
  }
}

int launch_nvfp4_tile_w1(const uint8_t* codes, const uint8_t* scales, int batch, int N, int K,
                         uint8_t* codes_t, uint8_t* scales_t, hipStream_t stream) {
  const size_t nchunks = (size_t)batch * N * (K / 2) / 16;
  size_t g = (nchunks + 255) / 256;
  if (g > 65536) g = 65536;
  hipLaunchKernelGGL(tile_w1_codes_kernel, dim3((unsigned)g), dim3(256), 0, stream, codes, N, K, nchunks, codes_t);
  if (hipGetLastError() != hipSuccess) return -5;
  const size_t nrows = (size_t)batch * N * g1_pieces(K);
  g = (nrows + 255) / 256;
  if (g > 65536) g = 65536;
  hipLaunchKernelGGL(tile_w1_scales_kernel, dim3((unsigned)g), dim3(256), 0, stream, scales, N, K, nrows, scales_t);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace mk

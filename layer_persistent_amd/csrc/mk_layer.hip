// Persistent fused decoder-layer kernel for gfx950 (MI355X).
//
// One launch = one decoder layer of the batch-one verify step, from attention of layer L to
// the next layer's q/k/v projection and KV write -- the fusion boundary of the LMSYS / SGLang
// "Muse Spark Open" megakernel (orcarouter.ai write-up, "where the kernel boundary sits").
// The grid is one workgroup per CU (the dynamic LDS request keeps a second one off any CU);
// the workgroups stay resident for the whole layer and hand work between phases through
// device-side flags or through the data itself, the role the pages give to device-side
// counters (alphasignal.ai, "A 12-warp pipeline takes over scheduling").
//
// Workgroup = 9 waves.  Waves 0..7 compute (MFMA, attention, routing, experts).  Wave 8 is
// the control wave: it stores each dense phase's output tile, signals this workgroup's flag
// and polls everyone else's at a grid hand-off.  Because compute waves never wait for their
// own global stores at a hand-off, the weight loads they issue for a later phase stay in
// flight across the grid-wide wait -- the pages' "weights do not depend on the previous output, so fetch the
// next operation's weights while the current one runs" (alphasignal.ai, "Four mechanisms
// keep work moving"), with the register file as the staging buffer.
//
// Phases (G: a grid-wide hand-off follows; D: the next phase reads the output as it arrives):
//   1 ATTN   tree-masked GQA attention over KV chunks -> per-chunk partial (m, l, o)      G
//   2 MERGE  merge partials per (token, head) -> attn (bf16), stats (m, l)              D
//   3 OPROJ  h1 = bf16(h_in + attn Wo^T)                                                 G
//   4 POOL   xp = bf16(h1 Wp^T)                                                          G
//   5 ROUTER logits = xp Wr^T (+ bias), fp32; the control wave of workgroup t reads row t as
//            it arrives and publishes its top-k experts and gates                        D
//   6 GEMM1  every workgroup: dispatch tables from the published routing (identical
//            everywhere); then (expert, 16-column block) tasks: u = xp W1^T ts1,
//            a = silu(u_gate) u_up, NVFP4 requantisation of a (bf16 for bf16 experts)    D
//   7 GEMM2  per 8-column slice of P: every active expert's down projection, then the combine
//            y = bf16(sum over the token's slots, in slot order, of gate * out)          G
//   8 UNPOOL h_out = bf16(h1 + y Wu^T)                                                   D
//     QKV    [q; k; v] = h_out Wqkv^T -> q_next, KV rows of the next layer (K split over up to
//            4 workgroups per tile; the last part to arrive adds the partials)
//
// Cross-workgroup hand-off, G: data is written with device-coherent (write-through) stores; the
// writer waits for them, then stores its per-phase flag; readers poll all flags with coherent
// loads and then read the data with ordinary loads.  D: the stage buffer holds all ones until
// written (no written 8-byte word ever does), and readers take 16-byte pieces with
// device-coherent loads as they arrive (arrived16).  Large broadcasts that every workgroup
// reads in full go by G, small ones by D.  Each hand-off buffer is written once per launch
// before any workgroup of the launch first reads it, so no cache can hold a stale copy.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_device.h"
#include "mk_internal.h"

namespace mk {


constexpr int kThreads = 576;      // 8 compute waves + 1 control wave
constexpr int kCompute = 512;
constexpr int kCtl = 512;          // first thread of the control wave
// The merge (one unit per (token, head) row) leaves about half the workgroups without work, and
// those skip the attention hand-off; they sleep this long before their first poll of the merged
// rows, so that their polls do not load the memory side while the merge runs (measured: 2 us
// beats 1 by ~0.1 us per layer; 4 or 5 us cost 0.3 and 1.0 us).  The pooler's idle workgroups
// sleep longer (see its hand-off).
constexpr int kIdleSleepUs = 2;
// Polls of stage data that has not arrived are repeated back to back, or after s_sleep
// MK_POLL_SLEEP (64-clock units)
#ifndef MK_POLL_SLEEP
#define MK_POLL_SLEEP 0
#endif
// workgroups without a router tile wait about MK_ROUTE_IDLE us before reading the routing
#ifndef MK_ROUTE_IDLE
#define MK_ROUTE_IDLE 0
#endif

// per-wave MFMA k-steps (32 k each) held in registers for each dense phase
constexpr int MAXS_O = 4;          // o-proj   K = Hq*d <= 1024
constexpr int MAXS_P = 16;         // pooler   K = H    <= 4096
constexpr int MAXS_R = 8;          // router   K = P    <= 2048
constexpr int MAXS_U = 8;          // unpooler K = P    <= 2048
constexpr int MAXS_Q = 16;         // qkv      K = H    <= 4096
// dynamic LDS layout (byte offsets; phases reuse the same space)
constexpr int XS_STRIDE_PAD = 8;                       // bf16 elements of padding per xp row
constexpr int G1_XS_BYTES = 32 * (1024 + 8) * 2;       // xp rows for GEMM1: 16 x (2048 + 8) or 32 x (1024 + 8)
constexpr int LDS_BYTES = 148 * 1024;                  // >= every phase's use (GEMM1: 136.5 KB)
// A pooler tile (16 x K <= 4096 bf16 = 128 KB) held in LDS from launch start, above the 17 KB of
// dense-phase reduction buffers and the merge scratch
constexpr int POOL_LDS_OFF = 20 * 1024;
static_assert(POOL_LDS_OFF + 16 * 4096 * 2 <= LDS_BYTES, "pooler tile in LDS");
// An unpooler tile (16 x P <= 2048 bf16 = 64 KB), filled during GEMM2 above GEMM2's own LDS use
constexpr int WU_LDS_OFF = 64 * 1024;
static_assert(WU_LDS_OFF + 16 * 2048 * 2 <= LDS_BYTES, "unpooler tile in LDS");
static_assert(G1_XS_BYTES + 16 * 16 * 128 + 2 * 16 * 16 * 17 * 4 <= LDS_BYTES, "GEMM1 LDS");

// This launch's stage buffers (copy `a.cur`), computed where they are used rather than held:
// nine pointers kept live through the launch would crowd the scalar registers.
__device__ __forceinline__ uint16_t* st_attn(const KArgs& a) { return (uint16_t*)(a.cur + kStageAttn); }
__device__ __forceinline__ uint16_t* st_h1(const KArgs& a) { return (uint16_t*)(a.cur + kStageH1); }
__device__ __forceinline__ uint16_t* st_h_frag(const KArgs& a) { return (uint16_t*)(a.cur + kStageHf); }
__device__ __forceinline__ uint16_t* st_xp(const KArgs& a) { return (uint16_t*)(a.cur + kStageXp); }
__device__ __forceinline__ float* st_logits(const KArgs& a) { return (float*)(a.cur + kStageLogits); }
__device__ __forceinline__ uint32_t* st_act_q(const KArgs& a) { return (uint32_t*)(a.cur + kStageAct); }
__device__ __forceinline__ uint16_t* st_act_bf(const KArgs& a) { return (uint16_t*)(a.cur + kStageAct); }
__device__ __forceinline__ uint16_t* st_y(const KArgs& a) { return (uint16_t*)(a.cur + kStageY); }
__device__ __forceinline__ float* st_g2_part(const KArgs& a) { return (float*)(a.cur + kStagePart); }
__device__ __forceinline__ uint64_t* st_route(const KArgs& a) { return (uint64_t*)(a.cur + kStageRoute); }

__device__ __forceinline__ void wg_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Timestamp event `ev` of this workgroup, written by thread `who` (timing build only).
// Events: 0 start, 1 setup done, 2p work of phase p done, 2p+1 its hand-off done (p = 1..8),
// 18 routing tables built, 19 end, 20+p control wave's wait for phase p done, 28+p compute
// waves' loads for a later phase issued, 37 / 38 first attention item staged / computed,
// 39 / 40 its key loop done / key groups' partials in LDS, 42 / 43 / 48 GEMM2 intermediate
// staged / experts done / first register batch done, 44 / 45 GEMM1 input rows built / first
// round multiplied, 46 / 47 routing logits staged / top-k done, 49 / 50 GEMM1 first pieces
// requested / row scales known, 53+p control wave's hand-off stores of phase p complete.
// Events are recorded in LDS and written out once at the end of the launch, so that the
// timing build issues no global stores (and waits for none) while the phases run.
__shared__ uint64_t ts_lds[MK_TS_EVENTS_DEV];
template <bool TS>
__device__ __forceinline__ void stamp(uint64_t* ts, int ev, int who = kCtl) {
  if constexpr (TS) {
    if ((int)threadIdx.x == who) ts_lds[ev] = wall_clock64();
  }
}

// ------------------------------------------------------------------ shared state

// Routing tables, identical in every workgroup, for up to NRT * 16 rows of k <= 8 pairs (16-bit
// entries keep the two-sequence tables within the LDS budget).
template <int NRT>
struct RouteT {
  static constexpr int kPairs = NRT * 16 * 8;
  int16_t idx[kPairs];    // [rows][k]
  float gate[kPairs];
  // GEMM1 entries: the active experts in ascending order, an expert with more than 16 pairs as
  // several entries of <= 16 (one 16-row MFMA tile each)
  int32_t n_active;
  int16_t act_expert[256 + kPairs / 17];
  int16_t act_off[256 + kPairs / 17];
  int16_t act_cnt[256 + kPairs / 17];
  int16_t pair_list[kPairs];  // pair id row*k + slot, grouped by expert (ascending), then by pair id
  float ts1[256], ts2[256];  // NVFP4 tensor scales of every expert (W1, W2)
  // GEMM2 slots: each GEMM1 entry's first (up to) 8 pairs, then the rest of every entry with
  // more than 8 pairs; a slot holds at most 8 pairs
  int32_t n_slots;
  int16_t slot_expert[kPairs];
  int16_t slot_off[kPairs];  // into pair_list
  int16_t slot_cnt[kPairs];
};

struct Tree {              // per row (sequence b's tokens on rows b Ts ..; ancestors within it)
  uint32_t anc[32];
  int32_t lo[32];         // first visible context row per token
  int32_t bad;
};

struct Ctl {              // control-wave state shared through LDS
  int32_t dead;           // a wait expired or the launch aborted
};

// ------------------------------------------------------------------ grid hand-off

struct Sync {
  uint32_t* flags;        // per-workgroup flags of the grid hand-off (see ctl_signal_wait)
  uint32_t* status;       // status word (status_word: epoch-tagged code)
  uint32_t epoch;         // this launch's epoch
  uint32_t base;          // epoch * 64
  int spin_limit;
  int skip_wg;
};

// Control wave only: signal this workgroup's flag for `phase`, then wait until every
// workgroup's flag has reached it.  Two polls (of every flag) stay in flight, back to back with
// no sleep between them (sleeping after a few polls measured 0.35 us slower per layer), so that
// a flag landing is seen about half a round trip later.  `idle_us` (about 1 us each) delays the
// first poll of a workgroup that had no work in a phase where the others work for ~2 us: its polls
// of the flags would only add memory traffic while they work.  A workgroup that does not read
// the phase's output (`wait` false) raises its flag and goes on: flags only grow, so the next
// wait it takes part in still covers it, and the others poll against less traffic.  Returns
// false when the wait expired or the launch was aborted (this launch's error code in the
// status word).
__device__ __forceinline__ bool ctl_signal_wait(const Sync& s, int phase, bool dead, int idle_us = 0,
                                                bool wait = true) {
  const int lane = threadIdx.x & 63;
  const int n = gridDim.x;
  __builtin_amdgcn_s_waitcnt(0);           // this wave's hand-off stores are complete
  // One flag per workgroup, 64 bytes apart; a poll reads all of them (4 loads per lane).
  const uint32_t target = s.base + (uint32_t)phase;
  if (lane == 0 && (int)blockIdx.x != s.skip_wg) st_coh_u32(s.flags + blockIdx.x * 16, target);
  if (dead) return false;
  if (!wait) return true;
  for (int i = 0; i < idle_us; ++i) __builtin_amdgcn_s_sleep(37);   // 37 x 64 clocks, ~1 us each
  const uint32_t* f = s.flags + lane * 16;
  auto poll = [&]() -> u32x4 {
    u32x4 x = {target, target, target, target};
    if (lane < n) x[0] = ld_coh_u32(f);
    if (lane + 64 < n) x[1] = ld_coh_u32(f + 64 * 16);
    if (lane + 128 < n) x[2] = ld_coh_u32(f + 128 * 16);
    if (lane + 192 < n) x[3] = ld_coh_u32(f + 192 * 16);
    return x;
  };
  auto done = [&](u32x4 x) {
    return __all((int32_t)(x[0] - target) >= 0 && (int32_t)(x[1] - target) >= 0 &&
                 (int32_t)(x[2] - target) >= 0 && (int32_t)(x[3] - target) >= 0);
  };
  u32x4 a = poll(), b = poll();
  int polls = 0;
  while (true) {
    if (done(a)) break;
    a = poll();
    if (done(b)) break;
    b = poll();
    polls += 2;
    if (polls >= s.spin_limit) {
      if (lane == 0) __hip_atomic_store(s.status, status_word(s.epoch, MK_ETIMEOUT_DEV), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
      return false;
    }
    if ((polls & 63) == 0) {
      // only an error raised by this launch aborts it (an earlier launch's code is stale)
      const uint32_t st = __hip_atomic_load(s.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__any(status_is_error_of(st, s.epoch))) { __builtin_amdgcn_s_waitcnt(0); return false; }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  return true;
}

// Reads n 16-byte pieces of a stage buffer as they arrive (arrived16): piece i is at byte
// offset off(i) of resource r, and use(i, v) consumes it.  This thread takes pieces tid,
// tid + nthr, ..., NB of them at a time, all loaded together with device-coherent loads; the
// pieces that have not arrived yet are loaded again, back to back.  Every wait is bounded: after
// spin_limit rounds this launch's status becomes MK_ETIMEOUT and the workgroup is marked dead
// (*dead_sh); an error another workgroup raised in this launch ends the wait too.  A dead
// workgroup's remaining pieces are skipped (the launch's outputs are then unspecified).
template <int NB, class OffF, class UseF>
__device__ __forceinline__ void poll_stage(const Sync& s, int32_t* dead_sh, rsrc_t r, int n, int tid, int nthr,
                                           OffF off, UseF use) {
  volatile int32_t* dead = dead_sh;
  for (int base = 0; base < n; base += NB * nthr) {
    bool need[NB];
    u32x4 v[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) need[j] = base + j * nthr + tid < n;
    for (int spins = 0;; ++spins) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
        if (need[j]) v[j] = ld_coh16(r, off(base + j * nthr + tid));
      bool more = false;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (need[j] && arrived16(v[j])) {
          use(base + j * nthr + tid, v[j]);
          need[j] = false;
        }
        more |= need[j];
      }
      if (!more || *dead) break;
#if MK_POLL_SLEEP > 0
      __builtin_amdgcn_s_sleep(MK_POLL_SLEEP);
#endif
      if (spins >= s.spin_limit) {
        __hip_atomic_store(s.status, status_word(s.epoch, MK_ETIMEOUT_DEV), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *dead = 1;
        break;
      }
      if ((spins & 63) == 63 &&
          status_is_error_of(__hip_atomic_load(s.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), s.epoch)) {
        *dead = 1;
        break;
      }
    }
    if (*dead) return;
  }
}

// ------------------------------------------------------------------ dense tiles
// Bounded-wait bookkeeping of one poll round: true when the wait must end (this workgroup is
// dead, its spin limit ran out -- this launch's status becomes MK_ETIMEOUT -- or another
// workgroup raised an error in this launch).
__device__ __forceinline__ bool poll_give_up(const Sync& s, volatile int32_t* dead, int spins) {
  if (*dead) return true;
  if (spins >= s.spin_limit) {
    __hip_atomic_store(s.status, status_word(s.epoch, MK_ETIMEOUT_DEV), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *dead = 1;
    return true;
  }
  if ((spins & 63) == 63 &&
      status_is_error_of(__hip_atomic_load(s.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), s.epoch)) {
    *dead = 1;
    return true;
  }
  return false;
}

// A stage buffer in MFMA fragment order ([16 rows][K] bf16: k-step s is the 1 KB at 1024 s,
// lane l's 16 bytes at 16 l).  Read as it arrives (`poll`, device-coherent loads that bypass
// the XCD's L2), or with plain loads once a grid hand-off has made it complete.  Broadcast
// data that every workgroup reads in full travels best the second way when it is large: the
// first workgroup of an XCD to read a line brings it into that XCD's L2 for the others, where
// polling reads it from the memory side once per workgroup and round.
struct XSrc {
  rsrc_t r;
  const uint16_t* x;
  const Sync* sy;
  int32_t* dead;
  bool poll;
};
__device__ __forceinline__ XSrc xsrc(const uint16_t* x, int K, const Sync& sy, int32_t* dead_sh) {
  return XSrc{make_rsrc(x, (uint32_t)K * 32u), x, &sy, dead_sh, true};
}
__device__ __forceinline__ XSrc xplain(const uint16_t* x, const Sync& sy, int32_t* dead_sh) {
  return XSrc{make_rsrc(x, 0u), x, &sy, dead_sh, false};
}
// Row tile r of a row-tiled stage buffer with K columns (tiles 16 K elements apart).
__device__ __forceinline__ XSrc xtile(const XSrc& x, int r, int K) {
  XSrc y = x;
  y.x = x.x + (size_t)r * 16 * K;
  y.r = make_rsrc(y.x, x.poll ? (uint32_t)K * 32u : 0u);
  return y;
}

// This lane's 16-byte pieces j < NB of a stage buffer (byte offsets off[j]; read when need[j],
// left zero otherwise), read as they arrive: every round reads all the pieces still missing,
// back to back (pieces from different producers arrive at different times; reading them one
// after another would add a round trip each).
template <int NB>
__device__ __forceinline__ void poll_pieces(const Sync& sy, int32_t* dead_sh, rsrc_t r, const uint32_t (&off)[NB],
                                            bool (&need)[NB], u32x4 (&v)[NB]) {
  volatile int32_t* dead = dead_sh;
#pragma unroll
  for (int j = 0; j < NB; ++j) v[j] = u32x4{0, 0, 0, 0};
  for (int spins = 0;; ++spins) {
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (need[j]) v[j] = ld_coh16(r, off[j]);
    bool more = false;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (need[j] && arrived16(v[j])) need[j] = false;
      more |= need[j];
    }
    if (!more || poll_give_up(sy, dead, spins)) return;
  }
}

// This lane's x fragments of k-steps s0 + j, j < NB: read as they arrive when j < cnt and the
// lane's row is valid (rv), zero otherwise.
template <int NB>
__device__ __forceinline__ void x_poll(const XSrc& x, int s0, int cnt, bool rv, u32x4 (&xa)[NB]) {
  const uint32_t lane16 = (uint32_t)(threadIdx.x & 63) * 16u;
  if (!x.poll) {
#pragma unroll
    for (int j = 0; j < NB; ++j)
      xa[j] = (rv && j < cnt) ? ld16((const char*)x.x + (size_t)(s0 + j) * 1024 + lane16) : u32x4{0, 0, 0, 0};
    return;
  }
  uint32_t off[NB];
  bool need[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    off[j] = (uint32_t)(s0 + j) * 1024u + lane16;
    need[j] = rv && j < cnt;
  }
  poll_pieces<NB>(*x.sy, x.dead, x.r, off, need, xa);
}

// One 8-byte word of a stage buffer, read as it arrives (device-coherent 8-byte loads).
__device__ __forceinline__ uint64_t poll_u64(const Sync& s, int32_t* dead_sh, const void* p) {
  volatile int32_t* dead = dead_sh;
  for (int spins = 0;; ++spins) {
    const uint64_t v = __hip_atomic_load((uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v != ~0ull || poll_give_up(s, dead, spins)) return v;
  }
}


// Weight fragments of one wave for one 16-column tile of W [N][K]: MFMA k-steps
// s = wave + 8j (j < MAXS) hold W[n0 + l%16][32 s + 8 (l/16) .. +8].
template <int MAXS>
struct WFrag {
  u32x4 v[MAXS > 0 ? MAXS : 1];
};

// Dense tiles split K over the 8 compute waves in contiguous blocks: wave w takes k-steps
// w * J .. w * J + J - 1, J = ceil(K / 256), so a wave's consecutive operand fetches are 64 B
// (weights) and 1 KB (fragment-order x) apart and fit the load instructions' immediate offsets.
__device__ __forceinline__ int kblock(int ksteps) { return (ksteps + 7) >> 3; }

// `ld` is the row stride in elements when the K columns are part of a longer row (0: K).
template <int MAXS>
__device__ __forceinline__ void wfrag_load(WFrag<MAXS>& f, const uint16_t* __restrict__ W, int K, int n0, int ld = 0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ksteps = K >> 5, J = kblock(ksteps);
  const uint16_t* row = W + (size_t)(n0 + (lane & 15)) * (ld > 0 ? ld : K) + (lane >> 4) * 8 + wave * J * 32;
#pragma unroll
  for (int j = 0; j < MAXS; ++j) {
    const int s = wave * J + j;
    f.v[j] = (j < J && s < ksteps) ? ld16(row + j * 32) : u32x4{0, 0, 0, 0};
  }
}

// Pull a tile's weight rows into the cache hierarchy without holding them in registers: each
// lane reads one dword of a different 128-byte line (a 16 x K tile is 16 * 2K bytes, covered
// by 16 * 2K / 8K loads per wave over the 8 compute waves).  The values are folded into one
// word that the caller keeps alive, so the loads are not dropped.
template <int NT>
__device__ __forceinline__ uint32_t touch_tile(const uint16_t* __restrict__ W, int K, int n0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const char* base = (const char*)(W + (size_t)n0 * K);
  const int lines = 16 * K * 2 / 128;
  uint32_t v[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int l = (wave + 8 * j) * 64 + lane;
    v[j] = l < lines ? *(const uint32_t*)(base + (size_t)l * 128) : 0u;
  }
  uint32_t x = 0;
#pragma unroll
  for (int j = 0; j < NT; ++j) x ^= v[j];
  return x;
}

// Speculative expert prefetch: pull the listed experts' W1 and W2 (codes and block scales for
// NVFP4, the bf16 matrices otherwise) into the device-side caches, one dword per 128-byte line.
// Worker w of nworkers takes every nworkers-th line of the concatenated slices; expert ids
// outside [0, E) are skipped.  Compute threads; the folded value must be kept alive.
__device__ __forceinline__ uint32_t expert_touch(const KArgs& a, int worker, int nworkers) {
  const size_t P = a.P, I = a.I;
  const bool fp4 = a.fmt == 1;
  // per expert: up to four contiguous regions
  const size_t r0 = fp4 ? 2 * I * P / 2 : 2 * I * P * 2;       // W1 codes | W1 bf16
  const size_t r1 = fp4 ? 2 * I * g1_scale_row_bytes(a.P) : 0; // W1 scales (GEMM1 operand order)
  const size_t r2 = fp4 ? P * I / 2 : P * I * 2;               // W2 codes | W2 bf16
  const size_t r3 = fp4 ? P * I / 16 : 0;                      // W2 scales
  const size_t per = (r0 + r1 + r2 + r3 + 127) / 128;          // lines per expert (regions rounded)
  const size_t lines = per * (size_t)a.n_prefetch;
  uint32_t v = 0;
  for (size_t l = (size_t)worker * kCompute + threadIdx.x; l < lines; l += (size_t)nworkers * kCompute) {
    const int e = a.prefetch[l / per];
    if (e < 0 || e >= a.E) continue;
    const size_t o = (l % per) * 128;
    const uint8_t* p;
    if (o < r0) p = (fp4 ? a.w1_codes : (const uint8_t*)a.w1) + (size_t)e * r0 + o;
    else if (o < r0 + r1) p = a.w1_scales + (size_t)e * r1 + (o - r0);
    else if (o < r0 + r1 + r2) p = (fp4 ? a.w2_codes : (const uint8_t*)a.w2) + (size_t)e * r2 + (o - r0 - r1);
    else if (o < r0 + r1 + r2 + r3) p = a.w2_scales + (size_t)e * r3 + (o - r0 - r1 - r2);
    else continue;
    v ^= *(const uint32_t*)p;
  }
  return v;
}

// Activations handed between phases ([16 rows][K] bf16, rows >= T unused) are kept in MFMA
// fragment order: element (t, c) at frag_off(t, c), so the B operand of k-step s -- lane
// (l % 16, l / 16) holding row l % 16, columns 32 s + 8 (l / 16) .. + 8 -- is the 1 KB at
// x + 512 s, 16 bytes per lane in lane order.  Row-major [16][K] would put the 64 lanes on 16
// rows 2K bytes apart; measured on gfx950, a workgroup then reads 128 KB in ~2.9 us against
// ~0.9 us for contiguous 1 KB per instruction.
__host__ __device__ __forceinline__ int frag_off(int t, int c) {
  return (((c >> 5) * 64 + ((c >> 3) & 3) * 16 + t) << 3) + (c & 7);
}

// This wave's partial of the tile: x (fragment order; rows >= T are zero) times the fragments.
// x: the stage buffer, read as it arrives; s_base: its first k-step used here.
template <int MAXS>
__device__ __forceinline__ f32x4 wfrag_mma(const WFrag<MAXS>& f, const XSrc& x, int s_base, int T, int K) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15;
  const bool xv = nl < T;
  const int ksteps = K >> 5, J = kblock(ksteps);
  constexpr int XB = MAXS < 8 ? MAXS : 8;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j0 = 0; j0 < MAXS; j0 += XB) {
    u32x4 xa[XB];
    x_poll<XB>(x, s_base + wave * J + j0, min(J - j0, ksteps - (wave * J + j0)), xv, xa);
#pragma unroll
    for (int j = 0; j < XB; ++j) {
      const int jj = j0 + j, s = wave * J + jj;
      if (jj < J && s < ksteps) acc = mfma_bf16(xa[j], f.v[jj], acc);
    }
  }
  return acc;
}

// This wave's partial of a tile whose weights are read now (typically from L2 after a touch
// prefetch): weights and x of 8 k-steps are loaded together, then multiplied.
__device__ __forceinline__ f32x4 stream_mma(const uint16_t* __restrict__ W, int K, int n0, const XSrc& x, int T) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15;
  const bool xv = nl < T;
  const int ksteps = K >> 5, J = kblock(ksteps);
  const uint16_t* wrow = W + (size_t)(n0 + nl) * K + (lane >> 4) * 8 + wave * J * 32;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < J; b += 8) {
    u32x4 w[8], xa[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int jj = b + j, s = wave * J + jj;
      w[j] = (jj < J && s < ksteps) ? ld16(wrow + jj * 32) : u32x4{0, 0, 0, 0};
    }
    x_poll<8>(x, wave * J + b, min(J - b, ksteps - (wave * J + b)), xv, xa);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int jj = b + j, s = wave * J + jj;
      if (jj < J && s < ksteps) acc = mfma_bf16(xa[j], w[j], acc);
    }
  }
  return acc;
}

// A 16 x K weight tile copied into LDS: chunk (s, l) -- row n0 + l % 16, k = 32 s + 8 (l / 16)
// .. + 8 -- at byte (64 s + l) * 16, so a wave reads 1 KB contiguous per k-step.  Compute
// threads; the caller synchronises before the tile is read.
__device__ __forceinline__ void lds_tile_fill(const uint16_t* __restrict__ W, int K, int n0, char* dst) {
  const int tid = threadIdx.x;
  if (tid >= kCompute) return;
  const int nch = (K / 32) * 64;
  for (int base = 0; base < nch; base += 8 * kCompute) {
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = base + j * kCompute + tid, sk = c >> 6, l = c & 63;
      if (c < nch) v[j] = ld16(W + (size_t)(n0 + (l & 15)) * K + 32 * sk + 8 * (l >> 4));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = base + j * kCompute + tid;
      if (c < nch) *(u32x4*)(dst + (size_t)c * 16) = v[j];
    }
  }
}

// The same tile layout filled by one wave through the LDS-DMA path (global_load_lds, 16 bytes
// per lane, lane l landing at base + 16 l): instruction s moves the 1 KB of k-step s.  No
// registers hold the data.  The LDS is written asynchronously: the wave must wait for its loads
// (s_waitcnt) before a workgroup barrier that precedes any read of the tile.
// Waves may share a tile: this wave moves k-steps first, first + stride, ...
__device__ __forceinline__ void lds_tile_dma(const uint16_t* __restrict__ W, int K, int n0, char* dst,
                                             int first = 0, int stride = 1) {
  const int lane = threadIdx.x & 63;
  const uint16_t* row = W + (size_t)(n0 + (lane & 15)) * K + 8 * (lane >> 4);
  for (int sk = first; sk < K / 32; sk += stride)
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(row + 32 * sk),
                                     (__attribute__((address_space(3))) void*)(dst + sk * 1024), 16, 0, 0);
}

// This wave's partial of a tile whose weights sit in LDS (lds_tile_fill layout); x rows are
// loaded 16 k-steps at a time.
__device__ __forceinline__ f32x4 lds_mma(const char* wl, const XSrc& x, int T, int K) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15;
  const bool xv = nl < T;
  const int ksteps = K >> 5, J = kblock(ksteps);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < J; b += 16) {
    u32x4 xa[16];
    x_poll<16>(x, wave * J + b, min(J - b, ksteps - (wave * J + b)), xv, xa);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int jj = b + j, sk = wave * J + jj;
      if (jj < J && sk < ksteps) acc = mfma_bf16(xa[j], *(const u32x4*)(wl + (size_t)(sk * 64 + lane) * 16), acc);
    }
  }
  return acc;
}

// wave partial -> LDS red[wave][row][col] (row stride 17)
__device__ __forceinline__ void red_store(float* red, f32x4 acc) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  float* p = red + wave * (16 * 17);
#pragma unroll
  for (int r = 0; r < 4; ++r) p[(4 * g + r) * 17 + nl] = acc[r];
}
__device__ __forceinline__ float red_sum(const float* red, int row, int col) {
  float v = 0.f;
#pragma unroll
  for (int w = 0; w < 8; ++w) v += red[w * (16 * 17) + row * 17 + col];
  return v;
}

// Control wave: the 4 outputs (row, c0..c0+3) of a tile, summed over the 8 waves.
__device__ __forceinline__ void ctl_tile_vals(const float* red, int row, int c0, float v[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = red_sum(red, row, c0 + j);
}

__device__ __forceinline__ uint64_t pack4_bf16(const float v[4]) {
  return (uint64_t)pack_bf2(v[0], v[1]) | ((uint64_t)pack_bf2(v[2], v[3]) << 32);
}

// tile index of this workgroup in a phase whose tile t runs on workgroup (t + off) % n_wg
__device__ __forceinline__ int first_tile(int off) {
  const int n = gridDim.x;
  return ((int)blockIdx.x - off % n + n) % n;
}

// Copy n 16-byte pieces to LDS with every load of a batch issued before any store (one
// memory round trip per batch of up to 16 pieces per thread instead of one per piece).
// piece(i) returns the global address of piece i, dst(i) its LDS address.  Compute
// threads only; the caller synchronises afterwards.
template <class SrcF, class DstF>
__device__ __forceinline__ void stage_pieces(int n, SrcF piece, DstF dst) {
  const int tid = threadIdx.x;
  if (tid >= kCompute) return;
  for (int base = 0; base < n; base += 8 * kCompute) {
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = base + j * kCompute + tid;
      if (i < n) v[j] = ld16(piece(i));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = base + j * kCompute + tid;
      if (i < n) *(u32x4*)dst(i) = v[j];
    }
  }
}

// ------------------------------------------------------------------ attention

// A work item is one (kv head g, key chunk, row block).  Chunk keys are context rows
// [kb, kb + nk) or, for the last chunk of a head, the tree's own slots.  Rows are the
// (token, q head of g) pairs, row = t * G + (h - g*G), R = T*G <= 128, in tiles of 16; a row
// block holds rw tiles.  The 8 compute waves split an item as rw row tiles x 8/rw key groups:
// wave w takes row tile rb*rw + w % rw and the w / rw-th of the chunk's keys.  S^T = K Q^T
// puts keys on the MFMA M axis so that the probabilities land in exactly the B-operand layout
// the P.V product needs.
struct AttnItem {
  int b, g, chunk, rb, kb, nk;      // b: the sequence (its KV cache, queries and tree)
  bool tree;
};
__device__ __forceinline__ AttnItem attn_item(const KArgs& a, int item) {
  AttnItem t;
  const int per_g = a.attn_chunks_per_head * a.attn_nrb;
  t.b = a.B == 1 ? 0 : item / (a.Hkv * per_g);   // (one sequence: a constant, no scalar registers)
  item -= t.b * a.Hkv * per_g;
  t.g = item / per_g;
  const int r = item % per_g;
  t.chunk = r / a.attn_nrb;
  t.rb = r % a.attn_nrb;
  t.tree = t.chunk == a.attn_chunks_per_head - 1;
  t.kb = t.tree ? a.ctx : a.attn_lo + t.chunk * a.ck;
  t.nk = t.tree ? a.Ts : min(a.ck, a.ctx - t.kb);
  return t;
}

// This lane's query fragments (B operand of S^T): row = 16 tile + l%16, d = 32 s + 8 (l/16).
__device__ __forceinline__ void attention_q(const KArgs& a, const AttnItem& it, u32x4 qf[4]) {
  const int d = a.d, G = a.Hq / a.Hkv, R = a.Ts * G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = (it.rb * a.attn_rw + wave % a.attn_rw) * 16 + (lane & 15), grp = lane >> 4;
  const bool rv = threadIdx.x < kCompute && row < R;
  const int tok = rv ? row / G : 0, head = it.g * G + (rv ? row % G : 0);
  // every lane loads, unconditionally (conditional loads would leave join copies that wait for
  // every load in flight): a row outside the item reads row 0, whose finite values only reach
  // scores that are masked for that row; k-steps past d/32 are never used
  const uint16_t* q = a.q_in + (size_t)(it.b * a.Ts + tok) * a.Hq * d + head * d + grp * 8;
#pragma unroll
  for (int s = 0; s < 4; ++s) qf[s] = ld16(q + (s < d / 32 ? s : 0) * 32);
}

__device__ __forceinline__ int vt_stride(int ck) { return ck / 2 + 2; }

// Staging of an item's K and V into LDS (keys nk..ck-1 zeroed), in batches of 4 K pieces and
// 2 V key-pair pieces per compute thread (at d = 128 a batch covers 128 keys): a batch's loads
// are all issued (stage_load) before its LDS stores (stage_store), so the first batch of a
// workgroup's first item can be in flight during the launch's setup.
struct StageRegs {
  u32x4 kv[4], v0[2], v1[2];
};
__device__ __forceinline__ int stage_batches(const KArgs& a) { return (a.ck * (a.d / 8) + 4 * kCompute - 1) / (4 * kCompute); }

__device__ __forceinline__ void stage_load(const KArgs& a, const AttnItem& it, int b, StageRegs& r) {
  // recomputed per item: indexing hoisted out of the item loop would hold registers
  // through the whole phase
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  if (tid >= kCompute) return;
  const int d = a.d, per_row = d / 8, nkp = a.ck / 2;
  const int kpieces = a.ck * per_row, vpieces = nkp * per_row;
  const size_t rstride = (size_t)a.Hkv * d;
  const size_t seq = (size_t)it.b * a.cap * a.Hkv * d;           // sequence it.b's cache
  const uint16_t* kbase = a.kc + seq + ((size_t)it.kb * a.Hkv + it.g) * d;
  const uint16_t* vbase = a.vc + seq + ((size_t)it.kb * a.Hkv + it.g) * d;
  // Every piece is loaded unconditionally from a valid address (a key past the chunk's rows
  // reads its last row, a piece past the chunk reads piece 0); stage_store zeroes or skips
  // those.  Conditional loads would leave join copies that wait for every load in flight.
  const int klast = it.nk - 1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int i = b * 4 * kCompute + tid + j * kCompute;
    i = i < kpieces ? i : 0;
    const int key = min(i / per_row, klast), c = (i % per_row) * 8;
    r.kv[j] = ld16(kbase + key * rstride + c);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int i = b * 2 * kCompute + tid + j * kCompute;
    i = i < vpieces ? i : 0;
    const int kp = i % nkp, c = (i / nkp) * 8;
    r.v0[j] = ld16(vbase + min(2 * kp, klast) * rstride + c);
    r.v1[j] = ld16(vbase + min(2 * kp + 1, klast) * rstride + c);
  }
}

// LDS of an item (ck <= 256 keys): K row-major [ck][d + 8] bf16, then V transposed as key
// pairs: VT32[dd][kp] = V[2kp][dd] | V[2kp+1][dd] << 16, row stride ck/2 + 2 dwords.
__device__ __forceinline__ void stage_store(const KArgs& a, const AttnItem& it, int b, const StageRegs& r, char* smem) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  if (tid >= kCompute) return;
  const int d = a.d, ck = a.ck, per_row = d / 8, nkp = ck / 2;
  const int ks_stride = d + 8, vs = vt_stride(ck);
  const int kpieces = ck * per_row, vpieces = nkp * per_row;
  uint16_t* Ks = (uint16_t*)smem;
  uint32_t* VT = (uint32_t*)(Ks + ck * ks_stride);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = b * 4 * kCompute + tid + j * kCompute, key = i / per_row, c = (i % per_row) * 8;
    if (i < kpieces) *(u32x4*)(Ks + key * ks_stride + c) = key < it.nk ? r.kv[j] : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = b * 2 * kCompute + tid + j * kCompute, kp = i % nkp, c = (i / nkp) * 8;
    if (i < vpieces) {
      const u32x4 z = {0, 0, 0, 0};
      const u32x4 a0 = 2 * kp < it.nk ? r.v0[j] : z, a1 = 2 * kp + 1 < it.nk ? r.v1[j] : z;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        VT[(c + 2 * q) * vs + kp] = (a0[q] & 0xFFFFu) | (a1[q] << 16);
        VT[(c + 2 * q + 1) * vs + kp] = (a0[q] >> 16) | (a1[q] & 0xFFFF0000u);
      }
    }
  }
}

// The compute half of an attention item, after the staging barrier.  Each wave runs an online
// softmax over its key group, 32 keys (two key tiles) a step: scores, a new running row max m,
// the running sum l and O^T rescaled by exp(m_old - m_new), then O^T += V^T P^T.  With one key
// group per row tile the wave stores its partial (O unnormalised, m, l); otherwise the key
// groups' partials of a row are combined in LDS, flash-decoding style, and stored once.
// Called by all threads (contains workgroup barriers when the item is split over keys).  RW is
// the item's row tiles (a.attn_rw), a template parameter so that the wave roles and the combine
// compile to shifts and unrolled loops.
template <int RW, bool TS>
__device__ __forceinline__ void attention_compute(const KArgs& a, const Tree& tr, const AttnItem& it, char* smem,
                                                  const u32x4 qf[4]) {
  const int d = a.d, G = a.Hq / a.Hkv, R = a.Ts * G, ck = a.ck;
  constexpr int rw = RW, nkw = 8 / RW;
  const int ks_stride = d + 8, vs = vt_stride(ck);
  const uint16_t* Ks = (const uint16_t*)smem;
  const uint32_t* VT = (const uint32_t*)(Ks + ck * ks_stride);
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));                 // (no per-thread indexing hoisted out of the item loop)
  const int lane = tid & 63, wave = tid >> 6;
  const int nl = lane & 15, grp = lane >> 4;
  const int rt = it.rb * rw + wave % rw, kg = wave / rw;
  const int row = rt * 16 + nl;                 // this lane's query row (MFMA column)
  const bool active = threadIdx.x < kCompute && rt * 16 < R;
  const bool rv = active && row < R;
  const int tok = rv ? row / G : 0;
  const int dsteps = d / 32, dtiles = d / 16;
  const float scale = 1.0f / sqrtf((float)d);
  // this wave's keys within the chunk: [k0, k1)
  const int kpg = ck / nkw;
  const int k0 = kg * kpg, k1 = min(k0 + kpg, it.nk);
  // visibility of chunk key kl for this lane's row: kl in [vis_lo, nk) for context chunks
  // (sliding-window lower bound), the ancestor mask for the tree chunk
  const int trow = it.b * a.Ts + tok;           // the token's row (its sequence's tree bits at b Ts)
  const int vis_lo = rv ? max(0, tr.lo[trow] - it.kb) : 0;
  const int vis_hi = rv ? it.nk : 0;
  const uint32_t anc_m = rv ? tr.anc[trow] >> (it.b * a.Ts) : 0u;
  float m = -INFINITY, lpart = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (active) {
    for (int kt = k0 / 16; kt * 16 < k1; kt += 2) {
      const bool two = kt * 16 + 16 < k1;
      u32x4 kf[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          if (s < dsteps && (h == 0 || two))
            kf[h][s] = *(const u32x4*)(Ks + ((kt + h) * 16 + nl) * ks_stride + s * 32 + grp * 8);
      f32x4 sc[2];
      float mx = -INFINITY;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (h == 0 || two) {
#pragma unroll
          for (int s = 0; s < 4; ++s)
            if (s < dsteps) acc = mfma_bf16(kf[h][s], qf[s], acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kl = (kt + h) * 16 + 4 * grp + r;   // key index within the chunk
          const bool vis = (h == 0 || two) && kl < vis_hi &&
                           (it.tree ? ((anc_m >> kl) & 1u) != 0 : kl >= vis_lo);
          sc[h][r] = vis ? acc[r] * scale : -INFINITY;
          mx = fmaxf(mx, sc[h][r]);
        }
      }
      const float mnew = fmaxf(m, xgroup_max(mx));
      // exp(-inf - x) = 0 for masked keys; with nothing visible yet the row uses 0 as its max
      const float msafe = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = __expf(m - msafe);
      uint32_t pb[2][2];
      float ps = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[r] = __expf(sc[h][r] - msafe);
          ps += p[r];
        }
        pb[h][0] = pack_bf2(p[0], p[1]);
        pb[h][1] = pack_bf2(p[2], p[3]);
      }
      lpart = lpart * alpha + ps;
      m = mnew;
      // O^T[dd][row] += sum_keys V^T[dd][key] P^T[key][row]; a 32-key step pairs the two key
      // tiles (lane group grp supplies keys 4grp..4grp+3 of both), a lone tile takes the
      // 16-key form
      const uint32_t* vt0 = VT + nl * vs + kt * 8 + 2 * grp;
      if (two) {
        const u32x4 pf = {pb[0][0], pb[0][1], pb[1][0], pb[1][1]};
#pragma unroll
        for (int h = 0; h < 2; ++h) {                 // d tiles in two groups of 4
          u32x4 vf[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (4 * h + j < dtiles) {
              const uint32_t* v = vt0 + (4 * h + j) * 16 * vs;
              const u32x2 v0 = *(const u32x2*)v, v1 = *(const u32x2*)(v + 8);
              vf[j] = u32x4{v0[0], v0[1], v1[0], v1[1]};
            }
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (4 * h + j < dtiles) o[4 * h + j] = mfma_bf16(vf[j], pf, o[4 * h + j] * alpha);
        }
      } else {
        u32x2 vf[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          if (dt < dtiles) vf[dt] = *(const u32x2*)(vt0 + dt * 16 * vs);
        const u32x2 pf = {pb[0][0], pb[0][1]};
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          if (dt < dtiles) o[dt] = mfma_bf16_k16(vf[dt], pf, o[dt] * alpha);
      }
    }
  }
  stamp<TS>(a.timestamps, 39, 0);
  const float lsum = xgroup_sum(lpart);
  const int slot = (it.b * a.Hkv + it.g) * a.attn_chunks_per_head + it.chunk;
  if (nkw == 1) {
    if (rv) {
      float* po = a.part_o + ((size_t)slot * 128 + row) * d;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        if (dt < dtiles) {
          u32x4 v = {__float_as_uint(o[dt][0]), __float_as_uint(o[dt][1]), __float_as_uint(o[dt][2]),
                     __float_as_uint(o[dt][3])};
          st_coh_u128(po + dt * 16 + 4 * grp, v);
        }
      }
      if (grp == 0)
        st_coh_u64(a.part_ml + ((size_t)slot * 128 + row) * 2,
                   (uint64_t)__float_as_uint(m) | ((uint64_t)__float_as_uint(lsum) << 32));
    }
    return;
  }
  // key groups combined in LDS over the staged chunk: [wave][16 rows][d + 4] fp32, then
  // [wave][16 rows] (m, l)
  const int cs = d + 4;
  float* cb = (float*)smem;
  float* cml = cb + 8 * 16 * cs;
  wg_sync();                                    // every wave is done with K and V
  if (active) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      if (dt < dtiles) *(f32x4*)(cb + (wave * 16 + nl) * cs + dt * 16 + 4 * grp) = o[dt];
    if (grp == 0) {
      cml[(wave * 16 + nl) * 2 + 0] = m;
      cml[(wave * 16 + nl) * 2 + 1] = lsum;
    }
  }
  wg_sync();
  stamp<TS>(a.timestamps, 40, 0);
  if (threadIdx.x < kCompute) {
    const int quads = d / 4;
    for (int e = threadIdx.x; e < rw * 16 * quads; e += kCompute) {
      const int lr = e / quads, dq = e % quads;
      const int j = lr / 16, r16 = lr % 16;
      const int grow = (it.rb * rw + j) * 16 + r16;
      if (grow >= R) continue;
      float M = -INFINITY;
#pragma unroll
      for (int q = 0; q < nkw; ++q) M = fmaxf(M, cml[((j + rw * q) * 16 + r16) * 2]);
      const float Ms = M == -INFINITY ? 0.f : M;
      float L = 0.f;
      f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < nkw; ++q) {
        const int w = j + rw * q;
        const float sw = __expf(cml[(w * 16 + r16) * 2] - Ms);
        L += cml[(w * 16 + r16) * 2 + 1] * sw;
        O += *(const f32x4*)(cb + (w * 16 + r16) * cs + 4 * dq) * sw;
      }
      float* po = a.part_o + ((size_t)slot * 128 + grow) * d;
      st_coh_u128(po + 4 * dq, u32x4{__float_as_uint(O[0]), __float_as_uint(O[1]), __float_as_uint(O[2]),
                                     __float_as_uint(O[3])});
      if (dq == 0)
        st_coh_u64(a.part_ml + ((size_t)slot * 128 + grow) * 2,
                   (uint64_t)__float_as_uint(M) | ((uint64_t)__float_as_uint(L) << 32));
    }
  }
}

// Merge of the per-chunk partials of one (kv head, row), flash-decoding style rescale.
// Compute waves: 16 chunk groups x 32 threads (4 d values each).  The first d/4 threads
// store the merged row (bf16, read by the o-proj as it arrives) and its stats.  Called by all
// threads; the caller synchronises before LDS `scratch` is used again.
template <bool TS>
__device__ __forceinline__ void merge_unit(const KArgs& a, int unit, float* scratch) {
  const int d = a.d;
  const int G = a.Hq / a.Hkv, R = a.Ts * G;
  const int b = a.B == 1 ? 0 : unit / (a.Hkv * R);       // the sequence
  unit -= b * a.Hkv * R;
  const int g_kv = b * a.Hkv + unit / R, row = unit % R;    // (partial slots are per sequence)
  const int tok = row / G, head = (unit / R) * G + row % G;
  const int nchunks = a.attn_chunks_per_head;
  const int quads = d / 4;
  const int ngroups = kCompute / 32;
  const int tq = threadIdx.x % 32, cg = threadIdx.x / 32;
  float M = -INFINITY, L = 0.f, O[4] = {0.f, 0.f, 0.f, 0.f};
  if (tq < quads && threadIdx.x < kCompute) {
    // four chunks' partials loaded together per round trip
    for (int c0 = cg; c0 < nchunks; c0 += 4 * ngroups) {
      f32x2 ml[4];
      f32x4 o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = c0 + j * ngroups;
        const size_t r = (size_t)(g_kv * nchunks + c) * 128 + row;
        ml[j] = c < nchunks ? *(const f32x2*)(a.part_ml + r * 2) : f32x2{-INFINITY, 0.f};
        o[j] = c < nchunks ? *(const f32x4*)(a.part_o + r * d + tq * 4) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float m = ml[j][0], l = ml[j][1];
        if (l <= 0.f) continue;
        const float Mn = fmaxf(M, m);
        const float s_old = (M == -INFINITY) ? 0.f : __expf(M - Mn);
        const float s_new = __expf(m - Mn);
        L = L * s_old + l * s_new;
#pragma unroll
        for (int q = 0; q < 4; ++q) O[q] = O[q] * s_old + o[j][q] * s_new;
        M = Mn;
      }
    }
  }
  stamp<TS>(a.timestamps, 61, 0);
  // The row's maximum over the groups' maxima (the threads of a group share theirs); every
  // thread rescales its group's sums to it, and the first 32 threads add the groups up in
  // group order.  LDS: the group maxima after 5 components x 16 groups x 32 threads.
  float* gmax = scratch + 5 * 16 * 32;
  if (threadIdx.x < kCompute && tq == 0) gmax[cg] = M;
  wg_sync();
  stamp<TS>(a.timestamps, 62, 0);
  float Mt = -INFINITY;
  if (threadIdx.x < kCompute) {
#pragma unroll
    for (int q = 0; q < 16; ++q) Mt = fmaxf(Mt, gmax[q]);
    const float s = M == -INFINITY ? 0.f : __expf(M - Mt);
    scratch[cg * 32 + tq] = L * s;
#pragma unroll
    for (int j = 0; j < 4; ++j) scratch[((1 + j) * 16 + cg) * 32 + tq] = O[j] * s;
  }
  wg_sync();
  if (threadIdx.x < quads) {
    float Lt = 0.f, Ot[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      Lt += scratch[q * 32 + threadIdx.x];
#pragma unroll
      for (int j = 0; j < 4; ++j) Ot[j] += scratch[((1 + j) * 16 + q) * 32 + threadIdx.x];
    }
    const float inv = 1.0f / Lt;
    st_coh_u64(st_attn(a) + (size_t)b * 16 * a.Hq * d + frag_off(tok, head * d + threadIdx.x * 4),
               (uint64_t)pack_bf2(Ot[0] * inv, Ot[1] * inv) | ((uint64_t)pack_bf2(Ot[2] * inv, Ot[3] * inv) << 32));
    if (threadIdx.x == 0 && a.attn_stats) {
      a.attn_stats[((size_t)(b * a.Ts + tok) * a.Hq + head) * 2 + 0] = Mt;
      a.attn_stats[((size_t)(b * a.Ts + tok) * a.Hq + head) * 2 + 1] = Lt;
    }
  }
  stamp<TS>(a.timestamps, 63, 0);
}

// ------------------------------------------------------------------ routing

// Top-k of one row of the logits (value desc, index asc) and softmax gates over the selected,
// published for every workgroup.  One wave per row: the control wave of workgroup t takes rows
// t, t + grid, ...  It reads the row as it arrives from the router workgroups, then writes the
// row's 8 routing slots (expert, gate bits) with coherent stores, zero past top-k.
template <bool TS>
__device__ __forceinline__ void publish_route(const KArgs& a, const Sync& sy, int32_t* dead_sh) {
  const int E = a.E, K = a.topk, lane = threadIdx.x & 63;
  for (int t = blockIdx.x; t < a.T; t += gridDim.x) {
    // lane l holds experts 4 l .. 4 l + 3
    u32x4 v = u32x4{0, 0, 0, 0};
    poll_stage<1>(sy, dead_sh, make_rsrc(st_logits(a) + (size_t)t * E, (uint32_t)E * 4), E / 4, lane, 64,
                  [](int i) { return (uint32_t)i * 16u; }, [&](int, u32x4 x) { v = x; });
    if (*(volatile int32_t*)dead_sh) return;
    stamp<TS>(a.timestamps, 51);
    // Each candidate is one 64-bit word: the logit's order-preserving integer with its sign bit
    // flipped (exact, so ties stay ties) above 0xFFFF - expert, so that a larger word comes
    // first in (logit desc, index asc) order; 0 stands for no expert.  One unsigned compare
    // then orders two candidates, with no branch on ties.
    uint64_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * lane + q;
      w[q] = e < E ? ((uint64_t)((uint32_t)f32_order_key(__uint_as_float(v[q])) ^ 0x80000000u) << 32) |
                         (uint32_t)(0xFFFF - e)
                   : 0ull;
    }
    auto cswap = [&](int i, int j) {
      const bool sw = w[j] > w[i];
      const uint64_t x = w[i], y = w[j];
      w[i] = sw ? y : x;
      w[j] = sw ? x : y;
    };
    cswap(0, 1); cswap(2, 3); cswap(0, 2); cswap(1, 3); cswap(1, 2);
    // each round the largest head wins (the lowest lane on ties, which holds the lowest index)
    // and its lane pops it; lane j keeps round j's logit key and expert
    int32_t kj = 0, ej = 0;
    for (int j = 0; j < K; ++j) {
      const int32_t head = (int32_t)((uint32_t)(w[0] >> 32) ^ 0x80000000u);
      const int32_t m = wave_max_i32_folded(head);
      const int lw = __ffsll((unsigned long long)__ballot(head == m)) - 1;
      const int be = 0xFFFF - __builtin_amdgcn_readlane((int)(uint32_t)w[0], lw);
      const bool take = lane == lw;
#pragma unroll
      for (int q = 0; q < 3; ++q) w[q] = take ? w[q + 1] : w[q];
      w[3] = take ? 0ull : w[3];
      kj = lane == j ? m : kj;
      ej = lane == j ? be : ej;
    }
    // gates: softmax over the k selected logits, summed in slot order
    auto rl = [](float x, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l)); };
    const float mj = f32_from_order_key(kj);
    const float z = __expf(mj - rl(mj, 0));
    float sum = 0.f;
    for (int j = 0; j < K; ++j) sum += rl(z, j);
    if (lane < 8)
      st_coh_u64(st_route(a) + (size_t)t * 8 + lane,
                 lane < K ? (uint64_t)(uint32_t)ej | ((uint64_t)__float_as_uint(z / sum) << 32) : 0ull);
    stamp<TS>(a.timestamps, 52);
  }
}

// The dispatch tables, from the published routing.  Every workgroup computes the same tables.
// Called by all threads; the work runs on the compute waves.
template <bool TS, class RT>
__device__ __forceinline__ void route_tables(const KArgs& a, RT& rt, uint32_t* lds, const Sync& sy, int32_t* dead_sh) {
  const int T = a.T, E = a.E, K = a.topk, tid = threadIdx.x;
  const int npairs = T * K;
  const bool cw = tid < kCompute;
  // (NVFP4) every expert's two tensor scales; then the routing, read as it arrives (one 16-byte
  // piece holds two slots)
  const int nts = a.fmt == 1 ? E / 4 : 0;
  stage_pieces(2 * nts, [&](int i) {
    return i < nts ? (const void*)(a.w1_ts + 4 * i) : (const void*)(a.w2_ts + 4 * (i - nts));
  }, [&](int i) {
    return i < nts ? (void*)(rt.ts1 + 4 * i) : (void*)(rt.ts2 + 4 * (i - nts));
  });
  if (cw)
    poll_stage<1>(sy, dead_sh, make_rsrc(st_route(a), (uint32_t)T * 64), T * 4, tid, kCompute,
                  [](int i) { return (uint32_t)i * 16u; }, [&](int i, u32x4 v) {
      const int t = i >> 2, j = (i & 3) * 2;
      if (j < K) { rt.idx[t * K + j] = (int16_t)v[0]; rt.gate[t * K + j] = __uint_as_float(v[1]); }
      if (j + 1 < K) { rt.idx[t * K + j + 1] = (int16_t)v[2]; rt.gate[t * K + j + 1] = __uint_as_float(v[3]); }
    });
  // per expert, a bitmask of the pairs routed there (kMW words), counts, offsets
  constexpr int kMW = RT::kPairs / 32;
  uint32_t* mask = lds;
  int32_t* ecnt = (int32_t*)(mask + E * kMW);
  int32_t* efirst = ecnt + E;
  for (int i = tid; cw && i < E * kMW; i += kCompute) mask[i] = 0u;
  wg_sync();
  stamp<TS>(a.timestamps, 46, 0);
  for (int p = tid; cw && p < npairs; p += kCompute) atomicOr(&mask[rt.idx[p] * kMW + (p >> 5)], 1u << (p & 31));
  wg_sync();
  for (int e = tid; cw && e < E; e += kCompute) {
    int c = 0;
#pragma unroll
    for (int q = 0; q < kMW; ++q) c += __popc(mask[e * kMW + q]);
    ecnt[e] = c;
  }
  wg_sync();
  stamp<TS>(a.timestamps, 20, 0);
  if (tid < 64) {
    // exclusive scans over experts: lane handles 4 consecutive experts; an expert takes
    // ceil(count / 16) GEMM1 entries
    int cnt[4], act[4], sumc = 0, suma = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid * 4 + q;
      cnt[q] = e < E ? ecnt[e] : 0;
      act[q] = (cnt[q] + 15) / 16;
      sumc += cnt[q];
      suma += act[q];
    }
    const int sc = wave_incl_scan_i32(sumc), sa = wave_incl_scan_i32(suma);
    int pc = sc - sumc, pa = sa - suma;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid * 4 + q;
      if (e < E) efirst[e] = pc;
#pragma unroll 1      // (kept small: this code runs once per launch, from a cold instruction cache)
      for (int j = 0; j < act[q]; ++j) {
        rt.act_expert[pa] = e;
        rt.act_off[pa] = pc + 16 * j;
        rt.act_cnt[pa] = min(16, cnt[q] - 16 * j);
        ++pa;
      }
      pc += cnt[q];
    }
    if (tid == 63) rt.n_active = sa;
  }
  wg_sync();
  stamp<TS>(a.timestamps, 22, 0);
  if (blockIdx.x == 0 && a.hist)
    for (int e = tid; e < E; e += kThreads) a.hist[e] += ecnt[e];
  if (!cw) {
    // GEMM2 slots (control wave): slot i is active expert i's first min(cnt, 8) pairs; the
    // experts with more than 8 pairs get a second slot each, after all the first slots
    const int lane = tid & 63, na = rt.n_active;
    int nsplit = 0;
    for (int base = 0; base < na; base += 64) {
      const int i = base + lane;
      const int c = i < na ? rt.act_cnt[i] : 0;
      const uint64_t split = __ballot(c > 8);
      if (i < na) {
        rt.slot_expert[i] = rt.act_expert[i];
        rt.slot_off[i] = rt.act_off[i];
        rt.slot_cnt[i] = min(c, 8);
        if (c > 8) {
          const int j = na + nsplit + __popcll(split & ((1ull << lane) - 1ull));
          rt.slot_expert[j] = rt.act_expert[i];
          rt.slot_off[j] = rt.act_off[i] + 8;
          rt.slot_cnt[j] = c - 8;
        }
      }
      nsplit += __popcll(split);
    }
    if (lane == 0) rt.n_slots = na + nsplit;
    stamp<TS>(a.timestamps, 25);
    // workgroup 0: this step's most-used experts, the next step's prefetch list, by a
    // tournament over keys (count, then lower index) that are unique per expert
    if (blockIdx.x == 0 && a.prefetch_next && a.n_prefetch_next > 0) {
      int32_t key[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = 4 * lane + q;
        key[q] = (e < E && ecnt[e] > 0) ? (ecnt[e] << 16) | (0xFFFF - e) : -1;
      }
      for (int j = 0; j < a.n_prefetch_next; ++j) {
        const int32_t best = max(max(key[0], key[1]), max(key[2], key[3]));
        const int32_t m = wave_max_i32(best);
#pragma unroll
        for (int q = 0; q < 4; ++q) key[q] = key[q] == m ? -1 : key[q];
        if (lane == 0) a.prefetch_next[j] = m < 0 ? -1 : 0xFFFF - (m & 0xFFFF);
      }
    }
  }
  for (int p = tid; cw && p < npairs; p += kCompute) {
    const int e = rt.idx[p];
    const uint32_t* m = mask + e * kMW;
    const int w = p >> 5;
    int r = __popc(m[w] & ((1u << (p & 31)) - 1u));
    for (int q = 0; q < w; ++q) r += __popc(m[q]);
    rt.pair_list[efirst[e] + r] = p;
  }
  stamp<TS>(a.timestamps, 26, 0);
  wg_sync();
}

// ------------------------------------------------------------------ experts

// GEMM1 for this workgroup's tasks.  A task is (active expert, block of 16 intermediate
// columns j0..j0+15); tasks are ordered by expert and each workgroup takes a contiguous
// range, so its tasks mostly share one expert.  A task has two units: the 16 gate rows
// (j0 + i) and the 16 up rows (I + j0 + i) of W1.  Each wave owns whole units over the full
// K = P, so no reduction across waves is needed: it loads all its codes at once (16 bytes
// per lane per 128 k), stages the unit's scales through LDS, reads the tokens' xp rows from
// LDS, and leaves the 16x16 tile u = xp W1^T ts1 in LDS.  The workgroup then forms
// a = silu(u_gate) * u_up and requantises it to NVFP4 (tensor scale 1) per 16-element block.
// Called by all threads.
constexpr int G1_UNITS = 16;                   // units per round (2 per compute wave)

// GEMM1 input rows.  NVFP4 experts multiply in fp16: xs[t][k] = fp16(xp[t][k] * 2^xk[t]),
// where 2^xk[t] puts the row's largest magnitude in [2^14, 2^15).  Every element whose
// magnitude is at least 2^-28 of the row maximum then converts exactly (a bf16 value has 8
// significant bits) and lies in fp16's normal range, and its product with an exactly decoded
// fp16 weight is exact in the fp32 accumulator; smaller elements may be rounded or flushed
// (relative effect below 2^-28).  The GEMM1 result is scaled back by 2^-xk[t].  bf16 experts
// take xs = xp unchanged.
//
// Part 1 (compute threads, no barrier; xp is complete since the pooler's hand-off): this
// thread's pieces of xp into registers and, for NVFP4, each piece's largest magnitude into
// pmax[t][c / 8] (LDS).  xp is in fragment order: piece i (8 bf16, 16 * P / 8 <= 4096 pieces)
// is row i % 16, columns 8 ((i / 64) * 4 + (i / 16) % 4) .. + 8; pieces of rows >= T are skipped.
__device__ __forceinline__ int piece_row(int i) { return i & 15; }
__device__ __forceinline__ int piece_col8(int i) { return ((i >> 6) << 2) + ((i >> 4) & 3); }
__device__ __forceinline__ void xp_fetch(const KArgs& a, u32x4 (&v)[8], uint32_t* pmax) {
  const int tid = threadIdx.x, n = 16 * (a.P / 8);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = j * kCompute + tid;
    if (i < n && piece_row(i) < a.T) v[j] = ld16(st_xp(a) + (size_t)i * 8);
  }
  if (a.fmt != 1) return;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = j * kCompute + tid;
    if (i < n && piece_row(i) < a.T) {
      // |x| of a bf16 orders like its bit pattern without the sign
      uint32_t m = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w = v[j][q] & 0x7FFF7FFFu;
        m = max(m, max(w & 0xFFFFu, w >> 16));
      }
      pmax[piece_row(i) * (a.P / 8) + piece_col8(i)] = m;
    }
  }
}

// Part 2 (all threads, after a barrier that follows part 1; returns with the workgroup
// synchronised): the row scales and xs.
template <bool TS>
__device__ __forceinline__ void xs_build(const KArgs& a, const u32x4 (&v)[8], uint16_t* xs, int xstride,
                                         const uint32_t* pmax, int32_t* xk) {
  const int T = a.T, tid = threadIdx.x, per_row = a.P / 8, n = T * per_row;
  const bool cw = tid < kCompute, fp4 = a.fmt == 1;
  const int lane = tid & 63, wave = tid >> 6;
  if (fp4) {
    for (int t = wave; cw && t < T; t += 8) {
      uint32_t m = 0;
      for (int i = lane; i < per_row; i += 64) m = max(m, pmax[t * per_row + i]);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
      // bf16 exponent field E: the row maximum lies in [2^(E-127), 2^(E-126))
      if (lane == 0) xk[t] = m == 0 ? 0 : min(126, max(-126, 141 - (int)(m >> 7)));
    }
    wg_sync();
    stamp<TS>(a.timestamps, 50, 0);
  }
  if (cw) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = j * kCompute + tid;
      if (i < 16 * per_row && piece_row(i) < T) {
        const int t = piece_row(i), c = piece_col8(i);
        u32x4 o = v[j];
        if (fp4) {
          const float f = __uint_as_float((uint32_t)(127 + xk[t]) << 23);   // 2^xk[t], exact
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float lo = __uint_as_float(v[j][q] << 16) * f, hi = __uint_as_float(v[j][q] & 0xFFFF0000u) * f;
            o[q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
          }
        }
        *(u32x4*)(xs + t * xstride + c * 8) = o;
      }
    }
  }
  wg_sync();
}

// Two sequences (32 rows, NVFP4 experts): the row scales from all of xp's two 16-row tiles
// (piece maxima in `pmax`, [32][P/8]), then GEMM1's input rows for columns [c_lo, c_lo + ncol)
// (all of them, or one K half when 32 rows of P do not fit), reloaded from xp.  Called by all
// threads; both return synchronised.
template <bool TS>
__device__ __forceinline__ void xs_rowscale2(const KArgs& a, uint32_t* pmax, int32_t* xk) {
  const int tid = threadIdx.x, per_row = a.P / 8, n = 16 * per_row;
  const bool cw = tid < kCompute;
  const int lane = tid & 63, wave = tid >> 6;
  for (int r = 0; r < 2; ++r) {
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = j * kCompute + tid;
      if (cw && i < n) v[j] = ld16(st_xp(a) + (size_t)r * 16 * a.P + (size_t)i * 8);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = j * kCompute + tid;
      if (cw && i < n) {
        uint32_t m = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w = v[j][q] & 0x7FFF7FFFu;
          m = max(m, max(w & 0xFFFFu, w >> 16));
        }
        pmax[(16 * r + piece_row(i)) * per_row + piece_col8(i)] = m;
      }
    }
  }
  wg_sync();
  for (int t = wave; cw && t < 32; t += 8) {
    uint32_t m = 0;
    for (int i = lane; i < per_row; i += 64) m = max(m, pmax[t * per_row + i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    if (lane == 0) xk[t] = m == 0 ? 0 : min(126, max(-126, 141 - (int)(m >> 7)));
  }
  wg_sync();
}
__device__ __forceinline__ void xs_fill2(const KArgs& a, uint16_t* xs, int xstride, int c_lo, int ncol,
                                         const int32_t* xk) {
  const int tid = threadIdx.x, per_row = a.P / 8, n = 16 * per_row;
  if (tid >= kCompute) return;
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = j * kCompute + tid;
      const int c = piece_col8(i) * 8;
      if (i < n && c >= c_lo && c < c_lo + ncol) {
        const int t = 16 * r + piece_row(i);
        const u32x4 v = ld16(st_xp(a) + (size_t)r * 16 * a.P + (size_t)i * 8);
        const float f = __uint_as_float((uint32_t)(127 + xk[t]) << 23);   // 2^xk[t], exact
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = __uint_as_float(v[q] << 16) * f, hi = __uint_as_float(v[q] & 0xFFFF0000u) * f;
          o[q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
        }
        *(u32x4*)(xs + t * xstride + (c - c_lo)) = o;
      }
    }
  }
}

// NVFP4 experts whose local intermediate is a multiple of 64 and at least 128 take gemm2_fp4;
// the others gemm2_staged
__device__ __forceinline__ bool g2_fast(const KArgs& a) { return a.fmt == 1 && a.I % 64 == 0 && a.I >= 128; }

// LDS of GEMM1: the input rows xs [T][P + 8] at 0, then 16 P bytes of piece scales (sbuf; the
// piece maxima while xs is built), then the partial tiles (ubuf).  The routing tables are built
// in the ubuf area, before GEMM1's first products.
__device__ __forceinline__ int g1_ubuf_off(int P) { return G1_XS_BYTES + 16 * P; }

template <bool TS, class RT>
__device__ __forceinline__ void gemm1_phase(const KArgs& a, const RT& rt, char* smem, int32_t* xk) {
  const int P = a.P, I = a.I, K = a.topk, T = a.T, tid = threadIdx.x;
  const bool cw = tid < kCompute;
  const int jblocks = I / 16;
  const int ntasks = rt.n_active * jblocks;
  const int nwg = gridDim.x;
  // contiguous shares of ntasks / nwg tasks, one more for ntasks % nwg workgroups; those extra
  // tasks go to the workgroups after the first T first (the first T published the routing and
  // start GEMM1 late), so that no share grows
  const int base = ntasks / nwg, rem = ntasks % nwg, npub = min(T, nwg);
  const int rem_o = min(rem, nwg - npub), rem_p = rem - rem_o;
  auto share_start = [&](int w) {
    return w * base + (w < npub ? min(w, rem_p) : rem_p + min(w - npub, rem_o));
  };
  const int t_begin = share_start(blockIdx.x), t_end = share_start(blockIdx.x + 1);
  if (t_begin >= t_end) return;                 // uniform over the workgroup
  const int nh = g1_pieces(P);                                   // pieces per unit
  const int hsteps = g1_hsteps(P);                               // load steps per piece (<= 8)
  // Two sequences of 16 with two pieces per unit: 32 rows of P do not fit, so xs holds one K
  // half -- the columns of pieces hf -- at a time (half 0 built before routing): a round runs
  // every half-0 piece, swaps in half 1 between two barriers, then runs the half-1 pieces, with
  // pieces dealt half-major (piece pc: unit pc % nu, half pc / nu).
  constexpr int NRT = RT::kPairs / 128;
  const bool kh = NRT == 2 && nh == 2;
  const int xstride = (kh ? hsteps * 128 : P) + XS_STRIDE_PAD;
  uint16_t* xs = (uint16_t*)smem;                                  // [T][cols + 8], built before routing
  // sbuf: the wave-private piece-scale buffers (16 rows x srow_b bytes each, 2 per wave: within
  // 16 P bytes for every P % 128 == 0 up to 2048)
  uint8_t* sbuf = (uint8_t*)(smem + G1_XS_BYTES);                  // 16 P bytes
  float* ubuf = (float*)(smem + g1_ubuf_off(P));                    // [16 units][2 K halves][16][17]
  const int lane = tid & 63, wave = tid >> 6, nl = lane & 15, grp = lane >> 4;
  const int lsteps = g1_lsteps(P);
  const int nunits = 2 * (t_end - t_begin);
  // NVFP4: a round's units are split into pieces (unit, K half) dealt to the compute waves
  // round-robin (piece pc: unit pc / nh, half pc % nh), so the waves carry equal work.  A wave
  // streams its pieces with the next piece's codes and block scales in flight while the
  // current one is multiplied; each piece leaves its partial tile in ubuf[unit][half].
  const int srow_b = g1_sb(P);                                   // scale bytes per row and piece
  auto piece_uh = [&](int u0, int pc, int& u, int& hf) {
    if (kh) {
      const int nu = min(G1_UNITS, nunits - u0);
      u = pc % nu;
      hf = pc / nu;
    } else {
      u = pc / nh;
      hf = pc % nh;
    }
  };
  // (two K halves) all threads: xs becomes the columns of pieces `h`
  auto xs_swap = [&](int h) {
    wg_sync();
    xs_fill2(a, xs, xstride, h * hsteps * 128, hsteps * 128, xk);
    wg_sync();
  };
  u32x4 cA[8], cB[8], sA, sB;
  // Piece pc of the round at unit u0 into cd / sv.  A piece that does not exist (`real` false)
  // loads the first bytes of W1 at one address for all lanes instead: a few cache lines whose
  // data is discarded.  Every lane of every wave thus issues the same loads in the same order
  // whatever its pieces, which keeps the compiler's load counters exact: a piece is waited for
  // while the next one stays in flight.  Past-the-end k-steps of a piece load its last k-step.
  auto load_piece = [&](int u0, int pc, bool real, u32x4 (&cd)[8], u32x4& sv) {
    const int pcr = real ? pc : 0;
    int u, hf;
    piece_uh(u0, pcr, u, hf);
    const int task = t_begin + (u0 + u) / 2, half = (u0 + u) & 1;
    const int ai = task / jblocks, j0 = (task % jblocks) * 16;
    // W1 is in GEMM1's operand order: k-step ls of the 16-row tile is 1 KB, lane l's 16 B at
    // 16 l; the piece's scales are 16 rows x srow_b bytes, one contiguous block
    const size_t tile = ((size_t)rt.act_expert[ai] * 2 * I + half * I + j0) / 16;
    const uint8_t* cp = real ? a.w1_codes + (tile * lsteps + hf * hsteps) * 1024 + lane * 16 : a.w1_codes;
    const uint8_t* spp = real ? a.w1_scales + (tile * nh + hf) * 16 * srow_b + min(lane * 16, 16 * srow_b - 16)
                              : a.w1_scales;
    // expert codes are read once per launch: non-temporal loads keep the stream from evicting
    // the hand-off activations every workgroup re-reads from L2 (about 1.5 us per layer)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ls = min(hf * hsteps + min(j, hsteps - 1), lsteps - 1) - hf * hsteps;
      cd[j] = __builtin_nontemporal_load((const u32x4*)(cp + (real ? ls : min(j, lsteps - 1)) * 1024));
    }
    sv = ld16(spp);
  };
  // SwiGLU + requantisation of the round at unit u0 (nu units, nu even).  A wave takes one task
  // (16 intermediate columns) at a time: lane = 4 m + q holds token row m, columns 4q..4q+3, so
  // a 16-column block's E4M3 scale is a maximum over a lane quad (DPP) and its 64-bit code word
  // is gathered into the quad's first lane.
  auto swiglu_round = [&](int u0, int nu) {
    const int m = lane >> 2, q = lane & 3;
    for (int tl = wave; cw && tl < nu / 2; tl += 8) {
      const int task = t_begin + u0 / 2 + tl;
      const int ai = task / jblocks, j0 = (task % jblocks) * 16;
      const bool valid = m < rt.act_cnt[ai];
      const int pair = valid ? rt.pair_list[rt.act_off[ai] + m] : 0;
      // the two K halves of the gate unit (2 tl) and of the up unit (2 tl + 1)
      const float* ug = ubuf + (4 * tl) * (16 * 17) + m * 17 + 4 * q;
      const float* uu = ubuf + (4 * tl + 2) * (16 * 17) + m * 17 + 4 * q;
      // NVFP4: the tensor scale, and undo the token row's power-of-two input scale (exact)
      const float f = a.fmt == 1 ? rt.ts1[rt.act_expert[ai]] * __uint_as_float((uint32_t)(127 - xk[pair / K]) << 23)
                                 : 1.0f;
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float g = (ug[j] + ug[16 * 17 + j]) * f;
        v[j] = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * ((uu[j] + uu[16 * 17 + j]) * f);
      }
      if (a.fmt == 1) {
        float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
        amax = fmaxf(amax, dpp_f32<0xB1>(amax));   // quad_perm [1,0,3,2]
        amax = fmaxf(amax, dpp_f32<0x4E>(amax));   // quad_perm [2,3,0,1]
        const uint32_t sc = e4m3_code_of_amax_over6(amax);
        const float sv = e4m3_to_f32(sc);
        uint32_t c = 0;
        if (sv > 0.f) {
#pragma unroll
          for (int j = 0; j < 4; ++j) c |= e2m1_code(v[j], sv) << (4 * j);
        }
        // codes of columns 8h..8h+7 on lanes q = 2h; the odd lane's half shifted in
        const uint32_t w = c | ((uint32_t)__builtin_amdgcn_update_dpp((int)c, (int)c, 0xB1, 0xF, 0xF, true) << 16);
        const uint32_t w1 = (uint32_t)__builtin_amdgcn_update_dpp((int)w, (int)w, 0x4E, 0xF, 0xF, true);
        // record: codes of elements 0-7 and the scale byte, codes of 8-15 and the scale byte
        // (each 8-byte half holds the scale, at most 0x7E, so neither is ever all ones)
        // (N-sharded layout: this rank's slice of the pair's gathered row)
        uint32_t* dst = a.ns_R ? a.act_recv + ((size_t)pair * (a.ns_R * I / 16) + a.ns_r * (I / 16) + j0 / 16) * 4
                               : st_act_q(a) + ((size_t)pair * (I / 16) + j0 / 16) * 4;
        if (valid && q == 0) st_coh_u128(dst, u32x4{w, sc, w1, sc});
      } else if (valid) {
        st_coh_u64(st_act_bf(a) + (size_t)pair * I + j0 + 4 * q, pack4_bf16(v));
      }
    }
  };
  // The first round's first piece is requested by every wave (the control wave's is a dummy).
  // Nothing useful is in flight here: the explicit wait lets the compiler's load counters start
  // from zero, so later waits count these loads exactly.
  if (a.fmt == 1) {
    __builtin_amdgcn_s_waitcnt(0);
    load_piece(0, wave, cw && wave < nh * min(G1_UNITS, nunits), cA, sA);
  }
  stamp<TS>(a.timestamps, 49, 0);
  for (int u0 = 0; u0 < nunits; u0 += G1_UNITS) {
    const int nu = min(G1_UNITS, nunits - u0);
    if (kh && u0 > 0) xs_swap(0);                 // (the last round ended on half 1)
    bool swapped = false;
    if (cw && a.fmt == 1) {
      const int npc = nh * nu;
      const int my = wave < npc ? (npc - 1 - wave) / 8 + 1 : 0;     // this wave's pieces
      const int mmax = (npc + 7) / 8;                                // wave 0's: uniform
      if (u0 > 0) load_piece(u0, wave, wave < npc, cA, sA);
      // piece jj of this wave (pc = wave + 8 jj) from cd / sv into ubuf[unit][half]; x picks
      // the wave's scale buffer
      auto piece_mma = [&](int jj, const u32x4 (&cd)[8], const u32x4& sv, int x) {
        const int pc = wave + 8 * jj;
        int u, hf;
        piece_uh(u0, pc, u, hf);
        const int task = t_begin + (u0 + u) / 2;
        const int ai = task / jblocks;
        const int cnt = rt.act_cnt[ai], off = rt.act_off[ai];
        // the piece's scales into this wave's LDS buffer (wave-private: no barrier)
        uint8_t* sd = sbuf + (wave * 2 + x) * 16 * srow_b;
        if (lane * 16 < 16 * srow_b) *(u32x4*)(sd + lane * 16) = sv;
        // rows past the expert's tokens read token 0 and are discarded after the product
        const uint16_t* xrow = xs + (nl < cnt ? rt.pair_list[off + nl] / K : 0) * xstride + grp * 32;
        const uint8_t* srow = sd + nl * srow_b + grp * 2;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int ls = hf * hsteps + k;
          if (k < hsteps && ls < lsteps) {
            const uint32_t sc = *(const uint16_t*)(srow + k * 8);
            const f16x2_t s0 = e4m3_to_f16x2(sc & 0xFF), s1 = e4m3_to_f16x2(sc >> 8);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const u32x4 xa = *(const u32x4*)(xrow + (kh ? k : ls) * 128 + q * 8);
              acc = mfma_f16(xa, fp4x8_to_f16(cd[k][q], q < 2 ? s0 : s1), acc);
            }
          }
        }
        float* ub = ubuf + (2 * u + hf) * (16 * 17);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          ub[(4 * grp + r) * 17 + nl] = acc[r];
          if (nh == 1) ub[16 * 17 + (4 * grp + r) * 17 + nl] = 0.f;
        }
      };
      // two pieces per trip, each loaded one piece ahead; the loads do not depend on which
      // pieces exist, only the products do
      // (two K halves: the swap to half 1 before this wave's first half-1 piece)
      auto maybe_swap = [&](int jj) {
        if (kh && !swapped && wave + 8 * jj >= nu) {
          xs_swap(1);
          swapped = true;
        }
      };
#pragma unroll 1
      for (int j = 0; j < mmax; j += 2) {
        load_piece(u0, wave + 8 * (j + 1), j + 1 < my, cB, sB);
        if (j < my) {
          maybe_swap(j);
          piece_mma(j, cA, sA, 0);
        }
        load_piece(u0, wave + 8 * (j + 2), j + 2 < my, cA, sA);
        if (j + 1 < my) {
          maybe_swap(j + 1);
          piece_mma(j + 1, cB, sB, 1);
        }
      }
    } else if (cw) {
      // bf16 experts: rows loaded as they are used
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int u = wave + 8 * h;
        if (u < nu) {
          const int task = t_begin + (u0 + u) / 2, half = (u0 + u) & 1;
          const int ai = task / jblocks, j0 = (task % jblocks) * 16;
          const int cnt = rt.act_cnt[ai], off = rt.act_off[ai];
          const bool mv = nl < cnt;
          const uint16_t* xrow = xs + (mv ? rt.pair_list[off + nl] / K : 0) * xstride + grp * 8;
          const uint16_t* wr = a.w1 + ((size_t)rt.act_expert[ai] * 2 * I + half * I + j0 + nl) * P + grp * 8;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          for (int st = 0; st < P / 32; ++st) {
            const u32x4 xa = mv ? *(const u32x4*)(xrow + st * 32) : u32x4{0, 0, 0, 0};
            acc = mfma_bf16(xa, ld16(wr + st * 32), acc);
          }
          float* ub = ubuf + (2 * u) * (16 * 17);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            ub[(4 * grp + r) * 17 + nl] = acc[r];
            ub[16 * 17 + (4 * grp + r) * 17 + nl] = 0.f;
          }
        }
      }
    }
    if (kh && !swapped) xs_swap(1);               // every wave takes part in the swap once
    wg_sync();
    if (u0 == 0) stamp<TS>(a.timestamps, 45, 0);
    swiglu_round(u0, nu);
    wg_sync();
  }
}

// ---- GEMM2 for NVFP4 experts: output columns [c0, c0+8) of P per workgroup
//
// Work comes in slots of at most 8 (token, slot) pairs of one expert (an expert with more
// than 8 pairs has two slots).  Unit U is the slot pair (2U, 2U+1), one 16x16 MFMA tile:
// token rows 0-7 and weight columns 0-7 belong to slot 2U, rows 8-15 and columns 8-15 to slot
// 2U+1, and the off-diagonal blocks are discarded.  Wave w takes units w, w+8, ...  Lane
// (nl, grp) holds weight row c0 + nl % 8 of its column's expert for the quarter k in
// [grp I/4, (grp+1) I/4) of the reduction: I/8 bytes of codes and I/64 E4M3 block scales,
// loaded straight into registers (a wave's first G2_UNITS units as soon as its workgroup's
// GEMM1 work ends).  The intermediate is read in the same permuted k order, which MFMA allows.
// Requires I % 64 == 0 and I >= 128.
constexpr int G2_UNITS = 2;   // units per register batch (4 and 3 measured slower)
constexpr int G2_MAXB = 4;    // I/64 <= 4
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
struct G2W {
  u32x2 c[G2_UNITS][G2_MAXB];
  u32x2 s[G2_UNITS];          // an 8-byte window of the row's scale bytes holding the lane's
};

// The lane's I/64 E4M3 scale bytes of a W2 row (I/16 bytes, I >= 128) come from one 8-byte
// window inside the row: it starts at the 4-aligned offset g2_swin(I, grp) and the lane's
// bytes begin g2_sshift(I, grp) bytes into it.
__device__ __forceinline__ int g2_swin(int I, int grp) { return min((grp * (I / 64)) & ~3, I / 16 - 8); }
__device__ __forceinline__ int g2_sshift(int I, int grp) { return grp * (I / 64) - g2_swin(I, grp); }
__device__ __forceinline__ uint32_t g2_sbyte(u32x2 win, int k) {
  return (uint32_t)((((uint64_t)win[1] << 32) | win[0]) >> (8 * k)) & 0xFFu;
}

// Loads unit U into register slot `i` of `w` for columns [c0, c0+8).  Compute waves only;
// `rt` must hold this launch's routing.
template <class RT>
__device__ __forceinline__ void g2_load_unit(const KArgs& a, const RT& rt, int c0, int U, G2W& w, int i) {
  const int lane = threadIdx.x & 63, nl = lane & 15, grp = lane >> 4;
  const int I = a.I, nb = I / 64, ns = rt.n_slots;
  if (2 * U < ns) {                                              // uniform over the wave
    const int sl = (nl >= 8 && 2 * U + 1 < ns) ? 2 * U + 1 : 2 * U;
    const size_t row = (size_t)rt.slot_expert[sl] * a.P + c0 + (nl & 7);
    const uint8_t* cp = a.w2_codes + row * (I / 2) + grp * (I / 8);   // 8-byte aligned
    // read once per launch, non-temporal as GEMM1's W1 codes (about 1.8 us per layer)
#pragma unroll
    for (int b = 0; b < G2_MAXB; ++b)
      if (b < nb) w.c[i][b] = __builtin_nontemporal_load((const u32x2*)(cp + 8 * b));
    const u32x2_a4 sw = __builtin_nontemporal_load((const u32x2_a4*)(a.w2_scales + row * (I / 16) + g2_swin(I, grp)));
    w.s[i] = u32x2{sw[0], sw[1]};
  }
}

// Batch `batch` of this wave: units wave + 8 (G2_UNITS batch + i), i < G2_UNITS.
template <class RT>
__device__ __forceinline__ void g2_load(const KArgs& a, const RT& rt, int c0, int batch, G2W& w) {
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < G2_UNITS; ++i) g2_load_unit(a, rt, c0, wave + 8 * (G2_UNITS * batch + i), w, i);
}

// One unit from register slot `i` of `w`.  urow[U][m] is the pair on token row m (-1: none).
// Writes the expert outputs (before gates) to outp[pair][8].
template <class RT>
__device__ __forceinline__ void g2_unit(const KArgs& a, const RT& rt, const G2W& w, int i, int U,
                                        const int32_t* urow, const uint16_t* actf, int astride, float* outp) {
  const int lane = threadIdx.x & 63, nl = lane & 15, grp = lane >> 4;
  const int I = a.I;
  const int32_t* ur = urow + U * 16;
  const int pair_m = ur[nl];
  // rows without a pair read pair 0; their outputs are discarded
  const uint16_t* arow = actf + (pair_m < 0 ? 0 : pair_m) * astride + grp * (I / 4);
  const int sl = (nl >= 8 && 2 * U + 1 < rt.n_slots) ? 2 * U + 1 : 2 * U;
  const float ts = rt.ts2[rt.slot_expert[sl]];
  const int sh = g2_sshift(I, grp);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < 2 * G2_MAXB; ++st) {
    if (st < I / 32) {
      const u32x4 x = *(const u32x4*)(arow + 8 * st);
      acc = mfma_f16(x, fp4x8_to_f16(w.c[i][st / 2][st & 1], e4m3_to_f16x2(g2_sbyte(w.s[i], sh + st / 2))), acc);
    }
  }
  // C lane: weight column nl, token rows 4 grp + r; keep the diagonal blocks
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * grp + r;
    const int pair = ur[row];
    if (pair >= 0 && (row >> 3) == (nl >> 3)) outp[pair * 8 + (nl & 7)] = acc[r] * ts;
  }
}

// Called by all threads.  `w0` holds batch 0 of this workgroup's first slice, requested as
// soon as this workgroup's GEMM1 work ended.
template <bool TS, class RT>
__device__ __forceinline__ void gemm2_fp4(const KArgs& a, const RT& rt, char* smem, uint32_t* ytile, G2W& w0,
                                          const Sync& sy, int32_t* dead_sh) {
  const int P = a.P, I = a.I, K = a.topk, T = a.T, tid = threadIdx.x;
  const bool cw = tid < kCompute;
  const int nwg = gridDim.x, nslices = P / 8;
  if ((int)blockIdx.x >= nslices) return;       // uniform over the workgroup
  const int npairs = T * K, ns = rt.n_slots, nu = (ns + 1) / 2;
  const int astride = I + 8;                                        // fp16 per pair row in LDS
  uint16_t* actf = (uint16_t*)smem;                                 // [pairs][I + 8]
  const int actb = (npairs * astride * 2 + 255) & ~255;
  float* outp = (float*)(smem + actb);                              // [pairs][8]
  int32_t* urow = (int32_t*)(smem + actb + RT::kPairs * 8 * 4);     // [units][16]
  const int wave = tid >> 6;
  for (int sl = blockIdx.x; sl < nslices; sl += nwg) {
    const int c0 = sl * 8;
    const bool first = sl == (int)blockIdx.x;
    if (first) {
      // token-row tables of the units
      for (int e = tid; cw && e < nu * 16; e += kCompute) {
        const int s2 = 2 * (e >> 4) + ((e >> 3) & 1), j = e & 7;
        urow[e] = (s2 < ns && j < rt.slot_cnt[s2]) ? rt.pair_list[rt.slot_off[s2] + j] : -1;
      }
      // the intermediate, read as it arrives from GEMM1: one 16-element block (codes and scale
      // byte) per record, decoded once
      const int nblk = npairs * (I / 16);                           // <= 4096
      if (cw)
        poll_stage<4>(sy, dead_sh, make_rsrc(st_act_q(a), (uint32_t)nblk * 16), nblk, tid, kCompute,
                      [](int i) { return (uint32_t)i * 16u; }, [&](int i, u32x4 v) {
                        const int pair = i / (I / 16), b = i % (I / 16);
                        const f16x2_t sc = e4m3_to_f16x2(v[1]);
                        uint16_t* dst = actf + pair * astride + b * 16;
                        *(u32x4*)dst = fp4x8_to_f16(v[0], sc);
                        *(u32x4*)(dst + 8) = fp4x8_to_f16(v[2], sc);
                      });
    } else if (cw) {
      g2_load(a, rt, c0, 0, w0);
    }
    wg_sync();
    if (first) stamp<TS>(a.timestamps, 42, 0);
    if (cw) {
      // batches of G2_UNITS units from the registers; each slot is refilled with the next
      // batch's unit as soon as it is used
      for (int b = 0; wave + 8 * G2_UNITS * b < nu; ++b) {
#pragma unroll
        for (int i = 0; i < G2_UNITS; ++i) {
          const int U = wave + 8 * (G2_UNITS * b + i);
          if (U < nu) g2_unit(a, rt, w0, i, U, urow, actf, astride, outp);
          g2_load_unit(a, rt, c0, U + 8 * G2_UNITS, w0, i);
        }
        if (first && b == 0) stamp<TS>(a.timestamps, 48, 0);
      }
    }
    wg_sync();
    if (first) stamp<TS>(a.timestamps, 43, 0);
    if (tid < T) {
      float y[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) y[c] = 0.f;
      for (int j = 0; j < K; ++j) {
        const float gt = rt.gate[tid * K + j];
        const float* o = outp + (tid * K + j) * 8;
#pragma unroll
        for (int c = 0; c < 8; ++c) y[c] += gt * o[c];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) ytile[tid * 4 + q] = pack_bf2(y[2 * q], y[2 * q + 1]);
    }
    wg_sync();
    if (tid >= kCompute && (tid - kCompute) < T) {
      const int t = tid - kCompute;
      uint16_t* dst = st_y(a) + (size_t)(t >> 4) * 16 * a.P + frag_off(t & 15, c0);   // 8 columns: 16 contiguous bytes
      st_coh_u64(dst, (uint64_t)ytile[t * 4] | ((uint64_t)ytile[t * 4 + 1] << 32));
      st_coh_u64(dst + 4, (uint64_t)ytile[t * 4 + 2] | ((uint64_t)ytile[t * 4 + 3] << 32));
    }
  }
}

// ---- GEMM2 of the N-sharded expert layout: rank r of R computes output columns
// [r P/R, (r+1) P/R) over the gathered intermediate (K2 = R I, the R ranks' NVFP4 slices in
// rank order, read from the receive buffer as they arrive), then combines its columns locally
// and writes them into the gathered y, where the other ranks' columns arrive the same way.
//
// Work: the unit tiles of gemm2_fp4 (two slots of <= 8 pairs, 8 columns each), dealt out as
// tasks (unit U, column block cb of 8 of the P/R columns), task U (P/(8R)) + cb, in contiguous
// ranges per workgroup: a workgroup's tasks span at most two units (the host checks that the
// grid covers P/(8R) blocks and T k / 2 units), so it decodes only those units' gathered rows
// (<= 32 rows of K2) into LDS.  Lane (nl, grp) holds W2 row c0 + nl % 8 of its slot's expert
// for the quarter [grp K2/4, (grp+1) K2/4) of the reduction, streamed in chunks of 64 values
// (32 code bytes, 4 scale bytes; NS_CH chunks in flight per wave); the intermediate is read in
// the same permuted k order.  Each task writes its products before gates as fp32 partials
// part[pair][c]; a combine step per column block then sums the 8 slots per token in slot order,
// reading the partials as they arrive.  Requires K2 % 256 == 0 and P % (8 R) == 0.
constexpr int NS_CH = 4;

template <bool TS, class RT>
__device__ __forceinline__ void gemm2_ns(const KArgs& a, const RT& rt, char* smem, uint32_t* ytile, const Sync& sy,
                                         int32_t* dead_sh) {
  const int R = a.ns_R, K2 = R * a.I, N2 = a.P / R, K = a.topk, T = a.T, tid = threadIdx.x;
  const bool cw = tid < kCompute;
  const int lane = tid & 63, wave = tid >> 6, nl = lane & 15, grp = lane >> 4;
  const int nblk = N2 / 8, ns = rt.n_slots, npairs = T * K;
  const long nt = (long)((ns + 1) / 2) * nblk;
  const int tb = (int)(nt * blockIdx.x / gridDim.x), te = (int)(nt * (blockIdx.x + 1) / gridDim.x);
  const int Ub = tb / nblk, nloc = te > tb ? (te - 1) / nblk - Ub + 1 : 0;      // <= 2
  const int astride = K2 + 8;
  uint16_t* actf = (uint16_t*)smem;                                   // [32][K2 + 8] fp16
  const int actb = 32 * astride * 2;
  float* outp = (float*)(smem + actb);                                // [pairs][8] (combine)
  int32_t* urow = (int32_t*)(smem + actb + 128 * 8 * 4);              // [32]: pair or -1
  int32_t* vrow = urow + 32;                                          // local rows with a pair
  int32_t* nvrow = vrow + 32;
  // local row (U - Ub) 16 + m: slot 2U's m-th pair (m < 8) or slot 2U+1's (m - 8)-th
  if (tid < 64) {
    const int lr = tid, U = Ub + (lr >> 4), m = lr & 15, s2 = 2 * U + (m >> 3), j = m & 7;
    const int pr = (lr < 16 * nloc && s2 < ns && j < rt.slot_cnt[s2]) ? rt.pair_list[rt.slot_off[s2] + j] : -1;
    const uint64_t has = __ballot(lr < 32 && pr >= 0);
    if (lr < 32) urow[lr] = pr;
    if (lr < 32 && pr >= 0) vrow[__popcll(has & ((1ull << lr) - 1ull))] = lr;
    if (lr == 0) *nvrow = __popcll(has);
  }
  wg_sync();
  // the units' gathered intermediate rows, as they arrive, decoded once into actf
  const int RB = K2 / 16, nrec = *nvrow * RB;
  if (cw && nrec > 0)
    poll_stage<4>(sy, dead_sh, make_rsrc(a.act_recv, (uint32_t)(npairs * RB) * 16u), nrec, tid, kCompute,
                  [&](int i) { return (uint32_t)(urow[vrow[i / RB]] * RB + i % RB) * 16u; }, [&](int i, u32x4 v) {
                    const f16x2_t sc = e4m3_to_f16x2(v[1]);
                    uint16_t* dst = actf + vrow[i / RB] * astride + (i % RB) * 16;
                    *(u32x4*)dst = fp4x8_to_f16(v[0], sc);
                    *(u32x4*)(dst + 8) = fp4x8_to_f16(v[2], sc);
                  });
  wg_sync();
  stamp<TS>(a.timestamps, 42, 0);
  const int kq = K2 / 4, nch = kq / 64;
  float* part = st_g2_part(a);
  if (cw && *dead_sh == 0) {
    const int my = te - tb > wave ? (te - tb - wave + 7) / 8 : 0;     // this wave's tasks
    const int nflat = my * nch;                                       // (task, chunk) in order
    u32x4 c0b[NS_CH], c1b[NS_CH];
    uint32_t scb[NS_CH];
    auto task_of = [&](int f, int& U, int& c0, int& e) {
      const int tau = tb + wave + 8 * (f / nch);
      U = tau / nblk;
      c0 = (tau % nblk) * 8;
      const int sl = (nl >= 8 && 2 * U + 1 < ns) ? 2 * U + 1 : 2 * U;
      e = rt.slot_expert[sl];
    };
    auto load_chunk = [&](int f, u32x4& x0, u32x4& x1, uint32_t& sv) {
      if (f < nflat) {
        int U, c0, e;
        task_of(f, U, c0, e);
        const int c = f % nch;
        const size_t row = (size_t)e * N2 + c0 + (nl & 7);
        const uint8_t* cp = a.w2_codes + row * (K2 / 2) + grp * (K2 / 8) + 32 * c;
        x0 = __builtin_nontemporal_load((const u32x4*)cp);
        x1 = __builtin_nontemporal_load((const u32x4*)(cp + 16));
        sv = __builtin_nontemporal_load((const uint32_t*)(a.w2_scales + row * (K2 / 16) + grp * (K2 / 64) + 4 * c));
      }
    };
#pragma unroll
    for (int q = 0; q < NS_CH; ++q) load_chunk(q, c0b[q], c1b[q], scb[q]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int f0 = 0; f0 < nflat; f0 += NS_CH) {
#pragma unroll
      for (int q = 0; q < NS_CH; ++q) {
        const int f = f0 + q;
        if (f < nflat) {
          int U, c0, e;
          task_of(f, U, c0, e);
          const int c = f % nch, lb = (U - Ub) * 16;
          // a local row without a pair holds stale LDS: its products land in discarded rows
          const uint16_t* arow = actf + (lb + nl) * astride + grp * kq + 64 * c;
#pragma unroll
          for (int st = 0; st < 8; ++st) {
            const u32x4 x = *(const u32x4*)(arow + 8 * st);
            const uint32_t cw4 = st < 4 ? c0b[q][st] : c1b[q][st - 4];
            acc = mfma_f16(x, fp4x8_to_f16(cw4, e4m3_to_f16x2((scb[q] >> (8 * (st / 2))) & 0xFFu)), acc);
          }
          if (c == nch - 1) {
            // C lane: weight column nl, token rows 4 grp + r; the diagonal blocks hold this
            // unit's (pair, column) products.  Even lanes store theirs with the odd neighbour's.
            const float ts = rt.ts2[e];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float v = acc[r] * ts;
              const float vn = dpp_f32<0xF5>(v);                    // lane nl + 1 (quad_perm 1,1,3,3)
              const int row = 4 * grp + r, pair = urow[lb + row];
              if (pair >= 0 && (row >> 3) == (nl >> 3) && (nl & 1) == 0)
                st_coh_u64(part + (size_t)pair * N2 + c0 + (nl & 7),
                           (uint64_t)__float_as_uint(v) | ((uint64_t)__float_as_uint(vn) << 32));
            }
            acc = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
        load_chunk(f + NS_CH, c0b[q], c1b[q], scb[q]);
      }
    }
  }
  wg_sync();
  stamp<TS>(a.timestamps, 43, 0);
  // combine: column blocks cb = blockIdx.x, + grid, ...: every pair's 8 partials, as they arrive
  for (int cb = blockIdx.x; cb < nblk && *dead_sh == 0; cb += gridDim.x) {
    const int c0 = cb * 8;
    if (cw)
      poll_stage<1>(sy, dead_sh, make_rsrc(part, (uint32_t)(npairs * N2) * 4u), 2 * npairs, tid, kCompute,
                    [&](int i) { return (uint32_t)((i >> 1) * N2 + c0 + 4 * (i & 1)) * 4u; },
                    [&](int i, u32x4 v) { *(u32x4*)(outp + (i >> 1) * 8 + 4 * (i & 1)) = v; });
    wg_sync();
    if (tid < T) {
      float y[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) y[c] = 0.f;
      for (int j = 0; j < K; ++j) {
        const float gt = rt.gate[tid * K + j];
        const float* o = outp + (tid * K + j) * 8;
#pragma unroll
        for (int c = 0; c < 8; ++c) y[c] += gt * o[c];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) ytile[tid * 4 + q] = pack_bf2(y[2 * q], y[2 * q + 1]);
    }
    wg_sync();
    if (tid >= kCompute && (tid - kCompute) < T) {
      const int t = tid - kCompute;
      uint16_t* dst = a.y_recv + frag_off(t, a.ns_r * N2 + c0);     // 8 columns: 16 contiguous bytes
      st_coh_u64(dst, (uint64_t)ytile[t * 4] | ((uint64_t)ytile[t * 4 + 1] << 32));
      st_coh_u64(dst + 4, (uint64_t)ytile[t * 4 + 2] | ((uint64_t)ytile[t * 4 + 3] << 32));
    }
  }
}

// ---- GEMM2 + combine, general form (bf16 experts, or NVFP4 with I % 64 != 0): output
// columns [c0, c0+8) of P.
//  * The fp4 intermediate of every (token, slot) pair is decoded once into LDS as bf16.
//  * The 8 weight rows of one expert for these columns are contiguous (codes, then scales);
//    the workgroup copies every active expert's rows into LDS with wide loads.
//  * Two experts share one 16x16 MFMA tile: rows 0-7 / columns 0-7 carry expert A's tokens
//    and columns, rows 8-15 / columns 8-15 expert B's, so every B-operand lane decodes real
//    weights; the off-diagonal blocks are discarded.  An expert with more than 8 tokens runs
//    alone (16 token rows, columns 0-7).
//  * Per token, the gate-weighted sum over its slots in slot order goes to LDS `ytile`
//    ([T][4] dwords of bf16 pairs) for the control wave to store.
// Called by all threads.
template <bool TS, class RT>
__device__ __forceinline__ void gemm2_staged(const KArgs& a, const RT& rt, char* smem, uint32_t* ytile,
                                             const Sync& sy, int32_t* dead_sh) {
  const int P = a.P, I = a.I, K = a.topk, T = a.T, tid = threadIdx.x;
  const bool cw = tid < kCompute;
  const int nwg = gridDim.x;
  const int nslices = P / 8;
  if ((int)blockIdx.x >= nslices) return;       // uniform over the workgroup
  const int npairs = T * K;
  const bool fp4 = a.fmt == 1;
  const int astride = I + 8;                                        // bf16 per pair row in LDS
  uint16_t* actbf = (uint16_t*)smem;                                // [pairs][I + 8]
  float* outp = (float*)(smem + ((npairs * astride * 2 + 255) & ~255));   // [pairs][8]
  char* wbuf = (char*)outp + 128 * 8 * 4;
  const int code_bytes = fp4 ? 8 * (I / 2) : 8 * I * 2;             // per expert, per slice
  const int chunk = code_bytes + (fp4 ? 8 * (I / 16) : 0);          // multiple of 16 (I % 32 == 0)
  const int cap = (LDS_BYTES - (int)(wbuf - smem)) / chunk;         // experts per round
  // the intermediate, read as it arrives from GEMM1 and decoded: one 16-element block (fp4
  // record) or 8 bf16 per 16-byte piece
  if (cw) {
    const int nblk = fp4 ? npairs * (I / 16) : npairs * (I / 8);
    const void* src = fp4 ? (const void*)st_act_q(a) : (const void*)st_act_bf(a);
    poll_stage<4>(sy, dead_sh, make_rsrc(src, (uint32_t)nblk * 16), nblk, tid, kCompute,
                  [](int i) { return (uint32_t)i * 16u; }, [&](int i, u32x4 v) {
                    if (fp4) {
                      const int pair = i / (I / 16), b = i % (I / 16);
                      const float sc = e4m3_to_f32(v[1]);
                      uint16_t* dst = actbf + pair * astride + b * 16;
                      *(u32x4*)dst = fp4x8_to_bf16(v[0], sc);
                      *(u32x4*)(dst + 8) = fp4x8_to_bf16(v[2], sc);
                    } else {
                      const int pair = i / (I / 8), b = i % (I / 8);
                      *(u32x4*)(actbf + pair * astride + b * 8) = v;
                    }
                  });
  }
  const int lane = tid & 63, wave = tid >> 6, nl = lane & 15, grp = lane >> 4;
  const int ksteps = I / 32;
  const int pieces = chunk / 16, code_pieces = code_bytes / 16;
  for (int sl = blockIdx.x; sl < nslices; sl += nwg) {
    const int c0 = sl * 8;
    for (int a0 = 0; a0 < rt.n_active; a0 += cap) {
      const int na = min(cap, rt.n_active - a0);
      stage_pieces(na * pieces, [&](int p) {
        const int ai = a0 + p / pieces, q = p % pieces;
        const size_t row0 = (size_t)rt.act_expert[ai] * P + c0;
        if (!fp4) return (const void*)((const char*)a.w2 + row0 * I * 2 + q * 16);
        if (q < code_pieces) return (const void*)(a.w2_codes + row0 * (I / 2) + q * 16);
        return (const void*)(a.w2_scales + row0 * (I / 16) + (q - code_pieces) * 16);
      }, [&](int p) { return (void*)(wbuf + (size_t)(p / pieces) * chunk + (p % pieces) * 16); });
      wg_sync();
      if (sl == (int)blockIdx.x && a0 == 0) stamp<TS>(a.timestamps, 42, 0);
      // units: experts (2u, 2u+1) of this round together when both have <= 8 tokens
      const int nunits = (na + 1) / 2;
      for (int u = wave; cw && u < nunits; u += 8) {
        const int iA = a0 + 2 * u, iB = iA + 1;
        const bool hasB = iB < a0 + na;
        const int cA = rt.act_cnt[iA], cB = hasB ? rt.act_cnt[iB] : 0;
        const bool pairm = hasB && cA <= 8 && cB <= 8;
        for (int pass = 0; pass < (pairm || !hasB ? 1 : 2); ++pass) {
          // pass 0: expert A (with B when paired); pass 1: expert B alone
          const int ia = pass == 0 ? iA : iB;
          const int cnt_a = rt.act_cnt[ia], off_a = rt.act_off[ia];
          const int cnt_b = pairm ? cB : 0, off_b = pairm ? rt.act_off[iB] : 0;
          // B operand: column nl -> expert (nl < 8 ? ia : iB), weight row nl % 8; unpaired, the
          // columns 8..15 repeat expert ia's rows and their outputs are discarded
          const int ib = nl < 8 || !pairm ? ia : iB;
          const char* wc = wbuf + (size_t)(ib - a0) * chunk;
          // A operand: row m -> pair of expert ia (m < cnt_a, or m < 8 when paired) or iB
          int pair_m = -1;
          if (pairm) {
            if (nl < 8) { if (nl < cnt_a) pair_m = rt.pair_list[off_a + nl]; }
            else if (nl - 8 < cnt_b) pair_m = rt.pair_list[off_b + nl - 8];
          } else if (nl < cnt_a) {
            pair_m = rt.pair_list[off_a + nl];
          }
          const uint16_t* arow = actbf + (pair_m < 0 ? 0 : pair_m) * astride + grp * 8;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          if (fp4) {
            const char* crow = wc + (nl & 7) * (I / 2) + 4 * grp;
            const uint8_t* srow = (const uint8_t*)wc + code_bytes + (nl & 7) * (I / 16) + (grp >> 1);
#pragma unroll
            for (int st = 0; st < 8; ++st) {
              if (st < ksteps) {
                // rows without a pair read pair 0; their outputs are discarded
                const u32x4 x = *(const u32x4*)(arow + st * 32);
                const uint32_t wcv = *(const uint32_t*)(crow + 16 * st);
                const float ws = e4m3_to_f32(srow[2 * st]);
                acc = mfma_bf16(x, fp4x8_to_bf16(wcv, ws), acc);
              }
            }
          } else {
            const uint16_t* wr = (const uint16_t*)wc + (nl & 7) * I + grp * 8;
            for (int st = 0; st < ksteps; ++st) {
              const u32x4 b = *(const u32x4*)(wr + st * 32);
              const u32x4 x = *(const u32x4*)(arow + st * 32);
              acc = mfma_bf16(x, b, acc);
            }
          }
          // C lane: column nl, rows 4 grp + r; keep the diagonal block(s)
          float ts = 1.0f;
          if (fp4) ts = rt.ts2[rt.act_expert[ib]];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 4 * grp + r;
            int pair = -1;
            if (pairm) {
              if (nl < 8 && row < 8 && row < cnt_a) pair = rt.pair_list[off_a + row];
              else if (nl >= 8 && row >= 8 && row - 8 < cnt_b) pair = rt.pair_list[off_b + row - 8];
            } else if (nl < 8 && row < cnt_a) {
              pair = rt.pair_list[off_a + row];
            }
            if (pair >= 0) outp[pair * 8 + (nl & 7)] = acc[r] * ts;
          }
        }
      }
      wg_sync();
    }
    if (sl == (int)blockIdx.x) stamp<TS>(a.timestamps, 43, 0);
    if (tid < T) {
      float y[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) y[c] = 0.f;
      for (int j = 0; j < K; ++j) {
        const float gt = rt.gate[tid * K + j];
        const float* o = outp + (tid * K + j) * 8;
#pragma unroll
        for (int c = 0; c < 8; ++c) y[c] += gt * o[c];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) ytile[tid * 4 + q] = pack_bf2(y[2 * q], y[2 * q + 1]);
    }
    wg_sync();
    if (tid >= kCompute && (tid - kCompute) < T) {
      const int t = tid - kCompute;
      uint16_t* dst = st_y(a) + (size_t)(t >> 4) * 16 * a.P + frag_off(t & 15, c0);   // 8 columns: 16 contiguous bytes
      st_coh_u64(dst, (uint64_t)ytile[t * 4] | ((uint64_t)ytile[t * 4 + 1] << 32));
      st_coh_u64(dst + 4, (uint64_t)ytile[t * 4 + 2] | ((uint64_t)ytile[t * 4 + 3] << 32));
    }
  }
}

// ------------------------------------------------------------------ dense phases

// One dense phase: this workgroup's tiles t = first, first + n_wg, ...  Compute waves form
// the wave partials (weights of the first tile already in `wf` when `have_pref`), the control
// wave sums them and runs `epi(n0, red, it)`.  Two reduction buffers alternate so a tile needs
// one workgroup barrier.  Called by all threads.
// Loads for the next phase are not issued here but inside the hand-off wait that follows
// (phase_end's `pf`): issued before the hand-off, a large tile's loads hold the issuing waves
// until the CU's load queue drains, and the grid waits for them at the barrier.
template <int NRT, bool TS = false, int MAXS, class Epi>
__device__ __forceinline__ void dense_phase(const KArgs& a, WFrag<MAXS>& wf, bool have_pref, const uint16_t* W,
                            const XSrc& x, int K, int N, int off, float* red2, Epi epi,
                            const char* wlds = nullptr, int ev = -1) {
  const int n = gridDim.x, ntiles = N / 16;
  int it = 0;
  for (int t = first_tile(off); t < ntiles; t += n, ++it) {
    // every row tile (sequence) with the same weights: registers or LDS, loaded once
#pragma unroll
    for (int r = 0; r < NRT; ++r) {
      float* red = red2 + ((it * NRT + r) & 1) * (8 * 16 * 17);
      if (threadIdx.x < kCompute) {
        const XSrc xr = NRT == 1 ? x : xtile(x, r, K);
        const int Tr = min(16, a.T - 16 * r);
        f32x4 acc;
        if (wlds && it == 0) {
          acc = lds_mma(wlds, xr, Tr, K);                // the first tile's weights are in LDS
        } else if constexpr (MAXS == 0) {
          acc = stream_mma(W, K, t * 16, xr, Tr);
        } else {
          if (!(have_pref && it == 0) && r == 0) wfrag_load(wf, W, K, t * 16);
          acc = wfrag_mma(wf, xr, 0, Tr, K);
        }
        if (ev >= 0 && it == 0 && r == 0) stamp<TS>(a.timestamps, ev, 0);
        red_store(red, acc);
      }
      wg_sync();
      if (threadIdx.x >= kCompute) epi(t * 16, red, it, r);
    }
  }
}

// End of a phase: compute waves run `pf` (loads for a later phase, left in flight) while the
// control wave signals and waits for the whole grid (first sleeping `idle_us`, see
// ctl_signal_wait).  Returns true when the launch is still alive.  Called by all threads; every
// compute-wave global store of the phase must be complete before the call.
template <bool TS, class PfF>
__device__ __forceinline__ bool phase_end(const KArgs& a, const Sync& s, int phase, int32_t* dead_sh, PfF pf,
                                          int idle_us = 0, bool wait = true) {
  wg_sync();
  stamp<TS>(a.timestamps, 2 * phase);
  if (threadIdx.x >= kCompute) {
    if constexpr (TS) {
      // the control wave's hand-off stores complete (just before the flag is raised)
      __builtin_amdgcn_s_waitcnt(0);
      stamp<TS>(a.timestamps, 53 + phase);
    }
    const bool ok = ctl_signal_wait(s, phase, *dead_sh != 0, idle_us, wait);
    if (!ok && threadIdx.x == kCtl) *dead_sh = 1;
    stamp<TS>(a.timestamps, 20 + phase);
  } else {
    pf();
    stamp<TS>(a.timestamps, 28 + phase, 0);
  }
  wg_sync();
  stamp<TS>(a.timestamps, 2 * phase + 1);
  return *dead_sh == 0;
}

// ------------------------------------------------------------------ split-K qkv

// The next layer's qkv projection has few 16-column tiles (N = (Hq + 2 Hkv) d) but a long K
// (= H), and every tile reads all of x, so with one workgroup per tile a few workgroups would
// each pull a 16 x K weight tile and all of x (32 K bytes each) while the rest idle.  Instead
// each tile's K is cut into `np` parts of `ps` k-steps (a multiple of 8, so the 8 waves get
// equal blocks) on np workgroups.  Each part's control wave stores its fp32 partial (64 lanes
// x 4 values, the epilogue's layout) and counts itself in on the tile's counter; the part that
// arrives last adds the np partials in part order, so the sum does not depend on the arrival
// order, writes q, k and v.  Tile t's counter is cleared at the start of every launch by the
// control wave of workgroup t, whose store completes before it first signals; every part
// counts in only after the last grid hand-off, so it always finds the cleared counter (also
// after an aborted launch left it part-way).
struct QkvSplit {
  int np, ps;
};

__device__ __forceinline__ QkvSplit qkv_split(int ksteps, int ntiles, int nwg) {
  QkvSplit q{1, ksteps};
  if (ntiles <= 0) return q;
  int np = nwg / ntiles;
  np = np > 4 ? 4 : np;
  if (np < 2) return q;
  const int ps = ((ksteps + np - 1) / np + 7) & ~7;
  np = (ksteps + ps - 1) / ps;
  if (np < 2 || ps > 64) return q;
  q.np = np;
  q.ps = ps;
  return q;
}

// Control wave of a workgroup holding part `part` of tile `tile`: the part's sums of every row
// tile r from the waves' partials in red + r * (8 * 16 * 17), the exchange, and (last part
// only) the tile's outputs.
template <int NRT>
__device__ __forceinline__ void qkv_split_epilogue(const KArgs& a, const float* red, int tile, int part, int np,
                                                   int crow, int cc0) {
  const int lane = threadIdx.x & 63;
  float v[NRT][4];
#pragma unroll
  for (int r = 0; r < NRT; ++r) {
    ctl_tile_vals(red + r * (8 * 16 * 17), crow, cc0, v[r]);
    float* mine = a.qkv_part + (((size_t)(tile * np + part) * NRT + r) * 64 + lane) * 4;
    st_coh_u64(mine, (uint64_t)__float_as_uint(v[r][0]) | ((uint64_t)__float_as_uint(v[r][1]) << 32));
    st_coh_u64(mine + 2, (uint64_t)__float_as_uint(v[r][2]) | ((uint64_t)__float_as_uint(v[r][3]) << 32));
  }
  __builtin_amdgcn_s_waitcnt(0);           // the partials are complete before they are counted
  uint32_t old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(a.qkv_cnt + tile * 16, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0);
  if (old != (uint32_t)(np - 1)) return;
  const int qd = a.Hq * a.d, kd = a.Hkv * a.d, n = tile * 16 + cc0;
#pragma unroll
  for (int r = 0; r < NRT; ++r) {
    float sum[4] = {0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < np; ++p) {
      float u[4] = {v[r][0], v[r][1], v[r][2], v[r][3]};
      if (p != part) {
        const uint32_t* o = (const uint32_t*)(a.qkv_part + (((size_t)(tile * np + p) * NRT + r) * 64 + lane) * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) u[j] = __uint_as_float(ld_coh_u32(o + j));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) sum[j] += u[j];
    }
    const int row = 16 * r + crow;
    if (row >= a.T) continue;
    const int sq = row / a.Ts, tok = row - sq * a.Ts;
    const size_t kvs = (size_t)sq * a.cap * kd;              // sequence sq's next-layer cache
    uint16_t* dst;
    if (n < qd) dst = a.q_next + (size_t)row * qd + n;
    else if (n < qd + kd) dst = a.kn + kvs + (size_t)(a.ctx + tok) * kd + (n - qd);
    else dst = a.vn + kvs + (size_t)(a.ctx + tok) * kd + (n - qd - kd);
    *(uint64_t*)dst = pack4_bf16(sum);
  }
}

// ------------------------------------------------------------------ kernel

// SPEC 1: the shard shape of the pages' model on one GPU (hidden 4096, 8 q heads / 1 kv head
// of 128, pooled 2048, 256 experts top-8, NVFP4 experts with local intermediate 192, a
// 16-token tree) with every shape a compile-time constant; SPEC 0 takes shapes at run time.
// NS: the N-sharded expert layout (a separate instantiation, so that the ordinary layout's
// code does not carry its registers).  NRT: 16-row tiles of the launch (1: one sequence of
// T <= 16 tokens; 2: two sequences of 16), SPEC 1 the shard shape at either.
template <bool TS, int SPEC, bool NS, int NRT>
__global__ void __launch_bounds__(kThreads) layer_kernel(KArgs a_in) {
  KArgs a = a_in;
  if constexpr (SPEC == 1) {
    a.H = 4096; a.Hq = 8; a.Hkv = 1; a.d = 128; a.P = 2048; a.E = 256; a.topk = 8; a.I = 192;
    a.fmt = 1; a.T = 16 * NRT;
  }
  if constexpr (NRT == 1) {
    a.B = 1;
    a.Ts = a.T;
  } else {
    a.B = NRT;
    a.Ts = 16;
    a.T = 16 * NRT;
  }
  if constexpr (!NS) a.ns_R = 0;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ RouteT<NRT> rt;
  __shared__ Tree tr;
  __shared__ int32_t dead_sh;
  __shared__ uint32_t epoch_sh;
  __shared__ int32_t par_sh[32];
  __shared__ int32_t xk_sh[16 * NRT];   // GEMM1 input row scales (NVFP4 experts)
  __shared__ uint32_t ytile[16 * NRT * 4];
  const int tid = threadIdx.x;
  const bool cw = tid < kCompute;
  const int lane = tid & 63;
  const int nwg = gridDim.x;
  if constexpr (TS) {
    if (tid >= kCtl && tid - kCtl < MK_TS_EVENTS_DEV) ts_lds[tid - kCtl] = 0;   // same wave as event 0
  }
  stamp<TS>(a.timestamps, 0);

  // control lanes: row (within a 16-row tile) / columns of the 4 outputs they store in a dense
  // tile epilogue; row tile r covers rows 16 r .. 16 r + 15
  const int crow = lane >> 2, cc0 = (lane & 3) * 4;
  auto crv = [&](int r) { return 16 * r + crow < a.T; };

  // weights of the o-proj tile, and (control wave) its residual, fetched at launch
  WFrag<MAXS_O> wo;
  WFrag<0> wp;
  WFrag<MAXS_R> wr;
  WFrag<MAXS_U> wu;
  WFrag<MAXS_Q> wq;
  WFrag<SPEC == 1 ? 6 : 8> wqs;       // a split-K part's fragments
  // pooler tiles run on the last P/16 workgroups, away from the attention items, so that
  // those workgroups can hold their tile in LDS from launch start
  const int off_p = nwg > a.P / 16 ? nwg - a.P / 16 : 0;
  const int t_o = first_tile(0), t_p = first_tile(off_p), t_u = first_tile(0);
  // router tiles: on workgroups with neither a pooler tile nor an attention item, just below
  // the pooler's, when there are enough; those hold their tile in LDS (where a pooler tile
  // would sit) from launch start.  Otherwise on the last workgroups, loaded into registers
  // during the pooler hand-off.
  const bool router_room = off_p - a.attn_items >= a.E / 16 && POOL_LDS_OFF + 32 * a.P <= LDS_BYTES;
  const int off_r = router_room ? off_p - a.E / 16 : nwg - a.E / 16, off_q = a.P / 16 < nwg ? a.P / 16 : 0;
  const int t_r = first_tile(off_r), t_q = first_tile(off_q);
  const int qkv_n = (a.Hq + 2 * a.Hkv) * a.d;
  // the stack's last layer (no next-layer weights) ends after the unpooler
  const bool has_qkv = a.w_qkv != nullptr;
  // qkv: K split over np workgroups per tile when the grid has room (item t_q is part
  // t_q / ntiles of tile t_q % ntiles), else one workgroup per tile over the full K
  // (shard shape: 80 tiles x 3 parts of 48, 48 and 32 k-steps; the host launches it on >= 240
  // workgroups)
  const QkvSplit qs = SPEC == 1 ? QkvSplit{3, 48} : qkv_split(a.H >> 5, qkv_n / 16, nwg);
  const bool q_split = has_qkv && qs.np > 1;
  const int q_nt = qkv_n / 16 > 0 ? qkv_n / 16 : 1;
  const int q_tile = t_q % q_nt, q_part = t_q / q_nt;
  const int q_s0 = q_part * qs.ps, q_ns = min(qs.ps, (a.H >> 5) - q_s0);
  const bool p_qs = q_split && q_part < qs.np;
  const bool p_o = t_o < a.H / 16, p_p = t_p < a.P / 16, p_r = t_r < a.E / 16, p_u = t_u < a.H / 16,
             p_q = has_qkv && !q_split && t_q < qkv_n / 16;
  // the pooler tile sits in LDS; a workgroup with an attention item fills it afterwards
  const bool pool_lds = p_p && POOL_LDS_OFF + 16 * a.H * 2 <= LDS_BYTES;
  const bool pool_dma = pool_lds && (int)blockIdx.x < a.attn_items;
  const bool router_lds = router_room && p_r;
  u32x2 res[NRT];
#pragma unroll
  for (int r = 0; r < NRT; ++r) {
    res[r] = u32x2{0, 0};
    if (!cw && p_o && crv(r)) res[r] = *(const u32x2*)(a.h_in + (size_t)(16 * r + crow) * a.H + t_o * 16 + cc0);
  }

  // the control wave reads the tree and this workgroup's epoch, both loads in flight together
  // (wave 0 issues its attention loads meanwhile)
  if (!cw) {
    const int l = tid - kCtl;
    const int32_t par = l < a.T ? a.parent[l] : 0;
    const uint32_t ep = ld_coh_u32(a.epoch + blockIdx.x * 16);
    if (l < a.T) par_sh[l] = par;
    if (l == 0) {
      epoch_sh = ep;
      dead_sh = 0;
      // this launch's split-K qkv arrival counter of tile blockIdx.x starts at zero
      if (q_split && (int)blockIdx.x < q_nt) st_coh_u32(a.qkv_cnt + blockIdx.x * 16, 0u);
    }
  }
  // the first attention item's queries and first K/V batch load during the setup
  u32x4 qf0[4];
  StageRegs sreg0;
  if ((int)blockIdx.x < a.attn_items) {
    const AttnItem it0 = attn_item(a, blockIdx.x);
    attention_q(a, it0, qf0);
    stage_load(a, it0, 0, sreg0);
  }
  wg_sync();
  if (tid < 64) {
    // lanes i < T (rows; sequence b's tree on lanes b Ts ..): ancestor-or-self set by pointer
    // jumping (4 rounds cover depth <= 15); depth = |ancestors| - 1
    const int lane = tid;
    const int sq = a.B == 1 ? 0 : lane / a.Ts, node = lane - sq * a.Ts;
    const int p = lane < a.T ? par_sh[lane] : -1;
    const bool ok = lane >= a.T || (node == 0 ? p == -1 : (p >= 0 && p < node));
    const bool bad = __ballot(!ok) != 0;
    uint32_t anc = lane < a.T ? 1u << lane : 0u;
    int jump = (lane < a.T && node > 0 && ok) ? sq * a.Ts + p : -1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t aj = __shfl(anc, jump < 0 ? lane : jump);
      const int jj = __shfl(jump, jump < 0 ? lane : jump);
      if (jump >= 0) {
        anc |= aj;
        jump = jj;
      }
    }
    if (lane < a.T) {
      const int pos = a.ctx + __popc(anc) - 1;
      tr.anc[lane] = bad ? 1u << lane : anc;
      tr.lo[lane] = a.window > 0 ? max(0, pos - a.window + 1) : 0;
    }
    if (lane == 0) {
      tr.bad = bad;
      if (bad && blockIdx.x == 0)
        __hip_atomic_store(a.status, status_word(epoch_sh, MK_EBADTREE_DEV), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  wg_sync();
  stamp<TS>(a.timestamps, 1);
  const uint32_t epoch = epoch_sh;
  // this launch's copy of the stage buffers; the control wave returns this workgroup's share of
  // the other copy to the sentinel for the next launch (plain stores: the next launch starts
  // after they are written back)
  {
    a.cur = a.stage + (size_t)(epoch & 1u) * kStageBytes;
    if (!cw) {
      u32x4* idle = (u32x4*)(a.stage + (size_t)((epoch & 1u) ^ 1u) * kStageBytes);
      constexpr uint32_t words = kStageBytes / 16;
      const uint32_t per = (words + nwg - 1) / nwg;
      for (uint32_t i = lane; i < per; i += 64) {
        const uint32_t w = blockIdx.x * per + i;
        if (w < words) idle[w] = u32x4{~0u, ~0u, ~0u, ~0u};
      }
    }
  }
  Sync s;
  s.flags = a.flags;
  s.status = a.status;
  s.epoch = epoch;
  s.base = epoch * 64u;
  s.spin_limit = a.spin_limit;
  s.skip_wg = a.skip_wg;
  float* red2 = (float*)smem;
  auto nop = [] {};

  if (!tr.bad) {
    bool alive = true;
    uint32_t touched = 0;     // folded values of the cache-touch prefetches
    // ---- 1 ATTN
    // one item: stage (its first batch already loaded), compute, store the partials
    auto attn_item_run = [&](const AttnItem& it, const StageRegs& r0, const u32x4 qf[4], bool first) {
      stage_store(a, it, 0, r0, smem);
      for (int b = 1; b < stage_batches(a); ++b) {
        StageRegs r;
        stage_load(a, it, b, r);
        stage_store(a, it, b, r, smem);
      }
      wg_sync();
      if (first) stamp<TS>(a.timestamps, 37, 0);
      switch (a.attn_rw) {                     // uniform over the grid
        case 1: attention_compute<1, TS>(a, tr, it, smem, qf); break;
        case 2: attention_compute<2, TS>(a, tr, it, smem, qf); break;
        case 4: attention_compute<4, TS>(a, tr, it, smem, qf); break;
        default: attention_compute<8, TS>(a, tr, it, smem, qf); break;
      }
      if (first) stamp<TS>(a.timestamps, 38, 0);
      wg_sync();
    };
    if ((int)blockIdx.x < a.attn_items) attn_item_run(attn_item(a, blockIdx.x), sreg0, qf0, true);
    for (int i = blockIdx.x + nwg; i < a.attn_items; i += nwg) {
      const AttnItem it = attn_item(a, i);
      u32x4 qf[4];
      StageRegs r;
      attention_q(a, it, qf);
      stage_load(a, it, 0, r);
      attn_item_run(it, r, qf, false);
    }
    if (pool_lds && !pool_dma) lds_tile_fill(a.w_pool, a.H, t_p * 16, smem + POOL_LDS_OFF);
    if (router_lds) lds_tile_fill(a.w_router, a.P, t_r * 16, smem + POOL_LDS_OFF);
    // workgroups without an attention item pull the previous step's most-used experts into
    // the device-side caches before the routing of this step is known.  (The unpooler and
    // qkv tiles are not touched here: that traffic slows the attention phase more than it
    // speeds up the end of the layer; the unpooler tile streams into LDS during GEMM2.)
    if (cw && (int)blockIdx.x >= a.attn_items && a.n_prefetch > 0 && nwg > a.attn_items)
      touched ^= expert_touch(a, blockIdx.x - a.attn_items, nwg - a.attn_items);
    if (cw) __builtin_amdgcn_s_waitcnt(0);   // partial stores complete
    // only the workgroups with a merge unit read the attention partials: the others raise their
    // flag and go on (the o-proj reads the merged rows as they arrive)
    const bool merge_wg = (int)blockIdx.x < a.B * a.Hkv * a.Ts * (a.Hq / a.Hkv);
    alive = phase_end<TS>(a, s, 1, &dead_sh, [&] {
      if (p_p && !pool_lds) touched ^= touch_tile<2>(a.w_pool, a.H, t_p * 16);
    }, 0, merge_wg);
    // ---- 2 MERGE
    if (alive) {
      const int units = a.B * a.Hkv * a.Ts * (a.Hq / a.Hkv);
      for (int u = blockIdx.x; u < units; u += nwg) {
        if (u != (int)blockIdx.x) wg_sync();     // LDS scratch reused
        merge_unit<TS>(a, u, (float*)smem);
        stamp<TS>(a.timestamps, 53, 0);
      }
    }
    // No grid hand-off after the merge: the o-proj reads attn as it arrives.  Meanwhile the
    // o-proj tile loads into registers and, on a workgroup that had an attention item, the
    // pooler tile into LDS by LDS-DMA (the merge and o-proj phases use LDS below POOL_LDS_OFF
    // only; the DMA is waited for before the pooler phase).  Workgroups without a merge unit
    // first wait about kIdleSleepUs: their polls would only add traffic while the merge runs.
    wg_sync();
    stamp<TS>(a.timestamps, 4);
    if (alive && cw) {
      if (p_o) wfrag_load(wo, a.w_o, a.Hq * a.d, t_o * 16);
      if (pool_dma) lds_tile_dma(a.w_pool, a.H, t_p * 16, smem + POOL_LDS_OFF, tid >> 6, kCompute / 64);
      if ((int)blockIdx.x >= a.B * a.Hkv * a.Ts * (a.Hq / a.Hkv))
        for (int i = 0; i < kIdleSleepUs; ++i) __builtin_amdgcn_s_sleep(37);
    }
    stamp<TS>(a.timestamps, 5, 0);
    // ---- 3 OPROJ: h1 = bf16(h_in + attn Wo^T).  The control wave keeps its first tile's h1
    // values: the unpooler's tiles are the same (N = H, same order), h1 is its residual.
    u32x2 res_u[NRT];
#pragma unroll
    for (int r = 0; r < NRT; ++r) res_u[r] = u32x2{0, 0};
    if (alive) {
      dense_phase<NRT, TS>(a, wo, p_o, a.w_o, xsrc(st_attn(a), a.Hq * a.d, s, &dead_sh), a.Hq * a.d, a.H, 0, red2,
                       [&](int n0, const float* red, int it, int rr) {
        if (!crv(rr)) return;
        const int row = 16 * rr + crow;
        float v[4];
        ctl_tile_vals(red, crow, cc0, v);
        const u32x2 r = it == 0 ? res[rr] : *(const u32x2*)(a.h_in + (size_t)row * a.H + n0 + cc0);
        v[0] += bf2f(r[0] & 0xFFFF); v[1] += bf2f(r[0] >> 16); v[2] += bf2f(r[1] & 0xFFFF); v[3] += bf2f(r[1] >> 16);
        const uint64_t hv = pack4_bf16(v);
        st_coh_u64(st_h1(a) + (size_t)rr * 16 * a.H + frag_off(crow, n0 + cc0), hv);
        if (it == 0) res_u[rr] = u32x2{(uint32_t)hv, (uint32_t)(hv >> 32)};
      }, nullptr, 47);
    }
    if (cw && pool_dma) __builtin_amdgcn_s_waitcnt(0);   // the pooler tile is in LDS
    // only the pooler's workgroups read h1 now; the others raise their flag and go on to the
    // pooler's hand-off
    alive = phase_end<TS>(a, s, 3, &dead_sh, nop, 0, p_p) && alive && dead_sh == 0;
    // ---- 4 POOL: xp = bf16(h1 Wp^T)
    if (alive) {
      dense_phase<NRT>(a, wp, false, a.w_pool, xplain(st_h1(a), s, &dead_sh), a.H, a.P, off_p, red2,
                       [&](int n0, const float* red, int, int rr) {
        if (!crv(rr)) return;
        float v[4];
        ctl_tile_vals(red, crow, cc0, v);
        st_coh_u64(st_xp(a) + (size_t)rr * 16 * a.P + frag_off(crow, n0 + cc0), pack4_bf16(v));
      }, pool_lds ? smem + POOL_LDS_OFF : nullptr);
    }
    // the router tile loads into registers (unless held in LDS) while the grid hands off
    // The workgroups without a pooler tile reach this wait right after their o-proj tile (they
    // skip the o-proj's wait) and sleep through the o-proj hand-off and the pooler's work, both
    // proportional to H: 1 + H/1024 us (5 at H = 4096, where 3, 4, 5, 6, 7, 8 us measured -0.09,
    // -0.18, -0.35, -0.34, -0.14, +0.36 us per layer against 2).
    alive = phase_end<TS>(a, s, 4, &dead_sh, [&] { if (p_r && !router_lds) wfrag_load(wr, a.w_router, a.P, t_r * 16); },
                          p_p ? 0 : 1 + a.H / 1024) && alive;
    // ---- 5 ROUTER: logits = xp Wr^T (+ bias)
    if (alive) {
      dense_phase<NRT>(a, wr, p_r && !router_lds, a.w_router, xplain(st_xp(a), s, &dead_sh), a.P, a.E, off_r, red2,
                       [&](int n0, const float* red, int, int rr) {
        if (!crv(rr)) return;
        const int row = 16 * rr + crow;
        float v[4];
        ctl_tile_vals(red, crow, cc0, v);
        if (a.bias) {
          const f32x4 b = *(const f32x4*)(a.bias + (size_t)row * a.E + n0 + cc0);
          v[0] += b[0]; v[1] += b[1]; v[2] += b[2]; v[3] += b[3];
        }
        st_coh_u128(st_logits(a) + (size_t)row * a.E + n0 + cc0,
                    u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
        if (a.router_logits) *(f32x4*)(a.router_logits + (size_t)row * a.E + n0 + cc0) = f32x4{v[0], v[1], v[2], v[3]};
      }, router_lds ? smem + POOL_LDS_OFF : nullptr);
    }
    // No grid hand-off after the router: the control waves of the first T workgroups read the
    // logits as they arrive and publish each row's routing, which every workgroup reads as it
    // arrives.  Meanwhile GEMM1's input rows (xs, in LDS at 0) are built from xp (piece maxima
    // go to the LDS area GEMM1 later uses for scales): they do not depend on the routing.
    wg_sync();
    stamp<TS>(a.timestamps, 10);
    if (alive) {
      if constexpr (NRT == 1) {
        u32x4 xpv[8];
        if (cw) xp_fetch(a, xpv, (uint32_t*)(smem + G1_XS_BYTES));
        else publish_route<TS>(a, s, &dead_sh);
        wg_sync();                              // every wave's piece maxima are in LDS
        xs_build<TS>(a, xpv, (uint16_t*)smem, a.P + XS_STRIDE_PAD, (const uint32_t*)(smem + G1_XS_BYTES), xk_sh);
      } else {
        // two sequences: all 32 rows, or (two pieces per unit) the first K half of them
        if (!cw) publish_route<TS>(a, s, &dead_sh);
        xs_rowscale2<TS>(a, (uint32_t*)(smem + G1_XS_BYTES), xk_sh);
        const int cols = g1_pieces(a.P) == 2 ? g1_hsteps(a.P) * 128 : a.P;
        xs_fill2(a, (uint16_t*)smem, cols + XS_STRIDE_PAD, 0, cols, xk_sh);
        wg_sync();
      }
    }
    stamp<TS>(a.timestamps, 11);
    // ---- 6 ROUTE + GEMM1
    if (alive) {
      if (!p_r)
        for (int i = 0; i < MK_ROUTE_IDLE; ++i) __builtin_amdgcn_s_sleep(37);
      route_tables<TS>(a, rt, (uint32_t*)(smem + g1_ubuf_off(a.P)), s, &dead_sh);
      stamp<TS>(a.timestamps, 18);
      alive = dead_sh == 0;                     // (route_tables ends synchronised)
      if (alive) gemm1_phase<TS>(a, rt, smem, xk_sh);
    }
    // No grid hand-off after GEMM1 either: GEMM2 reads the intermediate as it arrives.  This
    // workgroup's first W2 registers are requested now.
    G2W g2w;
    wg_sync();
    stamp<TS>(a.timestamps, 12);
    alive = alive && dead_sh == 0;
    if (alive && cw && !a.ns_R && g2_fast(a) && (int)blockIdx.x < a.P / 8) g2_load(a, rt, blockIdx.x * 8, 0, g2w);
    stamp<TS>(a.timestamps, 13, 0);
    // ---- 7 GEMM2 + combine
    // NVFP4 experts: GEMM2 leaves LDS above 64 KB free, so the control wave streams the
    // unpooler tile there while the experts run (waited for at this phase's hand-off)
    const int g2_lds_end = ((a.T * a.topk * (a.I + 8) * 2 + 255) & ~255) + 128 * 8 * 4 + 72 * 16 * 4;
    const bool wu_lds = !a.ns_R && g2_fast(a) && p_u && g2_lds_end <= WU_LDS_OFF &&
                        WU_LDS_OFF + 32 * a.P <= LDS_BYTES;
    if (alive) {
      if (!cw && wu_lds) lds_tile_dma(a.w_unpool, a.P, t_u * 16, smem + WU_LDS_OFF);
      if (a.ns_R) gemm2_ns<TS>(a, rt, smem, ytile, s, &dead_sh);
      else if (g2_fast(a)) gemm2_fp4<TS>(a, rt, smem, ytile, g2w, s, &dead_sh);
      else gemm2_staged<TS>(a, rt, smem, ytile, s, &dead_sh);
    }
    // the unpooler tile is in LDS (the control wave's LDS-DMA during GEMM2, waited for in the hand-off)
    // or loads into registers while the grid hands off
    alive = phase_end<TS>(a, s, 7, &dead_sh, [&] { if (p_u && !wu_lds) wfrag_load(wu, a.w_unpool, a.P, t_u * 16); })
            && alive;
    // ---- 8 UNPOOL: h_out = bf16(h1 + y Wu^T)
    if (alive) {
      // (N-sharded layout: the gathered y, the other ranks' columns read as they arrive)
      dense_phase<NRT>(a, wu, p_u && !wu_lds, a.w_unpool,
                       a.ns_R ? xsrc(a.y_recv, a.P, s, &dead_sh) : xplain(st_y(a), s, &dead_sh), a.P, a.H, 0, red2,
                       [&](int n0, const float* red, int it, int rr) {
        if (!crv(rr)) return;
        const int row = 16 * rr + crow;
        float v[4];
        ctl_tile_vals(red, crow, cc0, v);
        u32x2 r = res_u[rr];                // this workgroup's own o-proj output (first tile)
        if (it > 0) {
          const uint64_t w = poll_u64(s, &dead_sh, st_h1(a) + (size_t)rr * 16 * a.H + frag_off(crow, n0 + cc0));
          r = u32x2{(uint32_t)w, (uint32_t)(w >> 32)};
        }
        v[0] += bf2f(r[0] & 0xFFFF); v[1] += bf2f(r[0] >> 16); v[2] += bf2f(r[1] & 0xFFFF); v[3] += bf2f(r[1] >> 16);
        const uint64_t hv = pack4_bf16(v);
        st_coh_u64(a.h_out + (size_t)row * a.H + n0 + cc0, hv);                        // the output, row-major
        st_coh_u64(st_h_frag(a) + (size_t)rr * 16 * a.H + frag_off(crow, n0 + cc0), hv);  // the qkv phase's x
      }, wu_lds ? smem + WU_LDS_OFF : nullptr);
    }
    // No grid hand-off after the unpooler: the qkv projection reads h_out as it arrives; its
    // weights (a whole tile, or one K part of it) load meanwhile.
    wg_sync();
    stamp<TS>(a.timestamps, 16);
    if (alive && cw) {
      if (p_q) wfrag_load(wq, a.w_qkv, a.H, t_q * 16);
      if (p_qs) wfrag_load(wqs, a.w_qkv + q_s0 * 32, q_ns * 32, q_tile * 16, a.H);
    }
    stamp<TS>(a.timestamps, 17, 0);
    alive = alive && dead_sh == 0;
    // ---- QKV + KV write
    if (alive) {
      const int qd = a.Hq * a.d, kd = a.Hkv * a.d;
      const XSrc hx = xsrc(st_h_frag(a), a.H, s, &dead_sh);
      if (q_split) {
        // every row tile's part with the same weight registers, each into its own buffer
#pragma unroll
        for (int r = 0; r < NRT; ++r)
          if (cw && p_qs)
            red_store(red2 + r * (8 * 16 * 17), wfrag_mma(wqs, NRT == 1 ? hx : xtile(hx, r, a.H), q_s0,
                                                          min(16, a.T - 16 * r), q_ns * 32));
        wg_sync();
        if (!cw && p_qs) qkv_split_epilogue<NRT>(a, red2, q_tile, q_part, qs.np, crow, cc0);
      } else if (has_qkv) dense_phase<NRT>(a, wq, p_q, a.w_qkv, hx, a.H, qkv_n, off_q, red2,
                                           [&](int n0, const float* red, int, int rr) {
        if (!crv(rr)) return;
        const int row = 16 * rr + crow, sq = row / a.Ts, tok = row - sq * a.Ts;
        float v[4];
        ctl_tile_vals(red, crow, cc0, v);
        const int n = n0 + cc0;
        const size_t kvs = (size_t)sq * a.cap * kd;           // sequence sq's next-layer cache
        uint16_t* dst;
        if (n < qd) dst = a.q_next + (size_t)row * qd + n;
        else if (n < qd + kd) dst = a.kn + kvs + (size_t)(a.ctx + tok) * kd + (n - qd);
        else dst = a.vn + kvs + (size_t)(a.ctx + tok) * kd + (n - qd - kd);
        *(uint64_t*)dst = pack4_bf16(v);
      });
      if (blockIdx.x == 0) {
        for (int p = tid; p < a.T * a.topk; p += kThreads) {
          if (a.topk_idx) a.topk_idx[p] = rt.idx[p];
          if (a.topk_gate) a.topk_gate[p] = rt.gate[p];
        }
      }
    }
    stamp<TS>(a.timestamps, 19);
    if (touched == 0x9E3779B9u) ytile[0] = touched;   // keeps the touch loads alive
  }
  // the next launch on this workspace uses the next epoch
  if (tid == kCtl) st_coh_u32(a.epoch + blockIdx.x * 16, epoch + 1);
  if constexpr (TS) {
    wg_sync();
    if (tid < MK_TS_EVENTS_DEV) a.timestamps[blockIdx.x * MK_TS_EVENTS_DEV + tid] = ts_lds[tid];
  }
}

// Code placement.  The time per launch of the one-sequence shard-shape kernel depends on where
// its code sits in the code object: identical code measured up to ~1.4 us per launch apart
// between offsets 256 bytes apart, and 0x69400 was the best of the offsets measured for two
// versions of the kernel.  So it is emitted first, behind a kernel that is never launched and
// holds MK_CODE_PAD bytes of s_nop, which puts its code at that offset whatever the size of
// the other kernels (llvm-readelf -s on the device code object shows the offset).
#ifndef MK_CODE_PAD
#define MK_CODE_PAD 406784
#endif
#if MK_CODE_PAD > 0
__global__ void code_pad() { asm volatile(".fill %0, 4, 0xBF800000" ::"i"(MK_CODE_PAD / 4)); }
#endif
template __global__ void layer_kernel<false, 1, false, 1>(KArgs);
template __global__ void layer_kernel<false, 0, false, 1>(KArgs);
template __global__ void layer_kernel<true, 0, false, 1>(KArgs);
template __global__ void layer_kernel<true, 1, false, 1>(KArgs);
template __global__ void layer_kernel<false, 0, true, 1>(KArgs);
template __global__ void layer_kernel<true, 0, true, 1>(KArgs);
template __global__ void layer_kernel<false, 1, true, 1>(KArgs);
template __global__ void layer_kernel<true, 1, true, 1>(KArgs);
template __global__ void layer_kernel<false, 0, false, 2>(KArgs);
template __global__ void layer_kernel<true, 0, false, 2>(KArgs);
template __global__ void layer_kernel<false, 1, false, 2>(KArgs);
template __global__ void layer_kernel<true, 1, false, 2>(KArgs);

int layer_lds_bytes() { return LDS_BYTES; }

static bool is_spec1(const KArgs& a) {
  return a.H == 4096 && a.Hq == 8 && a.Hkv == 1 && a.d == 128 && a.P == 2048 && a.E == 256 && a.topk == 8 &&
         a.I == 192 && a.fmt == 1 && a.T == 16 * a.B && a.n_wg >= 240;
}

template <bool NS, int NRT>
void launch_v(const KArgs& a, int lds_bytes, hipStream_t stream) {
  const dim3 g(a.n_wg), b(kThreads);
  if (is_spec1(a)) {
    if (a.timestamps) hipLaunchKernelGGL((layer_kernel<true, 1, NS, NRT>), g, b, lds_bytes, stream, a);
    else hipLaunchKernelGGL((layer_kernel<false, 1, NS, NRT>), g, b, lds_bytes, stream, a);
  } else {
    if (a.timestamps) hipLaunchKernelGGL((layer_kernel<true, 0, NS, NRT>), g, b, lds_bytes, stream, a);
    else hipLaunchKernelGGL((layer_kernel<false, 0, NS, NRT>), g, b, lds_bytes, stream, a);
  }
}

int launch_layer(const KArgs& a, int lds_bytes, hipStream_t stream) {
  if (a.B == 2) launch_v<false, 2>(a, lds_bytes, stream);     // (the host admits no N-sharded batch)
  else if (a.ns_R) launch_v<true, 1>(a, lds_bytes, stream);
  else launch_v<false, 1>(a, lds_bytes, stream);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int set_layer_kernel_attrs(int lds_bytes) {
  const void* fns[] = {(const void*)layer_kernel<false, 0, false, 1>, (const void*)layer_kernel<true, 0, false, 1>,
                       (const void*)layer_kernel<false, 1, false, 1>, (const void*)layer_kernel<true, 1, false, 1>,
                       (const void*)layer_kernel<false, 0, true, 1>, (const void*)layer_kernel<true, 0, true, 1>,
                       (const void*)layer_kernel<false, 1, true, 1>, (const void*)layer_kernel<true, 1, true, 1>,
                       (const void*)layer_kernel<false, 0, false, 2>, (const void*)layer_kernel<true, 0, false, 2>,
                       (const void*)layer_kernel<false, 1, false, 2>, (const void*)layer_kernel<true, 1, false, 2>};
  for (const void* f : fns)
    if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes) != hipSuccess) return -5;
  return 0;
}

}  // namespace mk

// Device helpers for the gfx950 (CDNA4) kernels: bf16 packing, MFMA fragments, NVFP4
// dequantisation, coherent hand-off stores and wave reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace mk {

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(uint32_t b16) { return __uint_as_float(b16 << 16); }
// fp32 -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) { return f2bf(lo) | (f2bf(hi) << 16); }

// v_mfma_f32_16x16x32_bf16.  Lane l supplies A[l%16][8*(l/16) + j] and B[8*(l/16) + j][l%16]
// (j = 0..7, any common permutation of k is allowed); C lane l holds rows 4*(l/16)+r, col l%16.
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// v_mfma_f32_16x16x16_bf16: lane l supplies A[l%16][4*(l/16) + j] and B[4*(l/16) + j][l%16]
// (j = 0..3); C as in the 32-deep form.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma_bf16_k16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b),
                                                   c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_f16: the same lane layout as the bf16 form, fp16 operands.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Eight E2M1 codes times an E4M3 block scale -> eight fp16 in MFMA operand order, exactly:
// the codes are decoded at scale 1.0 (exact), then one packed fp16 multiply per pair applies
// the scale.  e2m1 x e4m3 products have <= 6 significant bits and lie in [2^-10, 2688], inside
// fp16's normal range, so the product is the exact value.  `s` holds the scale in both halves.
__device__ __forceinline__ u32x4 fp4x8_to_f16(uint32_t codes, f16x2_t s) {
  const f16x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s;
  const f16x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s;
  const f16x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s;
  const f16x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s;
  return u32x4{__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1),
               __builtin_bit_cast(uint32_t, v2), __builtin_bit_cast(uint32_t, v3)};
}
// an E4M3 byte as an fp16 pair (every E4M3 value is exact in fp16)
__device__ __forceinline__ f16x2_t e4m3_to_f16x2(uint32_t byte) {
  const _Float16 h = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
  return f16x2_t{h, h};
}

// Eight E2M1 codes (one dword, element 2q in the low nibble of byte q) times an fp32 block
// scale -> eight bf16 in MFMA operand order.  The hardware converter applies only the
// exponent of its scale operand, so it decodes the bare codes (scale 1.0, exact) and the
// E4M3 scale is applied by an fp32 multiply; e2m1 x e4m3 products have <= 6 significant
// bits, so truncating the fp32 product to its upper half is exact.
template <int Q>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t codes, float scale) {
  f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, Q);
  const uint32_t lo = __float_as_uint(v.x * scale), hi = __float_as_uint(v.y * scale);
  return __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}
__device__ __forceinline__ u32x4 fp4x8_to_bf16(uint32_t codes, float scale) {
  return u32x4{fp4x2_to_bf16x2<0>(codes, scale), fp4x2_to_bf16x2<1>(codes, scale),
               fp4x2_to_bf16x2<2>(codes, scale), fp4x2_to_bf16x2<3>(codes, scale)};
}

// OCP E4M3 byte -> fp32 (gfx950 converts the OCP "FN" encoding).
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// Coherent (device-scope, write-through) stores for data another workgroup reads in the
// same launch; plain loads see them because every hand-off buffer is written once per
// launch before any workgroup of the launch first reads it.
__device__ __forceinline__ void st_coh_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh_u64(void* p, uint64_t v) {
  __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh_u128(void* p, u32x4 v) {
  st_coh_u64(p, (uint64_t)v[0] | ((uint64_t)v[1] << 32));
  st_coh_u64((char*)p + 8, (uint64_t)v[2] | ((uint64_t)v[3] << 32));
}
__device__ __forceinline__ uint32_t ld_coh_u32(const uint32_t* p) {
  return __hip_atomic_load((uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }

// Hand-off data read as it arrives.  Producers write hand-off data with device-coherent
// 8-byte stores, and no 8-byte word of it is ever all ones (bf16 and fp32 results are never
// the all-ones NaN pattern; an NVFP4 intermediate record carries its scale byte, at most
// 0x7E, in each half); a stage buffer not yet written in this launch holds all ones.  A
// consumer loads 16 bytes with a device-coherent load -- a raw buffer load with the sc1
// cache policy, which sees other XCDs' coherent stores -- and takes them once neither
// 8-byte half is all ones.  Buffer loads outside the resource's range return zero.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 ld_coh16(rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 16 /* sc1 */);
}
__device__ __forceinline__ bool arrived16(u32x4 v) {
  return (v[0] & v[1]) != 0xFFFFFFFFu && (v[2] & v[3]) != 0xFFFFFFFFu;
}

// max / sum across the 4 lanes {l, l^16, l^32, l^48} (the four k-groups of an MFMA column)
__device__ __forceinline__ float xgroup_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float xgroup_sum(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// Maximum over the 64 lanes of a wave (all lanes active): DPP exchanges inside each row of
// 16 lanes (quad xor 1, quad xor 2, half-row mirror, row mirror), then the four row values.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f32<0x141>(v));   // row_half_mirror
  v = fmaxf(v, dpp_f32<0x140>(v));   // row_mirror
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)),
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)),
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48))));
}

// Maximum of a signed 32-bit value over the 64 lanes of a wave (all lanes active), returned
// uniform: DPP exchanges inside each row of 16, then row broadcasts 15 and 31 carry the row
// maxima up to lane 63.
template <int CTRL, int ROWS>
__device__ __forceinline__ int32_t dpp_i32(int32_t v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, ROWS, 0xF, false);
}
// Maxima of a signed 32-bit value over each half (lanes 0-31, 32-63) of a wave (all lanes
// active): lane 31 ends with the first half's, lane 63 with the second's.  Each step's DPP
// move takes no old value (all rows written) or the max identity (row broadcast into rows 1
// and 3 only), so the compiler folds it into the max as one DPP instruction.
template <int CTRL, int ROWS>
__device__ __forceinline__ int32_t dpp_max_i32(int32_t v) {
  const int32_t moved = ROWS == 0xF ? __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true)
                                    : __builtin_amdgcn_update_dpp((int32_t)0x80000000, v, CTRL, ROWS, 0xF, false);
  return max(v, moved);
}
__device__ __forceinline__ int32_t half_max_i32(int32_t v) {
  v = dpp_max_i32<0xB1, 0xF>(v);        // quad_perm [1,0,3,2]
  v = dpp_max_i32<0x4E, 0xF>(v);        // quad_perm [2,3,0,1]
  v = dpp_max_i32<0x141, 0xF>(v);       // row_half_mirror
  v = dpp_max_i32<0x140, 0xF>(v);       // row_mirror
  return dpp_max_i32<0x142, 0xA>(v);    // row_bcast:15 into rows 1 and 3
}
// wave_max_i32 with each exchange folded into the max (one DPP instruction per step)
__device__ __forceinline__ int32_t wave_max_i32_folded(int32_t v) {
  v = dpp_max_i32<0xB1, 0xF>(v);        // quad_perm [1,0,3,2]
  v = dpp_max_i32<0x4E, 0xF>(v);        // quad_perm [2,3,0,1]
  v = dpp_max_i32<0x141, 0xF>(v);       // row_half_mirror
  v = dpp_max_i32<0x140, 0xF>(v);       // row_mirror
  v = dpp_max_i32<0x142, 0xA>(v);       // row_bcast:15 into rows 1 and 3
  v = dpp_max_i32<0x143, 0xC>(v);       // row_bcast:31 into rows 2 and 3
  return __builtin_amdgcn_readlane(v, 63);
}
// Inclusive prefix sum over the 64 lanes of a wave (all lanes active): shifts right by 1, 2,
// 4 and 8 lanes inside each row of 16 (lanes with no source add 0), then row broadcasts add
// the preceding rows' totals (lane 15 into rows 1 and 3, then lane 31 into rows 2 and 3).
__device__ __forceinline__ int32_t wave_incl_scan_i32(int32_t v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31
  return v;
}
__device__ __forceinline__ int32_t wave_max_i32(int32_t v) {
  v = max(v, dpp_i32<0xB1, 0xF>(v));    // quad_perm [1,0,3,2]
  v = max(v, dpp_i32<0x4E, 0xF>(v));    // quad_perm [2,3,0,1]
  v = max(v, dpp_i32<0x141, 0xF>(v));   // row_half_mirror
  v = max(v, dpp_i32<0x140, 0xF>(v));   // row_mirror
  v = max(v, dpp_i32<0x142, 0xA>(v));   // row_bcast:15 into rows 1 and 3
  v = max(v, dpp_i32<0x143, 0xC>(v));   // row_bcast:31 into rows 2 and 3
  return __builtin_amdgcn_readlane(v, 63);
}

// fp32 -> signed integer with the same order (-0 counts as +0); finite or infinite inputs
__device__ __forceinline__ int32_t f32_order_key(float v) {
  const int32_t b = __float_as_int(v + 0.0f);
  return b >= 0 ? b : b ^ 0x7FFFFFFF;
}
__device__ __forceinline__ float f32_from_order_key(int32_t k) {
  return __int_as_float(k >= 0 ? k : k ^ 0x7FFFFFFF);
}

// E4M3 code of RNE(v / 6) for v >= 0 (fp32), saturating at 448, by binary search over the
// exact thresholds 6*mid (a midpoint of two neighbouring E4M3 values has <= 5 significant
// bits, so 6*mid is exact in fp32).  A tie goes to the even code.
__device__ __forceinline__ uint32_t e4m3_code_of_amax_over6(float v) {
  // passed(c): v lies above the midpoint between codes c and c+1 (or on it with c odd)
  int lo = 0, hi = 126;  // answer in [0, 126] = number of thresholds passed
  while (lo < hi) {
    int c = (lo + hi) >> 1;  // test threshold between c and c+1
    float mid = 0.5f * (e4m3_to_f32(c) + e4m3_to_f32(c + 1));
    float thr = 6.0f * mid;
    bool passed = v > thr || (v == thr && (c & 1));
    if (passed) lo = c + 1; else hi = c;
  }
  return (uint32_t)lo;
}

// E2M1 code of RNE(x / s) (s > 0 an E4M3 value), ties to the even code, saturating at 6;
// thresholds mid*s have <= 7 significant bits and are exact in fp32.
__device__ __forceinline__ uint32_t e2m1_code(float x, float s) {
  const float mids[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  float ax = fabsf(x);
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 7; ++i) {
    float thr = mids[i] * s;
    c += (ax > thr || (ax == thr && (i & 1))) ? 1u : 0u;
  }
  return (x < 0.f && c) ? (c | 8u) : c;
}

}  // namespace mk

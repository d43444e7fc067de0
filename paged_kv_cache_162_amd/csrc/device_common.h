// Device helpers shared by the pagedkv kernels (gfx950): vector types,
// 16-bit unpacking, DPP reductions, the fp8 (OCP E4M3) conversions, and the
// host-side launch helpers.
#ifndef PAGEDKV_DEVICE_COMMON_H_
#define PAGEDKV_DEVICE_COMMON_H_

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "../../include/pagedkv.h"
#include "status.h"

namespace pagedkv {
namespace dev {

using pagedkv::fail;

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

// ---- element conversion -----------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffffu));
}
__device__ __forceinline__ float f16hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}

// Unpack one 16-byte chunk into fp32 values (4 for fp32, 8 for 16-bit types).
template <int DT>
__device__ __forceinline__ void unpack16(const uint4& u, float* f) {
  if constexpr (DT == KV_F32) {
    f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
  } else if constexpr (DT == KV_BF16) {
    f[0] = bf16lo(u.x); f[1] = bf16hi(u.x); f[2] = bf16lo(u.y); f[3] = bf16hi(u.y);
    f[4] = bf16lo(u.z); f[5] = bf16hi(u.z); f[6] = bf16lo(u.w); f[7] = bf16hi(u.w);
  } else {
    f[0] = f16lo(u.x); f[1] = f16hi(u.x); f[2] = f16lo(u.y); f[3] = f16hi(u.y);
    f[4] = f16lo(u.z); f[5] = f16hi(u.z); f[6] = f16lo(u.w); f[7] = f16hi(u.w);
  }
}

// ---- cross-lane operations ---------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over groups of LPR consecutive lanes (LPR = 8, 16 or 32). Within a
// 16-lane DPP row: swap neighbours, swap pairs, mirror halves, mirror the row.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (LPR >= 16) x += dpp<0x140>(x);  // row_mirror
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16, 64);
  return x;
}

// ---- K/V loads ------------------------------------------------------------------
// With NT the load carries the non-temporal hint: cache data that nothing
// else reads again is streamed past the caches instead of being allocated in
// them, which lifts the decode step's throughput by 10-15% on batches without
// shared blocks (measured). Blocks that several sequences share are read
// many times in one step; for them plain loads keep the lines for the next
// reader. Program order within a lane is unchanged either way, so a lane
// still reads back what it stored before.
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
template <bool NT>
__device__ __forceinline__ uint4 load_kv(const uint4* p) {
  if constexpr (NT) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *p;
  }
}
template <bool NT>
__device__ __forceinline__ uint2 load_kv(const uint2* p) {
  if constexpr (NT) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    return make_uint2(v.x, v.y);
  } else {
    return *p;
  }
}

// ---- MFMA attention helpers (decode and prefill) ---------------------------
// Lazy rescale slack of the online softmax, in base-2 units.
constexpr float kRescaleSlack = 8.0f;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;

template <int DT>
__device__ __forceinline__ f32x4 mfma_qk(const uint4& a, const uint4& b, f32x4 c) {
  if constexpr (DT == KV_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ f32x4 mfma_pv(const uint2& a, const uint2& b, f32x4 c) {
  if constexpr (DT == KV_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// Two fp32 values rounded (to nearest even) into one packed 16-bit pair, and
// the two rounded values back as fp32.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (DT == KV_BF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}
template <int DT>
__device__ __forceinline__ void unpack2(uint32_t w, float& a, float& b) {
  if constexpr (DT == KV_BF16) {
    a = bf16lo(w);
    b = bf16hi(w);
  } else {
    a = f16lo(w);
    b = f16hi(w);
  }
}

// Weights of 4 tokens as a B operand: the 16-bit high parts when
// residual == 0, the 16-bit residuals x - high(x) when residual == 1.
template <int DT>
__device__ __forceinline__ uint2 weight_part(const float* x, float residual) {
  uint32_t o[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t h = pack2<DT>(x[2 * i], x[2 * i + 1]);
    float h0, h1;
    unpack2<DT>(h, h0, h1);
    o[i] = pack2<DT>(fmaf(-residual, h0, x[2 * i]), fmaf(-residual, h1, x[2 * i + 1]));
  }
  return make_uint2(o[0], o[1]);
}

// 16-bit element n (0..7) of the four V rows a lane holds, packed as an A
// operand (row of token 4g in the low half of the first dword).
__device__ __forceinline__ uint2 v_column(const uint4* v, int n) {
  auto word = [](const uint4& u, int k) -> uint32_t {
    return k == 0 ? u.x : (k == 1 ? u.y : (k == 2 ? u.z : u.w));
  };
  const uint32_t sel = (n & 1) ? 0x07060302u : 0x05040100u;
  const int k = n >> 1;
  return make_uint2(__builtin_amdgcn_perm(word(v[1], k), word(v[0], k), sel),
                    __builtin_amdgcn_perm(word(v[3], k), word(v[2], k), sel));
}

// Maximum and sum over the four lanes of an MFMA column (lanes l, l^16,
// l^32, l^48), with the gfx950 row-swap instructions: permlane16_swap of x
// with itself yields the values of rows (0,0,2,2) and (1,1,3,3), so
// combining the two results reduces over row pairs; permlane32_swap does the
// same for the two halves. The combination is symmetric, so every lane gets
// the same value in the same order.
__device__ __forceinline__ float column_max(float x) {
  uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  u = __float_as_uint(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
  auto t = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float column_sum(float x) {
  uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  u = __float_as_uint(__uint_as_float(r[0]) + __uint_as_float(r[1]));
  auto t = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}


// ---- fp8 (OCP E4M3) cache ---------------------------------------------------
// Four E4M3 codes (one dword, byte 0 first) as four 16-bit values of the
// query's type, in the same order. Every E4M3 value is exact in f16 and bf16;
// the gfx950 conversion takes a power-of-two scale, here 2^0.
template <int DT>
__device__ __forceinline__ uint2 e4m3x4_widen(uint32_t w) {
  if constexpr (DT == KV_BF16)
    return make_uint2(
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)));
  else
    return make_uint2(
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)));
}
template <int DT>
__device__ __forceinline__ uint4 e4m3x8_widen(uint32_t a, uint32_t b) {
  const uint2 lo = e4m3x4_widen<DT>(a), hi = e4m3x4_widen<DT>(b);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// The E4M3 code of x / scale: the quotient rounded to nearest even in fp32,
// then to the nearest E4M3 value (ties to even); magnitudes past 448 and
// infinities saturate to 448, NaN becomes 0x7F. The hardware conversion
// rounds to nearest even; the clamp before it gives the saturation. It
// writes every NaN as 0xFF, so the sign bit of a NaN byte is cleared after.
__device__ __forceinline__ float e4m3_operand(float x, float scale) {
  const float y = __fdiv_rn(x, scale);
  return y != y ? y : fminf(fmaxf(y, -448.0f), 448.0f);
}
__device__ __forceinline__ uint32_t e4m3x4_pack(float a, float b, float c, float d, float scale) {
  const float ya = e4m3_operand(a, scale), yb = e4m3_operand(b, scale);
  const float yc = e4m3_operand(c, scale), yd = e4m3_operand(d, scale);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ya, yb, 0, false);
  const uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(yc, yd, lo, true);
  const uint32_t nan_sign = (ya != ya ? 0x80u : 0u) | (yb != yb ? 0x8000u : 0u) |
                            (yc != yc ? 0x800000u : 0u) | (yd != yd ? 0x80000000u : 0u);
  return w & ~nan_sign;
}
// Eight 16-bit values (one uint4) of type DT as eight E4M3 codes.
template <int DT>
__device__ __forceinline__ uint2 e4m3x8_from16(const uint4& u, float scale) {
  float f[8];
  unpack16<DT>(u, f);
  return make_uint2(e4m3x4_pack(f[0], f[1], f[2], f[3], scale),
                    e4m3x4_pack(f[4], f[5], f[6], f[7], scale));
}

// ---- host-side helpers ------------------------------------------------------
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline kv_status launch_status(const char* who) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KV_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return KV_OK;
}

inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace dev
}  // namespace pagedkv

namespace pagedkv {
// At most this many key ranges of a shared prefix (the combining kernel holds
// one value per range in registers).
constexpr int kMaxSharedParts = 16;
// Key ranges the shared-prefix attention cuts shared_len positions into:
// returns their number (0 for invalid sizes) and sets *part_keys to the
// positions per range (a multiple of 32).
int32_t shared_prefix_parts(int32_t S, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t shared_len, int32_t* part_keys);
// Attention of S decode queries over the first shared_len positions of table
// row 0, which every sequence of the call shares, one launch over the ranges
// of shared_prefix_parts: range k's normalised outputs to o + k*S*Hq*D, log2
// of its softmax denominators (base-2 units) to lse + k*S*Hq. With kv8 the
// pools hold E4M3 codes: the K scale multiplies the scores (and so enters the
// denominators' units) and the V scale the outputs. Defined in
// shared_prefix.hip; the caller checks the arguments.
kv_status shared_prefix_attention(float* o, float* lse, const void* q, const void* k_pool,
                                  const void* v_pool, const int32_t* table_row0,
                                  int32_t max_blocks, int32_t S, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t block_size, int32_t num_blocks,
                                  float scale, kv_dtype dtype, int32_t shared_len, bool kv8,
                                  float k_scale, float v_scale, hipStream_t stream);
}  // namespace pagedkv

#endif  // PAGEDKV_DEVICE_COMMON_H_

// Device-side helpers shared by the OCTOPUS HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "octo_internal.hpp"

namespace octo {

enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

template <int D, int B>
struct Codec {
  static constexpr int T = (D + 2) / 3;          // triplets, zero padded
  static constexpr int BX = B + 1;               // bits of xi   ([YL] 非均匀比特分配:
  static constexpr int BE = B + 1;               // bits of eta    direction b+1,
  static constexpr int BR = B - 1;               // bits of rho    length b-1)
  static constexpr int BT = BX + BE + BR;        // bits per triplet (3b+1)
  static constexpr int W = (T * BT + 31) / 32;   // u32 words per key
  static constexpr int LX = 1 << BX, LE = 1 << BE, LR = 1 << BR;
  static constexpr int NDIR = 1 << (BX + BE);
  static constexpr uint32_t DIR_MASK = NDIR - 1;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return __half2float(__ushort_as_half((unsigned short)(w & 0xffffu)));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return __half2float(__ushort_as_half((unsigned short)(w >> 16)));
}

// Convert one 16-byte chunk of dtype DT to floats (8 for 16-bit types, 4 for f32).
template <int DT>
__device__ __forceinline__ void cvt_chunk(const uint4& c, float* out) {
  if constexpr (DT == DT_F32) {
    out[0] = __uint_as_float(c.x); out[1] = __uint_as_float(c.y);
    out[2] = __uint_as_float(c.z); out[3] = __uint_as_float(c.w);
  } else if constexpr (DT == DT_BF16) {
    out[0] = bf16_lo(c.x); out[1] = bf16_hi(c.x); out[2] = bf16_lo(c.y); out[3] = bf16_hi(c.y);
    out[4] = bf16_lo(c.z); out[5] = bf16_hi(c.z); out[6] = bf16_lo(c.w); out[7] = bf16_hi(c.w);
  } else {
    out[0] = f16_lo(c.x); out[1] = f16_hi(c.x); out[2] = f16_lo(c.y); out[3] = f16_hi(c.y);
    out[4] = f16_lo(c.z); out[5] = f16_hi(c.z); out[6] = f16_lo(c.w); out[7] = f16_hi(c.w);
  }
}

template <int DT> struct DtSize { static constexpr int v = DT == DT_F32 ? 4 : 2; };

// Unnormalised Walsh-Hadamard transform y = H_D x in registers, Sylvester
// order (H_2m = [[H_m, H_m], [H_m, -H_m]]): in-place butterflies of stride
// 1, 2, 4, ...  ([YL] 旋转魔法 / 工程实现: O(d log d) butterflies).
template <int D>
__device__ __forceinline__ void wht_regs(float (&v)[D]) {
#pragma unroll
  for (int h = 1; h < D; h <<= 1) {
#pragma unroll
    for (int i = 0; i < D; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        const float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
}

// Butterfly stages of stride h >= H0 only (the earlier ones already done).
template <int D, int H0>
__device__ __forceinline__ void wht_regs_from(float (&v)[D]) {
#pragma unroll
  for (int h = H0; h < D; h <<= 1) {
#pragma unroll
    for (int i = 0; i < D; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        const float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short bf16x4 __attribute__((ext_vector_type(4)));  // 4 bf16 bit patterns (MFMA operand)

__device__ __forceinline__ bf16x4 pack_bf16x4(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(bf16x4, make_uint2(lo, hi));
}
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// The first two butterfly stages (strides 1 and 2), i.e. H_4 applied to 4
// consecutive 16-bit elements, on the matrix cores: v_mfma_f32_4x4x4_16b_bf16
// (or _f16) with B = a lane's own 4 elements (the two packed words as they
// are stored, K = element order) and A = the 4 x 4 Sylvester H_4, row
// lane % 4 supplied by each lane of a 4-lane block, so lane l receives
// H_4 x of its own elements.  The products are exact (+-1 times a 16-bit
// value) and the sums fp32.  Every encoder forms these two stages this way,
// so all of them produce the same values.
typedef float wht4_t __attribute__((ext_vector_type(4)));
template <int DT>
__device__ __forceinline__ uint2 h4_row(int lane) {
  constexpr uint32_t one = DT == DT_BF16 ? 0x3f80u : 0x3c00u;
  const int m = lane & 3;
  uint32_t e[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) e[k] = one | ((uint32_t)(__builtin_popcount(m & k) & 1) << 15);
  return make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
}
template <int DT>
__device__ __forceinline__ wht4_t h4_apply(uint2 row, uint32_t w0, uint32_t w1) {
  const wht4_t z = {0.f, 0.f, 0.f, 0.f};
  if constexpr (DT == DT_BF16) {
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(pack_bf16x4(row.x, row.y), pack_bf16x4(w0, w1), z, 0, 0, 0);
  } else {
    typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(f16x4_t, make_uint2(row.x, row.y)),
                                              __builtin_bit_cast(f16x4_t, make_uint2(w0, w1)), z, 0, 0, 0);
  }
}

// s .* v where bit j of the mask means s_j = -1 (flip the IEEE sign bit).
template <int D>
__device__ __forceinline__ void apply_signs(float (&v)[D], const uint32_t (&bits)[8]) {
#pragma unroll
  for (int j = 0; j < D; ++j) {
    const uint32_t m = ((bits[j >> 5] >> (j & 31)) & 1u) << 31;
    v[j] = __uint_as_float(__float_as_uint(v[j]) ^ m);
  }
}

// Nearest centroid by the midpoint rule i = #{k : x > m_k}, from LDS tables.
__device__ __forceinline__ int quant_lookup(float x, const uint8_t* lut, const float* mid, float lo,
                                            float inv_w, float nbm1) {
  float f = (x - lo) * inv_w;
  f = __builtin_fminf(__builtin_fmaxf(f, 0.0f), nbm1);
  const int base = lut[(int)f];
  return base + (x > mid[base] ? 1 : 0) + (x > mid[base + 1] ? 1 : 0);
}

// Bit field [pos, pos+bits) of a little-endian u32 stream held in registers.
// Called from fully unrolled loops, so pos and bits fold to constants and the
// word array stays in registers (one v_bfe or v_alignbit + v_and).
template <int W>
__device__ __forceinline__ uint32_t field_at(const uint32_t (&w)[W], int pos, int bits) {
  const int wi = pos >> 5, off = pos & 31;
  const uint32_t lo = w[wi];
  const uint32_t hi = (wi + 1 < W) ? w[wi + 1] : 0u;
  const uint32_t v = (off + bits <= 32) ? (lo >> off) : __builtin_amdgcn_alignbit(hi, lo, off);
  return v & ((1u << bits) - 1u);
}

// Tile layout of a per-key word stream (packed codes, QJL sign words): in a
// tile of 64 keys, words 4g .. 4g+3 of all keys form group g, stored
// [key][4]; the last W % 4 words form the last group, stored [key][W % 4];
// groups follow each other.  A lane moves its key's whole stream with W/4
// 16-byte accesses (+ one narrower), each wavefront access 1 KiB contiguous.
template <int W>
struct TileWords {
  static constexpr int NG = W / 4, R = W % 4;
  __device__ static __forceinline__ void load(const uint32_t* tile, int lane, uint32_t (&w)[W]) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const uint4 u = *(const uint4*)(tile + 256 * g + 4 * lane);
      w[4 * g] = u.x; w[4 * g + 1] = u.y; w[4 * g + 2] = u.z; w[4 * g + 3] = u.w;
    }
    const uint32_t* r = tile + 256 * NG + R * lane;
    if constexpr (R == 1) {
      w[4 * NG] = r[0];
    } else if constexpr (R == 2) {
      const uint2 u = *(const uint2*)r;
      w[4 * NG] = u.x; w[4 * NG + 1] = u.y;
    } else if constexpr (R == 3) {
      w[4 * NG] = r[0]; w[4 * NG + 1] = r[1]; w[4 * NG + 2] = r[2];
    }
  }
  __device__ static __forceinline__ void store(uint32_t* tile, int lane, const uint32_t (&w)[W]) {
#pragma unroll
    for (int g = 0; g < NG; ++g)
      *(uint4*)(tile + 256 * g + 4 * lane) = make_uint4(w[4 * g], w[4 * g + 1], w[4 * g + 2], w[4 * g + 3]);
    uint32_t* r = tile + 256 * NG + R * lane;
    if constexpr (R == 1) {
      r[0] = w[4 * NG];
    } else if constexpr (R == 2) {
      *(uint2*)r = make_uint2(w[4 * NG], w[4 * NG + 1]);
    } else if constexpr (R == 3) {
      r[0] = w[4 * NG]; r[1] = w[4 * NG + 1]; r[2] = w[4 * NG + 2];
    }
  }
};

// Pointer into the constant address space: uniform loads through it become
// scalar loads (s_load) whose results feed VALU ops as SGPR operands.
typedef const __attribute__((address_space(4))) float cfloat;

// An SGPR zero the compiler cannot see through.  Adding it to a loop's
// constant-memory indices keeps those loads inside the loop (reloaded from
// the scalar cache) instead of being hoisted into hundreds of VGPRs.
__device__ __forceinline__ int opaque_zero() {
  int z = 0;
  asm volatile("" : "+s"(z));
  return z;
}

// Wave64 all-reduce with DPP: xor 1, xor 2 (quad_perm), half-row mirror,
// row mirror give every lane its 16-lane row result; the four rows are then
// combined through lanes 0, 16, 32, 48.
template <typename Op>
__device__ __forceinline__ float wave_allreduce(float x, Op op) {
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false)));
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false)));
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false)));
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false)));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return op(op(r0, r1), op(r2, r3));
}

struct OpMax { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };
struct OpAdd { __device__ float operator()(float a, float b) const { return a + b; } };

__device__ __forceinline__ float wave_max(float x) { return wave_allreduce(x, OpMax()); }
__device__ __forceinline__ float wave_sum(float x) { return wave_allreduce(x, OpAdd()); }

}  // namespace octo

// OCTOPUS online key encoder for gfx950.
//
// One wavefront encodes a tile of 64 keys, one key per lane, entirely in
// registers ([YL] 三元组分解, steps 1-4):
//   gamma = |k| (fp32, stored), y = H (s .* k) by in-register butterflies
//   ([YL] 旋转魔法 / 工程实现), triplets t_i of the zero-padded y, rho_i^2 =
//   |t_i|^2/|y|^2, octahedral (xi, eta) of t_i ([YL] 八面体折叠), Lloyd-Max
//   nearest-centroid indices from bucketed LDS tables, bit-pack, store.
// The key tile is read with coalesced 16-byte loads and handed to the lanes
// through a 16-row LDS buffer per wave in four phases (small LDS footprint,
// several waves per SIMD); packed words are stored in the tile's word-group
// layout (16-byte stores, 1 KiB contiguous per store instruction).  With QJL
// the same lane also forms the rotated residual r' = u' - u'^ and its fp16
// norm, and the wave the signs of S r' on the matrix cores
// ([YL] 可选的残差修正).  Joint rounding ([YL] 联合取整) is a template
// variant.  Included by k_encode_b<N>.hip, one translation unit per bit budget.
#pragma once

#include <algorithm>

#include "octo_device.hpp"
#include "octo_encode_dev.hpp"

// Floating-point expressions here are evaluated exactly as written (fma only
// where a builtin says so): the bulk and the one-key encoders then round the
// same operations the same way and write identical words and gamma.
#pragma clang fp contract(off)

namespace octo {

// Stage the key rows [r0, r0 + NR) of the wave's 64-key tile into LDS with
// coalesced 16-byte loads (consecutive lanes read consecutive chunks).  The
// WHT sign flips are applied here, on the raw chunk bits: every lane always
// handles the same chunk column, so one 16-byte mask per lane does it.
// NRW rows per phase: 16, or 8 where the block's LDS is short.
template <int D, int KT, int NRW = 16>
struct Stage {
  static constexpr int ES = DtSize<KT>::v;
  static constexpr int ROWB = D * ES;       // bytes per key row
  static constexpr int CPR = ROWB / 16;     // 16-byte chunks per row
  static constexpr int PITCH = ROWB + 16;   // padded pitch: conflict-free row reads
  static constexpr int VPC = 16 / ES;       // values per chunk
  static constexpr int NR = NRW;            // rows staged per phase
  static_assert(NR * CPR % 64 == 0 && kTile % NR == 0, "whole chunks per lane and phases per tile");
  static constexpr int NP = kTile / NR;     // phases
  static constexpr int PER_LANE = NR * CPR / 64;
};

// Sign mask of the chunk a lane stages: sign bit of every element whose WHT
// sign is -1 (bit 15 of a 16-bit element, bit 31 of an fp32 one).
template <int D, int KT>
__device__ __forceinline__ uint4 chunk_sign_mask(const uint32_t (&sign_bits)[8], int col) {
  using S = Stage<D, KT>;
  uint32_t m[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < S::VPC; ++e) {
    const int j = col * S::VPC + e;
    const uint32_t bit = (sign_bits[j >> 5] >> (j & 31)) & 1u;
    if constexpr (S::ES == 2) m[e >> 1] |= bit << (16 * (e & 1) + 15);
    else m[e] |= bit << 31;
  }
  return make_uint4(m[0], m[1], m[2], m[3]);
}

// Row pitch (bytes) up to which a full tile's offsets fit 32 bits.
constexpr int64_t kMaxFastRowBytes = int64_t(1) << 24;
// Fourth word of a raw (unformatted, stride 0) buffer descriptor on gfx9.
constexpr int kBufferDescWord3 = 0x00020000;

// The raw 16-byte chunks of the 64-key tile at j0: coalesced loads, NP
// phases of NR rows (rows past n_new re-read the last key, so the loads
// carry no conditions).  FAST (j0 wave-uniform): a full tile takes buffer
// loads at scalar row offsets instead, with one 32-bit lane offset for all
// of them.  That pays in the QJL encoder, whose waves walk several tiles;
// in the one-tile-per-wave encoder the cheaper issue measured 2-3 % slower
// (the tile's loads then leave in one burst, all waves in step).
template <int D, int KT, bool FAST, int NRW = 16>
__device__ __forceinline__ void load_rows(const EncodeArgs& a, int64_t seq, int64_t j0, int lane,
                                          uint4 (&raw)[Stage<D, KT, NRW>::NP][Stage<D, KT, NRW>::PER_LANE]) {
  using S = Stage<D, KT, NRW>;
  const unsigned char* kbase = (const unsigned char*)a.keys + (seq * a.seq_stride) * S::ES;
  const int col = lane % S::CPR;
  const int64_t rs = a.key_stride * S::ES;  // bytes between key rows
  if (FAST && j0 + kTile <= a.n_new && rs <= kMaxFastRowBytes) {
    // A full tile (j0 is wave-uniform): buffer loads from the tile's first
    // row, row h NR + lane / CPR + k (64 / CPR) at the lane's own 32-bit
    // offset plus a scalar one, no clamp and no 64-bit address arithmetic
    // per load.  The record range covers the tile's 64 rows.
    const unsigned char* tb = kbase + j0 * rs;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)tb, (short)0, (int)(63 * rs + S::ROWB), kBufferDescWord3);
    const int voff = (lane / S::CPR) * (int)rs + col * 16;
#pragma unroll
    for (int h = 0; h < S::NP; ++h) {
#pragma unroll
      for (int k = 0; k < S::PER_LANE; ++k) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(
            rsrc, voff, (h * S::NR + k * (64 / S::CPR)) * (int)rs, 0);
        raw[h][k] = make_uint4(x[0], x[1], x[2], x[3]);
      }
    }
    return;
  }
#pragma unroll
  for (int h = 0; h < S::NP; ++h) {
#pragma unroll
    for (int k = 0; k < S::PER_LANE; ++k) {
      const int f = lane + 64 * k;
      int64_t j = j0 + h * S::NR + f / S::CPR;
      j = j < a.n_new ? j : a.n_new - 1;
      raw[h][k] = *(const uint4*)(kbase + (j * a.key_stride) * S::ES + col * 16);
    }
  }
}

// Hand every lane its own key row (sign-flipped, raw bits) through the
// wave's LDS buffer of NR rows, one phase at a time.
template <int D, int KT, int NRW = 16>
__device__ __forceinline__ void stage_rows(const uint4 (&raw)[Stage<D, KT, NRW>::NP][Stage<D, KT, NRW>::PER_LANE],
                                           int lane, unsigned char* s_keys, const uint4& smask,
                                           uint4 (&rowbits)[Stage<D, KT, NRW>::CPR]) {
  using S = Stage<D, KT, NRW>;
  const int col = lane % S::CPR;
  const int my_phase = lane / S::NR;
  const unsigned char* row = s_keys + (lane % S::NR) * S::PITCH;
#pragma unroll
  for (int h = 0; h < S::NP; ++h) {
#pragma unroll
    for (int k = 0; k < S::PER_LANE; ++k) {
      const int f = lane + 64 * k;
      uint4 u = raw[h][k];
      u.x ^= smask.x; u.y ^= smask.y; u.z ^= smask.z; u.w ^= smask.w;
      *(uint4*)(s_keys + (f / S::CPR) * S::PITCH + col * 16) = u;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (my_phase == h) {
#pragma unroll
      for (int c = 0; c < S::CPR; ++c) rowbits[c] = *(const uint4*)(row + c * 16);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// The three bucket tables (nb + 2 <= kMaxLut + 2 entries each) into LDS
// by NTH threads: every thread requests all of its entries before it stores
// any, so the block waits one memory round trip for them, not one per table
// and per round of a copy loop.
template <int NTH>
__device__ __forceinline__ void copy_bucket_tables(const DevTables& t, uint2* s_qx, uint2* s_qe,
                                                   uint2* s_qr, int tid) {
  constexpr int R = (kMaxLut + 2 + NTH - 1) / NTH;
  const Bucket1* q[3] = {&t.qx, &t.qe, &t.qr2};
  uint2* dst[3] = {s_qx, s_qe, s_qr};
  uint2 v[3][R];
#pragma unroll
  for (int k = 0; k < 3; ++k)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = tid + NTH * r;
      v[k][r] = i < q[k]->nb + 2 ? q[k]->t[i] : make_uint2(0u, 0u);
    }
#pragma unroll
  for (int k = 0; k < 3; ++k)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = tid + NTH * r;
      if (i < q[k]->nb + 2) dst[k][i] = v[k][r];
    }
}

// Waves (64-key tiles in flight) per encoder block: 4, or 8 with QJL below
// 5 bits, where one block per CU holds the LDS copy of S and two waves per
// SIMD then overlap one wave's projection on the matrix cores with the
// other's VALU work (at b = 5 the 4096-entry direction table leaves no room
// for 8 waves' staging buffers).
template <bool QJL, int B>
constexpr int enc_waves() { return QJL && B < 5 ? 8 : 4; }

// Key rows staged per phase: 8 for fp32 keys with QJL at d = 128, b = 5,
// where the f16 QJL matrix (68 KiB) and the 4096-entry direction table
// (64 KiB) leave 26 KiB of LDS for the four waves' staging buffers; else 16.
template <int D, int B, int KT, bool QJL>
constexpr int enc_stage_rows() { return QJL && B >= 5 && KT == DT_F32 && D == 128 ? 8 : 16; }

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// v_writelane_b32: a wave-uniform value into one lane of a VGPR.
extern "C" __device__ int octo_writelane(int val, int lane, int old) __asm("llvm.amdgcn.writelane.i32");

// QJL matrix in LDS: planes [S_hi | S_lo] of f16 rows, padded so that the 32
// rows one B-operand load touches fall on distinct banks.
template <int D>
struct SLds {
  static constexpr int PITCH = 2 * D + 16;      // bytes per row
  static constexpr int BYTES = 2 * D * PITCH;   // both planes
  static constexpr int CPRS = 2 * D / 16;       // 16-byte chunks per row
  static constexpr int CHUNKS = 2 * D * CPRS;   // chunks copied (the whole f16 table)
  // 16-byte LDS slot past the last one the copy writes
  static constexpr int SLOT_END = ((CHUNKS - 1) / CPRS) * (PITCH / 16) + (CHUNKS - 1) % CPRS + 1;
  static_assert(PITCH % 16 == 0 && SLOT_END * 16 <= BYTES, "the S copy stays inside its LDS rows");
};

// QJL signs of the wave's 64 residuals on the matrix cores: P = R' S^T for
// the 64 keys x d projections, P[key][j] = <S_j, r'_key>, bit j of the key's
// sign words = (P >= 0) ([YL] 可选的残差修正; sgn(0) = +1).
//   r' (one key per lane, fp32, scaled by 2^12: signs unchanged, f16 range
//   kept) and S are split into f16 high and low parts, x = x_hi + x_lo with
//   both parts rounded to nearest; the product is summed from the three
//   terms hi*hi + hi*lo + lo*hi on v_mfma_f32_32x32x16_f16 (products exact,
//   fp32 accumulate).  The dropped lo*lo term and the rounding of the low
//   parts leave a relative error near 2^-23 |S_jk| |r'_k| per term.
//   A operands: rows = keys.  Lane (l % 32, g = l / 32) of the 32-key block
//   supplies dims 16 kb + 8 g .. + 7 of its row; a lane holds its own key's
//   dims, so v_permlane32_swap exchanges the upper half of the dims 0..7
//   words with the lower half of the dims 8..15 words, which yields the
//   operands of key block 0 (keys 0..31) and key block 1 (keys 32..63).
//   B operands: S rows j = 32 nb + l % 32, dims 16 kb + 8 g .. + 7, from LDS.
//   Output register r of lane (l % 32, g) is key 8 (r / 4) + 4 g + r % 4 of the
//   block and projection l % 32 of the block: a ballot over the wave gives the
//   32 sign bits of two keys at once, written into those keys' lanes.
template <int D>
__device__ __forceinline__ void qjl_signs(const float (&v)[D], const unsigned char* s_S, int lane,
                                          uint32_t (&sw)[D / 32]) {
  constexpr int NK = D / 16;  // 16-dim contraction blocks
  constexpr int NN = D / 32;  // 32-projection output blocks
  constexpr int PITCH = SLds<D>::PITCH;
  half8 ah[2][NK], al[2][NK];
#pragma unroll
  for (int kb = 0; kb < NK; ++kb) {
    uint32_t ph[8], pl[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const float x0 = v[16 * kb + 2 * p] * 4096.f, x1 = v[16 * kb + 2 * p + 1] * 4096.f;
      const __half2 h = __float22half2_rn(make_float2(x0, x1));
      const float2 hf = __half22float2(h);
      const __half2 l = __float22half2_rn(make_float2(x0 - hf.x, x1 - hf.y));
      ph[p] = __builtin_bit_cast(uint32_t, h);
      pl[p] = __builtin_bit_cast(uint32_t, l);
    }
    uint32_t h0[4], h1[4], l0[4], l1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto sh = __builtin_amdgcn_permlane32_swap(ph[i], ph[4 + i], false, false);
      h0[i] = sh[0];
      h1[i] = sh[1];
      const auto sl = __builtin_amdgcn_permlane32_swap(pl[i], pl[4 + i], false, false);
      l0[i] = sl[0];
      l1[i] = sl[1];
    }
    ah[0][kb] = __builtin_bit_cast(half8, make_uint4(h0[0], h0[1], h0[2], h0[3]));
    ah[1][kb] = __builtin_bit_cast(half8, make_uint4(h1[0], h1[1], h1[2], h1[3]));
    al[0][kb] = __builtin_bit_cast(half8, make_uint4(l0[0], l0[1], l0[2], l0[3]));
    al[1][kb] = __builtin_bit_cast(half8, make_uint4(l1[0], l1[1], l1[2], l1[3]));
  }
  // The B operands are the same for every tile: an offset the compiler
  // cannot see through (always 0) keeps their LDS reads inside the tile loop
  // instead of hoisting all of them into registers ahead of it.
  int opaque0;
  asm volatile("v_mov_b32 %0, 0" : "=v"(opaque0));
  const int ln = lane & 31, g = lane >> 5;
  s_S += opaque0;
#pragma unroll
  for (int nb = 0; nb < NN; ++nb) {
    floatx16 c[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) { c[0][r] = 0.f; c[1][r] = 0.f; }
    const unsigned char* row = s_S + (32 * nb + ln) * PITCH + 16 * g;
#pragma unroll
    for (int kb = 0; kb < NK; ++kb) {
      const half8 bh = *(const half8*)(row + 32 * kb);
      const half8 bl = *(const half8*)(row + D * PITCH + 32 * kb);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        c[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[mb][kb], bh, c[mb], 0, 0, 0);
        c[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[mb][kb], bl, c[mb], 0, 0, 0);
        c[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[mb][kb], bh, c[mb], 0, 0, 0);
      }
    }
    int w = 0;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint64_t m = __ballot(c[mb][r] >= 0.f);
        const int key = 32 * mb + 8 * (r >> 2) + (r & 3);
        w = octo_writelane((int)(uint32_t)m, key, w);
        w = octo_writelane((int)(uint32_t)(m >> 32), key + 4, w);
      }
    sw[nb] = (uint32_t)w;
  }
}

// Joint rounding of one unit triplet (x, y, z) ([YL] 联合取整): among the
// 3x3 direction codes around the scalar (xi, eta) indices c0 (clamped to the
// index range), each with its best rho^ (the centroid nearest s = <n^, t>,
// from the squared-midpoint table on max(s, 0)^2), the code with the least
// error |t - rho^ n^|^2 - |t|^2 = rho^ (rho^ - 2s); the first strict minimum
// in (xi, eta) offset order wins.
template <class C>
__device__ __forceinline__ uint32_t joint_code(float x, float y, float z, uint32_t c0,
                                               const float4* s_dir, const float* s_rho,
                                               const uint2* s_qr, float sr, float mr) {
  const int ix = (int)(c0 & (C::LX - 1)), ie = (int)(c0 >> C::BX);
  float best_e = INFINITY;
  uint32_t best = 0u;
#pragma unroll
  for (int da = -1; da <= 1; ++da) {
    const int ja = min(max(ix + da, 0), C::LX - 1);
#pragma unroll
    for (int dc = -1; dc <= 1; ++dc) {
      const int jc = min(max(ie + dc, 0), C::LE - 1);
      const uint32_t xe = (uint32_t)ja | ((uint32_t)jc << C::BX);
      const float4 n = s_dir[xe];
      const float sdot = __builtin_fmaf(n.x, x, __builtin_fmaf(n.y, y, n.z * z));
      const float sp = __builtin_fmaxf(sdot, 0.f);
      const uint32_t jr = quant1_clamp(sp * sp, s_qr, sr, mr);
      const float r = s_rho[jr];
      const float err = r * (r - 2.f * sdot);
      if (err < best_e) {
        best_e = err;
        best = xe | (jr << (C::BX + C::BE));
      }
    }
  }
  return best;
}

// The lane's key from the tile's raw rows: staged through LDS, then as fp32
// values (16-bit keys: after WHT strides 1 and 2, taken on the matrix cores
// straight from the packed elements by h4_apply).
template <int D, int KT, int NRW>
__device__ __forceinline__ void tile_values(const uint4 (&raw)[Stage<D, KT, NRW>::NP][Stage<D, KT, NRW>::PER_LANE],
                                            int lane, unsigned char* s_keys, const uint4& smask,
                                            float (&v)[D]) {
  using S = Stage<D, KT, NRW>;
  uint4 rowbits[S::CPR];
  stage_rows<D, KT, NRW>(raw, lane, s_keys, smask, rowbits);
  if constexpr (KT == DT_F32) {
#pragma unroll
    for (int c = 0; c < S::CPR; ++c) cvt_chunk<KT>(rowbits[c], &v[c * S::VPC]);
  } else {
    const uint2 h4 = h4_row<KT>(lane);
#pragma unroll
    for (int c = 0; c < S::CPR; ++c) {
      const wht4_t y0 = h4_apply<KT>(h4, rowbits[c].x, rowbits[c].y);
      const wht4_t y1 = h4_apply<KT>(h4, rowbits[c].z, rowbits[c].w);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[8 * c + k] = y0[k];
        v[8 * c + 4 + k] = y1[k];
      }
    }
  }
}

// Keys with entries far from 1 in magnitude are scaled by an exact power of
// two (changes no ratio) so that no triplet energy under- or overflows: the
// exponent of the largest value (after strides 1 and 2 for 16-bit keys, of
// the raw values for fp32 keys) decides, as in every encoder.  Returns it
// (0: not scaled).
template <int D>
__device__ __forceinline__ int prescale_scan(float (&v)[D]) {
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < D; ++j) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[j]));
  int ex = 0;
  __builtin_frexpf(amax, &ex);
  const int sexp = (ex > 50 || ex < -50) && amax > 0.f ? ex : 0;
  if (__any(sexp != 0)) {
    const float scale = __builtin_ldexpf(1.0f, -sexp);
#pragma unroll
    for (int j = 0; j < D; ++j) v[j] *= scale;
  }
  return sexp;
}

// A range of |y|^2 (y: the key after the whole unnormalised WHT) inside which
// prescale_scan leaves the key alone.  y's squared norm is F times that of the
// values prescale_scan looks at (F = D / 4 after strides 1 and 2, D for raw
// fp32 values), and that lies in [amax^2, D amax^2].  prescale_scan scales
// when amax >= 2^50 (then |y|^2 >= F 2^100) or 0 < amax < 2^-51 (then
// |y|^2 < F D 2^-102); with a factor 2 of margin for the rounding of the sum,
// |y|^2 in [F D 2^-101, F 2^99), or 0, means amax in [2^-51, 2^50) or 0.
template <int D, int KT>
struct NormRange {
  static constexpr float F = KT == DT_F32 ? (float)D : (float)(D / 4);
  static constexpr float LO = F * (float)D * 0x1p-101f;
  static constexpr float HI = F * 0x1p99f;
  __device__ static bool unscaled(float tot) { return tot == 0.f || (tot >= LO && tot < HI); }
};

// Encode the 64-key tile at j0 from its raw rows (load_rows): one key per
// lane, entirely in registers.
template <int D, int B, int KT, bool QJL, bool JR, int NRW = 16>
__device__ __forceinline__ void encode_tile(const EncodeArgs& a, int64_t seq, int64_t j0, int lane,
                                            const uint4 (&raw)[Stage<D, KT, NRW>::NP][Stage<D, KT, NRW>::PER_LANE],
                                            unsigned char* s_keys, const uint4& smask,
                                            const uint2* s_qx, const uint2* s_qe, const uint2* s_qr,
                                            const unsigned char* s_S, const float4* s_dir,
                                            const float* s_rho) {
  using C = Codec<D, B>;
  using S = Stage<D, KT, NRW>;
  constexpr int T = C::T, W = C::W;
  // The plain encoder skips the magnitude scan: it checks |y|^2 after the
  // transform instead, and only a tile with a key outside NormRange is
  // formed again with the scan.  A key inside the range is one the scan
  // leaves alone, so every key gets the same words as in the other encoders.
  constexpr bool CHECK = !QJL && !JR;
  float v[D];
  tile_values<D, KT, NRW>(raw, lane, s_keys, smask, v);
  int sexp = 0;
  if constexpr (!CHECK) sexp = prescale_scan<D>(v);
  if constexpr (KT == DT_F32) wht_regs<D>(v);
  else wht_regs_from<D, 4>(v);

  const float sx = a.t.qx.scale, bx = a.t.qx.bias;
  const float se = a.t.qe.scale, be = a.t.qe.bias;
  // (the rho^2 table starts at 0: bias 0)
  const float sr = a.t.qr2.scale, mr = (float)(a.t.qr2.nb - 1);
  uint32_t words[W];
#pragma unroll
  for (int w = 0; w < W; ++w) words[w] = 0u;
  const int64_t j = j0 + lane;
  const bool valid = j < a.n_new;
  const int64_t pos = a.pos0 + j;
  const int64_t tiles = a.cap / kTile;
  float tot = 0.f;
  if constexpr (CHECK) {
    // Pass 1: |y|^2 (the energies are formed again in pass 2, as the same
    // operations: holding all T of them would cost T registers)
#pragma unroll
    for (int i = 0; i < T; ++i) {
      float x, y, z;
      triplet_of<D>(v, i, x, y, z);
      tot += triplet_energy(x, y, z);
    }
    if (__any(!NormRange<D, KT>::unscaled(tot))) {
      // rare: a key far from unit magnitude; the tile again, with the scan
      // (the lane index passes through an empty asm, so that the compiler
      // cannot hoist these loads and their addresses out of the branch)
      int lane2 = lane;
      asm volatile("" : "+v"(lane2));
      uint4 raw2[S::NP][S::PER_LANE];
      load_rows<D, KT, false, NRW>(a, seq, j0, lane2, raw2);
      tile_values<D, KT, NRW>(raw2, lane2, s_keys, smask, v);
      sexp = prescale_scan<D>(v);
      if constexpr (KT == DT_F32) wht_regs<D>(v);
      else wht_regs_from<D, 4>(v);
      tot = 0.f;
#pragma unroll
      for (int i = 0; i < T; ++i) {
        float x, y, z;
        triplet_of<D>(v, i, x, y, z);
        tot += triplet_energy(x, y, z);
      }
    }
    // Pass 2: the (xi, eta) indices and the rho index from rho_i^2 =
    // e_i / |y|^2 against the squared midpoints, each code packed once.
    const RhoQuant<C::LR> rq(a.t, tot);
#pragma unroll
    for (int i = 0; i < T; ++i) {
      float x, y, z;
      triplet_of<D>(v, i, x, y, z);
      pack_code<C::BT>(words, i, xi_eta_code<C::BX>(x, y, z, s_qx, sx, bx, s_qe, se, be) |
                                     (rq.index(triplet_energy(x, y, z), s_qr, sr, mr) << (C::BX + C::BE)));
    }
  } else if constexpr (!JR) {
    // (QJL) Pass 1: |y|^2; pass 2: the codes, each packed once, with the
    // energies formed again rather than held (T registers fewer through the
    // residual and its projection).
#pragma unroll
    for (int i = 0; i < T; ++i) {
      float x, y, z;
      triplet_of<D>(v, i, x, y, z);
      tot += triplet_energy(x, y, z);
    }
    const RhoQuant<C::LR> rq(a.t, tot);
#pragma unroll
    for (int i = 0; i < T; ++i) {
      float x, y, z;
      triplet_of<D>(v, i, x, y, z);
      pack_code<C::BT>(words, i, xi_eta_code<C::BX>(x, y, z, s_qx, sx, bx, s_qe, se, be) |
                                     (rq.index(triplet_energy(x, y, z), s_qr, sr, mr) << (C::BX + C::BE)));
    }
  } else {
    // Joint rounding ([YL] 联合取整).  Pass 1: the energy and the scalar
    // (xi, eta) indices, the centre of the search.  Pass 2, per triplet t of
    // the unit key: for each of the 3x3 neighbouring direction codes (clamped
    // to the index range) with unit direction n^, the best rho^ is the
    // centroid nearest s = <n^, t> (the squared-midpoint table on max(s, 0)^2;
    // s <= 0 takes index 0), with error |t - rho^ n^|^2 - |t|^2 = rho^ (rho^ - 2s);
    // the first strict minimum in (xi, eta) offset order wins.
#pragma unroll
    for (int i = 0; i < T; ++i) {
      float x, y, z;
      triplet_of<D>(v, i, x, y, z);
      tot += triplet_energy(x, y, z);
      pack_code<C::BT>(words, i, xi_eta_code<C::BX>(x, y, z, s_qx, sx, bx, s_qe, se, be));
    }
    const float inv_norm = tot > 0.f ? __builtin_amdgcn_rsqf(tot) : 0.f;
    uint32_t wj[W];
#pragma unroll
    for (int w = 0; w < W; ++w) wj[w] = 0u;
    // (the search of joint_code, written out: the compiler schedules this
    // form of the loop better in this kernel)
#pragma unroll
    for (int i = 0; i < T; ++i) {
      float x, y, z;
      triplet_of<D>(v, i, x, y, z);
      x *= inv_norm;
      y *= inv_norm;
      z *= inv_norm;
      const uint32_t c0 = field_at<W>(words, i * C::BT, C::BX + C::BE);
      const int ix = (int)(c0 & (C::LX - 1)), ie = (int)(c0 >> C::BX);
      float best_e = INFINITY;
      uint32_t best = 0u;
#pragma unroll
      for (int da = -1; da <= 1; ++da) {
        const int ja = min(max(ix + da, 0), C::LX - 1);
#pragma unroll
        for (int dc = -1; dc <= 1; ++dc) {
          const int jc = min(max(ie + dc, 0), C::LE - 1);
          const uint32_t xe = (uint32_t)ja | ((uint32_t)jc << C::BX);
          const float4 n = s_dir[xe];
          const float sdot = __builtin_fmaf(n.x, x, __builtin_fmaf(n.y, y, n.z * z));
          const float sp = __builtin_fmaxf(sdot, 0.f);
          const uint32_t jr = quant1_clamp(sp * sp, s_qr, sr, mr);
          const float r = s_rho[jr];
          const float err = r * (r - 2.f * sdot);
          if (err < best_e) {
            best_e = err;
            best = xe | (jr << (C::BX + C::BE));
          }
        }
      }
      pack_code<C::BT>(wj, i, best);
    }
#pragma unroll
    for (int w = 0; w < W; ++w) words[w] = wj[w];
  }
  const float gamma = __builtin_ldexpf(__builtin_sqrtf(tot * (1.0f / D)), sexp);
  if (valid) {
    TileWords<W>::store(a.packed + (seq * tiles + (pos >> 6)) * W * kTile, (int)(pos & 63), words);
    a.gamma[seq * a.cap + pos] = gamma;
  }

  if constexpr (QJL) {
    if (a.qjl_bits != nullptr) {
      // Rotated unit-direction residual r' = u' - u'^ over the D real coordinates.
      const float inv_norm = tot > 0.f ? __builtin_amdgcn_rsqf(tot) : 0.f;
      float nu2 = 0.f;
#pragma unroll
      for (int i = 0; i < T; ++i) {
        const uint32_t code = field_at<W>(words, i * C::BT, C::BT);
        const float4 n = s_dir[code & C::DIR_MASK];
        const float rh = s_rho[code >> (C::BX + C::BE)];
        const float nc[3] = {n.x, n.y, n.z};
#pragma unroll
        for (int c = 0; c < 3; ++c) {
          if (3 * i + c < D) {
            const float r = __builtin_fmaf(v[3 * i + c], inv_norm, -rh * nc[c]);
            v[3 * i + c] = r;
            nu2 = __builtin_fmaf(r, r, nu2);
          }
        }
      }
      // the norm is formed here: left to itself the compiler sinks this sum
      // past the projection, keeping all D residuals live through it
      asm volatile("" : "+v"(nu2));
      const float nu = __builtin_sqrtf(nu2);
      uint32_t sbits[D / 32];
      qjl_signs<D>(v, s_S, lane, sbits);
      if (valid) {
        TileWords<D / 32>::store(a.qjl_bits + (seq * tiles + (pos >> 6)) * (D / 32) * kTile,
                                 (int)(pos & 63), sbits);
        a.qjl_norm[seq * a.cap + pos] = __half_as_ushort(__float2half_rn(nu));
      }
    }
  }
}

// Three waves per SIMD for the plain encoder of 16-bit keys (its state fits
// 168 registers once the triplet energies are formed again in the second
// pass instead of held); two otherwise (the one-key-per-lane state fits 256
// registers; left alone the allocator took 257 at b = 1 and halved the
// occupancy), except with QJL at 5 bits, where the LDS allows one wave per
// SIMD anyway.
template <int D, int B, int KT, bool QJL, bool JR>
__global__ __launch_bounds__((64 * enc_waves<QJL, B>()))
__attribute__((amdgpu_waves_per_eu(QJL && B >= 5 ? 1 : (!QJL && !JR && KT != DT_F32 ? 3 : 2)))) void k_encode(EncodeArgs a) {
  using C = Codec<D, B>;
  constexpr int NRW = enc_stage_rows<D, B, KT, QJL>();
  using S = Stage<D, KT, NRW>;
  constexpr int EW = enc_waves<QJL, B>();
  __shared__ __align__(16) unsigned char s_keys[EW][S::NR * S::PITCH];
  __shared__ uint2 s_qx[kMaxLut + 2], s_qe[kMaxLut + 2], s_qr[kMaxLut + 2];
  __shared__ __align__(16) unsigned char s_S[QJL ? SLds<D>::BYTES : 16];
  // unit directions and rho centroids (QJL residual, joint rounding)
  constexpr bool TABS = QJL || JR;
  __shared__ float4 s_dir[TABS ? C::NDIR : 1];
  __shared__ float s_rho[TABS ? C::LR : 1];

  // (with QJL the wave index is read as a scalar: tile bases and the
  // full-tile test of load_rows are then wave-uniform)
  const int lane = threadIdx.x & 63;
  const int wave = QJL ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : threadIdx.x >> 6;
  const int64_t seq = blockIdx.y;

  // the block's waves share the quantiser tables (and the QJL matrix)
  copy_bucket_tables<64 * EW>(a.t, s_qx, s_qe, s_qr, threadIdx.x);
  if constexpr (QJL) {
    constexpr int CPRS = SLds<D>::CPRS;
    for (int c = threadIdx.x; c < SLds<D>::CHUNKS; c += 64 * EW)
      *(uint4*)(s_S + (c / CPRS) * SLds<D>::PITCH + (c % CPRS) * 16) = a.t.S16[c];
  }
  if constexpr (TABS) {
    static_assert(C::LR <= 64 * EW, "one rho centroid per thread");
    for (int i = threadIdx.x; i < C::NDIR; i += 64 * EW) s_dir[i] = a.t.dirtab[i];
    if (threadIdx.x < C::LR) s_rho[threadIdx.x] = a.t.rho_tab[threadIdx.x];
  }
  __syncthreads();
  const uint4 smask = chunk_sign_mask<D, KT>(a.t.sign_bits, lane % S::CPR);
  // A wave encodes one 64-key tile; with QJL the grid is smaller than the
  // key count and the block's waves take tiles round-robin.
  for (int64_t j0 = ((int64_t)blockIdx.x * EW + wave) * kTile; j0 < a.n_new;
       j0 += (int64_t)gridDim.x * EW * kTile) {
    uint4 raw[S::NP][S::PER_LANE];
    load_rows<D, KT, QJL, NRW>(a, seq, j0, lane, raw);
    encode_tile<D, B, KT, QJL, JR, NRW>(a, seq, j0, lane, raw, s_keys[wave], smask, s_qx, s_qe, s_qr,
                                        s_S, s_dir, s_rho);
    if constexpr (!QJL) break;
  }
}

// ---------------------------------------------------------------------------
// Latency-optimised encoder for a few keys per sequence (the autoregressive
// step appends one key per sequence, [YL] 工程实现 / [AB] online): one
// wavefront per key (encode_one_key), words assembled in LDS, then stored.
// ---------------------------------------------------------------------------
template <int D, int B, int KT>
__global__ __launch_bounds__(256) void k_encode_one(EncodeArgs a) {
  using C = Codec<D, B>;
  constexpr int T = C::T, W = C::W;
  __shared__ float s_v[4][3 * T];
  __shared__ float s_e[4][T];
  __shared__ uint32_t s_w[4][W];
  __shared__ uint2 s_qx[kMaxLut + 2], s_qe[kMaxLut + 2], s_qr[kMaxLut + 2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  copy_bucket_tables<256>(a.t, s_qx, s_qe, s_qr, threadIdx.x);
  __syncthreads();
  const int64_t k = (int64_t)blockIdx.x * 4 + wave;  // keys flattened over (seq, new key)
  if (k >= a.n_new * a.seq_count) return;
  const int64_t seq = k / a.n_new, j = k % a.n_new;
  const int64_t pos = a.pos0 + j;
  const void* row = (const unsigned char*)a.keys +
                    (seq * a.seq_stride + j * a.key_stride) * DtSize<KT>::v;
  const float gamma = encode_one_key<D, B, KT>(row, a.t, s_qx, s_qe, s_qr, lane, s_v[wave],
                                               s_e[wave], s_w[wave]);
  if (lane < W) store_key_word<W>(a.packed, a.cap, seq, pos, lane, s_w[wave][lane]);
  if (lane == 0) a.gamma[seq * a.cap + pos] = gamma;
}

template <int D, int B, int KT>
inline hipError_t launch_encode_one_t(const EncodeArgs& a, int64_t n_seq, hipStream_t s) {
  if (a.t.qx.nb > kMaxLut || a.t.qe.nb > kMaxLut || a.t.qr2.nb > kMaxLut) return hipErrorInvalidValue;
  const int64_t keys = a.n_new * n_seq;
  hipLaunchKernelGGL((k_encode_one<D, B, KT>), dim3((unsigned)((keys + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Bulk encoder at d = 256: two lanes per key.  Lane l < 32 holds elements
// 0..127 of the wave's key l, lane l + 32 elements 128..255 of the same key;
// a wave encodes 32 keys.  Each lane runs the d = 128 machinery on its half
// (stride-1 butterflies from the packed pairs, strides 2..64 in registers),
// the stride-128 butterfly pairs the two lanes (v_permlane32_swap), and each
// lane quantises 43 triplets: triplets 0..42 (the last one takes element 128
// from the partner) and 43..85 (elements 129..255, zero padded).  The energy
// is summed serially in triplet order across the pair and every operation
// matches encode_one_key's, so both write identical words and gamma.
// ---------------------------------------------------------------------------
// The value lane ^ 32 holds.  A cross-lane read: call it with every lane
// active (never under a lane-dependent branch).
__device__ __forceinline__ uint32_t pair_xchg(uint32_t x, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return lane < 32 ? r[1] : r[0];
}
__device__ __forceinline__ float pair_xchg(float x, int lane) {
  return __uint_as_float(pair_xchg(__float_as_uint(x), lane));
}

template <int KT>
struct Half256 {
  using S = Stage<128, KT>;                 // a half row: 128 elements
  static constexpr int KPW = 32;            // keys per wave
};

// The 64 half rows of the wave's 32 keys at j0 (row r: key j0 + r % 32, half
// r / 32), loaded with coalesced 16-byte chunks as in load_rows; keys past
// n_new re-read the last key.
template <int KT>
__device__ __forceinline__ void load_half_rows(const EncodeArgs& a, int64_t seq, int64_t j0, int lane,
                                               uint4 (&raw)[Stage<128, KT>::NP][Stage<128, KT>::PER_LANE]) {
  using S = Stage<128, KT>;
  const unsigned char* kbase = (const unsigned char*)a.keys + (seq * a.seq_stride) * S::ES;
  const int col = lane % S::CPR;
#pragma unroll
  for (int h = 0; h < S::NP; ++h) {
#pragma unroll
    for (int k = 0; k < S::PER_LANE; ++k) {
      const int r = h * S::NR + (lane + 64 * k) / S::CPR;
      int64_t j = j0 + (r % 32);
      j = j < a.n_new ? j : a.n_new - 1;
      raw[h][k] = *(const uint4*)(kbase + (j * a.key_stride) * S::ES + (r / 32) * S::ROWB + col * 16);
    }
  }
}

// QJL signs of the wave's 32 keys at d = 256 (two lanes per key: lane l < 32
// holds dims 0..127 of key l's residual r', lane l + 32 dims 128..255) on
// the matrix cores, P = R' S^T, P[key][j] = <S_j, r'_key>, bit j of the key's
// sign words = (P >= 0) ([YL] 可选的残差修正; sgn(0) = +1).  The same three-term
// f16 split as qjl_signs; the contraction index is ordered so that every lane
// supplies its own dims: step kb of v_mfma_f32_32x32x16_f16 takes dims
// 128 g + 8 kb .. + 7 from lane (key, g) for the A operand and from S row
// j = 32 nb + l % 32 for the B operand, read straight from the f16 planes in
// global memory (S of d = 256 does not fit the LDS; 256 KiB, L2-resident).
// Output register r of lane (l % 32, g) is key 8 (r / 4) + 4 g + r % 4 and
// projection 32 nb + l % 32; the ballots give lane k (k < 32) key k's words.
__device__ __forceinline__ void qjl_signs256(const float (&v)[128], const uint4* S16, int lane,
                                             uint32_t (&sw)[8]) {
  constexpr int D = 256;
  half8 ah[16], al[16];
#pragma unroll
  for (int kb = 0; kb < 16; ++kb) {
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float x0 = v[8 * kb + 2 * p] * 4096.f, x1 = v[8 * kb + 2 * p + 1] * 4096.f;
      const __half2 h = __float22half2_rn(make_float2(x0, x1));
      const float2 hf = __half22float2(h);
      const __half2 l = __float22half2_rn(make_float2(x0 - hf.x, x1 - hf.y));
      ph[p] = __builtin_bit_cast(uint32_t, h);
      pl[p] = __builtin_bit_cast(uint32_t, l);
    }
    ah[kb] = __builtin_bit_cast(half8, make_uint4(ph[0], ph[1], ph[2], ph[3]));
    al[kb] = __builtin_bit_cast(half8, make_uint4(pl[0], pl[1], pl[2], pl[3]));
  }
  const int ln = lane & 31, g = lane >> 5;
  // 16-byte units: row j of a plane is 32 units, the lo plane follows the hi
#pragma unroll 1
  for (int nb = 0; nb < D / 32; ++nb) {
    const uint4* row = S16 + (32 * nb + ln) * (D / 8) + 16 * g;
    floatx16 c;
#pragma unroll
    for (int r = 0; r < 16; ++r) c[r] = 0.f;
#pragma unroll
    for (int kb = 0; kb < 16; ++kb) {
      const half8 bh = __builtin_bit_cast(half8, row[kb]);
      const half8 bl = __builtin_bit_cast(half8, row[D * D / 8 + kb]);
      c = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[kb], bh, c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[kb], bl, c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[kb], bh, c, 0, 0, 0);
    }
    int w = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint64_t m = __ballot(c[r] >= 0.f);
      const int key = 8 * (r >> 2) + (r & 3);
      w = octo_writelane((int)(uint32_t)m, key, w);
      w = octo_writelane((int)(uint32_t)(m >> 32), key + 4, w);
    }
    // (nb is not unrolled: a lane-indexed select keeps sw in registers)
#pragma unroll
    for (int k = 0; k < 8; ++k) sw[k] = nb == k ? (uint32_t)w : sw[k];
  }
}

template <int B, int KT, bool JR, bool QJL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(QJL || JR || KT == DT_F32 ? 2 : 3)))
void k_encode256(EncodeArgs a) {
  constexpr int D = 256;
  using C = Codec<D, B>;
  using S = Stage<128, KT>;
  constexpr int W = C::W;
  constexpr int TH = 43;                                   // triplets per lane
  constexpr int OFF = TH * C::BT;                          // first bit of triplet 43
  constexpr int WL = (OFF + 31) / 32 + 1;                  // local words per lane
  static_assert(C::T == 2 * TH, "d = 256 has 86 triplets");
  __shared__ __align__(16) unsigned char s_keys[4][S::NR * S::PITCH];
  __shared__ uint2 s_qx[kMaxLut + 2], s_qe[kMaxLut + 2], s_qr[kMaxLut + 2];
  __shared__ uint32_t s_w[4][32][W | 1];                   // odd pitch: conflict-free rows
  // unit directions and rho centroids (joint rounding, QJL residual)
  constexpr bool TABS = JR || QJL;
  __shared__ float4 s_dir[TABS ? C::NDIR : 1];
  __shared__ float s_rho[TABS ? C::LR : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t seq = blockIdx.y;
  copy_bucket_tables<256>(a.t, s_qx, s_qe, s_qr, threadIdx.x);
  if constexpr (TABS) {
    for (int i = threadIdx.x; i < C::NDIR; i += 256) s_dir[i] = a.t.dirtab[i];
    if (threadIdx.x < C::LR) s_rho[threadIdx.x] = a.t.rho_tab[threadIdx.x];
  }
  __syncthreads();
  const int64_t j0 = ((int64_t)blockIdx.x * 4 + wave) * 32;
  if (j0 >= a.n_new) return;  // (no block barrier past this point)
  const bool hi = lane >= 32;
  const int col = lane % S::CPR;
  // the sign masks of this lane's staging column in either half
  const uint4 m0 = chunk_sign_mask<D, KT>(a.t.sign_bits, col);
  const uint4 m1 = chunk_sign_mask<D, KT>(a.t.sign_bits, col + S::CPR);

  float v[128];
  {
    uint4 rowbits[S::CPR];
    {
      uint4 raw[S::NP][S::PER_LANE];
      load_half_rows<KT>(a, seq, j0, lane, raw);
      // stage the half rows (phases 0, 1: first halves; 2, 3: second halves)
      unsigned char* s_k = s_keys[wave];
      const int my_phase = lane / S::NR;
      const unsigned char* row = s_k + (lane % S::NR) * S::PITCH;
#pragma unroll
      for (int h = 0; h < S::NP; ++h) {
        const uint4 m = (h * S::NR) / 32 ? m1 : m0;
#pragma unroll
        for (int k = 0; k < S::PER_LANE; ++k) {
          uint4 u = raw[h][k];
          u.x ^= m.x; u.y ^= m.y; u.z ^= m.z; u.w ^= m.w;
          *(uint4*)(s_k + ((lane + 64 * k) / S::CPR) * S::PITCH + col * 16) = u;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (my_phase == h) {
#pragma unroll
          for (int c = 0; c < S::CPR; ++c) rowbits[c] = *(const uint4*)(row + c * 16);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
    if constexpr (KT == DT_F32) {
#pragma unroll
      for (int c = 0; c < S::CPR; ++c) cvt_chunk<KT>(rowbits[c], &v[c * S::VPC]);
    } else {
      // strides 1 and 2 on the matrix cores, straight from the packed 16-bit
      // elements (h4_apply)
      const uint2 h4 = h4_row<KT>(lane);
#pragma unroll
      for (int c = 0; c < S::CPR; ++c) {
        const wht4_t y0 = h4_apply<KT>(h4, rowbits[c].x, rowbits[c].y);
        const wht4_t y1 = h4_apply<KT>(h4, rowbits[c].z, rowbits[c].w);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[8 * c + k] = y0[k];
          v[8 * c + 4 + k] = y1[k];
        }
      }
    }
  }
  // the key's exponent scale (as encode_one_key: from the largest value after
  // the first two stages; fp32 keys: the raw values)
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 128; ++j) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[j]));
  amax = __builtin_fmaxf(amax, pair_xchg(amax, lane));
  int ex = 0;
  __builtin_frexpf(amax, &ex);
  const int sexp = (ex > 50 || ex < -50) && amax > 0.f ? ex : 0;
  if (__any(sexp != 0)) {
    const float scale = __builtin_ldexpf(1.0f, -sexp);
#pragma unroll
    for (int j = 0; j < 128; ++j) v[j] *= scale;
  }
  if constexpr (KT == DT_F32) wht_regs<128>(v);
  else wht_regs_from<128, 4>(v);
  // stride 128: y_j = a_j + a_{j+128} (first lane), a_j - a_{j+128} (second)
#pragma unroll
  for (int j = 0; j < 128; ++j) {
    const float p = pair_xchg(v[j], lane);
    v[j] = hi ? (p - v[j]) : (v[j] + p);
  }
  // element 128 for the first lane's last triplet; zero padding for the
  // second (the exchange runs on all lanes, outside any branch)
  const float x0 = pair_xchg(v[0], lane);
  const float ext = hi ? 0.f : x0;

  const float sx = a.t.qx.scale, bx = a.t.qx.bias;
  const float se = a.t.qe.scale, be = a.t.qe.bias;
  const float sr = a.t.qr2.scale, mr = (float)(a.t.qr2.nb - 1);
  auto trip = [&](int i, float& x, float& y, float& z) {
    // first lane: elements 3i .. 3i+2; second lane: 3i+1 .. 3i+3 (of its half)
    const float e0 = v[3 * i];
    const float e1 = v[3 * i + 1];
    const float e2 = 3 * i + 2 < 128 ? v[3 * i + 2] : ext;
    const float e3 = 3 * i + 3 < 128 ? v[3 * i + 3] : 0.f;
    x = hi ? e1 : e0;
    y = hi ? e2 : e1;
    z = hi ? e3 : e2;
  };
  uint32_t wl[WL];
#pragma unroll
  for (int w = 0; w < WL; ++w) wl[w] = 0u;
  float e[TH];
  float s1 = 0.f;
#pragma unroll
  for (int i = 0; i < TH; ++i) {
    float x, y, z;
    trip(i, x, y, z);
    e[i] = triplet_energy(x, y, z);
    s1 += e[i];
    pack_code<C::BT>(wl, i, xi_eta_code<C::BX>(x, y, z, s_qx, sx, bx, s_qe, se, be));
  }
  // serial energy over the pair: the second lane continues the first's sum
  float s2 = pair_xchg(s1, lane);
#pragma unroll
  for (int i = 0; i < TH; ++i) s2 += e[i];
  const float s2p = pair_xchg(s2, lane);
  const float tot = hi ? s2 : s2p;
  if constexpr (!JR) {
    const RhoQuant<C::LR> rq(a.t, tot);
#pragma unroll
    for (int i = 0; i < TH; ++i)
      pack_code<C::BT>(wl, i, rq.index(e[i], s_qr, sr, mr) << (C::BX + C::BE));
  } else {
    // joint rounding of every triplet of the unit key around its scalar
    // (xi, eta) indices
    const float inv_norm = tot > 0.f ? __builtin_amdgcn_rsqf(tot) : 0.f;
    uint32_t wj[WL];
#pragma unroll
    for (int w = 0; w < WL; ++w) wj[w] = 0u;
#pragma unroll
    for (int i = 0; i < TH; ++i) {
      float x, y, z;
      trip(i, x, y, z);
      x *= inv_norm;
      y *= inv_norm;
      z *= inv_norm;
      const uint32_t c0 = field_at<WL>(wl, i * C::BT, C::BX + C::BE);
      pack_code<C::BT>(wj, i, joint_code<C>(x, y, z, c0, s_dir, s_rho, s_qr, sr, mr));
    }
#pragma unroll
    for (int w = 0; w < WL; ++w) wl[w] = wj[w];
  }
  const float gamma = __builtin_ldexpf(__builtin_sqrtf(tot * (1.0f / D)), sexp);

  // QJL: the rotated unit-direction residual r' = u' - u'^ over the lane's
  // 128 dims, its norm over the pair, and the signs of S r'.  The first
  // lane's element j lies in its triplet j / 3 (component j % 3); the second
  // lane's element j >= 1 in its triplet (j - 1) / 3, and its element 0 (the
  // key's element 128) in the first lane's triplet 42.
  uint32_t sbits[QJL ? 8 : 1];
  float nu = 0.f;
  if constexpr (QJL) {
    const float inv_norm = tot > 0.f ? __builtin_amdgcn_rsqf(tot) : 0.f;
    const uint32_t c42 = pair_xchg(field_at<WL>(wl, 42 * C::BT, C::BT), lane);
    float cur[3], prev[3];
    {
      const float4 n = s_dir[c42 & C::DIR_MASK];
      const float rh = s_rho[c42 >> (C::BX + C::BE)];
      cur[0] = rh * n.x; cur[1] = rh * n.y; cur[2] = rh * n.z;
    }
    float nu2 = 0.f;
#pragma unroll
    for (int j = 0; j < 128; ++j) {
      const int c = j % 3;
      if (c == 0) {
#pragma unroll
        for (int k = 0; k < 3; ++k) prev[k] = cur[k];
        const uint32_t code = field_at<WL>(wl, (j / 3) * C::BT, C::BT);
        const float4 n = s_dir[code & C::DIR_MASK];
        const float rh = s_rho[code >> (C::BX + C::BE)];
        cur[0] = rh * n.x; cur[1] = rh * n.y; cur[2] = rh * n.z;
      }
      const float sub = hi ? (c == 0 ? prev[2] : cur[c - 1]) : cur[c];
      const float r = __builtin_fmaf(v[j], inv_norm, -sub);
      v[j] = r;
      nu2 = __builtin_fmaf(r, r, nu2);
    }
    nu2 += pair_xchg(nu2, lane);
    // formed here: left to itself the compiler may sink the sum past the
    // projection and keep all 128 residuals live through it
    asm volatile("" : "+v"(nu2));
    nu = __builtin_sqrtf(nu2);
#pragma unroll
    for (int k = 0; k < 8; ++k) sbits[k] = 0u;
    qjl_signs256(v, a.t.S16, lane, sbits);
  }

  // Assemble the key's word stream in LDS: the first lane's words hold bits
  // 0 .. OFF-1; the second lane's, shifted to bit OFF, are ORed in after.
  const int key = lane % 32;
  uint32_t* kw = s_w[wave][key];
  if (!hi) {
#pragma unroll
    for (int w = 0; w < (OFF + 31) / 32; ++w) kw[w] = wl[w];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (hi) {
    constexpr int W0 = OFF / 32, SH = OFF % 32;
#pragma unroll
    for (int k = 0; W0 + k < W; ++k) {
      const uint32_t lo = k > 0 ? wl[k - 1] : 0u;
      const uint32_t g = SH ? __builtin_amdgcn_alignbit(wl[k], lo, 32 - SH) : wl[k];
      if (k == 0) kw[W0] |= g;
      else kw[W0 + k] = g;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int64_t j = j0 + key;
  if (!hi && j < a.n_new) {
    uint32_t words[W];
#pragma unroll
    for (int w = 0; w < W; ++w) words[w] = kw[w];
    const int64_t pos = a.pos0 + j;
    TileWords<W>::store(a.packed + (seq * (a.cap / kTile) + (pos >> 6)) * W * kTile, (int)(pos & 63),
                        words);
    a.gamma[seq * a.cap + pos] = gamma;
    if constexpr (QJL) {
      TileWords<D / 32>::store(a.qjl_bits + (seq * (a.cap / kTile) + (pos >> 6)) * (D / 32) * kTile,
                               (int)(pos & 63), sbits);
      a.qjl_norm[seq * a.cap + pos] = __half_as_ushort(__float2half_rn(nu));
    }
  }
}

template <int B, int KT>
inline hipError_t launch_encode256_t(const EncodeArgs& a, bool joint, bool qjl, int64_t n_seq,
                                     hipStream_t s) {
  if (a.t.qx.nb > kMaxLut || a.t.qe.nb > kMaxLut || a.t.qr2.nb > kMaxLut) return hipErrorInvalidValue;
  if (qjl && (a.t.S16 == nullptr || a.qjl_bits == nullptr || a.qjl_norm == nullptr))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((a.n_new + 127) / 128), (unsigned)n_seq);
  if (qjl) {
    if (joint) hipLaunchKernelGGL((k_encode256<B, KT, true, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_encode256<B, KT, false, true>), grid, dim3(256), 0, s, a);
  } else {
    if (joint) hipLaunchKernelGGL((k_encode256<B, KT, true, false>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_encode256<B, KT, false, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <int D, int B, int KT, bool QJL, bool JR>
inline hipError_t launch_encode_t(const EncodeArgs& a, int64_t n_seq, hipStream_t s) {
  if (a.t.qx.nb > kMaxLut || a.t.qe.nb > kMaxLut || a.t.qr2.nb > kMaxLut) return hipErrorInvalidValue;
  constexpr int EW = enc_waves<QJL, B>();
  const int64_t per = (int64_t)EW * kTile;
  int64_t gx = (a.n_new + per - 1) / per;
  // With QJL each block first stages the matrix in LDS and then loops over
  // the tiles: a grid of about 512 blocks (one resident per compute unit).
  if (QJL) gx = std::min<int64_t>(gx, std::max<int64_t>(1, (512 + n_seq - 1) / n_seq));
  const dim3 grid((unsigned)gx, (unsigned)n_seq);
  hipLaunchKernelGGL((k_encode<D, B, KT, QJL, JR>), grid, dim3(64 * EW), 0, s, a);
  return hipGetLastError();
}

template <int D, int B, int KT>
inline hipError_t enc_q(bool qjl, bool joint, const EncodeArgs& a, int64_t n_seq, hipStream_t s) {
  if (joint)
    return qjl ? launch_encode_t<D, B, KT, true, true>(a, n_seq, s)
               : launch_encode_t<D, B, KT, false, true>(a, n_seq, s);
  return qjl ? launch_encode_t<D, B, KT, true, false>(a, n_seq, s)
             : launch_encode_t<D, B, KT, false, false>(a, n_seq, s);
}

template <int D, int B>
inline hipError_t enc_kt(int kdt, bool qjl, bool joint, const EncodeArgs& a, int64_t n_seq, hipStream_t s) {
  switch (kdt) {
    case DT_F32: return enc_q<D, B, DT_F32>(qjl, joint, a, n_seq, s);
    case DT_BF16: return enc_q<D, B, DT_BF16>(qjl, joint, a, n_seq, s);
    case DT_F16: return enc_q<D, B, DT_F16>(qjl, joint, a, n_seq, s);
  }
  return hipErrorInvalidValue;
}

// All encoder launches for bit budget B: d in {64, 128, 256}, the key dtypes,
// plain / QJL / joint rounding, and the one-key path for short appends.
// Each bit budget is instantiated in a translation unit of its own.
template <int B>
hipError_t launch_encode_b(int d, int kdt, bool qjl, bool joint, const EncodeArgs& a,
                           int64_t n_seq, hipStream_t s) {
  if (!qjl && !joint && a.n_new <= kEncodeOneMax) {
#define OCTO_ENC_ONE(DD)                                                          \
  switch (kdt) {                                                                \
    case DT_F32: return launch_encode_one_t<DD, B, DT_F32>(a, n_seq, s);        \
    case DT_BF16: return launch_encode_one_t<DD, B, DT_BF16>(a, n_seq, s);      \
    case DT_F16: return launch_encode_one_t<DD, B, DT_F16>(a, n_seq, s);        \
  }                                                                             \
  return hipErrorInvalidValue;
    if (d == 64) { OCTO_ENC_ONE(64) }
    if (d == 128) { OCTO_ENC_ONE(128) }
    if (d == 256) { OCTO_ENC_ONE(256) }
    return hipErrorInvalidValue;
  }
  // d = 256: two lanes per key (scalar or joint rounding, with or without QJL)
  if (d == 256) {
    switch (kdt) {
      case DT_F32: return launch_encode256_t<B, DT_F32>(a, joint, qjl, n_seq, s);
      case DT_BF16: return launch_encode256_t<B, DT_BF16>(a, joint, qjl, n_seq, s);
      case DT_F16: return launch_encode256_t<B, DT_F16>(a, joint, qjl, n_seq, s);
    }
    return hipErrorInvalidValue;
  }
#undef OCTO_ENC_ONE
  if (d == 64) return enc_kt<64, B>(kdt, qjl, joint, a, n_seq, s);
  if (d == 128) return enc_kt<128, B>(kdt, qjl, joint, a, n_seq, s);
  return hipErrorInvalidValue;
}

// LDS table copies of the encoder kernels (the octo_lds_copy records):
// the quantiser tables (loops bounded at run time by the table's nb + 2
// entries, which the launchers check against the kMaxLut + 2 LDS entries),
// and, where the variant holds them, the unit directions and rho centroids
// (QJL residual, joint rounding) and the f16 QJL matrix (SLDS: held in LDS;
// the d = 256 encoder reads it from global memory).
template <int D, int B, bool QJL, bool JR, int NTH, bool SLDS = QJL>
inline int enc_copy_recs(const char* kernel, LdsCopyRec* out, int n, int max) {
  using C = Codec<D, B>;
  for (int tab : {TAB_QX, TAB_QE, TAB_QR2})
    if (n < max) out[n++] = {kernel, D, B, QJL, tab, kMaxLut + 2, kMaxLut + 2, -1, -1, NTH, 1};
  if (QJL || JR) {
    using TC = TableCopy<C::NDIR, NTH>;
    if (n < max)
      out[n++] = {kernel, D, B, QJL, TAB_DIR, C::NDIR, TC::SLOTS, TC::ENTRIES, C::NDIR, NTH, TC::MASKED};
    if (n < max) out[n++] = {kernel, D, B, QJL, TAB_RHO, C::LR, C::LR, C::LR, C::LR, NTH, C::LR % NTH != 0};
  }
  if (SLDS) {
    using SL = SLds<D>;
    if (n < max)
      out[n++] = {kernel, D, B, QJL, TAB_S16, SL::BYTES / 16, SL::SLOT_END, SL::CHUNKS, SL::CHUNKS, NTH,
                  SL::CHUNKS % NTH != 0};
  }
  return n;
}

template <int B>
inline int enc_copy_recs_b(LdsCopyRec* out, int n, int max) {
#define OCTO_REC_D(D)                                                                            \
  n = enc_copy_recs<D, B, false, false, 64 * enc_waves<false, B>()>("k_encode", out, n, max);       \
  n = enc_copy_recs<D, B, false, true, 64 * enc_waves<false, B>()>("k_encode (joint)", out, n, max); \
  n = enc_copy_recs<D, B, true, false, 64 * enc_waves<true, B>()>("k_encode (qjl)", out, n, max);    \
  n = enc_copy_recs<D, B, true, true, 64 * enc_waves<true, B>()>("k_encode (qjl, joint)", out, n, max); \
  n = enc_copy_recs<D, B, false, false, 256>("k_encode_one", out, n, max);
  OCTO_REC_D(64)
  OCTO_REC_D(128)
#undef OCTO_REC_D
  n = enc_copy_recs<256, B, false, false, 256>("k_encode256", out, n, max);
  n = enc_copy_recs<256, B, false, true, 256>("k_encode256 (joint)", out, n, max);
  n = enc_copy_recs<256, B, true, false, 256, false>("k_encode256 (qjl)", out, n, max);
  n = enc_copy_recs<256, B, true, true, 256, false>("k_encode256 (qjl, joint)", out, n, max);
  n = enc_copy_recs<256, B, false, false, 256>("k_encode_one", out, n, max);
  return n;
}

}  // namespace octo

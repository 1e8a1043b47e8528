// Device helpers of the key encoders ([YL] 三元组分解, 八面体折叠): the
// per-triplet quantisers, the code packing, and the one-wavefront encode of
// a single key that both the append encoder and the attention kernel's
// append step use.  Floating-point expressions here are evaluated exactly as
// written (fma only where a builtin says so), so every encoder rounds the same
// operations the same way.
#pragma once

#include "octo_device.hpp"

namespace octo {

// #{k : x > m_k} from a centred one-midpoint-per-bucket table in LDS (see
// Bucket1), for x in [-1, 1] up to rounding: the fma rounds the bucket
// position to an integer in [0, nb] inside its own mantissa, so the bucket
// is its bits less kBucketMagicBits (one address add, no conversion).
__device__ __forceinline__ uint32_t quant1(float x, const uint2* t, float scale, float bias) {
  const uint2 e = t[__float_as_uint(__builtin_fmaf(x, scale, bias)) - kBucketMagicBits];
  return e.x + (x > __uint_as_float(e.y) ? 1u : 0u);
}

// The same for x >= 0 of unbounded range (rho^2), clamped to the last bucket.
__device__ __forceinline__ uint32_t quant1_clamp(float x, const uint2* t, float scale, float nbm1) {
  const uint2 e = t[(uint32_t)__builtin_fminf(x * scale, nbm1)];
  return e.x + (x > __uint_as_float(e.y) ? 1u : 0u);
}

// rho index of a triplet from its energy e = |t_i|^2 and the key's total
// energy tot = |y|^2: rho_i^2 = e / tot against the squared midpoints, i.e.
// #{k : e > m_k^2 tot}.  With at most 4 rho levels (b <= 3) the thresholds
// m_k^2 tot are formed once per key and each triplet takes one compare per
// midpoint; with more levels the index comes from the squared-midpoint
// bucket table on e / tot.  Every encoder takes its rho index through
// RhoQuant, so all of them round the same way.
template <int LR>
struct RhoQuant {
  static constexpr bool kDirect = LR <= 4;
  float thr[kDirect && LR > 1 ? LR - 1 : 1];
  float inv_tot;
  __device__ __forceinline__ RhoQuant(const DevTables& t, float tot) {
    if constexpr (kDirect) {
#pragma unroll
      for (int k = 0; k < LR - 1; ++k) thr[k] = t.rho_mid2[k] * tot;
      inv_tot = 0.f;
    } else {
      inv_tot = tot > 0.f ? __builtin_amdgcn_rcpf(tot) : 0.f;
    }
  }
  __device__ __forceinline__ uint32_t index(float e, const uint2* tqr, float scale, float nbm1) const {
    if constexpr (kDirect) {
      uint32_t i = 0u;
#pragma unroll
      for (int k = 0; k < LR - 1; ++k) i += e > thr[k] ? 1u : 0u;
      return i;
    } else {
      return quant1_clamp(e * inv_tot, tqr, scale, nbm1);
    }
  }
};

// Triplet i of the rotated key, zero padded past D.
template <int D>
__device__ __forceinline__ void triplet_of(const float (&v)[D], int i, float& x, float& y, float& z) {
  x = v[3 * i];
  y = (3 * i + 1 < D) ? v[3 * i + 1] : 0.f;
  z = (3 * i + 2 < D) ? v[3 * i + 2] : 0.f;
}

__device__ __forceinline__ float triplet_energy(float x, float y, float z) {
#pragma clang fp contract(off)
  return __builtin_fmaf(z, z, __builtin_fmaf(y, y, x * x));
}

// The octahedral (xi, eta) indices of a triplet, i_xi | i_eta << BX
// ([YL] 八面体折叠).  p = (x, y)/l1; in the lower hemisphere (z < 0) the fold
// (1 - |p_y|) sgn p_x equals p_x + sgn(p_x) |z|/l1 (likewise for y), with
// sgn(0) = +1 (the sign bit is copied; -0 only occurs for an all-zero
// triplet, where |z| = 0).  A zero triplet maps to (0, 0), i.e. n = (0,0,1).
template <int BX>
__device__ __forceinline__ uint32_t xi_eta_code(float x, float y, float z, const uint2* tx,
                                                float sx, float bx, const uint2* te, float se,
                                                float be) {
#pragma clang fp contract(off)
  const float l1 = __builtin_fabsf(x) + __builtin_fabsf(y) + __builtin_fabsf(z);
  const float il = __builtin_amdgcn_rcpf(__builtin_fmaxf(l1, 1e-37f));
  const float tz = __builtin_fmaxf(-z, 0.0f);
  const float xi = (x + __builtin_copysignf(tz, x)) * il;
  const float eta = (y + __builtin_copysignf(tz, y)) * il;
  return quant1(xi, tx, sx, bx) | (quant1(eta, te, se, be) << BX);
}

// OR a code into bits [i BT, (i + 1) BT) of the key's LSB-first word stream.
template <int BT, int W>
__device__ __forceinline__ void pack_code(uint32_t (&words)[W], int i, uint32_t code) {
  const int pos = i * BT, wi = pos >> 5, off = pos & 31;
  words[wi] |= code << off;
  if (off + BT > 32) words[wi + 1] |= code >> (32 - off);
}

// Store word w of the key at (seq, pos) into the tile's word-group layout.
template <int W>
__device__ __forceinline__ void store_key_word(uint32_t* packed, int64_t cap, int64_t seq,
                                               int64_t pos, int w, uint32_t val) {
  constexpr int NG = W / 4, R = W % 4;
  const int g = w / 4;
  const int width = g < NG ? 4 : R;
  uint32_t* tile = packed + (seq * (cap / kTile) + (pos >> 6)) * W * kTile;
  tile[256 * g + (int)(pos & 63) * width + (w & 3)] = val;
}

// Encode one key with one wavefront: the WHT butterflies run across lanes by
// shuffles (as in the query rotation), one triplet per lane.  Every value
// goes through the same fp32 operations in the same order as in the bulk
// encoders (for 16-bit keys the first two stages by the same H_4 MFMA on the
// sign-flipped words, the serial energy sum over triplets, the same
// quantisers), so all of them write identical words and gamma.
//   keyrow: the key's d elements (dtype KT); tqx/tqe/tqr: the quantiser
//   tables (LDS or global); sv (3T floats), se (T floats), sw (W words):
//   wave-private LDS scratch.  On return sw holds the packed words (visible
//   to the whole wave); the key's gamma is returned (every lane).
template <int D, int B, int KT>
__device__ __forceinline__ float encode_one_key(const void* keyrow, const DevTables& t,
                                                const uint2* tqx, const uint2* tqe,
                                                const uint2* tqr, int lane, float* sv, float* se,
                                                uint32_t* sw) {
#pragma clang fp contract(off)
  using C = Codec<D, B>;
  constexpr int T = C::T, W = C::W, NV = D / 64;
  int sexp = 0;
  if constexpr (KT == DT_F32) {
    // lane l holds elements l + 64 r of the sign-flipped key
    float x[NV];
    const float* row = (const float*)keyrow;
#pragma unroll
    for (int r = 0; r < NV; ++r) {
      const int e = lane + 64 * r;
      const uint32_t sb = (t.sign_bits[e >> 5] >> (e & 31)) & 1u;
      x[r] = __uint_as_float(__float_as_uint(row[e]) ^ (sb << 31));
    }
    float amax = 0.f;
#pragma unroll
    for (int r = 0; r < NV; ++r) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[r]));
    amax = wave_max(amax);
    int ex = 0;
    __builtin_frexpf(amax, &ex);
    const int sexp0 = (ex > 50 || ex < -50) && amax > 0.f ? ex : 0;
    if (sexp0 != 0) {
      const float scale = __builtin_ldexpf(1.0f, -sexp0);
#pragma unroll
      for (int r = 0; r < NV; ++r) x[r] *= scale;
    }
    sexp = sexp0;
    // butterflies of stride 1 .. 32 across lanes, then 64, 128, ... between a
    // lane's values
#pragma unroll
    for (int h = 1; h < 64 && h < D; h <<= 1) {
#pragma unroll
      for (int r = 0; r < NV; ++r) {
        const float o = __shfl_xor(x[r], h, 64);
        x[r] = (lane & h) ? (o - x[r]) : (x[r] + o);
      }
    }
#pragma unroll
    for (int hr = 1; hr < NV; hr <<= 1) {
#pragma unroll
      for (int r = 0; r < NV; ++r) {
        if (r & hr) continue;
        const float a0 = x[r], a1 = x[r + hr];
        x[r] = a0 + a1;
        x[r + hr] = a0 - a1;
      }
    }
#pragma unroll
    for (int r = 0; r < NV; ++r) sv[lane + 64 * r] = x[r];
  } else {
    // lane l takes the 4-element group g = l mod (D / 4) (lanes past D / 4
    // repeat the first ones): strides 1 and 2 on the matrix cores from the
    // two sign-flipped words (h4_apply, as the bulk encoders), then strides
    // 4, 8, ... as lane pairs g, g ^ (stride / 4)
    constexpr int NG = D / 4;
    static_assert(NG <= 64 && (NG & (NG - 1)) == 0, "one 4-element group per lane");
    const int g = lane & (NG - 1);
    const uint32_t* row = (const uint32_t*)keyrow;
    uint32_t w[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int m = 2 * g + k;   // elements 2m, 2m + 1
      const uint32_t s0 = (t.sign_bits[(2 * m) >> 5] >> ((2 * m) & 31)) & 1u;
      const uint32_t s1 = (t.sign_bits[(2 * m + 1) >> 5] >> ((2 * m + 1) & 31)) & 1u;
      w[k] = row[m] ^ ((s0 << 15) | (s1 << 31));
    }
    const wht4_t y = h4_apply<KT>(h4_row<KT>(lane), w[0], w[1]);
    float x[4] = {y[0], y[1], y[2], y[3]};
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
    amax = wave_max(amax);
    int ex = 0;
    __builtin_frexpf(amax, &ex);
    const int sexp0 = (ex > 50 || ex < -50) && amax > 0.f ? ex : 0;
    if (sexp0 != 0) {
      const float scale = __builtin_ldexpf(1.0f, -sexp0);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] *= scale;
    }
    sexp = sexp0;
#pragma unroll
    for (int h = 1; h < NG; h <<= 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float o = __shfl_xor(x[i], h, 64);
        x[i] = (g & h) ? (o - x[i]) : (x[i] + o);
      }
    }
    if (lane < NG) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[4 * g + i] = x[i];
    }
  }
  if (lane < 3 * T - D) sv[D + lane] = 0.f;
  for (int w = lane; w < W; w += 64) sw[w] = 0u;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // one triplet per lane (triplets lane + 64 m: two per lane up to d = 384)
  constexpr int NT = (T + 63) / 64;
  float e[NT];
  uint32_t xe[NT];
#pragma unroll
  for (int m = 0; m < NT; ++m) {
    const int i0 = lane + 64 * m;
    const int i = i0 < T ? i0 : T - 1;
    const float tx = sv[3 * i], ty = sv[3 * i + 1], tz = sv[3 * i + 2];
    e[m] = triplet_energy(tx, ty, tz);
    xe[m] = xi_eta_code<C::BX>(tx, ty, tz, tqx, t.qx.scale, t.qx.bias, tqe, t.qe.scale, t.qe.bias);
    if (i0 < T) se[i0] = e[m];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // the energy summed serially in triplet order, as the bulk encoder does
  float tot = 0.f;
  for (int i2 = 0; i2 < T; ++i2) tot += se[i2];
  const float gamma = __builtin_ldexpf(__builtin_sqrtf(tot * (1.0f / D)), sexp);
  const RhoQuant<C::LR> rq(t, tot);
#pragma unroll
  for (int m = 0; m < NT; ++m) {
    const int i0 = lane + 64 * m;
    const uint32_t rc = rq.index(e[m], tqr, t.qr2.scale, (float)(t.qr2.nb - 1));
    const uint32_t code = xe[m] | (rc << (C::BX + C::BE));
    if (i0 < T) {
      const int p = i0 * C::BT, wi = p >> 5, off = p & 31;
      atomicOr(&sw[wi], code << off);
      if (off + C::BT > 32) atomicOr(&sw[wi + 1], code >> (32 - off));
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  return gamma;
}

}  // namespace octo

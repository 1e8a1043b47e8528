// OCTOPUS online key encoder for gfx950.
//
// One wavefront encodes a tile of 64 keys, one key per lane, entirely in
// registers ([YL] 三元组分解, steps 1-4):
//   gamma = |k| (fp32, stored), y = H (s .* k) by in-register butterflies
//   ([YL] 旋转魔法 / 工程实现), triplets t_i of the zero-padded y, rho_i^2 =
//   |t_i|^2/|y|^2, octahedral (xi, eta) of t_i ([YL] 八面体折叠), Lloyd-Max
//   nearest-centroid indices from bucketed LDS tables, bit-pack, store.
// The key tile is read with coalesced 16-byte loads and handed to the lanes
// through LDS in two halves (small LDS footprint, several waves per SIMD);
// packed words are stored in the tile's word-group layout (16-byte stores,
// 1 KiB contiguous per store instruction).  With QJL the same lane also forms the rotated residual
// r' = u' - u'^, its fp16 norm and the signs of S r' ([YL] 可选的残差修正).
#include "octo_device.hpp"

namespace octo {

// Stage the key rows [r0, r0 + NR) of the wave's 64-key tile into LDS with
// coalesced 16-byte loads (consecutive lanes read consecutive chunks).  The
// WHT sign flips are applied here, on the raw chunk bits: every lane always
// handles the same chunk column, so one 16-byte mask per lane does it.
template <int D, int KT>
struct Stage {
  static constexpr int ES = DtSize<KT>::v;
  static constexpr int ROWB = D * ES;       // bytes per key row
  static constexpr int CPR = ROWB / 16;     // 16-byte chunks per row
  static constexpr int PITCH = ROWB + 16;   // padded pitch: conflict-free row reads
  static constexpr int VPC = 16 / ES;       // values per chunk
  static constexpr int NR = 16;             // rows staged per phase
  static constexpr int NP = kTile / NR;     // phases
  static constexpr int PER_LANE = NR * CPR / 64;
};

// Sign mask of the chunk a lane stages: sign bit of every element whose WHT
// sign is -1 (bit 15 of a 16-bit element, bit 31 of an fp32 one).
template <int D, int KT>
__device__ __forceinline__ uint4 chunk_sign_mask(const uint32_t (&sign_bits)[4], int col) {
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

// Bring the lane's own key row (already sign-flipped, raw bits) into
// registers: coalesced 16-byte global loads of the whole tile (rows past
// n_new re-read the last key, so the loads carry no conditions), then NP
// rounds through the wave's LDS buffer of NR rows.
template <int D, int KT>
__device__ __forceinline__ void gather_row(const EncodeArgs& a, int64_t seq, int64_t j0, int lane,
                                           unsigned char* s_keys, const uint4& smask,
                                           uint4 (&rowbits)[Stage<D, KT>::CPR]) {
  using S = Stage<D, KT>;
  const unsigned char* kbase = (const unsigned char*)a.keys + (seq * a.seq_stride) * S::ES;
  const int col = lane % S::CPR;
  uint4 raw[S::NP][S::PER_LANE];
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

// #{k : x > m_k} from a one-midpoint-per-bucket table in LDS (see Bucket1),
// for x in [-1, 1] up to rounding: the bucket position is then above -1, so
// truncation toward zero gives bucket 0 at the bottom, and the guard entries
// cover the top.
__device__ __forceinline__ uint32_t quant1(float x, const uint2* t, float scale, float bias) {
  const uint2 e = t[(int)__builtin_fmaf(x, scale, bias)];
  return e.x + (x > __uint_as_float(e.y) ? 1u : 0u);
}

// The same for x >= 0 of unbounded range (rho^2), clamped to the last bucket.
__device__ __forceinline__ uint32_t quant1_clamp(float x, const uint2* t, float scale, float nbm1) {
  const uint2 e = t[(uint32_t)__builtin_fminf(x * scale, nbm1)];
  return e.x + (x > __uint_as_float(e.y) ? 1u : 0u);
}

constexpr int kEncWaves = 4;  // waves (64-key tiles) per encoder block

template <int D, int B, int KT, bool QJL>
__global__ __launch_bounds__(64 * kEncWaves) void k_encode(EncodeArgs a) {
  using C = Codec<D, B>;
  using S = Stage<D, KT>;
  constexpr int T = C::T, W = C::W;

  __shared__ __align__(16) unsigned char s_keys[kEncWaves][S::NR * S::PITCH];
  __shared__ uint2 s_qx[kMaxLut + 2], s_qe[kMaxLut + 2], s_qr[kMaxLut + 2];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t seq = blockIdx.y;
  const int64_t j0 = ((int64_t)blockIdx.x * kEncWaves + wave) * kTile;

  // the block's waves share the quantiser tables
  for (int i = threadIdx.x; i < a.t.qx.nb + 2; i += 64 * kEncWaves) s_qx[i] = a.t.qx.t[i];
  for (int i = threadIdx.x; i < a.t.qe.nb + 2; i += 64 * kEncWaves) s_qe[i] = a.t.qe.t[i];
  for (int i = threadIdx.x; i < a.t.qr2.nb + 2; i += 64 * kEncWaves) s_qr[i] = a.t.qr2.t[i];
  __syncthreads();
  if (j0 >= a.n_new) return;
  const uint4 smask = chunk_sign_mask<D, KT>(a.t.sign_bits, lane % S::CPR);
  float v[D];
  {
    uint4 rowbits[S::CPR];
    gather_row<D, KT>(a, seq, j0, lane, s_keys[wave], smask, rowbits);
    if constexpr (KT == DT_F32) {
#pragma unroll
      for (int c = 0; c < S::CPR; ++c) cvt_chunk<KT>(rowbits[c], &v[c * S::VPC]);
    } else {
      // stride-1 butterflies straight from the packed 16-bit pairs
#pragma unroll
      for (int c = 0; c < S::CPR; ++c) {
        const uint32_t wd[4] = {rowbits[c].x, rowbits[c].y, rowbits[c].z, rowbits[c].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) stage1_pair<KT>(wd[k], v[8 * c + 2 * k], v[8 * c + 2 * k + 1]);
      }
    }
  }
  // Keys with entries far from 1 in magnitude are scaled by an exact power of
  // two (changes no ratio) so that no triplet energy under- or overflows.
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
  if constexpr (KT == DT_F32) wht_regs<D>(v);
  else wht_regs_from<D, 2>(v);

  const float sx = a.t.qx.scale, bx = a.t.qx.bias;
  const float se = a.t.qe.scale, be = a.t.qe.bias;
  uint32_t words[W];
#pragma unroll
  for (int w = 0; w < W; ++w) words[w] = 0u;
  uint32_t codes[QJL ? T : 1];
  float e[T];
  float tot = 0.f;

  // Pass 1: triplet energies and the octahedral (xi, eta) indices, packed
  // into place.  p = (x, y)/l1; in the lower hemisphere (z < 0) the fold
  // (1 - |p_y|) sgn p_x equals p_x + sgn(p_x) |z|/l1 (likewise for y), with
  // sgn(0) = +1 (the sign bit is copied; -0 only occurs for an all-zero
  // triplet, where |z| = 0).  A zero triplet maps to (0, 0), i.e. n = (0,0,1).
#pragma unroll
  for (int i = 0; i < T; ++i) {
    const float x = v[3 * i];
    const float y = (3 * i + 1 < D) ? v[3 * i + 1] : 0.f;
    const float z = (3 * i + 2 < D) ? v[3 * i + 2] : 0.f;
    e[i] = __builtin_fmaf(z, z, __builtin_fmaf(y, y, x * x));
    tot += e[i];
    const float l1 = __builtin_fabsf(x) + __builtin_fabsf(y) + __builtin_fabsf(z);
    const float il = __builtin_amdgcn_rcpf(__builtin_fmaxf(l1, 1e-37f));
    const float tz = __builtin_fmaxf(-z, 0.0f);
    const float xi = (x + __builtin_copysignf(tz, x)) * il;
    const float eta = (y + __builtin_copysignf(tz, y)) * il;
    const uint32_t code = quant1(xi, s_qx, sx, bx) | (quant1(eta, s_qe, se, be) << C::BX);
    if constexpr (QJL) codes[i] = code;
    const int pos = i * C::BT, wi = pos >> 5, off = pos & 31;
    words[wi] |= code << off;
    if (off + C::BT > 32) words[wi + 1] |= code >> (32 - off);
  }
  const float gamma = __builtin_ldexpf(__builtin_sqrtf(tot * (1.0f / D)), sexp);
  const float inv_tot = tot > 0.f ? __builtin_amdgcn_rcpf(tot) : 0.f;

  // Pass 2: rho index from rho_i^2 = e_i / |y|^2 against the squared midpoints.
  // (the rho^2 table starts at 0: bias 0)
  const float sr = a.t.qr2.scale, mr = (float)(a.t.qr2.nb - 1);
#pragma unroll
  for (int i = 0; i < T; ++i) {
    const uint32_t code = quant1_clamp(e[i] * inv_tot, s_qr, sr, mr) << (C::BX + C::BE);
    if constexpr (QJL) codes[i] |= code;
    const int pos = i * C::BT, wi = pos >> 5, off = pos & 31;
    words[wi] |= code << off;
    if (off + C::BT > 32) words[wi + 1] |= code >> (32 - off);
  }

  const int64_t j = j0 + lane;
  const bool valid = j < a.n_new;
  const int64_t pos = a.pos0 + j;
  const int64_t tiles = a.cap / kTile;
  if (valid) {
    TileWords<W>::store(a.packed + (seq * tiles + (pos >> 6)) * W * kTile, (int)(pos & 63), words);
    a.gamma[seq * a.cap + pos] = gamma;
  }

  if constexpr (QJL) {
    if (a.qjl_bits == nullptr) return;
    // Rotated unit-direction residual r' = u' - u'^ over the D real coordinates.
    const float inv_norm = tot > 0.f ? __builtin_amdgcn_rsqf(tot) : 0.f;
    float nu2 = 0.f;
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const float4 n = a.t.dirtab[codes[i] & C::DIR_MASK];
      const float rh = a.t.rho_tab[codes[i] >> (C::BX + C::BE)];
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
    const float nu = __builtin_sqrtf(nu2);
    uint32_t sbits[D / 32];
#pragma unroll
    for (int w = 0; w < D / 32; ++w) sbits[w] = 0u;
    const float* __restrict__ Sm = a.t.S;
#pragma unroll 1
    for (int r = 0; r < D; r += 32) {
      uint32_t m = 0u;
#pragma unroll 2
      for (int rr = 0; rr < 32; ++rr) {
        const float* __restrict__ srow = Sm + (int64_t)(r + rr) * D;
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < D; ++k) acc = __builtin_fmaf(srow[k], v[k], acc);
        m |= (acc >= 0.f ? 1u : 0u) << rr;
      }
#pragma unroll
      for (int w = 0; w < D / 32; ++w)
        if (w == r / 32) sbits[w] = m;
    }
    if (valid) {
      TileWords<D / 32>::store(a.qjl_bits + (seq * tiles + (pos >> 6)) * (D / 32) * kTile,
                               (int)(pos & 63), sbits);
      a.qjl_norm[seq * a.cap + pos] = __half_as_ushort(__float2half_rn(nu));
    }
  }
}

template <int D, int B, int KT, bool QJL>
static hipError_t launch_encode_t(const EncodeArgs& a, int64_t n_seq, hipStream_t s) {
  if (a.t.qx.nb > kMaxLut || a.t.qe.nb > kMaxLut || a.t.qr2.nb > kMaxLut) return hipErrorInvalidValue;
  const int64_t per = (int64_t)kEncWaves * kTile;
  const dim3 grid((unsigned)((a.n_new + per - 1) / per), (unsigned)n_seq);
  hipLaunchKernelGGL((k_encode<D, B, KT, QJL>), grid, dim3(64 * kEncWaves), 0, s, a);
  return hipGetLastError();
}

template <int D, int B, int KT>
static hipError_t enc_q(bool qjl, const EncodeArgs& a, int64_t n_seq, hipStream_t s) {
  return qjl ? launch_encode_t<D, B, KT, true>(a, n_seq, s)
             : launch_encode_t<D, B, KT, false>(a, n_seq, s);
}

template <int D, int B>
static hipError_t enc_kt(int kdt, bool qjl, const EncodeArgs& a, int64_t n_seq, hipStream_t s) {
  switch (kdt) {
    case DT_F32: return enc_q<D, B, DT_F32>(qjl, a, n_seq, s);
    case DT_BF16: return enc_q<D, B, DT_BF16>(qjl, a, n_seq, s);
    case DT_F16: return enc_q<D, B, DT_F16>(qjl, a, n_seq, s);
  }
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t enc_b(int b, int kdt, bool qjl, const EncodeArgs& a, int64_t n_seq, hipStream_t s) {
  switch (b) {
    case 2: return enc_kt<D, 2>(kdt, qjl, a, n_seq, s);
    case 3: return enc_kt<D, 3>(kdt, qjl, a, n_seq, s);
    case 4: return enc_kt<D, 4>(kdt, qjl, a, n_seq, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_encode(int d, int b, int kdt, bool qjl, const EncodeArgs& a, int64_t n_seq,
                         hipStream_t s) {
  if (a.n_new <= 0 || n_seq <= 0) return hipSuccess;
  switch (d) {
    case 64: return enc_b<64>(b, kdt, qjl, a, n_seq, s);
    case 128: return enc_b<128>(b, kdt, qjl, a, n_seq, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace octo

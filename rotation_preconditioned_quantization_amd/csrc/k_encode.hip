// OCTOPUS online key encoder for gfx950.
//
// One wavefront encodes a tile of 64 keys, one key per lane, entirely in
// registers ([YL] 三元组分解, steps 1-4):
//   gamma = |k| (fp32, stored), y = H (s .* k) by in-register butterflies
//   ([YL] 旋转魔法 / 工程实现), triplets t_i of the zero-padded y, rho_i^2 =
//   |t_i|^2/|y|^2, octahedral (xi, eta) of t_i ([YL] 八面体折叠), Lloyd-Max
//   nearest-centroid indices from bucketed LDS tables, bit-pack, store.
// The key tile is staged through LDS so that HBM reads are coalesced 16-byte
// loads; packed words are stored word-major per tile (256 contiguous bytes per
// store instruction).  With QJL the same lane also forms the rotated residual
// r' = u' - u'^, its fp16 norm and the signs of S r' ([YL] 可选的残差修正).
#include "octo_device.hpp"

namespace octo {

// y = H (s .* k * 2^-sexp) for the lane's staged key row, and the energies
// of its zero-padded triplets.
template <int D, int KT>
__device__ __forceinline__ void rotate_energy(const unsigned char* row, int sexp,
                                              const uint32_t (&sign_bits)[4], float (&v)[D],
                                              float (&e)[(D + 2) / 3], float& tot) {
  constexpr int T = (D + 2) / 3;
  constexpr int VPC = 16 / DtSize<KT>::v;
#pragma unroll
  for (int c = 0; c < D / VPC; ++c) {
    const uint4 w = *(const uint4*)(row + c * 16);
    cvt_chunk<KT>(w, &v[c * VPC]);
  }
  if (sexp != 0) {
    const float scale = __builtin_ldexpf(1.0f, -sexp);
#pragma unroll
    for (int j = 0; j < D; ++j) v[j] *= scale;
  }
  apply_signs<D>(v, sign_bits);
  wht_regs<D>(v);
  tot = 0.f;
#pragma unroll
  for (int i = 0; i < T; ++i) {
    const float x = v[3 * i];
    const float y = (3 * i + 1 < D) ? v[3 * i + 1] : 0.f;
    const float z = (3 * i + 2 < D) ? v[3 * i + 2] : 0.f;
    e[i] = __builtin_fmaf(z, z, __builtin_fmaf(y, y, x * x));
    tot += e[i];
  }
}

template <int D, int B, int KT, bool QJL>
__global__ __launch_bounds__(64) void k_encode(EncodeArgs a) {
  using C = Codec<D, B>;
  constexpr int T = C::T, W = C::W;
  constexpr int ES = DtSize<KT>::v;
  constexpr int ROWB = D * ES;            // bytes per key row
  constexpr int CPR = ROWB / 16;          // 16-byte chunks per row
  constexpr int PITCH = ROWB + 16;        // padded LDS row pitch: conflict-free row reads
  constexpr int VPC = 16 / ES;            // values per chunk

  __shared__ __align__(16) unsigned char s_keys[64 * PITCH];
  __shared__ float s_midx[C::LX + 1], s_mide[C::LE + 1], s_midr[C::LR + 1];
  __shared__ uint8_t s_lutx[kMaxLut], s_lute[kMaxLut], s_lutr[kMaxLut];

  const int lane = threadIdx.x;
  const int64_t seq = blockIdx.y;
  const int64_t j0 = (int64_t)blockIdx.x * kTile;

  for (int i = lane; i < a.t.qx.nb; i += 64) s_lutx[i] = a.t.qx.lut[i];
  for (int i = lane; i < a.t.qe.nb; i += 64) s_lute[i] = a.t.qe.lut[i];
  for (int i = lane; i < a.t.qr2.nb; i += 64) s_lutr[i] = a.t.qr2.lut[i];
  if (lane < C::LX + 1) s_midx[lane] = a.t.qx.mid[lane];
  if (lane < C::LE + 1) s_mide[lane] = a.t.qe.mid[lane];
  if (lane < C::LR + 1) s_midr[lane] = a.t.qr2.mid[lane];

  // Stage the 64 key rows: consecutive lanes read consecutive 16-byte chunks.
  const unsigned char* kbase =
      (const unsigned char*)a.keys + (seq * a.seq_stride) * ES;
#pragma unroll 4
  for (int f = lane; f < 64 * CPR; f += 64) {
    const int r = f / CPR, c = f % CPR;
    const int64_t j = j0 + r;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (j < a.n_new) val = *(const uint4*)(kbase + (j * a.key_stride) * ES + c * 16);
    *(uint4*)(s_keys + r * PITCH + c * 16) = val;
  }
  __syncthreads();

  // Rotate and take triplet energies; |y|^2 = D |k|^2.  Keys whose energy
  // would under- or overflow fp32 (norms far from 1, rare) are redone scaled
  // by an exact power of two, which changes no ratio.
  float v[D];
  float e[T];
  float tot = 0.f;
  int sexp = 0;
  const unsigned char* row = s_keys + lane * PITCH;
  rotate_energy<D, KT>(row, 0, a.t.sign_bits, v, e, tot);
  const bool redo = !(tot >= 0x1p-100f && tot <= 0x1p+100f);
  if (__any(redo)) {
    asm volatile("" ::: "memory");  // reload the row from LDS; keep no raw copy live
    if (redo) {
      float amax = 0.f;
#pragma unroll
      for (int c = 0; c < CPR; ++c) {
        float f[VPC];
        cvt_chunk<KT>(*(const uint4*)(row + c * 16), f);
#pragma unroll
        for (int k = 0; k < VPC; ++k) amax = __builtin_fmaxf(amax, __builtin_fabsf(f[k]));
      }
      int ex = 0;
      __builtin_frexpf(amax, &ex);   // amax = m * 2^ex, m in [0.5, 1)
      sexp = amax > 0.f ? ex : 0;
      rotate_energy<D, KT>(row, sexp, a.t.sign_bits, v, e, tot);
    }
  }
  const float gamma = __builtin_ldexpf(__builtin_sqrtf(tot * (1.0f / D)), sexp);
  const float inv_tot = tot > 0.f ? __builtin_amdgcn_rcpf(tot) : 0.f;

  const float lox = a.t.qx.lo, iwx = a.t.qx.inv_w, nbx = (float)(a.t.qx.nb - 1);
  const float loe = a.t.qe.lo, iwe = a.t.qe.inv_w, nbe = (float)(a.t.qe.nb - 1);
  const float lor = a.t.qr2.lo, iwr = a.t.qr2.inv_w, nbr = (float)(a.t.qr2.nb - 1);

  uint32_t words[W];
#pragma unroll
  for (int w = 0; w < W; ++w) words[w] = 0u;
  uint32_t codes[QJL ? T : 1];

  // Pass 2: quantise and pack.
#pragma unroll
  for (int i = 0; i < T; ++i) {
    const float x = v[3 * i];
    const float y = (3 * i + 1 < D) ? v[3 * i + 1] : 0.f;
    const float z = (3 * i + 2 < D) ? v[3 * i + 2] : 0.f;
    const int ir = quant_lookup(e[i] * inv_tot, s_lutr, s_midr, lor, iwr, nbr);
    const float l1 = __builtin_fabsf(x) + __builtin_fabsf(y) + __builtin_fabsf(z);
    const float il = l1 > 0.f ? __builtin_amdgcn_rcpf(l1) : 0.f;
    const float px = x * il, py = y * il;
    float xi = px, eta = py;
    if (z < 0.f) {  // fold the lower hemisphere onto the square's corners; sgn(0) = +1
      const float fx = 1.0f - __builtin_fabsf(py);
      const float fy = 1.0f - __builtin_fabsf(px);
      xi = px >= 0.f ? fx : -fx;
      eta = py >= 0.f ? fy : -fy;
    }
    const int ix = quant_lookup(xi, s_lutx, s_midx, lox, iwx, nbx);
    const int ie = quant_lookup(eta, s_lute, s_mide, loe, iwe, nbe);
    const uint32_t code = (uint32_t)ix | ((uint32_t)ie << C::BX) | ((uint32_t)ir << (C::BX + C::BE));
    if constexpr (QJL) codes[i] = code;
    const int pos = i * C::BT, wi = pos >> 5, off = pos & 31;
    words[wi] |= code << off;
    if (off + C::BT > 32) words[wi + 1] |= code >> (32 - off);
  }

  const int64_t j = j0 + lane;
  const bool valid = j < a.n_new;
  const int64_t pos = a.pos0 + j;
  const int64_t tiles = a.cap / kTile;
  if (valid) {
    uint32_t* dst = a.packed + ((seq * tiles + (pos >> 6)) * W) * kTile + (pos & 63);
#pragma unroll
    for (int w = 0; w < W; ++w) dst[w * kTile] = words[w];
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
    const float* __restrict__ S = a.t.S;
#pragma unroll 1
    for (int r = 0; r < D; r += 32) {
      uint32_t m = 0u;
#pragma unroll 2
      for (int rr = 0; rr < 32; ++rr) {
        const float* __restrict__ row = S + (int64_t)(r + rr) * D;
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < D; ++k) acc = __builtin_fmaf(row[k], v[k], acc);
        m |= (acc >= 0.f ? 1u : 0u) << rr;
      }
#pragma unroll
      for (int w = 0; w < D / 32; ++w)
        if (w == r / 32) sbits[w] = m;
    }
    if (valid) {
      uint32_t* dst = a.qjl_bits + ((seq * tiles + (pos >> 6)) * (D / 32)) * kTile + (pos & 63);
#pragma unroll
      for (int w = 0; w < D / 32; ++w) dst[w * kTile] = sbits[w];
      a.qjl_norm[seq * a.cap + pos] = __half_as_ushort(__float2half_rn(nu));
    }
  }
}

template <int D, int B, int KT, bool QJL>
static hipError_t launch_encode_t(const EncodeArgs& a, int64_t n_seq, hipStream_t s) {
  const dim3 grid((unsigned)((a.n_new + kTile - 1) / kTile), (unsigned)n_seq);
  hipLaunchKernelGGL((k_encode<D, B, KT, QJL>), grid, dim3(64), 0, s, a);
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

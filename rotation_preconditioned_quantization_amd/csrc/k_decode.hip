// OCTOPUS fused decode kernels for gfx950 ([YL] 工程实现: keys are rebuilt from
// the packed indices in registers, never written out; q.k, then online
// softmax and P.V, FlashAttention-style tiling).
//
//   k_rotate     q' = mult * R q once per query ([YL] 旋转魔法: R orthogonal, so
//                <q, k^> = gamma <R q, u'^> and keys are never inverse-rotated);
//                with QJL also p = sqrt(pi/2)/d * S q' ([YL] 可选的残差修正).
//   k_logits     one wavefront per 64-key tile, one key per lane: unpack the
//                word-major tile (coalesced), look up unit directions and rho
//                centroids in LDS, dot with the G query heads of the KV head.
//   k_attn       the same per-key logits, then a wave-wide online softmax and
//                P.V over bf16 V with 16 lanes per V row (coalesced), split-K
//                over the sequence; k_combine merges the splits (log-sum-exp).
//   k_reconstruct  test helper writing k^ = gamma R^T u'^.
#include "octo_device.hpp"

namespace octo {

// ---------------------------------------------------------------------------
// Query rotation.  One wavefront per query row; lane l holds elements
// l + 64 k.  Butterfly strides below 64 pair lanes l and l ^ h (shuffles),
// stride 64 pairs the two values a lane holds.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void k_rotate(RotateArgs a) {
  constexpr int T = (D + 2) / 3;
  constexpr int NV = D / 64;
  __shared__ float s_q[D];
  const int r = blockIdx.x;
  const int qi = r % a.n_q;
  const int h = (r / a.n_q) % a.Hq;
  const int b = r / (a.n_q * a.Hq);
  const int G = a.Hq / a.Hkv;
  const int orow = ((b * a.Hkv + h / G) * G + (h % G)) * a.n_q + qi;
  const int l = threadIdx.x;
  float x[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int j = l + 64 * k;
    float v;
    if (a.qdt == DT_F32) {
      v = ((const float*)a.q)[(int64_t)r * D + j];
    } else {
      const unsigned short u = ((const unsigned short*)a.q)[(int64_t)r * D + j];
      v = a.qdt == DT_BF16 ? __uint_as_float((uint32_t)u << 16) : __half2float(__ushort_as_half(u));
    }
    if ((a.t.sign_bits[j >> 5] >> (j & 31)) & 1u) v = -v;
    x[k] = v;
  }
#pragma unroll
  for (int hh = 1; hh < 64; hh <<= 1) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const float o = __shfl_xor(x[k], hh, 64);
      x[k] = (l & hh) ? (o - x[k]) : (x[k] + o);
    }
  }
  if constexpr (NV == 2) {
    const float a0 = x[0], a1 = x[1];
    x[0] = a0 + a1;
    x[1] = a0 - a1;
  }
  const float mult = a.mult * rsqrtf((float)D);
  float* out = a.qrot + (int64_t)orow * (3 * T);
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    x[k] *= mult;
    out[l + 64 * k] = x[k];
    s_q[l + 64 * k] = x[k];
  }
  if (l < 3 * T - D) out[D + l] = 0.f;
  if (a.qp != nullptr) {
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int j = l + 64 * k;
      const float* row = a.t.S + (int64_t)j * D;
      float acc = 0.f;
#pragma unroll 8
      for (int c = 0; c < D; ++c) acc = __builtin_fmaf(row[c], s_q[c], acc);
      a.qp[(int64_t)orow * D + j] = acc * (1.2533141373155003f / D);  // sqrt(pi/2)/d
    }
  }
}

// Shared per-block setup: direction / rho tables and the QJL byte table.
// lut[m][byte] holds, for the HP heads, sum_k (+1 if bit k of byte else -1) * p[8m+k].
template <int D, int B, int HP, bool QJL>
__device__ __forceinline__ void load_decode_tables(const DecodeArgs& a, int64_t seq, int g0,
                                                   float4* s_dir, float* s_rho, float4* s_lut) {
  using C = Codec<D, B>;
  const int tid = threadIdx.x;
  for (int i = tid; i < C::NDIR; i += blockDim.x) s_dir[i] = a.t.dirtab[i];
  if (tid < C::LR) s_rho[tid] = a.t.rho_tab[tid];
  if constexpr (QJL) {
    const float* p = a.qp + (seq * a.G + g0) * D;
    for (int e = tid; e < (D / 8) * 256; e += blockDim.x) {
      const int m = e >> 8, byte = e & 255;
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h = 0; h < HP; ++h) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float pv = p[h * D + 8 * m + k];
          acc[h] += ((byte >> k) & 1) ? pv : -pv;
        }
      }
      s_lut[e] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
  }
}

// Logits of the lane's key for HP query heads: acc[h] = <q'_h, u'^> (+ QJL).
template <int D, int B, int HP, bool QJL>
__device__ __forceinline__ void key_logits(const DecodeArgs& a, cfloat* qr,
                                           const float4* s_dir, const float* s_rho,
                                           const float4* s_lut, int64_t seq, int64_t t, int lane,
                                           float (&acc)[HP]) {
  using C = Codec<D, B>;
  constexpr int T = C::T, W = C::W;
  constexpr int kTripletGroup = HP >= 4 ? 4 : 8;
  const int64_t tiles = a.cap / kTile;
  const uint32_t* src = a.packed + ((seq * tiles + t) * W) * kTile + lane;
  uint32_t words[W];
#pragma unroll
  for (int w = 0; w < W; ++w) words[w] = src[w * kTile];
#pragma unroll
  for (int h = 0; h < HP; ++h) acc[h] = 0.f;
#pragma unroll
  for (int i = 0; i < T; ++i) {
    const uint32_t code = field_at<W>(words, i * C::BT, C::BT);
    const float4 n = s_dir[code & C::DIR_MASK];
    const float rh = s_rho[code >> (C::BX + C::BE)];
    const float tx = rh * n.x, ty = rh * n.y, tz = rh * n.z;
#pragma unroll
    for (int h = 0; h < HP; ++h) {
      cfloat* qh = qr + h * (3 * T) + 3 * i;
      acc[h] = __builtin_fmaf(tx, qh[0], __builtin_fmaf(ty, qh[1], __builtin_fmaf(tz, qh[2], acc[h])));
    }
    // Issue the LDS gathers and scalar q' loads a few triplets at a time: the
    // accumulators pass through an opaque asm with a memory clobber, so the
    // next group's loads cannot be hoisted above this group's FMAs (bounded
    // VGPR/SGPR live ranges instead of all 3T gathers in flight).
    if (i % kTripletGroup == kTripletGroup - 1) {
#pragma unroll
      for (int h = 0; h < HP; ++h) asm volatile("" : "+v"(acc[h])::"memory");
    }
  }
  if constexpr (QJL) {
    const uint32_t* sb = a.qjl_bits + ((seq * tiles + t) * (D / 32)) * kTile + lane;
    uint32_t sw[D / 32];
#pragma unroll
    for (int w = 0; w < D / 32; ++w) sw[w] = sb[w * kTile];
    const float nu = __half2float(__ushort_as_half(a.qjl_norm[seq * a.cap + t * kTile + lane]));
    float corr[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < D / 8; ++m) {
      const uint32_t byte = (sw[m >> 2] >> (8 * (m & 3))) & 255u;
      const float4 e = s_lut[(m << 8) + byte];
      corr[0] += e.x;
      if (HP > 1) corr[1] += e.y;
      if (HP > 2) { corr[2] += e.z; corr[3] += e.w; }
    }
#pragma unroll
    for (int h = 0; h < HP; ++h) acc[h] = __builtin_fmaf(nu, corr[h], acc[h]);
  }
}

// ---------------------------------------------------------------------------
// Logits.  grid = (blocks over key tiles, n_seq, G / HP); 4 waves per block.
// ---------------------------------------------------------------------------
template <int D, int B, int HP, bool QJL>
__global__ __launch_bounds__(256) void k_logits(DecodeArgs a) {
  using C = Codec<D, B>;
  constexpr int T = C::T;
  __shared__ float4 s_dir[C::NDIR];
  __shared__ float s_rho[C::LR];
  __shared__ float4 s_lut[QJL ? (D / 8) * 256 : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t seq = blockIdx.y;
  const int g0 = blockIdx.z * HP;
  load_decode_tables<D, B, HP, QJL>(a, seq, g0, s_dir, s_rho, s_lut);
  __syncthreads();
  cfloat* qr = (cfloat*)(a.qrot + (seq * a.G + g0) * (3 * T));
  const int64_t ntile = (a.n_keys + kTile - 1) / kTile;
  const int64_t bidx = seq / a.Hkv, kvh = seq % a.Hkv;
  for (int64_t t = (int64_t)blockIdx.x * 4 + wave; t < ntile; t += (int64_t)gridDim.x * 4) {
    // q' is read through the scalar cache every tile (SGPR operands), not
    // hoisted into 3T*HP vector registers.
    cfloat* qt = qr + opaque_zero();
    float acc[HP];
    key_logits<D, B, HP, QJL>(a, qt, s_dir, s_rho, s_lut, seq, t, lane, acc);
    const int64_t key = t * kTile + lane;
    if (key < a.n_keys) {
      const float gamma = a.gamma[seq * a.cap + key];
#pragma unroll
      for (int h = 0; h < HP; ++h) {
        const int64_t hq = kvh * a.G + g0 + h;
        a.logits[(bidx * a.Hq + hq) * a.n_keys + key] = gamma * acc[h];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Single-query split-K attention.  grid = (n_split, n_seq, G / HP), 4 waves.
// Partial (m, l, o) per (query head, split); m in log2 units.
// ---------------------------------------------------------------------------
template <int D, int B, int HP, bool QJL>
__global__ __launch_bounds__(256) void k_attn(DecodeArgs a) {
  using C = Codec<D, B>;
  constexpr int T = C::T;
  constexpr int DPL = D / 16;             // V dims per lane (16 lanes per V row)
  __shared__ float4 s_dir[C::NDIR];
  __shared__ float s_rho[C::LR];
  __shared__ float4 s_lut[QJL ? (D / 8) * 256 : 1];
  __shared__ float s_p[4][kTile][HP];
  __shared__ float s_ml[4][HP][2];
  __shared__ float s_o[4][HP][D];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gq = lane >> 4, li = lane & 15;
  const int64_t seq = blockIdx.y;
  const int g0 = blockIdx.z * HP;
  load_decode_tables<D, B, HP, QJL>(a, seq, g0, s_dir, s_rho, s_lut);
  __syncthreads();

  cfloat* qr = (cfloat*)(a.qrot + (seq * a.G + g0) * (3 * T));
  const int64_t ntile = (a.n_keys + kTile - 1) / kTile;
  const int64_t t_begin = (int64_t)blockIdx.x * a.tiles_per_split;
  int64_t t_end = t_begin + a.tiles_per_split;
  if (t_end > ntile) t_end = ntile;
  const unsigned short* vbase = (const unsigned short*)a.v + seq * a.cap * D + li * DPL;

  float m[HP], l[HP], o[HP][DPL];
#pragma unroll
  for (int h = 0; h < HP; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int c = 0; c < DPL; ++c) o[h][c] = 0.f;
  }

  for (int64_t t = t_begin + wave; t < t_end; t += 4) {
    // V rows of this tile: lane group gq takes keys 4*jj + gq.
    uint32_t vraw[16][DPL / 2];
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const int64_t kv = t * kTile + 4 * jj + gq;
      if (kv < a.n_keys) {
        const unsigned short* src = vbase + kv * D;
        if constexpr (DPL == 8) {
          const uint4 u = *(const uint4*)src;
          vraw[jj][0] = u.x; vraw[jj][1] = u.y; vraw[jj][2] = u.z; vraw[jj][3] = u.w;
        } else {
          const uint2 u = *(const uint2*)src;
          vraw[jj][0] = u.x; vraw[jj][1] = u.y;
        }
      } else {
#pragma unroll
        for (int c = 0; c < DPL / 2; ++c) vraw[jj][c] = 0u;
      }
    }
    cfloat* qt = qr + opaque_zero();
    float acc[HP];
    key_logits<D, B, HP, QJL>(a, qt, s_dir, s_rho, s_lut, seq, t, lane, acc);
    const int64_t key = t * kTile + lane;
    const bool valid = key < a.n_keys;
    const float gamma = valid ? a.gamma[seq * a.cap + key] : 0.f;
#pragma unroll
    for (int h = 0; h < HP; ++h) {
      const float sc = valid ? gamma * acc[h] : -INFINITY;
      const float mn = fmaxf(m[h], wave_max(sc));
      const float alpha = exp2f(m[h] - mn);
      const float p = exp2f(sc - mn);
      l[h] = __builtin_fmaf(l[h], alpha, p);
#pragma unroll
      for (int c = 0; c < DPL; ++c) o[h][c] *= alpha;
      m[h] = mn;
      s_p[wave][lane][h] = p;
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      float pv[HP];
#pragma unroll
      for (int h = 0; h < HP; ++h) pv[h] = s_p[wave][4 * jj + gq][h];
#pragma unroll
      for (int c = 0; c < DPL / 2; ++c) {
        const float v0 = bf16_lo(vraw[jj][c]), v1 = bf16_hi(vraw[jj][c]);
#pragma unroll
        for (int h = 0; h < HP; ++h) {
          o[h][2 * c] = __builtin_fmaf(pv[h], v0, o[h][2 * c]);
          o[h][2 * c + 1] = __builtin_fmaf(pv[h], v1, o[h][2 * c + 1]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // Reduce inside the wave: l over all lanes, o over the 4 lane groups.
#pragma unroll
  for (int h = 0; h < HP; ++h) {
    l[h] = wave_sum(l[h]);
#pragma unroll
    for (int c = 0; c < DPL; ++c) {
      float x = o[h][c];
      x += __shfl_xor(x, 16, 64);
      x += __shfl_xor(x, 32, 64);
      o[h][c] = x;
    }
  }
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < HP; ++h)
#pragma unroll
      for (int c = 0; c < DPL; ++c) s_o[wave][h][li * DPL + c] = o[h][c];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < HP; ++h) { s_ml[wave][h][0] = m[h]; s_ml[wave][h][1] = l[h]; }
  }
  __syncthreads();
  // Merge the 4 waves and write this block's partial.
  const int64_t bidx = seq / a.Hkv, kvh = seq % a.Hkv;
  for (int e = threadIdx.x; e < HP * (D + 2); e += blockDim.x) {
    const int h = e / (D + 2), c = e % (D + 2);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_ml[w][h][0]);
    float val;
    if (c == 0) {
      val = M;
    } else {
      val = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float sc = (s_ml[w][h][0] == -INFINITY) ? 0.f : exp2f(s_ml[w][h][0] - M);
        val += sc * (c == 1 ? s_ml[w][h][1] : s_o[w][h][c - 2]);
      }
    }
    const int64_t row = bidx * a.Hq + kvh * a.G + g0 + h;
    a.part[(row * a.n_split + blockIdx.x) * (D + 2) + c] = val;
  }
}

// out[row][c] = sum_s 2^(m_s - M) o_s[c] / sum_s 2^(m_s - M) l_s, one block per
// row.  The split weights are formed once in LDS; every thread then sums an
// independent strided slice of the splits for its output column, so the
// partial loads are issued back to back instead of one latency at a time.
constexpr int kCombineThreads = 256;
constexpr int kMaxSplit = 1024;

__global__ __launch_bounds__(kCombineThreads) void k_combine(CombineArgs a) {
  __shared__ float s_w[kMaxSplit];
  __shared__ float s_red[kCombineThreads];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int ns = a.n_split, stride = a.d + 2;
  const float* p = a.part + row * ns * stride;
  float mloc = -INFINITY;
  for (int s = tid; s < ns; s += kCombineThreads) {
    const float m = p[s * stride];
    s_w[s] = m;
    mloc = fmaxf(mloc, m);
  }
  s_red[tid] = mloc;
  __syncthreads();
  for (int o = kCombineThreads / 2; o > 0; o >>= 1) {
    if (tid < o) s_red[tid] = fmaxf(s_red[tid], s_red[tid + o]);
    __syncthreads();
  }
  const float M = s_red[0];
  __syncthreads();
  float lden = 0.f;
  for (int s = tid; s < ns; s += kCombineThreads) {
    const float m = s_w[s];
    const float w = (m == -INFINITY) ? 0.f : exp2f(m - M);
    s_w[s] = w;
    lden = __builtin_fmaf(w, p[s * stride + 1], lden);
  }
  s_red[tid] = lden;
  __syncthreads();
  for (int o = kCombineThreads / 2; o > 0; o >>= 1) {
    if (tid < o) s_red[tid] += s_red[tid + o];
    __syncthreads();
  }
  const float den = s_red[0];
  __syncthreads();
  // kCombineThreads / d threads per output column, each over a slice of splits
  const int per_col = kCombineThreads / a.d;
  const int c = tid % a.d, part = tid / a.d;
  float num = 0.f;
  if (part < per_col) {
#pragma unroll 4
    for (int s = part; s < ns; s += per_col) num = __builtin_fmaf(s_w[s], p[s * stride + 2 + c], num);
  }
  s_red[tid] = num;
  __syncthreads();
  if (tid < a.d) {
    float tot = 0.f;
    for (int k = 0; k < per_col; ++k) tot += s_red[k * a.d + tid];
    a.out[row * a.d + tid] = den > 0.f ? tot / den : 0.f;
  }
}

__global__ void k_fill_zero(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

// ---------------------------------------------------------------------------
// Test helper: k^ = gamma d^-1/2 s .* H u'^, one key per thread.
// ---------------------------------------------------------------------------
template <int D, int B>
__global__ __launch_bounds__(64) void k_reconstruct(ReconArgs a) {
  using C = Codec<D, B>;
  constexpr int T = C::T, W = C::W;
  const int64_t seq = blockIdx.y;
  const int64_t key = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (key >= a.n_keys) return;
  const int64_t tiles = a.cap / kTile;
  const uint32_t* src = a.packed + ((seq * tiles + (key >> 6)) * W) * kTile + (key & 63);
  uint32_t words[W];
#pragma unroll
  for (int w = 0; w < W; ++w) words[w] = src[w * kTile];
  float u[D];
#pragma unroll
  for (int i = 0; i < T; ++i) {
    const uint32_t code = field_at<W>(words, i * C::BT, C::BT);
    const float4 n = a.t.dirtab[code & C::DIR_MASK];
    const float rh = a.t.rho_tab[code >> (C::BX + C::BE)];
    u[3 * i] = rh * n.x;
    if (3 * i + 1 < D) u[3 * i + 1] = rh * n.y;
    if (3 * i + 2 < D) u[3 * i + 2] = rh * n.z;
  }
  wht_regs<D>(u);
  apply_signs<D>(u, a.t.sign_bits);
  const float g = a.gamma[seq * a.cap + key] * rsqrtf((float)D);
  float* dst = a.out + (seq * a.n_keys + key) * D;
#pragma unroll
  for (int j = 0; j < D; ++j) dst[j] = g * u[j];
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
hipError_t launch_rotate(int d, const RotateArgs& a, hipStream_t s) {
  const unsigned rows = (unsigned)(a.B * a.Hq * a.n_q);
  if (rows == 0) return hipSuccess;
  if (d == 64) hipLaunchKernelGGL(k_rotate<64>, dim3(rows), dim3(64), 0, s, a);
  else if (d == 128) hipLaunchKernelGGL(k_rotate<128>, dim3(rows), dim3(64), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int D, int B, int HP, bool QJL>
static hipError_t logits_t(const DecodeArgs& a, int64_t n_seq, int nbx, hipStream_t s) {
  hipLaunchKernelGGL((k_logits<D, B, HP, QJL>), dim3(nbx, (unsigned)n_seq, a.G / HP), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

template <int D, int B, int HP, bool QJL>
static hipError_t attn_t(const DecodeArgs& a, int64_t n_seq, hipStream_t s) {
  hipLaunchKernelGGL((k_attn<D, B, HP, QJL>), dim3(a.n_split, (unsigned)n_seq, a.G / HP),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

#define OCTO_DISPATCH_DBHQ(FN, ...)                                                      \
  switch (d * 100 + b * 10 + hp) {                                                       \
    case 6421: return qjl ? FN<64, 2, 1, true>(__VA_ARGS__) : FN<64, 2, 1, false>(__VA_ARGS__);     \
    case 6422: return qjl ? FN<64, 2, 2, true>(__VA_ARGS__) : FN<64, 2, 2, false>(__VA_ARGS__);     \
    case 6424: return qjl ? FN<64, 2, 4, true>(__VA_ARGS__) : FN<64, 2, 4, false>(__VA_ARGS__);     \
    case 6431: return qjl ? FN<64, 3, 1, true>(__VA_ARGS__) : FN<64, 3, 1, false>(__VA_ARGS__);     \
    case 6432: return qjl ? FN<64, 3, 2, true>(__VA_ARGS__) : FN<64, 3, 2, false>(__VA_ARGS__);     \
    case 6434: return qjl ? FN<64, 3, 4, true>(__VA_ARGS__) : FN<64, 3, 4, false>(__VA_ARGS__);     \
    case 6441: return qjl ? FN<64, 4, 1, true>(__VA_ARGS__) : FN<64, 4, 1, false>(__VA_ARGS__);     \
    case 6442: return qjl ? FN<64, 4, 2, true>(__VA_ARGS__) : FN<64, 4, 2, false>(__VA_ARGS__);     \
    case 6444: return qjl ? FN<64, 4, 4, true>(__VA_ARGS__) : FN<64, 4, 4, false>(__VA_ARGS__);     \
    case 12821: return qjl ? FN<128, 2, 1, true>(__VA_ARGS__) : FN<128, 2, 1, false>(__VA_ARGS__);  \
    case 12822: return qjl ? FN<128, 2, 2, true>(__VA_ARGS__) : FN<128, 2, 2, false>(__VA_ARGS__);  \
    case 12824: return qjl ? FN<128, 2, 4, true>(__VA_ARGS__) : FN<128, 2, 4, false>(__VA_ARGS__);  \
    case 12831: return qjl ? FN<128, 3, 1, true>(__VA_ARGS__) : FN<128, 3, 1, false>(__VA_ARGS__);  \
    case 12832: return qjl ? FN<128, 3, 2, true>(__VA_ARGS__) : FN<128, 3, 2, false>(__VA_ARGS__);  \
    case 12834: return qjl ? FN<128, 3, 4, true>(__VA_ARGS__) : FN<128, 3, 4, false>(__VA_ARGS__);  \
    case 12841: return qjl ? FN<128, 4, 1, true>(__VA_ARGS__) : FN<128, 4, 1, false>(__VA_ARGS__);  \
    case 12842: return qjl ? FN<128, 4, 2, true>(__VA_ARGS__) : FN<128, 4, 2, false>(__VA_ARGS__);  \
    case 12844: return qjl ? FN<128, 4, 4, true>(__VA_ARGS__) : FN<128, 4, 4, false>(__VA_ARGS__);  \
  }                                                                                      \
  return hipErrorInvalidValue;

hipError_t launch_logits(int d, int b, int hp, bool qjl, const DecodeArgs& a, int64_t n_seq,
                         int nbx, hipStream_t s) {
  OCTO_DISPATCH_DBHQ(logits_t, a, n_seq, nbx, s)
}

hipError_t launch_attn(int d, int b, int hp, bool qjl, const DecodeArgs& a, int64_t n_seq,
                       hipStream_t s) {
  OCTO_DISPATCH_DBHQ(attn_t, a, n_seq, s)
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (a.n_split > kMaxSplit || a.d > kCombineThreads) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_combine, dim3(a.rows), dim3(kCombineThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

template <int D, int B>
static hipError_t recon_t(const ReconArgs& a, int64_t n_seq, hipStream_t s) {
  hipLaunchKernelGGL((k_reconstruct<D, B>), dim3((unsigned)((a.n_keys + 63) / 64), (unsigned)n_seq),
                     dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_reconstruct(int d, int b, const ReconArgs& a, int64_t n_seq, hipStream_t s) {
  if (a.n_keys <= 0 || n_seq <= 0) return hipSuccess;
  switch (d * 10 + b) {
    case 642: return recon_t<64, 2>(a, n_seq, s);
    case 643: return recon_t<64, 3>(a, n_seq, s);
    case 644: return recon_t<64, 4>(a, n_seq, s);
    case 1282: return recon_t<128, 2>(a, n_seq, s);
    case 1283: return recon_t<128, 3>(a, n_seq, s);
    case 1284: return recon_t<128, 4>(a, n_seq, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace octo

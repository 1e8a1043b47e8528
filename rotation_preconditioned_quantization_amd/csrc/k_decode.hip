// OCTOPUS fused decode kernels for gfx950 ([YL] 工程实现: keys are rebuilt from
// the packed indices in registers, never written out; q.k, then online
// softmax and P.V, FlashAttention-style tiling).
//
//   k_rotate     q' = mult * R q per query row ([YL] 旋转魔法: R orthogonal, so
//                <q, k^> = gamma <R q, u'^> and keys are never inverse-rotated),
//                for the multi-query kernel; the single-query kernels rotate
//                their own heads in the prologue (with QJL also p = sqrt(pi/2)/d
//                * S q', [YL] 可选的残差修正).
//   k_logits     one wavefront per 64-key tile, one key per lane: unpack the
//                word-major tile (coalesced), rebuild rho^ n^ per triplet from
//                LDS tables, contract with 4 query heads on fp32 MFMA.
//   k_attn       the same per-key logits, then a wave-wide online softmax and
//                P.V over bf16 V (one coalesced row per load, fp32 MFMA),
//                split-K over the sequence; k_combine merges the splits.
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

typedef float floatx4 __attribute__((ext_vector_type(4)));

// LDS of the single-query kernels.  kCombined: for up to 10 bits per triplet
// one float4 per triplet code holds rho^ n^ directly; otherwise unit
// directions per (i_xi, i_eta) plus the rho centroids.  q holds the rotated
// queries of the (up to) 4 heads of this pass, rows padded with zeros; with
// QJL, qp holds p = sqrt(pi/2)/d S q' and lut its nibble sums.
template <int D, int B, bool QJL>
struct SQShared {
  using C = Codec<D, B>;
  static constexpr bool kCombined = C::BT <= 10;
  static constexpr int QD = ((3 * C::T + 3) / 4) * 4;
  float4 tab[kCombined ? (1 << C::BT) : C::NDIR];
  float rho[C::LR];
  float q[4][QD];
  float qp[QJL ? 4 : 1][QJL ? D : 1];
  float4 lut[QJL ? (D / 4) * 16 : 1];
};

// Query rotation in the block prologue: wave w rotates query head g0 + w of
// the block's KV head (q' = mult * R q, R = d^-1/2 H diag(s)), lane l holding
// elements l + 64 k; butterflies of stride < 64 pair lanes (shuffles).  With
// QJL the wave also forms p = sqrt(pi/2)/d * S q'.
template <int D, int B, bool QJL>
__device__ __forceinline__ void rotate_head(const DecodeArgs& a, int64_t seq, int g0, int hcount,
                                            SQShared<D, B, QJL>& sh) {
  using SH = SQShared<D, B, QJL>;
  constexpr int NV = D / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (w >= hcount) {
    for (int j = lane; j < SH::QD; j += 64) sh.q[w][j] = 0.f;
    return;
  }
  const int64_t bidx = seq / a.Hkv, kvh = seq % a.Hkv;
  const int64_t r = bidx * a.Hq + kvh * a.G + g0 + w;
  float x[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int j = lane + 64 * k;
    float v;
    if (a.qdt == DT_F32) {
      v = ((const float*)a.q)[r * D + j];
    } else {
      const unsigned short u = ((const unsigned short*)a.q)[r * D + j];
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
      x[k] = (lane & hh) ? (o - x[k]) : (x[k] + o);
    }
  }
  if constexpr (NV == 2) {
    const float a0 = x[0], a1 = x[1];
    x[0] = a0 + a1;
    x[1] = a0 - a1;
  }
  const float mult = a.mult * rsqrtf((float)D);
#pragma unroll
  for (int k = 0; k < NV; ++k) sh.q[w][lane + 64 * k] = x[k] * mult;
  for (int j = D + lane; j < SH::QD; j += 64) sh.q[w][j] = 0.f;
  if constexpr (QJL) {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int j = lane + 64 * k;
      const float* row = a.t.S + (int64_t)j * D;
      float acc = 0.f;
#pragma unroll 8
      for (int c = 0; c < D; ++c) acc = __builtin_fmaf(row[c], sh.q[w][c], acc);
      sh.qp[w][j] = acc * (1.2533141373155003f / D);  // sqrt(pi/2)/d
    }
  }
}

// Tables of the block (after the rotation; needs a block barrier before the
// QJL nibble table reads qp of all heads).
template <int D, int B, bool QJL>
__device__ __forceinline__ void load_sq_tables(const DecodeArgs& a, SQShared<D, B, QJL>& sh) {
  using C = Codec<D, B>;
  using SH = SQShared<D, B, QJL>;
  const int tid = threadIdx.x;
  if constexpr (SH::kCombined) {
    for (int i = tid; i < (1 << C::BT); i += blockDim.x) sh.tab[i] = a.t.trip_tab[i];
  } else {
    for (int i = tid; i < C::NDIR; i += blockDim.x) sh.tab[i] = a.t.dirtab[i];
  }
  if (tid < C::LR) sh.rho[tid] = a.t.rho_tab[tid];
}

// QJL nibble table: lut[m][nib] holds, per head, sum_k (+1 if bit k of nib
// else -1) * p[4m + k].
template <int D, int B, bool QJL>
__device__ __forceinline__ void build_qjl_lut(int hcount, SQShared<D, B, QJL>& sh) {
  if constexpr (QJL) {
    for (int e = threadIdx.x; e < (D / 4) * 16; e += blockDim.x) {
      const int m = e >> 4, nib = e & 15;
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if (h < hcount) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float pv = sh.qp[h][4 * m + k];
            acc[h] += ((nib >> k) & 1) ? pv : -pv;
          }
        }
      }
      sh.lut[e] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
  }
}

// The compressed words of one 64-key tile, as loaded by one wavefront.
template <int D, int B, bool QJL>
struct KTile {
  uint32_t words[Codec<D, B>::W];
  uint32_t sw[QJL ? D / 32 : 1];
  float gamma;
  float nu;
};

template <int D, int B, bool QJL>
__device__ __forceinline__ void load_ktile(const DecodeArgs& a, int64_t seq, int64_t t, int lane,
                                           KTile<D, B, QJL>& k) {
  constexpr int W = Codec<D, B>::W;
  const int64_t tiles = a.cap / kTile;
  const uint32_t* src = a.packed + ((seq * tiles + t) * W) * kTile + lane;
#pragma unroll
  for (int w = 0; w < W; ++w) k.words[w] = src[w * kTile];
  const int64_t key = t * kTile + lane;
  k.gamma = key < a.n_keys ? a.gamma[seq * a.cap + key] : 0.f;
  if constexpr (QJL) {
    const uint32_t* sb = a.qjl_bits + ((seq * tiles + t) * (D / 32)) * kTile + lane;
#pragma unroll
    for (int w = 0; w < D / 32; ++w) k.sw[w] = sb[w * kTile];
    k.nu = __half2float(__ushort_as_half(a.qjl_norm[seq * a.cap + key]));
  }
}

// Logits of a 64-key tile, one key per lane, for 4 query heads at once:
// returns acc[h] = <q'_h, u'^_key> (+ the QJL term).  The contraction over
// the rotated dims runs on v_mfma_f32_4x4x1_16b_f32: in every 4-lane block
// the A operand is q'[head = lane % 4][dim] and the B operand is the lane's
// own rebuilt coordinate, so block b produces the 4 x 4 outer product for
// keys 4b..4b+3 and lane l ends up holding the 4 heads of key l.  Exact fp32.
template <int D, int B, bool QJL>
__device__ __forceinline__ floatx4 tile_logits(const SQShared<D, B, QJL>& sh,
                                               const KTile<D, B, QJL>& k, int lane) {
  using C = Codec<D, B>;
  using SH = SQShared<D, B, QJL>;
  constexpr int T = C::T, W = C::W;
  constexpr int kGroup = 4;
  const float* qrow = sh.q[lane & 3];
  floatx4 acc[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < T; ++i) {
    const uint32_t code = field_at<W>(k.words, i * C::BT, C::BT);
    float tv[3];
    if constexpr (SH::kCombined) {
      const float4 e = sh.tab[code];
      tv[0] = e.x; tv[1] = e.y; tv[2] = e.z;
    } else {
      const float4 n = sh.tab[code & C::DIR_MASK];
      const float rh = sh.rho[code >> (C::BX + C::BE)];
      tv[0] = rh * n.x; tv[1] = rh * n.y; tv[2] = rh * n.z;
    }
#pragma unroll
    for (int c = 0; c < 3; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_4x4x1f32(qrow[3 * i + c], tv[c], acc[c], 0, 0, 0);
    // a few triplets at a time: keeps the LDS gathers from all being hoisted
    if (i % kGroup == kGroup - 1) asm volatile("" ::: "memory");
  }
  floatx4 r = acc[0] + acc[1] + acc[2];
  if constexpr (QJL) {
    float4 corr = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int m = 0; m < D / 4; ++m) {
      const uint32_t nib = (k.sw[m >> 3] >> (4 * (m & 7))) & 15u;
      const float4 e = sh.lut[(m << 4) + nib];
      corr.x += e.x; corr.y += e.y; corr.z += e.z; corr.w += e.w;
    }
    r[0] = __builtin_fmaf(k.nu, corr.x, r[0]);
    r[1] = __builtin_fmaf(k.nu, corr.y, r[1]);
    r[2] = __builtin_fmaf(k.nu, corr.z, r[2]);
    r[3] = __builtin_fmaf(k.nu, corr.w, r[3]);
  }
  return r;
}

// Prologue shared by both single-query kernels: rotation, tables, barrier.
template <int D, int B, bool QJL>
__device__ __forceinline__ void sq_prologue(const DecodeArgs& a, int64_t seq, int g0, int hcount,
                                            SQShared<D, B, QJL>& sh) {
  rotate_head<D, B, QJL>(a, seq, g0, hcount, sh);
  load_sq_tables<D, B, QJL>(a, sh);
  __syncthreads();
  if constexpr (QJL) {
    build_qjl_lut<D, B, QJL>(hcount, sh);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Logits.  grid = (blocks over key tiles, n_seq, ceil(G / 4)); 4 waves, each
// a stream of 64-key tiles with the next tile's words loaded ahead.
// ---------------------------------------------------------------------------
template <int D, int B, bool QJL>
__global__ __launch_bounds__(256) void k_logits(DecodeArgs a) {
  __shared__ SQShared<D, B, QJL> sh;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t seq = blockIdx.y;
  const int g0 = blockIdx.z * 4;
  const int hcount = a.G - g0 < 4 ? a.G - g0 : 4;
  const int64_t ntile = (a.n_keys + kTile - 1) / kTile;
  const int64_t stride = (int64_t)gridDim.x * 4;
  int64_t t = (int64_t)blockIdx.x * 4 + wave;
  KTile<D, B, QJL> cur;
  if (t < ntile) load_ktile<D, B, QJL>(a, seq, t, lane, cur);
  sq_prologue<D, B, QJL>(a, seq, g0, hcount, sh);
  const int64_t bidx = seq / a.Hkv, kvh = seq % a.Hkv;
  for (; t < ntile; t += stride) {
    KTile<D, B, QJL> nxt;
    if (t + stride < ntile) load_ktile<D, B, QJL>(a, seq, t + stride, lane, nxt);
    const floatx4 acc = tile_logits<D, B, QJL>(sh, cur, lane);
    const int64_t key = t * kTile + lane;
    if (key < a.n_keys) {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if (h < hcount) {
          const int64_t hq = kvh * a.G + g0 + h;
          a.logits[(bidx * a.Hq + hq) * a.n_keys + key] = cur.gamma * acc[h];
        }
      }
    }
    cur = nxt;
  }
}

// ---------------------------------------------------------------------------
// Single-query split-K attention.  grid = (n_split, n_seq, ceil(G / 4)), 4
// waves per block, each wave a stream of 64-key tiles whose next tile (V rows
// and compressed words) is loaded while the current one is computed.  Per
// tile: logits by tile_logits, a wave-wide online softmax per head (DPP
// max), then O[head][dim] += p[head][key] V[key][dim] on
// v_mfma_f32_4x4x1_16b_f32: the A operand is p[head = lane % 4][key], the B
// operand one bf16 of the V row the whole wave reads with one coalesced dword
// load, so lane l keeps O[0..3][2l] and O[0..3][2l+1] (d = 128; for d = 64
// the two half-waves take alternate keys).  Partial (m, l, o) per (query
// head, split); m in log2 units.
// ---------------------------------------------------------------------------
// The V rows of a 64-key tile as the PV MFMA wants them: lane l takes the
// dword (bf16 pair 2 dl, 2 dl + 1) of keys KPI * j + kk_off.  Full tiles
// use constant offsets from one base; the last partial tile checks each key.
template <int D, int NV, int KPI>
__device__ __forceinline__ void load_vtile(const uint32_t* vbase, int64_t t, int64_t n_keys,
                                           int kk_off, uint32_t (&vw)[NV]) {
  constexpr int ROWW = D / 2;  // dwords per V row
  const uint32_t* vt = vbase + (t * kTile + kk_off) * ROWW;
  if ((t + 1) * kTile <= n_keys) {
#pragma unroll
    for (int j = 0; j < NV; ++j) vw[j] = vt[j * KPI * ROWW];
  } else {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int64_t kv = t * kTile + KPI * j + kk_off;
      vw[j] = kv < n_keys ? vt[j * KPI * ROWW] : 0u;
    }
  }
}

template <int D, int B, bool QJL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_attn(DecodeArgs a) {
  constexpr int KPI = 128 / D;          // keys per V load / PV MFMA
  constexpr int NV = kTile / KPI;       // V loads per tile per lane
  __shared__ SQShared<D, B, QJL> sh;
  __shared__ float s_p[4][4][kTile + 4];   // padded rows: the 4 heads hit different banks
  __shared__ float s_ml[4][4][2];
  __shared__ float s_o[4][4][D];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t seq = blockIdx.y;
  const int g0 = blockIdx.z * 4;
  const int hcount = a.G - g0 < 4 ? a.G - g0 : 4;
  const int kk_off = KPI == 2 ? (lane >> 5) : 0;   // key of the pair this lane serves
  const int dl = KPI == 2 ? (lane & 31) : lane;     // dims 2 dl, 2 dl + 1
  const int64_t ntile = (a.n_keys + kTile - 1) / kTile;
  const int64_t t_begin = (int64_t)blockIdx.x * a.tiles_per_split;
  int64_t t_end = t_begin + a.tiles_per_split;
  if (t_end > ntile) t_end = ntile;
  const uint32_t* vbase = (const uint32_t*)a.v + (seq * a.cap * D) / 2 + dl;  // lane's dword column

  // first tile's loads go out before the prologue
  int64_t t = t_begin + wave;
  KTile<D, B, QJL> cur;
  uint32_t vw[NV];
  if (t < t_end) {
    load_vtile<D, NV, KPI>(vbase, t, a.n_keys, kk_off, vw);
    load_ktile<D, B, QJL>(a, seq, t, lane, cur);
  }
  sq_prologue<D, B, QJL>(a, seq, g0, hcount, sh);

  float m[4], l[4];
  floatx4 olo[2], ohi[2];
#pragma unroll
  for (int h = 0; h < 4; ++h) { m[h] = -INFINITY; l[h] = 0.f; }
#pragma unroll
  for (int k = 0; k < 2; ++k) { olo[k] = floatx4{0.f, 0.f, 0.f, 0.f}; ohi[k] = olo[k]; }

  // One tile: logits, online softmax per head, P.V.
  auto process = [&](const KTile<D, B, QJL>& kt, const uint32_t (&vv)[NV], int64_t tt) {
    const floatx4 acc = tile_logits<D, B, QJL>(sh, kt, lane);
    const int64_t key = tt * kTile + lane;
    const bool valid = key < a.n_keys;
    float al[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float sc = valid ? kt.gamma * acc[h] : -INFINITY;
      const float mn = fmaxf(m[h], wave_max(sc));
      al[h] = __builtin_amdgcn_exp2f(m[h] - mn);
      const float p = __builtin_amdgcn_exp2f(sc - mn);
      l[h] = __builtin_fmaf(l[h], al[h], p);
      m[h] = mn;
      s_p[wave][h][lane] = p;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r) { olo[k][r] *= al[r]; ohi[k][r] *= al[r]; }
    __builtin_amdgcn_wave_barrier();
    const float* prow = s_p[wave][lane & 3];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const float pa = prow[KPI * j + kk_off];
      olo[j & 1] = __builtin_amdgcn_mfma_f32_4x4x1f32(pa, bf16_lo(vv[j]), olo[j & 1], 0, 0, 0);
      ohi[j & 1] = __builtin_amdgcn_mfma_f32_4x4x1f32(pa, bf16_hi(vv[j]), ohi[j & 1], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  };

  // Two register sets, used alternately: the next tile loads while one computes.
  KTile<D, B, QJL> kb;
  uint32_t vb[NV];
  for (; t < t_end; t += 8) {
    if (t + 4 < t_end) {
      load_vtile<D, NV, KPI>(vbase, t + 4, a.n_keys, kk_off, vb);
      load_ktile<D, B, QJL>(a, seq, t + 4, lane, kb);
    }
    process(cur, vw, t);
    if (t + 4 >= t_end) break;
    if (t + 8 < t_end) {
      load_vtile<D, NV, KPI>(vbase, t + 8, a.n_keys, kk_off, vw);
      load_ktile<D, B, QJL>(a, seq, t + 8, lane, cur);
    }
    process(kb, vb, t + 4);
  }

  floatx4 olo_s = olo[0] + olo[1], ohi_s = ohi[0] + ohi[1];
  if constexpr (KPI == 2) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      olo_s[r] += __shfl_xor(olo_s[r], 32, 64);
      ohi_s[r] += __shfl_xor(ohi_s[r], 32, 64);
    }
  }
#pragma unroll
  for (int h = 0; h < 4; ++h) l[h] = wave_sum(l[h]);
  if (kk_off == 0) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      s_o[wave][h][2 * dl] = olo_s[h];
      s_o[wave][h][2 * dl + 1] = ohi_s[h];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < 4; ++h) { s_ml[wave][h][0] = m[h]; s_ml[wave][h][1] = l[h]; }
  }
  __syncthreads();
  // Merge the 4 waves and write this block's partial.
  const int64_t bidx = seq / a.Hkv, kvh = seq % a.Hkv;
  for (int e = threadIdx.x; e < hcount * (D + 2); e += blockDim.x) {
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
// row.  The o values of the first splits are loaded before anything else so
// they travel together with the (m, l) loads; the split weights are formed
// once in LDS; thread (c, part) sums the splits part, part + P, ... of column
// c and the P partial sums meet in LDS.
constexpr int kCombineThreads = 256;
constexpr int kMaxSplit = 1024;
constexpr int kCombinePre = 32;

__global__ __launch_bounds__(kCombineThreads) void k_combine(CombineArgs a) {
  __shared__ float s_w[kMaxSplit];
  __shared__ float s_l[kMaxSplit];
  __shared__ float s_red[kCombineThreads];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int ns = a.n_split, stride = a.d + 2;
  const int P = kCombineThreads / a.d;
  const int c = tid % a.d, part = tid / a.d;
  const bool worker = part < P;
  const float* p = a.part + row * ns * stride;
  float pre[kCombinePre];
#pragma unroll
  for (int k = 0; k < kCombinePre; ++k) {
    const int s = part + P * k;
    pre[k] = (worker && s < ns) ? p[s * stride + 2 + c] : 0.f;
  }
  for (int s = tid; s < ns; s += kCombineThreads) {
    s_w[s] = p[s * stride];
    s_l[s] = p[s * stride + 1];
  }
  __syncthreads();
  float mloc = -INFINITY;
  for (int s = tid; s < ns; s += kCombineThreads) mloc = fmaxf(mloc, s_w[s]);
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
    lden = __builtin_fmaf(w, s_l[s], lden);
  }
  s_red[tid] = lden;
  __syncthreads();
  for (int o = kCombineThreads / 2; o > 0; o >>= 1) {
    if (tid < o) s_red[tid] += s_red[tid + o];
    __syncthreads();
  }
  const float den = s_red[0];
  __syncthreads();
  float num = 0.f;
  if (worker) {
#pragma unroll
    for (int k = 0; k < kCombinePre; ++k) {
      const int s = part + P * k;
      if (s < ns) num = __builtin_fmaf(s_w[s], pre[k], num);
    }
    for (int s = part + P * kCombinePre; s < ns; s += P) num = __builtin_fmaf(s_w[s], p[s * stride + 2 + c], num);
  }
  s_red[tid] = num;
  __syncthreads();
  if (tid < a.d) {
    float tot = 0.f;
    for (int k = 0; k < P; ++k) tot += s_red[k * a.d + tid];
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

template <int D, int B, bool QJL>
static hipError_t logits_t(const DecodeArgs& a, int64_t n_seq, int nbx, hipStream_t s) {
  hipLaunchKernelGGL((k_logits<D, B, QJL>), dim3(nbx, (unsigned)n_seq, (a.G + 3) / 4), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

template <int D, int B, bool QJL>
static hipError_t attn_t(const DecodeArgs& a, int64_t n_seq, hipStream_t s) {
  hipLaunchKernelGGL((k_attn<D, B, QJL>), dim3(a.n_split, (unsigned)n_seq, (a.G + 3) / 4),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

#define OCTO_DISPATCH_DBQ(FN, ...)                                                              \
  switch (d * 10 + b) {                                                                         \
    case 642: return qjl ? FN<64, 2, true>(__VA_ARGS__) : FN<64, 2, false>(__VA_ARGS__);        \
    case 643: return qjl ? FN<64, 3, true>(__VA_ARGS__) : FN<64, 3, false>(__VA_ARGS__);        \
    case 644: return qjl ? FN<64, 4, true>(__VA_ARGS__) : FN<64, 4, false>(__VA_ARGS__);        \
    case 1282: return qjl ? FN<128, 2, true>(__VA_ARGS__) : FN<128, 2, false>(__VA_ARGS__);     \
    case 1283: return qjl ? FN<128, 3, true>(__VA_ARGS__) : FN<128, 3, false>(__VA_ARGS__);     \
    case 1284: return qjl ? FN<128, 4, true>(__VA_ARGS__) : FN<128, 4, false>(__VA_ARGS__);     \
  }                                                                                             \
  return hipErrorInvalidValue;

hipError_t launch_logits(int d, int b, bool qjl, const DecodeArgs& a, int64_t n_seq, int nbx,
                         hipStream_t s) {
  OCTO_DISPATCH_DBQ(logits_t, a, n_seq, nbx, s)
}

hipError_t launch_attn(int d, int b, bool qjl, const DecodeArgs& a, int64_t n_seq, hipStream_t s) {
  OCTO_DISPATCH_DBQ(attn_t, a, n_seq, s)
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

// Multi-query fused attention over the compressed cache (many query tokens
// per head, e.g. a block of video frames attending to the cache) on gfx950
// MFMA ([YL] 工程实现: keys rebuilt on the fly, FlashAttention tiling, online
// softmax; the block/chunk decoding of the video workloads in 实验结果).
//
// Workgroup = 8 wavefronts = 256 queries of one head over one split of the
// cache, so every rebuilt key serves 256 queries.  Per tile of 128 keys:
//   1. the keys are rebuilt from the packed stream into LDS as fp16 rotated
//      unit directions u'^ (gamma kept in fp32): wave w takes the 64 keys of
//      half w / 4 (one per lane) and the dim quarter w % 4 of each, i.e. only
//      the triplets that touch those dims;
//   2. the bf16 V tile is stored transposed in LDS as fp16;
//   3. each wave computes S^T = K^ Q'^T for its 32 queries with
//      v_mfma_f32_32x32x16_f16 (fp32 accumulate), scales by gamma, runs the
//      online softmax in the accumulator registers, and feeds P^T straight
//      from those registers into O^T += V^T P^T (same MFMA shape).
// Queries are the rotated q' = R q (keys are never inverse-rotated), scaled
// per row by a power of two so fp16 holds them without overflow.
#include "octo_device.hpp"

namespace octo {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kMQCompute = 8;                // matrix waves per workgroup
constexpr int kMQQueries = 32 * kMQCompute;  // queries per workgroup (32 per matrix wave)

// Workgroup shape.  At d = 64 the matrix waves fit three to a SIMD, so four
// more waves do the staging (key rebuild, V transpose, loads) next to them;
// at d = 128 the eight matrix waves stage the tiles themselves.
template <int D>
struct MQShape {
  static constexpr int KT = 128;                  // keys per tile
  static constexpr int KP = D * 2 + 16;           // K^ row pitch in bytes (fp16)
  // V^T row pitch in bytes (fp16): 66 dwords keep the 8-byte P.V operand
  // reads of 32 consecutive rows on distinct banks and halve the bank
  // collisions of the transposing writes against a 68-dword pitch
  static constexpr int VP = KT * 2 + 8;
  static constexpr int SW = D == 64 ? 4 : 0;      // staging-only waves
  static constexpr int NW = kMQCompute + SW;      // waves per workgroup
  static constexpr int NSW = SW ? SW : kMQCompute;  // waves that stage
  static constexpr int PARTS = NSW / 2;           // staging waves per 64-key half
  static constexpr int DQ = D / PARTS;            // dims rebuilt per lane
  static constexpr int NTH_S = 64 * NSW;          // staging threads
  static constexpr int KPT = KT * D / (8 * NTH_S);  // keys per thread of the V transpose
};

// Registers carrying one tile's global data from its loads (issued during
// the previous tile's matrix work) to its LDS staging.
template <int D, int B>
struct MQStage {
  uint32_t words[Codec<D, B>::W];   // the lane's key
  float gamma;
  uint4 v[MQShape<D>::KPT];         // KPT V rows, 8 dims each
};

// Loads of tile t by staging thread stid (rows past n_keys read the last
// key; they are masked later).  The waves of a key half all load the half's
// words (the same lines).
template <int D, int B>
__device__ __forceinline__ void mq_load(const MQArgs& a, int64_t seq, int64_t t, int stid,
                                        MQStage<D, B>& st) {
  using S = MQShape<D>;
  constexpr int W = Codec<D, B>::W;
  const int lane = stid & 63, sw = stid >> 6;
  const int64_t tiles64 = a.cap / kTile;
  int64_t key = t * S::KT + 64 * (sw / S::PARTS) + lane;
  key = key < a.n_keys ? key : a.n_keys - 1;
  TileWords<W>::load(a.packed + (seq * tiles64 + (key >> 6)) * W * kTile, (int)(key & 63), st.words);
  st.gamma = a.gamma[seq * a.cap + key];
  const int c = stid % (D / 8), kg = stid / (D / 8);
  const uint4* vseq = (const uint4*)a.v + seq * a.cap * (D / 8) + c;
#pragma unroll
  for (int i = 0; i < S::KPT; ++i) {
    int64_t kv = t * S::KT + kg * S::KPT + i;
    kv = kv < a.n_keys ? kv : a.n_keys - 1;
    st.v[i] = vseq[kv * (D / 8)];
  }
}

// bf16 pair -> f16 pair (V of the multi-query path must lie in fp16 range).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w << 16),
                                                                 __uint_as_float(w & 0xffff0000u)));
}

// Dims [PART DQ, (PART + 1) DQ) of the lane's rebuilt key u'^ = rho^ n^ per
// triplet, from the triplets that touch them, to the key's fp16 row in LDS.
template <int D, int B, int PART>
__device__ __forceinline__ void mq_rebuild(const MQStage<D, B>& st, bool ok, const float4* s_dir,
                                           const float* s_rho, unsigned char* krow) {
  using C = Codec<D, B>;
  constexpr int DQ = MQShape<D>::DQ, LO = PART * DQ, HI = LO + DQ;
  float u[DQ];
#pragma unroll
  for (int i = LO / 3; i <= (HI - 1) / 3; ++i) {
    const uint32_t code = field_at<C::W>(st.words, i * C::BT, C::BT);
    const float4 n = s_dir[code & C::DIR_MASK];
    const float rh = ok ? s_rho[code >> (C::BX + C::BE)] : 0.f;
    const float t3[3] = {rh * n.x, rh * n.y, rh * n.z};
#pragma unroll
    for (int c = 0; c < 3; ++c)
      if (3 * i + c >= LO && 3 * i + c < HI) u[3 * i + c - LO] = t3[c];
  }
  uint4* row = (uint4*)(krow + LO * 2);
#pragma unroll
  for (int j = 0; j < DQ / 8; ++j) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(u[8 * j + 2 * e], u[8 * j + 2 * e + 1]));
    row[j] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <int D, int B>
__global__ __launch_bounds__(64 * MQShape<D>::NW) void k_mq_attn(MQArgs a) {
  using C = Codec<D, B>;
  using S = MQShape<D>;
  constexpr int T = C::T;
  constexpr int KT = S::KT, KP = S::KP, VP = S::VP, NTH = 64 * S::NW;
  constexpr int NKS = D / 16;  // MFMA K-steps over the head dim
  constexpr int NMB = D / 32;  // 32-row blocks of O^T

  // two sets of tile buffers: tile t + 1 is staged while tile t is computed
  __shared__ __align__(16) unsigned char s_k[2][KT * KP];
  __shared__ __align__(16) unsigned char s_vt[2][D * VP];
  __shared__ __align__(16) float s_g[2][KT];
  __shared__ float4 s_dir[C::NDIR];
  __shared__ float s_rho[C::LR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, ln = lane & 31;
  const int bh = blockIdx.z;                 // b * Hq + h
  const int b = bh / a.H, h = bh % a.H;
  const int kvh = h / a.G;
  const int64_t seq = (int64_t)b * a.Hkv + kvh;
  const int q0 = blockIdx.y * kMQQueries + wave * 32;
  const int q = q0 + ln;
  const bool qvalid = wave < kMQCompute && q < a.n_q;
  const bool wave_q = wave < kMQCompute && q0 < a.n_q;   // a matrix wave with queries (uniform)
  const bool stager = S::SW == 0 || wave >= kMQCompute;  // (uniform)
  const int stid = S::SW == 0 ? tid : tid - 64 * kMQCompute;  // staging thread index

  for (int i = tid; i < C::NDIR; i += NTH) s_dir[i] = a.t.dirtab[i];
  if (tid < C::LR) s_rho[tid] = a.t.rho_tab[tid];

  // Q' fragment: B[k = dim][n = query], lane (ln, g) holds dims 16j + 8g + 0..7.
  half8 qf[NKS];
  float qscale_inv;
  {
    const float* qrow = a.qrot + (((seq * a.G + h % a.G) * a.n_q) + (qvalid ? q : 0)) * (3 * T);
    float v[NKS][8];
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < NKS; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[j][i] = qvalid ? qrow[16 * j + 8 * g + i] : 0.f;
        amax = fmaxf(amax, fabsf(v[j][i]));
      }
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    int ex = 0;
    __builtin_frexpf(amax, &ex);
    const int sh = amax > 0.f ? 7 - ex : 0;   // row max into [64, 128)
    const float sc = __builtin_ldexpf(1.0f, sh);
    qscale_inv = __builtin_ldexpf(1.0f, -sh);
#pragma unroll
    for (int j = 0; j < NKS; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) qf[j][i] = (_Float16)(v[j][i] * sc);
  }

  floatx16 o[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[mb][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int64_t ntile = (a.n_keys + KT - 1) / KT;
  const int64_t t_begin = (int64_t)blockIdx.x * a.tiles_per_split;
  const int64_t t_end = t_begin + a.tiles_per_split < ntile ? t_begin + a.tiles_per_split : ntile;
  constexpr int KPT = S::KPT;

  // Stage one tile from the registers of its loads into LDS buffer set bs:
  //   keys rebuilt by wave w for key half w / 4 and dim quarter w % 4;
  //   V transposed to [dim][key] fp16, this thread's KPT keys x 8 dims.
  MQStage<D, B> st;
  auto stage = [&](int64_t k0, int bs) {
    {
      const int sw = stid >> 6;
      const int kk = 64 * (sw / S::PARTS) + lane;
      const bool ok = k0 + kk < a.n_keys;
      unsigned char* krow = s_k[bs] + kk * KP;
      const int part = sw % S::PARTS;
      if (part == 0) {
        mq_rebuild<D, B, 0>(st, ok, s_dir, s_rho, krow);
        s_g[bs][kk] = ok ? st.gamma : 0.f;
      } else if (part == 1) {
        mq_rebuild<D, B, 1>(st, ok, s_dir, s_rho, krow);
      } else if constexpr (S::PARTS > 2) {
        if (part == 2) mq_rebuild<D, B, 2>(st, ok, s_dir, s_rho, krow);
        else mq_rebuild<D, B, 3>(st, ok, s_dir, s_rho, krow);
      }
    }
    const int c = stid % (D / 8), kg = stid / (D / 8);
    uint32_t hv[KPT][4];   // f16 pairs (dims 2e, 2e+1) per key
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const bool ok = k0 + kg * KPT + i < a.n_keys;
      const uint32_t src[4] = {st.v[i].x, st.v[i].y, st.v[i].z, st.v[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) hv[i][e] = ok ? bf16x2_to_f16x2(src[e]) : 0u;
    }
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
      uint32_t col[KPT / 2];
#pragma unroll
      for (int i = 0; i < KPT / 2; ++i)
        col[i] = __builtin_amdgcn_perm(hv[2 * i + 1][dd >> 1], hv[2 * i][dd >> 1], sel);
      unsigned char* dst = s_vt[bs] + (8 * c + dd) * VP + kg * KPT * 2;
      if constexpr (KPT == 2) *(uint32_t*)dst = col[0];
      else if constexpr (KPT == 4) *(uint2*)dst = make_uint2(col[0], col[1]);
      else *(uint4*)dst = make_uint4(col[0], col[1], col[2], col[3]);
    }
  };

  if (stager) mq_load<D, B>(a, seq, t_begin < ntile ? t_begin : 0, stid, st);
  __syncthreads();  // s_dir / s_rho
  if (stager && t_begin < t_end) {
    stage(t_begin * KT, 0);
    mq_load<D, B>(a, seq, t_begin + 1 < t_end ? t_begin + 1 : t_begin, stid, st);
  }
  __syncthreads();

  for (int64_t t = t_begin; t < t_end; ++t) {
    const int64_t k0 = t * KT;
    const int cb = (int)((t - t_begin) & 1);
    // stage the next tile into the other buffer set (its last reader, the
    // previous tile's matrix work, finished before the last barrier), then
    // request the tile after it
    if (stager && t + 1 < t_end) {
      stage(k0 + KT, cb ^ 1);
      mq_load<D, B>(a, seq, t + 2 < t_end ? t + 2 : t + 1, stid, st);
    }
    const unsigned char* sk = s_k[cb];
    const unsigned char* svt = s_vt[cb];
    const float* sg = s_g[cb];
    if (wave_q) {
    // 3. 64 keys at a time: S^T, online softmax, O^T += V^T P^T.  Scores stay
    // unscaled by the query's power of two (s' = q'.u'^ gamma 2^sh): the max
    // is taken on s', and exp2(s' 2^-sh - m) is one fma and one exp.
    const bool partial = k0 + KT > a.n_keys;
#pragma unroll 1
    for (int ch = 0; ch < KT / 64; ++ch) {
      floatx16 s[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const int kb = ch * 64 + sb * 32;
        floatx16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int j = 0; j < NKS; ++j) {
          const half8 kf = *(const half8*)(sk + (kb + ln) * KP + (16 * j + 8 * g) * 2);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[j], acc, 0, 0, 0);
        }
        // register r holds key row kb + 8 (r / 4) + 4 g + r % 4
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float4 gv = *(const float4*)(sg + kb + 8 * rr + 4 * g);
          acc[4 * rr] *= gv.x;
          acc[4 * rr + 1] *= gv.y;
          acc[4 * rr + 2] *= gv.z;
          acc[4 * rr + 3] *= gv.w;
        }
        if (partial) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (k0 + kb + 8 * (r >> 2) + 4 * g + (r & 3) >= a.n_keys) acc[r] = -INFINITY;
        }
        s[sb] = acc;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx * qscale_inv);
      // a row with no valid key yet keeps m = -inf; exponents use 0 then
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float lsum = 0.f;
      half8 pf[2][2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          pf[sb][r >> 3][r & 7] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][r], qscale_inv, -m_use));
      // l sums the fp16 p that P.V uses: v_dot2 over the packed pairs
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const half2v pp = {pf[sb][hh][2 * e], pf[sb][hh][2 * e + 1]};
            lsum = __builtin_amdgcn_fdot2(pp, half2v{(_Float16)1.0f, (_Float16)1.0f}, lsum, false);
          }
      l_run = __builtin_fmaf(l_run, alpha, lsum);
      m_run = m_new;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[mb][r] *= alpha;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int kbase = ch * 64 + sb * 32 + 16 * half + 4 * g;
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) {
            const unsigned char* vrow = svt + (32 * mb + ln) * VP;
            const half4 lo = *(const half4*)(vrow + kbase * 2);
            const half4 hi = *(const half4*)(vrow + (kbase + 8) * 2);
            const half8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[sb][half], o[mb], 0, 0, 0);
          }
        }
      }
    }
    }  // wave_q
    __syncthreads();  // this tile's buffers are free, the next tile's staged
  }

  l_run += __shfl_xor(l_run, 32, 64);
  if (qvalid) {
    float* dst = a.part + (((int64_t)bh * a.n_q + q) * a.n_split + blockIdx.x) * (D + 2);
    if (g == 0) {
      dst[0] = m_run;
      dst[1] = l_run;
    }
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[2 + 32 * mb + 8 * (r >> 2) + 4 * g + (r & 3)] = o[mb][r];
  }
}

template <int D, int B>
static hipError_t mq_t(const MQArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.n_split, (unsigned)((a.n_q + kMQQueries - 1) / kMQQueries),
                  (unsigned)(a.B * a.H));
  hipLaunchKernelGGL((k_mq_attn<D, B>), grid, dim3(64 * MQShape<D>::NW), 0, s, a);
  return hipGetLastError();
}

int mq_tile_keys(int d) { return d == 64 ? MQShape<64>::KT : MQShape<128>::KT; }
int mq_block_queries() { return kMQQueries; }

hipError_t launch_mq_attn(int d, int b, const MQArgs& a, hipStream_t s) {
  switch (d * 10 + b) {
    case 641: return mq_t<64, 1>(a, s);
    case 642: return mq_t<64, 2>(a, s);
    case 643: return mq_t<64, 3>(a, s);
    case 644: return mq_t<64, 4>(a, s);
    case 1282: return mq_t<128, 2>(a, s);
    case 1283: return mq_t<128, 3>(a, s);
    case 1284: return mq_t<128, 4>(a, s);
    case 645: return mq_t<64, 5>(a, s);
    case 1281: return mq_t<128, 1>(a, s);
    // d = 128 at b = 5: the 4096-entry direction table and the two tile
    // buffer sets do not fit the 160 KiB of LDS together (not supported)
  }
  return hipErrorInvalidValue;
}

}  // namespace octo

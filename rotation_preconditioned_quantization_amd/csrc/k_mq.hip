// Multi-query fused attention over the compressed cache (many query tokens
// per head, e.g. a block of video frames attending to the cache) on gfx950
// MFMA ([YL] 工程实现: keys rebuilt on the fly, FlashAttention tiling, online
// softmax; the block/chunk decoding of the video workloads in 实验结果).
//
// Workgroup = 8 wavefronts = 256 queries of one head over one split of the
// cache, so every rebuilt key serves 256 queries.  Per tile of 128 keys:
//   1. the keys are rebuilt from the packed stream into LDS as fp16 rows
//      gamma 2^-e u'^, with one power of two 2^e per 64-key half (the half's
//      largest gamma scaled into [1/2, 1)): wave w takes the 64 keys of half
//      w / PARTS (one per lane) and the dim range w % PARTS of each, i.e. only
//      the triplets that touch those dims;
//   2. the bf16 V tile is stored in LDS as fp16 key rows (64-byte segments
//      XOR-swizzled by row), and the P.V operands come out transposed from
//      ds_read_b64_tr_b16;
//   3. each wave computes S^T = K^ Q'^T for its 32 queries with
//      v_mfma_f32_32x32x16_f16 (fp32 accumulate), runs the online softmax in
//      the accumulator registers (the half's 2^e folded into the one scale
//      factor of the exponent), and feeds P^T straight from those registers
//      into O^T += V^T P^T (same MFMA shape).
// Folding gamma into the rows needs no per-score multiply, cannot overflow
// fp16 (every row element is at most 1), and leaves the absolute error of a
// score at most that of the half's largest-norm key, which fp16 rounding sets
// anyway: a key far smaller than its neighbours loses relative precision only
// below 2^-24 of the half's largest gamma.
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
// at d >= 128 the eight matrix waves stage the tiles themselves.  Tiles hold
// 128 keys, except at d = 128, b = 5, where the 4096-entry direction table
// (64 KiB) leaves room in LDS for two buffer sets of 64-key tiles only, and
// at d = 256 (K^ rows of 512 bytes).  At d = 256 the value dims are split
// over two workgroups (adjacent blocks, value part blockIdx.x % 2): each
// computes every score of its queries and the output of 128 value dims, so
// a matrix wave holds 64 accumulator registers of O^T, not 128.
template <int D, int B>
struct MQShape {
  static constexpr int KT = D == 256 || (D == 128 && B == 5) ? 64 : 128;  // keys per tile
  static constexpr int DV = D > 128 ? 128 : D;    // value dims per workgroup
  static constexpr int NVP = D / DV;              // value parts
  static constexpr int KP = D * 2 + 16;           // K^ row pitch in bytes (fp16)
  static constexpr int VR = DV * 2;               // V row bytes (fp16, unpadded)
  static constexpr int SW = D == 64 ? 4 : 0;      // staging-only waves
  static constexpr int NW = kMQCompute + SW;      // waves per workgroup
  static constexpr int NSW = SW ? SW : kMQCompute;  // waves that stage
  static constexpr int PARTS = NSW / (KT / 64);   // staging waves per 64-key half
  static constexpr int DQ = D / PARTS;            // dims rebuilt per lane
  static_assert(DQ % 8 == 0 && PARTS * DQ == D, "whole 16-byte row segments per lane");
  static constexpr int NTH_S = 64 * NSW;          // staging threads
  static constexpr int KPT = KT * DV / (8 * NTH_S);  // V rows staged per thread
  static constexpr int KGS = NTH_S / (DV / 8);       // key stride between them
};

// 64-byte segment swizzle of V row r in LDS: segment s is stored at s ^
// vswz(r).  The 4 rows one half-wave's transposing read touches (r = 4m ..
// 4m + 3) then cover all 64 banks, as do the 16-byte staging writes.
template <int DV>
__device__ __forceinline__ int vswz(int r) { return DV == 64 ? (r >> 1) & 1 : r & 3; }

// Registers carrying one tile's global data from its loads (issued during
// the previous tile's matrix work) to its LDS staging.
template <int D, int B>
struct MQStage {
  uint32_t words[Codec<D, B>::W];   // the lane's key
  float gamma;                      // its norm
  uint4 v[MQShape<D, B>::KPT];         // V rows kg + KGS i, 8 dims each
};

// Loads of tile t by staging thread stid (rows past n_keys read the last
// key; they are masked later).  The waves of a key half all load the half's
// words (the same lines).
template <int D, int B>
__device__ __forceinline__ void mq_load(const MQArgs& a, int64_t seq, int64_t t, int stid, int vp,
                                        MQStage<D, B>& st) {
  using S = MQShape<D, B>;
  constexpr int W = Codec<D, B>::W;
  const int lane = stid & 63, sw = stid >> 6;
  const int64_t tiles64 = a.cap / kTile;
  int64_t key = t * S::KT + 64 * (sw / S::PARTS) + lane;
  key = key < a.n_keys ? key : a.n_keys - 1;
  TileWords<W>::load(a.packed + (seq * tiles64 + (key >> 6)) * W * kTile, (int)(key & 63), st.words);
  st.gamma = a.gamma[seq * a.cap + key];
  const int c = stid % (S::DV / 8), kg = stid / (S::DV / 8);
  const uint4* vseq = (const uint4*)a.v + seq * a.cap * (D / 8) + vp * (S::DV / 8) + c;
#pragma unroll
  for (int i = 0; i < S::KPT; ++i) {
    int64_t kv = t * S::KT + kg + S::KGS * i;
    kv = kv < a.n_keys ? kv : a.n_keys - 1;
    st.v[i] = vseq[kv * (D / 8)];
  }
}

// max / sum of x over the lane pair (l, l ^ 32): v_permlane32_swap exchanges
// the two halves of the wavefront without a trip through the LDS
// (lane l < 32 finds its partner's value in the second result, lane l >= 32
// in the first; the other result is its own)
__device__ __forceinline__ float pair32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Transposing LDS read of 4 fp16 (ds_read_b64_tr_b16; the lane layout is
// described where the P.V operands are read).
typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 fp16x4_tr;
__device__ __forceinline__ half4 read_tr16(const unsigned char* p) {
  typedef __attribute__((address_space(3))) fp16x4_tr lds_fp16x4;
  return __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                                       (lds_fp16x4*)(const_cast<unsigned char*>(p))));
}

// bf16 pair -> f16 pair (V of the multi-query path must lie in fp16 range).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w << 16),
                                                                 __uint_as_float(w & 0xffff0000u)));
}

// Dims [PART DQ, (PART + 1) DQ) of the lane's rebuilt key gs u'^ (u'^ = rho^ n^
// per triplet, gs = gamma 2^-e, 0 for a row past the cache), from the
// triplets that touch them, to the key's fp16 row in LDS.
template <int D, int B, int PART>
__device__ __forceinline__ void mq_rebuild(const MQStage<D, B>& st, float gs, const float4* s_dir,
                                           const float* s_rho, unsigned char* krow) {
  using C = Codec<D, B>;
  constexpr int DQ = MQShape<D, B>::DQ, LO = PART * DQ, HI = LO + DQ;
  float u[DQ];
#pragma unroll
  for (int i = LO / 3; i <= (HI - 1) / 3; ++i) {
    const uint32_t code = field_at<C::W>(st.words, i * C::BT, C::BT);
    const float4 n = s_dir[code & C::DIR_MASK];
    const float rh = gs * s_rho[code >> (C::BX + C::BE)];
    const float t3[3] = {rh * n.x, rh * n.y, rh * n.z};
#pragma unroll
    for (int c = 0; c < 3; ++c)
      if (3 * i + c >= LO && 3 * i + c < HI) u[3 * i + c - LO] = t3[c];
  }
  // round to nearest: truncation would shrink every score by about 2^-12 on
  // average, an error that grows with the score's magnitude
  uint4* row = (uint4*)(krow + LO * 2);
#pragma unroll
  for (int j = 0; j < DQ / 8; ++j) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = __builtin_bit_cast(uint32_t, half2v{(_Float16)u[8 * j + 2 * e], (_Float16)u[8 * j + 2 * e + 1]});
    row[j] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// mq_rebuild of dim part `part` (wave-uniform), one of P .. PARTS - 1.
template <int D, int B, int P>
__device__ __forceinline__ void mq_rebuild_from(int part, const MQStage<D, B>& st, float gs,
                                                const float4* s_dir, const float* s_rho,
                                                unsigned char* krow) {
  if constexpr (P == MQShape<D, B>::PARTS - 1) {
    if (P > 1 || part == P) mq_rebuild<D, B, P>(st, gs, s_dir, s_rho, krow);
  } else {
    if (part == P) mq_rebuild<D, B, P>(st, gs, s_dir, s_rho, krow);
    else mq_rebuild_from<D, B, P + 1>(part, st, gs, s_dir, s_rho, krow);
  }
}

template <int D, int B>
__global__ __launch_bounds__((64 * MQShape<D, B>::NW)) void k_mq_attn(MQArgs a) {
  using C = Codec<D, B>;
  using S = MQShape<D, B>;
  constexpr int T = C::T;
  constexpr int KT = S::KT, KP = S::KP, VR = S::VR, NTH = 64 * S::NW;
  constexpr int NKS = D / 16;  // MFMA K-steps over the head dim
  constexpr int NMB = S::DV / 32;  // 32-row blocks of O^T

  // two sets of tile buffers: tile t + 1 is staged while tile t is computed
  __shared__ __align__(16) unsigned char s_k[2][KT * KP];
  __shared__ __align__(16) unsigned char s_v[2][KT * VR];
  __shared__ int s_e[2][KT / 64];   // the exponent e of each 64-key half
  // unit directions in LDS, except at d = 256, b = 5, where the 4096-entry
  // table (64 KiB) does not fit beside the tiles: the rebuild then reads it
  // from global memory (L2-resident)
  constexpr bool DIR_LDS = !(D == 256 && B == 5);
  __shared__ float4 s_dir[DIR_LDS ? C::NDIR : 1];
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

  static_assert(TableCopy<C::NDIR, NTH>::SLOTS <= C::NDIR && C::LR <= NTH, "table copies in bounds");
  const float4* dirp;
  if constexpr (DIR_LDS) {
    for (int i = tid; i < C::NDIR; i += NTH) s_dir[i] = a.t.dirtab[i];
    dirp = s_dir;
  } else {
    dirp = a.t.dirtab;
  }
  if (tid < C::LR) s_rho[tid] = a.t.rho_tab[tid];

  // Q' fragment: B[k = dim][n = query], lane (ln, g) holds dims 16j + 8g + 0..7.
  half8 qf[NKS];
  int qsh;   // queries held as q' 2^qsh
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
    amax = pair32_max(amax);
    int ex = 0;
    __builtin_frexpf(amax, &ex);
    const int sh = amax > 0.f ? 7 - ex : 0;   // row max into [64, 128)
    const float sc = __builtin_ldexpf(1.0f, sh);
    qsh = sh;
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
  const int split = blockIdx.x / S::NVP, vp = blockIdx.x % S::NVP;   // (uniform)
  const int64_t t_begin = (int64_t)split * a.tiles_per_split;
  const int64_t t_end = t_begin + a.tiles_per_split < ntile ? t_begin + a.tiles_per_split : ntile;
  constexpr int KPT = S::KPT;

  // Stage one tile from the registers of its loads into LDS buffer set bs:
  //   keys rebuilt by wave w for key half w / 4 and dim quarter w % 4;
  //   V rows as fp16, this thread's 8 dims of keys kg + KGS i.
  MQStage<D, B> st;
  auto stage = [&](int64_t k0, int bs) {
    {
      const int sw = stid >> 6;
      const int kk = 64 * (sw / S::PARTS) + lane;
      const bool ok = k0 + kk < a.n_keys;
      unsigned char* krow = s_k[bs] + kk * KP;
      const int part = sw % S::PARTS;
      // the half's exponent e: its largest gamma times 2^-e lies in [1/2, 1)
      // (every wave of the half computes the same value; clamped so that
      // 2^-e and 2^e are normal floats)
      const float gk = ok ? st.gamma : 0.f;
      int e = 0;
      __builtin_frexpf(wave_max(gk), &e);
      e = e < -126 ? -126 : (e > 126 ? 126 : e);
      const float gs = gk * __builtin_ldexpf(1.0f, -e);
      if (part == 0) {
        mq_rebuild<D, B, 0>(st, gs, dirp, s_rho, krow);
        if (lane == 0) s_e[bs][sw / S::PARTS] = e;
      } else {
        mq_rebuild_from<D, B, 1>(part, st, gs, dirp, s_rho, krow);
      }
    }
    const int c = stid % (S::DV / 8), kg = stid / (S::DV / 8);
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int key = kg + S::KGS * i;
      const bool ok = k0 + key < a.n_keys;
      const uint32_t src[4] = {st.v[i].x, st.v[i].y, st.v[i].z, st.v[i].w};
      uint32_t hv[4];   // f16 pairs (dims 2e, 2e+1)
#pragma unroll
      for (int e = 0; e < 4; ++e) hv[e] = ok ? bf16x2_to_f16x2(src[e]) : 0u;
      *(uint4*)(s_v[bs] + key * VR + ((16 * c) ^ (vswz<S::DV>(key) << 6))) = make_uint4(hv[0], hv[1], hv[2], hv[3]);
    }
  };

  if (stager) mq_load<D, B>(a, seq, t_begin < ntile ? t_begin : 0, stid, vp, st);
  __syncthreads();  // s_dir / s_rho
  if (stager && t_begin < t_end) {
    stage(t_begin * KT, 0);
    mq_load<D, B>(a, seq, t_begin + 1 < t_end ? t_begin + 1 : t_begin, stid, vp, st);
  }
  __syncthreads();

  // P.V operands by transposing reads (ds_read_b64_tr_b16: in each group of
  // 16 lanes, lane i receives element i % 4 of the 8 bytes that lanes
  // i / 4 + 4 k, k = 0..3, name).  Lane j of a group names V row 4 g + j / 4
  // of the chunk's 16-key half, dims 32 mb + 16 (ln / 16) + 4 (j % 4) ..
  // + 3, so lane (ln, g) receives dim 32 mb + ln of keys 4 g + 0..3, the
  // order P^T's registers hold them in (and keys + 8 from the row 8 below).
  int voff[NMB];
  {
    const int jt = lane & 15;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      voff[mb] = (4 * g + (jt >> 2)) * VR +
                 ((64 * mb + 32 * (ln >> 4) + 8 * (jt & 3)) ^ (vswz<S::DV>(jt >> 2) << 6));
  }

  for (int64_t t = t_begin; t < t_end; ++t) {
    const int64_t k0 = t * KT;
    const int cb = (int)((t - t_begin) & 1);
    // stage the next tile into the other buffer set (its last reader, the
    // previous tile's matrix work, finished before the last barrier), then
    // request the tile after it
    if (stager && t + 1 < t_end) {
      stage(k0 + KT, cb ^ 1);
      mq_load<D, B>(a, seq, t + 2 < t_end ? t + 2 : t + 1, stid, vp, st);
    }
    const unsigned char* sk = s_k[cb];
    const unsigned char* svt = s_v[cb];
    if (wave_q) {
    // 3. 64 keys (one half) at a time: S^T, online softmax, O^T += V^T P^T.
    // The accumulators hold s' = q'.(gamma 2^-e u'^) 2^qsh, so the score in
    // log2 units is s' 2^(e - qsh): one factor per half, folded into the
    // fma of the exponent.
    const bool partial = k0 + KT > a.n_keys;
#pragma unroll 1
    for (int ch = 0; ch < KT / 64; ++ch) {
      int ce = s_e[cb][ch] - qsh;
      ce = ce < -126 ? -126 : (ce > 127 ? 127 : ce);   // a normal, nonzero factor
      const float cs = __builtin_ldexpf(1.0f, ce);
      floatx16 s[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[sb][r] = 0.f;
      // the two 32-key blocks' chains interleaved: each MFMA's result is not
      // needed by the next one issued
#pragma unroll
      for (int j = 0; j < NKS; ++j)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const half8 kf = *(const half8*)(sk + (ch * 64 + sb * 32 + ln) * KP + (16 * j + 8 * g) * 2);
          s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[j], s[sb], 0, 0, 0);
        }
      // register r holds key row ch 64 + sb 32 + 8 (r / 4) + 4 g + r % 4
      if (partial) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (k0 + ch * 64 + sb * 32 + 8 * (r >> 2) + 4 * g + (r & 3) >= a.n_keys) s[sb][r] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sb][r]);
      mx = pair32_max(mx) * cs;
      // Lazily raised reference m (log2 units, one per query): raised to the
      // chunk's maximum, with l and o rescaled, only when a score exceeds it
      // by more than kLazyLog2 (any lane of the wave), so p = 2^(s - m) <=
      // 2^kLazyLog2, far inside fp16.  After the first chunk a raise is rare.
      constexpr float kLazyLog2 = 8.f;
      if (__any(mx > m_run + kLazyLog2)) {
        const float m_new = fmaxf(m_run, mx);
        // a row with no valid key yet keeps m = -inf (alpha is then moot)
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[mb][r] *= alpha;
        m_run = m_new;
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      float lsum = 0.f;
      half8 pf[2][2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          pf[sb][r >> 3][r & 7] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][r], cs, -m_use));
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
      l_run += lsum;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int kbase = ch * 64 + sb * 32 + 16 * half + 4 * g;
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) {
            const unsigned char* vp = svt + (kbase - 4 * g) * VR + voff[mb];
            const half4 lo = read_tr16(vp);
            const half4 hi = read_tr16(vp + 8 * VR);
            const half8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[sb][half], o[mb], 0, 0, 0);
          }
        }
      }
    }
    }  // wave_q
    __syncthreads();  // this tile's buffers are free, the next tile's staged
  }

  l_run = pair32_sum(l_run);
  if (qvalid) {
    float* dst = a.part + (((int64_t)bh * a.n_q + q) * a.n_split + split) * (D + 2);
    if (g == 0 && vp == 0) {
      dst[0] = m_run;
      dst[1] = l_run;
    }
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[2 + vp * S::DV + 32 * mb + 8 * (r >> 2) + 4 * g + (r & 3)] = o[mb][r];
  }
}

template <int D, int B>
static hipError_t mq_t(const MQArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.n_split * MQShape<D, B>::NVP),
                  (unsigned)((a.n_q + kMQQueries - 1) / kMQQueries), (unsigned)(a.B * a.H));
  hipLaunchKernelGGL((k_mq_attn<D, B>), grid, dim3((64 * MQShape<D, B>::NW)), 0, s, a);
  return hipGetLastError();
}

// LDS table copies of k_mq_attn<D, B>: unit directions and rho centroids.
template <int D, int B>
static int mq_copy_recs(LdsCopyRec* out, int n, int max) {
  using C = Codec<D, B>;
  constexpr int NTH = 64 * MQShape<D, B>::NW;
  using TC = TableCopy<C::NDIR, NTH>;
  if (n < max && !(D == 256 && B == 5))   // (d = 256, b = 5: no LDS copy of the directions)
    out[n++] = {"k_mq_attn", D, B, 0, TAB_DIR, C::NDIR, TC::SLOTS, TC::ENTRIES, C::NDIR, NTH, TC::MASKED};
  if (n < max) out[n++] = {"k_mq_attn", D, B, 0, TAB_RHO, C::LR, C::LR, C::LR, C::LR, NTH, C::LR % NTH != 0};
  return n;
}

int lds_copies_mq(LdsCopyRec* out, int max) {
  int n = 0;
  n = mq_copy_recs<64, 1>(out, n, max);
  n = mq_copy_recs<64, 2>(out, n, max);
  n = mq_copy_recs<64, 3>(out, n, max);
  n = mq_copy_recs<64, 4>(out, n, max);
  n = mq_copy_recs<64, 5>(out, n, max);
  n = mq_copy_recs<128, 1>(out, n, max);
  n = mq_copy_recs<128, 2>(out, n, max);
  n = mq_copy_recs<128, 3>(out, n, max);
  n = mq_copy_recs<128, 4>(out, n, max);
  n = mq_copy_recs<128, 5>(out, n, max);
  n = mq_copy_recs<256, 1>(out, n, max);
  n = mq_copy_recs<256, 2>(out, n, max);
  n = mq_copy_recs<256, 3>(out, n, max);
  n = mq_copy_recs<256, 4>(out, n, max);
  n = mq_copy_recs<256, 5>(out, n, max);
  return n;
}

int mq_tile_keys(int d, int b) {
  if (d == 64) return MQShape<64, 1>::KT;
  if (d == 256) return MQShape<256, 1>::KT;
  return b == 5 ? MQShape<128, 5>::KT : MQShape<128, 1>::KT;
}
int mq_value_parts(int d) { return d == 256 ? MQShape<256, 1>::NVP : 1; }
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
    case 1285: return mq_t<128, 5>(a, s);
    case 2561: return mq_t<256, 1>(a, s);
    case 2562: return mq_t<256, 2>(a, s);
    case 2563: return mq_t<256, 3>(a, s);
    case 2564: return mq_t<256, 4>(a, s);
    case 2565: return mq_t<256, 5>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace octo

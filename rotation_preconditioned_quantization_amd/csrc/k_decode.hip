// OCTOPUS fused decode kernels for gfx950 ([YL] 工程实现: keys are rebuilt from
// the packed indices in registers, never written out; q.k, then online
// softmax and P.V, FlashAttention-style tiling).
//
//   k_rotate     q' = mult * R q per query row ([YL] 旋转魔法: R orthogonal, so
//                <q, k^> = gamma <R q, u'^> and keys are never inverse-rotated),
//                for the multi-query kernel; the single-query kernels rotate
//                their own heads in the prologue (with QJL also p = kappa
//                * S q', [YL] 可选的残差修正).
//   k_logits     one wavefront per 64-key tile, one key per lane: unpack the
//                word-major tile (coalesced), rebuild rho^ n^ per triplet from
//                LDS tables, contract with 4 query heads on fp32 MFMA.
//   k_attn       the same per-key logits, then a wave-wide online softmax and
//                P.V over bf16 V (one coalesced row per load, fp32 MFMA),
//                split-K over the sequence; k_combine merges the splits.
//   k_reconstruct  test helper writing k^ = gamma R^T u'^.
#include <type_traits>

#include "octo_device.hpp"
#include "octo_encode_dev.hpp"

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
  // strides 64, 128: between the values a lane holds
#pragma unroll
  for (int hr = 1; hr < NV; hr <<= 1) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if (k & hr) continue;
      const float a0 = x[k], a1 = x[k + hr];
      x[k] = a0 + a1;
      x[k + hr] = a0 - a1;
    }
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
    float acc[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) acc[k] = 0.f;
#pragma unroll 8
    for (int c = 0; c < D; ++c) {
      const float qc = s_q[c];
      const float* col = a.t.St + (int64_t)c * D + l;   // coalesced column of S
#pragma unroll
      for (int k = 0; k < NV; ++k) acc[k] = __builtin_fmaf(col[64 * k], qc, acc[k]);
    }
#pragma unroll
    for (int k = 0; k < NV; ++k)
      a.qp[(int64_t)orow * D + l + 64 * k] = acc[k] * a.t.qjl_kappa;
  }
}

typedef float floatx4 __attribute__((ext_vector_type(4)));

// LDS of the single-query kernels.  kCombined: for up to 10 bits per triplet
// one float4 per triplet code holds rho^ n^ directly; otherwise unit
// directions per (i_xi, i_eta) plus the rho centroids.  REP (up to 10 bits per
// triplet): the combined table is held in NCOPY copies (as many as fit
// 128 KiB, at most 16), entry e of copy c at float4 slot NCOPY e + c, and lane
// l reads copy l % NCOPY.  The LDS serves 16 lanes per pass; with 16 copies
// they hit 16 different 4-bank groups whatever codes they look up, so random
// gathers are conflict-free (4 LDS cycles per wavefront read instead of about
// 11); with 8 copies (the 1024-entry table at 3 bits) only the 2 lanes of a
// copy can collide (8 copies measured 3.5 % faster than 4 in the logits
// kernel at 3 bits + QJL, whose LDS is busy most of the time).  q holds the rotated queries of the (up to) 4 heads of
// this pass, rows padded with zeros; with QJL, qp holds p = kappa S q'
// and lut its nibble sums.
template <int D, int B, bool QJL, bool REP>
struct SQShared {
  using C = Codec<D, B>;
  static_assert(!REP || C::BT <= 10, "replicated table needs the combined table");
  static constexpr bool kCombined = C::BT <= 10;
  static constexpr int NENT = kCombined ? (1 << C::BT) : C::NDIR;
  static constexpr int NCOPY = !REP ? 1 : (8192 / NENT < 16 ? 8192 / NENT : 16);
  static constexpr int QD = ((3 * C::T + 15) / 16) * 16;   // whole 16-dim groups (QRegs)
  // the nibble table first: its per-lookup offsets then fit the 16-bit
  // offset field of ds_read (no address add per lookup)
  float4 lut[QJL ? (D / 4) * 16 : 1];
  float4 tab[NENT * NCOPY];
  float rho[C::LR];
  float q[4][QD];
  float qp[QJL ? 4 : 1][QJL ? D : 1];
};

// The copy of a single-query kernel's code table into LDS by NTH threads.
template <int D, int B, bool QJL, bool REP, int NTH>
using SQTableCopy = TableCopy<SQShared<D, B, QJL, REP>::NENT * SQShared<D, B, QJL, REP>::NCOPY, NTH,
                              SQShared<D, B, QJL, REP>::NCOPY>;

// Replicated code table in k_logits (B <= 3) and in k_attn (B <= 2: at b = 3
// and 4 it measured no faster there).
template <int B>
constexpr bool logits_rep() { return B <= 3; }
template <int B>
constexpr bool attn_rep() { return B <= 2; }

// Waves per k_logits block: with the replicated table (B <= 3) 16 at 3 bits
// (its 128 KiB of copies allow one block per CU) and 8 below (two blocks per
// CU), else 4; always 4 waves per SIMD.
template <int B>
constexpr int logits_waves() { return !logits_rep<B>() ? 4 : (B == 3 ? 16 : 8); }

// Values the block prologue loads from global memory besides the LDS tables
// (which go to LDS directly): wave w's query head g0 + w (lane l holds the
// 32-bit words of elements l + 64 k) and the rho centroids.
template <int D, int B, bool QJL, bool REP>
struct SQPre {
  float rho;
  uint32_t qw[D / 64];
};

template <int D, int B, bool QJL, bool REP, int NTH = 256>
__device__ __forceinline__ void sq_issue_prologue(const DecodeArgs& a, int64_t seq, int g0,
                                                  int hcount, SQPre<D, B, QJL, REP>& pre,
                                                  SQShared<D, B, QJL, REP>& sh) {
  using C = Codec<D, B>;
  using SH = SQShared<D, B, QJL, REP>;
  using TC = SQTableCopy<D, B, QJL, REP, NTH>;
  static_assert(TC::SLOTS <= SH::NENT * SH::NCOPY && TC::ENTRIES <= SH::NENT,
                "the table copy stays inside the LDS table and the source table");
  static_assert(C::LR <= NTH, "one rho centroid per thread");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float4* src = SH::kCombined ? a.t.trip_tab : a.t.dirtab;
  // the table goes straight from global memory into LDS (no registers held);
  // slot i holds entry i / NCOPY.  The condition is per lane: a table of
  // fewer slots than threads (16 at one bit) is copied by the first lanes
  // only, and the others neither read past its end nor write past it in LDS.
#pragma unroll
  for (int k = 0; k < TC::ROUNDS; ++k) {
    const int i0 = NTH * k + 64 * w;  // this wave's 64 slots of round k
    if (!TC::MASKED || i0 + lane < SH::NENT * SH::NCOPY)
      __builtin_amdgcn_global_load_lds((const void*)(src + (i0 + lane) / SH::NCOPY),
                                       (__attribute__((address_space(3))) void*)(sh.tab + i0), 16,
                                       0, 0);
  }
  if (tid < C::LR) pre.rho = a.t.rho_tab[tid];
  // one 32-bit load per element whatever the dtype (the word holding a
  // 16-bit element), decoded by selects: no branch between these loads and
  // the tile loads that follow
  const int wq = w < hcount ? w : 0;
  const int64_t bidx = seq / a.Hkv, kvh = seq % a.Hkv;
  const int64_t r = bidx * a.Hq + kvh * a.G + g0 + wq;
  const int esz = a.qdt == DT_F32 ? 4 : 2;
  const unsigned char* qrow = (const unsigned char*)a.q + r * D * esz;
#pragma unroll
  for (int k = 0; k < D / 64; ++k) {
    const int j = lane + 64 * k;
    pre.qw[k] = *(const uint32_t*)(qrow + ((j * esz) & ~3));
  }
}

// Element l + 64 k of the wave's query from the raw words of sq_issue_prologue.
template <int D, int B, bool QJL, bool REP>
__device__ __forceinline__ float sq_query_elem(const DecodeArgs& a, const SQPre<D, B, QJL, REP>& pre,
                                               int k, int lane) {
  const uint32_t wd = pre.qw[k];
  const uint32_t h16 = (lane & 1) ? (wd >> 16) : (wd & 0xffffu);
  const float fb = __uint_as_float(h16 << 16);
  const float fh = __half2float(__ushort_as_half((unsigned short)h16));
  return a.qdt == DT_F32 ? __uint_as_float(wd) : (a.qdt == DT_BF16 ? fb : fh);
}

// Query rotation (q' = mult * R q, R = d^-1/2 H diag(s)): butterflies of
// stride < 64 pair lanes (shuffles), strides 64, 128 pair a lane's values.
// With QJL the wave also forms p = kappa * S q' (kappa: the estimator
// constant of the residual rotation S).
template <int D, int B, bool QJL, bool REP>
__device__ __forceinline__ void rotate_head(const DecodeArgs& a, int hcount,
                                            const SQPre<D, B, QJL, REP>& pre, SQShared<D, B, QJL, REP>& sh) {
  using SH = SQShared<D, B, QJL, REP>;
  constexpr int NV = D / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (w >= 4) return;   // blocks of more than 4 waves: the others only stream tiles
  // branch-free: a wave past hcount rotates a valid head and stores zeros
  const bool live = w < hcount;
  float x[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int j = lane + 64 * k;
    const float qv = sq_query_elem<D, B, QJL, REP>(a, pre, k, lane);
    const uint32_t sb = (lane < 32) ? a.t.sign_bits[2 * k] : a.t.sign_bits[2 * k + 1];
    x[k] = ((sb >> (j & 31)) & 1u) ? -qv : qv;
  }
#pragma unroll
  for (int hh = 1; hh < 64; hh <<= 1) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const float o = __shfl_xor(x[k], hh, 64);
      x[k] = (lane & hh) ? (o - x[k]) : (x[k] + o);
    }
  }
#pragma unroll
  for (int hr = 1; hr < NV; hr <<= 1) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if (k & hr) continue;
      const float a0 = x[k], a1 = x[k + hr];
      x[k] = a0 + a1;
      x[k + hr] = a0 - a1;
    }
  }
  const float mult = a.mult * rsqrtf((float)D);
#pragma unroll
  for (int k = 0; k < NV; ++k) sh.q[w][lane + 64 * k] = live ? x[k] * mult : 0.f;
  if (lane < SH::QD - D) sh.q[w][D + lane] = 0.f;
  if constexpr (QJL) {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    // p_j = sum_c S[j][c] q'_c: lane j reads element j of column c, so every
    // load is one contiguous row of St
    float acc[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) acc[k] = 0.f;
#pragma unroll 8
    for (int c = 0; c < D; ++c) {
      const float qc = sh.q[w][c];
      const float* col = a.t.St + (int64_t)c * D + lane;
#pragma unroll
      for (int k = 0; k < NV; ++k) acc[k] = __builtin_fmaf(col[64 * k], qc, acc[k]);
    }
#pragma unroll
    for (int k = 0; k < NV; ++k)
      sh.qp[w][lane + 64 * k] = live ? acc[k] * a.t.qjl_kappa : 0.f;
  }
}

template <int D, int B, bool QJL, bool REP>
__device__ __forceinline__ void store_sq_tables(const SQPre<D, B, QJL, REP>& pre,
                                                SQShared<D, B, QJL, REP>& sh) {
  using C = Codec<D, B>;
  if (threadIdx.x < C::LR) sh.rho[threadIdx.x] = pre.rho;
}

// QJL nibble table: lut[m][nib] holds, per head, sum_k (+1 if bit k of nib
// else -1) * p[4m + k].
template <int D, int B, bool QJL, bool REP>
__device__ __forceinline__ void build_qjl_lut(int hcount, SQShared<D, B, QJL, REP>& sh) {
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

// The rotated queries of the (up to) 4 heads in registers, in the layout the
// broadcast form of v_mfma_f32_4x4x1_16b_f32 reads: register r of lane
// 4 b + h holds q'[h][16 r + b], so one register carries 16 dims of all 4
// heads, and the MFMA with CBSZ = 4 (groups of 16 blocks) and ABID = j feeds
// block j's 4 values (dim 16 r + j) to all 16 blocks as the A operand.
template <int D, int B, bool QJL, bool REP>
struct QRegs {
  static constexpr int N = SQShared<D, B, QJL, REP>::QD / 16;
  float v[N];
};

template <int D, int B, bool QJL, bool REP>
__device__ __forceinline__ void load_qregs(const SQShared<D, B, QJL, REP>& sh, int lane,
                                           QRegs<D, B, QJL, REP>& qr) {
#pragma unroll
  for (int r = 0; r < QRegs<D, B, QJL, REP>::N; ++r) qr.v[r] = sh.q[lane & 3][16 * r + (lane >> 2)];
}

// f(std::integral_constant<int, I>) for I = I0 .. N-1, as straight-line code:
// the index is a constant expression in f (the MFMA broadcast controls must be).
template <int I0, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I0 < N) {
    f(std::integral_constant<int, I0>{});
    static_for<I0 + 1, N>(f);
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
  TileWords<W>::load(a.packed + (seq * tiles + t) * W * kTile, lane, k.words);
  const int64_t key = t * kTile + lane;   // < cap: in bounds (masked by the caller)
  k.gamma = a.gamma[seq * a.cap + key];
  if constexpr (QJL) {
    TileWords<D / 32>::load(a.qjl_bits + (seq * tiles + t) * (D / 32) * kTile, lane, k.sw);
    k.nu = __half2float(__ushort_as_half(a.qjl_norm[seq * a.cap + key]));
  }
}

// Logits of a 64-key tile, one key per lane, for 4 query heads at once:
// returns acc[h] = <q'_h, u'^_key> (+ the QJL term).  The contraction over
// the rotated dims runs on v_mfma_f32_4x4x1_16b_f32: in every 4-lane block
// the A operand is q'[head][dim] for the 4 heads (broadcast from the query
// registers, QRegs, or read from LDS beside the direction table) and the B
// operand is the lane's own rebuilt coordinate, so block b produces the 4 x 4
// outer product for keys 4b..4b+3 and lane l ends up holding the 4 heads of
// key l.  Exact fp32.
template <int D, int B, bool QJL, bool REP>
__device__ __forceinline__ floatx4 tile_logits(const SQShared<D, B, QJL, REP>& sh,
                                               const QRegs<D, B, QJL, REP>& qr,
                                               const KTile<D, B, QJL>& k, int lane) {
  using C = Codec<D, B>;
  using SH = SQShared<D, B, QJL, REP>;
  constexpr int T = C::T, W = C::W;
  constexpr int kGroup = 4;
  const float4* tab = sh.tab + (SH::NCOPY > 1 ? (lane & (SH::NCOPY - 1)) : 0);  // this lane's copy
  // two accumulator sets (even / odd triplets): the dependent-MFMA latency
  // then hides behind the other set's issue
  floatx4 acc[6];
#pragma unroll
  for (int c = 0; c < 6; ++c) acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};
  if constexpr (SH::kCombined) {
    // up to 10 bits per triplet: one table read per triplet, the queries from
    // registers (straight-line code: the broadcast controls are constants)
    static_for<0, T>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const uint32_t code = field_at<W>(k.words, i * C::BT, C::BT);
      const float4 e = tab[code * SH::NCOPY];
      // A: block (3i + c) % 16 of query register (3i + c) / 16, broadcast
      acc[3 * (i & 1)] = __builtin_amdgcn_mfma_f32_4x4x1f32(qr.v[(3 * i) >> 4], e.x, acc[3 * (i & 1)], 4,
                                                            (3 * i) & 15, 0);
      acc[3 * (i & 1) + 1] = __builtin_amdgcn_mfma_f32_4x4x1f32(qr.v[(3 * i + 1) >> 4], e.y,
                                                                acc[3 * (i & 1) + 1], 4, (3 * i + 1) & 15, 0);
      acc[3 * (i & 1) + 2] = __builtin_amdgcn_mfma_f32_4x4x1f32(qr.v[(3 * i + 2) >> 4], e.z,
                                                                acc[3 * (i & 1) + 2], 4, (3 * i + 2) & 15, 0);
      // a few triplets at a time: keeps the LDS gathers from all being hoisted
      if constexpr (i % kGroup == kGroup - 1) asm volatile("" ::: "memory");
    });
  } else {
    // direction table and rho centroids: the queries from LDS (measured
    // faster than the registers at 13 bits per triplet)
    const float* qrow = sh.q[lane & 3];
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const uint32_t code = field_at<W>(k.words, i * C::BT, C::BT);
      const float4 n = tab[(code & C::DIR_MASK) * SH::NCOPY];
      const float rh = sh.rho[code >> (C::BX + C::BE)];
      const float tv[3] = {rh * n.x, rh * n.y, rh * n.z};
#pragma unroll
      for (int c = 0; c < 3; ++c)
        acc[3 * (i & 1) + c] =
            __builtin_amdgcn_mfma_f32_4x4x1f32(qrow[3 * i + c], tv[c], acc[3 * (i & 1) + c], 0, 0, 0);
      if (i % kGroup == kGroup - 1) asm volatile("" ::: "memory");
    }
  }
  floatx4 r = (acc[0] + acc[3]) + (acc[1] + acc[4]) + (acc[2] + acc[5]);
  if constexpr (QJL) {
    float4 corr = sh.lut[k.sw[0] & 15u];   // nibble 0 (no adds to zero)
#pragma unroll
    for (int m = 1; m < D / 4; ++m) {
      const uint32_t nib = (k.sw[m >> 3] >> (4 * (m & 7))) & 15u;
      const float4 e = sh.lut[(m << 4) + nib];
      corr.x += e.x; corr.y += e.y; corr.z += e.z; corr.w += e.w;
      // 8 reads in flight, each group summed before the next is read (the
      // sums are pinned as live values here)
      if (m % 8 == 7)
        asm volatile("" : "+v"(corr.x), "+v"(corr.y), "+v"(corr.z), "+v"(corr.w) : : "memory");
    }
    r[0] = __builtin_fmaf(k.nu, corr.x, r[0]);
    r[1] = __builtin_fmaf(k.nu, corr.y, r[1]);
    r[2] = __builtin_fmaf(k.nu, corr.z, r[2]);
    r[3] = __builtin_fmaf(k.nu, corr.w, r[3]);
  }
  return r;
}

// Second half of the prologue shared by both single-query kernels: rotation,
// tables, barrier (and the QJL nibble table).
template <int D, int B, bool QJL, bool REP>
__device__ __forceinline__ void sq_finish_prologue(const DecodeArgs& a, int hcount,
                                                   const SQPre<D, B, QJL, REP>& pre,
                                                   SQShared<D, B, QJL, REP>& sh) {
  store_sq_tables<D, B, QJL, REP>(pre, sh);
  rotate_head<D, B, QJL, REP>(a, hcount, pre, sh);
  __syncthreads();
  if constexpr (QJL) {
    build_qjl_lut<D, B, QJL, REP>(hcount, sh);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Logits.  grid = (blocks over key tiles, n_seq, ceil(G / 4)); 4 or 8 waves
// (logits_waves), each a stream of 64-key tiles.
// ---------------------------------------------------------------------------
template <int D, int B, bool QJL>
__global__ __launch_bounds__(64 * logits_waves<B>())
__attribute__((amdgpu_waves_per_eu(logits_rep<B>() ? 4 : 2))) void k_logits(DecodeArgs a) {
  // replicated table where it fits (few or no gather conflicts), blocks of
  // logits_waves<B>() waves
  constexpr bool REP = logits_rep<B>();
  constexpr int NW = logits_waves<B>();
  __shared__ SQShared<D, B, QJL, REP> sh;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t seq = blockIdx.y;
  const int g0 = blockIdx.z * 4;
  const int hcount = a.G - g0 < 4 ? a.G - g0 : 4;
  const int64_t ntile = (a.n_keys + kTile - 1) / kTile;
  if (ntile == 0) return;
  const int64_t stride = (int64_t)gridDim.x * NW;
  int64_t t = (int64_t)blockIdx.x * NW + wave;
  SQPre<D, B, QJL, REP> pre;
  sq_issue_prologue<D, B, QJL, REP, 64 * NW>(a, seq, g0, hcount, pre, sh);
  sq_finish_prologue<D, B, QJL, REP>(a, hcount, pre, sh);
  QRegs<D, B, QJL, REP> qr;
  load_qregs<D, B, QJL, REP>(sh, lane, qr);
  // One tile at a time.  The kernel is bound by instruction issue and
  // latency (the 4x4x1 MFMAs, the code extraction, the table gathers), and
  // 16 waves per CU hide the load latency: loading a tile ahead measured no
  // faster (with the queries in registers) or slower (without).
  const int64_t bidx = seq / a.Hkv, kvh = seq % a.Hkv;
  for (; t < ntile; t += stride) {
    KTile<D, B, QJL> kt;
    load_ktile<D, B, QJL>(a, seq, t, lane, kt);
    const floatx4 acc = tile_logits<D, B, QJL, REP>(sh, qr, kt, lane);
    const float gamma = kt.gamma;
    const int64_t key = t * kTile + lane;
    if (key < a.n_keys) {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if (h < hcount) {
          const int64_t hq = kvh * a.G + g0 + h;
          a.logits[(bidx * a.Hq + hq) * a.n_keys + key] = gamma * acc[h];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Single-query split-K attention.  grid = (n_split x value parts, n_seq,
// ceil(G / 4)), 4 waves per block; wave w takes tiles t_begin + w, + 4, ... of the block's
// split, with the next tile (V rows and compressed words) in flight while
// the current one is computed.  Per tile: logits by tile_logits, a wave-wide
// online softmax per head (DPP max), then O[head][dim] += p[head][key]
// V[key][dim] on v_mfma_f32_4x4x4_16b_bf16.  V is read with 16-byte loads:
// lane l takes the 8 dims 8c .. 8c+7 (c = l % (d/8)) of keys KPL j + l/(d/8)
// (KPL = 512/d keys per wave load), so after 4 loads a lane holds 4 keys of
// each of its 8 dims: byte permutes turn them into the B operands (4 keys x
// 1 dim, bf16 exactly as stored).  Every 4-lane MFMA block shares its 4 keys;
// the A operand is p[head = lane % 4][those keys], split into bf16 high and
// low parts (p = hi + lo to 16 bits) and fed as two MFMAs.  Lanes serving
// different keys hold partial sums of the same dims, added at the end.  The
// block merges its 4 waves into one (m, l, o) partial per head (m in log2
// units); k_combine merges the splits.
// ---------------------------------------------------------------------------
// A block handles DV of the D value dims (DV = D up to 128; at d = 256 two
// blocks take a half each, so the V tile in flight stays at 64 registers).
template <int D>
struct VGeom {
  static constexpr int DV = D > 128 ? 128 : D;
  static constexpr int NVH = D / DV;       // value parts (blocks per head group)
  static constexpr int CPR = DV / 8;       // 16-byte chunks of a V row per block
  static constexpr int RP = D / 8;         // V row pitch in chunks
  static constexpr int KPL = 64 / CPR;     // keys per wavefront load
  static constexpr int NVL = kTile / KPL;  // loads per 64-key tile
};

// The block's part of the V rows of a 64-key tile.  V holds cap rows per
// sequence and cap is a multiple of 64, so the whole tile is always in
// bounds: the loads carry no conditions (rows past n_keys are zeroed where
// the tile is used).
template <int D>
__device__ __forceinline__ void load_vtile(const uint4* vlane, int64_t t, uint4 (&vv)[VGeom<D>::NVL]) {
  using VG = VGeom<D>;
  const uint4* vt = vlane + (t * kTile) * VG::RP;
#pragma unroll
  for (int j = 0; j < VG::NVL; ++j) vv[j] = vt[j * VG::KPL * VG::RP];
}

template <int D, int B, bool QJL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_attn(DecodeArgs a) {
  using VG = VGeom<D>;
  constexpr int NVL = VG::NVL;
  // replicated code table where it costs at most 32 KiB (b <= 2): about 1 %
  // at the extreme workload's shape
  constexpr bool REP = attn_rep<B>();
  __shared__ SQShared<D, B, QJL, REP> sh;
  // p of the tile per head, stored so that the 4 keys one MFMA block shares
  // are 4 consecutive floats; padded rows: the 4 heads hit different banks
  __shared__ __align__(16) float s_p[4][4][kTile + 4];
  __shared__ float s_ml[4][4][2];
  __shared__ float s_o[4][4][VG::DV];
  // append step: scratch of the one-wavefront encode and the new key's words
  __shared__ float s_ak[4 * Codec<D, B>::T];
  __shared__ uint32_t s_aw[Codec<D, B>::W];
  __shared__ float s_ag;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t seq = blockIdx.y;
  // the value parts of one split are adjacent blocks, so the second part's
  // reads of the split's code words hit the L2 the first part filled
  const int vh = VG::NVH > 1 ? (int)blockIdx.x % VG::NVH : 0;   // value part of this block
  const int split = VG::NVH > 1 ? (int)blockIdx.x / VG::NVH : (int)blockIdx.x;
  const int g0 = (int)blockIdx.z * 4;
  const int hcount = a.G - g0 < 4 ? a.G - g0 : 4;
  const int kq = lane / VG::CPR;                     // key of the wave load this lane serves
  // slot of this lane's key (= lane) in the p rows: key 4 KPL g + KPL j' + q
  // goes to 4 KPL g + 4 q + j'
  const int p_slot = (lane / (4 * VG::KPL)) * (4 * VG::KPL) + (lane % VG::KPL) * 4 +
                     (lane % (4 * VG::KPL)) / VG::KPL;
  const int64_t ntile = (a.n_keys + kTile - 1) / kTile;
  const int64_t t_begin = (int64_t)split * a.tiles_per_split;
  int64_t t_end = t_begin + a.tiles_per_split;
  if (t_end > ntile) t_end = ntile;
  const uint4* vlane0 = (const uint4*)a.v + kq * VG::RP + vh * VG::CPR + lane % VG::CPR;
  const uint4* vlane = vlane0 + seq * a.cap * VG::RP;

  // The wave's first tile is requested before the prologue (LDS tables by
  // DMA, the query words): the prologue's round trip then overlaps the
  // tile's, and the first LDS access waits for both.  Loads are issued
  // without conditions (a wave with no tile reads tile 0 of sequence 0
  // instead): no control flow between them keeps the compiler's
  // memory-counter waits exact.
  int64_t t = t_begin + wave;
  KTile<D, B, QJL> cur, nxt;
  uint4 vv[NVL];
  const bool any = t < t_end;
  load_ktile<D, B, QJL>(a, any ? seq : 0, any ? t : 0, lane, cur);
  load_vtile<D>(any ? vlane : vlane0, any ? t : 0, vv);
  SQPre<D, B, QJL, REP> pre;
  sq_issue_prologue<D, B, QJL, REP>(a, seq, g0, hcount, pre, sh);
  sq_finish_prologue<D, B, QJL, REP>(a, hcount, pre, sh);
  QRegs<D, B, QJL, REP> qr;
  load_qregs<D, B, QJL, REP>(sh, lane, qr);
  // Decode step with append: the block whose split holds position n_keys - 1
  // encodes the sequence's new key with one wavefront (the same code and
  // rounding as the append encoder), the first head pass writes it to the
  // cache, and the wave that owns the last tile substitutes it for the stale
  // words it loaded.
  const int64_t t_last = (a.n_keys - 1) / kTile;
  bool app = false;
  if constexpr (!QJL) {
    app = a.new_keys != nullptr && t_last >= t_begin && t_last < t_end;
    if (app) {
      if (wave == 0) {
        constexpr int T = Codec<D, B>::T, W = Codec<D, B>::W;
        const void* row = (const unsigned short*)a.new_keys + seq * a.new_key_stride;
        const float g = encode_one_key<D, B, DT_BF16>(row, a.t, a.t.qx.t, a.t.qe.t, a.t.qr2.t, lane,
                                                      s_ak, s_ak + 3 * T, s_aw);
        if (lane == 0) s_ag = g;
        if (blockIdx.z == 0 && vh == 0) {
          if (lane < W) store_key_word<W>(a.packed_w, a.cap, seq, a.n_keys - 1, lane, s_aw[lane]);
          if (lane == 0) a.gamma_w[seq * a.cap + a.n_keys - 1] = g;
        }
      }
      __syncthreads();
    }
  }
  const int new_lane = (int)((a.n_keys - 1) & (kTile - 1));
  auto patch = [&](KTile<D, B, QJL>& kt, int64_t tt) {
    if (app && tt == t_last && lane == new_lane) {
#pragma unroll
      for (int w = 0; w < Codec<D, B>::W; ++w) kt.words[w] = s_aw[w];
      kt.gamma = s_ag;
    }
  };

  float m[4], l[4];
  floatx4 o[8];
#pragma unroll
  for (int h = 0; h < 4; ++h) { m[h] = -INFINITY; l[h] = 0.f; }
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = floatx4{0.f, 0.f, 0.f, 0.f};

  // One tile: logits, online softmax per head, P.V.
  auto process = [&](const KTile<D, B, QJL>& kt, uint4 (&vv)[NVL], int64_t tt) {
    if ((tt + 1) * kTile > a.n_keys) {
      // last, partial tile: rows past n_keys hold arbitrary bits (p is 0 there,
      // but 0 * NaN is not)
#pragma unroll
      for (int j = 0; j < NVL; ++j)
        if (tt * kTile + VG::KPL * j + kq >= a.n_keys) vv[j] = make_uint4(0u, 0u, 0u, 0u);
    }
    const floatx4 acc = tile_logits<D, B, QJL, REP>(sh, qr, kt, lane);
    const int64_t key = tt * kTile + lane;
    const bool valid = key < a.n_keys;
    // Online softmax against a lazily raised reference m (log2 units, one
    // per head and wave): p = 2^(s - m).  m is raised to the wave's maximum,
    // and l and o rescaled, only when a score exceeds it by more than
    // kLazyLog2; p <= 2^kLazyLog2 stays far inside fp32 and its bf16 split.
    // After the first tile a raise is rare, so most tiles skip the max
    // reduction and the rescale.  (m, l, o) stay consistent, which is all
    // the merges of waves and splits need.
    constexpr float kLazyLog2 = 8.f;
    float sc[4];
    bool raise = false;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      sc[h] = valid ? kt.gamma * acc[h] : -INFINITY;
      raise |= sc[h] > m[h] + kLazyLog2;
    }
    if (__any(raise)) {
      float al[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float mn = fmaxf(m[h], wave_max(sc[h]));
        al[h] = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[h] - mn);
        l[h] *= al[h];
        m[h] = mn;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[k][r] *= al[r];
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float p = __builtin_amdgcn_exp2f(sc[h] - m[h]);
      l[h] += p;
      s_p[wave][h][p_slot] = p;
    }
    __builtin_amdgcn_wave_barrier();
    const float* prow = s_p[wave][lane & 3] + 4 * kq;
#pragma unroll
    for (int g = 0; g < NVL / 4; ++g) {
      // A: p of keys 4 KPL g + KPL j' + kq (j' = 0..3) as bf16 hi + lo parts
      const float4 pf = *(const float4*)(prow + 4 * VG::KPL * g);
      const uint32_t u0 = __float_as_uint(pf.x), u1 = __float_as_uint(pf.y);
      const uint32_t u2 = __float_as_uint(pf.z), u3 = __float_as_uint(pf.w);
      const float r0 = pf.x - __uint_as_float(u0 & 0xffff0000u);
      const float r1 = pf.y - __uint_as_float(u1 & 0xffff0000u);
      const float r2 = pf.z - __uint_as_float(u2 & 0xffff0000u);
      const float r3 = pf.w - __uint_as_float(u3 & 0xffff0000u);
      const bf16x4 phi = pack_bf16x4(__builtin_amdgcn_perm(u1, u0, 0x07060302u),
                                     __builtin_amdgcn_perm(u3, u2, 0x07060302u));
      const bf16x4 plo = pack_bf16x4(
          __builtin_amdgcn_perm(__float_as_uint(r1), __float_as_uint(r0), 0x07060302u),
          __builtin_amdgcn_perm(__float_as_uint(r3), __float_as_uint(r2), 0x07060302u));
      const uint4& e0 = vv[4 * g];
      const uint4& e1 = vv[4 * g + 1];
      const uint4& e2 = vv[4 * g + 2];
      const uint4& e3 = vv[4 * g + 3];
      const uint32_t w0[4] = {e0.x, e0.y, e0.z, e0.w}, w1[4] = {e1.x, e1.y, e1.z, e1.w};
      const uint32_t w2[4] = {e2.x, e2.y, e2.z, e2.w}, w3[4] = {e3.x, e3.y, e3.z, e3.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // B: dims 8c + 2k (low halves) and 8c + 2k + 1 (high halves), 4 keys each
        const bf16x4 blo = pack_bf16x4(__builtin_amdgcn_perm(w1[k], w0[k], 0x05040100u),
                                       __builtin_amdgcn_perm(w3[k], w2[k], 0x05040100u));
        const bf16x4 bhi = pack_bf16x4(__builtin_amdgcn_perm(w1[k], w0[k], 0x07060302u),
                                       __builtin_amdgcn_perm(w3[k], w2[k], 0x07060302u));
        o[2 * k] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(phi, blo, o[2 * k], 0, 0, 0);
        o[2 * k + 1] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(phi, bhi, o[2 * k + 1], 0, 0, 0);
        o[2 * k] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(plo, blo, o[2 * k], 0, 0, 0);
        o[2 * k + 1] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(plo, bhi, o[2 * k + 1], 0, 0, 0);
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // The next tile's code words load while this tile's logits are formed; its
  // V rows as soon as this tile's P.V has consumed the V registers.  Other
  // waves on the SIMD cover the remaining latency.  (Loading the next tile's
  // V a tile ahead, half or whole, measured slower: the registers it takes
  // cost spills or the compiler's schedule.)  The last tile is peeled off so
  // that no load is left in flight at the block's final barrier.
  for (; t + 4 < t_end; t += 4) {
    load_ktile<D, B, QJL>(a, seq, t + 4, lane, nxt);
    process(cur, vv, t);
    load_vtile<D>(vlane, t + 4, vv);
    cur = nxt;
  }
  // (the last tile of the cache is always the last one of its wave)
  if (t < t_end) {
    patch(cur, t);
    process(cur, vv, t);
  }

  // lanes serving different keys of a load hold partial sums of the same dims
#pragma unroll
  for (int sft = VG::CPR; sft < 64; sft <<= 1)
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[k][r] += __shfl_xor(o[k][r], sft, 64);
#pragma unroll
  for (int h = 0; h < 4; ++h) l[h] = wave_sum(l[h]);
  if (kq == 0) {
    const int c0 = 8 * (lane % VG::CPR);
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int k = 0; k < 8; ++k) s_o[wave][h][c0 + k] = o[k][h];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < 4; ++h) { s_ml[wave][h][0] = m[h]; s_ml[wave][h][1] = l[h]; }
  }
  __syncthreads();
  // Merge the 4 waves and write this block's partial.
  const int64_t bidx = seq / a.Hkv, kvh = seq % a.Hkv;
  for (int e = threadIdx.x; e < hcount * (VG::DV + 2); e += blockDim.x) {
    const int h = e / (VG::DV + 2), c = e % (VG::DV + 2);
    if (c < 2 && vh > 0) continue;  // (m, l) come from the first value part
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
        const float sc = (s_ml[w][h][0] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s_ml[w][h][0] - M);
        val += sc * (c == 1 ? s_ml[w][h][1] : s_o[w][h][c - 2]);
      }
    }
    const int64_t row = bidx * a.Hq + kvh * a.G + g0 + h;
    const int col = c < 2 ? c : c + vh * VG::DV;
    a.part[(row * a.n_split + split) * (D + 2) + col] = val;
  }
}

// out[row][c] = sum_s 2^(m_s - M) o_s[c] / sum_s 2^(m_s - M) l_s, M = max_s m_s,
// one 256-thread block per row.  Thread t handles the column pair 2 (t % (d/2))
// of the splits s = t / (d/2) (mod 256 / (d/2)), one 8-byte load per split;
// the (m, l) pairs are spread one per thread.  All of the row's loads are
// issued together, so the row costs one memory round trip plus three LDS
// reductions.
constexpr int kCombinePre = 16;

template <int D>
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  constexpr int LPS = D / 2;      // threads per split row
  constexpr int SPG = 256 / LPS;  // splits side by side
  constexpr int MLP = kMaxSplit / 256;
  __shared__ float s_w[kMaxSplit];
  __shared__ float s_red[2][4];
  __shared__ float2 s_num[SPG][LPS];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ns = a.n_split;
  const int cp = tid % LPS, so = tid / LPS;
  const float* p = a.part + row * ns * (D + 2);
  float2 pre[kCombinePre];
#pragma unroll
  for (int k = 0; k < kCombinePre; ++k) {
    const int sp = so + SPG * k;
    pre[k] = sp < ns ? *(const float2*)(p + (int64_t)sp * (D + 2) + 2 + 2 * cp) : make_float2(0.f, 0.f);
  }
  float2 ml[MLP];
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < MLP; ++k) {
    const int sp = tid + 256 * k;
    ml[k] = sp < ns ? *(const float2*)(p + (int64_t)sp * (D + 2)) : make_float2(-INFINITY, 0.f);
    M = fmaxf(M, ml[k].x);
  }
  M = wave_max(M);
  if (lane == 0) s_red[0][wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_red[0][0], s_red[0][1]), fmaxf(s_red[0][2], s_red[0][3]));
  float den = 0.f;
#pragma unroll
  for (int k = 0; k < MLP; ++k) {
    const int sp = tid + 256 * k;
    const float w = ml[k].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[k].x - M);
    if (sp < ns) s_w[sp] = w;
    den = __builtin_fmaf(w, ml[k].y, den);
  }
  den = wave_sum(den);
  if (lane == 0) s_red[1][wave] = den;
  __syncthreads();
  den = (s_red[1][0] + s_red[1][1]) + (s_red[1][2] + s_red[1][3]);
  float2 num = make_float2(0.f, 0.f);
#pragma unroll
  for (int k = 0; k < kCombinePre; ++k) {
    const int sp = so + SPG * k;
    if (sp < ns) {
      num.x = __builtin_fmaf(s_w[sp], pre[k].x, num.x);
      num.y = __builtin_fmaf(s_w[sp], pre[k].y, num.y);
    }
  }
#pragma unroll 8
  for (int sp = so + SPG * kCombinePre; sp < ns; sp += SPG) {
    const float2 o = *(const float2*)(p + (int64_t)sp * (D + 2) + 2 + 2 * cp);
    num.x = __builtin_fmaf(s_w[sp], o.x, num.x);
    num.y = __builtin_fmaf(s_w[sp], o.y, num.y);
  }
  s_num[so][cp] = num;
  __syncthreads();
  if (tid < LPS) {
    float2 tot = s_num[0][tid];
#pragma unroll
    for (int g = 1; g < SPG; ++g) { tot.x += s_num[g][tid].x; tot.y += s_num[g][tid].y; }
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    *(float2*)(a.out + row * D + 2 * tid) = make_float2(tot.x * inv, tot.y * inv);
  }
}

__global__ __launch_bounds__(256) void k_copy16(uint4* dst, const uint4* src, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

hipError_t launch_copy16(void* dst, const void* src, int64_t n16, hipStream_t s) {
  if (n16 <= 0) return hipSuccess;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_copy16, dim3((unsigned)blocks), dim3(256), 0, s, (uint4*)dst,
                     (const uint4*)src, n16);
  return hipGetLastError();
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
  uint32_t words[W];
  TileWords<W>::load(a.packed + (seq * tiles + (key >> 6)) * W * kTile, (int)(key & 63), words);
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
  else if (d == 256) hipLaunchKernelGGL(k_rotate<256>, dim3(rows), dim3(64), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int D, int B, bool QJL>
static hipError_t logits_t(const DecodeArgs& a, int64_t n_seq, int nbx, hipStream_t s) {
  // nbx counts 4-wave blocks; blocks of NW waves cover NW / 4 of them
  constexpr int NW = logits_waves<B>();
  const int nb = (nbx * 4 + NW - 1) / NW;
  hipLaunchKernelGGL((k_logits<D, B, QJL>), dim3(nb, (unsigned)n_seq, (a.G + 3) / 4), dim3(64 * NW),
                     0, s, a);
  return hipGetLastError();
}

template <int D, int B, bool QJL>
static hipError_t attn_t(const DecodeArgs& a, int64_t n_seq, hipStream_t s) {
  hipLaunchKernelGGL((k_attn<D, B, QJL>),
                     dim3(a.n_split * VGeom<D>::NVH, (unsigned)n_seq, (a.G + 3) / 4), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

#define OCTO_DISPATCH_DBQ(FN, ...)                                                              \
  switch (d * 10 + b) {                                                                         \
    case 2561: return qjl ? FN<256, 1, true>(__VA_ARGS__) : FN<256, 1, false>(__VA_ARGS__);     \
    case 2562: return qjl ? FN<256, 2, true>(__VA_ARGS__) : FN<256, 2, false>(__VA_ARGS__);     \
    case 2563: return qjl ? FN<256, 3, true>(__VA_ARGS__) : FN<256, 3, false>(__VA_ARGS__);     \
    case 2564: return qjl ? FN<256, 4, true>(__VA_ARGS__) : FN<256, 4, false>(__VA_ARGS__);     \
    case 2565: return qjl ? FN<256, 5, true>(__VA_ARGS__) : FN<256, 5, false>(__VA_ARGS__);     \
    case 641: return qjl ? FN<64, 1, true>(__VA_ARGS__) : FN<64, 1, false>(__VA_ARGS__);        \
    case 642: return qjl ? FN<64, 2, true>(__VA_ARGS__) : FN<64, 2, false>(__VA_ARGS__);        \
    case 643: return qjl ? FN<64, 3, true>(__VA_ARGS__) : FN<64, 3, false>(__VA_ARGS__);        \
    case 644: return qjl ? FN<64, 4, true>(__VA_ARGS__) : FN<64, 4, false>(__VA_ARGS__);        \
    case 1282: return qjl ? FN<128, 2, true>(__VA_ARGS__) : FN<128, 2, false>(__VA_ARGS__);     \
    case 1283: return qjl ? FN<128, 3, true>(__VA_ARGS__) : FN<128, 3, false>(__VA_ARGS__);     \
    case 1284: return qjl ? FN<128, 4, true>(__VA_ARGS__) : FN<128, 4, false>(__VA_ARGS__);     \
    case 645: return qjl ? FN<64, 5, true>(__VA_ARGS__) : FN<64, 5, false>(__VA_ARGS__);        \
    case 1281: return qjl ? FN<128, 1, true>(__VA_ARGS__) : FN<128, 1, false>(__VA_ARGS__);     \
    case 1285: return qjl ? FN<128, 5, true>(__VA_ARGS__) : FN<128, 5, false>(__VA_ARGS__);     \
  }                                                                                             \
  return hipErrorInvalidValue;

// LDS table copies of the single-query kernels: the code table (combined
// rho^ n^ per code, or unit directions) and the rho centroids, per
// instantiation, from the same constants as the copy loops.
template <int D, int B, bool QJL, bool REP, int NTH>
static int sq_copy_recs(const char* kernel, LdsCopyRec* out, int n, int max) {
  using SH = SQShared<D, B, QJL, REP>;
  using TC = SQTableCopy<D, B, QJL, REP, NTH>;
  using C = Codec<D, B>;
  if (n < max)
    out[n++] = {kernel, D, B, QJL, SH::kCombined ? TAB_TRIP : TAB_DIR, (int64_t)SH::NENT * SH::NCOPY,
                TC::SLOTS, TC::ENTRIES, (int64_t)SH::NENT * SH::NCOPY, NTH, TC::MASKED};
  if (n < max) out[n++] = {kernel, D, B, QJL, TAB_RHO, C::LR, C::LR, C::LR, C::LR, NTH, C::LR % NTH != 0};
  return n;
}

template <int D, int B, bool QJL>
static int decode_copy_recs(LdsCopyRec* out, int n, int max) {
  n = sq_copy_recs<D, B, QJL, logits_rep<B>(), 64 * logits_waves<B>()>("k_logits", out, n, max);
  n = sq_copy_recs<D, B, QJL, attn_rep<B>(), 256>("k_attn", out, n, max);
  return n;
}

int lds_copies_decode(LdsCopyRec* out, int max) {
  int n = 0;
#define OCTO_REC_B(D, QJL)                                                                     \
  n = decode_copy_recs<D, 1, QJL>(out, n, max); n = decode_copy_recs<D, 2, QJL>(out, n, max); \
  n = decode_copy_recs<D, 3, QJL>(out, n, max); n = decode_copy_recs<D, 4, QJL>(out, n, max); \
  n = decode_copy_recs<D, 5, QJL>(out, n, max);
  OCTO_REC_B(64, false)
  OCTO_REC_B(64, true)
  OCTO_REC_B(128, false)
  OCTO_REC_B(128, true)
  OCTO_REC_B(256, false)
  OCTO_REC_B(256, true)
#undef OCTO_REC_B
  return n;
}

hipError_t launch_logits(int d, int b, bool qjl, const DecodeArgs& a, int64_t n_seq, int nbx,
                         hipStream_t s) {
  OCTO_DISPATCH_DBQ(logits_t, a, n_seq, nbx, s)
}

hipError_t launch_attn(int d, int b, bool qjl, const DecodeArgs& a, int64_t n_seq, hipStream_t s) {
  OCTO_DISPATCH_DBQ(attn_t, a, n_seq, s)
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (a.n_split > kMaxSplit) return hipErrorInvalidValue;
  if (a.d == 64) hipLaunchKernelGGL(k_combine<64>, dim3(a.rows), dim3(256), 0, s, a);
  else if (a.d == 128) hipLaunchKernelGGL(k_combine<128>, dim3(a.rows), dim3(256), 0, s, a);
  else if (a.d == 256) hipLaunchKernelGGL(k_combine<256>, dim3(a.rows), dim3(256), 0, s, a);
  else return hipErrorInvalidValue;
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
    case 641: return recon_t<64, 1>(a, n_seq, s);
    case 642: return recon_t<64, 2>(a, n_seq, s);
    case 643: return recon_t<64, 3>(a, n_seq, s);
    case 644: return recon_t<64, 4>(a, n_seq, s);
    case 1282: return recon_t<128, 2>(a, n_seq, s);
    case 1283: return recon_t<128, 3>(a, n_seq, s);
    case 1284: return recon_t<128, 4>(a, n_seq, s);
    case 645: return recon_t<64, 5>(a, n_seq, s);
    case 1281: return recon_t<128, 1>(a, n_seq, s);
    case 1285: return recon_t<128, 5>(a, n_seq, s);
    case 2561: return recon_t<256, 1>(a, n_seq, s);
    case 2562: return recon_t<256, 2>(a, n_seq, s);
    case 2563: return recon_t<256, 3>(a, n_seq, s);
    case 2564: return recon_t<256, 4>(a, n_seq, s);
    case 2565: return recon_t<256, 5>(a, n_seq, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace octo

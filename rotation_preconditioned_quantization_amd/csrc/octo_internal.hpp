// Internal interface between the host library (octo_host.cpp) and the HIP
// kernels (k_*.hip).  Plain structs passed to kernels by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace octo {

constexpr int kTile = 64;          // keys per packed tile (one wavefront)
constexpr int kMaxLut = 1024;      // max buckets of an encoder lookup table
constexpr int kMaxLevels = 32;     // max centroids of one component (5 bits)
constexpr int kMaxSplit = 1024;    // max split-K partials per output row

// Nearest-centroid lookup for one scalar component (encoder).
// Bucket b covers [lo + b/inv_w, lo + (b+1)/inv_w); lut[b] is the number of
// midpoints below the bucket start minus a small margin, and at most two
// midpoints fall in the widened bucket, so the index #{k : x > m_k} is
// lut[b] + (x > mid[lut[b]]) + (x > mid[lut[b]+1]).  mid holds the sorted
// midpoints followed by two +inf sentinels.
struct QuantTable {
  const float* mid;
  const uint8_t* lut;
  float lo;
  float inv_w;
  int nb;
  int nmid;
};

// Encoder nearest-centroid for xi / eta: L uniform buckets over [-1, 1]; for
// x in bucket b the index #{k : x > m_k} is (b - 1) + (x > w[b]) + (x > w[b+1])
// with w = [-inf, m_0 .. m_{L-2}, +inf] (the host checks that the true index
// never leaves b-1 .. b+1, including a rounding margin at the bucket edges).
struct WindowTable {
  const float* w;  // L + 1 entries
  int levels;      // L
};

struct DevTables {
  QuantTable qx, qe, qr2;   // xi, eta, rho^2 (squared midpoints)
  WindowTable wx, we;       // xi, eta windows (encoder)
  float rho2_mid[8];        // squared rho midpoints (2^b_rho - 1 <= 7 used)
  const float4* dirtab;     // 2^(b_xi+b_eta) unit directions, index i_xi | i_eta << b_xi
  const float4* trip_tab;   // 2^B_t triplets rho^ n^ by full code (only for B_t <= 10)
  const float* rho_tab;     // 2^b_rho rho centroids
  const float* S;           // QJL matrix d x d row-major (nullptr without QJL)
  uint32_t sign_bits[4];    // bit j of the 128-bit mask set <=> WHT sign s_j = -1
};

struct EncodeArgs {
  DevTables t;
  const void* keys;
  int64_t seq_stride, key_stride;  // elements
  int64_t n_new, pos0, cap;
  uint32_t* packed;
  float* gamma;
  uint32_t* qjl_bits;
  uint16_t* qjl_norm;
};

// Query rotation: q' = mult * R q (pad zeros), rows r = ((b*Hkv + kvh)*G + g)*n_q + qi.
struct RotateArgs {
  DevTables t;
  const void* q;
  int qdt;
  int B, Hq, Hkv, n_q;
  float mult;          // folded into q' (attention: scale * log2(e))
  float* qrot;         // [rows][3T]
  float* qp;           // [rows][d] = (sqrt(pi/2)/d) * S q'[:d], QJL only (else nullptr)
};

struct DecodeArgs {
  DevTables t;
  const void* q;         // queries [B][Hq][d] (one token), rotated in each block's prologue
  int qdt;
  float mult;            // folded into q' (attention: scale * log2(e); logits: 1)
  const uint32_t* packed;
  const float* gamma;
  const uint32_t* qjl_bits;
  const uint16_t* qjl_norm;
  const void* v;
  int64_t n_keys, cap;
  int Hq, Hkv, G;
  int tiles_per_split;   // attention: key tiles of one split
  float* logits;         // [B][Hq][n_keys]
  float* part;           // attention partials [B*Hq][n_split][d + 2]
  int n_split;
};

struct CombineArgs {
  const float* part;
  float* out;
  int rows, n_split, d;
};

struct ReconArgs {
  DevTables t;
  const uint32_t* packed;
  const float* gamma;
  int64_t n_keys, cap;
  float* out;
};

struct MQArgs {
  DevTables t;
  const float* qrot;     // [H][n_q][3T] (scaled by scale*log2e)
  const uint32_t* packed;
  const float* gamma;
  const void* v;
  int64_t n_keys, cap;
  int B, n_q, H, Hkv, G;  // H = query heads
  int tiles_per_split, n_split;
  float* part;           // [B*H][n_q][n_split][d + 2]
};

hipError_t launch_encode(int d, int b, int kdt, bool qjl, const EncodeArgs& a, int64_t n_seq,
                         hipStream_t s);
hipError_t launch_rotate(int d, const RotateArgs& a, hipStream_t s);
hipError_t launch_logits(int d, int b, bool qjl, const DecodeArgs& a, int64_t n_seq,
                         int n_blocks_x, hipStream_t s);
hipError_t launch_attn(int d, int b, bool qjl, const DecodeArgs& a, int64_t n_seq, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);
hipError_t launch_reconstruct(int d, int b, const ReconArgs& a, int64_t n_seq, hipStream_t s);
hipError_t launch_mq_attn(int d, int b, const MQArgs& a, hipStream_t s);
int mq_tile_keys(int d);  // keys per tile of the multi-query kernel

}  // namespace octo

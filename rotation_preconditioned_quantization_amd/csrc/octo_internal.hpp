// Internal interface between the host library (octo_host.cpp) and the HIP
// kernels (k_*.hip).  Plain structs passed to kernels by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace octo {

constexpr int kTile = 64;          // keys per packed tile (one wavefront)
constexpr int kMaxLut = 256;       // max buckets of an encoder lookup table
constexpr int kMaxLevels = 32;     // max centroids of one component (5 bits)
constexpr int kMaxSplit = 1024;    // max split-K partials per output row
constexpr int kEncodeOneMax = 16;  // up to this many new keys per sequence: one-key encoder
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;  // octo_decode_attn_static's device array
constexpr int kMaxDevices = 64;

// Nearest-centroid lookup for one scalar component (encoder): the index
// #{k : x > m_k} of the midpoint rule.  The value range is cut into nb equal
// buckets; every bucket, widened by the rounding of the formula that finds
// it, holds at most one midpoint, so the index is t[b].x + (x > t[b].y as
// float): t[b].x counts the midpoints below the bucket, t[b].y is the one
// inside it (+inf if none).  The host checks the one-midpoint property when
// it builds the table.  Two layouts, both of nb + 2 entries:
//   xi, eta (centred on the integers): bucket b = bits of fmaf(x, scale,
//     bias) - kBucketMagicBits, where bias carries kBucketMagic, so the fma
//     itself rounds x scale + (bias - kBucketMagic) to the integer b in
//     [0, nb] for x in [-1, 1] up to rounding; one guard entry t[nb + 1];
//   rho^2 (from 0): b = (int) min(x scale, nb - 1) (the float-to-unsigned
//     conversion saturates below at 0), two guard entries.
struct Bucket1 {
  const uint2* t;     // nb + 2 entries
  float scale, bias;
  int nb;
};

// 1.5 * 2^23: floats in [2^23, 2^24) are spaced 1 apart, so adding this to a
// value of magnitude below 2^22 rounds the value to an integer, which the
// sum's low mantissa bits then hold (offset by kBucketMagicBits).
constexpr float kBucketMagic = 12582912.0f;
constexpr uint32_t kBucketMagicBits = 0x4B400000u;

struct DevTables {
  Bucket1 qx, qe, qr2;      // xi, eta over [-1, 1]; rho^2 (squared midpoints) over [0, inf)
  const float4* dirtab;     // 2^(b_xi+b_eta) unit directions, index i_xi | i_eta << b_xi
  const float4* trip_tab;   // 2^B_t triplets rho^ n^ by full code (only for B_t <= 10)
  const float* rho_tab;     // 2^b_rho rho centroids
  const float* St;          // QJL matrix S transposed, St[c * d + j] = S[j][c] (nullptr without QJL)
  const uint4* S16;         // S (row-major) as f16 planes [S_hi | S_lo], S_hi = f16(S), S_lo = f16(S - S_hi)
  uint32_t sign_bits[8];    // bit j of the 256-bit mask set <=> WHT sign s_j = -1
  float qjl_kappa;          // QJL estimator constant: <q', r'> ~ kappa |r'| <S q', sgn(S r')>
  float rho_mid2[3];        // the first 3 squared rho midpoints (fp32; +inf past the last)
};

struct EncodeArgs {
  DevTables t;
  const void* keys;
  int64_t seq_stride, key_stride;  // elements
  int64_t n_new, pos0, cap;
  int64_t seq_count;               // sequences (n_seq)
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
  float* qp;           // [rows][d] = kappa * S q'[:d], QJL only (else nullptr)
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
  // decode step with append (attention only, bf16 keys, no QJL): the new key
  // of sequence s at new_keys + s * new_key_stride (elements) is encoded
  // into position n_keys - 1 of packed_w / gamma_w by the block that owns
  // that position, which also uses it at once; nullptr otherwise
  const void* new_keys;
  int64_t new_key_stride;
  uint32_t* packed_w;
  float* gamma_w;
};

// Geometry of a copy of NS table entries into LDS by NTH threads, one entry
// per thread per round (global_load_lds or a strided loop).  When NTH does
// not divide NS the copy is masked per lane at NS; either way it writes LDS
// entries [0, SLOTS) only.  NCOPY > 1: LDS entry i holds table entry
// i / NCOPY (replicated tables), so the copy reads table entries
// [0, ENTRIES) only.  Kernels static_assert SLOTS and ENTRIES against their
// LDS array and table sizes; LdsCopyRec reports the same figures.
template <int NS, int NTH, int NCOPY = 1>
struct TableCopy {
  static constexpr int ROUNDS = (NS + NTH - 1) / NTH;
  static constexpr bool MASKED = NS % NTH != 0;
  static constexpr int SLOTS = MASKED ? NS : ROUNDS * NTH;
  static constexpr int ENTRIES = (SLOTS - 1) / NCOPY + 1;
};

// One table copy into LDS, as a kernel instantiation performs it (the
// octo_lds_copy record of the C ABI).  copied: entries moved, one per thread
// per round; entries_read = copied = -1: a loop bounded at run time by the
// table's own entry count (the launcher checks that count against
// lds_slots).
struct LdsCopyRec {
  const char* kernel;
  int d, b, qjl, table;
  int64_t lds_slots, slots_written, entries_read, copied;
  int threads, masked;
};

enum { TAB_DIR = 0, TAB_TRIP = 1, TAB_RHO = 2, TAB_QX = 3, TAB_QE = 4, TAB_QR2 = 5, TAB_S16 = 6,
       TAB_COUNT = 7 };

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

hipError_t launch_encode(int d, int b, int kdt, bool qjl, bool joint, const EncodeArgs& a,
                         int64_t n_seq, hipStream_t s);
hipError_t launch_rotate(int d, const RotateArgs& a, hipStream_t s);
hipError_t launch_logits(int d, int b, bool qjl, const DecodeArgs& a, int64_t n_seq,
                         int n_blocks_x, hipStream_t s);
hipError_t launch_attn(int d, int b, bool qjl, const DecodeArgs& a, int64_t n_seq, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);
hipError_t launch_copy16(void* dst, const void* src, int64_t n16, hipStream_t s);
hipError_t launch_reconstruct(int d, int b, const ReconArgs& a, int64_t n_seq, hipStream_t s);
hipError_t launch_mq_attn(int d, int b, const MQArgs& a, hipStream_t s);
// The LDS table copies of the kernels in each translation unit (records
// appended to out[0 .. max), count returned).
int lds_copies_decode(LdsCopyRec* out, int max);
int lds_copies_mq(LdsCopyRec* out, int max);
int lds_copies_encode(LdsCopyRec* out, int max);
// Device address of the static decode scratch on `device` (the current
// device), resolved once per device.
hipError_t static_scratch(int device, void** out);
int mq_tile_keys(int d, int b);  // keys per tile of the multi-query kernel
int mq_value_parts(int d);       // workgroups sharing one (query block, split): value dim parts
int mq_block_queries();   // queries per workgroup of the multi-query kernel

}  // namespace octo

/*
 * octo.h -- C ABI of the OCTOPUS key-codec library for MI355X (gfx950).
 *
 * OCTOPUS compresses attention keys.  Each key k (head dim d, a power of two)
 * is split into its fp32 norm gamma = |k| and a unit direction, the direction
 * is rotated by a seeded sign-flipped Walsh-Hadamard transform, cut into
 * zero-padded coordinate triplets, and every triplet is stored as a Lloyd-Max
 * quantised norm rho and an octahedral (xi, eta) pair.  Decode rebuilds the
 * keys in registers inside the attention kernels and never writes them out.
 *
 * Sources (the method description this library follows):
 *   [YL] youleyou.com summary of arXiv:2605.21226 "OCTOPUS", sections
 *        旋转魔法 (rotation), 八面体折叠 (octahedral folding), 三元组分解
 *        (triplet decomposition), 非均匀比特分配 (bit allocation),
 *        可选的残差修正 (OCTOPUS-QJL), 工程实现 (fused decode).
 *   [AR] agents-report.net "OCTOPUS：八面體參數化與 triplet 聯合量化優化
 *        Transformer KV 快取", sections 方法概覽, 位元分配, 實作要點, OCTOPUS-QJL.
 *   [AB] the paper's abstract (arxivlens / chatpaper pages): data-oblivious,
 *        online, deterministic given a seed; fused decode without
 *        materialising keys.
 *
 * Conventions for every call:
 *   - Device pointers are HIP device memory owned by the caller; host
 *     pointers are marked "host".  The library owns only the codebook.
 *     packed and qjl_bits must be 16-byte aligned, gamma and q 4-byte.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work: no call below synchronises the host, and no
 *     call allocates device memory except octo_codebook_build.
 *   - Arguments are checked before any launch.  A failed check returns a
 *     status and enqueues nothing; octo_last_error() then describes it
 *     (thread-local string).  Device faults surface at the caller's next
 *     synchronisation.
 *   - Codebooks are immutable after build, so concurrent calls on
 *     different streams may share one.
 */
#ifndef OCTO_H
#define OCTO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  OCTO_OK = 0,
  OCTO_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, n > cap ... */
  OCTO_ERR_UNSUPPORTED = 2, /* d, b or allocation without a compiled kernel  */
  OCTO_ERR_HIP = 3,         /* a HIP runtime call or launch failed           */
  OCTO_ERR_NOMEM = 4,       /* host or device allocation failed (build only) */
  OCTO_ERR_WORKSPACE = 5    /* workspace missing or smaller than required    */
} octo_status;

typedef enum { OCTO_F32 = 0, OCTO_BF16 = 1, OCTO_F16 = 2 } octo_dtype;

typedef struct octo_codebook octo_codebook; /* opaque, owned by the library */

/* Codebook parameters.  The codebook is a pure function of these fields
 * ([AR] 位元分配: it depends only on d and the bit budget; [AB]: deterministic
 * given a seed).
 *   d         head dim: 64, 128 and 256 have kernels (any power of two 4..1024
 *             for a host-only codebook).  At d = 256 the encoder gives each
 *             key two lanes.
 *   b         bit budget per coordinate; kernels exist for 1 .. 5.
 *   seed      seeds the WHT sign vector and the QJL projection.
 *   cb_seed   seeds the Monte-Carlo samples the Lloyd-Max tables are fit to.
 *   b_xi, b_eta, b_rho  bits per component; any value < 0 selects the pages'
 *             allocation (b+1, b+1, b-1) ([YL] 非均匀比特分配, direction one bit
 *             more, length one bit less), i.e. 3b+1 bits per triplet.  Kernels
 *             exist for that allocation only; others build host-only tables.
 *   qjl       1: also draw the residual's random rotation for OCTOPUS-QJL
 *             ([YL] 可选的残差修正: the residual is rotated independently and
 *             only the signs are kept): S = sqrt(d) P, P the Haar-random
 *             orthogonal Q factor of a seeded d x d Gaussian matrix.
 *   mc_vectors  Monte-Carlo vectors for the tables (0 = 65536).
 *   device    HIP device to upload the tables to, or -1 for a host-only
 *             codebook (octo_codebook_export / layout work; kernels refuse it).
 */
typedef struct {
  int d;
  int b;
  uint64_t seed;
  uint64_t cb_seed;
  int b_xi, b_eta, b_rho;
  int qjl;
  int mc_vectors;
  int device;
} octo_params;

/* Packed-cache geometry of a codebook.
 * Keys of one sequence (one batch x KV-head) live in tiles of tile_keys (64)
 * keys, W = words_per_key u32 words per key.  Inside a tile the words of all
 * keys are cut into groups of 4 consecutive words (the last group holds the
 * W % 4 left over); group g is stored key-major, [key][4] (last group
 * [key][W % 4]), and the groups follow each other: word w of key j is the u32
 * at packed[seq][j / 64][64 * 4 * (w / 4) + (j % 64) * width + w % 4], width =
 * 4 for full groups and W % 4 for the last.  Inside a key, triplet i occupies
 * bits [i*B_t, (i+1)*B_t) of its little-endian word stream, LSB first, as
 * code = i_xi | i_eta << b_xi | i_rho << (b_xi+b_eta); unused high bits are 0.
 * gamma is fp32 [seq][cap].  With QJL, the d/32 sign words of a key use the
 * same tile layout in qjl_bits (bit j%32 of word j/32 = sign j, 1 = positive)
 * and the residual norm is fp16 [seq][cap]. */
typedef struct {
  int d, n_triplets, pad_dim;
  int b_xi, b_eta, b_rho, bits_per_triplet, bits_per_key;
  int words_per_key, tile_keys, qjl, qjl_words_per_key;
  size_t packed_bytes_per_key_alloc; /* words_per_key * 4 */
} octo_layout;

/* Build a codebook ([AR] 位元分配, [AB] "implementation-matched marginals"):
 * SplitMix64 streams keyed by seed/cb_seed, WHT signs, Monte-Carlo samples of
 * the rotated triplet marginals, Lloyd-Max fits, encoder lookup tables,
 * unit-direction table, optional QJL matrix; then a synchronous upload to
 * `device`.  Host work of about a second.  *out receives the handle. */
octo_status octo_codebook_build(const octo_params* params, octo_codebook** out);
octo_status octo_codebook_free(octo_codebook* cb);
octo_status octo_codebook_layout(const octo_codebook* cb, octo_layout* out);

/* Host copies of the tables (tests).  Any pointer may be NULL to skip it.
 * c_xi: 2^b_xi, c_eta: 2^b_eta, c_rho: 2^b_rho doubles; signs: d int8 (+-1);
 * qjl_S: d*d floats row-major, S = sqrt(d) P (only if built with qjl). */
octo_status octo_codebook_export(const octo_codebook* cb, double* c_xi, double* c_eta,
                                 double* c_rho, int8_t* signs, float* qjl_S);

/* The codebook tables that kernels copy from global memory into LDS. */
typedef enum {
  OCTO_TABLE_DIR = 0,  /* unit directions by (i_xi, i_eta): 16-byte entries    */
  OCTO_TABLE_TRIP = 1, /* rho^ n^ by triplet code (B_t <= 10 only): 16 bytes  */
  OCTO_TABLE_RHO = 2,  /* rho centroids: 4-byte entries                        */
  OCTO_TABLE_QX = 3,   /* encoder bucket table of xi: 8-byte entries          */
  OCTO_TABLE_QE = 4,   /* encoder bucket table of eta                          */
  OCTO_TABLE_QR2 = 5,  /* encoder bucket table of rho^2                        */
  OCTO_TABLE_S16 = 6,  /* QJL matrix as f16 high/low planes: 16-byte entries  */
  OCTO_TABLE_COUNT = 7
} octo_table;

/* Entries of table `table` (octo_table) in the codebook's tables, device or
 * host-only (a host-only codebook computes the same tables without uploading
 * them); 0 for a table the codebook has no use for, -1 for a bad argument.
 * The device allocation ends with 1 KiB of zeros past the last table. */
int64_t octo_codebook_table_entries(const octo_codebook* cb, int table);

/* Bounds-check aid: one copy of a codebook table into LDS as a kernel
 * instantiation performs it, enumerated by index 0, 1, ... (returns
 * OCTO_ERR_INVALID_ARG past the last).  The figures come from the same
 * compile-time constants as the copy loops (which static_assert them):
 *   kernel, d, b, qjl   the kernel template and instantiation (string owned
 *                       by the library);
 *   table               the octo_table read;
 *   lds_slots           entries the LDS destination holds;
 *   slots_written       1 + the highest LDS entry the copy can write;
 *   entries_read        1 + the highest table entry it can read, or -1 for
 *                       a loop bounded by the table's own entry count at
 *                       run time (then that count must fit lds_slots);
 *   copied              entries moved, one per thread per round (-1 with
 *                       a run-time bound);
 *   threads, masked     threads sharing the copy; 1 when the copy bounds
 *                       each lane (needed when threads does not divide
 *                       copied).
 * A copy is in bounds when slots_written <= lds_slots and entries_read <=
 * octo_codebook_table_entries of the codebook it runs with. */
typedef struct {
  const char* kernel;
  int d, b, qjl, table;
  int64_t lds_slots, slots_written, entries_read, copied;
  int threads, masked;
} octo_lds_copy;
octo_status octo_debug_lds_copy(int index, octo_lds_copy* out);

/* Check aid for the encoder's nearest-centroid lookup ([YL] 三元组分解 step 4,
 * the midpoint rule): out[i] = the index the encoder kernels take for value
 * x[i] of xi (table OCTO_TABLE_QX) or eta (OCTO_TABLE_QE), by the kernels'
 * own formula (one fma, its bits less a magic constant, one bucket entry,
 * one compare) evaluated on the host over the codebook's table; it should
 * equal #{k : x[i] > m_k} over the component's fp32 midpoints m_k.  x, out:
 * host arrays of n entries.  Any codebook built with kernels (device or
 * host-only).  OCTO_ERR_INVALID_ARG for another table, a NULL array, or an
 * x whose bucket lies outside the table (the kernels are given values in
 * [-1, 1] up to rounding); OCTO_ERR_UNSUPPORTED for a codebook without
 * encoder tables. */
octo_status octo_debug_bucket_index(const octo_codebook* cb, int table, const float* x, int64_t n,
                                    uint32_t* out);

/* Bytes of the packed stream for n_seq sequences of capacity cap (cap % 64 == 0). */
size_t octo_packed_bytes(const octo_codebook* cb, int64_t n_seq, int64_t cap);
size_t octo_qjl_bits_bytes(const octo_codebook* cb, int64_t n_seq, int64_t cap);

/* Online key encoder ([YL] 三元组分解 steps 1-4, 八面体折叠; [AB] online).
 * keys: device, dtype kdt, key (s, j) at keys + s*seq_stride + j*key_stride
 *   (element strides; rows must be 16-byte aligned), s < n_seq, j < n_new.
 * Writes cache positions pos0 .. pos0+n_new-1 of every sequence:
 *   packed (octo_packed_bytes(cb, n_seq, cap) bytes), gamma fp32 [n_seq][cap],
 *   and with a QJL codebook also qjl_bits and qjl_norm (fp16 [n_seq][cap]);
 *   pass NULL for both to skip QJL.  Requires pos0 + n_new <= cap, cap % 64 == 0.
 * Rounding is scalar nearest-centroid (midpoint rule, ties to the lower
 * index).  Other positions of the cache are not touched.  Keys must be
 * finite: a key holding inf or NaN gets unspecified words and gamma (the
 * call still completes and touches no other key). */
octo_status octo_encode(const octo_codebook* cb, const void* keys, octo_dtype kdt,
                        int64_t n_seq, int64_t n_new, int64_t seq_stride, int64_t key_stride,
                        int64_t pos0, int64_t cap, void* packed, float* gamma,
                        void* qjl_bits, uint16_t* qjl_norm, void* stream);

/* The same encoder with joint rounding ([YL] 联合取整): per triplet t of the
 * rotated unit key, the direction code is chosen among the 3x3 neighbours of
 * the scalar-rounded (i_xi, i_eta) (clamped to the index range), each with
 * the rho centroid nearest s = <n^, t>, minimising |t - rho^ n^|^2; the first
 * strict minimum in (xi offset, eta offset) order -1, 0, +1 wins.  Arguments,
 * layout, ownership and errors as octo_encode; gamma and the QJL residual
 * (computed from the chosen codes) likewise.  Costs several times the
 * scalar encoder's arithmetic. */
octo_status octo_encode_joint(const octo_codebook* cb, const void* keys, octo_dtype kdt,
                              int64_t n_seq, int64_t n_new, int64_t seq_stride,
                              int64_t key_stride, int64_t pos0, int64_t cap, void* packed,
                              float* gamma, void* qjl_bits, uint16_t* qjl_norm, void* stream);

/* Workspace for the decode calls.  mode 0 = octo_decode_logits, 1 =
 * octo_decode_attn.  The workspace holds the rotated queries and, for
 * attention, the split-K partial results (one call at a time per
 * workspace). */
size_t octo_decode_workspace_bytes(const octo_codebook* cb, int mode, int B, int Hq, int Hkv,
                                   int n_q, int64_t n_keys);

/* Fused compressed-K logits ([YL] 工程实现: keys rebuilt in registers, q.k).
 * q: device [B][Hq][d] (dtype qdt), one query token per head.  Query head h
 * reads KV head h / (Hq/Hkv).  packed/gamma as written by octo_encode for
 * n_seq = B*Hkv sequences of capacity cap; the first n_keys positions are read.
 * logits: device fp32 [B][Hq][n_keys], the raw (unscaled) <q, k^>.  With
 * qjl_bits/qjl_norm non-NULL (QJL codebook) the OCTOPUS-QJL estimate
 *   gamma * (<q', u'^> + kappa_d * nu * <S q', sigma>)  is returned,
 * kappa_d = 1 / (d sqrt(d) E|u_1|) with E|u_1| = Gamma(d/2) / (sqrt(pi)
 * Gamma((d+1)/2)) (exactly unbiased for the rotation S). */
octo_status octo_decode_logits(const octo_codebook* cb, const void* q, octo_dtype qdt, int B,
                               int Hq, int Hkv, const void* packed, const float* gamma,
                               const void* qjl_bits, const uint16_t* qjl_norm, int64_t n_keys,
                               int64_t cap, float* logits, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Fused compressed-K attention ([YL] 工程实现: unpack, rebuild, q.k, online
 * softmax, FlashAttention-style tiling).
 * q: device [B][Hq][n_q][d]; v: device [B*Hkv][cap][d] (dtype vdt: bf16);
 * out: device fp32 [B][Hq][n_q][d] = softmax(scale * l) v over the first
 * n_keys keys, l the logits above (QJL-corrected when the QJL buffers are
 * given), no mask.  scale <= 0 selects 1/sqrt(d).  n_q == 1 runs the split-K
 * single-query kernels; n_q > 1 runs the multi-query MFMA kernel (refused
 * with OCTO_ERR_UNSUPPORTED for QJL buffers).
 * n_keys == 0 writes zeros.
 * Value range: the single-query kernels use V as stored (any bf16).  The
 * multi-query kernel multiplies in fp16: bf16 values with |v| in fp16's
 * normal range [2^-14, 65504] (and 0) are exact there, larger ones saturate
 * at +-65504 (round toward zero), smaller ones keep fp16's subnormal
 * precision (2^-24). */
octo_status octo_decode_attn(const octo_codebook* cb, const void* q, octo_dtype qdt, int B,
                             int Hq, int Hkv, int n_q, const void* packed, const float* gamma,
                             const void* qjl_bits, const uint16_t* qjl_norm, const void* v,
                             octo_dtype vdt, int64_t n_keys, int64_t cap, float scale, float* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory or hand in a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): octo_decode_attn with its scratch (the split-K partials and
 * rotated queries) in a static device array of OCTO_STATIC_SCRATCH_BYTES
 * that the library holds on every GPU it runs on until the process ends.
 * The call allocates nothing.  Arguments, layout, results and errors as
 * octo_decode_attn; a call whose scratch (octo_decode_workspace_bytes, mode
 * 1) exceeds the array returns OCTO_ERR_WORKSPACE and enqueues nothing.
 * All calls on one GPU share that GPU's array: calls that overlap in time on
 * one GPU (other streams, other host threads) race and give wrong results;
 * order them on one stream. */
#define OCTO_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
octo_status octo_decode_attn_static(const octo_codebook* cb, const void* q, octo_dtype qdt, int B,
                                    int Hq, int Hkv, int n_q, const void* packed,
                                    const float* gamma, const void* qjl_bits,
                                    const uint16_t* qjl_norm, const void* v, octo_dtype vdt,
                                    int64_t n_keys, int64_t cap, float scale, float* out,
                                    void* stream);

/* One autoregressive decode step ([YL] 工程实现; [AB] online): the new
 * token's key of every sequence is encoded into the cache at position
 * n_keys - 1, then the fused attention of one query token per head runs over
 * the n_keys cached keys, the new one included, exactly as octo_decode_attn
 * with n_q = 1.
 *   new_keys: device, dtype kdt, the key of sequence s = b*Hkv + kvh at
 *     new_keys + s * key_seq_stride (elements; 16-byte aligned rows).
 *   v must already hold the new token's value row at position n_keys - 1.
 *   For bf16 keys without QJL buffers the step is one fused pass: the
 *   attention block that owns position n_keys - 1 encodes the key with one
 *   wavefront (the same operations and rounding as octo_encode, so identical
 *   words and gamma), writes it to the cache and uses it at once.  Otherwise
 *   the key is encoded first (with the QJL encoder when QJL buffers are
 *   given; the QJL term is then used in the attention).
 * Requires 1 <= n_keys <= cap.  Other arguments, ownership and errors as
 * octo_encode and octo_decode_attn. */
octo_status octo_decode_attn_append(const octo_codebook* cb, const void* new_keys, octo_dtype kdt,
                                    int64_t key_seq_stride, const void* q, octo_dtype qdt, int B,
                                    int Hq, int Hkv, void* packed, float* gamma, void* qjl_bits,
                                    uint16_t* qjl_norm, const void* v, octo_dtype vdt,
                                    int64_t n_keys, int64_t cap, float scale, float* out,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* The launches of the two decode calls, for callers that schedule or time
 * them one by one: OCTO_STAGE_ROTATE writes the rotated queries into the
 * workspace (multi-query attention only; the other kernels rotate in their
 * prologue); OCTO_STAGE_MAIN runs the fused kernel; OCTO_STAGE_COMBINE
 * (attention only) merges the split-K partials into out.  Stages must run in
 * this order on one stream with the same arguments and workspace;
 * octo_decode_logits / octo_decode_attn run all of them. */
#define OCTO_STAGE_ROTATE 1
#define OCTO_STAGE_MAIN 2
#define OCTO_STAGE_COMBINE 4
#define OCTO_STAGE_ALL 7
octo_status octo_decode_logits_stages(const octo_codebook* cb, const void* q, octo_dtype qdt,
                                      int B, int Hq, int Hkv, const void* packed,
                                      const float* gamma, const void* qjl_bits,
                                      const uint16_t* qjl_norm, int64_t n_keys, int64_t cap,
                                      float* logits, void* workspace, size_t workspace_bytes,
                                      void* stream, int stages);
octo_status octo_decode_attn_stages(const octo_codebook* cb, const void* q, octo_dtype qdt, int B,
                                    int Hq, int Hkv, int n_q, const void* packed,
                                    const float* gamma, const void* qjl_bits,
                                    const uint16_t* qjl_norm, const void* v, octo_dtype vdt,
                                    int64_t n_keys, int64_t cap, float scale, float* out,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    int stages);

/* Test helper: rebuild keys k^ = gamma R^T u'^ into keys_out fp32
 * [n_seq][n_keys][d] (device). */
octo_status octo_debug_reconstruct(const octo_codebook* cb, const void* packed, const float* gamma,
                                   int64_t n_seq, int64_t n_keys, int64_t cap, float* keys_out,
                                   void* stream);

/* Measurement aid: copy `bytes` (a multiple of 16, both pointers 16-byte
 * aligned) from device src to device dst with 16-byte loads and stores, 1 KiB
 * contiguous per wavefront access -- the access pattern of the codec kernels.
 * Its reading of the HBM traffic counters (rocprofv3 FETCH_SIZE, WRITE_SIZE)
 * for a known byte count is the scale that turns their readings for the codec
 * kernels into bytes. */
octo_status octo_debug_copy(void* dst, const void* src, size_t bytes, void* stream);

const char* octo_status_str(octo_status s);
const char* octo_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* OCTO_H */

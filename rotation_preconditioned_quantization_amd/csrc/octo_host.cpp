// Host side of the OCTOPUS library: C ABI, codebook builder, argument checks
// and kernel dispatch.  The codebook builder runs on the host in fp64; the
// kernels live in k_*.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <limits>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/octo.h"
#include "octo_internal.hpp"

using namespace octo;

namespace {

thread_local std::string g_last_error;

octo_status fail(octo_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

// ---------------------------------------------------------------------------
// Seeded randomness ([AB]: deterministic given a seed).  SplitMix64 (Steele,
// Lea & Flood 2014) started at seed ^ tag; uniforms (x >> 11) * 2^-53;
// Box-Muller pairs g_2p = r cos(2 pi u2), g_2p+1 = r sin(2 pi u2),
// r = sqrt(-2 ln(1 - u1)).
// ---------------------------------------------------------------------------
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kTagSigns = 0x4F43544F5349474Eull;  // "OCTOSIGN"
constexpr uint64_t kTagMC = 0x4F43544F4D43534Dull;     // "OCTOMCSM"
constexpr uint64_t kTagQJL = 0x4F43544F514A4C53ull;    // "OCTOQJLS"

inline uint64_t splitmix_out(uint64_t state0, uint64_t i) {
  uint64_t z = state0 + (i + 1) * kGamma;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

inline double uniform_at(uint64_t state0, uint64_t i) {
  return (double)(splitmix_out(state0, i) >> 11) * (1.0 / 9007199254740992.0);
}

void gaussians(uint64_t seed, uint64_t tag, size_t n, double* out) {
  const uint64_t s0 = seed ^ tag;
  const double two_pi = 6.283185307179586;
  for (size_t p = 0; 2 * p < n; ++p) {
    const double u1 = uniform_at(s0, 2 * p), u2 = uniform_at(s0, 2 * p + 1);
    const double r = std::sqrt(-2.0 * std::log(1.0 - u1));
    const double th = two_pi * u2;
    out[2 * p] = r * std::cos(th);
    if (2 * p + 1 < n) out[2 * p + 1] = r * std::sin(th);
  }
}

// Octahedral encode of a unit (or zero-guarded) direction ([YL] 八面体折叠);
// sgn(0) = +1, z = 0 is the upper hemisphere.
inline void octa_encode(double x, double y, double z, double* xi, double* eta) {
  const double l1 = std::fabs(x) + std::fabs(y) + std::fabs(z);
  const double px = x / l1, py = y / l1;
  if (z < 0) {
    *xi = (1.0 - std::fabs(py)) * (px >= 0 ? 1.0 : -1.0);
    *eta = (1.0 - std::fabs(px)) * (py >= 0 ? 1.0 : -1.0);
  } else {
    *xi = px;
    *eta = py;
  }
}

inline void octa_decode(double xi, double eta, double* v) {
  const double r = 1.0 - std::fabs(xi) - std::fabs(eta);
  double x = xi, y = eta;
  if (r < 0) {
    x = (1.0 - std::fabs(eta)) * (xi >= 0 ? 1.0 : -1.0);
    y = (1.0 - std::fabs(xi)) * (eta >= 0 ? 1.0 : -1.0);
  }
  const double n = std::sqrt(x * x + y * y + r * r);
  v[0] = x / n;
  v[1] = y / n;
  v[2] = r / n;
}

// Lloyd-Max on samples ([YL] 三元组分解; [AB]): start at the sample quantiles
// (k + 1/2)/L, then c_k <- mean of the samples with m_{k-1} < x <= m_k (an
// empty cell keeps its centroid) until max |dc| <= 1e-12 or 2000 rounds.
// `x` must be sorted; cell sums come from prefix sums.
std::vector<double> lloyd_max_sorted(const std::vector<double>& x, int L) {
  const size_t N = x.size();
  std::vector<double> c(L);
  if (L == 1) {
    double s = 0;
    for (double v : x) s += v;
    c[0] = s / (double)N;
    return c;
  }
  std::vector<double> prefix(N + 1);
  prefix[0] = 0.0;
  for (size_t i = 0; i < N; ++i) prefix[i + 1] = prefix[i] + x[i];
  for (int k = 0; k < L; ++k) c[k] = x[(size_t)std::floor((k + 0.5) * (double)N / (double)L)];
  std::vector<size_t> edges(L - 1);
  for (int it = 0; it < 2000; ++it) {
    for (int k = 0; k + 1 < L; ++k) {
      const double m = 0.5 * (c[k] + c[k + 1]);
      edges[k] = (size_t)(std::upper_bound(x.begin(), x.end(), m) - x.begin());
    }
    double dmax = 0.0;
    for (int k = 0; k < L; ++k) {
      const size_t lo = k == 0 ? 0 : edges[k - 1];
      const size_t hi = k == L - 1 ? N : edges[k];
      double nc = c[k];
      if (hi > lo) nc = (prefix[hi] - prefix[lo]) / (double)(hi - lo);
      dmax = std::max(dmax, std::fabs(nc - c[k]));
      c[k] = nc;
    }
    if (dmax <= 1e-12) break;
  }
  return c;
}

std::vector<double> antisymmetrize(const std::vector<double>& c) {
  const size_t L = c.size();
  std::vector<double> o(L);
  for (size_t k = 0; k < L; ++k) o[k] = 0.5 * (c[k] - c[L - 1 - k]);
  return o;
}

// One-midpoint-per-bucket table (see Bucket1) for the value range [lo, hi)
// cut into nb buckets of width w; the first bucket extends to -inf, the last
// to +inf.  Takes the smallest bucket count (16 ... 256) that keeps <= 1
// midpoint in every bucket widened by the rounding margin of the device's
// bucket formula (a small table is copied into each encoder block's LDS
// sooner); false if none does.
//   plain: bucket b covers [lo + b w, lo + (b + 1) w), b < nb, found by
//     truncating x scale + bias; two guard buckets follow.
//   centred: bucket b covers [lo + (b - 1/2) w, lo + (b + 1/2) w), b <= nb,
//     found by rounding: with bias = -lo scale + kBucketMagic (lo scale an
//     integer), fmaf(x, scale, bias) holds kBucketMagic + round(x scale -
//     lo scale) exactly, so its bits minus kBucketMagicBits are the bucket
//     (one rounding of the exact value; a tie lands in either neighbour,
//     both of whose widened ranges hold x); one guard bucket follows.
// Either way the table has nb + 2 entries.
struct HostB1 {
  std::vector<uint32_t> t;  // 2 words per bucket: base, float bits of the midpoint
  float scale = 0, bias = 0;
  int nb = 0;
  bool centred = false;
};

bool build_bucket1(const std::vector<double>& mids, double lo, double hi, bool centred, HostB1* q) {
  const int nmid = (int)mids.size();
  std::vector<float> mf(nmid);
  for (int k = 0; k < nmid; ++k) mf[k] = (float)mids[k];
  const double eps = 1e-6 * (hi - lo);
  for (int nb : {16, 32, 64, 128, 256}) {
    if (nb > kMaxLut) continue;
    const double w = (hi - lo) / nb;
    const int nbk = centred ? nb + 1 : nb;   // buckets before the guards
    const double off = centred ? -0.5 : 0.0;
    std::vector<uint32_t> t(2 * (size_t)nbk);
    bool ok = true;
    for (int b = 0; b < nbk && ok; ++b) {
      const double L = b == 0 ? -INFINITY : lo + (b + off) * w - eps;
      const double U = b == nbk - 1 ? INFINITY : lo + (b + 1 + off) * w + eps;
      int below = 0, inside = 0;
      float m_in = INFINITY;
      for (int k = 0; k < nmid; ++k) {
        if ((double)mf[k] < L) ++below;
        else if ((double)mf[k] <= U) { ++inside; m_in = mf[k]; }
      }
      if (inside > 1) ok = false;
      uint32_t bits;
      std::memcpy(&bits, &m_in, 4);
      t[2 * b] = (uint32_t)below;
      t[2 * b + 1] = bits;
    }
    if (!ok) continue;
    // guard buckets repeating the last one (a value a rounding step above hi
    // lands in one without a clamp), up to nb + 2 entries
    while ((int)t.size() < 2 * (nb + 2)) { t.push_back(t[2 * (nbk - 1)]); t.push_back(t[2 * (nbk - 1) + 1]); }
    const double scale = nb / (hi - lo);
    if (centred) {
      const double bias = -lo * scale;
      if (bias != std::floor(bias) || std::fabs(bias) >= 1 << 20) continue;
      q->bias = (float)(bias + kBucketMagic);
    } else {
      q->bias = (float)(-lo * scale);
    }
    q->t = t;
    q->scale = (float)scale;
    q->nb = nb;
    q->centred = centred;
    return true;
  }
  return false;
}

std::vector<double> midpoints(const std::vector<double>& c) {
  std::vector<double> m(c.size() - 1);
  for (size_t k = 0; k + 1 < c.size(); ++k) m[k] = 0.5 * (c[k] + c[k + 1]);
  return m;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

struct octo_codebook {
  int d = 0, b = 0, bx = 0, be = 0, br = 0, T = 0, bt = 0, W = 0;
  uint64_t seed = 0, cb_seed = 0;
  int qjl = 0, mc = 0, device = -1;
  bool kernels = false;  // a compiled kernel exists for (d, allocation)
  std::vector<double> c_xi, c_eta, c_rho;
  std::vector<int8_t> signs;
  std::vector<float> S;
  uint32_t sign_bits[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  void* dev = nullptr;
  DevTables tables{};
  int64_t table_entries[TAB_COUNT] = {0, 0, 0, 0, 0, 0, 0};  // entries per table (octo_table)
  HostB1 qx, qe;           // host copies of the xi / eta bucket tables (octo_debug_bucket_index)
  float qjl_kappa = 0.f;   // QJL estimator constant of S
};

namespace {

// Bytes of zeros past the last table of the device allocation: a read a
// little past a table's end stays inside the allocation.
constexpr size_t kTableGuardBytes = 1024;

// The kernels' tables, built on the host.
struct HostTables {
  HostB1 qx, qe, qr2;
  std::vector<double> rho_mid2;   // squared rho midpoints
  std::vector<float> dir, rho, trip, st;
  std::vector<_Float16> s16;
};

octo_status make_host_tables(octo_codebook* cb, HostTables& h) {
  HostB1& qx = h.qx;
  HostB1& qe = h.qe;
  HostB1& qr2 = h.qr2;
  if (!build_bucket1(midpoints(cb->c_xi), -1.0, 1.0, true, &qx) ||
      !build_bucket1(midpoints(cb->c_eta), -1.0, 1.0, true, &qe))
    return fail(OCTO_ERR_UNSUPPORTED, "no bucket table fits the xi/eta midpoints");
  std::vector<double> m2 = midpoints(cb->c_rho);
  for (double& m : m2) m = m * m;
  const double hi = m2.empty() ? 1.0 : std::min(1.0, 1.25 * m2.back() + 1e-3);
  if (!build_bucket1(m2, 0.0, hi, false, &qr2))
    return fail(OCTO_ERR_UNSUPPORTED, "no bucket table fits the rho midpoints");
  h.rho_mid2 = m2;

  const int ndir = 1 << (cb->bx + cb->be);
  std::vector<float>& dir = h.dir;
  dir.resize(4 * (size_t)ndir);
  for (int ie = 0; ie < (1 << cb->be); ++ie)
    for (int ix = 0; ix < (1 << cb->bx); ++ix) {
      double v[3];
      octa_decode(cb->c_xi[ix], cb->c_eta[ie], v);
      const size_t o = 4 * (size_t)(ix | (ie << cb->bx));
      dir[o] = (float)v[0];
      dir[o + 1] = (float)v[1];
      dir[o + 2] = (float)v[2];
      dir[o + 3] = 0.f;
    }
  h.rho.assign(cb->c_rho.begin(), cb->c_rho.end());
  // rho^ n^ per full triplet code, for streams of at most 10 bits per triplet
  std::vector<float>& trip = h.trip;
  if (cb->bt <= 10) {
    trip.resize(4 * ((size_t)1 << cb->bt));
    for (int code = 0; code < (1 << cb->bt); ++code) {
      const int ix = code & ((1 << cb->bx) - 1);
      const int ie = (code >> cb->bx) & ((1 << cb->be) - 1);
      const int ir = code >> (cb->bx + cb->be);
      double v[3];
      octa_decode(cb->c_xi[ix], cb->c_eta[ie], v);
      for (int c = 0; c < 3; ++c) trip[4 * (size_t)code + c] = (float)(cb->c_rho[ir] * v[c]);
      trip[4 * (size_t)code + 3] = 0.f;
    }
  }

  // QJL matrix for the encoder's matrix-core projection: S = S_hi + S_lo with
  // S_hi = f16(S) and S_lo = f16(S - S_hi) (round to nearest even), planes
  // [hi | lo], each d x d row-major.  S_hi + S_lo carries 22 bits of S.
  std::vector<_Float16>& s16 = h.s16;
  if (!cb->S.empty()) {
    s16.resize(2 * cb->S.size());
    for (size_t i = 0; i < cb->S.size(); ++i) {
      const _Float16 h = (_Float16)cb->S[i];
      s16[i] = h;
      s16[cb->S.size() + i] = (_Float16)(cb->S[i] - (float)h);
    }
  }

  // S transposed (column-major S): the decode kernels form p = S q' with lane
  // j reading element j of column c, one contiguous row of St per load.
  std::vector<float>& st = h.st;
  if (!cb->S.empty()) {
    const int d = cb->d;
    st.resize(cb->S.size());
    for (int j = 0; j < d; ++j)
      for (int c = 0; c < d; ++c) st[(size_t)c * d + j] = cb->S[(size_t)j * d + c];
  }
  int64_t* n = cb->table_entries;
  n[TAB_DIR] = ndir;
  n[TAB_TRIP] = (int64_t)trip.size() / 4;
  n[TAB_RHO] = (int64_t)h.rho.size();
  n[TAB_QX] = (int64_t)qx.t.size() / 2;
  n[TAB_QE] = (int64_t)qe.t.size() / 2;
  n[TAB_QR2] = (int64_t)qr2.t.size() / 2;
  n[TAB_S16] = (int64_t)s16.size() / 8;
  return OCTO_OK;
}

octo_status upload_tables(octo_codebook* cb, const HostTables& h) {
  const HostB1& qx = h.qx;
  const HostB1& qe = h.qe;
  const HostB1& qr2 = h.qr2;
  const std::vector<float>& dir = h.dir;
  const std::vector<float>& rho = h.rho;
  const std::vector<float>& trip = h.trip;
  const std::vector<float>& st = h.st;
  const std::vector<_Float16>& s16 = h.s16;
  // One device allocation, 256-byte aligned regions, then a zeroed guard.
  struct Region { const void* src; size_t bytes; size_t off; };
  std::vector<Region> reg = {
      {dir.data(), dir.size() * 4, 0},           {rho.data(), rho.size() * 4, 0},
      {qx.t.data(), qx.t.size() * 4, 0},         {qe.t.data(), qe.t.size() * 4, 0},
      {qr2.t.data(), qr2.t.size() * 4, 0},
      {st.empty() ? nullptr : st.data(), st.size() * 4, 0},
      {trip.empty() ? nullptr : trip.data(), trip.size() * 4, 0},
      {s16.empty() ? nullptr : s16.data(), s16.size() * 2, 0}};
  size_t total = 0;
  for (auto& r : reg) { r.off = total; total += align256(r.bytes); }
  const size_t guard_off = total;
  total += kTableGuardBytes;
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess) return fail(OCTO_ERR_HIP, "hipGetDevice failed");
  if (hipSetDevice(cb->device) != hipSuccess)
    return fail(OCTO_ERR_HIP, "hipSetDevice(" + std::to_string(cb->device) + ") failed");
  // the static decode scratch of this device is resolved at set-up, with the
  // device current (octo_decode_attn_static)
  void* scr = nullptr;
  hipError_t e = static_scratch(cb->device, &scr);
  if (e != hipSuccess) {
    hipSetDevice(prev);
    return fail(OCTO_ERR_HIP, std::string("static scratch address: ") + hipGetErrorString(e));
  }
  void* dev = nullptr;
  e = hipMalloc(&dev, total);
  if (e != hipSuccess) {
    hipSetDevice(prev);
    return fail(OCTO_ERR_NOMEM, std::string("hipMalloc of codebook tables: ") + hipGetErrorString(e));
  }
  e = hipMemset((char*)dev + guard_off, 0, kTableGuardBytes);
  for (auto& r : reg) {
    if (r.bytes == 0 || e != hipSuccess) continue;
    e = hipMemcpy((char*)dev + r.off, r.src, r.bytes, hipMemcpyHostToDevice);
  }
  hipSetDevice(prev);
  if (e != hipSuccess) {
    hipFree(dev);
    return fail(OCTO_ERR_HIP, std::string("upload of codebook tables: ") + hipGetErrorString(e));
  }
  cb->dev = dev;
  char* base = (char*)dev;
  DevTables& t = cb->tables;
  t.dirtab = (const float4*)(base + reg[0].off);
  t.rho_tab = (const float*)(base + reg[1].off);
  auto qt = [&](const HostB1& h, int r) {
    Bucket1 q;
    q.t = (const uint2*)(base + reg[r].off);
    q.scale = h.scale;
    q.bias = h.bias;
    q.nb = h.nb;
    return q;
  };
  t.qx = qt(qx, 2);
  t.qe = qt(qe, 3);
  t.qr2 = qt(qr2, 4);
  t.St = st.empty() ? nullptr : (const float*)(base + reg[5].off);
  t.trip_tab = trip.empty() ? nullptr : (const float4*)(base + reg[6].off);
  t.S16 = s16.empty() ? nullptr : (const uint4*)(base + reg[7].off);
  for (int k = 0; k < 8; ++k) t.sign_bits[k] = cb->sign_bits[k];
  t.qjl_kappa = cb->qjl_kappa;
  for (int k = 0; k < 3; ++k)
    t.rho_mid2[k] = k < (int)h.rho_mid2.size() ? (float)h.rho_mid2[k] : INFINITY;
  return OCTO_OK;
}

int dtype_size(octo_dtype t) { return t == OCTO_F32 ? 4 : 2; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

octo_status check_cb(const octo_codebook* cb) {
  if (!cb) return fail(OCTO_ERR_INVALID_ARG, "codebook is NULL");
  if (cb->device < 0 || !cb->dev)
    return fail(OCTO_ERR_INVALID_ARG, "host-only codebook: build it with device >= 0");
  if (!cb->kernels) return fail(OCTO_ERR_UNSUPPORTED, "no kernel for this d / allocation");
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return fail(OCTO_ERR_HIP, "hipGetDevice failed");
  if (cur != cb->device)
    return fail(OCTO_ERR_INVALID_ARG, "current HIP device " + std::to_string(cur) +
                                          " differs from the codebook's device " +
                                          std::to_string(cb->device));
  return OCTO_OK;
}

octo_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return OCTO_OK;
  return fail(OCTO_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// The single-query kernels handle up to 4 query heads of a KV head per pass.
int head_passes(int G) { return (G + 3) / 4; }

struct Split { int n_split, tiles_per_split; };

// Blocks the single-query attention aims at (4-wave blocks, two resident per
// compute unit).
#ifndef OCTO_ATTN_TARGET_BLOCKS
#define OCTO_ATTN_TARGET_BLOCKS 1024
#endif

Split attn_split(int64_t n_keys, int64_t n_seq, int passes) {
  const int64_t ntile = std::max<int64_t>(1, (n_keys + kTile - 1) / kTile);
  const int64_t rows = std::max<int64_t>(1, n_seq * passes);
  int64_t ns = (OCTO_ATTN_TARGET_BLOCKS + rows - 1) / rows;
  ns = std::min<int64_t>(ns, (ntile + 7) / 8);
  ns = std::max<int64_t>(ns, 1);
  const int64_t tps = (ntile + ns - 1) / ns;
  ns = (ntile + tps - 1) / tps;
  return {(int)ns, (int)tps};
}

// Compute units of the current device (one multi-query workgroup each).
int64_t device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

// Multi-query split: the number of splits that minimises the tile steps of
// the slowest compute unit, ceil(rows * n_split / CUs) * tiles_per_split;
// among equal costs the fewest splits (least partial traffic).
Split mq_split(int64_t n_keys, int d, int b, int64_t rows) {
  const int kt = mq_tile_keys(d, b);
  const int64_t ntile = std::max<int64_t>(1, (n_keys + kt - 1) / kt);
  const int64_t slots = device_cus();
  rows = std::max<int64_t>(1, rows) * mq_value_parts(d);   // workgroups per split
  int64_t best_ns = 1, best_cost = INT64_MAX;
  for (int64_t ns = 1; ns <= std::min<int64_t>(ntile, kMaxSplit); ++ns) {
    const int64_t tps = (ntile + ns - 1) / ns;
    if ((ntile + tps - 1) / tps != ns) continue;  // same tiles per split as a smaller count
    const int64_t cost = ((rows * ns + slots - 1) / slots) * tps;
    if (cost < best_cost) { best_cost = cost; best_ns = ns; }
  }
  const int64_t tps = (ntile + best_ns - 1) / best_ns;
  return {(int)best_ns, (int)tps};
}

int64_t mq_rows(int B, int Hq, int n_q) {
  const int qb = mq_block_queries();
  return (int64_t)B * Hq * ((n_q + qb - 1) / qb);
}

struct WsLayout { size_t qrot, qp, part, total; };

WsLayout ws_layout(const octo_codebook* cb, int mode, int B, int Hq, int Hkv, int n_q,
                   int64_t n_keys) {
  WsLayout w{};
  const size_t rows = (size_t)B * Hq * n_q;
  w.qrot = 0;
  size_t off = align256(rows * 3 * cb->T * sizeof(float));
  w.qp = off;
  if (cb->qjl) off += align256(rows * cb->d * sizeof(float));
  w.part = off;
  if (mode == 1 && n_q > 1) {
    const Split sp = mq_split(n_keys, cb->d, cb->b, mq_rows(B, Hq, n_q));
    off += align256(rows * (size_t)sp.n_split * (cb->d + 2) * sizeof(float));
  } else if (mode == 1) {
    const int G = Hkv > 0 ? Hq / Hkv : 1;
    const Split sp = attn_split(n_keys, (int64_t)B * Hkv, head_passes(std::max(G, 1)));
    off += align256(rows * (size_t)sp.n_split * (cb->d + 2) * sizeof(float));
  }
  w.total = off;
  return w;
}

}  // namespace

extern "C" {

const char* octo_status_str(octo_status s) {
  switch (s) {
    case OCTO_OK: return "OCTO_OK";
    case OCTO_ERR_INVALID_ARG: return "OCTO_ERR_INVALID_ARG";
    case OCTO_ERR_UNSUPPORTED: return "OCTO_ERR_UNSUPPORTED";
    case OCTO_ERR_HIP: return "OCTO_ERR_HIP";
    case OCTO_ERR_NOMEM: return "OCTO_ERR_NOMEM";
    case OCTO_ERR_WORKSPACE: return "OCTO_ERR_WORKSPACE";
  }
  return "OCTO_ERR_UNKNOWN";
}

const char* octo_last_error(void) { return g_last_error.c_str(); }

octo_status octo_codebook_build(const octo_params* p, octo_codebook** out) {
  if (!p || !out) return fail(OCTO_ERR_INVALID_ARG, "params/out is NULL");
  *out = nullptr;
  const int d = p->d, b = p->b;
  if (d < 4 || d > 1024 || (d & (d - 1)))
    return fail(OCTO_ERR_INVALID_ARG, "d must be a power of two in [4, 1024]");
  const bool dflt = p->b_xi < 0 || p->b_eta < 0 || p->b_rho < 0;
  const int bx = dflt ? b + 1 : p->b_xi, be = dflt ? b + 1 : p->b_eta, br = dflt ? b - 1 : p->b_rho;
  if (b < 1 || b > 8 || bx < 1 || bx > 8 || be < 1 || be > 8 || br < 0 || br > 8)
    return fail(OCTO_ERR_INVALID_ARG, "bit allocation out of range");
  if (p->mc_vectors < 0) return fail(OCTO_ERR_INVALID_ARG, "mc_vectors < 0");
  const bool kernels = (d == 64 || d == 128 || d == 256) && (b >= 1 && b <= 5) && bx == b + 1 &&
                       be == b + 1 && br == b - 1;
  if (p->device >= 0 && !kernels)
    return fail(OCTO_ERR_UNSUPPORTED,
                "kernels exist for d in {64,128,256}, b in 1..5 and the (b+1,b+1,b-1) allocation; "
                "build with device = -1 for host-only tables");
  octo_codebook* cb = new (std::nothrow) octo_codebook();
  if (!cb) return fail(OCTO_ERR_NOMEM, "host allocation failed");
  cb->d = d;
  cb->b = b;
  cb->bx = bx;
  cb->be = be;
  cb->br = br;
  cb->T = (d + 2) / 3;
  cb->bt = bx + be + br;
  cb->W = (cb->T * cb->bt + 31) / 32;
  cb->seed = p->seed;
  cb->cb_seed = p->cb_seed;
  cb->qjl = p->qjl ? 1 : 0;
  cb->mc = p->mc_vectors ? p->mc_vectors : 65536;
  cb->device = p->device;
  cb->kernels = kernels;

  try {
    // WHT signs: s_j = +1 if the low bit of draw j is 0 ([YL] 旋转魔法).
    cb->signs.resize(d);
    for (int j = 0; j < d; ++j) {
      const bool neg = splitmix_out(p->seed ^ kTagSigns, (uint64_t)j) & 1ull;
      cb->signs[j] = neg ? -1 : 1;
      if (neg && j < 256) cb->sign_bits[j >> 5] |= 1u << (j & 31);
    }
    // The centroid tables depend only on (d, allocation, cb_seed, samples):
    // the last fit is kept, so codebooks that differ only in `seed` (signs,
    // QJL matrix) reuse it.
    static std::mutex fit_mutex;
    static std::vector<int64_t> fit_key;
    static std::vector<double> fit_xi, fit_eta, fit_rho;
    const std::vector<int64_t> key = {d, bx, be, br, (int64_t)p->cb_seed, cb->mc};
    bool fitted = false;
    {
      std::lock_guard<std::mutex> lock(fit_mutex);
      if (key == fit_key) {
        cb->c_xi = fit_xi;
        cb->c_eta = fit_eta;
        cb->c_rho = fit_rho;
        fitted = true;
      }
    }
    // Monte-Carlo samples of the rotated triplet marginals: normalised
    // Gaussian vectors are uniform on the sphere, so their rotation is too.
    const int T = cb->T, M = fitted ? 0 : cb->mc;
    std::vector<double> g((size_t)d);
    std::vector<double> rho;
    std::vector<double> dirs;
    rho.reserve((size_t)M * T);
    dirs.reserve((size_t)M * T * 4);
    std::vector<double> xs((size_t)M * T), es((size_t)M * T);
    std::vector<double> all((size_t)M * d);
    gaussians(p->cb_seed, kTagMC, (size_t)M * d, all.data());
    size_t n = 0;
    for (int v = 0; v < M; ++v) {
      const double* gv = &all[(size_t)v * d];
      double ss = 0.0;
      for (int j = 0; j < d; ++j) ss += gv[j] * gv[j];
      const double nrm = std::sqrt(ss);
      for (int i = 0; i < T; ++i) {
        double t[3];
        for (int c = 0; c < 3; ++c) t[c] = (3 * i + c < d) ? gv[3 * i + c] / nrm : 0.0;
        const double r = std::sqrt(t[0] * t[0] + t[1] * t[1] + t[2] * t[2]);
        double nx = 0, ny = 0, nz = 1;
        if (r > 0) { nx = t[0] / r; ny = t[1] / r; nz = t[2] / r; }
        double xi, eta;
        octa_encode(nx, ny, nz, &xi, &eta);
        rho.push_back(r);
        xs[n] = xi;
        es[n] = eta;
        ++n;
      }
    }
    // xi and eta pooled and symmetrised.
    dirs.insert(dirs.end(), xs.begin(), xs.end());
    dirs.insert(dirs.end(), es.begin(), es.end());
    const size_t half = dirs.size();
    for (size_t i = 0; i < half; ++i) dirs.push_back(-dirs[i]);
    std::vector<double>().swap(all);
    if (!fitted) {
      std::sort(rho.begin(), rho.end());
      std::sort(dirs.begin(), dirs.end());
      cb->c_xi = antisymmetrize(lloyd_max_sorted(dirs, 1 << bx));
      cb->c_eta = (be == bx) ? cb->c_xi : antisymmetrize(lloyd_max_sorted(dirs, 1 << be));
      cb->c_rho = lloyd_max_sorted(rho, 1 << br);
      std::lock_guard<std::mutex> lock(fit_mutex);
      fit_key = key;
      fit_xi = cb->c_xi;
      fit_eta = cb->c_eta;
      fit_rho = cb->c_rho;
    }
    if (cb->qjl) {
      std::vector<double> s((size_t)d * d);
      gaussians(p->seed, kTagQJL, s.size(), s.data());
      // The residual's random rotation ([YL] 可选的残差修正): the Haar-random
      // orthogonal P = Q of the seeded Gaussian matrix G = Q R with R's
      // diagonal positive (Mezzadri 2007), i.e. Gram-Schmidt of G's columns
      // (each projected out twice), kept as S = sqrt(d) P.
      std::vector<double> col((size_t)d * d);  // col[j * d + i] = G[i][j]
      for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) col[(size_t)j * d + i] = s[(size_t)i * d + j];
      for (int j = 0; j < d; ++j) {
        double* v = &col[(size_t)j * d];
        for (int pass = 0; pass < 2; ++pass)
          for (int k = 0; k < j; ++k) {
            const double* qk = &col[(size_t)k * d];
            double dot = 0.0;
            for (int i = 0; i < d; ++i) dot += qk[i] * v[i];
            for (int i = 0; i < d; ++i) v[i] -= dot * qk[i];
          }
        double nn = 0.0;
        for (int i = 0; i < d; ++i) nn += v[i] * v[i];
        const double inv = 1.0 / std::sqrt(nn);
        for (int i = 0; i < d; ++i) v[i] *= inv;
      }
      const double sd = std::sqrt((double)d);
      cb->S.resize((size_t)d * d);
      for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) cb->S[(size_t)i * d + j] = (float)(sd * col[(size_t)j * d + i]);
      // kappa_d = 1 / (d sqrt(d) E|u_1|), E|u_1| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))
      const double mean_abs = std::exp(std::lgamma(0.5 * d) - std::lgamma(0.5 * (d + 1))) / std::sqrt(M_PI);
      cb->qjl_kappa = (float)(1.0 / ((double)d * sd * mean_abs));
    }
  } catch (const std::bad_alloc&) {
    delete cb;
    return fail(OCTO_ERR_NOMEM, "host allocation failed during codebook build");
  }
  if (cb->kernels) {
    // the kernels' tables: uploaded for a device codebook; for a host-only
    // one only their sizes are kept (octo_codebook_table_entries)
    HostTables h;
    octo_status st = make_host_tables(cb, h);
    if (st == OCTO_OK) {
      cb->qx = h.qx;
      cb->qe = h.qe;
    }
    if (st == OCTO_OK && cb->device >= 0) st = upload_tables(cb, h);
    if (st != OCTO_OK && cb->device >= 0) {
      delete cb;
      return st;
    }
  }
  *out = cb;
  return OCTO_OK;
}

octo_status octo_codebook_free(octo_codebook* cb) {
  if (!cb) return OCTO_OK;
  if (cb->dev) {
    int prev = 0;
    hipGetDevice(&prev);
    hipSetDevice(cb->device);
    hipFree(cb->dev);
    hipSetDevice(prev);
  }
  delete cb;
  return OCTO_OK;
}

octo_status octo_codebook_layout(const octo_codebook* cb, octo_layout* o) {
  if (!cb || !o) return fail(OCTO_ERR_INVALID_ARG, "NULL argument");
  o->d = cb->d;
  o->n_triplets = cb->T;
  o->pad_dim = 3 * cb->T;
  o->b_xi = cb->bx;
  o->b_eta = cb->be;
  o->b_rho = cb->br;
  o->bits_per_triplet = cb->bt;
  o->bits_per_key = cb->T * cb->bt;
  o->words_per_key = cb->W;
  o->tile_keys = kTile;
  o->qjl = cb->qjl;
  o->qjl_words_per_key = cb->qjl ? cb->d / 32 : 0;
  o->packed_bytes_per_key_alloc = (size_t)cb->W * 4;
  return OCTO_OK;
}

octo_status octo_codebook_export(const octo_codebook* cb, double* c_xi, double* c_eta,
                                 double* c_rho, int8_t* signs, float* qjl_S) {
  if (!cb) return fail(OCTO_ERR_INVALID_ARG, "codebook is NULL");
  if (c_xi) std::memcpy(c_xi, cb->c_xi.data(), cb->c_xi.size() * sizeof(double));
  if (c_eta) std::memcpy(c_eta, cb->c_eta.data(), cb->c_eta.size() * sizeof(double));
  if (c_rho) std::memcpy(c_rho, cb->c_rho.data(), cb->c_rho.size() * sizeof(double));
  if (signs) std::memcpy(signs, cb->signs.data(), cb->signs.size());
  if (qjl_S) {
    if (cb->S.empty()) return fail(OCTO_ERR_INVALID_ARG, "codebook has no QJL matrix");
    std::memcpy(qjl_S, cb->S.data(), cb->S.size() * sizeof(float));
  }
  return OCTO_OK;
}

int64_t octo_codebook_table_entries(const octo_codebook* cb, int table) {
  if (!cb || table < 0 || table >= TAB_COUNT) return -1;
  return cb->table_entries[table];
}

octo_status octo_debug_bucket_index(const octo_codebook* cb, int table, const float* x, int64_t n,
                                    uint32_t* out) {
  if (!cb || (n > 0 && (!x || !out))) return fail(OCTO_ERR_INVALID_ARG, "NULL argument");
  if (table != TAB_QX && table != TAB_QE)
    return fail(OCTO_ERR_INVALID_ARG, "table must be OCTO_TABLE_QX or OCTO_TABLE_QE");
  const HostB1& q = table == TAB_QX ? cb->qx : cb->qe;
  if (q.t.empty()) return fail(OCTO_ERR_UNSUPPORTED, "codebook has no encoder tables");
  const int64_t entries = (int64_t)q.t.size() / 2;
  for (int64_t i = 0; i < n; ++i) {
    // the device formula: one fma, its bits less the magic, one compare
    uint32_t bits;
    const float f = std::fmaf(x[i], q.scale, q.bias);
    std::memcpy(&bits, &f, 4);
    const int64_t b = (int64_t)bits - (int64_t)kBucketMagicBits;
    if (b < 0 || b >= entries)
      return fail(OCTO_ERR_INVALID_ARG, "x[" + std::to_string(i) + "] lies outside the table's range");
    float mid;
    std::memcpy(&mid, &q.t[2 * b + 1], 4);
    out[i] = q.t[2 * b] + (x[i] > mid ? 1u : 0u);
  }
  return OCTO_OK;
}

octo_status octo_debug_lds_copy(int index, octo_lds_copy* out) {
  static const std::vector<LdsCopyRec> recs = [] {
    std::vector<LdsCopyRec> v(1024);
    int n = lds_copies_decode(v.data(), (int)v.size());
    n += lds_copies_mq(v.data() + n, (int)v.size() - n);
    n += lds_copies_encode(v.data() + n, (int)v.size() - n);
    v.resize(n);
    return v;
  }();
  if (!out) return fail(OCTO_ERR_INVALID_ARG, "out is NULL");
  if (index < 0 || index >= (int)recs.size())
    return fail(OCTO_ERR_INVALID_ARG, "index past the last table copy (" + std::to_string(recs.size()) + ")");
  const LdsCopyRec& r = recs[index];
  out->kernel = r.kernel;
  out->d = r.d;
  out->b = r.b;
  out->qjl = r.qjl;
  out->table = r.table;
  out->lds_slots = r.lds_slots;
  out->slots_written = r.slots_written;
  out->entries_read = r.entries_read;
  out->copied = r.copied;
  out->threads = r.threads;
  out->masked = r.masked;
  return OCTO_OK;
}

size_t octo_packed_bytes(const octo_codebook* cb, int64_t n_seq, int64_t cap) {
  if (!cb || n_seq < 0 || cap < 0) return 0;
  return (size_t)n_seq * (size_t)((cap + kTile - 1) / kTile) * kTile * cb->W * 4;
}

size_t octo_qjl_bits_bytes(const octo_codebook* cb, int64_t n_seq, int64_t cap) {
  if (!cb || n_seq < 0 || cap < 0 || !cb->qjl) return 0;
  return (size_t)n_seq * (size_t)((cap + kTile - 1) / kTile) * kTile * (cb->d / 32) * 4;
}

static octo_status encode_impl(const octo_codebook* cb, const void* keys, octo_dtype kdt,
                               int64_t n_seq, int64_t n_new, int64_t seq_stride,
                               int64_t key_stride, int64_t pos0, int64_t cap, void* packed,
                               float* gamma, void* qjl_bits, uint16_t* qjl_norm, void* stream,
                               bool joint) {
  octo_status st = check_cb(cb);
  if (st != OCTO_OK) return st;
  if (kdt != OCTO_F32 && kdt != OCTO_BF16 && kdt != OCTO_F16)
    return fail(OCTO_ERR_INVALID_ARG, "unknown key dtype");
  if (n_seq < 0 || n_new < 0 || pos0 < 0 || cap <= 0 || cap % kTile)
    return fail(OCTO_ERR_INVALID_ARG, "need n_seq, n_new, pos0 >= 0 and cap a positive multiple of 64");
  if (pos0 + n_new > cap) return fail(OCTO_ERR_INVALID_ARG, "pos0 + n_new exceeds cap");
  if (n_seq > 65535) return fail(OCTO_ERR_INVALID_ARG, "n_seq > 65535");
  if (n_seq == 0 || n_new == 0) return OCTO_OK;
  const int es = dtype_size(kdt);
  if (!keys || !packed || !gamma) return fail(OCTO_ERR_INVALID_ARG, "NULL keys/packed/gamma");
  if (key_stride < cb->d || (n_seq > 1 && seq_stride < 0))
    return fail(OCTO_ERR_INVALID_ARG, "key_stride < d or seq_stride < 0");
  if (!aligned(keys, 16) || (key_stride * es) % 16 || (seq_stride * es) % 16)
    return fail(OCTO_ERR_INVALID_ARG, "key rows must be 16-byte aligned");
  if (!aligned(packed, 16) || !aligned(gamma, 4))
    return fail(OCTO_ERR_INVALID_ARG, "packed must be 16-byte and gamma 4-byte aligned");
  if ((qjl_bits == nullptr) != (qjl_norm == nullptr))
    return fail(OCTO_ERR_INVALID_ARG, "pass both QJL buffers or neither");
  if (qjl_bits && !cb->qjl) return fail(OCTO_ERR_INVALID_ARG, "codebook built without QJL");
  if (qjl_bits && (!aligned(qjl_bits, 16) || !aligned(qjl_norm, 2)))
    return fail(OCTO_ERR_INVALID_ARG, "QJL buffers misaligned");
  EncodeArgs a{};
  a.t = cb->tables;
  a.keys = keys;
  a.seq_stride = seq_stride;
  a.key_stride = key_stride;
  a.n_new = n_new;
  a.pos0 = pos0;
  a.cap = cap;
  a.seq_count = n_seq;
  a.packed = (uint32_t*)packed;
  a.gamma = gamma;
  a.qjl_bits = (uint32_t*)qjl_bits;
  a.qjl_norm = qjl_norm;
  return hip_status(launch_encode(cb->d, cb->b, (int)kdt, qjl_bits != nullptr, joint, a, n_seq,
                                  (hipStream_t)stream),
                    "encode launch");
}

octo_status octo_encode(const octo_codebook* cb, const void* keys, octo_dtype kdt, int64_t n_seq,
                        int64_t n_new, int64_t seq_stride, int64_t key_stride, int64_t pos0,
                        int64_t cap, void* packed, float* gamma, void* qjl_bits,
                        uint16_t* qjl_norm, void* stream) {
  return encode_impl(cb, keys, kdt, n_seq, n_new, seq_stride, key_stride, pos0, cap, packed, gamma,
                     qjl_bits, qjl_norm, stream, false);
}

octo_status octo_encode_joint(const octo_codebook* cb, const void* keys, octo_dtype kdt,
                              int64_t n_seq, int64_t n_new, int64_t seq_stride,
                              int64_t key_stride, int64_t pos0, int64_t cap, void* packed,
                              float* gamma, void* qjl_bits, uint16_t* qjl_norm, void* stream) {
  return encode_impl(cb, keys, kdt, n_seq, n_new, seq_stride, key_stride, pos0, cap, packed, gamma,
                     qjl_bits, qjl_norm, stream, true);
}

size_t octo_decode_workspace_bytes(const octo_codebook* cb, int mode, int B, int Hq, int Hkv,
                                   int n_q, int64_t n_keys) {
  if (!cb || B < 0 || Hq < 0 || Hkv <= 0 || n_q < 0 || n_keys < 0) return 0;
  return ws_layout(cb, mode, B, Hq, Hkv, n_q, n_keys).total;
}

static octo_status check_decode_common(const octo_codebook* cb, const void* q, octo_dtype qdt,
                                       int B, int Hq, int Hkv, const void* packed,
                                       const float* gamma, const void* qjl_bits,
                                       const uint16_t* qjl_norm, int64_t n_keys, int64_t cap,
                                       void* workspace) {
  octo_status st = check_cb(cb);
  if (st != OCTO_OK) return st;
  if (qdt != OCTO_F32 && qdt != OCTO_BF16 && qdt != OCTO_F16)
    return fail(OCTO_ERR_INVALID_ARG, "unknown query dtype");
  if (B < 0 || Hq < 0 || Hkv <= 0 || (Hq % Hkv))
    return fail(OCTO_ERR_INVALID_ARG, "need B >= 0, Hkv > 0 and Hq a multiple of Hkv");
  if ((int64_t)B * Hkv > 65535) return fail(OCTO_ERR_INVALID_ARG, "B * Hkv > 65535");
  if (n_keys < 0 || cap <= 0 || cap % kTile || n_keys > cap)
    return fail(OCTO_ERR_INVALID_ARG, "need 0 <= n_keys <= cap and cap a positive multiple of 64");
  if (!q || !packed || !gamma) return fail(OCTO_ERR_INVALID_ARG, "NULL q/packed/gamma");
  if (!aligned(q, 4) || !aligned(packed, 16) || !aligned(gamma, 4))
    return fail(OCTO_ERR_INVALID_ARG, "q/packed/gamma misaligned");
  if ((qjl_bits == nullptr) != (qjl_norm == nullptr))
    return fail(OCTO_ERR_INVALID_ARG, "pass both QJL buffers or neither");
  if (qjl_bits && !cb->qjl) return fail(OCTO_ERR_INVALID_ARG, "codebook built without QJL");
  if (qjl_bits && (!aligned(qjl_bits, 16) || !aligned(qjl_norm, 2)))
    return fail(OCTO_ERR_INVALID_ARG, "qjl_bits/qjl_norm misaligned");
  if (!workspace || !aligned(workspace, 256))
    return fail(OCTO_ERR_WORKSPACE, "workspace missing or not 256-byte aligned");
  return OCTO_OK;
}

octo_status octo_decode_logits(const octo_codebook* cb, const void* q, octo_dtype qdt, int B,
                               int Hq, int Hkv, const void* packed, const float* gamma,
                               const void* qjl_bits, const uint16_t* qjl_norm, int64_t n_keys,
                               int64_t cap, float* logits, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return octo_decode_logits_stages(cb, q, qdt, B, Hq, Hkv, packed, gamma, qjl_bits, qjl_norm,
                                   n_keys, cap, logits, workspace, workspace_bytes, stream,
                                   OCTO_STAGE_ALL);
}

octo_status octo_decode_logits_stages(const octo_codebook* cb, const void* q, octo_dtype qdt,
                                      int B, int Hq, int Hkv, const void* packed,
                                      const float* gamma, const void* qjl_bits,
                                      const uint16_t* qjl_norm, int64_t n_keys, int64_t cap,
                                      float* logits, void* workspace, size_t workspace_bytes,
                                      void* stream, int stages) {
  octo_status st = check_decode_common(cb, q, qdt, B, Hq, Hkv, packed, gamma, qjl_bits, qjl_norm,
                                       n_keys, cap, workspace);
  if (st != OCTO_OK) return st;
  if (!logits || !aligned(logits, 4)) return fail(OCTO_ERR_INVALID_ARG, "logits NULL/misaligned");
  const WsLayout wl = ws_layout(cb, 0, B, Hq, Hkv, 1, n_keys);
  if (workspace_bytes < wl.total) return fail(OCTO_ERR_WORKSPACE, "workspace too small");
  if (B == 0 || Hq == 0 || n_keys == 0) return OCTO_OK;
  hipStream_t s = (hipStream_t)stream;
  const bool qjl = qjl_bits != nullptr;
  // the rotation runs in the fused kernel's prologue (OCTO_STAGE_ROTATE is a no-op here)
  if (!(stages & OCTO_STAGE_MAIN)) return OCTO_OK;
  const int G = Hq / Hkv;
  DecodeArgs a{};
  a.t = cb->tables;
  a.q = q;
  a.qdt = (int)qdt;
  a.mult = 1.0f;
  a.packed = (const uint32_t*)packed;
  a.gamma = gamma;
  a.qjl_bits = (const uint32_t*)qjl_bits;
  a.qjl_norm = qjl_norm;
  a.n_keys = n_keys;
  a.cap = cap;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = G;
  a.logits = logits;
  const int64_t n_seq = (int64_t)B * Hkv;
  const int64_t ntile = (n_keys + kTile - 1) / kTile;
  const int64_t rows = n_seq * head_passes(G);
  int64_t nbx = (2048 + rows - 1) / rows;
  nbx = std::max<int64_t>(1, std::min<int64_t>(nbx, (ntile + 3) / 4));
  return hip_status(launch_logits(cb->d, cb->b, qjl, a, n_seq, (int)nbx, s), "logits launch");
}

octo_status octo_decode_attn(const octo_codebook* cb, const void* q, octo_dtype qdt, int B,
                             int Hq, int Hkv, int n_q, const void* packed, const float* gamma,
                             const void* qjl_bits, const uint16_t* qjl_norm, const void* v,
                             octo_dtype vdt, int64_t n_keys, int64_t cap, float scale, float* out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return octo_decode_attn_stages(cb, q, qdt, B, Hq, Hkv, n_q, packed, gamma, qjl_bits, qjl_norm, v,
                                 vdt, n_keys, cap, scale, out, workspace, workspace_bytes, stream,
                                 OCTO_STAGE_ALL);
}

// The new-key arguments of a decode step with append (see DecodeArgs).
struct AppendKey {
  const void* keys;
  int64_t stride;
  void* packed;
  float* gamma;
};

static octo_status decode_attn_impl(const octo_codebook* cb, const void* q, octo_dtype qdt, int B,
                                    int Hq, int Hkv, int n_q, const void* packed,
                                    const float* gamma, const void* qjl_bits,
                                    const uint16_t* qjl_norm, const void* v, octo_dtype vdt,
                                    int64_t n_keys, int64_t cap, float scale, float* out,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    int stages, const AppendKey* app);

static_assert(OCTO_STATIC_SCRATCH_BYTES == kStaticScratchBytes, "one size of the static scratch");

octo_status octo_decode_attn_static(const octo_codebook* cb, const void* q, octo_dtype qdt, int B,
                                    int Hq, int Hkv, int n_q, const void* packed,
                                    const float* gamma, const void* qjl_bits,
                                    const uint16_t* qjl_norm, const void* v, octo_dtype vdt,
                                    int64_t n_keys, int64_t cap, float scale, float* out,
                                    void* stream) {
  octo_status st = check_cb(cb);
  if (st != OCTO_OK) return st;
  if (B < 0 || Hq < 0 || Hkv <= 0 || n_q < 1 || n_keys < 0)
    return fail(OCTO_ERR_INVALID_ARG, "bad B, Hq, Hkv, n_q or n_keys");
  const size_t need = ws_layout(cb, 1, B, Hq, Hkv, n_q, n_keys).total;
  if (need > kStaticScratchBytes)
    return fail(OCTO_ERR_WORKSPACE, "this call needs " + std::to_string(need) +
                                        " bytes of decode scratch; the static scratch holds " +
                                        std::to_string(kStaticScratchBytes));
  void* scr = nullptr;
  // (resolved when the codebook was built; check_cb made its device current)
  const hipError_t e = static_scratch(cb->device, &scr);
  if (e != hipSuccess) return hip_status(e, "static scratch address");
  return decode_attn_impl(cb, q, qdt, B, Hq, Hkv, n_q, packed, gamma, qjl_bits, qjl_norm, v, vdt,
                          n_keys, cap, scale, out, scr, kStaticScratchBytes, stream, OCTO_STAGE_ALL,
                          nullptr);
}

octo_status octo_decode_attn_append(const octo_codebook* cb, const void* new_keys, octo_dtype kdt,
                                    int64_t key_seq_stride, const void* q, octo_dtype qdt, int B,
                                    int Hq, int Hkv, void* packed, float* gamma, void* qjl_bits,
                                    uint16_t* qjl_norm, const void* v, octo_dtype vdt,
                                    int64_t n_keys, int64_t cap, float scale, float* out,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  // the decode's argument checks run before the encode writes anything
  octo_status st = check_decode_common(cb, q, qdt, B, Hq, Hkv, packed, gamma, qjl_bits, qjl_norm,
                                       n_keys, cap, workspace);
  if (st != OCTO_OK) return st;
  if (n_keys < 1) return fail(OCTO_ERR_INVALID_ARG, "need 1 <= n_keys <= cap");
  if (vdt != OCTO_BF16) return fail(OCTO_ERR_UNSUPPORTED, "V must be bf16");
  if (!v || !aligned(v, 16)) return fail(OCTO_ERR_INVALID_ARG, "v NULL or not 16-byte aligned");
  if (!out || !aligned(out, 4)) return fail(OCTO_ERR_INVALID_ARG, "out NULL/misaligned");
  if (workspace_bytes < ws_layout(cb, 1, B, Hq, Hkv, 1, n_keys).total)
    return fail(OCTO_ERR_WORKSPACE, "workspace too small");
  const int64_t n_seq = (int64_t)B * Hkv;
  if (n_seq == 0 || Hq == 0) return OCTO_OK;
  if (n_seq > 1 && key_seq_stride < cb->d) return fail(OCTO_ERR_INVALID_ARG, "key_seq_stride < d");
  if (!qjl_bits && kdt == OCTO_BF16) {
    // fused: the attention kernel encodes the new key itself (same code and
    // rounding as the append encoder)
    if (!new_keys || !aligned(new_keys, 16) || (key_seq_stride * 2) % 16)
      return fail(OCTO_ERR_INVALID_ARG, "new key rows must be 16-byte aligned");
    const AppendKey app{new_keys, key_seq_stride, packed, gamma};
    return decode_attn_impl(cb, q, qdt, B, Hq, Hkv, 1, packed, gamma, nullptr, nullptr, v, vdt,
                            n_keys, cap, scale, out, workspace, workspace_bytes, stream,
                            OCTO_STAGE_ALL, &app);
  }
  st = encode_impl(cb, new_keys, kdt, n_seq, 1, key_seq_stride, cb->d, n_keys - 1, cap, packed,
                   gamma, qjl_bits, qjl_norm, stream, false);
  if (st != OCTO_OK) return st;
  return octo_decode_attn_stages(cb, q, qdt, B, Hq, Hkv, 1, packed, gamma, qjl_bits, qjl_norm, v,
                                 vdt, n_keys, cap, scale, out, workspace, workspace_bytes, stream,
                                 OCTO_STAGE_ALL);
}

octo_status octo_decode_attn_stages(const octo_codebook* cb, const void* q, octo_dtype qdt, int B,
                                    int Hq, int Hkv, int n_q, const void* packed,
                                    const float* gamma, const void* qjl_bits,
                                    const uint16_t* qjl_norm, const void* v, octo_dtype vdt,
                                    int64_t n_keys, int64_t cap, float scale, float* out,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    int stages) {
  return decode_attn_impl(cb, q, qdt, B, Hq, Hkv, n_q, packed, gamma, qjl_bits, qjl_norm, v, vdt,
                          n_keys, cap, scale, out, workspace, workspace_bytes, stream, stages,
                          nullptr);
}

static octo_status decode_attn_impl(const octo_codebook* cb, const void* q, octo_dtype qdt, int B,
                                    int Hq, int Hkv, int n_q, const void* packed,
                                    const float* gamma, const void* qjl_bits,
                                    const uint16_t* qjl_norm, const void* v, octo_dtype vdt,
                                    int64_t n_keys, int64_t cap, float scale, float* out,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    int stages, const AppendKey* app) {
  octo_status st = check_decode_common(cb, q, qdt, B, Hq, Hkv, packed, gamma, qjl_bits, qjl_norm,
                                       n_keys, cap, workspace);
  if (st != OCTO_OK) return st;
  if (n_q < 1) return fail(OCTO_ERR_INVALID_ARG, "n_q < 1");
  if (vdt != OCTO_BF16) return fail(OCTO_ERR_UNSUPPORTED, "V must be bf16");
  if (!v || !aligned(v, 16)) return fail(OCTO_ERR_INVALID_ARG, "v NULL or not 16-byte aligned");
  if (!out || !aligned(out, 4)) return fail(OCTO_ERR_INVALID_ARG, "out NULL/misaligned");
  const WsLayout wl = ws_layout(cb, 1, B, Hq, Hkv, n_q, n_keys);
  if (workspace_bytes < wl.total) return fail(OCTO_ERR_WORKSPACE, "workspace too small");
  hipStream_t s = (hipStream_t)stream;
  const int64_t out_elems = (int64_t)B * Hq * n_q * cb->d;
  if (out_elems == 0) return OCTO_OK;
  if (n_keys == 0) {
    if (!(stages & OCTO_STAGE_COMBINE)) return OCTO_OK;
    return hip_status(launch_fill_zero(out, out_elems, s), "fill launch");
  }
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)cb->d);
  const bool qjl = qjl_bits != nullptr;
  RotateArgs r{};
  r.t = cb->tables;
  r.q = q;
  r.qdt = (int)qdt;
  r.B = B;
  r.Hq = Hq;
  r.Hkv = Hkv;
  r.n_q = n_q;
  r.mult = sc * 1.4426950408889634f;  // logits in log2 units for exp2
  r.qrot = (float*)((char*)workspace + wl.qrot);
  r.qp = nullptr;
  const int G = Hq / Hkv;
  if (n_q > 1) {
    if (qjl) return fail(OCTO_ERR_UNSUPPORTED, "multi-query path has no QJL variant");
    if (stages & OCTO_STAGE_ROTATE) {
      st = hip_status(launch_rotate(cb->d, r, s), "rotate launch");
      if (st != OCTO_OK) return st;
    }
    const Split sp = mq_split(n_keys, cb->d, cb->b, mq_rows(B, Hq, n_q));
    MQArgs m{};
    m.t = cb->tables;
    m.qrot = r.qrot;
    m.packed = (const uint32_t*)packed;
    m.gamma = gamma;
    m.v = v;
    m.n_keys = n_keys;
    m.cap = cap;
    m.B = B;
    m.n_q = n_q;
    m.H = Hq;
    m.Hkv = Hkv;
    m.G = G;
    m.tiles_per_split = sp.tiles_per_split;
    m.n_split = sp.n_split;
    m.part = (float*)((char*)workspace + wl.part);
    if (stages & OCTO_STAGE_MAIN) {
      st = hip_status(launch_mq_attn(cb->d, cb->b, m, s), "multi-query attention launch");
      if (st != OCTO_OK) return st;
    }
    if (!(stages & OCTO_STAGE_COMBINE)) return OCTO_OK;
    CombineArgs c{};
    c.part = m.part;
    c.out = out;
    c.rows = B * Hq * n_q;
    c.n_split = sp.n_split;
    c.d = cb->d;
    return hip_status(launch_combine(c, s), "combine launch");
  }
  const int64_t n_seq = (int64_t)B * Hkv;
  const Split sp = attn_split(n_keys, n_seq, head_passes(G));
  if (sp.n_split > kMaxSplit) return fail(OCTO_ERR_INVALID_ARG, "too many splits");
  // single query: the rotation runs in the fused kernel's prologue
  DecodeArgs a{};
  a.t = cb->tables;
  a.q = q;
  a.qdt = (int)qdt;
  a.mult = r.mult;
  a.packed = (const uint32_t*)packed;
  a.gamma = gamma;
  a.qjl_bits = (const uint32_t*)qjl_bits;
  a.qjl_norm = qjl_norm;
  a.v = v;
  a.n_keys = n_keys;
  a.cap = cap;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = G;
  a.tiles_per_split = sp.tiles_per_split;
  a.n_split = sp.n_split;
  a.part = (float*)((char*)workspace + wl.part);
  if (app) {
    a.new_keys = app->keys;
    a.new_key_stride = app->stride;
    a.packed_w = (uint32_t*)app->packed;
    a.gamma_w = app->gamma;
  }
  if (stages & OCTO_STAGE_MAIN) {
    st = hip_status(launch_attn(cb->d, cb->b, qjl, a, n_seq, s), "attention launch");
    if (st != OCTO_OK) return st;
  }
  if (!(stages & OCTO_STAGE_COMBINE)) return OCTO_OK;
  CombineArgs c{};
  c.part = a.part;
  c.out = out;
  c.rows = B * Hq;
  c.n_split = sp.n_split;
  c.d = cb->d;
  return hip_status(launch_combine(c, s), "combine launch");
}

octo_status octo_debug_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (!dst || !src || !aligned(dst, 16) || !aligned(src, 16) || bytes % 16)
    return fail(OCTO_ERR_INVALID_ARG, "copy needs 16-byte aligned pointers and size");
  return hip_status(launch_copy16(dst, src, (int64_t)(bytes / 16), (hipStream_t)stream),
                    "copy launch");
}

octo_status octo_debug_reconstruct(const octo_codebook* cb, const void* packed, const float* gamma,
                                   int64_t n_seq, int64_t n_keys, int64_t cap, float* keys_out,
                                   void* stream) {
  octo_status st = check_cb(cb);
  if (st != OCTO_OK) return st;
  if (n_seq < 0 || n_keys < 0 || cap <= 0 || cap % kTile || n_keys > cap || n_seq > 65535)
    return fail(OCTO_ERR_INVALID_ARG, "bad n_seq/n_keys/cap");
  if (!packed || !gamma || !keys_out) return fail(OCTO_ERR_INVALID_ARG, "NULL pointer");
  ReconArgs a{};
  a.t = cb->tables;
  a.packed = (const uint32_t*)packed;
  a.gamma = gamma;
  a.n_keys = n_keys;
  a.cap = cap;
  a.out = keys_out;
  return hip_status(launch_reconstruct(cb->d, cb->b, a, n_seq, (hipStream_t)stream),
                    "reconstruct launch");
}

}  // extern "C"

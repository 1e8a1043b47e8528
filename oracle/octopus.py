"""OCTOPUS oracle: fp64 NumPy, vectorised over keys but otherwise literal.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Nothing here is tuned;
every function follows one passage of the pages and says which.  Readings of
the pages where they are silent or ambiguous are marked "READING".

Parity status of each function (what pins it, tests/test_oracle_*.py):
  splitmix64 / gaussians     published SplitMix64 test vectors; N(0,1) moments+KS
  wht_signs / rotation       Sylvester H H^T = dI (exact), equals scipy.linalg.hadamard
  octa_encode / octa_decode  hand-computed golden points; round trip 1e-12 on 1e6 vectors
  triplet_polar              sum rho_i^2 = 1; rho^2 ~ Beta(3/2,(d-3)/2) (KS)
  lloyd_max                  Max (1960) Gaussian table; fixed-point property
  build_codebook             quadrature Lloyd-Max on the exact rho density
  quantize                   brute-force nearest centroid
  pack_codes / unpack_codes  golden hand-packed words; bijection on random codes
  encode / decode            identity-quantizer round trip 1e-12; printed MSEs
                             0.0071 (b=4) and 0.0897 (b=2) on d=128 Gaussian keys
  logits / attention         torch scaled_dot_product_attention (fp64, CPU)
  haar_rotation / qjl_scale  orthogonality; E|u_1| against the Beta(1/2, (d-1)/2)
                             moment (scipy); closed-form sign expectation over seeds
  qjl_encode / qjl_logits    unbiased over seeds; error ratio to the plain estimate
                             sqrt(pi/2 - 1) as the sign-estimator variance predicts
  joint_round                exhaustive 2^(b_xi+b_eta) search: identical on 10000
                             random triplets at b = 2, 3, 4, as the pages report
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# ----------------------------------------------------------------------------
# Seeded randomness.  The pages say only that the codec is deterministic given
# a seed ([AB]).  READING: SplitMix64 (Steele, Lea & Flood, OOPSLA 2014) keyed
# by seed XOR a per-purpose tag; uniforms (x >> 11) * 2^-53; Box-Muller pairs.
# ----------------------------------------------------------------------------
MASK64 = (1 << 64) - 1
SPLITMIX_GAMMA = 0x9E3779B97F4A7C15
TAG_SIGNS = 0x4F43544F5349474E  # "OCTOSIGN": WHT sign vector
TAG_MC = 0x4F43544F4D43534D     # "OCTOMCSM": Monte-Carlo codebook samples
TAG_QJL = 0x4F43544F514A4C53    # "OCTOQJLS": QJL Gaussian projection


def splitmix64(state0: int, n: int, start: int = 0) -> np.ndarray:
    """Outputs start..start+n-1 of SplitMix64 whose state starts at state0.

    Output i is mix(state0 + (i+1)*GAMMA) with the published mix function.
    """
    i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(state0 & MASK64) + i * np.uint64(SPLITMIX_GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        z = z ^ (z >> np.uint64(31))
    return z


def stream(seed: int, tag: int, n: int, start: int = 0) -> np.ndarray:
    return splitmix64((seed ^ tag) & MASK64, n, start)


def uniforms(seed: int, tag: int, n: int) -> np.ndarray:
    """U[0,1) doubles: the top 53 bits of each draw times 2^-53."""
    return (stream(seed, tag, n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def gaussians(seed: int, tag: int, n: int) -> np.ndarray:
    """N(0,1) by Box-Muller: draws (2p, 2p+1) give Gaussians (2p, 2p+1).

    r = sqrt(-2 ln(1-u1)); g_2p = r cos(2 pi u2); g_2p+1 = r sin(2 pi u2).
    """
    npairs = (n + 1) // 2
    u = uniforms(seed, tag, 2 * npairs)
    u1, u2 = u[0::2], u[1::2]
    r = np.sqrt(-2.0 * np.log(1.0 - u1))
    th = 2.0 * math.pi * u2
    g = np.empty(2 * npairs)
    g[0::2] = r * np.cos(th)
    g[1::2] = r * np.sin(th)
    return g[:n]


# ----------------------------------------------------------------------------
# Sign-flipped Walsh-Hadamard rotation ([YL] 旋转魔法; [AR] 方法概覽).
# READING: R(x) = d^-1/2 * H_d * (s .* x), H_d Sylvester-ordered, signs applied
# first; R is orthogonal so R^-1 = R^T.  d must be a power of two.
# ----------------------------------------------------------------------------
def wht_signs(d: int, seed: int) -> np.ndarray:
    """s_j = +1 if the low bit of draw j is 0, else -1."""
    bits = stream(seed, TAG_SIGNS, d) & np.uint64(1)
    return 1.0 - 2.0 * bits.astype(np.float64)


def sylvester(d: int) -> np.ndarray:
    """H_1 = [1]; H_2m = [[H_m, H_m], [H_m, -H_m]] (integer matrix)."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation(d: int, seed: int) -> np.ndarray:
    """The d x d matrix R = d^-1/2 H_d diag(s)."""
    return sylvester(d).astype(np.float64) * wht_signs(d, seed)[None, :] / math.sqrt(d)


# ----------------------------------------------------------------------------
# Triplets ([YL] 三元组分解): pad the rotated direction with zeros to a
# multiple of 3, split into adjacent triplets t_i = rho_i n_i.
# READING: a triplet with rho_i = 0 gets n_i = (0, 0, 1).
# ----------------------------------------------------------------------------
def n_triplets(d: int) -> int:
    return (d + 2) // 3


def split_triplets(u: np.ndarray) -> np.ndarray:
    """(..., d) -> (..., T, 3) with zero padding at the end."""
    d = u.shape[-1]
    T = n_triplets(d)
    pad = np.zeros(u.shape[:-1] + (3 * T - d,))
    return np.concatenate([u, pad], axis=-1).reshape(u.shape[:-1] + (T, 3))


def join_triplets(t: np.ndarray, d: int) -> np.ndarray:
    """(..., T, 3) -> (..., d), dropping the pad coordinates."""
    return t.reshape(t.shape[:-2] + (-1,))[..., :d]


def triplet_polar(t: np.ndarray):
    """rho = |t|, n = t / rho (n = (0,0,1) where rho == 0)."""
    rho = np.sqrt(np.sum(t * t, axis=-1))
    n = np.empty_like(t)
    nz = rho > 0
    n[nz] = t[nz] / rho[nz][:, None]
    n[~nz] = (0.0, 0.0, 1.0)
    return rho, n


# ----------------------------------------------------------------------------
# Octahedral map ([YL] 八面体折叠; [AR] 方法概覽 "piecewise-linear inverse").
# Encode: l = |x|+|y|+|z|, p = (x, y)/l; if z < 0 fold the lower hemisphere:
#   xi = (1 - |p_y|) sgn(p_x), eta = (1 - |p_x|) sgn(p_y).
# Decode: r = 1 - |xi| - |eta|; if r >= 0 take (xi, eta, r), otherwise unfold
#   to ((1-|eta|) sgn(xi), (1-|xi|) sgn(eta), r); then normalise.
# READING: sgn(0) = +1; z = 0 counts as the upper hemisphere.
# ----------------------------------------------------------------------------
def _sgn(x: np.ndarray) -> np.ndarray:
    return np.where(x >= 0, 1.0, -1.0)


def octa_encode(n: np.ndarray):
    x, y, z = n[..., 0], n[..., 1], n[..., 2]
    l1 = np.abs(x) + np.abs(y) + np.abs(z)
    px, py = x / l1, y / l1
    lower = z < 0
    xi = np.where(lower, (1.0 - np.abs(py)) * _sgn(px), px)
    eta = np.where(lower, (1.0 - np.abs(px)) * _sgn(py), py)
    return xi, eta


def octa_decode(xi: np.ndarray, eta: np.ndarray) -> np.ndarray:
    r = 1.0 - np.abs(xi) - np.abs(eta)
    lower = r < 0
    x = np.where(lower, (1.0 - np.abs(eta)) * _sgn(xi), xi)
    y = np.where(lower, (1.0 - np.abs(xi)) * _sgn(eta), eta)
    v = np.stack([x, y, r], axis=-1)
    return v / np.sqrt(np.sum(v * v, axis=-1, keepdims=True))


# ----------------------------------------------------------------------------
# 1-D Lloyd-Max quantiser ([YL] 三元组分解, last paragraphs; [AB]).
# READING (initialisation/stopping are not on the pages): start at the sample
# quantiles (k + 1/2)/L; repeat { m_k = (c_k + c_k+1)/2; c_k = mean of the
# samples x with m_k-1 < x <= m_k (an empty cell keeps its centroid) } until
# max |dc| <= 1e-12 or 2000 iterations.  The cell sums are taken from prefix
# sums of the sorted samples, which is the same definition evaluated faster.
# ----------------------------------------------------------------------------
LLOYD_TOL = 1e-12
LLOYD_MAX_ITER = 2000


def lloyd_max(samples: np.ndarray, levels: int, tol: float = LLOYD_TOL,
              max_iter: int = LLOYD_MAX_ITER) -> np.ndarray:
    x = np.sort(np.asarray(samples, dtype=np.float64))
    N = x.size
    if levels == 1:
        return np.array([x.mean()])
    prefix = np.concatenate([[0.0], np.cumsum(x)])
    c = x[np.floor((np.arange(levels) + 0.5) * N / levels).astype(np.int64)]
    for _ in range(max_iter):
        m = 0.5 * (c[:-1] + c[1:])
        edges = np.searchsorted(x, m, side="right")  # #{x_i <= m_k}
        lo = np.concatenate([[0], edges])
        hi = np.concatenate([edges, [N]])
        cnt = hi - lo
        new = np.where(cnt > 0, (prefix[hi] - prefix[lo]) / np.maximum(cnt, 1), c)
        done = np.max(np.abs(new - c)) <= tol
        c = new
        if done:
            break
    return c


def midpoints(c: np.ndarray) -> np.ndarray:
    return 0.5 * (c[:-1] + c[1:])


def quantize(x: np.ndarray, c: np.ndarray) -> np.ndarray:
    """Nearest centroid by the midpoint rule: i = #{k : x > m_k}.

    READING: a value exactly on a midpoint takes the lower index.
    """
    return np.searchsorted(midpoints(c), x, side="left").astype(np.int64)


# ----------------------------------------------------------------------------
# Codebooks: data-oblivious, pre-generated, depending only on d and the bit
# budget ([AR] 位元分配; [AB] "implementation-matched marginals").
# Bit allocation ([YL] 非均匀比特分配): direction b+1, length b-1.
# READING: xi and eta each get b+1 bits, rho gets b-1 (3b+1 bits per triplet);
# the allocation stays a parameter and (b, b, b) gives exactly 3b.
# READING: the marginals are sampled by Monte Carlo from the implementation's
# own pipeline: M Gaussian vectors, normalised (so their rotation is again
# uniform on the sphere), zero-padded, split into triplets; rho pooled over
# all T triplet positions; xi and eta pooled together and symmetrised by
# appending their negatives; the xi/eta codebook is made exactly antisymmetric
# by c_k <- (c_k - c_{L-1-k})/2 after Lloyd-Max.
# ----------------------------------------------------------------------------
MC_VECTORS = 65536


def default_alloc(b: int):
    return (b + 1, b + 1, b - 1)


_SAMPLE_CACHE: dict = {}


def mc_samples(d: int, cb_seed: int, M: int = MC_VECTORS):
    """Monte-Carlo samples (rho, xi/eta pool) of the rotated triplet marginals."""
    key = (d, cb_seed, M)
    if key not in _SAMPLE_CACHE:
        g = gaussians(cb_seed, TAG_MC, M * d).reshape(M, d)
        u = g / np.sqrt(np.sum(g * g, axis=1, keepdims=True))
        rho, n = triplet_polar(split_triplets(u).reshape(-1, 3))
        xi, eta = octa_encode(n)
        dirs = np.concatenate([xi, eta])
        _SAMPLE_CACHE[key] = (rho, np.concatenate([dirs, -dirs]))
    return _SAMPLE_CACHE[key]


@dataclass
class Codebook:
    d: int
    b: int
    alloc: tuple
    seed: int
    cb_seed: int
    c_xi: np.ndarray
    c_eta: np.ndarray
    c_rho: np.ndarray
    signs: np.ndarray
    R: np.ndarray = field(repr=False)

    @property
    def T(self) -> int:
        return n_triplets(self.d)

    @property
    def bits_per_triplet(self) -> int:
        return sum(self.alloc)

    @property
    def words_per_key(self) -> int:
        return (self.T * self.bits_per_triplet + 31) // 32


def antisymmetrize(c: np.ndarray) -> np.ndarray:
    return 0.5 * (c - c[::-1])


def build_codebook(d: int, b: int, seed: int = 0, cb_seed: int = 0, alloc=None,
                   M: int = MC_VECTORS) -> Codebook:
    alloc = tuple(alloc) if alloc is not None else default_alloc(b)
    b_xi, b_eta, b_rho = alloc
    rho, dirs = mc_samples(d, cb_seed, M)
    c_xi = antisymmetrize(lloyd_max(dirs, 1 << b_xi))
    c_eta = c_xi if b_eta == b_xi else antisymmetrize(lloyd_max(dirs, 1 << b_eta))
    c_rho = lloyd_max(rho, 1 << b_rho)
    return Codebook(d, b, alloc, seed, cb_seed, c_xi, c_eta, c_rho,
                    wht_signs(d, seed), rotation(d, seed))


# ----------------------------------------------------------------------------
# Encode / decode a batch of keys ([YL] 三元组分解 steps 1-4; 八面体折叠).
# gamma = |k|_2 kept as fp32; u = k / gamma (u = 0 when gamma = 0).
# ----------------------------------------------------------------------------
@dataclass
class Encoded:
    codes: np.ndarray        # (n, T, 3) int64: i_xi, i_eta, i_rho
    gamma: np.ndarray        # (n,) float32
    values: np.ndarray       # (n, T, 3) fp64 xi, eta, rho that were quantised
    rotated: np.ndarray      # (n, d) fp64 u' = R u


def encode(keys: np.ndarray, cb: Codebook, identity: bool = False,
           rounding: str = "scalar") -> Encoded:
    """Scalar (nearest-centroid) rounding, the encoder's hot-path rule, or
    with rounding="joint" the pages' joint rounding of each triplet
    ([YL] 联合取整, ``joint_round`` below).

    identity=True skips quantisation (codes are left empty and ``values``
    carries the exact components) so the rest of the chain can be checked
    for exactness.
    """
    k = np.asarray(keys, dtype=np.float64)
    gamma = np.sqrt(np.sum(k * k, axis=1))
    # u' = R (k / gamma) = H (s .* k) / (sqrt(d) gamma): R is linear, and the
    # integer Hadamard sums of fp32 / bf16 keys are exact in fp64, so a
    # coordinate that is exactly 0 (the signed entries cancel) stays exactly 0
    # (a rounded 1/gamma or 1/sqrt(d) before the sums would leave +-1e-17 of
    # either sign, turning zero triplets and sgn(0) into rounding noise)
    y = (k * cb.signs[None, :]) @ sylvester(cb.d).T.astype(np.float64)
    scale = np.where(gamma > 0, math.sqrt(cb.d) * gamma, 1.0)
    up = np.where(gamma[:, None] > 0, y / scale[:, None], 0.0)
    rho, n = triplet_polar(split_triplets(up).reshape(-1, 3))
    xi, eta = octa_encode(n)
    nk, T = k.shape[0], cb.T
    values = np.stack([xi, eta, rho], axis=-1).reshape(nk, T, 3)
    if identity:
        codes = np.zeros((nk, T, 3), dtype=np.int64)
    elif rounding == "joint":
        codes = joint_round(split_triplets(up), cb)
    else:
        codes = np.stack([quantize(xi, cb.c_xi), quantize(eta, cb.c_eta),
                          quantize(rho, cb.c_rho)], axis=-1).reshape(nk, T, 3)
    return Encoded(codes, gamma.astype(np.float32), values, up)


def dequantize(codes: np.ndarray, cb: Codebook) -> np.ndarray:
    """codes (..., T, 3) -> centroid values (..., T, 3) = (xi^, eta^, rho^)."""
    return np.stack([cb.c_xi[codes[..., 0]], cb.c_eta[codes[..., 1]],
                     cb.c_rho[codes[..., 2]]], axis=-1)


def reconstruct_rotated(vals: np.ndarray, d: int) -> np.ndarray:
    """(..., T, 3) of (xi, eta, rho) -> u'^ (..., d): t_i = rho octdec(xi, eta)."""
    t = vals[..., 2:3] * octa_decode(vals[..., 0], vals[..., 1])
    return join_triplets(t, d)


def decode_rotated(codes: np.ndarray, cb: Codebook) -> np.ndarray:
    """The rotated unit-direction estimate u'^ from packed codes."""
    return reconstruct_rotated(dequantize(codes, cb), cb.d)


def decode(codes: np.ndarray, gamma: np.ndarray, cb: Codebook) -> np.ndarray:
    """k^ = gamma R^T u'^ (gamma read as the stored fp32 value)."""
    uh = decode_rotated(codes, cb)
    return np.asarray(gamma, dtype=np.float64)[:, None] * (uh @ cb.R)


# ----------------------------------------------------------------------------
# Joint rounding ([YL] 联合取整): for a direction candidate n^, the best rho^
# is the codeword nearest s = <n^, t>; the candidates are the 3x3 neighbours
# of the scalar-rounded (i_xi, i_eta).  READING: candidates are clamped to the
# index range; error e = |t - rho^ n^|^2 - |t|^2 = (rho^ - s)^2 - s^2; the
# first strict minimum in (a, c) lexicographic order wins.
# ----------------------------------------------------------------------------
def joint_round(t: np.ndarray, cb: Codebook, exhaustive: bool = False) -> np.ndarray:
    """t (..., 3) exact rotated triplets -> codes (..., 3) by joint rounding.

    exhaustive=True searches all 2^(b_xi + b_eta) direction codes (the ground
    truth the 3x3 neighbourhood is compared with on the same page).
    """
    tt = np.asarray(t, dtype=np.float64).reshape(-1, 3)
    _, n = triplet_polar(tt)
    xi, eta = octa_encode(n)
    i_xi, i_eta = quantize(xi, cb.c_xi), quantize(eta, cb.c_eta)
    Lx, Le = cb.c_xi.size, cb.c_eta.size
    if exhaustive:
        cand = [(a, c) for a in range(Lx) for c in range(Le)]
    else:
        cand = [(a, c) for a in (-1, 0, 1) for c in (-1, 0, 1)]
    N = tt.shape[0]
    best_e = np.full(N, np.inf)
    best = np.zeros((N, 3), dtype=np.int64)
    for a, c in cand:
        if exhaustive:
            ja, jc = np.full(N, a), np.full(N, c)
        else:
            ja, jc = np.clip(i_xi + a, 0, Lx - 1), np.clip(i_eta + c, 0, Le - 1)
        nh = octa_decode(cb.c_xi[ja], cb.c_eta[jc])
        s = np.sum(nh * tt, axis=-1)
        jr = quantize(s, cb.c_rho)
        e = (cb.c_rho[jr] - s) ** 2 - s * s
        better = e < best_e
        best_e = np.where(better, e, best_e)
        best[better] = np.stack([ja, jc, jr], axis=-1)[better]
    return best.reshape(np.shape(t)[:-1] + (3,))


# ----------------------------------------------------------------------------
# Packed layout (the pages only say the decoder reads a compact bitstream,
# [YL] 工程实现).  READING: per key, triplet i occupies bits
# [i*B_t, (i+1)*B_t) of a little-endian stream of u32 words, LSB first, code
# = i_xi | i_eta << b_xi | i_rho << (b_xi + b_eta); unused bits are 0.
# Keys are stored in tiles of 64.  Inside a tile the W words of every key are
# cut into groups of 4 consecutive words (the last group holds the W % 4 left
# over); group g of all 64 keys is stored key-major, [key][words of group g],
# and the groups follow each other.  Word w of key j of sequence s is thus the
# element (j % 64) * width(g) + w % 4 of group g = w // 4 in tile j // 64, with
# width(g) = 4 for full groups and W % 4 for the last.  The same layout holds
# the d/32 QJL sign words of a key.
# ----------------------------------------------------------------------------
TILE = 64


def pack_codes(codes: np.ndarray, alloc) -> np.ndarray:
    """codes (n, T, 3) -> words (n, W) uint32."""
    b_xi, b_eta, b_rho = alloc
    bt = b_xi + b_eta + b_rho
    n, T, _ = codes.shape
    W = (T * bt + 31) // 32
    words = np.zeros((n, W + 1), dtype=np.uint64)
    code = (codes[..., 0] | (codes[..., 1] << b_xi) | (codes[..., 2] << (b_xi + b_eta))).astype(np.uint64)
    for i in range(T):
        pos = i * bt
        w, off = pos // 32, pos % 32
        v = code[:, i] << np.uint64(off)
        words[:, w] |= v & np.uint64(0xFFFFFFFF)
        words[:, w + 1] |= v >> np.uint64(32)
    return words[:, :W].astype(np.uint32)


def unpack_codes(words: np.ndarray, T: int, alloc) -> np.ndarray:
    """words (n, W) -> codes (n, T, 3)."""
    b_xi, b_eta, b_rho = alloc
    bt = b_xi + b_eta + b_rho
    n, W = words.shape
    ext = np.zeros((n, W + 1), dtype=np.uint64)
    ext[:, :W] = words
    codes = np.zeros((n, T, 3), dtype=np.int64)
    for i in range(T):
        pos = i * bt
        w, off = pos // 32, pos % 32
        window = ext[:, w] | (ext[:, w + 1] << np.uint64(32))
        c = (window >> np.uint64(off)) & np.uint64((1 << bt) - 1)
        c = c.astype(np.int64)
        codes[:, i, 0] = c & ((1 << b_xi) - 1)
        codes[:, i, 1] = (c >> b_xi) & ((1 << b_eta) - 1)
        codes[:, i, 2] = c >> (b_xi + b_eta)
    return codes


def tile_groups(W: int):
    """[(first word, width)] of the word groups of the tile layout."""
    return [(w0, min(4, W - w0)) for w0 in range(0, W, 4)]


def to_tiles(words: np.ndarray, cap: int) -> np.ndarray:
    """(n_seq, n <= cap, W) per-key words -> (n_seq, cap//64, 64*W) tiled buffer."""
    n_seq, n, W = words.shape
    full = np.zeros((n_seq, cap, W), dtype=np.uint32)
    full[:, :n] = words
    t = full.reshape(n_seq, cap // TILE, TILE, W)
    parts = [t[:, :, :, w0:w0 + wd].reshape(n_seq, cap // TILE, TILE * wd)
             for w0, wd in tile_groups(W)]
    return np.concatenate(parts, axis=2)


def from_tiles(tiles: np.ndarray, W: int, n: int) -> np.ndarray:
    """(n_seq, cap//64, 64*W) tiled buffer -> (n_seq, n, W) per-key words."""
    n_seq, nt = tiles.shape[:2]
    tiles = tiles.reshape(n_seq, nt, TILE * W)
    out = np.zeros((n_seq, nt, TILE, W), dtype=tiles.dtype)
    for w0, wd in tile_groups(W):
        out[:, :, :, w0:w0 + wd] = tiles[:, :, TILE * w0:TILE * (w0 + wd)].reshape(n_seq, nt, TILE, wd)
    return out.reshape(n_seq, nt * TILE, W)[:, :n]


# ----------------------------------------------------------------------------
# Decode-time arithmetic ([YL] 工程实现: keys rebuilt on the fly, q.k, then
# online softmax; FlashAttention tiling is an implementation detail that the
# plain definition below does not need).
# READING: logits are raw <q, k^>; attention scale 1/sqrt(d); no mask; query
# head h reads KV head floor(h / G); outputs fp64 here (fp32 on the device).
# ----------------------------------------------------------------------------
def logits(q: np.ndarray, khat: np.ndarray) -> np.ndarray:
    """q (..., d), khat (n, d) -> (..., n)."""
    return np.asarray(q, dtype=np.float64) @ khat.T


def logits_rotated(q: np.ndarray, uh: np.ndarray, gamma: np.ndarray, cb: Codebook) -> np.ndarray:
    """Same value through the rotated query: gamma * <R q, u'^>."""
    qr = np.asarray(q, dtype=np.float64) @ cb.R.T
    return (qr @ uh.T) * np.asarray(gamma, dtype=np.float64)


def softmax_attention(a: np.ndarray, v: np.ndarray) -> np.ndarray:
    """a (..., n) scaled scores, v (n, dv) -> softmax(a) v."""
    m = np.max(a, axis=-1, keepdims=True)
    p = np.exp(a - m)
    p = p / np.sum(p, axis=-1, keepdims=True)
    return p @ np.asarray(v, dtype=np.float64)


def attention(q: np.ndarray, khat: np.ndarray, v: np.ndarray, scale: float | None = None) -> np.ndarray:
    d = khat.shape[-1]
    s = 1.0 / math.sqrt(d) if scale is None else scale
    return softmax_attention(s * logits(q, khat), v)


def gqa_attention(q: np.ndarray, khat: np.ndarray, v: np.ndarray, scale: float | None = None) -> np.ndarray:
    """q (B, Hq, nq, d), khat (B, Hkv, n, d), v (B, Hkv, n, dv) -> (B, Hq, nq, dv)."""
    B, Hq = q.shape[:2]
    Hkv = khat.shape[1]
    G = Hq // Hkv
    out = np.zeros(q.shape[:3] + (v.shape[-1],))
    for bb in range(B):
        for h in range(Hq):
            out[bb, h] = attention(q[bb, h], khat[bb, h // G], v[bb, h // G], scale)
    return out


# ----------------------------------------------------------------------------
# OCTOPUS-QJL ([YL] 可选的残差修正; [AR] OCTOPUS-QJL; the 1-bit sign estimator
# of QJL, [TQ] 四/五).
# READING: the residual is taken in the rotated unit domain over the d real
# coordinates, r' = u'[:d] - u'^[:d]; its length is stored as fp16; the page's
# "independent random rotation" is a Haar-random orthogonal d x d matrix P
# drawn from the seed; one sign per rotated coordinate, sgn(0) = +1, bit j = 1
# when sign j is +1.  The matrix is kept as S = sqrt(d) P (rows of norm
# sqrt(d), like Gaussian rows; the signs of S r' are those of P r'), and
#   l = gamma * ( <q', u'^> + kappa_d * nu * <S q', sigma> ),
#   kappa_d = 1 / (d sqrt(d) E|u_1|),  E|u_1| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))
# the mean |coordinate| of a uniform unit vector in R^d.  For a Haar P the
# rotated residual direction is uniform on the sphere, so
# E[<P q', sgn(P r')>] = d E|u_1| <q', r'> / |r'| and the estimate is exactly
# unbiased.  (A Gaussian S, the other reading, is unbiased too with
# kappa = sqrt(pi/2)/d, but its sign estimate has about pi/2 times the
# variance; gaussian_projection keeps it for that comparison.)
# ----------------------------------------------------------------------------
def gaussian_projection(d: int, seed: int) -> np.ndarray:
    """The seeded iid N(0,1) d x d matrix (row-major draws)."""
    return gaussians(seed, TAG_QJL, d * d).reshape(d, d)


def haar_rotation(d: int, seed: int) -> np.ndarray:
    """Haar-random orthogonal P: the Q factor of the seeded Gaussian matrix
    with the signs fixed so that R has a positive diagonal (Mezzadri 2007),
    i.e. the Gram-Schmidt orthonormalisation of its columns."""
    Q, R = np.linalg.qr(gaussian_projection(d, seed))
    return Q * np.where(np.diag(R) < 0, -1.0, 1.0)[None, :]


def qjl_matrix(d: int, seed: int) -> np.ndarray:
    """S = sqrt(d) P: the rotation the residual signs are taken in."""
    return math.sqrt(d) * haar_rotation(d, seed)


def mean_abs_coordinate(d: int) -> float:
    """E|u_1| for u uniform on the unit sphere of R^d."""
    return math.exp(math.lgamma(d / 2.0) - math.lgamma((d + 1) / 2.0)) / math.sqrt(math.pi)


def qjl_scale(d: int) -> float:
    """kappa_d with <q', r'> = kappa_d |r'| E<S q', sgn(S r')> for S = sqrt(d) P."""
    return 1.0 / (d * math.sqrt(d) * mean_abs_coordinate(d))


@dataclass
class QJLEncoded:
    signs: np.ndarray        # (n, d) +-1
    nu: np.ndarray           # (n,) float16 residual norms
    proj: np.ndarray         # (n, d) fp64 S r' (for boundary margins)
    resid: np.ndarray        # (n, d) fp64 r'


def qjl_encode(rotated: np.ndarray, uh: np.ndarray, S: np.ndarray) -> QJLEncoded:
    d = S.shape[0]
    r = rotated[:, :d] - uh[:, :d]
    nu = np.sqrt(np.sum(r * r, axis=1)).astype(np.float16)
    proj = r @ S.T
    signs = np.where(proj >= 0, 1.0, -1.0)
    return QJLEncoded(signs, nu, proj, r)


def qjl_logits(q: np.ndarray, uh: np.ndarray, gamma: np.ndarray, enc: QJLEncoded,
               S: np.ndarray, cb: Codebook, kappa: float | None = None) -> np.ndarray:
    """q (..., d) -> (..., n) QJL-corrected raw logits (kappa: the estimator
    constant of S; qjl_scale(d) for the rotation reading)."""
    d = cb.d
    kappa = qjl_scale(d) if kappa is None else kappa
    qr = np.asarray(q, dtype=np.float64) @ cb.R.T
    base = qr @ uh.T
    sq = qr @ S.T
    corr = (sq @ enc.signs.T) * enc.nu.astype(np.float64) * kappa
    return np.asarray(gamma, dtype=np.float64) * (base + corr)


def pack_signs(signs: np.ndarray) -> np.ndarray:
    """(n, d) +-1 -> (n, d/32) uint32, bit j%32 of word j//32 = (sign_j > 0)."""
    n, d = signs.shape
    bits = (signs > 0).astype(np.uint64).reshape(n, d // 32, 32)
    return np.sum(bits << np.arange(32, dtype=np.uint64), axis=-1).astype(np.uint32)


def unpack_signs(words: np.ndarray, d: int) -> np.ndarray:
    n = words.shape[0]
    bits = (words.astype(np.uint64)[:, :, None] >> np.arange(32, dtype=np.uint64)) & np.uint64(1)
    return np.where(bits.reshape(n, d) > 0, 1.0, -1.0)


# ----------------------------------------------------------------------------
# Sizes.
# ----------------------------------------------------------------------------
def layout(d: int, alloc) -> dict:
    T = n_triplets(d)
    bt = sum(alloc)
    return {"d": d, "n_triplets": T, "pad_dim": 3 * T, "bits_per_triplet": bt,
            "bits_per_key": T * bt, "words_per_key": (T * bt + 31) // 32}


__all__ = [n for n in dir() if not n.startswith("_")]

// Matrix-core (bf16 MFMA, fp32 accumulate) PaTH prefill for head dim 64, chunk 64.
//
// Scheme (PaTH summary, gist.science/ko/paper/2505.16381, section 3): each chunk's
// transitions are held in compact UT form, H_0...H_{C-1} = I - W^T T^{-1} W; per
// chunk we precompute boundary-adjusted rows (queries carry the chunk prefix up to
// and including themselves, keys carry the chunk suffix strictly after them), the
// chunk product P_c and the in-chunk logits; the attention kernel then scans key
// chunks right to left, moving its running queries across each finished chunk
// with P_c (the notes on PaTH, "WY" block: a dense d x d matrix per chunk applied
// to the whole query tile, a prefix product between chunks).
//
// Kernel 1 (prep), one workgroup of 4 waves per (b, h, chunk):
//   A = I + diag(beta) strict_upper(W W^T)   (unit upper triangular, fp32)
//   Z = A^{-1} by 16x16-blocked back substitution (fp32), T^{-1} = Z diag(beta)
//   U^T[a][t] = q_a.w_t (t <= a), R[b][s] = k_b.w_s (s > b), X = T^{-1} U, Y = R T^{-1}
//   qtilde = Q - X^T W, ktilde = K - Y W, P = I - W^T (T^{-1} W),
//   S[a][b] = q_a.k_b - (Y U)[b][a]   (b <= a; in-chunk logits before scaling)
// T^{-1} and T^{-1} W enter the matrix cores as hi+lo bf16 pairs so that P is
// accurate enough to be split again into hi+lo for the long-range transport.
//
// Kernel 2 (attention), one workgroup of 4 waves per 4 consecutive query chunks
// (wave w owns chunk 4p+w, 64 queries = four 16-query MFMA column tiles), longest
// rows first.  The waves share one LDS stream of key chunks n = 4p+3 ... 0
// (ktilde_n, V_n straight from the value tensor, P_n; double-buffered, filled by
// direct global->LDS loads); each A-fragment read from LDS feeds four MFMAs (one
// per query tile).  A wave scores its own chunk from the precomputed in-chunk
// logits when the stream reaches it, and earlier chunks as follows:
//   S^T = ktilde_n Q_run^T       (keys x queries: each lane holds one query column)
//   online softmax (exp2), P^T kept in registers as the PV B-operand
//   O^T += V_n^T P^T
//   Q_run^T <- P_n Q_run^T       (fp32 accumulate, re-rounded to bf16 [hi+lo])
// Column permutation: an MFMA accumulator gives each lane rows 4g..4g+3 of every
// 16-row tile, while a B-operand wants rows 8g..8g+7 of every 32-row k-step.  The
// contraction order is free, so qtilde, ktilde and P (columns) are stored with
// stored slot 8g+j of each 32-block holding index 16(j/4)+4g+(j%4), and V^T
// fragments are read (LDS transpose reads) in the same key order; accumulators then
// convert to B-operands in registers with no data movement.
#include "common.h"

namespace pathattn {

namespace {

constexpr int kD = 64;      // head dim
constexpr int kC = 64;      // chunk
constexpr int kLDB = 72;    // bf16 LDS row stride (144 B: conflict-free 16-byte row reads)
constexpr int kLDF = 68;    // fp32 LDS row stride
constexpr int kMat = kC * kLDB;  // elements of one padded 64x64 bf16 LDS matrix

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_frag(const __bf16* m, int row, int col) {
  return *reinterpret_cast<const bf16x8*>(m + row * kLDB + col);
}

// acc += X[m0..m0+15][0..63] . Y[n0..n0+15][0..63]^T; lane (r = l%16, g = l/16) receives
// acc[i] = D[m0 + 4g + i][n0 + r].
__device__ __forceinline__ f32x4 mm_tile(const __bf16* X, const __bf16* Y, int m0, int n0, f32x4 acc) {
  const int l = threadIdx.x & 63, r = l & 15, g = l >> 4;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    acc = mfma16(lds_frag(X, m0 + r, ks * 32 + g * 8), lds_frag(Y, n0 + r, ks * 32 + g * 8), acc);
  return acc;
}

// Stored slot of original column c (0..63) under the in-block permutation.
__device__ __forceinline__ int perm_pos(int c) {
  const int c32 = c & 31;
  return (c & 32) + ((c32 >> 2) & 3) * 8 + (c32 >> 4) * 4 + (c32 & 3);
}

__device__ __forceinline__ bf16x4 pack4(float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  v[2] = (__bf16)c;
  v[3] = (__bf16)d;
  return v;
}

__device__ __forceinline__ void split_hi_lo(float v, __bf16& hi, __bf16& lo) {
  hi = (__bf16)v;
  lo = (__bf16)(v - (float)hi);
}

// Four values -> hi and lo bf16 quads with v ~= hi + lo.
__device__ __forceinline__ void split4(float v0, float v1, float v2, float v3, bf16x4& h, bf16x4& l) {
  const float v[4] = {v0, v1, v2, v3};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const __bf16 hi = (__bf16)v[i];
    h[i] = hi;
    l[i] = (__bf16)(v[i] - (float)hi);
  }
}

}  // namespace

// =========================================================================== kernel 1: prep
// LDS plan (bytes): 13 padded bf16 64x64 matrices + beta + an fp32 region for A, Z = A^{-1}
// and block temporaries.  Regions are reused once their contents are dead:
//   R1 (4 mats): W, Q, K in phases A-B; X^T hi/lo and Y hi/lo in phases E-F
//   R2 (1 mat):  W^T throughout
//   R3 (4 mats): U^T hi/lo, R hi/lo
//   R4 (4 mats): T^{-1} hi/lo, T^{-T} hi/lo
//   R5 (fp32):   A, Z, temporaries in phases B-D; (T^{-1}W)^T hi/lo in phases E-F
constexpr size_t kPrepLds = 13 * kMat * 2 + 64 * 4 + 2 * kC * kLDF * 4 + 3 * 256 * 4;
static_assert(kPrepLds <= 160 * 1024, "prep LDS plan exceeds 160 KiB");

__global__ __launch_bounds__(256) void mfma_prep_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ w,
    const float* __restrict__ beta, const float* __restrict__ logf, int64_t L, int64_t M, __bf16* __restrict__ qt,
    __bf16* __restrict__ qt_lo, __bf16* __restrict__ kt, __bf16* __restrict__ p_hi, __bf16* __restrict__ p_lo,
    float* __restrict__ Sm, float* __restrict__ fl, float* __restrict__ ftot) {
  extern __shared__ __align__(16) char smem[];
  __bf16* R1 = reinterpret_cast<__bf16*>(smem);
  __bf16* Ws = R1;                 // W [s][x]
  __bf16* Qs = R1 + kMat;          // Q [a][x]
  __bf16* Ks = R1 + 2 * kMat;      // K [b][x]
  __bf16* XTH = R1;                // X^T [a][s] hi / lo   (after phase B)
  __bf16* XTL = R1 + kMat;
  __bf16* YH = R1 + 2 * kMat;      // Y [b][t] hi / lo     (after phase B)
  __bf16* YL = R1 + 3 * kMat;
  __bf16* WTs = R1 + 4 * kMat;     // W^T [x][s]
  __bf16* UTH = R1 + 5 * kMat;     // U^T [a][t] hi / lo
  __bf16* UTL = R1 + 6 * kMat;
  __bf16* RH = R1 + 7 * kMat;      // R [b][s] hi / lo
  __bf16* RL = R1 + 8 * kMat;
  __bf16* TiH = R1 + 9 * kMat;     // T^{-1} [s][t] hi / lo
  __bf16* TiL = R1 + 10 * kMat;
  __bf16* TiTH = R1 + 11 * kMat;   // T^{-T} [t][s] hi / lo
  __bf16* TiTL = R1 + 12 * kMat;
  float* Bs = reinterpret_cast<float*>(R1 + 13 * kMat);  // beta [64]
  float* Af = Bs + 64;                                   // A [64][kLDF]
  float* Zf = Af + kC * kLDF;                            // Z = A^{-1} [64][kLDF]
  float* Tmp = Zf + kC * kLDF;                           // 3 x 16 x 16 block temporaries
  __bf16* Z2H = reinterpret_cast<__bf16*>(Af);           // (T^{-1} W)^T [y][s] hi / lo (after phase D)
  __bf16* Z2L = Z2H + kMat;

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63, r = l & 15, g = l >> 4;
  const int c = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t Lp = M * kC;
  const int64_t row0 = (int64_t)c * kC;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  // ---------------------------------------------------------------- A: stage W, W^T, Q, K, beta
  for (int e = tid; e < 512; e += 256) {
    const int a = e >> 3, c8 = (e & 7) * 8;
    const int64_t i = row0 + a;
    const bool ok = i < L;
    const size_t go = ((size_t)bh * L + (ok ? i : 0)) * kD + c8;
    const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
    const uint4 wv = ok ? *reinterpret_cast<const uint4*>(w + go) : z4;
    *reinterpret_cast<uint4*>(Ws + a * kLDB + c8) = wv;
    *reinterpret_cast<uint4*>(Qs + a * kLDB + c8) = ok ? *reinterpret_cast<const uint4*>(q + go) : z4;
    *reinterpret_cast<uint4*>(Ks + a * kLDB + c8) = ok ? *reinterpret_cast<const uint4*>(k + go) : z4;
    const bf16x8 wb = __builtin_bit_cast(bf16x8, wv);
#pragma unroll
    for (int j = 0; j < 8; ++j) WTs[(c8 + j) * kLDB + a] = wb[j];
  }
  if (tid < 64) {
    const int64_t i = row0 + tid;
    Bs[tid] = i < L ? beta[bh * L + i] : 0.f;  // padded tokens: identity transitions
  }
  for (int e = tid; e < kC * kLDF; e += 256) Zf[e] = 0.f;
  if (logf != nullptr && wave == 0) {  // chunk-local inclusive prefix sum of the log-forget gates
    const int64_t i = row0 + l;
    float f = i < L ? logf[bh * L + i] : 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(f, o, 64);
      if (l >= o) f += y;
    }
    fl[bh * Lp + i] = f;
    if (l == 63) ftot[bh * M + c] = f;
  }
  __syncthreads();

  // ---------------------------------------------------------------- B: A, U^T, R, K Q^T
  f32x4 kq[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    // A[s][t] = beta_s (w_s . w_t) for s < t  (rows s in block `wave`)
    const f32x4 ga = mm_tile(Ws, Ws, 16 * wave, 16 * nb, zero);
    // D[t][a] = w_t . q_a  ->  U^T[a][t], t <= a
    const f32x4 ua = mm_tile(Ws, Qs, 16 * wave, 16 * nb, zero);
    // D[s][b] = w_s . k_b  ->  R[b][s], s > b
    const f32x4 ra = mm_tile(Ws, Ks, 16 * wave, 16 * nb, zero);
    const int col = 16 * nb + r;
    float um[4], rm[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * wave + 4 * g + i;
      Af[row * kLDF + col] = (row < col) ? Bs[row] * ga[i] : 0.f;
      um[i] = (row <= col) ? ua[i] : 0.f;
      rm[i] = (row > col) ? ra[i] : 0.f;
    }
    bf16x4 uh, ul, rh, rl;
    split4(um[0], um[1], um[2], um[3], uh, ul);
    split4(rm[0], rm[1], rm[2], rm[3], rh, rl);
    *reinterpret_cast<bf16x4*>(UTH + col * kLDB + 16 * wave + 4 * g) = uh;
    *reinterpret_cast<bf16x4*>(UTL + col * kLDB + 16 * wave + 4 * g) = ul;
    *reinterpret_cast<bf16x4*>(RH + col * kLDB + 16 * wave + 4 * g) = rh;
    *reinterpret_cast<bf16x4*>(RL + col * kLDB + 16 * wave + 4 * g) = rl;
    // D[b][a] = k_b . q_a for queries a in block `wave`
    kq[nb] = mm_tile(Ks, Qs, 16 * nb, 16 * wave, zero);
  }
  __syncthreads();

  // ---------------------------------------------------------------- C: diagonal 16x16 blocks of Z = A^{-1}
  if (l < 16) {
    const int base = 16 * wave;
    float z[16];
#pragma unroll
    for (int ii = 15; ii >= 0; --ii) {
      float s = 0.f;
#pragma unroll
      for (int kk = ii + 1; kk < 16; ++kk) s += Af[(base + ii) * kLDF + base + kk] * z[kk];
      z[ii] = (ii == l) ? 1.f : (ii < l ? -s : 0.f);
    }
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) Zf[(base + ii) * kLDF + base + l] = z[ii];
  }
  __syncthreads();

  // ---------------------------------------------------------------- D: off-diagonal blocks, by distance
  // Z_IJ = -Z_II sum_{K=I+1..J} A_IK Z_KJ
  for (int lv = 1; lv < 4; ++lv) {
    const int nblk = 4 - lv;
    for (int e = tid; e < nblk * 256; e += 256) {
      const int I = e >> 8, ii = (e >> 4) & 15, jj = e & 15, J = I + lv;
      float s = 0.f;
      for (int K = I + 1; K <= J; ++K)
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) s += Af[(16 * I + ii) * kLDF + 16 * K + kk] * Zf[(16 * K + kk) * kLDF + 16 * J + jj];
      Tmp[e] = s;
    }
    __syncthreads();
    for (int e = tid; e < nblk * 256; e += 256) {
      const int I = e >> 8, ii = (e >> 4) & 15, jj = e & 15, J = I + lv;
      float s = 0.f;
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) s += Zf[(16 * I + ii) * kLDF + 16 * I + kk] * Tmp[(I << 8) + (kk << 4) + jj];
      Zf[(16 * I + ii) * kLDF + 16 * J + jj] = -s;
    }
    __syncthreads();
  }

  // T^{-1} = Z diag(beta) as hi/lo bf16, row-major and transposed
  for (int e = tid; e < kC * kC; e += 256) {
    const int s = e >> 6, t = e & 63;
    __bf16 hi, lo;
    split_hi_lo(Zf[s * kLDF + t] * Bs[t], hi, lo);
    TiH[s * kLDB + t] = hi;
    TiL[s * kLDB + t] = lo;
    TiTH[t * kLDB + s] = hi;
    TiTL[t * kLDB + s] = lo;
  }
  __syncthreads();

  // ---------------------------------------------------------------- E: X^T, Y, (T^{-1}W)^T, each hi/lo
  // (hi+lo)(hi+lo) products drop the lo*lo term.
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int col = 16 * nb + r, m0 = 16 * wave, n0 = 16 * nb;
    bf16x4 h4, l4;
    // D[s][a] = X[s][a]  ->  X^T[a][s]
    f32x4 xa = mm_tile(TiH, UTH, m0, n0, zero);
    xa = mm_tile(TiH, UTL, m0, n0, xa);
    xa = mm_tile(TiL, UTH, m0, n0, xa);
    split4(xa[0], xa[1], xa[2], xa[3], h4, l4);
    *reinterpret_cast<bf16x4*>(XTH + col * kLDB + m0 + 4 * g) = h4;
    *reinterpret_cast<bf16x4*>(XTL + col * kLDB + m0 + 4 * g) = l4;
    // D[t][b] = Y[b][t]  ->  Y[b][t]
    f32x4 ya = mm_tile(TiTH, RH, m0, n0, zero);
    ya = mm_tile(TiTH, RL, m0, n0, ya);
    ya = mm_tile(TiTL, RH, m0, n0, ya);
    split4(ya[0], ya[1], ya[2], ya[3], h4, l4);
    *reinterpret_cast<bf16x4*>(YH + col * kLDB + m0 + 4 * g) = h4;
    *reinterpret_cast<bf16x4*>(YL + col * kLDB + m0 + 4 * g) = l4;
    // D[s][y] = (T^{-1} W)[s][y]  ->  Z2^T[y][s]
    f32x4 za = mm_tile(TiH, WTs, m0, n0, zero);
    za = mm_tile(TiL, WTs, m0, n0, za);
    split4(za[0], za[1], za[2], za[3], h4, l4);
    *reinterpret_cast<bf16x4*>(Z2H + col * kLDB + m0 + 4 * g) = h4;
    *reinterpret_cast<bf16x4*>(Z2L + col * kLDB + m0 + 4 * g) = l4;
  }
  __syncthreads();

  // ---------------------------------------------------------------- F: outputs
  const size_t chunk_rows = (size_t)bh * Lp + row0;
  const size_t chunk_mat = ((size_t)bh * M + c) * kD * kD;
  const int a = 16 * wave + r;  // query / key / P-row handled by this lane
  const int64_t ia = row0 + a;
  const bool aok = ia < L;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int x0 = 16 * mb + 4 * g;  // first of this lane's four consecutive columns
    const int pos = perm_pos(x0);
    const size_t gin = ((size_t)bh * L + (aok ? ia : 0)) * kD + x0;
    // qtilde[a][x] = q_a[x] - sum_s X[s][a] w_s[x]
    {
      f32x4 d4 = mm_tile(WTs, XTH, 16 * mb, 16 * wave, zero);
      d4 = mm_tile(WTs, XTL, 16 * mb, 16 * wave, d4);
      bf16x4 q4 = {};
      if (aok) q4 = *reinterpret_cast<const bf16x4*>(q + gin);
      bf16x4 h4, l4;
      split4((float)q4[0] - d4[0], (float)q4[1] - d4[1], (float)q4[2] - d4[2], (float)q4[3] - d4[3], h4, l4);
      *reinterpret_cast<bf16x4*>(qt + (chunk_rows + a) * kD + pos) = h4;
      if (qt_lo != nullptr) *reinterpret_cast<bf16x4*>(qt_lo + (chunk_rows + a) * kD + pos) = l4;
    }
    // ktilde[b][x] = k_b[x] - sum_t Y[b][t] w_t[x]
    {
      f32x4 d4 = mm_tile(WTs, YH, 16 * mb, 16 * wave, zero);
      d4 = mm_tile(WTs, YL, 16 * mb, 16 * wave, d4);
      bf16x4 k4 = {};
      if (aok) k4 = *reinterpret_cast<const bf16x4*>(k + gin);
      *reinterpret_cast<bf16x4*>(kt + (chunk_rows + a) * kD + pos) =
          pack4((float)k4[0] - d4[0], (float)k4[1] - d4[1], (float)k4[2] - d4[2], (float)k4[3] - d4[3]);
    }
    // P[x][y] = delta - sum_s w_s[x] Z2[s][y]   (lane: row x = a, columns y = x0..x0+3)
    {
      f32x4 d4 = mm_tile(Z2H, WTs, 16 * mb, 16 * wave, zero);
      d4 = mm_tile(Z2L, WTs, 16 * mb, 16 * wave, d4);
      bf16x4 ph, pl;
      split4((x0 == a ? 1.f : 0.f) - d4[0], (x0 + 1 == a ? 1.f : 0.f) - d4[1], (x0 + 2 == a ? 1.f : 0.f) - d4[2],
             (x0 + 3 == a ? 1.f : 0.f) - d4[3], ph, pl);
      *reinterpret_cast<bf16x4*>(p_hi + chunk_mat + (size_t)a * kD + pos) = ph;
      if (p_lo != nullptr) *reinterpret_cast<bf16x4*>(p_lo + chunk_mat + (size_t)a * kD + pos) = pl;
    }
    // S[a][b] = q_a.k_b - (Y U)[b][a]   (lane: query a, keys b = x0..x0+3)
    {
      f32x4 d4 = mm_tile(YH, UTH, 16 * mb, 16 * wave, zero);
      d4 = mm_tile(YH, UTL, 16 * mb, 16 * wave, d4);
      d4 = mm_tile(YL, UTH, 16 * mb, 16 * wave, d4);
      const float4 s4 = make_float4(kq[mb][0] - d4[0], kq[mb][1] - d4[1], kq[mb][2] - d4[2], kq[mb][3] - d4[3]);
      *reinterpret_cast<float4*>(Sm + (((size_t)bh * M + c) * kC + a) * kC + x0) = s4;
    }
  }
}

// =========================================================================== kernel 2: attention
// LDS tiles of the key-chunk stream are 64 rows x 128 B with no padding; the 16-byte chunk c of
// row r sits at slot c ^ (r & 7) (an XOR swizzle), so the 16 rows an MFMA fragment read touches
// land in distinct banks.  Tiles are filled by direct global->LDS loads (16 B per lane, lane i
// of an instruction writes slot i of a 1 KiB run), so no staging registers are needed: each lane
// simply fetches the global chunk that belongs in its slot.
constexpr int kTile = kC * kD;  // bf16 elements of one swizzled 64x64 tile

__device__ __forceinline__ int swz(int row, int chunk) { return row * 64 + ((chunk ^ (row & 7)) << 3); }

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));

// Direct global->LDS copy of one 64x64 bf16 tile (row stride `gstride` elements in global) by
// one wave: instructions i0, i0+1 each cover 8 rows.  Rows at or beyond `rmax` are clamped to
// rmax - 1 (finite data that only ever meets masked or discarded positions).
__device__ __forceinline__ void dma_tile(__bf16* tile, const __bf16* src, int64_t gstride, int rmax, int i0) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int i = i0; i < i0 + 2; ++i) {
    const int row = 8 * i + (l >> 3), slot = l & 7;
    const int rs = row < rmax ? row : rmax - 1;
    const __bf16* g = src + (int64_t)rs * gstride + ((slot ^ (row & 7)) << 3);
    __builtin_amdgcn_global_load_lds((const void*)g, (lds_void*)(tile + i * 512), 16, 0, 0);
  }
}

__device__ __forceinline__ bf16x8 tile_frag(const __bf16* tile, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(tile + swz(row, chunk));
}

// V^T A-fragment from a row-major V tile ([key][d]) with two LDS transpose reads: lane (r, g) of
// d-tile dt, k-step ks receives V[key][16dt + r] for keys 32ks + 16h + 4g + (0..3), h = 0, 1
// (the same key order as the P^T B-operand).  Within a 16-lane group the transpose read gives
// lane d element (d & 3) of source lanes (d >> 2) + 4j; source lane s therefore points at
// row base + (s >> 2), columns 16dt + 4(s & 3) .. +3.
__device__ __forceinline__ bf16x8 vt_frag(const __bf16* tile, int dt, int ks) {
  const int l = threadIdx.x & 63, g = l >> 4, s = l & 15;
  const int col = 16 * dt + 4 * (s & 3);
  bf16x8 out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 32 * ks + 16 * h + 4 * g + (s >> 2);
    const __bf16* p = tile + swz(row, col >> 3) + (col & 7);
    const v4i16 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(p));
#pragma unroll
    for (int j = 0; j < 4; ++j) out[4 * h + j] = __builtin_bit_cast(__bf16, (short)t[j]);
  }
  return out;
}

#ifndef PATHATTN_SCAN_WAVES_PER_SIMD
#define PATHATTN_SCAN_WAVES_PER_SIMD 2
#endif

// Max / sum over the 4 lanes holding the same query column (lanes l, l^16, l^32, l^48): each
// permlane swap returns the value pair {own, partner} for the two lane halves it exchanges.
// The maxima use the NaN-propagating maximum, which needs no input canonicalisation.
__device__ __forceinline__ float max2(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max3(float a, float b, float c) { return max2(max2(a, b), c); }
__device__ __forceinline__ float colmax4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max2(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max2(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float colsum4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Blocks are laid out for the 8 XCDs (workgroup b runs on XCD b % 8, each with its own L2):
// every query block of one (batch, head) lands on the same XCD, heads are dealt round-robin
// to XCDs, and within a head the longest rows go first.
constexpr int kXcd = 8;
// Work split: a block of 4 waves owns kCpb consecutive query chunks; each chunk's 64 queries
// are shared by kWpc waves of kQt 16-query MFMA column tiles each.
constexpr int kQt = 2;
constexpr int kWpc = 4 / kQt;
constexpr int kCpb = 4 / kWpc;

// Waves per SIMD the scan is built for (register budget 512 / waves).
template <bool FOX, bool X3>
__global__ __launch_bounds__(256, X3 ? 2 : PATHATTN_SCAN_WAVES_PER_SIMD) void mfma_attn_kernel(
    const __bf16* __restrict__ qt, const __bf16* __restrict__ qt_lo, const __bf16* __restrict__ kt,
    const __bf16* __restrict__ v, const __bf16* __restrict__ p_hi, const __bf16* __restrict__ p_lo,
    const float* __restrict__ Sm, const float* __restrict__ fl, const float* __restrict__ ftot,
    __bf16* __restrict__ out, float* __restrict__ lse, int64_t L, int64_t M, int64_t BH, float sc) {
  constexpr int NM = X3 ? 4 : 3;  // ktilde, V, P hi [, P lo]
  constexpr float kRescale = 8.f;  // log2 headroom before the running max must be raised
  __shared__ __align__(1024) __bf16 lds[2][NM][kTile];
  __shared__ __align__(16) float lfl[2][64];

  const int64_t nP = (M + kCpb - 1) / kCpb;
  const int xcd = (int)(blockIdx.x % kXcd);
  const int64_t slot = blockIdx.x / kXcd;
  const int64_t heads_here = (BH - xcd + kXcd - 1) / kXcd;
  if (slot >= heads_here * nP) return;  // whole block: this XCD has fewer heads
  const int64_t bh = xcd + kXcd * (slot / nP);
  const int64_t p = nP - 1 - slot % nP;

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63, r = l & 15, g = l >> 4;
  const int64_t m = kCpb * p + wave / kWpc;  // this wave's query chunk
  const int q0 = 16 * kQt * (wave % kWpc);   // first query (within the chunk) of this wave
  const bool active = m < M;
  const int64_t Lp = M * kC;
  const int64_t mtop = (kCpb * p + kCpb - 1 < M - 1) ? kCpb * p + kCpb - 1 : M - 1;  // highest chunk here
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  f32x4 o[4][kQt];  // O^T tiles [d tile][query tile]
  float lsum[kQt];  // this lane's share of each column's softmax denominator (fp32)
  float mref[kQt];  // running reference max per query column (log2 units)
  bf16x8 qb[kQt][2], ql[kQt][2];
#pragma unroll
  for (int a = 0; a < kQt; ++a) {
    mref[a] = -INFINITY;
    lsum[a] = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) o[b][a] = zero;
#pragma unroll
    for (int b = 0; b < 2; ++b) qb[a][b] = ql[a][b] = bf16x8{};
  }
  int buf = 0;  // LDS buffer holding the chunk being scored

  // Online softmax over one 32-key half (key tiles 2h, 2h+1) of a chunk.  z holds logits in
  // log2 units.  The reference max is raised only when some column's max exceeds it by more
  // than kRescale, so most halves skip the O rescale.  pb receives P^T for k-step h.
  auto absorb = [&](f32x4 (&z)[2][kQt], bf16x8 (&pb)[kQt]) {
    float mz[kQt];
    bool raise = false;
#pragma unroll
    for (int qi = 0; qi < kQt; ++qi) {
      const float m0 = max3(z[0][qi][0], z[0][qi][1], z[0][qi][2]);
      const float m1 = max3(z[0][qi][3], z[1][qi][0], z[1][qi][1]);
      mz[qi] = colmax4(max3(max3(m0, m1, z[1][qi][2]), z[1][qi][3], -INFINITY));
      raise |= mz[qi] > mref[qi] + kRescale;
    }
    if (__any(raise)) {
#pragma unroll
      for (int qi = 0; qi < kQt; ++qi) {
        const float mnew = max2(mref[qi], mz[qi]);
        const float base = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = fast_exp2(mref[qi] - base);
        lsum[qi] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt][qi] *= alpha;
        mref[qi] = base;
      }
    }
#pragma unroll
    for (int qi = 0; qi < kQt; ++qi) {
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = fast_exp2(z[u][qi][i] - mref[qi]);
          ps += pv;
          pb[qi][4 * u + i] = (__bf16)pv;
        }
      lsum[qi] += ps;
    }
  };
  auto pv_update = [&](const __bf16* Vn, int ks, const bf16x8 (&pb)[kQt]) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const bf16x8 a = vt_frag(Vn, dt, ks);
#pragma unroll
      for (int qi = 0; qi < kQt; ++qi) o[dt][qi] = mfma16(a, pb[qi], o[dt][qi]);
    }
  };
  // Scaled logits (log2 units) of key tiles 2h, 2h+1 against the running queries, plus the
  // PaTH-FoX bias sum_{s=j+1..i} f_s = (chunk-local prefix at i) + off - (prefix at j), whose
  // row-constant first term cancels in the softmax.
  auto logits_half = [&](const __bf16* Kn, int h, float offv, f32x4 (&z)[2][kQt]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int qi = 0; qi < kQt; ++qi) z[u][qi] = zero;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 a = tile_frag(Kn, 16 * (2 * h + u) + r, 4 * ks + g);
#pragma unroll
        for (int qi = 0; qi < kQt; ++qi) {
          z[u][qi] = mfma16(a, qb[qi][ks], z[u][qi]);
          if (X3) z[u][qi] = mfma16(a, ql[qi][ks], z[u][qi]);  // logits see the query residual
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float bias = FOX ? kLog2e * (offv - lfl[buf][16 * (2 * h + u) + 4 * g + i]) : 0.f;
#pragma unroll
        for (int qi = 0; qi < kQt; ++qi) z[u][qi][i] = __builtin_fmaf(z[u][qi][i], sc, bias);
      }
  };

  // Stage key chunk n into LDS buffer b (each wave moves a quarter of every tile).
  auto stage = [&](int64_t n, int b) {
    const int i0 = 2 * wave;
    dma_tile(lds[b][0], kt + ((size_t)bh * Lp + n * kC) * kD, kD, kC, i0);
    const int64_t vrows = L - n * kC;
    dma_tile(lds[b][1], v + ((size_t)bh * L + n * kC) * kD, kD, vrows < kC ? (int)vrows : kC, i0);
    dma_tile(lds[b][2], p_hi + ((size_t)bh * M + n) * kD * kD, kD, kC, i0);
    if (X3) dma_tile(lds[b][NM - 1], p_lo + ((size_t)bh * M + n) * kD * kD, kD, kC, i0);
    if (FOX && wave == 0)
      __builtin_amdgcn_global_load_lds((const void*)(fl + bh * Lp + n * kC + l), (lds_void*)lfl[b], 4, 0, 0);
  };

  stage(mtop, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's LDS writes have landed
  __syncthreads();
  float off = 0.f;
  for (int64_t n = mtop; n >= 0; --n) {
    if (n > 0) stage(n - 1, buf ^ 1);  // safe: every wave finished reading buf^1 before the last barrier
    const __bf16* Kn = lds[buf][0];
    const __bf16* Vn = lds[buf][1];
    const __bf16* Pn = lds[buf][2];
    if (active && n == m) {
      // ---------------------------------------------------------- own chunk: in-chunk logits
      const float* Sb = Sm + ((size_t)bh * M + m) * kC * kC;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 z[2][kQt];
#pragma unroll
        for (int qi = 0; qi < kQt; ++qi)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int kti = 2 * h + u, a = q0 + 16 * qi + r;
            const float4 s4 = *reinterpret_cast<const float4*>(Sb + a * kC + 16 * kti + 4 * g);
            const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int b = 16 * kti + 4 * g + i;
              const float fb = FOX ? kLog2e * lfl[buf][b] : 0.f;
              z[u][qi][i] = (b <= a) ? sv[i] * sc - fb : -INFINITY;
            }
          }
        bf16x8 pb[kQt];
        absorb(z, pb);
        pv_update(Vn, h, pb);
      }
#pragma unroll
      for (int qi = 0; qi < kQt; ++qi)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const size_t qo = ((size_t)bh * Lp + m * kC + q0 + 16 * qi + r) * kD + 32 * ks + 8 * g;
          qb[qi][ks] = *reinterpret_cast<const bf16x8*>(qt + qo);
          if (X3) ql[qi][ks] = *reinterpret_cast<const bf16x8*>(qt_lo + qo);
        }
    } else if (active && n < m) {
      // ---------------------------------------------------------- earlier chunk: transported queries
      // Per 32-key half: logits S^T = ktilde_n Q_run^T, online softmax, O^T += V^T P^T.  The
      // transport Q_run^T <- P_n Q_run^T for the next chunk is issued after the second half's
      // logits (the last reader of the current queries), so the matrix cores run it while the
      // vector units do that half's softmax.
      if (FOX) off += ftot[bh * M + n];
      {
        f32x4 z[2][kQt];
        logits_half(Kn, 0, off, z);
        bf16x8 pb[kQt];
        absorb(z, pb);
        pv_update(Vn, 0, pb);
      }
      {
        f32x4 z[2][kQt];
        logits_half(Kn, 1, off, z);
        if (n > 0) {
          f32x4 qn[4][kQt];
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
            for (int qi = 0; qi < kQt; ++qi) qn[dt][qi] = zero;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
              const bf16x8 a = tile_frag(Pn, 16 * dt + r, 4 * ks + g);
#pragma unroll
              for (int qi = 0; qi < kQt; ++qi) qn[dt][qi] = mfma16(a, qb[qi][ks], qn[dt][qi]);
              if (X3) {
                const bf16x8 alo = tile_frag(lds[buf][NM - 1], 16 * dt + r, 4 * ks + g);
#pragma unroll
                for (int qi = 0; qi < kQt; ++qi) {
                  qn[dt][qi] = mfma16(a, ql[qi][ks], qn[dt][qi]);
                  qn[dt][qi] = mfma16(alo, qb[qi][ks], qn[dt][qi]);
                }
              }
            }
          }
#pragma unroll
          for (int qi = 0; qi < kQt; ++qi)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const float vq = qn[2 * ks + (j >> 2)][qi][j & 3];
                const __bf16 hi = (__bf16)vq;
                qb[qi][ks][j] = hi;
                if (X3) ql[qi][ks][j] = (__bf16)(vq - (float)hi);
              }
        }
        bf16x8 pb[kQt];
        absorb(z, pb);
        pv_update(Vn, 1, pb);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next chunk's LDS writes from this wave have landed
    __syncthreads();
    buf ^= 1;
  }

  // ---------------------------------------------------------------- epilogue
#pragma unroll
  for (int qi = 0; qi < kQt; ++qi) {
    const float lt = colsum4(lsum[qi]);
    const int a = q0 + 16 * qi + r;
    const int64_t i = m * kC + a;
    if (active && i < L) {
      const float inv = 1.f / lt;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        *reinterpret_cast<bf16x4*>(out + ((size_t)bh * L + i) * kD + 16 * dt + 4 * g) =
            pack4(o[dt][qi][0] * inv, o[dt][qi][1] * inv, o[dt][qi][2] * inv, o[dt][qi][3] * inv);
      if (lse != nullptr && g == 0)
        lse[bh * L + i] = (mref[qi] + fast_log2(lt)) * kLn2 + (FOX ? fl[bh * Lp + i] : 0.f);
    }
  }
}

// =========================================================================== host
bool mfma_supported(int d, int chunk) { return d == kD && chunk == kC; }

template <bool FOX, bool X3>
static void launch_attn(dim3 grid, hipStream_t st, const __bf16* qt, const __bf16* qt_lo, const __bf16* kt,
                        const __bf16* v, const __bf16* p_hi, const __bf16* p_lo, const float* Sm, const float* fl,
                        const float* ftot, __bf16* out, float* lse, int64_t L, int64_t M, int64_t BH, float sc) {
  mfma_attn_kernel<FOX, X3><<<grid, 256, 0, st>>>(qt, qt_lo, kt, v, p_hi, p_lo, Sm, fl, ftot, out, lse, L, M, BH,
                                                  sc);
}

// phases: bit 0 = per-chunk prep, bit 1 = attention scan (reads what the prep left in the workspace).
hipError_t mfma_run(int phases, int chunk, int transport, const void* q, const void* k, const void* v,
                    const void* w, const float* beta, const float* logf, void* out, float* lse, int64_t BH,
                    int64_t L, float scale, void* qt, void* qt_lo, void* kt, void* p_hi, void* p_lo,
                    float* Sm, float* fl, float* ftot, hipStream_t st) {
  if (chunk != kC) return hipErrorInvalidValue;
  const int64_t M = (L + kC - 1) / kC;
  const bool x3 = transport == 1;
  hipError_t e = hipSuccess;
  if (phases & 1) {
    e = hipFuncSetAttribute((const void*)mfma_prep_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)kPrepLds);
    if (e != hipSuccess) return e;
    mfma_prep_kernel<<<dim3((unsigned)M, (unsigned)BH), 256, kPrepLds, st>>>(
        (const __bf16*)q, (const __bf16*)k, (const __bf16*)w, beta, logf, L, M, (__bf16*)qt,
        x3 ? (__bf16*)qt_lo : nullptr, (__bf16*)kt, (__bf16*)p_hi, x3 ? (__bf16*)p_lo : nullptr, Sm, fl, ftot);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & 2) {
    const int64_t heads_per_xcd = (BH + kXcd - 1) / kXcd;
    const dim3 grid((unsigned)(kXcd * heads_per_xcd * ((M + kCpb - 1) / kCpb)));
    const float sc = scale * kLog2e;
    const bool fox = logf != nullptr;
    auto args = [&](auto fn) {
      fn(grid, st, (const __bf16*)qt, (const __bf16*)qt_lo, (const __bf16*)kt, (const __bf16*)v,
         (const __bf16*)p_hi, (const __bf16*)p_lo, Sm, fl, ftot, (__bf16*)out, lse, L, M, BH, sc);
    };
    if (fox && x3) args(launch_attn<true, true>);
    else if (fox) args(launch_attn<true, false>);
    else if (x3) args(launch_attn<false, true>);
    else args(launch_attn<false, false>);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace pathattn

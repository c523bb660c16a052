// Matrix-core (bf16 MFMA, fp32 accumulate) PaTH prefill for head dim 64, chunk 64 or 128.
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
//   S[a][b] = q_a.k_b - (Y U)[b][a]   (b <= a; in-chunk logits)
// qtilde and S are stored multiplied by scale * log2(e), the scan's logit unit.
// T^{-1} and T^{-1} W enter the matrix cores as hi+lo bf16 pairs so that P is
// accurate enough to be split again into hi+lo for the long-range transport.
//
// Kernel 2 (attention), one workgroup of 4 waves per 2 consecutive query chunks (two waves of
// 32 queries per chunk), longest rows first.  The waves share one LDS stream of key chunks
// n = top ... 0 (ktilde_n, V_n straight from the value tensor, P_n; a ring of direct global->LDS
// copies issued one step ahead).  A wave scores its own chunk from the precomputed in-chunk logits
// when the stream reaches it, and earlier chunks as follows (queries pre-scaled by
// scale * log2(e), so logits come out in log2 units):
//   S^T = ktilde_n Q_run^T - m    (keys x queries; the running max m seeds the accumulator)
//   p = exp2(S^T), lazily checked against the running max; P^T kept as the PV B-operand
//   O^T += V_n^T P^T
//   Q_run^T <- P_n Q_run^T       (fp32 accumulate, re-rounded to bf16 [hi+lo])
// Column permutation: an MFMA accumulator gives each lane rows 4g..4g+3 of every
// 16-row tile, while a B-operand wants rows 8g..8g+7 of every 32-row k-step.  The
// contraction order is free, so qtilde, ktilde and P (columns) are stored with
// stored slot 8g+j of each 32-block holding index 16(j/4)+4g+(j%4), and V^T
// fragments are read (LDS transpose reads) in the same key order; accumulators then
// convert to B-operands in registers with no data movement.
#include <type_traits>

#include "tiles.h"

namespace pathattn {

// =========================================================================== kernel 1: prep
// One block of 4 waves per (b, h, chunk).  Operand conventions (16x16x32 MFMA, lane l, r = l%16,
// g = l/16): an accumulator gives lane (r, g) rows 4g..4g+3 of column r; converted in registers it
// serves directly as an A- or B-operand whose k index runs over those rows in the key order of
// tr_frag.  Every product below pairs such an operand with a tr_frag read or with a tile stored in
// permuted-column form, so the 64x64 intermediates X, Y, T^{-1}W, U and R never touch LDS:
// wave w owns query block a = 16w.. (X, U, KQ), key block b = 16w.. (Y, R, S) and y block 16w.. of
// T^{-1}W (for P).  LDS holds the DMA-loaded W, Q, K tiles, A (strict upper) with Z = A^{-1}
// stored transposed in its lower triangle, T^{-T} (hi, lo) and U^T (hi, lo, for S); T^{-T} reuses the
// space of Q and K (dead once the products of phase B are done; the few q and k values the final
// phase needs are kept in registers), U^T that of A (written once T^{-T} has been formed), so that
// three blocks share a CU.
//   A      = I + diag(beta) strict_upper(W W^T)        (fp32)
//   Z      = A^{-1}: 16x16 diagonal blocks by back substitution, then Z_IJ = -Z_II sum_K A_IK Z_KJ
//   T^{-1} = Z diag(beta)                              (hi + lo bf16)
//   X = T^{-1} U, U[t][a] = w_t.q_a (t <= a);  Y = R T^{-1}, R[b][s] = k_b.w_s (s > b)
//   qtilde = Q - X^T W,  ktilde = K - Y W,  P = I - W^T (T^{-1} W),  S^T = K Q^T - Y U
// hi/lo products drop lo*lo.  Padded tokens of a ragged last chunk are clamped copies of the last
// row with beta = 0, which makes every T^{-1} entry that would touch them exactly zero.
constexpr int kLDF = 68;  // fp32 row stride of A/Z
constexpr size_t kPrepLds = 3 * kTile * 2 + kC * kLDF * 4 + 2 * 64 * 4;
static_assert(kC * kLDF * 4 >= 2 * kTile * 2, "U^T hi/lo must fit in the space of A");
static_assert(kPrepLds <= 160 * 1024 / 3, "prep LDS plan must allow three blocks per CU");

__device__ __forceinline__ int perm_col(int c) { return perm_pos(c); }


// X3: the lo halves of qtilde and P (bf16x3 transport) are formed and stored; without it only hi.
// Zo (optional): Z = A^{-1} as well ([chunk][i][j] fp32, unit upper triangular, zeros below the
// diagonal), which the backward's gradient kernel needs.
template <bool X3>
__global__ __launch_bounds__(256, 3) void mfma_prep_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ w,
    const float* __restrict__ beta, const float* __restrict__ logf, int64_t L, int64_t M, float qs,
    __bf16* __restrict__ qt, __bf16* __restrict__ qt_lo, __bf16* __restrict__ kt, __bf16* __restrict__ p_hi, __bf16* __restrict__ p_lo,
    float* __restrict__ Sm, float* __restrict__ fl, float* __restrict__ ftot, float* __restrict__ Zo) {
  extern __shared__ __align__(1024) char smem[];
  __bf16* Wt = reinterpret_cast<__bf16*>(smem);  // W [s][x]            (swizzled, natural columns)
  __bf16* Qt = Wt + kTile;                       // Q [a][x]
  __bf16* Kt = Qt + kTile;                       // K [b][x]
  __bf16* TiH = Qt;                              // later: T^{-T} [t][s] hi / lo (swizzled, permuted columns)
  __bf16* TiL = Kt;
  float* Af = reinterpret_cast<float*>(Kt + kTile);  // A strict upper, Z^T lower incl. diagonal
  __bf16* UH = reinterpret_cast<__bf16*>(Af);        // later: U^T [a][t] hi / lo (swizzled, permuted columns)
  __bf16* UL = UH + kTile;
  float* Bs = Af + kC * kLDF;                        // beta
  float* Fs = Bs + 64;                               // unused pad (keeps the plan aligned)
  (void)Fs;

  // the wave index is wave-uniform: keep it in a scalar register, so that branches on it are uniform
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, r = l & 15, g = l >> 4;
  const int c = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t Lp = M * kC;
  const int64_t row0 = (int64_t)c * kC;
  const int64_t vr = L - row0;
  const int valid = vr < kC ? (int)vr : kC;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  auto mm = [](const bf16x8& a, const bf16x8& b, const f32x4& acc) { return mfma16(a, b, acc); };
  auto row_frag = [](const __bf16* tile, int row, int ks) {  // tile[row][32ks + 8g .. +7]
    const int g_ = (threadIdx.x & 63) >> 4;
    return tile_frag(tile, row, 4 * ks + g_);
  };

  // ---------------------------------------------------------------- A: stage W, Q, K, beta, FoX prefix
  {
    const int i0 = 2 * wave;
    const size_t base = ((size_t)bh * L + row0) * kD;
    dma_tile(Wt, w + base, valid, i0);
    dma_tile(Qt, q + base, valid, i0);
    dma_tile(Kt, k + base, valid, i0);
  }
  if (tid < 64) Bs[tid] = tid < valid ? beta[bh * L + row0 + tid] : 0.f;  // padded tokens: identity
  if (logf != nullptr && wave == 0) {  // chunk-local inclusive prefix sum of the log-forget gates
    float f = l < valid ? logf[bh * L + row0 + l] : 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(f, o, 64);
      if (l >= o) f += y;
    }
    fl[bh * Lp + row0 + l] = f;
    if (l == 63) ftot[bh * M + c] = f;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's tile loads have landed
  __syncthreads();

  // ---------------------------------------------------------------- B: A, U, R, K Q^T; diagonal block of Z
  bf16x8 ubh[2], ubl[2], rbh[2], rbl[2];
  f32x4 kq[4];
  {
    f32x4 ua[4], ra[4];
    const float4 bw = *reinterpret_cast<const float4*>(Bs + 16 * wave + 4 * g);  // beta of rows 16 wave + 4g + i
    const float bwi[4] = {bw.x, bw.y, bw.z, bw.w};
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      f32x4 ga = zero, u4 = zero, r4 = zero, k4 = zero;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 wr = row_frag(Wt, 16 * wave + r, ks);  // W rows of block `wave`
        const bf16x8 wc = row_frag(Wt, 16 * tt + r, ks);    // W rows of block tt
        ga = mm(wr, wc, ga);                                // D[s in wave][t in tt] = w_s . w_t
        u4 = mm(wc, row_frag(Qt, 16 * wave + r, ks), u4);   // D[t in tt][a in wave] = w_t . q_a
        r4 = mm(wc, row_frag(Kt, 16 * wave + r, ks), r4);   // D[s in tt][b in wave] = w_s . k_b
        k4 = mm(row_frag(Kt, 16 * wave + r, ks), row_frag(Qt, 16 * tt + r, ks), k4);  // D[b][a] = k_b.q_a
      }
      const int col_wave = 16 * wave + r;  // a or b of this lane
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rw = 16 * tt + 4 * g + i;  // t (for U) or s (for R)
        u4[i] = (rw <= col_wave) ? u4[i] : 0.f;
        r4[i] = (rw > col_wave) ? r4[i] : 0.f;
        // the lower triangle (zeros here) is overwritten by Z^T before anything reads it
        const int srow = 16 * wave + 4 * g + i, tcol = 16 * tt + r;
        Af[srow * kLDF + tcol] = (srow < tcol) ? bwi[i] * ga[i] : 0.f;
      }
      ua[tt] = u4;
      ra[tt] = r4;
      kq[tt] = k4;
    }
    acc_to_op(ua, ubh, ubl);
    acc_to_op(ra, rbh, rbl);
  }
  // the q and k values the final phase needs (row 16 wave + r, columns 16 xt + 4g ..), taken from the
  // tiles before their space is reused
  bf16x4 q4s[4], k4s[4];
#pragma unroll
  for (int xt = 0; xt < 4; ++xt) {
    const int row = 16 * wave + r, x0 = 16 * xt + 4 * g;
    q4s[xt] = *reinterpret_cast<const bf16x4*>(Qt + swz(row, x0 >> 3) + (x0 & 7));
    k4s[xt] = *reinterpret_cast<const bf16x4*>(Kt + swz(row, x0 >> 3) + (x0 & 7));
  }
  __builtin_amdgcn_wave_barrier();
  // Z_II (block I = wave) by back substitution, lane l < 16 owning column l = A_II^{-1} e_l; stored
  // transposed.  Column-oriented: once z[kk] is final its multiple of column kk of A leaves the rows
  // above, so the 15 dependent steps each carry up to 15 independent FMAs.
  if (l < 16) {
    const int base = 16 * wave;
    float z[16];
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) z[ii] = (ii == l) ? 1.f : 0.f;
#pragma unroll
    for (int kk = 15; kk >= 1; --kk)
#pragma unroll
      for (int ii = 0; ii < kk; ++ii) z[ii] = __builtin_fmaf(-Af[(base + ii) * kLDF + base + kk], z[kk], z[ii]);
    // (z[ii] = 0 for ii > l: those stores clear the block's upper half, whose A entries are no longer read)
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) Af[(base + l) * kLDF + base + ii] = z[ii];
  }
  __syncthreads();

  // ---------------------------------------------------------------- C: off-diagonal blocks of Z, two levels
  // Z[i][j] (i <= j) lives at Af[j][i]; the upper halves of the diagonal blocks' storage are zero.  With
  // 16 x 16 blocks I, J = 0..3:
  //   level 1 (waves 0, 2):  Z_{I,I+1} = -Z_II A_{I,I+1} Z_{I+1,I+1}, the 32 x 32 diagonal blocks of Z;
  //   level 2 (wave w: i = w / 2, j = 2 + w % 2):  the 32 x 32 corner
  //     T_kj = sum_{k'=2..j} A_{k k'} Z_{k' j}  (k = 0, 1),   Z_ij = -sum_{k=i..1} Z_ik T_kj,
  //   each wave forming every T it needs itself (T_1j twice), so the corner needs no barrier inside.
  // Products on the fp32 matrix cores (16x16x4: lane (r, q) brings A[r][q] and B[q][r]) from the fp32
  // LDS copy of A and Z; in Z T the contraction index kk = 4q + m of step m makes T's accumulator slot m
  // the B-operand of the same lane.  The first sums run in two accumulators.
  auto t_prod = [&](int row0, int k0, int steps, int J) PA_INLINE {  // sum_kk A[row0 + r][kk] Z[kk][16J + r]
    f32x4 t2[2] = {zero, zero};
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st < steps) {
        const int kk = k0 + 4 * st + g;
        const float a = Af[(row0 + r) * kLDF + kk];
        const float zv = Af[(16 * J + r) * kLDF + kk];
        const float b = (kk >= 16 * J && kk - 16 * J > r) ? 0.f : zv;  // Z_JJ is upper triangular
        t2[st & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, t2[st & 1], 0, 0, 0);
      }
    }
    return t2[0] + t2[1];
  };
  // zacc += Z[16I + r][16K + 4g + m] (block (I, K)) times T's slot m
  auto z_prod = [&](f32x4 zacc, int I, int K, const f32x4& t) PA_INLINE {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int kk = 4 * g + m;
      const float zv = Af[(16 * K + kk) * kLDF + 16 * I + r];
      const float a = (I == K && kk < r) ? 0.f : zv;
      zacc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, t[m], zacc, 0, 0, 0);
    }
    return zacc;
  };
  // lane (r, g) holds Z_IJ[4g + e][r] = Z[16I + 4g + e][16J + r], stored at Af[16J + r][16I + 4g + e]
  auto z_store = [&](int I, int J, const f32x4& z) PA_INLINE {
    *reinterpret_cast<float4*>(Af + (16 * J + r) * kLDF + 16 * I + 4 * g) = make_float4(-z[0], -z[1], -z[2], -z[3]);
  };
  if ((wave & 1) == 0) {  // level 1
    const int I = wave, J = wave + 1;
    z_store(I, J, z_prod(zero, I, I, t_prod(16 * I, 16 * J, 4, J)));
  }
  __syncthreads();
  {  // level 2
    const int i = wave >> 1, J = 2 + (wave & 1), steps = 4 * (J - 1);
    const f32x4 t1 = t_prod(16, 32, steps, J);
    if (i == 1) {
      z_store(1, J, z_prod(zero, 1, 1, t1));
    } else {
      const f32x4 t0 = t_prod(0, 32, steps, J);
      z_store(0, J, z_prod(z_prod(zero, 0, 0, t0), 0, 1, t1));
    }
  }
  __syncthreads();
  if (Zo != nullptr) {  // Z for the backward: Z[i][j] (i <= j) from Af[j][i]
    float* zc = Zo + ((size_t)bh * M + c) * kC * kC;
    for (int e = tid; e < kC * kC; e += 256) {
      const int i = e >> 6, j = e & 63;
      zc[e] = i <= j ? Af[j * kLDF + i] : 0.f;
    }
  }

  // T^{-T}[t][s] = Z[s][t] beta_t (t >= s), hi/lo, stored with permuted columns: stored slots 8 ch + j
  // of row t hold columns c0 + 16 (j / 4) + j % 4, c0 = 32 (ch / 4) + 4 (ch % 4)
  for (int e = tid; e < 512; e += 256) {
    const int t = e >> 3, ch = e & 7, c0 = 32 * (ch >> 2) + 4 * (ch & 3);
    const float4 v0 = *reinterpret_cast<const float4*>(Af + t * kLDF + c0);
    const float4 v1 = *reinterpret_cast<const float4*>(Af + t * kLDF + c0 + 16);
    const float zt[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    const float bt = Bs[t];
    bf16x8 h8, l8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sc_ = c0 + 16 * (j >> 2) + (j & 3);  // column held
      const float v = (t >= sc_) ? zt[j] * bt : 0.f;
      const __bf16 hh = (__bf16)v;
      h8[j] = hh;
      l8[j] = (__bf16)(v - (float)hh);
    }
    *reinterpret_cast<bf16x8*>(TiH + swz(t, ch)) = h8;
    *reinterpret_cast<bf16x8*>(TiL + swz(t, ch)) = l8;
  }
  __syncthreads();
  // A is no longer needed: U^T[a][t] (hi/lo) for the S product of the other waves, from this wave's U
  // operand (4 consecutive t of column a = 16 wave + r per accumulator tile, in permuted order)
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int ks = tt >> 1, h = tt & 1;
    const bf16x4 h4 = {ubh[ks][4 * h], ubh[ks][4 * h + 1], ubh[ks][4 * h + 2], ubh[ks][4 * h + 3]};
    const bf16x4 l4 = {ubl[ks][4 * h], ubl[ks][4 * h + 1], ubl[ks][4 * h + 2], ubl[ks][4 * h + 3]};
    const int pc = perm_pos(16 * tt + 4 * g), col_wave = 16 * wave + r;
    *reinterpret_cast<bf16x4*>(UH + swz(col_wave, pc >> 3) + (pc & 7)) = h4;
    *reinterpret_cast<bf16x4*>(UL + swz(col_wave, pc >> 3) + (pc & 7)) = l4;
  }

  // ---------------------------------------------------------------- D: register-resident products
  const int a = 16 * wave + r;  // query / key row of this lane's output column
  const int64_t ia = row0 + a;
  const size_t chunk_rows = (size_t)bh * Lp + row0;
  const size_t chunk_mat = ((size_t)bh * M + c) * kD * kD;
  // X[s][a] = sum_t T^{-1}[s][t] U[t][a]          (s tiles st; a in this wave's block)
  // Y^T[t][b] = sum_s T^{-T}[t][s] R[b][s]         (t tiles tt; b in this wave's block)
  // Z2[s][y] = sum_t T^{-1}[s][t] W[t][y]          (s tiles st; y in this wave's block)
  bf16x8 xbh[2], xbl[2], ybh[2], ybl[2], zbh[2], zbl[2];
  {
    f32x4 xa[4], ya[4], za[4];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      f32x4 x4 = zero, y4 = zero, z4 = zero;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 th = tr_frag(TiH, 16 * t4, ks, perm_col);  // T^{-1} rows s = 16 t4 + r, k = t
        const bf16x8 tl = tr_frag(TiL, 16 * t4, ks, perm_col);
        x4 = mm(th, ubh[ks], x4);
        x4 = mm(th, ubl[ks], x4);
        x4 = mm(tl, ubh[ks], x4);
        const bf16x8 wy = tr_frag(Wt, 16 * wave, ks, col_identity);  // W[t][y], y in this block
        z4 = mm(th, wy, z4);
        z4 = mm(tl, wy, z4);
        const bf16x8 gh = row_frag(TiH, 16 * t4 + r, ks);  // T^{-T} rows t = 16 t4 + r, k = s
        const bf16x8 gl = row_frag(TiL, 16 * t4 + r, ks);
        y4 = mm(gh, rbh[ks], y4);
        y4 = mm(gh, rbl[ks], y4);
        y4 = mm(gl, rbh[ks], y4);
      }
      xa[t4] = x4;
      ya[t4] = y4;
      za[t4] = z4;
    }
    acc_to_op(xa, xbh, xbl);  // X as an operand over k = s, column a
    acc_to_op(ya, ybh, ybl);  // Y as an operand over k = t, row/column b
    acc_to_op(za, zbh, zbl);  // (T^{-1}W)^T as an operand over k = s, row y
  }
  __syncthreads();  // every wave's U^T is in place
#pragma unroll
  for (int xt = 0; xt < 4; ++xt) {
    const int x0 = 16 * xt + 4 * g;  // this lane's four consecutive output columns
    const int pos = perm_pos(x0);
    f32x4 dq = zero, dk = zero, dp = zero, ds = zero;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 wtx = tr_frag(Wt, 16 * xt, ks, col_identity);  // W^T rows x = 16 xt + r, k = s
      dq = mm(wtx, xbh[ks], dq);  // D[x][a] = sum_s W[s][x] X[s][a]
      dq = mm(wtx, xbl[ks], dq);
      dk = mm(wtx, ybh[ks], dk);  // D[x][b] = sum_t W[t][x] Y[b][t]
      dk = mm(wtx, ybl[ks], dk);
      dp = mm(zbh[ks], wtx, dp);  // D[y][x] = sum_s Z2[s][y] W[s][x]
      dp = mm(zbl[ks], wtx, dp);
      const bf16x8 uh = row_frag(UH, 16 * xt + r, ks);  // U^T rows a = 16 xt + r, k = t
      const bf16x8 ul = row_frag(UL, 16 * xt + r, ks);
      ds = mm(ybh[ks], uh, ds);  // D[b][a] = sum_t Y[b][t] U[t][a]
      ds = mm(ybh[ks], ul, ds);
      ds = mm(ybl[ks], uh, ds);
    }
    // qtilde[a][x] = (q_a[x] - D[x][a]) * qs  (lane: row a, columns x0..x0+3)
    {
      const bf16x4 q4 = q4s[xt];
      const float v0 = ((float)q4[0] - dq[0]) * qs, v1 = ((float)q4[1] - dq[1]) * qs,
                  v2 = ((float)q4[2] - dq[2]) * qs, v3 = ((float)q4[3] - dq[3]) * qs;
      if constexpr (X3) {
        bf16x4 h4, l4;
        split4(v0, v1, v2, v3, h4, l4);
        *reinterpret_cast<bf16x4*>(qt + (chunk_rows + a) * kD + pos) = h4;
        *reinterpret_cast<bf16x4*>(qt_lo + (chunk_rows + a) * kD + pos) = l4;
      } else {
        *reinterpret_cast<bf16x4*>(qt + (chunk_rows + a) * kD + pos) = pack4(v0, v1, v2, v3);
      }
    }
    // ktilde[b][x] = k_b[x] - D[x][b]
    {
      const bf16x4 k4 = k4s[xt];
      const float u0 = (float)k4[0] - dk[0], u1 = (float)k4[1] - dk[1], u2 = (float)k4[2] - dk[2],
                  u3 = (float)k4[3] - dk[3];
      *reinterpret_cast<bf16x4*>(kt + (chunk_rows + a) * kD + pos) = pack4(u0, u1, u2, u3);
    }
    // P[x][y] = delta - D[y][x]  (lane: row x = 16 xt + r, columns y = 16 wave + 4g .. +3)
    {
      const int xr = 16 * xt + r, y0 = 16 * wave + 4 * g;
      const float e0 = (y0 == xr ? 1.f : 0.f) - dp[0], e1 = (y0 + 1 == xr ? 1.f : 0.f) - dp[1],
                  e2 = (y0 + 2 == xr ? 1.f : 0.f) - dp[2], e3 = (y0 + 3 == xr ? 1.f : 0.f) - dp[3];
      const int py = perm_pos(y0);
      if constexpr (X3) {
        bf16x4 ph, pl;
        split4(e0, e1, e2, e3, ph, pl);
        *reinterpret_cast<bf16x4*>(p_hi + chunk_mat + (size_t)xr * kD + py) = ph;
        *reinterpret_cast<bf16x4*>(p_lo + chunk_mat + (size_t)xr * kD + py) = pl;
      } else {
        *reinterpret_cast<bf16x4*>(p_hi + chunk_mat + (size_t)xr * kD + py) = pack4(e0, e1, e2, e3);
      }
    }
    // S[a][b] = (q_a.k_b - D[b][a]) * qs  (lane: query a = 16 xt + r, keys b = 16 wave + 4g .. +3), as the
    // packed lower triangle
    {
      const int aq = 16 * xt + r, b0 = 16 * wave + 4 * g;
      const float4 s4 = make_float4((kq[xt][0] - ds[0]) * qs, (kq[xt][1] - ds[1]) * qs, (kq[xt][2] - ds[2]) * qs,
                                    (kq[xt][3] - ds[3]) * qs);
      if (b0 <= aq)
        *reinterpret_cast<float4*>(Sm + (((size_t)bh * M + c) * kSGroups + s_row_group(aq) + (b0 >> 2)) * 4) = s4;
    }
  }
  (void)ia;
}

// =========================================================================== kernel 2: attention
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


// Blocks are laid out for the 8 XCDs (workgroup b runs on XCD b % 8, each with its own L2):
// every query block of one (batch, head) lands on the same XCD, heads are dealt round-robin
// to XCDs, and within a head the longest rows go first.
constexpr int kXcd = 8;
#ifndef PATHATTN_SCAN_HGROUP
#define PATHATTN_SCAN_HGROUP 4
#endif
constexpr int64_t kHeadGroup = PATHATTN_SCAN_HGROUP;

#ifndef PATHATTN_SCAN_QT
#define PATHATTN_SCAN_QT 2
#endif
#ifndef PATHATTN_SCAN_BLOCK_WAVES
#define PATHATTN_SCAN_BLOCK_WAVES 4
#endif
// Work split: a block of W waves owns consecutive query chunks; each chunk's 64 queries are shared
// by 4 / QT waves of QT 16-query MFMA column tiles each.  QT = 2 runs two waves per SIMD, QT = 4
// one (each LDS fragment then feeds four MFMAs instead of two).  With W = 8 the two waves of a SIMD
// belong to one block and every key chunk copied to LDS serves twice the queries.
template <bool X3, int QT, int W>
struct ScanShape {
  static_assert(QT == 2 || QT == 4, "16-query tiles per wave");
  static_assert(W == 4 || W == 8, "waves per block");
  static constexpr int kWpc = 4 / QT;                  // waves per query chunk
  static constexpr int kCpb = W / kWpc;                // query chunks per block
  static constexpr int kWaves = QT == 2 ? 2 : 1;       // waves per SIMD
  static constexpr int kNm = X3 ? 4 : 3;               // tiles per key chunk (ktilde, V, P hi [, P lo])
  static constexpr int kBuf = (X3 && QT == 2 && W == 4) ? 2 : 3;  // LDS ring depth
  static constexpr int kCopies = 8 / W;                // copy instructions per wave per tile
  static constexpr int kOps = kNm * kCopies;           // copy instructions per wave per chunk (+1 FoX)
};

// Attention scan.  Block-wide stream of key chunks n = top chunk ... 0, each {ktilde_n (or its
// carried form), V_n, P_n [, P_lo n] (or the group product), FoX prefix of chunk n}.  Per wave, with
// its query chunk m (chunks above m are skipped):
//   n == m (own chunk):  logits from the precomputed in-chunk S (masked), exact row max, P^T V_m;
//                        running queries Q_run = qtilde.
//   n <  m:              z = ktilde_n Q_run^T minus the running max (which seeds the MFMA
//                        accumulator), p = exp2(z), O^T += V_n^T p^T, and, when a chunk below
//                        follows, Q_run^T <- P_n Q_run^T.
// The running max is raised lazily: a lane whose partial row sum exceeds 2^kRescale (so possibly
// some p > 2^kRescale) sends the wave through the exact max, which raises the reference of any
// column whose max exceeds it by more than kRescale and rescales O, the sums and the pending logits.
template <bool FOX, bool X3, int G, int QT, int W>
__global__ __launch_bounds__(64 * W, (ScanShape<X3, QT, W>::kWaves)) void mfma_attn_kernel(
    const __bf16* __restrict__ qt, const __bf16* __restrict__ qt_lo, const __bf16* __restrict__ kt,
    const __bf16* __restrict__ v, const __bf16* __restrict__ p_hi, const __bf16* __restrict__ p_lo,
    const __bf16* __restrict__ ktc, const __bf16* __restrict__ pg_hi, const __bf16* __restrict__ pg_lo,
    const float* __restrict__ Sm, const float* __restrict__ fl, const float* __restrict__ ftot,
    __bf16* __restrict__ out, float* __restrict__ lse, int64_t L, int64_t M, int64_t BH) {
  using Sh = ScanShape<X3, QT, W>;
  constexpr int NM = Sh::kNm, NB = Sh::kBuf, kWpc = Sh::kWpc, kCpb = Sh::kCpb, kCp = Sh::kCopies;
  constexpr int OPS = Sh::kOps + (FOX ? 1 : 0);
  constexpr float kRescale = 8.f;     // log2 headroom before the running max must be raised
  constexpr float kSumCap = 256.f;    // 2^kRescale
  __shared__ __align__(1024) __bf16 lds[NB][NM][kTile];
  __shared__ __align__(16) float lfl[NB][64];

  const int64_t nP = (M + kCpb - 1) / kCpb;
  const int xcd = (int)(blockIdx.x % kXcd);
  const int64_t slot = blockIdx.x / kXcd;
  const int64_t heads_here = (BH - xcd + kXcd - 1) / kXcd;
  if (slot >= heads_here * nP) return;  // whole block: this XCD has fewer heads
  // Heads are taken in groups of kHeadGroup; within a group the blocks go longest first across the
  // group's heads, so the short blocks of one group fill in behind the long ones of the next.
  const int64_t grp = slot / (kHeadGroup * nP), in_grp = slot % (kHeadGroup * nP);
  const int64_t grp_heads = (heads_here - grp * kHeadGroup < kHeadGroup) ? heads_here - grp * kHeadGroup : kHeadGroup;
  const int64_t bh = xcd + kXcd * (grp * kHeadGroup + in_grp % grp_heads);
  const int64_t p = nP - 1 - in_grp / grp_heads;

  // the wave index is wave-uniform: keep it (and everything derived from it) in scalar registers
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, r = l & 15, g = l >> 4;
  const int64_t m = kCpb * p + wave / kWpc;  // this wave's query chunk
  const int q0 = 16 * QT * (wave % kWpc);    // first query (within the chunk) of this wave
  const bool active = m < M;
  const int64_t Lp = M * kC;
  const int64_t mtop = (kCpb * p + kCpb - 1 < M - 1) ? kCpb * p + kCpb - 1 : M - 1;  // highest chunk here
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  f32x4 o[4][QT];    // O^T tiles [d tile][query tile]
  float lsum[QT];    // this lane's share of each column's softmax denominator
  float mref[QT];    // running reference max per query column (log2 units)
  f32x4 negm[QT];    // -mref in all four accumulator slots: the logits' MFMA seed
  bf16x8 qb[QT][2], ql[QT][2];  // running queries as the logits' B-operand (hi [, lo])
#pragma unroll
  for (int a = 0; a < QT; ++a) {
    mref[a] = 0.f;
    lsum[a] = 0.f;
    negm[a] = zero;
#pragma unroll
    for (int b = 0; b < 4; ++b) o[b][a] = zero;
#pragma unroll
    for (int b = 0; b < 2; ++b) qb[a][b] = ql[a][b] = bf16x8{};
  }
  float off = 0.f;  // FoX: sum of the chunk totals from the chunk being scored up to chunk m - 1

  // ---------------------------------------------------------------- step pieces
  // Logits (log2 units, minus the running max) of a key chunk against the running queries, plus the
  // PaTH-FoX bias sum_{s=j+1..i} f_s = (chunk-local prefix at i) + off - (prefix at j), whose
  // row-constant first term cancels in the softmax (it returns in the lse).  kfrag(t, ks) gives the
  // A-fragment of key rows 16t.., lf the chunk-local prefix of the key chunk.
  auto logits = [&](auto kfrag, const float* lf, float offv, f32x4 (&z)[4][QT]) PA_INLINE {
    // FoX: seed = -mref + log2e (off - prefix_j) = fma(-log2e, prefix_j, base), base per query column
    float base[QT];
    if constexpr (FOX) {
#pragma unroll
      for (int qi = 0; qi < QT; ++qi) base[qi] = __builtin_fmaf(kLog2e, offv, negm[qi][0]);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x4 seed[QT];
      if constexpr (FOX) {
        const float4 f4 = *reinterpret_cast<const float4*>(lf + 16 * t + 4 * g);
        const float fb[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
        for (int qi = 0; qi < QT; ++qi)
#pragma unroll
          for (int i = 0; i < 4; ++i) seed[qi][i] = __builtin_fmaf(-kLog2e, fb[i], base[qi]);
      } else {
#pragma unroll
        for (int qi = 0; qi < QT; ++qi) seed[qi] = negm[qi];
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 a = kfrag(t, ks);
#pragma unroll
        for (int qi = 0; qi < QT; ++qi) {
          z[t][qi] = mfma16(a, qb[qi][ks], ks == 0 ? seed[qi] : z[t][qi]);
          if constexpr (X3) z[t][qi] = mfma16(a, ql[qi][ks], z[t][qi]);  // logits see the query residual
        }
      }
    }
  };
  auto lds_keys = [&](const __bf16* Kt_) PA_INLINE {
    return [=](int t, int ks) PA_INLINE { return tile_frag(Kt_, 16 * t + r, 4 * ks + g); };
  };
  // Q_run^T <- P_n Q_run^T (fp32 accumulate).
  auto transport = [&](const __bf16* Pt, const __bf16* Plt, f32x4 (&qn)[4][QT]) PA_INLINE {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int qi = 0; qi < QT; ++qi) qn[dt][qi] = zero;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 a = tile_frag(Pt, 16 * dt + r, 4 * ks + g);
#pragma unroll
        for (int qi = 0; qi < QT; ++qi) qn[dt][qi] = mfma16(a, qb[qi][ks], qn[dt][qi]);
        if constexpr (X3) {
          const bf16x8 alo = tile_frag(Plt, 16 * dt + r, 4 * ks + g);
#pragma unroll
          for (int qi = 0; qi < QT; ++qi) {
            qn[dt][qi] = mfma16(a, ql[qi][ks], qn[dt][qi]);
            qn[dt][qi] = mfma16(alo, qb[qi][ks], qn[dt][qi]);
          }
        }
      }
    }
  };
  // Accumulator tiles -> the logits' B-operand (bf16 hi [+ lo]).
  auto requeue = [&](const f32x4 (&qn)[4][QT]) PA_INLINE {
#pragma unroll
    for (int qi = 0; qi < QT; ++qi)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float vq = qn[2 * ks + (j >> 2)][qi][j & 3];
          const __bf16 hi = (__bf16)vq;
          qb[qi][ks][j] = hi;
          if constexpr (X3) ql[qi][ks][j] = (__bf16)(vq - (float)hi);
        }
  };
  // p = exp2(z - shift): this lane's partial row sums and P^T as the PV B-operand.
  auto exps = [&](const f32x4 (&z)[4][QT], const float (&shift)[QT], bf16x8 (&pb)[QT][2], float (&ps)[QT]) PA_INLINE {
#pragma unroll
    for (int qi = 0; qi < QT; ++qi) {
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = fast_exp2(z[t][qi][i] - shift[qi]);
          s = (t == 0 && i == 0) ? pv : s + pv;
          pb[qi][t >> 1][4 * (t & 1) + i] = (__bf16)pv;
        }
      ps[qi] = s;
    }
  };
  auto pv = [&](const __bf16* Vt, const bf16x8 (&pb)[QT][2]) PA_INLINE {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 a = vt_frag(Vt, dt, ks);
#pragma unroll
        for (int qi = 0; qi < QT; ++qi) o[dt][qi] = mfma16(a, pb[qi][ks], o[dt][qi]);
      }
  };
  // Exact column max of z (relative to the reference); raise every column's reference to its max
  // when some column exceeds it by more than kRescale.  Returns false when nothing moved.
  auto raise_ref = [&](const f32x4 (&z)[4][QT], float (&d)[QT]) PA_INLINE {
    bool up = false;
#pragma unroll
    for (int qi = 0; qi < QT; ++qi) {
      float mx = max3(z[0][qi][0], z[0][qi][1], z[0][qi][2]);
      mx = max3(mx, z[0][qi][3], z[1][qi][0]);
      mx = max3(mx, z[1][qi][1], z[1][qi][2]);
      mx = max3(mx, z[1][qi][3], z[2][qi][0]);
      mx = max3(mx, z[2][qi][1], z[2][qi][2]);
      mx = max3(mx, z[2][qi][3], z[3][qi][0]);
      mx = max3(mx, z[3][qi][1], z[3][qi][2]);
      mx = max2(mx, z[3][qi][3]);
      d[qi] = max2(colmax4(mx), 0.f);
      up |= d[qi] > kRescale;
    }
    if (!__any(up)) return false;
#pragma unroll
    for (int qi = 0; qi < QT; ++qi) {
      const float alpha = fast_exp2(-d[qi]);
      mref[qi] += d[qi];
      negm[qi] = f32x4{-mref[qi], -mref[qi], -mref[qi], -mref[qi]};
      lsum[qi] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt][qi] *= alpha;
    }
    return true;
  };

  // Own chunk: logits from the in-chunk S (already in log2 units), exact max, P^T V_m; then the
  // running queries start at qtilde.  The in-chunk logits, FoX prefix and qtilde rows are fetched
  // into registers at the block's start (own_load), while the first key chunk streams in.
  float4 own_s[4][QT], own_f[4];
  bf16x8 own_q[QT][2], own_ql[QT][2];
  auto own_load = [&]() PA_INLINE {
    // packed S: a group past row a's last (columns beyond the diagonal, masked below) re-reads the last
    const float* Sb = Sm + ((size_t)bh * M + m) * kSGroups * 4;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if constexpr (FOX) own_f[t] = *reinterpret_cast<const float4*>(fl + bh * Lp + m * kC + 16 * t + 4 * g);
#pragma unroll
      for (int qi = 0; qi < QT; ++qi) {
        const int a = q0 + 16 * qi + r, last = a >> 2;
        const int grp = (4 * t + g < last) ? 4 * t + g : last;
        own_s[t][qi] = *reinterpret_cast<const float4*>(Sb + (s_row_group(a) + grp) * 4);
      }
    }
#pragma unroll
    for (int qi = 0; qi < QT; ++qi)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const size_t qo = ((size_t)bh * Lp + m * kC + q0 + 16 * qi + r) * kD + 32 * ks + 8 * g;
        own_q[qi][ks] = *reinterpret_cast<const bf16x8*>(qt + qo);
        if constexpr (X3) own_ql[qi][ks] = *reinterpret_cast<const bf16x8*>(qt_lo + qo);
      }
  };
  auto diag = [&](const __bf16* Vt_) PA_INLINE {
    f32x4 z[4][QT];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float fb[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (FOX) {
        fb[0] = kLog2e * own_f[t].x, fb[1] = kLog2e * own_f[t].y, fb[2] = kLog2e * own_f[t].z,
        fb[3] = kLog2e * own_f[t].w;
      }
#pragma unroll
      for (int qi = 0; qi < QT; ++qi) {
        const int a = q0 + 16 * qi + r;
        const float sv[4] = {own_s[t][qi].x, own_s[t][qi].y, own_s[t][qi].z, own_s[t][qi].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) z[t][qi][i] = (16 * t + 4 * g + i <= a) ? sv[i] - fb[i] : -INFINITY;
      }
    }
    float shift[QT], ps[QT];
#pragma unroll
    for (int qi = 0; qi < QT; ++qi) {
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t) mx = max3(mx, max2(z[t][qi][0], z[t][qi][1]), max2(z[t][qi][2], z[t][qi][3]));
      mref[qi] = colmax4(mx);  // finite: key a itself is never masked
      negm[qi] = f32x4{-mref[qi], -mref[qi], -mref[qi], -mref[qi]};
      shift[qi] = mref[qi];
    }
    bf16x8 pb[QT][2];
    exps(z, shift, pb, ps);
#pragma unroll
    for (int qi = 0; qi < QT; ++qi) lsum[qi] = ps[qi];
    pv(Vt_, pb);
#pragma unroll
    for (int qi = 0; qi < QT; ++qi)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        qb[qi][ks] = own_q[qi][ks];
        if constexpr (X3) ql[qi][ks] = own_ql[qi][ks];
      }
  };

  // Earlier chunk n (< m); NEXT: chunk n - 1 exists (the running queries move on).  Logits of
  // chunk n (seeded with -reference, plus the FoX bias), exponentials with the lazy check, then the
  // transport and O^T += V_n^T P^T on the matrix cores; the requeue of the moved queries comes last
  // so that the transport has drained by then.  The two waves of a SIMD overlap one's vector phase
  // with the other's MFMAs.
  auto step = [&](auto next_tag, const __bf16* Kt_, const __bf16* Vt_, const __bf16* Pt_, const __bf16* Plt_,
                  const float* lf) PA_INLINE {
    constexpr bool NEXT = decltype(next_tag)::value;
    f32x4 z[4][QT];
    logits(lds_keys(Kt_), lf, off, z);
    f32x4 qn[4][QT];
    if constexpr (NEXT) transport(Pt_, Plt_, qn);
    const float none[QT] = {};
    bf16x8 pb[QT][2];
    float ps[QT];
    exps(z, none, pb, ps);
    // Issue order: the logits' MFMAs first, then the transport's MFMAs interleaved with the
    // exponentials, which only wait for the logits.
    if constexpr (!X3 && !FOX && QT == 2) {
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // key fragments
      __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);  // logits
      if constexpr (NEXT) {
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // transition fragments
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
        }
      }
    }
    bool big = false;
#pragma unroll
    for (int qi = 0; qi < QT; ++qi) big |= ps[qi] > kSumCap;
    if (__any(big)) {  // rare: some p may exceed 2^kRescale
      float d[QT];
      if (raise_ref(z, d)) exps(z, d, pb, ps);
    }
#pragma unroll
    for (int qi = 0; qi < QT; ++qi) lsum[qi] += ps[qi];
    pv(Vt_, pb);
    if constexpr (NEXT) requeue(qn);
  };

  // ---------------------------------------------------------------- key-group stream
  // Key chunk n = ktilde_n, V_n, P_n [, P_lo n] and the FoX prefix of chunk n.  Each wave moves a
  // 1/W share of every tile (rows 8i.., i = kCp wave .. kCp wave + kCp - 1; lane l carries 16 B of
  // row 8i + l/8, written to slot l of the tile's i-th 1 KiB run) and of the prefix.
  const int i0 = kCp * wave;
  const int64_t mlow = kCpb * p;  // lowest query chunk of the block
  // With chunks of G > 1 sub-chunks the stream below the block takes whole groups from galign down:
  // each sub-chunk with its keys carried to the group's top and no transport, except the group's
  // bottom sub-chunk, which moves the queries across the whole group (P_group).  Sub-chunks between
  // the block's own chunks and galign (the group boundary at or below them) step one by one.
  static_assert(G == 1 || G == 2 || G == 4, "sub-chunks per chunk");
  const int64_t MG = M / G;
  const int64_t galign = (mlow / G) * G;
  auto chunk_src = [&](int64_t n, int t) PA_INLINE -> const __bf16* {
    const bool grouped = G > 1 && n < galign;
    if (t == 0)
      return (grouped && n % G != G - 1 ? ktc : kt) + ((size_t)bh * Lp + n * kC) * kD;
    if (t == 1) return v + ((size_t)bh * L + n * kC) * kD;
    if (grouped && n % G == 0) return (t == 2 ? pg_hi : pg_lo) + ((size_t)bh * MG + n / G) * kD * kD;
    return (t == 2 ? p_hi : p_lo) + ((size_t)bh * M + n) * kD * kD;
  };
  auto chunk_rows = [&](int64_t n, int t) PA_INLINE -> int {
    const int64_t vrows = L - n * kC;
    return (t == 1 && vrows < kC) ? (int)vrows : kC;
  };
  // full: chunk n is known to be whole (n < M - 1), so no value row needs the clamp
  auto stage = [&](int64_t n, int s, bool full = false) PA_INLINE {
#pragma unroll
    for (int t = 0; t < NM; ++t) dma_tile<kCp>(lds[s][t], chunk_src(n, t), full ? kC : chunk_rows(n, t), i0);
    if constexpr (FOX) {
      if (l < 64 / W)
        __builtin_amdgcn_global_load_lds((const void*)(fl + bh * Lp + n * kC + (64 / W) * wave + l),
                                         (lds_void*)(lfl[s] + (64 / W) * wave), 4, 0, 0);
    }
  };

  int cur = 0;
  // The own-chunk loads go out first, so waiting for the first key chunk covers them too.
  if (active) own_load();
  __asm__ __volatile__("" ::: "memory");  // keep them ahead of the copies in issue order
  stage(mtop, 0);
  if constexpr (NB == 3) {
    if (mtop >= 1) {
      stage(mtop - 1, 1);
      wait_vm<OPS>();
    } else {
      wait_vm<0>();
    }
  } else {
    wait_vm<0>();
  }
  lds_barrier();
  // With a 3-slot ring the copy of chunk n-2 is issued after the step's last LDS read (the compiler
  // waits for outstanding copies before any LDS transpose read, so a copy issued earlier in the step
  // would stall it); with 2 slots the copy of chunk n-1 has to go out first.
  auto prefetch = [&](int64_t n) PA_INLINE {
    if constexpr (NB == 2) {
      if (n >= 1) stage(n - 1, cur ^ 1);
    }
  };
  auto advance = [&](int64_t n) PA_INLINE {
    if constexpr (NB == 3) {
      if (n >= 2) {
        stage(n - 2, cur == 0 ? 2 : cur - 1);
        wait_vm<OPS>();  // chunk n-1 (issued one step earlier) has landed
      } else {
        wait_vm<0>();
      }
    } else {
      wait_vm<0>();
    }
    lds_barrier();
    cur = (cur + 1 == NB) ? 0 : cur + 1;
  };
  auto run_step = [&](auto next_tag, int64_t n) PA_INLINE {
    if constexpr (FOX) off += lfl[cur][63];  // the chunk's total: its last inclusive prefix, already staged
    step(next_tag, lds[cur][0], lds[cur][1], lds[cur][2], lds[cur][NM - 1], lfl[cur]);
  };

  // Head: the block's own query chunks mtop .. mlow.  A wave idles above its chunk, scores its own
  // chunk from the in-chunk logits and steps below it.
  int64_t n = mtop;
#pragma unroll
  for (int it = 0; it < kCpb; ++it, --n) {
    if (n < mlow) break;
    prefetch(n);
    if (active && n == m) {
      diag(lds[cur][1]);
    } else if (active && n < m) {
      if (n > 0)
        run_step(std::true_type{}, n);
      else
        run_step(std::false_type{}, n);
    }
    advance(n);
  }
  // Body: every wave steps (a wave past the end of the sequence works on zero queries and stores
  // nothing), so the loop has a single path.
  if constexpr (G > 1) {
    if constexpr (kCpb % G != 0) {
      for (; n >= galign && n >= 1; --n) {  // down to the group boundary, one sub-chunk at a time
        prefetch(n);
        run_step(std::true_type{}, n);
        advance(n);
      }
    }
    // from here n is the top of a group (n % G == G - 1) or 0
    for (; n >= 2 * G - 1; n -= G) {  // whole groups with more below: transport at the bottom only
#pragma unroll
      for (int j = 0; j < G - 1; ++j) {
        prefetch(n - j);
        run_step(std::false_type{}, n - j);
        advance(n - j);
      }
      prefetch(n - G + 1);
      run_step(std::true_type{}, n - G + 1);
      advance(n - G + 1);
    }
#pragma unroll
    for (int j = 0; j < G - 1; ++j) {  // the lowest group: nothing below it
      if (n >= 1) {
        prefetch(n);
        run_step(std::false_type{}, n);
        advance(n);
        --n;
      }
    }
  } else if constexpr (NB == 3) {
    // Three steps per turn of the ring, so that every step's slot (and with it every LDS address) is
    // a compile-time constant; the chunks staged here (n - 2 <= M - 3) are whole.
    auto body_step = [&](auto slot_c) PA_INLINE {
      constexpr int S = decltype(slot_c)::value;
      if constexpr (FOX) off += lfl[S][63];
      step(std::true_type{}, lds[S][0], lds[S][1], lds[S][2], lds[S][NM - 1], lfl[S]);
      if (n >= 2) {
        stage(n - 2, (S + 2) % 3, true);
        wait_vm<OPS>();  // chunk n-1 (issued one step earlier) has landed
      } else {
        wait_vm<0>();
      }
      lds_barrier();
      --n;
    };
    while (n >= 1) {
      if (cur == 0) {
        body_step(std::integral_constant<int, 0>{});
        cur = 1;
        if (n < 1) break;
      }
      if (cur == 1) {
        body_step(std::integral_constant<int, 1>{});
        cur = 2;
        if (n < 1) break;
      }
      body_step(std::integral_constant<int, 2>{});
      cur = 0;
    }
  } else {
    for (; n >= 1; --n) {
      prefetch(n);
      run_step(std::true_type{}, n);
      advance(n);
    }
  }
  if (n == 0) run_step(std::false_type{}, 0);

  // ---------------------------------------------------------------- epilogue
#pragma unroll
  for (int qi = 0; qi < QT; ++qi) {
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

// =========================================================================== chains of chunk products
// Kernels 3 and 4 carry a running product R of consecutive chunk matrices from right to left,
// R <- P_s R, and emit rows ktilde_s R on the way.  Columns of R evolve independently, so compute
// wave w of a block carries the 64 x 16 column block y = 16w .. 16w+15 in fp32 accumulators (lane
// (r, g): rows 16jt + 4g + e, column 16w + r).  That accumulator is already the B-operand of the next
// product in the stored key order (acc_to_op), and the A-operand of the key product taken transposed
// (key^T = R^T ktilde^T), so R never leaves registers.  R enters the matrix cores as hi + lo bf16, P
// as hi (+ lo with bf16x3 transport).  A fifth wave streams the P and ktilde tiles of the coming steps
// into an NB-slot LDS ring (direct global->LDS copies) and is the only wave that waits for them, so
// its wait counts are exact while the compute waves store their results.
struct ChainFrags {
  bf16x8 ph[4][2], pl[4][2], k[4][2];
};

constexpr int kChainThreads = 320;  // 4 compute waves + the copy wave

__device__ __forceinline__ void chain_identity(f32x4 (&racc)[4]) {
  const int l = threadIdx.x & 63, r = l & 15, g = l >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
#pragma unroll
    for (int e = 0; e < 4; ++e) racc[jt][e] = (16 * jt + 4 * g + e == 16 * wave + r) ? 1.f : 0.f;
}

// key^T[y][b] = sum_m R[m][y] ktilde[b][m] for key tile bt: lane gets key b = 16 bt + r, y = 16w + 4g ..
__device__ __forceinline__ f32x4 chain_keys(const bf16x8 (&rh)[2], const bf16x8 (&rl)[2], const bf16x8 (&k)[2]) {
  f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    a = mfma16(rh[ks], k[ks], a);
    a = mfma16(rl[ks], k[ks], a);
  }
  return a;
}

// R <- P R
template <bool X3>
__device__ __forceinline__ void chain_advance(const ChainFrags& F, const bf16x8 (&rh)[2], const bf16x8 (&rl)[2],
                                              f32x4 (&racc)[4]) {
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      a = mfma16(F.ph[jt][ks], rh[ks], a);
      a = mfma16(F.ph[jt][ks], rl[ks], a);
      if constexpr (X3) a = mfma16(F.pl[jt][ks], rh[ks], a);
    }
    racc[jt] = a;
  }
}

// Run `steps` chain steps.  src(i, t) is the global tile of step i (t = 0: P hi, 1: ktilde, 2: P lo;
// without KEYS no ktilde tile is streamed); emit(i, rh, rl, F) runs on the compute waves before the
// step's R <- P R (skipped for the last step unless advance_last).  All waves of the block call this.
template <bool X3, bool KEYS>
struct ChainTiles {
  static constexpr int value = (KEYS ? 2 : 1) + (X3 ? 1 : 0);
};
template <bool X3, bool KEYS>
using ChainSlot = __bf16[ChainTiles<X3, KEYS>::value][kTile];  // one ring slot: the step's tiles
template <bool X3, int NB, bool KEYS = true, typename Src, typename Emit>
__device__ __forceinline__ void chain_run(ChainSlot<X3, KEYS>* ring, int64_t steps, bool advance_last,
                                          f32x4 (&racc)[4], Src src, Emit emit) {
  constexpr int NT = ChainTiles<X3, KEYS>::value;
  constexpr int D = 8 * NT;  // copy instructions per step (the copy wave moves whole tiles)
  static_assert((NB - 2) * D <= 63, "vmcnt field");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = threadIdx.x & 15, g = (threadIdx.x & 63) >> 4;
  const bool copier = wave == 4;
  auto stage = [&](int64_t i) PA_INLINE {
#pragma unroll
    for (int t = 0; t < NT; ++t) dma_tile<8>(ring[i % NB][t], src(i, (KEYS || t == 0) ? t : 2), kC, 0);
  };
  if (copier) {
    for (int64_t i = 0; i < NB - 1 && i < steps; ++i) stage(i);
    wait_vm<0>();
  }
  lds_barrier();
  for (int64_t i = 0; i < steps; ++i) {
    if (copier) {
      if (i + NB - 1 < steps) {
        stage(i + NB - 1);
        wait_vm<(NB - 2) * D>();  // step i + 1 has landed
      } else {
        wait_vm<0>();
      }
    } else {
      ChainFrags F;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          F.ph[t][ks] = tile_frag(ring[i % NB][0], 16 * t + r, 4 * ks + g);
          if constexpr (KEYS) F.k[t][ks] = tile_frag(ring[i % NB][1], 16 * t + r, 4 * ks + g);
          if constexpr (X3) F.pl[t][ks] = tile_frag(ring[i % NB][NT - 1], 16 * t + r, 4 * ks + g);
        }
      bf16x8 rh[2], rl[2];
      acc_to_op(racc, rh, rl);
      emit(i, rh, rl, F);
      if (i + 1 < steps || advance_last) chain_advance<X3>(F, rh, rl, racc);
    }
    lds_barrier();
  }
}

// =========================================================================== kernel 3: grouped chunks
// Chunks of 64 G tokens (G = 2, 4) are built from G 64-token sub-chunks (kernel 1); this kernel adds,
// per group g of sub-chunks s0 = gG .. s0+G-1, what the scan needs below a query's own chunks:
//   carried keys  ktilde_s (P_{s+1} ... P_{s0+G-1})   for s < s0+G-1  (keys moved to the group's top)
//   P_group       P_{s0} ... P_{s0+G-1}                (the group's transition product)
// so that the scan moves its queries once per group.  One block of 4 waves per (group, b, h): every
// tile of the group arrives in LDS at once, then the chain above runs top first without further
// barriers; the last product is taken transposed (P_group^T = R^T P_{s0}^T, the key product's shape)
// so that each lane stores four consecutive columns.  Only whole groups are materialised.
template <bool X3, int G>
__global__ __launch_bounds__(256) void mfma_group_kernel(const __bf16* __restrict__ kt,
                                                         const __bf16* __restrict__ p_hi,
                                                         const __bf16* __restrict__ p_lo, int64_t M,
                                                         __bf16* __restrict__ ktc, __bf16* __restrict__ pg_hi,
                                                         __bf16* __restrict__ pg_lo) {
  __shared__ __align__(1024) __bf16 tp[G][kTile], tpl[X3 ? G : 1][kTile], tk[G - 1][kTile];
  const int64_t grp = blockIdx.x, bh = blockIdx.y, Lp = M * kC, MG = M / G, s0 = grp * G;
  const int l = threadIdx.x & 63, r = l & 15, g = l >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int j = 0; j < G; ++j) {
    dma_tile<2>(tp[j], p_hi + ((size_t)bh * M + s0 + j) * kD * kD, kC, 2 * wave);
    if constexpr (X3) dma_tile<2>(tpl[j], p_lo + ((size_t)bh * M + s0 + j) * kD * kD, kC, 2 * wave);
    if (j < G - 1) dma_tile<2>(tk[j], kt + ((size_t)bh * Lp + (s0 + j) * kC) * kD, kC, 2 * wave);
  }
  wait_vm<0>();
  __syncthreads();
  f32x4 racc[4];
  chain_identity(racc);
#pragma unroll
  for (int j = G - 1; j >= 0; --j) {
    bf16x8 rh[2], rl[2];
    acc_to_op(racc, rh, rl);
    if (j < G - 1) {  // keys of sub-chunk s0 + j carried to the group's top
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        const bf16x8 k[2] = {tile_frag(tk[j], 16 * bt + r, g), tile_frag(tk[j], 16 * bt + r, 4 + g)};
        const f32x4 a = chain_keys(rh, rl, k);
        *reinterpret_cast<bf16x4*>(ktc + ((size_t)bh * Lp + (s0 + j) * kC + 16 * bt + r) * kD +
                                   perm_pos(16 * wave + 4 * g)) = pack4(a[0], a[1], a[2], a[3]);
      }
    }
    if (j > 0) {  // R <- P_j R
      ChainFrags F;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          F.ph[t][ks] = tile_frag(tp[j], 16 * t + r, 4 * ks + g);
          if constexpr (X3) F.pl[t][ks] = tile_frag(tpl[j], 16 * t + r, 4 * ks + g);
        }
      chain_advance<X3>(F, rh, rl, racc);
    } else {  // P_group^T[y][x] = sum_m R[m][y] P_{s0}[x][m]: lane gets row x = 16xt + r, y = 16 wave + 4g ..
#pragma unroll
      for (int xt = 0; xt < 4; ++xt) {
        const bf16x8 ph[2] = {tile_frag(tp[0], 16 * xt + r, g), tile_frag(tp[0], 16 * xt + r, 4 + g)};
        f32x4 a = chain_keys(rh, rl, ph);
        if constexpr (X3) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) a = mfma16(rh[ks], tile_frag(tpl[0], 16 * xt + r, 4 * ks + g), a);
        }
        bf16x4 h4, l4;
        split4(a[0], a[1], a[2], a[3], h4, l4);
        const size_t o = ((size_t)bh * MG + grp) * kD * kD + (size_t)(16 * xt + r) * kD + perm_pos(16 * wave + 4 * g);
        *reinterpret_cast<bf16x4*>(pg_hi + o) = h4;
        if constexpr (X3) *reinterpret_cast<bf16x4*>(pg_lo + o) = l4;
      }
    }
  }
}

// =========================================================================== kernel 4: decode cache
// Prefill -> decode hand-off (PaTH summary, section 3, inference: a decode cache slot j holds
// the key after every later transition, H_{L-1} ... H_{j+1} k_j).  In chunk terms, with R_n the
// product of the chunk matrices after chunk n,
//   R_{M-1} = I,   R_{n-1} = P_n R_n,   cache rows of chunk n = ktilde_n R_n   (row form),
// the chain above over all 64-token (sub-)chunks, reusing the prep's ktilde and P.  With few (b, h)
// pairs one chain per pair would leave most of the chip idle (a 32768-token prompt is a 512-step chain
// on 24 blocks), so each pair's chain is cut into segments s of chunks lo_s .. hi_s:
//   Q_s = P_{lo_s} ... P_{hi_s}                          (kernel 4a, segments s >= 1, in parallel)
//   S_s = Q_{s+1} ... Q_{last} = Q_{s+1} S_{s+1}        (kernel 4b, one short chain per pair)
//   R_{hi_s} = S_s, then the chain above down to lo_s   (kernel 4c, every segment in parallel)
// Q_s is kept as hi + lo bf16 in the P tile layout (rows natural, columns permuted) and S_s in fp32.
int64_t mfma_handoff_segment_chunks(int64_t BH, int64_t M) {
  if (BH >= 128 || BH <= 0 || M < 8) return M > 0 ? M : 1;  // one segment (about a block per CU or more)
  const int64_t want = (512 + BH - 1) / BH, most = M / 4;  // about 512 blocks, segments of >= 4 chunks
  const int64_t nseg = want < most ? want : most;
  return (M + nseg - 1) / nseg;
}
constexpr size_t kSegBytes = 2 * kTile * 2 + kD * kD * 4;  // Q_s hi, lo (bf16) and S_s (fp32) per segment

// Kernel 4a: one block (4 compute waves + the copy wave) per (segment s >= 1, b, h).  The chain runs
// from hi_s down to lo_s + 1 (R = P_{lo_s + 1} ... P_{hi_s}); the last product, with P_{lo_s}, is taken
// transposed (Q_s^T = R^T P_{lo_s}^T, the key product's shape) so that each lane stores four
// consecutive columns of Q_s.
template <bool X3>
__global__ __launch_bounds__(kChainThreads, 1) void mfma_handoff_prod_kernel(const __bf16* __restrict__ p_hi,
                                                                             const __bf16* __restrict__ p_lo,
                                                                             int64_t M, int64_t Gs, int64_t nseg,
                                                                             char* __restrict__ seg) {
  constexpr int NB = 4;
  __shared__ __align__(1024) __bf16 ring[NB][ChainTiles<X3, false>::value][kTile];
  const int64_t sg = blockIdx.x + 1, bh = blockIdx.y;
  const int64_t lo = sg * Gs, hi = (lo + Gs < M ? lo + Gs : M) - 1;
  const int l = threadIdx.x & 63, r = l & 15, g = l >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  f32x4 racc[4];
  if (wave < 4) chain_identity(racc);
  char* base = seg + ((size_t)bh * nseg + sg) * kSegBytes;
  __bf16* qh = reinterpret_cast<__bf16*>(base);
  __bf16* ql = qh + kTile;
  auto src = [&](int64_t i, int t) -> const __bf16* {
    return (t == 0 ? p_hi : p_lo) + ((size_t)bh * M + (hi - i)) * kD * kD;
  };
  const int64_t steps = hi - lo + 1;
  auto emit = [&](int64_t i, const bf16x8 (&rh)[2], const bf16x8 (&rl)[2], const ChainFrags& F) PA_INLINE {
    if (i != steps - 1) return;
    // Q_s^T[y][x] = sum_m R[m][y] P_lo[x][m]: lane gets row x = 16 xt + r, columns y = 16 wave + 4g ..
#pragma unroll
    for (int xt = 0; xt < 4; ++xt) {
      f32x4 a = chain_keys(rh, rl, F.ph[xt]);
      if constexpr (X3) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) a = mfma16(rh[ks], F.pl[xt][ks], a);
      }
      bf16x4 h4, l4;
      split4(a[0], a[1], a[2], a[3], h4, l4);
      const size_t o = (size_t)(16 * xt + r) * kD + perm_pos(16 * wave + 4 * g);
      *reinterpret_cast<bf16x4*>(qh + o) = h4;
      *reinterpret_cast<bf16x4*>(ql + o) = l4;
    }
  };
  chain_run<X3, NB, false>(ring, steps, false, racc, src, emit);
}

// Kernel 4b: one block of 4 waves per (b, h): S_{last} = I, S_s = Q_{s+1} S_{s+1} down to s = 0, each
// wave carrying a 64 x 16 column block of S in fp32 accumulators (the chain step with Q_{s+1} as a hi + lo
// "P"), stored in fp32 with natural columns.
__global__ __launch_bounds__(256) void mfma_handoff_suffix_kernel(int64_t nseg, char* __restrict__ seg) {
  const int64_t bh = blockIdx.x;
  const int l = threadIdx.x & 63, r = l & 15, g = l >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  f32x4 racc[4];
  chain_identity(racc);
  for (int64_t sg = nseg - 2; sg >= 0; --sg) {
    const char* qb = seg + ((size_t)bh * nseg + sg + 1) * kSegBytes;
    const __bf16* qh = reinterpret_cast<const __bf16*>(qb);
    const __bf16* ql = qh + kTile;
    ChainFrags F;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const size_t o = (size_t)(16 * t + r) * kD + 8 * (4 * ks + g);
        F.ph[t][ks] = *reinterpret_cast<const bf16x8*>(qh + o);
        F.pl[t][ks] = *reinterpret_cast<const bf16x8*>(ql + o);
      }
    bf16x8 rh[2], rl[2];
    acc_to_op(racc, rh, rl);
    chain_advance<true>(F, rh, rl, racc);
    float* so = reinterpret_cast<float*>(seg + ((size_t)bh * nseg + sg) * kSegBytes + 2 * kTile * 2);
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int e = 0; e < 4; ++e) so[(16 * jt + 4 * g + e) * kD + 16 * wave + r] = racc[jt][e];
  }
}

// Kernel 4c: one block (4 compute waves + the copy wave) per (b, h, segment), 1-D grid; the chain
// starts from S_s (the identity for the last segment) at hi_s and emits the segment's key slots; each
// compute wave also copies its quarter of the chunk's value rows.
template <bool X3>
__global__ __launch_bounds__(kChainThreads, 1) void mfma_cache_kernel(const __bf16* __restrict__ kt,
                                                                      const __bf16* __restrict__ p_hi,
                                                                      const __bf16* __restrict__ p_lo,
                                                                      const __bf16* __restrict__ v, int64_t L,
                                                                      int64_t M, int64_t cap, int64_t Gs,
                                                                      int64_t nseg, const char* __restrict__ seg,
                                                                      __bf16* __restrict__ kc,
                                                                      __bf16* __restrict__ vc) {
  constexpr int NB = 4;
  __shared__ __align__(1024) __bf16 ring[NB][ChainTiles<X3, true>::value][kTile];
  __shared__ __align__(1024) __bf16 kst[2][kTile];  // finished key rows of the last two chunks (swizzled)
  const int64_t bh = blockIdx.x / nseg, sg = blockIdx.x % nseg, Lp = M * kC;
  const int64_t lo = sg * Gs, hi = (lo + Gs < M ? lo + Gs : M) - 1;
  const int l = threadIdx.x & 63, r = l & 15, g = l >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  f32x4 racc[4];
  if (wave < 4) {
    if (sg == nseg - 1) {
      chain_identity(racc);
    } else {  // S_s, fp32 with natural columns: lane (r, g) holds rows 16 jt + 4g + e of column 16 wave + r
      const float* si = reinterpret_cast<const float*>(seg + ((size_t)bh * nseg + sg) * kSegBytes + 2 * kTile * 2);
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int e = 0; e < 4; ++e) racc[jt][e] = si[(16 * jt + 4 * g + e) * kD + 16 * wave + r];
    }
  }
  auto src = [&](int64_t i, int t) -> const __bf16* {
    const int64_t n = hi - i;
    if (t == 1) return kt + ((size_t)bh * Lp + n * kC) * kD;
    return (t == 0 ? p_hi : p_lo) + ((size_t)bh * M + n) * kD * kD;
  };
  // values of chunk n: rows 16 wave .. 16 wave + 15, 32 B per lane, loaded one chunk ahead
  uint4 va = {}, vb = {};
  auto vload = [&](int64_t n) PA_INLINE {
    const int64_t j = n * kC + 16 * wave + (l >> 2);
    if (n >= lo && j < L) {
      const uint4* s = reinterpret_cast<const uint4*>(v + ((size_t)bh * L + j) * kD + 16 * (l & 3));
      va = s[0];
      vb = s[1];
    }
  };
  if (wave < 4) vload(hi);
  // key rows 16 wave .. 16 wave + 15 of chunk n from a staging tile: 8 lanes per 128-byte row
  auto flush = [&](int64_t n, const __bf16* tile) PA_INLINE {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 16 * wave + 8 * h + (l >> 3), c = l & 7;
      const int64_t j = n * kC + row;
      if (j < L)
        *reinterpret_cast<bf16x8*>(kc + ((size_t)bh * cap + j) * kD + 8 * c) = tile_frag(tile, row, c);
    }
  };
  auto emit = [&](int64_t i, const bf16x8 (&rh)[2], const bf16x8 (&rl)[2], const ChainFrags& F) PA_INLINE {
    const int64_t n = hi - i;
    {
      const int64_t j = n * kC + 16 * wave + (l >> 2);
      if (j < L) {
        uint4* d = reinterpret_cast<uint4*>(vc + ((size_t)bh * cap + j) * kD + 16 * (l & 3));
        d[0] = va;
        d[1] = vb;
      }
      vload(n - 1);
    }
    // keys: this wave's 16 columns go to the staging tile; the previous chunk's tile, complete since
    // the last barrier, is stored as whole 128-byte rows
    if (i > 0) flush(n + 1, kst[(i - 1) & 1]);
#pragma unroll
    for (int bt = 0; bt < 4; ++bt) {
      const f32x4 a = chain_keys(rh, rl, F.k[bt]);
      const int row = 16 * bt + r, c0 = 16 * wave + 4 * g;
      *reinterpret_cast<bf16x4*>(kst[i & 1] + swz(row, c0 >> 3) + (c0 & 7)) = pack4(a[0], a[1], a[2], a[3]);
    }
  };
  const int64_t steps = hi - lo + 1;
  chain_run<X3, NB>(ring, steps, false, racc, src, emit);
  if (wave < 4) flush(lo, kst[(steps - 1) & 1]);
}

// =========================================================================== host
bool mfma_supported(int d, int chunk) { return d == kD && (chunk == kC || chunk == 2 * kC || chunk == 4 * kC); }

template <bool FOX, bool X3, int G>
static void launch_attn(dim3 grid, hipStream_t st, const __bf16* qt, const __bf16* qt_lo, const __bf16* kt,
                        const __bf16* v, const __bf16* p_hi, const __bf16* p_lo, const __bf16* ktc,
                        const __bf16* pg_hi, const __bf16* pg_lo, const float* Sm, const float* fl,
                        const float* ftot, __bf16* out, float* lse, int64_t L, int64_t M, int64_t BH) {
  mfma_attn_kernel<FOX, X3, G, PATHATTN_SCAN_QT, PATHATTN_SCAN_BLOCK_WAVES>
      <<<grid, 64 * PATHATTN_SCAN_BLOCK_WAVES, 0, st>>>(qt, qt_lo, kt, v, p_hi, p_lo, ktc, pg_hi, pg_lo, Sm, fl, ftot,
                                                        out, lse, L, M, BH);
}

template <int G>
static void launch_attn_g(bool fox, bool x3, dim3 grid, hipStream_t st, const __bf16* qt, const __bf16* qt_lo,
                          const __bf16* kt, const __bf16* v, const __bf16* p_hi, const __bf16* p_lo,
                          const __bf16* ktc, const __bf16* pg_hi, const __bf16* pg_lo, const float* Sm,
                          const float* fl, const float* ftot, __bf16* out, float* lse, int64_t L, int64_t M,
                          int64_t BH) {
  auto go = [&](auto fn) { fn(grid, st, qt, qt_lo, kt, v, p_hi, p_lo, ktc, pg_hi, pg_lo, Sm, fl, ftot, out, lse, L, M, BH); };
  if (fox && x3) go(launch_attn<true, true, G>);
  else if (fox) go(launch_attn<true, false, G>);
  else if (x3) go(launch_attn<false, true, G>);
  else go(launch_attn<false, false, G>);
}

// phases: bit 0 = per-chunk prep, bit 1 = attention scan (reads what the prep left in the workspace).
// The prep stores qtilde and the in-chunk logits multiplied by scale * log2(e).  Chunks of 128 or 256
// tokens run the prep on 64-token sub-chunks and group them (kernel 3) before the scan.
hipError_t mfma_run(int phases, int chunk, int transport, const void* q, const void* k, const void* v,
                    const void* w, const float* beta, const float* logf, void* out, float* lse, int64_t BH,
                    int64_t L, float scale, void* qt, void* qt_lo, void* kt, void* p_hi, void* p_lo, void* ktc,
                    void* pg_hi, void* pg_lo, float* Sm, float* fl, float* ftot, hipStream_t st) {
  if (!mfma_supported(kD, chunk)) return hipErrorInvalidValue;
  const int G = chunk / kC;
  const int64_t M = (L + kC - 1) / kC;  // 64-token (sub-)chunks
  const int64_t MG = M / G;             // whole groups
  const bool x3 = transport == 1;
  hipError_t e = hipSuccess;
  if (phases & 1) {
    auto prep = [&](auto kernel) {
      hipError_t err = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)kPrepLds);
      if (err != hipSuccess) return err;
      kernel<<<dim3((unsigned)M, (unsigned)BH), 256, kPrepLds, st>>>(
          (const __bf16*)q, (const __bf16*)k, (const __bf16*)w, beta, logf, L, M, scale * kLog2e, (__bf16*)qt,
          x3 ? (__bf16*)qt_lo : nullptr, (__bf16*)kt, (__bf16*)p_hi, x3 ? (__bf16*)p_lo : nullptr, Sm, fl, ftot,
          nullptr);
      return hipGetLastError();
    };
    e = x3 ? prep(mfma_prep_kernel<true>) : prep(mfma_prep_kernel<false>);
    if (e != hipSuccess) return e;
    if (G > 1 && MG > 0) {
      const dim3 gg((unsigned)MG, (unsigned)BH);
      const auto* a_kt = (const __bf16*)kt;
      const auto* a_ph = (const __bf16*)p_hi;
      const auto* a_pl = x3 ? (const __bf16*)p_lo : nullptr;
      auto* a_kc = (__bf16*)ktc;
      auto* a_gh = (__bf16*)pg_hi;
      auto* a_gl = x3 ? (__bf16*)pg_lo : nullptr;
      if (G == 4 && x3)
        mfma_group_kernel<true, 4><<<gg, 256, 0, st>>>(a_kt, a_ph, a_pl, M, a_kc, a_gh, a_gl);
      else if (G == 4)
        mfma_group_kernel<false, 4><<<gg, 256, 0, st>>>(a_kt, a_ph, a_pl, M, a_kc, a_gh, a_gl);
      else if (x3)
        mfma_group_kernel<true, 2><<<gg, 256, 0, st>>>(a_kt, a_ph, a_pl, M, a_kc, a_gh, a_gl);
      else
        mfma_group_kernel<false, 2><<<gg, 256, 0, st>>>(a_kt, a_ph, a_pl, M, a_kc, a_gh, a_gl);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (phases & 2) {
    constexpr int kCpb = ScanShape<false, PATHATTN_SCAN_QT, PATHATTN_SCAN_BLOCK_WAVES>::kCpb;
    static_assert(kCpb % 2 == 0, "blocks must cover whole 128-token chunks");
    const int64_t heads_per_xcd = (BH + kXcd - 1) / kXcd;
    const dim3 grid((unsigned)(kXcd * heads_per_xcd * ((M + kCpb - 1) / kCpb)));
    const bool fox = logf != nullptr;
    const auto* a_qt = (const __bf16*)qt;
    const auto* a_qtl = (const __bf16*)qt_lo;
    const auto* a_kt = (const __bf16*)kt;
    const auto* a_v = (const __bf16*)v;
    const auto* a_ph = (const __bf16*)p_hi;
    const auto* a_pl = (const __bf16*)p_lo;
    const auto* a_kc = (const __bf16*)ktc;
    const auto* a_gh = (const __bf16*)pg_hi;
    const auto* a_gl = (const __bf16*)pg_lo;
    if (G == 4)
      launch_attn_g<4>(fox, x3, grid, st, a_qt, a_qtl, a_kt, a_v, a_ph, a_pl, a_kc, a_gh, a_gl, Sm, fl, ftot,
                       (__bf16*)out, lse, L, M, BH);
    else if (G == 2)
      launch_attn_g<2>(fox, x3, grid, st, a_qt, a_qtl, a_kt, a_v, a_ph, a_pl, a_kc, a_gh, a_gl, Sm, fl, ftot,
                       (__bf16*)out, lse, L, M, BH);
    else
      launch_attn_g<1>(fox, x3, grid, st, a_qt, a_qtl, a_kt, a_v, a_ph, a_pl, a_kc, a_gh, a_gl, Sm, fl, ftot,
                       (__bf16*)out, lse, L, M, BH);
    e = hipGetLastError();
  }
  return e;
}

// Bytes of one 64-token chunk's packed in-chunk logits (bf16 forms).
size_t mfma_s_chunk_bytes() { return (size_t)kSGroups * 4 * sizeof(float); }

// Scratch the hand-off needs in the prefill workspace (segment products), bytes.
size_t mfma_handoff_scratch_bytes(int64_t BH, int64_t M) {
  if (BH <= 0 || M <= 0) return 0;
  const int64_t Gs = mfma_handoff_segment_chunks(BH, M);
  const int64_t nseg = (M + Gs - 1) / Gs;
  return nseg > 1 ? (size_t)(BH * nseg) * kSegBytes : 0;
}

// The prefill's per-chunk terms (bf16 transport form) for the backward pass of bf16 inputs, plus
// Z = A^{-1} per chunk for its gradient kernel.
hipError_t mfma_prep_bwd_run(const void* q, const void* k, const void* w, const float* beta, const float* logf,
                             int64_t BH, int64_t L, float qs, void* qt, void* kt, void* Pm, float* Sm, float* fl,
                             float* ftot, float* Zi, hipStream_t st) {
  const int64_t M = (L + kC - 1) / kC;
  hipError_t e = hipFuncSetAttribute((const void*)mfma_prep_kernel<false>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kPrepLds);
  if (e != hipSuccess) return e;
  mfma_prep_kernel<false><<<dim3((unsigned)M, (unsigned)BH), 256, kPrepLds, st>>>(
      (const __bf16*)q, (const __bf16*)k, (const __bf16*)w, beta, logf, L, M, qs, reinterpret_cast<__bf16*>(qt),
      nullptr, reinterpret_cast<__bf16*>(kt), reinterpret_cast<__bf16*>(Pm), nullptr, Sm, fl, ftot, Zi);
  return hipGetLastError();
}

// Decode cache from a prefill workspace (kernel 4): segment products and their suffix products when
// the chain is cut, then one block (4 compute waves + the copy wave) per (b, h, segment).
hipError_t mfma_cache_run(int transport, const void* kt, const void* p_hi, const void* p_lo, const void* v,
                          int64_t BH, int64_t L, int64_t cap, void* scratch, void* kc, void* vc, hipStream_t st) {
  const int64_t M = (L + kC - 1) / kC;
  const int64_t Gs = mfma_handoff_segment_chunks(BH, M), nseg = (M + Gs - 1) / Gs;
  char* seg = static_cast<char*>(scratch);
  if (nseg > 1 && seg == nullptr) return hipErrorInvalidValue;
  const bool x3 = transport == 1;
  const auto* ph = (const __bf16*)p_hi;
  const auto* pl = x3 ? (const __bf16*)p_lo : nullptr;
  if (nseg > 1) {
    if (x3)
      mfma_handoff_prod_kernel<true><<<dim3((unsigned)(nseg - 1), (unsigned)BH), kChainThreads, 0, st>>>(ph, pl, M, Gs,
                                                                                                      nseg, seg);
    else
      mfma_handoff_prod_kernel<false><<<dim3((unsigned)(nseg - 1), (unsigned)BH), kChainThreads, 0, st>>>(ph, pl, M,
                                                                                                       Gs, nseg, seg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    mfma_handoff_suffix_kernel<<<dim3((unsigned)BH), 256, 0, st>>>(nseg, seg);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const dim3 grid((unsigned)(BH * nseg));
  if (x3)
    mfma_cache_kernel<true><<<grid, kChainThreads, 0, st>>>((const __bf16*)kt, ph, pl, (const __bf16*)v, L, M, cap,
                                                            Gs, nseg, seg, (__bf16*)kc, (__bf16*)vc);
  else
    mfma_cache_kernel<false><<<grid, kChainThreads, 0, st>>>((const __bf16*)kt, ph, nullptr, (const __bf16*)v, L, M,
                                                             cap, Gs, nseg, seg, (__bf16*)kc, (__bf16*)vc);
  return hipGetLastError();
}

}  // namespace pathattn

// PaTH / PaTH-FoX backward, chunk-pair kernels for bf16 inputs at d = chunk = 64, in the operand
// conventions of the matrix-core prefill (tiles.h).  The recurrences are those of backward.hip
// (PaTH summary, gist.science/ko/paper/2505.16381, section 3, differentiated):
//   forward per query chunk m:  r^(m-1) = qtilde_m,  z_mn = r^(n) ktilde_n^T,  r^(n-1) = r^(n) P_n^T
//   backward:                   dr^(n) = g_mn ktilde_n + dr^(n-1) P_n   (n = 0 .. m-1, g = ln2 dz)
//                               dP_n = sum_m dr^(n-1)_m^T r^(n)_m,  dktilde_n = sum_m g_mn^T r^(n)_m,
//                               dv_n = sum_m p_mn^T dO_m
// The forward's own per-chunk terms are used (qtilde, ktilde and P in bf16 with permuted columns, the
// packed in-chunk logits), and the running states are rounded to bf16 after every transition exactly
// as the forward's bf16 transport rounds its running queries, so the recomputed logits are the
// forward's.  Chains are held transposed (d x queries, as accumulator tiles), so an accumulator turns
// into an MFMA operand in registers (acc_to_op); a state's operand form is also a row of a tile with
// permuted columns, so the pair states r^(n) and dr^(n-1) are stored as such tiles with one 16-byte
// store per lane and k-step, and the key-side kernel reads them back as row fragments (tile_frag) and
// as column fragments (LDS transpose reads, tr_frag).  The streamed tiles (ktilde, V and P on the query
// side, the pair states and dO on the key side) pass through rings of LDS slots (two on the query side,
// three on the key side) filled by direct global->LDS copies, as in the prefill's scan.
#include <type_traits>

#include "backward.h"
#include "tiles.h"

namespace pathattn {

namespace {

constexpr int kRingSlots = 3;  // ring slots of the key-side kernel
constexpr int kPairTiles = 3;  // tiles per ring slot

// Copies of one ring slot per wave: three tiles (2 instructions each) and `extra` 4-byte row loads.
template <int EXTRA>
constexpr int slot_ops() { return kPairTiles * 2 + EXTRA; }

// 16 lanes of every wave copy 16 floats of a 64-float row into LDS (lane l < 16 of wave w writes
// dst[16 w + l]).
__device__ __forceinline__ void row_to_lds(float* dst, const float* src, int wave, int l) {
  if (l < 16)
    __builtin_amdgcn_global_load_lds((const void*)(src + 16 * wave + l), (lds_void*)(dst + 16 * wave), 4, 0, 0);
}

// One slot of the chunk-pair kernels' LDS rings: three tiles and up to two 64-float rows, each an LDS
// variable of its own.  The ring loops are unrolled over the slots, so each LDS access names its
// variable at compile time, and an address is at most a few steps from it: the compiler then keeps the
// variable's alias scope on the access, sees that a read of one slot cannot touch the copies still in
// flight into the others, and does not drain them before it.  (A read whose scope is lost waits for
// every copy in flight.)
struct PairSlot {
  __bf16* t[kPairTiles];
  float* rows[2];
};
template <int S>
using slot_c = std::integral_constant<int, S>;

}  // namespace

// The query-side kernel's two ring slots take 49 KB of LDS, so three blocks share a CU when their registers
// fit (launch bound): 760 against 795 us per band with two blocks and three slots.
#ifndef PATHATTN_QUERY_BLOCKS_PER_CU
#define PATHATTN_QUERY_BLOCKS_PER_CU 3
#endif
constexpr int kQueryBlocksPerCu = PATHATTN_QUERY_BLOCKS_PER_CU;

// Query-chunk kernel: one block of 4 waves per (query chunk m of the band, batch*head); wave w owns the
// queries a = 16w .. 16w+15 of the chunk (lane (r, g) query 16w + r).  Writes the states r^(n) and the
// incoming gradients dr^(n-1) of every pair (m, n < m) (bf16 tiles [query][d], columns permuted), the
// FoX offsets of each pair, the row statistics (lse2, D), the in-chunk logit gradient dS (unscaled
// units, fp32 square), d qtilde (unscaled, fp32) and the row sums of dz.
template <bool FOX>
__global__ __launch_bounds__(256, kQueryBlocksPerCu) void bwd_query_tile_kernel(
    const __bf16* __restrict__ qt, const __bf16* __restrict__ kt, const __bf16* __restrict__ Pm,
    const float* __restrict__ Sm, const float* __restrict__ fl, const float* __restrict__ ftot,
    const __bf16* __restrict__ v, const __bf16* __restrict__ out, const __bf16* __restrict__ dout,
    const float* __restrict__ lse, int64_t L, int64_t M, float scale, pair_band band, __bf16* __restrict__ St,
    __bf16* __restrict__ Gst, float* __restrict__ Off, float* __restrict__ lse2w, float* __restrict__ Dw,
    float* __restrict__ drow, float* __restrict__ dqt, float* __restrict__ dSm, int64_t BH) {
  // two ring slots of ktilde_n, V_n, P_n tiles and the FoX chunk-local prefix of chunk n, every tile and
  // row an LDS variable of its own (as in PairSlot; the loops below name their slots at compile time)
  __shared__ __align__(1024) __bf16 qk0[kTile], qv0[kTile], qp0[kTile], qk1[kTile], qv1[kTile], qp1[kTile];
  __shared__ __align__(16) float qf0[64], qf1[64];
  auto qslot = [&](auto S) PA_INLINE -> PairSlot {
    if constexpr (decltype(S)::value == 0) return PairSlot{{qk0, qv0, qp0}, {qf0, nullptr}};
    else return PairSlot{{qk1, qv1, qp1}, {qf1, nullptr}};
  };

  int64_t bh, q;
  if (!bwd_pair_block(BH, band.me - band.mb, bh, q)) return;  // whole block
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, r = l & 15, g = l >> 4;
  const int64_t m = band.me - 1 - q;  // longest of the band first
  const int64_t Lp = M * 64;
  const size_t row0 = (size_t)bh * Lp + (size_t)m * 64;
  const int a = 16 * wave + r;   // this lane's query within chunk m
  const int64_t ia = m * 64 + a;
  const bool qvalid = ia < L;
  const int i0 = 2 * wave;       // this wave's share of every tile copy (rows 16 wave .. +15)
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  // dO_a (natural columns) as the B-operand of V dO^T; D_a = dO_a . o_a; the row statistics
  bf16x8 dob[2];
  float Da, l2a;
  {
    const size_t ro = ((size_t)bh * L + (size_t)(qvalid ? ia : L - 1)) * 64;
    float ds = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(dout + ro + 32 * ks + 8 * g);
      const bf16x8 o = *reinterpret_cast<const bf16x8*>(out + ro + 32 * ks + 8 * g);
      dob[ks] = qvalid ? x : bf16x8{};
#pragma unroll
      for (int j = 0; j < 8; ++j) ds = __builtin_fmaf((float)dob[ks][j], (float)o[j], ds);
    }
    Da = colsum4(ds);  // over the four lanes of query a
    const float Fa = FOX ? fl[row0 + a] : 0.f;
    const float lv = lse[bh * L + (qvalid ? ia : L - 1)];
    l2a = qvalid ? kLog2e * (lv - Fa) : INFINITY;  // padded query: p = 0
    if (g == 0) {
      lse2w[row0 + a] = l2a;
      Dw[row0 + a] = Da;
    }
  }

  // ---------------------------------------------------------------- pass 1: the states r^(n)
  // r^(n) of this wave's queries as the operand rb (query a, d in the permuted key order), stored per
  // pair and moved across P_n (n >= 1), rounded to bf16 after every transition.  P_{m-1} .. P_1 stream
  // through the LDS ring (one copy per block; P_{n-2} is issued after the transport of step n).  A
  // step's stores go out after its copy wait, so that the next step's wait covers them.
  bf16x8 rb[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) rb[ks] = *reinterpret_cast<const bf16x8*>(qt + (row0 + a) * 64 + 32 * ks + 8 * g);
  {
    auto stage_p = [&](int64_t n, const PairSlot& sl) PA_INLINE {
      dma_tile<2>(sl.t[2], Pm + ((size_t)bh * M + (size_t)n) * 4096, 64, i0);
    };
    if (m >= 2) {
      stage_p(m - 1, qslot(slot_c<0>{}));
      wait_vm<0>();
      lds_barrier();
    }
    float off = 0.f;
    // step i of the pass (n = m - 1 - i) reads slot i & 1 and first sends P_{n-1} into the other slot
    // (last read in step i - 1, which every wave has left)
    auto p1step = [&](auto S, int64_t n) PA_INLINE {
      constexpr int sc = decltype(S)::value;
      const size_t pr = band.slot(bh, m, n);
      if constexpr (FOX) off += ftot[bh * M + n];
      bf16x8 rn[2] = {rb[0], rb[1]};
      if (n > 0) {
        if (n - 1 >= 1) stage_p(n - 1, qslot(slot_c<sc ^ 1>{}));
        const __bf16* Pt = qslot(S).t[2];
        f32x4 rt[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          rt[dt] = zero;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) rt[dt] = mfma16(tile_frag(Pt, 16 * dt + r, 4 * ks + g), rb[ks], rt[dt]);
        }
        wait_vm<0>();
        lds_barrier();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int j = 0; j < 8; ++j) rn[ks][j] = (__bf16)rt[2 * ks + (j >> 2)][j & 3];
      }
      if (l == 0) Off[pr] = off;  // every wave writes the same value
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        *reinterpret_cast<bf16x8*>(St + pr * 4096 + a * 64 + 32 * ks + 8 * g) = rb[ks];
      rb[0] = rn[0];
      rb[1] = rn[1];
    };
    for (int64_t i = 0; i < m; i += 2) {
      p1step(slot_c<0>{}, m - 1 - i);
      if (i + 1 < m) p1step(slot_c<1>{}, m - 2 - i);
    }
  }
  lds_barrier();  // every wave is done with the P slots before the ring below reuses them

  // ---------------------------------------------------------------- key chunks through the LDS ring
  // stream position j: 0 = the own chunk m (in-chunk block), then n = j - 1 = 0 .. m-1
  auto chunk_at = [&](int64_t j) PA_INLINE -> int64_t { return j == 0 ? m : j - 1; };
  auto stage = [&](int64_t j, const PairSlot& sl) PA_INLINE {
    const int64_t n = chunk_at(j);
    const int64_t vr = L - n * 64;
    dma_tile<2>(sl.t[0], kt + ((size_t)bh * Lp + (size_t)n * 64) * 64, 64, i0);
    dma_tile<2>(sl.t[1], v + ((size_t)bh * L + (size_t)n * 64) * 64, vr < 64 ? (int)vr : 64, i0);
    dma_tile<2>(sl.t[2], Pm + ((size_t)bh * M + (size_t)n) * 4096, 64, i0);
    if constexpr (FOX) row_to_lds(sl.rows[0], fl + (size_t)bh * Lp + (size_t)n * 64, wave, l);
  };
  const int64_t steps = m + 1;
  stage(0, qslot(slot_c<0>{}));
  wait_vm<0>();
  lds_barrier();
  // the first key chunk and its state are requested before the in-chunk block (which reads slot 0 only)
  bf16x8 rn[2];  // r^(n) of the next step, from the pair states
  float offn = 0.f;
  auto fetch_state = [&](int64_t n) PA_INLINE {
    const size_t pr = band.slot(bh, m, n);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) rn[ks] = *reinterpret_cast<const bf16x8*>(St + pr * 4096 + a * 64 + 32 * ks + 8 * g);
    if constexpr (FOX) offn = Off[pr];
  };
  if (m > 0) {
    fetch_state(0);
    stage(1, qslot(slot_c<1>{}));
  }

  float rs = 0.f;  // row sum of dz for query a, this lane's keys
  // in-chunk block: logits from the packed S, dO V_m^T on the matrix cores
  {
    const PairSlot s0 = qslot(slot_c<0>{});
    const __bf16* Vt = s0.t[1];
    f32x4 dp[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      dp[t] = zero;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) dp[t] = mfma16(tile_frag(Vt, 16 * t + r, 4 * ks + g), dob[ks], dp[t]);
    }
    const float* Sb = Sm + ((size_t)bh * M + (size_t)m) * kSGroups * 4;
    float* dSc = dSm + ((size_t)bh * M + (size_t)m) * 4096 + (size_t)a * 64;
    const int last = a >> 2;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int grp = (4 * t + g < last) ? 4 * t + g : last;  // groups past the diagonal re-read the last
      const float4 s4 = *reinterpret_cast<const float4*>(Sb + (s_row_group(a) + grp) * 4);
      const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
      float dz4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = 16 * t + 4 * g + i;
        // computed for every key, kept on and below the diagonal (entries past it are unspecified)
        const float z2 = sv[i] - (FOX ? kLog2e * s0.rows[0][b] : 0.f);
        const float dze = fast_exp2(z2 - l2a) * (dp[t][i] - Da);
        const float dz = b <= a ? dze : 0.f;
        rs += dz;
        dz4[i] = scale * dz;
      }
      *reinterpret_cast<float4*>(dSc + 16 * t + 4 * g) = make_float4(dz4[0], dz4[1], dz4[2], dz4[3]);
    }
  }

  // key chunks n = 0 .. m-1: z^T = ktilde_n r^(n)T, p, dz; dr^(n)T = ktilde_n^T g^T + P_n^T dr^(n-1)T
  f32x4 dR[4];  // dr^(n-1) transposed: [d 16 dt + 4g + i][query a]
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) dR[dt] = zero;
  // step j reads slot j & 1; it waits for everything (its chunk and state, requested one step earlier),
  // then requests the next step's state and chunk (into the slot of step j - 1, which every wave has left)
  auto p2step = [&](auto S, int64_t j) PA_INLINE {
    constexpr int sc = decltype(S)::value;
    wait_vm<0>();
    lds_barrier();
    bf16x8 rcur[2] = {rn[0], rn[1]};
    const float ofs = offn;
    if (j + 1 < steps) {
      fetch_state(j);  // r^(j), the state of step j + 1 (requested before the copies, into live registers)
      stage(j + 1, qslot(slot_c<sc ^ 1>{}));
    }
    const int64_t n = j - 1;
    const size_t pr = band.slot(bh, m, n);
    const PairSlot cur = qslot(S);
    const __bf16* Kt = cur.t[0];
    const __bf16* Vt = cur.t[1];
    const __bf16* Pt = cur.t[2];
    // dr^(n-1) as the operand (hi + lo); its hi part is the pair's stored gradient state
    bf16x8 dh[2], dl[2];
    acc_to_op(dR, dh, dl);
    if (n > 0) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) *reinterpret_cast<bf16x8*>(Gst + pr * 4096 + a * 64 + 32 * ks + 8 * g) = dh[ks];
    }
    f32x4 zt[4], dp[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      zt[t] = zero;
      dp[t] = zero;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        zt[t] = mfma16(tile_frag(Kt, 16 * t + r, 4 * ks + g), rcur[ks], zt[t]);
        dp[t] = mfma16(tile_frag(Vt, 16 * t + r, 4 * ks + g), dob[ks], dp[t]);
      }
    }
    f32x4 gt[4];  // ln2 dz, transposed: [key 16t + 4g + i][query a]
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = 16 * t + 4 * g + i;
        const float z2 = zt[t][i] + (FOX ? kLog2e * (ofs - cur.rows[0][b]) : 0.f);
        const float dz = fast_exp2(z2 - l2a) * (dp[t][i] - Da);
        rs += dz;
        gt[t][i] = kLn2 * dz;
      }
    bf16x8 gh[2];
    acc_to_bf(gt, gh);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      f32x4 acc = zero;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 kx = tr_frag(Kt, 16 * dt, ks, perm_pos);  // ktilde_n^T rows d = 16 dt + r, k = keys
        acc = mfma16(kx, gh[ks], acc);
      }
      if (n > 0) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 px = tr_frag(Pt, 16 * dt, ks, perm_pos);  // P_n^T rows d = 16 dt + r, k = d'
          acc = mfma16(px, dh[ks], acc);
          acc = mfma16(px, dl[ks], acc);
        }
      }
      dR[dt] = acc;
    }
   };
  for (int64_t j = 1; j < steps; j += 2) {
    p2step(slot_c<1>{}, j);
    if (j + 1 < steps) p2step(slot_c<0>{}, j + 1);
  }

  // d qtilde = dr^(m-1) (qtilde entered the scan scaled by scale * log2e), row sums of dz
  {
    const float sq = scale * kLog2e;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      *reinterpret_cast<float4*>(dqt + (row0 + a) * 64 + 16 * dt + 4 * g) =
          make_float4(sq * dR[dt][0], sq * dR[dt][1], sq * dR[dt][2], sq * dR[dt][3]);
    const float s = colsum4(rs);
    if (g == 0) drow[row0 + a] = s;
  }
}

// Key-chunk kernel: one block of 4 waves per (key chunk n < me, batch*head); wave w owns the keys
// b = 16w .. 16w+15 of the chunk (lane (r, g) key 16w + r).  The band's share of dv, d ktilde, dP_n and
// the column sums of dz, added to the earlier bands' sums (fixed order: deterministic).  Per query chunk
// m the pair states r^(n)_m, dr^(n-1)_m and the rows of dO_m stream through a ring of LDS slots.
//   z[a][b] = r^(n)_m[a] . ktilde_n[b]  (queries x keys; accumulator rows a, column b)
//   dv^T += dO_m^T p,  dktilde^T += r^T g,  dP_n[x][y] += sum_a dr[a][x] r[a][y]
template <bool FOX>
__global__ __launch_bounds__(256, 2) void bwd_key_tile_kernel(
    const __bf16* __restrict__ kt, const float* __restrict__ Sm, const float* __restrict__ fl,
    const __bf16* __restrict__ v, const __bf16* __restrict__ dout, const __bf16* __restrict__ St,
    const __bf16* __restrict__ Gst, const float* __restrict__ Off, const float* __restrict__ lse2w,
    const float* __restrict__ Dw, int64_t L, int64_t M, pair_band band, __bf16* __restrict__ dv,
    float* __restrict__ dva, float* __restrict__ dkt, float* __restrict__ dPm, float* __restrict__ dcol,
    int64_t BH) {
  // ring slots: r^(n)_m, dr^(n-1)_m, dO_m tiles; lse2 and D rows of chunk m
  __shared__ __align__(1024) __bf16 kr0[kTile], kg0[kTile], ko0[kTile], kr1[kTile], kg1[kTile], ko1[kTile];
  __shared__ __align__(1024) __bf16 kr2[kTile], kg2[kTile], ko2[kTile];
  __shared__ __align__(16) float kl0[64], kd0[64], kl1[64], kd1[64], kl2[64], kd2[64];
  auto ring = [&](auto S) PA_INLINE -> PairSlot {
    constexpr int sidx = decltype(S)::value;
    static_assert(sidx >= 0 && sidx < kRingSlots, "ring slot");
    if constexpr (sidx == 0) return PairSlot{{kr0, kg0, ko0}, {kl0, kd0}};
    else if constexpr (sidx == 1) return PairSlot{{kr1, kg1, ko1}, {kl1, kd1}};
    else return PairSlot{{kr2, kg2, ko2}, {kl2, kd2}};
  };

  int64_t bh, n;
  if (!bwd_pair_block(BH, band.me, bh, n)) return;  // whole block; low key chunks first
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, r = l & 15, g = l >> 4;
  const int64_t Lp = M * 64;
  const size_t rown = (size_t)bh * Lp + (size_t)n * 64;
  const bool first = n >= band.mb;  // key chunk n's own query chunk is in this band: the sums start here
  const bool last = band.me == M;   // the sums end here
  const bool trans = n > 0;         // pairs (m, n) carry a transition below them (dr^(n-1) exists)
  const int b = 16 * wave + r;      // this lane's key within chunk n
  const int64_t ib = n * 64 + b;
  const int i0 = 2 * wave;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  // ktilde_b (d in the permuted key order) and v_b (natural) as B-operands
  bf16x8 kb[2], vb[2];
  {
    const size_t rv = ((size_t)bh * L + (size_t)(ib < L ? ib : L - 1)) * 64;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      kb[ks] = *reinterpret_cast<const bf16x8*>(kt + (rown + b) * 64 + 32 * ks + 8 * g);
      vb[ks] = *reinterpret_cast<const bf16x8*>(v + rv + 32 * ks + 8 * g);
    }
  }
  const float Fb = FOX ? fl[rown + b] : 0.f;

  f32x4 aV[4], aK[4], aP[4];  // dv^T, dktilde^T: [x 16 xt + 4g + i][key b];  dP: [x 16 wave + 4g + i][y 16 yt + r]
  float cs = 0.f;             // column sum of dz for key b, this lane's queries
  const size_t pbase = ((size_t)bh * M + (size_t)n) * 4096;
  if (!first) {  // the sums of the earlier bands
#pragma unroll
    for (int xt = 0; xt < 4; ++xt) {
      const float4 x = *reinterpret_cast<const float4*>(dva + (rown + b) * 64 + 16 * xt + 4 * g);
      const float4 y = *reinterpret_cast<const float4*>(dkt + (rown + b) * 64 + 16 * xt + 4 * g);
      aV[xt] = f32x4{x.x, x.y, x.z, x.w};
      aK[xt] = f32x4{y.x, y.y, y.z, y.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) aP[xt][i] = dPm[pbase + (16 * wave + 4 * g + i) * 64 + 16 * xt + r];
    }
  } else {
#pragma unroll
    for (int xt = 0; xt < 4; ++xt) aV[xt] = aK[xt] = aP[xt] = zero;
  }

  // p of a step as the k = queries operand (bf16)
  auto dv_update = [&](const __bf16* Ot, const f32x4 (&pt)[4]) PA_INLINE {
    bf16x8 ph[2];
    acc_to_bf(pt, ph);
#pragma unroll
    for (int xt = 0; xt < 4; ++xt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 ox = tr_frag(Ot, 16 * xt, ks, col_identity);  // dO_m^T rows x = 16 xt + r, k = queries
        aV[xt] = mfma16(ox, ph[ks], aV[xt]);
      }
  };
  auto stage_rows = [&](int64_t mm, const PairSlot& sl) PA_INLINE {
    const int64_t vr = L - mm * 64;
    dma_tile<2>(sl.t[2], dout + ((size_t)bh * L + (size_t)mm * 64) * 64, vr < 64 ? (int)vr : 64, i0);
    row_to_lds(sl.rows[0], lse2w + (size_t)bh * Lp + (size_t)mm * 64, wave, l);
    row_to_lds(sl.rows[1], Dw + (size_t)bh * Lp + (size_t)mm * 64, wave, l);
  };

  // in-chunk block (m = n): logits from the packed S; dv only
  if (first) {
    const PairSlot s0 = ring(slot_c<0>{});
    stage_rows(n, s0);
    wait_vm<0>();
    lds_barrier();
    const __bf16* Ot = s0.t[2];
    const float* Sb = Sm + ((size_t)bh * M + (size_t)n) * kSGroups * 4;
    f32x4 pt[4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      f32x4 dp = zero;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) dp = mfma16(tile_frag(Ot, 16 * qt + r, 4 * ks + g), vb[ks], dp);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int a = 16 * qt + 4 * g + i;
        // every lane loads (entries past the diagonal read the diagonal's), then selects: no load waits
        // inside a branch
        const float sab = Sb[s_row_group(a) * 4 + (b <= a ? b : a)];
        const float z2 = sab - (FOX ? kLog2e * Fb : 0.f);
        const float pe = fast_exp2(z2 - s0.rows[0][a]);
        const float p = b <= a ? pe : 0.f;
        const float dz = p * (dp[i] - s0.rows[1][a]);
        cs += dz;
        pt[qt][i] = p;
      }
    }
    dv_update(Ot, pt);
    lds_barrier();  // every wave is done with slot 0 before the ring reuses it
  }

  // the band's query chunks m > n
  const int64_t m0 = n + 1 > band.mb ? n + 1 : band.mb;
  const int64_t steps = band.me - m0;
  if (steps > 0) {
    auto stage = [&](int64_t k, const PairSlot& sl) PA_INLINE {
      const int64_t mm = m0 + k;
      const size_t pr = band.slot(bh, mm, n);
      dma_tile<2>(sl.t[0], St + pr * 4096, 64, i0);
      dma_tile<2>(sl.t[1], Gst + pr * 4096, 64, i0);  // (not written for n = 0: copied, not used)
      stage_rows(mm, sl);
    };
    constexpr int OPS = slot_ops<2>();
    float offn = FOX ? Off[band.slot(bh, m0, n)] : 0.f;
    stage(0, ring(slot_c<0>{}));
    if (steps > 1) {
      stage(1, ring(slot_c<1>{}));
      wait_vm<OPS>();
    } else {
      wait_vm<0>();
    }
    lds_barrier();
    // step k reads slot k % 3; query chunk k + 2 goes into slot (k + 2) % 3, last read in step k - 1
    auto step = [&](auto S, int64_t k) PA_INLINE {
      constexpr int sc = decltype(S)::value;
      const PairSlot cur = ring(S);
      const __bf16* Rt = cur.t[0];
      const __bf16* Gt = cur.t[1];
      const __bf16* Ot = cur.t[2];
      const float* l2r = cur.rows[0];
      const float* Dr = cur.rows[1];
      const float ofs = offn;
      if constexpr (FOX) offn = Off[band.slot(bh, m0 + (k + 1 < steps ? k + 1 : k), n)];
      f32x4 pt[4], gt[4];
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        f32x4 z = zero, dp = zero;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          z = mfma16(tile_frag(Rt, 16 * qt + r, 4 * ks + g), kb[ks], z);
          dp = mfma16(tile_frag(Ot, 16 * qt + r, 4 * ks + g), vb[ks], dp);
        }
        const float4 l4 = *reinterpret_cast<const float4*>(l2r + 16 * qt + 4 * g);
        const float4 d4 = *reinterpret_cast<const float4*>(Dr + 16 * qt + 4 * g);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float z2 = z[i] + (FOX ? kLog2e * (ofs - Fb) : 0.f);
          const float p = fast_exp2(z2 - lv[i]);
          const float dz = p * (dp[i] - dv4[i]);
          cs += dz;
          pt[qt][i] = p;
          gt[qt][i] = kLn2 * dz;
        }
      }
      dv_update(Ot, pt);
      {
        bf16x8 gh[2];
        acc_to_bf(gt, gh);
#pragma unroll
        for (int xt = 0; xt < 4; ++xt)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 rx = tr_frag(Rt, 16 * xt, ks, perm_pos);  // r^T rows x = 16 xt + r, k = queries
            aK[xt] = mfma16(rx, gh[ks], aK[xt]);
          }
      }
      if (trans) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 gx = tr_frag(Gt, 16 * wave, ks, perm_pos);  // dr^T rows x = 16 wave + r, k = queries
#pragma unroll
          for (int yt = 0; yt < 4; ++yt) aP[yt] = mfma16(gx, tr_frag(Rt, 16 * yt, ks, perm_pos), aP[yt]);
        }
      }
      // ring: query chunk k + 2 into the slot two ahead, chunk k + 1 has landed
      if (k + 2 < steps) {
        stage(k + 2, ring(slot_c<(sc + 2) % kRingSlots>{}));
        wait_vm<OPS>();
      } else {
        wait_vm<0>();
      }
      lds_barrier();
    };
    for (int64_t k = 0; k < steps; k += kRingSlots) {
      step(slot_c<0>{}, k);
      if (k + 1 < steps) step(slot_c<1>{}, k + 1);
      if (k + 2 < steps) step(slot_c<2>{}, k + 2);
    }
  }

  // outputs
#pragma unroll
  for (int xt = 0; xt < 4; ++xt) {
    const size_t o = (rown + b) * 64 + 16 * xt + 4 * g;
    *reinterpret_cast<float4*>(dkt + o) = make_float4(aK[xt][0], aK[xt][1], aK[xt][2], aK[xt][3]);
    if (!last) {
      *reinterpret_cast<float4*>(dva + o) = make_float4(aV[xt][0], aV[xt][1], aV[xt][2], aV[xt][3]);
    } else if (ib < L) {
      bf16x4 h;
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = (__bf16)aV[xt][i];
      *reinterpret_cast<bf16x4*>(dv + ((size_t)bh * L + (size_t)ib) * 64 + 16 * xt + 4 * g) = h;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) dPm[pbase + (16 * wave + 4 * g + i) * 64 + 16 * xt + r] = aP[xt][i];
  }
  const float s = colsum4(cs);
  if (g == 0) dcol[rown + b] = (first ? 0.f : dcol[rown + b]) + s;
}

// ------------------------------------------------------------------------------- per-chunk gradients
// Gradients of a chunk's terms (d qtilde, d ktilde, dP, dS) back through the UT transform to dq, dk, dw,
// dbeta, for bf16 inputs (the math of bwd_chunk_grad_mfma_kernel in backward.hip):
//   dX = -W dqtilde^T      dY = -dktilde W^T - dS^T U^T      dU = Ti^T dX - (dS Y)^T      dR = dY Ti^T
//   dTi = dX U^T + R^T dY - W dP W^T,  M1 = A^{-T} dTi,  dA = -M1 Ti^T (strict upper)
//   dbeta = diag(M1) + rowsum(dA o W W^T),  dN = diag(beta) dA
//   dW = -X dqtilde - Y^T dktilde - Ti W dP^T - Ti^T W dP + dU Q + dR^T K + (dN + dN^T) W
//   dQ = dqtilde + dS K + dU^T W,   dK = dktilde + dS^T Q + dR W
// Every operand is a bf16 LDS tile with permuted columns (swizzled): w, q and k exactly, every fp32 matrix
// (the inputs d qtilde, d ktilde, dS, dP, A^{-1} and the intermediates) as a hi + lo pair split once when
// it is stored, so that a fragment in either orientation is one LDS read (tile_frag by rows, tr_frag by
// columns) in the accumulator key order.  Eight waves: wave 4h + w works on rows 16 w .. 16 w + 15 and
// column blocks 2h, 2h + 1 of every product.
namespace {

struct GradOp {
  const __bf16* hi;
  const __bf16* lo;  // (split tiles; unused for exact ones)
};

// fragment of rows (TR = false: M[base16 + r][k]) or columns (TR = true: M[k][base16 + r]), k in the
// accumulator key order 32 ks + 16 (j / 4) + 4g + j % 4
template <bool SPLIT, bool TR>
__device__ __forceinline__ void grad_frag(const GradOp& o, int base16, int ks, bf16x8& h, bf16x8& l) {
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  if constexpr (TR) {
    h = tr_frag(o.hi, base16, ks, perm_pos);
    if constexpr (SPLIT) l = tr_frag(o.lo, base16, ks, perm_pos);
  } else {
    h = tile_frag(o.hi, base16 + r, 4 * ks + g);
    if constexpr (SPLIT) l = tile_frag(o.lo, base16 + r, 4 * ks + g);
  }
}

#ifndef PATHATTN_GRAD_WAVES
#define PATHATTN_GRAD_WAVES 8
#endif
// Waves of the per-chunk gradient kernel: 4 row blocks x (waves / 4) column groups of 16 / (waves / 4) * 16
// columns each.
constexpr int kGradWaves = PATHATTN_GRAD_WAVES, kGradThreads = 64 * kGradWaves;
constexpr int kGradGroups = kGradWaves / 4, kGradNc = 4 / kGradGroups;
static_assert(kGradWaves == 8 || kGradWaves == 16, "gradient kernel waves");

// acc[c] += sum_k A(16w + r', k) B(k, 16(cb0 + c) + r''); AT: A(i, k) = A[k][i], else A[i][k]; BK:
// B(k, j) = B[k][j], else B[j][k].  An exact operand contributes one bf16 product, a split one its hi and
// lo parts (hi*hi + hi*lo + lo*hi; lo*lo dropped).
template <bool SA, bool AT, bool SB, bool BK>
__device__ __forceinline__ void gmm(f32x4 (&acc)[kGradNc], const GradOp& A, const GradOp& B, int w, int cb0) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    bf16x8 ah, al;
    grad_frag<SA, AT>(A, 16 * w, ks, ah, al);
#pragma unroll
    for (int c = 0; c < kGradNc; ++c) {
      bf16x8 bh, bl;
      grad_frag<SB, BK>(B, 16 * (cb0 + c), ks, bh, bl);
      acc[c] = mfma16(ah, bh, acc[c]);
      if constexpr (SB) acc[c] = mfma16(ah, bl, acc[c]);
      if constexpr (SA) acc[c] = mfma16(al, bh, acc[c]);
    }
  }
}
constexpr bool kE = false, kS2 = true;  // exact / split operand

__device__ __forceinline__ int tile_slot(int row, int col) {
  const int pp = perm_pos(col);
  return swz(row, pp >> 3) + (pp & 7);
}
// accumulator (rows 16w + 4g + e, columns 16(cb0 + c) + r) -> split tile pair, through f(i, j, x)
template <typename F>
__device__ __forceinline__ void gstore(const f32x4 (&acc)[kGradNc], __bf16* hi, __bf16* lo, int w, int cb0, F f) {
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int c = 0; c < kGradNc; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * w + 4 * g + e, j = 16 * (cb0 + c) + r;
      const float v = f(i, j, acc[c][e]);
      const __bf16 hv = (__bf16)v;
      hi[tile_slot(i, j)] = hv;
      lo[tile_slot(i, j)] = (__bf16)(v - (float)hv);
    }
}
// A [64][64] fp32 matrix in global memory (row stride 64) as float4 pieces held by the block's threads
// (piece tid + kGradThreads it), and those pieces, times a per-column factor, into a split tile pair.
constexpr int kGradPieces = 1024 / kGradThreads;
__device__ __forceinline__ void load_pieces(float4 (&f)[kGradPieces], const float* __restrict__ m, int tid) {
#pragma unroll
  for (int it = 0; it < kGradPieces; ++it) {
    const int e = tid + kGradThreads * it;
    f[it] = *reinterpret_cast<const float4*>(m + (e >> 4) * 64 + (e & 15) * 4);
  }
}
template <bool COLSCALE>
__device__ __forceinline__ void put_split(__bf16* hi, __bf16* lo, const float4 (&f)[kGradPieces], const float* cs,
                                          int tid) {
#pragma unroll
  for (int it = 0; it < kGradPieces; ++it) {
    const int e = tid + kGradThreads * it, row = e >> 4, c4 = (e & 15) * 4;
    float4 x = f[it];
    if constexpr (COLSCALE) x.x *= cs[c4], x.y *= cs[c4 + 1], x.z *= cs[c4 + 2], x.w *= cs[c4 + 3];
    bf16x4 h, l;
    split4(x.x, x.y, x.z, x.w, h, l);
    const int sl = tile_slot(row, c4);
    *reinterpret_cast<bf16x4*>(hi + sl) = h;
    *reinterpret_cast<bf16x4*>(lo + sl) = l;
  }
}
__device__ __forceinline__ void zero2(f32x4 (&acc)[kGradNc]) {
#pragma unroll
  for (int c = 0; c < kGradNc; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
}
__device__ __forceinline__ void sub2(f32x4 (&acc)[kGradNc], const f32x4 (&t)[kGradNc]) {
#pragma unroll
  for (int c = 0; c < kGradNc; ++c) acc[c] -= t[c];
}
// rows of a global fp32 [64][64] matrix into the accumulator layout
__device__ __forceinline__ void glob_acc(f32x4 (&acc)[kGradNc], const float* m, int w, int cb0) {
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int c = 0; c < kGradNc; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[c][e] = m[(16 * w + 4 * g + e) * 64 + 16 * (cb0 + c) + r];
}

}  // namespace

__global__ __launch_bounds__(kGradThreads) void bwd_chunk_grad_tile_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ w,
    const float* __restrict__ beta, const float* __restrict__ dqt, const float* __restrict__ dkt,
    const float* __restrict__ dPm, const float* __restrict__ dSm, const float* __restrict__ Zi, int64_t L,
    int64_t M, __bf16* __restrict__ dq, __bf16* __restrict__ dk, __bf16* __restrict__ dw,
    float* __restrict__ dbeta) {
  __shared__ __align__(1024) __bf16 te[3][kTile];  // W, Q, K (exact)
  // split pairs: Ti | U, dU, dTi | R, dR, M1 | dS, A^{-1} | X, dX, W dP, dN | Y, dY, W dP^T | dqtilde, dP | dktilde
  __shared__ __align__(1024) __bf16 ts[8][2][kTile];
  __shared__ float Bs[64];
  __shared__ float dB[64 * kGradGroups];  // dbeta partials, one row of 64 per column group (each address
                                         // filled by a single wave)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wv = wave & 3, cgrp = wave >> 2, cb0 = kGradNc * cgrp;
  const int r = lane & 15, g = lane >> 4;
  const int64_t c = blockIdx.x, bh = blockIdx.y, Lp = M * 64;
  const size_t row0 = (size_t)bh * Lp + (size_t)c * 64;
  const GradOp W{te[0], nullptr}, Q{te[1], nullptr}, K{te[2], nullptr};
  auto split = [&](int i) PA_INLINE { return GradOp{ts[i][0], ts[i][1]}; };
  const GradOp S3 = split(0), S4 = split(1), S5 = split(2), S6 = split(3), S7 = split(4), S8 = split(5);
  const GradOp dS = split(3), dQ = split(6), dP = split(6), dK = split(7);
  const float* zc = Zi + ((size_t)bh * M + c) * 64 * 64;  // A^{-1}
  const float* dSg = dSm + ((size_t)bh * M + c) * 64 * 64;
  auto keep = [](int, int, float x) { return x; };
  auto neg = [](int, int, float x) { return -x; };

  // Every global input of the first phases is requested before any is waited for (one memory round
  // trip): W, Q, K of the chunk (rows past L zero), beta (padded tokens: identity), d qtilde, d ktilde,
  // dS, A^{-1} and the rows of d qtilde, d ktilde that seed dq, dk; dP follows once the first tiles
  // are stored, and A^{-1} stays in registers until its tile is free.
  constexpr int kWqk = 3 * 1024 / kGradThreads;  // bf16x4 pieces of W, Q, K per thread
  bf16x4 wqk[kWqk];
  {
    const size_t base = (size_t)bh * L * 64;
#pragma unroll
    for (int i = 0; i < kWqk; ++i) {
      const int e = tid + kGradThreads * i, tt = e >> 10, row = (e >> 4) & 63, c4 = (e & 15) * 4;
      const __bf16* src = tt == 0 ? w : (tt == 1 ? q : k);
      const int64_t tok = c * 64 + row;
      wqk[i] = *reinterpret_cast<const bf16x4*>(src + base + (size_t)(tok < L ? tok : L - 1) * 64 + c4);
    }
  }
  float bv = 0.f;
  if (tid < 64) bv = beta[bh * L + (c * 64 + tid < L ? c * 64 + tid : L - 1)];
  float4 fS[kGradPieces], fQ[kGradPieces], fK[kGradPieces], fZ[kGradPieces], fP[kGradPieces];
  load_pieces(fS, dSg, tid);
  load_pieces(fQ, dqt + row0 * 64, tid);
  load_pieces(fK, dkt + row0 * 64, tid);
  load_pieces(fZ, zc, tid);
  f32x4 aq[kGradNc], ak[kGradNc], aw[kGradNc], t[kGradNc], u[kGradNc], rU[kGradNc], rG[kGradNc];
  glob_acc(aq, dqt + row0 * 64, wv, cb0);  // dq = d qtilde + ...
  glob_acc(ak, dkt + row0 * 64, wv, cb0);  // dk = d ktilde + ...
  if (tid < 64 * kGradGroups) dB[tid] = 0.f;
  if (tid < 64) Bs[tid] = c * 64 + tid < L ? bv : 0.f;
#pragma unroll
  for (int i = 0; i < kWqk; ++i) {
    const int e = tid + kGradThreads * i, tt = e >> 10, row = (e >> 4) & 63, c4 = (e & 15) * 4;
    *reinterpret_cast<bf16x4*>(te[tt] + tile_slot(row, c4)) = c * 64 + row < L ? wqk[i] : bf16x4{};
  }
  put_split<false>(ts[3][0], ts[3][1], fS, nullptr, tid);
  put_split<false>(ts[6][0], ts[6][1], fQ, nullptr, tid);
  put_split<false>(ts[7][0], ts[7][1], fK, nullptr, tid);
  __syncthreads();
  load_pieces(fP, dPm + ((size_t)bh * M + c) * 64 * 64, tid);
  put_split<true>(ts[0][0], ts[0][1], fZ, Bs, tid);  // Ti = A^{-1} diag(beta)
  zero2(t);
  gmm<kE, false, kE, false>(t, W, Q, wv, cb0);  // w_t . q_a
  gstore(t, ts[1][0], ts[1][1], wv, cb0, [](int i, int j, float x) { return i <= j ? x : 0.f; });
  zero2(t);
  gmm<kE, false, kE, false>(t, K, W, wv, cb0);  // k_b . w_s
  gstore(t, ts[2][0], ts[2][1], wv, cb0, [](int i, int j, float x) { return j > i ? x : 0.f; });
  __syncthreads();

  zero2(aw);
  zero2(t);
  gmm<kS2, false, kS2, true>(t, S3, S4, wv, cb0);  // X = Ti U
  gstore(t, ts[4][0], ts[4][1], wv, cb0, keep);
  zero2(t);
  gmm<kS2, false, kS2, true>(t, S5, S3, wv, cb0);  // Y = R Ti
  gstore(t, ts[5][0], ts[5][1], wv, cb0, keep);
  gmm<kS2, false, kE, true>(aq, dS, K, wv, cb0);  // dq += dS K
  gmm<kS2, true, kE, true>(ak, dS, Q, wv, cb0);   // dk += dS^T Q
  __syncthreads();
  zero2(t);
  gmm<kS2, false, kS2, true>(t, S7, dQ, wv, cb0);  // X dqtilde
  gmm<kS2, true, kS2, true>(t, S8, dK, wv, cb0);   // + Y^T dktilde
  sub2(aw, t);
  zero2(u);
  gmm<kE, false, kS2, false>(u, W, dQ, wv, cb0);  // -dX = W dqtilde^T
  zero2(t);
  gmm<kS2, false, kE, false>(t, dK, W, wv, cb0);   // -dY = dktilde W^T
  gmm<kS2, true, kS2, false>(t, dS, S4, wv, cb0);  //       + dS^T U^T
  zero2(rU);
  gmm<kS2, true, kS2, false>(rU, S8, dS, wv, cb0);  // (dS Y)^T
  __syncthreads();
  gstore(u, ts[4][0], ts[4][1], wv, cb0, neg);  // dX
  gstore(t, ts[5][0], ts[5][1], wv, cb0, neg);  // dY
  put_split<false>(ts[6][0], ts[6][1], fP, nullptr, tid);  // dP
  put_split<false>(ts[3][0], ts[3][1], fZ, nullptr, tid);  // A^{-1}
  __syncthreads();
  zero2(u);
  gmm<kS2, true, kS2, true>(u, S3, S7, wv, cb0);  // dU = Ti^T dX - (dS Y)^T
  sub2(u, rU);
  zero2(rG);
  gmm<kS2, false, kS2, false>(rG, S7, S4, wv, cb0);  // dTi = dX U^T
  gmm<kS2, true, kS2, true>(rG, S5, S8, wv, cb0);    //     + R^T dY
  zero2(t);
  gmm<kS2, false, kS2, false>(t, S8, S3, wv, cb0);  // dR = dY Ti^T
  __syncthreads();
  gstore(u, ts[1][0], ts[1][1], wv, cb0, [](int i, int j, float x) { return i <= j ? x : 0.f; });
  gstore(t, ts[2][0], ts[2][1], wv, cb0, [](int i, int j, float x) { return j > i ? x : 0.f; });
  __syncthreads();
  gmm<kS2, false, kE, true>(aw, S4, Q, wv, cb0);  // dW += dU Q
  gmm<kS2, true, kE, true>(aw, S5, K, wv, cb0);   //     + dR^T K
  gmm<kS2, true, kE, true>(aq, S4, W, wv, cb0);   // dq += dU^T W
  gmm<kS2, false, kE, true>(ak, S5, W, wv, cb0);  // dk += dR W
  zero2(t);
  gmm<kE, false, kS2, true>(t, W, dP, wv, cb0);  // W dP
  zero2(u);
  gmm<kE, false, kS2, false>(u, W, dP, wv, cb0);  // W dP^T
  gstore(t, ts[4][0], ts[4][1], wv, cb0, keep);
  gstore(u, ts[5][0], ts[5][1], wv, cb0, keep);
  __syncthreads();
  zero2(t);
  gmm<kS2, false, kE, false>(t, S7, W, wv, cb0);  // dTi -= W dP W^T
  sub2(rG, t);
  zero2(t);
  gmm<kS2, false, kS2, true>(t, S3, S8, wv, cb0);  // dW -= Ti W dP^T
  gmm<kS2, true, kS2, true>(t, S3, S7, wv, cb0);   //      + Ti^T W dP
  sub2(aw, t);
  __syncthreads();
  gstore(rG, ts[1][0], ts[1][1], wv, cb0, keep);
  __syncthreads();
  zero2(t);
  gmm<kS2, true, kS2, true>(t, S6, S4, wv, cb0);  // M1 = A^{-T} dTi; dbeta += diag(M1)
#pragma unroll
  for (int cc = 0; cc < kGradNc; ++cc)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (16 * wv + 4 * g + e == 16 * (cb0 + cc) + r) atomicAdd(&dB[64 * cgrp + 16 * (cb0 + cc) + r], t[cc][e]);
  gstore(t, ts[2][0], ts[2][1], wv, cb0, keep);
  __syncthreads();
  zero2(t);
  gmm<kS2, false, kS2, false>(t, S5, S3, wv, cb0);  // M1 Ti^T
  zero2(u);
  gmm<kE, false, kE, false>(u, W, W, wv, cb0);  // w_r . w_s
  {
    float rowp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < kGradNc; ++cc)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * wv + 4 * g + e, j = 16 * (cb0 + cc) + r;
        const float z = i < j ? -t[cc][e] : 0.f;  // dA[i][j]
        rowp[e] += z * u[cc][e];
        t[cc][e] = Bs[i] * z;  // dN
      }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = rowp[e];
      x += __shfl_xor(x, 1);
      x += __shfl_xor(x, 2);
      x += __shfl_xor(x, 4);
      x += __shfl_xor(x, 8);
      if (r == 0) atomicAdd(&dB[64 * cgrp + 16 * wv + 4 * g + e], x);
    }
  }
  gstore(t, ts[4][0], ts[4][1], wv, cb0, keep);
  __syncthreads();
  gmm<kS2, false, kE, true>(aw, S7, W, wv, cb0);  // dW += dN W
  gmm<kS2, true, kE, true>(aw, S7, W, wv, cb0);   //      + dN^T W
  __syncthreads();
#pragma unroll
  for (int cc = 0; cc < kGradNc; ++cc)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int a = 16 * wv + 4 * g + e, x = 16 * (cb0 + cc) + r;
      const int64_t i = c * 64 + a;
      if (i < L) {
        const size_t o = ((size_t)bh * L + i) * 64 + x;
        dq[o] = (__bf16)aq[cc][e];
        dk[o] = (__bf16)ak[cc][e];
        dw[o] = (__bf16)aw[cc][e];
      }
    }
  if (tid < 64 && c * 64 + tid < L) {
    float sb = dB[tid];
#pragma unroll
    for (int h = 1; h < kGradGroups; ++h) sb += dB[64 * h + tid];
    dbeta[bh * L + c * 64 + tid] = sb;
  }
}

hipError_t bwd_chunk_grad_tiles_run(const void* q, const void* k, const void* w, const float* beta, int64_t BH,
                                    int64_t L, const bwd_buffers& b, void* dq, void* dk, void* dw, float* dbeta,
                                    hipStream_t st) {
  const int64_t M = (L + 63) / 64;
  bwd_chunk_grad_tile_kernel<<<dim3((unsigned)M, (unsigned)BH), kGradThreads, 0, st>>>(
      (const __bf16*)q, (const __bf16*)k, (const __bf16*)w, beta, b.dqt, b.dkt, b.dPm, b.dSm, b.Zi, L, M,
      (__bf16*)dq, (__bf16*)dk, (__bf16*)dw, dbeta);
  return hipGetLastError();
}

// One band of query chunks: the query-side kernel, then the key-side kernel.
hipError_t bwd_pair_tiles_run(bool fox, const void* v, const void* out, const void* dout, const float* lse,
                              int64_t BH, int64_t L, float scale, pair_band band, const bwd_buffers& b,
                              void* dv, hipStream_t st) {
  const int64_t M = (L + 63) / 64;
  const int64_t xh = kBwdXcd * ((BH + kBwdXcd - 1) / kBwdXcd);
  const __bf16* qt = reinterpret_cast<const __bf16*>(b.qt);
  const __bf16* kt = reinterpret_cast<const __bf16*>(b.kt);
  const __bf16* Pm = reinterpret_cast<const __bf16*>(b.Pm);
  __bf16* St = reinterpret_cast<__bf16*>(b.St);
  __bf16* Gst = reinterpret_cast<__bf16*>(b.Gst);
  const dim3 gq((unsigned)(xh * (band.me - band.mb))), gk((unsigned)(xh * band.me));
  auto q = [&](auto kernel) {
    kernel<<<gq, 256, 0, st>>>(qt, kt, Pm, b.Sm, fox ? b.fl : nullptr, b.ftot, (const __bf16*)v, (const __bf16*)out,
                              (const __bf16*)dout, lse, L, M, scale, band, St, Gst, b.Off, b.lse2, b.Dv, b.drow,
                              b.dqt, b.dSm, BH);
  };
  if (fox) q(bwd_query_tile_kernel<true>);
  else q(bwd_query_tile_kernel<false>);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  auto k = [&](auto kernel) {
    kernel<<<gk, 256, 0, st>>>(kt, b.Sm, fox ? b.fl : nullptr, (const __bf16*)v, (const __bf16*)dout, St, Gst, b.Off,
                              b.lse2, b.Dv, L, M, band, (__bf16*)dv, b.dva, b.dkt, b.dPm, b.dcol, BH);
  };
  if (fox) k(bwd_key_tile_kernel<true>);
  else k(bwd_key_tile_kernel<false>);
  return hipGetLastError();
}

}  // namespace pathattn

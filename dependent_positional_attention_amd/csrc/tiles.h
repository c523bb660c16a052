// bf16 64 x 64 tiles in LDS and the MFMA operand conventions shared by the matrix-core prefill and
// backward kernels (gfx950 only).
//
// Column permutation: an MFMA accumulator gives each lane rows 4g..4g+3 of every 16-row tile, while a
// B-operand wants rows 8g..8g+7 of every 32-row k-step.  The contraction order is free, so tiles whose
// columns are contracted against accumulator-derived operands are stored with slot 8g+j of each
// 32-block holding index 16(j/4)+4g+(j%4); accumulators then convert to operands in registers with no
// data movement, and a row-fragment read of such a tile is already in that key order.
#pragma once

#include "common.h"

namespace pathattn {

namespace {

constexpr int kD = 64;  // head dim
constexpr int kC = 64;  // chunk

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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

// =========================================================================== swizzled LDS tiles
// LDS tiles of the key-chunk stream are 64 rows x 128 B with no padding; the 16-byte chunk c of
// row r sits at slot c ^ (r & 7) (an XOR swizzle), so the 16 rows an MFMA fragment read touches
// land in distinct banks.  Tiles are filled by direct global->LDS loads (16 B per lane, lane i
// of an instruction writes slot i of a 1 KiB run), so no staging registers are needed: each lane
// simply fetches the global chunk that belongs in its slot.
constexpr int kTile = kC * kD;  // bf16 elements of one swizzled 64x64 tile

__device__ __forceinline__ int swz(int row, int chunk) { return row * 64 + ((chunk ^ (row & 7)) << 3); }

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));

// Direct global->LDS copy of one 64x64 bf16 tile (64 contiguous rows of 128 B in global) by one
// wave: instructions i0 .. i0+CNT-1 each cover 8 rows.  Rows at or beyond `rmax` are clamped to
// rmax - 1 (finite data that only ever meets masked or discarded positions).  The per-lane part of
// the address is a 32-bit byte offset from the wave-uniform tile base (scalar base + vector offset).
template <int CNT = 2>
__device__ __forceinline__ void dma_tile(__bf16* tile, const __bf16* src, int rmax, int i0) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int i = i0; i < i0 + CNT; ++i) {
    const int row = 8 * i + (l >> 3), slot = l & 7;
    const int rs = row < rmax ? row : rmax - 1;
    uint32_t off = (uint32_t)(rs * 128 + ((slot ^ (row & 7)) << 4));
    // (an empty asm keeps the offset a fresh 32-bit register, so that the copy takes the scalar-base +
    // 32-bit-offset form instead of a 64-bit vector address rebuilt with a vector add per copy)
    __asm__ volatile("" : "+v"(off));
    __builtin_amdgcn_global_load_lds((const void*)(reinterpret_cast<const char*>(src) + off),
                                     (lds_void*)(tile + i * 512), 16, 0, 0);
  }
}

__device__ __forceinline__ bf16x8 tile_frag(const __bf16* tile, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(tile + swz(row, chunk));
}

// Transposed fragment: operand row/column index c0 + (l % 16) runs over the tile's COLUMNS and
// the k index over its ROWS, in the key order an accumulator-derived operand uses: lane (r, g)
// of k-step ks receives tile[row][c0 + r] for rows 32ks + 16h + 4g + (0..3), h = 0, 1.  Two LDS
// transpose reads: within a 16-lane group the transpose read gives lane d element (d & 3) of
// source lanes (d >> 2) + 4j, so source lane s points at row base + (s >> 2), columns
// c0 + 4(s & 3) .. +3.  `pcol` maps a logical column to its stored slot (identity, or the
// in-block permutation of tiles stored that way); it must keep aligned quads contiguous.
template <typename ColMap>
__device__ __forceinline__ bf16x8 tr_frag(const __bf16* tile, int c0, int ks, ColMap pcol) {
  const int l = threadIdx.x & 63, g = l >> 4, s = l & 15;
  const int col = pcol(c0 + 4 * (s & 3));
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
__device__ __forceinline__ int col_identity(int c) { return c; }

// V^T A-fragment from a row-major V tile ([key][d]): rows d = 16dt + r, keys in the order of
// the P^T B-operand.
__device__ __forceinline__ bf16x8 vt_frag(const __bf16* tile, int dt, int ks) {
  return tr_frag(tile, 16 * dt, ks, col_identity);
}

// Accumulator tiles D[16t + 4g + i][col] (t = 0..3) as the k = 0..63 operand (k order above).
__device__ __forceinline__ void acc_to_op(const f32x4 (&acc)[4], bf16x8 (&hi)[2], bf16x8 (&lo)[2]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = acc[2 * ks + (j >> 2)][j & 3];
      const __bf16 h = (__bf16)v;
      hi[ks][j] = h;
      lo[ks][j] = (__bf16)(v - (float)h);
    }
}

// The same operand rounded to bf16 once (no lo part).
__device__ __forceinline__ void acc_to_bf(const f32x4 (&acc)[4], bf16x8 (&hi)[2]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int j = 0; j < 8; ++j) hi[ks][j] = (__bf16)acc[2 * ks + (j >> 2)][j & 3];
}

// In-chunk logits S of the bf16 forms, packed: only entries on or below the diagonal are ever read, so
// row a keeps its 4-float groups 0 .. a/4 (columns 0 .. 4(a/4) + 3; the entries of the last group
// past the diagonal are unspecified), rows back to back.  Row a starts at group
// a + sum_{b<a} floor(b/4) = a + 2u(u - 1) + uv (u = a/4, v = a%4); a 64-token chunk takes 544
// groups, 53% of the square.
constexpr int kSGroups = 544;
__host__ __device__ constexpr int s_row_group(int a) { return a + 2 * (a >> 2) * ((a >> 2) - 1) + (a >> 2) * (a & 3); }
static_assert(s_row_group(kC) == kSGroups, "packed S size");

// Sum of x over the four lanes r, r + 16, r + 32, r + 48 (the g index of an accumulator), in all four.
__device__ __forceinline__ float colsum4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Workgroup barrier that leaves outstanding global->LDS copies in flight (the plain
// __syncthreads() drains every memory counter first).  LDS reads issued before it have
// returned; the copies a later step reads are waited for explicitly, per wave, before it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// s_waitcnt vmcnt(n) (expcnt, lgkmcnt untouched), n < 64: the count's low 4 bits sit in bits 3:0 of
// the immediate, its high 2 bits in bits 15:14
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

}  // namespace pathattn

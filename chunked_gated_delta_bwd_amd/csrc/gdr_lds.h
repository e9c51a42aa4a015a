// LDS tile helpers shared by the chain and gradient kernels (gfx950): XOR-swizzled
// unpadded bf16 tiles, MFMA fragments read from them, direct-to-LDS loads, and a
// workgroup barrier that orders LDS traffic only.
#pragma once

#include <hip/hip_runtime.h>

#include "gdr_device.h"

namespace gdr {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

// ---------------------------------------------------------------------------
// swizzled LDS tiles
// ---------------------------------------------------------------------------
// Piece p (16 bytes) of row r of a W-column bf16 tile sits at piece p ^ swz(r).
// The functions were chosen by measuring LDS bank conflicts on gfx950:
//   W = 128: (r ^ 2r) mod 16 is conflict-free for both row-fragment reads (16
//            rows at one piece, ds_read_b128) and transposed reads (rows
//            r..r+3 and r+8..r+11 at two adjacent pieces, ds_read_b64_tr_b16);
//   W = 64, kind 0: conflict-free transposed reads (the P tile, 64-wide tiles);
//   W = 64, kind 1: r mod 8, conflict-free row-fragment reads (16-row tiles);
//   W = 16: no swizzle, but rows 8-11 and 12-15 of every 16 swap places, so
//            that the two 16-lane halves of a transposed read hit different banks.
template <int W, int KIND>
__device__ __forceinline__ int swz(int r) {
  if constexpr (W == 128) return (r ^ (r << 1)) & 15;
  else if constexpr (W == 64 && KIND == 0) return 4 * ((r >> 1) & 1) + 2 * ((r & 1) ^ ((r >> 3) & 1)) + ((r >> 2) & 1);
  else if constexpr (W == 64) return r & 7;
  else return 0;
}

// physical row of logical row r (only 16-wide tiles permute rows)
template <int W>
__device__ __forceinline__ int prow(int r) {
  if constexpr (W == 16) return r ^ (((r >> 3) & 1) << 2);
  else return r;
}

// byte offset of element (r, c) of a swizzled W-column bf16 tile
template <int W, int KIND = 0>
__device__ __forceinline__ int soff(int r, int c) {
  return prow<W>(r) * (2 * W) + (((c >> 3) ^ swz<W, KIND>(r)) << 4) + ((c & 7) << 1);
}

// Fragment addresses.  Every fragment read below takes tile-aligned arguments: its
// first row r0 or column c0 is a multiple of 16, its K offset k0 a multiple of 32.
// Then the swizzle of each row a lane touches depends on the lane alone (every
// swz depends on r mod 16 only), and the aligned offsets either add whole rows or
// flip bits that the lane's own part leaves clear, so (q = lane % 16, g = lane / 16)
//   soff(r0 + q, k0 + 8g)                    = r0 2W + (rk_lane ^ 2 k0)
//   soff(k0 + 8g + q/4 (+4), c0 + 4 (q % 4)) = k0 2W + (kc_lane(0 or 4) ^ 2 c0)
// and likewise for the split K orders.  A read then costs one XOR with a
// compile-time or wave-uniform value (shared by the reads with the same one)
// instead of the swizzle arithmetic per read.  The identities hold for every tile
// width and swizzle kind here (checked exhaustively against soff on the host).
template <int W, int KIND>
__device__ __forceinline__ int rk_lane() {
  const int l = lane_id(), q = l & 15, g = l >> 4;
  return prow<W>(q) * (2 * W) + ((g ^ swz<W, KIND>(q)) << 4);
}

// transposed reads: rows 8g + q/4 + d (d = 0, 4), column piece of 4 (q % 4)
template <int W, int KIND>
__device__ __forceinline__ int kc_lane(int d) {
  const int l = lane_id(), q = l & 15, g = l >> 4;
  const int rl = 8 * g + (q >> 2) + d;
  return prow<W>(rl) * (2 * W) + 8 * (q & 1) + ((((q >> 1) & 1) ^ swz<W, KIND>(rl)) << 4);
}

// T[r0 + j][k0 + 8g .. 8g+7] (see frag_rk)
template <int W, int KIND = 0>
__device__ __forceinline__ bf16x8 frag_rk_s(const char* T, int r0, int k0) {
  return *reinterpret_cast<const bf16x8*>(T + r0 * (2 * W) + (rk_lane<W, KIND>() ^ (2 * k0)));
}

__device__ __forceinline__ bf16x8 tr_pair(const char* p0, const char* p1) {
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((lds_short*)(p0)));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((lds_short*)(p1)));
  const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo);
  const bf16x4 h4 = __builtin_bit_cast(bf16x4, hi);
  return __builtin_shufflevector(l4, h4, 0, 1, 2, 3, 4, 5, 6, 7);
}

// T[k0 + 8g .. 8g+7][c0 + j] by transposed reads (see frag_kc)
template <int W, int KIND = 0>
__device__ __forceinline__ bf16x8 frag_kc_s(const char* T, int c0, int k0) {
  const char* base = T + k0 * (2 * W);
  return tr_pair(base + (kc_lane<W, KIND>(0) ^ (2 * c0)), base + (kc_lane<W, KIND>(4) ^ (2 * c0)));
}

// T[m_e][c0 + j] with rows m_e = k0 + 4g + e (e < 4) and k0 + 16 + 4g + e - 4
// (e >= 4): the K order of an MFMA operand is free as long as both operands
// share it, and this one matches a B operand assembled from the accumulators
// of two 16-row MFMA tiles (lane group g holds rows 4g .. 4g+3 of each)
template <int W, int KIND>
__device__ __forceinline__ int kcs_lane() {
  const int l = lane_id(), q = l & 15, g = l >> 4;
  const int rl = 4 * g + (q >> 2);
  return prow<W>(rl) * (2 * W) + 8 * (q & 1) + ((((q >> 1) & 1) ^ swz<W, KIND>(rl)) << 4);
}

template <int W, int KIND = 0>
__device__ __forceinline__ bf16x8 frag_kc_split_s(const char* T, int c0, int k0) {
  const int o = kcs_lane<W, KIND>() ^ (2 * c0);
  return tr_pair(T + k0 * (2 * W) + o, T + (k0 + 16) * (2 * W) + o);
}

// T[r0 + j][m_e], m_e as in frag_kc_split_s: the row-fragment form of the same
// K order (two 8-byte reads: columns k0 + 4g and k0 + 16 + 4g)
template <int W, int KIND>
__device__ __forceinline__ int rks_lane() {
  const int l = lane_id(), q = l & 15, g = l >> 4;
  return prow<W>(q) * (2 * W) + 8 * (g & 1) + (((g >> 1) ^ swz<W, KIND>(q)) << 4);
}

template <int W, int KIND = 0>
__device__ __forceinline__ bf16x8 frag_rk_split_s(const char* T, int r0, int k0) {
  const char* base = T + r0 * (2 * W);
  const int o = rks_lane<W, KIND>();
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(base + (o ^ (2 * k0)));
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(base + (o ^ (2 * k0 + 32)));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Lane (q, g)'s four consecutive elements of row r0 + q, columns c0 + 4g .. +3
// (r0, c0 multiples of 16: an accumulator tile's layout), as bytes from the tile:
// the 8-byte pieces frag_rk_split_s reads, so the same per-lane part serves
template <int W, int KIND = 0>
__device__ __forceinline__ int quad_off(int r0, int c0) {
  return r0 * (2 * W) + (rks_lane<W, KIND>() ^ (2 * c0));
}

template <int W, int KIND = 0>
__device__ __forceinline__ void st4_q(char* T, int r0, int c0, float a, float b, float d, float e) {
  *reinterpret_cast<uint2*>(T + quad_off<W, KIND>(r0, c0)) = pack4_bf16(a, b, d, e);
}

template <int W, int KIND = 0>
__device__ __forceinline__ bf16x4 ld4_q(const char* T, int r0, int c0) {
  return *reinterpret_cast<const bf16x4*>(T + quad_off<W, KIND>(r0, c0));
}

// x - bf16(x): the low part of a two-part bf16 value
__device__ __forceinline__ float lo_part(float x) { return x - float(to_bf16(x)); }

// one 16-byte direct-to-LDS load per lane: lane l's bytes land at lds + 16 l
__device__ __forceinline__ void dma16(const void* src, char* lds) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)((lds_char_t*)lds), 16, 0, 0);
}

// a 4-byte direct-to-LDS load: used to pull a cache line into L2 ahead of time
__device__ __forceinline__ void dma4(const void* src, char* lds) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)((lds_char_t*)lds), 4, 0, 0);
}

// Workgroup barrier that orders LDS traffic only: each wave's LDS reads and
// writes complete first (lgkmcnt), while its global stores and loads stay in
// flight (a __syncthreads fence would drain them every chunk step; the movers
// wait for exactly the loads a barrier publishes).  The signal fences keep the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void chain_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt untouched
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// s_waitcnt vmcnt(N), other counters untouched
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}


// Direct-to-LDS copy of a ROWS x W bf16 tile (rows of 2W bytes) into a swizzled
// LDS tile at `dst`; row_src(row) is the global address of the row's first byte.
// The tile's 1 KB loads are dealt to NW waves: wave `iw` issues loads iw,
// iw + NW, ...  dma_piece issues the wave's load number `it` alone, so that the
// copies can be spread over compute (a wave that issues many loads back to back
// stalls until the memory pipeline takes them).
template <int W, int ROWS, int NW>
struct DmaTile {
  static constexpr int kLoads = ROWS * 2 * W / 1024;
  static_assert(kLoads % NW == 0, "loads split evenly over the issuing waves");
  static constexpr int kPerWave = kLoads / NW;
};

template <int W, int KIND, int ROWS, int NW, typename F>
__device__ __forceinline__ void dma_piece(char* dst, F row_src, int iw, int it) {
  const int i = iw + NW * it;
  const int pos = i * 1024 + 16 * lane_id();
  const int row = pos / (2 * W), lp = ((pos % (2 * W)) >> 4) ^ swz<W, KIND>(row);
  dma16(row_src(row) + 16 * lp, dst + i * 1024);
}

template <int W, int KIND, int ROWS, int NW, typename F>
__device__ __forceinline__ void dma_tile(char* dst, F row_src, int iw) {
  // the trip count is a compile-time constant, so the loop unrolls and the
  // compiler can count the loads in flight (an unknown count makes it wait for all)
#pragma unroll
  for (int it = 0; it < DmaTile<W, ROWS, NW>::kPerWave; ++it) dma_piece<W, KIND, ROWS, NW>(dst, row_src, iw, it);
}

}  // namespace gdr

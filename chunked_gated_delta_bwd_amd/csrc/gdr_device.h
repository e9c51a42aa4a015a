// Device helpers for gfx950: bf16 conversion, MFMA 16x16x32 bf16 fragments,
// LDS transpose reads, typed global loads/stores and wave reductions.
//
// MFMA v_mfma_f32_16x16x32_bf16 lane layout (wave64, lane l, g = l/16, j = l%16):
//   A operand: A[m = j][k = 8g .. 8g+7]      (8 bf16 per lane)
//   B operand: B[k = 8g .. 8g+7][n = j]
//   C/D:       C[m = 4g + i][n = j], i = 0..3 (4 fp32 per lane)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) short lds_short;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16x16x4 fp32 MFMA: lane l gives A[l%16][l/16] and B[l/16][l%16]
__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Fragment of a tile stored T[row][k] (k contiguous, pitch P elements):
// lane gets T[r0 + j][k0 + 8g .. 8g+7].  Serves as the A operand (m = row) or
// as the B operand when B[k][n] = T[n][k].
__device__ __forceinline__ bf16x8 frag_rk(const bf16* T, int P, int r0, int k0) {
  const int l = lane_id();
  return *reinterpret_cast<const bf16x8*>(T + (r0 + (l & 15)) * P + k0 + 8 * (l >> 4));
}

// Fragment of a tile stored T[k][col] (col contiguous, pitch P elements):
// lane gets T[k0 + 8g .. 8g+7][c0 + j], gathered by two ds_read_b64_tr_b16.
// Within each 16-lane group, lane i of the transposed read receives element
// i%4 of the 64-bit chunk addressed by lane 4r + i/4 (r = result slot), so lane
// q addresses row k0 + 8g + q/4, columns c0 + 4(q%4) .. +3.
__device__ __forceinline__ bf16x8 frag_kc(const bf16* T, int P, int c0, int k0) {
  const int l = lane_id();
  const int g = l >> 4, q = l & 15;
  const bf16* p0 = T + (k0 + 8 * g + (q >> 2)) * P + c0 + 4 * (q & 3);
  const bf16* p1 = p0 + 4 * P;
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((lds_short*)(p0)));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((lds_short*)(p1)));
  // whole-vector bit casts: extracting 16-bit lanes one at a time through a
  // scalar bf16 bit cast miscompiles on this toolchain (element 0 is splat)
  const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo);
  const bf16x4 h4 = __builtin_bit_cast(bf16x4, hi);
  return __builtin_shufflevector(l4, h4, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t u) { return __uint_as_float(uint32_t(u) << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (bf16)x); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Four fp32 -> four bf16 (round to nearest even) packed into 8 bytes, one packed
// conversion per pair.
__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
  uint2 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
  r.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{c, d}, bf16x2));
  return r;
}

// ---- typed token-tensor access (storage bf16 or fp32, math in fp32) ----
template <typename T> struct IO;

template <> struct IO<bf16> {
  // raw (still packed) register images, so that a prefetch keeps loads in
  // flight and unpacks only where the data is consumed
  static constexpr int kRaw8Loads = 1;   // global load instructions per Raw8
  typedef u32x4 Raw8;
  typedef unsigned int __attribute__((ext_vector_type(2))) Raw4;
  static __device__ __forceinline__ Raw8 load_raw8(const void* base, int64_t off) {
    return *reinterpret_cast<const Raw8*>(static_cast<const uint16_t*>(base) + off);
  }
  static __device__ __forceinline__ Raw4 load_raw4(const void* base, int64_t off) {
    return *reinterpret_cast<const Raw4*>(static_cast<const uint16_t*>(base) + off);
  }
  static __device__ __forceinline__ void unpack8(const Raw8& u, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(u[i] << 16);
      x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void unpack4(const Raw4& u, float (&x)[4]) {
    x[0] = __uint_as_float(u[0] << 16);
    x[1] = __uint_as_float(u[0] & 0xffff0000u);
    x[2] = __uint_as_float(u[1] << 16);
    x[3] = __uint_as_float(u[1] & 0xffff0000u);
  }
  static __device__ __forceinline__ void load8(const void* base, int64_t off, float (&x)[8]) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void load4(const void* base, int64_t off, float (&x)[4]) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + off);
    x[0] = __uint_as_float(u.x << 16);
    x[1] = __uint_as_float(u.x & 0xffff0000u);
    x[2] = __uint_as_float(u.y << 16);
    x[3] = __uint_as_float(u.y & 0xffff0000u);
  }
  static __device__ __forceinline__ float load1(const void* base, int64_t off) {
    return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[off]);
  }
  static __device__ __forceinline__ void store8(void* base, int64_t off, const float (&x)[8]) {
    uint4 u;
    const uint2 a = pack4_bf16(x[0], x[1], x[2], x[3]);
    const uint2 b = pack4_bf16(x[4], x[5], x[6], x[7]);
    u.x = a.x; u.y = a.y; u.z = b.x; u.w = b.y;
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off) = u;
  }
  static __device__ __forceinline__ void store4(void* base, int64_t off, float a, float b, float c, float d) {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + off) = pack4_bf16(a, b, c, d);
  }
  static __device__ __forceinline__ void store1(void* base, int64_t off, float x) {
    static_cast<uint16_t*>(base)[off] = f32_to_bf16_bits(x);
  }
};

template <> struct IO<float> {
  static constexpr int kRaw8Loads = 2;
  struct Raw8 { f32x4 a, b; };
  typedef f32x4 Raw4;
  static __device__ __forceinline__ Raw8 load_raw8(const void* base, int64_t off) {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + off);
    return Raw8{p[0], p[1]};
  }
  static __device__ __forceinline__ Raw4 load_raw4(const void* base, int64_t off) {
    return *reinterpret_cast<const Raw4*>(static_cast<const float*>(base) + off);
  }
  static __device__ __forceinline__ void unpack8(const Raw8& u, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = u.a[i];
      x[4 + i] = u.b[i];
    }
  }
  static __device__ __forceinline__ void unpack4(const Raw4& u, float (&x)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = u[i];
  }
  static __device__ __forceinline__ void load8(const void* base, int64_t off, float (&x)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  static __device__ __forceinline__ void load4(const void* base, int64_t off, float (&x)[4]) {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  }
  static __device__ __forceinline__ float load1(const void* base, int64_t off) {
    return static_cast<const float*>(base)[off];
  }
  static __device__ __forceinline__ void store8(void* base, int64_t off, const float (&x)[8]) {
    float* p = static_cast<float*>(base) + off;
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
  }
  static __device__ __forceinline__ void store4(void* base, int64_t off, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(static_cast<float*>(base) + off) = make_float4(a, b, c, d);
  }
  static __device__ __forceinline__ void store1(void* base, int64_t off, float x) {
    static_cast<float*>(base)[off] = x;
  }
};

// Sum over groups of `width` consecutive lanes (width a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = WIDTH / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// lane exchange inside the 16-lane DPP rows of a wave
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// sum over the 16 lanes 16k .. 16k+15 of a wave, returned to all of them (DPP
// row rotations by 8 and 4, then two quad permutations; no LDS traffic)
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<0x128>(x);   // row_ror:8
  x += dpp_f<0x124>(x);   // row_ror:4
  x += dpp_f<0x4E>(x);    // quad_perm [2, 3, 0, 1]
  x += dpp_f<0xB1>(x);    // quad_perm [1, 0, 3, 2]
  return x;
}

// sum over aligned groups of W lanes (W = 16: the DPP row; W = 8: half rows,
// by a mirror within each half and two quad permutations), on every lane
template <int W>
__device__ __forceinline__ float group_sum_dpp(float x) {
  static_assert(W == 16 || W == 8, "DPP group width");
  if constexpr (W == 16) {
    return row16_sum(x);
  } else {
    x += dpp_f<0x141>(x);   // row_half_mirror
    x += dpp_f<0x4E>(x);    // quad_perm [2, 3, 0, 1]
    x += dpp_f<0xB1>(x);    // quad_perm [1, 0, 3, 2]
    return x;
  }
}

// x + (x of lane l ^ 16): v_permlane16_swap exchanges the odd 16-lane rows of
// one register with the even rows of another; on two copies of x the two
// registers then hold both rows of each pair, and their sum is the same on both.
// (Inline assembly: the compiler builtin returns its first result twice.  The
// compiler does not pad inline assembly for hazards: a VALU write of an operand
// needs two wait states before the swap, a v_cmpx write of EXEC four; the
// trailing nop separates the swap from the VALU that reads its results.)
#define GDR_SWAP_ASM(op) "s_nop 4\n\t" op " %0, %1\n\ts_nop 1"
__device__ __forceinline__ float pair16_sum(float x) {
  float a = x, b = x;
  asm volatile(GDR_SWAP_ASM("v_permlane16_swap_b32") : "+v"(a), "+v"(b));
  return a + b;
}
// x + (x of lane l ^ 32), by the same exchange of the two 32-lane halves
__device__ __forceinline__ float pair32_sum(float x) {
  float a = x, b = x;
  asm volatile(GDR_SWAP_ASM("v_permlane32_swap_b32") : "+v"(a), "+v"(b));
  return a + b;
}
// sum over lanes l, l^16, l^32, l^48 (the four 16-lane rows), on every lane
__device__ __forceinline__ float xrow_sum(float x) { return pair32_sum(pair16_sum(x)); }
// sum over the whole wave, on every lane (no LDS traffic)
__device__ __forceinline__ float wave_sum(float x) { return xrow_sum(row16_sum(x)); }

// ---- tile geometry shared by the kernels ----
constexpr int C = 64;       // tokens per chunk
constexpr int PC = C + 8;   // LDS pitch of 64-wide bf16 tiles (elements)

template <int D>
struct Dims {
  static constexpr int PD = D + 8;             // LDS pitch of D-wide bf16 tiles
  static constexpr int TPR = D / 8;            // threads per row in row sweeps (8 elements each)
  static constexpr int RPP = 256 / TPR;        // rows per pass for 256 threads
  static constexpr int NPASS = C / RPP;        // passes over the 64 rows
  static constexpr int NJB = D / 16;           // 16-wide blocks along D
  static constexpr int NJW = NJB / 4;          // D-blocks per compute wave in the chain kernels
};

__device__ __forceinline__ int64_t tok(int t, int H, int h) { return int64_t(t) * H + h; }
// token row of the q, k tensors for value head h: with grouped heads q and k have
// Hk heads, value head h reading key head h / (H / Hk) (P is the kernels' Params)
template <typename P>
__device__ __forceinline__ int64_t qk_tok(const P& p, int t, int h) { return int64_t(t) * p.Hk + h / p.G; }

// (chunk, value head) of a per-(chunk, head) workgroup on an NC x H grid.  With
// grouped heads the G value heads of a key head read the same q, k rows, so their
// workgroups for one chunk are dealt to one XCD back to back (workgroups go
// round-robin over the 8 XCDs: ids j 8G + 8 i + x, i < G, all land on XCD x), where
// that XCD's L2 serves the rows after the first read.  A bijection of the grid:
// the (chunk, key head) pairs past the last whole set of eight keep their members
// consecutive.
// chunk_head_at: the same for the workgroup with linear id L (x fastest).
template <typename P>
__device__ __forceinline__ void chunk_head_at(const P& p, int L, int& c, int& h) {
  if (p.G == 1) {
    c = L % p.NC;
    h = L / p.NC;
    return;
  }
  const int G = p.G;
  const int npair = p.NC * p.Hk, p8 = npair / 8 * 8;
  int pair, gi;
  if (L < p8 * G) {
    const int j = L / (8 * G), r = L % (8 * G);
    pair = 8 * j + r % 8;
    gi = r / 8;
  } else {
    const int rem = L - p8 * G;
    pair = p8 + rem / G;
    gi = rem % G;
  }
  c = pair / p.Hk;
  h = (pair % p.Hk) * G + gi;
}

template <typename P>
__device__ __forceinline__ void chunk_head(const P& p, int& c, int& h) {
  if (p.G == 1) {
    c = blockIdx.x;
    h = blockIdx.y;
    return;
  }
  chunk_head_at(p, int(blockIdx.x + p.NC * blockIdx.y), c, h);
}

__device__ __forceinline__ void st_bf16x4(bf16* dst, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(dst) = pack4_bf16(a, b, c, d);
}
__device__ __forceinline__ void st_bf16x4(uint16_t* dst, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(dst) = pack4_bf16(a, b, c, d);
}

__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }
// 2^x on the hardware exponential alone (fast_exp(x) is this of x log2(e)): for
// exponents kept in base-2 units, which saves the multiply per factor
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float sigmoidf(float x) { return 1.0f / (1.0f + __expf(-x)); }
// softplus(x) = max(x, 0) + log(1 + exp(-|x|)), stable for every x.  The
// argument of the log lies in (1, 2], where the hardware log is accurate; rounding
// 1 + e for tiny e costs at most 2^-24 absolute, far below the bf16 data.
__device__ __forceinline__ float softplusf(float x) { return fmaxf(x, 0.0f) + __logf(1.0f + __expf(-fabsf(x))); }

}  // namespace gdr

// k_chain: the two serial chunk recursions of the chunked gated delta rule.
//
//   forward state pass      U = U' - W S_n^T,  S_{n+1} = S_n Diag(e^GamC) + U^T Khat
//   reverse state gradient  dU = P^T dO + Khat dS_{n+1}^T,
//                           dS_n = dS_{n+1} Diag(e^GamC) + Qbar^T dO - W^T dU
//
// (the second is the recursion the FlashQLA overview describes, running strictly
// from the last chunk to the first, dh <- g_last dh + R^T dO + X^T Y with
// X = A_beta K).  One workgroup per (sequence, head, 16-wide V slice) and
// direction; neither recursion depends on the other, so the fused entry point
// runs both in one grid.  The fp32 state / state gradient of a slice lives in
// registers for the whole sequence.
//
// Workgroups are 512 threads: waves 0-3 compute, waves 4-7 load and stage the
// chunk tiles ("producers"), so the compute waves never wait on global loads.
// Every chunk step has two barriers, B1 and B2.  A tile is written in the window
// where no compute wave reads it, so the large tiles need one LDS buffer each:
//   reverse: Khat, P (read in the first window) are staged after B2 of the
//            previous step; Qbar (hi + lo) and W (read after B2) are staged
//            between B1 and B2 of their own step; dO is double-buffered.
//   forward: W and U' (first window) after B2 of the previous step; Khat and
//            the decay (second window) between B1 and B2.
// Producers keep two register sets of raw prefetched chunk data (chunk k in set
// k % 2) and issue every load unconditionally (clamped to the last chunk), so the
// compiler never has to wait for a load before its data is staged.
//
// Qbar^T dO carries the dominant part of dh0, so Qbar is split into bf16 high and
// low parts (two MFMAs); for fp32 inputs dO is split too.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

constexpr int kChainThreads = 512;
constexpr int kChainCompute = 256;   // threads of the compute waves (0-3)

template <int D>
struct ChainLayout {
  static constexpr int PD = D + 8, PO = 24;
  // reverse role, bf16 element offsets
  static constexpr int bKh = 0;
  static constexpr int bP = bKh + C * PD;
  static constexpr int bQh = bP + C * PC;
  static constexpr int bQl = bQh + C * PD;
  static constexpr int bW = bQl + C * PD;
  static constexpr int bdOh = bW + C * PD;     // two buffers
  static constexpr int bdOl = bdOh + 2 * C * PO;  // two buffers
  static constexpr int bdS = bdOl + 2 * C * PO;
  static constexpr int bdU = bdS + 16 * PD;
  static constexpr int bEnd = bdU + 16 * PC;   // then 2 x D fp32 decay values
  static constexpr size_t bBytes = size_t(bEnd) * 2 + 2 * D * 4;
  // forward role
  static constexpr int fW = 0;
  static constexpr int fKh = fW + C * PD;
  static constexpr int fUq = fKh + C * PD;     // U' slice as [v][r]
  static constexpr int fS = fUq + 16 * PC;
  static constexpr int fU = fS + 16 * PD;
  static constexpr int fEnd = fU + 16 * PC;    // then D fp32 decay values
  static constexpr size_t fBytes = size_t(fEnd) * 2 + D * 4;
  static constexpr size_t bytes = bBytes > fBytes ? bBytes : fBytes;
};

// ---------------------------------------------------------------------------
// producer register sets
// ---------------------------------------------------------------------------
template <int D, typename TIO, int GATE>
struct FwdSet {
  using Dm = Dims<D>;
  u32x4 w[Dm::NPASS];
  typename IO<TIO>::Raw8 k[Dm::NPASS];   // scalar gate: raw k (Khat formed at the stash)
  u32x4 kh[Dm::NPASS];                   // per-channel gate: Khat tile from the prologue kernel
  float rk[Dm::NPASS], g[Dm::NPASS], m[Dm::NPASS], gC;
  f32x4 gCv[2];                          // per-channel gate: GamC of this thread's 8 columns
  uint2 up;                              // U' slice: 4 values of one row
};

template <int D, typename TIO, int GATE>
struct BwdSet {
  using Dm = Dims<D>;
  u32x4 w[Dm::NPASS], pm[2];
  typename IO<TIO>::Raw8 k[Dm::NPASS], q[Dm::NPASS];   // scalar gate
  u32x4 kh[Dm::NPASS], qh[Dm::NPASS], ql[Dm::NPASS];   // per-channel gate
  float rk[Dm::NPASS], rq[Dm::NPASS], g[Dm::NPASS], m[Dm::NPASS], gC;
  f32x4 gCv[2];
  typename IO<TIO>::Raw4 dO;
  float m_do;
};

struct ChunkGeo {
  int64_t ch;   // chunk-head index
  int t0, len;  // first token, valid rows
};

__device__ __forceinline__ ChunkGeo geo(const Params& p, const SeqEntry& se, int h, int c) {
  ChunkGeo r;
  r.ch = int64_t(h) * p.NC + c;
  r.t0 = se.t_start + (c - se.c0) * C;
  r.len = min(C, se.len - (c - se.c0) * C);
  return r;
}

// ---- forward role ----
template <int D, typename TIO, int GATE>
__device__ __forceinline__ void fwd_load(FwdSet<D, TIO, GATE>& f, const Params& p, const SeqEntry& se, int h,
                                         int v0, int c, int pt) {
  using Dm = Dims<D>;
  const ChunkGeo cg = geo(p, se, h, c);
#pragma unroll
  for (int ps = 0; ps < Dm::NPASS; ++ps) {
    const int r = ps * Dm::RPP + pt / Dm::TPR, c0 = (pt % Dm::TPR) * 8;
    f.w[ps] = *reinterpret_cast<const u32x4*>(p.W + (cg.ch * C + r) * D + c0);
    if constexpr (GATE == 0) {
      f.k[ps] = IO<TIO>::load_raw8(p.k, tok(cg.t0 + min(r, cg.len - 1), p.H, h) * D + c0);
      f.m[ps] = r < cg.len ? 1.f : 0.f;
      f.rk[ps] = p.rho[cg.ch * 2 * C + C + r];
      f.g[ps] = p.gam[cg.ch * C + r];
    } else {
      f.kh[ps] = *reinterpret_cast<const u32x4*>(p.Kh + (cg.ch * C + r) * D + c0);
    }
  }
  const int c0 = (pt % Dm::TPR) * 8;
  if constexpr (GATE == 0) {
    f.gC = p.gam[cg.ch * C + C - 1];
  } else {
    const f32x4* gc = reinterpret_cast<const f32x4*>(p.gam + (cg.ch * C + C - 1) * D + c0);
    f.gCv[0] = gc[0];
    f.gCv[1] = gc[1];
  }
  const int r = pt / 4, cc = (pt % 4) * 4;
  f.up = *reinterpret_cast<const uint2*>(p.Up + (cg.ch * C + r) * D + v0 + cc);
}

// window before B1 (after B2 of the previous step): W and U' of the chunk
template <int D, typename TIO, int GATE>
__device__ __forceinline__ void fwd_stash_w(const FwdSet<D, TIO, GATE>& f, bf16* L, int pt) {
  using Dm = Dims<D>;
  using Ly = ChainLayout<D>;
  constexpr int PD = Dm::PD;
#pragma unroll
  for (int ps = 0; ps < Dm::NPASS; ++ps) {
    const int r = ps * Dm::RPP + pt / Dm::TPR, c0 = (pt % Dm::TPR) * 8;
    *reinterpret_cast<u32x4*>(L + Ly::fW + r * PD + c0) = f.w[ps];
  }
  const int r = pt / 4, cc = (pt % 4) * 4;
  uint16_t* uq = reinterpret_cast<uint16_t*>(L + Ly::fUq);
  uq[(cc + 0) * PC + r] = uint16_t(f.up.x & 0xffffu);
  uq[(cc + 1) * PC + r] = uint16_t(f.up.x >> 16);
  uq[(cc + 2) * PC + r] = uint16_t(f.up.y & 0xffffu);
  uq[(cc + 3) * PC + r] = uint16_t(f.up.y >> 16);
}

// window between B1 and B2: Khat and the per-column decay of the chunk
template <int D, typename TIO, int GATE>
__device__ __forceinline__ void fwd_stash_k(const FwdSet<D, TIO, GATE>& f, bf16* L, float* dec, int pt) {
  using Dm = Dims<D>;
  using Ly = ChainLayout<D>;
  constexpr int PD = Dm::PD;
#pragma unroll
  for (int ps = 0; ps < Dm::NPASS; ++ps) {
    const int r = ps * Dm::RPP + pt / Dm::TPR, c0 = (pt % Dm::TPR) * 8;
    if constexpr (GATE == 0) {
      const float s = f.m[ps] * f.rk[ps] * fast_exp(f.gC - f.g[ps]);
      float kx[8];
      IO<TIO>::unpack8(f.k[ps], kx);
      bf16x8 kb;
#pragma unroll
      for (int e = 0; e < 8; ++e) kb[e] = to_bf16(kx[e] * s);
      *reinterpret_cast<bf16x8*>(L + Ly::fKh + r * PD + c0) = kb;
    } else {
      *reinterpret_cast<u32x4*>(L + Ly::fKh + r * PD + c0) = f.kh[ps];
    }
  }
  if (pt < Dm::TPR) {
    const int c0 = pt * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) dec[c0 + e] = fast_exp(GATE == 0 ? f.gC : f.gCv[e / 4][e % 4]);
  }
}

// ---- reverse role ----
template <int D, typename TIO, int GATE>
__device__ __forceinline__ void bwd_load(BwdSet<D, TIO, GATE>& f, const Params& p, const SeqEntry& se, int h,
                                         int v0, int c, int pt) {
  using Dm = Dims<D>;
  const ChunkGeo cg = geo(p, se, h, c);
#pragma unroll
  for (int ps = 0; ps < Dm::NPASS; ++ps) {
    const int r = ps * Dm::RPP + pt / Dm::TPR, c0 = (pt % Dm::TPR) * 8;
    f.w[ps] = *reinterpret_cast<const u32x4*>(p.W + (cg.ch * C + r) * D + c0);
    if constexpr (GATE == 0) {
      const int64_t o = tok(cg.t0 + min(r, cg.len - 1), p.H, h) * D + c0;
      f.k[ps] = IO<TIO>::load_raw8(p.k, o);
      f.q[ps] = IO<TIO>::load_raw8(p.q, o);
      f.m[ps] = r < cg.len ? 1.f : 0.f;
      f.rk[ps] = p.rho[cg.ch * 2 * C + C + r];
      f.rq[ps] = p.rho[cg.ch * 2 * C + r];
      f.g[ps] = p.gam[cg.ch * C + r];
    } else {
      const int64_t o = (cg.ch * C + r) * D + c0;
      f.kh[ps] = *reinterpret_cast<const u32x4*>(p.Kh + o);
      f.qh[ps] = *reinterpret_cast<const u32x4*>(p.Qh + o);
      f.ql[ps] = *reinterpret_cast<const u32x4*>(p.Ql + o);
    }
  }
  const int c0 = (pt % Dm::TPR) * 8;
  if constexpr (GATE == 0) {
    f.gC = p.gam[cg.ch * C + C - 1];
  } else {
    const f32x4* gc = reinterpret_cast<const f32x4*>(p.gam + (cg.ch * C + C - 1) * D + c0);
    f.gCv[0] = gc[0];
    f.gCv[1] = gc[1];
  }
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int pc = pt + x * 256;   // 16-byte piece of the 64x64 P tile
    f.pm[x] = *reinterpret_cast<const u32x4*>(p.P + (cg.ch * C + pc / 8) * C + (pc % 8) * 8);
  }
  const int r = pt / 4, cc = (pt % 4) * 4;
  f.dO = IO<TIO>::load_raw4(p.dO, tok(cg.t0 + min(r, cg.len - 1), p.H, h) * D + v0 + cc);
  f.m_do = r < cg.len ? 1.f : 0.f;
}

// window between B1 and B2: Qbar (hi + lo) and W of the chunk
template <int D, typename TIO, int GATE>
__device__ __forceinline__ void bwd_stash_q(const BwdSet<D, TIO, GATE>& f, bf16* L, float scale, int pt) {
  using Dm = Dims<D>;
  using Ly = ChainLayout<D>;
  constexpr int PD = Dm::PD;
#pragma unroll
  for (int ps = 0; ps < Dm::NPASS; ++ps) {
    const int r = ps * Dm::RPP + pt / Dm::TPR, c0 = (pt % Dm::TPR) * 8;
    *reinterpret_cast<u32x4*>(L + Ly::bW + r * PD + c0) = f.w[ps];
    if constexpr (GATE == 0) {
      const float s = f.m[ps] * scale * f.rq[ps] * fast_exp(f.g[ps]);
      float qx[8];
      IO<TIO>::unpack8(f.q[ps], qx);
      bf16x8 qh, ql;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = qx[e] * s;
        qh[e] = to_bf16(x);
        ql[e] = to_bf16(x - float(qh[e]));
      }
      *reinterpret_cast<bf16x8*>(L + Ly::bQh + r * PD + c0) = qh;
      *reinterpret_cast<bf16x8*>(L + Ly::bQl + r * PD + c0) = ql;
    } else {
      *reinterpret_cast<u32x4*>(L + Ly::bQh + r * PD + c0) = f.qh[ps];
      *reinterpret_cast<u32x4*>(L + Ly::bQl + r * PD + c0) = f.ql[ps];
    }
  }
}

// window after B2: Khat, P, dO (buffer `buf`) and the decay (buffer `buf`) of the chunk
template <int D, typename TIO, int GATE>
__device__ __forceinline__ void bwd_stash_k(const BwdSet<D, TIO, GATE>& f, bf16* L, float* dec, int buf, int pt) {
  using Dm = Dims<D>;
  using Ly = ChainLayout<D>;
  constexpr int PD = Dm::PD, PO = Ly::PO;
#pragma unroll
  for (int ps = 0; ps < Dm::NPASS; ++ps) {
    const int r = ps * Dm::RPP + pt / Dm::TPR, c0 = (pt % Dm::TPR) * 8;
    if constexpr (GATE == 0) {
      const float s = f.m[ps] * f.rk[ps] * fast_exp(f.gC - f.g[ps]);
      float kx[8];
      IO<TIO>::unpack8(f.k[ps], kx);
      bf16x8 kb;
#pragma unroll
      for (int e = 0; e < 8; ++e) kb[e] = to_bf16(kx[e] * s);
      *reinterpret_cast<bf16x8*>(L + Ly::bKh + r * PD + c0) = kb;
    } else {
      *reinterpret_cast<u32x4*>(L + Ly::bKh + r * PD + c0) = f.kh[ps];
    }
  }
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int pc = pt + x * 256;
    *reinterpret_cast<u32x4*>(L + Ly::bP + (pc / 8) * PC + (pc % 8) * 8) = f.pm[x];
  }
  const int r = pt / 4, cc = (pt % 4) * 4;
  float dx[4], hi[4], lo[4];
  IO<TIO>::unpack4(f.dO, dx);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    dx[e] *= f.m_do;
    hi[e] = float(to_bf16(dx[e]));
    lo[e] = dx[e] - hi[e];   // zero for bf16 inputs
  }
  st_bf16x4(L + Ly::bdOh + buf * C * PO + r * PO + cc, hi[0], hi[1], hi[2], hi[3]);
  st_bf16x4(L + Ly::bdOl + buf * C * PO + r * PO + cc, lo[0], lo[1], lo[2], lo[3]);
  if (pt < Dm::TPR) {
    const int c0 = pt * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) dec[buf * D + c0 + e] = fast_exp(GATE == 0 ? f.gC : f.gCv[e / 4][e % 4]);
  }
}

// ---------------------------------------------------------------------------
// the two roles
// ---------------------------------------------------------------------------
template <int D, typename TIO, int GATE>
__device__ __forceinline__ void chain_fwd(const Params& p, char* smem, int si, int h, int sl) {
  using Dm = Dims<D>;
  using Ly = ChainLayout<D>;
  constexpr int PD = Dm::PD, NJW = Dm::NJW;
  bf16* const L = reinterpret_cast<bf16*>(smem);
  float* const dec = reinterpret_cast<float*>(smem + size_t(Ly::fEnd) * 2);
  const bf16* Wl = L + Ly::fW;
  const bf16* Khl = L + Ly::fKh;
  const bf16* Uq = L + Ly::fUq;
  bf16* Ss = L + Ly::fS;
  bf16* Ut = L + Ly::fU;

  const int tid = threadIdx.x;
  const bool compute = tid < kChainCompute;
  const int pt = tid - kChainCompute;   // producer thread index (valid when !compute)
  const int l = lane_id(), w = wave_id();
  const int g = l >> 4, jj = l & 15;
  const SeqEntry se = p.stab[si];
  const int v0 = 16 * sl;
  const int nck = se.nchunks;

  f32x4 acc[NJW];
#pragma unroll
  for (int x = 0; x < NJW; ++x) acc[x] = zero4();
  if (compute && p.h0) {
#pragma unroll
    for (int x = 0; x < NJW; ++x) {
      const int j = 16 * (w * NJW + x) + 4 * g;
      const float4 t = *reinterpret_cast<const float4*>(p.h0 + ((int64_t(se.seq) * p.H + h) * D + v0 + jj) * D + j);
      acc[x] = f32x4{t.x, t.y, t.z, t.w};
    }
  }

  // The two roles run separate loops (live ranges do not overlap); each executes
  // exactly two workgroup barriers per chunk step.
  if (compute) {
    for (int k = 0; k < nck; ++k) {
      const int64_t ch = int64_t(h) * p.NC + se.c0 + k;
#pragma unroll
      for (int x = 0; x < NJW; ++x) {
        const int j = 16 * (w * NJW + x) + 4 * g;
        st_bf16x4(Ss + jj * PD + j, acc[x][0], acc[x][1], acc[x][2], acc[x][3]);
        st_bf16x4(p.S + (ch * D + v0 + jj) * D + j, acc[x][0], acc[x][1], acc[x][2], acc[x][3]);
      }
      __syncthreads();   // B1
      // U = U' - W S^T, rows 16w.., columns of this slice
      f32x4 au = zero4();
#pragma unroll
      for (int k0 = 0; k0 < D; k0 += 32) au = mma(frag_rk(Wl, PD, 16 * w, k0), frag_rk(Ss, PD, 0, k0), au);
      const uint2 up = *reinterpret_cast<const uint2*>(Uq + jj * PC + 16 * w + 4 * g);
      float u[4];
      u[0] = __uint_as_float(up.x << 16) - au[0];
      u[1] = __uint_as_float(up.x & 0xffff0000u) - au[1];
      u[2] = __uint_as_float(up.y << 16) - au[2];
      u[3] = __uint_as_float(up.y & 0xffff0000u) - au[3];
#pragma unroll
      for (int i = 0; i < 4; ++i) p.U[(ch * C + 16 * w + 4 * g + i) * D + v0 + jj] = f32_to_bf16_bits(u[i]);
      st_bf16x4(Ut + jj * PC + 16 * w + 4 * g, u[0], u[1], u[2], u[3]);
      __syncthreads();   // B2
      // S_{k+1}^T = S_k^T Diag(e^GamC) + Khat^T U
#pragma unroll
      for (int x = 0; x < NJW; ++x) {
        const int jb = w * NJW + x;
        const float4 d = *reinterpret_cast<const float4*>(dec + 16 * jb + 4 * g);
        f32x4 a = acc[x] * f32x4{d.x, d.y, d.z, d.w};
#pragma unroll
        for (int k0 = 0; k0 < C; k0 += 32) a = mma(frag_kc(Khl, PD, 16 * jb, k0), frag_rk(Ut, PC, 0, k0), a);
        acc[x] = a;
      }
    }
  } else if (nck > 0) {
    // three register sets: chunk k lives in set k % 3 from its load (step k - 3)
    // until its last stash (step k), so every load has two steps to arrive
    FwdSet<D, TIO, GATE> s0, s1, s2;
    auto step = [&](int k, FwdSet<D, TIO, GATE>& cur, FwdSet<D, TIO, GATE>& nxt) __attribute__((always_inline)) {
      __syncthreads();   // B1
      fwd_stash_k<D, TIO, GATE>(cur, L, dec, pt);
      __syncthreads();   // B2
      if (k + 1 < nck) fwd_stash_w<D, TIO, GATE>(nxt, L, pt);
      fwd_load<D, TIO, GATE>(cur, p, se, h, v0, se.c0 + min(k + 3, nck - 1), pt);
    };
    fwd_load<D, TIO, GATE>(s0, p, se, h, v0, se.c0, pt);
    fwd_load<D, TIO, GATE>(s1, p, se, h, v0, se.c0 + min(1, nck - 1), pt);
    fwd_load<D, TIO, GATE>(s2, p, se, h, v0, se.c0 + min(2, nck - 1), pt);
    fwd_stash_w<D, TIO, GATE>(s0, L, pt);
    for (int k = 0; k < nck; k += 3) {
      step(k, s0, s1);
      if (k + 1 < nck) step(k + 1, s1, s2);
      if (k + 2 < nck) step(k + 2, s2, s0);
    }
  }
  if (compute && p.ht) {
#pragma unroll
    for (int x = 0; x < NJW; ++x) {
      const int j = 16 * (w * NJW + x) + 4 * g;
      *reinterpret_cast<float4*>(p.ht + ((int64_t(se.seq) * p.H + h) * D + v0 + jj) * D + j) =
          make_float4(acc[x][0], acc[x][1], acc[x][2], acc[x][3]);
    }
  }
}

template <int D, typename TIO, int GATE>
__device__ __forceinline__ void chain_bwd(const Params& p, char* smem, int si, int h, int sl) {
  using Dm = Dims<D>;
  using Ly = ChainLayout<D>;
  constexpr int PD = Dm::PD, NJW = Dm::NJW, PO = Ly::PO;
  constexpr bool kLo = std::is_same<TIO, float>::value;   // fp32 dO is not exact in bf16
  bf16* const L = reinterpret_cast<bf16*>(smem);
  float* const dec = reinterpret_cast<float*>(smem + size_t(Ly::bEnd) * 2);
  const bf16* Khl = L + Ly::bKh;
  const bf16* Pl = L + Ly::bP;
  const bf16* Qhl = L + Ly::bQh;
  const bf16* Qll = L + Ly::bQl;
  const bf16* Wl = L + Ly::bW;
  bf16* dSl = L + Ly::bdS;
  bf16* dUt = L + Ly::bdU;

  const int tid = threadIdx.x;
  const bool compute = tid < kChainCompute;
  const int pt = tid - kChainCompute;
  const int l = lane_id(), w = wave_id();
  const int g = l >> 4, jj = l & 15;
  const SeqEntry se = p.stab[si];
  const int v0 = 16 * sl;
  const int nck = se.nchunks;
  const float scale = p.scale;

  f32x4 acc[NJW];
#pragma unroll
  for (int x = 0; x < NJW; ++x) acc[x] = zero4();
  if (compute && p.dht) {
#pragma unroll
    for (int x = 0; x < NJW; ++x) {
      const int j = 16 * (w * NJW + x) + 4 * g;
      const float4 t = *reinterpret_cast<const float4*>(p.dht + ((int64_t(se.seq) * p.H + h) * D + v0 + jj) * D + j);
      acc[x] = f32x4{t.x, t.y, t.z, t.w};
    }
  }

  // step k walks chunk c0 + nck - 1 - k (last to first); the two roles run
  // separate loops, each with exactly two workgroup barriers per step
  auto chunk_of = [&](int k) { return se.c0 + nck - 1 - min(k, nck - 1); };
  if (compute) {
    for (int k = 0; k < nck; ++k) {
      const int buf = k & 1;
      const int64_t ch = int64_t(h) * p.NC + chunk_of(k);
      const bf16* dOh = L + Ly::bdOh + buf * C * PO;
      const bf16* dOl = L + Ly::bdOl + buf * C * PO;
#pragma unroll
      for (int x = 0; x < NJW; ++x) {
        const int j = 16 * (w * NJW + x) + 4 * g;
        st_bf16x4(dSl + jj * PD + j, acc[x][0], acc[x][1], acc[x][2], acc[x][3]);
        st_bf16x4(p.dS + (ch * D + v0 + jj) * D + j, acc[x][0], acc[x][1], acc[x][2], acc[x][3]);
      }
      __syncthreads();   // B1
      // dU = P^T dO + Khat dS^T, rows 16w.., columns of this slice
      f32x4 ad = zero4();
#pragma unroll
      for (int k0 = 0; k0 < C; k0 += 32) {
        const bf16x8 pa = frag_kc(Pl, PC, 16 * w, k0);
        ad = mma(pa, frag_kc(dOh, PO, 0, k0), ad);
        if constexpr (kLo) ad = mma(pa, frag_kc(dOl, PO, 0, k0), ad);
      }
#pragma unroll
      for (int k0 = 0; k0 < D; k0 += 32) ad = mma(frag_rk(Khl, PD, 16 * w, k0), frag_rk(dSl, PD, 0, k0), ad);
#pragma unroll
      for (int i = 0; i < 4; ++i) p.dU[(ch * C + 16 * w + 4 * g + i) * D + v0 + jj] = f32_to_bf16_bits(ad[i]);
      st_bf16x4(dUt + jj * PC + 16 * w + 4 * g, -ad[0], -ad[1], -ad[2], -ad[3]);
      __syncthreads();   // B2
      // dS_n^T = dS_{n+1}^T Diag(e^GamC) + Qbar^T dO - W^T dU
#pragma unroll
      for (int x = 0; x < NJW; ++x) {
        const int jb = w * NJW + x;
        const float4 d = *reinterpret_cast<const float4*>(dec + buf * D + 16 * jb + 4 * g);
        f32x4 a = acc[x] * f32x4{d.x, d.y, d.z, d.w};
#pragma unroll
        for (int k0 = 0; k0 < C; k0 += 32) {
          const bf16x8 qh = frag_kc(Qhl, PD, 16 * jb, k0);
          const bf16x8 bh = frag_kc(dOh, PO, 0, k0);
          a = mma(qh, bh, a);
          a = mma(frag_kc(Qll, PD, 16 * jb, k0), bh, a);
          if constexpr (kLo) a = mma(qh, frag_kc(dOl, PO, 0, k0), a);
          a = mma(frag_kc(Wl, PD, 16 * jb, k0), frag_rk(dUt, PC, 0, k0), a);
        }
        acc[x] = a;
      }
    }
  } else if (nck > 0) {
    // three register sets: chunk k lives in set k % 3 from its load (step k - 3)
    // until its last stash (step k), so every load has two steps to arrive
    BwdSet<D, TIO, GATE> s0, s1, s2;
    auto step = [&](int k, BwdSet<D, TIO, GATE>& cur, BwdSet<D, TIO, GATE>& nxt) __attribute__((always_inline)) {
      __syncthreads();   // B1
      bwd_stash_q<D, TIO, GATE>(cur, L, scale, pt);
      __syncthreads();   // B2
      if (k + 1 < nck) bwd_stash_k<D, TIO, GATE>(nxt, L, dec, (k + 1) & 1, pt);
      bwd_load<D, TIO, GATE>(cur, p, se, h, v0, chunk_of(k + 3), pt);
    };
    bwd_load<D, TIO, GATE>(s0, p, se, h, v0, chunk_of(0), pt);
    bwd_load<D, TIO, GATE>(s1, p, se, h, v0, chunk_of(1), pt);
    bwd_load<D, TIO, GATE>(s2, p, se, h, v0, chunk_of(2), pt);
    bwd_stash_k<D, TIO, GATE>(s0, L, dec, 0, pt);
    for (int k = 0; k < nck; k += 3) {
      step(k, s0, s1);
      if (k + 1 < nck) step(k + 1, s1, s2);
      if (k + 2 < nck) step(k + 2, s2, s0);
    }
  }
  if (compute && p.dh0) {
#pragma unroll
    for (int x = 0; x < NJW; ++x) {
      const int j = 16 * (w * NJW + x) + 4 * g;
      *reinterpret_cast<float4*>(p.dh0 + ((int64_t(se.seq) * p.H + h) * D + v0 + jj) * D + j) =
          make_float4(acc[x][0], acc[x][1], acc[x][2], acc[x][3]);
    }
  }
}

// blockIdx -> (one (sequence, head), V slice): the slices of one (sequence, head)
// share its chunk tiles, so they are placed on the same XCD (workgroups are
// dealt round-robin over the 8 XCDs).
template <int D, typename TIO, int GATE>
__global__ __launch_bounds__(kChainThreads) void k_chain(const Params p, int mode, int nb_role) {
  __shared__ __attribute__((aligned(16))) char smem[ChainLayout<D>::bytes];
  int b = blockIdx.x;
  int role;
  if (mode == kChainBoth) {
    role = b < nb_role ? 0 : 1;
    if (role) b -= nb_role;
  } else {
    role = mode == kChainFwd ? 0 : 1;
  }
  constexpr int ns = D / 16;
  const int xcd = b % 8, y = b / 8;
  const int sl = y % ns;
  const int gidx = (y / ns) * 8 + xcd;
  if (gidx >= p.N * p.H) return;
  const int si = gidx / p.H, h = gidx % p.H;
  if (role == 0)
    chain_fwd<D, TIO, GATE>(p, smem, si, h, sl);
  else
    chain_bwd<D, TIO, GATE>(p, smem, si, h, sl);
}

namespace {
template <int D, typename TIO, int GATE>
void run_chain(const Params& p, int mode, hipStream_t s) {
  constexpr int ns = D / 16;
  const int groups = p.N * p.H;
  const int nb = ((groups + 7) / 8) * 8 * ns;
  const int nroles = mode == kChainBoth ? 2 : 1;
  k_chain<D, TIO, GATE><<<dim3(nb * nroles), kChainThreads, 0, s>>>(p, mode, nb);
}
}  // namespace

int launch_chain(const Params& p, int mode, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const bool bf = p.dtype == GDR_BF16;
  if (p.K == 128 && bf && p.gate == 0) run_chain<128, bf16, 0>(p, mode, s);
  else if (p.K == 128 && bf && p.gate == 1) run_chain<128, bf16, 1>(p, mode, s);
  else if (p.K == 128 && !bf && p.gate == 0) run_chain<128, float, 0>(p, mode, s);
  else if (p.K == 128 && !bf && p.gate == 1) run_chain<128, float, 1>(p, mode, s);
  else if (p.K == 64 && bf && p.gate == 0) run_chain<64, bf16, 0>(p, mode, s);
  else if (p.K == 64 && bf && p.gate == 1) run_chain<64, bf16, 1>(p, mode, s);
  else if (p.K == 64 && !bf && p.gate == 0) run_chain<64, float, 0>(p, mode, s);
  else if (p.K == 64 && !bf && p.gate == 1) run_chain<64, float, 1>(p, mode, s);
  else return static_cast<int>(hipErrorInvalidValue);
  return static_cast<int>(hipGetLastError());
}

}  // namespace gdr

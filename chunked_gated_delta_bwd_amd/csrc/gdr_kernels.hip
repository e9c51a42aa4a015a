// HIP kernels for gfx950: the chunked gated delta-rule forward recompute and
// backward.  Four launches per backward:
//
//   k_prep    one workgroup per (chunk, head): L2 norms, beta, in-chunk gate
//             cumsum Gamma, M = Kn Kn^T o E and P = scale Qn Kn^T o E on MFMA,
//             the UT/WY inverse A = (I + StrictLower(diag(beta) M))^-1, and
//             W = A diag(beta) Kbar, U' = A diag(beta) V on MFMA.
//   k_chain   the two serial chunk recursions, one workgroup per
//             (sequence, head, 16-wide V slice) per direction: the forward state
//             pass S_{n+1} = S_n Diag(e^GamC) + (U' - W S_n^T)^T Khat and the
//             reverse state-gradient pass dS_n = dS_{n+1} Diag(e^GamC) +
//             dO^T Qbar - dU^T W with dU = P^T dO + Khat dS_{n+1}^T.  Neither
//             depends on the other, so the fused entry point runs both side by
//             side in one grid.  The fp32 accumulators stay in registers.
//   k_grads   one workgroup per (chunk, head): the chunk-local gradients on MFMA.
//   k_finish  one workgroup per (chunk, head), bandwidth bound: L2-norm and
//             sigmoid backward, reverse cumsum of the gate gradient plus the
//             chunk-total term.
//
// The recursion is the one the FlashQLA overview describes (state gradient
// strictly from the last chunk to the first, dh <- g_last dh + R^T dO + X^T Y
// with X = A_beta K); the prepare-stage formulas follow the FlashKDA backward
// (K1) page, sections 3-6.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

constexpr int C = kChunk;
constexpr int PC = C + 8;   // LDS pitch of 64-wide bf16 tiles (elements)

template <int D>
struct Dims {
  static constexpr int PD = D + 8;             // LDS pitch of D-wide bf16 tiles
  static constexpr int TPR = D / 8;            // threads per row in row sweeps (8 elements each)
  static constexpr int RPP = kThreads / TPR;   // rows per pass
  static constexpr int NPASS = C / RPP;        // passes over the 64 rows
  static constexpr int NJB = D / 16;           // 16-wide blocks along D
  static constexpr int NJW = NJB / 4;          // D-blocks per wave in the chain kernels
};

__device__ __forceinline__ int64_t tok(int t, int H, int h) { return int64_t(t) * H + h; }

__device__ __forceinline__ void st_bf16x4(bf16* dst, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(dst) = pack4_bf16(a, b, c, d);
}
__device__ __forceinline__ void st_bf16x4(uint16_t* dst, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(dst) = pack4_bf16(a, b, c, d);
}

// ===========================================================================
// k_prep (scalar gate)
// ===========================================================================
template <int D, typename TIO>
__global__ __launch_bounds__(kThreads) void k_prep_gdn(const Params p) {
  using Dm = Dims<D>;
  constexpr int PD = Dm::PD, TPR = Dm::TPR, RPP = Dm::RPP, NPASS = Dm::NPASS;
  constexpr int PL = C + 4;
  __shared__ __attribute__((aligned(16))) bf16 Qs[C * PD];
  __shared__ __attribute__((aligned(16))) bf16 Ks[C * PD];
  __shared__ __attribute__((aligned(16))) bf16 Vs[C * PD];
  __shared__ __attribute__((aligned(16))) bf16 As[C * PC];
  __shared__ __attribute__((aligned(16))) float Lf[C * PL];
  __shared__ float gam_s[C], beta_s[C];

  const int c = blockIdx.x, h = blockIdx.y;
  const ChunkEntry ce = p.ctab[c];
  const int t0 = ce.t_start, len = ce.len;
  const int tid = threadIdx.x, l = lane_id(), w = wave_id();
  const int64_t ch = int64_t(h) * p.NC + c;
  const int H = p.H;

  // --- rows: L2 norms; qn, kn to LDS; kn and v kept in registers ---
  float kn_r[NPASS][8], v_r[NPASS][8];
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int r = ps * RPP + tid / TPR, c0 = (tid % TPR) * 8;
    float qv[8], kv[8];
    {
      // unconditional loads from a clamped row, masked afterwards (no branch
      // around the loads, so they are not serialised)
      const int64_t off = tok(t0 + min(r, len - 1), H, h) * D + c0;
      IO<TIO>::load8(p.q, off, qv);
      IO<TIO>::load8(p.k, off, kv);
      IO<TIO>::load8(p.v, off, v_r[ps]);
      const float m = r < len ? 1.f : 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qv[e] *= m;
        kv[e] *= m;
        v_r[ps][e] *= m;
      }
    }
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) { sq += qv[e] * qv[e]; sk += kv[e] * kv[e]; }
    sq = group_sum<TPR>(sq);
    sk = group_sum<TPR>(sk);
    const float rq = 1.0f / sqrtf(sq + 1e-6f), rk = 1.0f / sqrtf(sk + 1e-6f);
    bf16x8 qb, kb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kn_r[ps][e] = kv[e] * rk;
      qb[e] = to_bf16(qv[e] * rq);
      kb[e] = to_bf16(kn_r[ps][e]);
    }
    *reinterpret_cast<bf16x8*>(Qs + r * PD + c0) = qb;
    *reinterpret_cast<bf16x8*>(Ks + r * PD + c0) = kb;
    if (tid % TPR == 0) {
      p.rho[ch * 2 * C + r] = rq;
      p.rho[ch * 2 * C + C + r] = rk;
    }
  }
  // --- beta and the in-chunk cumsum of the log decay (wave 0) ---
  if (w == 0) {
    const int64_t o = tok(t0 + min(l, len - 1), H, h);
    const float m = l < len ? 1.f : 0.f;
    float lam = m * IO<TIO>::load1(p.g, o);
    const float bt = m * sigmoidf(IO<TIO>::load1(p.b, o));
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const float y = __shfl_up(lam, m, 64);
      if (l >= m) lam += y;
    }
    gam_s[l] = lam;
    beta_s[l] = bt;
    p.gam[ch * C + l] = lam;
  }
  __syncthreads();

  // --- M and P, transposed tiles so that each lane owns 4 consecutive s ---
  {
    const int R = w;
    const int r = 16 * R + (l & 15);
    const float gr = gam_s[r], br = beta_s[r];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      float Lv[4] = {0.f, 0.f, 0.f, 0.f}, Pv[4] = {0.f, 0.f, 0.f, 0.f};
      const int s0 = 16 * sb + 4 * (l >> 4);
      if (sb <= R) {
        f32x4 aM = zero4(), aP = zero4();
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += 32) {
          const bf16x8 a = frag_rk(Ks, PD, 16 * sb, k0);
          aM = mma(a, frag_rk(Ks, PD, 16 * R, k0), aM);
          aP = mma(a, frag_rk(Qs, PD, 16 * R, k0), aP);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = s0 + i;
          if (r >= s) {
            const float E = fast_exp(gr - gam_s[s]);
            Pv[i] = p.scale * aP[i] * E;
            if (r > s) Lv[i] = br * aM[i] * E;
          }
        }
      }
      *reinterpret_cast<float4*>(Lf + r * PL + s0) = make_float4(Lv[0], Lv[1], Lv[2], Lv[3]);
      st_bf16x4(p.P + (ch * C + r) * C + s0, Pv[0], Pv[1], Pv[2], Pv[3]);
    }
  }
  __syncthreads();

  // --- beta * Kbar and beta * V overwrite the operand tiles ---
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int r = ps * RPP + tid / TPR, c0 = (tid % TPR) * 8;
    const float fk = beta_s[r] * fast_exp(gam_s[r]), fv = beta_s[r];
    bf16x8 kb, vb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kb[e] = to_bf16(kn_r[ps][e] * fk);
      vb[e] = to_bf16(v_r[ps][e] * fv);
    }
    *reinterpret_cast<bf16x8*>(Ks + r * PD + c0) = kb;
    *reinterpret_cast<bf16x8*>(Vs + r * PD + c0) = vb;
  }

  // --- A = (I + L)^-1 by forward substitution, one column per lane (wave 0) ---
  if (w == 0) {
    float a[C];
#pragma unroll
    for (int r = 0; r < C; ++r) {
      float acc = (r == l) ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < (r & ~3); s += 4) {
        const float4 L4 = *reinterpret_cast<const float4*>(Lf + r * PL + s);
        acc -= L4.x * a[s] + L4.y * a[s + 1] + L4.z * a[s + 2] + L4.w * a[s + 3];
      }
#pragma unroll
      for (int s = (r & ~3); s < r; ++s) acc -= Lf[r * PL + s] * a[s];
      a[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < C; ++r) {
      As[r * PC + l] = to_bf16(a[r]);
      p.A[(ch * C + r) * C + l] = f32_to_bf16_bits(a[r]);
    }
  }
  __syncthreads();

  // --- W^T and U'^T tiles: lane owns W[r][j .. j+3] ---
  {
    const int r = 16 * w + (l & 15);
#pragma unroll
    for (int jb = 0; jb < D / 16; ++jb) {
      f32x4 aW = zero4(), aU = zero4();
#pragma unroll
      for (int k0 = 0; k0 < C; k0 += 32) {
        const bf16x8 b = frag_rk(As, PC, 16 * w, k0);  // B[s][r] = A[r][s]
        aW = mma(frag_kc(Ks, PD, 16 * jb, k0), b, aW);
        aU = mma(frag_kc(Vs, PD, 16 * jb, k0), b, aU);
      }
      const int j0 = 16 * jb + 4 * (l >> 4);
      st_bf16x4(p.W + (ch * C + r) * D + j0, aW[0], aW[1], aW[2], aW[3]);
      st_bf16x4(p.Up + (ch * C + r) * D + j0, aU[0], aU[1], aU[2], aU[3]);
    }
  }
}

// ===========================================================================
// k_chain: serial recursions over the chunks of one (sequence, head, V slice)
// ===========================================================================
template <int D, typename TIO>
struct ChainSmem {
  using Dm = Dims<D>;
  static constexpr int PD = Dm::PD, PO = 24;
  static constexpr size_t tile = size_t(C) * PD * 2;
  // fp32 inputs are not exact in bf16: q also gets a low-order tile (where it fits)
  static constexpr bool kQlo = std::is_same<TIO, float>::value && D == 64;
  static constexpr size_t fwd = 4 * tile + 16 * PD * 2 + 16 * PC * 2 + 2 * 4;
  static constexpr size_t bwd = (kQlo ? 8 : 6) * tile + 2 * C * PC * 2 + 3 * 2 * C * PO * 2 + 16 * PD * 2 +
                                16 * PC * 2 + 2 * 4;
  static constexpr size_t bytes = fwd > bwd ? fwd : bwd;
};

// Each recursion keeps two register sets of prefetched chunk data (raw, not
// unpacked): the set stashed into LDS at step k was loaded at step k-2, so every
// load has two full steps to arrive while vmcnt waits only for the older set.
template <int D, typename TIO>
struct FwdPrefetch {
  using Dm = Dims<D>;
  u32x4 w[Dm::NPASS];
  typename IO<TIO>::Raw8 k[Dm::NPASS];
  float rk[Dm::NPASS], g[Dm::NPASS], m[Dm::NPASS], gC;
  uint16_t u[4];
};

template <int D, typename TIO>
struct BwdPrefetch {
  using Dm = Dims<D>;
  u32x4 w[Dm::NPASS], pm[2];
  typename IO<TIO>::Raw8 k[Dm::NPASS], q[Dm::NPASS];
  typename IO<TIO>::Raw4 dO;
  float rk[Dm::NPASS], g[Dm::NPASS], m[Dm::NPASS], gC, rq_do, g_do, m_do;
};

// Loads of one chunk into registers: unconditional (rows past the sequence end
// read its last row and are masked at the stash) and with no arithmetic on the
// loaded values, so nothing waits for them before the stash.
template <int D, typename TIO>
__device__ __forceinline__ void fwd_load(FwdPrefetch<D, TIO>& f, const Params& p, const SeqEntry& se, int h,
                                         int v0, int c) {
  using Dm = Dims<D>;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int64_t ch = int64_t(h) * p.NC + c;
  const int ct0 = se.t_start + (c - se.c0) * C;
  const int clen = min(C, se.len - (c - se.c0) * C);
#pragma unroll
  for (int ps = 0; ps < Dm::NPASS; ++ps) {
    const int r = ps * Dm::RPP + tid / Dm::TPR, c0 = (tid % Dm::TPR) * 8;
    f.w[ps] = *reinterpret_cast<const u32x4*>(p.W + (ch * C + r) * D + c0);
    f.k[ps] = IO<TIO>::load_raw8(p.k, tok(ct0 + min(r, clen - 1), p.H, h) * D + c0);
    f.m[ps] = r < clen ? 1.f : 0.f;
    f.rk[ps] = p.rho[ch * 2 * C + C + r];
    f.g[ps] = p.gam[ch * C + r];
  }
  f.gC = p.gam[ch * C + C - 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) f.u[i] = p.Up[(ch * C + 16 * w + 4 * (l >> 4) + i) * D + v0 + (l & 15)];
}

// Khat = kn e^(GamC - Gam) and W into LDS buffer `buf`; U' into registers.
template <int D, typename TIO>
__device__ __forceinline__ void fwd_stash(const FwdPrefetch<D, TIO>& f, bf16* Ws, bf16* Kh, float* dec,
                                          float (&up)[4]) {
  using Dm = Dims<D>;
  constexpr int PD = Dm::PD;
  const int tid = threadIdx.x;
#pragma unroll
  for (int ps = 0; ps < Dm::NPASS; ++ps) {
    const int r = ps * Dm::RPP + tid / Dm::TPR, c0 = (tid % Dm::TPR) * 8;
    *reinterpret_cast<u32x4*>(Ws + r * PD + c0) = f.w[ps];
    const float s = f.m[ps] * f.rk[ps] * fast_exp(f.gC - f.g[ps]);
    float kx[8];
    IO<TIO>::unpack8(f.k[ps], kx);
    bf16x8 kb;
#pragma unroll
    for (int e = 0; e < 8; ++e) kb[e] = to_bf16(kx[e] * s);
    *reinterpret_cast<bf16x8*>(Kh + r * PD + c0) = kb;
  }
  if (tid == 0) *dec = fast_exp(f.gC);
#pragma unroll
  for (int i = 0; i < 4; ++i) up[i] = bf16_bits_to_f32(f.u[i]);
}

template <int D, typename TIO>
__device__ __forceinline__ void bwd_load(BwdPrefetch<D, TIO>& f, const Params& p, const SeqEntry& se, int h,
                                         int v0, int c) {
  using Dm = Dims<D>;
  const int tid = threadIdx.x;
  const int64_t ch = int64_t(h) * p.NC + c;
  const int ct0 = se.t_start + (c - se.c0) * C;
  const int clen = min(C, se.len - (c - se.c0) * C);
#pragma unroll
  for (int ps = 0; ps < Dm::NPASS; ++ps) {
    const int r = ps * Dm::RPP + tid / Dm::TPR, c0 = (tid % Dm::TPR) * 8;
    f.w[ps] = *reinterpret_cast<const u32x4*>(p.W + (ch * C + r) * D + c0);
    const int64_t o = tok(ct0 + min(r, clen - 1), p.H, h) * D + c0;
    f.k[ps] = IO<TIO>::load_raw8(p.k, o);
    f.q[ps] = IO<TIO>::load_raw8(p.q, o);
    f.m[ps] = r < clen ? 1.f : 0.f;
    f.rk[ps] = p.rho[ch * 2 * C + C + r];
    f.g[ps] = p.gam[ch * C + r];
  }
  f.gC = p.gam[ch * C + C - 1];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int pc = tid + x * kThreads;   // 16-byte piece of the 64x64 P tile
    f.pm[x] = *reinterpret_cast<const u32x4*>(p.P + (ch * C + pc / 8) * C + (pc % 8) * 8);
  }
  const int r = tid / 4, c0 = (tid % 4) * 4;
  f.dO = IO<TIO>::load_raw4(p.dO, tok(ct0 + min(r, clen - 1), p.H, h) * D + v0 + c0);
  f.m_do = r < clen ? 1.f : 0.f;
  f.rq_do = p.rho[ch * 2 * C + r];
  f.g_do = p.gam[ch * C + r];
}

// Khat, raw q (exact in bf16; high/low parts for fp32 inputs), W, P, the raw dO
// slice and the scaled slice f*dO (f_r = scale rho_r e^Gam_r) split into bf16
// high + low parts.  The Qbar^T dO term is then q^T (f dO) with no rounding of
// Qbar: it dominates dh0.
template <int D, typename TIO, bool QLO>
__device__ __forceinline__ void bwd_stash(const BwdPrefetch<D, TIO>& f, float scale, bf16* Kh, bf16* Qb, bf16* Ql,
                                          bf16* Ws, bf16* Ps, bf16* dOr, bf16* dFh, bf16* dFl, float* dec) {
  using Dm = Dims<D>;
  constexpr int PD = Dm::PD, PO = 24;
  const int tid = threadIdx.x;
#pragma unroll
  for (int ps = 0; ps < Dm::NPASS; ++ps) {
    const int r = ps * Dm::RPP + tid / Dm::TPR, c0 = (tid % Dm::TPR) * 8;
    *reinterpret_cast<u32x4*>(Ws + r * PD + c0) = f.w[ps];
    const float fk = f.m[ps] * f.rk[ps] * fast_exp(f.gC - f.g[ps]);
    float kx[8], qx[8];
    IO<TIO>::unpack8(f.k[ps], kx);
    IO<TIO>::unpack8(f.q[ps], qx);
    bf16x8 kb, qb, ql;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float qv = qx[e] * f.m[ps];
      kb[e] = to_bf16(kx[e] * fk);
      qb[e] = to_bf16(qv);
      if constexpr (QLO) ql[e] = to_bf16(qv - float(qb[e]));
    }
    *reinterpret_cast<bf16x8*>(Kh + r * PD + c0) = kb;
    *reinterpret_cast<bf16x8*>(Qb + r * PD + c0) = qb;
    if constexpr (QLO) *reinterpret_cast<bf16x8*>(Ql + r * PD + c0) = ql;
  }
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int pc = tid + x * kThreads;
    *reinterpret_cast<u32x4*>(Ps + (pc / 8) * PC + (pc % 8) * 8) = f.pm[x];
  }
  const int r = tid / 4, c0 = (tid % 4) * 4;
  const float fs = f.m_do * scale * f.rq_do * fast_exp(f.g_do);
  float dx[4], fh[4], fl[4];
  IO<TIO>::unpack4(f.dO, dx);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float x = dx[e] * fs;
    fh[e] = float(to_bf16(x));
    fl[e] = x - fh[e];
    dx[e] *= f.m_do;
  }
  st_bf16x4(dOr + r * PO + c0, dx[0], dx[1], dx[2], dx[3]);
  st_bf16x4(dFh + r * PO + c0, fh[0], fh[1], fh[2], fh[3]);
  st_bf16x4(dFl + r * PO + c0, fl[0], fl[1], fl[2], fl[3]);
  if (tid == 0) *dec = fast_exp(f.gC);
}

template <int D, typename TIO>
__device__ __forceinline__ void chain_fwd(const Params& p, char* smem, int si, int h, int sl) {
  using Dm = Dims<D>;
  constexpr int PD = Dm::PD, NJW = Dm::NJW;
  // double-buffered tiles: buffer b of X starts at X0 + b * C * PD
  bf16* const Ws0 = reinterpret_cast<bf16*>(smem);
  bf16* const Kh0 = Ws0 + 2 * C * PD;
  bf16* Ss = Kh0 + 2 * C * PD;   // S[v][j], 16 rows
  bf16* Ut = Ss + 16 * PD;       // U[r][v] stored as Ut[v][r]
  float* dec = reinterpret_cast<float*>(Ut + 16 * PC);

  const int l = lane_id(), w = wave_id();
  const int g = l >> 4, jj = l & 15;
  const int H = p.H;
  const SeqEntry se = p.stab[si];
  const int v0 = 16 * sl;
  const int nck = se.nchunks;

  f32x4 acc[NJW];
#pragma unroll
  for (int x = 0; x < NJW; ++x) {
    const int j = 16 * (w * NJW + x) + 4 * g;
    if (p.h0) {
      const float4 t = *reinterpret_cast<const float4*>(p.h0 + ((int64_t(se.seq) * H + h) * D + v0 + jj) * D + j);
      acc[x] = f32x4{t.x, t.y, t.z, t.w};
    } else {
      acc[x] = zero4();
    }
  }

  FwdPrefetch<D, TIO> A, Bp;
  float up[4];
  // one chunk k (0-based in this sequence) on LDS buffer `buf`; `nx` holds chunk
  // k+1 (stashed into the other buffer here) and is refilled with chunk k+3
  auto step = [&](int k, int buf, FwdPrefetch<D, TIO>& nx) __attribute__((always_inline)) {
    const int c = se.c0 + k;
    const int64_t ch = int64_t(h) * p.NC + c;
    // S_k: to LDS (operand of U) and to the workspace
#pragma unroll
    for (int x = 0; x < NJW; ++x) {
      const int j = 16 * (w * NJW + x) + 4 * g;
      st_bf16x4(Ss + jj * PD + j, acc[x][0], acc[x][1], acc[x][2], acc[x][3]);
      st_bf16x4(p.S + (ch * D + v0 + jj) * D + j, acc[x][0], acc[x][1], acc[x][2], acc[x][3]);
    }
    __syncthreads();
    // U = U' - W S^T for rows 16w.., columns of this slice
    const bf16* Wb = Ws0 + buf * C * PD;
    const bf16* Khb = Kh0 + buf * C * PD;
    f32x4 au = zero4();
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += 32) au = mma(frag_rk(Wb, PD, 16 * w, k0), frag_rk(Ss, PD, 0, k0), au);
    float u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u[i] = up[i] - au[i];
      p.U[(ch * C + 16 * w + 4 * g + i) * D + v0 + jj] = f32_to_bf16_bits(u[i]);
    }
    st_bf16x4(Ut + jj * PC + 16 * w + 4 * g, u[0], u[1], u[2], u[3]);
    if (k + 1 < nck) fwd_stash<D, TIO>(nx, Ws0 + (buf ^ 1) * C * PD, Kh0 + (buf ^ 1) * C * PD, dec + (buf ^ 1), up);
    // unconditional (clamped to the last chunk): a branch here would make the
    // compiler wait for the loaded registers at the join
    fwd_load<D, TIO>(nx, p, se, h, v0, se.c0 + min(k + 3, nck - 1));
    __syncthreads();
    // S_{k+1}^T = S_k^T e^GamC + Khat^T U
    const float d = dec[buf];
#pragma unroll
    for (int x = 0; x < NJW; ++x) {
      const int jb = w * NJW + x;
      f32x4 a = acc[x] * d;
#pragma unroll
      for (int k0 = 0; k0 < C; k0 += 32) a = mma(frag_kc(Khb, PD, 16 * jb, k0), frag_rk(Ut, PC, 0, k0), a);
      acc[x] = a;
    }
  };

  if (nck > 0) {
    fwd_load<D, TIO>(A, p, se, h, v0, se.c0);
    fwd_load<D, TIO>(Bp, p, se, h, v0, se.c0 + min(1, nck - 1));
    fwd_stash<D, TIO>(A, Ws0, Kh0, dec, up);
    fwd_load<D, TIO>(A, p, se, h, v0, se.c0 + min(2, nck - 1));
    __syncthreads();
    for (int k = 0; k < nck; k += 2) {
      step(k, 0, Bp);
      if (k + 1 < nck) step(k + 1, 1, A);
    }
  }
  if (p.ht) {
#pragma unroll
    for (int x = 0; x < NJW; ++x) {
      const int j = 16 * (w * NJW + x) + 4 * g;
      *reinterpret_cast<float4*>(p.ht + ((int64_t(se.seq) * H + h) * D + v0 + jj) * D + j) =
          make_float4(acc[x][0], acc[x][1], acc[x][2], acc[x][3]);
    }
  }
}

template <int D, typename TIO>
__device__ __forceinline__ void chain_bwd(const Params& p, char* smem, int si, int h, int sl) {
  using Dm = Dims<D>;
  constexpr int PD = Dm::PD, NJW = Dm::NJW;
  constexpr int PO = ChainSmem<D, TIO>::PO;
  constexpr bool QLO = ChainSmem<D, TIO>::kQlo;
  // Double-buffered tiles: buffer b of X starts at X0 + b * (tile size).
  bf16* const Kh0 = reinterpret_cast<bf16*>(smem);
  bf16* const Qb0 = Kh0 + 2 * C * PD;   // raw q (high part for fp32 inputs)
  bf16* const Ws0 = Qb0 + 2 * C * PD;
  bf16* const Ql0 = Ws0 + 2 * C * PD;   // low part of q (fp32 inputs only)
  bf16* const Ps0 = Ql0 + (QLO ? 2 * C * PD : 0);
  bf16* const dO0 = Ps0 + 2 * C * PC;   // raw dO slice
  bf16* const dFh0 = dO0 + 2 * C * PO;  // f * dO, high part
  bf16* const dFl0 = dFh0 + 2 * C * PO; // f * dO, low part
  bf16* dSl = dFl0 + 2 * C * PO;  // dS[v][j], 16 rows
  bf16* dUt = dSl + 16 * PD;     // -dU stored as [v][r]
  float* dec = reinterpret_cast<float*>(dUt + 16 * PC);

  const int l = lane_id(), w = wave_id();
  const int g = l >> 4, jj = l & 15;
  const int H = p.H;
  const SeqEntry se = p.stab[si];
  const int v0 = 16 * sl;
  const int nck = se.nchunks;
  const float scale = p.scale;

  f32x4 acc[NJW];
#pragma unroll
  for (int x = 0; x < NJW; ++x) {
    const int j = 16 * (w * NJW + x) + 4 * g;
    if (p.dht) {
      const float4 t = *reinterpret_cast<const float4*>(p.dht + ((int64_t(se.seq) * H + h) * D + v0 + jj) * D + j);
      acc[x] = f32x4{t.x, t.y, t.z, t.w};
    } else {
      acc[x] = zero4();
    }
  }

  auto stash = [&](const BwdPrefetch<D, TIO>& f, int buf) __attribute__((always_inline)) {
    bwd_stash<D, TIO, QLO>(f, scale, Kh0 + buf * C * PD, Qb0 + buf * C * PD, Ql0 + buf * C * PD,
                           Ws0 + buf * C * PD, Ps0 + buf * C * PC, dO0 + buf * C * PO, dFh0 + buf * C * PO,
                           dFl0 + buf * C * PO, dec + buf);
  };
  // chunks are walked last to first: step k handles chunk c0 + nck - 1 - k
  BwdPrefetch<D, TIO> A, Bp;
  auto step = [&](int k, int buf, BwdPrefetch<D, TIO>& nx) __attribute__((always_inline)) {
    const int c = se.c0 + nck - 1 - k;
    const int64_t ch = int64_t(h) * p.NC + c;
    // dS_{n+1}: to LDS (operand of dU) and to the workspace
#pragma unroll
    for (int x = 0; x < NJW; ++x) {
      const int j = 16 * (w * NJW + x) + 4 * g;
      st_bf16x4(dSl + jj * PD + j, acc[x][0], acc[x][1], acc[x][2], acc[x][3]);
      st_bf16x4(p.dS + (ch * D + v0 + jj) * D + j, acc[x][0], acc[x][1], acc[x][2], acc[x][3]);
    }
    __syncthreads();
    const bf16* Khb = Kh0 + buf * C * PD;
    const bf16* Qbb = Qb0 + buf * C * PD;
    const bf16* Wb = Ws0 + buf * C * PD;
    const bf16* Pb = Ps0 + buf * C * PC;
    const bf16* dOb = dO0 + buf * C * PO;
    const bf16* dFh = dFh0 + buf * C * PO;
    const bf16* dFl = dFl0 + buf * C * PO;
    const bf16* Qlb = Ql0 + buf * C * PD;
    // dU = P^T dO + Khat dS^T for rows 16w.., columns of this slice
    f32x4 ad = zero4();
#pragma unroll
    for (int k0 = 0; k0 < C; k0 += 32) ad = mma(frag_kc(Pb, PC, 16 * w, k0), frag_kc(dOb, PO, 0, k0), ad);
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += 32) ad = mma(frag_rk(Khb, PD, 16 * w, k0), frag_rk(dSl, PD, 0, k0), ad);
#pragma unroll
    for (int i = 0; i < 4; ++i) p.dU[(ch * C + 16 * w + 4 * g + i) * D + v0 + jj] = f32_to_bf16_bits(ad[i]);
    st_bf16x4(dUt + jj * PC + 16 * w + 4 * g, -ad[0], -ad[1], -ad[2], -ad[3]);
    if (k + 1 < nck) stash(nx, buf ^ 1);
    bwd_load<D, TIO>(nx, p, se, h, v0, se.c0 + max(nck - 4 - k, 0));  // chunk k+3, clamped
    __syncthreads();
    // dS_n^T = dS_{n+1}^T e^GamC + q^T (f dO) - W^T dU
    const float d = dec[buf];
#pragma unroll
    for (int x = 0; x < NJW; ++x) {
      const int jb = w * NJW + x;
      f32x4 a = acc[x] * d;
#pragma unroll
      for (int k0 = 0; k0 < C; k0 += 32) {
        const bf16x8 aq = frag_kc(Qbb, PD, 16 * jb, k0);
        const bf16x8 bh = frag_kc(dFh, PO, 0, k0);
        a = mma(aq, bh, a);
        a = mma(aq, frag_kc(dFl, PO, 0, k0), a);
        if constexpr (QLO) a = mma(frag_kc(Qlb, PD, 16 * jb, k0), bh, a);
        a = mma(frag_kc(Wb, PD, 16 * jb, k0), frag_rk(dUt, PC, 0, k0), a);
      }
      acc[x] = a;
    }
  };

  if (nck > 0) {
    const int cl = se.c0 + nck - 1;
    bwd_load<D, TIO>(A, p, se, h, v0, cl);
    bwd_load<D, TIO>(Bp, p, se, h, v0, max(cl - 1, se.c0));
    stash(A, 0);
    bwd_load<D, TIO>(A, p, se, h, v0, max(cl - 2, se.c0));
    __syncthreads();
    for (int k = 0; k < nck; k += 2) {
      step(k, 0, Bp);
      if (k + 1 < nck) step(k + 1, 1, A);
    }
  }
  if (p.dh0) {
#pragma unroll
    for (int x = 0; x < NJW; ++x) {
      const int j = 16 * (w * NJW + x) + 4 * g;
      *reinterpret_cast<float4*>(p.dh0 + ((int64_t(se.seq) * H + h) * D + v0 + jj) * D + j) =
          make_float4(acc[x][0], acc[x][1], acc[x][2], acc[x][3]);
    }
  }
}

// blockIdx -> (work group of one (sequence, head), V slice): the slices of one
// (sequence, head) share its chunk tiles, so they are placed on the same XCD
// (workgroups are dealt round-robin over the 8 XCDs).
template <int D, typename TIO>
__global__ __launch_bounds__(kThreads) void k_chain(const Params p, int mode, int nb_role) {
  __shared__ __attribute__((aligned(16))) char smem[ChainSmem<D, TIO>::bytes];
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
    chain_fwd<D, TIO>(p, smem, si, h, sl);
  else
    chain_bwd<D, TIO>(p, smem, si, h, sl);
}

// ===========================================================================
// k_grads (scalar gate): chunk-local gradients
// ===========================================================================
template <int D>
struct GradSmem {
  static constexpr int PD = Dims<D>::PD;
  static constexpr int rs = 2 * C * PD;                                  // elements
  static constexpr int rds = (D * PD > 2 * C * PC) ? D * PD : 2 * C * PC;  // elements
};

template <int D, typename TIO>
__global__ __launch_bounds__(kThreads) void k_grads_gdn(const Params p) {
  using Dm = Dims<D>;
  constexpr int PD = Dm::PD, TPR = Dm::TPR, RPP = Dm::RPP, NPASS = Dm::NPASS, NJB = Dm::NJB;
  __shared__ __attribute__((aligned(16))) bf16 RS[GradSmem<D>::rs];
  __shared__ __attribute__((aligned(16))) bf16 RdS[GradSmem<D>::rds];
  __shared__ __attribute__((aligned(16))) bf16 dOs[C * PD];
  __shared__ __attribute__((aligned(16))) bf16 Us[C * PD];
  __shared__ __attribute__((aligned(16))) bf16 dYs[C * PD];
  __shared__ float gam_s[C], beta_s[C], rq_s[C], rk_s[C];
  // fixed-order partial sums (deterministic): column sums of the pairwise dGamma
  // term per wave, row sums per row, and two per-wave chunk scalars
  __shared__ float colsum_s[4][C], rowsum_s[C], red_s[4][2];

  const int c = blockIdx.x, h = blockIdx.y;
  const ChunkEntry ce = p.ctab[c];
  const int t0 = ce.t_start, len = ce.len;
  const int tid = threadIdx.x, l = lane_id(), w = wave_id();
  const int g = l >> 4, jj = l & 15;
  const int64_t ch = int64_t(h) * p.NC + c;
  const int H = p.H;
  const float scale = p.scale;

  bf16* dUs = RS;     // phase 1
  bf16* As = RdS;     // phase 1
  if (tid < C) {
    gam_s[tid] = p.gam[ch * C + tid];
    rq_s[tid] = p.rho[ch * 2 * C + tid];
    rk_s[tid] = p.rho[ch * 2 * C + C + tid];
    beta_s[tid] = (tid < len ? 1.f : 0.f) * sigmoidf(IO<TIO>::load1(p.b, tok(t0 + min(tid, len - 1), H, h)));
#pragma unroll
    for (int x = 0; x < 4; ++x) colsum_s[x][tid] = 0.f;
  }
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int r = ps * RPP + tid / TPR, c0 = (tid % TPR) * 8;
    *reinterpret_cast<uint4*>(dUs + r * PD + c0) = *reinterpret_cast<const uint4*>(p.dU + (ch * C + r) * D + c0);
    *reinterpret_cast<uint4*>(Us + r * PD + c0) = *reinterpret_cast<const uint4*>(p.U + (ch * C + r) * D + c0);
    float x[8];
    IO<TIO>::load8(p.dO, tok(t0 + min(r, len - 1), H, h) * D + c0, x);
    const float m = r < len ? 1.f : 0.f;
    bf16x8 xb;
#pragma unroll
    for (int e = 0; e < 8; ++e) xb[e] = to_bf16(x[e] * m);
    *reinterpret_cast<bf16x8*>(dOs + r * PD + c0) = xb;
  }
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int pc = tid + x * kThreads;
    *reinterpret_cast<uint4*>(As + (pc / 8) * PC + (pc % 8) * 8) =
        *reinterpret_cast<const uint4*>(p.A + (ch * C + pc / 8) * C + (pc % 8) * 8);
  }
  __syncthreads();

  // ---- phase 1: dY = A^T dU (lane owns dY[r][v .. v+3], r = 16w + jj); dv; sum dY*v ----
  const int r = 16 * w + jj;
  const float br = beta_s[r];
  float dbeta_row = 0.f, dgam_row = 0.f;
#pragma unroll
  for (int vb = 0; vb < NJB; ++vb) {
    f32x4 a = zero4();
#pragma unroll
    for (int k0 = 0; k0 < C; k0 += 32) a = mma(frag_kc(dUs, PD, 16 * vb, k0), frag_kc(As, PC, 16 * w, k0), a);
    const int v = 16 * vb + 4 * g;
    st_bf16x4(dYs + r * PD + v, a[0], a[1], a[2], a[3]);
    // rows past the end: dY is exactly zero there, so the clamped v row adds nothing
    const int64_t o = tok(t0 + min(r, len - 1), H, h) * D + v;
    float vv[4];
    IO<TIO>::load4(p.v, o, vv);
    dbeta_row += a[0] * vv[0] + a[1] * vv[1] + a[2] * vv[2] + a[3] * vv[3];
    if (r < len) IO<TIO>::store4(p.dv, o, br * a[0], br * a[1], br * a[2], br * a[3]);
  }
  __syncthreads();
  // ---- load S (RS) and dS (RdS), both [v][j] ----
  {
    constexpr int PIECES = D * D / 8;
    for (int pc = tid; pc < PIECES; pc += kThreads) {
      const int row = pc / (D / 8), col = (pc % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(RS + row * PD + col) = *reinterpret_cast<const uint4*>(p.S + (ch * D + row) * D + col);
      *reinterpret_cast<uint4*>(RdS + row * PD + col) = *reinterpret_cast<const uint4*>(p.dS + (ch * D + row) * D + col);
    }
  }
  __syncthreads();
  // ---- phase 2: Z = dY S, dQbar = dO S, dKhat = U dS (transposed tiles) ----
  f32x4 aZ[NJB], aQ[NJB], aK[NJB];
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb) {
    aZ[jb] = aQ[jb] = aK[jb] = zero4();
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += 32) {
      const bf16x8 aS = frag_kc(RS, PD, 16 * jb, k0);
      const bf16x8 aD = frag_kc(RdS, PD, 16 * jb, k0);
      aZ[jb] = mma(aS, frag_rk(dYs, PD, 16 * w, k0), aZ[jb]);
      aQ[jb] = mma(aS, frag_rk(dOs, PD, 16 * w, k0), aQ[jb]);
      aK[jb] = mma(aD, frag_rk(Us, PD, 16 * w, k0), aK[jb]);
    }
  }
  // state term of dGamma_C: sum_{v,j} dS * S
  float sdot = 0.f;
  {
    constexpr int PIECES = D * D / 8;
    for (int pc = tid; pc < PIECES; pc += kThreads) {
      const int row = pc / (D / 8), col = (pc % (D / 8)) * 8;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(RS + row * PD + col);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(RdS + row * PD + col);
#pragma unroll
      for (int e = 0; e < 8; ++e) sdot += float(a[e]) * float(b[e]);
    }
  }
  __syncthreads();
  // ---- load Kn, Qn (RS rows 0..63 and 64..127) ----
  bf16* Kn = RS;
  bf16* Qn = RS + C * PD;
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int rr = ps * RPP + tid / TPR, c0 = (tid % TPR) * 8;
    float qv[8], kv[8];
    const int64_t o = tok(t0 + min(rr, len - 1), H, h) * D + c0;
    IO<TIO>::load8(p.q, o, qv);
    IO<TIO>::load8(p.k, o, kv);
    const float m = rr < len ? 1.f : 0.f;
    const float fq = m * rq_s[rr], fk = m * rk_s[rr];
    bf16x8 qb, kb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qb[e] = to_bf16(qv[e] * fq);
      kb[e] = to_bf16(kv[e] * fk);
    }
    *reinterpret_cast<bf16x8*>(Qn + rr * PD + c0) = qb;
    *reinterpret_cast<bf16x8*>(Kn + rr * PD + c0) = kb;
  }
  __syncthreads();
  // ---- phase 3: M, P, dP, dL (transposed tiles: lane owns X[r][s .. s+3]) ----
  bf16* dMEs = RdS;
  bf16* dPEs = RdS + C * PC;
  const float gr = gam_s[r];
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
    const int s0 = 16 * sb + 4 * g;
    float dme[4] = {0.f, 0.f, 0.f, 0.f}, dpe[4] = {0.f, 0.f, 0.f, 0.f};
    if (sb <= w) {
      f32x4 G1 = zero4(), G2 = zero4(), Mr = zero4(), Pr = zero4();
#pragma unroll
      for (int k0 = 0; k0 < D; k0 += 32) {
        const bf16x8 aU = frag_rk(Us, PD, 16 * sb, k0);
        G1 = mma(aU, frag_rk(dOs, PD, 16 * w, k0), G1);
        G2 = mma(aU, frag_rk(dYs, PD, 16 * w, k0), G2);
        const bf16x8 aK = frag_rk(Kn, PD, 16 * sb, k0);
        Mr = mma(aK, frag_rk(Kn, PD, 16 * w, k0), Mr);
        Pr = mma(aK, frag_rk(Qn, PD, 16 * w, k0), Pr);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = s0 + i;
        float qv = 0.f;
        if (r >= s) {
          const float E = fast_exp(gr - gam_s[s]);
          const float P = scale * Pr[i] * E;
          const float dP = G1[i];
          qv = dP * P;
          dpe[i] = scale * dP * E;
          if (r > s) {
            const float M = Mr[i] * E;
            const float dL = -G2[i];
            const float dM = br * dL;
            dbeta_row += dL * M;
            qv += dM * M;
            dme[i] = dM * E;
          }
        }
        dgam_row += qv;
        const float col = group_sum<16>(qv);   // sum over the 16 rows r of this tile
        if (jj == 0) colsum_s[w][s] = -col;
      }
    }
    st_bf16x4(dMEs + r * PC + s0, dme[0], dme[1], dme[2], dme[3]);
    st_bf16x4(dPEs + r * PC + s0, dpe[0], dpe[1], dpe[2], dpe[3]);
  }
  // ---- fold the state-side terms (lane owns (r, j .. j+3)) ----
  const float eg = fast_exp(gr), eh = fast_exp(gam_s[C - 1] - gr);
  float dgc_loc = 0.f;
  f32x4 dkn[NJB], dqn[NJB];
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb) {
    const int j = 16 * jb + 4 * g;
    const bf16x4 kb = *reinterpret_cast<const bf16x4*>(Kn + r * PD + j);
    const bf16x4 qb = *reinterpret_cast<const bf16x4*>(Qn + r * PD + j);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float kn = float(kb[i]), qn = float(qb[i]);
      const float z = aZ[jb][i], dkh = aK[jb][i], dqb = aQ[jb][i];
      // dKbar = -beta Z, Kbar = kn e^Gam, Khat = kn e^(GamC-Gam), Qbar = scale qn e^Gam
      dgam_row += -br * z * kn * eg - dkh * kn * eh + dqb * scale * qn * eg;
      dbeta_row -= kn * eg * z;
      dgc_loc += dkh * kn * eh;
      dkn[jb][i] = -br * z * eg + dkh * eh;
      dqn[jb][i] = scale * dqb * eg;
    }
  }
  __syncthreads();
  // ---- phase 4: pairwise terms, dkn += (dME + dME^T) Kn + scale dPE^T Qn, dqn += scale dPE Kn ----
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb) {
#pragma unroll
    for (int k0 = 0; k0 < C; k0 += 32) {
      const bf16x8 aK = frag_kc(Kn, PD, 16 * jb, k0);
      const bf16x8 aQ2 = frag_kc(Qn, PD, 16 * jb, k0);
      dkn[jb] = mma(aK, frag_rk(dMEs, PC, 16 * w, k0), dkn[jb]);
      dkn[jb] = mma(aK, frag_kc(dMEs, PC, 16 * w, k0), dkn[jb]);
      dkn[jb] = mma(aQ2, frag_kc(dPEs, PC, 16 * w, k0), dkn[jb]);
      dqn[jb] = mma(aK, frag_rk(dPEs, PC, 16 * w, k0), dqn[jb]);
    }
    const int j = 16 * jb + 4 * g;
    *reinterpret_cast<float4*>(p.dqn + (ch * C + r) * D + j) = make_float4(dqn[jb][0], dqn[jb][1], dqn[jb][2], dqn[jb][3]);
    *reinterpret_cast<float4*>(p.dkn + (ch * C + r) * D + j) = make_float4(dkn[jb][0], dkn[jb][1], dkn[jb][2], dkn[jb][3]);
  }
  // ---- row and chunk reductions ----
  dgam_row += __shfl_xor(dgam_row, 16, 64);
  dgam_row += __shfl_xor(dgam_row, 32, 64);
  dbeta_row += __shfl_xor(dbeta_row, 16, 64);
  dbeta_row += __shfl_xor(dbeta_row, 32, 64);
  if (g == 0) {
    rowsum_s[r] = dgam_row;
    p.dbeta[ch * C + r] = dbeta_row;
  }
  const float tot = group_sum<64>(dgc_loc);
  const float st = group_sum<64>(sdot);
  if (l == 0) {
    red_s[w][0] = tot;
    red_s[w][1] = st;
  }
  __syncthreads();
  if (tid < C)
    p.dgam[ch * C + tid] = rowsum_s[tid] + ((colsum_s[0][tid] + colsum_s[1][tid]) + (colsum_s[2][tid] + colsum_s[3][tid]));
  if (tid == 0) {
    const float a = (red_s[0][0] + red_s[1][0]) + (red_s[2][0] + red_s[3][0]);
    const float b = (red_s[0][1] + red_s[1][1]) + (red_s[2][1] + red_s[3][1]);
    p.dgamc[ch] = a + b * fast_exp(gam_s[C - 1]);
  }
}

// ===========================================================================
// k_finish (scalar gate): L2-norm / sigmoid backward, gate reverse cumsum
// ===========================================================================
template <int D, typename TIO>
__global__ __launch_bounds__(kThreads) void k_finish_gdn(const Params p) {
  using Dm = Dims<D>;
  constexpr int TPR = Dm::TPR, RPP = Dm::RPP, NPASS = Dm::NPASS;
  const int c = blockIdx.x, h = blockIdx.y;
  const ChunkEntry ce = p.ctab[c];
  const int t0 = ce.t_start, len = ce.len;
  const int tid = threadIdx.x, l = lane_id(), w = wave_id();
  const int64_t ch = int64_t(h) * p.NC + c;
  const int H = p.H;
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int r = ps * RPP + tid / TPR, c0 = (tid % TPR) * 8;
    const bool ok = r < len;
    float q[8], k[8], dq[8], dk[8];
    const int64_t o = tok(t0 + min(r, len - 1), H, h) * D + c0;
    const float m = ok ? 1.f : 0.f;
    const float rq = m * p.rho[ch * 2 * C + r], rk = m * p.rho[ch * 2 * C + C + r];
    IO<TIO>::load8(p.q, o, q);
    IO<TIO>::load8(p.k, o, k);
    {
      const float4* a = reinterpret_cast<const float4*>(p.dqn + (ch * C + r) * D + c0);
      const float4* b = reinterpret_cast<const float4*>(p.dkn + (ch * C + r) * D + c0);
      const float4 a0 = a[0], a1 = a[1], b0 = b[0], b1 = b[1];
      dq[0] = a0.x; dq[1] = a0.y; dq[2] = a0.z; dq[3] = a0.w; dq[4] = a1.x; dq[5] = a1.y; dq[6] = a1.z; dq[7] = a1.w;
      dk[0] = b0.x; dk[1] = b0.y; dk[2] = b0.z; dk[3] = b0.w; dk[4] = b1.x; dk[5] = b1.y; dk[6] = b1.z; dk[7] = b1.w;
    }
    float pq = 0.f, pk = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      q[e] *= rq;
      k[e] *= rk;
      pq += q[e] * dq[e];
      pk += k[e] * dk[e];
    }
    pq = group_sum<TPR>(pq);
    pk = group_sum<TPR>(pk);
    if (ok) {
      float oq[8], ok8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        oq[e] = rq * (dq[e] - q[e] * pq);
        ok8[e] = rk * (dk[e] - k[e] * pk);
      }
      IO<TIO>::store8(p.dq, o, oq);
      IO<TIO>::store8(p.dk, o, ok8);
    }
  }
  if (w == 0) {
    // dlam_s = sum_{r >= s} dGam_r + dGamC (suffix sum; FlashKDA backward page, §5)
    float x = p.dgam[ch * C + l];
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const float y = __shfl_down(x, m, 64);
      if (l + m < 64) x += y;
    }
    const int64_t o = tok(t0 + min(l, len - 1), H, h);
    const float bt = sigmoidf(IO<TIO>::load1(p.b, o));
    const float dgc = p.dgamc[ch], dbs = p.dbeta[ch * C + l];
    if (l < len) {
      IO<TIO>::store1(p.dg, o, x + dgc);
      IO<TIO>::store1(p.db, o, dbs * bt * (1.f - bt));
    }
  }
}

__global__ void k_zero(float* a, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) a[i] = 0.f;
}

// ===========================================================================
// launchers
// ===========================================================================
namespace {

int last_error() { return static_cast<int>(hipGetLastError()); }

template <template <int, typename> class F>
int dispatch(const Params& p, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (p.K == 128 && p.dtype == GDR_BF16) F<128, bf16>::run(p, s);
  else if (p.K == 128 && p.dtype == GDR_F32) F<128, float>::run(p, s);
  else if (p.K == 64 && p.dtype == GDR_BF16) F<64, bf16>::run(p, s);
  else if (p.K == 64 && p.dtype == GDR_F32) F<64, float>::run(p, s);
  else return static_cast<int>(hipErrorInvalidValue);
  return last_error();
}

template <int D, typename TIO>
struct RunPrep {
  static void run(const Params& p, hipStream_t s) {
    k_prep_gdn<D, TIO><<<dim3(p.NC, p.H), kThreads, 0, s>>>(p);
  }
};
template <int D, typename TIO>
struct RunGrads {
  static void run(const Params& p, hipStream_t s) {
    k_grads_gdn<D, TIO><<<dim3(p.NC, p.H), kThreads, 0, s>>>(p);
  }
};
template <int D, typename TIO>
struct RunFinish {
  static void run(const Params& p, hipStream_t s) {
    k_finish_gdn<D, TIO><<<dim3(p.NC, p.H), kThreads, 0, s>>>(p);
  }
};

int g_chain_mode = 0;
template <int D, typename TIO>
struct RunChain {
  static void run(const Params& p, hipStream_t s) {
    constexpr int ns = D / 16;
    const int groups = p.N * p.H;
    const int nb = ((groups + 7) / 8) * 8 * ns;
    const int nroles = g_chain_mode == kChainBoth ? 2 : 1;
    k_chain<D, TIO><<<dim3(nb * nroles), kThreads, 0, s>>>(p, g_chain_mode, nb);
  }
};

}  // namespace

int launch_prep(const Params& p, void* stream) { return dispatch<RunPrep>(p, stream); }
int launch_grads(const Params& p, void* stream) { return dispatch<RunGrads>(p, stream); }
int launch_finish(const Params& p, void* stream) { return dispatch<RunFinish>(p, stream); }
int launch_chain(const Params& p, int mode, void* stream) {
  g_chain_mode = mode;
  return dispatch<RunChain>(p, stream);
}
int launch_zero_params(const Params& p, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (p.dA_log) k_zero<<<(p.H + 255) / 256, 256, 0, s>>>(p.dA_log, p.H);
  if (p.ddt_bias) k_zero<<<(p.H * p.K + 255) / 256, 256, 0, s>>>(p.ddt_bias, p.H * p.K);
  return last_error();
}
const char* hip_error_string(int err) { return hipGetErrorString(static_cast<hipError_t>(err)); }

}  // namespace gdr

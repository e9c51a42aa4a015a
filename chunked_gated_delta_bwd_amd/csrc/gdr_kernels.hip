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

static_assert(C == kChunk, "chunk size");
static_assert(Dims<128>::RPP * Dims<128>::TPR == kThreads, "row sweep covers the workgroup");

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
  __shared__ float gam_s[C], beta_s[C], rq_s[C], rk_s[C];
  // fp32 inputs: the recursions take materialised Khat / Qbar tiles (Qbar split
  // into bf16 high and low parts); bf16 inputs use the raw rows and row factors
  constexpr bool kMat = std::is_same<TIO, float>::value;

  const int c = blockIdx.x, h = blockIdx.y;
  const ChunkEntry ce = p.ctab[c];
  const int t0 = ce.t_start, len = ce.len;
  const int tid = threadIdx.x, l = lane_id(), w = wave_id();
  const int64_t ch = int64_t(h) * p.NC + c;
  const int H = p.H;

  // --- rows: L2 norms; qn, kn to LDS; kn and v kept in registers ---
  float kn_r[NPASS][8], v_r[NPASS][8];
  float qn_r[kMat ? NPASS : 1][8];
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
      if constexpr (kMat) qn_r[ps][e] = qv[e] * rq;
      qb[e] = to_bf16(qv[e] * rq);
      kb[e] = to_bf16(kn_r[ps][e]);
    }
    *reinterpret_cast<bf16x8*>(Qs + r * PD + c0) = qb;
    *reinterpret_cast<bf16x8*>(Ks + r * PD + c0) = kb;
    if (tid % TPR == 0) {
      p.rho[ch * 2 * C + r] = rq;
      p.rho[ch * 2 * C + C + r] = rk;
      rq_s[r] = rq;
      rk_s[r] = rk;
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

  // --- operands of the two recursions: row factors, chunk decay, and for fp32
  // inputs the Khat and Qbar (high + low) tiles ---
  if (tid < C) {
    const float m = tid < len ? 1.f : 0.f, gC = gam_s[C - 1], gr = gam_s[tid];
    p.fac[ch * 2 * C + tid] = m * p.scale * rq_s[tid] * fast_exp(gr);
    p.fac[ch * 2 * C + C + tid] = m * rk_s[tid] * fast_exp(gC - gr);
    if (tid == 0) p.edec[ch * 4] = fast_exp(gC);
  }
  if constexpr (kMat) {
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int r = ps * RPP + tid / TPR, c0 = (tid % TPR) * 8;
      const float fk = fast_exp(gam_s[C - 1] - gam_s[r]), fq = p.scale * fast_exp(gam_s[r]);
      bf16x8 kh, qh, ql;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = qn_r[ps][e] * fq;
        kh[e] = to_bf16(kn_r[ps][e] * fk);
        qh[e] = to_bf16(x);
        ql[e] = to_bf16(x - float(qh[e]));
      }
      const int64_t o = (ch * C + r) * D + c0;
      *reinterpret_cast<bf16x8*>(p.Kh + o) = kh;
      *reinterpret_cast<bf16x8*>(p.Qh + o) = qh;
      *reinterpret_cast<bf16x8*>(p.Ql + o) = ql;
    }
  }

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
  __shared__ __attribute__((aligned(16))) bf16 UsT[D * PC];   // U^T: [v][r]
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

  bf16* dUsT = RS;    // phase 1: dU^T [v][r]
  bf16* As = RdS;     // phase 1
  if (tid < C) {
    gam_s[tid] = p.gam[ch * C + tid];
    rq_s[tid] = p.rho[ch * 2 * C + tid];
    rk_s[tid] = p.rho[ch * 2 * C + C + tid];
    beta_s[tid] = (tid < len ? 1.f : 0.f) * sigmoidf(IO<TIO>::load1(p.b, tok(t0 + min(tid, len - 1), H, h)));
#pragma unroll
    for (int x = 0; x < 4; ++x) colsum_s[x][tid] = 0.f;
  }
  // U and dU are stored transposed, [v][r]
  for (int pc = tid; pc < D * C / 8; pc += kThreads) {
    const int v = pc / (C / 8), c0 = (pc % (C / 8)) * 8;
    *reinterpret_cast<uint4*>(dUsT + v * PC + c0) = *reinterpret_cast<const uint4*>(p.dU + (ch * D + v) * C + c0);
    *reinterpret_cast<uint4*>(UsT + v * PC + c0) = *reinterpret_cast<const uint4*>(p.U + (ch * D + v) * C + c0);
  }
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int r = ps * RPP + tid / TPR, c0 = (tid % TPR) * 8;
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
    for (int k0 = 0; k0 < C; k0 += 32) a = mma(frag_rk(dUsT, PC, 16 * vb, k0), frag_kc(As, PC, 16 * w, k0), a);
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
      aK[jb] = mma(aD, frag_kc(UsT, PC, 16 * w, k0), aK[jb]);
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
        const bf16x8 aU = frag_kc(UsT, PC, 16 * sb, k0);
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

}  // namespace

int launch_prep(const Params& p, void* stream) { return dispatch<RunPrep>(p, stream); }
int launch_grads(const Params& p, void* stream) { return dispatch<RunGrads>(p, stream); }
int launch_finish(const Params& p, void* stream) { return dispatch<RunFinish>(p, stream); }
int launch_zero_params(const Params& p, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (p.dA_log) k_zero<<<(p.H + 255) / 256, 256, 0, s>>>(p.dA_log, p.H);
  if (p.ddt_bias) k_zero<<<(p.H * p.K + 255) / 256, 256, 0, s>>>(p.ddt_bias, p.H * p.K);
  return last_error();
}
const char* hip_error_string(int err) { return hipGetErrorString(static_cast<hipError_t>(err)); }

}  // namespace gdr

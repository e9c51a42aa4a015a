// HIP kernels for gfx950, scalar gate (GDN): the chunk-parallel parts of the
// chunked gated delta-rule forward recompute and backward.  Three launches per
// backward (the per-channel gate has its own kernels in gdr_kda.hip):
//
//   k_prep    one workgroup per (chunk, head): L2 norms, beta, in-chunk gate
//             cumsum Gamma, M = Kn Kn^T o E and P = scale Qn Kn^T o E on MFMA,
//             the UT/WY inverse A = (I + StrictLower(diag(beta) M))^-1, and
//             W = A diag(beta) Kbar, U' = A diag(beta) V on MFMA.
//   k_chain   (gdr_chain.hip) the two serial chunk recursions.
//   k_grads   one workgroup per (chunk, head): the chunk-local gradients on MFMA,
//             and in its tail the prepare-backward: L2-norm and sigmoid backward,
//             reverse cumsum of the gate gradient plus the chunk-total term.
//
// The recursion is the one the FlashQLA overview describes (state gradient
// strictly from the last chunk to the first, dh <- g_last dh + R^T dO + X^T Y
// with X = A_beta K); the prepare-stage formulas follow the FlashKDA backward
// (K1) page, sections 3-6.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gdr_device.h"
#include "gdr_internal.h"
#include "gdr_lds.h"

namespace gdr {

static_assert(C == kChunk, "chunk size");
static_assert(Dims<128>::RPP * Dims<128>::TPR == kThreads, "row sweep covers the workgroup");

// ===========================================================================
// k_prep (scalar gate)
// ===========================================================================
// The prologue runs eight waves (two per SIMD).  Tiles (rb, sb), sb <= rb, of the
// 10 lower / diagonal 16x16 blocks of a 64x64 chunk matrix, dealt over them: slot
// 0 of wave w is tile w, slot 1 of waves 0 and 1 tiles 8 and 9 (nibble w of these
// words, then nibbles 8 and 9, give rb / sb); the other waves have no slot 1.
constexpr int kPrepThreads = 2 * kThreads;
constexpr uint64_t kTileRb = 0x3333222110ull;   // tile t: rb = nibble t
constexpr uint64_t kTileSb = 0x3210210100ull;   // tile t: sb = nibble t
__device__ __forceinline__ int tile_of(int w, int slot) { return slot == 0 || w >= 2 ? w : 8 + w; }
__device__ __forceinline__ int tile_rb(int w, int slot) { return int(kTileRb >> (4 * tile_of(w, slot))) & 15; }
__device__ __forceinline__ int tile_sb(int w, int slot) { return int(kTileSb >> (4 * tile_of(w, slot))) & 15; }
__device__ __forceinline__ bool tile_valid(int w, int slot) { return slot == 0 || w < 2; }


template <int D, typename TIO>
__global__ __launch_bounds__(kPrepThreads) void k_prep_gdn(const Params p) {
  using Dm = Dims<D>;
  constexpr int PD = Dm::PD, TPR = Dm::TPR;
  constexpr int kT = kPrepThreads;
  constexpr int RPP = kT / TPR, NPASS = C / RPP;   // row sweeps of 8 channels a thread
  constexpr int PL = C + 4;   // pitch (floats) of the fp32 64x64 tiles L and X
  constexpr int kQX = C * PD * 2 > C * PL * 4 ? C * PD * 2 : C * PL * 4;
  __shared__ __attribute__((aligned(16))) char QX[kQX];          // Qn; from the inverse on: X = A, fp32
  __shared__ __attribute__((aligned(16))) bf16 Ks[C * PD];
  __shared__ __attribute__((aligned(16))) bf16 Vs[C * PD];
  __shared__ __attribute__((aligned(16))) bf16 As[C * PC];       // P on its way out; inverse scratch; A
  __shared__ __attribute__((aligned(16))) float Lf[C * PL];
  __shared__ float gam_s[C], beta_s[C], rq_s[C], rk_s[C];
  bf16* const Qs = reinterpret_cast<bf16*>(QX);
  float* const Xf = reinterpret_cast<float*>(QX);
  // fp32 inputs: the recursions take materialised Khat / Qbar tiles (Qbar split
  // into bf16 high and low parts); bf16 inputs use the raw rows and row factors
  constexpr bool kMat = std::is_same<TIO, float>::value;
  // and at kMatTwoPartK-wide heads the low tiles of Khat and W as well, for the
  // reverse recursion's two-part steps
  constexpr bool kMat2 = kMat && D == kMatTwoPartK;
  // fp32 inputs: low bf16 parts of qn, kn (then beta Kbar) and A, so that M, P and
  // W are formed from two-part operands (hi hi + lo hi + hi lo); bf16 inputs' rows
  // are exact in bf16 after the row norm only up to its rounding, which the
  // recursions' row factors carry instead
  constexpr int kLoT = kMat ? C * PD : 8, kLoA = kMat ? C * PC : 8;
  __shared__ __attribute__((aligned(16))) bf16 Qsl[kLoT];
  __shared__ __attribute__((aligned(16))) bf16 Ksl[kLoT];
  __shared__ __attribute__((aligned(16))) bf16 Asl[kLoA];

  int c, h;
  chunk_head(p, c, h);
  const ChunkEntry ce = p.ctab[c];
  const int t0 = ce.t_start, len = ce.len;
  const int tid = threadIdx.x, l = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id());
  const int g = l >> 4, jj = l & 15;
  // wave w: row block rb = w % 4; the two waves of a row block (one SIMD) split
  // its work where it splits, else the first one works
  const int rb = w & 3, hf = w >> 2;
  const int64_t ch = int64_t(h) * p.NC + c;
  const int H = p.H;

  // --- rows: every load issued first (unconditional, from a clamped row, masked
  // afterwards), so that their latencies overlap ---
  typename IO<TIO>::Raw8 qraw[NPASS], kraw[NPASS], vraw[NPASS];
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int r = ps * RPP + tid / TPR, c0 = (tid % TPR) * 8;
    const int64_t off = tok(t0 + min(r, len - 1), H, h) * D + c0;
    const int64_t qoff = qk_tok(p, t0 + min(r, len - 1), h) * D + c0;
    qraw[ps] = IO<TIO>::load_raw8(p.q, qoff);
    kraw[ps] = IO<TIO>::load_raw8(p.k, qoff);
    vraw[ps] = IO<TIO>::load_raw8(p.v, off);
  }
  float graw = 0.f, braw = 0.f;
  if (w == 0) {
    const int64_t o = tok(t0 + min(l, len - 1), H, h);
    graw = IO<TIO>::load1(p.g, o);
    braw = IO<TIO>::load1(p.b, o);
  }
  // the P tile goes out through As, which starts at zero (tiles above the diagonal)
  for (int o = 16 * tid; o < C * PC * 2; o += 16 * kT)
    *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(As) + o) = u32x4{0u, 0u, 0u, 0u};

  // --- L2 norms; qn, kn to LDS; kn and v kept in registers ---
  float kn_r[NPASS][8], v_r[NPASS][8];
  float qn_r[kMat ? NPASS : 1][8];
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int r = ps * RPP + tid / TPR, c0 = (tid % TPR) * 8;
    float qv[8], kv[8];
    IO<TIO>::unpack8(qraw[ps], qv);
    IO<TIO>::unpack8(kraw[ps], kv);
    IO<TIO>::unpack8(vraw[ps], v_r[ps]);
    const float m = r < len ? 1.f : 0.f;
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qv[e] *= m;
      kv[e] *= m;
      v_r[ps][e] *= m;
      sq += qv[e] * qv[e];
      sk += kv[e] * kv[e];
    }
    sq = group_sum_dpp<TPR>(sq);
    sk = group_sum_dpp<TPR>(sk);
    const float rq = 1.0f / sqrtf(sq + 1e-6f), rk = 1.0f / sqrtf(sk + 1e-6f);
    bf16x8 qb, kb, ql, kl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kn_r[ps][e] = kv[e] * rk;
      if constexpr (kMat) qn_r[ps][e] = qv[e] * rq;
      // bf16 inputs: the raw rows (exact in bf16) for M and P, whose products
      // take the row norms in fp32 afterwards; fp32 inputs: qn, kn in two parts
      qb[e] = to_bf16(kMat ? qv[e] * rq : qv[e]);
      kb[e] = to_bf16(kMat ? kn_r[ps][e] : kv[e]);
      if constexpr (kMat) {
        ql[e] = to_bf16(qn_r[ps][e] - float(qb[e]));
        kl[e] = to_bf16(kn_r[ps][e] - float(kb[e]));
      }
    }
    *reinterpret_cast<bf16x8*>(Qs + r * PD + c0) = qb;
    *reinterpret_cast<bf16x8*>(Ks + r * PD + c0) = kb;
    if constexpr (kMat) {
      *reinterpret_cast<bf16x8*>(Qsl + r * PD + c0) = ql;
      *reinterpret_cast<bf16x8*>(Ksl + r * PD + c0) = kl;
    }
    if (tid % TPR == 0) {
      p.rho[ch * 3 * C + r] = rq;
      p.rho[ch * 3 * C + C + r] = rk;
      rq_s[r] = rq;
      rk_s[r] = rk;
    }
  }
  // --- beta and the in-chunk cumsum of the log decay (wave 0) ---
  if (w == 0) {
    const float m = l < len ? 1.f : 0.f;
    float lam = m * graw;
    const float bt = m * sigmoidf(braw);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const float y = __shfl_up(lam, m, 64);
      if (l >= m) lam += y;
    }
    gam_s[l] = lam;
    beta_s[l] = bt;
    p.gam[ch * C + l] = lam;
    p.rho[ch * 3 * C + 2 * C + l] = bt;
  }
  __syncthreads();

  // --- operands of the two recursions: row factors, chunk decay, and for fp32
  // inputs the Khat and Qbar (high + low) tiles ---
  if (tid < C) {
    const float m = tid < len ? 1.f : 0.f, gC = gam_s[C - 1], gr = gam_s[tid];
    p.fac[ch * 3 * C + tid] = m * p.scale * rq_s[tid] * fast_exp(gr);
    p.fac[ch * 3 * C + C + tid] = m * rk_s[tid] * fast_exp(gC - gr);
    p.fac[ch * 3 * C + 2 * C + tid] = beta_s[tid] * rk_s[tid] * fast_exp(gr);   // W = A Diag(this) k
    if (tid == 0) p.edec[ch * 4] = fast_exp(gC);
  }
  if constexpr (kMat) {
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int r = ps * RPP + tid / TPR, c0 = (tid % TPR) * 8;
      const float fk = fast_exp(gam_s[C - 1] - gam_s[r]), fq = p.scale * fast_exp(gam_s[r]);
      bf16x8 kh, kl, qh, ql;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = qn_r[ps][e] * fq, y = kn_r[ps][e] * fk;
        kh[e] = to_bf16(y);
        kl[e] = to_bf16(y - float(kh[e]));
        qh[e] = to_bf16(x);
        ql[e] = to_bf16(x - float(qh[e]));
      }
      const int64_t o = (ch * C + r) * D + c0;
      *reinterpret_cast<bf16x8*>(p.Kh + o) = kh;
      if constexpr (kMat2) *reinterpret_cast<bf16x8*>(p.Khl + o) = kl;
      *reinterpret_cast<bf16x8*>(p.Qh + o) = qh;
      *reinterpret_cast<bf16x8*>(p.Ql + o) = ql;
    }
  }

  // --- M and P on the lower / diagonal tiles: lane owns X[r][s .. s+3],
  // r = 16 rb + jj, s = 16 sb + 4g + i ---
#pragma unroll
  for (int slot = 0; slot < 2; ++slot) {
    if (!tile_valid(w, slot)) break;
    const int tb = tile_rb(w, slot), sb = tile_sb(w, slot);
    const int r = 16 * tb + jj, s0 = 16 * sb + 4 * g;
    f32x4 aM = zero4(), aP = zero4();
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += 32) {
      const bf16x8 a = frag_rk(Ks, PD, 16 * sb, k0);
      const bf16x8 bk = frag_rk(Ks, PD, 16 * tb, k0), bq = frag_rk(Qs, PD, 16 * tb, k0);
      aM = mma(a, bk, aM);
      aP = mma(a, bq, aP);
      if constexpr (kMat) {
        const bf16x8 al = frag_rk(Ksl, PD, 16 * sb, k0);
        aM = mma(al, bk, aM);
        aM = mma(a, frag_rk(Ksl, PD, 16 * tb, k0), aM);
        aP = mma(al, bq, aP);
        aP = mma(a, frag_rk(Qsl, PD, 16 * tb, k0), aP);
      }
    }
    const float gr = gam_s[r], br = beta_s[r];
    // bf16 inputs: the row norms of the raw-row products
    const float fm = kMat ? 1.f : rk_s[r], fp = kMat ? 1.f : rq_s[r];
    float Lv[4], Pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = s0 + i;
      // Gamma is non-increasing, so the exponent is <= 0 wherever it is used
      const float E = fast_exp(fminf(gr - gam_s[s], 0.f));
      const float fs = kMat ? 1.f : rk_s[s];
      Pv[i] = r >= s ? p.scale * (aP[i] * (fp * fs)) * E : 0.f;
      Lv[i] = r > s ? br * (aM[i] * (fm * fs)) * E : 0.f;
    }
    if (tile_valid(w, slot)) {
      *reinterpret_cast<float4*>(Lf + r * PL + s0) = make_float4(Lv[0], Lv[1], Lv[2], Lv[3]);
      st_bf16x4(As + r * PC + s0, Pv[0], Pv[1], Pv[2], Pv[3]);
    }
  }
  __syncthreads();

  // --- P out: rows of 128 bytes, 16 bytes per lane ---
#pragma unroll
  for (int it = 0; it < C * C / 8 / kT; ++it) {
    const int idx = tid + kT * it, row = idx / 8, c8 = (idx % 8) * 8;
    *reinterpret_cast<u32x4*>(p.P + (ch * C + row) * C + c8) = *reinterpret_cast<const u32x4*>(As + row * PC + c8);
  }

  // --- beta * Kbar (for W; fp32 inputs only, bf16 inputs leave W to the
  // recursions as A Diag(fw) k) and beta * V overwrite the operand tiles ---
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int r = ps * RPP + tid / TPR, c0 = (tid % TPR) * 8;
    const float fk = beta_s[r] * fast_exp(gam_s[r]), fv = beta_s[r];
    bf16x8 kb, kl, vb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = kn_r[ps][e] * fk;
      kb[e] = to_bf16(x);
      kl[e] = to_bf16(x - float(kb[e]));
      vb[e] = to_bf16(v_r[ps][e] * fv);
    }
    if constexpr (kMat) {
      *reinterpret_cast<bf16x8*>(Ks + r * PD + c0) = kb;
      *reinterpret_cast<bf16x8*>(Ksl + r * PD + c0) = kl;
    }
    *reinterpret_cast<bf16x8*>(Vs + r * PD + c0) = vb;
  }

  // --- A = (I + L)^-1 in 16x16 blocks X_ij (fp32): wave i inverts the diagonal
  // block I + L_ii by forward substitution (lane = column) ... ---
  if (hf == 0) {
    const int i0 = 16 * rb;
    float a[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = r == jj ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < r; ++s) acc -= Lf[(i0 + r) * PL + i0 + s] * a[s];
      a[r] = acc;
    }
    if (l < 16) {
#pragma unroll
      for (int r = 0; r < 16; ++r) Xf[(i0 + r) * PL + i0 + jj] = a[r];
    }
  }
  __syncthreads();
  // ... then wave j walks down block column j on fp32 MFMA:
  //   X_ij = -X_ii (sum_{m=j}^{i-1} L_im X_mj),  i = j+1 .. 3
  if (hf == 0) {
    const int j0 = 16 * rb;
    float* const scr = reinterpret_cast<float*>(As) + 256 * rb;   // 16x16 per wave
    for (int i = rb + 1; i < 4; ++i) {
      const int i0 = 16 * i;
      f32x4 sacc = zero4();
      for (int m = rb; m < i; ++m) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          sacc = mma_f32(Lf[(i0 + jj) * PL + 16 * m + 4 * kk + g], Xf[(16 * m + 4 * kk + g) * PL + j0 + jj], sacc);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) scr[(4 * g + e) * 16 + jj] = sacc[e];
      f32x4 x = zero4();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) x = mma_f32(Xf[(i0 + jj) * PL + i0 + 4 * kk + g], scr[(4 * kk + g) * 16 + jj], x);
#pragma unroll
      for (int e = 0; e < 4; ++e) Xf[(i0 + 4 * g + e) * PL + j0 + jj] = -x[e];
    }
  }
  __syncthreads();
  // --- A out (bf16): the operand tile for W, U' and the workspace copy; the
  // blocks above the diagonal are zero ---
#pragma unroll
  for (int it = 0; it < C * C / 8 / kT; ++it) {
    const int idx = tid + kT * it, row = idx / 8, c8 = (idx % 8) * 8;
    const bool on = (c8 >> 4) <= (row >> 4);
    bf16x8 v, vl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = on ? Xf[row * PL + c8 + e] : 0.f;
      v[e] = to_bf16(x);
      vl[e] = to_bf16(x - float(v[e]));
    }
    *reinterpret_cast<bf16x8*>(As + row * PC + c8) = v;
    if constexpr (kMat) *reinterpret_cast<bf16x8*>(Asl + row * PC + c8) = vl;
    *reinterpret_cast<bf16x8*>(p.A + (ch * C + row) * C + c8) = v;
  }
  __syncthreads();

  // --- W (fp32 inputs) and U' tiles: lane owns W[r][j .. j+3]; staged in the
  // inverse's scratch (free by now) and stored as 16-byte row pieces ---
  static_assert(C * PD * 2 <= kQX && C * PD * 2 <= C * PL * 4, "staging tiles fit");
  bf16* const Wst = reinterpret_cast<bf16*>(QX);
  bf16* const Ust = reinterpret_cast<bf16*>(Lf);
  {
    const int r = 16 * rb + (l & 15);
#pragma unroll
    for (int q = 0; q < D / 32; ++q) {   // this wave's half of the 16-wide column blocks
      const int jb = hf * (D / 32) + q;
      f32x4 aW = zero4(), aU = zero4();
#pragma unroll
      for (int k0 = 0; k0 < C; k0 += 32) {
        const bf16x8 b = frag_rk(As, PC, 16 * rb, k0);  // B[s][r] = A[r][s]
        if constexpr (kMat) {
          const bf16x8 kf = frag_kc(Ks, PD, 16 * jb, k0);
          aW = mma(kf, b, aW);
          aW = mma(frag_kc(Ksl, PD, 16 * jb, k0), b, aW);
          aW = mma(kf, frag_rk(Asl, PC, 16 * rb, k0), aW);
        }
        aU = mma(frag_kc(Vs, PD, 16 * jb, k0), b, aU);
      }
      const int j0 = 16 * jb + 4 * (l >> 4);
      if constexpr (kMat) st_bf16x4(Wst + r * PD + j0, aW[0], aW[1], aW[2], aW[3]);
      if constexpr (kMat2)   // (fp32 inputs only: stored from the lane, 8 bytes a row)
        st_bf16x4(p.Wl + (ch * C + r) * D + j0, lo_part(aW[0]), lo_part(aW[1]), lo_part(aW[2]), lo_part(aW[3]));
      st_bf16x4(Ust + r * PD + j0, aU[0], aU[1], aU[2], aU[3]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < C * D / 8 / kT; ++it) {
    const int idx = tid + kT * it, row = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
    if constexpr (kMat)
      *reinterpret_cast<u32x4*>(p.W + (ch * C + row) * D + c8) = *reinterpret_cast<const u32x4*>(Wst + row * PD + c8);
    *reinterpret_cast<u32x4*>(p.Up + (ch * C + row) * D + c8) = *reinterpret_cast<const u32x4*>(Ust + row * PD + c8);
  }
}

// ===========================================================================
// k_grads_gdn (scalar gate): chunk-local gradients, fused with the
// prepare-backward (L2-norm and sigmoid backward, the gate's reverse cumsum)
// ===========================================================================
// The tiles a chunk needs (dU^T, A, U^T, dO, v, S, dS) are copied global -> LDS
// with direct-to-LDS loads issued as the workgroup starts, in two groups: phase 1
// waits for the first only, so the state tiles arrive while it runs.  Raw q and
// k rows are copied the same way at the start of phase 2, into the space phase 1
// has freed.  Each tile is its own LDS object, so the compiler can tell that a
// read of one tile does not depend on the copies into another.
//
// A wave with direct-to-LDS loads in flight must not consume an ordinary
// register load: the compiler then waits for every load in flight.  With bf16
// inputs the kernel therefore reads nothing from global memory into registers
// until all copies have landed; fp32 inputs (rounded to bf16 on the way into
// LDS) are loaded into registers and lose that overlap.
template <int D, typename TIO>
struct GradLds {
  static constexpr bool kDma = !std::is_same<TIO, float>::value;
  static constexpr int TS = D * D * 2;   // S, dS tiles [v][j]
  static constexpr int TU = D * C * 2;   // dU^T, U^T tiles [v][r]
  static constexpr int TR = C * D * 2;   // row tiles [r][*]: dO, dY, v, q, k, Kn, Qn
  static constexpr int TA = C * C * 2;   // A, dME, dPE
  // the S tile later holds Kn and Qn, the dS tile dME and dPE
  static constexpr int TSx = TS > 2 * TR ? TS : 2 * TR;
  static constexpr int TdSx = TS > 2 * TA ? TS : 2 * TA;
  static_assert(TU == TR, "raw q rows reuse the dU^T tile");
};

// Eight waves: wave w works on row block rb = w % 4 (rows 16 rb ..) and column
// half hf = w / 4 of every D-wide result; waves w and w + 4 share a SIMD.
constexpr int kGradWaves = 8;
constexpr int kGradThreads = 64 * kGradWaves;

// how many workgroups ahead a gradient workgroup prefetches (one per CU run at once)
constexpr int kGradAhead = 256;

// L2 prefetch of the first tile group of the gradient workgroup with linear id L:
// dU^T, A, U^T and (bf16 inputs) the dO and v rows; rows past the end clamped
template <int D, typename TIO>
__device__ __forceinline__ void grads_prefetch(const Params& p, int L, char* sink) {
  constexpr bool kRows = !std::is_same<TIO, float>::value;
  constexpr int SR = D * 2 / 64;                                  // sectors per token row
  constexpr int NU = D * C * 2 / 64, NA = C * C * 2 / 64, NR = C * SR;
  constexpr int NTOT = 2 * NU + NA + (kRows ? 2 * NR : 0);
  int c, h;
  chunk_head_at(p, L, c, h);
  const ChunkEntry ce = p.ctab[c];
  const int64_t ch = int64_t(h) * p.NC + c;
  const char* dU = reinterpret_cast<const char*>(p.dU + ch * D * C);
  const char* A = reinterpret_cast<const char*>(p.A + ch * C * C);
  const char* U = reinterpret_cast<const char*>(p.U + ch * D * C);
  for (int u = threadIdx.x; u < NTOT; u += blockDim.x) {
    const char* a;
    if (u < NU) {
      a = dU + 64 * u;
    } else if (u < NU + NA) {
      a = A + 64 * (u - NU);
    } else if (u < 2 * NU + NA) {
      a = U + 64 * (u - NU - NA);
    } else {
      const int i = u - 2 * NU - NA, k = i % NR, row = min(k / SR, ce.len - 1);
      const void* base = i < NR ? p.dO : p.v;
      a = reinterpret_cast<const char*>(base) + tok(ce.t_start + row, p.H, h) * D * 2 + 64 * (k % SR);
    }
    dma4(a, sink);
  }
}

// phase-3 tiles (rb, sb), sb <= rb: slot 0 of every wave, slot 1 of waves 0 and 1
// (so that each SIMD gets two or three of the ten tiles)
__device__ __forceinline__ int g3_rb(int w, int slot) {
  return slot == 0 ? (w < 4 ? 3 : w < 7 ? 2 : 1) : (w == 0 ? 1 : 0);
}
__device__ __forceinline__ int g3_sb(int w, int slot) {
  return slot == 0 ? (w < 4 ? w : w < 7 ? w - 4 : 0) : (w == 0 ? 1 : 0);
}

template <int D, typename TIO>
__global__ __launch_bounds__(kGradThreads) void k_grads_gdn(const Params p) {
  using Ly = GradLds<D, TIO>;
  constexpr bool kDma = Ly::kDma;
  constexpr int NJB = D / 16, NJH = NJB / 2;                 // 16-wide blocks along D; per half
  constexpr int TPR = D / 8, RPP = kGradThreads / TPR, NPASS = C / RPP;   // row sweeps, 8 elements a thread
  static_assert(NPASS >= 1 && C % RPP == 0, "row sweep");
  __shared__ __attribute__((aligned(1024))) char Sx[Ly::TSx];         // S; phases 3-4: Kn, Qn
  __shared__ __attribute__((aligned(1024))) char dSx[Ly::TdSx];       // dS; phases 3-4: dME, dPE
  __shared__ __attribute__((aligned(1024))) char dUT[Ly::TU];         // phase 1: dU^T; then raw q
  __shared__ __attribute__((aligned(1024))) char At[Ly::TA];
  __shared__ __attribute__((aligned(1024))) char UT[Ly::TU];
  __shared__ __attribute__((aligned(1024))) char dOt[Ly::TR];
  __shared__ __attribute__((aligned(1024))) char dYt[Ly::TR];
  __shared__ __attribute__((aligned(1024))) char Vt[kDma ? Ly::TR : 16];   // phase 1: v; then raw k
  // per-row scalars: Gamma, 1/|q|, 1/|k|, beta (0 past the end)
  __shared__ __attribute__((aligned(256))) float sc_s[4][C];
  // fixed-order partial sums (deterministic): column sums of the pairwise dGamma
  // term per row block, row sums and dbeta per column half, phase-3 row sums per
  // column block (written for sb <= r / 16), the L2-norm dot products per half,
  // two per-wave chunk scalars
  __shared__ float colsum_s[4][C], rowsum_s[2][C], dbeta_s[2][C], rowq_s[4][C], rowb_s[4][C];
  __shared__ float l2_s[2][2][C], red_s[kGradWaves][2];
  const float* const gam_s = sc_s[0];
  const float* const rq_s = sc_s[1];
  const float* const rk_s = sc_s[2];
  const float* const beta_s = sc_s[3];

  int c, h;
  chunk_head(p, c, h);
  const ChunkEntry ce = p.ctab[c];
  const int t0 = ce.t_start, len = ce.len;
  const int tid = threadIdx.x, l = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rb = w & 3, hf = w >> 2;
  const int g = l >> 4, jj = l & 15;
  const int64_t ch = int64_t(h) * p.NC + c;
  const int H = p.H;
  const float scale = p.scale;
  char* const Kn = Sx;
  char* const Qn = Sx + Ly::TR;
  char* const dME = dSx;
  char* const dPE = dSx + Ly::TA;
  const int r = 16 * rb + jj;
  const int64_t trow = tok(t0 + min(r, len - 1), H, h) * D;
  auto u16 = [](const uint16_t* x) { return reinterpret_cast<const char*>(x); };
  auto row_of = [&](const void* x, int rr) {
    return reinterpret_cast<const char*>(x) + tok(t0 + min(rr, len - 1), H, h) * D * 2;
  };
  auto qk_row_of = [&](const void* x, int rr) {   // q, k rows (key head of this value head)
    return reinterpret_cast<const char*>(x) + qk_tok(p, t0 + min(rr, len - 1), h) * D * 2;
  };
  const int64_t qtrow = qk_tok(p, t0 + min(r, len - 1), h) * D;

  // ---- first group: per-row scalars, phase-1 tiles, dO (and v) ----
  if (w < 4)
    dma4(w == 0 ? static_cast<const void*>(p.gam + ch * C + l) : static_cast<const void*>(p.rho + (ch * 3 + w - 1) * C + l),
         reinterpret_cast<char*>(sc_s[w]));
  dma_tile<C, 1, D, kGradWaves>(dUT, [&](int v) { return u16(p.dU + (ch * D + v) * C); }, w);
  dma_tile<C, 0, C, kGradWaves>(At, [&](int rr) { return u16(p.A + (ch * C + rr) * C); }, w);
  dma_tile<C, 0, D, kGradWaves>(UT, [&](int v) { return u16(p.U + (ch * D + v) * C); }, w);
  if constexpr (kDma) {
    dma_tile<D, 0, C, kGradWaves>(dOt, [&](int rr) { return row_of(p.dO, rr); }, w);
    dma_tile<D, 0, C, kGradWaves>(Vt, [&](int rr) { return row_of(p.v, rr); }, w);
  }
  // ---- second group: S, dS ----
  dma_tile<D, 0, D, kGradWaves>(Sx, [&](int v) { return u16(p.S + (ch * D + v) * D); }, w);
  dma_tile<D, 0, D, kGradWaves>(dSx, [&](int v) { return u16(p.dS + (ch * D + v) * D); }, w);
  constexpr int G2 = 2 * DmaTile<D, D, kGradWaves>::kPerWave;   // loads of the second group per wave

  // fp32 inputs: dO rounded into its tile, v and raw q, k rows kept in registers
  typename IO<TIO>::Raw4 vraw[kDma ? 1 : NJH];
  typename IO<TIO>::Raw8 qraw[kDma ? 1 : NPASS], kraw[kDma ? 1 : NPASS];
  if constexpr (!kDma) {
#pragma unroll
    for (int q = 0; q < NJH; ++q) vraw[q] = IO<TIO>::load_raw4(p.v, trow + 16 * (hf * NJH + q) + 4 * g);
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int rr = ps * RPP + tid / TPR, c0 = (tid % TPR) * 8;
      const int64_t o = tok(t0 + min(rr, len - 1), H, h) * D + c0;
      const int64_t qo = qk_tok(p, t0 + min(rr, len - 1), h) * D + c0;
      qraw[ps] = IO<TIO>::load_raw8(p.q, qo);
      kraw[ps] = IO<TIO>::load_raw8(p.k, qo);
      float x[8];
      IO<TIO>::load8(p.dO, o, x);
      bf16x8 xb;
#pragma unroll
      for (int e = 0; e < 8; ++e) xb[e] = to_bf16(x[e]);
      *reinterpret_cast<bf16x8*>(dOt + soff<D>(rr, c0)) = xb;
    }
  }
  if (tid < C) {
#pragma unroll
    for (int x = 0; x < 4; ++x) colsum_s[x][tid] = 0.f;
  }
  if constexpr (kDma) wait_vm<G2>();   // the first group has landed
  else wait_vm<0>();
  chain_barrier();   // B_a

  // ---- phase 1: dY = A^T dU (lane owns dY[r][v .. v+3], r = 16 rb + jj, v in
  // this wave's half); dv; sum dY*v ----
  const float br = beta_s[r];
  float dbeta_row = 0.f, dgam_row = 0.f;
  f32x4 dvv[NJH];
#pragma unroll
  for (int q = 0; q < NJH; ++q) {
    const int vb = hf * NJH + q;
    f32x4 a = zero4();
#pragma unroll
    for (int k0 = 0; k0 < C; k0 += 32) a = mma(frag_rk_s<C, 1>(dUT, 16 * vb, k0), frag_kc_s<C, 0>(At, 16 * rb, k0), a);
    st4_q<D>(dYt, 16 * rb, 16 * vb, a[0], a[1], a[2], a[3]);
    // rows past the end: dY is exactly zero there, so the clamped v row adds nothing
    float vv[4];
    if constexpr (kDma) {
      const bf16x4 vb4 = ld4_q<D>(Vt, 16 * rb, 16 * vb);
#pragma unroll
      for (int i = 0; i < 4; ++i) vv[i] = float(vb4[i]);
    } else {
      IO<TIO>::unpack4(vraw[q], vv);
    }
    dbeta_row += a[0] * vv[0] + a[1] * vv[1] + a[2] * vv[2] + a[3] * vv[3];
    dvv[q] = a;
  }
  wait_vm<0>();
  chain_barrier();   // B_b: S, dS and all of dY in LDS; dU^T, A and v are no longer read

  // ---- raw q, k rows (bf16 inputs) into the freed dU^T and v tiles; dv ----
  if constexpr (kDma) {
    dma_tile<D, 0, C, kGradWaves>(dUT, [&](int rr) { return qk_row_of(p.q, rr); }, w);
    dma_tile<D, 0, C, kGradWaves>(Vt, [&](int rr) { return qk_row_of(p.k, rr); }, w);
  }
  if (r < len) {
#pragma unroll
    for (int q = 0; q < NJH; ++q)
      IO<TIO>::store4(p.dv, trow + 16 * (hf * NJH + q) + 4 * g, br * dvv[q][0], br * dvv[q][1], br * dvv[q][2],
                      br * dvv[q][3]);
  }

  // ---- phase 2: Z = dY S, dQbar = dO S, dKhat = U dS (transposed tiles), this
  // wave's column half ----
  f32x4 aZ[NJH], aQ[NJH], aK[NJH];
#pragma unroll
  for (int q = 0; q < NJH; ++q) {
    const int jb = hf * NJH + q;
    aZ[q] = aQ[q] = aK[q] = zero4();
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += 32) {
      const bf16x8 aS = frag_kc_s<D>(Sx, 16 * jb, k0);
      aZ[q] = mma(aS, frag_rk_s<D>(dYt, 16 * rb, k0), aZ[q]);
      aQ[q] = mma(aS, frag_rk_s<D>(dOt, 16 * rb, k0), aQ[q]);
      aK[q] = mma(frag_kc_s<D>(dSx, 16 * jb, k0), frag_kc_s<C, 0>(UT, 16 * rb, k0), aK[q]);
    }
  }
  // state term of dGamma_C: sum_{v,j} S dS, the trace of S dS^T taken over its
  // diagonal 16x16 blocks on MFMA (one block per wave; lane holds block rows
  // 4g+i, column jj)
  float sdot = 0.f;
  if (w < NJB) {
    const int vb = 16 * w;
    f32x4 t = zero4();
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += 32) t = mma(frag_rk_s<D>(Sx, vb, k0), frag_rk_s<D>(dSx, vb, k0), t);
#pragma unroll
    for (int i = 0; i < 4; ++i) sdot += 4 * g + i == jj ? t[i] : 0.f;
  }
  wait_vm<0>();
  chain_barrier();   // B_c: S and dS are no longer read; raw q, k in LDS

  // The workgroup dealt kGradAhead places later runs on this XCD (workgroups go
  // round-robin over the 8 XCDs) at about the time this one ends: pull its first
  // tile group into this XCD's L2 now, so that its start does not wait for HBM
  // (4-byte direct-to-LDS loads, one per 64-byte sector, into the A tile, which is
  // not read again; waited for at the end).  bf16 inputs only: with fp32 inputs
  // ordinary register loads follow, and their waits would take the prefetch along
  if constexpr (kDma) {
    if (const int L = blockIdx.x + p.NC * blockIdx.y + kGradAhead; L < p.NC * p.H)
      grads_prefetch<D, TIO>(p, L, At);
  }

  // ---- Kn, Qn (over S) ----
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int rr = ps * RPP + tid / TPR, c0 = (tid % TPR) * 8;
    float qv[8], kv[8];
    if constexpr (kDma) {
      const bf16x8 qb8 = *reinterpret_cast<const bf16x8*>(dUT + soff<D>(rr, c0));
      const bf16x8 kb8 = *reinterpret_cast<const bf16x8*>(Vt + soff<D>(rr, c0));
#pragma unroll
      for (int e = 0; e < 8; ++e) { qv[e] = float(qb8[e]); kv[e] = float(kb8[e]); }
    } else {
      IO<TIO>::unpack8(qraw[ps], qv);
      IO<TIO>::unpack8(kraw[ps], kv);
    }
    const float m = rr < len ? 1.f : 0.f;
    const float fq = m * rq_s[rr], fk = m * rk_s[rr];
    bf16x8 qb, kb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qb[e] = to_bf16(qv[e] * fq);
      kb[e] = to_bf16(kv[e] * fk);
    }
    *reinterpret_cast<bf16x8*>(Qn + soff<D>(rr, c0)) = qb;
    *reinterpret_cast<bf16x8*>(Kn + soff<D>(rr, c0)) = kb;
  }
  // dME, dPE start at zero: phase 3 writes only the tiles on and below the diagonal
  for (int o = 16 * tid; o < 2 * Ly::TA; o += 16 * kGradThreads) *reinterpret_cast<u32x4*>(dME + o) = u32x4{0u, 0u, 0u, 0u};
  chain_barrier();   // B_d

  // ---- fold the state-side terms (lane owns (r, j .. j+3), j in this wave's half) ----
  // dKbar = -beta Z, Kbar = kn e^Gam, Khat = kn e^(GamC-Gam), Qbar = scale qn e^Gam:
  //   dkn = -beta e^Gam Z + e^(GamC-Gam) dKhat,  dqn = scale e^Gam dQbar,
  //   dGam_r  += <kn, dkn> - 2 e^(GamC-Gam) <kn, dKhat> + <qn, dqn>,
  //   dbeta_r -= e^Gam <kn, Z>,   dGam_C += e^(GamC-Gam) <kn, dKhat>
  const float gr = gam_s[r];
  const float eg = fast_exp(gr), eh = fast_exp(gam_s[C - 1] - gr);
  const float cz = -br * eg, cq = scale * eg;
  float s_kdkn = 0.f, s_kdkh = 0.f, s_qdqn = 0.f, s_kz = 0.f;
  f32x4 dkn[NJH], dqn[NJH];
#pragma unroll
  for (int q = 0; q < NJH; ++q) {
    const int jc = 16 * (hf * NJH + q);
    const bf16x4 kb = ld4_q<D>(Kn, 16 * rb, jc);
    const bf16x4 qb = ld4_q<D>(Qn, 16 * rb, jc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float kn = float(kb[i]), qn = float(qb[i]);
      const float z = aZ[q][i], dkh = aK[q][i];
      dkn[q][i] = fmaf(cz, z, eh * dkh);
      dqn[q][i] = cq * aQ[q][i];
      s_kdkn = fmaf(kn, dkn[q][i], s_kdkn);
      s_kdkh = fmaf(kn, dkh, s_kdkh);
      s_qdqn = fmaf(qn, dqn[q][i], s_qdqn);
      s_kz = fmaf(kn, z, s_kz);
    }
  }
  dgam_row += s_kdkn - 2.f * eh * s_kdkh + s_qdqn;
  dbeta_row -= eg * s_kz;
  const float dgc_loc = eh * s_kdkh;

  // ---- phase 3: M, P, dP, dL on the 10 lower / diagonal tiles (tb, sb), slot 0
  // of every wave and slot 1 of waves 0, 1 (g3_rb / g3_sb).  Lane owns X[rr][s .. s+3],
  // rr = 16 tb + jj, s = 16 sb + 4g + i. ----
  float dme[2][4], dpe[2][4];
#pragma unroll
  for (int slot = 0; slot < 2; ++slot) {
    if (slot == 1 && w >= 2) break;
    const int tb = g3_rb(w, slot), sb = g3_sb(w, slot);
    const int rr = 16 * tb + jj, s0 = 16 * sb + 4 * g;
    f32x4 G1 = zero4(), G2 = zero4(), Mr = zero4(), Pr = zero4();
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += 32) {
      const bf16x8 aU = frag_kc_s<C, 0>(UT, 16 * sb, k0);
      G1 = mma(aU, frag_rk_s<D>(dOt, 16 * tb, k0), G1);
      G2 = mma(aU, frag_rk_s<D>(dYt, 16 * tb, k0), G2);
      const bf16x8 aK = frag_rk_s<D>(Kn, 16 * sb, k0);
      Mr = mma(aK, frag_rk_s<D>(Kn, 16 * tb, k0), Mr);
      Pr = mma(aK, frag_rk_s<D>(Qn, 16 * tb, k0), Pr);
    }
    const float grr = gam_s[rr], brr = beta_s[rr];
    float rq = 0.f, rbt = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = s0 + i;
      // Gamma is non-increasing, so the exponent is <= 0 wherever it is used
      const float E = fast_exp(fminf(grr - gam_s[s], 0.f));
      const float le = rr >= s ? 1.f : 0.f, lt = rr > s ? 1.f : 0.f;
      const float dP = G1[i];
      const float M = lt * Mr[i] * E;
      const float dL = -G2[i];
      const float dM = brr * dL;
      const float qv = le * dP * scale * Pr[i] * E + dM * M;
      dpe[slot][i] = le * scale * dP * E;
      dme[slot][i] = lt * dM * E;
      rbt = fmaf(dL, M, rbt);
      rq += qv;
      // column sum over the 16 rows of the tile
      const float col = row16_sum(qv);
      if (jj == 0) colsum_s[tb][s] = -col;
    }
    // row sums over the 16 columns of the tile
    rq = xrow_sum(rq);
    rbt = xrow_sum(rbt);
    if (g == 0) {
      rowq_s[sb][rr] = rq;
      rowb_s[sb][rr] = rbt;
    }
  }
#pragma unroll
  for (int slot = 0; slot < 2; ++slot) {
    if (slot == 0 || w < 2) {
      const int r0 = 16 * g3_rb(w, slot), c0 = 16 * g3_sb(w, slot);
      st4_q<C, 0>(dME, r0, c0, dme[slot][0], dme[slot][1], dme[slot][2], dme[slot][3]);
      st4_q<C, 0>(dPE, r0, c0, dpe[slot][0], dpe[slot][1], dpe[slot][2], dpe[slot][3]);
    }
  }
  // raw q, k of this lane's outputs, for the L2-norm backward at the end
  typename IO<TIO>::Raw4 qo[kDma ? 1 : NJH], ko[kDma ? 1 : NJH];
  if constexpr (!kDma) {
#pragma unroll
    for (int q = 0; q < NJH; ++q) {
      qo[q] = IO<TIO>::load_raw4(p.q, qtrow + 16 * (hf * NJH + q) + 4 * g);
      ko[q] = IO<TIO>::load_raw4(p.k, qtrow + 16 * (hf * NJH + q) + 4 * g);
    }
  }
  chain_barrier();   // B_e: dME, dPE complete

  // ---- phase 4: pairwise terms, dkn += (dME + dME^T) Kn + scale dPE^T Qn, dqn += scale dPE Kn ----
#pragma unroll
  for (int q = 0; q < NJH; ++q) {
    const int jb = hf * NJH + q;
#pragma unroll
    for (int k0 = 0; k0 < C; k0 += 32) {
      const bf16x8 aK = frag_kc_s<D>(Kn, 16 * jb, k0);
      const bf16x8 aQ2 = frag_kc_s<D>(Qn, 16 * jb, k0);
      dkn[q] = mma(aK, frag_rk_s<C, 0>(dME, 16 * rb, k0), dkn[q]);
      dkn[q] = mma(aK, frag_kc_s<C, 0>(dME, 16 * rb, k0), dkn[q]);
      dkn[q] = mma(aQ2, frag_kc_s<C, 0>(dPE, 16 * rb, k0), dkn[q]);
      dqn[q] = mma(aK, frag_rk_s<C, 0>(dPE, 16 * rb, k0), dqn[q]);
    }
  }
  // ---- L2-norm backward: dq = rq (dqn - qn <qn, dqn>), dk likewise (K1 page, 3.3);
  // the dot products add the two column halves ----
  const float m = r < len ? 1.f : 0.f;
  const float rq = m * rq_s[r], rk = m * rk_s[r];
  float qn[NJH][4], kn[NJH][4];
  {
    float pq = 0.f, pk = 0.f;
#pragma unroll
    for (int q = 0; q < NJH; ++q) {
      if constexpr (kDma) {
        const bf16x4 q4 = ld4_q<D>(dUT, 16 * rb, 16 * (hf * NJH + q));
        const bf16x4 k4 = ld4_q<D>(Vt, 16 * rb, 16 * (hf * NJH + q));
#pragma unroll
        for (int i = 0; i < 4; ++i) { qn[q][i] = float(q4[i]); kn[q][i] = float(k4[i]); }
      } else {
        IO<TIO>::unpack4(qo[q], qn[q]);
        IO<TIO>::unpack4(ko[q], kn[q]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qn[q][i] *= rq;
        kn[q][i] *= rk;
        pq += qn[q][i] * dqn[q][i];
        pk += kn[q][i] * dkn[q][i];
      }
    }
    pq = xrow_sum(pq);
    pk = xrow_sum(pk);
    if (g == 0) {
      l2_s[hf][0][r] = pq;
      l2_s[hf][1][r] = pk;
    }
  }
  // ---- row and chunk reductions ----
  dgam_row = xrow_sum(dgam_row);
  dbeta_row = xrow_sum(dbeta_row);
  if (g == 0) {
    rowsum_s[hf][r] = dgam_row;
    dbeta_s[hf][r] = dbeta_row;
  }
  const float tot = wave_sum(dgc_loc);
  const float st = wave_sum(sdot);
  if (l == 0) {
    red_s[w][0] = tot;
    red_s[w][1] = st;
  }
  chain_barrier();   // B_f
  {
    const float pq = l2_s[0][0][r] + l2_s[1][0][r], pk = l2_s[0][1][r] + l2_s[1][1][r];
    if constexpr (kDma) {
      // bf16 rows go out through LDS (the dO and dY tiles are free now), below
#pragma unroll
      for (int q = 0; q < NJH; ++q) {
        const int jc = 16 * (hf * NJH + q);
        st4_q<D>(dOt, 16 * rb, jc, rq * (dqn[q][0] - qn[q][0] * pq), rq * (dqn[q][1] - qn[q][1] * pq),
                 rq * (dqn[q][2] - qn[q][2] * pq), rq * (dqn[q][3] - qn[q][3] * pq));
        st4_q<D>(dYt, 16 * rb, jc, rk * (dkn[q][0] - kn[q][0] * pk), rk * (dkn[q][1] - kn[q][1] * pk),
                 rk * (dkn[q][2] - kn[q][2] * pk), rk * (dkn[q][3] - kn[q][3] * pk));
      }
    } else if (r < len) {
#pragma unroll
      for (int q = 0; q < NJH; ++q) {
        const int64_t o = trow + 16 * (hf * NJH + q) + 4 * g;
        IO<TIO>::store4(p.dq, o, rq * (dqn[q][0] - qn[q][0] * pq), rq * (dqn[q][1] - qn[q][1] * pq),
                        rq * (dqn[q][2] - qn[q][2] * pq), rq * (dqn[q][3] - qn[q][3] * pq));
        IO<TIO>::store4(p.dk, o, rk * (dkn[q][0] - kn[q][0] * pk), rk * (dkn[q][1] - kn[q][1] * pk),
                        rk * (dkn[q][2] - kn[q][2] * pk), rk * (dkn[q][3] - kn[q][3] * pk));
      }
    }
  }
  if (w == 0) {
    // dlam_s = sum_{r >= s} dGam_r + dGamC (suffix sum; FlashKDA backward page, section 5)
    float rs = 0.f, ss = 0.f;
#pragma unroll
    for (int x = 0; x < kGradWaves; ++x) {
      rs += red_s[x][0];
      ss += red_s[x][1];
    }
    const float dgc = rs + ss * fast_exp(gam_s[C - 1]);
    float x = (rowsum_s[0][l] + rowsum_s[1][l]) + ((colsum_s[0][l] + colsum_s[1][l]) + (colsum_s[2][l] + colsum_s[3][l]));
    float dbt = dbeta_s[0][l] + dbeta_s[1][l];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {   // entries exist for sb <= l / 16 only
      x += sb <= (l >> 4) ? rowq_s[sb][l] : 0.f;
      dbt += sb <= (l >> 4) ? rowb_s[sb][l] : 0.f;
    }
    // suffix sums inside each 16-lane row (DPP shifts toward lower lanes, zero
    // filled), then the totals of the rows above
#pragma unroll
    for (int sh = 1; sh < 16; sh <<= 1) {
      const float y = sh == 1 ? dpp_f<0x101>(x) : sh == 2 ? dpp_f<0x102>(x) : sh == 4 ? dpp_f<0x104>(x) : dpp_f<0x108>(x);
      x += (l & 15) + sh < 16 ? y : 0.f;
    }
    const float t1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
    const float t2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
    const float t3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
    x += g == 0 ? t1 + (t2 + t3) : g == 1 ? t2 + t3 : g == 2 ? t3 : 0.f;
    if (l < len) {
      const int64_t o = tok(t0 + l, H, h);
      const float bt = beta_s[l];   // sigma(b) on valid rows
      IO<TIO>::store1(p.dg, o, x + dgc);
      IO<TIO>::store1(p.db, o, dbt * bt * (1.f - bt));
    }
  }
  if constexpr (kDma) {
    chain_barrier();   // B_g: dq, dk rows staged
    // dq, dk rows: 1 KB (four rows) per wave instruction, 16 bytes per lane
#pragma unroll
    for (int it = 0; it < Ly::TR / 1024 / kGradWaves; ++it) {
      const int pos = (w + kGradWaves * it) * 1024 + 16 * l;
      const int row = pos / (2 * D), c0 = (pos % (2 * D)) / 2;
      if (row < len) {
        const int64_t o = tok(t0 + row, H, h) * D + c0;
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.dq) + o) = *reinterpret_cast<const u32x4*>(dOt + soff<D>(row, c0));
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.dk) + o) = *reinterpret_cast<const u32x4*>(dYt + soff<D>(row, c0));
      }
    }
  }
  wait_vm<0>();   // the prefetch's direct-to-LDS loads land before the workgroup's LDS is released
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
    k_prep_gdn<D, TIO><<<dim3(p.NC, p.H), kPrepThreads, 0, s>>>(p);
  }
};
template <int D, typename TIO>
struct RunGrads {
  static void run(const Params& p, hipStream_t s) {
    k_grads_gdn<D, TIO><<<dim3(p.NC, p.H), kGradThreads, 0, s>>>(p);
  }
};
}  // namespace

int launch_prep(const Params& p, void* stream) { return dispatch<RunPrep>(p, stream); }
int launch_grads(const Params& p, void* stream) { return dispatch<RunGrads>(p, stream); }
int launch_zero_params(const Params& p, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (p.dA_log) k_zero<<<(p.H + 255) / 256, 256, 0, s>>>(p.dA_log, p.H);
  if (p.ddt_bias) k_zero<<<(p.H * p.K + 255) / 256, 256, 0, s>>>(p.ddt_bias, p.H * p.K);
  return last_error();
}
const char* hip_error_string(int err) { return hipGetErrorString(static_cast<hipError_t>(err)); }

}  // namespace gdr

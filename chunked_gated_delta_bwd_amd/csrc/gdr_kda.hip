// HIP kernels for gfx950: the chunk-parallel parts of the per-channel (KDA) gate.
//
// The gate is lambda = -exp(A_log) softplus(g_raw + dt_bias), or in the bounded
// form lambda = gate_scale sigmoid(exp(A_log) (g_raw + dt_bias)), one value per
// token, head and key channel (FlashKDA backward (K1) page, section 5).  Its in-chunk
// cumsum Gamma is per channel, so the decay between rows r and s of a chunk is
// the per-channel factor E_rsc = exp(Gamma_rc - Gamma_sc) inside every
// contraction over channels:
//   M_rs = sum_c kn_rc kn_sc E_rsc,   P_rs = scale sum_c qn_rc kn_sc E_rsc.
// Between different 16-row blocks the factor splits at a reference row that lies
// between them, E = exp(Gamma_r - Gamma_ref) exp(Gamma_ref - Gamma_s) with both
// exponents <= 0 (Gamma never increases), so those blocks go to MFMA on operands
// scaled in registers; inside a diagonal 16-row block it splits at the block's
// middle row (factors bounded by the half-spans of the block, fp32 MFMA), and a
// channel whose half-span is too wide for that is evaluated exactly per element.
// The chunk recursions then take materialised Khat = kn e^(GamC - Gam), Qbar =
// scale qn e^Gam (high + low bf16 parts) and the per-channel chunk decay.
//
//   k_prep_kda    per (chunk, head): norms, gate and its cumsum, M and P, the
//                 UT/WY inverse, W and U', Khat / Qbar tiles, chunk decay.
//   k_grads_kda   per (chunk, head): the chunk-local gradients; the pairwise
//                 terms are four E-weighted products (row and column sides of
//                 dM o E and dP o E) on K = 16 MFMAs plus the diagonal blocks
//                 on fp32 MFMA (exactly where their decay is too steep); then,
//                 fused, the prepare-backward: L2-norm and sigmoid backward, the
//                 per-channel reverse cumsum of dGamma plus the chunk-total term,
//                 the gate backward, per-chunk partial sums of dA_log, ddt_bias.
//   k_params_kda  per head: the partial sums reduced in a fixed order.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gdr_device.h"
#include "gdr_internal.h"
#include "gdr_lds.h"

namespace gdr {

// The per-channel gate function of x = g_raw + dt_bias, with ea = e^A_log:
//   softplus form         lambda = -ea softplus(x)
//   bounded sigmoid form  lambda = gate_scale sigmoid(ea x)
__device__ __forceinline__ float gate_lambda(const Params& p, float ea, float x) {
  return p.gate_fn ? p.gate_scale * sigmoidf(ea * x) : -ea * softplusf(x);
}

namespace {

typedef short s16x4v __attribute__((ext_vector_type(4)));

// largest exponent of a factor of the in-block decay (per channel) for which a
// diagonal 16-row block is factored at its middle row: the factors e^(Gam_r - Gam_m)
// and e^(Gam_m - Gam_s) and their products stay normal fp32 numbers far from
// overflow and underflow
constexpr float kSpanMax = 60.f;

// v_mfma_f32_16x16x16_bf16: A lane (m = l % 16, k = 4 (l / 16) .. +3),
// B lane (k = 4 (l / 16) .. +3, n = l % 16), C as for the K = 32 form.
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4v, a), __builtin_bit_cast(s16x4v, b), c, 0,
                                                   0, 0);
}

// K = 16 fragment of a tile stored T[k][col]: lane gets T[k0 + 4g .. +3][c0 + j]
// (one transposed read; lane q addresses row k0 + 4g + q/4, columns c0 + 4(q%4)).
__device__ __forceinline__ bf16x4 frag16_kc(const bf16* T, int P, int c0, int k0) {
  const int l = lane_id();
  const int g = l >> 4, q = l & 15;
  const bf16* p0 = T + (k0 + 4 * g + (q >> 2)) * P + c0 + 4 * (q & 3);
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((lds_short*)(p0)));
  return __builtin_bit_cast(bf16x4, v);
}

// K = 16 fragment of a tile stored T[row][k]: lane gets T[r0 + j][k0 + 4g .. +3]
__device__ __forceinline__ bf16x4 frag16_rk(const bf16* T, int P, int r0, int k0) {
  const int l = lane_id();
  return *reinterpret_cast<const bf16x4*>(T + (r0 + (l & 15)) * P + k0 + 4 * (l >> 4));
}

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float el(const float4& v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

}  // namespace

// ===========================================================================
// k_prep_kda
// ===========================================================================
// the prologue runs eight waves (two per SIMD)
constexpr int kKdaPrepThreads = 2 * kThreads;

template <int D, typename TIO>
__global__ __launch_bounds__(kKdaPrepThreads) void k_prep_kda(const Params p) {
  using Dm = Dims<D>;
  constexpr int PD = Dm::PD, TPR = Dm::TPR;
  constexpr int kT = kKdaPrepThreads;
  constexpr int RPP = kT / TPR, NPASS = C / RPP;   // row sweeps of 8 channels a thread
  constexpr int NPART = kT / D, RP = C / NPART;    // per-channel scans: row ranges per channel
  constexpr int PL = C + 4, PG = D + 4;
  constexpr int kQX = C * PD * 2 > C * PL * 4 ? C * PD * 2 : C * PL * 4;
  __shared__ __attribute__((aligned(16))) char QX[kQX];   // Qn; from the inverse on: X = A, fp32
  bf16* const Qs = reinterpret_cast<bf16*>(QX);
  float* const Xf = reinterpret_cast<float*>(QX);
  __shared__ __attribute__((aligned(16))) bf16 Ks[C * PD];
  __shared__ __attribute__((aligned(16))) bf16 Vs[C * PD];
  __shared__ __attribute__((aligned(16))) bf16 As[C * PC];
  __shared__ __attribute__((aligned(16))) float Lf[C * PL];
  __shared__ __attribute__((aligned(16))) float Gs[C * PG];   // Gamma [r][c]
  // low bf16 parts of A and beta V: U' = A beta V is formed to ~fp32 accuracy
  __shared__ __attribute__((aligned(16))) bf16 Asl[C * PC];
  __shared__ __attribute__((aligned(16))) bf16 Vsl[C * PD];
  __shared__ float beta_s[C], tot_s[NPART][D];
  // bf16 inputs: Ks, Qs hold the raw k, q rows (exact in bf16) until the M, P
  // blocks are formed, and these the row norms 1/|k|, 1/|q| (kn = k / |k| in fp32);
  // fp32 inputs: kn, qn in bf16 and factors 1.  They share space with Asl, which
  // is written only later.
  constexpr bool kRawRows = !std::is_same<TIO, float>::value;
  float* const rk_s = reinterpret_cast<float*>(Asl);
  float* const rq_s = rk_s + C;
  static_assert(2 * C * 4 <= C * PC * 2, "row norms fit in Asl");

  int c, h;
  chunk_head(p, c, h);
  const ChunkEntry ce = p.ctab[c];
  const int t0 = ce.t_start, len = ce.len;
  const int tid = threadIdx.x, l = lane_id(), w = wave_id();
  // eight waves: wave w works on row block rb = w % 4; the two waves of a row block
  // (w, w + 4: one SIMD) split its work where it splits, else the first one works
  const int rb = __builtin_amdgcn_readfirstlane(w & 3), hf = __builtin_amdgcn_readfirstlane(w >> 2);
  const int g = l >> 4, jj = l & 15;
  const int64_t ch = int64_t(h) * p.NC + c;
  const int H = p.H;
  const float scale = p.scale;

  // --- rows: every load issued first (unconditional, from a clamped row, masked
  // afterwards), so that their latencies overlap: q, k, v, the raw gate, beta ---
  typename IO<TIO>::Raw8 qraw[NPASS], kraw[NPASS], vraw[NPASS], graw[NPASS];
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int r = ps * RPP + tid / TPR, c0 = (tid % TPR) * 8;
    const int64_t off = tok(t0 + min(r, len - 1), H, h) * D + c0;
    const int64_t qoff = qk_tok(p, t0 + min(r, len - 1), h) * D + c0;
    qraw[ps] = IO<TIO>::load_raw8(p.q, qoff);
    kraw[ps] = IO<TIO>::load_raw8(p.k, qoff);
    vraw[ps] = IO<TIO>::load_raw8(p.v, off);
    graw[ps] = IO<TIO>::load_raw8(p.g, off);
  }
  const int cg0 = (tid % TPR) * 8;   // this thread's 8 channels in the row sweeps
  const float4 bias0 = ld4(p.dt_bias + h * D + cg0), bias1 = ld4(p.dt_bias + h * D + cg0 + 4);
  const float ea = fast_exp(p.A_log[h]);
  float braw = 0.f;
  if (tid >= kT - C) braw = IO<TIO>::load1(p.b, tok(t0 + min(tid - (kT - C), len - 1), H, h));

  // --- L2 norms; qn, kn to LDS; kn, qn, v kept in registers; the log decay
  // lambda = gate_lambda(g + dt_bias) (0 past the end) to Gs ---
  float kn_r[NPASS][8], qn_r[NPASS][8], v_r[NPASS][8];
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int r = ps * RPP + tid / TPR, c0 = cg0;
    float qv[8], kv[8], gv[8];
    IO<TIO>::unpack8(qraw[ps], qv);
    IO<TIO>::unpack8(kraw[ps], kv);
    IO<TIO>::unpack8(vraw[ps], v_r[ps]);
    IO<TIO>::unpack8(graw[ps], gv);
    const float m = r < len ? 1.f : 0.f;
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qv[e] *= m;
      kv[e] *= m;
      v_r[ps][e] *= m;
      sq += qv[e] * qv[e];
      sk += kv[e] * kv[e];
      gv[e] = m * gate_lambda(p, ea, gv[e] + (e < 4 ? el(bias0, e) : el(bias1, e - 4)));
    }
    *reinterpret_cast<float4*>(Gs + r * PG + c0) = make_float4(gv[0], gv[1], gv[2], gv[3]);
    *reinterpret_cast<float4*>(Gs + r * PG + c0 + 4) = make_float4(gv[4], gv[5], gv[6], gv[7]);
    sq = group_sum_dpp<TPR>(sq);
    sk = group_sum_dpp<TPR>(sk);
    const float rq = 1.0f / sqrtf(sq + 1e-6f), rk = 1.0f / sqrtf(sk + 1e-6f);
    bf16x8 qb, kb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kn_r[ps][e] = kv[e] * rk;
      qn_r[ps][e] = qv[e] * rq;
      qb[e] = to_bf16(kRawRows ? qv[e] : qn_r[ps][e]);
      kb[e] = to_bf16(kRawRows ? kv[e] : kn_r[ps][e]);
    }
    *reinterpret_cast<bf16x8*>(Qs + r * PD + c0) = qb;
    *reinterpret_cast<bf16x8*>(Ks + r * PD + c0) = kb;
    if (tid % TPR == 0) {
      rk_s[r] = kRawRows ? rk : 1.f;
      rq_s[r] = kRawRows ? rq : 1.f;
      p.rho[ch * 3 * C + r] = rq;
      p.rho[ch * 3 * C + C + r] = rk;
    }
  }
  if (tid >= kT - C) {
    const int r = tid - (kT - C);
    const float bt = (r < len ? 1.f : 0.f) * sigmoidf(braw);
    beta_s[r] = bt;
    p.rho[ch * 3 * C + 2 * C + r] = bt;
  }
  __syncthreads();
  // --- in-chunk cumsum Gamma per channel: thread = (channel, one of NPART row
  // ranges) scans its range in registers, then adds the totals of the ranges before ---
  {
    const int cc = tid % D, part = tid / D;
    float x[RP];
#pragma unroll
    for (int i = 0; i < RP; ++i) x[i] = Gs[(part * RP + i) * PG + cc];
#pragma unroll
    for (int i = 1; i < RP; ++i) x[i] += x[i - 1];
    tot_s[part][cc] = x[RP - 1];
    __syncthreads();
    float before = 0.f;
#pragma unroll
    for (int q = 0; q < NPART - 1; ++q) before += q < part ? tot_s[q][cc] : 0.f;
#pragma unroll
    for (int i = 0; i < RP; ++i) {
      const float v = x[i] + before;
      // kept in base-2 units (log2(e) Gamma) from here on: every use below is an
      // exponent of 2; the workspace copy is Gamma itself
      Gs[(part * RP + i) * PG + cc] = kLog2e * v;
      p.gam[(ch * C + part * RP + i) * D + cc] = v;
    }
  }
  __syncthreads();

  // --- M and P between blocks (the second waves of the row blocks): block (R, sb),
  // sb < R, rows 16R.., reference row 16R (so both factors are <= 1); lane owns
  // M[r][s .. s+3].  The operands kn e^(Gam - Gam_ref) and qn e^(Gam - Gam_ref)
  // are formed in fp32 and taken in two bf16 parts (products hi hi + lo hi + hi
  // lo): the gate-parameter gradients sum terms that cancel strongly, and these
  // blocks' bf16 roundings are among the largest terms of their error.  The six
  // blocks are dealt two, two, one and one to the four waves, the pairs sharing
  // their row operands: (3,0) (3,1) | (2,0) (2,1) | (3,2) | (1,0) ---
  if (hf == 1) {
    const int R = rb == 0 || rb == 2 ? 3 : rb == 1 ? 2 : 1;
    const int sb0 = rb == 2 ? 2 : 0, nsb = rb < 2 ? 2 : 1;
    const int r = 16 * R + jj;
    f32x4 aM[2], aP[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) aM[x] = aP[x] = zero4();
    const float rkr = rk_s[r], rqr = rq_s[r];
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += 32) {
      const int c0 = k0 + 8 * g;
      const float4 gr0 = ld4(Gs + r * PG + c0), gr1 = ld4(Gs + r * PG + c0 + 4);
      const float4 gf0 = ld4(Gs + 16 * R * PG + c0), gf1 = ld4(Gs + 16 * R * PG + c0 + 4);
      const bf16x8 kr = *reinterpret_cast<const bf16x8*>(Ks + r * PD + c0);
      const bf16x8 qr = *reinterpret_cast<const bf16x8*>(Qs + r * PD + c0);
      bf16x8 bk, bq, bkl, bql;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = fast_exp2(e < 4 ? el(gr0, e) - el(gf0, e) : el(gr1, e - 4) - el(gf1, e - 4));
        const float xk = float(kr[e]) * (rkr * d), xq = float(qr[e]) * (rqr * d);
        bk[e] = to_bf16(xk);
        bq[e] = to_bf16(xq);
        bkl[e] = to_bf16(xk - float(bk[e]));
        bql[e] = to_bf16(xq - float(bq[e]));
      }
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        if (x < nsb) {
          const int s = 16 * (sb0 + x) + jj;
          const float4 gs0 = ld4(Gs + s * PG + c0), gs1 = ld4(Gs + s * PG + c0 + 4);
          const bf16x8 ks = *reinterpret_cast<const bf16x8*>(Ks + s * PD + c0);
          const float rks = rk_s[s];
          bf16x8 ak, akl;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float d = fast_exp2(e < 4 ? el(gf0, e) - el(gs0, e) : el(gf1, e - 4) - el(gs1, e - 4));
            const float xs = float(ks[e]) * (rks * d);
            ak[e] = to_bf16(xs);
            akl[e] = to_bf16(xs - float(ak[e]));
          }
          aM[x] = mma(ak, bk, aM[x]);
          aM[x] = mma(akl, bk, aM[x]);
          aM[x] = mma(ak, bkl, aM[x]);
          aP[x] = mma(ak, bq, aP[x]);
          aP[x] = mma(akl, bq, aP[x]);
          aP[x] = mma(ak, bql, aP[x]);
        }
      }
    }
    const float br = beta_s[r];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      if (x < nsb) {
        const int s0 = 16 * (sb0 + x) + 4 * g;
        float Lv[4], Pv[4], Mv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Mv[i] = aM[x][i];
          Pv[i] = scale * aP[x][i];
          Lv[i] = br * Mv[i];
        }
        *reinterpret_cast<float4*>(Lf + r * PL + s0) = make_float4(Lv[0], Lv[1], Lv[2], Lv[3]);
        st_bf16x4(p.P + (ch * C + r) * C + s0, Pv[0], Pv[1], Pv[2], Pv[3]);
        st_bf16x4(p.Mk + (ch * C + r) * C + s0, Mv[0], Mv[1], Mv[2], Mv[3]);
      }
    }
    // the zero blocks above the diagonal of row block rb
    const int rz = 16 * rb + jj;
    for (int sb = rb + 1; sb < 4; ++sb) {
      const int s0 = 16 * sb + 4 * g;
      *reinterpret_cast<float4*>(Lf + rz * PL + s0) = make_float4(0.f, 0.f, 0.f, 0.f);
      st_bf16x4(p.P + (ch * C + rz) * C + s0, 0.f, 0.f, 0.f, 0.f);
      st_bf16x4(p.Mk + (ch * C + rz) * C + s0, 0.f, 0.f, 0.f, 0.f);
    }
  }
  // --- diagonal blocks: wave R's block factored at its middle row m = f + 8,
  // E_rs = e^(Gam_r - Gam_m) e^(Gam_m - Gam_s), on 16x16x4 fp32 MFMA with fp32
  // operands (contraction over channels; lane group g takes channels g D/4 .. +D/4).
  // Every factor's exponent is bounded by the larger half-span of the block in its
  // channel, max(Gam_f - Gam_m, Gam_m - Gam_(f+15)); a channel where that reaches
  // kSpanMax is left out of the products (its operands are zero) and added exactly,
  // one channel at a time, thread owns row r and four columns s (the first wave
  // of each row block) ---
  if (hf == 0) {
    const int f = 16 * rb, m = f + 8, rr = f + jj;
    auto wide_ch = [&](int cc) {
      const float gm = Gs[m * PG + cc];
      return fmaxf(Gs[f * PG + cc] - gm, gm - Gs[(f + 15) * PG + cc]) >= kLog2e * kSpanMax;
    };
    // wave-uniform masks of the wide channels: lane l tests channels l and 64 + l
    const uint64_t wide0 = __builtin_amdgcn_ballot_w64(wide_ch(l));
    uint64_t wide1 = 0;
    if constexpr (D > 64) wide1 = __builtin_amdgcn_ballot_w64(wide_ch(64 + l));
    f32x4 aM = zero4(), aP = zero4();
    const float rkr = rk_s[rr], rqr = rq_s[rr];
#pragma unroll
    for (int kq = 0; kq < D / 16; ++kq) {
      const int c4 = (D / 4) * g + 4 * kq;
      const float4 gr4 = ld4(Gs + rr * PG + c4), gm4 = ld4(Gs + m * PG + c4);
      const bf16x4 k4 = *reinterpret_cast<const bf16x4*>(Ks + rr * PD + c4);
      const bf16x4 q4 = *reinterpret_cast<const bf16x4*>(Qs + rr * PD + c4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int cc = c4 + e;
        const bool wd = ((cc < 64 ? wide0 >> cc : wide1 >> (cc & 63)) & 1) != 0;
        const float ea = wd ? 0.f : fast_exp2(el(gr4, e) - el(gm4, e));   // row as r
        const float eb = wd ? 0.f : fast_exp2(el(gm4, e) - el(gr4, e));   // row as s
        const float kn = float(k4[e]) * rkr;
        aM = mma_f32(kn * eb, kn * ea, aM);
        aP = mma_f32(kn * eb, float(q4[e]) * rqr * ea, aP);
      }
    }
    const int s0 = f + 4 * g;
    // the wide channels, exactly: E = exp(-|Gamma_r - Gamma_s|) (Gamma does not increase)
    uint64_t rest0 = wide0, rest1 = wide1;
    while (rest0 | rest1) {
      int cc;
      if (rest0) {
        cc = __builtin_ctzll(rest0);
        rest0 &= rest0 - 1;
      } else {
        cc = 64 + __builtin_ctzll(rest1);
        rest1 &= rest1 - 1;
      }
      const float gr = Gs[rr * PG + cc], kr = float(Ks[rr * PD + cc]) * rkr, qr = float(Qs[rr * PD + cc]) * rqr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int sc = s0 + i;
        const float kk = float(Ks[sc * PD + cc]) * rk_s[sc] * fast_exp2(-fabsf(gr - Gs[sc * PG + cc]));
        aM[i] += kr * kk;
        aP[i] += qr * kk;
      }
    }
    const float br = beta_s[rr];
    float Mv[4], Pv[4], Lv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sc = s0 + i;
      Mv[i] = sc < rr ? aM[i] : 0.f;
      Pv[i] = sc <= rr ? scale * aP[i] : 0.f;
      Lv[i] = br * Mv[i];
    }
    *reinterpret_cast<float4*>(Lf + rr * PL + s0) = make_float4(Lv[0], Lv[1], Lv[2], Lv[3]);
    st_bf16x4(p.P + (ch * C + rr) * C + s0, Pv[0], Pv[1], Pv[2], Pv[3]);
    st_bf16x4(p.Mk + (ch * C + rr) * C + s0, Mv[0], Mv[1], Mv[2], Mv[3]);
  }
  __syncthreads();

  // --- beta Kbar (Kbar = kn e^Gam) and beta V overwrite the operand tiles; the
  // recursions' Khat / Qbar tiles and the chunk decay go to the workspace; a weak
  // chunk (some channel decays by less than kTwoPartDecay) also Khat's low part ---
  int wf = 0;
  for (int j = l; j < D; j += 64) wf |= fast_exp2(Gs[(C - 1) * PG + j]) >= kTwoPartDecay;
  const bool weak = __any(wf);
  if (tid == 0) p.weak[ch] = weak ? 1 : 0;
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int r = ps * RPP + tid / TPR, c0 = (tid % TPR) * 8;
    const float fb = beta_s[r];
    bf16x8 kb, vb, vl, kh, khl, qh, ql;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float gr = Gs[r * PG + c0 + e], gC = Gs[(C - 1) * PG + c0 + e];
      const float eg = fast_exp2(gr), eh = fast_exp2(gC - gr);
      kb[e] = to_bf16(fb * kn_r[ps][e] * eg);
      const float bv = fb * v_r[ps][e];
      vb[e] = to_bf16(bv);
      vl[e] = to_bf16(bv - float(vb[e]));
      const float kx = kn_r[ps][e] * eh;
      kh[e] = to_bf16(kx);
      khl[e] = to_bf16(kx - float(kh[e]));
      const float x = scale * qn_r[ps][e] * eg;
      qh[e] = to_bf16(x);
      ql[e] = to_bf16(x - float(qh[e]));
    }
    *reinterpret_cast<bf16x8*>(Ks + r * PD + c0) = kb;
    *reinterpret_cast<bf16x8*>(Vs + r * PD + c0) = vb;
    *reinterpret_cast<bf16x8*>(Vsl + r * PD + c0) = vl;
    const int64_t o = (ch * C + r) * D + c0;
    *reinterpret_cast<bf16x8*>(p.Kh + o) = kh;
    if (weak) *reinterpret_cast<bf16x8*>(p.Khl + o) = khl;
    *reinterpret_cast<bf16x8*>(p.Qh + o) = qh;
    *reinterpret_cast<bf16x8*>(p.Ql + o) = ql;
  }
  if (tid < D) p.edec[ch * D + tid] = fast_exp2(Gs[(C - 1) * PG + tid]);

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
  // --- A out: high and low bf16 parts for the W, U' products, the high part to the
  // workspace; the blocks above the diagonal are zero ---
#pragma unroll
  for (int it = 0; it < C * C / 8 / kT; ++it) {
    const int idx = tid + kT * it, row = idx / 8, c8 = (idx % 8) * 8;
    const bool on = (c8 >> 4) <= (row >> 4);
    bf16x8 vh, vl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = on ? Xf[row * PL + c8 + e] : 0.f;
      vh[e] = to_bf16(x);
      vl[e] = to_bf16(x - float(vh[e]));
    }
    *reinterpret_cast<bf16x8*>(As + row * PC + c8) = vh;
    *reinterpret_cast<bf16x8*>(Asl + row * PC + c8) = vl;
    *reinterpret_cast<bf16x8*>(p.A + (ch * C + row) * C + c8) = vh;
  }
  __syncthreads();

  // --- W^T and U'^T tiles: lane owns W[r][j .. j+3]; U' = A_h V_h + A_h V_l + A_l V_h,
  // stored as bf16 high + low parts.  The three tiles are staged in LDS no longer
  // read (W over Qn / X, U' high over Gamma, U' low over L) and leave in 16-byte
  // row pieces ---
  bf16* const Wst = reinterpret_cast<bf16*>(QX);
  bf16* const Uhst = reinterpret_cast<bf16*>(Gs);
  bf16* const Ulst = reinterpret_cast<bf16*>(Lf);
  static_assert(C * PD * 2 <= kQX && C * PD * 2 <= C * PG * 4 && C * PD * 2 <= C * PL * 4, "staging fits");
  {
    const int r = 16 * rb + jj;
#pragma unroll
    for (int q = 0; q < D / 32; ++q) {   // this wave's half of the 16-wide column blocks
      const int jb = hf * (D / 32) + q;
      f32x4 aW = zero4(), aU = zero4();
#pragma unroll
      for (int k0 = 0; k0 < C; k0 += 32) {
        const bf16x8 b = frag_rk(As, PC, 16 * rb, k0);
        const bf16x8 bl = frag_rk(Asl, PC, 16 * rb, k0);
        const bf16x8 vh = frag_kc(Vs, PD, 16 * jb, k0);
        aW = mma(frag_kc(Ks, PD, 16 * jb, k0), b, aW);
        aU = mma(vh, b, aU);
        aU = mma(frag_kc(Vsl, PD, 16 * jb, k0), b, aU);
        aU = mma(vh, bl, aU);
      }
      const int j0 = 16 * jb + 4 * g;
      st_bf16x4(Wst + r * PD + j0, aW[0], aW[1], aW[2], aW[3]);
      float hi[4], lo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hi[i] = float(to_bf16(aU[i]));
        lo[i] = aU[i] - hi[i];
      }
      st_bf16x4(Uhst + r * PD + j0, hi[0], hi[1], hi[2], hi[3]);
      st_bf16x4(Ulst + r * PD + j0, lo[0], lo[1], lo[2], lo[3]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < C * D / 8 / kT; ++it) {
    const int idx = tid + kT * it, row = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
    const int64_t o = (ch * C + row) * D + c8;
    *reinterpret_cast<u32x4*>(p.W + o) = *reinterpret_cast<const u32x4*>(Wst + row * PD + c8);
    *reinterpret_cast<u32x4*>(p.Up + o) = *reinterpret_cast<const u32x4*>(Uhst + row * PD + c8);
    *reinterpret_cast<u32x4*>(p.Uplo + o) = *reinterpret_cast<const u32x4*>(Ulst + row * PD + c8);
  }
}

// ===========================================================================
// k_grads_kda
// ===========================================================================
// The gate gradient feeds per-head sums (dA_log, ddt_bias) whose terms cancel
// by one to two orders of magnitude, so everything on its path is carried to
// about fp32 accuracy: U, S and dS enter as bf16 high + low parts (two or three
// MFMAs per product), kn and qn are fp32, dM and dP are split into two parts,
// and the operands of the pairwise products are split likewise.
// the gradient kernel runs eight waves (two per SIMD: phases alternate between them)
constexpr int kKdaGradThreads = 2 * kThreads;
// one workgroup per CU: the workgroup dealt this many places later runs on the
// same XCD (workgroups go round-robin over the 8 XCDs) at about the time this one
// ends
constexpr int kKdaGradAhead = 256;

// L2 prefetch of the first loads of the gradient workgroup with linear id L (dU^T,
// U^T high and low, A, and the dO and v rows; rows past the end clamped): one
// 4-byte direct-to-LDS load per 64-byte sector into a sink that is never read
template <int D>
__device__ __forceinline__ void kda_grads_prefetch(const Params& p, int L, char* sink) {
  constexpr int SR = D * 2 / 64;                     // sectors per bf16 token row
  constexpr int NU = D * C * 2 / 64, NA = C * C * 2 / 64, NR = C * SR;
  constexpr int NTOT = 3 * NU + NA + 2 * NR;
  int c, h;
  chunk_head_at(p, L, c, h);
  const ChunkEntry ce = p.ctab[c];
  const int64_t ch = int64_t(h) * p.NC + c;
  const char* tiles[3] = {reinterpret_cast<const char*>(p.dU + ch * D * C), reinterpret_cast<const char*>(p.U + ch * D * C),
                          reinterpret_cast<const char*>(p.Ulo + ch * D * C)};
  const char* A = reinterpret_cast<const char*>(p.A + ch * C * C);
  for (int u = threadIdx.x; u < NTOT; u += blockDim.x) {
    const char* a;
    if (u < 3 * NU) {
      a = (u < NU ? tiles[0] : u < 2 * NU ? tiles[1] : tiles[2]) + 64 * (u % NU);
    } else if (u < 3 * NU + NA) {
      a = A + 64 * (u - 3 * NU);
    } else {
      const int i = u - 3 * NU - NA, k = i % NR, row = min(k / SR, ce.len - 1);
      const void* base = i < NR ? p.dO : p.v;
      a = reinterpret_cast<const char*>(base) + tok(ce.t_start + row, p.H, h) * D * 2 + 64 * (k % SR);
    }
    dma4(a, sink);
  }
}

template <int D>
struct KdaGradSmem {
  static constexpr int PD = Dims<D>::PD;
  static constexpr int PG = D + 4;
  // region X: phase 1 dU^T + A | phase 2 S, dS tiles | phase 4 kn, qn in fp32
  static constexpr int x_p1 = (D * PC + C * PC) * 2;
  static constexpr int x_p2 = 2 * D * PD * 2;
  static constexpr int x_p4 = 2 * C * PG * 4;
  static constexpr int xb = x_p1 > x_p2 ? (x_p1 > x_p4 ? x_p1 : x_p4) : (x_p2 > x_p4 ? x_p2 : x_p4);
  // region Y: phases 1-3 dO, dY, U^T high, U^T low [, dO low for fp32 inputs] |
  // phase 4 dM, dP (high, low), Gamma
  static constexpr int y_p1 = (3 * C * PD + 2 * D * PC) * 2;
  static constexpr int y_p4 = 4 * C * PC * 2 + C * PG * 4;
  static constexpr int yb = y_p1 > y_p4 ? y_p1 : y_p4;
  // from phase 4 on, region Y's bytes past the phase-4 tiles are free
  static constexpr int y_tail = yb - y_p4;
};

template <int D, typename TIO>
__global__ __launch_bounds__(kKdaGradThreads) void k_grads_kda(const Params p) {
  constexpr bool kLo = std::is_same<TIO, float>::value;   // fp32 dO is not exact in bf16
  using Dm = Dims<D>;
  using Sm = KdaGradSmem<D>;
  constexpr int PD = Dm::PD, TPR = Dm::TPR, NJB = Dm::NJB;
  constexpr int kT = kKdaGradThreads;
  constexpr int RPP = kT / TPR, NPASS = C / RPP;   // row sweeps of 8 channels a thread
  constexpr int NJH = NJB / 2;                     // 16-wide channel blocks per column half
  constexpr int PG = Sm::PG;
  __shared__ __attribute__((aligned(16))) char RX[Sm::xb];
  __shared__ __attribute__((aligned(16))) char RY[Sm::yb];
  __shared__ float beta_s[C], rq_s[C], rk_s[C];
  // fixed-order partial sums for the per-channel chunk-total gradient
  __shared__ float csum_s[4][D], ssum_s[4][D];
  // the fused prepare-backward's small arrays: in region Y's tail where it has room
  constexpr int NPART = kT / D, RP = C / NPART;   // per-channel scans: row ranges per channel
  constexpr int kTailFloats = 2 * NPART * D + kT / 64 + 4 * C + C + D;
  constexpr bool kTailInY = Sm::y_tail >= kTailFloats * 4;
  __shared__ __attribute__((aligned(16))) float TX[kTailInY ? 4 : kTailFloats];
  // bf16 inputs: the sink of the successor's L2 prefetch
  constexpr bool kPf = !kLo;
  __shared__ __attribute__((aligned(256))) char pf_sink[kPf ? 256 : 4];

  int c, h;
  chunk_head(p, c, h);
  const ChunkEntry ce = p.ctab[c];
  const int t0 = ce.t_start, len = ce.len;
  const int tid = threadIdx.x, l = lane_id(), w = wave_id();
  const int g = l >> 4, jj = l & 15;
  // eight waves: wave w owns row block rb = w % 4 (rows 16 rb ..) and column half
  // hf = w / 4 of every channel-wide result; waves w and w + 4 share a SIMD
  const int rb = __builtin_amdgcn_readfirstlane(w & 3), hf = __builtin_amdgcn_readfirstlane(w >> 2);
  const int64_t ch = int64_t(h) * p.NC + c;
  const int H = p.H;
  const float scale = p.scale;

  bf16* dUsT = reinterpret_cast<bf16*>(RX);          // phase 1: dU^T [v][r]
  bf16* As = dUsT + D * PC;                           // phase 1
  bf16* Sx = reinterpret_cast<bf16*>(RX);             // phase 2: S part [v][j]
  bf16* dSx = Sx + D * PD;                            // phase 2: dS part [v][j]
  float* Knf = reinterpret_cast<float*>(RX);          // phase 3-4: kn [r][c] fp32
  float* Qnf = Knf + C * PG;                          // phase 3-4: qn [r][c] fp32
  bf16* dOs = reinterpret_cast<bf16*>(RY);            // phases 1-3
  bf16* dYs = dOs + C * PD;
  bf16* UsT = dYs + C * PD;                           // U^T high [v][r]
  bf16* UsTl = UsT + D * PC;                          // U^T low
  bf16* dOl = UsTl + D * PC;                          // dO low (fp32 inputs)
  bf16* dMh = reinterpret_cast<bf16*>(RY);            // phase 4: dM, dP high / low [r][s]
  bf16* dMl = dMh + C * PC;
  bf16* dPh = dMl + C * PC;
  bf16* dPl = dPh + C * PC;
  float* Gs = reinterpret_cast<float*>(dPl + C * PC); // phase 4: Gamma [r][c]
  float* Dg_s = reinterpret_cast<float*>(RY);         // after phase 4: dGamma [r][c]
  float* const tail = kTailInY ? reinterpret_cast<float*>(RY + Sm::y_p4) : TX;
  float* const tot_s = tail;                  // [NPART][D] range totals of the reverse cumsum
  float* const pd_s = tot_s + NPART * D;      // [NPART][D] ddt_bias partials
  float* const pa_s = pd_s + NPART * D;       // [waves]    dA_log partials
  float* const l2_s = pa_s + kT / 64;         // [half][q, k][C] row dot products
  float* const dbt_s = l2_s + 4 * C;          // [C] the second column half's dbeta partials
  float* const dgc_s = dbt_s + C;             // [D] dGamma_C

  if (tid < C) {
    rq_s[tid] = p.rho[ch * 3 * C + tid];
    rk_s[tid] = p.rho[ch * 3 * C + C + tid];
    beta_s[tid] = p.rho[ch * 3 * C + 2 * C + tid];
  }
  // every tile load issued first (their latencies overlap), then the LDS writes
  constexpr int NU = D * C / 8 / kT;   // 16-byte pieces per thread of a [D][64] tile
  static_assert(C * C / 8 == kT, "one 16-byte piece of A per thread");
  uint4 du_r[NU], u_r[NU], ul_r[NU], a_r;
  typename IO<TIO>::Raw8 do_r[NPASS];
#pragma unroll
  for (int i = 0; i < NU; ++i) {
    const int pc = tid + i * kT, v = pc / (C / 8), c0 = (pc % (C / 8)) * 8;
    const int64_t o = (ch * D + v) * C + c0;
    du_r[i] = *reinterpret_cast<const uint4*>(p.dU + o);
    u_r[i] = *reinterpret_cast<const uint4*>(p.U + o);
    ul_r[i] = *reinterpret_cast<const uint4*>(p.Ulo + o);
  }
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int r = ps * RPP + tid / TPR, c0 = (tid % TPR) * 8;
    do_r[ps] = IO<TIO>::load_raw8(p.dO, tok(t0 + min(r, len - 1), H, h) * D + c0);
  }
  a_r = *reinterpret_cast<const uint4*>(p.A + (ch * C + tid / 8) * C + (tid % 8) * 8);
  // phase 1's v values (row 16 rb + jj, columns 16 vb + 4g .., vb in this wave's
  // half): loaded here, since a load placed after the dv stores could not be
  // moved above them
  const int r = 16 * rb + jj;
  const int64_t trow = tok(t0 + min(r, len - 1), H, h) * D;
  typename IO<TIO>::Raw4 v_raw[NJH];
#pragma unroll
  for (int q = 0; q < NJH; ++q) v_raw[q] = IO<TIO>::load_raw4(p.v, trow + 16 * (hf * NJH + q) + 4 * g);
#pragma unroll
  for (int i = 0; i < NU; ++i) {
    const int pc = tid + i * kT, v = pc / (C / 8), c0 = (pc % (C / 8)) * 8;
    *reinterpret_cast<uint4*>(dUsT + v * PC + c0) = du_r[i];
    *reinterpret_cast<uint4*>(UsT + v * PC + c0) = u_r[i];
    *reinterpret_cast<uint4*>(UsTl + v * PC + c0) = ul_r[i];
  }
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int r = ps * RPP + tid / TPR, c0 = (tid % TPR) * 8;
    float x[8];
    IO<TIO>::unpack8(do_r[ps], x);
    const float m = r < len ? 1.f : 0.f;
    bf16x8 xb, xl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      xb[e] = to_bf16(x[e] * m);
      xl[e] = to_bf16(x[e] * m - float(xb[e]));
    }
    *reinterpret_cast<bf16x8*>(dOs + r * PD + c0) = xb;
    if constexpr (kLo) *reinterpret_cast<bf16x8*>(dOl + r * PD + c0) = xl;
  }
  *reinterpret_cast<uint4*>(As + (tid / 8) * PC + (tid % 8) * 8) = a_r;
  __syncthreads();

  // the high parts of S and dS for phase 2, in flight during phase 1; thread =
  // (8 channels c8, rows vg + VG i), the same entries in both passes of phase 2
  constexpr int NSL = D * D / 8 / kT;   // 16-byte pieces per thread of a [D][D] tile
  constexpr int CG = D / 8, VG = kT / CG;
  static_assert(NSL * VG == D, "one row set per thread");
  const int c8 = (tid % CG) * 8, vg = tid / CG;
  uint4 s_r[NSL], d_r[NSL];
#pragma unroll
  for (int i = 0; i < NSL; ++i) {
    const int64_t o = (ch * D + vg + VG * i) * D + c8;
    s_r[i] = *reinterpret_cast<const uint4*>(p.S + o);
    d_r[i] = *reinterpret_cast<const uint4*>(p.dS + o);
  }

  // ---- phase 1: dY = A^T dU (lane owns dY[r][v .. v+3], r = 16 rb + jj, v in this
  // wave's half); dv; sum dY*v ----
  const float br = beta_s[r];
  float dbeta_row = 0.f;
#pragma unroll
  for (int q = 0; q < NJH; ++q) {
    const int vb = hf * NJH + q;
    f32x4 a = zero4();
#pragma unroll
    for (int k0 = 0; k0 < C; k0 += 32) a = mma(frag_rk(dUsT, PC, 16 * vb, k0), frag_kc(As, PC, 16 * rb, k0), a);
    const int v = 16 * vb + 4 * g;
    st_bf16x4(dYs + r * PD + v, a[0], a[1], a[2], a[3]);
    float vv[4];
    IO<TIO>::unpack4(v_raw[q], vv);
    dbeta_row += a[0] * vv[0] + a[1] * vv[1] + a[2] * vv[2] + a[3] * vv[3];
    if (r < len) IO<TIO>::store4(p.dv, trow + v, br * a[0], br * a[1], br * a[2], br * a[3]);
  }
  __syncthreads();

  // ---- phase 2: Z = dY S, dQbar = dO S, dKhat = U dS in two passes (high, low
  // parts of S and dS); lane owns (r, j .. j+3), j in this wave's half ----
  f32x4 aZ[NJH], aQ[NJH], aK[NJH];
#pragma unroll
  for (int q = 0; q < NJH; ++q) aZ[q] = aQ[q] = aK[q] = zero4();
  // per-channel state sum sum_v S dS with S = high + low, dS likewise (fp32
  // products), over this thread's entries: the high parts read back from LDS, the
  // low parts from the registers that carry them there
  float acc8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // raw q, k rows (for kn, qn in fp32 below) and the M entries phase 3 needs,
  // loaded during the second pass
  typename IO<TIO>::Raw8 q_raw[NPASS], k_raw[NPASS];
  uint2 mk_r[2];   // phase 3's blocks of this wave: sb = hf, hf + 2
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int i = 0; i < NSL; ++i) {
      const int row = vg + VG * i;
      *reinterpret_cast<uint4*>(Sx + row * PD + c8) = s_r[i];
      *reinterpret_cast<uint4*>(dSx + row * PD + c8) = d_r[i];
    }
    if (pass == 0) {
#pragma unroll
      for (int i = 0; i < NSL; ++i) {
        const int64_t o = (ch * D + vg + VG * i) * D + c8;
        s_r[i] = *reinterpret_cast<const uint4*>(p.Slo + o);
        d_r[i] = *reinterpret_cast<const uint4*>(p.dSlo + o);
      }
    } else {
#pragma unroll
      for (int ps = 0; ps < NPASS; ++ps) {
        const int rr = ps * RPP + tid / TPR, c0 = (tid % TPR) * 8;
        const int64_t o = qk_tok(p, t0 + min(rr, len - 1), h) * D + c0;
        q_raw[ps] = IO<TIO>::load_raw8(p.q, o);
        k_raw[ps] = IO<TIO>::load_raw8(p.k, o);
      }
#pragma unroll
      for (int x = 0; x < 2; ++x)
        mk_r[x] = *reinterpret_cast<const uint2*>(p.Mk + (ch * C + r) * C + 16 * (hf + 2 * x) + 4 * g);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NJH; ++q) {
      const int jb = hf * NJH + q;
#pragma unroll
      for (int k0 = 0; k0 < D; k0 += 32) {
        const bf16x8 aS = frag_kc(Sx, PD, 16 * jb, k0);
        const bf16x8 aD = frag_kc(dSx, PD, 16 * jb, k0);
        aZ[q] = mma(aS, frag_rk(dYs, PD, 16 * rb, k0), aZ[q]);
        aQ[q] = mma(aS, frag_rk(dOs, PD, 16 * rb, k0), aQ[q]);
        if (kLo && pass == 0) aQ[q] = mma(aS, frag_rk(dOl, PD, 16 * rb, k0), aQ[q]);
        aK[q] = mma(aD, frag_kc(UsT, PC, 16 * rb, k0), aK[q]);
        if (pass == 0) aK[q] = mma(aD, frag_kc(UsTl, PC, 16 * rb, k0), aK[q]);
      }
    }
    if (pass == 0) {   // the state sum over this thread's entries (high parts: its own LDS writes)
#pragma unroll
      for (int i = 0; i < NSL; ++i) {
        const int row = vg + VG * i;
        float a[8], b[8], c2[8], d2[8];
        IO<bf16>::unpack8(*reinterpret_cast<const u32x4*>(Sx + row * PD + c8), a);
        IO<bf16>::unpack8(*reinterpret_cast<const u32x4*>(&s_r[i]), b);
        IO<bf16>::unpack8(*reinterpret_cast<const u32x4*>(dSx + row * PD + c8), c2);
        IO<bf16>::unpack8(*reinterpret_cast<const u32x4*>(&d_r[i]), d2);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc8[e] = fmaf(a[e] + b[e], c2[e] + d2[e], acc8[e]);
      }
    }
    __syncthreads();
  }
  // ---- the state sum: row groups summed across lanes, then waves ----
  {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (CG == 8) acc8[e] += dpp_f<0x128>(acc8[e]);   // lanes l and l + 8 of a row
      acc8[e] = xrow_sum(acc8[e]);
    }
    // waves 4 .. 7 leave their partials here; waves 0 .. 3 add theirs after the
    // next barrier (a fixed order)
    if (hf == 1 && l < CG) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ssum_s[rb][c8 + e] = acc8[e];
    }
  }

  // ---- kn, qn in fp32 (region X) ----
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int rr = ps * RPP + tid / TPR, c0 = (tid % TPR) * 8;
    float qv[8], kv[8];
    IO<TIO>::unpack8(q_raw[ps], qv);
    IO<TIO>::unpack8(k_raw[ps], kv);
    const float m = rr < len ? 1.f : 0.f;
    const float fq = m * rq_s[rr], fk = m * rk_s[rr];
#pragma unroll
    for (int e = 0; e < 8; e += 4) {
      *reinterpret_cast<float4*>(Qnf + rr * PG + c0 + e) =
          make_float4(qv[e] * fq, qv[e + 1] * fq, qv[e + 2] * fq, qv[e + 3] * fq);
      *reinterpret_cast<float4*>(Knf + rr * PG + c0 + e) =
          make_float4(kv[e] * fk, kv[e + 1] * fk, kv[e + 2] * fk, kv[e + 3] * fk);
    }
  }
  // Gamma rows for phase 4 (in flight during phase 3; region Y is rewritten below)
  constexpr int NGL = C * D / 4 / kT;
  float4 g_r[NGL];
#pragma unroll
  for (int i = 0; i < NGL; ++i) {
    const int pc = tid + i * kT, rr = pc / (D / 4), c4 = (pc % (D / 4)) * 4;
    g_r[i] = ld4(p.gam + (ch * C + rr) * D + c4);
  }
  // ---- phase 3: dP = dO U^T, dL = -dY U^T (U high + low); dM = beta dL; this
  // wave takes the column blocks sb = hf, hf + 2 of its row block (zero above it) ----
  float dmv[2][4], dpv[2][4];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int sb = hf + 2 * x;
    const int s0 = 16 * sb + 4 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) dmv[x][i] = dpv[x][i] = 0.f;
    if (sb <= rb) {
      f32x4 G1 = zero4(), G2 = zero4();
#pragma unroll
      for (int k0 = 0; k0 < D; k0 += 32) {
        const bf16x8 uh = frag_kc(UsT, PC, 16 * sb, k0), ul = frag_kc(UsTl, PC, 16 * sb, k0);
        const bf16x8 bo = frag_rk(dOs, PD, 16 * rb, k0), by = frag_rk(dYs, PD, 16 * rb, k0);
        G1 = mma(uh, bo, G1);
        G1 = mma(ul, bo, G1);
        if constexpr (kLo) G1 = mma(uh, frag_rk(dOl, PD, 16 * rb, k0), G1);
        G2 = mma(uh, by, G2);
        G2 = mma(ul, by, G2);
      }
      const uint2 mk = mk_r[x];
      const float Mv[4] = {__uint_as_float(mk.x << 16), __uint_as_float(mk.x & 0xffff0000u),
                           __uint_as_float(mk.y << 16), __uint_as_float(mk.y & 0xffff0000u)};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = s0 + i;
        if (r >= s) dpv[x][i] = G1[i];
        if (r > s) {
          const float dL = -G2[i];
          dbeta_row += dL * Mv[i];
          dmv[x][i] = br * dL;
        }
      }
    }
  }
  __syncthreads();
  if (hf == 0 && l < CG) {   // the state sum, waves 0 .. 3 after waves 4 .. 7
#pragma unroll
    for (int e = 0; e < 8; ++e) ssum_s[rb][c8 + e] += acc8[e];
  }
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int sb = hf + 2 * x;
    const int s0 = 16 * sb + 4 * g;
    float hm[4], lm[4], hp[4], lp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hm[i] = float(to_bf16(dmv[x][i]));
      lm[i] = dmv[x][i] - hm[i];
      hp[i] = float(to_bf16(dpv[x][i]));
      lp[i] = dpv[x][i] - hp[i];
    }
    st_bf16x4(dMh + r * PC + s0, hm[0], hm[1], hm[2], hm[3]);
    st_bf16x4(dMl + r * PC + s0, lm[0], lm[1], lm[2], lm[3]);
    st_bf16x4(dPh + r * PC + s0, hp[0], hp[1], hp[2], hp[3]);
    st_bf16x4(dPl + r * PC + s0, lp[0], lp[1], lp[2], lp[3]);
  }
#pragma unroll
  for (int i = 0; i < NGL; ++i) {
    const int pc = tid + i * kT, rr = pc / (D / 4), c4 = (pc % (D / 4)) * 4;
    // in base-2 units (log2(e) Gamma): every use below is an exponent of 2
    *reinterpret_cast<float4*>(Gs + rr * PG + c4) =
        make_float4(kLog2e * g_r[i].x, kLog2e * g_r[i].y, kLog2e * g_r[i].z, kLog2e * g_r[i].w);
  }
  __syncthreads();

  // the successor's first loads into this XCD's L2 (waited for at the end); phase
  // 4 is long enough for them to land before the tail's register loads are waited
  // for (their waits would take the prefetch along)
  if constexpr (kPf) {
    if (const int L = blockIdx.x + p.NC * blockIdx.y + kKdaGradAhead; L < p.NC * p.H)
      kda_grads_prefetch<D>(p, L, pf_sink);
  }

  // ---- phase 4: pairwise terms ----
  //   X1_rc = sum_{s<r} dM_rs kn_sc E_rsc     -> dkn_r, dGamma_r (+ kn_r X1)
  //   X3_rc = scale sum_{s<=r} dP_rs kn_sc E  -> dqn_r, dGamma_r (+ qn_r X3)
  //   X2_sc = sum_{r>s} dM_rs kn_rc E_rsc     -> dkn_s, dGamma_s (- kn_s X2)
  //   X4_sc = scale sum_{r>=s} dP_rs qn_rc E  -> dkn_s, dGamma_s (- kn_s X4)
  // the waves of row block rb own its 16 rows on both sides, each for the channel
  // tiles of its half; products with split operands take a_h b_h + a_h b_l + a_l b_h.  One 16-channel tile at a time: its state-side
  // terms are folded in first, and its results are stored at the end of its step,
  // so that only one tile's gradients are held in registers.
  // K = 16 B fragments of the off-diagonal block pairs (the same for every channel
  // tile): row side blocks sb < rb, column side blocks cb > rb
  bf16x4 fr_mh[3], fr_ml[3], fr_ph[3], fr_pl[3], fc_mh[3], fc_ml[3], fc_ph[3], fc_pl[3];
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    if (x < rb) {
      fr_mh[x] = frag16_rk(dMh, PC, 16 * rb, 16 * x);
      fr_ml[x] = frag16_rk(dMl, PC, 16 * rb, 16 * x);
      fr_ph[x] = frag16_rk(dPh, PC, 16 * rb, 16 * x);
      fr_pl[x] = frag16_rk(dPl, PC, 16 * rb, 16 * x);
    }
    if (x + 1 > rb) {
      const int rs = 16 * (x + 1);
      fc_mh[x] = frag16_kc(dMh, PC, 16 * rb, rs);
      fc_ml[x] = frag16_kc(dMl, PC, 16 * rb, rs);
      fc_ph[x] = frag16_kc(dPh, PC, 16 * rb, rs);
      fc_pl[x] = frag16_kc(dPl, PC, 16 * rb, rs);
    }
  }
  // B operands of the diagonal block's fp32 products (lane: k = 4 kk + g, n = jj):
  // dM[f+n][f+k] and dP[f+n][f+k] (row side), dM[f+k][f+n] and dP[f+k][f+n] (column side)
  float dm_row[4], dp_row[4], dm_col[4], dp_col[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int f = 16 * rb, kx = f + 4 * kk + g, nx = f + jj;
    dm_row[kk] = float(dMh[nx * PC + kx]) + float(dMl[nx * PC + kx]);
    dp_row[kk] = float(dPh[nx * PC + kx]) + float(dPl[nx * PC + kx]);
    dm_col[kk] = float(dMh[kx * PC + nx]) + float(dMl[kx * PC + nx]);
    dp_col[kk] = float(dPh[kx * PC + nx]) + float(dPl[kx * PC + nx]);
  }
  auto split4 = [](const float (&x)[4], bf16x4& hi, bf16x4& lo) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hi[i] = to_bf16(x[i]);
      lo[i] = to_bf16(x[i] - float(hi[i]));
    }
  };
  // every tile's dqn, dkn, dGamma stay in registers for the prepare-backward below
  f32x4 oq[NJH], ok[NJH], og[NJH];
  // the prepare-backward's per-channel operands (thread = channel gc, row range gpart)
  const int gc = tid % D, gpart = tid / D;
  float x_r[RP], bias = 0.f, a_log = 0.f, braw = 0.f;
#pragma unroll
  for (int q = 0; q < NJH; ++q) {
    if (q == NJH - 1) {   // in flight during the last tile
#pragma unroll
      for (int i = 0; i < RP; ++i)
        x_r[i] = IO<TIO>::load1(p.g, tok(t0 + min(gpart * RP + i, len - 1), H, h) * D + gc);
      bias = p.dt_bias[h * D + gc];
      a_log = p.A_log[h];
      braw = IO<TIO>::load1(p.b, tok(t0 + min(r, len - 1), H, h));
    }
    const int jb = hf * NJH + q;
    const int c0 = 16 * jb;
    const int cm = c0 + jj;          // channel of this lane in an A fragment (m = lane % 16)
    const int j = c0 + 4 * g;        // channels of this lane in the outputs
    const float4 kr = ld4(Knf + r * PG + j), qr = ld4(Qnf + r * PG + j);
    // fold the state-side terms (lane owns (r, c = j + i)): Kbar = kn e^Gam
    // (dKbar = -beta Z), Khat = kn e^(GamC - Gam), Qbar = scale qn e^Gam
    f32x4 dkn, dqn, dgm, Gr;
    {
      const float4 gr = ld4(Gs + r * PG + j), gC = ld4(Gs + (C - 1) * PG + j);
      float csum[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float kn = el(kr, i), qn = el(qr, i);
        const float eg = fast_exp2(el(gr, i)), eh = fast_exp2(el(gC, i) - el(gr, i));
        const float z = aZ[q][i], dkh = aK[q][i], dqb = aQ[q][i];
        dgm[i] = -br * z * kn * eg - dkh * kn * eh + dqb * scale * qn * eg;
        dbeta_row -= kn * eg * z;
        csum[i] = dkh * kn * eh;
        dkn[i] = -br * z * eg + dkh * eh;
        dqn[i] = scale * dqb * eg;
        Gr[i] = el(gr, i);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float col = row16_sum(csum[i]);   // over the 16 rows of this wave
        if (jj == 0) csum_s[rb][j + i] = col;
      }
    }
    // row side, earlier blocks sb < rb: reference = last row of block sb
#pragma unroll
    for (int sb = 0; sb < 3; ++sb) {
      if (sb >= rb) break;
      const int se = 16 * sb + 15;
      const float ge = Gs[se * PG + cm];
      float av[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = 16 * sb + 4 * g + i;
        av[i] = Knf[s * PG + cm] * fast_exp2(ge - Gs[s * PG + cm]);
      }
      bf16x4 ah, al;
      split4(av, ah, al);
      const bf16x4 mh = fr_mh[sb], ml = fr_ml[sb], ph = fr_ph[sb], pl = fr_pl[sb];
      const f32x4 t1 = mma16(al, mh, mma16(ah, ml, mma16(ah, mh, zero4())));
      const f32x4 t3 = mma16(al, ph, mma16(ah, pl, mma16(ah, ph, zero4())));
      const float4 gend = ld4(Gs + se * PG + j);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float mlt = fast_exp2(Gr[i] - el(gend, i));
        const float x1 = t1[i] * mlt, x3 = scale * t3[i] * mlt;
        dkn[i] += x1;
        dqn[i] += x3;
        dgm[i] += el(kr, i) * x1 + el(qr, i) * x3;
      }
    }
    // column side, later blocks cb > rb: reference = first row of block cb
#pragma unroll
    for (int cb = 1; cb < 4; ++cb) {
      if (cb <= rb) continue;
      const int rs = 16 * cb;
      const float gst = Gs[rs * PG + cm];
      float kv[4], qv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = rs + 4 * g + i;
        const float d = fast_exp2(Gs[rr * PG + cm] - gst);
        kv[i] = Knf[rr * PG + cm] * d;
        qv[i] = Qnf[rr * PG + cm] * d;
      }
      bf16x4 kh, kl, qh, ql;
      split4(kv, kh, kl);
      split4(qv, qh, ql);
      const bf16x4 mh = fc_mh[cb - 1], ml = fc_ml[cb - 1], ph = fc_ph[cb - 1], pl = fc_pl[cb - 1];
      const f32x4 t2 = mma16(kl, mh, mma16(kh, ml, mma16(kh, mh, zero4())));
      const f32x4 t4 = mma16(ql, ph, mma16(qh, pl, mma16(qh, ph, zero4())));
      const float4 gsv = ld4(Gs + rs * PG + j);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float mlt = fast_exp2(el(gsv, i) - Gr[i]);
        const float x = (t2[i] + scale * t4[i]) * mlt;
        dkn[i] += x;
        dgm[i] -= el(kr, i) * x;
      }
    }
    bool fact_ok;
    // diagonal block rb, factored at its middle row m = 16 rb + 8: E_rt =
    // e^(Gam_r - Gam_m) e^(Gam_m - Gam_t).  The products run on fp32 MFMA (16x16x4,
    // four k-steps) with fp32 operands, so they keep the exact path's accuracy.
    // Valid while the block's larger half-span max(Gam_f - Gam_m, Gam_m - Gam_(f+15))
    // (f = 16 rb, the bound of every factor's exponent) stays below kSpanMax for all
    // 16 channels of this tile (no overflow, no underflow of the small factors);
    // otherwise the tile takes the exact per-element path below.
    {
      const int f = 16 * rb, m = f + 8;
      const float gm = Gs[m * PG + cm];
      const bool wide = fmaxf(Gs[f * PG + cm] - gm, gm - Gs[(f + 15) * PG + cm]) >= kLog2e * kSpanMax;
      fact_ok = __builtin_amdgcn_ballot_w64(wide) == 0;
      if (fact_ok) {
        f32x4 t1 = zero4(), t2 = zero4(), t3 = zero4(), t4 = zero4();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int s = f + 4 * kk + g;   // A: m = channel cm, k = s - f
          const float gs = Gs[s * PG + cm];
          const float kb = Knf[s * PG + cm] * fast_exp2(gm - gs);   // kn_s b_s
          const float d = fast_exp2(gs - gm);                        // a_s
          t1 = mma_f32(kb, dm_row[kk], t1);
          t3 = mma_f32(kb, dp_row[kk], t3);
          t2 = mma_f32(Knf[s * PG + cm] * d, dm_col[kk], t2);
          t4 = mma_f32(Qnf[s * PG + cm] * d, dp_col[kk], t4);
        }
        const float4 gmv = ld4(Gs + m * PG + j);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float arow = fast_exp2(Gr[i] - el(gmv, i));   // a_r
          const float bcol = fast_exp2(el(gmv, i) - Gr[i]);   // b_r
          const float x1 = t1[i] * arow, x3 = scale * t3[i] * arow;
          const float x24 = (t2[i] + scale * t4[i]) * bcol;
          dkn[i] += x1 + x24;
          dqn[i] += x3;
          dgm[i] += el(kr, i) * (x1 - x24) + el(qr, i) * x3;
        }
      }
    }
    // a tile whose decay is too steep for the factored form, exactly:
    // E = exp(-|Gamma_r - Gamma_t|) for both orders
    if (!fact_ok) {
      for (int t = 16 * rb; t < 16 * rb + 16; ++t) {
        const float mrt = float(dMh[r * PC + t]) + float(dMl[r * PC + t]);
        const float prt = scale * (float(dPh[r * PC + t]) + float(dPl[r * PC + t]));
        const float mtr = float(dMh[t * PC + r]) + float(dMl[t * PC + r]);
        const float ptr = scale * (float(dPh[t * PC + r]) + float(dPl[t * PC + r]));
        const float4 gt = ld4(Gs + t * PG + j);
        const float4 kt = ld4(Knf + t * PG + j), qt = ld4(Qnf + t * PG + j);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float E = fast_exp2(-fabsf(Gr[i] - el(gt, i)));
          const float ke = el(kt, i) * E, qe = el(qt, i) * E;
          const float x1 = mrt * ke, x3 = prt * ke, x24 = mtr * ke + ptr * qe;
          dkn[i] += x1 + x24;
          dqn[i] += x3;
          dgm[i] += el(kr, i) * (x1 - x24) + el(qr, i) * x3;
        }
      }
    }
    oq[q] = dqn;
    ok[q] = dkn;
    og[q] = dgm;
  }

  // ---- prepare-backward, fused (FlashKDA backward (K1) page, sections 3.3 and 5):
  // the L2-norm backward of dqn, dkn (row dot products over both column halves),
  // the sigmoid backward of dbeta, the per-channel reverse cumsum of dGamma plus the
  // chunk-total term, the gate backward, per-chunk partials of dA_log and ddt_bias ----
  float pq = 0.f, pk = 0.f;
#pragma unroll
  for (int q = 0; q < NJH; ++q) {
    const int j = 16 * (hf * NJH + q) + 4 * g;
    const float4 qn4 = ld4(Qnf + r * PG + j), kn4 = ld4(Knf + r * PG + j);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pq = fmaf(el(qn4, i), oq[q][i], pq);
      pk = fmaf(el(kn4, i), ok[q][i], pk);
    }
  }
  pq = xrow_sum(pq);
  pk = xrow_sum(pk);
  dbeta_row += __shfl_xor(dbeta_row, 16, 64);
  dbeta_row += __shfl_xor(dbeta_row, 32, 64);
  __syncthreads();   // phase 4 is done everywhere: dM, dP are free (Gamma's last row is read below)
#pragma unroll
  for (int q = 0; q < NJH; ++q) {
    const int j = 16 * (hf * NJH + q) + 4 * g;
    *reinterpret_cast<float4*>(Dg_s + r * PG + j) = make_float4(og[q][0], og[q][1], og[q][2], og[q][3]);
  }
  if (g == 0) {
    l2_s[(2 * hf) * C + r] = pq;
    l2_s[(2 * hf + 1) * C + r] = pk;
    if (hf == 1) dbt_s[r] = dbeta_row;
  }
  if (tid < D) {
    const float st = (ssum_s[0][tid] + ssum_s[1][tid]) + (ssum_s[2][tid] + ssum_s[3][tid]);
    const float a = (csum_s[0][tid] + csum_s[1][tid]) + (csum_s[2][tid] + csum_s[3][tid]);
    dgc_s[tid] = a + st * fast_exp2(Gs[(C - 1) * PG + tid]);
  }
  __syncthreads();
  // L2-norm backward (K1 page, 3.3): dq = rq (dqn - qn <qn, dqn>), dk likewise
  {
    const bool valid = r < len;
    const float m = valid ? 1.f : 0.f;
    const float rq = m * rq_s[r], rk = m * rk_s[r];
    const float pqf = l2_s[r] + l2_s[2 * C + r], pkf = l2_s[C + r] + l2_s[3 * C + r];
#pragma unroll
    for (int q = 0; q < NJH; ++q) {
      const int j = 16 * (hf * NJH + q) + 4 * g;
      const float4 qn4 = ld4(Qnf + r * PG + j), kn4 = ld4(Knf + r * PG + j);
      float dq[4], dk[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dq[i] = rq * (oq[q][i] - el(qn4, i) * pqf);
        dk[i] = rk * (ok[q][i] - el(kn4, i) * pkf);
      }
      if (valid) {
        IO<TIO>::store4(p.dq, tok(t0 + r, H, h) * D + j, dq[0], dq[1], dq[2], dq[3]);
        IO<TIO>::store4(p.dk, tok(t0 + r, H, h) * D + j, dk[0], dk[1], dk[2], dk[3]);
      }
    }
  }
  // sigmoid backward of beta (w.r.t. its logit)
  if (hf == 0 && g == 0 && r < len) {
    const float bt = sigmoidf(braw);
    IO<TIO>::store1(p.db, tok(t0 + r, H, h), (dbeta_row + dbt_s[r]) * bt * (1.f - bt));
  }
  // per channel: dlam_r = sum_{r' >= r} dGamma_r' + dGamma_C (K1 page, section 5),
  // then through the gate function: softplus form dx = dlam (-e^A sigmoid(x)),
  // d/dA_log: dlam lambda; bounded sigmoid form (z = e^A x) dx = dlam gate_scale
  // sigma(z) (1 - sigma(z)) e^A, d/dA_log: dx x.  Thread = (channel, one of NPART
  // row ranges): a suffix scan of its range in registers plus the totals of the
  // ranges after it
  float xs[RP];
#pragma unroll
  for (int i = RP - 1; i >= 0; --i) xs[i] = Dg_s[(gpart * RP + i) * PG + gc] + (i < RP - 1 ? xs[i + 1] : 0.f);
  tot_s[gpart * D + gc] = xs[0];
  __syncthreads();
  float after = dgc_s[gc];
#pragma unroll
  for (int qq = NPART - 1; qq > 0; --qq) after += qq > gpart ? tot_s[qq * D + gc] : 0.f;
  const float ea = fast_exp(a_log);
  float pd = 0.f, pa = 0.f;
#pragma unroll
  for (int i = 0; i < RP; ++i) {
    const int rr = gpart * RP + i;
    if (rr < len) {
      const float acc = xs[i] + after;
      const float xg = x_r[i] + bias;
      float dx;
      if (p.gate_fn) {
        // sigma'(z) = sigma(z) sigma(-z) = t / (1 + t)^2 with t = e^-|z|: no
        // cancellation where sigma saturates (1 - sigma(z) in fp32 loses the
        // relative accuracy of sigma' there, and dA_log sums these terms with
        // strong cancellation)
        const float t = fast_exp(-fabsf(ea * xg));
        dx = acc * p.gate_scale * (t / ((1.f + t) * (1.f + t))) * ea;
        pa += dx * xg;
      } else {
        dx = acc * (-ea * sigmoidf(xg));
        pa += acc * (-ea * softplusf(xg));
      }
      IO<TIO>::store1(p.dg, tok(t0 + rr, H, h) * D + gc, dx);
      pd += dx;
    }
  }
  pd_s[gpart * D + gc] = pd;
  pa = wave_sum(pa);
  if (l == 0) pa_s[w] = pa;
  __syncthreads();
  if (tid < D) {
    float sdt = 0.f;
#pragma unroll
    for (int qq = 0; qq < NPART; ++qq) sdt += pd_s[qq * D + tid];
    p.pddt[ch * D + tid] = sdt;
  }
  if (tid == 0) {
    float sa = 0.f;
#pragma unroll
    for (int x = 0; x < kT / 64; ++x) sa += pa_s[x];
    p.pdA[ch] = sa;
  }
  if constexpr (kPf) wait_vm<0>();   // the prefetch's direct-to-LDS loads land before the LDS is released
}

// dA_log[h] and ddt_bias[h][:] from the per-chunk partials, in a fixed order:
// thread (channel, part) sums chunks part, part + NP, ... (loads independent of
// each other), then the parts are added in order; dA_log likewise over one wave.
constexpr int kParamThreads = 1024;
template <int D>
__global__ __launch_bounds__(kParamThreads) void k_params_kda(const Params p) {
  constexpr int NP = kParamThreads / D;
  __shared__ float part_s[NP][D];
  const int h = blockIdx.x, t = threadIdx.x, cc = t % D, part = t / D;
  const int64_t base = int64_t(h) * p.NC;
  float s = 0.f;
#pragma unroll 8
  for (int c = part; c < p.NC; c += NP) s += p.pddt[(base + c) * D + cc];
  part_s[part][cc] = s;
  float a = 0.f;
  if (t < 64) {
#pragma unroll 8
    for (int c = t; c < p.NC; c += 64) a += p.pdA[base + c];
    a = wave_sum(a);
  }
  __syncthreads();
  if (t < D) {
    float x = 0.f;
#pragma unroll
    for (int q = 0; q < NP; ++q) x += part_s[q][t];
    p.ddt_bias[h * D + t] = x;
  }
  if (t == 0) p.dA_log[h] = a;
}

// ===========================================================================
// launchers
// ===========================================================================
namespace {
template <int D, typename TIO>
void run_kda(const Params& p, int stage, hipStream_t s) {
  const dim3 grid(p.NC, p.H);
  if (stage == 0) k_prep_kda<D, TIO><<<grid, kKdaPrepThreads, 0, s>>>(p);
  else if (stage == 1) k_grads_kda<D, TIO><<<grid, kKdaGradThreads, 0, s>>>(p);
  else if (stage == 2) k_params_kda<D><<<p.H, kParamThreads, 0, s>>>(p);
}
}  // namespace

int launch_kda(const Params& p, int stage, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (p.K == 128 && p.dtype == GDR_BF16) run_kda<128, bf16>(p, stage, s);
  else if (p.K == 128 && p.dtype == GDR_F32) run_kda<128, float>(p, stage, s);
  else if (p.K == 64 && p.dtype == GDR_BF16) run_kda<64, bf16>(p, stage, s);
  else if (p.K == 64 && p.dtype == GDR_F32) run_kda<64, float>(p, stage, s);
  else return static_cast<int>(hipErrorInvalidValue);
  return static_cast<int>(hipGetLastError());
}

}  // namespace gdr

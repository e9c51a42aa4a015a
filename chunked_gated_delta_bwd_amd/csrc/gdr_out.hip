// k_output: the forward output of the chunked gated delta rule, per (chunk, head),
// from what the forward recompute leaves in the workspace:
//
//   O = Qbar S_n^T + P U      (64 x V)
//
// with S_n the state at the chunk start, U = U' - W S_n^T the chunk's new values
// (v_new), P = scale (Qn Kn^T o E) on and below the diagonal, and
// Qbar = scale qn e^Gam (per row for the scalar gate, per channel for the
// per-channel gate).  This is the chunked form of o_t = scale S_t qn_t: the state
// carried into the chunk reaches row r through Qbar, the chunk's own tokens
// through P (FlashQLA GDN overview, section 3; FlashKDA K1 page, section 2).
//
// One workgroup of four waves per (chunk, head); wave w owns rows 16w .. 16w+15.
// The tiles (S_n, the Qbar rows, P, U^T) are copied global -> LDS with
// direct-to-LDS loads and read as row fragments.  The products are taken
// transposed (O^T = S_n Qbar^T + U^T P^T) so that a lane ends up with four
// consecutive columns of one output row.  For the scalar gate with bf16 inputs
// Qbar is the raw q row times the row factor fq = scale e^Gam / |q|, applied to
// the accumulator; otherwise the prologue's Qbar (high part) tile is used.  The
// low parts the per-channel gate carries for S and U are not needed at the
// output's bf16 / fp32-rounding accuracy.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gdr_device.h"
#include "gdr_internal.h"
#include "gdr_lds.h"

namespace gdr {

constexpr int kOutWaves = 4;
constexpr int kOutThreads = 64 * kOutWaves;

template <int D, typename TIO, bool RAW>
__global__ __launch_bounds__(kOutThreads) void k_output(const Params p) {
  constexpr int NVB = D / 16;   // 16-wide output column blocks
  __shared__ __attribute__((aligned(1024))) char Ss[D * D * 2];   // S_n [v][k]
  __shared__ __attribute__((aligned(1024))) char Qs[C * D * 2];   // Qbar rows or raw q rows [r][k]
  __shared__ __attribute__((aligned(1024))) char Ps[C * C * 2];   // P [r][s]
  __shared__ __attribute__((aligned(1024))) char Us[D * C * 2];   // U^T [v][s]
  __shared__ __attribute__((aligned(256))) float fq_s[C];

  int c, h;
  chunk_head(p, c, h);
  const ChunkEntry ce = p.ctab[c];
  const int t0 = ce.t_start, len = ce.len;
  const int l = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = l >> 4, jj = l & 15;
  const int64_t ch = int64_t(h) * p.NC + c;
  auto u16 = [](const uint16_t* x) { return reinterpret_cast<const char*>(x); };

  dma_tile<D, 0, D, kOutWaves>(Ss, [&](int v) { return u16(p.S + (ch * D + v) * D); }, w);
  if constexpr (RAW) {
    dma_tile<D, 0, C, kOutWaves>(Qs, [&](int r) {
      return reinterpret_cast<const char*>(p.q) + qk_tok(p, t0 + min(r, len - 1), h) * D * 2;
    }, w);
    if (w == 0) dma4(p.fac + ch * 3 * C + l, reinterpret_cast<char*>(fq_s));   // fq: row factor 0
  } else {
    dma_tile<D, 0, C, kOutWaves>(Qs, [&](int r) { return u16(p.Qh + (ch * C + r) * D); }, w);
  }
  dma_tile<C, 1, C, kOutWaves>(Ps, [&](int r) { return u16(p.P + (ch * C + r) * C); }, w);
  dma_tile<C, 1, D, kOutWaves>(Us, [&](int v) { return u16(p.U + (ch * D + v) * C); }, w);
  wait_vm<0>();
  chain_barrier();

  // this wave's rows: Qbar (or q) and P fragments, read once for every column block
  const int rb = w;
  bf16x8 qf[D / 32], pf[C / 32];
#pragma unroll
  for (int k = 0; k < D / 32; ++k) qf[k] = frag_rk_s<D>(Qs, 16 * rb, 32 * k);
#pragma unroll
  for (int k = 0; k < C / 32; ++k) pf[k] = frag_rk_s<C, 1>(Ps, 16 * rb, 32 * k);
  const int r = 16 * rb + jj;
  const float fr = RAW ? fq_s[r] : 1.f;
  const bool store = r < len;
  const int64_t orow = tok(t0 + min(r, len - 1), p.H, h) * D;
#pragma unroll
  for (int vb = 0; vb < NVB; ++vb) {
    // lane: O^T[16 vb + 4g + i][r] = O[r][16 vb + 4g + i]
    f32x4 a = zero4();
#pragma unroll
    for (int k = 0; k < D / 32; ++k) a = mma(frag_rk_s<D>(Ss, 16 * vb, 32 * k), qf[k], a);
    if constexpr (RAW) a *= f32x4{fr, fr, fr, fr};
#pragma unroll
    for (int k = 0; k < C / 32; ++k) a = mma(frag_rk_s<C, 1>(Us, 16 * vb, 32 * k), pf[k], a);
    if (store) IO<TIO>::store4(p.o, orow + 16 * vb + 4 * g, a[0], a[1], a[2], a[3]);
  }
}

namespace {
template <int D, typename TIO, bool RAW>
void run_output(const Params& p, hipStream_t s) {
  k_output<D, TIO, RAW><<<dim3(p.NC, p.H), kOutThreads, 0, s>>>(p);
}
}  // namespace

int launch_output(const Params& p, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const bool bf = p.dtype == GDR_BF16;
  const bool raw = bf && p.gate == 0;   // the scalar gate with bf16 inputs has no Qbar tile
  if (p.K == 128 && raw) run_output<128, bf16, true>(p, s);
  else if (p.K == 128 && bf) run_output<128, bf16, false>(p, s);
  else if (p.K == 128) run_output<128, float, false>(p, s);
  else if (p.K == 64 && raw) run_output<64, bf16, true>(p, s);
  else if (p.K == 64 && bf) run_output<64, bf16, false>(p, s);
  else if (p.K == 64) run_output<64, float, false>(p, s);
  else return static_cast<int>(hipErrorInvalidValue);
  return static_cast<int>(hipGetLastError());
}

}  // namespace gdr

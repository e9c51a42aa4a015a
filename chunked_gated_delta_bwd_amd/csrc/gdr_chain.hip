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
// Workgroups have nine waves with fixed jobs (thirteen with two V slices a
// workgroup: compute waves 4-7 for the second slice, the converter and movers
// after them):
//   waves 0-3  compute: the MFMA products of one chunk step, two barriers a step;
//              their results for later kernels (S, U or dS, dU of the chunk) go
//              to LDS only; for the scalar gate with bf16 inputs they also turn
//              the next chunk's dO slice into fq dO in bf16 high + low parts;
//   wave  4    converter: writes those slices from LDS to global memory with
//              16-byte stores (dU one step late, from a second buffer, where LDS
//              allows), and for fp32 inputs forms dO high + low from registers
//              loaded one step ahead;
//   waves 5-8  movers: copy the chunk tiles and the small per-chunk data (dO
//              slice, row factors, decay) global -> LDS with direct-to-LDS loads
//              (no registers, no ALU), up to two chunks ahead.
// Every big tile has two LDS buffers (chunk k in buffer k % 2), the small data
// three rotating slots.  Set A, read only in the first window of a step (between
// its barriers B1 and B2), is refilled after B2 with the chunk two steps ahead
// (one and a half steps to land); set B, read in the second window (and in the
// reverse role in the first as well), is refilled after the next B1 with the
// next chunk (one step to land).  The movers wait for their own loads with
// vmcnt before the barrier that publishes them.
//
// Sequences may be split into segments (runs of whole chunks; one segment per
// sequence unless the host splits them): both recursions are affine in the
// carried state, S_{n+1} = S_n F_n + U'^T Khat with F_n = Diag(e^GamC) - W^T Khat,
// and dS_n = dS_{n+1} F_n^T + (Qbar^T dO - (P^T dO)^T W).  A local pass runs each
// segment from a zero state (the first one of a role from h0 / dht) and carries
// the transfer product of its chunks as D more rows of the state, started at the
// identity with the U' and dO terms left out; k_chain_fix composes the true
// boundary states in order, and the final pass runs every segment from its true
// state and stores the per-chunk outputs.  (The FlashQLA overview, section 3,
// shards the state-gradient recursion over devices with warm-up chunks instead;
// here the composition is exact.)
//
// Tiles are stored unpadded with an XOR swizzle of their 16-byte pieces (one
// direct-to-LDS load writes 1 KB contiguously, so the swizzle is applied by
// choosing which global piece each lane fetches).
//
// The scalar gate with bf16 inputs reads the raw q and k rows and applies the
// row factors of Qbar = q (scale e^Gam / |q|) and Khat = k (e^(GamC - Gam) / |k|)
// to the small operands instead (dO rows, U rows, dU rows); the per-channel
// gate and fp32 inputs take the Khat / Qbar tiles the prologue kernel formed.
// Qbar^T dO carries the dominant part of dh0, so that product is taken in two
// bf16 parts (Qbar high + low, or the scaled dO high + low).
//
// Where the gate barely decays, a step's bf16 roundings are not damped by the
// following steps and accumulate over the sequence.  The scalar gate's reverse
// steps whose error reaches dh0 with little damping then take dS, dU and (raw
// mode) Y in two parts (a second launch, k_chain<..., TWO = true>, for the
// segments that have such steps; with fp32 inputs where the LDS holds the low
// parts, D = 64); the per-channel gate's forward steps on chunks with a barely
// decaying channel take Khat in two parts (the same launch, chain_fwd<..., TWO>).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gdr_device.h"
#include "gdr_internal.h"
#include "gdr_lds.h"

namespace gdr {


// ---------------------------------------------------------------------------
// LDS plan
// ---------------------------------------------------------------------------
// NSL: V slices per workgroup (two share the chunk tiles: raw mode only, where
// LDS allows; waves 0-3 compute for the first slice, 4-7 for the second)
template <int D, typename TIO, int GATE, int NSL = 1>
struct ChainCfg {
  static constexpr bool LO = std::is_same<TIO, float>::value;  // fp32 inputs: dO split in two parts
  static constexpr bool MAT = GATE == 1 || LO;                 // materialised Khat / Qbar tiles
  static constexpr bool RAW = !MAT;                            // raw q, k rows and row factors
  static constexpr bool SPLIT = GATE == 1;   // U', U, S, dS also carried as bf16 high + low parts
  static_assert(NSL == 1 || (NSL == 2 && RAW), "two slices a workgroup in raw mode only");
  static constexpr int NCW = 4 * NSL;                      // compute waves
  static constexpr int CONV = NCW, MOVE0 = NCW + 1;        // converter, first of four movers
  static constexpr int WAVES = NCW + 5, THREADS = 64 * WAVES;
  static constexpr int NPF = NSL;                          // L2 prefetch loads per mover wave and step
  static constexpr int DG = GATE == 1 ? D : 16;    // decay floats per slot (scalar: one value, 64-byte slot part)
  static constexpr int TB = C * D * 2;             // one 64 x D bf16 tile
  static constexpr int PB = C * C * 2;             // the 64 x 64 P tile
  static constexpr int XB = C * 16 * 2;            // a 64 x 16 bf16 slice
  static constexpr int NJ = TB / 4096;             // 1 KB loads per mover wave per 64 x D tile
  // small per-chunk data, three rotating slots: the raw dO slices (bf16 inputs, one
  // per V slice), the row factors fq, fk, fw (raw mode) and the decay
  static constexpr int NFAC = 3;
  static constexpr int sDO = 0;
  static constexpr int sFac = sDO + (LO ? 0 : NSL * XB);
  static constexpr int sDec = sFac + (RAW ? NFAC * C * 4 : 0);
  static constexpr int SLOT = sDec + DG * 4;
  // reverse role, byte offsets; the tile buffers first.  Materialised tiles:
  // Khat, Qbar high, low, W, P.  Raw mode: q, P (set A), k, A (set B), where
  // W^T dU is formed as k^T (Diag(fw) A^T dU) from the raw k rows already there
  static constexpr int bK = 0, bQh = TB, bQl = 2 * TB, bW = 3 * TB;
  static constexpr int bP = MAT ? 4 * TB : 2 * TB;
  static constexpr int bA = 2 * TB + PB;                           // raw mode
  // The reverse steps of weakly decaying chunks take dS and dU^T in two bf16
  // parts: in raw mode always; with materialised tiles (fp32 inputs, scalar gate)
  // at kMatTwoPartK-wide heads, where Khat and W come in two parts as well (their
  // low tiles, set A and set B, loaded by the two-part kernel only)
  static constexpr bool TWOM = LO && GATE == 0 && D == kMatTwoPartK;
  static constexpr bool LOWB = RAW || TWOM;
  static constexpr int bKl = 4 * TB + PB, bWl = 5 * TB + PB;       // TWOM
  static constexpr int bufB = MAT ? 4 * TB + PB + (TWOM ? 2 * TB : 0) : 2 * TB + 2 * PB;
  // per-slice parts: slice s, buffer b at X + (2 s + b) XB
  static constexpr int bX1 = 2 * bufB;                             // LO: dO high part
  static constexpr int bX2 = bX1 + (LO ? 2 * XB : 0);              // RAW: fq dO high; LO: dO low
  static constexpr int bX3 = bX2 + ((RAW || LO) ? 2 * NSL * XB : 0);   // RAW: fq dO low
  static constexpr int bSlot = bX3 + (RAW ? 2 * NSL * XB : 0);
  static constexpr int bdS = bSlot + 3 * SLOT;                     // 16 x D state-gradient slice, each slice
  static constexpr int dUB = 16 * C * 2;
  // the low parts of the dS slices and of the dU^T buffers, each a fixed distance
  // above its high part (one lane address serves both)
  static constexpr int bdSl = bdS + NSL * 16 * D * 2;
  static constexpr int bdU = bdSl + (LOWB ? NSL * 16 * D * 2 : 0);  // 16 x 64: dU^T, each slice
  // dU^T in two buffers (step parity) where LDS allows: the converter then stores
  // it during the next step instead of holding up the first barrier
  static constexpr int NDU = bdU + (LOWB ? 4 : 2) * NSL * dUB + 256 <= 160 * 1024 ? 2 : 1;
  static constexpr int bdUl = bdU + NSL * NDU * dUB;
  static constexpr int bPF = bdUl + (LOWB ? NSL * NDU * dUB : 0);  // 256 B sink of the L2 prefetches
  static constexpr int bEnd = bPF + 256;
  // forward role
  // forward role: materialised tiles W, Khat; raw mode A (in W's place) and k,
  // with W S^T formed as A (Diag(fw) k S^T)
  // (the U' slices of the NSL slices in one region: element (s, r, c) at
  // ((r / 16) NSL + s) 512 + (r % 16) 32 + 2c bytes, one mover load covering 16 rows of all)
  // (per-channel gate: Khat's low part for the weak-chunk kernel, fKl)
  static constexpr int fW = 0, fA = 0, fK = MAT ? TB : PB, fUp = fK + TB, fUpl = fUp + NSL * XB;
  static constexpr int fKl = fUpl + (SPLIT ? XB : 0);
  static constexpr int bufF = fKl + (SPLIT ? TB : 0);
  static constexpr int fSlot = 2 * bufF;
  static constexpr int fS = fSlot + 3 * SLOT;                      // 16 x D state slice, each slice
  static constexpr int fU = fS + NSL * 16 * D * 2;                 // 16 x 64: U^T as the MFMA takes it, each slice
  static constexpr int fUo = fU + NSL * 16 * C * 2;                // RAW: unscaled U^T, to be stored, each slice
  static constexpr int fUl = fUo + (RAW ? NSL * 16 * C * 2 : 0);   // SPLIT: low part of U^T
  static constexpr int fSl = fUl + (SPLIT ? 16 * C * 2 : 0);       // SPLIT: low part of the state slice
  static constexpr int fPF = fSl + (SPLIT ? 16 * D * 2 : 0);
  static constexpr int fEnd = fPF + 256;
  static constexpr int bytes = bEnd > fEnd ? bEnd : fEnd;
  // mover loads per wave per chunk: first-window set A, second-window set B
  // (set B carries the small data of the chunk after its own)
  // small data loads per mover wave and chunk, counted as one (movers that issue
  // none wait for one fewer: wait_mover)
  static constexpr int nSb = 1;
  static constexpr int nSf = 1;
  static constexpr int bwdA = NJ + 2, bwdB = (MAT ? 3 * NJ : NJ + 2) + nSb;
  // the two-part kernel's counts (TWOM: the low tiles of Khat and W too)
  static constexpr int bwdA2 = bwdA + (TWOM ? NJ : 0), bwdB2 = bwdB + (TWOM ? NJ : 0);
  // L2 prefetch distance in chunk steps (one prefetch load per mover wave per
  // step), the best of 2 .. 6 measured for each form: raw rows with one slice a
  // workgroup 5, two slices 3 (each step twice as long), materialised tiles 4
  static constexpr int PFD = MAT ? 4 : NSL == 2 ? 3 : 5;
  static constexpr int fwdA = (MAT ? NJ : 2) + 1 + (SPLIT ? 1 : 0), fwdB = NJ + nSf;
  static_assert(bytes <= 160 * 1024, "LDS budget");
  static_assert(2 * bwdA2 + bwdB2 + (PFD - 2) * NPF < 64 && 2 * fwdA + fwdB + (PFD - 2) * NPF < 64, "vmcnt range");
};

// The segment entry of a workgroup, read once into scalar registers (left in
// memory, the compiler may reload it with a vector load inside a chunk loop, and
// a mover's wait for that load drains all of its tile loads in flight)
__device__ __forceinline__ SeqEntry seq_entry(const Params& p, int si) {
  const SeqEntry e = p.stab[si];
  SeqEntry r;
  r.seq = __builtin_amdgcn_readfirstlane(e.seq);
  r.len = __builtin_amdgcn_readfirstlane(e.len);
  r.c0 = __builtin_amdgcn_readfirstlane(e.c0);
  r.nchunks = __builtin_amdgcn_readfirstlane(e.nchunks);
  r.t_start = __builtin_amdgcn_readfirstlane(e.t_start);
  r.seg = __builtin_amdgcn_readfirstlane(e.seg);
  r.nseg = __builtin_amdgcn_readfirstlane(e.nseg);
  r.slot = __builtin_amdgcn_readfirstlane(e.slot);
  return r;
}

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

// ---------------------------------------------------------------------------
// movers: mover wave mw fills bytes [mw T/4, (mw+1) T/4) of a tile T
// ---------------------------------------------------------------------------
// Every address is a per-chunk scalar base plus a lane offset.  The lane offsets
// (the swizzle, the lane's row and piece) are computed once and hidden from the
// compiler (keep()), which would otherwise recompute them, with a division and
// 64-bit arithmetic, for every load of every chunk step on the SIMDs the compute
// waves run on; only the last, partial chunk of a sequence takes clamped offsets.
__device__ __forceinline__ void keep(int& x) { asm volatile("" : "+v"(x)); }

template <int D>
struct MoverLane {
  int rD[4], pD[4], tD[4];   // 64 x D tile, load j: row, swizzled piece byte offset, in-tile offset
  int rowoff[4];             // q / k token rows of a whole chunk, load j: byte offset from its first row
  int tP[2];                 // P tile, load j: in-tile offset
  int up;                    // the U' slices' part of a 64 x D tile: row * 2D + byte offset
  int drow, doff;            // dO halves (movers 0, 1): logical row; byte offset, whole chunk
  int rs, ds;                // byte strides of q / k rows and of dO rows (scalars)
  int hk;                    // the key head of value head h (scalar)
  template <int NSL>
  __device__ __forceinline__ void init(const Params& p, int h, int mw, int l, int dsz) {
    constexpr int RB = 2 * D, TB = C * RB, NJ = TB / 4096;
    rs = __builtin_amdgcn_readfirstlane(p.Hk * D * 2);
    ds = __builtin_amdgcn_readfirstlane(p.H * D * dsz);
    hk = __builtin_amdgcn_readfirstlane(h / p.G);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pos = mw * (TB / 4) + (j < NJ ? j : 0) * 1024 + 16 * l;
      const int row = pos / RB, lp = ((pos % RB) >> 4) ^ swz<D, 0>(row);
      rD[j] = row;
      pD[j] = lp << 4;
      tD[j] = row * RB + (lp << 4);
      rowoff[j] = row * rs + (lp << 4);
      keep(rD[j]);
      keep(pD[j]);
      keep(tD[j]);
      keep(rowoff[j]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int pos = mw * 2048 + j * 1024 + 16 * l;
      const int row = pos >> 7, lp = ((pos & 127) >> 4) ^ swz<64, 0>(row);
      tP[j] = row * 128 + (lp << 4);
      keep(tP[j]);
    }
    // U' slices: one slice, lanes 0-31, 16 rows x 32 bytes; two slices, lane l
    // 16 rows x 64 bytes (slice l / 32 in the upper half of the lanes)
    up = NSL == 1 ? (16 * mw + ((l & 31) >> 1)) * RB + ((l & 1) << 4)
                  : (16 * mw + ((l & 31) >> 1)) * RB + (l >> 5) * 32 + ((l & 1) << 4);
    drow = prow<16>(32 * (mw & 1) + (l >> 1));   // logical row landing at physical row 32 mw + l/2
    doff = drow * ds + (l & 1) * 16;
    keep(up);
    keep(drow);
    keep(doff);
  }
};

// a 64 x D tile stored contiguously at `src` (workspace layout [64][D])
template <int D>
__device__ __forceinline__ void move_tile(const MoverLane<D>& ml, const void* src, char* dst, int mw) {
  constexpr int TB = C * D * 2, NJ = TB / 4096;
  const char* s = static_cast<const char*>(src);
#pragma unroll
  for (int j = 0; j < NJ; ++j) dma16(s + uint32_t(ml.tD[j]), dst + mw * (TB / 4) + j * 1024);
}

// a 64 x D tile of raw token rows (q or k of the key head that value head h reads),
// rows past the end clamped
template <int D>
__device__ __forceinline__ void move_rows(const MoverLane<D>& ml, const void* base, const ChunkGeo& cg, char* dst,
                                          int mw) {
  constexpr int TB = C * D * 2, NJ = TB / 4096;
  const char* s = static_cast<const char*>(base) + (int64_t(cg.t0) * (ml.rs / (D * 2)) + ml.hk) * (D * 2);
  if (cg.len == C) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) dma16(s + uint32_t(ml.rowoff[j]), dst + mw * (TB / 4) + j * 1024);
  } else {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      dma16(s + uint32_t(min(ml.rD[j], cg.len - 1) * ml.rs + ml.pD[j]), dst + mw * (TB / 4) + j * 1024);
  }
}

template <int D>
__device__ __forceinline__ void move_p(const MoverLane<D>& ml, const void* src, char* dst, int mw) {
  const char* s = static_cast<const char*>(src);
#pragma unroll
  for (int j = 0; j < 2; ++j) dma16(s + uint32_t(ml.tP[j]), dst + mw * 2048 + j * 1024);
}

// small data of chunk c into a slot: the dO slice (reverse role), fq / fk, decay,
// in as few whole-wave loads as possible (a load costs about the same however few
// bytes it carries): reverse role, movers 0 and 1 one half of the dO slice each
// (rows 32 mw .. 32 mw + 31, two pieces a row), mover 2 the row factors and the
// decay together (contiguous in the slot); forward role, mover 0 the latter.
// small_loads() is the number of loads a mover issues here (0 or 1).
template <int D, typename TIO, int GATE, int NSL>
__device__ __forceinline__ bool small_loads(int mw, bool with_dO) {
  using Cf = ChainCfg<D, TIO, GATE, NSL>;
  if constexpr (Cf::LO) return false;
  return with_dO ? mw < 2 * NSL + 1 : mw == 0;
}

// (two slices: movers 0, 1 the halves of the first dO slice, 2, 3 of the second,
// mover 0 the row factors and decay as well)
template <int D, typename TIO, int GATE, int NSL>
__device__ __forceinline__ void move_small(const MoverLane<D>& ml, const Params& p, const SeqEntry& se, int h, int c,
                                           int v0, char* slot, int mw, bool with_dO) {
  using Cf = ChainCfg<D, TIO, GATE, NSL>;
  if constexpr (!Cf::LO) {
    const ChunkGeo cg = geo(p, se, h, c);
    const int l = lane_id();
    if (with_dO && mw < 2 * NSL) {
      const int sv = mw >> 1;   // the slice
      const char* s = reinterpret_cast<const char*>(p.dO) + ((int64_t(cg.t0) * p.H + h) * D + v0 + 16 * sv) * 2;
      const int o = cg.len == C ? ml.doff : min(ml.drow, cg.len - 1) * ml.ds + (l & 1) * 16;
      dma16(s + uint32_t(o), slot + Cf::sDO + sv * Cf::XB + (mw & 1) * 1024);
    }
    if (mw == (with_dO && NSL == 1 ? 2 : 0)) {
      if constexpr (Cf::RAW) {
        // fq, fk, fw (768 bytes, lanes 0-47), then the decay (lane 48) right behind them
        constexpr int NL = Cf::NFAC * C * 4 / 16;
        static_assert(Cf::sDec == Cf::sFac + NL * 16, "decay follows the row factors");
        if (l < NL) dma16(reinterpret_cast<const char*>(p.fac + cg.ch * Cf::NFAC * C) + l * 16, slot + Cf::sFac);
        else if (l == NL) dma16(p.edec + cg.ch * 4, slot + Cf::sFac);
      } else {
        if (l < D / 4) dma16(reinterpret_cast<const char*>(p.edec + cg.ch * D) + l * 16, slot + Cf::sDec);
      }
    }
  }
}

// s_waitcnt vmcnt for the movers: every wait below counts one small load; a mover
// that issues none (small_loads() false) waits for one fewer
template <int N>
__device__ __forceinline__ void wait_mover(bool has_small) {
  static_assert(N >= 1, "count includes the small load");
  if (has_small) wait_vm<N>();
  else wait_vm<N - 1>();
}

// reverse role: set A (Khat, P; raw mode q, P), set B (Qbar high + low, W; raw
// mode k, A); TWO with materialised tiles: the low tiles of Khat (set A) and W
// (set B) as well
template <int D, typename TIO, int GATE, bool TWO = false>
__device__ __forceinline__ void move_bwd_a(const MoverLane<D>& ml, const Params& p, const SeqEntry& se, int h, int c,
                                           char* buf, int mw) {
  using Cf = ChainCfg<D, TIO, GATE>;
  const ChunkGeo cg = geo(p, se, h, c);
  if constexpr (Cf::RAW)
    move_rows<D>(ml, p.q, cg, buf + Cf::bQh, mw);
  else
    move_tile<D>(ml, p.Kh + cg.ch * C * D, buf + Cf::bK, mw);
  move_p<D>(ml, p.P + cg.ch * C * C, buf + Cf::bP, mw);
  if constexpr (TWO && Cf::TWOM) move_tile<D>(ml, p.Khl + cg.ch * C * D, buf + Cf::bKl, mw);
}

template <int D, typename TIO, int GATE, bool TWO = false>
__device__ __forceinline__ void move_bwd_b(const MoverLane<D>& ml, const Params& p, const SeqEntry& se, int h, int c,
                                           char* buf, int mw) {
  using Cf = ChainCfg<D, TIO, GATE>;
  const ChunkGeo cg = geo(p, se, h, c);
  if constexpr (Cf::RAW) {
    move_rows<D>(ml, p.k, cg, buf + Cf::bK, mw);
    move_p<D>(ml, p.A + cg.ch * C * C, buf + Cf::bA, mw);
  } else {
    move_tile<D>(ml, p.Qh + cg.ch * C * D, buf + Cf::bQh, mw);
    move_tile<D>(ml, p.Ql + cg.ch * C * D, buf + Cf::bQl, mw);
    move_tile<D>(ml, p.W + cg.ch * C * D, buf + Cf::bW, mw);
    if constexpr (TWO && Cf::TWOM) move_tile<D>(ml, p.Wl + cg.ch * C * D, buf + Cf::bWl, mw);
  }
}

// forward role: set A (W or, raw mode, A; the U' slice), set B (Khat or k)
template <int D, typename TIO, int GATE, int NSL>
__device__ __forceinline__ void move_fwd_a(const MoverLane<D>& ml, const Params& p, const SeqEntry& se, int h, int c,
                                           int v0, char* buf, int mw) {
  using Cf = ChainCfg<D, TIO, GATE, NSL>;
  const ChunkGeo cg = geo(p, se, h, c);
  if constexpr (Cf::MAT)
    move_tile<D>(ml, p.W + cg.ch * C * D, buf + Cf::fW, mw);
  else
    move_p<D>(ml, p.A + cg.ch * C * C, buf + Cf::fA, mw);
  if (NSL == 2 || lane_id() < 32)
    dma16(reinterpret_cast<const char*>(p.Up + cg.ch * C * D + v0) + ml.up, buf + Cf::fUp + mw * 512 * NSL);
  if constexpr (Cf::SPLIT) {
    if (lane_id() < 32)
      dma16(reinterpret_cast<const char*>(p.Uplo + cg.ch * C * D + v0) + ml.up, buf + Cf::fUpl + mw * 512);
  }
}

// (TWO, per-channel gate: Khat's low part too, written by the prologue for weak
// chunks only; the tile of another chunk is loaded but not read)
template <int D, typename TIO, int GATE, bool TWO = false>
__device__ __forceinline__ void move_fwd_b(const MoverLane<D>& ml, const Params& p, const SeqEntry& se, int h, int c,
                                           char* buf, int mw) {
  using Cf = ChainCfg<D, TIO, GATE>;
  const ChunkGeo cg = geo(p, se, h, c);
  if constexpr (Cf::RAW) {
    move_rows<D>(ml, p.k, cg, buf + Cf::fK, mw);
  } else {
    move_tile<D>(ml, p.Kh + cg.ch * C * D, buf + Cf::fK, mw);
    if constexpr (TWO) move_tile<D>(ml, p.Khl + cg.ch * C * D, buf + Cf::fKl, mw);
  }
}

// L2 prefetch of chunk c, three steps beyond the direct-to-LDS loads: the V
// slices of one (sequence, head) read the same tiles, so slice sl touches only
// rows [sl R, (sl+1) R) of them (R = 64 / slices), mover wave mw a quarter of
// those, one 4-byte load per 64-byte sector into a sink that is never read.  The
// lane plan (which rows a lane touches, its row and byte offset) is computed once;
// a step adds the chunk's scalar base of the lane's kind of rows.
template <int D, typename TIO, int GATE, bool BWD>
struct PfLane {
  using Cf = ChainCfg<D, TIO, GATE>;
  static constexpr int ns = D / 16, R = C / ns, RW = R / 4;
  static constexpr int LB = 64;                                   // bytes per prefetch load
  static constexpr int LPR = (2 * D) / LB;                        // loads per row of a 64 x D bf16 tile
  static constexpr int DOL = int(D * sizeof(TIO)) / LB;           // loads per dO row of one head
  static constexpr int NP = 128 / LB;                             // loads per row of a 64 x 64 tile
  static constexpr int NT = BWD ? (Cf::MAT ? 4 : 2) : (Cf::MAT ? 2 : 1);   // tiles with D-wide rows
  static constexpr int NT64 = BWD ? (Cf::MAT ? 1 : 2) : (Cf::MAT ? 0 : 1);  // 64 x 64 tiles (P, A)
  static constexpr int NTAIL = (Cf::RAW ? Cf::NFAC * C * 4 : 512) / LB;   // row factors or the decay
  static constexpr int N1 = NT * RW * LPR, N2 = N1 + NT64 * RW * NP, N3 = N2 + (BWD ? RW * DOL : RW * LPR);
  static_assert(N3 + NTAIL <= 64, "one prefetch load per wave");
  // kinds: 0 .. NT - 1 the D-wide tiles (reverse: Khat, Qbar high, low, W; raw
  // mode k, q; forward: W, Khat; raw mode k), then the 64 x 64 tiles (reverse: P,
  // raw mode A too; forward, raw mode: A), then the dO rows (reverse) or U' rows
  // (forward), then the row factors or decay; -1 idle
  static constexpr int KR = NT + NT64, KT = KR + 1, NK = KR + 2;
  int kind, row, col, stride, off;
  bool tok;   // token rows (clamped at the end of a sequence)

  __device__ __forceinline__ void init(const Params& p, int sl, int mw, int l) {
    const int r0 = sl * R + mw * RW;
    kind = -1;
    row = 0;
    col = 0;
    stride = 0;
    tok = false;
    if (l < N1) {
      const int t = l / (RW * LPR), rem = l % (RW * LPR);
      kind = t;
      row = r0 + rem / LPR;
      col = (rem % LPR) * LB;
      tok = Cf::RAW;
      stride = tok ? p.Hk * D * 2 : D * 2;
    } else if (l < N2) {
      const int i = l - N1, t = i / (RW * NP), rem = i % (RW * NP);
      kind = NT + t;
      row = r0 + rem / NP;
      col = (rem % NP) * LB;
      stride = C * 2;
    } else if (l < N3) {
      const int i = l - N2;
      kind = KR;
      if constexpr (BWD) {
        row = r0 + i / DOL;
        col = (i % DOL) * LB;
        tok = true;
        stride = p.H * D * int(sizeof(TIO));
      } else {
        row = r0 + i / LPR;
        col = (i % LPR) * LB;
        stride = D * 2;
      }
    } else if (sl == 0 && mw == 0 && l < N3 + NTAIL) {
      const int i = l - N3;
      kind = KT;
      col = Cf::RAW ? i * LB : (i * LB) % (GATE == 1 ? D * 4 : 16);
    }
    off = row * stride + col;
    keep(kind);
    keep(row);
    keep(col);
    keep(stride);
    keep(off);
  }
};

// a pointer the whole wave holds, pinned in scalar registers (a choice between
// such pointers per lane is then register moves; chosen among Params fields
// directly, the compiler turns it into a per-lane load from the kernel arguments,
// and the wait for that load drains every load in flight)
__device__ __forceinline__ const char* wave_ptr(const void* q) {
  const uint64_t u = reinterpret_cast<uint64_t>(q);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(u)), hi = __builtin_amdgcn_readfirstlane(uint32_t(u >> 32));
  return reinterpret_cast<const char*>((uint64_t(hi) << 32) | lo);
}

template <int D, typename TIO, int GATE, bool BWD>
__device__ __forceinline__ void prefetch_chunk(const PfLane<D, TIO, GATE, BWD>& pf, const MoverLane<D>& ml,
                                               const Params& p, const SeqEntry& se, int h, int c, char* sink) {
  using Cf = ChainCfg<D, TIO, GATE>;
  using Pl = PfLane<D, TIO, GATE, BWD>;
  const ChunkGeo cg = geo(p, se, h, c);
  const int64_t tb = cg.ch * C * D * 2;                                    // a workspace 64 x D tile
  const int64_t qk = (int64_t(cg.t0) * p.Hk + ml.hk) * D * 2;             // q, k rows of the key head
  auto base = [&](int kd) -> const char* {
    if (kd < Pl::NT) {
      if constexpr (BWD) {
        if constexpr (Cf::RAW)
          return reinterpret_cast<const char*>(kd == 0 ? p.k : p.q) + qk;
        else
          return reinterpret_cast<const char*>(kd == 0 ? p.Kh : kd == 1 ? p.Qh : kd == 2 ? p.Ql : p.W) + tb;
      } else {
        if constexpr (Cf::RAW)
          return reinterpret_cast<const char*>(p.k) + qk;
        else
          return reinterpret_cast<const char*>(kd == 0 ? p.W : p.Kh) + tb;
      }
    }
    if (kd < Pl::KR) return reinterpret_cast<const char*>(BWD && kd == Pl::NT ? p.P : p.A) + cg.ch * C * C * 2;
    if (kd == Pl::KR) {
      if constexpr (BWD)
        return reinterpret_cast<const char*>(p.dO) + (int64_t(cg.t0) * p.H + h) * D * int64_t(sizeof(TIO));
      else
        return reinterpret_cast<const char*>(p.Up) + tb;
    }
    if constexpr (Cf::RAW) return reinterpret_cast<const char*>(p.fac + cg.ch * Cf::NFAC * C);
    else return reinterpret_cast<const char*>(p.edec + cg.ch * (GATE == 1 ? D : 4));
  };
  const char* a = wave_ptr(base(0));
#pragma unroll
  for (int kd = 1; kd < Pl::NK; ++kd) {
    const char* b = wave_ptr(base(kd));
    a = pf.kind == kd ? b : a;
  }
  const int o = pf.tok && cg.len < C ? min(pf.row, cg.len - 1) * pf.stride + pf.col : pf.off;
  if (pf.kind >= 0) dma4(a + uint32_t(o), sink);
}

// ---------------------------------------------------------------------------
// converter (wave 4)
// ---------------------------------------------------------------------------
// Copies a 16-row slice tile (W columns, swizzled in LDS) to 16 contiguous global
// rows with 16-byte stores.
template <int W, int KIND = 0>
__device__ __forceinline__ void store_slice(const char* T, uint16_t* dst) {
  constexpr int BYTES = 16 * W * 2;
  const int l = lane_id();
#pragma unroll
  for (int i = 0; i < BYTES / 1024; ++i) {
    const int pos = i * 1024 + 16 * l;
    const int row = pos / (2 * W), piece = (pos % (2 * W)) >> 4;
    const u32x4 v = *reinterpret_cast<const u32x4*>(T + soff<W, KIND>(row, piece * 8));
    *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(dst) + pos) = v;
  }
}

// fp32 inputs: the converter loads the chunk's dO rows and decay into registers
// one step ahead and writes dO high / low parts and the decay to LDS
template <int D, typename TIO, int GATE>
struct LoRegs {
  static constexpr int ND = GATE == 1 ? D / 64 : 1;
  typename IO<TIO>::Raw8 d0, d1;   // 16 dO values of row l
  float m;
  float dec[ND];

  __device__ __forceinline__ void load(const Params& p, const SeqEntry& se, int h, int c, int v0, bool with_dO) {
    const int l = lane_id();
    const ChunkGeo cg = geo(p, se, h, c);
    if (with_dO) {
      const int64_t o = tok(cg.t0 + min(l, cg.len - 1), p.H, h) * D + v0;
      d0 = IO<TIO>::load_raw8(p.dO, o);
      d1 = IO<TIO>::load_raw8(p.dO, o + 8);
    }
    m = l < cg.len ? 1.f : 0.f;
    if constexpr (GATE == 1) {
#pragma unroll
      for (int i = 0; i < ND; ++i) dec[i] = p.edec[cg.ch * D + ND * l + i];
    } else {
      dec[0] = p.edec[cg.ch * 4];
    }
  }

  __device__ __forceinline__ void store_dO(char* x1, char* x2) const {
    const int l = lane_id();
    float a[8], b[8];
    IO<TIO>::unpack8(d0, a);
    IO<TIO>::unpack8(d1, b);
    bf16x8 h0, h1, l0, l1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xa = m * a[e], xb = m * b[e];
      h0[e] = to_bf16(xa);
      h1[e] = to_bf16(xb);
      l0[e] = to_bf16(xa - float(h0[e]));
      l1[e] = to_bf16(xb - float(h1[e]));
    }
    const int o = prow<16>(l) * 32;
    *reinterpret_cast<bf16x8*>(x1 + o) = h0;
    *reinterpret_cast<bf16x8*>(x1 + o + 16) = h1;
    *reinterpret_cast<bf16x8*>(x2 + o) = l0;
    *reinterpret_cast<bf16x8*>(x2 + o + 16) = l1;
  }

  __device__ __forceinline__ void store_dec(float* dst) const {
    const int l = lane_id();
    if constexpr (GATE == 1) {
#pragma unroll
      for (int i = 0; i < ND; ++i) dst[ND * l + i] = dec[i];
    } else {
      if (l == 0) dst[0] = dec[0];
    }
  }
};

// scalar gate, bf16 inputs: fq dO of the chunk's dO slice in bf16 high + low
// parts (X2, X3), rows 16w .. 16w+15 by compute wave w (lane: row 16w + l/4,
// columns 4(l%4) .. +3)
template <int D, typename TIO, int GATE, int NSL>
__device__ __forceinline__ void convert_raw_rows(const char* slot, int sv, char* x2, char* x3, int w, bool lo) {
  using Cf = ChainCfg<D, TIO, GATE, NSL>;
  const int l = lane_id();
  const int row = 16 * w + (l >> 2), o = prow<16>(row) * 32 + (l & 3) * 8;
  const uint2 r = *reinterpret_cast<const uint2*>(slot + Cf::sDO + sv * Cf::XB + o);
  const float fq = reinterpret_cast<const float*>(slot + Cf::sFac)[row];
  const float a[4] = {bf16_bits_to_f32(r.x & 0xffffu), bf16_bits_to_f32(r.x >> 16), bf16_bits_to_f32(r.y & 0xffffu),
                      bf16_bits_to_f32(r.y >> 16)};
  float hv[4], lv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float y = fq * a[e];
    hv[e] = float(to_bf16(y));
    lv[e] = y - hv[e];
  }
  *reinterpret_cast<uint2*>(x2 + o) = pack4_bf16(hv[0], hv[1], hv[2], hv[3]);
  if (lo) *reinterpret_cast<uint2*>(x3 + o) = pack4_bf16(lv[0], lv[1], lv[2], lv[3]);
}

// the decay of this lane's four accumulator rows j = 16 jb + 4 g .. +3
template <int D, int GATE>
__device__ __forceinline__ f32x4 decay4(const float* dec, int jb, int g) {
  if constexpr (GATE == 1) {
    const float4 d = *reinterpret_cast<const float4*>(dec + 16 * jb + 4 * g);
    return f32x4{d.x, d.y, d.z, d.w};
  } else {
    const float d = dec[0];
    return f32x4{d, d, d, d};
  }
}

// ---------------------------------------------------------------------------
// what one workgroup's recursion starts from, where its end state goes, and
// whether it stores the per-chunk outputs
// ---------------------------------------------------------------------------
struct ChainJob {
  const float* init;   // the 16 x D slice it starts from (row stride D), or NULL: zero / identity
  float* fin;          // where the 16 x D end slice goes (row stride D), or NULL
  bool store;          // per-chunk outputs (S, U / dS, dU) to the workspace
  bool xfer;           // transfer rows: start at identity rows i0 .. i0 + 15, no U' / dO terms
  int i0;
  int v0l;             // V offset of the slice for loads of U' and dO (a state slice's own)
};

template <int D>
__device__ __forceinline__ void job_init(const ChainJob& job, f32x4 (&acc)[Dims<D>::NJW], int w, int g, int jj) {
  constexpr int NJW = Dims<D>::NJW;
#pragma unroll
  for (int x = 0; x < NJW; ++x) {
    const int j = 16 * (w * NJW + x) + 4 * g;
    if (job.init) {
      const float4 t = *reinterpret_cast<const float4*>(job.init + jj * D + j);
      acc[x] = f32x4{t.x, t.y, t.z, t.w};
    } else if (job.xfer) {
      const int r = job.i0 + jj;
      acc[x] = f32x4{r == j ? 1.f : 0.f, r == j + 1 ? 1.f : 0.f, r == j + 2 ? 1.f : 0.f, r == j + 3 ? 1.f : 0.f};
    } else {
      acc[x] = zero4();
    }
  }
}

template <int D>
__device__ __forceinline__ void job_fin(const ChainJob& job, const f32x4 (&acc)[Dims<D>::NJW], int w, int g, int jj) {
  constexpr int NJW = Dims<D>::NJW;
  if (!job.fin) return;
#pragma unroll
  for (int x = 0; x < NJW; ++x) {
    const int j = 16 * (w * NJW + x) + 4 * g;
    *reinterpret_cast<float4*>(job.fin + jj * D + j) = make_float4(acc[x][0], acc[x][1], acc[x][2], acc[x][3]);
  }
}

// ---------------------------------------------------------------------------
// the two roles
// ---------------------------------------------------------------------------
// the job of slice sv (0 .. NSL - 1), chosen by selects (a dynamic index into
// the array would put it in scratch memory)
template <int NSL>
__device__ __forceinline__ ChainJob job_of(const ChainJob (&jobs)[NSL], int sv) {
  if constexpr (NSL == 1) {
    return jobs[0];
  } else {
    const bool b = sv != 0;
    ChainJob j;
    j.init = b ? jobs[1].init : jobs[0].init;
    j.fin = b ? jobs[1].fin : jobs[0].fin;
    j.store = jobs[0].store;
    j.xfer = jobs[0].xfer;
    j.i0 = b ? jobs[1].i0 : jobs[0].i0;
    j.v0l = b ? jobs[1].v0l : jobs[0].v0l;
    return j;
  }
}

// TWO (per-channel gate): the form for segments with weak chunks, whose steps take
// Khat in two parts in the state update where the chunk is weak
template <int D, typename TIO, int GATE, int NSL, bool TWO = false>
__device__ __forceinline__ void chain_fwd(const Params& p, char* smem, int si, int h, int sl,
                                          const ChainJob (&jobs)[NSL]) {
  using Dm = Dims<D>;
  using Cf = ChainCfg<D, TIO, GATE, NSL>;
  static_assert(!TWO || Cf::SPLIT, "two-part forward steps for the per-channel gate only");
  // mover loads per wave in a chunk's second set (TWO: Khat's low part as well)
  constexpr int FB = Cf::fwdB + (TWO ? Cf::NJ : 0);
  static_assert(2 * Cf::fwdA + FB + (Cf::PFD - 2) * Cf::NPF < 64, "vmcnt range");
  constexpr int NJW = Dm::NJW;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = lane_id();
  const int g = l >> 4, jj = l & 15;
  const SeqEntry se = seq_entry(p, si);
  const int v0 = 16 * sl, v0l = jobs[0].v0l;   // the first slice's (the others follow, 16 apart)
  const int nck = se.nchunks;
  // slice sv's state, U^T and unscaled U^T tiles
  auto Ss_of = [&](int sv) { return smem + Cf::fS + sv * (16 * D * 2); };
  auto Ut_of = [&](int sv) { return smem + Cf::fU + sv * (16 * C * 2); };
  auto Uo_of = [&](int sv) { return smem + (Cf::RAW ? Cf::fUo : Cf::fU) + sv * (16 * C * 2); };
  auto chunk = [&](int k) { return se.c0 + min(k, nck - 1); };
  auto slot = [&](int k) { return smem + Cf::fSlot + (k % 3) * Cf::SLOT; };

  if (wv < Cf::NCW) {
    const int sv = wv >> 2, w = wv & 3;
    const ChainJob job = job_of<NSL>(jobs, sv);
    char* Ss = Ss_of(sv);
    char* Ut = Ut_of(sv);
    char* Uo = Uo_of(sv);
    f32x4 acc[NJW];
    job_init<D>(job, acc, w, g, jj);
    if (nck > 0) chain_barrier();   // B0
    for (int k = 0; k < nck; ++k) {
      const char* Fb = smem + (k & 1) * Cf::bufF;
      const char* sl_k = slot(k);
      // a weak chunk (TWO): read ahead of its use after the second barrier
      const bool wk = TWO && p.weak[int64_t(h) * p.NC + chunk(k)] != 0;
#pragma unroll
      for (int x = 0; x < NJW; ++x) {
        const int jc = 16 * (w * NJW + x);
        st4_q<D>(Ss, 0, jc, acc[x][0], acc[x][1], acc[x][2], acc[x][3]);
        if constexpr (Cf::SPLIT)
          st4_q<D>(smem + Cf::fSl, 0, jc, lo_part(acc[x][0]), lo_part(acc[x][1]), lo_part(acc[x][2]),
                   lo_part(acc[x][3]));
      }
      chain_barrier();   // B1
      // U = U' - W S^T, rows 16w.., columns of this slice
      f32x4 au = zero4();
      if constexpr (Cf::RAW) {
        // W S^T = A Y with Y = Diag(fw) k S^T (W = A Diag(fw) k): every wave forms all
        // 64 rows of Y (straight-line code schedules better than skipping the blocks
        // that A's zero upper blocks do not need) and feeds its accumulators, rounded
        // to bf16, straight back as the B operand, K-step kk pairing the row blocks
        // 2kk and 2kk+1 (frag_rk_split_s reads the rows of A in that column order)
        const float* fw = reinterpret_cast<const float*>(sl_k + Cf::sFac) + 2 * C;
        f32x4 y[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          y[rb] = zero4();
#pragma unroll
          for (int k0 = 0; k0 < D; k0 += 32)
            y[rb] = mma(frag_rk_s<D>(Fb + Cf::fK, 16 * rb, k0), frag_rk_s<D>(Ss, 0, k0), y[rb]);
          const float4 f = *reinterpret_cast<const float4*>(fw + 16 * rb + 4 * g);
          y[rb] *= f32x4{f.x, f.y, f.z, f.w};
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          bf16x8 yb;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            yb[i] = to_bf16(y[2 * kk][i]);
            yb[4 + i] = to_bf16(y[2 * kk + 1][i]);
          }
          au = mma(frag_rk_split_s<C>(Fb + Cf::fA, 16 * w, 32 * kk), yb, au);
        }
      } else {
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += 32) au = mma(frag_rk_s<D>(Fb + Cf::fW, 16 * w, k0), frag_rk_s<D>(Ss, 0, k0), au);
      }
      const uint16_t* Up = reinterpret_cast<const uint16_t*>(Fb + Cf::fUp);
      float u[4];
      // transfer rows: U' = 0
      const float um = job.xfer ? 0.f : 1.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) u[i] = um * bf16_bits_to_f32(Up[(w * NSL + sv) * 256 + (4 * g + i) * 16 + jj]) - au[i];
      if constexpr (Cf::SPLIT) {
        const uint16_t* Upl = reinterpret_cast<const uint16_t*>(Fb + Cf::fUpl);
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] += um * bf16_bits_to_f32(Upl[(16 * w + 4 * g + i) * 16 + jj]);
        st4_q<C, 1>(smem + Cf::fUl, 0, 16 * w, lo_part(u[0]), lo_part(u[1]), lo_part(u[2]), lo_part(u[3]));
      }
      if constexpr (Cf::RAW) {
        st4_q<C, 1>(Uo, 0, 16 * w, u[0], u[1], u[2], u[3]);
        const float4 f = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(sl_k + Cf::sFac) + C +
                                                          16 * w + 4 * g);
        u[0] *= f.x;
        u[1] *= f.y;
        u[2] *= f.z;
        u[3] *= f.w;
      }
      st4_q<C, 1>(Ut, 0, 16 * w, u[0], u[1], u[2], u[3]);
      chain_barrier();   // B2
      // S_{k+1}^T = Diag(e^GamC) S_k^T + Khat^T U (per-channel gate: U in two parts,
      // the low one also stored for the gradient kernel; U's bf16 rounding here is
      // the largest single term of the gate-parameter gradients' error, Khat's the
      // next one, which only weak chunks pay for)
      const float* dec = reinterpret_cast<const float*>(sl_k + Cf::sDec);
#pragma unroll
      for (int x = 0; x < NJW; ++x) {
        const int jb = w * NJW + x;
        f32x4 a = acc[x] * decay4<D, GATE>(dec, jb, g);
#pragma unroll
        for (int k0 = 0; k0 < C; k0 += 32) {
          const bf16x8 kh = frag_kc_s<D>(Fb + Cf::fK, 16 * jb, k0);
          const bf16x8 ut = frag_rk_s<C, 1>(Ut, 0, k0);
          a = mma(kh, ut, a);
          if constexpr (Cf::SPLIT) a = mma(kh, frag_rk_s<C, 1>(smem + Cf::fUl, 0, k0), a);
          if (TWO && wk) a = mma(frag_kc_s<D>(Fb + Cf::fKl, 16 * jb, k0), ut, a);
        }
        acc[x] = a;
      }
    }
    job_fin<D>(job, acc, w, g, jj);
  } else if (wv == Cf::CONV) {
    if (nck == 0) return;
    LoRegs<D, TIO, GATE> R;
    if constexpr (Cf::LO) {
      R.load(p, se, h, chunk(0), v0l, false);
      R.store_dec(reinterpret_cast<float*>(slot(0) + Cf::sDec));
      R.load(p, se, h, chunk(1), v0l, false);
    }
    const bool store = jobs[0].store;
    chain_barrier();   // B0
    for (int k = 0; k < nck; ++k) {
      const int64_t ch = int64_t(h) * p.NC + chunk(k);
      chain_barrier();   // B1
      if (store) {
#pragma unroll
        for (int sv = 0; sv < NSL; ++sv) store_slice<D>(Ss_of(sv), p.S + (ch * D + v0 + 16 * sv) * D);
        if constexpr (Cf::SPLIT) store_slice<D>(smem + Cf::fSl, p.Slo + (ch * D + v0) * D);
      }
      chain_barrier();   // B2
      if (store) {
#pragma unroll
        for (int sv = 0; sv < NSL; ++sv) store_slice<C, 1>(Uo_of(sv), p.U + (ch * D + v0 + 16 * sv) * C);
        if constexpr (Cf::SPLIT) store_slice<C, 1>(smem + Cf::fUl, p.Ulo + (ch * D + v0) * C);
      }
      if constexpr (Cf::LO) {
        R.store_dec(reinterpret_cast<float*>(slot(k + 1) + Cf::sDec));
        R.load(p, se, h, chunk(k + 2), v0l, false);
      }
    }
    wait_vm<0>();
  } else {
    if (nck == 0) return;
    constexpr int NPF = Cf::NPF;
    const int mw = wv - Cf::MOVE0;
    const bool hs = small_loads<D, TIO, GATE, NSL>(mw, false);
    MoverLane<D> ml;
    ml.template init<NSL>(p, h, mw, l, int(sizeof(TIO)));
    // the rows of the state slices whose U' this workgroup loads, one prefetch a slice
    PfLane<D, TIO, GATE, false> pf[NSL];
#pragma unroll
    for (int i = 0; i < NSL; ++i) pf[i].init(p, v0l / 16 + i, mw, l);
    auto prefetch = [&](int c) {
#pragma unroll
      for (int i = 0; i < NSL; ++i) prefetch_chunk<D, TIO, GATE, false>(pf[i], ml, p, se, h, c, smem + Cf::fPF);
    };
    move_small<D, TIO, GATE, NSL>(ml, p, se, h, chunk(0), v0l, slot(0), mw, false);
    move_fwd_a<D, TIO, GATE, NSL>(ml, p, se, h, chunk(0), v0l, smem, mw);
    move_fwd_b<D, TIO, GATE, TWO>(ml, p, se, h, chunk(0), smem, mw);
    move_small<D, TIO, GATE, NSL>(ml, p, se, h, chunk(1), v0l, slot(1), mw, false);
    move_fwd_a<D, TIO, GATE, NSL>(ml, p, se, h, chunk(1), v0l, smem + Cf::bufF, mw);
    for (int c = 2; c < Cf::PFD; ++c) prefetch(chunk(c));
    wait_mover<Cf::fwdA + FB + Cf::fwdA + (Cf::PFD - 2) * NPF>(hs);
    chain_barrier();   // B0
    // raw mode reads set B (k) in the first window too: both sets of chunk 0 land
    // before B1; otherwise set B may land by B2
    if constexpr (Cf::RAW) wait_mover<Cf::fwdA + 1 + (Cf::PFD - 2) * NPF>(hs);
    else wait_mover<FB + Cf::fwdA + (Cf::PFD - 2) * NPF>(hs);
    for (int k = 0; k < nck; ++k) {
      chain_barrier();   // B1
      move_fwd_b<D, TIO, GATE, TWO>(ml, p, se, h, chunk(k + 1), smem + ((k + 1) & 1) * Cf::bufF, mw);
      move_small<D, TIO, GATE, NSL>(ml, p, se, h, chunk(k + 2), v0l, slot(k + 2), mw, false);
      wait_mover<Cf::fwdA + NPF + FB>(hs);
      chain_barrier();   // B2
      move_fwd_a<D, TIO, GATE, NSL>(ml, p, se, h, chunk(k + 2), v0l, smem + (k & 1) * Cf::bufF, mw);
      prefetch(chunk(k + Cf::PFD));
      if constexpr (Cf::RAW) wait_mover<Cf::fwdA + NPF + 1>(hs);   // set B of chunk k + 1 before the next B1
      else wait_mover<FB + Cf::fwdA + 2 * NPF>(hs);
    }
    wait_vm<0>();
  }
}

// Raw mode: the reverse steps two_part_last() picks take the operands dS (in Khat
// dS^T), dU (in A^T dU) and Y (in k^T Y) in two bf16 parts.  A step's rounding
// error is proportional to e^GamC (Khat^T W is), and the earlier chunks damp it by
// their own decays on its way to dh0; with little decay it accumulates over the
// whole sequence (float64 model of the state-gradient recursion with each
// rounding switched on alone: at e^GamC = 1 each of the three gives 8e-4 relative
// error in dh0 over four chunks, 1.5e-3 together; at 1/16 all of them 5e-4).
// With materialised tiles (fp32 inputs, D = 64) the same steps take dS (in Khat
// dS^T) and dU (in W^T dU) in two parts.

// TWO: the kernel that runs the segments with weakly decaying chunks (their steps
// take two-part operands; the other steps the common ones)
template <int D, typename TIO, int GATE, int NSL, bool TWO>
__device__ __forceinline__ void chain_bwd(const Params& p, char* smem, int si, int h, int sl,
                                          const ChainJob (&jobs)[NSL], int two_last) {
  using Dm = Dims<D>;
  using Cf = ChainCfg<D, TIO, GATE, NSL>;
  constexpr int NJW = Dm::NJW;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = lane_id();
  const int g = l >> 4, jj = l & 15;
  const SeqEntry se = seq_entry(p, si);
  const int v0 = 16 * sl, v0l = jobs[0].v0l;   // the first slice's (the others follow, 16 apart)
  const int nck = se.nchunks;
  auto dS_of = [&](int sv) { return smem + Cf::bdS + sv * (16 * D * 2); };
  // slice sv's dU^T of step k (buffer k & 1 when there are two)
  auto dUbuf = [&](int sv, int k) {
    return smem + Cf::bdU + (sv * Cf::NDU + (Cf::NDU == 2 ? (k & 1) : 0)) * Cf::dUB;
  };
  // step k walks chunk c0 + nck - 1 - k (last to first), clamped past the end
  auto chunk = [&](int k) { return se.c0 + nck - 1 - min(k, nck - 1); };
  auto slot = [&](int k) { return smem + Cf::bSlot + (k % 3) * Cf::SLOT; };

  if (wv < Cf::NCW) {
    const int sv = wv >> 2, w = wv & 3;
    const ChainJob job = job_of<NSL>(jobs, sv);
    char* dSl = dS_of(sv);
    char* dSlo = dSl + (Cf::bdSl - Cf::bdS);
    // slice sv's fq dO high / low parts, buffer b
    auto X2_of = [&](int b) { return smem + Cf::bX2 + (2 * sv + b) * Cf::XB; };
    auto X3_of = [&](int b) { return smem + Cf::bX3 + (2 * sv + b) * Cf::XB; };
    f32x4 acc[NJW];
    job_init<D>(job, acc, w, g, jj);
    if (nck > 0) chain_barrier();   // B0
    // Qbar^T dO's low part (raw mode the fq dO low slice, else the Qbar low tile).
    // Scalar gate: a chunk's term reaches the segment's end state damped by the
    // decays of the chunks before it, so the common kernel takes it for the
    // segment's first chunk (its last step) only, the two-part kernel on every
    // step.  Per-channel gate: every step, since its dS also leaves in two parts
    // for the gate-parameter gradients, whose sums cancel strongly.
    auto qlo_step = [&](int k) { return TWO || Cf::SPLIT || k == nck - 1; };
    // raw mode: the compute waves form fq dO (high and, where it is taken, low) of
    // each chunk's dO slice one step ahead, a quarter each (chunk 0 here, chunk
    // k + 1 in the first window of step k; published by the next barrier)
    if constexpr (Cf::RAW)
      if (nck > 0) convert_raw_rows<D, TIO, GATE, NSL>(slot(0), sv, X2_of(0), X3_of(0), w, qlo_step(0));
    for (int k = 0; k < nck; ++k) {
      const int buf = k & 1;
      const char* Bb = smem + buf * Cf::bufB;
      const char* sl_k = slot(k);
      const char* X1 = Cf::LO ? smem + Cf::bX1 + buf * Cf::XB : sl_k + Cf::sDO + sv * Cf::XB;
      const char* X2 = X2_of(buf);
      const char* X3 = X3_of(buf);
      char* dUt = dUbuf(sv, k);
      char* dUlo = dUt + (Cf::bdUl - Cf::bdU);
      // a weakly decaying chunk: two-part operands (uniform over the workgroup)
      const bool two = TWO && chunk(k) <= two_last;
#pragma unroll
      for (int x = 0; x < NJW; ++x) {
        const int jc = 16 * (w * NJW + x), j = jc + 4 * g;
        st4_q<D>(dSl, 0, jc, acc[x][0], acc[x][1], acc[x][2], acc[x][3]);
        if (TWO && two)
          st4_q<D>(dSlo, 0, jc, lo_part(acc[x][0]), lo_part(acc[x][1]), lo_part(acc[x][2]), lo_part(acc[x][3]));
        if (Cf::SPLIT && job.store)   // no LDS left for a low tile: stored directly
          st_bf16x4(p.dSlo + (int64_t(h) * p.NC + chunk(k)) * D * D + (v0 + 16 * sv + jj) * D + j, lo_part(acc[x][0]),
                    lo_part(acc[x][1]), lo_part(acc[x][2]), lo_part(acc[x][3]));
      }
      chain_barrier();   // B1
      // raw mode: fq dO (high, low) of the next chunk first, so that its LDS round
      // trip overlaps the fragment reads below
      if constexpr (Cf::RAW)
        convert_raw_rows<D, TIO, GATE, NSL>(slot(k + 1), sv, X2_of(buf ^ 1), X3_of(buf ^ 1), w, qlo_step(k + 1));
      // dU = P^T dO + Khat dS^T, rows 16w.., columns of this slice
      f32x4 ad = zero4(), ak = zero4();
      if (!job.xfer) {   // transfer rows: dO = 0
#pragma unroll
        for (int k0 = 0; k0 < C; k0 += 32) {
          const bf16x8 pa = frag_kc_s<C>(Bb + Cf::bP, 16 * w, k0);
          ad = mma(pa, frag_kc_s<16>(X1, 0, k0), ad);
          if constexpr (Cf::LO) ad = mma(pa, frag_kc_s<16>(X2, 0, k0), ad);
        }
      }
      if (TWO && two) {
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += 32) {
          const bf16x8 kf = frag_rk_s<D>(Bb + Cf::bK, 16 * w, k0);
          const bf16x8 sh = frag_rk_s<D>(dSl, 0, k0);
          ak = mma(kf, sh, ak);
          ak = mma(kf, frag_rk_s<D>(dSlo, 0, k0), ak);
          if constexpr (Cf::TWOM) ak = mma(frag_rk_s<D>(Bb + Cf::bKl, 16 * w, k0), sh, ak);
        }
      } else {
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += 32)
          ak = mma(frag_rk_s<D>(Bb + Cf::bK, 16 * w, k0), frag_rk_s<D>(dSl, 0, k0), ak);
      }
      if constexpr (Cf::RAW) {
        const float4 f = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(sl_k + Cf::sFac) + C +
                                                          16 * w + 4 * g);
        ad += ak * f32x4{f.x, f.y, f.z, f.w};
      } else {
        ad += ak;
      }
      st4_q<C, 1>(dUt, 0, 16 * w, ad[0], ad[1], ad[2], ad[3]);
      if (TWO && two) st4_q<C, 1>(dUlo, 0, 16 * w, lo_part(ad[0]), lo_part(ad[1]), lo_part(ad[2]), lo_part(ad[3]));
      // dS_n^T = Diag(e^GamC) dS_{n+1}^T + Qbar^T dO - W^T dU: the first two terms do
      // not depend on dU and are issued before the barrier
      const float* dec = reinterpret_cast<const float*>(sl_k + Cf::sDec);
      f32x4 an[NJW];
      // the dO fragments (B operands: raw mode fq dO high, low; else dO high and,
      // for fp32 inputs, low) serve every x: read once
      constexpr int NK = C / 32;
      const char* XH = Cf::RAW ? X2 : X1;
      const char* XL = Cf::RAW ? X3 : X2;
      const bool qlo = qlo_step(k);
      bf16x8 xh[NK], xl[NK];
      if (!job.xfer) {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          xh[kk] = frag_kc_s<16>(XH, 0, 32 * kk);
          if constexpr (Cf::LO) xl[kk] = frag_kc_s<16>(XL, 0, 32 * kk);
          if constexpr (Cf::RAW)
            if (qlo) xl[kk] = frag_kc_s<16>(XL, 0, 32 * kk);
        }
      }
#pragma unroll
      for (int x = 0; x < NJW; ++x) {
        const int jb = w * NJW + x;
        f32x4 a = acc[x] * decay4<D, GATE>(dec, jb, g);
        if (!job.xfer) {   // transfer rows: dO = 0
#pragma unroll
          for (int kk = 0; kk < NK; ++kk) {
            const bf16x8 qa = frag_kc_s<D>(Bb + Cf::bQh, 16 * jb, 32 * kk);
            a = mma(qa, xh[kk], a);
            if constexpr (Cf::RAW) {
              if (qlo) a = mma(qa, xl[kk], a);
            } else {
              if (qlo) a = mma(frag_kc_s<D>(Bb + Cf::bQl, 16 * jb, 32 * kk), xh[kk], a);
              if constexpr (Cf::LO) a = mma(qa, xl[kk], a);
            }
          }
        }
        an[x] = a;
      }
      chain_barrier();   // B2
      if constexpr (Cf::RAW) {
        // W^T dU = k^T Y with Y = Diag(fw) A^T dU (W = A Diag(fw) k).  Every wave
        // forms all 64 rows of Y (A is block lower triangular: row block rb takes
        // dU rows from 16 rb on) and feeds its accumulators, rounded to bf16,
        // straight back as the B operand of k^T Y, K-step kk pairing the row
        // blocks 2kk and 2kk+1 (frag_kc_split_s reads k^T in that row order)
        const bf16x8 du0 = frag_rk_s<C, 1>(dUt, 0, 0), du1 = frag_rk_s<C, 1>(dUt, 0, 32);
        // fw of this lane's Y rows 16 rb + 4g .. +3 and the k^T fragments, read in
        // the same round trip as dU
        const float* fw = reinterpret_cast<const float*>(sl_k + Cf::sFac) + 2 * C;
        f32x4 fwv[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const float4 f = *reinterpret_cast<const float4*>(fw + 16 * rb + 4 * g);
          fwv[rb] = f32x4{f.x, f.y, f.z, f.w};
        }
        f32x4 y[4];
        bf16x8 yb[2];
        if (TWO && two) {
          // (the rare path: fragments read where they are used, to keep the
          // registers of the common path's schedule free)
          const bf16x8 dl0 = frag_rk_s<C, 1>(dUlo, 0, 0), dl1 = frag_rk_s<C, 1>(dUlo, 0, 32);
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) {
            y[rb] = zero4();
            if (rb < 2) {
              const bf16x8 a0 = frag_kc_s<C>(Bb + Cf::bA, 16 * rb, 0);
              y[rb] = mma(a0, du0, y[rb]);
              y[rb] = mma(a0, dl0, y[rb]);
            }
            const bf16x8 a1 = frag_kc_s<C>(Bb + Cf::bA, 16 * rb, 32);
            y[rb] = mma(a1, du1, y[rb]);
            y[rb] = mma(a1, dl1, y[rb]);
            y[rb] *= fwv[rb];
          }
          bf16x8 yl[2];
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              yb[kk][i] = to_bf16(y[2 * kk][i]);
              yb[kk][4 + i] = to_bf16(y[2 * kk + 1][i]);
              yl[kk][i] = to_bf16(lo_part(y[2 * kk][i]));
              yl[kk][4 + i] = to_bf16(lo_part(y[2 * kk + 1][i]));
            }
#pragma unroll
          for (int x = 0; x < NJW; ++x) {
            f32x4 aw = zero4();
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
              const bf16x8 kf = frag_kc_split_s<D>(Bb + Cf::bK, 16 * (w * NJW + x), 32 * kk);
              aw = mma(kf, yb[kk], aw);
              aw = mma(kf, yl[kk], aw);
            }
            acc[x] = an[x] - aw;
          }
        } else {
          bf16x8 kfr[NJW][2];
#pragma unroll
          for (int x = 0; x < NJW; ++x)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) kfr[x][kk] = frag_kc_split_s<D>(Bb + Cf::bK, 16 * (w * NJW + x), 32 * kk);
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) {
            y[rb] = zero4();
            if (rb < 2) y[rb] = mma(frag_kc_s<C>(Bb + Cf::bA, 16 * rb, 0), du0, y[rb]);
            y[rb] = mma(frag_kc_s<C>(Bb + Cf::bA, 16 * rb, 32), du1, y[rb]);
            y[rb] *= fwv[rb];
          }
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              yb[kk][i] = to_bf16(y[2 * kk][i]);
              yb[kk][4 + i] = to_bf16(y[2 * kk + 1][i]);
            }
#pragma unroll
          for (int x = 0; x < NJW; ++x) {
            f32x4 aw = zero4();
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) aw = mma(kfr[x][kk], yb[kk], aw);
            acc[x] = an[x] - aw;
          }
        }
      } else {
#pragma unroll
        for (int x = 0; x < NJW; ++x) {
          const int jb = w * NJW + x;
          f32x4 aw = zero4();
#pragma unroll
          for (int k0 = 0; k0 < C; k0 += 32) {
            const bf16x8 wf = frag_kc_s<D>(Bb + Cf::bW, 16 * jb, k0);
            const bf16x8 uh = frag_rk_s<C, 1>(dUt, 0, k0);
            aw = mma(wf, uh, aw);
            if (TWO && two) {
              aw = mma(wf, frag_rk_s<C, 1>(dUlo, 0, k0), aw);
              if constexpr (Cf::TWOM) aw = mma(frag_kc_s<D>(Bb + Cf::bWl, 16 * jb, k0), uh, aw);
            }
          }
          acc[x] = an[x] - aw;
        }
      }
    }
    job_fin<D>(job, acc, w, g, jj);
  } else if (wv == Cf::CONV) {
    if (nck == 0) return;
    LoRegs<D, TIO, GATE> R;
    const bool store = jobs[0].store;
    if constexpr (Cf::LO) {
      R.load(p, se, h, chunk(0), v0l, true);
      R.store_dO(smem + Cf::bX1, smem + Cf::bX2);
      R.store_dec(reinterpret_cast<float*>(slot(0) + Cf::sDec));
      R.load(p, se, h, chunk(1), v0l, true);
    }
    chain_barrier();   // B0
    for (int k = 0; k < nck; ++k) {
      const int64_t ch = int64_t(h) * p.NC + chunk(k);
      const int nb = (k + 1) & 1;
      chain_barrier();   // B1
      if (store) {
#pragma unroll
        for (int sv = 0; sv < NSL; ++sv) {
          store_slice<D>(dS_of(sv), p.dS + (ch * D + v0 + 16 * sv) * D);
          // two dU buffers: dU of the previous step (its buffer is not written again
          // before the next B2); one buffer: this step's, after B2
          if (Cf::NDU == 2 && k > 0)
            store_slice<C, 1>(dUbuf(sv, k - 1), p.dU + ((int64_t(h) * p.NC + chunk(k - 1)) * D + v0 + 16 * sv) * C);
        }
      }
      chain_barrier();   // B2
      if (Cf::NDU == 1 && store) {
#pragma unroll
        for (int sv = 0; sv < NSL; ++sv) store_slice<C, 1>(dUbuf(sv, k), p.dU + (ch * D + v0 + 16 * sv) * C);
      }
      if constexpr (Cf::LO) {
        R.store_dO(smem + Cf::bX1 + nb * Cf::XB, smem + Cf::bX2 + nb * Cf::XB);
        R.store_dec(reinterpret_cast<float*>(slot(k + 1) + Cf::sDec));
        R.load(p, se, h, chunk(k + 2), v0l, true);
      }
    }
    if (Cf::NDU == 2 && store) {
#pragma unroll
      for (int sv = 0; sv < NSL; ++sv)
        store_slice<C, 1>(dUbuf(sv, nck - 1), p.dU + ((int64_t(h) * p.NC + chunk(nck - 1)) * D + v0 + 16 * sv) * C);
    }
    wait_vm<0>();
  } else {
    if (nck == 0) return;
    constexpr int NPF = Cf::NPF;
    constexpr int BA = TWO ? Cf::bwdA2 : Cf::bwdA, BB = TWO ? Cf::bwdB2 : Cf::bwdB;
    const int mw = wv - Cf::MOVE0;
    const bool hs = small_loads<D, TIO, GATE, NSL>(mw, true);
    MoverLane<D> ml;
    ml.template init<NSL>(p, h, mw, l, int(sizeof(TIO)));
    // the rows of the state slices whose dO this workgroup loads, one prefetch a slice
    PfLane<D, TIO, GATE, true> pf[NSL];
#pragma unroll
    for (int i = 0; i < NSL; ++i) pf[i].init(p, v0l / 16 + i, mw, l);
    auto prefetch = [&](int c) {
#pragma unroll
      for (int i = 0; i < NSL; ++i) prefetch_chunk<D, TIO, GATE, true>(pf[i], ml, p, se, h, c, smem + Cf::bPF);
    };
    move_small<D, TIO, GATE, NSL>(ml, p, se, h, chunk(0), v0l, slot(0), mw, true);
    move_bwd_a<D, TIO, GATE, TWO>(ml, p, se, h, chunk(0), smem, mw);
    move_bwd_b<D, TIO, GATE, TWO>(ml, p, se, h, chunk(0), smem, mw);
    move_small<D, TIO, GATE, NSL>(ml, p, se, h, chunk(1), v0l, slot(1), mw, true);
    move_bwd_a<D, TIO, GATE, TWO>(ml, p, se, h, chunk(1), smem + Cf::bufB, mw);
    for (int c = 2; c < Cf::PFD; ++c) prefetch(chunk(c));
    wait_mover<BA + BB + BA + (Cf::PFD - 2) * NPF>(hs);
    chain_barrier();   // B0
    // both sets of chunk 0 and the small data of chunk 1 land before B1 (set B is
    // read in the first window too, and so is the next chunk's small data)
    wait_vm<BA + (Cf::PFD - 2) * NPF>();
    for (int k = 0; k < nck; ++k) {
      chain_barrier();   // B1
      move_bwd_b<D, TIO, GATE, TWO>(ml, p, se, h, chunk(k + 1), smem + ((k + 1) & 1) * Cf::bufB, mw);
      move_small<D, TIO, GATE, NSL>(ml, p, se, h, chunk(k + 2), v0l, slot(k + 2), mw, true);
      wait_mover<BA + NPF + BB>(hs);
      chain_barrier();   // B2
      move_bwd_a<D, TIO, GATE, TWO>(ml, p, se, h, chunk(k + 2), smem + (k & 1) * Cf::bufB, mw);
      prefetch(chunk(k + Cf::PFD));
      // set B of chunk k + 1 and the small data of chunk k + 2 land before the
      // next B1: only set A of chunk k + 2 and the prefetch stay in flight
      wait_vm<BA + NPF>();
    }
    wait_vm<0>();
  }
}

// Scalar gate, reverse role: a step's rounding reaches the segment's end state
// (dh0 for a sequence's first segment) damped by the decays of the chunks before
// it, so the steps that take two-part operands are those of the chunks whose
// decay from the segment's start, e^(sum of GamC up to and including the chunk),
// is at least kTwoPartDecay: the segment's first chunks (GamC <= 0).  Returns the
// global index of the last of them, or -1.  Every wave scans the chunk decays
// itself (a wave-wide prefix sum of their logarithms): a uniform answer with no
// barrier.
__device__ __forceinline__ int two_part_last(const Params& p, const SeqEntry& se, int h) {
  const int l = lane_id();
  const float thr = logf(kTwoPartDecay);
  float carry = 0.f;
  int last = -1;
  for (int b = 0; b < se.nchunks; b += 64) {
    const int i = b + l;
    const float e = i < se.nchunks ? p.edec[(int64_t(h) * p.NC + se.c0 + i) * 4] : 0.f;
    float x = e > 0.f ? logf(e) : -INFINITY;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(x, o, 64);
      if (l >= o) x += y;
    }
    x += carry;
    const uint64_t m = __ballot(x >= thr);
    if (m) last = se.c0 + b + 63 - __clzll(m);
    carry = __shfl(x, 63, 64);
    if (!(carry >= thr)) break;   // the sums only decrease from here
  }
  return __builtin_amdgcn_readfirstlane(last);
}

// Per-channel gate, forward role: whether segment se has a weak chunk before its
// last one (the last step's rounding reaches only the end state, through one
// step: it does not accumulate).  Every wave reads the prologue's flags itself.
__device__ __forceinline__ bool weak_segment(const Params& p, const SeqEntry& se, int h) {
  int f = 0;
  for (int i = lane_id(); i < se.nchunks - 1; i += 64) f |= p.weak[int64_t(h) * p.NC + se.c0 + i];
  return __any(f);
}

// blockIdx -> (one (segment, head), slice): the slices of one (segment, head)
// share its chunk tiles, so they are placed on the same XCD (workgroups are
// dealt round-robin over the 8 XCDs).  The final pass has D / 16 slices per
// (segment, head), the state rows; the local pass twice that many, the state
// rows and then the transfer-product rows; a workgroup takes NSL consecutive slices.
// TWO (Cf::LOWB): the reverse role of the segments two_part_last() picks (the
// common kernel leaves them out).  The per-channel gate's forward role takes its
// two-part form in the common kernel, for the segments weak_segment() picks.
template <int D, typename TIO, int GATE, int NSL, bool TWO = false>
__global__ __launch_bounds__((ChainCfg<D, TIO, GATE, NSL>::THREADS)) void k_chain(const Params p, int mode, int nb_role,
                                                                                  int pass) {
  using Cf = ChainCfg<D, TIO, GATE, NSL>;
  static_assert(!TWO || Cf::LOWB, "a kernel of two-part steps: where the LDS holds the low parts");
  __shared__ __attribute__((aligned(1024))) char smem[ChainCfg<D, TIO, GATE, NSL>::bytes];
  int b = blockIdx.x;
  int role;
  if (mode == kChainBoth) {
    role = b < nb_role ? 0 : 1;
    if (role) b -= nb_role;
  } else {
    role = mode == kChainFwd ? 0 : 1;
  }
  constexpr int ns = D / 16;
  const int nsl = pass == kPassLocal ? 2 * ns : ns;
  const int nsg = nsl / NSL;   // slice groups per (segment, head)
  const int xcd = b % 8, y = b / 8;
  const int sl = (y % nsg) * NSL, t = y / nsg;   // sl: the group's first slice
  // (segment, head) of slot t on this XCD.  With grouped heads the G value heads
  // of a key head read the same q, k rows, so they take consecutive slots of one
  // XCD (its L2 then serves the rows they share); the (segment, key head) pairs
  // past the last whole set of eight keep the plain order.
  int gidx;
  if (p.G == 1) {
    gidx = t * 8 + xcd;
  } else {
    const int npair = p.NS * p.Hk, p8 = npair / 8 * 8;
    const int L = t * 8 + xcd;
    int pair, gi;
    if (L < p8 * p.G) {
      pair = (t / p.G) * 8 + xcd;
      gi = t % p.G;
    } else {
      const int rem = L - p8 * p.G;
      pair = p8 + rem / p.G;
      gi = rem % p.G;
    }
    gidx = (pair / p.Hk) * p.H + (pair % p.Hk) * p.G + gi;
  }
  if (gidx >= p.NS * p.H) return;
  const int si = gidx / p.H, h = gidx % p.H;
  const SeqEntry se = seq_entry(p, si);
  const bool first = role == 0 ? se.seg == 0 : se.seg == se.nseg - 1;   // the role's first segment
  const bool last = role == 0 ? se.seg == se.nseg - 1 : se.seg == 0;    // the role's last segment
  const int64_t sh = int64_t(se.seq) * p.H + h;                           // (sequence, head)
  const int64_t gh = (int64_t(role) * p.NS + se.slot) * p.H + h;           // (role, segment slot, head)
  const float* start = role == 0 ? p.h0 : p.dht;
  float* end = role == 0 ? p.ht : p.dh0;
  // the slices of a group lie on one side of ns (ns is even): all state rows or
  // all transfer rows
  const bool xfer = sl >= ns;
  // only segments that a later one (in the role's order) starts from, and the
  // transfer product only where the segment does not start from h0 / dht
  if (pass == kPassLocal && (last || (xfer && first))) return;
  int two_last = -1;   // reverse role: the last chunk of two-part steps
  if constexpr (Cf::LOWB) {
    if (role == 1) {
      two_last = two_part_last(p, se, h);
      if ((two_last >= 0) != TWO) return;
    }
  }
  ChainJob jobs[NSL];
#pragma unroll
  for (int i = 0; i < NSL; ++i) {
    const int sx = sl + i;
    ChainJob& job = jobs[i];
    job.xfer = xfer;
    job.i0 = 16 * (sx - ns);
    job.v0l = 16 * (sx % ns);
    if (pass == kPassLocal) {
      job.init = first && !xfer && start ? start + (sh * D + 16 * sx) * D : nullptr;
      job.fin = p.xf + (gh * 2 * D + 16 * sx) * D;
      job.store = false;
    } else {
      job.init = first ? (start ? start + (sh * D + 16 * sx) * D : nullptr) : p.sb + (gh * D + 16 * sx) * D;
      job.fin = last && end ? end + (sh * D + 16 * sx) * D : nullptr;
      job.store = true;
    }
  }
  if constexpr (TWO) {
    chain_bwd<D, TIO, GATE, NSL, true>(p, smem, si, h, sl, jobs, two_last);
  } else {
    if (role == 0) {
      if (Cf::SPLIT && weak_segment(p, se, h))
        chain_fwd<D, TIO, GATE, NSL, Cf::SPLIT>(p, smem, si, h, sl, jobs);
      else
        chain_fwd<D, TIO, GATE, NSL>(p, smem, si, h, sl, jobs);
    } else {
      chain_bwd<D, TIO, GATE, NSL, false>(p, smem, si, h, sl, jobs, -1);
    }
  }
}

// The boundary states of split sequences, in order: one workgroup per (first
// segment of a split sequence, head, 16 state rows, role).  Forward: segment 1
// starts from the local pass's end state of segment 0 (run from h0), and
// segment j + 1 from S_j T_j + E_j (T_j the transfer product of segment j, E_j its
// end state from zero); reverse likewise from the last segment down.  Each row of
// the state composes on its own, so a workgroup carries its 16 rows through all
// the boundaries.  The products run on 16x16x4 fp32 MFMA: wave w owns columns
// [w D/4, (w + 1) D/4), the state rows (the A operand) come from LDS, and T_j
// (the B operand) goes straight from global memory into registers, the next
// boundary's while this one computes.  Over the MFMA's four k lanes the sum
// index is taken as k = g (D/4) + kk at step kk, so each lane reads a contiguous
// run of its state row.
template <int D>
__global__ __launch_bounds__(256) void k_chain_fix(const Params p, int mode) {
  constexpr int KK = D / 4;        // MFMA steps over the sum index
  constexpr int NT = D / 64;       // 16-column tiles per wave
  constexpr int PIT = D + 4;       // LDS row pitch (floats)
  constexpr int ns = D / 16, CPT = D / 16;
  __shared__ __align__(16) float cur[16 * PIT];
  int b = blockIdx.x;
  const int per_role = p.NS * p.H * ns;
  int role = mode == kChainBwd ? 1 : 0;
  if (mode == kChainBoth && b >= per_role) {
    role = 1;
    b -= per_role;
  }
  const int sl = b % ns, gidx = b / ns;
  const int si = gidx / p.H, h = gidx % p.H;
  const SeqEntry se = seq_entry(p, si);
  if (se.seg != 0 || se.nseg < 2) return;
  const int tid = threadIdx.x, r = tid >> 4, c0 = (tid & 15) * CPT;
  const int l = lane_id(), q = l & 15, g = l >> 4, n0 = wave_id() * (D / 4);
  auto xf = [&](int slot) { return p.xf + ((int64_t(role) * p.NS + slot) * p.H + h) * 2 * D * D; };
  auto sbuf = [&](int slot) { return p.sb + (((int64_t(role) * p.NS + slot) * p.H + h) * D + 16 * sl) * D; };
  const int P = se.nseg, s0 = se.slot;
  // the role's first segment ran from h0 / dht: its end state is already true
  const int j0 = role == 0 ? 0 : P - 1;
  const int step = role == 0 ? 1 : -1;
  const int jlast = j0 + step * (P - 1);
  {
    const float* e0 = xf(s0 + j0) + (16 * sl + r) * D + c0;
#pragma unroll
    for (int i = 0; i < CPT; ++i) cur[r * PIT + c0 + i] = e0[i];
  }
  // B operand of boundary j: T_j[g KK + kk][n0 + 16 n + q]; the accumulators
  // start from E_j at the MFMA output positions (rows 4 g + v, column n0 + 16 n + q)
  auto load_t = [&](float (&bt)[NT][KK], float (&e)[NT][4], int j) {
    const float* T = xf(s0 + j) + D * D + (g * KK) * D + n0 + q;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int n = 0; n < NT; ++n) bt[n][kk] = T[kk * D + 16 * n];
    const float* E = xf(s0 + j) + (16 * sl + 4 * g) * D + n0 + q;
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int v = 0; v < 4; ++v) e[n][v] = E[v * D + 16 * n];
  };
  // one boundary: cur holds the state segment s0 + j starts from
  auto compose = [&](const float (&bt)[NT][KK], const float (&e)[NT][4], int j) {
    float* dst = sbuf(s0 + j) + r * D + c0;
#pragma unroll
    for (int i = 0; i < CPT; ++i) dst[i] = cur[r * PIT + c0 + i];
    float a[KK];
#pragma unroll
    for (int i = 0; i < KK; i += 4) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(&cur[q * PIT + g * KK + i]);
      a[i] = t[0];
      a[i + 1] = t[1];
      a[i + 2] = t[2];
      a[i + 3] = t[3];
    }
    f32x4 acc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = f32x4{e[n][0], e[n][1], e[n][2], e[n][3]};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n] = mma_f32(a[kk], bt[n][kk], acc[n]);
    chain_barrier();   // every read of cur is done (the next T_j stays in flight)
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int v = 0; v < 4; ++v) cur[(4 * g + v) * PIT + n0 + 16 * n + q] = acc[n][v];
    chain_barrier();
  };
  float bt0[NT][KK], bt1[NT][KK], e0[NT][4], e1[NT][4];
  int j = j0 + step;
  if (j != jlast) load_t(bt0, e0, j);
  __syncthreads();
  while (j != jlast) {
    if (j + step != jlast) load_t(bt1, e1, j + step);
    compose(bt0, e0, j);
    j += step;
    if (j == jlast) break;
    if (j + step != jlast) load_t(bt0, e0, j + step);
    compose(bt1, e1, j);
    j += step;
  }
  // the state of the role's last segment
  float* dst = sbuf(s0 + jlast) + r * D + c0;
#pragma unroll
  for (int i = 0; i < CPT; ++i) dst[i] = cur[r * PIT + c0 + i];
}

namespace {
template <int D, typename TIO, int GATE, int NSL, bool TWO = false>
void launch_nsl(const Params& p, int mode, int pass, hipStream_t s) {
  constexpr int ns = D / 16;
  const int nsl = pass == kPassLocal ? 2 * ns : ns;
  const int groups = p.NS * p.H;
  const int nb = ((groups + 7) / 8) * 8 * (nsl / NSL);
  const int nroles = mode == kChainBoth ? 2 : 1;
  k_chain<D, TIO, GATE, NSL, TWO><<<dim3(nb * nroles), ChainCfg<D, TIO, GATE, NSL>::THREADS, 0, s>>>(p, mode, nb, pass);
}

// One slice a workgroup while every workgroup gets a CU of its own (one fits per
// CU); beyond that, in raw mode, two slices a workgroup: they share the chunk
// tiles (one set of loads for two slices), so the grid stays in one round
// instead of two.
template <int D, typename TIO, int GATE>
void run_chain(const Params& p, int mode, int pass, hipStream_t s) {
  constexpr int ns = D / 16;
  const int nsl = pass == kPassLocal ? 2 * ns : ns;
  const int64_t nb1 = int64_t((p.NS * p.H + 7) / 8) * 8 * nsl * (mode == kChainBoth ? 2 : 1);
  if constexpr (ChainCfg<D, TIO, GATE>::RAW) {
    if (nb1 > kGpuCUs)
      launch_nsl<D, TIO, GATE, 2>(p, mode, pass, s);
    else
      launch_nsl<D, TIO, GATE, 1>(p, mode, pass, s);
    // the reverse role of the segments with weakly decaying chunks (their
    // workgroups in the launch above return at once, as do the others here)
    if (mode != kChainFwd) launch_nsl<D, TIO, GATE, 1, true>(p, kChainBwd, pass, s);
    return;
  }
  launch_nsl<D, TIO, GATE, 1>(p, mode, pass, s);
  if constexpr (ChainCfg<D, TIO, GATE>::TWOM)
    if (mode != kChainFwd) launch_nsl<D, TIO, GATE, 1, true>(p, kChainBwd, pass, s);
}
}  // namespace

int launch_chain(const Params& p, int mode, int pass, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (pass == kPassLocal && (!p.xf || !p.sb)) return static_cast<int>(hipErrorInvalidValue);
  const bool bf = p.dtype == GDR_BF16;
  if (p.K == 128 && bf && p.gate == 0) run_chain<128, bf16, 0>(p, mode, pass, s);
  else if (p.K == 128 && bf && p.gate == 1) run_chain<128, bf16, 1>(p, mode, pass, s);
  else if (p.K == 128 && !bf && p.gate == 0) run_chain<128, float, 0>(p, mode, pass, s);
  else if (p.K == 128 && !bf && p.gate == 1) run_chain<128, float, 1>(p, mode, pass, s);
  else if (p.K == 64 && bf && p.gate == 0) run_chain<64, bf16, 0>(p, mode, pass, s);
  else if (p.K == 64 && bf && p.gate == 1) run_chain<64, bf16, 1>(p, mode, pass, s);
  else if (p.K == 64 && !bf && p.gate == 0) run_chain<64, float, 0>(p, mode, pass, s);
  else if (p.K == 64 && !bf && p.gate == 1) run_chain<64, float, 1>(p, mode, pass, s);
  else return static_cast<int>(hipErrorInvalidValue);
  return static_cast<int>(hipGetLastError());
}

int launch_chain_fix(const Params& p, int mode, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (!p.xf || !p.sb) return static_cast<int>(hipErrorInvalidValue);
  const int nroles = mode == kChainBoth ? 2 : 1;
  const int per_role = p.NS * p.H * (p.K / 16);
  if (per_role == 0) return 0;
  if (p.K == 128) k_chain_fix<128><<<dim3(per_role * nroles), 256, 0, s>>>(p, mode);
  else if (p.K == 64) k_chain_fix<64><<<dim3(per_role * nroles), 256, 0, s>>>(p, mode);
  else return static_cast<int>(hipErrorInvalidValue);
  return static_cast<int>(hipGetLastError());
}

}  // namespace gdr

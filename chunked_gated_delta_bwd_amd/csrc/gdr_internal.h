// Internal declarations shared by the host API (gdr_api.cpp) and the kernels
// (gdr_kernels.hip): workspace layout, the chunk/sequence tables and the
// parameter block every kernel receives by value.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/gdr.h"

namespace gdr {

constexpr int kChunk = 64;     // tokens per chunk
// A recursion step's bf16 rounding error is proportional to the chunk's decay
// e^GamC, and with little decay the following steps do not damp it.  Steps whose
// error is damped by less than this take some operands in two bf16 parts (x = hi
// + lo): the scalar gate's reverse steps dS, dU and Y where the decay from the
// segment's start to the chunk's end is at least this, the per-channel gate's
// forward steps Khat where some channel's e^GamC is (a "weak" chunk).
constexpr float kTwoPartDecay = 1.f / 16;
// With fp32 inputs the scalar gate's recursions take Khat and W as materialised
// bf16 tiles, whose rounding weighs as much as that of dS and dU there.  At this
// head size the reverse recursion's two-part steps take them in two parts too,
// from low tiles the prologue writes (at 128-wide heads the recursion's LDS has
// no room for them).
constexpr int kMatTwoPartK = 64;
constexpr int kThreads = 256;  // threads per workgroup in every kernel (4 wave64s)

// One row per chunk (global chunk index c).
struct ChunkEntry {
  int32_t t_start;   // first token (packed token axis)
  int32_t len;       // valid rows, 1..64
  int32_t seq;       // sequence index
  int32_t idx;       // chunk index inside its sequence
};

// One row per segment of a sequence: the recursions run over segments, each a
// run of whole chunks of one sequence (a sequence that is not split is one
// segment).  The recursion kernel's table is ordered longest first so that the
// longest chains start first.
// MI355X compute units; one recursion workgroup fits per CU
constexpr int kGpuCUs = 256;

struct SeqEntry {
  int32_t seq;       // sequence index (addresses h0/dht/dh0/ht)
  int32_t len;       // tokens
  int32_t c0;        // global index of its first chunk
  int32_t nchunks;   // ceil(len / 64)
  int32_t t_start;   // first token (packed token axis)
  int32_t seg;       // segment index inside the sequence, 0 .. nseg - 1
  int32_t nseg;      // segments of the sequence
  int32_t slot;      // boundary-state slot: the sequence's segments take nseg consecutive slots
};

// Table entries handed to k_tables by value, kTableBatch per launch.
//   kind 0 (dense): `n` dense sequences of dense_T tokens numbered from `first`,
//                   each split into nseg equal runs of chunks; writes chunk and
//                   segment rows; `e` is not read
//   kind 1:         `n` whole sequences in e[]: writes their chunk rows
//   kind 2:         `n` segments in e[]: writes segment-table rows first .. first + n - 1
constexpr int kTableBatch = 56;
struct TableBatch {
  int32_t n;
  int32_t first;
  int32_t kind;
  int32_t dense_T;
  int32_t nseg;
  int32_t pad[3];
  SeqEntry e[kTableBatch];
};
static_assert(sizeof(TableBatch) <= 2048, "kernel argument size");

// Segments per sequence chosen by the host for a shape (the same choice sizes
// the workspace and builds the tables).
constexpr int kMaxSegments = 16;

// Byte offsets of every workspace region (all 256-byte aligned).
struct WsLayout {
  int64_t NC = 0;    // total chunks
  int64_t NS = 0;    // segments (rows of the segment table)
  int32_t split = 0; // 1 when some sequence is split into several segments
  size_t ctab = 0, stab = 0;
  size_t gam = 0;    // fp32 [H][NC][64] or [H][NC][64][K]: in-chunk cumsum of the log decay
  size_t rho = 0;    // fp32 [H][NC][3][64]: 1/|q|, 1/|k|, beta per row (beta 0 past the end)
  size_t fac = 0;    // fp32 [H][NC][3][64]: scalar gate row factors of the recursions,
                     //   fq = scale e^Gam / |q|, fk = e^(GamC - Gam) / |k|,
                     //   fw = beta e^Gam / |k| (W = A Diag(fw) k; all zero past the end)
  size_t edec = 0;   // fp32 [H][NC][4] (value, 3 pad) or [H][NC][K]: chunk decay e^GamC
  size_t A = 0;      // bf16 [H][NC][64][64]: UT/WY inverse
  size_t P = 0;      // bf16 [H][NC][64][64]: scale * (Qn Kn^T o E), lower incl. diagonal
  size_t W = 0;      // bf16 [H][NC][64][K]:  A diag(beta) Kbar (materialised tiles only)
  size_t Up = 0;     // bf16 [H][NC][64][V]:  U' = A diag(beta) V
  size_t U = 0;      // bf16 [H][NC][V][64]:  v_new = U' - W S^T (forward state pass), transposed
  size_t S = 0;      // bf16 [H][NC][V][K]:   state at chunk start
  size_t dS = 0;     // bf16 [H][NC][V][K]:   gradient w.r.t. the state at chunk end
  size_t dU = 0;     // bf16 [H][NC][V][64]:  gradient w.r.t. v_new, transposed
  // per-channel gate or fp32 inputs: the recursions' operand tiles formed by the
  // prologue (the scalar gate with bf16 inputs applies row factors instead)
  size_t Kh = 0;     // bf16 [H][NC][64][K]: Khat = kn e^(GamC - Gam)
  size_t Qh = 0;     // bf16 [H][NC][64][K]: Qbar = scale qn e^Gam, high part
  size_t Ql = 0;     // bf16 [H][NC][64][K]: Qbar low part
  // per-channel gate only
  size_t Mk = 0;     // bf16 [H][NC][64][64]: M = Kn Kn^T weighted by the per-channel decay
  size_t pdA = 0;    // fp32 [H][NC]:    per-chunk partial sums of dA_log
  size_t pddt = 0;   // fp32 [H][NC][K]: per-chunk partial sums of ddt_bias
  // per-channel gate only: low bf16 parts (x = hi + lo) of U', U, S and dS, for
  // the gate gradient, whose per-head sums cancel strongly
  size_t Uplo = 0;   // bf16 [H][NC][64][V]
  size_t Ulo = 0;    // bf16 [H][NC][V][64]
  size_t Slo = 0;    // bf16 [H][NC][V][K]
  size_t dSlo = 0;   // bf16 [H][NC][V][K]
  size_t Khl = 0;    // bf16 [H][NC][64][K]: Khat's low part (per-channel gate: weak chunks only;
                     //   fp32 inputs, scalar gate, K = kMatTwoPartK: every chunk)
  size_t Wl = 0;     // bf16 [H][NC][64][K]: W's low part (fp32 inputs, scalar gate, K = kMatTwoPartK)
  size_t weak = 0;   // int32 [H][NC]: 1 for a weak chunk (see kTwoPartDecay)
  // split sequences only: the first recursion pass's segment-end states and
  // transfer products, and the composed segment boundary states
  size_t xf = 0;     // fp32 [2 roles][NS][H][2 D][D]: rows 0..D-1 end state from zero (or from
                     //   h0 / dht for the first segment of a role), rows D..2D-1 transfer product
  size_t sb = 0;     // fp32 [2 roles][NS][H][D][D]: the state a segment's recursion starts from
  // grouped heads only (Hk < H): dq, dk per value head before the group sum
  size_t dqv = 0;    // dtype [tokens][H][K]
  size_t dkv = 0;    // dtype [tokens][H][K]
  size_t total = 0;
};

struct Params {
  int32_t H, K, V, N, NC, T;     // T = total tokens
  int32_t NS;                     // rows of the segment table
  int32_t Hk, G;                  // q, k heads and value heads per key head (H = Hk G)
  int32_t gate, dtype;            // gate: 0 scalar, 1 per-channel (either gate function)
  float scale;
  int32_t gate_fn;                // per-channel: 0 -e^A_log softplus(x), 1 gate_scale sigmoid(e^A_log x)
  float gate_scale;
  // inputs
  const void *q, *k, *v, *g, *b, *dO;
  const float *A_log, *dt_bias, *h0, *dht;
  // outputs
  void *dq, *dk, *dv, *dg, *db;
  float *dh0, *dA_log, *ddt_bias, *ht;
  void* o;   // forward output (gdr_fwd only)
  // workspace
  const ChunkEntry* ctab;
  const SeqEntry* stab;
  float* gam;
  float* rho;
  float *fac, *edec;
  uint16_t *A, *P, *W, *Up, *U, *S, *dS, *dU;   // bf16 bit patterns
  uint16_t *Kh, *Qh, *Ql;                        // materialised operand tiles (see WsLayout)
  uint16_t* Mk;                                  // per-channel gate only
  float *pdA, *pddt;
  uint16_t *Uplo, *Ulo, *Slo, *dSlo;             // per-channel gate only: low parts
  uint16_t *Khl, *Wl;                            // low tiles of Khat and W (see WsLayout)
  int32_t* weak;                                 // per-channel gate only
  float *xf, *sb;                                // split sequences only
};

// Chain-kernel roles.
enum ChainMode { kChainFwd = 1, kChainBwd = 2, kChainBoth = 3 };
// Passes of the recursions over segments.  kPassFinal runs every segment from
// its true starting state (h0 / dht, or the composed boundary state) and stores
// the per-chunk outputs; a problem with no split sequence runs only this pass.
// kPassLocal runs every segment that some later (forward) or earlier (reverse)
// segment depends on, from zero (or h0 / dht), with the transfer product as D
// more state rows, and stores only the segment-end rows.
enum ChainPass { kPassFinal = 0, kPassLocal = 1 };

// Chunk and sequence tables from one batch of sequence entries (gdr_tables.hip).
int launch_tables(const ChunkEntry* ctab, const SeqEntry* stab, const TableBatch& tb, void* stream);
// Kernel launchers (gdr_kernels.hip).  Return a hipError_t as int.
int launch_prep(const Params& p, void* stream);
int launch_chain(const Params& p, int mode, int pass, void* stream);
// The serial composition of the segment boundary states from the local pass's
// segment-end states and transfer products (split sequences only).
int launch_chain_fix(const Params& p, int mode, void* stream);
int launch_grads(const Params& p, void* stream);
int launch_zero_params(const Params& p, void* stream);
// Forward output from the forward recompute's workspace (gdr_out.hip).
int launch_output(const Params& p, void* stream);
// Grouped heads (gdr_group.hip): dst[t][j][:] = sum over i < G of src[t][j G + i][:],
// for the T tokens, Hk key heads and K channels of p, in p.dtype.
int launch_group_sum(const Params& p, const void* src, void* dst, void* stream);
// Per-channel gate kernels (gdr_kda.hip): stage 0 prologue, 1 gradients with the
// prepare-backward, 2 dA_log / ddt_bias reduction.
int launch_kda(const Params& p, int stage, void* stream);
const char* hip_error_string(int err);
// Records the message gdr_last_error() returns to this thread and returns `st`
// (gdr_api.cpp).
gdr_status set_error(gdr_status st, const char* fmt, ...);

}  // namespace gdr

// Host side of the C ABI declared in include/gdr.h: argument validation,
// workspace layout, the chunk and sequence tables, and the launch sequence.
// Nothing here allocates or synchronises; everything is enqueued on the
// caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "gdr_internal.h"

namespace {

thread_local std::string g_last_error;

gdr_status fail(gdr_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validates the shape and computes the chunk count.
gdr_status check_shape(const gdr_shape* s, int64_t* NC_out) {
  if (!s) return fail(GDR_EINVAL, "shape is NULL");
  if (s->gate != GDR_GATE_SCALAR && s->gate != GDR_GATE_CHANNEL && s->gate != GDR_GATE_CHANNEL_SIGMOID)
    return fail(GDR_EINVAL, "unknown gate %d", s->gate);
  if (s->gate == GDR_GATE_CHANNEL_SIGMOID && !(s->gate_scale <= 0.f && s->gate_scale > -1e30f))
    return fail(GDR_EINVAL, "gate_scale %g must be finite and <= 0 (a log decay)", double(s->gate_scale));
  if (s->dtype != GDR_BF16 && s->dtype != GDR_F32) return fail(GDR_EINVAL, "unknown dtype %d", s->dtype);
  if (s->Dk != s->Dv) return fail(GDR_EUNSUPPORTED, "Dk (%d) != Dv (%d)", s->Dk, s->Dv);
  if (s->Dk != 64 && s->Dk != 128) return fail(GDR_EUNSUPPORTED, "head dim %d not in {64, 128}", s->Dk);
  if (s->H < 1 || s->B < 1 || s->T < 0 || s->N < 0) return fail(GDR_EINVAL, "bad B/T/H/N");
  if (s->Hk < 0 || s->Hk > s->H || (s->Hk > 0 && s->H % s->Hk != 0))
    return fail(GDR_EINVAL, "Hk (%d) must be 0 or divide H (%d)", s->Hk, s->H);
  if (s->seq_split < 0) return fail(GDR_EINVAL, "seq_split %d must be >= 0", s->seq_split);
  int64_t NC = 0;
  if (s->cu_seqlens_host == nullptr) {
    if (s->N != s->B) return fail(GDR_EINVAL, "dense shape needs N == B (N=%d, B=%d)", s->N, s->B);
    NC = int64_t(s->B) * ((int64_t(s->T) + gdr::kChunk - 1) / gdr::kChunk);
  } else {
    if (s->B != 1) return fail(GDR_EINVAL, "varlen shape needs B == 1");
    if (s->N < 1) return fail(GDR_EINVAL, "varlen shape needs N >= 1");
    const int64_t* cu = s->cu_seqlens_host;
    if (cu[0] != 0) return fail(GDR_EINVAL, "cu_seqlens[0] = %lld, expected 0", (long long)cu[0]);
    for (int n = 0; n < s->N; ++n) {
      if (cu[n + 1] < cu[n]) return fail(GDR_EINVAL, "cu_seqlens decreases at %d", n);
      NC += (cu[n + 1] - cu[n] + gdr::kChunk - 1) / gdr::kChunk;
    }
    if (cu[s->N] != s->T)
      return fail(GDR_EINVAL, "cu_seqlens[N] = %lld != T = %d", (long long)cu[s->N], s->T);
  }
  const int64_t tokens = int64_t(s->B) * s->T;
  if (tokens * s->H * s->Dk >= (int64_t(1) << 40) || NC * s->H * gdr::kChunk >= (int64_t(1) << 31))
    return fail(GDR_EUNSUPPORTED, "problem too large for 32-bit chunk indexing");
  *NC_out = NC;
  return GDR_OK;
}

// ---------------------------------------------------------------------------
// Sequence split of the recursions (exact: both recursions are affine in the
// carried state, so a segment run from zero plus the transfer product of its
// chunks gives its end state for any starting state).
// ---------------------------------------------------------------------------
constexpr int kCUs = gdr::kGpuCUs;
constexpr int kMinSegChunks = 8;    // automatic splits keep at least this many chunks per segment

int64_t seq_chunks(const gdr_shape* s, int n) {
  const int64_t len = s->cu_seqlens_host ? s->cu_seqlens_host[n + 1] - s->cu_seqlens_host[n] : s->T;
  return (len + gdr::kChunk - 1) / gdr::kChunk;
}

// Segments of a sequence of nck chunks when P per sequence are asked for.
int segments_for(int64_t nck, int P, int min_chunks) {
  if (P <= 1 || nck < 2) return 1;
  return int(std::max<int64_t>(1, std::min<int64_t>(P, nck / min_chunks)));
}

struct SplitPlan {
  int P = 1;           // segments asked per sequence
  int min_chunks = 1;  // per segment
  int64_t NS = 0;      // total segments
  bool split = false;  // some sequence has more than one
};

// Time of a plan in chunk steps of a one-slice recursion workgroup (about a
// microsecond each on the headline shape). Each pass (for a split, the local
// pass and then the final one) takes the longest segment's chunks once per round
// of workgroups over the CUs; the launch pads the (segment, head) groups to a
// multiple of 8. Raw-row recursions with more slices than CUs run two slices a
// workgroup, whose step takes about 1.6 times as long. Partial rounds count as
// fractions: workgroups of unequal length leave room for the extra ones. The
// boundary composition walks a sequence's segments in order, about 1.8 steps
// each. The constants are fitted to timings of 2 .. 16 segments on sequences of
// 512 chunks with 2 and 4 heads.
constexpr double kTwoSliceStep = 1.6;
constexpr double kFixStepsPerSegment = 1.8;

double plan_steps(const gdr_shape* s, int P, int min_chunks, SplitPlan* out) {
  const int64_t ns = s->Dk / 16;
  const bool raw = s->gate == GDR_GATE_SCALAR && s->dtype == GDR_BF16;
  int64_t longest = 0, nseg = 0;
  int pmax = 1;
  for (int n = 0; n < s->N; ++n) {
    const int64_t nck = seq_chunks(s, n);
    const int Pn = segments_for(nck, P, min_chunks);
    nseg += Pn;
    pmax = std::max(pmax, Pn);
    longest = std::max<int64_t>(longest, (nck + Pn - 1) / Pn);
    if (!s->cu_seqlens_host) {                // dense: every sequence alike
      nseg *= s->N;
      break;
    }
  }
  const int64_t groups = (nseg * s->H + 7) / 8 * 8;
  auto pass = [&](int64_t slices) {           // slices of both roles
    double wg = double(slices), step = 1.0;
    if (raw && slices > kCUs) {
      wg = 0.5 * double(slices);
      step = kTwoSliceStep;
    }
    return std::max(1.0, wg / kCUs) * step * double(longest);
  };
  double steps = pass(groups * ns * 2);
  if (pmax > 1) steps += pass(groups * 2 * ns * 2) + kFixStepsPerSegment * pmax;
  if (out) {
    out->P = P;
    out->min_chunks = min_chunks;
    out->NS = nseg;
    out->split = pmax > 1;
  }
  return steps;
}

SplitPlan plan_split(const gdr_shape* s) {
  SplitPlan best;
  // the unsplit recursions already give every compute unit a workgroup: a split
  // would only add work
  const bool full = int64_t(2) * s->H * (s->Dk / 16) * s->N >= kCUs;
  if (s->seq_split == 1 || (s->seq_split == 0 && full)) {
    plan_steps(s, 1, 1, &best);
  } else if (s->seq_split >= 2) {
    plan_steps(s, std::min(s->seq_split, gdr::kMaxSegments), 1, &best);
  } else {
    double best_steps = plan_steps(s, 1, 1, &best);
    for (int P = 2; P <= gdr::kMaxSegments; ++P) {
      SplitPlan cand;
      const double st = plan_steps(s, P, kMinSegChunks, &cand);
      if (st < best_steps) {
        best_steps = st;
        best = cand;
      }
    }
  }
  return best;
}

gdr::WsLayout layout(const gdr_shape* s, int64_t NC) {
  gdr::WsLayout L;
  L.NC = NC;
  const SplitPlan sp = plan_split(s);
  L.NS = sp.NS;
  L.split = sp.split ? 1 : 0;
  const size_t H = s->H, K = s->Dk, V = s->Dv, C = gdr::kChunk, NS = size_t(sp.NS);
  const size_t gk = s->gate != GDR_GATE_SCALAR ? K : 1;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  L.ctab = take(NC * sizeof(gdr::ChunkEntry));
  L.stab = take(NS * sizeof(gdr::SeqEntry));
  L.gam = take(H * NC * C * gk * 4);
  L.rho = take(H * NC * 3 * C * 4);
  L.fac = take(H * NC * 3 * C * 4);
  L.edec = take(H * NC * (gk == 1 ? 4 : gk) * 4);
  // materialised Khat / Qbar / W tiles: the per-channel gate and fp32 inputs (the
  // scalar gate with bf16 inputs works from the raw rows, row factors and A)
  const size_t mat = (s->gate != GDR_GATE_SCALAR || s->dtype == GDR_F32) ? 1 : 0;
  L.A = take(H * NC * C * C * 2);
  L.P = take(H * NC * C * C * 2);
  L.W = take(mat * H * NC * C * K * 2);
  L.Up = take(H * NC * C * V * 2);
  L.U = take(H * NC * C * V * 2);
  L.S = take(H * NC * V * K * 2);
  L.dS = take(H * NC * V * K * 2);
  L.dU = take(H * NC * C * V * 2);
  L.Kh = take(mat * H * NC * C * K * 2);
  L.Qh = take(mat * H * NC * C * K * 2);
  L.Ql = take(mat * H * NC * C * K * 2);
  const size_t kda = s->gate != GDR_GATE_SCALAR ? 1 : 0;
  L.Mk = take(kda * H * NC * C * C * 2);
  L.pdA = take(kda * H * NC * 4);
  L.pddt = take(kda * H * NC * K * 4);
  L.Uplo = take(kda * H * NC * C * V * 2);
  L.Ulo = take(kda * H * NC * C * V * 2);
  L.Slo = take(kda * H * NC * V * K * 2);
  L.dSlo = take(kda * H * NC * V * K * 2);
  // fp32 inputs, scalar gate, K = kMatTwoPartK: the low tiles of Khat and W
  const size_t mat2 = (s->gate == GDR_GATE_SCALAR && s->dtype == GDR_F32 && K == size_t(gdr::kMatTwoPartK)) ? 1 : 0;
  L.Khl = take((kda | mat2) * H * NC * C * K * 2);
  L.Wl = take(mat2 * H * NC * C * K * 2);
  L.weak = take(kda * H * NC * 4);
  L.xf = take(L.split * 2 * NS * H * 2 * K * K * 4);
  L.sb = take(L.split * 2 * NS * H * K * K * 4);
  const size_t grouped = s->Hk > 0 && s->Hk < s->H ? 1 : 0;
  const size_t esz = s->dtype == GDR_BF16 ? 2 : 4;
  L.dqv = take(grouped * size_t(s->B) * size_t(s->T) * H * K * esz);
  L.dkv = take(grouped * size_t(s->B) * size_t(s->T) * H * K * esz);
  L.total = off;
  return L;
}

// Token tensors may be NULL only when there are no tokens (an empty tensor has
// no storage); everything else the call reads or writes is required.
bool no_tokens(const gdr_shape* s) { return int64_t(s->B) * s->T == 0; }

gdr_status check_inputs(const gdr_shape* s, const gdr_inputs* in) {
  if (!in) return fail(GDR_EINVAL, "inputs is NULL");
  const void* req[] = {in->q, in->k, in->v, in->g, in->beta_logit};
  const char* names[] = {"q", "k", "v", "g", "beta_logit"};
  for (int i = 0; i < 5; ++i) {
    if (!req[i] && no_tokens(s)) continue;
    if (!req[i]) return fail(GDR_EINVAL, "input %s is NULL", names[i]);
    if (!aligned16(req[i])) return fail(GDR_EINVAL, "input %s is not 16-byte aligned", names[i]);
  }
  if (in->h0 && !aligned16(in->h0)) return fail(GDR_EINVAL, "h0 is not 16-byte aligned");
  if (s->gate != GDR_GATE_SCALAR) {
    if (!in->A_log || !in->dt_bias) return fail(GDR_EINVAL, "per-channel gate needs A_log and dt_bias");
    if (!aligned16(in->A_log) || !aligned16(in->dt_bias))
      return fail(GDR_EINVAL, "A_log/dt_bias not 16-byte aligned");
  } else if (in->A_log || in->dt_bias) {
    return fail(GDR_EINVAL, "scalar gate takes no A_log/dt_bias");
  }
  return GDR_OK;
}

gdr_status check_grads(const gdr_shape* s, const void* dO, const float* dht, const gdr_grads* gr) {
  if (!dO && !no_tokens(s)) return fail(GDR_EINVAL, "dO is NULL");
  if (!aligned16(dO)) return fail(GDR_EINVAL, "dO is not 16-byte aligned");
  if (dht && !aligned16(dht)) return fail(GDR_EINVAL, "dht is not 16-byte aligned");
  if (!gr) return fail(GDR_EINVAL, "grads is NULL");
  const void* req[] = {gr->dq, gr->dk, gr->dv, gr->dg, gr->dbeta};
  const char* names[] = {"dq", "dk", "dv", "dg", "dbeta"};
  for (int i = 0; i < 5; ++i) {
    if (!req[i] && no_tokens(s)) continue;
    if (!req[i]) return fail(GDR_EINVAL, "output %s is NULL", names[i]);
    if (!aligned16(req[i])) return fail(GDR_EINVAL, "output %s is not 16-byte aligned", names[i]);
  }
  if (gr->dh0 && !aligned16(gr->dh0)) return fail(GDR_EINVAL, "dh0 is not 16-byte aligned");
  if (s->gate != GDR_GATE_SCALAR) {
    if (!gr->dA_log || !gr->ddt_bias) return fail(GDR_EINVAL, "per-channel gate needs dA_log and ddt_bias outputs");
    if (!aligned16(gr->dA_log) || !aligned16(gr->ddt_bias))
      return fail(GDR_EINVAL, "dA_log/ddt_bias not 16-byte aligned");
  } else if (gr->dA_log || gr->ddt_bias) {
    return fail(GDR_EINVAL, "scalar gate has no dA_log/ddt_bias outputs");
  }
  return GDR_OK;
}

gdr_status check_ws(const gdr::WsLayout& L, const void* ws, size_t ws_bytes) {
  if (ws_bytes < L.total) return fail(GDR_EWORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, L.total);
  if (!ws && L.total) return fail(GDR_EINVAL, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(GDR_EINVAL, "workspace is not 256-byte aligned");
  return GDR_OK;
}

gdr_status hip_status(int err, const char* what) {
  if (err == 0) return GDR_OK;
  return fail(GDR_EHIP, "%s: %s", what, gdr::hip_error_string(err));
}

// Enqueues the writes of the chunk and segment tables (k_tables).  Dense
// problems take one launch that derives every entry from (B, T) and the number
// of segments per sequence; varlen problems split and order their segments here
// (longest first) and pass the entries by value in batches.  No host memory is
// read after this returns.
gdr_status enqueue_tables(const gdr_shape* s, const gdr::WsLayout& L, void* ws, hipStream_t stream) {
  const int N = s->N;
  if (N == 0) return GDR_OK;
  char* w = static_cast<char*>(ws);
  auto* ctab = reinterpret_cast<const gdr::ChunkEntry*>(w + L.ctab);
  auto* stab = reinterpret_cast<const gdr::SeqEntry*>(w + L.stab);
  const SplitPlan sp = plan_split(s);
  gdr::TableBatch tb;
  std::memset(&tb, 0, sizeof(tb));
  if (!s->cu_seqlens_host) {
    tb.n = N;
    tb.first = 0;
    tb.kind = 0;
    tb.dense_T = s->T;
    tb.nseg = segments_for(seq_chunks(s, 0), sp.P, sp.min_chunks);
    return hip_status(gdr::launch_tables(ctab, stab, tb, stream), "table kernel");
  }
  std::vector<gdr::SeqEntry> seqs(N), segs;
  segs.reserve(size_t(L.NS));
  int64_t c = 0;
  for (int n = 0; n < N; ++n) {
    const int64_t b = s->cu_seqlens_host[n], e = s->cu_seqlens_host[n + 1];
    const int len = int(e - b);
    const int nck = int((len + gdr::kChunk - 1) / gdr::kChunk);
    seqs[n] = gdr::SeqEntry{n, len, int32_t(c), nck, int32_t(b), 0, 1, 0};
    const int P = segments_for(nck, sp.P, sp.min_chunks);
    const int slot0 = int(segs.size());
    for (int j = 0; j < P; ++j) {
      const int a0 = j * nck / P, a1 = (j + 1) * nck / P;
      const int slen = std::min(len, a1 * gdr::kChunk) - a0 * gdr::kChunk;
      segs.push_back(gdr::SeqEntry{n, slen, int32_t(c + a0), a1 - a0, int32_t(b + int64_t(a0) * gdr::kChunk), j, P,
                                   slot0 + j});
    }
    c += nck;
  }
  std::stable_sort(segs.begin(), segs.end(),
                   [](const gdr::SeqEntry& x, const gdr::SeqEntry& y) { return x.len > y.len; });
  for (int kind = 1; kind <= 2; ++kind) {
    const std::vector<gdr::SeqEntry>& v = kind == 1 ? seqs : segs;
    const int n_all = int(v.size());
    for (int first = 0; first < n_all; first += gdr::kTableBatch) {
      tb.n = std::min(gdr::kTableBatch, n_all - first);
      tb.first = first;
      tb.kind = kind;
      tb.dense_T = -1;
      for (int i = 0; i < tb.n; ++i) tb.e[i] = v[first + i];
      gdr_status r = hip_status(gdr::launch_tables(ctab, stab, tb, stream), "table kernel");
      if (r != GDR_OK) return r;
    }
  }
  return GDR_OK;
}

gdr::Params make_params(const gdr_shape* s, const gdr::WsLayout& L, const gdr_inputs* in, void* ws) {
  gdr::Params p;
  std::memset(&p, 0, sizeof(p));
  p.H = s->H; p.K = s->Dk; p.V = s->Dv; p.N = s->N; p.NC = int32_t(L.NC); p.T = s->B * s->T;
  p.NS = int32_t(L.NS);
  p.Hk = s->Hk > 0 ? s->Hk : s->H;
  p.G = s->H / p.Hk;
  // the kernels tell the scalar gate from the per-channel one; the per-channel
  // gate function (softplus or bounded sigmoid) matters only where it is applied
  p.gate = s->gate == GDR_GATE_SCALAR ? 0 : 1;
  p.gate_fn = s->gate == GDR_GATE_CHANNEL_SIGMOID ? 1 : 0;
  p.gate_scale = s->gate_scale;
  p.dtype = s->dtype; p.scale = s->scale;
  p.q = in->q; p.k = in->k; p.v = in->v; p.g = in->g; p.b = in->beta_logit;
  p.A_log = in->A_log; p.dt_bias = in->dt_bias; p.h0 = in->h0;
  char* w = static_cast<char*>(ws);
  p.ctab = reinterpret_cast<const gdr::ChunkEntry*>(w + L.ctab);
  p.stab = reinterpret_cast<const gdr::SeqEntry*>(w + L.stab);
  p.gam = reinterpret_cast<float*>(w + L.gam);
  p.rho = reinterpret_cast<float*>(w + L.rho);
  p.fac = reinterpret_cast<float*>(w + L.fac);
  p.edec = reinterpret_cast<float*>(w + L.edec);
  p.A = reinterpret_cast<uint16_t*>(w + L.A);
  p.P = reinterpret_cast<uint16_t*>(w + L.P);
  p.W = reinterpret_cast<uint16_t*>(w + L.W);
  p.Up = reinterpret_cast<uint16_t*>(w + L.Up);
  p.U = reinterpret_cast<uint16_t*>(w + L.U);
  p.S = reinterpret_cast<uint16_t*>(w + L.S);
  p.dS = reinterpret_cast<uint16_t*>(w + L.dS);
  p.dU = reinterpret_cast<uint16_t*>(w + L.dU);
  p.Kh = reinterpret_cast<uint16_t*>(w + L.Kh);
  p.Qh = reinterpret_cast<uint16_t*>(w + L.Qh);
  p.Ql = reinterpret_cast<uint16_t*>(w + L.Ql);
  p.Mk = reinterpret_cast<uint16_t*>(w + L.Mk);
  p.pdA = reinterpret_cast<float*>(w + L.pdA);
  p.pddt = reinterpret_cast<float*>(w + L.pddt);
  p.Uplo = reinterpret_cast<uint16_t*>(w + L.Uplo);
  p.Ulo = reinterpret_cast<uint16_t*>(w + L.Ulo);
  p.Slo = reinterpret_cast<uint16_t*>(w + L.Slo);
  p.dSlo = reinterpret_cast<uint16_t*>(w + L.dSlo);
  p.Khl = reinterpret_cast<uint16_t*>(w + L.Khl);
  p.Wl = reinterpret_cast<uint16_t*>(w + L.Wl);
  p.weak = reinterpret_cast<int32_t*>(w + L.weak);
  p.xf = L.split ? reinterpret_cast<float*>(w + L.xf) : nullptr;
  p.sb = L.split ? reinterpret_cast<float*>(w + L.sb) : nullptr;
  return p;
}

// With grouped heads the kernels write dq, dk per value head into the workspace;
// group_sum then reduces them into the caller's [tokens][Hk][K] outputs.
void set_grads(gdr::Params& p, const gdr::WsLayout& L, void* ws, const void* dO, const float* dht,
               const gdr_grads* gr) {
  p.dO = dO; p.dht = dht;
  p.dq = gr->dq; p.dk = gr->dk; p.dv = gr->dv; p.dg = gr->dg; p.db = gr->dbeta;
  if (p.G > 1) {
    p.dq = static_cast<char*>(ws) + L.dqv;
    p.dk = static_cast<char*>(ws) + L.dkv;
  }
  p.dh0 = gr->dh0; p.dA_log = gr->dA_log; p.ddt_bias = gr->ddt_bias;
}

enum Stage { kFwd = 1, kBwd = 2, kFused = 3 };

// `only` >= 0 restricts the launch sequence to one GDR_STAGE_* kernel.
gdr_status run(int stage, const gdr_shape* s, const gdr_inputs* in, const void* dO, const float* dht,
               void* ws, size_t ws_bytes, const gdr_grads* gr, float* ht, void* stream, int only = -1,
               void* o = nullptr) {
  int64_t NC = 0;
  gdr_status st = check_shape(s, &NC);
  if (st != GDR_OK) return st;
  if ((st = check_inputs(s, in)) != GDR_OK) return st;
  if (stage != kFwd && (st = check_grads(s, dO, dht, gr)) != GDR_OK) return st;
  if (ht && !aligned16(ht)) return fail(GDR_EINVAL, "ht is not 16-byte aligned");
  if (o && !aligned16(o)) return fail(GDR_EINVAL, "o is not 16-byte aligned");
  const gdr::WsLayout L = layout(s, NC);
  if ((st = check_ws(L, ws, ws_bytes)) != GDR_OK) return st;

  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  // a single stage reuses the tables the full call before it wrote
  if (only < 0 && (st = enqueue_tables(s, L, ws, hs)) != GDR_OK) return st;
  gdr::Params p = make_params(s, L, in, ws);
  p.ht = ht;
  p.o = o;
  if (stage != kFwd) set_grads(p, L, ws, dO, dht, gr);

  const bool kda = s->gate != GDR_GATE_SCALAR;
  auto prep = [&]() { return kda ? gdr::launch_kda(p, 0, stream) : gdr::launch_prep(p, stream); };
  auto grads = [&]() { return kda ? gdr::launch_kda(p, 1, stream) : gdr::launch_grads(p, stream); };
  // both gates' prepare-backward is fused into their gradient kernels; what is
  // left: the per-head reduction of the per-channel gate's parameter partial
  // sums and, with grouped heads, the dq, dk group sums
  auto finish = [&]() {
    int e = 0;
    if (kda && !e) e = gdr::launch_kda(p, 2, stream);
    if (p.G > 1 && !e) e = gdr::launch_group_sum(p, p.dq, gr->dq, stream);
    if (p.G > 1 && !e) e = gdr::launch_group_sum(p, p.dk, gr->dk, stream);
    return e;
  };
  // the recursions: for split sequences the local pass and the boundary
  // composition first, then the final pass over every segment
  auto chain = [&](int mode) {
    int e = 0;
    if (L.split) {
      e = gdr::launch_chain(p, mode, gdr::kPassLocal, stream);
      if (!e) e = gdr::launch_chain_fix(p, mode, stream);
    }
    if (!e) e = gdr::launch_chain(p, mode, gdr::kPassFinal, stream);
    return e;
  };
  if (only >= 0) {
    switch (only) {
      case GDR_STAGE_PREP: return NC > 0 ? hip_status(prep(), "prep kernel") : GDR_OK;
      case GDR_STAGE_CHAIN_FWD: return hip_status(chain(gdr::kChainFwd), "chain kernel");
      case GDR_STAGE_CHAIN_BWD: return hip_status(chain(gdr::kChainBwd), "chain kernel");
      case GDR_STAGE_CHAIN_BOTH: return hip_status(chain(gdr::kChainBoth), "chain kernel");
      case GDR_STAGE_GRADS: return NC > 0 ? hip_status(grads(), "gradient kernel") : GDR_OK;
      case GDR_STAGE_FINISH:
        if (NC > 0) return hip_status(finish(), "parameter reduction kernel");
        return kda ? hip_status(gdr::launch_zero_params(p, stream), "zero kernel") : GDR_OK;
      default: return fail(GDR_EINVAL, "unknown stage %d", only);
    }
  }
  if (stage != kBwd && NC > 0) {
    if ((st = hip_status(prep(), "prep kernel")) != GDR_OK) return st;
  }
  const int mode = stage == kFwd ? gdr::kChainFwd : stage == kBwd ? gdr::kChainBwd : gdr::kChainBoth;
  if ((st = hip_status(chain(mode), "chain kernel")) != GDR_OK) return st;
  if (o && NC > 0) {
    if ((st = hip_status(gdr::launch_output(p, stream), "output kernel")) != GDR_OK) return st;
  }
  if (stage != kFwd) {
    if (NC > 0) {
      if ((st = hip_status(grads(), "gradient kernel")) != GDR_OK) return st;
      if ((st = hip_status(finish(), "parameter reduction kernel")) != GDR_OK) return st;
    } else if (kda) {
      // no tokens: the per-head parameter gradients are zero
      if ((st = hip_status(gdr::launch_zero_params(p, stream), "zero kernel")) != GDR_OK) return st;
    }
  }
  return GDR_OK;
}

}  // namespace

namespace gdr {
gdr_status set_error(gdr_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}
}  // namespace gdr

extern "C" {

gdr_status gdr_workspace_bytes(const gdr_shape* shape, size_t* bytes) {
  int64_t NC = 0;
  gdr_status st = check_shape(shape, &NC);
  if (st != GDR_OK) return st;
  if (!bytes) return fail(GDR_EINVAL, "bytes is NULL");
  *bytes = layout(shape, NC).total;
  return GDR_OK;
}

gdr_status gdr_fwd_recompute(const gdr_shape* shape, const gdr_inputs* in, void* ws, size_t ws_bytes, void* o,
                             float* ht, void* stream) {
  return run(kFwd, shape, in, nullptr, nullptr, ws, ws_bytes, nullptr, ht, stream, -1, o);
}

gdr_status gdr_fwd(const gdr_shape* shape, const gdr_inputs* in, void* ws, size_t ws_bytes, void* o, float* ht,
                   void* stream) {
  if (!o && !(shape && no_tokens(shape))) return fail(GDR_EINVAL, "o is NULL");
  return run(kFwd, shape, in, nullptr, nullptr, ws, ws_bytes, nullptr, ht, stream, -1, o);
}

gdr_status gdr_bwd(const gdr_shape* shape, const gdr_inputs* in, const void* dO, const float* dht, void* ws,
                   size_t ws_bytes, gdr_grads* grads, void* stream) {
  return run(kBwd, shape, in, dO, dht, ws, ws_bytes, grads, nullptr, stream);
}

gdr_status gdr_fwd_bwd(const gdr_shape* shape, const gdr_inputs* in, const void* dO, const float* dht, void* ws,
                       size_t ws_bytes, gdr_grads* grads, float* ht, void* stream) {
  return run(kFused, shape, in, dO, dht, ws, ws_bytes, grads, ht, stream);
}

gdr_status gdr_run_stage(const gdr_shape* shape, const gdr_inputs* in, const void* dO, const float* dht, void* ws,
                         size_t ws_bytes, gdr_grads* grads, float* ht, int32_t stage, void* stream) {
  if (stage < GDR_STAGE_PREP || stage > GDR_STAGE_FINISH) return fail(GDR_EINVAL, "unknown stage %d", stage);
  return run(kFused, shape, in, dO, dht, ws, ws_bytes, grads, ht, stream, stage);
}

gdr_status gdr_workspace_region(const gdr_shape* shape, int32_t which, size_t* offset, size_t* bytes) {
  int64_t NC = 0;
  gdr_status st = check_shape(shape, &NC);
  if (st != GDR_OK) return st;
  if (!offset || !bytes) return fail(GDR_EINVAL, "offset/bytes is NULL");
  const gdr::WsLayout L = layout(shape, NC);
  const size_t H = shape->H, K = shape->Dk, V = shape->Dv, C = gdr::kChunk;
  const size_t gk = shape->gate != GDR_GATE_SCALAR ? K : 1;
  switch (which) {
    case GDR_WS_STATE: *offset = L.S; *bytes = H * NC * V * K * 2; break;
    case GDR_WS_DSTATE: *offset = L.dS; *bytes = H * NC * V * K * 2; break;
    case GDR_WS_U: *offset = L.U; *bytes = H * NC * C * V * 2; break;
    case GDR_WS_A: *offset = L.A; *bytes = H * NC * C * C * 2; break;
    case GDR_WS_GAMMA: *offset = L.gam; *bytes = H * NC * C * gk * 4; break;
    default: return fail(GDR_EINVAL, "unknown workspace region %d", which);
  }
  return GDR_OK;
}

const char* gdr_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

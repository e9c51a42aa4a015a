// k_tables: writes the chunk table and the segment table into the workspace.
//
// The host decides how sequences split into segments (runs of whole chunks the
// recursions treat as units) and hands the entries to this kernel by value, up
// to kTableBatch per launch; each workgroup writes one entry.  Nothing is
// copied from host memory: the launch arguments are captured with the launch,
// so the enqueue neither waits for the host nor depends on host memory staying
// alive, and it can be recorded into a graph like every other launch of the
// library.
#include <hip/hip_runtime.h>

#include "gdr_internal.h"

namespace gdr {

__device__ __forceinline__ void write_chunks(ChunkEntry* ctab, const SeqEntry& se) {
  for (int c = threadIdx.x; c < se.nchunks; c += blockDim.x)
    ctab[se.c0 + c] = ChunkEntry{se.t_start + c * kChunk, min(kChunk, se.len - c * kChunk), se.seq, c};
}

__global__ __launch_bounds__(256) void k_tables(ChunkEntry* ctab, SeqEntry* stab, const TableBatch tb) {
  const int i = blockIdx.x;
  if (i >= tb.n) return;
  if (tb.kind == 0) {
    // dense sequence n: dense_T tokens from token n dense_T, chunks from n nck; its
    // segment j covers chunks [j nck / nseg, (j + 1) nck / nseg)
    const int n = tb.first + i;
    const int nck = (tb.dense_T + kChunk - 1) / kChunk;
    const SeqEntry sq{n, tb.dense_T, n * nck, nck, n * tb.dense_T, 0, 1, n};
    write_chunks(ctab, sq);
    if (threadIdx.x < tb.nseg) {
      const int j = threadIdx.x;
      const int a = j * nck / tb.nseg, b = (j + 1) * nck / tb.nseg;
      const int len = min(tb.dense_T, b * kChunk) - a * kChunk;
      stab[n * tb.nseg + j] = SeqEntry{n, len, sq.c0 + a, b - a, sq.t_start + a * kChunk, j, tb.nseg, n * tb.nseg + j};
    }
  } else if (tb.kind == 1) {
    write_chunks(ctab, tb.e[i]);
  } else {
    if (threadIdx.x == 0) stab[tb.first + i] = tb.e[i];
  }
}

int launch_tables(const ChunkEntry* ctab, const SeqEntry* stab, const TableBatch& tb, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (tb.n <= 0) return 0;
  k_tables<<<dim3(tb.n), 256, 0, s>>>(const_cast<ChunkEntry*>(ctab), const_cast<SeqEntry*>(stab), tb);
  return static_cast<int>(hipGetLastError());
}

}  // namespace gdr

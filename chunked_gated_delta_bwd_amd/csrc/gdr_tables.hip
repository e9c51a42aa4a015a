// k_tables: writes the chunk table and the sequence table into the workspace.
//
// The host orders the sequences (longest first, so the serial kernels start the
// longest chains first) and hands their entries to this kernel by value, up to
// kTableBatch per launch; each workgroup writes one sequence entry and the chunk
// entries of that sequence.  Nothing is copied from host memory: the launch
// arguments are captured with the launch, so the enqueue neither waits for the
// host nor depends on host memory staying alive, and it can be recorded into a
// graph like every other launch of the library.
#include <hip/hip_runtime.h>

#include "gdr_internal.h"

namespace gdr {

__global__ __launch_bounds__(256) void k_tables(ChunkEntry* ctab, SeqEntry* stab, const TableBatch tb) {
  const int i = blockIdx.x;
  if (i >= tb.n) return;
  SeqEntry se;
  if (tb.dense_T >= 0) {
    // B sequences of dense_T tokens in their natural order (all equally long)
    const int n = tb.first + i;
    const int nck = (tb.dense_T + kChunk - 1) / kChunk;
    se = SeqEntry{n, tb.dense_T, n * nck, nck, n * tb.dense_T, {0, 0, 0}};
  } else {
    se = tb.seqs[i];
  }
  if (threadIdx.x == 0) stab[tb.first + i] = se;
  for (int c = threadIdx.x; c < se.nchunks; c += blockDim.x)
    ctab[se.c0 + c] = ChunkEntry{se.t_start + c * kChunk, min(kChunk, se.len - c * kChunk), se.seq, c};
}

int launch_tables(const ChunkEntry* ctab, const SeqEntry* stab, const TableBatch& tb, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (tb.n <= 0) return 0;
  k_tables<<<dim3(tb.n), 256, 0, s>>>(const_cast<ChunkEntry*>(ctab), const_cast<SeqEntry*>(stab), tb);
  return static_cast<int>(hipGetLastError());
}

}  // namespace gdr

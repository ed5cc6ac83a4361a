// GELU of the adapter and of the audio encoder (model card "ark-asr-3b-onnx",
// "Inference" steps 1 and 3; the activation is a reading: the erf GELU of
// the Whisper encoder).  y <- fp32(0.5 y (1 + erf(y / sqrt 2))) in fp64, in
// place, optionally plus a row of a table (the encoder's positional rows,
// added in fp32 after the rounding), and optionally the per-sequence range
// of the result for the dynamic quantisation that follows (folded like
// every other producer's range).
#include "common.hpp"
#include "kernels.hpp"

namespace ark {

// grid (column blocks, row blocks); 256 threads, each a run of columns of
// rows blockIdx.y, blockIdx.y + gridDim.y, ...
__global__ __launch_bounds__(256) void k_gelu_stats(int R, int N, int rows_per_seq,
                                                    float* __restrict__ y, int ldy,
                                                    const float* __restrict__ add, int ldadd,
                                                    SeqStats S) {
  const bool stats = S.cur != nullptr;
  if (stats) stats_clear_other(S);
  for (int r = blockIdx.y; r < R; r += gridDim.y) {
    float* row = y + (size_t)r * ldy;
    const float* arow = add ? add + (size_t)(r % rows_per_seq) * ldadd : nullptr;
    float lo = INFINITY, hi = -INFINITY;
    for (int c = blockIdx.x * 256 + threadIdx.x; c < N; c += gridDim.x * 256) {
      const double x = row[c];
      // the same operations as the definition: x / sqrt(2) with sqrt(2)
      // rounded to fp64, erf in fp64, one rounding to fp32
      float g = (float)(0.5 * x * (1.0 + erf(x / 1.4142135623730951)));
      if (arow) g = g + arow[c];
      row[c] = g;
      lo = fminf(lo, g);
      hi = fmaxf(hi, g);
    }
    if (stats) {
      lo = wave_min(lo);
      hi = wave_max(hi);
      if ((threadIdx.x & 63) == 0)
        stats_fold(S, (r * gridDim.x + blockIdx.x) * 4 + (threadIdx.x >> 6), r / rows_per_seq, lo,
                   hi);
    }
  }
}

hipError_t launch_gelu_stats(hipStream_t st, int R, int N, int rows_per_seq, float* y, int ldy,
                             const SeqStats& S, const float* add, int ldadd) {
  const int cx = std::max(1, std::min(8, (N + 1023) / 1024));
  const int cy = std::min(R, 65535);
  hipLaunchKernelGGL(k_gelu_stats, dim3(cx, cy), dim3(256), 0, st, R, N, rows_per_seq, y, ldy, add,
                     ldadd, S);
  return hipGetLastError();
}

}  // namespace ark

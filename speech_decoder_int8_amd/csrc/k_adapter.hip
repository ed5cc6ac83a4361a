// The adapter's activation (model card "ark-asr-3b-onnx", "Inference" step
// 3; the activation is a reading: the erf GELU of the Whisper encoder whose
// frames the adapter merges).  y <- fp32(0.5 y (1 + erf(y / sqrt 2))) in
// fp64, in place, and the per-sequence range of the result for the dynamic
// quantisation that follows (folded like every other producer's range).
#include "common.hpp"
#include "kernels.hpp"

namespace ark {

// grid (column blocks, rows); 256 threads, each a run of columns.
__global__ __launch_bounds__(256) void k_gelu_stats(int N, int rows_per_seq, float* __restrict__ y,
                                                    int ldy, SeqStats S) {
  stats_clear_other(S);
  const int r = blockIdx.y;
  float* row = y + (size_t)r * ldy;
  float lo = INFINITY, hi = -INFINITY;
  for (int c = blockIdx.x * 256 + threadIdx.x; c < N; c += gridDim.x * 256) {
    const double x = row[c];
    // the same operations as the definition: x / sqrt(2) with sqrt(2)
    // rounded to fp64, erf in fp64, one rounding to fp32
    const float g = (float)(0.5 * x * (1.0 + erf(x / 1.4142135623730951)));
    row[c] = g;
    lo = fminf(lo, g);
    hi = fmaxf(hi, g);
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  if ((threadIdx.x & 63) == 0)
    stats_fold(S, (blockIdx.y * gridDim.x + blockIdx.x) * 4 + (threadIdx.x >> 6),
               r / rows_per_seq, lo, hi);
}

hipError_t launch_gelu_stats(hipStream_t st, int R, int N, int rows_per_seq, float* y, int ldy,
                             const SeqStats& S) {
  const int cx = std::max(1, std::min(8, (N + 1023) / 1024));
  hipLaunchKernelGGL(k_gelu_stats, dim3(cx, R), dim3(256), 0, st, N, rows_per_seq, y, ldy, S);
  return hipGetLastError();
}

}  // namespace ark

// int8 x int8 -> int32 GEMM for few activation rows (M <= 64: batched decode
// and the LM head of a batch), weight-stream bound, on gfx950 matrix cores
// (v_mfma_i32_32x32x32_i8), with the same dequantising epilogues as k_gemm
// (store (+bias), residual add, SwiGLU over paired gate/up rows).
//
// One 32x32x32 instruction covers a block of 32 rows; up to two blocks (MB)
// share each weight fragment, so every weight byte is read from HBM once
// per pass of up to 64 rows.  A workgroup of 4 waves
// owns 128 weight rows (wave w: rows 32 w .. 32 w + 31; for SwiGLU 16 gate
// rows and the 16 up rows of the same outputs) and a range of K, walked in
// 128-byte steps.  Each step's tiles (128 weight rows and the 32 activation
// rows, 128 bytes each) go from global memory straight into LDS with
// 16-byte LDS-DMA loads: one instruction moves 8 whole 128-byte row
// segments; three steps are in flight.  In LDS the 16-byte chunk c of row r
// sits at chunk c ^ ((r >> 1) & 7), so the 16 rows one fragment read
// touches cover all 64 banks; each lane fetches the global chunk that
// belongs at its LDS position.  Fragment layout: lane l supplies row l % 32
// of its activation and weight fragments with K bytes 32 c + 16 (l / 32) ..
// +16 for instruction c = 0..3 of the step.
//
// Small weight matrices are split along K over ks workgroups per row tile
// (so that a launch still spreads over the whole chip): each adds its int32
// sums into the tile's block with device-scope atomic additions, and the
// last one to arrive (tile counter) reads the block, clears it and the
// counter for the next launch, and runs the epilogue.  Integer sums are
// exact, so the result does not depend on the split or the order.
//
// Accumulator layout (32x32 int32 in 16 registers): register r of lane l
// holds row (r / 4) * 8 + (l / 32) * 4 + r % 4, column l % 32.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace ark {

typedef int i32x16 __attribute__((ext_vector_type(16)));

namespace sk {
constexpr int NT = 256, ROWS = 128, SS = 128, NS = 3;
constexpr int B_BYTES = ROWS * SS;
// MB blocks of 32 activation rows (1, or 2 for 33..64 rows: the weights are
// streamed once for all of them)
template <int MB>
struct Cfg {
  static constexpr int A_BYTES = 32 * MB * SS, STAGE = B_BYTES + A_BYTES, LDS = NS * STAGE;
  static constexpr int LPW = 4 + MB;  // loads per wave per step
};
constexpr int MAX_MB = 2;
}  // namespace sk

struct GemmSkParams {
  int M, K, ncols, epi, rows_per_seq, nseg, tiles, ks, nss;
  int row0;  // first row of this launch in the caller's row space (sequence of row m: (row0 + m) / rows_per_seq)
  const int8_t* A;
  const float* qs;
  const int* qz;
  Seg seg[3];
  int seg_start[4];
  int32_t* part;     // [tiles][32 MB][ROWS] int32 sums of split launches, zero between launches
  uint32_t* ctr;     // [tiles] arrival counters, zero between launches
  int32_t* acc_out;  // optional [M][ncols]: raw sums (tests)
  int32_t* pout;     // optional [ks][M][ncols]: each split's int32 sums, no epilogue
};

__device__ __forceinline__ int sk_swz(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

template <int N>
__device__ __forceinline__ void sk_wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

template <int MB>
__global__ __launch_bounds__(256, 2) void k_gemm_sk(GemmSkParams P) {
  using namespace sk;
  constexpr int STAGE = Cfg<MB>::STAGE, LPW = Cfg<MB>::LPW;
  extern __shared__ __align__(16) int8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool swiglu = P.epi == EPI_SWIGLU;
  const int tile = blockIdx.x % P.tiles, kp = blockIdx.x / P.tiles;
  const int K = P.K;
  const int j = lane & 31, half = lane >> 5;

  // DMA sources: weight instruction i (0..3) of this wave covers tile rows
  // 8 (4 w + i) .. +8, the activation instruction rows 8 w .. 8 w + 7; lane l
  // lands at LDS chunk l % 8 of row l / 8 and fetches the chunk stored there.
  // Rows past ncols or M read row 0 instead (their products only reach
  // outputs that are never stored), so every wave issues exactly 5 loads per
  // step and the waits below can count them.
  const int8_t* bsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * (4 * wave + i) + (lane >> 3);  // tile row
    const int c = (lane & 7) ^ ((r >> 1) & 7);       // global chunk at this position
    bsrc[i] = P.seg[0].w + 16 * c;
    if (swiglu) {
      // tile rows 32 v .. 32 v + 15: gate outputs 16 v.., rows 32 v + 16..: up
      const int v = r >> 5, q = r & 31;
      const int n = tile * (ROWS / 2) + v * 16 + (q & 15);
      if (n < P.ncols) bsrc[i] = (q < 16 ? P.seg[0].w : P.seg[1].w) + (size_t)n * K + 16 * c;
    } else {
      const int n = tile * ROWS + r;
      if (n < P.ncols) {
        int s = 0;
        while (s + 1 < P.nseg && n >= P.seg_start[s + 1]) ++s;
        bsrc[i] = P.seg[s].w + (size_t)(n - P.seg_start[s]) * K + 16 * c;
      }
    }
  }
  // activation instruction a of this wave covers rows 8 (MB wave + a) .. + 7
  const int8_t* asrc[MB];
#pragma unroll
  for (int a = 0; a < MB; ++a) {
    const int r = 8 * (MB * wave + a) + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    asrc[a] = P.A + (size_t)(r < P.M ? r : 0) * K + 16 * c;
  }
  const int s0 = kp * P.nss, s1 = min(s0 + P.nss, K / SS);
  const int nk = s1 - s0;

  auto issue = [&](int st, int buf) {
    int8_t* base = lds + buf * STAGE;
    const size_t o = (size_t)(s0 + st) * SS;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(bsrc[i] + o),
          (void __attribute__((address_space(3)))*)(base + (4 * wave + i) * 1024), 16, 0, 2);
#pragma unroll
    for (int a = 0; a < MB; ++a)
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(asrc[a] + o),
          (void __attribute__((address_space(3)))*)(base + B_BYTES + (MB * wave + a) * 1024), 16,
          0, 0);
  };
  for (int st = 0; st < NS - 1; ++st)
    if (st < nk) issue(st, st);

  i32x16 acc[MB];
#pragma unroll
  for (int bI = 0; bI < MB; ++bI)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[bI][r] = 0;
  for (int st = 0; st < nk; ++st) {
    if (st + 1 < nk)
      sk_wait_vm<LPW>();  // this wave's loads of step st are done (step st+1's may be in flight)
    else
      sk_wait_vm<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();         // every wave's step-st loads landed; buffer st+2 free
    if (st + NS - 1 < nk) issue(st + NS - 1, (st + NS - 1) % NS);
    const int8_t* Bs = lds + (st % NS) * STAGE;
    const int8_t* As = Bs + B_BYTES;
    i32x4 fa[MB][4], fb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int bI = 0; bI < MB; ++bI)
        fa[bI][c] = *(const i32x4*)(As + sk_swz(32 * bI + j, 2 * c + half));
      fb[c] = *(const i32x4*)(Bs + sk_swz(32 * wave + j, 2 * c + half));
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int bI = 0; bI < MB; ++bI)
        acc[bI] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[bI][c], fb[c], acc[bI], 0, 0, 0);
  }

  if (P.pout) {
    // this K range's sums as they are; a row kernel adds the splits and
    // runs the epilogue
    const int col = tile * ROWS + wave * 32 + j;
    if (col < P.ncols) {
      int32_t* dst = P.pout + (size_t)kp * P.M * P.ncols + col;
#pragma unroll
      for (int bI = 0; bI < MB; ++bI)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = 32 * bI + (r / 4) * 8 + half * 4 + r % 4;
          if (m < P.M) dst[(size_t)m * P.ncols] = acc[bI][r];
        }
    }
    return;
  }

  if (P.ks > 1) {
    // add this K range's sums into the tile's block (device-scope atomics,
    // performed at the coherence point); the last arrival reads the block
    // back, clears it for the next launch and runs the epilogue
    int32_t* blk = P.part + (size_t)tile * 32 * MB * ROWS;
#pragma unroll
    for (int bI = 0; bI < MB; ++bI)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 32 * bI + (r / 4) * 8 + half * 4 + r % 4;
        __hip_atomic_fetch_add(blk + m * ROWS + wave * 32 + j, acc[bI][r], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's additions are performed
    __syncthreads();
    __shared__ uint32_t last;
    if (tid == 0) {
      const uint32_t old = __hip_atomic_fetch_add(P.ctr + tile, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      last = (old == (uint32_t)P.ks - 1);
    }
    __syncthreads();
    if (!last) return;
#pragma unroll
    for (int bI = 0; bI < MB; ++bI)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 32 * bI + (r / 4) * 8 + half * 4 + r % 4;
        int32_t* a = blk + m * ROWS + wave * 32 + j;
        acc[bI][r] = __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
    for (int bI = 0; bI < MB; ++bI)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 32 * bI + (r / 4) * 8 + half * 4 + r % 4;
        __hip_atomic_store(blk + m * ROWS + wave * 32 + j, 0, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    if (tid == 0)
      __hip_atomic_store(P.ctr + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- epilogue, once per block of 32 activation rows (rows mb .. mb + 31)
#pragma unroll
  for (int bI = 0; bI < MB; ++bI) {
  const int mb = 32 * bI;
  const i32x16 accb = acc[bI];
  // ---- epilogue: row m = mb + (r / 4) * 8 + half * 4 + r % 4, weight row j.
  // Parameter-block fields are taken as wave-uniform values (a per-lane
  // choice between them would become a vector load of the block), and every
  // per-row parameter and residual input is requested in one batch before
  // the first is used: the rows share one wait instead of one each.
  const gptr<const float> qs = uniform_ptr(P.qs);
  const gptr<const int> qz = uniform_ptr(P.qz);
  const int M = P.M, rps = P.rows_per_seq, row0 = P.row0;
  const gptr<int32_t> acc_out = uniform_ptr(P.acc_out);
  float rs[16];
  int rz[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = min(mb + (r / 4) * 8 + half * 4 + r % 4, M - 1);
    const int b = (row0 + m) / rps;
    rs[r] = qs[b];
    rz[r] = qz[b];
  }
  // one wait for the whole batch: the values pass through this (empty)
  // statement, so no use of them can be scheduled before every load is out
  asm volatile("" : "+v"(rs[0]), "+v"(rs[1]), "+v"(rs[2]), "+v"(rs[3]), "+v"(rs[4]), "+v"(rs[5]),
               "+v"(rs[6]), "+v"(rs[7]), "+v"(rs[8]), "+v"(rs[9]), "+v"(rs[10]), "+v"(rs[11]),
               "+v"(rs[12]), "+v"(rs[13]), "+v"(rs[14]), "+v"(rs[15]));
  asm volatile("" : "+v"(rz[0]), "+v"(rz[1]), "+v"(rz[2]), "+v"(rz[3]), "+v"(rz[4]), "+v"(rz[5]),
               "+v"(rz[6]), "+v"(rz[7]), "+v"(rz[8]), "+v"(rz[9]), "+v"(rz[10]), "+v"(rz[11]),
               "+v"(rz[12]), "+v"(rz[13]), "+v"(rz[14]), "+v"(rz[15]));
#pragma unroll
  for (int r = 0; r < 16; ++r) rz[r] = 128 - rz[r];
  if (swiglu) {
    const gptr<const float> gsw = uniform_ptr(P.seg[0].sw), usw = uniform_ptr(P.seg[1].sw);
    const gptr<const int32_t> gcs = uniform_ptr(P.seg[0].cs), ucs = uniform_ptr(P.seg[1].cs);
    const gptr<float> out = uniform_ptr(P.seg[0].out);
    const int ldo = __builtin_amdgcn_readfirstlane(P.seg[0].ldo);
    const int n = tile * (ROWS / 2) + wave * 16 + (j & 15);
    const int nn = min(n, P.ncols - 1);
    const float sg = gsw[nn], su = usw[nn];
    const int cg = gcs[nn], cu = ucs[nn];
    const SwigluK SK = swiglu_consts();
    float y[16];
    int ag[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int up = __shfl_down(accb[r], 16, 32);  // lane j < 16 gets row j's up sum
      ag[r] = accb[r] + rz[r] * cg;
      const float g = dequant(ag[r], rs[r], sg);
      const float u = dequant(up + rz[r] * cu, rs[r], su);
      y[r] = swiglu_f64(g, u, SK);
    }
    // computed here, ahead of the guarded stores (sunk into them, each
    // store would wait for every earlier memory operation, stores included)
    asm volatile("" : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3]), "+v"(y[4]), "+v"(y[5]),
                 "+v"(y[6]), "+v"(y[7]), "+v"(y[8]), "+v"(y[9]), "+v"(y[10]), "+v"(y[11]),
                 "+v"(y[12]), "+v"(y[13]), "+v"(y[14]), "+v"(y[15]));
    if (j < 16 && n < P.ncols) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = mb + (r / 4) * 8 + half * 4 + r % 4;
        if (m >= M) continue;
        out[(size_t)m * ldo + n] = y[r];
        if (acc_out) acc_out[(size_t)m * P.ncols + n] = ag[r];
      }
    }
  } else {
    const int col = tile * ROWS + wave * 32 + j;
    const int cc = min(col, P.ncols - 1);
    const int nseg = P.nseg;
    const int sb1 = __builtin_amdgcn_readfirstlane(nseg > 1 ? P.seg_start[1] : P.ncols);
    const int sb2 = __builtin_amdgcn_readfirstlane(nseg > 2 ? P.seg_start[2] : P.ncols);
    gptr<const float> usw[3], ubias[3];
    gptr<const int32_t> ucs[3];
    gptr<float> uout[3];
    int uldo[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const Seg& S = P.seg[k < nseg ? k : 0];
      usw[k] = uniform_ptr(S.sw);
      ucs[k] = uniform_ptr(S.cs);
      ubias[k] = uniform_ptr(S.bias);
      uout[k] = uniform_ptr(S.out);
      uldo[k] = __builtin_amdgcn_readfirstlane(S.ldo);
    }
    const bool in1 = cc >= sb1, in2 = cc >= sb2;
    const int n = cc - (in2 ? sb2 : (in1 ? sb1 : 0));
    const gptr<const float> sw = in2 ? usw[2] : (in1 ? usw[1] : usw[0]);
    const gptr<const int32_t> cs = in2 ? ucs[2] : (in1 ? ucs[1] : ucs[0]);
    const gptr<const float> bias = in2 ? ubias[2] : (in1 ? ubias[1] : ubias[0]);
    const gptr<float> out = in2 ? uout[2] : (in1 ? uout[1] : uout[0]);
    const int ldo = in2 ? uldo[2] : (in1 ? uldo[1] : uldo[0]);
    const bool resid = P.epi == EPI_RESID;
    const float swv = sw[n];
    const int csv = cs[n];
    const float bv = bias ? bias[n] : 0.f;
    float old[16];
    if (resid) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = min(mb + (r / 4) * 8 + half * 4 + r % 4, M - 1);
        old[r] = out[(size_t)m * ldo + n];
      }
    }
    // every row's value first (one wait for the residual inputs), then the
    // guarded stores
    float val[16];
    int at[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      at[r] = accb[r] + rz[r] * csv;
      float y = dequant(at[r], rs[r], swv);
      if (bias) y = y + bv;
      val[r] = resid ? old[r] + y : y;
    }
    asm volatile("" : "+v"(val[0]), "+v"(val[1]), "+v"(val[2]), "+v"(val[3]), "+v"(val[4]),
                 "+v"(val[5]), "+v"(val[6]), "+v"(val[7]), "+v"(val[8]), "+v"(val[9]),
                 "+v"(val[10]), "+v"(val[11]), "+v"(val[12]), "+v"(val[13]), "+v"(val[14]),
                 "+v"(val[15]));
    if (col < P.ncols) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = mb + (r / 4) * 8 + half * 4 + r % 4;
        if (m >= M) continue;
        out[(size_t)m * ldo + n] = val[r];
        if (acc_out) acc_out[(size_t)m * P.ncols + col] = at[r];
      }
    }
  }
  }
}

bool gemm_skinny_supported(int M, int K) { return M >= 1 && M < 128 && K % sk::SS == 0; }

constexpr int SK_MAX_SPLIT_TILES = 256;  // row tiles of a K-split launch

size_t gemm_skinny_ws_bytes() {
  // sum blocks of the tiles of a split launch, then the tile counters
  return (size_t)SK_MAX_SPLIT_TILES * 32 * sk::MAX_MB * sk::ROWS * 4 + SK_MAX_SPLIT_TILES * 4;
}

__global__ void k_zero_u32(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

hipError_t launch_zero_u32(hipStream_t st, uint32_t* p, int n) {
  hipLaunchKernelGGL(k_zero_u32, dim3(std::max(1, std::min(256, (n + 255) / 256))), dim3(256), 0, st,
                     p, n);
  return hipGetLastError();
}

hipError_t gemm_skinny_reset(hipStream_t st, void* scratch) {
  const int n = (int)(gemm_skinny_ws_bytes() / 4);
  hipLaunchKernelGGL(k_zero_u32, dim3(256), dim3(256), 0, st, (uint32_t*)scratch, n);
  return hipGetLastError();
}

size_t gemm_ws_bytes(size_t max_rows) {
  return gemm_skinny_ws_bytes() + (max_rows >= 128 ? gemm_big_split_ws_bytes() : 0);
}

hipError_t gemm_scratch_reset(hipStream_t st, void* scratch, size_t max_rows) {
  const int n = (int)(gemm_ws_bytes(max_rows) / 4);
  hipLaunchKernelGGL(k_zero_u32, dim3(256), dim3(256), 0, st, (uint32_t*)scratch, n);
  return hipGetLastError();
}

static hipError_t launch_gemm_skinny_rows(hipStream_t st, int M, int row0, int K,
                                          const int8_t* codes, const float* s, const int* z,
                                          int rows_per_seq, const Seg* segs, int nseg, Epi epi,
                                          int32_t* acc_out, void* scratch,
                                          int32_t* pout = nullptr, int* ks_out = nullptr);

hipError_t launch_gemm_skinny(hipStream_t st, int M, int K, const int8_t* codes, const float* s,
                              const int* z, int rows_per_seq, const Seg* segs, int nseg, Epi epi,
                              int32_t* acc_out, void* scratch) {
  using namespace sk;
  // more than 64 rows: one launch per 64 rows (the weights are streamed once
  // per launch; a few extra passes cost far less than a row-tiled GEMM with
  // a handful of workgroups)
  if (M > 32 * MAX_MB) {
    for (int r0 = 0; r0 < M; r0 += 32 * MAX_MB) {
      Seg sub[3];
      for (int i = 0; i < nseg; ++i) {
        sub[i] = segs[i];
        sub[i].out = segs[i].out + (size_t)r0 * segs[i].ldo;
      }
      int ncols = 0;
      for (int i = 0; i < nseg; ++i) ncols += segs[i].n;
      if (epi == EPI_SWIGLU) ncols = segs[0].n;
      const hipError_t e = launch_gemm_skinny_rows(
          st, min(32 * MAX_MB, M - r0), r0, K, codes + (size_t)r0 * K, s, z, rows_per_seq, sub, nseg, epi,
          acc_out ? acc_out + (size_t)r0 * ncols : nullptr, scratch);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  return launch_gemm_skinny_rows(st, M, 0, K, codes, s, z, rows_per_seq, segs, nseg, epi, acc_out,
                                 scratch);
}

template <int MB>
static hipError_t launch_sk(hipStream_t st, const GemmSkParams& P) {
  // one-time attribute set-up (a function-local static: initialised once,
  // thread-safe)
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)k_gemm_sk<MB>, hipFuncAttributeMaxDynamicSharedMemorySize, sk::Cfg<MB>::LDS);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(k_gemm_sk<MB>, dim3(P.tiles * P.ks), dim3(sk::NT), sk::Cfg<MB>::LDS, st, P);
  return hipGetLastError();
}

static hipError_t launch_gemm_skinny_rows(hipStream_t st, int M, int row0, int K,
                                          const int8_t* codes, const float* s, const int* z,
                                          int rows_per_seq, const Seg* segs, int nseg, Epi epi,
                                          int32_t* acc_out, void* scratch, int32_t* pout,
                                          int* ks_out) {
  using namespace sk;
  GemmSkParams P = {};
  P.M = M;
  P.row0 = row0;
  P.K = K;
  P.A = codes;
  P.qs = s;
  P.qz = z;
  P.rows_per_seq = rows_per_seq;
  P.nseg = nseg;
  P.epi = epi;
  P.acc_out = acc_out;
  P.seg_start[0] = 0;
  for (int i = 0; i < nseg; ++i) {
    P.seg[i] = segs[i];
    P.seg_start[i + 1] = P.seg_start[i] + segs[i].n;
  }
  P.ncols = (epi == EPI_SWIGLU) ? segs[0].n : P.seg_start[nseg];
  const int per_tile = epi == EPI_SWIGLU ? ROWS / 2 : ROWS;
  P.tiles = (P.ncols + per_tile - 1) / per_tile;
  const int nss = K / SS;
  // split K (at most 8 ways) until the launch has about one workgroup per
  // CU, with at least 2 steps per split (a split costs every workgroup its
  // atomic additions, so a launch that already covers the chip, such as the
  // 172 gate/up tiles of an 11008-wide MLP, is not split); launches of more
  // than SK_MAX_SPLIT_TILES tiles are not split
  int ks = 1;
  if (P.tiles <= SK_MAX_SPLIT_TILES)
    while (ks < 8 && P.tiles * ks * 2 <= 256 && nss / (ks * 2) >= 2) ks *= 2;
  P.nss = (nss + ks - 1) / ks;
  P.ks = (nss + P.nss - 1) / P.nss;
  P.part = (int32_t*)scratch;
  P.ctr = (uint32_t*)((char*)scratch + (size_t)SK_MAX_SPLIT_TILES * 32 * MAX_MB * ROWS * 4);
  P.pout = pout;
  if (ks_out) *ks_out = P.ks;
  return M > 32 ? launch_sk<2>(st, P) : launch_sk<1>(st, P);
}

bool gemm_rows_supported(int M, int K, Epi epi, int ncols) {
  return gemm_skinny_supported(M, K) && M <= 32 * sk::MAX_MB && epi != EPI_SWIGLU &&
         ncols >= 1 && row_epi_supported(ncols);
}

size_t gemm_rows_part_bytes(int M, int ncols) { return (size_t)8 * M * ncols * 4; }

hipError_t launch_gemm_rows(hipStream_t st, int M, int K, const int8_t* codes, const float* s,
                            const int* z, const Seg* segs, int nseg, Epi epi, int32_t* part,
                            const RowNorm* norm) {
  int ncols = 0;
  for (int i = 0; i < nseg; ++i) ncols += segs[i].n;
  if (!part || !gemm_rows_supported(M, K, epi, ncols) || (norm && (epi != EPI_RESID || nseg != 1)))
    return hipErrorInvalidValue;
  int ks = 0;
  hipError_t e = launch_gemm_skinny_rows(st, M, 0, K, codes, s, z, 1, segs, nseg, epi, nullptr,
                                         nullptr, part, &ks);
  if (e != hipSuccess) return e;
  return launch_row_epi(st, M, ks, part, s, z, segs, nseg, epi, norm);
}

}  // namespace ark

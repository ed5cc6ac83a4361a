// Large int8 x int8 -> int32 GEMM for prefill on gfx950 matrix cores
// (v_mfma_i32_32x32x32_i8), with the same dequantising epilogues as k_gemm
// (store (+bias), residual add, SwiGLU over paired gate/up columns).
//
// Tiles of BM x BN x BK (128 x 256 x 64 on 256 threads as 2 x 2 waves, or
// 256 x 256 x 128 on 512 threads as 4 x 2 waves), each wave 64 x 128 of
// 32x32 accumulators.  Operand tiles go from global memory straight into
// LDS with 16-byte LDS-DMA loads (no register staging), NS stages deep, so
// the loads of step k+NS-1 overlap the matrix work of step k; one barrier
// per K step.
//
// LDS tile layout: 64-byte rows; the 16-byte chunk c of row r sits at chunk
// position c ^ ((r >> 2) & 3), so the 16 lanes served together by a 16-byte
// read (16 consecutive rows, same chunk) cover all 64 banks of gfx950's LDS.
// The DMA writes 1 KiB per instruction at lane-contiguous positions; each
// lane picks the global (row, chunk) that belongs at its position.
//
// With 256 threads two workgroups share a CU (launch bounds 256 x 2), so
// one's epilogue and prologue overlap the other's main loop; with 512 one
// workgroup has the CU (and its LDS) alone.  Workgroup ids are dealt
// round-robin over the 8 XCDs, so the tile order gives each XCD a
// contiguous run of tiles (groups of 8 M-tiles, M fastest) and its L2 sees
// few distinct operand tiles at a time.
//
// Fragment layout: lane l supplies row (l % 32) of its A and of its B
// fragment, both with K bytes [16*(l/32), +16) of the 32-wide K substep; the
// 32x32 result sits in lane (j + 32*((i/4)%2)), register (i/8)*4 + i%4 for
// row i, column j.  A and B share the lane -> K assignment, so each output
// is the full sum over K whatever order the instruction walks it.
#include "common.hpp"
#include "kernels.hpp"

namespace ark {

constexpr int kBigSplitMaxTiles = 64;  // launches of at most this many tiles may split K

typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t2 __attribute__((ext_vector_type(8)));

struct Gemm2Params {
  int M, K, ncols, epi, rows_per_seq, nseg, tiles_m, tiles;
  const int8_t* A;
  const float* qs;
  const int* qz;
  Seg seg[3];
  int seg_start[4];
  int32_t* acc_out;
  SeqStats stats;  // EPI_SWIGLU: per-sequence min/max of the output (cur == nullptr: off)
  // bf16 operands (the instantiation with BF): A and the weight rows are bf16
  // matrices read as bytes (K = 2 x the element count), the epilogue is
  // bf_out / bf_swiglu over these segments
  BSeg bs[3];
  int bepi;
  // K split over ks workgroups per tile (ks > 1 only for the int8 GEMM of a
  // launch with few tiles): nks K steps each; each split adds its int32
  // sums into the tile's block of part (device-scope atomics), and a second
  // kernel reads the totals, clears the blocks and runs the epilogue
  int ks, nks;
  int32_t* part;  // [tiles][BM * BN], zero between launches
};

__device__ __forceinline__ void dma16(const int8_t* src, int8_t* lds_base) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                   (void __attribute__((address_space(3)))*)lds_base, 16, 0, 0);
}

// s_waitcnt vmcnt(n) for a compile-time n, expcnt/lgkmcnt untouched
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Epilogue of one BM x BN tile held as FM x FN 32x32 accumulators per wave
// (wave (wm, wn) owns rows wm * 64 + [0, 64) and columns wn * 128 + [0,
// 128)): dequantisation, bias, residual add or SwiGLU, and for SwiGLU the
// per-sequence range of the output into P.stats (replica rep).
template <int FM, int FN>
__device__ __forceinline__ void g2_epilogue(const Gemm2Params& P, i32x16 (&acc)[FM][FN], int m0,
                                            int nb, int wm, int wn, int lane, int rep) {
  constexpr int RW = FM * 32;
  const bool swiglu = P.epi == EPI_SWIGLU, resid = P.epi == EPI_RESID;
  const int lr = lane & 31, lc = lane >> 5;
  const int rps = P.rows_per_seq;
  // Row i of a 32x32 block is in register (i/8)*4 + i%4 of lanes with
  // (l/32) == (i/4)%2 (every index below is a compile-time constant, so the
  // accumulators stay in registers).  Every parameter and every residual
  // input is requested in one batch before the first is used: a kernel that
  // keeps operand loads in flight behind the epilogue pays one wait for the
  // batch, not one per request.  Segment fields are taken as wave-uniform
  // values (a per-lane choice between parameter-block fields would become a
  // vector load of the parameter block).
  const int nseg = P.nseg;
  const int sb1 = __builtin_amdgcn_readfirstlane(nseg > 1 ? P.seg_start[1] : P.ncols);
  const int sb2 = __builtin_amdgcn_readfirstlane(nseg > 2 ? P.seg_start[2] : P.ncols);
  struct {
    gptr<const float> sw[3];
    gptr<const int32_t> cs[3];
    gptr<const float> bias[3];
    gptr<float> out[3];
    int ldo[3];
  } U;
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const Seg& S = P.seg[k < nseg ? k : 0];
    U.sw[k] = uniform_ptr(S.sw);
    U.cs[k] = uniform_ptr(S.cs);
    U.bias[k] = uniform_ptr(S.bias);
    U.out[k] = uniform_ptr(S.out);
    U.ldo[k] = __builtin_amdgcn_readfirstlane(S.ldo);
  }
  const gptr<const float> qs = uniform_ptr(P.qs);
  const gptr<const int> qz = uniform_ptr(P.qz);
  const gptr<int32_t> acc_out = uniform_ptr(P.acc_out);
  float csw[FN], cbias[FN], usw[FN / 2];
  int ccs[FN], ucs[FN / 2];
  gptr<float> cout[FN];
  int cldo[FN];
  bool cok[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    cbias[j] = 0.f;
    if (swiglu) {
      if (j % 2 == 0) {
        const int n = nb + (wn * (FN / 2) + j / 2) * 32 + lr;
        const int nn = min(n, P.ncols - 1);
        cok[j] = n < P.ncols;
        csw[j] = U.sw[0][nn];
        ccs[j] = U.cs[0][nn];
        usw[j / 2] = U.sw[1][nn];
        ucs[j / 2] = U.cs[1][nn];
        cout[j] = U.out[0] + nn;
        cldo[j] = U.ldo[0];
      }
    } else {
      const int col = nb + wn * (FN * 32) + j * 32 + lr;
      const int cc = min(col, P.ncols - 1);
      const bool in1 = cc >= sb1, in2 = cc >= sb2;
      const int n = cc - (in2 ? sb2 : (in1 ? sb1 : 0));
      const gptr<const float> sw = in2 ? U.sw[2] : (in1 ? U.sw[1] : U.sw[0]);
      const gptr<const int32_t> cs = in2 ? U.cs[2] : (in1 ? U.cs[1] : U.cs[0]);
      const gptr<const float> bias = in2 ? U.bias[2] : (in1 ? U.bias[1] : U.bias[0]);
      const gptr<float> out = in2 ? U.out[2] : (in1 ? U.out[1] : U.out[0]);
      cldo[j] = in2 ? U.ldo[2] : (in1 ? U.ldo[1] : U.ldo[0]);
      cok[j] = col < P.ncols;
      csw[j] = sw[n];
      ccs[j] = cs[n];
      if (bias) cbias[j] = bias[n];
      cout[j] = out + n;
    }
  }
  // per group (i, q) of 4 rows: the parameters of the first row's sequence
  // (rows past its end, where a sequence starts inside the group, load their
  // own below)
  const int rbase = m0 + wm * RW + lc * 4;
  float rs[FM][4];
  int rz[FM][4], rnext[FM][4];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int b = min(rbase + i * 32 + q * 8, P.M - 1) / rps;
      rnext[i][q] = (b + 1) * rps;
      rs[i][q] = qs[b];
      rz[i][q] = 128 - qz[b];
    }
  // SwiGLU outputs' min / max per row of this lane (neutral where no output)
  float elo[FM][16], ehi[FM][16];
  // rows per batch of requests: 4, or all 16 of a block where a wave holds
  // only one or two 32x32 blocks (the separate epilogue of a K-split launch,
  // whose chain of dependent loads is its whole run time)
  constexpr int VB = FM * FN <= 2 ? 16 : 4;
  const SwigluK SK = swiglu_consts();
#pragma clang loop unroll(full)
  for (int i = 0; i < FM; ++i) {
#pragma clang loop unroll(full)
   for (int vh = 0; vh < 16; vh += VB) {
    // residual inputs of these VB rows, all requested before any store
    float old[VB][FN];
    if (resid) {
#pragma clang loop unroll(full)
      for (int v = vh; v < vh + VB; ++v) {
        const int row = min(rbase + i * 32 + (v >> 2) * 8 + (v & 3), P.M - 1);
#pragma clang loop unroll(full)
        for (int j = 0; j < FN; ++j) old[v - vh][j] = cout[j][(size_t)row * cldo[j]];
      }
    }
    if (swiglu) {
      // the VB rows' values first, with no branch between them (independent
      // fp64 chains the scheduler can interleave), then the guarded stores
      float sv[VB];
      int zv[VB];
#pragma clang loop unroll(full)
      for (int v = vh; v < vh + VB; ++v) {
        const int row = rbase + i * 32 + (v >> 2) * 8 + (v & 3);
        float s = rs[i][v >> 2];
        int zc = rz[i][v >> 2];
        if (row < P.M && row >= rnext[i][v >> 2]) {
          const int b = row / rps;
          s = qs[b];
          zc = 128 - qz[b];
        }
        sv[v - vh] = s;
        zv[v - vh] = zc;
      }
      float y[VB][FN / 2];
      int agc[VB][FN / 2];
#pragma clang loop unroll(full)
      for (int v = vh; v < vh + VB; ++v)
#pragma clang loop unroll(full)
        for (int j = 0; j < FN; j += 2) {
          agc[v - vh][j / 2] = acc[i][j][v] + zv[v - vh] * ccs[j];
          const float g = dequant(agc[v - vh][j / 2], sv[v - vh], csw[j]);
          const float u = dequant(acc[i][j + 1][v] + zv[v - vh] * ucs[j / 2], sv[v - vh], usw[j / 2]);
          y[v - vh][j / 2] = swiglu_f64(g, u, SK);
        }
      // computed here for every lane (not sunk into the guarded stores)
#pragma clang loop unroll(full)
      for (int v = 0; v < VB; ++v)
#pragma clang loop unroll(full)
        for (int j = 0; j < FN / 2; ++j) asm volatile("" : "+v"(y[v][j]));
#pragma clang loop unroll(full)
      for (int v = vh; v < vh + VB; ++v) {
        elo[i][v] = INFINITY;
        ehi[i][v] = -INFINITY;
        const int row = rbase + i * 32 + (v >> 2) * 8 + (v & 3);
        if (row >= P.M) continue;
#pragma clang loop unroll(full)
        for (int j = 0; j < FN; j += 2) {
          if (cok[j]) {
            const float yv = y[v - vh][j / 2];
            cout[j][(size_t)row * cldo[j]] = yv;
            elo[i][v] = fminf(elo[i][v], yv);
            ehi[i][v] = fmaxf(ehi[i][v], yv);
            if (acc_out)
              acc_out[(size_t)row * P.ncols + nb + (wn * (FN / 2) + j / 2) * 32 + lr] = agc[v - vh][j / 2];
          }
        }
      }
      continue;
    }
#pragma clang loop unroll(full)
    for (int v = vh; v < vh + VB; ++v) {
      elo[i][v] = INFINITY;
      ehi[i][v] = -INFINITY;
      const int row = rbase + i * 32 + (v >> 2) * 8 + (v & 3);
      if (row >= P.M) continue;
      float s = rs[i][v >> 2];
      int zc = rz[i][v >> 2];
      if (row >= rnext[i][v >> 2]) {
        const int b = row / rps;
        s = qs[b];
        zc = 128 - qz[b];
      }
      {
#pragma clang loop unroll(full)
        for (int j = 0; j < FN; ++j) {
          if (cok[j]) {
            const int at = acc[i][j][v] + zc * ccs[j];
            float y = dequant(at, s, csw[j]);
            y = y + cbias[j];
            const gptr<float> o = cout[j] + (size_t)row * cldo[j];
            *o = resid ? old[v - vh][j] + y : y;
            if (acc_out) acc_out[(size_t)row * P.ncols + nb + wn * (FN * 32) + j * 32 + lr] = at;
          }
        }
      }
    }
   }
  }
  if (swiglu && P.stats.cur) {
    // fold this wave's 64 rows into their sequences (one or two unless
    // sequences are shorter than the wave's rows): lanes' values of rows in
    // sequence b, then the wave's min / max, one atomic pair per sequence
    const int r0 = m0 + wm * RW;
    const int rl = min(r0 + RW, P.M) - 1;
    for (int b = r0 / rps; b <= rl / rps; ++b) {
      const int ra = b * rps, rb = ra + rps;
      float lo = INFINITY, hi = -INFINITY;
#pragma clang loop unroll(full)
      for (int i = 0; i < FM; ++i)
#pragma clang loop unroll(full)
        for (int v = 0; v < 16; ++v) {
          const int row = rbase + i * 32 + (v >> 2) * 8 + (v & 3);
          const bool in = row >= ra && row < rb;
          lo = fminf(lo, in ? elo[i][v] : INFINITY);
          hi = fmaxf(hi, in ? ehi[i][v] : -INFINITY);
        }
      lo = wave_min(lo);
      hi = wave_max(hi);
      if (lane == 0) stats_fold(P.stats, rep, b, lo, hi);
    }
  }
}

// BM x BN x BK tiles on NTH / 64 waves arranged (BM / 64) x 2: every wave
// owns a 64 x BN/2 block (2 x BN/64 accumulators of 32 x 32).  Tile rows are
// BK bytes in LDS; one LDS-DMA instruction moves 1024 / BK rows, each lane
// the 16-byte chunk that belongs at its LDS position (chunk c of row r sits
// at chunk c ^ ((r / (256 / BK)) % (BK / 16)), so the 16 rows of one
// fragment read fall on all 64 banks).  128-byte rows make every request a
// whole cache line, which streams markedly faster than 64-byte halves.
// Epilogue of the bf16 instantiation: fp32 sums of bf16 products, rounded
// to bf16 by the variant's rules (bf_out), SwiGLU pairs by bf_swiglu.
template <int FM, int FN>
__device__ __forceinline__ void bf16_epilogue(const Gemm2Params& P, f32x16 (&acc)[FM][FN], int m0,
                                              int nb, int wm, int wn, int lane) {
  constexpr int RW = FM * 32;
  const bool swiglu = P.epi == EPI_SWIGLU;
  const int lr = lane & 31, lc = lane >> 5;
  const int rbase = m0 + wm * RW + lc * 4;
  // output address, row stride and bias of each of this lane's columns,
  // chosen once by selects (all indices into acc below are compile-time
  // constants, so it stays in registers)
  const int sb1 = P.nseg > 1 ? P.seg_start[1] : P.ncols;
  const int sb2 = P.nseg > 2 ? P.seg_start[2] : P.ncols;
  const int epi = P.bepi;
  char* cout[FN];
  int cldo[FN];
  float cb[FN];
  bool cok[FN];
#pragma clang loop unroll(full)
  for (int j = 0; j < FN; ++j) {
    const int col = swiglu ? nb + (wn * (FN / 2) + j / 2) * 32 + lr : nb + wn * (FN * 32) + j * 32 + lr;
    cok[j] = col < P.ncols;
    const int cc = min(col, P.ncols - 1);
    const bool in1 = cc >= sb1, in2 = cc >= sb2;
    const int n = cc - (in2 ? sb2 : (in1 ? sb1 : 0));
    const BSeg& S0 = P.bs[0];
    const BSeg& S1 = P.bs[1];
    const BSeg& S2 = P.bs[2];
    char* base = (char*)(in2 ? S2.out : (in1 ? S1.out : S0.out));
    const uint16_t* bias = in2 ? S2.bias : (in1 ? S1.bias : S0.bias);
    cldo[j] = in2 ? S2.ldo : (in1 ? S1.ldo : S0.ldo);
    cout[j] = base + (size_t)n * (epi == BE_F32 ? 4 : 2);
    cb[j] = (bias && !swiglu && epi != BE_F32) ? bf2f(bias[n]) : 0.0f;
  }
#pragma clang loop unroll(full)
  for (int i = 0; i < FM; ++i)
#pragma clang loop unroll(full)
    for (int v = 0; v < 16; ++v) {
      const int row = rbase + i * 32 + (v >> 2) * 8 + (v & 3);
      if (row < P.M) {
        if (swiglu) {
#pragma clang loop unroll(full)
          for (int j = 0; j < FN; j += 2)
            if (cok[j])
              ((uint16_t*)cout[j])[(size_t)row * cldo[j]] = bf_swiglu(acc[i][j][v], acc[i][j + 1][v]);
        } else if (epi == BE_F32) {
#pragma clang loop unroll(full)
          for (int j = 0; j < FN; ++j)
            if (cok[j]) ((float*)cout[j])[(size_t)row * cldo[j]] = acc[i][j][v];
        } else {
#pragma clang loop unroll(full)
          for (int j = 0; j < FN; ++j)
            if (cok[j]) {
              uint16_t* o = (uint16_t*)cout[j] + (size_t)row * cldo[j];
              const float y = acc[i][j][v] + cb[j];
              *o = epi == BE_RESID ? f2bf(bf2f(*o) + rbf(y)) : f2bf(y);
            }
        }
      }
    }
}

// First row and column of tile t: tiles walk groups of 8 m-tiles x all
// n-tiles, m fastest (SwiGLU tiles hold BN / 2 output columns).
template <int BM, int BN>
__device__ __forceinline__ void tile_origin(const Gemm2Params& P, int t, int& m0, int& nb) {
  const int tiles_n = P.tiles / P.tiles_m;
  const int grp = t / (8 * tiles_n);
  const int gm = min(8, P.tiles_m - grp * 8);
  const int tg = t - grp * 8 * tiles_n;
  m0 = (grp * 8 + tg % gm) * BM;
  nb = (tg / gm) * (P.epi == EPI_SWIGLU ? BN / 2 : BN);
}

// SPLIT: one K range of a K-split launch (P.ks ranges of P.nks steps per
// tile): the int32 sums go to the tile's block of P.part and
// k_gemm_big_epi runs the epilogue afterwards.
template <int BM, int BN, int BK, int NS, int NTH, bool BF = false, bool SPLIT = false>
__global__ __launch_bounds__(NTH, NTH == 256 ? 2 : 1) void k_gemm_big(Gemm2Params P) {
  constexpr int NWV = NTH / 64;             // waves
  constexpr int RW = 64;                    // rows per wave
  static_assert(NWV * RW == BM * 2, "(BM / 64) x 2 waves");
  constexpr int FM = RW / 32;               // 32-row blocks per wave
  constexpr int FN = BN / 64;               // 32-column blocks per wave
  constexpr int KK = BK / 32;               // 32-wide K substeps per step
  constexpr int CPR = BK / 16;              // 16-byte chunks per tile row
  constexpr int RPI = 1024 / BK;            // tile rows per DMA instruction
  constexpr int RPL = 256 / BK;             // tile rows per 256 bytes (all banks)
  constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK, STAGE = A_BYTES + B_BYTES;
  constexpr int A_INS = A_BYTES / 1024 / NWV, B_INS = B_BYTES / 1024 / NWV;  // per wave per stage
  static_assert(A_INS * NWV * 1024 == A_BYTES && B_INS * NWV * 1024 == B_BYTES, "DMA split");
  static_assert(FN % 2 == 0 && (BK == 64 || BK == 128), "tile shape");
  constexpr int INS = A_INS + B_INS;
  extern __shared__ __align__(16) int8_t lds[];
  auto sw = [](int r, int c) { return r * BK + ((c ^ ((r / RPL) % CPR)) << 4); };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const bool swiglu = P.epi == EPI_SWIGLU;

  // XCD-aware tile order: the workgroups of one XCD (bid % 8) take a
  // contiguous run of tiles, and runs walk groups of 8 m-tiles x all
  // n-tiles m-fastest, so the ~64 concurrent workgroups of an XCD share
  // about 8 activation and 8 weight tiles in their L2.
  if (P.stats.cur) stats_clear_other(P.stats);
  static_assert(!(BF && SPLIT), "K split: int8 only");
  const int ks = SPLIT ? P.ks : 1;
  const int per = (P.tiles * ks + 7) / 8;
  const int u = (blockIdx.x % 8) * per + blockIdx.x / 8;  // split-major: an XCD's run
  if (u >= P.tiles * ks) return;                           // is mostly one split
  const int t = u % P.tiles, split = u / P.tiles;
  int m0, nb;
  tile_origin<BM, BN>(P, t, m0, nb);
  const int K = P.K;
  // this workgroup's K steps: kb .. kb + nk - 1
  const int kb = SPLIT ? split * P.nks : 0;
  const int nk = SPLIT ? min(P.nks, K / BK - kb) : K / BK;

  // per-lane DMA sources: A instructions wave*A_INS + i, B instructions
  // wave*B_INS + i; instruction u covers rows RPI u .. RPI u + RPI - 1
  const int8_t* asrc[A_INS];
#pragma unroll
  for (int i = 0; i < A_INS; ++i) {
    const int r = RPI * (wave * A_INS + i) + lane / CPR;
    const int c = (lane % CPR) ^ ((r / RPL) % CPR);
    asrc[i] = P.A + (size_t)min(m0 + r, P.M - 1) * K + 16 * c;
  }
  const int8_t* bsrc[B_INS];
#pragma unroll
  for (int i = 0; i < B_INS; ++i) {
    const int r = RPI * (wave * B_INS + i) + lane / CPR;
    const int c = (lane % CPR) ^ ((r / RPL) % CPR);
    const int8_t* w;
    if (swiglu) {
      const int blk = r >> 5;
      const int n = min(nb + (blk >> 1) * 32 + (r & 31), P.ncols - 1);
      w = ((blk & 1) ? P.seg[1].w : P.seg[0].w) + (size_t)n * K;
    } else {
      const int col = min(nb + r, P.ncols - 1);
      int s = 0;
      while (s + 1 < P.nseg && col >= P.seg_start[s + 1]) ++s;
      w = P.seg[s].w + (size_t)(col - P.seg_start[s]) * K;
    }
    bsrc[i] = w + 16 * c;
  }

  auto issue = [&](int st, int buf) {
    int8_t* base = lds + buf * STAGE;
    const int k0 = (kb + st) * BK;
#pragma unroll
    for (int i = 0; i < A_INS; ++i) dma16(asrc[i] + k0, base + (wave * A_INS + i) * 1024);
#pragma unroll
    for (int i = 0; i < B_INS; ++i)
      dma16(bsrc[i] + k0, base + A_BYTES + (wave * B_INS + i) * 1024);
  };

  using AccT = typename std::conditional<BF, f32x16, i32x16>::type;
  AccT acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) issue(s, s);

  const int lr = lane & 31, lc = lane >> 5;
  for (int ks = 0; ks < nk; ++ks) {
    // this wave's loads of step ks are done once at most the later issued
    // stages' loads are outstanding
    if (NS == 3 && ks + 1 < nk)
      wait_vm<INS>();
    else
      wait_vm<0>();
    // every wave's step-ks loads are in LDS and every wave is done reading
    // the buffer refilled next; a plain barrier (no wait for the loads that
    // stay in flight)
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
    __builtin_amdgcn_s_barrier();
    if (ks + NS - 1 < nk) issue(ks + NS - 1, (ks + NS - 1) % NS);
    const int8_t* As = lds + (ks % NS) * STAGE;
    const int8_t* Bs = As + A_BYTES;
    // the K substeps' fragments are read up front into separate registers,
    // so no read waits for a matrix instruction still using its sources
    i32x4 fa[KK][FM], fb[KK][FN];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int c = 2 * kk + lc;
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[kk][i] = *(const i32x4*)(As + sw(wm * RW + i * 32 + lr, c));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        fb[kk][j] = *(const i32x4*)(Bs + sw(wn * (BN / 2) + j * 32 + lr, c));
    }
    // pin all fragments live at once (keeps the reads ahead of the MFMAs)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(fa[kk][i]));
#pragma unroll
      for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(fb[kk][j]));
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          if constexpr (BF)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t2, fa[kk][i]), __builtin_bit_cast(bf16x8_t2, fb[kk][j]),
                acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[kk][i], fb[kk][j], acc[i][j], 0, 0, 0);
  }

  if constexpr (SPLIT) {
    // this K range's sums into the tile's block (device-scope atomics,
    // lane-contiguous words); k_gemm_big_epi applies the epilogue to the
    // totals after the launch
    int32_t* blk = P.part + (size_t)t * BM * BN + (size_t)wave * FM * FN * 16 * 64 + lane;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          __hip_atomic_fetch_add(blk + ((i * FN + j) * 16 + v) * 64, acc[i][j][v], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if constexpr (BF)
    bf16_epilogue<FM, FN>(P, acc, m0, nb, wm, wn, lane);
  else
    g2_epilogue<FM, FN>(P, acc, m0, nb, wm, wn, lane, blockIdx.x * NWV + wave);
}

// The epilogue of a K-split launch: one workgroup per tile, one wave per
// 32 rows x 64 columns (two 32x32 blocks: a SwiGLU pair, or two adjacent
// store/residual blocks) of the k_gemm_big wave that summed them, so each
// wave's chain of dependent loads is short.  It reads the tile's int32
// totals from its block of P.part (in k_gemm_big's accumulator layout) and
// clears the block for the next launch.
template <int BM, int BN, int NTH>
struct EpiShape {
  static constexpr int NWV = NTH / 64, RW = 2 * BM / NWV, FM = RW / 32, FN = BN / 64;
  static constexpr int SUB = FM * (FN / 2);                 // epilogue waves per summing wave
  static constexpr int EW = NWV * SUB;                      // epilogue waves per tile
  static constexpr int EPW = EW > 8 ? 8 : EW;               // of them per workgroup
  static_assert(EW % EPW == 0, "epilogue waves");
};

template <int BM, int BN, int NTH>
__global__ __launch_bounds__((EpiShape<BM, BN, NTH>::EPW * 64)) void k_gemm_big_epi(Gemm2Params P) {
  using E = EpiShape<BM, BN, NTH>;
  constexpr int NWV = E::NWV, RW = E::RW, FM = E::FM, FN = E::FN, SUB = E::SUB;
  const int tid = threadIdx.x, lane = tid & 63, ew = blockIdx.y * E::EPW + (tid >> 6);
  const int wave = ew / SUB, i = (ew % SUB) / (FN / 2), j0 = 2 * ((ew % SUB) % (FN / 2));
  const int wm = wave >> 1, wn = wave & 1;
  const int t = blockIdx.x;
  int m0, nb;
  tile_origin<BM, BN>(P, t, m0, nb);
  int32_t* blk = P.part + (size_t)t * BM * BN + (size_t)wave * FM * FN * 16 * 64 + lane;
  i32x16 acc[1][2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[0][jj][v] = blk[((i * FN + j0 + jj) * 16 + v) * 64];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int v = 0; v < 16; ++v) blk[((i * FN + j0 + jj) * 16 + v) * 64] = 0;
  // the two blocks as a one-wave 32 x 64 tile: rows m0 + wm RW + 32 i, and
  // columns nb + wn (BN / 2) + 32 j0 (SwiGLU: output columns nb + (wn FN / 2
  // + j0 / 2) 32, the pair j0, j0 + 1)
  const int m1 = m0 + wm * RW + 32 * i;
  const int n1 = P.epi == EPI_SWIGLU ? nb + (wn * (FN / 2) + j0 / 2) * 32 : nb + wn * (BN / 2) + 32 * j0;
  g2_epilogue<1, 2>(P, acc, m1, n1, 0, 0, lane, t * E::EW + ew);
}

template <int BM, int BN, int BK, int NS, int NTH, bool BF = false>
static hipError_t launch_big(hipStream_t st, Gemm2Params P) {
  constexpr int bytes = NS * (BM + BN) * BK;
  // one-time attribute set-up (a function-local static: initialised once,
  // thread-safe)
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)k_gemm_big<BM, BN, BK, NS, NTH, BF>, hipFuncAttributeMaxDynamicSharedMemorySize,
      bytes);
  if (attr != hipSuccess) return attr;
  const int tn = P.epi == EPI_SWIGLU ? BN / 2 : BN;
  P.tiles_m = (P.M + BM - 1) / BM;
  P.tiles = P.tiles_m * ((P.ncols + tn - 1) / tn);
  // a launch of few tiles (a single 387-row prompt: 32 tiles for o and down)
  // would leave most CUs idle: split K (at most 8 ways, at least 4 steps per
  // split) until about 256 workgroups run
  P.ks = 1;
  if (!BF && P.part && P.tiles <= kBigSplitMaxTiles) {
    const int nkt = P.K / BK;
    int ks = 1;
    while (ks < 8 && P.tiles * ks * 2 <= 256 && nkt / (ks * 2) >= 4) ks *= 2;
    P.nks = (nkt + ks - 1) / ks;
    P.ks = (nkt + P.nks - 1) / P.nks;  // every split non-empty
  }
  const int grid = 8 * ((P.tiles * P.ks + 7) / 8);
  if constexpr (!BF) {
    if (P.ks > 1) {
      static const hipError_t attr_s = hipFuncSetAttribute(
          (const void*)k_gemm_big<BM, BN, BK, NS, NTH, false, true>,
          hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
      if (attr_s != hipSuccess) return attr_s;
      hipLaunchKernelGGL((k_gemm_big<BM, BN, BK, NS, NTH, false, true>), dim3(grid), dim3(NTH), bytes,
                         st, P);
      using E = EpiShape<BM, BN, NTH>;
      hipLaunchKernelGGL((k_gemm_big_epi<BM, BN, NTH>), dim3(P.tiles, E::EW / E::EPW), dim3(E::EPW * 64),
                         0, st, P);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((k_gemm_big<BM, BN, BK, NS, NTH, BF>), dim3(grid), dim3(NTH), bytes, st, P);
  return hipGetLastError();
}

bool gemm_big_supported(int M, int K) { return M >= 128 && K % 64 == 0; }

size_t gemm_big_split_ws_bytes() {
  return (size_t)kBigSplitMaxTiles * 256 * 256 * 4;
}

hipError_t launch_gemm_big(hipStream_t st, int M, int K, const int8_t* codes, const float* s,
                           const int* z, int rows_per_seq, const Seg* segs, int nseg, Epi epi,
                           int32_t* acc_out, const SeqStats* stats, void* split_ws) {
  Gemm2Params P = {};
  if (split_ws) P.part = (int32_t*)split_ws;
  if (stats && epi == EPI_SWIGLU) P.stats = *stats;
  P.M = M;
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
  // The main loop is bound by the operand bytes a CU keeps in flight over
  // their latency (LDS holds the stages).  Store and residual epilogues are
  // light: one workgroup per CU with 256 x 256 tiles and whole 128-byte K
  // steps in two stages (256 int8 ops per operand byte, whole-line loads)
  // is fastest there, once the rows fill enough tiles (16x387 prefill: q|k|v
  // 60 -> 54 us, o 68 -> 64.5 us, down 201 -> 179 us per layer).  The SwiGLU
  // epilogue's fp64 gate is as long as a good part of the main loop, so there
  // two workgroups share each CU (one's epilogue overlaps the other's main
  // loop): 128 x 256 tiles with 64-byte K steps in three stages.  Measured
  // alternatives, slower for both: 256 x 256 with 64-byte steps in three or
  // four stages, 256 x 128 with 128-byte steps in three stages, 128 x 256 or
  // 128 x 128 with 128-byte steps in two stages.
  if (epi != EPI_SWIGLU && M >= 1024) return launch_big<256, 256, 128, 2, 512>(st, P);
  return launch_big<128, 256, 64, 3, 256>(st, P);
}

// The bf16 variant's GEMM at 128+ rows on the same tiles: x [M][K] bf16
// (row stride K), weight rows bf16; K counted in bytes for the byte-level
// staging (one 32-byte K substep is one 32x32x16 bf16 instruction).
hipError_t launch_gemm_big_bf16(hipStream_t st, int M, int K, const uint16_t* x, const BSeg* segs,
                                int nseg, int epi) {
  Gemm2Params P = {};
  P.M = M;
  P.K = 2 * K;
  P.A = (const int8_t*)x;
  P.rows_per_seq = M;
  P.nseg = nseg;
  P.epi = epi == BE_SWIGLU ? EPI_SWIGLU : EPI_STORE;
  P.bepi = epi;
  P.seg_start[0] = 0;
  for (int i = 0; i < nseg; ++i) {
    P.seg[i].w = (const int8_t*)segs[i].w;
    P.seg[i].n = segs[i].n;
    P.bs[i] = segs[i];
    P.seg_start[i + 1] = P.seg_start[i] + segs[i].n;
  }
  P.ncols = (epi == BE_SWIGLU) ? segs[0].n : P.seg_start[nseg];
  if (epi != BE_SWIGLU && M >= 1024) return launch_big<256, 256, 128, 2, 512, true>(st, P);
  return launch_big<128, 256, 64, 3, 256, true>(st, P);
}

}  // namespace ark

// Persistent decode step for the ARK-ASR-3B geometry at batch 1.
//
// One launch runs all 36 layers and the LM head of a decode
// token (model card "ark-asr-3b-onnx", sections Shapes and Files: hidden
// 2048, 16 query / 2 KV heads of 128, int8 per-channel MatMuls with dynamic
// activation quantisation, full static-cache attention, int8 LM head).
//
// Why one kernel: a batch-1 token streams 3.09 GB of int8 weights but has
// five all-to-all dependencies per layer (each MatMul needs the whole
// quantised input vector).  Separate kernels pay launch gaps and short,
// latency-bound streams; here the weight stream runs ahead of the
// dependency chain instead.
//
// Work split: 256 workgroups x 16 waves.  In the layers every wave streams
// weights: it owns fixed output rows (or, for the down projection, half a
// row) of each phase and issues the loads of a phase's weights into
// registers ahead of the phase's input.  The attention of a token runs on at
// most 16 workgroups (items of 4 query heads of one KV head over a share of
// the live 64-key chunks); the gate/up rows are spread over the other
// workgroups only, which stream them while the attention runs.
//
// Data exchange between workgroups (which sit on different XCDs with
// separate L2s) uses 64-bit words (fp32 value | tag << 32) written with
// device-scope stores and read with device-scope loads, so no cache
// write-back/invalidate fence is needed.  The tag is a per-launch epoch kept
// in the workspace, so words of earlier launches never match.  Every wait is
// bounded: on time-out the kernel records an error and runs to completion.
//
// Residency: the exchanges need all 256 workgroups on the device at once.
// One fits per CU (decode_mega_init checks it), so an ordinary launch on a
// GPU that is not running another kernel places them all at once; a
// kernel on another stream that holds CUs only delays the late
// workgroups, and a delay beyond the wait bound ends the step with the
// time-out error.  ARK_DECODE_LAUNCH=cooperative selects the cooperative
// launch, which guarantees residency at about 20 us more per launch.
#include <float.h>
#include <limits.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace ark {
namespace mk {

constexpr int H = 2048, NH = 16, NKV = 2, D = kHeadDim, Q = NH * D, KVD = NKV * D, I = 11008;
constexpr int G = NH / NKV;               // query heads per KV head
constexpr int NQKV = Q + 2 * KVD;         // 2560 q|k|v rows
constexpr int NWG = 256, NT = 1024, NW = 16, NS = NW - 1;
constexpr int KEYS = 64;                  // cache rows per attention chunk
constexpr int HPI = 4;                    // query heads per attention item
constexpr int HH = G / HPI;               // items side by side per KV head (head groups)
constexpr int NIH = 4;                    // items per (KV head, head group) along the cache
constexpr int NATT = NKV * HH * NIH;      // workgroups that may hold an attention item
constexpr int PART = 2 + D;               // fp64 words of one partial softmax state
constexpr uint32_t SPIN_LIMIT = 1u << 15;  // ~30-60 ms per wait: a failure ends in seconds
// The error word of a launch and the bound of its waits (rounds): a wait
// that gives up sets a bit of the word and the kernel runs to completion.
struct Err {
  uint32_t* word;
  uint32_t limit;
};
constexpr int NREP = 8;                   // replicas of each broadcast vector (one per XCD)
constexpr unsigned long long MAGIC = 0x41524b5f58434831ull;

// per-layer exchange words: q|k|v once (read by the attention workgroups),
// every vector that all workgroups read in NREP replicas, so each replica is
// read by the 32 workgroups of one XCD instead of all 256 reading one copy
// The SwiGLU vector is exchanged already quantised, in two rounds: each
// producer workgroup's min and max (OFF_AMM, 2 words per producer), then its
// codes packed 4 per word (OFF_AC, word k = codes of rows 4k..4k+3).
constexpr int OFF_QKV = 0, OFF_X0 = NQKV, OFF_ATT = OFF_X0 + NREP * H,
              OFF_X1 = OFF_ATT + NREP * Q, OFF_AMM = OFF_X1 + NREP * H,
              OFF_AC = OFF_AMM + NREP * 2 * NWG, XCH_LAYER = OFF_AC + NREP * (I / 4);
static_assert(I % 4 == 0, "packed codes");

// rows per workgroup of the q|k|v, o and down phases (wave s owns row s of
// q|k|v and o; waves 2r and 2r+1 split down row r); the gate/up rows are
// spread at run time over the workgroups without attention work, at most
// GU_ROWS per wave
constexpr int R_QKV = NQKV / NWG, R_O = H / NWG, R_D = H / NWG;
static_assert(R_QKV * NWG == NQKV && R_O * NWG == H && R_D * NWG == H, "row split");
static_assert(R_QKV <= NW && R_O <= NW && 2 * R_D == NW, "rows per wave");
constexpr int GU_ROWS = 3;
static_assert(GU_ROWS <= 4, "SwiGLU rows of a wave sit on lanes of one DPP quad");
static_assert((((I + (NWG - NATT) - 1) / (NWG - NATT) + 3) & ~3) <= GU_ROWS * NW, "gate/up rows");
constexpr int STAGE = 112 * 1024;             // LDS staging bytes
constexpr int GU_LDS = 16 * 1024;             // stage offset of the gate/up units in LDS
// down projection: waves 8..15 ("loaders") each own one of the 8 rows (11
// units of 1 KiB, the last one partial), all in LDS: units 8..10 at DN_LDS +
// 3 KiB x loader (requested early, while the attention runs), units 0..7 at
// DN_HEAD + 8 KiB x loader (requested once the gate/up units in LDS are
// used, so they are in before the SwiGLU codes are awaited); waves 0..7
// poll and unpack its input
constexpr int D_UNITS = (I + 1023) / 1024;    // 11
constexpr int D_HEAD_UNITS = 8;
constexpr int D_LDS_UNITS = D_UNITS - D_HEAD_UNITS;  // 3
constexpr int NPOLL = NW - R_D;               // 8 polling waves
constexpr int DN_LDS = 88 * 1024;
constexpr int DN_HEAD = 24 * 1024;
static_assert(DN_LDS + R_D * D_LDS_UNITS * 1024 <= STAGE, "down units exceed LDS stage");
static_assert(GU_LDS + NW * 4096 <= DN_LDS, "gate/up units overlap the down units");
static_assert(DN_HEAD >= (I / 4) * 8 && DN_HEAD + R_D * D_HEAD_UNITS * 1024 <= DN_LDS,
              "down head units between the codes' staging and the early down units");

typedef unsigned long long u64;
typedef __attribute__((address_space(1))) const i32x4 gi32x4;

// 16-byte streaming load through a global (not flat) pointer: flat loads
// would also count against the LDS wait counter.
__device__ __forceinline__ i32x4 ldg_nt(const void* p) {
  return __builtin_nontemporal_load((gi32x4*)p);
}
template <typename T>
__device__ __forceinline__ T ldg(const T* p) {
  return *(const __attribute__((address_space(1))) T*)p;
}
// Wave-uniform read of data that no kernel writes (per-row scales, column
// sums, biases) through the constant address space: a scalar load into an
// SGPR, waited on with the LDS counter, never behind the weight stream.
template <typename T>
__device__ __forceinline__ T ldc(const T* p, int i) {
  return ((const __attribute__((address_space(4))) T*)(uintptr_t)p)[__builtin_amdgcn_readfirstlane(i)];
}

__device__ __forceinline__ void xput(u64* p, float v, uint32_t tag) {
  __hip_atomic_store(p, ((u64)tag << 32) | (u64)__float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
// element i of a replicated vector of length n
__device__ __forceinline__ void xput_rep(u64* base, int n, int i, float v, uint32_t tag) {
#pragma unroll
  for (int r = 0; r < NREP; ++r) xput(base + (size_t)r * n + i, v, tag);
}
__device__ __forceinline__ unsigned xcc_id() {
  unsigned x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  return x & (NREP - 1);
}
__device__ __forceinline__ u64 xget(const u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_f64(double* p, double v) {
  __hip_atomic_store((u64*)p, (u64)__double_as_longlong(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// DMA of `bytes` (multiple of 1024) from global to LDS by one wave, 1 KiB per
// instruction; device-scope loads when `coherent`.
template <bool coherent>
__device__ __forceinline__ void dma_wave(const void* src, void* lds, int bytes, int lane16) {
  const char* s = (const char*)src + lane16;
  char* d = (char*)lds;
  for (int off = 0; off < bytes; off += 1024) {
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(s + off),
                                     (void __attribute__((address_space(3)))*)(d + off), 16, 0,
                                     coherent ? 16 : 0);
  }
}

struct LayerW {
  const int8_t* w[7];  // q, k, v, o, gate, up, down
  const float* sw[7];
  const int32_t* cs[7];
  const float* bias[3];
  const float* ln1;
  const float* ln2;
  const float* kc;  // [T][NKV][D]
  const float* vc;
};

struct MegaArgs {
  const LayerW* layers;
  int L, T, V, pos;
  double eps;
  const float* final_norm;
  const int8_t* lm_w;
  const float* lm_sw;
  const int32_t* lm_cs;
  const uint8_t* lm4_w;
  const float* lm4_s;
  const uint8_t* lm4_z;
  const double* rcos;
  const double* rsin;
  float* kdelta;
  float* vdelta;
  float* logits;
  float* hidden_out;
  const uint8_t* mask;
  int32_t* out_token;
  u64* xch;
  u64* part;
  uint32_t* ctr;
  float* amax_v;
  int* amax_i;
  Err err;
  u64* trace;  // optional phase timestamps [3 workgroups][L + 1][16]
  u64* marker;
  u64 marker_value;
  uint32_t* epoch;  // [0] last launch's tag, [1] this launch's tag
  DumpRec dump;     // re-anchored parity record (instantiation with DUMP only)
};

// Fields of a layer record of the parity dump (the order of the public
// layout: h1, q|k|v, attention output, x1, h2, SwiGLU output, x2, the four
// code arrays, then s and z of the four quantisation points).
enum { F_H1, F_QKV, F_ATTN, F_X1, F_H2, F_A, F_X2, F_C1, F_C2, F_C3, F_C4, F_S, F_Z };
template <typename T>
__device__ __forceinline__ T* dump_at(const DumpRec& d, int l, int f) {
  if (!d.base || !((d.mask >> l) & 1)) return nullptr;
  return (T*)(d.base + (size_t)__popcll(d.mask & ((1ull << l) - 1)) * d.rec + d.f[f]);
}

// Phase timestamps (100 MHz real-time counter) of workgroups 0, 1 and the
// last one for every layer, and of every workgroup for one layer, when a
// trace buffer is given: [3][L + 1][32] then [NWG][16].
constexpr int TRACE_WIDE_LAYER = 2;
__device__ __forceinline__ void trace_at(const MegaArgs& A, int w, int l, int ev) {
  if (A.trace && threadIdx.x == 0) {
    const u64 t = __builtin_amdgcn_s_memrealtime();
    const int slot = w == 0 ? 0 : (w == 1 ? 1 : (w == NWG - 1 ? 2 : -1));
    if (slot >= 0) A.trace[((size_t)slot * (A.L + 1) + l) * 32 + ev] = t;
    if (l == (A.L > TRACE_WIDE_LAYER ? TRACE_WIDE_LAYER : 0))
      A.trace[(size_t)3 * (A.L + 1) * 32 + (size_t)w * 16 + ev] = t;
  }
}

// The latest of the streaming waves' timestamps for a phase's end (each
// wave's lane 0 calls this once).
__device__ __forceinline__ void trace_done(const MegaArgs& A, int w, int l, int ev, int lane) {
  if (A.trace && lane == 0) {
    const u64 t = __builtin_amdgcn_s_memrealtime();
    const int slot = w == 0 ? 0 : (w == 1 ? 1 : (w == NWG - 1 ? 2 : -1));
    if (slot >= 0)
      __hip_atomic_fetch_max(A.trace + ((size_t)slot * (A.L + 1) + l) * 32 + ev, t,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (l == (A.L > TRACE_WIDE_LAYER ? TRACE_WIDE_LAYER : 0))
      __hip_atomic_fetch_max(A.trace + (size_t)3 * (A.L + 1) * 32 + (size_t)w * 16 + ev, t,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ void trace_val(const MegaArgs& A, int w, int l, int ev, uint32_t v) {
  if (A.trace && threadIdx.x == 0 && l == (A.L > TRACE_WIDE_LAYER ? TRACE_WIDE_LAYER : 0))
    A.trace[(size_t)3 * (A.L + 1) * 32 + (size_t)w * 16 + ev] = v;
}
// Wide-trace slot of a poll count (workgroup w, layer TRACE_WIDE_LAYER), or null.
__device__ __forceinline__ uint32_t* trace_stat(const MegaArgs& A, int w, int l, int ev) {
  if (!A.trace || l != (A.L > TRACE_WIDE_LAYER ? TRACE_WIDE_LAYER : 0)) return nullptr;
  return (uint32_t*)(A.trace + (size_t)3 * (A.L + 1) * 32 + (size_t)w * 16 + ev);
}
// Slot of a sub-phase timestamp (events 16..31) of workgroups 0, 1 and the
// last one, or null.
__device__ __forceinline__ u64* trace_sub(const MegaArgs& A, int w, int l, int ev) {
  const int slot = w == 0 ? 0 : (w == 1 ? 1 : (w == NWG - 1 ? 2 : -1));
  return (A.trace && slot >= 0) ? A.trace + ((size_t)slot * (A.L + 1) + l) * 32 + ev : nullptr;
}
__device__ __forceinline__ void stamp(u64* t, int i, int lane) {
  if (t && lane == 0) t[i] = __builtin_amdgcn_s_memrealtime();
}

// exp(x) in fp64, written out so its constants come from LDS at the point
// of use (kept in registers across the kernel they would be spilled):
// x = k ln2 + r with |r| <= ln2 / 2 (two-part ln2, k ln2_hi exact for
// |k| < 2^11), e^r by its Taylor series to degree 13 (the first dropped term
// is below 5e-18), times 2^k.  A few fp64 ulp from the correctly rounded
// value; every caller rounds its result to fp32 afterwards.
// Table: 1/k! for k = 0..13 (each correctly rounded), ln2_hi (ln2 with the
// low 21 mantissa bits cleared), ln2_lo = ln2 - ln2_hi, 1/ln2.
__constant__ double kExpTab[17] = {
    0x1.0p+0, 0x1.0p+0, 0x1.0p-1, 0x1.5555555555555p-3, 0x1.5555555555555p-5,
    0x1.1111111111111p-7, 0x1.6c16c16c16c17p-10, 0x1.a01a01a01a01ap-13,
    0x1.a01a01a01a01ap-16, 0x1.71de3a556c734p-19, 0x1.27e4fb7789f5cp-22,
    0x1.ae64567f544e4p-26, 0x1.1eed8eff8d898p-29, 0x1.6124613a86d09p-33,
    0x1.62e42fee00000p-1, 0x1.a39ef35793c76p-33, 0x1.71547652b82fep+0};

__device__ __forceinline__ double exp_t(double x, const double* t) {
  // the table in two groups, each requested before its first use: two LDS
  // round trips instead of one per coefficient, few registers held at once
  const double2* t2 = (const double2*)t;
  const double2 c7 = t2[7], c6 = t2[6], c5 = t2[5], c4 = t2[4];
  const double inv_ln2 = t[16];
  asm volatile("" ::"v"(c7.x), "v"(c7.y), "v"(c6.x), "v"(c6.y), "v"(c5.x), "v"(c5.y), "v"(c4.x),
               "v"(c4.y), "v"(inv_ln2));
  const bool tiny = !(x > -746.0);  // also NaN
  const bool huge = x > 709.8;
  const double xs = (tiny || huge) ? 0.0 : x;
  const double k = rint(xs * inv_ln2);
  const double r = fma(-k, c7.y, fma(-k, c7.x, xs));
  const double2 c3 = t2[3], c2 = t2[2], c1 = t2[1], c0 = t2[0];
  double p = c6.y;  // 1/13!
  p = fma(p, r, c6.x);
  p = fma(p, r, c5.y);
  p = fma(p, r, c5.x);
  p = fma(p, r, c4.y);
  p = fma(p, r, c4.x);
  asm volatile("" ::"v"(c3.x), "v"(c3.y), "v"(c2.x), "v"(c2.y), "v"(c1.x), "v"(c1.y), "v"(c0.x),
               "v"(c0.y));
  p = fma(p, r, c3.y);
  p = fma(p, r, c3.x);
  p = fma(p, r, c2.y);
  p = fma(p, r, c2.x);
  p = fma(p, r, c1.y);
  p = fma(p, r, c1.x);
  p = fma(p, r, c0.y);
  p = fma(p, r, c0.x);
  const double e = ldexp(p, (int)k);
  return tiny ? ((x != x) ? x : 0.0) : (huge ? (double)INFINITY : e);
}

struct Shared {
  float xs[H];         // layer input (kept for the o residual)
  float x1s[H];        // input of the MLP half (kept for the down residual)
  float gain[H];
  int8_t codes[11264];
  alignas(16) unsigned char stage[STAGE];
  double redd[NW];
  alignas(16) float redf[2 * NW];
  float bestv[NW];
  int besti[NW];
  LayerW lt[2];        // weight table of layers l and l + 1 (slot l % 2)
  float aval[GU_ROWS * NW];  // this workgroup's SwiGLU values
  alignas(16) double expc[17];  // exp_t table
  double rcos[D / 2];  // rotary table row of the position (attention workgroups)
  double rsin[D / 2];
  float qpf;           // quantisation parameters handed from the computing waves
  int qpz;
  int flag;
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Workgroup barrier that orders LDS only: every wave's LDS reads and writes
// are complete, while its global loads (prefetched weights) stay in flight.
// Data a wave copied into LDS by DMA is covered only once that wave has
// waited for its own loads (vmcnt) before the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), no vmcnt wait
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Reduce the 16 per-wave partials that lanes 0..15 of the calling wave hold
// (one DPP row), result in every lane.  All 64 lanes must be active.
template <typename T, typename Op>
__device__ __forceinline__ T reduce16(T v, Op op) {
  static_assert(NW == 16, "one partial per lane of a DPP row");
  v = op(v, dpp::mov<dpp::kXor1>(v));
  v = op(v, dpp::mov<dpp::kXor2>(v));
  v = op(v, dpp::mov<dpp::kHalfMirror>(v));
  v = op(v, dpp::mov<dpp::kMirror>(v));
  return dpp::lane_read(v, 0);
}
// Min and max of the 16 per-wave (min, max) pairs in red.
__device__ __forceinline__ void minmax16(const float* red, int lane, float& lo, float& hi) {
  const float2 m = ((const float2*)red)[lane & 15];
  lo = reduce16(m.x, [](float a, float b) { return fminf(a, b); });
  hi = reduce16(m.y, [](float a, float b) { return fmaxf(a, b); });
}

// ------------------------------------------------------------- waiting --
// One wave: wait until words [c0, c1) of v carry the tag and copy them to
// dst (word c0 first).  The range is first copied straight into LDS with
// device-scope loads and every tag checked: data that is already there (the
// usual case) costs one round trip.  Otherwise producers write v in blocks
// of blk words (block b = words [b*blk, b*blk + blk)): the wave polls the
// first word of each block that meets the range (or, given flags, the
// block's flag word), which keeps the polling traffic small, then copies
// and checks again until all tags match.  The copy is whole KiB: dst needs
// room up to the next KiB boundary.  Bounded: after err.limit rounds the
// error word is set and the wave goes on.  Returns the number of sparse
// polls plus 65536 x the number of copies.
__device__ uint32_t poll_range(const u64* v, int c0, int c1, int blk, unsigned char* dst,
                               Err err, int lane, uint32_t tag, u64* tr = nullptr,
                               const u64* flags = nullptr, bool dense = false) {
  const int bytes = ((c1 - c0) * 8 + 1023) & ~1023;
  // dense: copy again until every tag matches, without the sparse phase
  // (for short waits while little else is in flight)
  for (uint32_t n = 0;; ++n) {
    dma_wave<true>(v + c0, dst, bytes, lane * 16);
    __builtin_amdgcn_s_waitcnt(0);
    const u64* s = (const u64*)dst;
    bool ok = true;
#pragma unroll 4
    for (int i = lane; i < c1 - c0; i += 64) ok &= (uint32_t)(s[i] >> 32) == tag;
    if (__all(ok)) {
      stamp(tr, 1, lane);
      return (n + 1) << 16;
    }
    if (!dense) break;
    if (n >= err.limit) {
      if (lane == 0) atomicOr(err.word, 2u);
      return (n + 1) << 16;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  uint32_t spins = 0;
  const int b0 = c0 / blk, b1 = (c1 - 1) / blk;
  for (;;) {
    bool ok = true;
    for (int b = b0 + lane; b <= b1; b += 64)
      ok &= (uint32_t)(xget(flags ? flags + b : v + max(c0, b * blk)) >> 32) == tag;
    if (__all(ok)) break;
    if (++spins > err.limit) {
      if (lane == 0) atomicOr(err.word, 1u);
      break;
    }
  }
  const uint32_t pre = spins;
  stamp(tr, 1, lane);
  for (;;) {
    dma_wave<true>(v + c0, dst, bytes, lane * 16);
    __builtin_amdgcn_s_waitcnt(0);
    const u64* s = (const u64*)dst;
    bool ok = true;
#pragma unroll 4
    for (int i = lane; i < c1 - c0; i += 64) ok &= (uint32_t)(s[i] >> 32) == tag;
    if (__all(ok)) break;
    if (++spins > err.limit) {
      if (lane == 0) atomicOr(err.word, 2u);
      break;
    }
  }
  return pre + ((spins - pre + 2) << 16);
}

// All waves: poll_range over words [0, n) of v, split into one chunk of
// whole KiB per wave, staged at stage + 8 i.  Also waits for every load the
// wave has in flight.  Returns wave 0's poll_range count.
__device__ uint32_t poll_all(const u64* v, int n, int blk, unsigned char* stage, Err err,
                             int lane, int wave, uint32_t tag, u64* tr = nullptr,
                             const u64* flags = nullptr, int np = NW, bool dense = false) {
  if (wave >= np) return 0;  // not a polling wave: its loads in flight stay in flight
  if (wave == 0) stamp(tr, 0, lane);
  const int chunk = ((n + np - 1) / np + 127) & ~127;
  const int c0 = wave * chunk, c1 = min(n, c0 + chunk);
  uint32_t r = 0;
  if (c0 < c1)
    r = poll_range(v, c0, c1, blk, stage + (size_t)c0 * 8, err, lane, tag, wave == 0 ? tr : nullptr,
                   flags, dense);
  __builtin_amdgcn_s_waitcnt(0);
  if (wave == 0) stamp(tr, 2, lane);
  return r;
}

// Waves 0..7: start copying an H-float gain vector into LDS (completes by the
// next poll_all).
__device__ __forceinline__ void load_gain(const float* g, float* dst, int wave, int lane16) {
  if (wave < H / 256) dma_wave<false>(g + wave * 256, dst + wave * 256, 1024, lane16);
}

// All threads: staged words -> fp32 values.
__device__ __forceinline__ void unstage(const unsigned char* stage, float* dst, int n, int tid) {
  const u64* s = (const u64*)stage;
#pragma unroll 2
  for (int i = tid; i < n; i += NT) dst[i] = __uint_as_float((uint32_t)s[i]);
}

// ----------------------------------------------------------- prologues --
// RMSNorm (fp64 inside) of x with gain g, then the dynamic uint8 quantiser;
// shifted codes to sh.codes.  All 512 threads.
template <bool DUMP>
__device__ QParam prologue_norm(const float* x, const float* g, double eps, Shared& sh, int tid,
                                u64* tr = nullptr, const DumpRec* dump = nullptr) {
  if (tid == 0) stamp(tr, 0, 0);
  double ss = 0.0;
  for (int i = tid; i < H; i += NT) {
    const double v = x[i];
    ss += v * v;
  }
  ss = block_sum<NT>(ss, sh.redd);
  if (tid == 0) stamp(tr, 1, 0);
  const double rs = 1.0 / sqrt(ss / (double)H + eps);
  float hv[H / NT];
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll
  for (int j = 0; j < H / NT; ++j) {
    const int i = tid + j * NT;
    hv[j] = (float)(((double)x[i] * rs) * (double)g[i]);
    lo = fminf(lo, hv[j]);
    hi = fmaxf(hi, hv[j]);
  }
  block_minmax<NT>(lo, hi, sh.redf);
  if (tid == 0) stamp(tr, 2, 0);
  const QParam p = quant_param(lo, hi);
#pragma unroll
  for (int j = 0; j < H / NT; ++j) sh.codes[tid + j * NT] = shift_code(quant_code(hv[j], p));
  if constexpr (DUMP) {
    if (dump && dump->base) {
#pragma unroll
      for (int j = 0; j < H / NT; ++j) {
        ((float*)(dump->base + dump->head[0]))[tid + j * NT] = hv[j];
        ((int8_t*)(dump->base + dump->head[1]))[tid + j * NT] = sh.codes[tid + j * NT];
      }
      if (tid == 0) {
        *(float*)(dump->base + dump->head[2]) = p.s;
        *(int*)(dump->base + dump->head[3]) = p.z;
      }
    }
  }
  __syncthreads();
  if (tid == 0) stamp(tr, 3, 0);
  return p;
}

// The final RMSNorm of the int4 LM tier: x (in LDS) replaced by
// fp32((x * rs) * g), the arithmetic of prologue_norm, without quantisation
// (the int4 tier's activations stay fp32).
template <bool DUMP>
__device__ void norm_in_place(float* x, const float* g, double eps, Shared& sh, int tid,
                              const DumpRec* dump = nullptr) {
  double ss = 0.0;
  for (int i = tid; i < H; i += NT) {
    const double v = x[i];
    ss += v * v;
  }
  ss = block_sum<NT>(ss, sh.redd);
  const double rs = 1.0 / sqrt(ss / (double)H + eps);
#pragma unroll
  for (int j = 0; j < H / NT; ++j) {
    const int i = tid + j * NT;
    x[i] = (float)(((double)x[i] * rs) * (double)g[i]);
    if constexpr (DUMP)
      if (dump && dump->base) ((float*)(dump->base + dump->head[0]))[i] = x[i];
  }
  __syncthreads();
}

// Dynamic uint8 quantiser straight from the staged exchange words.
__device__ QParam prologue_plain(const unsigned char* stage, int n, Shared& sh, int tid) {
  const u64* x = (const u64*)stage;
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll 2
  for (int i = tid; i < n; i += NT) {
    const float v = __uint_as_float((uint32_t)x[i]);
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  block_minmax<NT>(lo, hi, sh.redf);
  const QParam p = quant_param(lo, hi);
#pragma unroll 2
  for (int i = tid; i < n; i += NT)
    sh.codes[i] = shift_code(quant_code(__uint_as_float((uint32_t)x[i]), p));
  __syncthreads();
  return p;
}

// All waves: poll_all of an H-word vector whose wave chunks are 128 words,
// then RMSNorm (fp64 inside) with gain sh.gain and the dynamic uint8
// quantiser: the values go to x (fp32), the shifted codes to sh.codes.
// Waves 0..3 (one per SIMD) do the arithmetic, 512 elements each: the
// wave-uniform part (sum, square root, division, quantisation parameters)
// then runs once per SIMD instead of once per wave.  Four barriers.
constexpr int NORM_WAVES = 4;
constexpr int NORM_PER_LANE = H / (NORM_WAVES * 64);
// `after_poll` runs in every wave once its share of the vector has arrived
// (loads it issues then do not delay this wait).
// With DUMP and dh != nullptr the values, codes and (s, z) are also written
// to dh, dc, ds, dz.
template <bool DUMP, typename AfterPoll>
__device__ QParam poll_norm(const u64* v, int blk, float* x, Shared& sh, double eps, int lane,
                            int wave, int tid, uint32_t tag, Err err, AfterPoll after_poll,
                            u64* tr = nullptr, uint32_t* stat = nullptr, u64* tn0 = nullptr,
                            u64* tn1 = nullptr, u64* tn2 = nullptr, float* dh = nullptr,
                            int8_t* dc = nullptr, float* ds = nullptr, int* dz = nullptr) {
  static_assert(H == NW * 128, "one 128-word chunk per wave");
  const uint32_t r = poll_all(v, H, blk, sh.stage, err, lane, wave, tag, tr);
  after_poll();
  if (stat && tid == 0) *stat = r;
  lds_barrier();
  const u64* st = (const u64*)sh.stage;
  const bool mine = wave < NORM_WAVES;
  const int i0 = wave * (H / NORM_WAVES) + lane;  // element i0 + 64 k
  float xv[NORM_PER_LANE];
  if (mine) {
    double ss = 0.0;
#pragma unroll
    for (int k = 0; k < NORM_PER_LANE; ++k) {
      xv[k] = __uint_as_float((uint32_t)st[i0 + 64 * k]);
      x[i0 + 64 * k] = xv[k];
      ss += (double)xv[k] * (double)xv[k];
    }
    ss = wave_sum(ss);
    if (lane == 0) sh.redd[wave] = ss;
  }
  lds_barrier();
  if (tid == 0) stamp(tn0, 0, 0);
  float hv[NORM_PER_LANE];
  if (mine) {
    const double ss = ((sh.redd[0] + sh.redd[1]) + sh.redd[2]) + sh.redd[3];
    const double rs = 1.0 / sqrt(ss / (double)H + eps);
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int k = 0; k < NORM_PER_LANE; ++k) {
      hv[k] = (float)(((double)xv[k] * rs) * (double)sh.gain[i0 + 64 * k]);
      lo = fminf(lo, hv[k]);
      hi = fmaxf(hi, hv[k]);
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (lane == 0) {
      sh.redf[2 * wave] = lo;
      sh.redf[2 * wave + 1] = hi;
    }
  }
  lds_barrier();
  if (tid == 0) stamp(tn1, 0, 0);
  QParam p;
  if (mine) {
    const float4 m0 = *(const float4*)sh.redf, m1 = *(const float4*)(sh.redf + 4);
    const float lo = fminf(fminf(m0.x, m0.z), fminf(m1.x, m1.z));
    const float hi = fmaxf(fmaxf(m0.y, m0.w), fmaxf(m1.y, m1.w));
    p = quant_param(lo, hi);
#pragma unroll
    for (int k = 0; k < NORM_PER_LANE; ++k) sh.codes[i0 + 64 * k] = shift_code(quant_code(hv[k], p));
    if (wave == 0 && lane == 0) {
      sh.qpf = p.s;
      sh.qpz = p.z;
    }
    if constexpr (DUMP) {
      if (dh) {
#pragma unroll
        for (int k = 0; k < NORM_PER_LANE; ++k) {
          dh[i0 + 64 * k] = hv[k];
          dc[i0 + 64 * k] = sh.codes[i0 + 64 * k];
        }
        if (wave == 0 && lane == 0) {
          *ds = p.s;
          *dz = p.z;
        }
      }
    }
  }
  lds_barrier();
  if (tid == 0) stamp(tn2, 0, 0);
  if (!mine) {
    p.s = sh.qpf;
    p.z = sh.qpz;
  }
  return p;
}

// All waves (barriers): poll_all of an n-word vector by waves below np,
// then the dynamic uint8 quantiser on it (each wave on its own chunk when
// all waves poll, else all waves on the whole vector after a barrier);
// shifted codes to sh.codes.
template <bool DUMP>
__device__ QParam poll_quant(const u64* v, int n, int blk, Shared& sh, int lane, int wave,
                             uint32_t tag, Err err, u64* tr = nullptr,
                             const u64* flags = nullptr, uint32_t* stat = nullptr, int np = NW,
                             bool pairs = false, float* dh = nullptr, int8_t* dc = nullptr,
                             float* ds = nullptr, int* dz = nullptr) {
  const int tid = wave * 64 + lane;
  const uint32_t r = poll_all(v, n, blk, sh.stage, err, lane, wave, tag, tr, flags, np);
  if (stat && tid == 0) *stat = r;
  const u64* st = (const u64*)sh.stage;
  float lo = INFINITY, hi = -INFINITY;
  int c0, c1, step;
  if (np == NW) {  // every wave scans its own chunk
    const int chunk = ((n + np - 1) / np + 127) & ~127;
    c0 = wave * chunk + lane;
    c1 = min(n, wave * chunk + chunk);
    step = 64;
  } else {  // the vector is complete once every poller is past the barrier
    lds_barrier();
    c0 = tid;
    c1 = n;
    step = NT;
  }
  for (int i = c0; i < c1; i += step) {
    const float x = __uint_as_float((uint32_t)st[i]);
    // pairs: the words are (min, max) pairs of the producers
    if (!pairs || !(i & 1)) lo = fminf(lo, x);
    if (!pairs || (i & 1)) hi = fmaxf(hi, x);
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  if (lane == 0) {
    sh.redf[2 * wave] = lo;
    sh.redf[2 * wave + 1] = hi;
  }
  lds_barrier();
  minmax16(sh.redf, lane, lo, hi);
  const QParam p = quant_param(lo, hi);
  if (pairs) return p;  // the quantisation parameters only
  for (int i = c0; i < c1; i += step)
    sh.codes[i] = shift_code(quant_code(__uint_as_float((uint32_t)st[i]), p));
  if constexpr (DUMP) {
    if (dh) {
      for (int i = c0; i < c1; i += step) {
        dh[i] = __uint_as_float((uint32_t)st[i]);
        dc[i] = sh.codes[i];
      }
      if (tid == 0) {
        *ds = p.s;
        *dz = p.z;
      }
    }
  }
  lds_barrier();
  return p;
}

typedef int i32x16 __attribute__((ext_vector_type(16)));

// All waves: wait for the (min, max) word pairs of all NWG workgroups in v
// (workgroups without SwiGLU rows publish +inf, -inf) and reduce them to the
// quantisation parameters (every wave gets them).  The words are read with
// coherent scalar loads: they take the scalar path to memory, so this wait
// does not queue behind the vector loads (weights) the workgroup has in
// flight.  Wave w checks words [32 w, 32 w + 32) with four 64-byte loads per
// round.  Bounded like poll_range.
__device__ QParam poll_amm(const u64* v, Shared& sh, int lane, int wave, uint32_t tag,
                           Err err, u64* tr = nullptr) {
  static_assert(NW * 32 == 2 * NWG, "one 32-word slice per wave covers every workgroup");
  if (wave == 0) stamp(tr, 0, lane);
  // the address in scalar registers (readfirstlane) whether or not this
  // function is inlined into a caller that knows it is wave-uniform
  const u64* vw = (const u64*)uniform_ptr(v + wave * 32);
  i32x16 q[4];
  uint32_t spins = 0;
  for (;;) {
    asm volatile(
        "s_load_dwordx16 %0, %4, 0x0 glc\n\t"
        "s_load_dwordx16 %1, %4, 0x40 glc\n\t"
        "s_load_dwordx16 %2, %4, 0x80 glc\n\t"
        "s_load_dwordx16 %3, %4, 0xc0 glc\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&s"(q[0]), "=&s"(q[1]), "=&s"(q[2]), "=&s"(q[3])
        : "s"(vw)
        : "memory");
    uint32_t bad = 0;
#pragma unroll
    for (int k = 0; k < 32; ++k) bad |= (uint32_t)q[k / 8][2 * (k % 8) + 1] ^ tag;
    if (bad == 0) break;
    if (++spins > err.limit) {
      if (lane == 0) atomicOr(err.word, 8u);
      break;
    }
    __builtin_amdgcn_s_sleep(4);  // ~0.1 us: 4096 polling waves would crowd the scalar path
  }
  // word 2 i is workgroup i's min, word 2 i + 1 its max
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll
  for (int k = 0; k < 32; k += 2) {
    lo = fminf(lo, __int_as_float(q[k / 8][2 * (k % 8)]));
    hi = fmaxf(hi, __int_as_float(q[k / 8][2 * (k % 8) + 2]));
  }
  if (wave == 0) stamp(tr, 1, lane);
  if (lane == 0) {
    sh.redf[2 * wave] = lo;
    sh.redf[2 * wave + 1] = hi;
  }
  lds_barrier();
  if (wave == 0) stamp(tr, 2, lane);
  minmax16(sh.redf, lane, lo, hi);
  return quant_param(lo, hi);
}

// Waves below NPOLL: poll n words of packed codes (4 per word, producer
// blocks of blk words) and unpack them to sh.codes; all waves end at a
// barrier.  The staging of each polling wave ends before DN_LDS.
__device__ void poll_codes(const u64* v, int n, int blk, Shared& sh, int lane, int wave,
                           uint32_t tag, Err err, u64* tr = nullptr) {
  poll_all(v, n, blk, sh.stage, err, lane, wave, tag, tr, nullptr, NPOLL, true);
  if (wave < NPOLL) {
    const int chunk = ((n + NPOLL - 1) / NPOLL + 127) & ~127;
    const int c1 = min(n, wave * chunk + chunk);
    const u64* st = (const u64*)sh.stage;
    for (int i = wave * chunk + lane; i < c1; i += 64) ((uint32_t*)sh.codes)[i] = (uint32_t)st[i];
  }
  lds_barrier();
}

// ------------------------------------------------------ weight streams --
// Rows of a phase: workgroup w owns rows [w*R, (w+1)*R); wave s owns local
// rows i = (s + rot) % 16 + 16k.
__device__ __forceinline__ int row_local(int s, int rot, int k) { return (s + rot) % NW + NW * k; }

// Load NR rows x U units (1 KiB per unit: 16 bytes per lane) of a K-byte
// row-major int8 matrix into registers, plus per-row metadata.
template <int NR, int U>
__device__ __forceinline__ void load_rows(i32x4 (&r)[NR][U], float (&msw)[NR], int (&mcs)[NR],
                                          const int8_t* W, const float* sw, const int32_t* cs,
                                          int K, int row0, int R, int s, int rot, int lane16) {
  // metadata first: a later wait on it must not also wait for the weights
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const int i = row_local(s, rot, k);
    const bool valid = i < R;
    msw[k] = valid ? ldc(sw, row0 + i) : 0.0f;
    mcs[k] = valid ? ldc(cs, row0 + i) : 0;
  }
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const int i = row_local(s, rot, k);
    const bool valid = i < R;
    const int8_t* p = W + (size_t)(row0 + (valid ? i : 0)) * K;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int off = u * 1024 + lane16;
      r[k][u] = (valid && off < K) ? ldg_nt(p + off)
                                   : i32x4{0, 0, 0, 0};
    }
  }
}

__device__ __forceinline__ int dot16(const i32x4 w, const i32x4 a, int acc) {
  acc = __builtin_amdgcn_sdot4(w[0], a[0], acc, false);
  acc = __builtin_amdgcn_sdot4(w[1], a[1], acc, false);
  acc = __builtin_amdgcn_sdot4(w[2], a[2], acc, false);
  acc = __builtin_amdgcn_sdot4(w[3], a[3], acc, false);
  return acc;
}

// Dot products of NR register-resident rows with the LDS codes: each 16-byte
// code chunk is read once and used for every row; returns wave totals.
template <int NR, int U>
__device__ __forceinline__ void dot_rows(const i32x4 (&r)[NR][U], const int8_t* codes,
                                         int (&out)[NR], int lane16) {
#pragma unroll
  for (int k = 0; k < NR; ++k) out[k] = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const i32x4 a = *(const i32x4*)(codes + u * 1024 + lane16);
#pragma unroll
    for (int k = 0; k < NR; ++k) out[k] = dot16(r[k][u], a, out[k]);
  }
#pragma unroll
  for (int k = 0; k < NR; ++k) out[k] = wave_sum(out[k]);
}

// Rolling window over a streamer's units (16 bytes per lane each): the first
// W are issued by prime(), run() consumes unit i and refills its slot with
// unit i + W.  Fully unrolled, so every slot is a fixed register.
template <int N, int W, typename Addr>
__device__ __forceinline__ void prime_units(i32x4 (&buf)[W], Addr addr) {
#pragma unroll
  for (int j = 0; j < W; ++j) {
    if (j < N) {
      const int8_t* a = addr(j);
      buf[j] = a ? ldg_nt(a) : i32x4{0, 0, 0, 0};
    }
  }
}
template <int N, int W, typename Addr, typename Use>
__device__ __forceinline__ void run_units(i32x4 (&buf)[W], Addr addr, Use use) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int j = i % W;
    use(i, buf[j]);
    if (i + W < N) {
      const int8_t* a = addr(i + W);
      buf[j] = a ? ldg_nt(a) : i32x4{0, 0, 0, 0};
    }
  }
}

// ---------------------------------------------------------- attention --
// Work items: (KV head g, head group hh of 4 query heads, item sp < 4) on
// workgroup 8 g + 4 hh + sp.  With nchunk live 64-key chunks (those holding
// a key at or before the position) each (g, hh) uses nitem = min(4, nchunk)
// items, item sp taking chunks sp, sp + nitem, ...: a second chunk in the
// same item costs more than the merge of two items' states.
constexpr int ATT_RED = 0;                             // fp64 partial sums, 16 KiB
constexpr int ATT_KV = 16 * 1024;                      // byte offset in stage
constexpr int ATT_QKV = ATT_KV + 2 * (KEYS / 2) * 260 * 4;
constexpr int ATT_Q = ATT_QKV + 10 * 1024;             // rotated q, fp64 [HPI][D]
constexpr int ATT_KR = ATT_Q + HPI * D * 8;            // rotated k and v, fp32 [D] each
constexpr int ATT_P = ATT_KR + 2 * D * 4;              // softmax weights, fp64 [KEYS][HPI]
constexpr int ATT_HM = ATT_P + HPI * KEYS * 8;         // per-head max and sum, fp64
constexpr int ATT_END = ATT_HM + HPI * 2 * 8;
constexpr int SC_SLICES = 8;                           // score waves: 16 dims each
constexpr int PV_SLICES = 4;                           // P V key slices: 16 keys each
constexpr int PSTATE = 2 * PART;                       // words per (item, head)
constexpr int MERGE_BATCH = 4;                         // items merged per pass
static_assert(ATT_END <= STAGE, "attention staging exceeds LDS stage");  // the down units are loaded after it
static_assert(SC_SLICES * HPI * KEYS * 8 <= ATT_KV && PV_SLICES * HPI * D * 8 <= ATT_KV,
              "partial sums exceed their region");
static_assert(MERGE_BATCH * HPI * PSTATE * 8 + 1024 <= ATT_QKV - ATT_KV, "merge batch too large");
static_assert(SC_SLICES * 16 == D && PV_SLICES * 16 == KEYS && HPI * D <= NT, "attention split");

__device__ __forceinline__ int kv_row(int k) { return (k >> 1) * 260 + (k & 1) * D; }

// All waves: start copying the live cache rows of KV head g in the chunk
// starting at j0 into LDS, keys (which = 0) or values (which = 1) or both
// (which = 2); two rows per 1 KiB instruction, pairs spread over the waves.
// Completes by the wave's next full wait.
__device__ __forceinline__ void load_kv(const MegaArgs& A, int l, int g, int j0, Shared& sh,
                                        int wave, int lane, int which = 2) {
  const int npair = (min(KEYS, A.pos + 1 - j0) + 1) / 2;
  const LayerW& Lw = sh.lt[l & 1];
  float* Ks = (float*)(sh.stage + ATT_KV);
  float* Vs = Ks + (KEYS / 2) * 260;
  for (int pr = wave; pr < npair; pr += NW) {
    const int j = j0 + 2 * pr + (lane >> 5);
    const size_t off = ((size_t)j * NKV + g) * D + (lane & 31) * 4;
    if (which != 1)
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(Lw.kc + off),
                                       (void __attribute__((address_space(3)))*)(Ks + pr * 260),
                                       16, 0, 0);
    if (which != 0)
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(Lw.vc + off),
                                       (void __attribute__((address_space(3)))*)(Vs + pr * 260),
                                       16, 0, 0);
  }
}

__device__ __forceinline__ void put_half(u64* p, uint32_t v, uint32_t tag) {
  __hip_atomic_store(p, ((u64)tag << 32) | (u64)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_tagged_f64(u64* p, double v, uint32_t tag) {
  const u64 b = (u64)__double_as_longlong(v);
  put_half(p, (uint32_t)b, tag);
  put_half(p + 1, (uint32_t)(b >> 32), tag);
}
__device__ __forceinline__ double get_tagged_f64(const u64* p) {
  return __longlong_as_double((long long)((p[0] & 0xffffffffull) | (p[1] << 32)));
}

// Online-softmax merge of a state (m, l, o) into (M, L, O).
__device__ __forceinline__ void softmax_merge(double& M, double& L, double& O, double m, double l,
                                              double o, const double* et) {
  const double Mn = fmax(M, m);
  const double a = exp_t(M - Mn, et);   // 0 while M is still -inf
  const double b = exp_t(m - Mn, et);
  L = L * a + l * b;
  O = O * a + o * b;
  M = Mn;
}

// One attention item: query heads h0 .. h0 + 3 of KV head g (h0 = 8 g + 4 hh)
// over the chunks c = sp, sp + nitem, ... of the cache, folded with the
// online-softmax update; fp64 inside (the products of two fp32 values are
// exact in fp64).  Every step spreads over the waves so that no SIMD
// repeats wave-uniform work: scores as 8 slices of 16 dims (lane = key, all
// four heads per lane, so each key value is widened once), partial sums
// through LDS, the softmax of head h on wave h, the weighted values as 4
// slices of 16 keys x 2 halves of the dims (lane = dim), partial sums
// through LDS, and thread (h, d) < 512 keeps the running state of output
// (h, d).  With more than one item, items sp > 0 publish their states (fp64
// as two tagged 32-bit halves) and item 0 waits for them, merges and
// publishes the output.
//
// LDS (stage offsets): partial sums [0, 16K); keys and values of the chunk
// as pairs of rows 1040 bytes apart (key k at float offset kv_row(k)); the
// q|k|v words; rotated q (fp64), k and v; the softmax weights; per-head
// max and sum.
__device__ void attention_item(const MegaArgs& A, uint32_t epoch, int l, int g, int hh, int sp,
                               int nitem, int nchunk, Shared& sh, u64* xl, u64* tr, int tid,
                               int lane, int wave) {
  const int p = A.pos;
  float* Ks = (float*)(sh.stage + ATT_KV);
  float* Vs = Ks + (KEYS / 2) * 260;
  unsigned char* qst = sh.stage + ATT_QKV;
  double* qd = (double*)(sh.stage + ATT_Q);
  float* kr = (float*)(sh.stage + ATT_KR);
  float* vv = kr + D;
  double* pw = (double*)(sh.stage + ATT_P);
  double* hm = (double*)(sh.stage + ATT_HM);
  double* red = (double*)(sh.stage + ATT_RED);
  const int h0 = g * G + hh * HPI;

  // The first chunk's keys are requested first; the wait for q|k|v queues
  // only behind them (a workgroup's loads are served in order), and the
  // values, first needed for the weighted sum, are requested after it.
  load_kv(A, l, g, sp * KEYS, sh, wave, lane, 0);
  // q of heads h0..h0+3 (waves 0..3), k and v of KV head g (waves 4, 5)
  if (wave < HPI + 2) {
    const int n0 = wave < HPI ? (h0 + wave) * D : (wave == HPI ? Q + g * D : Q + KVD + g * D);
    poll_range(xl + OFF_QKV, n0, n0 + D, R_QKV, qst + wave * D * 8, A.err, lane, epoch);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of the first chunk's keys
  lds_barrier();
  load_kv(A, l, g, sp * KEYS, sh, wave, lane, 1);
  if (tid == 0) stamp(tr, 0, lane);
  // rotary embedding (fp64) at position p, rounded to fp32; q kept widened
  {
    const u64* s = (const u64*)qst;
    const double* cs = sh.rcos;
    const double* sn = sh.rsin;
    for (int t = tid; t < (HPI + 1) * (D / 2); t += NT) {
      const int head = t / (D / 2), j = t % (D / 2);
      const double x1 = __uint_as_float((uint32_t)s[head * D + j]);
      const double x2 = __uint_as_float((uint32_t)s[head * D + j + D / 2]);
      const double c = cs[j], sv = sn[j];
      const float r1 = (float)(x1 * c - x2 * sv);
      const float r2 = (float)(x2 * c + x1 * sv);
      if (head < HPI) {
        qd[head * D + j] = r1;
        qd[head * D + j + D / 2] = r2;
      } else {
        kr[j] = r1;
        kr[j + D / 2] = r2;
      }
    }
    for (int t = tid; t < D; t += NT) vv[t] = __uint_as_float((uint32_t)s[(HPI + 1) * D + t]);
  }
  lds_barrier();
  // the first item of head group 0 publishes the deltas (stores left in flight)
  if (hh == 0 && sp == 0)
    for (int t = tid; t < D; t += NT) {
      A.kdelta[(size_t)l * KVD + g * D + t] = kr[t];
      A.vdelta[(size_t)l * KVD + g * D + t] = vv[t];
    }
  const bool mine = tid < HPI * D;
  const int oh = tid >> 7, od = tid & (D - 1);  // output (head, dim) of a state thread
  double M = -INFINITY, Lsum = 0.0, O = 0.0;
  for (int c = sp; c < nchunk; c += nitem) {
    const int j0 = c * KEYS;
    const int nk = min(KEYS, p + 1 - j0);  // keys at or before the position
    if (c != sp) {
      lds_barrier();  // the previous chunk's values and partial sums are used
      load_kv(A, l, g, j0, sh, wave, lane);
      __builtin_amdgcn_s_waitcnt(0);
      lds_barrier();
    }
    // this call's key row replaces cache row p
    const bool here = p >= j0 && p < j0 + KEYS;
    if (here)
      for (int t = tid; t < D; t += NT) Ks[kv_row(p - j0) + t] = kr[t];
    lds_barrier();
    if (tid == 0) stamp(tr, 1, lane);
    // scores, partial over dims [16 w, 16 w + 16) on waves 0..7, lane = key;
    // keys past the position are selected away below (their rows are stale)
    if (wave < SC_SLICES) {
      const float4* kp = (const float4*)(Ks + kv_row(lane) + 16 * wave);
      double acc[HPI];
#pragma unroll
      for (int h = 0; h < HPI; ++h) acc[h] = 0.0;
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4) {
        // the group's key and q values are all requested before the first use
        const float4 kv = kp[d4];
        double2 qa[HPI], qb[HPI];
#pragma unroll
        for (int h = 0; h < HPI; ++h) {
          const double2* qh = (const double2*)(qd + h * D + 16 * wave + 4 * d4);
          qa[h] = qh[0];
          qb[h] = qh[1];
        }
        asm volatile("" ::"v"(kv.x), "v"(qa[0].x), "v"(qa[1].x), "v"(qa[2].x), "v"(qa[3].x),
                     "v"(qb[0].x), "v"(qb[1].x), "v"(qb[2].x), "v"(qb[3].x));
        const double k0 = kv.x, k1 = kv.y, k2 = kv.z, k3 = kv.w;
#pragma unroll
        for (int h = 0; h < HPI; ++h) {
          acc[h] = fma(qa[h].x, k0, acc[h]);
          acc[h] = fma(qa[h].y, k1, acc[h]);
          acc[h] = fma(qb[h].x, k2, acc[h]);
          acc[h] = fma(qb[h].y, k3, acc[h]);
        }
      }
#pragma unroll
      for (int h = 0; h < HPI; ++h) red[(wave * HPI + h) * KEYS + lane] = acc[h];
    }
    lds_barrier();
    // softmax of head h on wave h, lane = key
    if (wave < HPI) {
      double sc = 0.0;
#pragma unroll
      for (int s = 0; s < SC_SLICES; ++s) sc += red[(s * HPI + wave) * KEYS + lane];
      sc = lane < nk ? sc / sqrt((double)D) : -INFINITY;
      const double m = wave_max(sc);
      const double e = lane < nk ? exp_t(sc - m, sh.expc) : 0.0;
      const double ls = wave_sum(e);
      pw[lane * HPI + wave] = e;
      if (lane == 0) {
        hm[2 * wave] = m;
        hm[2 * wave + 1] = ls;
      }
    }
    // this wave's copies of the values are in (the first chunk's were
    // requested after the keys)
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    if (tid == 0) stamp(tr, 2, lane);
    // this call's value row replaces cache row p; the value rows past it
    // (stale LDS, weight 0) are zeroed so that the weighted sum needs no mask
    if (here) {
      for (int t = tid; t < D; t += NT) Vs[kv_row(p - j0) + t] = vv[t];
      for (int t = tid + nk * D; t < KEYS * D; t += NT) Vs[kv_row(t >> 7) + (t & (D - 1))] = 0.f;
      lds_barrier();
    }
    // weighted values, partial over keys [16 ks, 16 ks + 16) on waves 0..7
    // (ks = w / 2): lane = dim within half w % 2, all four heads per lane;
    // keys past the position have weight 0 and zeroed rows
    if (wave < 2 * PV_SLICES) {
      const int d = 64 * (wave & 1) + lane, ks = wave >> 1;
      double acc[HPI];
#pragma unroll
      for (int h = 0; h < HPI; ++h) acc[h] = 0.0;
      for (int k4 = 16 * ks; k4 < min(nk, 16 * ks + 16); k4 += 4) {
        float vf[4];
        double2 pa[4], pb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // the group's loads are requested together
          vf[i] = Vs[kv_row(k4 + i) + d];
          pa[i] = *(const double2*)(pw + (k4 + i) * HPI);
          pb[i] = *(const double2*)(pw + (k4 + i) * HPI + 2);
        }
        asm volatile("" ::"v"(vf[0]), "v"(vf[1]), "v"(vf[2]), "v"(vf[3]), "v"(pa[0].x),
                     "v"(pa[3].x), "v"(pb[0].x), "v"(pb[3].x));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const double v = vf[i];
          acc[0] = fma(pa[i].x, v, acc[0]);
          acc[1] = fma(pa[i].y, v, acc[1]);
          acc[2] = fma(pb[i].x, v, acc[2]);
          acc[3] = fma(pb[i].y, v, acc[3]);
        }
      }
#pragma unroll
      for (int h = 0; h < HPI; ++h) red[(ks * HPI + h) * D + d] = acc[h];
    }
    lds_barrier();
    if (nitem == 1 && tid == 0) stamp(tr, 3, lane);
    // fold the chunk into the running state of output (h, d)
    if (mine) {
      double o = 0.0;
#pragma unroll
      for (int s = 0; s < PV_SLICES; ++s) o += red[(s * HPI + oh) * D + od];
      if (c == sp) {  // the merge into the empty state, written out
        M = hm[2 * oh];
        Lsum = hm[2 * oh + 1];
        O = o;
      } else {
        softmax_merge(M, Lsum, O, hm[2 * oh], hm[2 * oh + 1], o, sh.expc);
      }
    }
  }
  if (nitem == 1) {
    if (tid == 0) stamp(tr, 4, lane);
    if (mine) xput_rep(xl + OFF_ATT, Q, (h0 + oh) * D + od, (float)(O / Lsum), epoch);
    return;
  }
  u64* part = A.part + (((size_t)l * NKV + g) * HH + hh) * NIH * HPI * PSTATE;  // item 0's slot unused
  if (sp > 0) {
    if (mine) {
      u64* pst = part + ((size_t)sp * HPI + oh) * PSTATE;
      if (od == 0) {
        put_tagged_f64(pst, M, epoch);
        put_tagged_f64(pst + 2, Lsum, epoch);
      }
      put_tagged_f64(pst + 4 + 2 * od, O, epoch);
    }
    return;
  }
  if (tid == 0) stamp(tr, 3, lane);
  // item 0: merge the other items' states, MERGE_BATCH per pass
  const u64* pb = (const u64*)(sh.stage + ATT_KV);
  for (int s0 = 1; s0 < nitem; s0 += MERGE_BATCH) {
    const int ns = min(MERGE_BATCH, nitem - s0);
    const int n = ns * HPI * PSTATE;
    const int chunk = ((n + NW - 1) / NW + 127) & ~127;
    const int c0 = wave * chunk, c1 = min(n, c0 + chunk);
    lds_barrier();  // the chunk's values (or the previous batch) are used
    if (c0 < c1)
      poll_range(part + (size_t)s0 * HPI * PSTATE, c0, c1, HPI * PSTATE,
                 sh.stage + ATT_KV + c0 * 8, A.err, lane, epoch);
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    if (mine)
      for (int s = 0; s < ns; ++s) {
        const u64* q = pb + ((size_t)s * HPI + oh) * PSTATE;
        softmax_merge(M, Lsum, O, get_tagged_f64(q), get_tagged_f64(q + 2),
                      get_tagged_f64(q + 4 + 2 * od), sh.expc);
      }
  }
  if (tid == 0) stamp(tr, 4, lane);
  if (mine) xput_rep(xl + OFF_ATT, Q, (h0 + oh) * D + od, (float)(O / Lsum), epoch);
}

// ------------------------------------------------------------ the kernel --
template <bool DUMP>
__global__ __launch_bounds__(1024, 1) void k_decode(MegaArgs A) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Shared& sh = *(Shared*)smem_raw;
  int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(wave_id());
  int w = blockIdx.x;
  // Per-lane byte offset and wave index, redefined opaquely in every layer so
  // the compiler recomputes addresses in the loop instead of keeping dozens
  // of hoisted 64-bit addresses live next to the prefetched weights.
  int lane16 = lane * 16;
  int s = wave;

  // attention items (see attention_item): workgroup w < NATT holds item
  // sp = w % NIH of head group hh = (w / NIH) % HH of KV head g = w / (NIH HH)
  const int nchunk = A.pos / KEYS + 1;
  const int nitem = min(NIH, nchunk);
  const bool att = w < NATT && (w % NIH) < nitem;
  // gate/up rows: rg per workgroup without attention work, by rank
  const int natt = NKV * HH * nitem;
  const int rank = w - (w >= NATT ? natt : (w / NIH) * nitem + min(w % NIH, nitem));
  const int rg = ((I + (NWG - natt) - 1) / (NWG - natt) + 3) & ~3;  // whole code words
  const int nprod = (I + rg - 1) / rg;                                  // ranks with rows
  const int gu0 = att ? 0 : rank * rg;
  const int ngu = att ? 0 : max(0, min(rg, I - gu0));

  // weight registers
  constexpr int W = 8;                      // units in flight per wave (big phases)
  constexpr int NGU = GU_ROWS * 2 * 2;      // gate/up units: rows x {gate, up} x 2
  static_assert(NGU == W + 4, "gate/up: 8 units in registers, 4 in LDS");
  static_assert(sizeof(LayerW) % 8 == 0 && sizeof(LayerW) / 8 <= 64, "layer table");
  i32x4 wq[1][2], wo[1][2], win[W];
  float sq[1], so[1], sg[GU_ROWS], su[GU_ROWS], sd;
  int cq[1], co[1], cg[GU_ROWS], cu[GU_ROWS], cd;
  float bq[1] = {0.f};

  auto issue_qkv = [&](int l) {
    const LayerW& Lw = sh.lt[l & 1];
    // rows of the concatenated q|k|v space: [w*10, w*10+10), row s
    const bool valid = s < R_QKV;
    const int n = w * R_QKV + (valid ? s : 0);
    const int seg = n < Q ? 0 : (n < Q + KVD ? 1 : 2);
    const int nl = n - (seg == 0 ? 0 : (seg == 1 ? Q : Q + KVD));
    const int8_t* p = Lw.w[seg] + (size_t)nl * H;
    sq[0] = valid ? ldc(Lw.sw[seg], nl) : 0.f;
    cq[0] = valid ? ldc(Lw.cs[seg], nl) : 0;
    bq[0] = valid ? ldc(Lw.bias[seg], nl) : 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) wq[0][u] = valid ? ldg_nt(p + u * 1024 + lane16) : i32x4{0, 0, 0, 0};
  };
  auto issue_o = [&](int l) {
    const LayerW& Lw = sh.lt[l & 1];
    load_rows<1, 2>(wo, so, co, Lw.w[3], Lw.sw[3], Lw.cs[3], Q, w * R_O, R_O, s, 0, lane16);
  };
  // unit i of the gate/up phase: row s + 16 (i / 4), matrix (i / 2) % 2, unit i % 2
  auto gu_addr = [&](const LayerW& Lw, int i) -> const int8_t* {
    const int k = i / 4, m = (i / 2) % 2, u = i % 2;
    const int r = s + NW * k;
    if (r >= ngu) return nullptr;
    return Lw.w[4 + m] + (size_t)(gu0 + r) * H + u * 1024 + lane16;
  };
  // unit u of the down phase: bytes [u KiB, u KiB + 1 KiB) of row s - NPOLL
  // (a lane past the row's end reads the row start; its code is zero)
  auto down_addr = [&](const LayerW& Lw, int u) -> const int8_t* {
    const int off = u * 1024 + lane16;
    return Lw.w[6] + (size_t)(w * R_D + s - NPOLL) * I + (off < I ? off : 0);
  };
  auto issue_gate_up = [&](int l) {
    const LayerW& Lw = sh.lt[l & 1];
#pragma unroll
    for (int k = 0; k < GU_ROWS; ++k) {
      const int r = s + NW * k;
      const bool valid = r < ngu;
      sg[k] = valid ? ldc(Lw.sw[4], gu0 + r) : 0.f;
      cg[k] = valid ? ldc(Lw.cs[4], gu0 + r) : 0;
      su[k] = valid ? ldc(Lw.sw[5], gu0 + r) : 0.f;
      cu[k] = valid ? ldc(Lw.cs[5], gu0 + r) : 0;
    }
    // units 0..7 into registers
    prime_units<W, W>(win, [&](int i) { return gu_addr(Lw, i); });
  };
  // the last row's four units into this wave's 4 KiB of LDS (stage bytes
  // [16K, 80K): on workgroups without attention work they are free from the
  // end of the q|k|v phase); requested with the register units, so that they
  // are in before the o projection's stores, which would otherwise queue
  // behind them
  auto issue_gate_up_lds = [&](int l) {
    const LayerW& Lw = sh.lt[l & 1];
    if (s + NW * 2 < ngu) {
#pragma unroll
      for (int i = W; i < NGU; ++i)
        __builtin_amdgcn_global_load_lds(
            (const void __attribute__((address_space(1)))*)gu_addr(Lw, i),
            (void __attribute__((address_space(3)))*)(sh.stage + GU_LDS + s * 4096 + (i - W) * 1024),
            16, 0, 2);
    }
  };
  // loaders: the LDS part of their down row (any time the region is free)
  auto issue_down_lds = [&](int l) {
    if (s < NPOLL) return;
    const LayerW& Lw = sh.lt[l & 1];
#pragma unroll
    for (int u = D_HEAD_UNITS; u < D_UNITS; ++u)
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)down_addr(Lw, u),
          (void __attribute__((address_space(3)))*)(sh.stage + DN_LDS +
                                                    ((s - NPOLL) * D_LDS_UNITS + u - D_HEAD_UNITS) *
                                                        1024),
          16, 0, 2);
  };
  // loaders: the other units of their down row, into LDS as well (the stage
  // region between the codes' staging and DN_LDS must be free)
  auto issue_down_head = [&](int l) {
    if (s < NPOLL) return;
    const LayerW& Lw = sh.lt[l & 1];
    sd = ldc(Lw.sw[6], w * R_D + s - NPOLL);
    cd = ldc(Lw.cs[6], w * R_D + s - NPOLL);
#pragma unroll
    for (int u = 0; u < D_HEAD_UNITS; ++u)
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)down_addr(Lw, u),
          (void __attribute__((address_space(3)))*)(sh.stage + DN_HEAD +
                                                    ((s - NPOLL) * D_HEAD_UNITS + u) * 1024),
          16, 0, 2);
  };

  const size_t rep = xcc_id();
  const uint32_t epoch = __builtin_amdgcn_readfirstlane(A.epoch[1]);
  if (w == 0 && tid == 0) {
    A.epoch[0] = epoch;           // the next launch counts on from here
    *A.marker = A.marker_value;   // the exchange area is initialised
  }
  // the weight table lives in LDS: pointers read from global memory with
  // vector loads would make every address wait for all loads in flight
  constexpr int LTW = sizeof(LayerW) / 8;
  if (tid < LTW) ((u64*)&sh.lt[0])[tid] = ((const u64*)&A.layers[0])[tid];
  if (A.L > 1 && tid >= 64 && tid < 64 + LTW)
    ((u64*)&sh.lt[1])[tid - 64] = ((const u64*)&A.layers[1])[tid - 64];
  if (tid < 17) sh.expc[tid] = kExpTab[tid];
  // codes past the SwiGLU vector stay zero: the tail of the last down unit
  // multiplies them
  for (int i = I + tid; i < (int)sizeof(sh.codes); i += NT) sh.codes[i] = 0;
  __syncthreads();
  issue_qkv(0);
  if (att && tid < D / 2) {
    sh.rcos[tid] = A.rcos[(size_t)A.pos * (D / 2) + tid];
    sh.rsin[tid] = A.rsin[(size_t)A.pos * (D / 2) + tid];
  }

  for (int l = 0; l < A.L; ++l) {
    asm volatile("" : "+v"(lane16), "+v"(tid), "+v"(lane), "+s"(w), "+s"(s));
    const LayerW& Lw = sh.lt[l & 1];
    u64* xl = A.xch + (size_t)l * XCH_LAYER;
    u64* xn = A.xch + (size_t)(l + 1) * XCH_LAYER;   // next layer's input lives at its OFF_X0
    // table of layer l + 1 into the other slot (layer l - 1 is done with it;
    // read after this layer's barriers)
    if (l >= 1 && l + 1 < A.L && tid < LTW)
      ((u64*)&sh.lt[(l + 1) & 1])[tid] = ((const u64*)&A.layers[l + 1])[tid];

    // parity record of this layer (workgroup 0 records what every
    // workgroup computes alike; the producers record their own rows)
    float *d_qkv = nullptr, *d_x1 = nullptr, *d_a = nullptr, *d_x2 = nullptr, *d_s = nullptr;
    int8_t* d_c4 = nullptr;
    int* d_z = nullptr;
    const bool d0 = DUMP && w == 0;
    if constexpr (DUMP) {
      d_qkv = dump_at<float>(A.dump, l, F_QKV);
      d_x1 = dump_at<float>(A.dump, l, F_X1);
      d_a = dump_at<float>(A.dump, l, F_A);
      d_x2 = dump_at<float>(A.dump, l, F_X2);
      d_c4 = dump_at<int8_t>(A.dump, l, F_C4);
      d_s = dump_at<float>(A.dump, l, F_S);
      d_z = dump_at<int>(A.dump, l, F_Z);
    }

    // ---- q, k, v
    trace_at(A, w, l, 0);
    load_gain(Lw.ln1, sh.gain, wave, lane16);
    QParam qp = poll_norm<DUMP>(xl + OFF_X0 + rep * H, R_D, sh.xs, sh, A.eps, lane, wave, tid, epoch,
                          A.err, [] {}, trace_sub(A, w, l, 27), trace_stat(A, w, l, 11),
                          trace_sub(A, w, l, 11), trace_sub(A, w, l, 12), trace_sub(A, w, l, 13),
                          d0 ? dump_at<float>(A.dump, l, F_H1) : nullptr,
                          d0 ? dump_at<int8_t>(A.dump, l, F_C1) : nullptr, d0 ? d_s : nullptr,
                          d0 ? d_z : nullptr);
    trace_at(A, w, l, 2);
    {
      int accs[1];
      dot_rows<1, 2>(wq, sh.codes, accs, lane16);
      if (lane == 0 && s < R_QKV) {
        float y = dequant(accs[0] + (128 - qp.z) * cq[0], qp.s, sq[0]);
        y = y + bq[0];
        xput(xl + OFF_QKV + w * R_QKV + s, y, epoch);
        if constexpr (DUMP)
          if (d_qkv) d_qkv[w * R_QKV + s] = y;
      }
    }
    trace_done(A, w, l, 3, lane);

    // ---- attention; the other workgroups stream the o rows and their
    // gate/up rows meanwhile
    if (att) {
      lds_barrier();  // the codes are used (the stores of the q|k|v rows stay in flight)
      attention_item(A, epoch, l, w / (NIH * HH), (w / NIH) % HH, w % NIH, nitem, nchunk, sh, xl,
                     trace_sub(A, w, l, 22), tid, lane, s);  // s: wave index, opaque per layer
      lds_barrier();  // the staging area is free again
      // no SwiGLU rows here: the neutral (min, max) pair, one replica per lane
      if (wave == 0 && lane < NREP) {
        float pinf = INFINITY;
        asm volatile("" : "+v"(pinf));  // made here, not kept (spilled) across the loop
        u64* mm = xl + OFF_AMM + lane * 2 * NWG + 2 * w;
        xput(mm, pinf, epoch);
        xput(mm + 1, -pinf, epoch);
      }
      issue_o(l);
      issue_down_lds(l);
    } else {
      issue_o(l);
      issue_gate_up(l);
      issue_gate_up_lds(l);
      issue_down_lds(l);
    }

    // ---- o projection + residual
    asm volatile("" : "+v"(lane16), "+v"(tid), "+v"(lane));
    trace_at(A, w, l, 4);
    qp = poll_quant<DUMP>(xl + OFF_ATT + rep * Q, Q, HPI * D, sh, lane, wave, epoch, A.err, nullptr,
                          nullptr, trace_stat(A, w, l, 12), NW, false,
                          d0 ? dump_at<float>(A.dump, l, F_ATTN) : nullptr,
                          d0 ? dump_at<int8_t>(A.dump, l, F_C2) : nullptr, d0 ? d_s + 1 : nullptr,
                          d0 ? d_z + 1 : nullptr);
    trace_at(A, w, l, 5);
    {
      int accs[1];
      dot_rows<1, 2>(wo, sh.codes, accs, lane16);
      if (lane == 0 && s < R_O) {
        const int n = w * R_O + s;
        const float y = dequant(accs[0] + (128 - qp.z) * co[0], qp.s, so[0]);
        xput_rep(xl + OFF_X1, H, n, sh.xs[n] + y, epoch);
        if constexpr (DUMP)
          if (d_x1) d_x1[n] = sh.xs[n] + y;
      }
    }
    trace_done(A, w, l, 6, lane);
    // attention workgroups have no gate/up rows: their down rows next
    if (att) issue_down_head(l);

    // ---- gate/up + SwiGLU
    asm volatile("" : "+v"(lane16), "+v"(tid), "+v"(lane));
    load_gain(Lw.ln2, sh.gain, wave, lane16);
    qp = poll_norm<DUMP>(xl + OFF_X1 + rep * H, R_O, sh.x1s, sh, A.eps, lane, wave, tid, epoch,
                         A.err, [] {}, trace_sub(A, w, l, 16), trace_stat(A, w, l, 13),
                         trace_sub(A, w, l, 14), trace_sub(A, w, l, 15), trace_sub(A, w, l, 30),
                         d0 ? dump_at<float>(A.dump, l, F_H2) : nullptr,
                         d0 ? dump_at<int8_t>(A.dump, l, F_C3) : nullptr, d0 ? d_s + 2 : nullptr,
                         d0 ? d_z + 2 : nullptr);
    trace_at(A, w, l, 7);
    if (!att) {
      const int zc = 128 - qp.z;
      int aggs[GU_ROWS] = {}, aus[GU_ROWS] = {};
      const i32x4 c0 = *(const i32x4*)(sh.codes + lane16);
      const i32x4 c1 = *(const i32x4*)(sh.codes + 1024 + lane16);
      run_units<W, W>(win, [&](int i) { return gu_addr(Lw, i); }, [&](int i, const i32x4 v) {
        const int k = i / 4, m = (i / 2) % 2, u = i % 2;
        int& acc = m ? aus[k] : aggs[k];
        acc = dot16(v, u ? c1 : c0, acc);
      });
      if (s + NW * 2 < ngu) {
#pragma unroll
        for (int i = W; i < NGU; ++i) {
          const i32x4 v = *(const i32x4*)(sh.stage + GU_LDS + s * 4096 + (i - W) * 1024 + lane16);
          const int m = (i / 2) % 2, u = i % 2;
          int& acc = m ? aus[2] : aggs[2];
          acc = dot16(v, u ? c1 : c0, acc);
        }
      }
#pragma unroll
      for (int k = 0; k < GU_ROWS; ++k) {
        aggs[k] = wave_sum(aggs[k]);
        aus[k] = wave_sum(aus[k]);
      }
      // SwiGLU of row s + 16 k on lane k (the rows' exponentials side by side)
      int ag = aggs[0], au = aus[0], cgk = cg[0], cuk = cu[0];
      float sgk = sg[0], suk = su[0];
#pragma unroll
      for (int k = 1; k < GU_ROWS; ++k)
        if (lane == k) {
          ag = aggs[k];
          au = aus[k];
          cgk = cg[k];
          cuk = cu[k];
          sgk = sg[k];
          suk = su[k];
        }
      const int i = s + NW * lane;
      const bool live = lane < GU_ROWS && i < ngu;
      const float gv = dequant(ag + zc * cgk, qp.s, sgk);
      const float uv = dequant(au + zc * cuk, qp.s, suk);
      // silu(g) u = (g >= 0 ? g u : g u t) / (1 + t) with t = e^-|g| in
      // [0, 1]: the denominator lies in [1, 2], so two Newton steps on the
      // reciprocal estimate replace a general fp64 division
      const double gd = gv;
      const double t = exp_t(-fabs(gd), sh.expc);
      const double gu = gd * (double)uv;
      const double num = gd >= 0.0 ? gu : gu * t;
      const double den = 1.0 + t;
      double rq = __builtin_amdgcn_rcp(den);
      rq = fma(rq, fma(-den, rq, 1.0), rq);
      rq = fma(rq, fma(-den, rq, 1.0), rq);
      const float a = (float)(num * rq);
      if (live) sh.aval[i] = a;
      if constexpr (DUMP)
        if (live && d_a) d_a[gu0 + i] = a;
      float lo = live ? a : INFINITY, hi = live ? a : -INFINITY;
      lo = fminf(lo, fminf(dpp::mov<dpp::kXor1>(lo), dpp::mov<dpp::kXor2>(lo)));
      hi = fmaxf(hi, fmaxf(dpp::mov<dpp::kXor1>(hi), dpp::mov<dpp::kXor2>(hi)));
      if (lane == 0) {
        sh.redf[2 * s] = lo;
        sh.redf[2 * s + 1] = hi;
      }
      trace_done(A, w, l, 8, lane);
      lds_barrier();  // the down units bound for LDS may still be in flight
      // round 1: this workgroup's min and max (+inf, -inf without rows), one
      // replica per lane
      if (wave == 0) {
        minmax16(sh.redf, lane, lo, hi);
        if (lane < NREP) {
          u64* mm = xl + OFF_AMM + lane * 2 * NWG + 2 * w;
          xput(mm, lo, epoch);
          xput(mm + 1, hi, epoch);
        }
      }
      // the rest of the down rows are requested now, behind the (min, max)
      // stores (a workgroup's memory requests are served in order) and into
      // the LDS the gate/up units have left: they stream during the
      // (min, max) wait (which takes the scalar path) and are in before the
      // codes are awaited
      lds_barrier();
      if (tid == 0) stamp(trace_sub(A, w, l, 31), 0, 0);
      issue_down_head(l);
    }

    // ---- SwiGLU quantisation parameters from all producers' min/max
    asm volatile("" : "+v"(lane16), "+v"(tid), "+v"(lane));
    qp = poll_amm(xl + OFF_AMM + rep * 2 * NWG, sh, lane, wave, epoch, A.err, trace_sub(A, w, l, 19));
    if constexpr (DUMP)
      if (d0 && d_s && tid == 0) {
        d_s[3] = qp.s;
        d_z[3] = qp.z;
      }
    // round 2: producers quantise their rows and publish the packed codes
    if (!att && tid == 0) stamp(trace_sub(A, w, l, 25), 0, 0);
    if (!att && tid < ngu / 4) {
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        word |= (uint32_t)(uint8_t)shift_code(quant_code(sh.aval[4 * tid + j], qp)) << (8 * j);
      const int k = gu0 / 4 + tid;
      if constexpr (DUMP)
        if (d_c4) ((uint32_t*)d_c4)[k] = word;
#pragma unroll
      for (int r = 0; r < NREP; ++r)
        __hip_atomic_store(xl + OFF_AC + (size_t)r * (I / 4) + k, ((u64)epoch << 32) | word,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // ---- down + residual: waves 0..7 poll and unpack the SwiGLU codes;
    // loader 8 + r computes row r from its units in LDS
    asm volatile("" : "+v"(lane16), "+v"(tid), "+v"(lane));
    poll_codes(xl + OFF_AC + rep * (I / 4), I / 4, rg / 4, sh, lane, wave, epoch, A.err,
               att ? nullptr : trace_sub(A, w, l, 22));
    trace_at(A, w, l, 9);
    if (s >= NPOLL) {
      int acc = 0;
      const int8_t* cb = sh.codes + lane16;
      __builtin_amdgcn_s_waitcnt(0);  // this wave's LDS units
#pragma unroll
      for (int u = 0; u < D_HEAD_UNITS; ++u) {
        const i32x4 v =
            *(const i32x4*)(sh.stage + DN_HEAD + ((s - NPOLL) * D_HEAD_UNITS + u) * 1024 + lane16);
        acc = dot16(v, *(const i32x4*)(cb + u * 1024), acc);
      }
#pragma unroll
      for (int u = D_HEAD_UNITS; u < D_UNITS; ++u) {
        const i32x4 v = *(const i32x4*)(sh.stage + DN_LDS +
                                        ((s - NPOLL) * D_LDS_UNITS + u - D_HEAD_UNITS) * 1024 +
                                        lane16);
        acc = dot16(v, *(const i32x4*)(cb + u * 1024), acc);
      }
      acc = wave_sum(acc);
      if (lane == 0) {
        const int n = w * R_D + s - NPOLL;
        const float y = dequant(acc + (128 - qp.z) * cd, qp.s, sd);
        xput_rep(xn + OFF_X0, H, n, sh.x1s[n] + y, epoch);
        if constexpr (DUMP)
          if (d_x2) d_x2[n] = sh.x1s[n] + y;
      }
    }
    trace_done(A, w, l, 10, lane);
    if (l + 1 < A.L) issue_qkv(l + 1);
  }

  // ---- final norm + LM head + masked argmax
  u64* xf = A.xch + (size_t)A.L * XCH_LAYER;
  if (A.final_norm) load_gain(A.final_norm, sh.gain, wave, lane16);
  poll_all(xf + OFF_X0 + rep * H, H, R_D, sh.stage, A.err, lane, wave, epoch);
  __syncthreads();
  unstage(sh.stage, sh.xs, H, tid);
  __syncthreads();
  trace_at(A, w, A.L, 0);
  if (w == 0 && A.hidden_out)
    for (int i = tid; i < H; i += NT) A.hidden_out[i] = sh.xs[i];
  if (!A.lm_w && !A.lm4_w) return;
  const int r0 = (int)(((long long)w * A.V) / NWG), r1 = (int)(((long long)(w + 1) * A.V) / NWG);
  float bv = -INFINITY;
  int bi = INT_MAX;
  if (A.lm4_w) {
    // int4 LM tier: the normed row stays fp32; each streamer wave takes
    // whole 1 KB code rows (lane l: codes of k = 32 l .. 32 l + 31, block
    // l / 4) and forms s (sum h q - z sum h) per lane, then the wave sum
    norm_in_place<DUMP>(sh.xs, sh.gain, A.eps, sh, tid, (DUMP && w == 0) ? &A.dump : nullptr);
    if (wave > 0) {
      const int s = wave - 1;
      float hv[32];
#pragma unroll
      for (int i = 0; i < 32; i += 4) {
        const float4 t = *(const float4*)(sh.xs + 32 * lane + i);
        hv[i] = t.x;
        hv[i + 1] = t.y;
        hv[i + 2] = t.z;
        hv[i + 3] = t.w;
      }
      float hsum = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) hsum += hv[i];
      const int blk = lane / 4;
      constexpr int GR = 4;
      i32x4 b0[GR], b1[GR];
      float s0[GR], s1[GR];
      uint32_t z0[GR], z1[GR];
      int m0[GR], m1[GR];
      const int nmine = (r1 - r0 - s + NS - 1) / NS;
      const int ngroups = (nmine + GR - 1) / GR;
      auto load_group = [&](int gidx, i32x4 (&b)[GR], float (&sc)[GR], uint32_t (&zb)[GR],
                            int (&mk)[GR]) {
#pragma unroll
        for (int k = 0; k < GR; ++k) {
          const int n = r0 + s + NS * (gidx * GR + k);
          const bool valid = n < r1;
          const int nn = valid ? n : r0;
          b[k] = ldg_nt((const int8_t*)A.lm4_w + (size_t)nn * (H / 2) + 16 * lane);
          sc[k] = ldg(A.lm4_s + (size_t)nn * (H / 128) + blk);
          zb[k] = A.lm4_z[(size_t)nn * (H / 256) + blk / 2];
          mk[k] = (valid && A.mask) ? (int)ldg(A.mask + n) : 1;
        }
      };
      auto use_group = [&](int gidx, const i32x4 (&b)[GR], const float (&sc)[GR],
                           const uint32_t (&zb)[GR], const int (&mk)[GR]) {
#pragma unroll
        for (int k = 0; k < GR; ++k) {
          float a = 0.0f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t x = (uint32_t)b[k][j];
            uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
            asm volatile("" : "+v"(lo), "+v"(hi));  // keeps the byte conversions direct
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              a = fmaf(hv[8 * j + 2 * m], (float)((lo >> (8 * m)) & 0xffu), a);
              a = fmaf(hv[8 * j + 2 * m + 1], (float)((hi >> (8 * m)) & 0xffu), a);
            }
          }
          const float zf = (float)((zb[k] >> (4 * (blk & 1))) & 15u);
          const float y = wave_sum_f32(sc[k] * (a - zf * hsum));
          const int n = r0 + s + NS * (gidx * GR + k);
          if (lane == 0 && n < r1) {
            A.logits[n] = y;
            if (mk[k] == 0 && !isnan(y) && (y > bv || (y == bv && n < bi))) {
              bv = y;
              bi = n;
            }
          }
        }
      };
      if (ngroups > 0) load_group(0, b0, s0, z0, m0);
      for (int gg = 0; gg < ngroups; gg += 2) {
        if (gg + 1 < ngroups) load_group(gg + 1, b1, s1, z1, m1);
        use_group(gg, b0, s0, z0, m0);
        if (gg + 1 < ngroups) {
          if (gg + 2 < ngroups) load_group(gg + 2, b0, s0, z0, m0);
          use_group(gg + 1, b1, s1, z1, m1);
        }
      }
    }
  } else {
  const QParam qp = prologue_norm<DUMP>(sh.xs, sh.gain, A.eps, sh, tid, nullptr,
                                        (DUMP && w == 0) ? &A.dump : nullptr);
  if (wave > 0) {
    const int s = wave - 1;  // streamer 0..14
    const int zc = 128 - qp.z;
    constexpr int GR = 4;  // rows per group of one streamer; two groups in flight
    i32x4 b0[GR][2], b1[GR][2];
    float w0[GR], w1[GR];
    int c0[GR], c1[GR], m0[GR], m1[GR];
    const int nmine = (r1 - r0 - s + NS - 1) / NS;  // rows of this streamer
    const int ngroups = (nmine + GR - 1) / GR;
    // the metadata is loaded with the weights so no later load has to wait
    // behind the prefetched group
    auto load_group = [&](int gidx, i32x4 (&b)[GR][2], float (&sw)[GR], int (&cs)[GR],
                          int (&mk)[GR]) {
#pragma unroll
      for (int k = 0; k < GR; ++k) {
        const int n = r0 + s + NS * (gidx * GR + k);
        const bool valid = n < r1;
        const int8_t* p = A.lm_w + (size_t)(valid ? n : r0) * H;
#pragma unroll
        for (int u = 0; u < 2; ++u)
          b[k][u] = valid ? ldg_nt(p + u * 1024 + lane16)
                          : i32x4{0, 0, 0, 0};
        sw[k] = valid ? ldg(A.lm_sw + n) : 0.f;
        cs[k] = valid ? ldg(A.lm_cs + n) : 0;
        mk[k] = (valid && A.mask) ? (int)ldg(A.mask + n) : 1;
      }
    };
    auto use_group = [&](int gidx, const i32x4 (&b)[GR][2], const float (&sw)[GR],
                         const int (&cs)[GR], const int (&mk)[GR]) {
      int accs[GR];
      dot_rows<GR, 2>(b, sh.codes, accs, lane16);
#pragma unroll
      for (int k = 0; k < GR; ++k) {
        const int n = r0 + s + NS * (gidx * GR + k);
        const int acc = accs[k];
        if (lane == 0 && n < r1) {
          const float y = dequant(acc + zc * cs[k], qp.s, sw[k]);
          A.logits[n] = y;
          if (mk[k] == 0 && !isnan(y) && (y > bv || (y == bv && n < bi))) {
            bv = y;
            bi = n;
          }
        }
      }
    };
    if (ngroups > 0) load_group(0, b0, w0, c0, m0);
    for (int gg = 0; gg < ngroups; gg += 2) {
      if (gg + 1 < ngroups) load_group(gg + 1, b1, w1, c1, m1);
      use_group(gg, b0, w0, c0, m0);
      if (gg + 1 < ngroups) {
        if (gg + 2 < ngroups) load_group(gg + 2, b0, w0, c0, m0);
        use_group(gg + 1, b1, w1, c1, m1);
      }
    }
  }
  }
  trace_at(A, w, A.L, 1);
  if (!A.mask) return;
  // workgroup best -> partial; the last workgroup reduces all partials
  if (lane == 0) {
    sh.bestv[wave] = bv;
    sh.besti[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int k = 1; k < NW; ++k)
      if (sh.besti[k] != INT_MAX && (sh.bestv[k] > bv || (sh.bestv[k] == bv && sh.besti[k] < bi))) {
        bv = sh.bestv[k];
        bi = sh.besti[k];
      }
    __hip_atomic_store((uint32_t*)A.amax_v + w, __float_as_uint(bv), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store((uint32_t*)A.amax_i + w, (uint32_t)bi, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    const uint32_t old = __hip_atomic_fetch_add(A.ctr + 2 * A.L, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    sh.flag = (old == NWG - 1);
  }
  __syncthreads();
  if (!sh.flag || wave != 0) return;
  bv = -INFINITY;
  bi = INT_MAX;
  for (int k = lane; k < NWG; k += 64) {
    const float v = __uint_as_float(__hip_atomic_load((uint32_t*)A.amax_v + k, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT));
    const int i = (int)__hip_atomic_load((uint32_t*)A.amax_i + k, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    if (i != INT_MAX && (v > bv || (v == bv && i < bi))) {
      bv = v;
      bi = i;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v = __shfl_xor(bv, o, 64);
    const int i = __shfl_xor(bi, o, 64);
    if (i != INT_MAX && (v > bv || (v == bv && i < bi))) {
      bv = v;
      bi = i;
    }
  }
  if (lane == 0) *A.out_token = (bi == INT_MAX) ? -1 : bi;
}

// Zero the counters (and, on the first use of a workspace, the exchange
// words and partial states), pick this launch's tag, then publish the embedding of the token as
// the first layer's input in every replica, carrying that tag.  The tag
// counter lives in the workspace, so exchange words left by any earlier
// launch on it carry a different tag; a workspace whose marker does not hold
// this layout's value is cleared and counts from 1.
__global__ __launch_bounds__(256) void k_decode_prep(u64* xch, size_t nwords, uint32_t* ctr,
                                                     int nctr, uint32_t* err, const u64* marker,
                                                     u64 marker_value, uint32_t* epoch,
                                                     const int32_t* token, const uint16_t* table,
                                                     int V) {
  const bool fresh = *marker != marker_value;
  uint32_t e = fresh ? 1u : epoch[0] + 1u;
  if (e == 0) e = 1;
  if (fresh) {
    // the first layer's input block is written below, not cleared
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < nwords; i += stride)
      if (i < OFF_X0 || i >= OFF_X0 + (size_t)NREP * H) xch[i] = 0;
  }
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < nctr; i += 256) ctr[i] = 0;
    if (threadIdx.x == 0) {
      *err = 0;
      epoch[1] = e;
    }
  }
  if (blockIdx.x == 1) {
    const int id = *token;
    for (int i = threadIdx.x; i < H; i += 256) {
      const float v = (id >= 0 && id < V) ? half_bits_to_float(table[(size_t)id * H + i])
                                          : __int_as_float(0x7fc00000);
      for (int r = 0; r < NREP; ++r)
        xch[OFF_X0 + (size_t)r * H + i] = ((u64)e << 32) | (u64)__float_as_uint(v);
    }
  }
}


// Between two tokens of the greedy loop on this path: the deltas of the
// token just decoded written into the caches at its row (the arithmetic of
// k_cache_write), the stop rule (k_greedy_post), and, when another token
// follows, the preparation of its launch as k_decode_prep does it on an
// initialised workspace (counters cleared, the next tag, the embedding of
// the next input id in every replica of the first layer's input).  The
// error word is left as it is: a wait that timed out in any step of the
// loop stays recorded until the host reads it.  Workgroups 0 .. L-1 write the cache rows of their layer;
// workgroup L + r publishes replica r, and workgroup L also applies the
// stop rule.  Each of them derives the next input id itself: it equals the
// stored id whether or not workgroup L has already written it back.
struct BetweenArgs {
  float* kc[kMaxLayers];
  float* vc[kMaxLayers];
  int L, pos;              // layers; cache row of the token just decoded
  const float* kd;         // [L][KVD] deltas of that token
  const float* vd;
  int32_t* token;          // the greedy id, replaced by the next input id
  int32_t* out_row;
  int32_t end_id;
  int32_t* done;
  int prep;                // prepare the next launch
  u64* xch;
  uint32_t* ctr;
  int nctr;
  uint32_t* epoch;
  const uint16_t* table;
  int V;
};

__global__ __launch_bounds__(256) void k_decode_between(BetweenArgs A) {
  const int blk = blockIdx.x, tid = threadIdx.x;
  if (blk < A.L) {
    const float4* kd = (const float4*)(A.kd + (size_t)blk * KVD);
    const float4* vd = (const float4*)(A.vd + (size_t)blk * KVD);
    float4* kc = (float4*)(A.kc[blk] + (size_t)A.pos * KVD);
    float4* vc = (float4*)(A.vc[blk] + (size_t)A.pos * KVD);
    for (int e = tid; e < KVD / 4; e += 256) {
      kc[e] = kd[e];
      vc[e] = vd[e];
    }
    return;
  }
  const int r = blk - A.L;  // replica
  const int id = *A.done ? A.end_id : *A.token;
  __syncthreads();          // this workgroup has read the id before it is written back
  if (r == 0 && tid == 0) {
    *A.token = id;
    *A.out_row = id;
    if (id == A.end_id) *A.done = 1;
  }
  if (!A.prep) return;
  uint32_t e = A.epoch[0] + 1u;
  if (e == 0) e = 1;
  if (r == 0) {
    for (int i = tid; i < A.nctr; i += 256) A.ctr[i] = 0;
    if (tid == 0) A.epoch[1] = e;
  }
  for (int i = tid; i < H; i += 256) {
    const float v = (id >= 0 && id < A.V) ? half_bits_to_float(A.table[(size_t)id * H + i])
                                          : __int_as_float(0x7fc00000);
    A.xch[OFF_X0 + (size_t)r * H + i] = ((u64)e << 32) | (u64)__float_as_uint(v);
  }
}
}  // namespace mk

// ------------------------------------------------------------------ host --
// exchange words: L layers plus the final hidden state (the next layer's
// input block of the last layer)
static size_t mega_xch_words(int L) {
  return (size_t)L * mk::XCH_LAYER + mk::OFF_X0 + (size_t)mk::NREP * mk::H;
}

size_t decode_mega_ws_bytes(int L, int T) {
  const size_t xch = mega_xch_words(L) * 8;
  const size_t part = (size_t)L * mk::NKV * mk::HH * mk::NIH * mk::HPI * mk::PSTATE * 8;
  const size_t ctr = (size_t)(2 * L + 64) * 4;
  const size_t amax = (size_t)mk::NWG * 8;
  const size_t table = (size_t)L * sizeof(mk::LayerW);
  const size_t trace = ((size_t)3 * (L + 1) * 32 + mk::NWG * 16) * 8;
  auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
  return al(xch) + al(part) + al(ctr) + al(amax) + al(table) + al(trace) + 256;
}

bool decode_mega_supported(int H, int NH, int NKV, int D, int I, int T, int L) {
  // attention chunks are 64 whole cache rows
  return H == mk::H && NH == mk::NH && NKV == mk::NKV && D == mk::D && I == mk::I &&
         T % mk::KEYS == 0 && T >= mk::KEYS && T <= 8192 && L >= 1 && L <= kMaxLayers;
}

struct MegaLayout {
  mk::u64* xch;
  mk::u64* part;
  uint32_t* ctr;
  float* amax_v;
  int* amax_i;
  mk::LayerW* table;
  uint32_t* err;
  mk::u64* trace;
  mk::u64* marker;
  uint32_t* epoch;
};

static MegaLayout mega_layout(void* ws, int L, int T) {
  auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
  char* p = (char*)ws;
  MegaLayout m;
  m.xch = (mk::u64*)p;
  p += al(mega_xch_words(L) * 8);
  m.part = (mk::u64*)p;
  p += al((size_t)L * mk::NKV * mk::HH * mk::NIH * mk::HPI * mk::PSTATE * 8);
  m.ctr = (uint32_t*)p;
  m.err = m.ctr + 2 * L + 32;
  m.marker = (mk::u64*)(m.ctr + 2 * L + 48);
  m.epoch = m.ctr + 2 * L + 52;
  p += al((size_t)(2 * L + 64) * 4);
  m.amax_v = (float*)p;
  m.amax_i = (int*)(p + mk::NWG * 4);
  p += al((size_t)mk::NWG * 8);
  m.table = (mk::LayerW*)p;
  p += al((size_t)L * sizeof(mk::LayerW));
  m.trace = (mk::u64*)p;
  return m;
}

hipError_t decode_mega_upload(hipStream_t st, void* ws, int L, int T, const MegaLayer* layers) {
  MegaLayout lay = mega_layout(ws, L, T);
  mk::LayerW tab[kMaxLayers];
  for (int l = 0; l < L; ++l) {
    for (int i = 0; i < 7; ++i) {
      tab[l].w[i] = layers[l].w[i];
      tab[l].sw[i] = layers[l].sw[i];
      tab[l].cs[i] = layers[l].cs[i];
    }
    for (int i = 0; i < 3; ++i) tab[l].bias[i] = layers[l].bias[i];
    tab[l].ln1 = layers[l].ln1;
    tab[l].ln2 = layers[l].ln2;
    tab[l].kc = layers[l].kc;
    tab[l].vc = layers[l].vc;
  }
  return hipMemcpyAsync(lay.table, tab, sizeof(mk::LayerW) * L, hipMemcpyHostToDevice, st);
}

bool decode_mega_cooperative() {
  const char* e = getenv("ARK_DECODE_LAUNCH");
  return e && strcmp(e, "cooperative") == 0;
}

hipError_t decode_mega_launch(hipStream_t st, void* ws, const MegaStep& S, hipEvent_t ev_begin,
                              hipEvent_t ev_end, bool prep) {
  MegaLayout lay = mega_layout(ws, S.L, S.T);
  // the exchange words and the partial attention states that follow them
  const size_t part_words = (size_t)S.L * mk::NKV * mk::HH * mk::NIH * mk::HPI * mk::PSTATE;
  const size_t nwords = (size_t)(lay.part - lay.xch) + part_words;
  const mk::u64 marker = mk::MAGIC ^ (mk::u64)nwords ^ ((mk::u64)S.T << 40);
  hipError_t e = hipSuccess;
  if (prep) {
    hipLaunchKernelGGL(mk::k_decode_prep, dim3(mk::NWG), dim3(256), 0, st, lay.xch, nwords, lay.ctr,
                       2 * S.L + 32, lay.err, lay.marker, marker, lay.epoch, S.token, S.table, S.V);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  mk::MegaArgs A;
  A.layers = lay.table;
  A.L = S.L;
  A.T = S.T;
  A.V = S.V;
  A.pos = S.pos;
  A.eps = S.eps;
  A.final_norm = S.final_norm;
  A.lm_w = S.lm_w;
  A.lm_sw = S.lm_sw;
  A.lm_cs = S.lm_cs;
  A.lm4_w = S.lm4_w;
  A.lm4_s = S.lm4_s;
  A.lm4_z = S.lm4_z;
  A.rcos = S.rcos;
  A.rsin = S.rsin;
  A.kdelta = S.kdelta;
  A.vdelta = S.vdelta;
  A.logits = S.logits;
  A.hidden_out = S.hidden_out;
  A.mask = S.mask;
  A.out_token = S.out_token;
  A.xch = lay.xch;
  A.part = lay.part;
  A.ctr = lay.ctr;
  A.amax_v = lay.amax_v;
  A.amax_i = lay.amax_i;
  A.err.word = lay.err;
  A.err.limit = S.spin_limit < 0 ? mk::SPIN_LIMIT : (uint32_t)std::min<int64_t>(S.spin_limit, 0xffffffffll);
  A.dump = S.dump;
  const char* tr = getenv("ARK_MEGA_TRACE");
  A.trace = (tr && tr[0] == '1') ? lay.trace : nullptr;
  A.marker = lay.marker;
  A.marker_value = marker;
  A.epoch = lay.epoch;
  void* args[] = {&A};
  if (ev_begin) hipEventRecord(ev_begin, st);
  const void* fn = S.dump.base ? (const void*)mk::k_decode<true> : (const void*)mk::k_decode<false>;
  e = decode_mega_cooperative()
          ? hipLaunchCooperativeKernel(fn, dim3(mk::NWG), dim3(mk::NT), args, sizeof(mk::Shared), st)
          : hipLaunchKernel(fn, dim3(mk::NWG), dim3(mk::NT), args, sizeof(mk::Shared), st);
  if (ev_end) hipEventRecord(ev_end, st);
  return e;
}

hipError_t decode_mega_between(hipStream_t st, void* ws, const MegaStep& S, float* const* k_cache,
                               float* const* v_cache, int32_t* out_row, int32_t end_id,
                               int32_t* done, bool prep) {
  if (S.L < 1 || S.L > kMaxLayers) return hipErrorInvalidValue;
  MegaLayout lay = mega_layout(ws, S.L, S.T);
  mk::BetweenArgs A;
  for (int l = 0; l < S.L; ++l) {
    A.kc[l] = k_cache[l];
    A.vc[l] = v_cache[l];
  }
  A.L = S.L;
  A.pos = S.pos;
  A.kd = S.kdelta;
  A.vd = S.vdelta;
  A.token = const_cast<int32_t*>(S.token);
  A.out_row = out_row;
  A.end_id = end_id;
  A.done = done;
  A.prep = prep ? 1 : 0;
  A.xch = lay.xch;
  A.ctr = lay.ctr;
  A.nctr = 2 * S.L + 32;
  A.epoch = lay.epoch;
  A.table = S.table;
  A.V = S.V;
  hipLaunchKernelGGL(mk::k_decode_between, dim3(S.L + mk::NREP), dim3(256), 0, st, A);
  return hipGetLastError();
}

uint64_t* decode_mega_marker(void* ws, int L, int T) { return (uint64_t*)mega_layout(ws, L, T).marker; }

const uint32_t* decode_mega_err_word(const void* ws, int L, int T) {
  return mega_layout(const_cast<void*>(ws), L, T).err;
}

size_t decode_mega_trace_offset(int L, int T) {
  MegaLayout lay = mega_layout(nullptr, L, T);
  return (size_t)((char*)lay.trace - (char*)nullptr);
}

// One-time set-up of both instantiations (the record-writing one only for
// the parity tests): dynamic LDS size, and the check that all NWG
// workgroups fit on the device at once, which the exchanges rely on (and
// that the device can launch them cooperatively, for ARK_DECODE_LAUNCH).
// Thread-safe: std::call_once.
hipError_t decode_mega_init() {
  static std::once_flag once;
  static hipError_t status = hipSuccess;
  std::call_once(once, [] {
    const void* fns[2] = {(const void*)mk::k_decode<false>, (const void*)mk::k_decode<true>};
    for (const void* fn : fns) {
      status = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   sizeof(mk::Shared));
      if (status != hipSuccess) return;
      int dev = 0, ncu = 0, coop = 0, nblk = 0;
      hipGetDevice(&dev);
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
      hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev);
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&nblk, fn, mk::NT, sizeof(mk::Shared));
      if (!coop || (long)ncu * nblk < mk::NWG) {
        status = hipErrorCooperativeLaunchTooLarge;
        return;
      }
    }
  });
  return status;
}

}  // namespace ark

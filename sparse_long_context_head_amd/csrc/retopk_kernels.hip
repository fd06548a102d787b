// ReTopK decode-step kernels for CDNA4 (gfx950, wave64).
//
// Method: "Recall Before You Rank: Similarity-Guided Top-K Reuse for
// Efficient Long-Context Attention", Methodology section. A decode step (or an
// exact call) is one launch of k_step, whose work groups take two roles by
// block index:
//
//   head   one per query head: recall (Eqs. 5-7) and the path rule (Eq. 13),
//          published at once through a device-scope flag tagged with the call;
//          a reuse head then runs its whole path in the same work group:
//          candidate union (Eqs. 8-9), candidate scores (Eq. 10), rerank
//          (Eq. 11), softmax-V (Eq. 12) and the cache update;
//   score  full-history scores (Eq. 4) and a score histogram of every exact
//          head, GQA-grouped on MFMA, the rows of the exact KV groups spread
//          over all score work groups and kept in LDS; then the scores in the
//          histogram's boundary bin or above, per segment in position order,
//          and, in the work group each exact head is assigned to, the
//          selection inside the boundary bin (global Top-K, Eq. 1),
//          softmax-V and the cache update.
//
// Data passes between work groups only through device-scope (sc1) stores and
// loads and device-scope atomics, which are coherent across the XCDs' L2s on
// their own: no whole-L2 write-back or invalidate is needed (those cost more
// than a launch on this part). Head work groups never wait; a score work group
// waits only for earlier phases of the others, and every wait is bounded in
// time. Reuse heads need no full-history work at all, and the host never waits
// on the path decision. Every phase issues its global loads before consuming
// them, so a phase costs about one memory round trip rather than one per loop
// iteration.

#include "retopk_internal.h"

#include <algorithm>
#include <cmath>

namespace retopk {

namespace {

// The buffer table as the kernels see it: the same layout, every pointer in
// the global address space, so that accesses through it compile to global
// (not flat) instructions once the table is read from device memory.
// (the host pass, which only parses device code, sees plain pointers)
#if defined(__HIP_DEVICE_COMPILE__)
template <typename T>
using gptr = __attribute__((address_space(1))) T*;
#else
template <typename T>
using gptr = T*;
#endif

struct BufsDev {
  gptr<float> cache_qbar;
  gptr<int32_t> cache_supp;
  gptr<int32_t> cache_len;
  gptr<int32_t> fifo;
  gptr<int32_t> path;
  gptr<double> rho;
  gptr<int32_t> ret;
  gptr<int32_t> retslot;
  gptr<int32_t> m;
  gptr<int32_t> cand;
  gptr<float> score;
  gptr<uint32_t> hist;
  gptr<uint2> hits;
  gptr<uint2> ccnt;
  gptr<int32_t> dec;
  gptr<int32_t> err;
  gptr<int32_t> wdone;
  gptr<uint64_t> bkeys;
  gptr<int32_t> sel;
  gptr<float> selsc;
  gptr<int32_t> sellen;
  gptr<uint8_t> st_path;
  gptr<double> st_rho;
  gptr<int32_t> st_m;
  gptr<int32_t> hint;
  Bufs* self;
};
static_assert(sizeof(BufsDev) == sizeof(Bufs), "device view of the buffer table");

// The table as the head role reads it: in the constant address space, since
// it does not change while a kernel runs, so that its fields are read with
// scalar loads through the scalar cache (one round trip for the whole table,
// see prefetch_table) rather than vector loads that the compiler serialises.
#if defined(__HIP_DEVICE_COMPILE__)
typedef __attribute__((address_space(4))) const BufsDev ConstBufs;
#else
typedef const BufsDev ConstBufs;
#endif


constexpr float kNegInf = -INFINITY;
constexpr float kPosInf = INFINITY;
constexpr float kInvSqrtD = 0.08838834764831845f;  // 1 / sqrt(128)

// Every block of the step kernel has kHeadThreads threads (its only launch
// shape), and its device code uses that constant rather than blockDim.x: the
// runtime group size lives in the dispatch packet and, being memory, would be
// read again (a dependent global round trip) after every barrier that clobbers
// memory.

// Barrier for data shared through LDS only: this wave's LDS operations are
// complete, then s_barrier. Unlike __syncthreads() it does not wait for the
// wave's outstanding global loads and stores (which no other wave of the
// work group reads), so global traffic stays in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wait until this wave's global stores, atomics and loads have completed
// (vmcnt counts all of them on gfx9-family parts). A work group publishes data
// to other work groups by having every wave that wrote a part of it execute
// this before the barrier that precedes the flag store: s_barrier alone (and
// __syncthreads(), which compiles to it with an LDS wait only) lets a wave
// arrive with stores still in flight, so the flag could become visible first.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Order-preserving map of a float32 to uint32 (larger float, larger key).
// Negative zero is folded into positive zero so that the two compare equal.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// acc + a.lo * b.lo + a.hi * b.hi for two packed bf16 pairs (v_dot2, fp32 accumulation).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
}

// ---- cross-lane primitives on DPP row operations (no LDS traffic) ----
// A DPP "row" is 16 consecutive lanes. Lanes whose source is out of range
// read 0.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- 7 - i within each 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <- 15 - i within each row
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;

template <int Ctrl>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, Ctrl, 0xF, 0xF, false);
}
template <int Ctrl>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(dpp_i<Ctrl>(__float_as_int(x)));
}
template <int Ctrl>
__device__ __forceinline__ double dpp_d(double x) {
  const unsigned long long u = static_cast<unsigned long long>(__double_as_longlong(x));
  const int lo = dpp_i<Ctrl>(static_cast<int>(u & 0xffffffffull));
  const int hi = dpp_i<Ctrl>(static_cast<int>(u >> 32));
  return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(static_cast<unsigned>(hi)) << 32) |
                                                     static_cast<unsigned>(lo)));
}

// Sum / maximum over each 16-lane row; every lane of the row gets the result.
__device__ __forceinline__ float row_sum(float x) {
  x += dpp_f<kDppXor1>(x);
  x += dpp_f<kDppXor2>(x);
  x += dpp_f<kDppHalfMirror>(x);
  x += dpp_f<kDppMirror>(x);
  return x;
}
__device__ __forceinline__ double row_sum(double x) {
  x += dpp_d<kDppXor1>(x);
  x += dpp_d<kDppXor2>(x);
  x += dpp_d<kDppHalfMirror>(x);
  x += dpp_d<kDppMirror>(x);
  return x;
}
__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, dpp_f<kDppXor1>(x));
  x = fmaxf(x, dpp_f<kDppXor2>(x));
  x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
  x = fmaxf(x, dpp_f<kDppMirror>(x));
  return x;
}

__device__ __forceinline__ double row_max(double x) {
  x = fmax(x, dpp_d<kDppXor1>(x));
  x = fmax(x, dpp_d<kDppXor2>(x));
  x = fmax(x, dpp_d<kDppHalfMirror>(x));
  x = fmax(x, dpp_d<kDppMirror>(x));
  return x;
}

__device__ __forceinline__ double readlane_d(double x, int lane) {
  const unsigned long long u = static_cast<unsigned long long>(__double_as_longlong(x));
  const unsigned lo = __builtin_amdgcn_readlane(static_cast<int>(u & 0xffffffffull), lane);
  const unsigned hi = __builtin_amdgcn_readlane(static_cast<int>(u >> 32), lane);
  return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}

// Wave-wide sum (fixed order: rows 0+1, 2+3, then both), in every lane.
__device__ __forceinline__ double wave_sum_f64(double x) {
  x = row_sum(x);
  return (readlane_d(x, 0) + readlane_d(x, 16)) + (readlane_d(x, 32) + readlane_d(x, 48));
}

__device__ __forceinline__ double wave_max_f64(double x) {
  x = row_max(x);
  return fmax(fmax(readlane_d(x, 0), readlane_d(x, 16)), fmax(readlane_d(x, 32), readlane_d(x, 48)));
}

__device__ __forceinline__ float wave_max_f32(float x) {
  x = row_max(x);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_i<kDppShr1>(x);
  x += dpp_i<kDppShr2>(x);
  x += dpp_i<kDppShr4>(x);
  x += dpp_i<kDppShr8>(x);
  const int t0 = __builtin_amdgcn_readlane(x, 15);
  const int t1 = __builtin_amdgcn_readlane(x, 31);
  const int t2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row > 0 ? t0 : 0) + (row > 1 ? t1 : 0) + (row > 2 ? t2 : 0);
}

// Slot for every lane with `pred` in an LDS list whose length is *counter:
// one atomic per wave (ballot, then rank by mbcnt). The value is meaningful
// only where pred holds. Every lane of the wave must call it.
__device__ __forceinline__ int wave_slot(bool pred, int* counter) {
  const uint64_t m = __ballot(pred);
  const uint32_t lo = static_cast<uint32_t>(m), hi = static_cast<uint32_t>(m >> 32);
  const int rank = __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
  int base = 0;
  if (m != 0ull) {
    const int leader = __builtin_amdgcn_readfirstlane(__ffsll(static_cast<long long>(m)) - 1);
    if ((threadIdx.x & 63) == leader) base = atomicAdd(counter, __popcll(m));
    base = __builtin_amdgcn_readlane(base, leader);
  }
  return base + rank;
}

// Block-wide exclusive prefix sum of one int per thread. `tmp` holds at
// least kHeadThreads / 64 ints. With kTail, a barrier at the end lets the
// caller reuse tmp at once; without it, tmp must not be written again before
// the next barrier. Every thread of the block must call it.
template <bool kTail = true>
__device__ __forceinline__ int block_exclusive_scan(int v, int* total, int* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = kHeadThreads >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) tmp[wave] = incl;
  lds_barrier();
  int before = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    const int x = tmp[w];
    if (w < wave) before += x;
    tot += x;
  }
  if (kTail) lds_barrier();
  *total = tot;
  return before + incl - v;
}

// Block-wide minimum and maximum of one float per thread (tmp: 2 * waves floats).
__device__ __forceinline__ void block_minmax_f32(float lo, float hi, float* tmp, float* mn, float* mx) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = kHeadThreads >> 6;
  hi = wave_max_f32(hi);
  lo = -wave_max_f32(-lo);
  if (lane == 0) {
    tmp[2 * wave] = lo;
    tmp[2 * wave + 1] = hi;
  }
  lds_barrier();
  float a = kPosInf, b = kNegInf;
  for (int w = 0; w < nw; ++w) {
    a = fminf(a, tmp[2 * w]);
    b = fmaxf(b, tmp[2 * w + 1]);
  }
  lds_barrier();
  *mn = a;
  *mx = b;
}

// Two block-wide exclusive prefix sums at once (one pair of barriers). tmp:
// 2 * kHeadThreads / 64 ints.
__device__ __forceinline__ void block_exclusive_scan2(int a, int b, int* ea, int* eb, int* ta, int* tb, int* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = kHeadThreads >> 6;
  const int ia = wave_incl_scan(a), ib = wave_incl_scan(b);
  if (lane == 63) {
    tmp[2 * wave] = ia;
    tmp[2 * wave + 1] = ib;
  }
  lds_barrier();
  int pa = 0, pb = 0, sa = 0, sb = 0;
  for (int w = 0; w < nw; ++w) {
    const int xa = tmp[2 * w], xb = tmp[2 * w + 1];
    if (w < wave) {
      pa += xa;
      pb += xb;
    }
    sa += xa;
    sb += xb;
  }
  lds_barrier();
  *ea = pa + ia - a;
  *eb = pb + ib - b;
  *ta = sa;
  *tb = sb;
}

// Whether p holds in every thread of the block; also a barrier. votes: two
// sets of per-wave words, used in turn (par flips at each call, in every
// thread alike), so that a wave casting the next vote cannot overwrite one
// that a slower wave is still reading. Every thread of the block must call it.
__device__ __forceinline__ bool block_all(bool p, int* votes, int& par) {
  int* v = votes + par * (kHeadThreads / 64);
  par ^= 1;
  const uint64_t m = __ballot(!p);
  if ((threadIdx.x & 63) == 0) v[threadIdx.x >> 6] = m != 0ull ? 1 : 0;
  lds_barrier();
  int any = 0;
#pragma unroll
  for (int w = 0; w < kHeadThreads / 64; ++w) any |= v[w];
  return any == 0;
}

__device__ __forceinline__ float block_max_f32(float v, float* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = kHeadThreads >> 6;
  v = wave_max_f32(v);
  if (lane == 0) tmp[wave] = v;
  lds_barrier();
  float m = kNegInf;
  for (int w = 0; w < nw; ++w) m = fmaxf(m, tmp[w]);
  lds_barrier();
  return m;
}

// LDS bitmap windows of kBitmapWords words. Each thread owns a slice of 16
// consecutive words; word w is stored at w + w/16 so that the 64 lanes of a
// wave reading "their" i-th word hit distinct banks.
constexpr int kSliceWords = kBitmapWords / kHeadThreads;
static_assert(kSliceWords == 16, "bitmap slice layout");
constexpr int kBitmapLdsWords = kBitmapWords + kBitmapWords / kSliceWords;

__device__ __forceinline__ int bm_at(int w) { return w + (w >> 4); }

__device__ __forceinline__ void bitmap_clear(uint32_t* bm) {
  uint32_t* p = bm + threadIdx.x * (kSliceWords + 1);
#pragma unroll
  for (int i = 0; i <= kSliceWords; ++i) p[i] = 0u;
}

__device__ __forceinline__ void bitmap_set(uint32_t* bm, int x) { atomicOr(&bm[bm_at(x >> 5)], 1u << (x & 31)); }

// Per-word prefix counts of an LDS bitmap window, for ranking its set bits.
// Thread t owns the slice of words 16t .. 16t+15 (the layout bitmap_clear
// clears). pfx receives, for every word w, the number of set bits in words
// [0, w), as 16-bit counts packed two per dword, with one pad dword after
// every 32 so that the 64 lanes' stores spread over the banks. Returns the
// total number of set bits (the same value in every thread). Ends with a
// barrier. Every thread of the block must call it.
constexpr int kPfxDwords = kBitmapWords / 2 + kBitmapWords / 64;
__device__ __forceinline__ int bitmap_prefix(const uint32_t* bm, uint32_t* pfx, int* tmp) {
  const int t = threadIdx.x;
  const uint32_t* p = bm + t * (kSliceWords + 1);
  int c[kSliceWords];
  int run = 0;
#pragma unroll
  for (int i = 0; i < kSliceWords; ++i) {
    c[i] = run;
    run += __popc(p[i]);
  }
  int tot;
  const int base = block_exclusive_scan<false>(run, &tot, tmp);  // (tmp is next written after the barrier below)
  uint32_t* o = pfx + t * (kSliceWords / 2) + (t >> 2);
#pragma unroll
  for (int i = 0; i < kSliceWords / 2; ++i)
    o[i] = static_cast<uint32_t>(base + c[2 * i]) | (static_cast<uint32_t>(base + c[2 * i + 1]) << 16);
  lds_barrier();
  return tot;
}

// Rank of set bit y of the window among its set bits (the number of set bits
// below it), from the prefix counts of bitmap_prefix.
__device__ __forceinline__ int bitmap_rank(const uint32_t* bm, const uint32_t* pfx, int y) {
  const int w = y >> 5;
  const uint32_t below = (pfx[(w >> 1) + (w >> 6)] >> ((w & 1) << 4)) & 0xffffu;
  return static_cast<int>(below) + __popc(bm[bm_at(w)] & ((1u << (y & 31)) - 1u));
}

// First dynamic-LDS region of the head kernel: the bitmap window, later S_hat
// with its scores (8K bytes) and one flag byte per candidate.
__host__ __device__ inline size_t head_region0(const Dims& d) {
  const size_t sel = 8 * static_cast<size_t>(d.K) + static_cast<size_t>(d.cand_cap);
  const size_t bm = static_cast<size_t>(kBitmapLdsWords) * 4;
  return ((bm > sel ? bm : sel) + 15) / 16 * 16;
}

// Shared scratch of the per-head kernels (static LDS).
struct HeadShared {
  float q[kHeadDim];                   // raw query as float
  float qbar[kHeadDim];                // normalised query
  double rho[64];                      // rho of each held entry, by FIFO position
  int len[64];                         // support size of each ring slot
  int rslot[64];                       // ring slots of the retrieved entries, best first
  int moff[65];                        // merged union: start of each retrieved list's part below the window
  __align__(16) int whist[kHeadThreads / 64][256];   // one radix histogram per wave
  int tmp[32];
  __align__(16) float red[kHeadThreads / 16][kHeadDim + 4];  // one row per 16-lane row group (before
                                                             // that, the union's bitmap prefix counts)
  int i0, i1, i2, i3;
  int vote[2 * (kHeadThreads / 64)];  // block_all's votes
};
static_assert(sizeof(HeadShared::red) >= kPfxDwords * 4, "bitmap prefix counts in the reduction rows");
// the per-head kernels add at most 2 KiB of their own to it; LDS is 160 KiB per work group
static_assert(sizeof(HeadShared) + 2048 + kLdsLimit <= 160 * 1024, "static + dynamic LDS of a per-head kernel");

// Wave 0 turns the per-wave histograms into the digit holding the rem-th
// largest key (digits scanned from 255 down): sh.i0 = digit, sh.i1 = rank
// within it, sh.i2 = its count. Called by every thread; only wave 0 works.
__device__ __forceinline__ void pick_digit(HeadShared& sh, int rem) {
  const int lane = threadIdx.x & 63;
  if ((threadIdx.x >> 6) != 0) return;
  // lane owns digits 255-4*lane .. 252-4*lane, read as one 128-bit word per wave histogram
  int4 acc = make_int4(0, 0, 0, 0);
#pragma unroll
  for (int w = 0; w < kHeadThreads / 64; ++w) {
    const int4 h = *reinterpret_cast<const int4*>(&sh.whist[w][252 - 4 * lane]);
    acc.x += h.x;
    acc.y += h.y;
    acc.z += h.z;
    acc.w += h.w;
  }
  const int c[4] = {acc.w, acc.z, acc.y, acc.x};  // digits 255-4l, 254-4l, 253-4l, 252-4l
  const int s4 = c[0] + c[1] + c[2] + c[3];
  int run = wave_incl_scan(s4) - s4;
  if (run < rem && run + s4 >= rem) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (run + c[j] >= rem) {
        sh.i0 = 255 - 4 * lane - j;
        sh.i1 = rem - run;
        sh.i2 = c[j];
        break;
      }
      run += c[j];
    }
  }
}

// From a 2048-bin histogram in sh.whist, the bin holding the rem-th largest
// (bins scanned from 2047 down): sh.i0 = bin, sh.i1 = rank within it, sh.i2 =
// its count. Every thread of a 512-thread block must call it; ends with a
// barrier.
__device__ __forceinline__ void pick_bin2048(HeadShared& sh, int rem) {
  const int* bins = &sh.whist[0][0];
  const int4 h = reinterpret_cast<const int4*>(bins)[511 - threadIdx.x];  // bins 2047-4t .. 2044-4t
  const int c[4] = {h.w, h.z, h.y, h.x};
  const int s4 = c[0] + c[1] + c[2] + c[3];
  int tot;
  int run = block_exclusive_scan<false>(s4, &tot, sh.tmp);  // (tmp is next written after the barrier below)
  if (run < rem && run + s4 >= rem) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (run + c[j] >= rem) {
        sh.i0 = 2047 - 4 * static_cast<int>(threadIdx.x) - j;
        sh.i1 = rem - run;
        sh.i2 = c[j];
        break;
      }
      run += c[j];
    }
  }
  lds_barrier();
}

__device__ __forceinline__ void clear_whist(HeadShared& sh) {
  int4* w = reinterpret_cast<int4*>(&sh.whist[0][0]);
  for (int i = threadIdx.x; i < (kHeadThreads / 64) * 64; i += kHeadThreads) w[i] = make_int4(0, 0, 0, 0);
}

// Radix select of the k largest of n scores (LDS) under (score desc,
// position asc) on the order-preserving keys: a first pass over the top 11
// bits (2048 bins), then 8-, 8- and 5-bit passes over the remaining bits,
// stopping as soon as every remaining candidate is needed. On return the
// kept entries are those with (key & *mask) > T, plus the first *need (by
// position) with (key & *mask) == T. Every thread of the block must call it.
__device__ __forceinline__ uint32_t radix_kth(const float* sc, int n, int k, HeadShared& sh, uint32_t* mask_out,
                                              int* need) {
  const int wave = threadIdx.x >> 6;
  int* bins = &sh.whist[0][0];  // 2048 bins for the first pass
  reinterpret_cast<int4*>(bins)[threadIdx.x] = make_int4(0, 0, 0, 0);
  lds_barrier();
  for (int i = threadIdx.x; i < n; i += kHeadThreads) atomicAdd(&bins[order_key(sc[i]) >> 21], 1);
  lds_barrier();
  {
    const int4 h = reinterpret_cast<const int4*>(bins)[511 - threadIdx.x];  // bins 2047-4t .. 2044-4t
    const int c[4] = {h.w, h.z, h.y, h.x};
    const int s4 = c[0] + c[1] + c[2] + c[3];
    int tot;
    int run = block_exclusive_scan<false>(s4, &tot, sh.tmp);  // (tmp is next written after the barrier below)
    if (run < k && run + s4 >= k) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (run + c[j] >= k) {
          sh.i0 = 2047 - 4 * static_cast<int>(threadIdx.x) - j;
          sh.i1 = k - run;
          sh.i2 = c[j];
          break;
        }
        run += c[j];
      }
    }
    lds_barrier();
  }
  uint32_t prefix = static_cast<uint32_t>(sh.i0) << 21, mask = 0x7FFu << 21;
  int rem = sh.i1, ncand = sh.i2;
  const int shifts[3] = {13, 5, 0};
  for (int p = 0; p < 3 && ncand > rem; ++p) {
    const int shift = shifts[p];
    const uint32_t dmask = shift == 0 ? 31u : 255u;
    clear_whist(sh);
    lds_barrier();
    for (int i = threadIdx.x; i < n; i += kHeadThreads) {
      const uint32_t u = order_key(sc[i]);
      if ((u & mask) == prefix) atomicAdd(&sh.whist[wave][(u >> shift) & dmask], 1);
    }
    lds_barrier();
    pick_digit(sh, rem);
    lds_barrier();
    prefix |= static_cast<uint32_t>(sh.i0) << shift;
    mask |= dmask << shift;
    rem = sh.i1;
    ncand = sh.i2;
  }
  *mask_out = mask;
  *need = rem;
  return prefix;
}

// Keep, in position order, the entries with (key & mask) > T and the first
// `need` entries with (key & mask) == T; write idx[i] of the kept positions
// to out_idx and g_idx, their weight exp((sc[i] - mx) / sqrt(d)) to out_w and
// sc[i] to g_sc. Returns the number kept. Every thread must call it.
__device__ __forceinline__ int select_in_order(const int32_t* idx, const float* sc, int n, uint32_t T, uint32_t mask,
                                               int need, float mx, int32_t* out_idx, float* out_w, int32_t* g_idx,
                                               float* g_sc, HeadShared& sh) {
  const int per = (n + kHeadThreads - 1) / kHeadThreads;
  const int i0 = threadIdx.x * per, i1 = min(i0 + per, n);
  int gt = 0, eq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t u = order_key(sc[i]) & mask;
    gt += u > T;
    eq += u == T;
  }
  int tot;
  const int pre = block_exclusive_scan<false>((eq << 16) | gt, &tot, sh.tmp);  // n < 2^15; barrier below
  int e = pre >> 16;
  int o = (pre & 0xffff) + min(e, need);
  for (int i = i0; i < i1; ++i) {
    const uint32_t u = order_key(sc[i]) & mask;
    if ((u > T) || (u == T && e < need)) {
      out_idx[o] = idx[i];
      out_w[o] = expf((sc[i] - mx) * kInvSqrtD);
      g_idx[o] = idx[i];
      g_sc[o] = sc[i];
      ++o;
    }
    e += (u == T);
  }
  lds_barrier();
  return (tot & 0xffff) + min(tot >> 16, need);
}

// Rerank (Eq. 11) of M > K candidates in LDS, first pass on scores binned
// linearly between their minimum mn and maximum mx (mx > mn): the bin of a
// score is monotone in the score, so every bin above the one holding the
// K-th largest is kept whole. When only some entries of that boundary bin are
// kept (at most 64 of them), one wave ranks them exactly by (score desc,
// index asc) and flags the kept ones. The kept entries are written in
// candidate order (ascending index): their indices to out_idx and g_idx,
// their weights exp((sc - mx) / sqrt(d)) to out_w and their scores to g_sc.
// Returns K, or -1 (nothing written) when the boundary bin is too crowded,
// for the caller's order-key radix select. The caller zeroes the 2048 bins
// (sh.whist) and sh.i3 beforehand, with a barrier since. flag: M bytes of LDS
// scratch. Every thread must call it.
__device__ __forceinline__ int rerank_linear(const int32_t* idx, const float* sc, int M, int K, float mn, float mx,
                                             int32_t* out_idx, float* out_w, int32_t* g_idx, float* g_sc,
                                             uint8_t* flag, HeadShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float scale = 2048.f / (mx - mn);
  auto bin_of = [&](float v) { return min(2047, static_cast<int>((v - mn) * scale)); };
  int* bins = &sh.whist[0][0];  // 2048 bins
  for (int i = tid; i < M; i += kHeadThreads) atomicAdd(&bins[bin_of(sc[i])], 1);
  lds_barrier();
  if (wave == 0) {
    // the bin holding the K-th largest, from the top: lane l sums bins
    // 2047 - 32l .. 2016 - 32l; then the lanes take the 32 bins of the lane
    // where the count reaches K, one each (M > K, so there is one)
    const int4* b4 = reinterpret_cast<const int4*>(bins) + (2016 - 32 * lane) / 4;
    int s32 = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int4 h = b4[k];
      s32 += h.x + h.y + h.z + h.w;
    }
    const int incl = wave_incl_scan(s32);
    const int L = __ffsll(static_cast<long long>(__ballot(incl - s32 < K && incl >= K))) - 1;
    const int runL = __builtin_amdgcn_readlane(incl - s32, L);
    const int c = lane < 32 ? bins[2047 - 32 * L - lane] : 0;
    const int ci = wave_incl_scan(c);
    const int j = __ffsll(static_cast<long long>(__ballot(lane < 32 && runL + ci >= K))) - 1;
    if (lane == j) {
      sh.i0 = 2047 - 32 * L - j;
      sh.i1 = K - (runL + ci - c);
      sh.i2 = c;
    }
  }
  lds_barrier();
  const int b1 = sh.i0, need = sh.i1, cnt = sh.i2;
  if (need < cnt) {
    if (cnt > 64) return -1;  // uniform
    // the boundary bin's entries, listed by one wave-aggregated pass
    for (int i0 = 0; i0 < M; i0 += kHeadThreads) {
      const int i = i0 + tid;
      const bool in = i < M && bin_of(sc[min(i, M - 1)]) == b1;
      const int o = wave_slot(in, &sh.i3);
      if (in) sh.rslot[o] = i;
    }
    lds_barrier();
    if (wave == 0) {
      const int p = sh.rslot[min(lane, cnt - 1)];
      const float v = sc[p];
      const int x = idx[p];
      int rank = 0;
      for (int j = 0; j < cnt; ++j) {
        const float u = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
        const int y = __builtin_amdgcn_readlane(x, j);
        rank += (u > v) || (u == v && y < x);
      }
      if (lane < cnt) flag[p] = rank < need ? 1 : 0;
    }
    lds_barrier();
  }
  // kept: bin > b1, or bin == b1 and (all of the bin kept, or flagged)
  const int per = (M + kHeadThreads - 1) / kHeadThreads;
  const int i0 = tid * per, i1 = min(i0 + per, M);
  auto kept = [&](int i) {
    const int bn = bin_of(sc[i]);
    return bn > b1 || (bn == b1 && (need == cnt || flag[i] != 0));
  };
  int k = 0;
  for (int i = i0; i < i1; ++i) k += kept(i);
  int tot;
  int o = block_exclusive_scan<false>(k, &tot, sh.tmp);  // (tmp is next written after the barrier below)
  for (int i = i0; i < i1; ++i) {
    if (kept(i)) {
      out_idx[o] = idx[i];
      out_w[o] = expf((sc[i] - mx) * kInvSqrtD);
      g_idx[o] = idx[i];
      g_sc[o] = sc[i];
      ++o;
    }
  }
  lds_barrier();
  return tot;
}

// End of softmax-V: every thread holds the weighted sums of 8 value dims
// (lane & 15 picks the dims) over its rows and, in lane & 15 == 0, the sum of
// their weights. Each 16-lane row group stores one row of sh.red; then 128
// threads add the rows of one dim each (conflict-free LDS columns) and write
// out (see attend). Every thread of the block must call it.
__device__ __forceinline__ void attend_reduce(float (&acc)[8], float z, float* out, float* out_z, HeadShared& sh) {
  const int sub = threadIdx.x & 15, rg = threadIdx.x >> 4, nrg = kHeadThreads >> 4;
  float4* r = reinterpret_cast<float4*>(&sh.red[rg][8 * sub]);
  r[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  r[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  if (sub == 0) sh.red[rg][kHeadDim] = z;
  lds_barrier();
  if (out != nullptr && threadIdx.x < kHeadDim) {
    float a = 0.f, zz = 0.f;
    for (int g2 = 0; g2 < nrg; ++g2) {
      a += sh.red[g2][threadIdx.x];
      zz += sh.red[g2][kHeadDim];
    }
    if (out_z == nullptr) {
      out[threadIdx.x] = zz > 0.f ? a / zz : 0.f;  // an empty support gives the zero vector
    } else {
      out[threadIdx.x] = a;
      if (threadIdx.x == 0) *out_z = zz;
    }
  }
  lds_barrier();
}

// Sparse softmax-V (Eq. 12) over n selected rows (indices and unscaled
// scores in LDS; mx = the maximum over the whole support). The scores are
// first replaced in place by their weights exp((s - mx) / sqrt(d)), one
// thread per row; then 16 lanes per value row (16 bytes each), 16 row loads
// in flight per thread. With out_z NULL it writes the normalised output
// out[0 .. 127]; otherwise the unnormalised sums to out[0 .. 127] and the sum
// of the weights to *out_z, so that disjoint slices of one support can be
// merged by adding them. Nothing is written when out is NULL. Every thread of
// the block must call it.
__device__ __forceinline__ void attend_w(const int32_t* sel, const float* sc, int n, const uint16_t* vb, float* out,
                                         float* out_z, HeadShared& sh);
__device__ __forceinline__ void attend(const int32_t* sel, float* sc, int n, float mx, const uint16_t* vb, float* out,
                                       float* out_z, HeadShared& sh) {
  for (int i = threadIdx.x; i < n; i += kHeadThreads) sc[i] = expf((sc[i] - mx) * kInvSqrtD);
  lds_barrier();
  attend_w(sel, sc, n, vb, out, out_z, sh);
}

// The same with the weights already in sc[0 .. n) (LDS, published by a
// barrier). Every thread of the block must call it.
__device__ __forceinline__ void attend_w(const int32_t* sel, const float* sc, int n, const uint16_t* vb, float* out,
                                         float* out_z, HeadShared& sh) {
  const int sub = threadIdx.x & 15, rg = threadIdx.x >> 4, rpr = kHeadThreads >> 4;
  constexpr int U = 16;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float z = 0.f;
  for (int r0 = 0; r0 < n; r0 += rpr * U) {
    uint4 w[U];
    float p[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // clamped row: always a valid address, weight 0 past the end
      const int i = min(r0 + u * rpr + rg, n - 1);
      w[u] = *reinterpret_cast<const uint4*>(vb + static_cast<long>(sel[i]) * kHeadDim + 8 * sub);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = r0 + u * rpr + rg;
      p[u] = (i < n) ? sc[min(i, n - 1)] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc[0] = fmaf(p[u], bf16_lo(w[u].x), acc[0]);
      acc[1] = fmaf(p[u], bf16_hi(w[u].x), acc[1]);
      acc[2] = fmaf(p[u], bf16_lo(w[u].y), acc[2]);
      acc[3] = fmaf(p[u], bf16_hi(w[u].y), acc[3]);
      acc[4] = fmaf(p[u], bf16_lo(w[u].z), acc[4]);
      acc[5] = fmaf(p[u], bf16_hi(w[u].z), acc[5]);
      acc[6] = fmaf(p[u], bf16_lo(w[u].w), acc[6]);
      acc[7] = fmaf(p[u], bf16_hi(w[u].w), acc[7]);
      if (sub == 0) z += p[u];
    }
  }
  attend_reduce(acc, z, out, out_z, sh);
}

// q_bar = x / ||x|| (Eqs. 5-6) of one bf16 query row, by one wave: w2 holds
// elements 2l and 2l+1 in lane l, which gets their normalised values. Sum of
// squares, square root and division in fp64, one rounding to fp32; the zero
// query gives 0. The head and the score work groups both call it, so both
// get the same bits without a hand-off.
__device__ __forceinline__ void normalize_row(uint32_t w2, float& qb0, float& qb1) {
  const double x0 = bf16_lo(w2), x1 = bf16_hi(w2);
  const double nrm = sqrt(wave_sum_f64(x0 * x0 + x1 * x1));
  qb0 = 0.f;
  qb1 = 0.f;
  if (nrm > 0.0) {
    qb0 = static_cast<float>(x0 / nrm);
    qb1 = static_cast<float>(x1 / nrm);
  }
}

// Push (q_bar_t, S_hat_t) into the head's FIFO (Query-support cache
// paragraph: after either path; the oldest entry is overwritten when full).
// slot / count: the FIFO state read at the start of the kernel (the caller's
// threads must not re-read it here, since thread 0 updates it).
template <typename Table>
__device__ __forceinline__ void cache_push(const Dims& d, Table& b, int bh, int slot, int count, const float* qbar,
                                           const int32_t* sel, int n) {
  const long e = static_cast<long>(bh) * d.C + slot;
  for (int t = threadIdx.x; t < kHeadDim; t += kHeadThreads) b.cache_qbar[e * kHeadDim + t] = qbar[t];
  for (int i = threadIdx.x; i < n; i += kHeadThreads) b.cache_supp[e * d.K + i] = sel[i];
  if (threadIdx.x == 0) {
    b.cache_len[e] = n;
    b.fifo[2 * bh] = (slot + 1) % d.C;
    b.fifo[2 * bh + 1] = min(count + 1, d.C);
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) float lds_float;  // a float in LDS (ds_* accesses)
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

}  // namespace

size_t head_lds_bytes(const Dims& d) {
  return head_region0(d) + 8 * static_cast<size_t>(d.cand_cap);
}

size_t score_lds_bytes(const Dims& d) { return static_cast<size_t>(d.G) * kNumBins * 4; }

// Every launch takes kLdsLimit: one 512-thread work group per CU is resident
// anyway (registers), and a score work group keeps its scores in what its
// histograms leave free.
size_t step_lds_bytes(const Dims& d) {
  return std::max({head_lds_bytes(d), score_lds_bytes(d), finish_lds_bytes(d), static_cast<size_t>(kLdsLimit)});
}

size_t finish_lds_bytes(const Dims& d) {
  const size_t nw = static_cast<size_t>(std::min(d.n_cu, kHeadThreads));
  return 8 * static_cast<size_t>(kBoundaryLds) + 4 * ((nw + 4) / 4 * 4 + (nw + 3) / 4 * 4) +
         8 * static_cast<size_t>(d.K);
}

constexpr long kLongShare = 8192;  // key rows per score work group from which exact calls take every CU
constexpr int kKbDecodeLen = 1 << 21;  // visible keys from which decode steps use the K-best variant

int score_grid(const Dims& d, int length, int mode, bool wide) {
  // One 512-thread work group per CU beside the head work groups, so that all
  // are resident at once and none starts late (a reuse head's work group holds
  // its CU for the whole reuse path), but at least half the CUs. Exact calls
  // with many heads, and decode steps expected to be mostly exact, take every
  // CU instead: their head work groups only publish the decision and leave,
  // and half the CUs cannot stream the keys at the HBM rate (with few heads
  // the late starters cost more than they add). At most one per thread of a
  // work group (the finish reads one segment per thread), and never more than
  // the CUs, so that all score work groups, which wait for one another, can be
  // resident together.
  const long bh = static_cast<long>(d.B) * d.Hq;
  // (an exact call whose share per work group is long: the head work groups'
  // CUs are free within a few us, and the scan then gains their bandwidth)
  const long share = static_cast<long>(d.B) * d.Hkv * length / std::max<long>(1, d.n_cu - bh);
  const bool all_cu = ((mode == kModeExact || wide) && bh >= d.n_cu / 8) || (mode == kModeExact && share >= kLongShare);
  const long free_cu = all_cu ? d.n_cu : std::max<long>(d.n_cu - bh, d.n_cu / 2);
  const long cap = std::min<long>(free_cu, kHeadThreads);
  const long groups = static_cast<long>(d.B) * d.Hkv;
  const long want = groups * ((length + kExactMinRows - 1) / kExactMinRows);
  return static_cast<int>(std::max(1L, std::min(cap, want)));
}

int score_keep_rows(const Dims& d, int length, int n_score) {
  // the largest share a score work group can get (every KV group exact), its
  // segments each starting at a 16-row boundary of LDS
  const long T = static_cast<long>(d.B) * d.Hkv * length;
  const long rows = (T + n_score - 1) / n_score + 16;
  const long segs = (rows + length - 1) / length + 1;
  const long keep = (rows + 16 * segs + 15) / 16 * 16;
  const long bytes = static_cast<long>(d.G) * kNumBins * 4 + static_cast<long>(d.G) * (keep + 4) * 4;
  return bytes <= kLdsLimit ? static_cast<int>(keep) : 0;
}
// static LDS of k_step: the head role's shared state and rank table, the score
// role's group list and exact bits, the survivor pass's boundaries
static_assert(sizeof(HeadShared) + 2048 + 4 * 1024 + 2048 + 512 + kLdsLimit <= 160 * 1024, "k_step LDS");

// ---------------------------------------------------------------------------
// Reset the FIFO bookkeeping before cache initialisation. One thread per head.
// ---------------------------------------------------------------------------
__global__ void k_reset(Dims d, Bufs b) {
  const int bh = blockIdx.x * blockDim.x + threadIdx.x;
  if (bh >= d.B * d.Hq) return;
  b.fifo[2 * bh] = 0;
  b.fifo[2 * bh + 1] = 0;
}

namespace {
// Data handed from one work group to another inside a launch goes through
// device-scope (sc1) stores and loads, which are coherent across the XCDs'
// L2s on their own (as are the device-scope atomics): a hand-off then needs
// only the stores to be complete before the flag or counter that publishes
// them, not a whole-L2 write-back and invalidate.
__device__ __forceinline__ void store_shared(uint2* p, uint2 v) {
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p),
                     (static_cast<unsigned long long>(v.y) << 32) | v.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_shared(int32_t* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint2 load_shared(const uint2* p) {
  const unsigned long long u = __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
  return make_uint2(static_cast<uint32_t>(u), static_cast<uint32_t>(u >> 32));
}
__device__ __forceinline__ int load_shared(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_shared(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_shared(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// two consecutive floats (8-byte aligned) as one device-scope store
__device__ __forceinline__ void store_shared2(float* p, float a, float b) {
  store_shared(reinterpret_cast<uint2*>(p), make_uint2(__float_as_uint(a), __float_as_uint(b)));
}

constexpr int kPollSleep = 2;                 // s_sleep between polls of a flag (128 clocks, about 0.05 us)
constexpr long long kWaitTicks = 20000000;    // give up a wait after 200 ms (s_memrealtime is 100 MHz)

constexpr int kQkUnroll = 4;  // 16-row tiles per wave per stage: 512 rows per 8-wave work group

struct QkTiles {
  uint4 a[kQkUnroll][4];
};

__device__ __forceinline__ void qk_load(QkTiles& t, const uint16_t* kb, int t0, int rend, int wave, int nw, int j,
                                        int kq) {
#pragma unroll
  for (int u = 0; u < kQkUnroll; ++u) {
    const int r = min(t0 + (u * nw + wave) * 16 + j, rend - 1);
    const uint16_t* row = kb + static_cast<long>(r) * kHeadDim + 8 * kq;
#pragma unroll
    for (int s = 0; s < 4; ++s) t.a[u][s] = *reinterpret_cast<const uint4*>(row + 32 * s);
  }
}

// Row r goes to ldst[r + off] (to_lds) or gdst[r + off]: two typed pointers,
// so that each store is a plain LDS or global store.
__device__ __forceinline__ void qk_score(const QkTiles& t, const bf16x8 (&bq)[4], int t0, int rend, int wave, int nw,
                                         int kq, bool hv, bool to_lds, lds_float* ldst, float* gdst, int off,
                                         uint32_t* hrow) {
#pragma unroll
  for (int u = 0; u < kQkUnroll; ++u) {
    const int rbase = t0 + (u * nw + wave) * 16;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(t.a[u][s]), bq[s], acc, 0, 0, 0);
    // lane holds query head j for rows rbase + 4*kq + 0..3
    if (hv) {
      const int r = rbase + 4 * kq;
      if (r + 3 < rend) {
        if (to_lds)
          *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(ldst + r + off) = acc;
        else
          *reinterpret_cast<f32x4*>(gdst + r + off) = acc;
#pragma unroll
        for (int e = 0; e < 4; ++e) atomicAdd(&hrow[order_key(acc[e]) >> kHistShift], 1u);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (r + e < rend) {
            if (to_lds)
              ldst[r + e + off] = acc[e];
            else
              gdst[r + e + off] = acc[e];
            atomicAdd(&hrow[order_key(acc[e]) >> kHistShift], 1u);
          }
        }
      }
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// K1, one work group per query head: recall, path decision and the whole
// reuse path.
//
// Recall (Eqs. 5-7): q_bar = fp32(x / ||x||) with fp64 sum of squares, sqrt
// and divide; rho = fp64 dot of the fp32 q_bar values for every ring slot
// (16 threads per slot, all slots loaded at once); R_t = the R largest rho
// over the held entries, ranked by counting in parallel over all waves (ties:
// older entry); rho_max. Path (Eq. 13): exact if refresh, empty cache or
// rho_max < tau. Exact heads clear their score histogram and stop.
//
// Reuse heads, same work group:
//   union (Eqs. 8-9): retrieved supports and the window [max(0, L-W), L) set
//     bits of an LDS bitmap over token positions (windows of 262144), read
//     back in ascending order -> A_t, M_t;
//   scores (Eq. 10): q . k_i for i in A_t straight from the KV cache, 16 lanes
//     per key row, 18 rows in flight per 16-lane group, bf16 pair products with fp32
//     accumulation;
//   rerank (Eq. 11): a pass over scores binned linearly between their minimum
//     and maximum finds the bin of the K-th largest, whose entries are ranked
//     exactly (else a radix select on the ordered keys); kept in candidate
//     (= ascending index) order, ties to the lower index;
//   softmax-V (Eq. 12) and the cache update.
//
// In kModeExact (no cache: the exact Top-K baseline and the cache
// initialisation) every head is exact.
//
// LDS (dynamic): region0 = bitmap window (34 KiB), later S_hat and its scores
// (K each) and one flag byte per candidate; then A_t and its scores
// (cand_cap each).
// ---------------------------------------------------------------------------
constexpr int kCandU = 18;     // candidate rows per 16-lane group in flight: 576 per round
constexpr int kCandWide = 24;  // ... for 577 .. 768 candidates: one round of 768

// Candidate scores (Eq. 10): 16 lanes per key row (16 bytes each), U rows in
// flight per 16-lane group, bf16 pair products accumulated in fp32 (dot2).
// Every thread of the block must call it.
template <int U>
__device__ __forceinline__ void cand_scores(const uint16_t* kb, const int32_t* s_cand, int M, uint4 qw, int rg,
                                            int rpr, int part, float* s_sc, float& mn, float& mx) {
  for (int r0 = 0; r0 < M; r0 += rpr * U) {
    uint4 kv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = min(r0 + u * rpr + rg, M - 1);  // clamped: a valid row, its score is not stored
      kv[u] = *reinterpret_cast<const uint4*>(kb + static_cast<long>(s_cand[i]) * kHeadDim + 8 * part);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = r0 + u * rpr + rg;
      float sc = dot2_bf16(kv[u].x, qw.x, 0.f);
      sc = dot2_bf16(kv[u].y, qw.y, sc);
      sc = dot2_bf16(kv[u].z, qw.z, sc);
      sc = dot2_bf16(kv[u].w, qw.w, sc);
      sc = row_sum(sc);
      if (i < M) {
        if (part == 0) s_sc[i] = sc;
        mn = fminf(mn, sc);
        mx = fmaxf(mx, sc);
      }
    }
  }
}
constexpr int kMergeR = 8;                      // retrieved lists the merged union takes
constexpr int kMergeE = 4;                      // entries per thread: R K <= 4 * 512

// Candidate union (Eqs. 8-9) below the window by merging the retrieved
// supports, each held in ascending order (the cache's canonical form): its
// cost depends on R K, not on the context length (one LDS bitmap window
// covers 262144 positions; longer contexts would need a sweep per window).
// The n_ret <= kMergeR lists are staged in LDS (lists, K ints each) and cut
// at the first entry >= wlo (the window [wlo, L) is appended after; entries
// past the visible length lie beyond it too). Each thread takes up to kMergeE
// consecutive entries and finds, for each entry x and each list, the number
// of that list's entries below x: all these searches advance together, one
// power-of-two step per round. An entry is kept unless a lower-numbered list
// holds x; its place in the output is the sum over the lists of the kept
// entries below x (a prefix count of the kept flags, pre). Writes the
// distinct positions ascending to out and returns their number. Requires
// n_ret * K <= kMergeE * 512. Every thread of the block must call it.
template <int NR>
__device__ __forceinline__ int union_merge_n(const Dims& d, ConstBufs& b, int bh, int n_ret, int wlo, int32_t* out,
                                             int* lists, int* pre, HeadShared& sh) {
  const int tid = threadIdx.x;
  for (int j0 = 0; j0 < d.K; j0 += kHeadThreads) {
    const int j = j0 + tid;
    for (int r0 = 0; r0 < n_ret; r0 += 4) {
      int x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = min(r0 + u, n_ret - 1);  // clamped: a valid address, not stored when out of range
        x[u] = b.cache_supp[(static_cast<long>(bh) * d.C + sh.rslot[r]) * d.K + min(j, d.K - 1)];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = r0 + u;
        if (r < n_ret && j < sh.len[sh.rslot[min(r, n_ret - 1)]]) lists[r * d.K + j] = x[u];
      }
    }
  }
  lds_barrier();
  // list r (lane r of wave 0): its entries below wlo, then their offsets
  if (tid < 64) {
    const int len = tid < n_ret ? sh.len[sh.rslot[tid]] : 0;
    const int* L = lists + min(tid, n_ret - 1) * d.K;
    int cut = 0;
    for (int st = kHeadThreads * kMergeE; st > 0; st >>= 1) {
      const int c = cut + st;
      const int x = L[max(min(c, len) - 1, 0)];
      cut = (c <= len && x < wlo) ? c : cut;
    }
    const int incl = wave_incl_scan(cut);
    if (tid < NR) sh.moff[tid + 1] = incl;  // (a list past n_ret: empty, at F)
    if (tid == 0) sh.moff[0] = 0;
  }
  lds_barrier();
  int nmax = 0;
  for (int r = 0; r < n_ret; ++r) nmax = max(nmax, sh.moff[r + 1] - sh.moff[r]);
  const int F = sh.moff[n_ret];
  const int f0 = min(tid * kMergeE, F);
  int xe[kMergeE], re[kMergeE];
  {
    int r = 0;
#pragma unroll
    for (int e = 0; e < kMergeE; ++e) {
      const int f = min(f0 + e, max(F - 1, 0));
      while (r + 1 < n_ret && sh.moff[r + 1] <= f) ++r;
      re[e] = r;
      xe[e] = F > 0 ? lists[r * d.K + (f - sh.moff[r])] : 0;
    }
  }
  // lb[e][r2]: entries of list r2 below xe[e]
  int lb[kMergeE][NR];
#pragma unroll
  for (int e = 0; e < kMergeE; ++e)
#pragma unroll
    for (int r2 = 0; r2 < NR; ++r2) lb[e][r2] = 0;
  int step = 1;
  while (step * 2 <= nmax) step *= 2;
  // NR lists, those past n_ret empty (their searches never move) and read at
  // list 0: no branch depends on n_ret, which keeps the loop's uniform values
  // few (a branch per list held a lane mask per list through the loop)
  int nl[NR], lo[NR];
#pragma unroll
  for (int r2 = 0; r2 < NR; ++r2) {
    nl[r2] = sh.moff[r2 + 1] - sh.moff[r2];
    lo[r2] = (r2 < n_ret ? r2 : 0) * d.K;
  }
  // (every read is issued unconditionally at a clamped, valid index, so that
  // a round's reads are all in flight together)
  for (; step > 0; step >>= 1) {
    int v[kMergeE][NR];
#pragma unroll
    for (int r2 = 0; r2 < NR; ++r2)
#pragma unroll
      for (int e = 0; e < kMergeE; ++e) v[e][r2] = lists[lo[r2] + max(min(lb[e][r2] + step, nl[r2]) - 1, 0)];
#pragma unroll
    for (int r2 = 0; r2 < NR; ++r2)
#pragma unroll
      for (int e = 0; e < kMergeE; ++e)
        lb[e][r2] = (lb[e][r2] + step <= nl[r2] && v[e][r2] < xe[e]) ? lb[e][r2] + step : lb[e][r2];
  }
  uint32_t keep = 0u;
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < kMergeE; ++e) {
    bool dup = f0 + e >= F;
#pragma unroll
    for (int r2 = 0; r2 < NR - 1; ++r2) {  // (the last list is never below another)
      const int at = lists[lo[r2] + min(lb[e][r2], max(nl[r2] - 1, 0))];
      dup = dup || (r2 < re[e] && lb[e][r2] < nl[r2] && at == xe[e]);
    }
    if (!dup) {
      keep |= 1u << e;
      ++cnt;
    }
  }
  int total;
  int run = block_exclusive_scan<false>(cnt, &total, sh.tmp);  // (tmp is next written after the barrier below)
#pragma unroll
  for (int e = 0; e < kMergeE; ++e) {
    if (f0 + e < F) pre[f0 + e] = run;
    run += (keep >> e) & 1u;
  }
  if (tid == 0) pre[F] = total;
  lds_barrier();
#pragma unroll
  for (int e = 0; e < kMergeE; ++e) {
    if (!((keep >> e) & 1u)) continue;
    int pos = 0;
#pragma unroll
    for (int r2 = 0; r2 < NR; ++r2) {
      const int o2 = sh.moff[r2];
      // (an entry's own list: lb is its index there, as the list is ascending;
      // an empty list at F adds pre[F] - pre[F] = 0)
      pos += pre[o2 + lb[e][r2]] - pre[o2];
    }
    out[pos] = xe[e];
  }
  lds_barrier();
  return total;
}
__device__ __forceinline__ int union_merge(const Dims& d, ConstBufs& b, int bh, int n_ret, int wlo, int32_t* out,
                                           int* lists, int* pre, HeadShared& sh) {
  return n_ret <= 4 ? union_merge_n<4>(d, b, bh, n_ret, wlo, out, lists, pre, sh)
                    : union_merge_n<kMergeR>(d, b, bh, n_ret, wlo, out, lists, pre, sh);
}

// Bring all four 64-byte lines of the buffer table into the scalar cache at
// once. The head role reads its pointers from the table where it needs them,
// and the first read of each line after a launch would otherwise wait a
// memory round trip of its own in the middle of a phase. (The loads complete
// inside the block, so their unused results are safe.)
__device__ __forceinline__ void prefetch_table(const void* t) {
  uint32_t a, b2, c, e;
  asm volatile(
      "s_load_dword %0, %4, 0x0\n\ts_load_dword %1, %4, 0x40\n\ts_load_dword %2, %4, 0x80\n\t"
      "s_load_dword %3, %4, 0xc0\n\ts_waitcnt lgkmcnt(0)"
      : "=s"(a), "=s"(b2), "=s"(c), "=s"(e)
      : "s"(t)
      : "memory");
}
static_assert(sizeof(Bufs) > 0xc0 && sizeof(Bufs) <= 0x100, "the buffer table spans four 64-byte lines");

// A uniform int read with a scalar load (constant address space): only for
// words no work group of the running launch writes before the read.
__device__ __forceinline__ int scalar_read_ptr(const int32_t* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return *(__attribute__((address_space(4))) const int32_t*)(reinterpret_cast<uintptr_t>(p));
#else
  return *p;
#endif
}
__device__ __forceinline__ int scalar_read(gptr<int32_t> p) {
  return scalar_read_ptr(reinterpret_cast<const int32_t*>(reinterpret_cast<uintptr_t>(p)));
}

__device__ __forceinline__ void head_role(const Dims& d, ConstBufs& b, const uint16_t* q, long q_sb, long q_sh,
                                          const uint16_t* k, const uint16_t* v, float* out, int length, int t_dec,
                                          int mode, int stats_slot, int call_flag, int bh, HeadShared& sh) {
  const int bb = bh / d.Hq, h = bh % d.Hq, g = h / d.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int s_rank[8][64];
  extern __shared__ __align__(16) unsigned char dyn[];
  const size_t region0 = head_region0(d);
  uint32_t* bm = reinterpret_cast<uint32_t*>(dyn);
  int32_t* s_sel = reinterpret_cast<int32_t*>(dyn);
  float* s_selsc = reinterpret_cast<float*>(dyn + 4 * static_cast<size_t>(d.K));
  int32_t* s_cand = reinterpret_cast<int32_t*>(dyn + region0);
  float* s_sc = reinterpret_cast<float*>(dyn + region0 + 4 * static_cast<size_t>(d.cand_cap));

  // ---- one round of loads: query, FIFO state, every ring slot's q_bar and support size ----
  // (all requested before any of them is used, so that they cost one round trip)
  const int part = tid & 15;
  const uint32_t qw2 = wave == 0 ? *reinterpret_cast<const uint32_t*>(q + bb * q_sb + h * q_sh + 2 * lane) : 0u;
  prefetch_table(&b);
  // The FIFO state through the scalar cache: written only by earlier launches
  // (this launch's push comes after this read), so the scalar load is safe.
  const int fifo_head = scalar_read(b.fifo + 2 * bh);
  const int count = scalar_read(b.fifo + 2 * bh + 1);
  // (also in the exact mode, which does not use them: a branch here made the
  // compiler consume the loads inside it, before the rest were requested)
  // (a second round of 32 entries only for caches of more than 32)
  const bool two = d.C > kHeadThreads / 16;
  float4 ent[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    ent[i][0] = ent[i][1] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i == 0 || two) {
      const int c = min(i * (kHeadThreads / 16) + (tid >> 4), d.C - 1);
      const float* e = b.cache_qbar + (static_cast<long>(bh) * d.C + c) * kHeadDim + 8 * part;
      ent[i][0] = *reinterpret_cast<const float4*>(e);
      ent[i][1] = *reinterpret_cast<const float4*>(e + 4);
    }
  }
  const int len_c = b.cache_len[static_cast<long>(bh) * d.C + min(tid, d.C - 1)];

  if (wave == 0) {
    float qb0, qb1;
    normalize_row(qw2, qb0, qb1);
    sh.qbar[2 * lane] = qb0;
    sh.qbar[2 * lane + 1] = qb1;
  }
  if (mode == kModeDecode) bitmap_clear(bm);  // first bitmap window, while the loads are in flight
  if (mode == kModeDecode && tid < d.C) sh.len[tid] = len_c;
  lds_barrier();

  bool exact = true, refresh = false;
  double rho_max = -INFINITY;
  int n_ret = 0;
  const int oldest = (fifo_head - count + d.C) % d.C;
  if (mode == kModeDecode) {
    refresh = d.Tr > 0 && (t_dec % d.Tr) == 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (i == 1 && !two) break;
      const int c = i * (kHeadThreads / 16) + (tid >> 4);
      const float* t = sh.qbar + 8 * part;
      double s = 0.0;
      s = fma(static_cast<double>(t[0]), static_cast<double>(ent[i][0].x), s);
      s = fma(static_cast<double>(t[1]), static_cast<double>(ent[i][0].y), s);
      s = fma(static_cast<double>(t[2]), static_cast<double>(ent[i][0].z), s);
      s = fma(static_cast<double>(t[3]), static_cast<double>(ent[i][0].w), s);
      s = fma(static_cast<double>(t[4]), static_cast<double>(ent[i][1].x), s);
      s = fma(static_cast<double>(t[5]), static_cast<double>(ent[i][1].y), s);
      s = fma(static_cast<double>(t[6]), static_cast<double>(ent[i][1].z), s);
      s = fma(static_cast<double>(t[7]), static_cast<double>(ent[i][1].w), s);
      s = row_sum(s);
      // FIFO position p (0 = oldest) lives in ring slot (oldest + p) mod C
      if (part == 0 && c < d.C) {
        int p = c - oldest;
        if (p < 0) p += d.C;
        sh.rho[p] = s;
      }
    }
    lds_barrier();
    // the path rule needs only rho_max: publish the decision before ranking
    // (recent-R retrieval: rho_max over the R newest entries only). Every
    // wave finds it, and every wave finds the ranks below, so that the union
    // needs no further barrier.
    const double v = lane < count ? sh.rho[lane] : -INFINITY;  // FIFO position lane
    const int lo = d.recent ? max(0, count - d.R) : 0;
    const double mxr = wave_max_f64(lane < count && lane >= lo ? v : -INFINITY);
    if (tid == 0)
      store_shared(b.dec + bh * kFlagStride, call_flag | ((refresh || count == 0 || mxr < d.tau) ? 1 : 0));
    // Rank of FIFO position p under (rho desc, position asc), counted in
    // parallel: wave w compares every position with positions w, w+8, ...
    {
      int r = 0;
      for (int p2 = wave; p2 < count; p2 += kHeadThreads / 64) {
        const double u = sh.rho[p2];
        r += (u > v) || (u == v && p2 < lane);
      }
      s_rank[wave][lane] = r;
    }
    lds_barrier();
    {
      int rank = 0;
#pragma unroll
      for (int w = 0; w < kHeadThreads / 64; ++w) rank += s_rank[w][lane];
      if (d.recent) rank = count - 1 - lane;  // the newest first
      if (lane < count && rank < d.R) {
        int slot = oldest + lane;
        if (slot >= d.C) slot -= d.C;
        sh.rslot[rank] = slot;  // the same value from every wave; each reads back its own
        if (wave == 0) {
          b.ret[bh * d.R + rank] = lane;
          b.retslot[bh * d.R + rank] = slot;
        }
      }
    }
    n_ret = min(d.R, count);
    // (the best entry's rho is the maximum: mxr over every entry, or over the
    // R newest for recent-R, where the path rule takes it)
    if (count > 0) rho_max = mxr;
    exact = refresh || count == 0 || rho_max < d.tau;
  }
  if (tid >= n_ret && tid < d.R) {
    b.ret[bh * d.R + tid] = -1;
    b.retslot[bh * d.R + tid] = -1;
  }
  if (tid == 0) {
    b.path[bh] = exact ? 1 : 0;
    b.rho[bh] = rho_max;
    if (stats_slot >= 0) {
      const long o = static_cast<long>(stats_slot) * d.B * d.Hq + bh;
      b.st_path[o] = static_cast<uint8_t>((exact ? 1 : 0) | (refresh ? 2 : 0));
      b.st_rho[o] = rho_max;
      if (exact) b.st_m[o] = 0;
    }
  }
  // publish the decision to the score work groups (decode mode did so above;
  // the histogram half of this call was cleared during the previous one)
  if (tid == 0 && mode != kModeDecode) store_shared(b.dec + bh * kFlagStride, call_flag | (exact ? 1 : 0));
  if (exact) {
    if (tid == 0) b.m[bh] = 0;
    return;
  }

  // ---- candidate union (Eqs. 8-9) ----
  // Support entries below the window go through the LDS bitmap and come out
  // ascending and de-duplicated; the window [max(0, L-W), L) holds the
  // largest positions and is appended after them (support entries inside it
  // are already covered).
  const int wlo = max(0, length - d.W);
  int M = 0;
  // while the scores are not there yet: each retrieved support entry's
  // position relative to the bitmap window, or -1 (outside it, or past the
  // entry's support size)
  int32_t* stash = reinterpret_cast<int32_t*>(s_sc);
  uint32_t* pfx = reinterpret_cast<uint32_t*>(&sh.red[0][0]);
  // positions beyond one bitmap window: merge the sorted supports instead of
  // sweeping window after window
  const bool merged = wlo > kBitmapWords * 32 && n_ret <= kMergeR && n_ret * d.K <= kMergeE * kHeadThreads;
  if (merged) M = union_merge(d, b, bh, n_ret, wlo, s_cand, reinterpret_cast<int*>(s_sc), reinterpret_cast<int*>(dyn), sh);
  for (int base = 0; !merged && base < wlo; base += kBitmapWords * 32) {
    const int nbits = min(kBitmapWords * 32, wlo - base);
    if (base > 0) {
      bitmap_clear(bm);
      lds_barrier();
    }
    for (int j0 = 0; j0 < d.K; j0 += kHeadThreads) {
      const int j = j0 + tid;
      for (int r0 = 0; r0 < n_ret; r0 += 4) {
        int x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          // clamped entry: always a valid address, discarded when out of range
          const int r = min(r0 + u, n_ret - 1);
          x[u] = b.cache_supp[(static_cast<long>(bh) * d.C + sh.rslot[r]) * d.K + min(j, d.K - 1)];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = r0 + u;
          const int y = x[u] - base;
          const bool in = r < n_ret && j < sh.len[sh.rslot[min(r, n_ret - 1)]] && y >= 0 && y < nbits;
          if (in) bitmap_set(bm, y);
          if (r < n_ret && j < d.K) stash[r * d.K + j] = in ? y : -1;
        }
      }
    }
    lds_barrier();
    // Every entry goes to its position's rank among the window's set bits, so
    // the positions come out ascending; copies of one position in several
    // supports write the same value to the same slot.
    const int nset = bitmap_prefix(bm, pfx, sh.tmp);
    const int nrk = n_ret * d.K;
    for (int i0 = 0; i0 < nrk; i0 += 4 * kHeadThreads) {
      // four entries per thread at once, so that their LDS reads overlap
      int y[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * kHeadThreads + tid;
        y[u] = i < nrk ? stash[i] : -1;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (y[u] >= 0) s_cand[M + bitmap_rank(bm, pfx, y[u])] = base + y[u];
    }
    M += nset;
    if (base + kBitmapWords * 32 < wlo) lds_barrier();  // (the next window clears the bitmap; after the
                                                        // last one, the window append below is disjoint)
  }
  for (int x = wlo + tid; x < length; x += kHeadThreads) s_cand[M + (x - wlo)] = x;
  M += length - wlo;
  lds_barrier();
  // the rerank's 2048 bins, zeroed now (ordered before it by the barriers in between)
  reinterpret_cast<int4*>(&sh.whist[0][0])[tid] = make_int4(0, 0, 0, 0);
  if (tid == 0) sh.i3 = 0;
  for (int i = tid; i < M; i += kHeadThreads) b.cand[static_cast<long>(bh) * d.cand_cap + i] = s_cand[i];
  if (tid == 0) {
    b.m[bh] = M;
    if (stats_slot >= 0) b.st_m[static_cast<long>(stats_slot) * d.B * d.Hq + bh] = M;
  }

  // ---- candidate scores (Eq. 10) ----
  const uint16_t* kb = k + static_cast<long>(bb * d.Hkv + g) * d.max_len * kHeadDim;
  const uint16_t* vb = v + static_cast<long>(bb * d.Hkv + g) * d.max_len * kHeadDim;
  const int rg = tid >> 4, rpr = kHeadThreads >> 4;
  float mx = kNegInf, mn = kPosInf;
  {
    // kCandU rows in flight per 16-lane group; a wider round for candidate
    // sets that one such round misses only by a little, so that they do not
    // pay a second dependent round trip
    const uint4 qw = *reinterpret_cast<const uint4*>(q + bb * q_sb + h * q_sh + 8 * part);
    if (M > rpr * kCandU && M <= rpr * kCandWide)
      cand_scores<kCandWide>(kb, s_cand, M, qw, rg, rpr, part, s_sc, mn, mx);
    else
      cand_scores<kCandU>(kb, s_cand, M, qw, rg, rpr, part, s_sc, mn, mx);
  }
  // the scores' extremes: per wave before the barrier that publishes the
  // scores, across the waves after it
  {
    float* tmpf = reinterpret_cast<float*>(sh.tmp);
    mx = wave_max_f32(mx);
    mn = -wave_max_f32(-mn);
    if (lane == 0) {
      tmpf[2 * wave] = mn;
      tmpf[2 * wave + 1] = mx;
    }
    lds_barrier();
    mn = kPosInf;
    mx = kNegInf;
#pragma unroll
    for (int w = 0; w < kHeadThreads / 64; ++w) {
      mn = fminf(mn, tmpf[2 * w]);
      mx = fmaxf(mx, tmpf[2 * w + 1]);
    }
  }

  // ---- rerank (Eq. 11) ----
  // LDS after S_hat and its scores in region0: boundary flags of the linear rerank
  uint8_t* flag = reinterpret_cast<uint8_t*>(dyn + 8 * static_cast<size_t>(d.K));
  // S_t (ascending index) with the softmax weights of Eq. 12 in LDS, and
  // with its scores to the step outputs
  int32_t* g_sel = b.sel + static_cast<long>(bh) * d.K;
  float* g_selsc = b.selsc + static_cast<long>(bh) * d.K;
  int n;
  if (M <= d.K) {
    for (int i = tid; i < M; i += kHeadThreads) {
      const int x = s_cand[i];
      const float sv = s_sc[i];
      s_sel[i] = x;
      s_selsc[i] = expf((sv - mx) * kInvSqrtD);
      g_sel[i] = x;
      g_selsc[i] = sv;
    }
    n = M;
    lds_barrier();
  } else {
    n = (mx > mn) ? rerank_linear(s_cand, s_sc, M, d.K, mn, mx, s_sel, s_selsc, g_sel, g_selsc, flag, sh) : -1;
    if (n < 0) {
      int need;
      uint32_t mask;
      const uint32_t T = radix_kth(s_sc, M, d.K, sh, &mask, &need);
      n = select_in_order(s_cand, s_sc, M, T, mask, need, mx, s_sel, s_selsc, g_sel, g_selsc, sh);
    }
  }

  // ---- reuse path: softmax-V (Eq. 12) and cache update ----
  if (tid == 0) b.sellen[bh] = n;
  attend_w(s_sel, s_selsc, n, vb, out + static_cast<long>(bh) * kHeadDim, nullptr, sh);
  cache_push(d, b, bh, fifo_head, count, sh.qbar, s_sel, n);
}

// ---------------------------------------------------------------------------
// Composite keys of the exact Top-K: ordered score << 32 | ~index, so that a
// larger key is a higher score, then a lower index; all keys are distinct.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t comp_key(float s, uint32_t idx) {
  return (static_cast<uint64_t>(order_key(s)) << 32) | static_cast<uint64_t>(0xffffffffu - idx);
}

// ---------------------------------------------------------------------------
// Shared end of the exact finish: S_t (n indices, ascending) and their scores
// are in LDS. Writes them out, aggregates the values (Eq. 12) and pushes
// (q_bar_t, S_t) when `push`. Every thread of the block must call it.
// ---------------------------------------------------------------------------
// qb0 / qb1: elements 2 lane and 2 lane + 1 of q_bar_t in wave 0 (normalize_row).
__device__ __forceinline__ void finish_tail(const Dims& d, const BufsDev& b, int bh, int n, const uint16_t* v, float* out,
                                            int32_t* sel_out, int push, int fifo_slot, int fifo_count, HeadShared& sh,
                                            const int32_t* s_sel, float* s_selsc, float qb0, float qb1) {
  const int tid = threadIdx.x;
  const int bb = bh / d.Hq, g = (bh % d.Hq) / d.G;
  float mx = kNegInf;
  for (int i = tid; i < n; i += kHeadThreads) {
    mx = fmaxf(mx, s_selsc[i]);
    b.sel[static_cast<long>(bh) * d.K + i] = s_sel[i];
    b.selsc[static_cast<long>(bh) * d.K + i] = s_selsc[i];
  }
  mx = block_max_f32(mx, reinterpret_cast<float*>(sh.tmp));
  if (tid == 0) b.sellen[bh] = n;
  if (sel_out != nullptr)
    for (int i = tid; i < d.K; i += kHeadThreads) sel_out[static_cast<long>(bh) * d.K + i] = i < n ? s_sel[i] : -1;
  if (v != nullptr && out != nullptr) {
    const uint16_t* vb = v + static_cast<long>(bb * d.Hkv + g) * d.max_len * kHeadDim;
    attend(s_sel, s_selsc, n, mx, vb, out + static_cast<long>(bh) * kHeadDim, nullptr, sh);
  }
  if (push) {
    if (tid < 64) {
      sh.qbar[2 * tid] = qb0;
      sh.qbar[2 * tid + 1] = qb1;
    }
    lds_barrier();
    cache_push(d, b, bh, fifo_slot, fifo_count, sh.qbar, s_sel, n);
  }
}

// ---------------------------------------------------------------------------
// The exact heads of a call, GQA-grouped: full-history scores (Eq. 4,
// unscaled), Global Top-K (Eq. 1), softmax-V (Eq. 12) and the cache update,
// all run by the score work groups.
//
// Rows: the KV groups holding at least one exact head are listed in order;
// their rows, concatenated (T = ne * L of them), are split evenly over the nW
// score work groups: work group w owns [x_w, x_{w+1}), x_w = floor(w T / nW).
// Inside a group a work group's rows start at a 16-row boundary; its rows of
// one group are a segment [row0, rend).
//
// Phase 1, scores: every segment is streamed once and scored for all query
//   heads of its group with MFMA 16x16x32 bf16 tiles (A = 16 key rows x 32
//   dims, B = 32 dims x 16 query heads, fp32 accumulation), the loads of the
//   next 512 rows in flight while the current ones are scored. The scores of
//   exact heads stay in LDS when a work group's share fits (else they go to
//   the score workspace) and are counted in a per-head histogram of the top
//   10 bits of their ordered keys (LDS, then added into the call's half of
//   the global one). The work group then sets its scored flag (the call
//   flag, device scope).
// Phase 2, survivors: once the group of a segment is fully scored (the scored
//   flag of every work group with rows in it is the call's), one wave
//   per exact head reads the head's histogram, finds the bin b1 holding the
//   K-th largest score, and writes the segment's positions and scores in bin
//   b1 or above, in ascending position order, to the segment's own region of
//   the head's survivor row (starting at row0); once they are stored, the
//   wave publishes their count together with the call flag (one 8-byte
//   store per head and work group).
// Phase 3, finish: exact head m (of n_ex) of group e belongs to the work group
//   whose rows hold x = e L + floor((2m + 1) L / (2 n_ex)). That work group
//   finds b1 and the counts above and in it from the histogram, polls the
//   head's survivor counts of the group's work groups until each carries the
//   call flag, selects the K best survivors
//   (radix select over the key bits below bin b1), writes S_t, aggregates the
//   values and pushes (q_bar_t, S_t).
//
// A head's histogram has a half per call parity: a call fills one while the
// score work groups clear the other (used by the previous call) for the next.
// A phase waits only for earlier phases, which never wait for later ones, and
// every wait is bounded in time (a timeout sets the device error word and the
// work group gives up the call). Head work groups never wait, so score work
// groups not yet resident get a CU as the head work groups end.
// ---------------------------------------------------------------------------
constexpr int kMaxExactGroups = 1024;  // KV groups (batch x KV heads) the row split can list
constexpr int kPollRounds = 20000;     // polls of the decision flags before giving up (tens of ms)

// Where work group ww's share starts: list position e and row r (rounded
// down to 16 inside the group; e == ne, r == 0 at the end). The share starts
// at x = floor(ww T / nW) of the T = ne * length concatenated rows; with
// ww ne = a nW + b (b < nW) that is x = a length + floor(b length / nW), whose
// second term is below length: so e = a and r = floor(b length / nW), without
// 64-bit integer divisions (they expand to long instruction sequences, and
// every waiting thread evaluates this for its work group). b length < 2^42 is
// exact in a double, and the quotient, below 2^24, is at least 1 / nW away
// from the next integer unless it is one, far more than the division's
// rounding error: its floor is exact.
__device__ __forceinline__ void share_start(int nW, int length, int ne, int ww, int& a, int& rr) {
  const uint32_t q = static_cast<uint32_t>(ww) * static_cast<uint32_t>(ne);  // <= 2^10 * 2^10
  const uint32_t qa = q / static_cast<uint32_t>(nW), bq = q - qa * static_cast<uint32_t>(nW);
  const double bl = static_cast<double>(bq) * static_cast<double>(length);
  a = static_cast<int>(qa);
  rr = static_cast<int>(bl / static_cast<double>(nW));
}
__device__ __forceinline__ void split_at(long T, int nW, int length, int ne, int ww, int& e, int& r) {
  (void)T;  // = ne * length
  int rr;
  share_start(nW, length, ne, ww, e, rr);
  r = e < ne ? rr & ~15 : 0;
}

// Rows [lo, hi) of group e in work group ww's share (empty when lo >= hi).
__device__ __forceinline__ void seg_rows(long T, int nW, int length, int ne, int ww, int e, int& lo, int& hi) {
  int ea, ra, eb, rb;
  split_at(T, nW, length, ne, ww, ea, ra);
  split_at(T, nW, length, ne, ww + 1, eb, rb);
  lo = ea < e ? 0 : (ea == e ? ra : length);
  hi = eb > e ? length : (eb == e ? rb : 0);
}

// Lanes below this one with their bit set in m.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

// Wait until flags[ww * kFlagStride] == call_flag for every work group ww with rows in list
// group e (one thread per work group; bounded in time, a timeout sets the
// device error word). Every thread of the block must call it.
__device__ __forceinline__ bool wait_group(const int32_t* flags, long T, int nW, int length, int ne, int e,
                                           int call_flag, int32_t* err, int* s_go, int* votes, int& vpar) {
  const int tid = threadIdx.x;
  bool chk = false;
  if (tid < nW) {
    int lo, hi;
    seg_rows(T, nW, length, ne, tid, e, lo, hi);
    chk = lo < hi;
  }
  const long long t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    const bool ok = !chk || load_shared(flags + tid * kFlagStride) == call_flag;
    if (block_all(ok, votes, vpar)) return true;
    if (tid == 0) *s_go = __builtin_amdgcn_s_memrealtime() - t0 >= kWaitTicks ? -1 : 0;
    lds_barrier();
    if (*s_go < 0) {
      if (tid == 0) store_shared(err, 1);
      return false;
    }
    __builtin_amdgcn_s_sleep(kPollSleep);
  }
}

// Index of the m-th set bit of mask (m < popcount(mask)).
__device__ __forceinline__ int nth_bit(unsigned mask, int m) {
  for (int i = 0; i < m; ++i) mask &= mask - 1;
  return __ffs(mask) - 1;
}

// One wave: the bin b1 holding the keff-th largest key of a histogram
// (kNumBins counters, read with device-scope loads), the count above b1 and
// the count in b1 ({0, 0, 0} if the counts fall short of keff). Lane l holds
// the 16 bins below kNumBins - 16 l. Every lane of the wave must call it.
__device__ __forceinline__ int3 wave_boundary(const uint32_t* hist, int keff) {
  const int lane = threadIdx.x & 63;
  const int lo = kNumBins - 16 * (lane + 1);
  uint32_t c[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint2 v = load_shared(reinterpret_cast<const uint2*>(hist + lo + 2 * i));
    c[2 * i] = v.x;
    c[2 * i + 1] = v.y;
  }
  int tot = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) tot += static_cast<int>(c[i]);
  const int incl = wave_incl_scan(tot);  // counts of this lane's bins and all above
  int run = incl - tot;
  int3 r = make_int3(0, 0, 0);
  const bool here = run < keff && incl >= keff;
  if (here) {
    bool found = false;
#pragma unroll
    for (int i = 15; i >= 0; --i) {
      if (!found && run + static_cast<int>(c[i]) >= keff) {
        r = make_int3(lo + i, run, static_cast<int>(c[i]));
        found = true;
      }
      run += static_cast<int>(c[i]);
    }
  }
  const uint64_t m = __ballot(here);
  if (m == 0) return make_int3(0, 0, 0);
  const int src = __ffsll(static_cast<long long>(m)) - 1;
  return make_int3(__builtin_amdgcn_readlane(r.x, src), __builtin_amdgcn_readlane(r.y, src),
                   __builtin_amdgcn_readlane(r.z, src));
}

// Phase 2 for one segment [row0, rend) of KV group (bb, g), whose rows are all
// scored: the survivors of every exact head jj of the group (bit jj of
// emask), one wave per head: b1 from the head's histogram, then 64 rows per
// ballot in position order with a running count (kEmitU ballots' worth of
// scores read at once from LDS, kEmitUGlobal from the score workspace, whose
// round trips are far longer). Scores from LDS (kLds: head jj's row row0 + i
// at sc[jj * stride + i]) or from the score workspace. Every thread of the
// block must call it.
constexpr int kEmitU = 8;
constexpr int kEmitUGlobal = 32;

// End of phase 2 for one segment in one wave: lane i holds the survivor count
// of the wave's i-th head (jj = wave + 8 i, 8 waves). Once the wave's survivor
// stores are complete, each exact head's count goes out with the call flag as
// one 8-byte device-scope store; the finishing work group polls these words,
// so the count arrives with the flag that publishes it.
__device__ __forceinline__ void publish_counts(uint2* ccnt, int h0, int n_cu, int w, int G, unsigned emask, int run,
                                               int call_flag) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = kHeadThreads >> 6;
  const int jj = wave + nw * lane;
  wait_vmem();
  if (jj < G && ((emask >> (jj & 31)) & 1u))
    store_shared(ccnt + static_cast<long>(h0 + jj) * n_cu + w,
                 make_uint2(static_cast<uint32_t>(run), static_cast<uint32_t>(call_flag)));
}

template <bool kLds>
__device__ __forceinline__ void emit_segment(const Dims& d, const BufsDev& b, int bb, int g, unsigned emask, int row0,
                                             int rend, int length, int w, int par, int call_flag, const float* sc,
                                             int stride) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = kHeadThreads >> 6;
  const int G = d.G;
  const int h0 = bb * d.Hq + g * G;  // query head of jj = 0
  const int nrows = rend - row0;
  int my_run = 0;  // lane i: the count of this wave's i-th head
  for (int jj = wave, slot = 0; jj < G; jj += nw, ++slot) {
    if (!((emask >> jj) & 1u)) continue;
    const int b1 = wave_boundary(b.hist + (static_cast<long>(h0 + jj) * 2 + par) * kNumBins, min(d.K, length)).x;
    // bin(x) >= b1 as one unsigned compare: s ^ ((s >> 31) | 2^31) orders the
    // raw bits like order_key except that -0.0 lands just below +0.0, which
    // only matters at b1 = 512 and is covered by lowering that threshold by one
    const uint32_t k0 = b1 == kNumBins / 2 ? 0x7fffffffu : static_cast<uint32_t>(b1) << kHistShift;
    const float* srow = kLds ? sc + jj * stride : b.score + static_cast<long>(h0 + jj) * d.score_stride + row0;
    uint2* region = b.hits + static_cast<long>(h0 + jj) * d.max_len + row0;
    int run = 0;
    constexpr int U = kLds ? kEmitU : kEmitUGlobal;
    for (int c0 = 0; c0 < nrows; c0 += 64 * U) {
      float x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = srow[min(c0 + 64 * u + lane, nrows - 1)];  // clamped, masked below
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = c0 + 64 * u + lane;
        const int sb = __float_as_int(x[u]);
        const bool sv = (i < nrows) & ((static_cast<uint32_t>(sb) ^ (static_cast<uint32_t>(sb >> 31) | 0x80000000u)) >= k0);
        const uint64_t m = __ballot(sv);
        if (sv)
          store_shared(region + run + lanes_below(m), make_uint2(static_cast<uint32_t>(row0 + i), __float_as_uint(x[u])));
        run += __popcll(m);
      }
    }
    if (lane == slot) my_run = run;
  }
  publish_counts(b.ccnt, h0, d.n_cu, w, G, emask, my_run, call_flag);
}

// ---------------------------------------------------------------------------
// Long histories: per-segment K-best lists instead of stored scores.
//
// When a score work group's share of rows does not fit its LDS as scores, it
// keeps, per exact head of each of its segments, only the entries that can
// still be among the segment's K best: a key outside its own segment's K best
// cannot be among the K best of the whole history (the segment alone holds K
// better ones). Entries are (ordered score key, row) in LDS, admitted when
// their composite key (ordered score << 32 | ~row: higher score first, then
// lower row; all keys distinct) reaches the head's admission threshold. Each
// stage's admitted entries are placed in row order (a scan of per-tile
// counts), so a list is always sorted by row. When a head's list could
// overflow during the next stage, one wave cuts it (in place, in order) to the
// entries at or above a new threshold that keeps at least its K best: a
// 256-bin histogram of the 8 score-key bits below the common prefix of the
// list's key range (tracked per head as entries are admitted), refined 8 bits
// at a time; on the full composite keys only when scores tie. At the end of a
// segment, the lists of a work group's first segment (of two) are cut to the
// next power of two >= K entries and moved to that stride; only the lists'
// entries enter the call's score histogram: the K best of the union of all
// lists are the K best of the history, so the boundary bin b1, the counts
// above and in it, and the survivors (list entries in b1 or above, already in
// position order) are those of the full history.
// ---------------------------------------------------------------------------
constexpr int kKbSlack = 1024;   // list room beyond K: the next stage's arrivals never overflow it
constexpr int kKbCutSlack = 64;  // a cut during the scan keeps at most K + this many entries
constexpr int kKbMaxSeg = 2;     // segments per work group the lists are kept for (else stored scores)
constexpr int kKbTc = 16 * kQkUnroll * (kHeadThreads / kWave) / 4;  // (tile, row quad) slots per head and stage
// Rows per score work group from which the lists beat stored scores (below,
// the stored scores' write and re-read cost less than the lists' per-stage
// ordering and cuts)
constexpr long kKbMinShare = 8192;

__device__ __forceinline__ uint64_t kb_key(uint2 e) {
  return (static_cast<uint64_t>(e.x) << 32) | static_cast<uint64_t>(0xffffffffu - e.y);
}

// The float bits of an ordered score key (negative zero comes back as +0).
__device__ __forceinline__ uint32_t okey_bits(uint32_t k) { return (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k; }

__host__ __device__ inline int kb_stride(int K) {
  int p = 1;
  while (p < K) p <<= 1;
  return p;
}

// Dynamic LDS of the K-best path: two stages' tile counts, then the lists.
__host__ __device__ inline long kb_tc_bytes(const Dims& d) { return (8L * d.G * kKbTc + 15) / 16 * 16; }

// Entries per head of segment si's working list (after the finished lists of
// segments 0 .. si-1, at stride kb_stride(K)).
__host__ __device__ inline int kb_cap(const Dims& d, int si) {
  const long list_bytes = 8L * d.G * kb_stride(d.K);
  return static_cast<int>((kLdsLimit - kb_tc_bytes(d) - si * list_bytes) / (8L * d.G));
}

// Whether a work group with nseg non-empty segments keeps K-best lists: each
// segment's working list holds K + kKbSlack entries per head.
__host__ __device__ inline bool kb_fits(const Dims& d, int nseg) {
  if (nseg < 1 || nseg > kKbMaxSeg) return false;
  for (int si = 0; si < nseg; ++si)
    if (kb_cap(d, si) < d.K + kKbSlack) return false;
  return true;
}

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t y = static_cast<uint64_t>(__shfl_xor(static_cast<long long>(x), o));
    x = y < x ? y : x;
  }
  return x;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t y = static_cast<uint64_t>(__shfl_xor(static_cast<long long>(x), o));
    x = y > x ? y : x;
  }
  return x;
}

// One wave: the digit holding the need-th largest of a 256-bin histogram
// (bins scanned from 255 down): returns false if the bins hold fewer; else
// *dg, the count above it (*above) and in it (*cnt).
__device__ __forceinline__ bool kb_pick(const int* bins, int need, int* dg_out, int* above_out, int* cnt_out) {
  const int lane = threadIdx.x & 63;
  const int4 h = reinterpret_cast<const int4*>(bins)[63 - lane];  // lane l: digits 255-4l .. 252-4l
  const int c[4] = {h.w, h.z, h.y, h.x};
  const int s4 = c[0] + c[1] + c[2] + c[3];
  const int incl = wave_incl_scan(s4);
  int run = incl - s4;
  int dg = -1, above = 0, cnt = 0;
  if (run < need && incl >= need) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (dg < 0 && run + c[j] >= need) {
        dg = 255 - 4 * lane - j;
        above = run;
        cnt = c[j];
      }
      run += c[j];
    }
  }
  const uint64_t m = __ballot(dg >= 0);
  if (m == 0) return false;
  const int src = __ffsll(static_cast<long long>(m)) - 1;
  *dg_out = __builtin_amdgcn_readlane(dg, src);
  *above_out = __builtin_amdgcn_readlane(above, src);
  *cnt_out = __builtin_amdgcn_readlane(cnt, src);
  return true;
}

// One wave: cut buf[0, n) (n > limit >= k) in place and in order to the
// entries whose score key is at least a threshold that keeps at least the k
// largest and at most `limit` of them. lo, hi bound the list's score keys.
// Entries with equal scores are kept or dropped together: returns false, with
// buf untouched, when ties leave more than `limit` entries at the finest
// score resolution; else sets *theta (as a composite-key threshold) and
// *n_out. bins: 256 ints of this wave's own LDS.
__device__ __forceinline__ bool kb_cut32(uint2* buf, int n, int k, int limit, uint32_t lo, uint32_t hi, int* bins,
                                         uint64_t* theta, int* n_out) {
  const int lane = threadIdx.x & 63;
  constexpr int U = 8;
  if (lo >= hi) return false;
  // the first digit: the 8 bits whose top one is the highest bit where lo and hi differ
  const int hb = 31 - __clz(static_cast<int>(lo ^ hi));
  int shift = max(hb - 7, 0), width = min(hb + 1, 8);
  uint32_t mask = hb >= 31 ? 0u : ~0u << (hb + 1);
  uint32_t pre = lo & mask;
  int need = k, kept = 0;
  for (;;) {
    const uint32_t dm = (1u << width) - 1u;
    reinterpret_cast<int4*>(bins)[lane] = make_int4(0, 0, 0, 0);
    for (int c0 = 0; c0 < n; c0 += 64 * U) {
      uint32_t x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = buf[min(c0 + 64 * u + lane, n - 1)].x;  // (clamped, masked below)
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (c0 + 64 * u + lane < n && (x[u] & mask) == pre) atomicAdd(&bins[(x[u] >> shift) & dm], 1);
    }
    int dg, above, cnt;
    if (!kb_pick(bins, need, &dg, &above, &cnt)) return false;  // (cannot happen: lo, hi bound the keys)
    pre |= static_cast<uint32_t>(dg) << shift;
    mask |= dm << shift;
    kept += above;
    need -= above;
    if (kept + cnt <= limit) break;
    if (shift == 0) return false;
    width = min(shift, 8);
    shift -= width;
  }
  int run = 0;
  for (int c0 = 0; c0 < n; c0 += 64 * U) {
    uint2 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = buf[min(c0 + 64 * u + lane, n - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool kp = (c0 + 64 * u + lane < n) && (x[u].x & mask) >= pre;
      const uint64_t b = __ballot(kp);
      if (kp) buf[run + lanes_below(b)] = x[u];
      run += __popcll(b);
    }
  }
  *n_out = run;
  *theta = static_cast<uint64_t>(pre) << 32;
  return true;
}

// The same cut on the full composite keys (all distinct), for lists whose
// scores tie: always succeeds.
__device__ __forceinline__ uint64_t kb_cut64(uint2* buf, int n, int k, int limit, int* bins, int* n_out) {
  const int lane = threadIdx.x & 63;
  constexpr int U = 8;
  uint64_t lo = ~0ull, hi = 0ull;
  for (int c0 = 0; c0 < n; c0 += 64 * U) {
    uint2 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = buf[min(c0 + 64 * u + lane, n - 1)];  // (clamped repeats change nothing)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t key = kb_key(x[u]);
      lo = key < lo ? key : lo;
      hi = key > hi ? key : hi;
    }
  }
  lo = wave_min_u64(lo);
  hi = wave_max_u64(hi);
  const int hb = 63 - __clzll(static_cast<long long>(lo ^ hi));  // (n > 1 distinct keys: lo != hi)
  int shift = max(hb - 7, 0), width = min(hb + 1, 8);
  uint64_t mask = hb >= 63 ? 0ull : ~0ull << (hb + 1);
  uint64_t pre = lo & mask;
  int need = k, kept = 0;
  for (;;) {
    const uint64_t dm = (1ull << width) - 1;
    reinterpret_cast<int4*>(bins)[lane] = make_int4(0, 0, 0, 0);
    for (int c0 = 0; c0 < n; c0 += 64 * U) {
      uint2 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = buf[min(c0 + 64 * u + lane, n - 1)];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t key = kb_key(x[u]);
        if (c0 + 64 * u + lane < n && (key & mask) == pre) atomicAdd(&bins[(key >> shift) & dm], 1);
      }
    }
    int dg, above, cnt;
    if (!kb_pick(bins, need, &dg, &above, &cnt)) break;  // (cannot happen: lo, hi bound the keys)
    pre |= static_cast<uint64_t>(dg) << shift;
    mask |= dm << shift;
    kept += above;
    need -= above;
    if (kept + cnt <= limit || shift == 0) break;
    width = min(shift, 8);
    shift -= width;
  }
  int run = 0;
  for (int c0 = 0; c0 < n; c0 += 64 * U) {
    uint2 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = buf[min(c0 + 64 * u + lane, n - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool kp = (c0 + 64 * u + lane < n) && (kb_key(x[u]) & mask) >= pre;
      const uint64_t b = __ballot(kp);
      if (kp) buf[run + lanes_below(b)] = x[u];
      run += __popcll(b);
    }
  }
  *n_out = run;
  return pre;
}

__device__ __forceinline__ uint64_t kb_cut(uint2* buf, int n, int k, int limit, uint32_t lo, uint32_t hi, int* bins,
                                           int* n_out) {
  uint64_t th;
  if (kb_cut32(buf, n, k, limit, lo, hi, bins, &th, n_out)) return th;
  return kb_cut64(buf, n, k, limit, bins, n_out);
}

// Per-head state of the lists of the current segment (static LDS).
struct KbState {
  int n[kMaxGroup];          // entries
  uint64_t theta[kMaxGroup]; // admission threshold (composite key)
  uint32_t lo[kMaxGroup];    // a lower bound of the entries' score keys
  uint32_t hi[kMaxGroup];    // their maximum
  int full[kMaxGroup];       // to be cut after this stage
  int cnt[kKbMaxSeg][kMaxGroup];  // final length per segment
};

// One stage of scores (as qk_score) into the K-best lists, in row order:
//  1. every lane with an exact head j finds, per tile, its four rows whose keys
//     reach theta and writes their count to the stage's slot table (and folds
//     their score keys into the head's range);
//  2. a wave per head scans the head's table (slot order = row order) into
//     list positions and moves the head's length on;
//  3. the lanes write their entries;
//  4. when a head's list could overflow during the next stage, its wave cuts
//     it and raises its threshold.
// tc: this stage's table (the other one serves the neighbouring stages, so
// no barrier is needed between step 3 of one stage and step 1 of the next).
// Every thread of the block must call it.
__device__ __forceinline__ void qk_score_kb(const Dims& d, const QkTiles& t, const bf16x8 (&bq)[4], int t0, int rend,
                                            int wave, int nw, int j, int kq, bool hv, uint64_t& theta, uint2* lists,
                                            int cap, int* tc, KbState& ks, unsigned emask, HeadShared& sh) {
  const int lane = threadIdx.x & 63;
  uint32_t ok[kQkUnroll][4];
  unsigned pass = 0u;
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int u = 0; u < kQkUnroll; ++u) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(t.a[u][s]), bq[s], acc, 0, 0, 0);
    const int r = t0 + (u * nw + wave) * 16 + 4 * kq;
    int c = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ok[u][e] = order_key(acc[e]);
      const uint64_t ck = (static_cast<uint64_t>(ok[u][e]) << 32) |
                          static_cast<uint64_t>(0xffffffffu - static_cast<uint32_t>(r + e));
      const bool pe = hv & (r + e < rend) & (ck >= theta);
      pass |= static_cast<unsigned>(pe) << (4 * u + e);
      c += pe;
      if (pe) {
        lo = min(lo, ok[u][e]);
        hi = max(hi, ok[u][e]);
      }
    }
    if (hv) tc[j * kKbTc + (u * nw + wave) * 4 + kq] = c;
  }
  if (pass) {
    atomicMin(&ks.lo[j], lo);
    atomicMax(&ks.hi[j], hi);
  }
  lds_barrier();
  const int room = cap - 16 * kQkUnroll * nw;  // a stage adds at most one entry per row
  for (int jj = wave; jj < d.G; jj += nw) {
    if (!((emask >> jj) & 1u)) continue;
    int* row = tc + jj * kKbTc;
    const int a = row[2 * lane], b2 = row[2 * lane + 1];
    const int incl = wave_incl_scan(a + b2);
    const int base = ks.n[jj];
    const int ex = base + incl - a - b2;
    row[2 * lane] = ex;
    row[2 * lane + 1] = ex + a;
    const int n = base + __builtin_amdgcn_readlane(incl, 63);
    if (lane == 0) {
      ks.n[jj] = n;
      ks.full[jj] = n > room;
    }
  }
  lds_barrier();
  if (pass) {
    uint2* buf = lists + static_cast<long>(j) * cap;
#pragma unroll
    for (int u = 0; u < kQkUnroll; ++u) {
      if (!((pass >> (4 * u)) & 0xfu)) continue;
      int slot = tc[j * kKbTc + (u * nw + wave) * 4 + kq];
      const int r = t0 + (u * nw + wave) * 16 + 4 * kq;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if ((pass >> (4 * u + e)) & 1u) {
          if (slot < cap) buf[slot] = make_uint2(ok[u][e], static_cast<uint32_t>(r + e));
          ++slot;
        }
      }
    }
  }
  bool any = false;
  for (int jj = 0; jj < d.G; ++jj) any |= ks.full[jj] != 0;  // (set before the last barrier; uniform)
  if (any) {
    lds_barrier();  // the entries are in
    for (int jj = wave; jj < d.G; jj += nw) {
      if (!ks.full[jj]) continue;
      int kept;
      const uint64_t th = kb_cut(lists + static_cast<long>(jj) * cap, min(ks.n[jj], cap), d.K, d.K + kKbCutSlack,
                                 ks.lo[jj], ks.hi[jj], &sh.whist[wave][0], &kept);
      if (lane == 0) {
        ks.theta[jj] = th;
        ks.n[jj] = kept;
        ks.lo[jj] = static_cast<uint32_t>(th >> 32);  // every kept score key reaches the threshold's
        ks.full[jj] = 0;
      }
    }
    lds_barrier();
  }
  theta = ks.theta[j < d.G ? j : 0];
}

// End of segment si's scan (of nseg). The first of two segments cuts its lists
// to at most kp entries (keeping their K best) and moves them to stride kp,
// making room for the next segment's; the last leaves them in place at stride
// cap. Records the lists' lengths and adds their histograms into the call's
// half of the heads' global histograms: one wave per head, over the bins the
// head's score keys span, 256 at a time in the wave's own LDS. Returns the
// lists' stride. Every thread of the block must call it.
__device__ __forceinline__ int kb_close(const Dims& d, ConstBufs& b, int bb, int g, unsigned emask, int par,
                                        uint2* lists, int cap, int kp, bool last, KbState& ks, int* kcnt,
                                        HeadShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = kHeadThreads >> 6;
  lds_barrier();
  int stride = cap;
  for (int jj = wave; jj < d.G; jj += nw) {
    int n = min(ks.n[jj], cap);
    if (!last && n > kp) kb_cut(lists + static_cast<long>(jj) * cap, n, d.K, kp, ks.lo[jj], ks.hi[jj],
                                &sh.whist[wave][0], &n);
    if (lane == 0) kcnt[jj] = n;
  }
  lds_barrier();
  if (!last) {
    // move: read a chunk into registers, then write it (a destination never
    // lies past its own source, nor in the source of a later chunk)
    const int total = d.G * kp;
    for (int base = 0; base < total; base += 8 * kHeadThreads) {
      uint2 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int xi = base + u * kHeadThreads + tid;
        const int jj = xi / kp, i = xi - jj * kp;
        x[u] = make_uint2(0u, 0xffffffffu);
        if (xi < total && i < kcnt[jj]) x[u] = lists[static_cast<long>(jj) * cap + i];
      }
      lds_barrier();
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int xi = base + u * kHeadThreads + tid;
        if (xi < total) lists[xi] = x[u];
      }
      lds_barrier();
    }
    stride = kp;
  }
  for (int jj = wave; jj < d.G; jj += nw) {
    if (!((emask >> jj) & 1u)) continue;
    const int n = kcnt[jj];
    const uint2* list = lists + static_cast<long>(jj) * stride;
    int* bins = &sh.whist[wave][0];
    uint32_t* ghist = b.hist + (static_cast<long>(bb * d.Hq + g * d.G + jj) * 2 + par) * kNumBins;
    const int blo = static_cast<int>(ks.lo[jj] >> kHistShift), bhi = static_cast<int>(ks.hi[jj] >> kHistShift);
    for (int b0 = blo; n > 0 && b0 <= bhi; b0 += 256) {
      reinterpret_cast<int4*>(bins)[lane] = make_int4(0, 0, 0, 0);
      for (int c0 = 0; c0 < n; c0 += 64 * 8) {
        uint32_t x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = list[min(c0 + 64 * u + lane, n - 1)].x;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int bn = static_cast<int>(x[u] >> kHistShift) - b0;
          if (c0 + 64 * u + lane < n && bn >= 0 && bn < 256) atomicAdd(&bins[bn], 1);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = bins[lane + 64 * i];
        if (c && b0 + lane + 64 * i < kNumBins) atomicAdd(&ghist[b0 + lane + 64 * i], static_cast<uint32_t>(c));
      }
    }
  }
  return stride;
}

// Phase 2 from a list (sorted by row): as emit_segment, reading (score key,
// row) entries.
__device__ __forceinline__ void emit_kb(const Dims& d, const BufsDev& b, int bb, int g, unsigned emask, int row0,
                                        int length, int w, int par, int call_flag, const uint2* lists, int stride,
                                        const int* kcnt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = kHeadThreads >> 6;
  const int G = d.G;
  const int h0 = bb * d.Hq + g * G;
  int my_run = 0;  // lane i: the count of this wave's i-th head
  for (int jj = wave, slot = 0; jj < G; jj += nw, ++slot) {
    if (!((emask >> jj) & 1u)) continue;
    const int b1 = wave_boundary(b.hist + (static_cast<long>(h0 + jj) * 2 + par) * kNumBins, min(d.K, length)).x;
    const uint32_t k0 = static_cast<uint32_t>(b1) << kHistShift;
    const uint2* list = lists + static_cast<long>(jj) * stride;
    uint2* region = b.hits + static_cast<long>(h0 + jj) * d.max_len + row0;
    const int n = kcnt[jj];
    int run = 0;
    for (int c0 = 0; c0 < n; c0 += 64 * kEmitU) {
      uint2 x[kEmitU];
#pragma unroll
      for (int u = 0; u < kEmitU; ++u) x[u] = list[min(c0 + 64 * u + lane, max(n - 1, 0))];
#pragma unroll
      for (int u = 0; u < kEmitU; ++u) {
        const bool sv = (c0 + 64 * u + lane < n) & (x[u].x >= k0);
        const uint64_t m = __ballot(sv);
        if (sv) store_shared(region + run + lanes_below(m), make_uint2(x[u].y, okey_bits(x[u].x)));
        run += __popcll(m);
      }
    }
    if (lane == slot) my_run = run;
  }
  publish_counts(b.ccnt, h0, d.n_cu, w, G, emask, my_run, call_flag);
}

// ---------------------------------------------------------------------------
// Phase 4 (finish) for head bh of list group e, run by the work group the head
// belongs to.
//  1. The survivor counts of the group's segments give each segment's offset
//     in the head's survivor list (ascending positions: the segments are in
//     order).
//  2. Each thread takes kSU consecutive survivors and classifies them: above
//     b1 (all kept) or in b1 (candidates). The candidates' composite keys
//     (score desc, index asc) are compacted (LDS, else the global spill row)
//     and a radix select over the bits below their shared top 10 keeps the
//     `need` = keff - (count above b1) best.
//  3. A block scan over "kept" flags writes S_t in ascending index order.
//
// LDS (dynamic): segment offsets (nW + 1) and first rows (nW), S_t and its
// scores (K each), then the candidate keys (the rest: at least kBoundaryLds).
// ---------------------------------------------------------------------------
constexpr int kSU = 8;  // survivors per thread per round

// Every thread of the block must call it. sh.i0 .. i2 hold (b1, count above
// b1, count in b1), written by wave 0 before the call. Returns false when the
// survivor-count poll timed out (the device error word is then set).
__device__ __forceinline__ bool finish_phase(const Dims& d, const BufsDev& b, int bh, const uint16_t* q, long q_sb,
                                             long q_sh, const uint16_t* v, float* out, int32_t* sel_out, int length,
                                             int push, int call_flag, long T, int nW, int ne, int e, HeadShared& sh,
                                             unsigned char* dyn, int& vpar) {
  const int tid = threadIdx.x;
  // one round of loads: this thread's segment count, the FIFO state and (for
  // the push) q_bar_t
  // q_bar_t for the push, normalised here from the query (the same bits as the
  // head work group's, with normalize_row; the word is loaded in this round)
  const uint32_t qw2 = push && tid < 64 ? *reinterpret_cast<const uint32_t*>(q + (bh / d.Hq) * q_sb +
                                                                               (bh % d.Hq) * q_sh + 2 * tid)
                                        : 0u;
  int slo = 0, shi = 0;
  if (tid < nW) seg_rows(T, nW, length, ne, tid, e, slo, shi);
  const int fifo_slot = b.fifo[2 * bh], fifo_count = b.fifo[2 * bh + 1];
  // the survivor count of every segment of the group, polled until each
  // carries this call's flag (one thread per work group; bounded in time)
  int cc = 0;
  {
    const bool chk = tid < nW && slo < shi;
    const uint2* crow = b.ccnt + static_cast<long>(bh) * d.n_cu + tid;
    const long long t0 = __builtin_amdgcn_s_memrealtime();
    for (;;) {
      const uint2 c2 = chk ? load_shared(crow) : make_uint2(0u, static_cast<uint32_t>(call_flag));
      cc = static_cast<int>(c2.x);
      if (block_all(c2.y == static_cast<uint32_t>(call_flag), sh.vote, vpar)) break;
      if (tid == 0) sh.i3 = __builtin_amdgcn_s_memrealtime() - t0 >= kWaitTicks ? -1 : 0;
      lds_barrier();
      if (sh.i3 < 0) {
        if (tid == 0) store_shared(b.err, 1);
        return false;
      }
      __builtin_amdgcn_s_sleep(kPollSleep);
    }
  }
  // (b1, count above b1, count in b1), from wave 0 before the poll's barriers
  const int3 bd = make_int3(sh.i0, sh.i1, sh.i2);
  int* aoff = reinterpret_cast<int*>(dyn);
  int* srow0 = aoff + (nW + 4) / 4 * 4;
  const size_t off_c = 4 * static_cast<size_t>((nW + 4) / 4 * 4 + (nW + 3) / 4 * 4);
  int32_t* s_sel = reinterpret_cast<int32_t*>(dyn + off_c);
  float* s_selsc = reinterpret_cast<float*>(dyn + off_c + 4 * static_cast<size_t>(d.K));
  // the candidate keys take the rest of the LDS (at least kBoundaryLds of them)
  const size_t off_k = (off_c + 8 * static_cast<size_t>(d.K) + 15) / 16 * 16;
  uint64_t* lkeys = reinterpret_cast<uint64_t*>(dyn + off_k);
  const int key_cap = static_cast<int>((kLdsLimit - off_k) / 8);
  const int keff = min(d.K, length);
  // (clamped: consistent scores and histogram never need it, but every index below stays in its row)
  const int b1 = bd.x, n_above = min(max(bd.y, 0), keff - 1), n_bd = min(max(bd.z, 0), length);
  const bool keys_lds = n_bd <= key_cap;
  uint64_t* gkeys = b.bkeys + static_cast<long>(bh) * d.max_len;
  const uint2* hits_row = b.hits + static_cast<long>(bh) * d.max_len;

  // ---- 1. segment offsets ----
  {
    int tot;
    const int o = block_exclusive_scan(cc, &tot, sh.tmp);
    if (tid < nW) {
      aoff[tid] = o;
      srow0[tid] = slo;
    }
    if (tid == 0) aoff[nW] = tot;
    lds_barrier();
  }
  const int ns = aoff[nW];
  float qb0 = 0.f, qb1 = 0.f;
  if (push && tid < 64) normalize_row(qw2, qb0, qb1);

  // ---- 2. classification, candidate keys, radix select ----
  const int nrounds = (ns + kHeadThreads * kSU - 1) / (kHeadThreads * kSU);
  int pos[kSU];
  uint32_t sb[kSU];
  auto load_round = [&](int rd) {
    const int i0 = rd * kHeadThreads * kSU + tid * kSU;
    // the segment holding survivor i0 (the last whose offset is <= i0), then
    // forward from there for the following ones
    int sg = 0;
    if (i0 < ns) {
      int hi = nW;
      while (hi - sg > 1) {
        const int mid = (sg + hi) >> 1;
        if (aoff[mid] <= i0) sg = mid; else hi = mid;
      }
    }
    uint2 e[kSU];
#pragma unroll
    for (int u = 0; u < kSU; ++u) {
      const int i = i0 + u;
      e[u] = make_uint2(0xffffffffu, 0u);
      if (i < ns) {
        while (aoff[sg + 1] <= i) ++sg;  // aoff[nW] = ns > i ends it
        e[u] = load_shared(hits_row + srow0[sg] + (i - aoff[sg]));
      }
    }
#pragma unroll
    for (int u = 0; u < kSU; ++u) {
      pos[u] = static_cast<int>(e[u].x);  // -1 past the end
      sb[u] = e[u].y;
    }
  };
  auto bin_of = [&](int u) { return static_cast<int>(order_key(__uint_as_float(sb[u])) >> kHistShift); };
  auto in_b1 = [&](int u) { return (pos[u] >= 0) & (bin_of(u) == b1); };
  auto above = [&](int u) { return (pos[u] >= 0) & (bin_of(u) > b1); };

  // candidate keys, compacted in position order
  {
    int krun = 0;
    for (int rd = 0; rd < nrounds; ++rd) {
      load_round(rd);
      int c = 0;
#pragma unroll
      for (int u = 0; u < kSU; ++u) c += in_b1(u);
      int tot;
      int o = krun + block_exclusive_scan(c, &tot, sh.tmp);
#pragma unroll
      for (int u = 0; u < kSU; ++u) {
        if (in_b1(u)) {
          const uint64_t key = comp_key(__uint_as_float(sb[u]), static_cast<uint32_t>(pos[u]));
          if (o < n_bd) {
            if (keys_lds) lkeys[o] = key;
            else gkeys[o] = key;
          }
          ++o;
        }
      }
      krun += tot;
    }
  }
  lds_barrier();
  // Radix select of the `need` best candidates. Their composite keys share
  // the top 10 bits (the bin b1), so the digits start below them, 11 bits at
  // a time: bits 53-43, 42-32 (score), 31-21, 20-10, 9-0 (index).
  int need = keff - n_above;
  int ncand = n_bd;
  uint64_t mask = 0x3FFull << 54, prefix = static_cast<uint64_t>(b1) << 54;
  int* bins = &sh.whist[0][0];
  for (int shift = 43; ncand > need && need > 0; shift = shift >= 11 ? shift - 11 : 0) {
    const uint64_t dmask = shift == 0 ? 0x3FFull : 0x7FFull;
    reinterpret_cast<int4*>(bins)[tid] = make_int4(0, 0, 0, 0);
    lds_barrier();
    if (keys_lds) {
      for (int i = tid; i < n_bd; i += kHeadThreads) {
        const uint64_t u = lkeys[i];
        if ((u & mask) == prefix) atomicAdd(&bins[(u >> shift) & dmask], 1);
      }
    } else {
      for (int i = tid; i < n_bd; i += kHeadThreads) {
        const uint64_t u = gkeys[i];
        if ((u & mask) == prefix) atomicAdd(&bins[(u >> shift) & dmask], 1);
      }
    }
    lds_barrier();
    pick_bin2048(sh, need);
    prefix |= static_cast<uint64_t>(sh.i0) << shift;
    mask |= dmask << shift;
    need = sh.i1;
    ncand = sh.i2;
    if (shift == 0) break;
  }

  // ---- 3. S_t in ascending index order: survivors above b1 and the kept candidates ----
  int n = 0;
  for (int rd = 0; rd < nrounds; ++rd) {
    if (nrounds > 1) load_round(rd);  // one round: still in registers
    bool keep[kSU];
    int c = 0;
#pragma unroll
    for (int u = 0; u < kSU; ++u) {
      keep[u] = above(u) |
                (in_b1(u) & ((comp_key(__uint_as_float(sb[u]), static_cast<uint32_t>(pos[u])) & mask) >= prefix));
      c += keep[u];
    }
    int tot;
    int o = n + block_exclusive_scan(c, &tot, sh.tmp);
#pragma unroll
    for (int u = 0; u < kSU; ++u) {
      if (keep[u]) {
        if (o < d.K) {
          s_sel[o] = pos[u];
          s_selsc[o] = __uint_as_float(sb[u]);
        }
        ++o;
      }
    }
    n += tot;
  }
  n = min(n, keff);
  lds_barrier();
  finish_tail(d, b, bh, n, v, out, sel_out, push, fifo_slot, fifo_count, sh, s_sel, s_selsc, qb0, qb1);
  return true;
}

// Clears the other half (the next call's) of score work group w's slice of
// the heads' histograms. (w BH < 2^29: 32-bit divisions)
__device__ __forceinline__ void clear_next_half(ConstBufs& b, int w, int nW, int BH, int par) {
  for (int hh = static_cast<int>(static_cast<uint32_t>(w * BH) / static_cast<uint32_t>(nW));
       hh < static_cast<int>(static_cast<uint32_t>((w + 1) * BH) / static_cast<uint32_t>(nW)); ++hh) {
    uint4* hz = reinterpret_cast<uint4*>(b.hist + (static_cast<long>(hh) * 2 + (par ^ 1)) * kNumBins);
    for (int i = threadIdx.x; i < kNumBins / 4; i += kHeadThreads) hz[i] = make_uint4(0u, 0u, 0u, 0u);
  }
}

// w: this score work group's index among the nW of them. all_exact: every
// head of the call is exact (no flags to wait for). keep: rows per head of
// LDS for the scores of phase 1 (a multiple of 16; 0: they go to the score
// workspace, or, with kLong, into K-best lists where those fit).
template <bool kLong>
__device__ __forceinline__ void score_role(const Dims& d, ConstBufs& bt, const uint16_t* q, long q_sb, long q_sh,
                                           const uint16_t* k, const uint16_t* v, float* out, int32_t* sel_out,
                                           int length, int push, int call_flag, int w, int nW, bool all_exact,
                                           int keep, HeadShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = kHeadThreads >> 6;
  const int j = lane & 15, kq = lane >> 4;
  const int NG = d.B * d.Hkv, BH = d.B * d.Hq;
  const int par = (call_flag >> 1) & 1;
  int vpar = 0;  // block_all's vote set
  __shared__ int s_eg[kMaxExactGroups];  // listed group | its exact heads << 16 (bit jj: head jj of the group)
  __shared__ int s_tmp[8];
  __shared__ uint32_t s_ex[kMaxExactGroups * kMaxGroup / 32];  // exact bit of every head
  __shared__ KbState s_kb;                          // K-best lists of the current segment
  __shared__ int s_kbstride[kKbMaxSeg];             // ... finished lists' stride per segment
  extern __shared__ __align__(16) unsigned char dyn[];
  // LDS: histograms [G, kNumBins] (phase 1), then the kept scores
  // [G, keep + 4] (phase 1 -> 3); phase 4 reuses all of it
  uint32_t* s_hist = reinterpret_cast<uint32_t*>(dyn);
  const int stride = keep + 4;
  float* s_sc = reinterpret_cast<float*>(dyn + static_cast<size_t>(d.G) * kNumBins * 4);

  // clear the other half of a slice of the heads' histograms for the next
  // call: once on every way out of the work group, in phase 1 after the first
  // key loads are requested (the table read it needs then waits beside them)
  // (w BH < 2^29: 32-bit divisions)
  bool cleared = false;

  // every head's decision of this call, published by the head work groups
  // (lower block indices, so already running); bounded wait
  if (!all_exact) {
    int done = 0;
    for (int it = 0; it < kPollRounds; ++it) {
      for (int i = threadIdx.x; i < (BH + 31) / 32; i += kHeadThreads) s_ex[i] = 0u;
      lds_barrier();
      int mine = 1;
      for (int i = threadIdx.x; i < BH; i += kHeadThreads) {
        const int x = load_shared(bt.dec + i * kFlagStride);
        mine &= (x | 1) == (call_flag | 1);
        if (x & 1) atomicOr(&s_ex[i >> 5], 1u << (i & 31));
      }
      done = block_all(mine, sh.vote, vpar);
      if (done) break;
      __builtin_amdgcn_s_sleep(kPollSleep);
    }
    if (!done) {
      clear_next_half(bt, w, nW, BH, par);
      if (threadIdx.x == 0) store_shared(bt.err, 1);
      return;
    }
  }

  // ordered list of the KV groups holding an exact head
  int ne;
  {
    const int per = (NG + kHeadThreads - 1) / kHeadThreads;
    const int g0 = min(static_cast<int>(threadIdx.x) * per, NG), g1 = min(g0 + per, NG);
    int cnt = 0;
    for (int bg = g0; bg < g1; ++bg) {
      const int bb = bg / d.Hkv, g = bg % d.Hkv;
      int m = all_exact ? (1 << d.G) - 1 : 0;
      for (int jj = 0; !all_exact && jj < d.G; ++jj) {
        const int hh = bb * d.Hq + g * d.G + jj;
        m |= ((s_ex[hh >> 5] >> (hh & 31)) & 1) << jj;
      }
      cnt += m != 0;
    }
    int o = block_exclusive_scan(cnt, &ne, s_tmp);
    if (!all_exact && w == 0 && threadIdx.x == 0) bt.hint[0] = ne;  // (host-mapped; sizes later launches)
    for (int bg = g0; bg < g1; ++bg) {
      const int bb = bg / d.Hkv, g = bg % d.Hkv;
      int m = all_exact ? (1 << d.G) - 1 : 0;
      for (int jj = 0; !all_exact && jj < d.G; ++jj) {
        const int hh = bb * d.Hq + g * d.G + jj;
        m |= ((s_ex[hh >> 5] >> (hh & 31)) & 1) << jj;
      }
      if (m != 0) s_eg[o++] = bg | (m << 16);
    }
  }
  lds_barrier();
  if (ne == 0) {
    clear_next_half(bt, w, nW, BH, par);
    return;
  }
  const long T = static_cast<long>(ne) * length;
  int e0, r0, e1, r1;
  split_at(T, nW, length, ne, w, e0, r0);
  split_at(T, nW, length, ne, w + 1, e1, r1);
  // long histories: K-best lists when this work group's segments allow them
  bool use_kb = false;
  int nseg = 0;
  if constexpr (kLong) {
    for (int e = e0, r = r0; e < e1 || (e == e1 && r < r1); ++e, r = 0) nseg += r < (e == e1 ? r1 : length);
    use_kb = T >= kKbMinShare * nW && kb_fits(d, nseg);
  }
  const int kp = kb_stride(d.K);

  // ---- phase 1: scores and histograms ----
  if constexpr (kLong) {
    for (int e = e0, r = r0, si = 0; use_kb && (e < e1 || (e == e1 && r < r1)); ++e, r = 0) {
      const int row0 = r, rend = e == e1 ? r1 : length;
      if (row0 >= rend) continue;
      const int bg = s_eg[e] & 0xffff;
      const int bb = bg / d.Hkv, g = bg % d.Hkv;
      const int h = g * d.G + j;
      const unsigned emask = static_cast<unsigned>(s_eg[e]) >> 16;
      const bool hv = (j < d.G) && ((emask >> j) & 1u);
      bf16x8 bq[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint4 u = make_uint4(0u, 0u, 0u, 0u);
        if (hv) u = *reinterpret_cast<const uint4*>(q + bb * q_sb + h * q_sh + 8 * kq + 32 * s);
        bq[s] = as_bf16x8(u);
      }
      const uint16_t* kb = k + static_cast<long>(bb * d.Hkv + g) * d.max_len * kHeadDim;
      QkTiles ta, tb;
      qk_load(ta, kb, row0, rend, wave, nw, j, kq);
      if (!cleared) {
        clear_next_half(bt, w, nW, BH, par);
        cleared = true;
      }
      const int cap = kb_cap(d, si);
      int* tc = reinterpret_cast<int*>(dyn);  // two stages' slot tables
      uint2* lists = reinterpret_cast<uint2*>(dyn + kb_tc_bytes(d)) + static_cast<long>(si) * d.G * kp;
      if (threadIdx.x < d.G) {
        s_kb.n[threadIdx.x] = 0;
        s_kb.theta[threadIdx.x] = 0ull;
        s_kb.lo[threadIdx.x] = 0xffffffffu;
        s_kb.hi[threadIdx.x] = 0u;
        s_kb.full[threadIdx.x] = 0;
      }
      lds_barrier();  // (also: the previous segment's histogram is read out)
      uint64_t theta = 0ull;
      const int kStage = 16 * kQkUnroll * nw;  // rows per stage
      for (int t0 = row0; t0 < rend; t0 += 2 * kStage) {
        qk_load(tb, kb, t0 + kStage, rend, wave, nw, j, kq);
        qk_score_kb(d, ta, bq, t0, rend, wave, nw, j, kq, hv, theta, lists, cap, tc, s_kb, emask, sh);
        if (t0 + kStage >= rend) break;
        qk_load(ta, kb, t0 + 2 * kStage, rend, wave, nw, j, kq);
        qk_score_kb(d, tb, bq, t0 + kStage, rend, wave, nw, j, kq, hv, theta, lists, cap, tc + d.G * kKbTc, s_kb,
                    emask, sh);
      }
      const int stride = kb_close(d, bt, bb, g, emask, par, lists, cap, kp, si == nseg - 1, s_kb, s_kb.cnt[si], sh);
      if (threadIdx.x == 0) s_kbstride[si] = stride;
      ++si;
    }
  }
  for (int e = e0, r = r0, lb = 0; !use_kb && (e < e1 || (e == e1 && r < r1)); ++e, r = 0) {
    const int row0 = r, rend = e == e1 ? r1 : length;
    if (row0 >= rend) continue;
    const int bg = s_eg[e] & 0xffff;
    const int bb = bg / d.Hkv, g = bg % d.Hkv;
    const int h = g * d.G + j;
    const bool hv = (j < d.G) && ((static_cast<unsigned>(s_eg[e]) >> (16 + j)) & 1u);
    bf16x8 bq[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 u = make_uint4(0u, 0u, 0u, 0u);
      if (hv) u = *reinterpret_cast<const uint4*>(q + bb * q_sb + h * q_sh + 8 * kq + 32 * s);
      bq[s] = as_bf16x8(u);
    }
    const uint16_t* kb = k + static_cast<long>(bb * d.Hkv + g) * d.max_len * kHeadDim;
    QkTiles ta, tb;
    qk_load(ta, kb, row0, rend, wave, nw, j, kq);
    if (!cleared) {
      clear_next_half(bt, w, nW, BH, par);
      cleared = true;
    }
    const unsigned emask = static_cast<unsigned>(s_eg[e]) >> 16;
    lds_barrier();  // the previous segment's histogram flush is done
    for (int jj = 0; jj < d.G; ++jj)
      if ((emask >> jj) & 1)
        for (int i = threadIdx.x; i < kNumBins; i += kHeadThreads) s_hist[jj * kNumBins + i] = 0u;
    lds_barrier();
    // row r of the segment goes to LDS row lb + (r - row0) of head j, or to
    // the workspace row
    const bool to_lds = keep > 0;
    lds_float* ldst = (lds_float*)(s_sc + (j < d.G ? j : 0) * stride);  // (address-space cast)
    float* gdst = bt.score + static_cast<long>(bb * d.Hq + h) * d.score_stride;
    const int off = to_lds ? lb - row0 : 0;
    uint32_t* hrow = s_hist + j * kNumBins;
    const int kStage = 16 * kQkUnroll * nw;  // rows per stage
    for (int t0 = row0; t0 < rend; t0 += 2 * kStage) {
      qk_load(tb, kb, t0 + kStage, rend, wave, nw, j, kq);
      qk_score(ta, bq, t0, rend, wave, nw, kq, hv, to_lds, ldst, gdst, off, hrow);
      if (t0 + kStage >= rend) break;
      qk_load(ta, kb, t0 + 2 * kStage, rend, wave, nw, j, kq);
      qk_score(tb, bq, t0 + kStage, rend, wave, nw, kq, hv, to_lds, ldst, gdst, off, hrow);
    }
    lds_barrier();
    for (int jj = 0; jj < d.G; ++jj) {
      if (!((emask >> jj) & 1)) continue;
      uint32_t* ghist = bt.hist + (static_cast<long>(bb * d.Hq + g * d.G + jj) * 2 + par) * kNumBins;
      for (int i = threadIdx.x; i < kNumBins; i += kHeadThreads) {
        const uint32_t c = s_hist[jj * kNumBins + i];
        if (c) atomicAdd(&ghist[i], c);
      }
    }
    lb += (rend - row0 + 15) & ~15;
  }
  if (!cleared) clear_next_half(bt, w, nW, BH, par);  // (no rows in this call)
  wait_vmem();      // this wave's histogram adds (and workspace scores) have completed ...
  __syncthreads();  // ... in every wave, before the flag that publishes them
  if (threadIdx.x == 0) store_shared(bt.wdone + w * kFlagStride, call_flag);

  // a copy of the table for the later phases (read while this work group
  // scans: phase 1 reads its fields in place, so that its first key loads
  // do not wait for the table)
  const BufsDev b = bt;

  // the heads this work group finishes: head m of group e when x_m (see
  // above) falls in [xa, xb)
  // (no 64-bit divisions: the share bounds as in split_at, and
  // (2m + 1) length < 2^29)
  int ea, rra, ebb, rrb;
  share_start(nW, length, ne, w, ea, rra);
  share_start(nW, length, ne, w + 1, ebb, rrb);
  const long xa = static_cast<long>(ea) * length + rra, xb = static_cast<long>(ebb) * length + rrb;
  const int eb = xb > xa ? (rrb > 0 ? ebb : ebb - 1) : ea - 1;  // the group of row xb - 1
  auto owned = [&](int e, int m, int nex) {
    const long xm = static_cast<long>(e) * length +
                    static_cast<uint32_t>((2 * m + 1) * length) / static_cast<uint32_t>(2 * nex);
    return xa <= xm && xm < xb;
  };

  // ---- phase 2: survivors of every segment ----
  uint64_t seen = 0;  // bit e - e0: list group e is known to be fully scored
  for (int e = e0, r = r0, lb = 0, si = 0; e < e1 || (e == e1 && r < r1); ++e, r = 0) {
    const int row0 = r, rend = e == e1 ? r1 : length;
    if (row0 >= rend) continue;
    const int bg = s_eg[e] & 0xffff;
    if (!wait_group(b.wdone, T, nW, length, ne, e, call_flag, b.err, &sh.i3, sh.vote, vpar)) return;
    if (e - e0 < 64) seen |= 1ull << (e - e0);
    if (use_kb) {
      emit_kb(d, b, bg / d.Hkv, bg % d.Hkv, static_cast<unsigned>(s_eg[e]) >> 16, row0, length, w, par, call_flag,
              reinterpret_cast<const uint2*>(dyn + kb_tc_bytes(d)) + static_cast<long>(si) * d.G * kp,
              s_kbstride[si], s_kb.cnt[si]);
      ++si;
    } else if (keep > 0)
      emit_segment<true>(d, b, bg / d.Hkv, bg % d.Hkv, static_cast<unsigned>(s_eg[e]) >> 16, row0, rend, length, w,
                         par, call_flag, s_sc + lb, stride);
    else
      emit_segment<false>(d, b, bg / d.Hkv, bg % d.Hkv, static_cast<unsigned>(s_eg[e]) >> 16, row0, rend, length, w,
                          par, call_flag, nullptr, stride);
    lb += (rend - row0 + 15) & ~15;
  }

  // ---- phase 3: finish the owned heads ----
  for (int e = ea; e <= eb; ++e) {
    const int bg = s_eg[e] & 0xffff;
    const unsigned emask = static_cast<unsigned>(s_eg[e]) >> 16;
    const int nex = __popc(emask);
    for (int m = 0; m < nex; ++m) {
      if (!owned(e, m, nex)) continue;
      const int bh = (bg / d.Hkv) * d.Hq + (bg % d.Hkv) * d.G + nth_bit(emask, m);
      // the head's boundary (its group is fully scored once this work group's
      // own segment of it has passed phase 2; else wait for that here), read
      // by wave 0 into sh.i0 .. i2 while the finish polls the survivor counts
      const bool scored = e - e0 < 64 && ((seen >> (e - e0)) & 1);
      if (!scored && !wait_group(b.wdone, T, nW, length, ne, e, call_flag, b.err, &sh.i3, sh.vote, vpar)) return;
      if ((threadIdx.x >> 6) == 0) {
        const int3 bd = wave_boundary(b.hist + (static_cast<long>(bh) * 2 + par) * kNumBins, min(d.K, length));
        if (threadIdx.x == 0) {
          sh.i0 = bd.x;
          sh.i1 = bd.y;
          sh.i2 = bd.z;
        }
      }
      if (!finish_phase(d, b, bh, q, q_sb, q_sh, v, out, sel_out, length, push, call_flag, T, nW, ne, e, sh, dyn,
                        vpar))
        return;
      lds_barrier();  // the next finish reuses the LDS
    }
  }
}

// ---------------------------------------------------------------------------
// A decode step (or an exact call), one launch over the work-group index space
//   [0, BH)        head work groups (query heads);
//   [BH, BH + NS)  score work groups (also the exact heads' Top-K and finish).
// ---------------------------------------------------------------------------
template <bool kLong>
__global__ __launch_bounds__(kHeadThreads) void k_step(Dims d, const Bufs* __restrict__ bp, const uint16_t* q, long q_sb, long q_sh,
                                                       const uint16_t* k, const uint16_t* v, float* out,
                                                       int32_t* sel_out, int length, int t_dec, int mode,
                                                       int stats_slot, int push, int call_flag, int n_score,
                                                       int keep, const int32_t* ctl, int layer) {
  __shared__ HeadShared sh;
  if (ctl != nullptr) {
    // A step replayed from a graph: the position and the call's sequence
    // number come from the control words that k_advance moved on at the head
    // of the replay (an earlier launch on the stream); this layer's call is
    // `layer` steps after the replay's first.
    length = scalar_read_ptr(ctl);
    t_dec = scalar_read_ptr(ctl + 1);
    const int seq = (scalar_read_ptr(ctl + 2) + layer) & kSeqMask;
    call_flag = 2 * seq;
    if (stats_slot >= 0) stats_slot = (t_dec - 1) % kStatsCap;
  }
  // The buffer table is not held in the kernel's argument registers, which
  // would keep it live through both roles: each role reads its own copy.
  const int BH = d.B * d.Hq;
  const int w = static_cast<int>(blockIdx.x);
  // (marked likely so that the head role's code comes first: its addresses
  // then stay put when the score role's code changes size)
  if (__builtin_expect(w < BH, 1)) {
    head_role(d, *(ConstBufs*)(reinterpret_cast<uintptr_t>(bp)), q, q_sb, q_sh, k, v, out, length, t_dec, mode, stats_slot,
              call_flag, w, sh);
  } else {
    ConstBufs& b = *(ConstBufs*)(reinterpret_cast<uintptr_t>(bp));
    // every head is exact in an exact call and on a refresh step (Eq. 13):
    // then there are no decisions to wait for
    const bool all_exact = mode == kModeExact || (d.Tr > 0 && t_dec % d.Tr == 0);
    score_role<kLong>(d, b, q, q_sb, q_sh, k, v, out, sel_out, length, push, call_flag, w - BH, n_score, all_exact,
                      keep, sh);
  }
}

// ---------------------------------------------------------------------------
// Launch helpers
// ---------------------------------------------------------------------------
hipError_t configure_kernels(const Dims& d) {
  const int lds = static_cast<int>(step_lds_bytes(d));
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_step<false>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_step<true>), hipFuncAttributeMaxDynamicSharedMemorySize,
                            lds);
  return e;
}

const char* kernel_name(int id) {
  static const char* names[kNumKernels] = {"k_step", "k_reset", "k_dense", "k_dense_merge", "k_advance"};
  return (id >= 0 && id < kNumKernels) ? names[id] : "";
}

hipError_t launch_reset(const Dims& d, const Bufs& b, hipStream_t s) {
  const int bh = d.B * d.Hq;
  hipLaunchKernelGGL(k_reset, dim3((bh + 255) / 256), dim3(256), 0, s, d, b);
  return hipGetLastError();
}

hipError_t launch_step(const Dims& d, const Bufs& b, const uint16_t* q, long q_sb, long q_sh, const uint16_t* k,
                       const uint16_t* v, float* out, int32_t* sel_out, int length, int t_dec, int mode,
                       int stats_slot, int push, int call_flag, bool wide, hipStream_t s, const int32_t* ctl,
                       int layer) {
  // (a replayed step is sized for `length`, the longest of its replays)
  const int n_score = score_grid(d, length, mode, wide);
  const int keep = score_keep_rows(d, length, n_score);
  // Scores that do not fit the score work groups' LDS: the variant with K-best
  // lists, for calls expected to be mostly exact. Its larger score role costs
  // the head role about 1 us of register spills, so decode steps take it only
  // from kKbDecodeLen keys on, where its refresh steps save more than that.
  if (keep == 0 && (mode == kModeExact || wide || length >= kKbDecodeLen))
    hipLaunchKernelGGL(k_step<true>, dim3(d.B * d.Hq + n_score), dim3(kHeadThreads), step_lds_bytes(d), s, d, b.self,
                       q, q_sb, q_sh, k, v, out, sel_out, length, t_dec, mode, stats_slot, push, call_flag, n_score,
                       keep, ctl, layer);
  else
    hipLaunchKernelGGL(k_step<false>, dim3(d.B * d.Hq + n_score), dim3(kHeadThreads), step_lds_bytes(d), s, d,
                       b.self, q, q_sb, q_sh, k, v, out, sel_out, length, t_dec, mode, stats_slot, push, call_flag,
                       n_score, keep, ctl, layer);
  return hipGetLastError();
}

// The control words of graph-replayed steps: {length, t_dec, seq}. k_advance
// moves them on by one token (n_layers calls); k_set_position sets them.
__global__ void k_advance(int32_t* ctl, int n_layers) {
  if (threadIdx.x == 0) {
    ctl[0] += 1;
    ctl[1] += 1;
    ctl[2] = (ctl[2] + n_layers) & kSeqMask;
  }
}

__global__ void k_set_position(int32_t* ctl, int length, int t_dec, int seq) {
  if (threadIdx.x == 0) {
    ctl[0] = length;
    ctl[1] = t_dec;
    ctl[2] = seq & kSeqMask;
  }
}

hipError_t launch_advance(int32_t* ctl, int n_layers, hipStream_t s) {
  hipLaunchKernelGGL(k_advance, dim3(1), dim3(64), 0, s, ctl, n_layers);
  return hipGetLastError();
}

hipError_t launch_set_position(int32_t* ctl, int length, int t_dec, int seq, hipStream_t s) {
  hipLaunchKernelGGL(k_set_position, dim3(1), dim3(64), 0, s, ctl, length, t_dec, seq);
  return hipGetLastError();
}

}  // namespace retopk

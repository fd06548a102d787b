// ReTopK decode-step kernels for CDNA4 (gfx950, wave64).
//
// Method: "Recall Before You Rank: Similarity-Guided Top-K Reuse for
// Efficient Long-Context Attention", Methodology section. A decode step is
// four launches on one stream:
//
//   k_head      one work group per query head: recall (Eqs. 5-7) and the path
//               rule (Eq. 13); for reuse heads, in the same work group, the
//               candidate union (Eqs. 8-9), candidate scores (Eq. 10), the
//               rerank to K (Eq. 11), sparse softmax-V (Eq. 12) and the cache
//               update. No data crosses work groups, so no inter-group sync.
//   k_exact_qk  full-history scores (Eq. 4) for the KV groups holding at least
//               one exact head, GQA-grouped on MFMA, plus a score histogram;
//   k_collect   global Top-K (Eq. 1), step 1: threshold bin and collection;
//   k_finish    global Top-K, step 2: boundary resolution and ascending order;
//               then softmax-V and the cache update for exact heads.
//
// The path flag stays on the device: the exact-path kernels read it and
// return at once where no head of theirs is exact, so the host never waits.
// Every phase issues its global loads before consuming them, so a phase costs
// about one memory round trip rather than one per loop iteration.

#include "retopk_internal.h"

#include <algorithm>
#include <cmath>

namespace retopk {

namespace {

constexpr float kNegInf = -INFINITY;
constexpr float kInvSqrtD = 0.08838834764831845f;  // 1 / sqrt(128)

// Order-preserving map of a float32 to uint32 (larger float, larger key).
// Negative zero is folded into positive zero so that the two compare equal.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ float wave_max_f32(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// Block-wide exclusive prefix sum of one int per thread. `tmp` holds at
// least blockDim.x / 64 ints. Every thread of the block must call it.
__device__ int block_exclusive_scan(int v, int* total, int* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    const int x = tmp[w];
    if (w < wave) before += x;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return before + incl - v;
}

__device__ float block_max_f32(float v, float* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_max_f32(v);
  if (lane == 0) tmp[wave] = v;
  __syncthreads();
  float m = kNegInf;
  for (int w = 0; w < nw; ++w) m = fmaxf(m, tmp[w]);
  __syncthreads();
  return m;
}

// Emit, in ascending order, the positions base + bit of every set bit of an
// LDS bitmap of `nwords` words to out[0 ..). Returns the number emitted (the
// same value in every thread). Every thread of the block must call it.
__device__ int bitmap_emit(const uint32_t* bm, int nwords, int base, int32_t* out, int* tmp) {
  const int per = (nwords + blockDim.x - 1) / blockDim.x;
  const int w0 = threadIdx.x * per;
  const int w1 = min(w0 + per, nwords);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bm[w]);
  int total;
  int off = block_exclusive_scan(cnt, &total, tmp);
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = bm[w];
    while (bits) {
      const int b = __ffs(bits) - 1;
      out[off++] = base + w * 32 + b;
      bits &= bits - 1;
    }
  }
  return total;
}

// Shared scratch of the per-head kernels (static LDS).
struct HeadShared {
  float q[kHeadDim];           // raw query as float
  float qbar[kHeadDim];        // normalised query
  double rho[64];
  int slot[64], len[64];       // retrieved ring slots and their support sizes
  int hist[256];
  int tmp[16];
  float red[kHeadThreads / 64][kHeadDim + 4];
  int i0, i1, i2, i3;
  double d0;
};

// K-th largest of n scores (LDS) under (score desc, position asc): radix
// select over the order-preserving keys, 8 bits per pass. Returns the key T of
// the K-th largest; *need receives how many entries equal to T are taken (the
// lowest positions first). Every thread of the block must call it.
__device__ uint32_t radix_kth(const float* sc, int n, int k, HeadShared& sh, int* need) {
  uint32_t prefix = 0u, mask = 0u;
  int rem = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (threadIdx.x < 256) sh.hist[threadIdx.x] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const uint32_t u = order_key(sc[i]);
      if ((u & mask) == prefix) atomicAdd(&sh.hist[(u >> shift) & 255u], 1);
    }
    __syncthreads();
    const int digit = 255 - static_cast<int>(threadIdx.x & 255);
    const int c = threadIdx.x < 256 ? sh.hist[digit] : 0;
    int tot;
    const int above = block_exclusive_scan(c, &tot, sh.tmp);
    if (threadIdx.x < 256 && above < rem && above + c >= rem) {
      sh.i0 = digit;
      sh.i1 = rem - above;
    }
    __syncthreads();
    prefix |= static_cast<uint32_t>(sh.i0) << shift;
    mask |= 255u << shift;
    rem = sh.i1;
    __syncthreads();
  }
  *need = rem;
  return prefix;
}

// Keep, in position order, the entries with key > T and the first `need`
// entries with key == T; write their positions' values idx[i] / sc[i] to
// out_idx / out_sc. Returns the number kept. Every thread must call it.
__device__ int select_in_order(const int32_t* idx, const float* sc, int n, uint32_t T, int need,
                               int32_t* out_idx, float* out_sc, HeadShared& sh) {
  const int per = (n + blockDim.x - 1) / blockDim.x;
  const int i0 = threadIdx.x * per, i1 = min(i0 + per, n);
  int eq = 0;
  for (int i = i0; i < i1; ++i) eq += (order_key(sc[i]) == T);
  int tot;
  const int eq_before = block_exclusive_scan(eq, &tot, sh.tmp);
  int nsel = 0, e = eq_before;
  for (int i = i0; i < i1; ++i) {
    const uint32_t u = order_key(sc[i]);
    nsel += (u > T) || (u == T && e < need);
    e += (u == T);
  }
  int kept;
  int o = block_exclusive_scan(nsel, &kept, sh.tmp);
  e = eq_before;
  for (int i = i0; i < i1; ++i) {
    const uint32_t u = order_key(sc[i]);
    if ((u > T) || (u == T && e < need)) {
      out_idx[o] = idx[i];
      out_sc[o] = sc[i];
      ++o;
    }
    e += (u == T);
  }
  __syncthreads();
  return kept;
}

// Sparse softmax-V (Eq. 12) over n selected rows (indices and unscaled
// scores in LDS; mx = their maximum): 16 lanes per value row (16 bytes
// each), 8 row loads in flight per thread. Writes out[0 .. 127] when out is
// not NULL. Every thread of the block must call it.
__device__ void attend(const int32_t* sel, const float* sc, int n, float mx, const uint16_t* vb, float* out,
                       HeadShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int sub = threadIdx.x & 15, rg = threadIdx.x >> 4, rpr = blockDim.x >> 4;
  constexpr int U = 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float z = 0.f;
  for (int r0 = 0; r0 < n; r0 += rpr * U) {
    uint4 w[U];
    float p[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = r0 + u * rpr + rg;
      if (i < n) {
        w[u] = *reinterpret_cast<const uint4*>(vb + static_cast<long>(sel[i]) * kHeadDim + 8 * sub);
        p[u] = expf((sc[i] - mx) * kInvSqrtD);
      } else {
        w[u] = make_uint4(0u, 0u, 0u, 0u);
        p[u] = 0.f;
      }
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
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    acc[e] += __shfl_xor(acc[e], 16);
    acc[e] += __shfl_xor(acc[e], 32);
  }
  z += __shfl_xor(z, 16);
  z += __shfl_xor(z, 32);
  if (lane < 16) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sh.red[wave][8 * sub + e] = acc[e];
    if (lane == 0) sh.red[wave][kHeadDim] = z;
  }
  __syncthreads();
  if (out != nullptr && threadIdx.x < kHeadDim) {
    float a = 0.f, zz = 0.f;
    for (int w = 0; w < nw; ++w) {
      a += sh.red[w][threadIdx.x];
      zz += sh.red[w][kHeadDim];
    }
    out[threadIdx.x] = a / zz;
  }
  __syncthreads();
}

// Push (q_bar_t, S_hat_t) into the head's FIFO (Query-support cache
// paragraph: after either path; the oldest entry is overwritten when full).
__device__ void cache_push(const Dims& d, const Bufs& b, int bh, const float* qbar, const int32_t* sel, int n) {
  const int slot = b.fifo[2 * bh];
  const int count = b.fifo[2 * bh + 1];
  const long e = static_cast<long>(bh) * d.C + slot;
  for (int t = threadIdx.x; t < kHeadDim; t += blockDim.x) b.cache_qbar[e * kHeadDim + t] = qbar[t];
  for (int i = threadIdx.x; i < n; i += blockDim.x) b.cache_supp[e * d.K + i] = sel[i];
  if (threadIdx.x == 0) {
    b.cache_len[e] = n;
    b.fifo[2 * bh] = (slot + 1) % d.C;
    b.fifo[2 * bh + 1] = min(count + 1, d.C);
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

}  // namespace

size_t head_lds_bytes(const Dims& d) {
  const size_t region0 = std::max<size_t>(kBitmapWords * 4, 8 * static_cast<size_t>(d.K));
  return region0 + 8 * static_cast<size_t>(d.cand_cap);
}

size_t finish_lds_bytes(const Dims& d) {
  return std::max<size_t>(kBoundaryLds * 8, kBitmapWords * 4) + 8 * static_cast<size_t>(d.K);
}

// ---------------------------------------------------------------------------
// Reset the FIFO bookkeeping before cache initialisation. One thread per head.
// ---------------------------------------------------------------------------
__global__ void k_reset(Dims d, Bufs b) {
  const int bh = blockIdx.x * blockDim.x + threadIdx.x;
  if (bh >= d.B * d.Hq) return;
  b.fifo[2 * bh] = 0;
  b.fifo[2 * bh + 1] = 0;
}

// ---------------------------------------------------------------------------
// Per-head kernel: recall, path decision, and the reuse path.
//
// Recall (Eqs. 5-7): q_bar = fp32(x / ||x||) with fp64 sum of squares, sqrt
// and divide; rho_c = fp64 dot of the fp32 q_bar values for each held entry
// (16 threads per entry); R_t = the R largest rho (ties: older entry);
// rho_max. Path (Eq. 13): exact if refresh, empty cache or rho_max < tau.
// Exact heads clear the counters and histogram of the exact-path kernels and
// stop here.
//
// Reuse path, same work group:
//   union (Eqs. 8-9): retrieved supports and the window [max(0, L-W), L) set
//     bits of an LDS bitmap over token positions (windows of 262144), read
//     back in ascending order -> A_t in LDS, M_t;
//   scores (Eq. 10): q . k_i for i in A_t straight from the KV cache, 16 lanes
//     per key row, 8 rows in flight per thread, fp32 accumulation of exact
//     bf16 products;
//   rerank (Eq. 11): radix select of the K-th largest, kept in candidate
//     (= ascending index) order, ties to the lower index;
//   softmax-V (Eq. 12) and the cache update.
//
// LDS (dynamic): region0 = bitmap window (32 KiB), later the selected indices
// and scores (K each); then A_t and its scores (cand_cap each).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kHeadThreads) void k_head(Dims d, Bufs b, const uint16_t* q, long q_sb,
                                                       long q_sh, const uint16_t* k, const uint16_t* v,
                                                       float* out, int length, int t_dec, int mode,
                                                       int stats_slot) {
  const int bh = blockIdx.x;
  const int bb = bh / d.Hq, h = bh % d.Hq, g = h / d.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ HeadShared sh;
  extern __shared__ __align__(16) unsigned char dyn[];
  const size_t region0 = (kBitmapWords * 4 > 8 * d.K) ? kBitmapWords * 4 : 8 * d.K;
  uint32_t* bm = reinterpret_cast<uint32_t*>(dyn);
  int32_t* s_sel = reinterpret_cast<int32_t*>(dyn);
  float* s_selsc = reinterpret_cast<float*>(dyn + 4 * static_cast<size_t>(d.K));
  int32_t* s_cand = reinterpret_cast<int32_t*>(dyn + region0);
  float* s_sc = reinterpret_cast<float*>(dyn + region0 + 4 * static_cast<size_t>(d.cand_cap));

  // ---- normalised query (wave 0) ----
  if (wave == 0) {
    const uint32_t w2 = *reinterpret_cast<const uint32_t*>(q + bb * q_sb + h * q_sh + 2 * lane);
    const double x0 = bf16_lo(w2), x1 = bf16_hi(w2);
    const double nrm = sqrt(wave_sum_f64(x0 * x0 + x1 * x1));
    float qb0 = 0.f, qb1 = 0.f;
    if (nrm > 0.0) {
      qb0 = static_cast<float>(x0 / nrm);
      qb1 = static_cast<float>(x1 / nrm);
    }
    sh.q[2 * lane] = static_cast<float>(x0);
    sh.q[2 * lane + 1] = static_cast<float>(x1);
    sh.qbar[2 * lane] = qb0;
    sh.qbar[2 * lane + 1] = qb1;
    *reinterpret_cast<float2*>(b.qbar + static_cast<long>(bh) * kHeadDim + 2 * lane) = make_float2(qb0, qb1);
  }
  const int count = b.fifo[2 * bh + 1];
  const int oldest = (b.fifo[2 * bh] - count + d.C) % d.C;
  __syncthreads();

  bool exact = true, refresh = false;
  double rho_max = -INFINITY;
  int n_ret = 0;
  if (mode == kModeDecode) {
    refresh = d.Tr > 0 && (t_dec % d.Tr) == 0;
    // rho for entry c by 16 threads, 8 dimensions each
    for (int c0 = 0; c0 < count; c0 += kHeadThreads / 16) {
      const int c = c0 + (tid >> 4), part = tid & 15;
      double s = 0.0;
      if (c < count) {
        const float* e = b.cache_qbar + (static_cast<long>(bh) * d.C + (oldest + c) % d.C) * kHeadDim + 8 * part;
        const float4 e0 = *reinterpret_cast<const float4*>(e);
        const float4 e1 = *reinterpret_cast<const float4*>(e + 4);
        const float* t = sh.qbar + 8 * part;
        s = fma(static_cast<double>(t[0]), static_cast<double>(e0.x), s);
        s = fma(static_cast<double>(t[1]), static_cast<double>(e0.y), s);
        s = fma(static_cast<double>(t[2]), static_cast<double>(e0.z), s);
        s = fma(static_cast<double>(t[3]), static_cast<double>(e0.w), s);
        s = fma(static_cast<double>(t[4]), static_cast<double>(e1.x), s);
        s = fma(static_cast<double>(t[5]), static_cast<double>(e1.y), s);
        s = fma(static_cast<double>(t[6]), static_cast<double>(e1.z), s);
        s = fma(static_cast<double>(t[7]), static_cast<double>(e1.w), s);
      }
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s += __shfl_xor(s, 4);
      s += __shfl_xor(s, 8);
      if (part == 0 && c < count) sh.rho[c] = s;
    }
    __syncthreads();
    if (tid < count) {
      const double mine = sh.rho[tid];
      int rank = 0;
      for (int j = 0; j < count; ++j) {
        const double o = sh.rho[j];
        rank += (o > mine) || (o == mine && j < tid);
      }
      if (rank < d.R) {
        b.ret[bh * d.R + rank] = tid;
        b.retslot[bh * d.R + rank] = (oldest + tid) % d.C;
      }
      if (rank == 0) sh.d0 = mine;
    }
    n_ret = min(d.R, count);
    __syncthreads();
    if (count > 0) rho_max = sh.d0;
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
  if (exact) {
    if (tid == 0) b.m[bh] = 0;
    if (tid < 4) b.cnt[bh * 4 + tid] = 0;
    for (int i = tid; i < kNumBins; i += blockDim.x) b.hist[static_cast<long>(bh) * kNumBins + i] = 0u;
    return;
  }

  // ---- candidate union (Eqs. 8-9) ----
  const int wlo = max(0, length - d.W);
  if (tid < n_ret) {
    const int slot = b.retslot[bh * d.R + tid];
    sh.slot[tid] = slot;
    sh.len[tid] = b.cache_len[static_cast<long>(bh) * d.C + slot];
  }
  __syncthreads();
  int M = 0;
  for (int base = 0; base < length; base += kBitmapWords * 32) {
    const int nbits = min(kBitmapWords * 32, length - base);
    const int nwords = (nbits + 31) >> 5;
    for (int i = tid; i < nwords; i += blockDim.x) bm[i] = 0u;
    __syncthreads();
    const int total = n_ret * d.K;
    for (int i0 = 0; i0 < total; i0 += blockDim.x * 4) {
      int x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * blockDim.x + tid;
        x[u] = -1;
        if (i < total) {
          const int r = i / d.K, j = i - r * d.K;
          if (j < sh.len[r]) x[u] = b.cache_supp[(static_cast<long>(bh) * d.C + sh.slot[r]) * d.K + j] - base;
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (x[u] >= 0 && x[u] < nbits) atomicOr(&bm[x[u] >> 5], 1u << (x[u] & 31));
    }
    for (int x = max(wlo, base) + tid; x < base + nbits; x += blockDim.x) {
      const int y = x - base;
      atomicOr(&bm[y >> 5], 1u << (y & 31));
    }
    __syncthreads();
    M += bitmap_emit(bm, nwords, base, s_cand + M, sh.tmp);
    __syncthreads();
  }
  for (int i = tid; i < M; i += blockDim.x) b.cand[static_cast<long>(bh) * d.cand_cap + i] = s_cand[i];
  if (tid == 0) {
    b.m[bh] = M;
    if (stats_slot >= 0) b.st_m[static_cast<long>(stats_slot) * d.B * d.Hq + bh] = M;
  }

  // ---- candidate scores (Eq. 10) ----
  const uint16_t* kb = k + static_cast<long>(bb * d.Hkv + g) * d.max_len * kHeadDim;
  {
    const int sub = tid & 15, rg = tid >> 4, rpr = blockDim.x >> 4;
    float qf[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[e] = sh.q[8 * sub + e];
    constexpr int U = 8;
    for (int r0 = 0; r0 < M; r0 += rpr * U) {
      uint4 kv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = r0 + u * rpr + rg;
        kv[u] = (i < M) ? *reinterpret_cast<const uint4*>(kb + static_cast<long>(s_cand[i]) * kHeadDim + 8 * sub)
                        : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = r0 + u * rpr + rg;
        float s = qf[0] * bf16_lo(kv[u].x);
        s = fmaf(qf[1], bf16_hi(kv[u].x), s);
        s = fmaf(qf[2], bf16_lo(kv[u].y), s);
        s = fmaf(qf[3], bf16_hi(kv[u].y), s);
        s = fmaf(qf[4], bf16_lo(kv[u].z), s);
        s = fmaf(qf[5], bf16_hi(kv[u].z), s);
        s = fmaf(qf[6], bf16_lo(kv[u].w), s);
        s = fmaf(qf[7], bf16_hi(kv[u].w), s);
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 4);
        s += __shfl_xor(s, 8);
        if (sub == 0 && i < M) s_sc[i] = s;
      }
    }
  }
  __syncthreads();
  float mx = kNegInf;
  for (int i = tid; i < M; i += blockDim.x) {
    mx = fmaxf(mx, s_sc[i]);
    b.cscore[static_cast<long>(bh) * d.cand_cap + i] = s_sc[i];
  }
  mx = block_max_f32(mx, reinterpret_cast<float*>(sh.tmp));

  // ---- rerank (Eq. 11) ----
  int n;
  if (M <= d.K) {
    for (int i = tid; i < M; i += blockDim.x) {
      s_sel[i] = s_cand[i];
      s_selsc[i] = s_sc[i];
    }
    n = M;
    __syncthreads();
  } else {
    int need;
    const uint32_t T = radix_kth(s_sc, M, d.K, sh, &need);
    n = select_in_order(s_cand, s_sc, M, T, need, s_sel, s_selsc, sh);
  }
  for (int i = tid; i < n; i += blockDim.x) {
    b.sel[static_cast<long>(bh) * d.K + i] = s_sel[i];
    b.selsc[static_cast<long>(bh) * d.K + i] = s_selsc[i];
  }
  if (tid == 0) b.sellen[bh] = n;

  // ---- softmax-V (Eq. 12) and cache update ----
  const uint16_t* vb = v + static_cast<long>(bb * d.Hkv + g) * d.max_len * kHeadDim;
  attend(s_sel, s_selsc, n, mx, vb, out + static_cast<long>(bh) * kHeadDim, sh);
  cache_push(d, b, bh, sh.qbar, s_sel, n);
}

// ---------------------------------------------------------------------------
// Full-history scores (Eq. 4, unscaled) for every exact head, GQA-grouped:
// the rows of one KV head are split evenly over `wpg` work groups; each
// streams its rows exactly once and scores them for all query heads of the
// group with MFMA 16x16x32 bf16 tiles (A = 16 key rows x 32 dims, B = 32 dims
// x 16 query heads, fp32 accumulation). Scores go to the workspace and into a
// per-head histogram of the top 10 bits of their ordered keys (LDS, flushed
// with global atomics); the collect kernel finds the Top-K boundary from it.
// Work groups whose KV group has no exact head return at once.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_exact_qk(Dims d, Bufs b, const uint16_t* q, long q_sb, long q_sh,
                                                  const uint16_t* k, int length, int wpg) {
  const int bg = blockIdx.x / wpg, part = blockIdx.x % wpg;
  const int bb = bg / d.Hkv, g = bg % d.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, kq = lane >> 4;
  const int h = g * d.G + j;
  const bool hv = (j < d.G) && b.path[bb * d.Hq + h];
  if (__ballot(hv) == 0) return;  // same answer in every wave
  const int row0 = static_cast<int>((static_cast<long>(part) * length / wpg) & ~15L);
  const int rend = (part == wpg - 1) ? length : static_cast<int>((static_cast<long>(part + 1) * length / wpg) & ~15L);
  if (row0 >= rend) return;
  extern __shared__ uint32_t s_hist[];  // [G, kNumBins]
  bf16x8 bq[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (hv) u = *reinterpret_cast<const uint4*>(q + bb * q_sb + h * q_sh + 8 * kq + 32 * s);
    bq[s] = as_bf16x8(u);
  }
  for (int i = threadIdx.x; i < d.G * kNumBins; i += blockDim.x) s_hist[i] = 0u;
  __syncthreads();
  const uint16_t* kb = k + static_cast<long>(bb * d.Hkv + g) * d.max_len * kHeadDim;
  float* srow = b.score + static_cast<long>(bb * d.Hq + h) * d.score_stride;
  uint32_t* hrow = s_hist + j * kNumBins;
  constexpr int kUnroll = 4;
  for (int t0 = row0; t0 < rend; t0 += 64 * kUnroll) {
    uint4 a[kUnroll][4];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int r = t0 + (u * 4 + wave) * 16 + j;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        a[u][s] = (r < rend) ? *reinterpret_cast<const uint4*>(kb + static_cast<long>(r) * kHeadDim + 8 * kq + 32 * s)
                             : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int rbase = t0 + (u * 4 + wave) * 16;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[u][s]), bq[s], acc, 0, 0, 0);
      // lane holds query head j for rows rbase + 4*kq + 0..3
      if (hv) {
        const int r = rbase + 4 * kq;
        if (r + 3 < rend) {
          *reinterpret_cast<float4*>(srow + r) = make_float4(acc[0], acc[1], acc[2], acc[3]);
#pragma unroll
          for (int e = 0; e < 4; ++e) atomicAdd(&hrow[order_key(acc[e]) >> kHistShift], 1u);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (r + e < rend) {
              srow[r + e] = acc[e];
              atomicAdd(&hrow[order_key(acc[e]) >> kHistShift], 1u);
            }
          }
        }
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < d.G * kNumBins; i += blockDim.x) {
    const uint32_t c = s_hist[i];
    if (c) {
      const int hh = g * d.G + i / kNumBins;
      atomicAdd(&b.hist[static_cast<long>(bb * d.Hq + hh) * kNumBins + (i % kNumBins)], c);
    }
  }
}

// ---------------------------------------------------------------------------
// Global Top-K (Eq. 1), step 1, for exact heads: from the histogram find the
// boundary bin (the bin holding the K-th largest score), then classify a
// chunk of scores: indices in higher bins go to the "above" list (fewer than
// K in all), those in the boundary bin to the boundary list. Hits are staged
// in LDS; one atomic per list and work group reserves the global space.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_collect(Dims d, Bufs b, int length) {
  const int bh = blockIdx.x;
  if (!b.path[bh]) return;
  const int c0 = blockIdx.y * kCollectChunk;
  if (c0 >= length) return;
  __shared__ int tmp[8];
  __shared__ int s_b1;
  __shared__ int32_t s_list[kCollectChunk];
  __shared__ int s_nu, s_nb, s_gu, s_gb;
  const int keff = min(d.K, length);
  const float* srow = b.score + static_cast<long>(bh) * d.score_stride;
  // this thread's 16 consecutive scores, loaded before the histogram scan
  constexpr int kPerThread = kCollectChunk / 256;
  const int i0 = c0 + threadIdx.x * kPerThread;
  float v[kPerThread];
  if (i0 + kPerThread <= length) {
#pragma unroll
    for (int u = 0; u < kPerThread; u += 4) {
      const float4 f = *reinterpret_cast<const float4*>(srow + i0 + u);
      v[u] = f.x;
      v[u + 1] = f.y;
      v[u + 2] = f.z;
      v[u + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) v[u] = (i0 + u < length) ? srow[i0 + u] : 0.f;
  }
  const uint32_t* hist = b.hist + static_cast<long>(bh) * kNumBins;
  constexpr int kPer = kNumBins / 256;
  int c[kPer];
  int csum = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    c[i] = static_cast<int>(hist[kNumBins - 1 - (kPer * threadIdx.x + i)]);
    csum += c[i];
  }
  if (threadIdx.x == 0) {
    s_nu = 0;
    s_nb = 0;
    s_b1 = 0;
  }
  int tot;
  const int ex = block_exclusive_scan(csum, &tot, tmp);
  if (ex < keff && ex + csum >= keff) {
    int run = ex;
    for (int i = 0; i < kPer; ++i) {
      if (run + c[i] >= keff) {
        s_b1 = kNumBins - 1 - (kPer * threadIdx.x + i);
        break;
      }
      run += c[i];
    }
  }
  __syncthreads();
  const uint32_t b1 = static_cast<uint32_t>(s_b1);
  int nu = 0, nbd = 0;
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const bool valid = i0 + u < length;
    const uint32_t bin = order_key(v[u]) >> kHistShift;
    nu += valid && bin > b1;
    nbd += valid && bin == b1;
  }
  int ou = 0, ob = 0;
  if (nu) ou = atomicAdd(&s_nu, nu);
  if (nbd) ob = atomicAdd(&s_nb, nbd);
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    if (i0 + u < length) {
      const uint32_t bin = order_key(v[u]) >> kHistShift;
      if (bin > b1) s_list[kCollectChunk - 1 - (ou++)] = i0 + u;
      else if (bin == b1) s_list[ob++] = i0 + u;
    }
  }
  __syncthreads();
  const int tu = s_nu, tb = s_nb;
  if (threadIdx.x == 0) {
    s_gu = tu ? atomicAdd(&b.cnt[bh * 4 + 0], tu) : 0;
    s_gb = tb ? atomicAdd(&b.cnt[bh * 4 + 1], tb) : 0;
  }
  __syncthreads();
  int32_t* above = b.above + static_cast<long>(bh) * d.K;
  int32_t* bnd = b.bnd + static_cast<long>(bh) * d.max_len;
  // (fewer than K scores lie above the boundary bin; the guards only keep a
  // broken invariant from writing out of bounds)
  for (int t = threadIdx.x; t < tu; t += blockDim.x)
    if (s_gu + t < d.K) above[s_gu + t] = s_list[kCollectChunk - 1 - t];
  for (int t = threadIdx.x; t < tb; t += blockDim.x)
    if (s_gb + t < d.max_len) bnd[s_gb + t] = s_list[t];
}

// ---------------------------------------------------------------------------
// Global Top-K, step 2, for exact heads, then softmax-V and the cache update.
// Of the boundary-bin entries keep the `need` best under (score desc, index
// asc): a radix select over 64-bit keys (ordered score << 32 | ~index), in
// LDS when the boundary holds at most 4096 entries, else over global memory.
// Then the K indices are put in ascending order through an LDS bitmap (S_t,
// stored as the cache entry's support), the values are aggregated (Eq. 12)
// and (q_bar_t, S_t) is pushed. One work group per head.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t comp_key(float s, int idx) {
  return (static_cast<uint64_t>(order_key(s)) << 32) |
         static_cast<uint64_t>(0xffffffffu - static_cast<uint32_t>(idx));
}

__global__ __launch_bounds__(kHeadThreads) void k_finish(Dims d, Bufs b, const uint16_t* v, float* out,
                                                         int32_t* sel_out, int length, int push) {
  const int bh = blockIdx.x;
  if (!b.path[bh]) return;
  const int bb = bh / d.Hq, h = bh % d.Hq, g = h / d.G;
  const int tid = threadIdx.x;
  __shared__ HeadShared sh;
  extern __shared__ __align__(16) unsigned char dyn[];
  const size_t region0 = (kBoundaryLds * 8 > kBitmapWords * 4) ? kBoundaryLds * 8 : kBitmapWords * 4;
  uint64_t* keys = reinterpret_cast<uint64_t*>(dyn);
  uint32_t* bm = reinterpret_cast<uint32_t*>(dyn);
  int32_t* s_sel = reinterpret_cast<int32_t*>(dyn + region0);
  float* s_selsc = reinterpret_cast<float*>(dyn + region0 + 4 * static_cast<size_t>(d.K));
  const int keff = min(d.K, length);
  const int n_above = min(b.cnt[bh * 4 + 0], keff);
  const int nb = min(b.cnt[bh * 4 + 1], length);
  const float* srow = b.score + static_cast<long>(bh) * d.score_stride;
  int32_t* above = b.above + static_cast<long>(bh) * d.K;
  const int32_t* bnd = b.bnd + static_cast<long>(bh) * d.max_len;
  const bool in_lds = nb <= kBoundaryLds;
  if (in_lds) {
    for (int i0 = 0; i0 < nb; i0 += blockDim.x * 4) {
      int ix[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * blockDim.x + tid;
        ix[u] = i < nb ? bnd[i] : 0;
      }
      float sv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) sv[u] = (i0 + u * blockDim.x + tid < nb) ? srow[ix[u]] : 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * blockDim.x + tid;
        if (i < nb) keys[i] = comp_key(sv[u], ix[u]);
      }
    }
  }
  if (tid == 0) sh.i3 = 0;
  __syncthreads();
  uint64_t prefix = 0ull, mask = 0ull;
  int need = keff - n_above;
  int ncand = nb;
  for (int shift = 56; shift >= 0 && ncand > need; shift -= 8) {
    if (tid < 256) sh.hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < nb; i += blockDim.x) {
      const uint64_t u = in_lds ? keys[i] : comp_key(srow[bnd[i]], bnd[i]);
      if ((u & mask) == prefix) atomicAdd(&sh.hist[(u >> shift) & 255ull], 1);
    }
    __syncthreads();
    const int digit = 255 - static_cast<int>(tid & 255);
    const int c = (tid < 256) ? sh.hist[digit] : 0;
    int tot;
    const int above_cnt = block_exclusive_scan(c, &tot, sh.tmp);
    if (tid < 256 && above_cnt < need && above_cnt + c >= need) {
      sh.i0 = digit;
      sh.i1 = need - above_cnt;
      sh.i2 = c;
    }
    __syncthreads();
    prefix |= static_cast<uint64_t>(sh.i0) << shift;
    mask |= 255ull << shift;
    need = sh.i1;
    ncand = sh.i2;
    __syncthreads();
  }
  // boundary entries whose masked key is >= prefix are exactly the kept ones
  for (int i = tid; i < nb; i += blockDim.x) {
    const int ix = bnd[i];
    const uint64_t u = in_lds ? keys[i] : comp_key(srow[ix], ix);
    if ((u & mask) >= prefix) {
      const int o = atomicAdd(&sh.i3, 1);
      if (n_above + o < d.K) above[n_above + o] = ix;
    }
  }
  __syncthreads();
  // ascending order through the bitmap
  int total = 0;
  for (int base = 0; base < length; base += kBitmapWords * 32) {
    const int nbits = min(kBitmapWords * 32, length - base);
    const int nwords = (nbits + 31) >> 5;
    for (int i = tid; i < nwords; i += blockDim.x) bm[i] = 0u;
    __syncthreads();
    for (int i = tid; i < keff; i += blockDim.x) {
      const int x = above[i] - base;
      if (x >= 0 && x < nbits) atomicOr(&bm[x >> 5], 1u << (x & 31));
    }
    __syncthreads();
    total += bitmap_emit(bm, nwords, base, s_sel + total, sh.tmp);
    __syncthreads();
  }
  const int n = min(total, keff);
  float mx = kNegInf;
  for (int i = tid; i < n; i += blockDim.x) {
    const float s = srow[s_sel[i]];
    s_selsc[i] = s;
    mx = fmaxf(mx, s);
  }
  mx = block_max_f32(mx, reinterpret_cast<float*>(sh.tmp));
  for (int i = tid; i < n; i += blockDim.x) {
    b.sel[static_cast<long>(bh) * d.K + i] = s_sel[i];
    b.selsc[static_cast<long>(bh) * d.K + i] = s_selsc[i];
  }
  if (tid == 0) b.sellen[bh] = n;
  if (sel_out != nullptr)
    for (int i = tid; i < d.K; i += blockDim.x) sel_out[static_cast<long>(bh) * d.K + i] = i < n ? s_sel[i] : -1;
  if (v != nullptr && out != nullptr) {
    const uint16_t* vb = v + static_cast<long>(bb * d.Hkv + g) * d.max_len * kHeadDim;
    attend(s_sel, s_selsc, n, mx, vb, out + static_cast<long>(bh) * kHeadDim, sh);
  }
  if (push) {
    for (int t = tid; t < kHeadDim; t += blockDim.x) sh.qbar[t] = b.qbar[static_cast<long>(bh) * kHeadDim + t];
    __syncthreads();
    cache_push(d, b, bh, sh.qbar, s_sel, n);
  }
}

// ---------------------------------------------------------------------------
// Launch helpers
// ---------------------------------------------------------------------------
hipError_t configure_kernels(const Dims& d) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_head),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(head_lds_bytes(d)));
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_finish), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(finish_lds_bytes(d)));
  return e;
}

const char* kernel_name(int id) {
  static const char* names[kNumKernels] = {"k_head", "k_exact_qk", "k_collect", "k_finish", "k_reset"};
  return (id >= 0 && id < kNumKernels) ? names[id] : "";
}

hipError_t launch_reset(const Dims& d, const Bufs& b, hipStream_t s) {
  const int bh = d.B * d.Hq;
  hipLaunchKernelGGL(k_reset, dim3((bh + 255) / 256), dim3(256), 0, s, d, b);
  return hipGetLastError();
}

hipError_t launch_head(const Dims& d, const Bufs& b, const uint16_t* q, long q_sb, long q_sh,
                       const uint16_t* k, const uint16_t* v, float* out, int length, int t_dec, int mode,
                       int stats_slot, hipStream_t s) {
  hipLaunchKernelGGL(k_head, dim3(d.B * d.Hq), dim3(kHeadThreads), head_lds_bytes(d), s, d, b, q, q_sb, q_sh,
                     k, v, out, length, t_dec, mode, stats_slot);
  return hipGetLastError();
}

hipError_t launch_exact_qk(const Dims& d, const Bufs& b, const uint16_t* q, long q_sb, long q_sh,
                           const uint16_t* k, int length, hipStream_t s) {
  const int groups = d.B * d.Hkv;
  int wpg = (kExactWGTarget + groups - 1) / groups;
  wpg = std::max(1, std::min(wpg, (length + kExactMinRows - 1) / kExactMinRows));
  hipLaunchKernelGGL(k_exact_qk, dim3(groups * wpg), dim3(256), d.G * kNumBins * sizeof(uint32_t), s, d, b,
                     q, q_sb, q_sh, k, length, wpg);
  return hipGetLastError();
}

hipError_t launch_collect(const Dims& d, const Bufs& b, int length, hipStream_t s) {
  const int ny = (length + kCollectChunk - 1) / kCollectChunk;
  hipLaunchKernelGGL(k_collect, dim3(d.B * d.Hq, ny), dim3(256), 0, s, d, b, length);
  return hipGetLastError();
}

hipError_t launch_finish(const Dims& d, const Bufs& b, const uint16_t* v, float* out, int32_t* sel_out,
                         int length, int push, hipStream_t s) {
  hipLaunchKernelGGL(k_finish, dim3(d.B * d.Hq), dim3(kHeadThreads), finish_lds_bytes(d), s, d, b, v, out,
                     sel_out, length, push);
  return hipGetLastError();
}

}  // namespace retopk

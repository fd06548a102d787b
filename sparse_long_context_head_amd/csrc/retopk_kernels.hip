// ReTopK decode-step kernels for CDNA4 (gfx950, wave64).
//
// Method: "Recall Before You Rank: Similarity-Guided Top-K Reuse for
// Efficient Long-Context Attention", Methodology section. One decode step runs
//   recall      (Eqs. 5-7 and the path rule of Eq. 13)   k_recall
//   reuse path: candidate union (Eqs. 8-9)                k_union
//               candidate scores (Eq. 10)                 k_cand_qk
//               rerank to K (Eq. 11)                      k_rerank
//   exact path: full-history scores (Eq. 4) + histogram   k_exact_qk  (MFMA)
//               global Top-K (Eq. 1), threshold + collect k_collect
//               boundary resolution + ascending order     k_finish
//   both:       sparse softmax-V (Eq. 12) + cache update  k_attend
// Every kernel reads the per-head path flag written by k_recall and returns
// at once for heads (or KV groups) that take the other path, so the host
// never waits for the decision.

#include "retopk_internal.h"

#include <cmath>

namespace retopk {

namespace {

constexpr float kNegInf = -INFINITY;

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

__device__ __forceinline__ double wave_max_f64(double x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmax(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_max_f32(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// Number of lanes below this one whose bit is set in `mask`.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
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

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

}  // namespace

// ---------------------------------------------------------------------------
// Reset the FIFO bookkeeping (before cache initialisation) and the arrival
// counters. One thread per head.
// ---------------------------------------------------------------------------
__global__ void k_reset(Dims d, Bufs b) {
  const int bh = blockIdx.x * blockDim.x + threadIdx.x;
  if (bh >= d.B * d.Hq) return;
  b.fifo[2 * bh] = 0;
  b.fifo[2 * bh + 1] = 0;
  b.done[bh] = 0;
}

// ---------------------------------------------------------------------------
// Recall (Eqs. 5-7) and path decision (Eq. 13).
// One work group per (batch, KV group); one wave per query head of the group.
//   q_bar = fp32(x / ||x||), fp64 sum of squares, sqrt and divide
//   rho_c = fp64 dot of the fp32 q_bar values, c over the held entries
//   R_t   = the R entries of largest rho (ties: older entry), rho_max
//   exact = refresh or empty cache or rho_max < tau
// Also clears the per-head counters and (for exact heads) the histogram that
// the exact-path kernels accumulate into.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kMaxGroup * kWave) void k_recall(Dims d, Bufs b, const uint16_t* q,
                                                              long q_sb, long q_sh, int mode,
                                                              int t_dec, int stats_slot) {
  const int bb = blockIdx.x / d.Hkv, g = blockIdx.x % d.Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = g * d.G + wave;
  const int bh = bb * d.Hq + h;
  __shared__ float s_qbar[kMaxGroup][kHeadDim];
  __shared__ double s_rho[kMaxGroup][kWave];
  __shared__ int s_exact[kMaxGroup];

  const uint32_t w2 = *reinterpret_cast<const uint32_t*>(q + bb * q_sb + h * q_sh + 2 * lane);
  const double x0 = bf16_lo(w2), x1 = bf16_hi(w2);
  const double ss = wave_sum_f64(x0 * x0 + x1 * x1);
  const double nrm = sqrt(ss);
  float qb0 = 0.f, qb1 = 0.f;
  if (nrm > 0.0) {
    qb0 = static_cast<float>(x0 / nrm);
    qb1 = static_cast<float>(x1 / nrm);
  }
  s_qbar[wave][2 * lane] = qb0;
  s_qbar[wave][2 * lane + 1] = qb1;
  *reinterpret_cast<float2*>(b.qbar + static_cast<long>(bh) * kHeadDim + 2 * lane) =
      make_float2(qb0, qb1);

  const int count = b.fifo[2 * bh + 1];
  const int oldest = (b.fifo[2 * bh] - count + d.C) % d.C;
  bool exact = true, refresh = false;
  double rho_max = -INFINITY;
  __syncthreads();
  if (mode == kModeDecode) {
    refresh = d.Tr > 0 && (t_dec % d.Tr) == 0;
    // lane c computes rho for the entry at FIFO position c (0 = oldest)
    double part = 0.0;
    if (lane < count) {
      const float* e = b.cache_qbar + (static_cast<long>(bh) * d.C + (oldest + lane) % d.C) * kHeadDim;
      const float* t = s_qbar[wave];
#pragma unroll 4
      for (int j = 0; j < kHeadDim; j += 4) {
        const float4 ev = *reinterpret_cast<const float4*>(e + j);
        part = fma(static_cast<double>(t[j]), static_cast<double>(ev.x), part);
        part = fma(static_cast<double>(t[j + 1]), static_cast<double>(ev.y), part);
        part = fma(static_cast<double>(t[j + 2]), static_cast<double>(ev.z), part);
        part = fma(static_cast<double>(t[j + 3]), static_cast<double>(ev.w), part);
      }
    }
    const double mine = (lane < count) ? part : -INFINITY;
    s_rho[wave][lane] = mine;
    __syncthreads();
    rho_max = wave_max_f64(mine);
    if (lane < count) {
      int rank = 0;
      for (int j = 0; j < count; ++j) {
        const double o = s_rho[wave][j];
        rank += (o > mine) || (o == mine && j < lane);
      }
      if (rank < d.R) {
        b.ret[bh * d.R + rank] = lane;
        b.retslot[bh * d.R + rank] = (oldest + lane) % d.C;
      }
    }
    exact = refresh || count == 0 || rho_max < d.tau;
  } else {
    __syncthreads();
  }
  const int n_ret = (mode == kModeDecode) ? min(d.R, count) : 0;
  if (lane >= n_ret && lane < d.R) {
    b.ret[bh * d.R + lane] = -1;
    b.retslot[bh * d.R + lane] = -1;
  }
  if (lane == 0) {
    b.path[bh] = exact ? 1 : 0;
    b.rho[bh] = rho_max;
    if (exact) b.m[bh] = 0;
    if (stats_slot >= 0) {
      const long o = static_cast<long>(stats_slot) * d.B * d.Hq + bh;
      b.st_path[o] = static_cast<uint8_t>((exact ? 1 : 0) | (refresh ? 2 : 0));
      b.st_rho[o] = rho_max;
      if (exact) b.st_m[o] = 0;
    }
  }
  if (lane < 4) b.cnt[bh * 4 + lane] = 0;
  if (exact) {
    for (int i = lane; i < kNumBins; i += kWave) b.hist[static_cast<long>(bh) * kNumBins + i] = 0u;
  }
  if (lane == 0) s_exact[wave] = exact ? 1 : 0;
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    for (int w = 0; w < d.G; ++w) n += s_exact[w];
    b.gexact[bb * d.Hkv + g] = n;
  }
}

// ---------------------------------------------------------------------------
// Candidate union (Eqs. 8-9) for reuse heads: the retrieved supports and the
// window [max(0, L-W), L) are set in an LDS bitmap over token positions
// (processed in windows of 262144 positions), which is then read back in
// ascending order. Duplicates vanish in the bitmap. One work group per head.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_union(Dims d, Bufs b, int length, int stats_slot) {
  const int bh = blockIdx.x;
  if (b.path[bh]) return;
  extern __shared__ uint32_t bm[];
  __shared__ int tmp[8];
  const int wlo = max(0, length - d.W);
  int32_t* out = b.cand + static_cast<long>(bh) * d.cand_cap;
  int total = 0;
  for (int base = 0; base < length; base += kBitmapWords * 32) {
    const int nbits = min(kBitmapWords * 32, length - base);
    const int nwords = (nbits + 31) >> 5;
    for (int i = threadIdx.x; i < nwords; i += blockDim.x) bm[i] = 0u;
    __syncthreads();
    for (int r = 0; r < d.R; ++r) {
      const int slot = b.retslot[bh * d.R + r];
      if (slot < 0) break;
      const long e = static_cast<long>(bh) * d.C + slot;
      const int len = b.cache_len[e];
      const int32_t* s = b.cache_supp + e * d.K;
      for (int i = threadIdx.x; i < len; i += blockDim.x) {
        const int x = s[i] - base;
        if (x >= 0 && x < nbits) atomicOr(&bm[x >> 5], 1u << (x & 31));
      }
    }
    for (int x = max(wlo, base) + threadIdx.x; x < base + nbits; x += blockDim.x) {
      const int y = x - base;
      atomicOr(&bm[y >> 5], 1u << (y & 31));
    }
    __syncthreads();
    total += bitmap_emit(bm, nwords, base, out + total, tmp);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    b.m[bh] = total;
    if (stats_slot >= 0) b.st_m[static_cast<long>(stats_slot) * d.B * d.Hq + bh] = total;
  }
}

// ---------------------------------------------------------------------------
// Candidate scores (Eq. 10, unscaled): s_i = q . k_i for i in A_t, read
// straight from the KV cache through the index list (no gathered key
// tensor). 16 lanes per key row (16 bytes each), 4 rows per wave step,
// 128 rows per work group; fp32 accumulation of exact bf16 products.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_cand_qk(Dims d, Bufs b, const uint16_t* q,
                                                 const uint16_t* k) {
  const int bh = blockIdx.x;
  if (b.path[bh]) return;
  const int M = b.m[bh];
  const int r0 = blockIdx.y * kCandRowsPerBlock;
  if (r0 >= M) return;
  const int bb = bh / d.Hq, h = bh % d.Hq, g = h / d.G;
  const uint16_t* kb = k + static_cast<long>(bb * d.Hkv + g) * d.max_len * kHeadDim;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & 15, rg = lane >> 4;
  const uint4 qv = *reinterpret_cast<const uint4*>(q + static_cast<long>(bh) * kHeadDim + 8 * sub);
  float qf[8] = {bf16_lo(qv.x), bf16_hi(qv.x), bf16_lo(qv.y), bf16_hi(qv.y),
                 bf16_lo(qv.z), bf16_hi(qv.z), bf16_lo(qv.w), bf16_hi(qv.w)};
  const int32_t* cand = b.cand + static_cast<long>(bh) * d.cand_cap;
  float* cs = b.cscore + static_cast<long>(bh) * d.cand_cap;
  const int rend = min(M, r0 + kCandRowsPerBlock);
  constexpr int kPer = kCandRowsPerBlock / 16;  // rows per lane group
  uint4 kv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int r = r0 + wave * (kPer * 4) + i * 4 + rg;
    if (r < rend) {
      const int idx = cand[r];
      kv[i] = *reinterpret_cast<const uint4*>(kb + static_cast<long>(idx) * kHeadDim + 8 * sub);
    } else {
      kv[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int r = r0 + wave * (kPer * 4) + i * 4 + rg;
    float s = qf[0] * bf16_lo(kv[i].x);
    s = fmaf(qf[1], bf16_hi(kv[i].x), s);
    s = fmaf(qf[2], bf16_lo(kv[i].y), s);
    s = fmaf(qf[3], bf16_hi(kv[i].y), s);
    s = fmaf(qf[4], bf16_lo(kv[i].z), s);
    s = fmaf(qf[5], bf16_hi(kv[i].z), s);
    s = fmaf(qf[6], bf16_lo(kv[i].w), s);
    s = fmaf(qf[7], bf16_hi(kv[i].w), s);
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    s += __shfl_xor(s, 8);
    if (sub == 0 && r < rend) cs[r] = s;
  }
}

// ---------------------------------------------------------------------------
// Rerank (Eq. 11): the K largest candidate scores, ties to the lower index.
// Radix select over the order-preserving score keys in LDS (4 passes of 8
// bits) finds the K-th largest key T; every key > T is kept, and of the keys
// equal to T the first ones in (ascending) candidate order. The kept
// candidates are written in candidate order, hence ascending.
// One work group per reuse head.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_rerank(Dims d, Bufs b) {
  const int bh = blockIdx.x;
  if (b.path[bh]) return;
  extern __shared__ uint32_t skey[];
  __shared__ int hist[256];
  __shared__ int tmp[8];
  __shared__ int s_digit, s_need;
  const int M = b.m[bh], K = d.K;
  const float* sc = b.cscore + static_cast<long>(bh) * d.cand_cap;
  const int32_t* cd = b.cand + static_cast<long>(bh) * d.cand_cap;
  int32_t* sel = b.sel + static_cast<long>(bh) * K;
  float* selsc = b.selsc + static_cast<long>(bh) * K;
  if (M <= K) {
    for (int i = threadIdx.x; i < M; i += blockDim.x) {
      sel[i] = cd[i];
      selsc[i] = sc[i];
    }
    if (threadIdx.x == 0) b.sellen[bh] = M;
    return;
  }
  for (int i = threadIdx.x; i < M; i += blockDim.x) skey[i] = order_key(sc[i]);
  __syncthreads();
  uint32_t prefix = 0u, mask = 0u;
  int need = K;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[threadIdx.x] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < M; i += blockDim.x) {
      const uint32_t u = skey[i];
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1);
    }
    __syncthreads();
    const int digit = 255 - static_cast<int>(threadIdx.x);
    const int c = hist[digit];
    int tot;
    const int above = block_exclusive_scan(c, &tot, tmp);
    if (above < need && above + c >= need) {
      s_digit = digit;
      s_need = need - above;
    }
    __syncthreads();
    prefix |= static_cast<uint32_t>(s_digit) << shift;
    mask |= 255u << shift;
    need = s_need;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const int per = (M + blockDim.x - 1) / blockDim.x;
  const int i0 = threadIdx.x * per, i1 = min(i0 + per, M);
  int eq = 0;
  for (int i = i0; i < i1; ++i) eq += (skey[i] == T);
  int tot;
  const int eq_before = block_exclusive_scan(eq, &tot, tmp);
  int nsel = 0;
  int e = eq_before;
  for (int i = i0; i < i1; ++i) {
    const uint32_t u = skey[i];
    nsel += (u > T) || (u == T && e < need);
    e += (u == T);
  }
  int o = block_exclusive_scan(nsel, &tot, tmp);
  e = eq_before;
  for (int i = i0; i < i1; ++i) {
    const uint32_t u = skey[i];
    if ((u > T) || (u == T && e < need)) {
      sel[o] = cd[i];
      selsc[o] = sc[i];
      ++o;
    }
    e += (u == T);
  }
  if (threadIdx.x == 0) b.sellen[bh] = K;
}

// ---------------------------------------------------------------------------
// Full-history scores (Eq. 4, unscaled) for every exact head, GQA-grouped:
// each work item streams 1024 rows of one KV head exactly once and scores
// them for all query heads of the group with MFMA 16x16x32 bf16 tiles
// (A = 16 key rows x 32 dims, B = 32 dims x 16 query heads, fp32 accumulate).
// The scores go to the workspace and into a per-head histogram of the top 10
// bits of their ordered keys (LDS, flushed with global atomics), which the
// threshold kernel uses to find the Top-K boundary without a sort.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_exact_qk(Dims d, Bufs b, const uint16_t* q, long q_sb,
                                                  long q_sh, const uint16_t* k, int length,
                                                  int nchunk) {
  const int chunk = blockIdx.x % nchunk;
  const int bg = blockIdx.x / nchunk;
  if (b.gexact[bg] == 0) return;
  const int bb = bg / d.Hkv, g = bg % d.Hkv;
  extern __shared__ uint32_t s_hist[];  // [G, kNumBins]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, kq = lane >> 4;
  const int h = g * d.G + j;
  const bool hv = (j < d.G) && b.path[bb * d.Hq + h];
  bf16x8 bq[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (hv) u = *reinterpret_cast<const uint4*>(q + bb * q_sb + h * q_sh + 8 * kq + 32 * s);
    bq[s] = as_bf16x8(u);
  }
  for (int i = threadIdx.x; i < d.G * kNumBins; i += blockDim.x) s_hist[i] = 0u;
  __syncthreads();
  const int row0 = chunk * kExactChunk;
  const int rend = min(row0 + kExactChunk, length);
  const uint16_t* kb = k + static_cast<long>(bb * d.Hkv + g) * d.max_len * kHeadDim;
  float* srow = b.score + static_cast<long>(bb * d.Hq + h) * d.score_stride;
  uint32_t* hrow = s_hist + j * kNumBins;
  constexpr int kTiles = kExactChunk / 16;  // 16-row tiles per chunk
  constexpr int kUnroll = 4;
  for (int t0 = 0; t0 < kTiles; t0 += 4 * kUnroll) {
    uint4 a[kUnroll][4];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int rbase = row0 + (t0 + u * 4 + wave) * 16;
      const int r = rbase + j;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (r < rend)
          a[u][s] = *reinterpret_cast<const uint4*>(kb + static_cast<long>(r) * kHeadDim + 8 * kq + 32 * s);
        else
          a[u][s] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int rbase = row0 + (t0 + u * 4 + wave) * 16;
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
          for (int v = 0; v < 4; ++v) atomicAdd(&hrow[order_key(acc[v]) >> kHistShift], 1u);
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            if (r + v < rend) {
              srow[r + v] = acc[v];
              atomicAdd(&hrow[order_key(acc[v]) >> kHistShift], 1u);
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
// Global Top-K (Eq. 1), step 1 of 2, for exact heads. From the histogram,
// find the boundary bin: the bin holding the K-th largest score. Then scan a
// chunk of scores and append (wave-aggregated atomics) the indices of scores
// in higher bins to the "above" list (fewer than K in total) and those in the
// boundary bin to the boundary list.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_collect(Dims d, Bufs b, int length) {
  const int bh = blockIdx.x;
  if (!b.path[bh]) return;
  const int c0 = blockIdx.y * kCollectChunk;
  if (c0 >= length) return;
  __shared__ int tmp[8];
  __shared__ int s_b1;
  const int keff = min(d.K, length);
  const uint32_t* hist = b.hist + static_cast<long>(bh) * kNumBins;
  constexpr int kPer = kNumBins / 256;
  int c[kPer];
  int csum = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    c[i] = static_cast<int>(hist[kNumBins - 1 - (kPer * threadIdx.x + i)]);
    csum += c[i];
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
  const float* srow = b.score + static_cast<long>(bh) * d.score_stride;
  int32_t* above = b.above + static_cast<long>(bh) * d.K;
  int32_t* bnd = b.bnd + static_cast<long>(bh) * d.max_len;
  const int lane = threadIdx.x & 63;
  const int cend = min(c0 + kCollectChunk, length);
  for (int base = c0; base < cend; base += blockDim.x) {
    const int i = base + threadIdx.x;
    bool up = false, bd = false;
    if (i < cend) {
      const uint32_t bin = order_key(srow[i]) >> kHistShift;
      up = bin > b1;
      bd = bin == b1;
    }
    const uint64_t mu = __ballot(up), mb = __ballot(bd);
    int ou = 0, ob = 0;
    if (lane == 0) {
      if (mu) ou = atomicAdd(&b.cnt[bh * 4 + 0], __popcll(mu));
      if (mb) ob = atomicAdd(&b.cnt[bh * 4 + 1], __popcll(mb));
    }
    ou = __shfl(ou, 0);
    ob = __shfl(ob, 0);
    // (fewer than K scores lie above the boundary bin; the guards only keep a
    // broken invariant from writing out of bounds)
    if (up && ou + lanes_below(mu) < d.K) above[ou + lanes_below(mu)] = i;
    if (bd && ob + lanes_below(mb) < d.max_len) bnd[ob + lanes_below(mb)] = i;
  }
}

// ---------------------------------------------------------------------------
// Global Top-K, step 2 of 2, for exact heads. Of the boundary-bin entries,
// keep the `need` best under the total order (score desc, index asc): a
// radix select over 64-bit keys (ordered score << 32 | ~index), in LDS when
// the boundary holds at most 4096 entries, else over global memory. The kept
// entries join the "above" list; then the K indices are put in ascending order
// through an LDS bitmap and written with their scores. One work group per head.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t comp_key(const float* srow, int idx) {
  return (static_cast<uint64_t>(order_key(srow[idx])) << 32) |
         static_cast<uint64_t>(0xffffffffu - static_cast<uint32_t>(idx));
}

__global__ __launch_bounds__(512) void k_finish(Dims d, Bufs b, int length) {
  const int bh = blockIdx.x;
  if (!b.path[bh]) return;
  extern __shared__ uint64_t lds[];  // boundary keys, later reused as the bitmap
  __shared__ int hist[256];
  __shared__ int tmp[16];
  __shared__ int s_digit, s_need, s_ncand, s_napp;
  const int keff = min(d.K, length);
  const int n_above = min(b.cnt[bh * 4 + 0], keff);
  const int nb = min(b.cnt[bh * 4 + 1], length);
  const float* srow = b.score + static_cast<long>(bh) * d.score_stride;
  int32_t* above = b.above + static_cast<long>(bh) * d.K;
  const int32_t* bnd = b.bnd + static_cast<long>(bh) * d.max_len;
  const bool in_lds = nb <= kBoundaryLds;
  if (in_lds)
    for (int i = threadIdx.x; i < nb; i += blockDim.x) lds[i] = comp_key(srow, bnd[i]);
  if (threadIdx.x == 0) s_napp = 0;
  __syncthreads();
  uint64_t prefix = 0ull, mask = 0ull;
  int need = keff - n_above;
  int ncand = nb;
  for (int shift = 56; shift >= 0 && ncand > need; shift -= 8) {
    if (threadIdx.x < 256) hist[threadIdx.x] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < nb; i += blockDim.x) {
      const uint64_t u = in_lds ? lds[i] : comp_key(srow, bnd[i]);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255ull], 1);
    }
    __syncthreads();
    const int digit = 255 - static_cast<int>(threadIdx.x & 255);
    const int c = (threadIdx.x < 256) ? hist[digit] : 0;
    int tot;
    const int above_cnt = block_exclusive_scan(c, &tot, tmp);
    if (threadIdx.x < 256 && above_cnt < need && above_cnt + c >= need) {
      s_digit = digit;
      s_need = need - above_cnt;
      s_ncand = c;
    }
    __syncthreads();
    prefix |= static_cast<uint64_t>(s_digit) << shift;
    mask |= 255ull << shift;
    need = s_need;
    ncand = s_ncand;
    __syncthreads();
  }
  // boundary entries whose masked key is >= prefix are exactly the kept ones
  for (int i = threadIdx.x; i < nb; i += blockDim.x) {
    const uint64_t u = in_lds ? lds[i] : comp_key(srow, bnd[i]);
    if ((u & mask) >= prefix) {
      const int o = atomicAdd(&s_napp, 1);
      if (n_above + o < d.K) above[n_above + o] = bnd[i];
    }
  }
  __syncthreads();
  // ascending order through the bitmap; scores looked up again
  uint32_t* bm = reinterpret_cast<uint32_t*>(lds);
  int32_t* sel = b.sel + static_cast<long>(bh) * d.K;
  float* selsc = b.selsc + static_cast<long>(bh) * d.K;
  int total = 0;
  for (int base = 0; base < length; base += kBitmapWords * 32) {
    const int nbits = min(kBitmapWords * 32, length - base);
    const int nwords = (nbits + 31) >> 5;
    for (int i = threadIdx.x; i < nwords; i += blockDim.x) bm[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < keff; i += blockDim.x) {
      const int x = above[i] - base;
      if (x >= 0 && x < nbits) atomicOr(&bm[x >> 5], 1u << (x & 31));
    }
    __syncthreads();
    total += bitmap_emit(bm, nwords, base, sel + total, tmp);
    __syncthreads();
  }
  for (int i = threadIdx.x; i < keff; i += blockDim.x) selsc[i] = srow[sel[i]];
  if (threadIdx.x == 0) b.sellen[bh] = keff;
}

// ---------------------------------------------------------------------------
// Sparse softmax-V (Eq. 12) over S_hat_t, and the cache update. The support
// is split over kAttendSplit work groups per head; all of them use the same
// maximum score, so their partial sums add directly. The last work group to
// arrive adds the partials in fixed order, writes the output, and pushes
// (q_bar_t, S_hat_t) into the head's FIFO (after either path).
// 16 lanes per value row (16 bytes each), 4 rows per wave step.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_attend(Dims d, Bufs b, const uint16_t* v, float* out,
                                                int32_t* sel_out, int push) {
  const int bh = blockIdx.x, part = blockIdx.y;
  const int n = b.sellen[bh];
  const int bb = bh / d.Hq, h = bh % d.Hq, g = h / d.G;
  const float* sc = b.selsc + static_cast<long>(bh) * d.K;
  const int32_t* sel = b.sel + static_cast<long>(bh) * d.K;
  __shared__ float red[4][kHeadDim + 4];
  __shared__ float tmpf[8];
  __shared__ int s_last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & 15, rg = lane >> 4;
  float* pp = b.part + (static_cast<long>(bh) * kAttendSplit + part) * (kHeadDim + 4);
  if (out != nullptr) {
    float mx = kNegInf;
    for (int i = threadIdx.x; i < n; i += blockDim.x) mx = fmaxf(mx, sc[i]);
    mx = block_max_f32(mx, tmpf);
    const float inv_sqrt_d = 0.08838834764831845f;  // 1 / sqrt(128)
    const int per = (n + kAttendSplit - 1) / kAttendSplit;
    const int i0 = part * per, i1 = min(n, i0 + per);
    const uint16_t* vb = v + static_cast<long>(bb * d.Hkv + g) * d.max_len * kHeadDim;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float z = 0.f;
    for (int i = i0 + wave * 4 + rg; i < i1; i += 16) {
      const float p = expf((sc[i] - mx) * inv_sqrt_d);
      const uint4 w = *reinterpret_cast<const uint4*>(vb + static_cast<long>(sel[i]) * kHeadDim + 8 * sub);
      acc[0] = fmaf(p, bf16_lo(w.x), acc[0]);
      acc[1] = fmaf(p, bf16_hi(w.x), acc[1]);
      acc[2] = fmaf(p, bf16_lo(w.y), acc[2]);
      acc[3] = fmaf(p, bf16_hi(w.y), acc[3]);
      acc[4] = fmaf(p, bf16_lo(w.z), acc[4]);
      acc[5] = fmaf(p, bf16_hi(w.z), acc[5]);
      acc[6] = fmaf(p, bf16_lo(w.w), acc[6]);
      acc[7] = fmaf(p, bf16_hi(w.w), acc[7]);
      z += p;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[e] += __shfl_xor(acc[e], 16);
      acc[e] += __shfl_xor(acc[e], 32);
    }
    z += __shfl_xor(z, 16);
    z += __shfl_xor(z, 32);
    if (rg == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave][8 * sub + e] = acc[e];
      if (sub == 0) red[wave][kHeadDim] = z;
    }
    __syncthreads();
    if (threadIdx.x <= kHeadDim) {
      const int t = threadIdx.x;
      pp[t] = red[0][t] + red[1][t] + red[2][t] + red[3][t];
    }
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(&b.done[bh], 1) == kAttendSplit - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (out != nullptr && threadIdx.x < kHeadDim) {
    const float* p0 = b.part + static_cast<long>(bh) * kAttendSplit * (kHeadDim + 4);
    float a = 0.f, zz = 0.f;
    for (int s = 0; s < kAttendSplit; ++s) {
      a += p0[s * (kHeadDim + 4) + threadIdx.x];
      zz += p0[s * (kHeadDim + 4) + kHeadDim];
    }
    out[static_cast<long>(bh) * kHeadDim + threadIdx.x] = a / zz;
  }
  if (sel_out != nullptr)
    for (int i = threadIdx.x; i < d.K; i += blockDim.x)
      sel_out[static_cast<long>(bh) * d.K + i] = i < n ? sel[i] : -1;
  if (push) {
    const int slot = b.fifo[2 * bh];
    const long e = static_cast<long>(bh) * d.C + slot;
    for (int t = threadIdx.x; t < kHeadDim; t += blockDim.x)
      b.cache_qbar[e * kHeadDim + t] = b.qbar[static_cast<long>(bh) * kHeadDim + t];
    for (int i = threadIdx.x; i < n; i += blockDim.x) b.cache_supp[e * d.K + i] = sel[i];
    __syncthreads();
    if (threadIdx.x == 0) {
      b.cache_len[e] = n;
      b.fifo[2 * bh] = (slot + 1) % d.C;
      b.fifo[2 * bh + 1] = min(b.fifo[2 * bh + 1] + 1, d.C);
    }
  }
  if (threadIdx.x == 0) b.done[bh] = 0;
}

// ---------------------------------------------------------------------------
// Launch helpers
// ---------------------------------------------------------------------------
const char* kernel_name(int id) {
  static const char* names[kNumKernels] = {"k_recall", "k_union",  "k_cand_qk", "k_rerank", "k_exact_qk",
                                           "k_collect", "k_finish", "k_attend", "k_reset"};
  return (id >= 0 && id < kNumKernels) ? names[id] : "";
}

hipError_t launch_reset(const Dims& d, const Bufs& b, hipStream_t s) {
  const int bh = d.B * d.Hq;
  hipLaunchKernelGGL(k_reset, dim3((bh + 255) / 256), dim3(256), 0, s, d, b);
  return hipGetLastError();
}

hipError_t launch_recall(const Dims& d, const Bufs& b, const uint16_t* q, long q_sb, long q_sh,
                         int mode, int t_dec, int stats_slot, hipStream_t s) {
  hipLaunchKernelGGL(k_recall, dim3(d.B * d.Hkv), dim3(d.G * kWave), 0, s, d, b, q, q_sb, q_sh, mode,
                     t_dec, stats_slot);
  return hipGetLastError();
}

hipError_t launch_union(const Dims& d, const Bufs& b, int length, int stats_slot, hipStream_t s) {
  hipLaunchKernelGGL(k_union, dim3(d.B * d.Hq), dim3(256), kBitmapWords * sizeof(uint32_t), s, d, b,
                     length, stats_slot);
  return hipGetLastError();
}

hipError_t launch_cand_qk(const Dims& d, const Bufs& b, const uint16_t* q, const uint16_t* k,
                          hipStream_t s) {
  const int ny = (d.cand_cap + kCandRowsPerBlock - 1) / kCandRowsPerBlock;
  hipLaunchKernelGGL(k_cand_qk, dim3(d.B * d.Hq, ny), dim3(256), 0, s, d, b, q, k);
  return hipGetLastError();
}

hipError_t launch_rerank(const Dims& d, const Bufs& b, hipStream_t s) {
  hipLaunchKernelGGL(k_rerank, dim3(d.B * d.Hq), dim3(256), d.cand_cap * sizeof(uint32_t), s, d, b);
  return hipGetLastError();
}

hipError_t launch_exact_qk(const Dims& d, const Bufs& b, const uint16_t* q, long q_sb, long q_sh,
                           const uint16_t* k, int length, hipStream_t s) {
  const int nchunk = (length + kExactChunk - 1) / kExactChunk;
  hipLaunchKernelGGL(k_exact_qk, dim3(d.B * d.Hkv * nchunk), dim3(256),
                     d.G * kNumBins * sizeof(uint32_t), s, d, b, q, q_sb, q_sh, k, length, nchunk);
  return hipGetLastError();
}

hipError_t launch_collect(const Dims& d, const Bufs& b, int length, hipStream_t s) {
  const int ny = (length + kCollectChunk - 1) / kCollectChunk;
  hipLaunchKernelGGL(k_collect, dim3(d.B * d.Hq, ny), dim3(256), 0, s, d, b, length);
  return hipGetLastError();
}

hipError_t launch_finish(const Dims& d, const Bufs& b, int length, hipStream_t s) {
  const size_t lds = kBoundaryLds * sizeof(uint64_t) > kBitmapWords * sizeof(uint32_t)
                         ? kBoundaryLds * sizeof(uint64_t)
                         : kBitmapWords * sizeof(uint32_t);
  hipLaunchKernelGGL(k_finish, dim3(d.B * d.Hq), dim3(512), lds, s, d, b, length);
  return hipGetLastError();
}

hipError_t launch_attend(const Dims& d, const Bufs& b, const uint16_t* v, float* out,
                         int32_t* sel_out, int push, hipStream_t s) {
  hipLaunchKernelGGL(k_attend, dim3(d.B * d.Hq, kAttendSplit), dim3(256), 0, s, d, b, v, out, sel_out,
                     push);
  return hipGetLastError();
}

}  // namespace retopk

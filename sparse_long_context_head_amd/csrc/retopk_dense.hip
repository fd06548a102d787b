// Dense softmax attention of one decode step over every cached key: the "Full
// Attention" column the ReTopK paper sets beside Exact Top-K (Experimental
// Results, Table 1; Kernel efficiency analysis, Figure 9). For each query head
// the scores are those of Eq. (4) for all i < L_t and the output is Eq. (12)'s
// softmax-value aggregation with the support taken as every position.
//
// Split over the key rows. k_dense gives each work group one (batch, KV group)
// pair and a contiguous slice of its rows, for all G query heads of the group
// at once, so that each key and value row is read from HBM once per group.
// The slice is streamed in stages of 128 rows; the key and value rows of the
// next two stages are in flight while the current one is processed (three
// register buffers in rotation):
//   - scores: MFMA 16x16x32 bf16 tiles (16 key rows x 32 dims times 32 dims x
//     16 query heads, fp32 accumulation), 16 rows per wave;
//   - a running maximum m and weight sum Z per head (online softmax): each
//     stage's maximum raises m, the earlier sums are scaled by exp(m_old - m);
//   - the weights exp((s - m) / sqrt(d)) go through LDS to the value side,
//     where 16 lanes per value row (8 dims each) accumulate all heads' weighted
//     sums in fp32 on the vector ALUs.
// A work group leaves, per query head of its group, (weighted value sum, m, Z)
// of its slice. k_dense_merge then combines the slices of each head with the
// merge of disjoint partial softmax results of the RetrievalAttention reading
// notes (Method, CPU-GPU two-path computation): common maximum m = max m_s,
// weights exp(m_s - m) Z_s, normalised sum.

#include "retopk_internal.h"

#include <mutex>

// Scratch of the entry point that allocates nothing (retopk_dense_attn_noalloc):
// the row slices' partial results, reserved in device memory on every GPU the
// library runs on, from load time until the process ends. Host code never
// passes this name to a kernel (on the host it does not denote the device
// address); it takes the address hipGetSymbolAddress returns per device.
static __device__ __align__(256) float scratch[retopk::kNoAllocScratchFloats];

namespace retopk {
namespace {

constexpr int kDThreads = 512;  // 8 waves
constexpr int kDWaves = kDThreads / kWave;
constexpr int kDStage = 128;    // rows per stage: 16 per wave for the scores, 4 per thread for the values
constexpr int kDVRows = kDStage / (kDThreads / 16);  // value rows per thread and stage
constexpr float kDInvSqrtD = 0.08838834764831845f;  // 1 / sqrt(128)

typedef __bf16 dbf16x8 __attribute__((ext_vector_type(8)));
typedef float df32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ dbf16x8 d_as_bf16x8(uint4 u) { return __builtin_bit_cast(dbf16x8, u); }
__device__ __forceinline__ float d_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float d_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// LDS-only barrier: waits for this wave's LDS accesses, not for its global
// loads, so that the next stage's row loads stay in flight across it.
__device__ __forceinline__ void d_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One stage's rows in registers.
struct DTiles {
  uint4 k[4];        // key row t0 + 16 wave + (lane & 15), dims 32 s + 8 (lane >> 4) .. + 8
  uint4 v[kDVRows];  // value row t0 + (tid >> 4) + 32 i, dims 8 (tid & 15) .. + 8
};

struct __align__(16) DShared {  // (16-byte rows of p are read as float4)
  float p[kDStage][kDenseMaxGroup];       // the stage's weights, [row][head]
  float wmax[kDWaves][16];                // per wave and head: the stage's maximum score
  float wz[kDWaves][16];                  // per wave and head: the stage's weight sum
  float alpha[kDenseMaxGroup];            // per head: exp((m_old - m_new) / sqrt(d))
  float red[kDWaves][kDenseMaxGroup][kHeadDim];  // the slice's value sums per wave
};

// Rows past rend are clamped to rend - 1 (a valid row; its weight is zero).
__device__ __forceinline__ void d_load(DTiles& t, const uint16_t* kb, const uint16_t* vb, int t0, int rend) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, kq = lane >> 4;
  const uint16_t* row = kb + static_cast<long>(min(t0 + 16 * wave + j, rend - 1)) * kHeadDim + 8 * kq;
#pragma unroll
  for (int s = 0; s < 4; ++s) t.k[s] = *reinterpret_cast<const uint4*>(row + 32 * s);
  const int sub = threadIdx.x & 15, rg = threadIdx.x >> 4;
#pragma unroll
  for (int i = 0; i < kDVRows; ++i) {
    const int r = min(t0 + rg + 32 * i, rend - 1);
    t.v[i] = *reinterpret_cast<const uint4*>(vb + static_cast<long>(r) * kHeadDim + 8 * sub);
  }
}

// One stage. m, z: the running maximum and weight sum of head (lane & 15),
// the same in every wave. acc[h][c]: this thread's weighted sum of value dim
// 8 (tid & 15) + c for head h, relative to the running maximum.
__device__ __forceinline__ void d_stage(const DTiles& t, const dbf16x8 (&bq)[4], int t0, int rend, float& m, float& z,
                                        float (&acc)[kDenseMaxGroup][8], DShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, kq = lane >> 4;
  // scores: lane holds head j for rows 16 wave + 4 kq + e of the stage
  float s[4];
  {
    df32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q) a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(d_as_bf16x8(t.k[q]), bq[q], a, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] = (t0 + 16 * wave + 4 * kq + e < rend) ? a[e] : -INFINITY;
  }
  float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  if (kq == 0) sh.wmax[wave][j] = mx;
  d_barrier();
  // the new running maximum (row t0 of every stage is below rend, so it is
  // finite from the first stage on)
  float mn = m;
#pragma unroll
  for (int w = 0; w < kDWaves; ++w) mn = fmaxf(mn, sh.wmax[w][j]);
  const float alpha = m == -INFINITY ? 0.f : expf((m - mn) * kDInvSqrtD);
  float ps = 0.f;
  float p[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    p[e] = expf((s[e] - mn) * kDInvSqrtD);  // rows past rend: exp(-inf) = 0
    ps += p[e];
  }
  if (j < kDenseMaxGroup) {
#pragma unroll
    for (int e = 0; e < 4; ++e) sh.p[16 * wave + 4 * kq + e][j] = p[e];
  }
  ps += __shfl_xor(ps, 16);
  ps += __shfl_xor(ps, 32);
  if (kq == 0) sh.wz[wave][j] = ps;
  if (wave == 0 && kq == 0 && j < kDenseMaxGroup) sh.alpha[j] = alpha;
  m = mn;
  d_barrier();
  float zs = 0.f;
#pragma unroll
  for (int w = 0; w < kDWaves; ++w) zs += sh.wz[w][j];
  z = alpha * z + zs;
  // values
  const int rg = threadIdx.x >> 4;
  float al[kDenseMaxGroup];
#pragma unroll
  for (int h = 0; h < kDenseMaxGroup; ++h) al[h] = sh.alpha[h];
#pragma unroll
  for (int h = 0; h < kDenseMaxGroup; ++h)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[h][c] *= al[h];
#pragma unroll
  for (int i = 0; i < kDVRows; ++i) {
    const float4 pa = *reinterpret_cast<const float4*>(&sh.p[rg + 32 * i][0]);
    const float4 pb = *reinterpret_cast<const float4*>(&sh.p[rg + 32 * i][4]);
    const float pw[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
    const uint4 w4 = t.v[i];
    const float x[8] = {d_lo(w4.x), d_hi(w4.x), d_lo(w4.y), d_hi(w4.y),
                        d_lo(w4.z), d_hi(w4.z), d_lo(w4.w), d_hi(w4.w)};
#pragma unroll
    for (int h = 0; h < kDenseMaxGroup; ++h)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[h][c] = fmaf(pw[h], x[c], acc[h][c]);
  }
}

// Work group (bg, split): KV group bg = b * Hkv + g, rows [split * rows,
// min((split + 1) * rows, length)). part[(b Hq + g G + jj) * n_split + split]
// receives [0, 128) the value sums, [128] m (the unscaled maximum score), [129]
// Z. An empty slice writes m = -inf, Z = 0.
__global__ __launch_bounds__(kDThreads) void k_dense(Dims d, const uint16_t* q, const uint16_t* k,
                                                     const uint16_t* v, int length, float* part, int n_split,
                                                     int rows) {
  __shared__ DShared sh;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, kq = lane >> 4;
  const int bg = static_cast<int>(blockIdx.x) / n_split, split = static_cast<int>(blockIdx.x) % n_split;
  const int bb = bg / d.Hkv, g = bg % d.Hkv;
  const int r0 = split * rows, r1 = min(r0 + rows, length);
  const int h0 = bb * d.Hq + g * d.G;
  dbf16x8 bq[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (j < d.G) u = *reinterpret_cast<const uint4*>(q + static_cast<long>(h0 + j) * kHeadDim + 8 * kq + 32 * s);
    bq[s] = d_as_bf16x8(u);
  }
  float m = -INFINITY, z = 0.f;
  float acc[kDenseMaxGroup][8];
#pragma unroll
  for (int h = 0; h < kDenseMaxGroup; ++h)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[h][c] = 0.f;
  if (r0 < r1) {
    const uint16_t* kb = k + static_cast<long>(bg) * d.max_len * kHeadDim;
    const uint16_t* vb = v + static_cast<long>(bg) * d.max_len * kHeadDim;
    DTiles ta, tb, tc;
    d_load(ta, kb, vb, r0, r1);
    if (r0 + kDStage < r1) d_load(tb, kb, vb, r0 + kDStage, r1);
    for (int t0 = r0; t0 < r1; t0 += 3 * kDStage) {
      if (t0 + 2 * kDStage < r1) d_load(tc, kb, vb, t0 + 2 * kDStage, r1);
      d_stage(ta, bq, t0, r1, m, z, acc, sh);
      if (t0 + kDStage >= r1) break;
      if (t0 + 3 * kDStage < r1) d_load(ta, kb, vb, t0 + 3 * kDStage, r1);
      d_stage(tb, bq, t0 + kDStage, r1, m, z, acc, sh);
      if (t0 + 2 * kDStage >= r1) break;
      if (t0 + 4 * kDStage < r1) d_load(tb, kb, vb, t0 + 4 * kDStage, r1);
      d_stage(tc, bq, t0 + 2 * kDStage, r1, m, z, acc, sh);
    }
  }
  // the slice's sums: the four row groups of a wave, then the waves
#pragma unroll
  for (int h = 0; h < kDenseMaxGroup; ++h)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      acc[h][c] += __shfl_xor(acc[h][c], 16);
      acc[h][c] += __shfl_xor(acc[h][c], 32);
    }
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < kDenseMaxGroup; ++h)
#pragma unroll
      for (int c = 0; c < 8; ++c) sh.red[wave][h][8 * lane + c] = acc[h][c];
  }
  d_barrier();
  const int dim = threadIdx.x & (kHeadDim - 1);
  for (int h = threadIdx.x / kHeadDim; h < d.G; h += kDThreads / kHeadDim) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < kDWaves; ++w) a += sh.red[w][h][dim];
    part[(static_cast<long>(h0 + h) * n_split + split) * kDensePart + dim] = a;
  }
  if (wave == 0 && kq == 0 && j < d.G) {
    float* pm = part + (static_cast<long>(h0 + j) * n_split + split) * kDensePart + kHeadDim;
    pm[0] = m;
    pm[1] = z;
  }
}

// One work group per query head: thread (dim, sg) takes output dim `dim` over
// the slices s = sg, sg + 4, ... (16 of them per round, all loads issued
// together), with a maximum of its own; the four slice groups are then merged
// the same way through LDS.
constexpr int kDMergeThreads = 512;
constexpr int kDMergeGroups = kDMergeThreads / kHeadDim;  // 4
constexpr int kDMergeU = 16;                               // slices per thread per round

__global__ __launch_bounds__(kDMergeThreads) void k_dense_merge(const float* part, int n_split, float* out) {
  __shared__ float red[3][kDMergeGroups][kHeadDim];  // per slice group: maximum, value sum, weight sum
  const long bh = blockIdx.x;
  const int dim = threadIdx.x & (kHeadDim - 1), sg = threadIdx.x / kHeadDim;
  const float* pr = part + bh * n_split * kDensePart;
  float m = -INFINITY, num = 0.f, den = 0.f;
  for (int c0 = sg; c0 < n_split; c0 += kDMergeGroups * kDMergeU) {
    float a[kDMergeU], ms[kDMergeU], zs[kDMergeU];
#pragma unroll
    for (int i = 0; i < kDMergeU; ++i) {
      const int sl = c0 + kDMergeGroups * i;
      const float* ps = pr + static_cast<long>(min(sl, n_split - 1)) * kDensePart;
      a[i] = ps[dim];
      ms[i] = sl < n_split ? ps[kHeadDim] : -INFINITY;
      zs[i] = ps[kHeadDim + 1];
    }
    float mn = m;
#pragma unroll
    for (int i = 0; i < kDMergeU; ++i) mn = fmaxf(mn, ms[i]);
    if (mn == -INFINITY) continue;  // only empty slices so far
    const float sc = m == -INFINITY ? 0.f : expf((m - mn) * kDInvSqrtD);
    num *= sc;
    den *= sc;
#pragma unroll
    for (int i = 0; i < kDMergeU; ++i) {
      const float w = ms[i] == -INFINITY ? 0.f : expf((ms[i] - mn) * kDInvSqrtD);
      num = fmaf(w, a[i], num);
      den = fmaf(w, zs[i], den);
    }
    m = mn;
  }
  red[0][sg][dim] = m;
  red[1][sg][dim] = num;
  red[2][sg][dim] = den;
  d_barrier();
  if (threadIdx.x < kHeadDim) {
    float mx = red[0][0][dim];
#pragma unroll
    for (int g = 1; g < kDMergeGroups; ++g) mx = fmaxf(mx, red[0][g][dim]);
    float tn = 0.f, td = 0.f;
#pragma unroll
    for (int g = 0; g < kDMergeGroups; ++g) {
      const float mg = red[0][g][dim];
      const float w = mg == -INFINITY ? 0.f : expf((mg - mx) * kDInvSqrtD);
      tn = fmaf(w, red[1][g][dim], tn);
      td = fmaf(w, red[2][g][dim], td);
    }
    out[bh * kHeadDim + dim] = tn / td;
  }
}

}  // namespace

int dense_max_split(const Dims& d) {
  const int groups = d.B * d.Hkv;
  return max(1, (d.n_cu + groups - 1) / groups);
}

void dense_split(const Dims& d, int length, int* n_split, int* rows) {
  const int ns = max(1, min(dense_max_split(d), (length + 15) / 16));
  const int r = ((length + ns - 1) / ns + 15) / 16 * 16;
  *rows = r;
  *n_split = (length + r - 1) / r;
}

hipError_t dense_scratch(float** ptr) {
  static std::mutex mu;
  static float* per_device[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (per_device[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // this device's copy of the array
    if (e != hipSuccess) return e;
    per_device[dev] = static_cast<float*>(p);
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

hipError_t launch_dense(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v, float* out,
                        int length, float* part, hipStream_t s, int phase) {
  int n_split = 1, rows = 1;
  dense_split(d, length, &n_split, &rows);
  if (phase == 0) {
    hipLaunchKernelGGL(k_dense, dim3(d.B * d.Hkv * n_split), dim3(kDThreads), 0, s, d, q, k, v, length, part,
                       n_split, rows);
  } else {
    hipLaunchKernelGGL(k_dense_merge, dim3(d.B * d.Hq), dim3(kDMergeThreads), 0, s, part, n_split, out);
  }
  return hipGetLastError();
}

}  // namespace retopk

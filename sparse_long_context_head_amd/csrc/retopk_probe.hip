// A plain streaming read of device memory: the rate a kernel that does nothing
// but read reaches on the device at hand. It is the measured ceiling that the
// HBM rates of the attention kernels are set against, beside the published
// peak (8 TB/s on MI355X).
//
// Every work group reads 32 KiB per round: each of its 256 threads issues 8
// 16-byte loads at once, a wave's loads of one round covering 1 KiB of
// consecutive bytes; the rounds stride over the buffer by the whole grid. The
// words read are folded into one value per thread that is stored only when it
// equals a fixed pattern, which keeps every load live without writing memory.

#include "retopk_internal.h"

namespace retopk {
namespace {

constexpr int kPThreads = 256;
constexpr int kPUnroll = 8;
constexpr long kPChunk = static_cast<long>(kPThreads) * kPUnroll;  // 16-byte words per work group and round

__global__ __launch_bounds__(kPThreads) void k_stream_read(const uint4* __restrict__ src, long n16, uint32_t* sink) {
  uint32_t x = 0u;
  for (long c = static_cast<long>(blockIdx.x) * kPChunk; c < n16; c += static_cast<long>(gridDim.x) * kPChunk) {
    uint4 w[kPUnroll];
#pragma unroll
    for (int u = 0; u < kPUnroll; ++u) {
      const long i = c + u * kPThreads + threadIdx.x;
      w[u] = i < n16 ? src[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kPUnroll; ++u) x ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
  }
  if (x == 0x9e3779b9u) sink[0] = x;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int n_cu, hipStream_t s) {
  const long n16 = static_cast<long>(bytes / 16);
  const long chunks = (n16 + kPChunk - 1) / kPChunk;
  const long grid = std::max(1L, std::min<long>(chunks, 8L * n_cu));
  hipLaunchKernelGGL(k_stream_read, dim3(static_cast<unsigned>(grid)), dim3(kPThreads), 0, s,
                     static_cast<const uint4*>(buf), n16, sink);
  return hipGetLastError();
}

}  // namespace retopk

// Scoring A/B: the full-history score pass of one KV group (the 7 query heads
// of a Qwen2.5-7B-shaped GQA layer against every key row of their KV head),
// written twice with the same row streaming, once on the matrix cores and once
// on the vector ALUs. Each work group of 8 waves takes a contiguous slice of
// rows; a wave reads 16-row tiles (a lane holds 16 bytes of four 64-byte
// column chunks of one row), two register stages of 4 tiles per wave in
// flight (scheduling barriers keep the compiler from sinking the next stage's
// loads down to their use, which it otherwise does in the matrix form). The matrix form multiplies each tile by the queries in a
// 16x16x32 bf16 MFMA (query heads as the 16 columns, 7 used); the vector form
// keeps each lane's 32 query dimensions per head in registers and takes 16
// bf16 pair dot products per head and row, then sums the four lanes of a row
// with two cross-lane adds. Both keep only a running maximum, stored when it
// equals a fixed value, so that the scores stay live without being written.
namespace retopk {
namespace {

constexpr int kQHeads = 7;
constexpr int kQThreads = 512;
constexpr int kQTiles = 4;                       // 16-row tiles per wave and stage
constexpr int kQRowsPerStage = kQThreads / kWave * kQTiles * 16;

typedef __bf16 pbf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 pbf16x2 __attribute__((ext_vector_type(2)));
typedef float pf32x4 __attribute__((ext_vector_type(4)));

struct QStage {
  uint4 a[kQTiles][4];
};

__device__ __forceinline__ void q_stage_load(QStage& t, const uint16_t* k, int base, int rend, int wave, int j,
                                             int kq) {
#pragma unroll
  for (int u = 0; u < kQTiles; ++u) {
    const int r = min(base + (u * (kQThreads / kWave) + wave) * 16 + j, rend - 1);
    const uint16_t* row = k + static_cast<long>(r) * kHeadDim + 8 * kq;
#pragma unroll
    for (int s = 0; s < 4; ++s) t.a[u][s] = *reinterpret_cast<const uint4*>(row + 32 * s);
  }
}

template <bool kMfma>
__global__ __launch_bounds__(kQThreads) void k_score_probe(const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ q, int n_rows,
                                                           int rows_per_wg, float* sink) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave, j = lane & 15, kq = lane >> 4;
  const int row0 = blockIdx.x * rows_per_wg, rend = min(row0 + rows_per_wg, n_rows);
  if (row0 >= rend) return;
  float best = -3.0e38f;
  QStage ta, tb;
  if constexpr (kMfma) {
    pbf16x8 bq[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 u = make_uint4(0u, 0u, 0u, 0u);
      if (j < kQHeads) u = *reinterpret_cast<const uint4*>(q + j * kHeadDim + 8 * kq + 32 * s);
      bq[s] = __builtin_bit_cast(pbf16x8, u);
    }
    auto score = [&](const QStage& t) {
#pragma unroll
      for (int u = 0; u < kQTiles; ++u) {
        pf32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(pbf16x8, t.a[u][s]), bq[s], acc, 0, 0,
                                                        0);
        best = fmaxf(best, fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3])));
      }
    };
    q_stage_load(ta, k, row0, rend, wave, j, kq);
    for (int t0 = row0; t0 < rend; t0 += 2 * kQRowsPerStage) {
      q_stage_load(tb, k, t0 + kQRowsPerStage, rend, wave, j, kq);
      __builtin_amdgcn_sched_barrier(0);  // the next stage's loads stay ahead of this stage's math
      score(ta);
      if (t0 + kQRowsPerStage >= rend) break;
      q_stage_load(ta, k, t0 + 2 * kQRowsPerStage, rend, wave, j, kq);
      __builtin_amdgcn_sched_barrier(0);
      score(tb);
    }
  } else {
    uint32_t qv[kQHeads][16];
#pragma unroll
    for (int h = 0; h < kQHeads; ++h)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 u = *reinterpret_cast<const uint4*>(q + h * kHeadDim + 8 * kq + 32 * s);
        qv[h][4 * s] = u.x;
        qv[h][4 * s + 1] = u.y;
        qv[h][4 * s + 2] = u.z;
        qv[h][4 * s + 3] = u.w;
      }
    auto dot2 = [](uint32_t a, uint32_t b, float c) {
      return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(pbf16x2, a), __builtin_bit_cast(pbf16x2, b), c,
                                             false);
    };
    auto score = [&](const QStage& t) {
#pragma unroll
      for (int u = 0; u < kQTiles; ++u) {
#pragma unroll
        for (int h = 0; h < kQHeads; ++h) {
          float acc = 0.f;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            acc = dot2(t.a[u][s].x, qv[h][4 * s], acc);
            acc = dot2(t.a[u][s].y, qv[h][4 * s + 1], acc);
            acc = dot2(t.a[u][s].z, qv[h][4 * s + 2], acc);
            acc = dot2(t.a[u][s].w, qv[h][4 * s + 3], acc);
          }
          acc += __shfl_xor(acc, 16);
          acc += __shfl_xor(acc, 32);
          best = fmaxf(best, acc);
        }
      }
    };
    q_stage_load(ta, k, row0, rend, wave, j, kq);
    for (int t0 = row0; t0 < rend; t0 += 2 * kQRowsPerStage) {
      q_stage_load(tb, k, t0 + kQRowsPerStage, rend, wave, j, kq);
      __builtin_amdgcn_sched_barrier(0);  // the next stage's loads stay ahead of this stage's math
      score(ta);
      if (t0 + kQRowsPerStage >= rend) break;
      q_stage_load(ta, k, t0 + 2 * kQRowsPerStage, rend, wave, j, kq);
      __builtin_amdgcn_sched_barrier(0);
      score(tb);
    }
  }
  if (best == 1.5e38f) sink[0] = best;
}

}  // namespace

hipError_t launch_score_probe(int use_mfma, const uint16_t* k, long n_rows, const uint16_t* q, float* sink, int n_cu,
                              hipStream_t s) {
  const int per = static_cast<int>(((n_rows + n_cu - 1) / n_cu + 15) / 16 * 16);
  const int grid = static_cast<int>((n_rows + per - 1) / per);
  if (use_mfma)
    hipLaunchKernelGGL(k_score_probe<true>, dim3(grid), dim3(kQThreads), 0, s, k, q, static_cast<int>(n_rows),
                       per, sink);
  else
    hipLaunchKernelGGL(k_score_probe<false>, dim3(grid), dim3(kQThreads), 0, s, k, q, static_cast<int>(n_rows),
                       per, sink);
  return hipGetLastError();
}

}  // namespace retopk

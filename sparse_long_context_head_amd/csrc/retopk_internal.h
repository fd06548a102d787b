// Internal declarations shared by the ReTopK kernels and the C-ABI host code.
// Not part of the public interface (that is include/retopk.h).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdint>

namespace retopk {

constexpr int kHeadDim = 128;        // D; one bf16 key row is 256 bytes
constexpr int kWave = 64;            // CDNA wavefront width
constexpr int kMaxGroup = 16;        // query heads per KV head handled by one MFMA tile
constexpr int kHistBits = 10;        // first-level histogram: top 10 bits of the ordered key
constexpr int kNumBins = 1 << kHistBits;
constexpr int kHistShift = 32 - kHistBits;
constexpr int kStatsCap = 4096;      // decode steps kept in the statistics ring
constexpr int kExactMinRows = 512;   // key rows per score work group of the full-history pass, at least
constexpr int kBoundaryLds = 4096;   // boundary-bin candidates resolved in LDS, at least (32 KiB of 64-bit keys)
constexpr int kHeadThreads = 512;    // threads of the per-head kernels
constexpr int kBitmapWords = 8192;   // LDS bitmap window: 262144 token positions (32 KiB)
constexpr int kLdsLimit = 124 * 1024;  // dynamic LDS a per-head kernel may use (static LDS <= 36 KiB)
constexpr int kMaxCand = 16384;      // R*K + W limit (candidate keys kept in LDS for reranking)
constexpr int kDenseMaxGroup = 8;    // query heads per KV head the dense-attention kernel handles
constexpr int kDensePart = 132;      // floats per (query head, row slice) partial: 128 sums, m, Z, 2 pad
// Ints between two polled flags (decisions, hand-off flags): one per 128-byte
// line, so that many work groups polling many flags do not all queue on the
// same few lines.
constexpr int kFlagStride = 32;

// Problem dimensions, passed by value to every kernel.
struct Dims {
  int B, Hq, Hkv, G;       // G = Hq / Hkv query heads per KV head
  int max_len;             // rows of the k / v buffers
  int score_stride;        // row stride of the full-history score workspace (max_len rounded to 16)
  int K, C, W, R, Tr;
  int cand_cap;            // R*K + W
  int n_cu;                // compute units of the device
  int recent;              // 1: recent-R retrieval (the R newest entries, rho_max over them)
  double tau;
};

// Device buffers owned by a handle. BH = B * Hq.
struct Bufs {
  // query-support cache (Eq. 5), a ring per head
  float* cache_qbar;       // [BH, C, D]
  int32_t* cache_supp;     // [BH, C, K]
  int32_t* cache_len;      // [BH, C]
  int32_t* fifo;           // [BH, 2]: next slot to write, entries held
  // per-step workspaces
  int32_t* path;           // [BH]      1 exact, 0 reuse
  double* rho;             // [BH]      rho_max
  int32_t* ret;            // [BH, R]   retrieved FIFO positions, -1 pad
  int32_t* retslot;        // [BH, R]   their ring slots
  int32_t* m;              // [BH]      M_t
  int32_t* cand;           // [BH, cand_cap]  A_t ascending
  float* score;            // [BH, score_stride]  full-history q.k
  uint32_t* hist;          // [BH, 2, kNumBins]  histogram of ordered score keys, a half per call parity
  uint2* hits;             // [BH, max_len] survivors (scores in the boundary bin or above) as
                           //   (position, score bits); a score work group's segment [row0, rend)
                           //   writes its own in ascending position order from row0 on
  uint2* ccnt;             // [BH, n_cu] (survivors of a score work group's segment, call flag),
                           //   one 8-byte device-scope store once the survivors are out
  int32_t* dec;            // [BH, kFlagStride] path decision of the current call: call flag | exact
                           //   (one per 128-byte line)
  int32_t* err;            // [1]  sticky device error word (1: a wait of the step kernel timed out)
  int32_t* wdone;          // [n_cu, kFlagStride] per score work group (one per 128-byte line), the
                           //   call flag once its scores and histogram adds are out
  uint64_t* bkeys;         // [BH, max_len] boundary-bin composite keys when more than the LDS holds
  int32_t* sel;            // [BH, K]   S_hat_t ascending
  float* selsc;            // [BH, K]   q.k of S_hat_t
  int32_t* sellen;         // [BH]
  // statistics ring
  uint8_t* st_path;        // [kStatsCap, BH]
  double* st_rho;          // [kStatsCap, BH]
  int32_t* st_m;           // [kStatsCap, BH]
  int32_t* hint;           // [1] host-mapped: exact KV groups of the latest decode step (sizes the next
                           //   launch; read by the host without synchronising)
  Bufs* self;              // device copy of this table (what the step kernel is given)
};

enum KernelId : int { kKStep = 0, kKReset, kKDense, kKDenseMerge, kKAdvance, kNumKernels };

const char* kernel_name(int id);

// Dynamic LDS of the kernels for the given dimensions.
size_t head_lds_bytes(const Dims& d);
size_t score_lds_bytes(const Dims& d);
size_t step_lds_bytes(const Dims& d);
size_t finish_lds_bytes(const Dims& d);
// Score work groups of a call at this length and mode (HeadMode); wide: the
// call is expected to hold exact heads in at least half the KV groups.
int score_grid(const Dims& d, int length, int mode, bool wide);
// Rows per query head of LDS a score work group keeps its scores in (0: they
// go to the score workspace).
int score_keep_rows(const Dims& d, int length, int n_score);

// Launch helpers (retopk_kernels.hip). Each returns the hipError_t of the
// launch. A decode step, the exact Top-K baseline and the cache
// initialisation are each one k_step launch per call on one stream.
enum HeadMode : int { kModeDecode = 0, kModeExact = 1 };

// Raise the dynamic-LDS limit of the kernels to what `d` needs.
hipError_t configure_kernels(const Dims& d);
hipError_t launch_reset(const Dims& d, const Bufs& b, hipStream_t s);
// The whole call in one launch: recall, path decision and the reuse path of
// reuse heads (k, v, out are used by reuse heads only; in kModeExact every
// head is marked exact, with no recall), the full-history scores and
// histogram of exact heads, and their global Top-K, softmax-V (skipped when v
// or out is NULL), S_t to sel_out (when not NULL) and cache update (when
// push). call_flag: an even number, different from the previous call's, that
// tags this call's decision flags; its bit 1 selects the half of `scored`.
// ctl: NULL for a step whose length, t_dec and call flag are the arguments;
// else the device control words {length, t_dec, seq} of graph-replayed steps
// (length then sizes the launch: the longest of the replays), the call flag
// being 2 * ((seq + layer) & kSeqMask) and stats_slot >= 0 meaning "record".
hipError_t launch_step(const Dims& d, const Bufs& b, const uint16_t* q, long q_sb, long q_sh, const uint16_t* k,
                       const uint16_t* v, float* out, int32_t* sel_out, int length, int t_dec, int mode,
                       int stats_slot, int push, int call_flag, bool wide, hipStream_t s, const int32_t* ctl,
                       int layer);
constexpr int kSeqMask = (1 << 29) - 1;  // call sequence numbers, mod 2^29 (the call flag is twice one)
hipError_t launch_advance(int32_t* ctl, int n_layers, hipStream_t s);
hipError_t launch_set_position(int32_t* ctl, int length, int t_dec, int seq, hipStream_t s);

// Dense softmax attention (retopk_dense.hip): row slices per KV group of a
// call at this length, and the most any length gives (the partials workspace
// holds B * Hq * dense_max_split(d) * kDensePart floats).
int dense_max_split(const Dims& d);
// The static scratch of the no-allocation dense entry point: 4 MiB of floats
// (the partials of B * Hq * dense_max_split(d) slices must fit), and this
// device's address of it (looked up once per device with that device current).
constexpr size_t kNoAllocScratchFloats = (static_cast<size_t>(4) << 20) / 4;
constexpr int kMaxDevices = 64;
hipError_t dense_scratch(float** ptr);
void dense_split(const Dims& d, int length, int* n_split, int* rows);
// phase 0: the slices' partial results (k_dense); phase 1: their merge into
// out (k_dense_merge). Both on stream s, one launch each.
hipError_t launch_dense(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v, float* out,
                        int length, float* part, hipStream_t s, int phase);

// Plain streaming read of `bytes` (a multiple of 16) at buf (retopk_probe.hip).
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int n_cu, hipStream_t s);
// Score pass of 7 query heads over n_rows key rows, on MFMA (use_mfma) or on
// the vector ALUs (retopk_probe.hip); q holds 7 rows of kHeadDim bf16.
hipError_t launch_score_probe(int use_mfma, const uint16_t* k, long n_rows, const uint16_t* q, float* sink, int n_cu,
                              hipStream_t s);
}  // namespace retopk

// Internal declarations shared by the kernels and the C-ABI host code.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lfattn {

// Keys per tile staged in LDS, and query rows per wavefront (one 32x32 MFMA
// block of queries).
constexpr int kTileKeys = 64;
constexpr int kWaveRows = 32;
// Waves per band workgroup; a band workgroup covers kBandWaves * 32 query rows.
constexpr int kBandWaves = 4;
constexpr int kBandRows = kBandWaves * kWaveRows;
// The bf16 band kernel stages the global positions in LDS; this many at most.
constexpr int kMaxGlobalBf16 = 512;
// Key chunks of the global rows are merged from one batch of loads; the
// chunk count per row set is at most this.
constexpr int kMergeBatch = 16;
// The band launch merges a set of global rows itself (the last of its chunk
// items to finish, from one round of loads) when the set has at most this
// many key chunks; otherwise a separate merge kernel does.
constexpr int kFuseChunks = 16;

// One band workgroup's work: batch-head bh, dilation residue r, and the first
// position t0 (in the residue's subsequence r, r+d, r+2d, ...) of its rows.
// A global-row item (dil = 0, kernels that take global-row work in the same
// launch) is instead one workgroup's worth of global rows (set r of its batch
// element's sorted global list) against key chunk t0, and it writes a partial
// (m, l, acc) record per row.  Either kind carries its batch element b and
// that element's global list: ng positions from BandArgs::glob + g0.
struct BandWork {
  int bh;
  int r;
  int t0;
  int dil;  // band item: its head's dilation (>= 1); global-row item: 0
  int g0;   // offset of the batch element's global list
  int ng;   // its length
  int b;    // batch element (bh / H)
  int pad;
};

struct BandArgs {
  const void* Q;
  const void* K;
  const void* V;
  // The global rows' projections (the same pointers as Q, K, V when the
  // caller gives none): global-row items read these.
  const void* Qg;
  const void* Kg;
  const void* Vg;
  void* O;
  const BandWork* work;        // one entry per workgroup
  const int* glob;             // the sorted global lists, one after another
  const unsigned char* is_glob;  // [B or 1][N]: 1 where the position is global
  long long isg_stride;        // N (one row per batch element) or 0 (one shared row)
  int H, N, hw, n_glob;        // n_glob: the longest global list
  int hr;                      // keys a row scores after itself: hw, or 0 (causal)
  int chunk;                   // > 0: chunked attention, chunks of this many keys
  int cbase;                   // first position of the chunked main sequence
  float* lse;                  // [B, H, N] log-sum-exp of the band rows' scores, or null
  float sl2;                   // softmax scale times log2(e)
  int rows_per_wg;             // rows per band workgroup (bf16: 64 or 128)
  // Global-row items (dil 0): partial records laid out as GlobArgs::part
  // with rows_per_wg rows per set, and the chunking of the keys; gcount:
  // one arrival count per (b*H + h, set), zero between calls (the workgroup
  // that merges a set resets it), or null when a separate kernel merges.
  float* part;
  unsigned* gcount;
  int n_sets, n_chunks, chunk_keys;
  // Nonzero when every workgroup of the launch is resident at once: the
  // wavefronts then take issue priority by the steps they have left (the
  // furthest behind first), so that the workgroups finish together.
  int lrf;
};

struct GlobArgs {
  const void* Q;               // the global rows' projections
  const void* K;
  const void* V;
  void* O;
  const int* glob;             // the sorted global lists, one after another
  const int2* gsel;            // [B]: (offset into glob, length) of each batch element's list
  float* part;                 // partial (m, l, 2 pad, acc[D]) records
  int H, N, n_glob;            // n_glob: the longest global list
  int n_bh;                    // B * H
  int rows_per_set;            // waves * 32
  int n_sets;                  // sets of up to waves*32 global rows per head
  int n_chunks;                // key chunks per (bh, set)
  int chunk_keys;              // keys per chunk, a multiple of kTileKeys
  float sl2;
  float* lse;                  // [B, H, N] log-sum-exp of the global rows' scores, or null
};

// Backward pass (bf16, D = 64 or 128): gradients of the band + global attention.
// Each side's work table holds band items of 64 or 128 rows (row side) or
// keys (key side), ks = 2 or 1, and global items of as many global positions
// against a chunk of chunk_keys keys (row side) or rows (key side).
struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  const float* lse;            // [B, H, N] natural log-sum-exp from the forward
  // Workspace the row side writes for the key side, three planes of
  // [B, H, N]: -Delta (Delta = dO . O), -lse / scale, and -lse / scale with
  // -inf at global positions.
  float* terms;
  float* dQ;                   // [B, H, N, D] fp32 outputs
  float* dK;
  float* dV;
  // The global rows' own projections (the same pointers as Q, K, V when the
  // forward shared them) and, with proj set, their gradients: the global
  // rows' terms go to dQg, dKg, dVg ([B, H, N, D] fp32) instead of dQ, dK, dV.
  const void* Qg;
  const void* Kg;
  const void* Vg;
  float* dQg;
  float* dKg;
  float* dVg;
  int proj;
  const BandWork* work;
  const int* glob;
  const unsigned char* is_glob;
  long long isg_stride;
  int H, N, D, n_bh, hw, hr, chunk, cbase, chunk_keys, n_glob;
  int ks;                      // 1: 128 rows (keys) per item; 2: 64, tiles split in two
  // Query side, D = 64: wavefronts per SIMD of its kernel, 3 (168 registers)
  // or 4 (128; more workgroups per round for launches of several rounds).
  int rows_wpe;
  float sl2, scale;
  // Global items' partial gradients, three planes (dQ, dK, dV) of
  // [B*H][n_gch chunks][n_glob][D] fp32, summed by the merge kernel; gsel:
  // (offset, length) of each batch element's global list.
  float* gpart;
  int n_gch;
  const int2* gsel;
};

// Optional events around one launch: start and stop take the kernel's own
// begin and end timestamps (hipExtLaunchKernel), so their elapsed time is the
// kernel's duration without the stream's marker overhead.  Null: untimed.
struct Timing {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

template <typename A>
inline hipError_t launch_kernel(void (*k)(A), dim3 grid, dim3 block, hipStream_t s, const A& a,
                                const Timing& t) {
  void* args[] = {const_cast<A*>(&a)};
  return hipExtLaunchKernel(reinterpret_cast<const void*>(k), grid, block, args, 0, s, t.start,
                            t.stop, 0);
}

// Kernels that take the work table as a separate first argument: the build
// preloads the first kernel-argument dwords into scalar registers, so each
// wavefront's load of its work item goes out at once instead of after the
// load of the argument block.
template <typename A>
inline hipError_t launch_kernel(void (*k)(const BandWork*, A), dim3 grid, dim3 block,
                                hipStream_t s, const A& a, const Timing& t) {
  const BandWork* work = a.work;
  void* args[] = {const_cast<BandWork**>(&work), const_cast<A*>(&a)};
  return hipExtLaunchKernel(reinterpret_cast<const void*>(k), grid, block, args, 0, s, t.start,
                            t.stop, 0);
}

// Launchers (defined next to the kernels).  dtype: 0 fp32, 1 bf16.
hipError_t launch_band(int dtype, int D, const BandArgs& a, int n_wg, hipStream_t s, const Timing& t);
hipError_t launch_band_bf16(int D, const BandArgs& a, int n_wg, hipStream_t s, const Timing& t);
// Whether the band kernel for this element type and D also takes the
// global-row items (kind 1) in its launch (one workgroup's rows per set).
bool band_takes_global_items(int dtype, int D);
// Band workgroups one compute unit holds at once (registers and LDS).
int band_workgroups_per_cu(int dtype, int D);
// Rows per set of the global-row items of a bf16 band launch (D = 64: sets
// of 64 rows in every launch; D = 128: the band workgroup's rows).
int global_set_rows(int D, int band_rows);
hipError_t launch_glob(int dtype, int D, int waves, const GlobArgs& a, int n_wg, hipStream_t s,
                       const Timing& t);
hipError_t launch_glob_merge(int dtype, int D, const GlobArgs& a, hipStream_t s, const Timing& t);
// The row-side and key-side launches take their own work tables (rows.work,
// keys.work; n_*_wg items); t: events around the rows, keys and merge
// kernels (null events: untimed).
hipError_t launch_backward_bf16(const BwdArgs& rows, const BwdArgs& keys, int n_rows_wg,
                                int n_keys_wg, hipStream_t s, const Timing t[3]);

}  // namespace lfattn

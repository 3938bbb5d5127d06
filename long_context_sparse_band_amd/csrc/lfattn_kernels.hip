// HIP kernels for band + global sparse attention on gfx950 (MI355X): the
// fp32 band and global-row partial kernels, and the merge of global-row
// partials shared by both dtypes (the bf16 band kernel is in band_bf16.hip).
//
// Band kernel (fp32): one workgroup of 4 wavefronts takes 128 consecutive
// query rows of one (batch, head, dilation residue) and walks the 64-key tiles
// of their band (staged in LDS through registers), then the tiles of gathered
// global keys.  Each wavefront owns 32 query rows and computes, per tile,
//   S^T = K_tile Q^T          (v_mfma_f32_32x32x2f32)
//   online softmax on S^T     (running max and sum per query row)
//   O^T += V_tile^T P^T       (same MFMA shape, fp32 accumulators)
// Scores are kept transposed (keys down the MFMA rows, queries across lanes)
// so that one lane holds 16 keys of a single query: the row maximum is a
// per-lane reduction plus one exchange between lane l and lane l+32, and the
// exponentiated scores already sit in the lane layout of the next MFMA's B
// operand.
//
// Global-row kernels: the rows of global tokens attend to all N keys.  Each
// workgroup of the partial kernel scores a chunk of keys for up to 128 global
// rows and writes a partial (max, sum, unnormalised output); the merge kernel,
// launched after the band kernel on the same stream, combines the chunks of
// every global row and writes those output rows.
//
// The math is Eq. (1) of the Unlimiformer page (section 2.3) over the
// Longformer pattern (Ultralytics glossary "Longformer", section on how the
// attention works); the running maximum relies on softmax ignoring a constant
// added to all its inputs (Unlimiformer section 2.3, footnote 3).
#include "lfattn_internal.h"

namespace lfattn {
namespace {

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int TK = kTileKeys;
// Running maximum before any key is seen: finite, so that exp2(m - m_new) is
// 0 rather than NaN.
constexpr float kNegInit = -1.0e30f;
// The running maximum is only moved when a tile's maximum exceeds it by more
// than this (log2 units); weights then stay below 2^8, far inside fp32 and
// bf16 range, and most tiles skip rescaling the accumulators.
constexpr float kSlack = 8.0f;

__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Key of accumulator register i (0..15) of a 32x32 MFMA result block, for the
// lane half hi = lane / 32: row 8*(i/4) + 4*hi + i%4 of the block.
__device__ __forceinline__ int block_row(int i, int hi) { return 8 * (i >> 2) + 4 * hi + (i & 3); }

// ---------------------------------------------------------------------------
// LDS tiles and the cooperative loaders.
// ---------------------------------------------------------------------------

// fp32: K and V both row-major [key][d]; the pitches spread the MFMA operand
// reads over the LDS banks.
template <int D>
struct Tile {
  static constexpr int KP = D + 4;
  static constexpr int VP = D + 8;
  float k[TK * KP];
  float v[TK * VP];
};

template <int D, int NT>
struct Loader {
  static constexpr int C4 = D / 4;           // 16-byte chunks per row
  static constexpr int NC = TK * C4 / NT;    // chunks per thread, each of K and V
  static_assert(NC >= 1, "tile too small for the workgroup");
  float4 k[NC];
  float4 v[NC];

  template <typename RowOf>
  __device__ __forceinline__ void fetch(const float* Kp, const float* Vp, RowOf row_of, int tid) {
#pragma unroll
    for (int e = 0; e < NC; ++e) {
      const int c = tid + NT * e;
      const int kk = c / C4, c4 = c % C4;
      const int row = row_of(kk);
      const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
      k[e] = row >= 0 ? *(const float4*)(Kp + (size_t)row * D + c4 * 4) : z;
      v[e] = row >= 0 ? *(const float4*)(Vp + (size_t)row * D + c4 * 4) : z;
    }
  }

  __device__ __forceinline__ void store(Tile<D>& t, int tid) const {
#pragma unroll
    for (int e = 0; e < NC; ++e) {
      const int c = tid + NT * e;
      const int kk = c / C4, c4 = c % C4;
      *(float4*)&t.k[kk * Tile<D>::KP + c4 * 4] = k[e];
      *(float4*)&t.v[kk * Tile<D>::VP + c4 * 4] = v[e];
    }
  }
};

// ---------------------------------------------------------------------------
// Per-wavefront attention state for 32 query rows, and one tile step.
// ---------------------------------------------------------------------------

template <int D>
struct WaveAttn {
  // B operand of the fp32 MFMA k-steps: step t pairs d = t (hi = 0) with
  // d = t + D/2 (hi = 1); any fixed pairing of d values is a valid split.
  float q[D / 2];
  f32x16 acc[D / 32];
  float m, l;

  __device__ __forceinline__ void load_q(const float* Qp, int row, int hi) {
#pragma unroll
    for (int t4 = 0; t4 < D / 8; ++t4) {
      float4 x = row >= 0 ? *(const float4*)(Qp + (size_t)row * D + (D / 2) * hi + 4 * t4)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
      q[4 * t4] = x.x; q[4 * t4 + 1] = x.y; q[4 * t4 + 2] = x.z; q[4 * t4 + 3] = x.w;
    }
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[b][i] = 0.0f;
    m = kNegInit;
    l = 0.0f;
  }

  __device__ __forceinline__ void scores(const Tile<D>& t, int lane, f32x16 (&s)[2]) const {
    const int hi = lane >> 5, r = lane & 31;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.0f;
#pragma unroll
      for (int t4 = 0; t4 < D / 8; ++t4) {
        const float4 a = *(const float4*)&t.k[(32 * kb + r) * Tile<D>::KP + (D / 2) * hi + 4 * t4];
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, q[4 * t4], s[kb], 0, 0, 0);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, q[4 * t4 + 1], s[kb], 0, 0, 0);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, q[4 * t4 + 2], s[kb], 0, 0, 0);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, q[4 * t4 + 3], s[kb], 0, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void accumulate(const Tile<D>& t, int lane, const f32x16 (&p)[2]) {
    const int hi = lane >> 5, r = lane & 31;
    // k-step (kb, i) pairs key 32*kb + block_row(i, 0) (hi = 0) with
    // 32*kb + block_row(i, 1) (hi = 1): exactly the keys whose weights the two
    // lane halves hold in register i of score block kb.
#pragma unroll
    for (int b = 0; b < D / 32; ++b) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float a = t.v[(32 * kb + block_row(i, hi)) * Tile<D>::VP + 32 * b + r];
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p[kb][i], acc[b], 0, 0, 0);
        }
      }
    }
  }

  __device__ __forceinline__ void store_row(float* Op, int row, int hi, float inv) const {
#pragma unroll
    for (int b = 0; b < D / 32; ++b) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 o = make_float4(acc[b][4 * g] * inv, acc[b][4 * g + 1] * inv,
                               acc[b][4 * g + 2] * inv, acc[b][4 * g + 3] * inv);
        *(float4*)(Op + (size_t)row * D + 32 * b + 8 * g + 4 * hi) = o;
      }
    }
  }
};

// Online softmax over one tile of transposed scores s (raw, -inf where the
// pair is not scored), then the P.V accumulation.  m is kept in log2 units
// of the scaled scores.
template <int D, typename Tl>
__device__ __forceinline__ void softmax_accumulate(WaveAttn<D>& st, const Tl& tile,
                                                   int lane, f32x16 (&s)[2], float sl2) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
  mx = pair_max(mx) * sl2;
  if (__any(mx > st.m + kSlack)) {
    const float mn = fmaxf(st.m, mx);
    const float alpha = fast_exp2(st.m - mn);
    st.l *= alpha;
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.acc[b][i] *= alpha;
    st.m = mn;
  }
  float ls = 0.0f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(fmaf(s[kb][i], sl2, -st.m));
      s[kb][i] = p;
      ls += p;
    }
  st.l += ls;
  st.accumulate(tile, lane, s);
}

template <bool BF16>
struct ElemT;
template <>
struct ElemT<true> { typedef unsigned short type; };
template <>
struct ElemT<false> { typedef float type; };

// ---------------------------------------------------------------------------
// Band kernel.
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(kBandWaves * 64) void band_kernel(BandArgs a) {
  typedef float E;
  constexpr int NT = kBandWaves * 64;
  __shared__ Tile<D> tile;
  __shared__ __attribute__((aligned(16))) int gsub[TK];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hi = lane >> 5;
  const BandWork w = a.work[blockIdx.x];
  const int d = w.dil;
  // A row u scores the keys u - hl .. u + hr of its subsequence (hl = hr =
  // the half-width; causal: hr = 0).
  const int r = w.r, t0 = w.t0, hl = a.hw, hr = a.hr, N = a.N;
  // Chunked attention (d = 1): row u scores its chunk c0 .. c0 + C - 1,
  // c0 = cb + C * floor((u - cb) / C), instead; rows before cb are the memory.
  const int cC = a.chunk, cb = a.cbase;
  auto lo_of = [&](int uu) -> int {
    return cC == 0 ? uu - hl : (uu < cb ? uu : cb + (uu - cb) / cC * cC);
  };
  auto hi_of = [&](int uu) -> int {
    return cC == 0 ? uu + hr : (uu < cb ? uu : cb + (uu - cb) / cC * cC + cC - 1);
  };
  // The global list of this item's batch element.
  const int* gl = a.glob + w.g0;
  const int n_glob = w.ng;
  const int Lr = (N - r + d - 1) / d;  // length of the residue's subsequence
  const size_t base = (size_t)w.bh * N * D;
  const E* Qp = (const E*)a.Q + base;
  const E* Kp = (const E*)a.K + base;
  const E* Vp = (const E*)a.V + base;

  // This wave's query rows: subsequence positions ua .. ub (ub < Lr).
  const int ua = t0 + kWaveRows * wave;
  const int ub = min(ua + kWaveRows - 1, Lr - 1);
  const bool wave_live = ua < Lr;
  const int u = ua + (lane & 31);
  const int qrow = u < Lr ? r + d * u : -1;

  WaveAttn<D> st;
  st.load_q(Qp, qrow, hi);

  // Key range of the workgroup's band, in subsequence positions.
  const int s_lo = max(0, lo_of(t0));
  const int s_hi = min(Lr - 1, hi_of(t0 + kBandRows - 1));
  const int lo_a = lo_of(ua), hi_a = hi_of(ua), lo_b = lo_of(ub), hi_b = hi_of(ub);
  const int n_band = (s_hi - s_lo) / TK + 1;
  const int n_glob_tiles = (n_glob + TK - 1) / TK;
  const int n_tiles = n_band + n_glob_tiles;

  auto row_of_tile = [&](int tt) {
    return [=](int kk) -> int {
      if (tt < n_band) {
        const int s = s_lo + TK * tt + kk;
        return s <= s_hi ? r + d * s : -1;
      }
      const int slot = TK * (tt - n_band) + kk;
      return slot < n_glob ? gl[slot] : -1;
    };
  };

  // Keys a row may score inside a band tile form the interval [lo, hi] of
  // subsequence positions.  Rows past the end of the subsequence get an empty
  // interval.
  int lo = max(lo_of(u), 0), hi_key = min(hi_of(u), s_hi);
  if (u >= Lr || hi_key < lo) {
    lo = 0x3fffffff;
    hi_key = lo;
  }
  const unsigned rng = (unsigned)(hi_key - lo);
  constexpr int kNotInClass = 0x40000000;

  Loader<D, NT> ld;
  ld.fetch(Kp, Vp, row_of_tile(0), tid);

  for (int tt = 0; tt < n_tiles; ++tt) {
    ld.store(tile, tid);
    if (tt >= n_band && tid < TK) {
      // Position of each global key in this residue's subsequence, or a value
      // no row's band reaches when the key belongs to another residue class.
      const int slot = TK * (tt - n_band) + tid;
      int sp = kNotInClass;
      if (slot < n_glob) {
        const int off = gl[slot] - r;
        if (off >= 0 && off % d == 0) sp = off / d;
      }
      gsub[tid] = sp;
    }
    __syncthreads();
    if (tt + 1 < n_tiles) ld.fetch(Kp, Vp, row_of_tile(tt + 1), tid);

    if (wave_live) {
      f32x16 s[2];
      if (tt < n_band) {
        const int s0 = s_lo + TK * tt;
        const int kb_ = min(s0 + TK - 1, s_hi);  // last real key of the tile
        const bool any = s0 <= hi_b && kb_ >= lo_a;
        if (any) {
          const bool full = (kb_ == s0 + TK - 1) && (s0 + TK - 1 <= hi_a) && (s0 >= lo_b);
          st.scores(tile, lane, s);
          if (!full) {
            const int base = s0 + 4 * hi - lo;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const unsigned x = (unsigned)(base + 32 * kb + block_row(i, 0));
                s[kb][i] = x > rng ? -INFINITY : s[kb][i];
              }
          }
          softmax_accumulate(st, tile, lane, s, a.sl2);
        }
      } else {
        // Global keys, minus those already inside this row's band.
        const int nvalid = min(TK, n_glob - TK * (tt - n_band));

        bool any = false;
        unsigned keep = 0;  // bit 16*kb + i
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int kk0 = 32 * kb + 8 * g + 4 * hi;
            const int4 sp = *(const int4*)&gsub[kk0];
            const int spv[4] = {sp.x, sp.y, sp.z, sp.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const bool k = (kk0 + c < nvalid) && u < Lr &&
                             (unsigned)(spv[c] - lo) > rng;
              keep |= (unsigned)k << (16 * kb + 4 * g + c);
              any |= k;
            }
          }
        if (__any(any)) {
          st.scores(tile, lane, s);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              s[kb][i] = ((keep >> (16 * kb + i)) & 1u) ? s[kb][i] : -INFINITY;
          softmax_accumulate(st, tile, lane, s, a.sl2);
        }
      }
    }
    __syncthreads();
  }

  if (wave_live) {
    const float lt = pair_sum(st.l);
    if (qrow >= 0 && !a.is_glob[w.b * a.isg_stride + qrow])
      st.store_row((E*)a.O + base, qrow, hi, 1.0f / lt);
  }
}

// ---------------------------------------------------------------------------
// Global-row partial kernel: one (batch-head, row set, key chunk) per workgroup.
// ---------------------------------------------------------------------------

template <int D, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void glob_kernel(GlobArgs a) {
  typedef float E;
  constexpr int NT = WAVES * 64;
  constexpr int ROWS = WAVES * kWaveRows;   // global rows per set
  constexpr int REC = D + 4;                // partial record: m, l, 2 pad, acc[D]
  __shared__ Tile<D> tile;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hi = lane >> 5;
  const int chunk = blockIdx.x % a.n_chunks;
  const int bhs = blockIdx.x / a.n_chunks;
  const int bh = bhs / a.n_sets, set = bhs % a.n_sets;
  const int N = a.N;
  const size_t base = (size_t)bh * N * D;
  const E* Qp = (const E*)a.Q + base;
  const E* Kp = (const E*)a.K + base;
  const E* Vp = (const E*)a.V + base;

  // The global list of this batch element (sets past its end have no rows).
  const int2 gs = a.gsel[bh / a.H];
  const int* gl = a.glob + gs.x;
  const int gfirst = set * ROWS + kWaveRows * wave;  // first global slot of this wave
  const bool wave_live = gfirst < gs.y;
  const int gslot = gfirst + (lane & 31);
  const int qrow = gslot < gs.y ? gl[gslot] : -1;

  WaveAttn<D> st;
  st.load_q(Qp, qrow, hi);

  const int c0 = chunk * a.chunk_keys;
  const int c1 = min(N, c0 + a.chunk_keys);
  const int n_tiles = (c1 - c0 + TK - 1) / TK;
  auto row_of_tile = [&](int tt) {
    return [=](int kk) -> int {
      const int j = c0 + TK * tt + kk;
      return j < c1 ? j : -1;
    };
  };

  Loader<D, NT> ld;
  ld.fetch(Kp, Vp, row_of_tile(0), tid);
  for (int tt = 0; tt < n_tiles; ++tt) {
    ld.store(tile, tid);
    __syncthreads();
    if (tt + 1 < n_tiles) ld.fetch(Kp, Vp, row_of_tile(tt + 1), tid);
    if (wave_live) {
      f32x16 s[2];
      st.scores(tile, lane, s);
      const int j0 = c0 + TK * tt;
      if (j0 + TK > c1) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (j0 + 32 * kb + block_row(i, hi) >= c1) s[kb][i] = -INFINITY;
      }
      softmax_accumulate(st, tile, lane, s, a.sl2);
    }
    __syncthreads();
  }

  // Partial record of this wave's 32 rows for this chunk.
  float* part = a.part + ((size_t)bhs * a.n_chunks + chunk) * ROWS * REC;
  if (wave_live) {
    const float lt = pair_sum(st.l);
    float* rec = part + (size_t)(kWaveRows * wave + (lane & 31)) * REC;
    if (hi == 0) {
      rec[0] = st.m;
      rec[1] = lt;
    }
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(float4*)(rec + 4 + 32 * b + 8 * g + 4 * hi) =
            make_float4(st.acc[b][4 * g], st.acc[b][4 * g + 1], st.acc[b][4 * g + 2],
                        st.acc[b][4 * g + 3]);
  }
}

// Merge of the global-row partials: one workgroup per (batch-head, global
// row) of NG groups of 16 threads; thread (g, q) combines chunks g, g + NG,
// ... for columns 4q .. 4q+3 (D = 64: 16 column quads; D = 128: each thread
// takes two quads), then the NG chunk groups are combined through LDS.  Every
// chunk record is loaded once: the first 16 chunks in one round (16 / NG per
// thread), later ones two per thread at a time.  The records' base and
// geometry, the per-batch list extents and the lists come ahead of the
// argument block as scalars the build preloads into SGPRs (per_b: workgroups
// per batch element), so that the record loads, the list-extent load and the
// row-position load go out before any argument load returns (a slot past the
// end of its batch element's list reads records that exist but hold nothing,
// and stores none).
template <bool BF16, int D, int NG>
__global__ __launch_bounds__(NG * 16) void glob_merge_kernel(const float* __restrict__ part,
                                                         const int2* __restrict__ gsel,
                                                         const int* glob, int n_glob, int rows,
                                                         int n_sets, int n_chunks, int per_b,
                                                         GlobArgs a) {
  typedef typename ElemT<BF16>::type E;
  constexpr int REC = D + 4;
  constexpr int NQ = D / 4;          // column quads
  constexpr int QPT = NQ / 16;       // quads per thread
  // NG chunk groups of 16 threads; the first round loads FIRST chunks per
  // thread (16 chunks over the groups).
  constexpr int FIRST = 16 / NG;
  static_assert(NG * FIRST == 16, "chunk groups");
  __shared__ float sm_m[NG][16], sm_l[NG][16];
  __shared__ float4 sm_a[NG][NQ];
  const int slot = blockIdx.x % n_glob;
  const int bh = blockIdx.x / n_glob;
  const int q0 = threadIdx.x & 15, g = threadIdx.x >> 4;
  const int set = slot / rows, rr = slot % rows;
  const float* part0 = part + ((size_t)(bh * n_sets + set) * n_chunks * rows + rr) * REC;
  const size_t cs = (size_t)rows * REC;
  float m = kNegInit, l = 0.0f;
  float4 acc[QPT];
#pragma unroll
  for (int t = 0; t < QPT; ++t) acc[t] = make_float4(0.f, 0.f, 0.f, 0.f);
  auto combine = [&](const float2 ml, const float4* v) {
    const float mn = fmaxf(m, ml.x);
    const float a0 = fast_exp2(m - mn), a1 = fast_exp2(ml.x - mn);
    l = l * a0 + ml.y * a1;
#pragma unroll
    for (int t = 0; t < QPT; ++t) {
      acc[t].x = acc[t].x * a0 + v[t].x * a1;
      acc[t].y = acc[t].y * a0 + v[t].y * a1;
      acc[t].z = acc[t].z * a0 + v[t].z * a1;
      acc[t].w = acc[t].w * a0 + v[t].w * a1;
    }
    m = mn;
  };
  // The first chunks of this thread's group, g + NG f for f < FIRST (clamped:
  // a chunk past the last loads the last record and combines an empty state
  // instead), then the batch element's list extent, taken before anything is
  // combined so that its load is in flight with the records'.
  int2 gs;
  int orow;
  {
    float2 ml0[FIRST];
    float4 v0[FIRST][QPT];
#pragma unroll
    for (int f = 0; f < FIRST; ++f) {
      const float* r0 = part0 + (size_t)min(g + NG * f, n_chunks - 1) * cs;
      ml0[f] = *(const float2*)r0;
#pragma unroll
      for (int t = 0; t < QPT; ++t) v0[f][t] = *(const float4*)(r0 + 4 + 4 * (q0 + 16 * t));
    }
    gs = gsel[blockIdx.x / per_b];
    // (The output arguments are taken here too, so that their loads go out
    // with this one instead of after the combine.)
    asm volatile("" ::"s"(gs.x), "s"(gs.y), "s"(a.O), "s"(a.lse), "s"(a.N) : "memory");
    // The row's position, its load issued now (an index clamped into the
    // list for a slot past its end, whose value is not used).
    orow = glob[gs.y > 0 ? gs.x + min(slot, gs.y - 1) : 0];
    asm volatile("" ::: "memory");
#pragma unroll
    for (int f = 0; f < FIRST; ++f) {
      // (An empty state, maximum kNegInit and no weight, leaves (m, l, acc)
      // as they are.)
      const bool have = g + NG * f < n_chunks;
      ml0[f] = have ? ml0[f] : make_float2(kNegInit, 0.0f);
#pragma unroll
      for (int t = 0; t < QPT; ++t)
        v0[f][t] = have ? v0[f][t] : make_float4(0.f, 0.f, 0.f, 0.f);
      combine(ml0[f], v0[f]);
    }
  }
  for (int c = g + 16; c < n_chunks; c += 2 * NG) {
    // Chunks c and c + NG (the second when there is one), both loaded
    // before either is combined.
    const bool two = c + NG < n_chunks;
    const float* r0 = part0 + (size_t)c * cs;
    const float2 ml0 = *(const float2*)r0;
    float4 v0[QPT], v1[QPT];
    float2 ml1 = make_float2(0.f, 0.f);
#pragma unroll
    for (int t = 0; t < QPT; ++t) v0[t] = *(const float4*)(r0 + 4 + 4 * (q0 + 16 * t));
    if (two) {
      const float* r1 = r0 + (size_t)NG * cs;
      ml1 = *(const float2*)r1;
#pragma unroll
      for (int t = 0; t < QPT; ++t) v1[t] = *(const float4*)(r1 + 4 + 4 * (q0 + 16 * t));
    }
    combine(ml0, v0);
    if (two) combine(ml1, v1);
  }
  // Slots past the end of this batch element's global list have no row.
  if (slot >= gs.y) return;
  sm_m[g][q0] = m;
  sm_l[g][q0] = l;
#pragma unroll
  for (int t = 0; t < QPT; ++t) sm_a[g][q0 + 16 * t] = acc[t];
  __syncthreads();
  if (g != 0) return;
  float mt = kNegInit;
#pragma unroll
  for (int x = 0; x < NG; ++x) mt = fmaxf(mt, sm_m[x][q0]);
  float lt = 0.0f;
  float4 at[QPT];
#pragma unroll
  for (int t = 0; t < QPT; ++t) at[t] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int x = 0; x < NG; ++x) {
    const float wgt = fast_exp2(sm_m[x][q0] - mt);
    lt += sm_l[x][q0] * wgt;
#pragma unroll
    for (int t = 0; t < QPT; ++t) {
      const float4 v = sm_a[x][q0 + 16 * t];
      at[t].x += v.x * wgt;
      at[t].y += v.y * wgt;
      at[t].z += v.z * wgt;
      at[t].w += v.w * wgt;
    }
  }
  const float inv = 1.0f / lt;
  if (a.lse && q0 == 0)
    a.lse[(size_t)bh * a.N + orow] = (mt + __log2f(lt)) * 0.6931471805599453f;
  E* Orow = (E*)a.O + (size_t)bh * a.N * D + (size_t)orow * D;
#pragma unroll
  for (int t = 0; t < QPT; ++t) {
    E* Op = Orow + 4 * (q0 + 16 * t);
    if constexpr (BF16) {
      bf16x4 o;
      o[0] = (__bf16)(at[t].x * inv); o[1] = (__bf16)(at[t].y * inv);
      o[2] = (__bf16)(at[t].z * inv); o[3] = (__bf16)(at[t].w * inv);
      *(bf16x4*)Op = o;
    } else {
      *(float4*)Op = make_float4(at[t].x * inv, at[t].y * inv, at[t].z * inv, at[t].w * inv);
    }
  }
}

}  // namespace

hipError_t launch_band(int dtype, int D, const BandArgs& a, int n_wg, hipStream_t s, const Timing& t) {
  if (n_wg <= 0) return hipSuccess;
  if (dtype == 1) return launch_band_bf16(D, a, n_wg, s, t);
  const dim3 grid(n_wg), block(kBandWaves * 64);
  if (dtype == 0 && D == 64) return launch_kernel(band_kernel<64>, grid, block, s, a, t);
  if (dtype == 0 && D == 128) return launch_kernel(band_kernel<128>, grid, block, s, a, t);
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t launch_glob_f32(int waves, const GlobArgs& a, int n_wg, hipStream_t s, const Timing& t) {
  const dim3 grid(n_wg);
  if (waves == 1) return launch_kernel(glob_kernel<D, 1>, grid, dim3(64), s, a, t);
  if (waves == 2) return launch_kernel(glob_kernel<D, 2>, grid, dim3(128), s, a, t);
  if (waves == 4) return launch_kernel(glob_kernel<D, 4>, grid, dim3(256), s, a, t);
  return hipErrorInvalidValue;
}

hipError_t launch_glob(int dtype, int D, int waves, const GlobArgs& a, int n_wg, hipStream_t s,
                       const Timing& t) {
  if (n_wg <= 0) return hipSuccess;
  // (bf16: the band launch takes the global rows; no separate kernel.)
  if (dtype == 0 && D == 64) return launch_glob_f32<64>(waves, a, n_wg, s, t);
  if (dtype == 0 && D == 128) return launch_glob_f32<128>(waves, a, n_wg, s, t);
  return hipErrorInvalidValue;
}

hipError_t launch_glob_merge(int dtype, int D, const GlobArgs& a, hipStream_t s, const Timing& t) {
  const long long n_wg = (long long)a.n_bh * a.n_glob;
  if (n_wg <= 0) return hipSuccess;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)n_wg);
  // Sets of at most 16 chunks: one wavefront per row (4 chunk groups, each
  // loading its 4 chunks at once); more: 16 groups.
  const bool small = a.n_chunks <= 16;
  const dim3 blk(small ? 64 : 256);
  void (*k)(const float*, const int2*, const int*, int, int, int, int, int, GlobArgs) = nullptr;
  if (dtype == 1 && D == 64) k = small ? glob_merge_kernel<true, 64, 4> : glob_merge_kernel<true, 64, 16>;
  if (dtype == 1 && D == 128) k = small ? glob_merge_kernel<true, 128, 4> : glob_merge_kernel<true, 128, 16>;
  if (dtype == 0 && D == 64) k = small ? glob_merge_kernel<false, 64, 4> : glob_merge_kernel<false, 64, 16>;
  if (dtype == 0 && D == 128) k = small ? glob_merge_kernel<false, 128, 4> : glob_merge_kernel<false, 128, 16>;
  if (!k || a.n_glob <= 0 || a.rows_per_set <= 0 || a.n_sets <= 0 || a.n_chunks <= 0)
    return hipErrorInvalidValue;
  if ((long long)a.n_glob * a.H > 0x7fffffffLL) return hipErrorInvalidValue;
  const float* part = a.part;
  const int2* gsel = a.gsel;
  const int* glob = a.glob;
  int n_glob = a.n_glob, rows = a.rows_per_set, n_sets = a.n_sets, n_chunks = a.n_chunks;
  int per_b = a.n_glob * a.H;
  void* args[] = {const_cast<float**>(&part), const_cast<int2**>(&gsel),
                  const_cast<int**>(&glob), &n_glob, &rows, &n_sets, &n_chunks, &per_b,
                  const_cast<GlobArgs*>(&a)};
  return hipExtLaunchKernel(reinterpret_cast<const void*>(k), grid, blk, args, 0, s, t.start,
                            t.stop, 0);
}

}  // namespace lfattn

// bf16 band kernel for gfx950 (MI355X): band32_kernel<D, KS, CHUNK>, D = 64 or 128.
//
// A workgroup of 4 wavefronts takes 32*4/KS consecutive query rows of one
// (batch, head, dilation residue) and walks the 32-key tiles of their band,
// then the tiles of gathered global keys.  Each wavefront owns one block of
// 32 rows (one 32x32 MFMA column block).  With KS = 2 the tile list is split
// between two wavefront pairs (even and odd tiles) and the two partial
// softmax states of a row are merged through LDS at the end, which keeps
// twice as many wavefronts busy on short sequences; with KS = 1 four row
// blocks share one tile stream.  The same launch also takes the global rows:
// items that run the same code over a chunk of plain key positions with Q
// gathered from the global positions and write partial softmax records.
//
// Memory path: the K and V tiles of a step go global -> LDS with direct loads
// (global_load_lds_dwordx4) into a two-stage ring; nothing is staged in
// registers.  Rows are 16-byte-chunk swizzled so that the MFMA operand reads
// of consecutive rows hit distinct LDS banks.  V stays row-major: the A
// operand of O^T += V^T P^T is read with ds_read_b64_tr_b16, whose lane
// transpose delivers the 8 keys of one value column that a lane feeds to a
// 32x32x16 k-step.  The global positions (and their place in the residue's
// subsequence) are staged in LDS once, so issuing a global tile never waits
// on a plain global load.
//
// Per tile and wavefront: S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys on
// the MFMA rows, queries across lanes, so a lane holds 16 keys of one query);
// weights exp2(s*scale*log2e - m) against the running maximum m; P rounded to
// bf16 is already the B operand of the P.V MFMA, and its row sum is taken
// with v_dot2_f32_bf16 on the packed pairs (the same rounded weights as the
// numerator).  The first scored tile sets the maximum; after that it is not
// computed in the common case: a tile whose weights sum past 2^8 on any lane
// is redone against its true maximum, rescaling the accumulators.  That is
// exact because softmax ignores a constant added to all its inputs
// (Unlimiformer, section 2.3, footnote 3).  Tiles that no row of the wave
// may score are skipped; only tiles cut by a band edge evaluate the band
// predicate.
//
// The math is Eq. (1) of the Unlimiformer page (section 2.3) over the pattern
// of the Ultralytics glossary page "Longformer" (section on how the attention
// works): band |i-j| <= window//2 (dilated: j = i + d*k), global rows and
// columns, a global key inside a row's band counted once.
#include <type_traits>

#include "lfattn_internal.h"

namespace lfattn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
#define LDS_AS __attribute__((address_space(3)))

constexpr float kNegInit = -1.0e30f;
constexpr float kSumLimit = 256.0f;
constexpr int kNotInClass = 0x40000000;

// s_waitcnt with vmcnt = VM and lgkmcnt = 0 (gfx9-family encoding:
// vmcnt[3:0] in bits 3:0, expcnt in 6:4, lgkmcnt in 11:8, vmcnt[5:4] in 15:14).
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(VM >= 0 && VM < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | ((VM >> 4) << 14));
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ds_read_b64_tr_b16 at lds_addr + OFF issued as inline assembly.  The
// compiler's builtin for it
// is treated as possibly aliasing the in-flight direct-to-LDS loads and gets a
// full vmcnt(0) wait in front of it, which would drain the load ring; the
// ring's own waits already order these reads.  The result must not be used
// before lgkm_wait() has been passed the same registers.
template <unsigned OFF>
__device__ __forceinline__ s16x4 ds_read_tr16(unsigned lds_addr) {
  s16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(lds_addr), "n"(OFF));
  return r;
}
// 16-byte LDS read at lds_addr + OFF, the same way (the result must pass
// lgkm_wait_n() before use).
template <unsigned OFF>
__device__ __forceinline__ bf16x8 ds_read_b128(unsigned lds_addr) {
  bf16x8 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(lds_addr), "n"(OFF));
  return r;
}
// Wait until at most N LDS reads are outstanding, with x (the result of the
// read issued N before the last one) ready afterwards.  LDS reads complete
// in order; scalar loads in flight only make the wait longer.
template <int N>
__device__ __forceinline__ void lgkm_wait_n(bf16x8& x) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "n"(N));
}
__device__ __forceinline__ void lgkm_wait(s16x4& a0, s16x4& a1, s16x4& a2, s16x4& a3,
                                          s16x4& a4, s16x4& a5, s16x4& a6, s16x4& a7) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7));
}

// The lane's index in the wavefront, computed afresh where it is called (the
// compiler cannot merge it with another call), so that lane-derived values
// used only on rare paths are recomputed there instead of being kept live in
// registers across the step loop.
__device__ __forceinline__ int lane_id() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Partial records of the global rows are exchanged between workgroups that
// may run on different XCDs (whose L2 caches are not coherent with each
// other): they are written and read with agent-scope atomic accesses
// (coherent at the device level without flushing the whole L2), 8 bytes at a
// time.
__device__ __forceinline__ void store_agent(float* p, float x, float y) {
  const unsigned long long v =
      (unsigned long long)__float_as_uint(x) | ((unsigned long long)__float_as_uint(y) << 32);
  __hip_atomic_store((unsigned long long*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_agent(const float* p) {
  const unsigned long long v = __hip_atomic_load((const unsigned long long*)p, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((unsigned)v), __uint_as_float((unsigned)(v >> 32)));
}

// Key of register i (0..15) of a 32x32 MFMA result block for lane half hi.
__device__ __forceinline__ constexpr int block_row(int i, int hi) {
  return 8 * (i >> 2) + 4 * hi + (i & 3);
}

constexpr int kGlobCap = kMaxGlobalBf16;  // global positions staged in LDS

// 16-byte direct global -> LDS loads: lane i's 16 bytes land at LDS byte
// address M0 + 16*i.  Written as inline assembly so that the compiler does
// not treat every later LDS read as depending on them (which made it drain
// all outstanding loads before the transposed reads); the ring's explicit
// waits order the accesses.  (M0 is written here only: nothing else in these
// kernels uses it.)
//
// dma16_s: from a wave-uniform base address plus a 32-bit per-lane offset.
__device__ __forceinline__ void dma16_s(const void* sbase, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(sbase)
               : "memory", "m0");
}
// dma16_2: from a per-lane 64-bit address, with the LDS address given as a
// sum of two wave-uniform parts (one scalar add into M0).
__device__ __forceinline__ void dma16_2(const void* gaddr, unsigned lds_a, unsigned lds_b) {
  asm volatile("s_add_u32 m0, %0, %1\n\tglobal_load_lds_dwordx4 %2, off"
               :
               : "s"(lds_a), "s"(lds_b), "v"(gaddr)
               : "memory", "m0", "scc");
}


// ---------------------------------------------------------------------------
// bf16 band kernel with 32-key steps (band32_kernel<D>, D = 64 or 128).
//
// A workgroup of 4 wavefronts takes 64 consecutive rows of one (batch, head,
// dilation residue): wavefronts 0,1 own rows 0-31 and 32-63 over the first
// half of the workgroup's 32-key tiles, wavefronts 2,3 the same rows over the
// second half (partial softmax states merged through LDS at the end).  Each
// wavefront's state is one 32x32 MFMA block.  D = 64: a wavefront fits in
// 128 registers and four workgroups (a 2-stage ring of 32-key K/V tiles, 36
// KB of LDS each) share a compute unit, four wavefronts per SIMD hiding each
// other's latencies; D = 128: 256 registers, 68 KB, two per compute unit.
// Per step and wavefront: S^T = K Q^T (D/16 MFMAs), mask where a band edge
// or global dedupe cuts the tile, weights with the lazy rescale,
// O^T += V^T P^T (D/16 MFMAs).
// ---------------------------------------------------------------------------
template <int D, int KS_>
struct B32 {
  static constexpr int TK = 32;          // keys per step
  static constexpr int RB = 2 * D;       // bytes per key row
  static constexpr int CPR = RB / 16;    // 16-byte chunks per row
  static constexpr int RPI = 1024 / RB;  // rows one wave-wide direct load fills
  static constexpr int MAT = TK * RB;    // bytes of one K (or V) tile
  static constexpr int KS = KS_, NS = 2;  // key halves, ring stages
  static constexpr int QBLKS = 4 / KS;   // 32-row query blocks per workgroup
  static constexpr int ROWS = 32 * QBLKS;  // rows per workgroup
  static constexpr int RPW = TK / QBLKS;   // tile rows each wavefront loads
  static constexpr int NE = RPW / RPI;   // loads per matrix and wavefront per step
  // Wavefronts per SIMD: D = 64 fits 128 registers (4); D = 128 fits 168
  // (3) with the 36 KB ring of one key split, 256 (2) with two.
  static constexpr int WPE = D == 64 ? 4 : (KS_ == 1 ? 3 : 2);
  // Physical 16-byte chunk of logical chunk c in row `row` (an involution),
  // chosen for 64 LDS banks (256 bytes per cycle): a K-operand read (chunk c
  // of 32 consecutive rows) is served 16 lanes = 16 rows at a time, a
  // transposed V read 32 lanes = 4 consecutive rows x 4 adjacent chunks at a
  // time.  D = 64 (two rows per 256 bytes): the XOR term is a bijection of
  // row/2 and moves the 4-chunk block of row pairs 2 apart; D = 128: a
  // bijection of the row whose block bits differ over any 4 consecutive rows.
  // Neither read then repeats a bank.
  static __device__ __forceinline__ int swz(int row, int c) {
    if constexpr (D == 64) {
      const int j = (row >> 1) & 7;
      return c ^ (((j & 1) << 2) | ((j >> 1) & 3));
    } else {
      return c ^ (((row & 3) << 2) | ((row >> 2) & 3));
    }
  }
};

// Global-row items of D = 64 launches run in the key-split layout (two
// 32-row blocks of global rows, even and odd tiles on two wavefront pairs),
// whatever the launch's band layout: all four wavefronts score.
template <int D, int KS>
constexpr int global_ks() { return D == 64 ? 2 : KS; }

// LDS of one band workgroup: the tile ring (sized for the wider of the
// launch's band and global-row layouts), the staged global positions, the
// band rows that are global positions, and a flag.
template <int D, int KS>
struct BandSmem {
  static constexpr int KSMAX = KS > global_ks<D, KS>() ? KS : global_ks<D, KS>();
  unsigned char st[B32<D, KS>::NS * KSMAX * 2 * B32<D, KS>::MAT];
  int gpos[kGlobCap];
  int gsp[kGlobCap];
  unsigned char rowg[128];   // band rows that are global positions
  int last;                  // global-row item: this workgroup merges the set
};

// The merge of one set of global rows (slots ROWS*set .. of the batch
// element's list) from its n_chunks (at most kFuseChunks) partial records:
// each thread takes one row and 8 output columns, loads that row's records in
// rounds of 4 chunks of independent loads, combines the chunks' (max, sum,
// acc) with the log-sum-exp rule, and writes 16 bytes of the row (bf16) and,
// where asked, its log-sum-exp.
template <int D, int ROWS>
__device__ __forceinline__ void merge_global_set(const BandArgs& a, const BandWork& w,
                                                 const float* set_part, int tid) {
  constexpr int TPR = D / 8;          // threads per row
  constexpr int RPP = 256 / TPR;      // rows per pass
  constexpr int REC = D + 4;
  constexpr int CB = 4;               // chunks loaded per round
  const int n_rows = min(ROWS, w.ng - ROWS * w.r);
  const int cg = tid % TPR;
  const int* gl = a.glob + w.g0;
  for (int r = tid / TPR; r < n_rows; r += RPP) {
    float m = kNegInit, l = 0.0f;
    float o[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) o[x] = 0.0f;
    for (int c0 = 0; c0 < a.n_chunks; c0 += CB) {
      float2 ml[CB], v[CB][4];
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        const int c = min(c0 + u, a.n_chunks - 1);
        const float* rec = set_part + ((size_t)c * ROWS + r) * REC;
        ml[u] = load_agent(rec);
#pragma unroll
        for (int x = 0; x < 4; ++x) v[u][x] = load_agent(rec + 4 + 8 * cg + 2 * x);
      }
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        if (c0 + u >= a.n_chunks) break;
        const float mn = fmaxf(m, ml[u].x);
        const float a0 = fast_exp2(m - mn), a1 = fast_exp2(ml[u].x - mn);
        l = l * a0 + ml[u].y * a1;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          o[2 * x] = o[2 * x] * a0 + v[u][x].x * a1;
          o[2 * x + 1] = o[2 * x + 1] * a0 + v[u][x].y * a1;
        }
        m = mn;
      }
    }
    const int orow = gl[ROWS * w.r + r];
    if (a.lse && cg == 0) a.lse[(size_t)w.bh * a.N + orow] = (m + __log2f(l)) * 0.6931471805599453f;
    const float inv = 1.0f / l;
    bf16x8 ob;
#pragma unroll
    for (int x = 0; x < 8; ++x) ob[x] = (__bf16)(o[x] * inv);
    *(bf16x8*)((unsigned short*)a.O + (size_t)w.bh * a.N * D + (size_t)orow * D + 8 * cg) = ob;
  }
}

// One work item of the band launch in the layout KS_ (a band item, or a
// global-row item when w.dil == 0).  CHUNK: GMAT chunked attention
// (a.chunk > 0) instead of a band; a separate instantiation, so that the band
// kernels carry none of its arithmetic.
template <int D, int KS_, bool CHUNK, class SM>
__device__ __forceinline__ void band_item(const BandArgs& a, const BandWork& w, SM& sm) {
  using C = B32<D, KS_>;
  constexpr int TK = C::TK, RB = C::RB, CPR = C::CPR, RPI = C::RPI, MAT = C::MAT;
  constexpr int NE = C::NE, KS = C::KS, NS = C::NS, ROWS = C::ROWS, QBLKS = C::QBLKS;
  constexpr int RPW = C::RPW;
  static_assert(QBLKS * NE * RPI == TK, "the wavefronts of a key half load its 32-row tiles");
  static_assert(sizeof(sm.st) >= (size_t)NS * KS * 2 * MAT, "tile ring");
  auto swz = [](int row, int c) { return C::swz(row, c); };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hi = lane >> 5, l32 = lane & 31;
  const int qblk = wave % QBLKS, kh = wave / QBLKS;
  // A global-row item is the band problem over plain key positions (d = 1),
  // with a half-width no key reaches past and its rows taken from the global
  // list, restricted to one key chunk.
  const bool gi = w.dil == 0;
  const int d = gi ? 1 : w.dil;
  const int r = gi ? 0 : w.r, t0 = gi ? 0 : w.t0, N = a.N;
  // A row u scores the keys u - hl .. u + hr of its subsequence (hl = hr =
  // the half-width; causal: hr = 0).
  const int hl = gi ? (1 << 29) : a.hw;
  const int hr = gi ? (1 << 29) : a.hr;
  // Chunked attention (band items, d = 1): row u scores its chunk instead,
  // positions c0 .. c0 + C - 1 with c0 = cb + C * floor((u - cb) / C); rows
  // before cb are the memory (global rows, whose band output is not kept).
  const int cC = (!CHUNK || gi) ? 0 : a.chunk, cb = a.cbase;
  auto lo_of = [&](int uu) -> int {
    return cC == 0 ? uu - hl : (uu < cb ? uu : cb + (uu - cb) / cC * cC);
  };
  auto hi_of = [&](int uu) -> int {
    return cC == 0 ? uu + hr : (uu < cb ? uu : cb + (uu - cb) / cC * cC + cC - 1);
  };
  const int Lr = d == 1 ? N - r : (N - r + d - 1) / d;
  const size_t base = (size_t)w.bh * N * D;
  // A global-row item reads the global rows' own projections.
  const unsigned short* Qp = (const unsigned short*)(gi ? a.Qg : a.Q) + base;
  const unsigned short* Kp = (const unsigned short*)(gi ? a.Kg : a.K) + base;
  const unsigned short* Vp = (const unsigned short*)(gi ? a.Vg : a.V) + base;
  // The global list of this item's batch element.
  const int* gl = a.glob + w.g0;
  const int n_glob = w.ng;

  // Global positions this thread stages (loaded first so that their latency
  // overlaps the Q loads and the first tile loads).
  constexpr int kStageIters = (kGlobCap + 255) / 256;
  int gv[kStageIters];
#pragma unroll
  for (int it = 0; it < kStageIters; ++it) {
    const int x = tid + 256 * it;
    gv[it] = x < n_glob ? gl[x] : 0;
  }

  // This wave's rows: subsequence positions ua .. ub (one per lane % 32); for
  // a global-row item, slots of the global list, and keys s_lo .. s_hi.
  const int n_rows = gi ? n_glob : Lr;
  const int ua = (gi ? ROWS * w.r : t0) + 32 * qblk;
  const int ub = min(ua + 31, n_rows - 1);
  const bool live = ua < n_rows;
  const int s_lo = gi ? w.t0 * a.chunk_keys : max(0, lo_of(t0));
  const int s_hi = gi ? min(N, s_lo + a.chunk_keys) - 1 : min(Lr - 1, hi_of(t0 + ROWS - 1));
  // Keys of this wave's first and last rows (both ends are non-decreasing in
  // the row): a tile reaches some row when k0 <= hi_b and k1 >= lo_a, and
  // every row wholly when k0 >= lo_b and k1 <= hi_a.
  const int lo_a = lo_of(ua), hi_a = hi_of(ua), lo_b = lo_of(ub), hi_b = hi_of(ub);
  const int u = ua + l32;
  const bool row_ok = u < n_rows;

  // Whether the lane's band row is itself a global position (its output is
  // the merge kernel's), read now (a plain load, waited for with the others)
  // so that the epilogue finds it in LDS.  Meaningless for global-row items.
  const unsigned char own_glob =
      a.is_glob[w.b * a.isg_stride + min(r + d * (row_ok ? u : 0), N - 1)];

  // Q operand (B of S^T = K Q^T): Q[row][16ks + 8hi + 0..7].
  bf16x8 q[D / 16];
  {
    const size_t row =
        gi ? (size_t)(row_ok ? gl[u] : 0) : (size_t)(r + d * (row_ok ? u : 0));
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      q[ks] = *(const bf16x8*)(Qp + row * D + 16 * ks + 8 * hi);
      if (!row_ok) q[ks] = bf16x8{};
    }
  }
  // A key at position k is in the band of the lane's row u when
  // -hl <= k - u <= hr and k <= s_hi (keys below 0 never occur: tiles start at
  // s_lo >= 0).  Rows past the end are never stored, so they need no mask.

  const int n_band = (s_hi - s_lo) / TK + 1;
  const int n_tiles = n_band + (gi ? 0 : (n_glob + TK - 1) / TK);
  const int n_steps = (n_tiles + KS - 1) / KS;  // half kh takes tiles KS*j + kh

  // Direct loads of step j into the stage at byte offset soff: the wavefronts
  // of a key half load that half's K and V tiles, wavefront w rows
  // RPW*qblk + RPI*e + lane/CPR (e < NE): 2*NE loads each (tiles past the end
  // load a real row so that every wavefront issues the same count).
  const int rbase = RPW * qblk;
  const unsigned st_base = (unsigned)(uintptr_t)(LDS_AS void*)(sm.st + kh * 2 * MAT);
  constexpr unsigned kStageBytes = KS * 2 * MAT;
  const int rlane = rbase + lane / CPR;
  // LDS destination of load e of K within a stage (V: + MAT).
  const unsigned ld_k = st_base + rbase * RB;
  // Byte offset of this lane's 16 bytes of row rlane + RPI*e of a band tile
  // from the tile's first key row (rows d apart in memory).
  unsigned boff[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e)
    boff[e] = (unsigned)(d * (rlane + RPI * e) * RB) + 16u * swz(rlane + RPI * e, lane % CPR);
  // Tile of step j.  KS = 2: tile KS*j + kh.  KS = 1: the band tiles in a
  // rotated order, chosen so that the workgroups of one (head, residue) read
  // tiles whose index from the sequence start is congruent mod n_band at the
  // same step: the workgroups that share a tile (their bands overlap) read it
  // at nearly the same time, and a tile stays in L2 only briefly.  Then the
  // gathered global tiles.
  const int rot = KS == 1 ? (n_band - (s_lo / TK) % n_band) % n_band : 0;
  auto tile_of = [&](int j) -> int {
    if constexpr (KS == 1) {
      if (j >= n_band) return j;
      const int t = j + rot;
      return t >= n_band ? t - n_band : t;
    } else {
      return KS * j + kh;
    }
  };
  // First key row of band tile t: Kp/Vp + kt0 + t*tstep elements.
  const size_t kt0 = (size_t)(r + d * s_lo) * D;
  const size_t tstep = (size_t)d * TK * D;
  // Loads of a band tile that lies wholly in the key range, from its first
  // K and V rows.
  auto issue_band = [&](const unsigned short* kb, const unsigned short* vb, unsigned soff) {
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      dma16_s(kb, boff[e], ld_k + 1024 * e + soff);
      dma16_s(vb, boff[e], ld_k + MAT + 1024 * e + soff);
    }
  };
  // Loads of any tile of step j: gathered global keys, or band rows clamped
  // to s_hi (the last band tile, or a tile past the end).
  auto issue = [&](int j, unsigned soff) {
    const int tj = tile_of(j);
    const bool glob_tile = tj >= n_band && tj < n_tiles;
    if (!glob_tile && s_lo + TK * tj + TK - 1 <= s_hi) {
      const size_t row0 = kt0 + (size_t)tj * tstep;
      issue_band(Kp + row0, Vp + row0, soff);
      return;
    }
    const int ln = lane_id(), rl = rbase + ln / CPR;
    int g[NE];
    if (glob_tile) {
      const int x0 = TK * (tj - n_band);
#pragma unroll
      for (int e = 0; e < NE; ++e) g[e] = sm.gpos[min(x0 + rl + RPI * e, n_glob - 1)];
    } else {
      const int k0 = s_lo + TK * tj;
#pragma unroll
      for (int e = 0; e < NE; ++e) g[e] = r + d * min(k0 + rl + RPI * e, s_hi);
    }
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const size_t off = (size_t)g[e] * D + 8 * swz(rl + RPI * e, ln % CPR);
      dma16_2(Kp + off, ld_k + 1024 * e, soff);
      dma16_2(Vp + off, ld_k + MAT + 1024 * e, soff);
    }
  };

  // The first stage goes out before the global positions are staged unless
  // its tile is a gathered global tile.
  static_assert(NS == 2, "the step loop alternates two stages");
  const bool early = !(tile_of(0) >= n_band && tile_of(0) < n_tiles);
  if (early) issue(0, 0);
#pragma unroll
  for (int it = 0; it < kStageIters; ++it) {
    const int x = tid + 256 * it;
    if (x < n_glob) {
      const int g = gv[it];
      const int off = g - r;
      sm.gpos[x] = g;
      // (d = 1: every position is in the one residue class, r = 0.)
      sm.gsp[x] = d == 1 ? off : ((off >= 0 && off % d == 0) ? off / d : kNotInClass);
    }
  }
  if (!gi && kh == 0 && hi == 0) sm.rowg[32 * qblk + l32] = own_glob;
  __syncthreads();  // staged global positions visible
  if (!early) issue(0, 0);

  // Whether a global key lies in the band of one of this wave's rows (then
  // global tiles need the per-pair dedupe test).
  bool gdup = false;
  if (live) {
    const int lo_w = lo_a;
    const unsigned span_w = (unsigned)(hi_b - lo_a);
    for (int x = lane; x < n_glob; x += 64) gdup |= (unsigned)(sm.gsp[x] - lo_w) <= span_w;
  }
  gdup = __any(gdup);

  f32x16 acc[D / 32];
#pragma unroll
  for (int b = 0; b < D / 32; ++b) acc[b] = f32x16{};
  float m = kNegInit, l = 0.0f;
  bool fresh = true;  // no tile scored yet: maximum unset

  // Per-step flags for steps j0 .. j0+63, one step per lane: act, the wave
  // scores some key of the step's tile; fast, an active band tile that needs
  // no mask and is not the wave's first scored tile (the common case, taken
  // without any of the tests below); nfast, the next step's tile is a band
  // tile wholly in the key range (its loads take the short path).
  unsigned long long act_m = 0, fast_m = 0, nfast_m = 0;
  auto flags = [&](int j0) {
    const int x = j0 + lane_id();
    const int tt = tile_of(x);
    bool fa = false, ff = false;
    if (live && x < n_steps && tt < n_tiles) {
      if (tt < n_band) {
        const int k0 = s_lo + TK * tt, k1 = min(k0 + TK - 1, s_hi);
        fa = (k0 <= hi_b) & (k1 >= lo_a);
        ff = fa & (k1 == k0 + TK - 1) & (k1 <= hi_a) & (k0 >= lo_b);
      } else {
        fa = true;
      }
    }
    act_m = __ballot(fa);
    fast_m = __ballot(ff);
    if (fresh) fast_m &= ~(act_m & (0 - act_m));  // the first scored tile
    const int tn = tile_of(x + 1);
    nfast_m = __ballot(tn < n_band && s_lo + TK * tn + TK - 1 <= s_hi);
  };

  // Per-lane LDS addresses of the MFMA operands in stage 0 (stage 1: plus
  // kStageBytes, an immediate offset).
  unsigned koff[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) koff[ks] = st_base + l32 * RB + 16 * swz(l32, 2 * ks + hi);
  unsigned voff[D / 32][2];
  {
    const int g16 = lane >> 4, t16 = lane & 15;
#pragma unroll
    for (int b = 0; b < D / 32; ++b) {
      const int dcol = 32 * b + 16 * (g16 & 1) + 4 * (t16 & 3);
      const int c = dcol >> 3, half = (dcol >> 2) & 1;
      const int row0 = 4 * (g16 >> 1) + (t16 >> 2), row1 = row0 + 8;
      voff[b][0] = st_base + MAT + row0 * RB + 16 * swz(row0, c) + 8 * half;
      voff[b][1] = st_base + MAT + row1 * RB + 16 * swz(row1, c) + 8 * half;
    }
  }
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // Scoring of step j's tile t = KS*j + kh from the stage at SOFF.  fast: a
  // band tile with no mask, not the first scored one (the tests are skipped).
  auto score = [&](const int j, auto stage, const bool fast) {
    constexpr unsigned SOFF = decltype(stage)::value * kStageBytes;
    const int t = tile_of(j);
    const bool band = t < n_band;

    // Global tiles: which slots the rows keep (with the dedupe test: one
    // bit per register; without: the slots before glim, counted from this
    // lane half's first key).
    bool edge = false;
    unsigned keep = 0;
    int glim = TK;
    if (!fast) {
      if (band) {
        const int k0 = s_lo + TK * t, k1 = min(k0 + TK - 1, s_hi);
        edge = !((k1 == k0 + TK - 1) & (k1 <= hi_a) & (k0 >= lo_b));
      } else {
        bool act;
        const int ln = lane_id(), lh = ln >> 5, lu = ua + (ln & 31);
        const int g0 = TK * (t - n_band);
        const int nvalid = min(TK, n_glob - g0);
        if (!gdup) {
          glim = nvalid - 4 * lh;
          act = true;
          edge = nvalid < TK;
        } else {
          // Keep a valid slot unless its key lies in the row's band (then the
          // band already scored it).  One group of 4 slots at a time, so that
          // this rare path stays small in registers.
          const int lo_u = lo_of(lu);
          const unsigned span = (unsigned)(hi_of(lu) - lo_u);
#pragma unroll 1
          for (int g4 = 0; g4 < 4; ++g4) {
            const int kk0 = 8 * g4 + 4 * lh;
            const i32x4 sp = *(const LDS_AS i32x4*)&sm.gsp[min(g0 + kk0, kGlobCap - 4)];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const bool k = (kk0 + c < nvalid) & (lu < n_rows) & ((unsigned)(sp[c] - lo_u) > span);
              keep |= (unsigned)k << (4 * g4 + c);
            }
          }
          act = __any(keep != 0);
          edge = true;
        }
        if (!act) return;
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // S^T = K Q^T.
    f32x16 S;
    {
      bf16x8 kv[D / 16];
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) kv[ks] = ds_read_b128<SOFF>(koff[ks]);
      S = f32x16{};
      auto kstep1 = [&](auto ksc) {
        constexpr int ks = decltype(ksc)::value;
        lgkm_wait_n<D / 16 - 1 - ks>(kv[ks]);
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv[ks], q[ks], S, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      };
      kstep1(std::integral_constant<int, 0>{});
      kstep1(std::integral_constant<int, 1>{});
      kstep1(std::integral_constant<int, 2>{});
      kstep1(std::integral_constant<int, 3>{});
      if constexpr (D == 128) {
        kstep1(std::integral_constant<int, 4>{});
        kstep1(std::integral_constant<int, 5>{});
        kstep1(std::integral_constant<int, 6>{});
        kstep1(std::integral_constant<int, 7>{});
      }
    }
    if (!fast) {
      if (edge) {
        if (band) {
          const int s0 = s_lo + TK * t;
          const int ln = lane_id(), lh = ln >> 5, lu = ua + (ln & 31);
          // lo(u) <= key <= hi(u)  <=>  0 <= e + br <= hi(u) - lo(u)
          const int lo_u = lo_of(lu);
          const unsigned span = (unsigned)(hi_of(lu) - lo_u);
          const int e = s0 + 4 * lh - lo_u;
          if (s0 + TK - 1 <= s_hi) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
              S[i] = (unsigned)(e + block_row(i, 0)) > span ? -INFINITY : S[i];
          } else {
            const int last = s_hi - s0 - 4 * lh;  // keys past s_hi: block row > last
#pragma unroll
            for (int i = 0; i < 16; ++i)
              S[i] = ((int)((unsigned)(e + block_row(i, 0)) > span) | (int)(block_row(i, 0) > last))
                         ? -INFINITY : S[i];
          }
        } else if (!gdup) {
#pragma unroll
          for (int i = 0; i < 16; ++i) S[i] = block_row(i, 0) < glim ? S[i] : -INFINITY;
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) S[i] = ((keep >> i) & 1u) ? S[i] : -INFINITY;
        }
      }
      if (fresh) {
        // First scored tile: start the running maximum at its own maximum.
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, S[i]);
        m = fmaxf(kNegInit, pair_max(mx) * a.sl2);
        fresh = false;
      }
    }

    __builtin_amdgcn_sched_barrier(0);
    // Weights, packed to bf16 (the B operand of P.V), and their sum.
    unsigned P[8];
    float ls;
    auto weights = [&](float mq) {
      float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        f32x2 pf;
        pf[0] = fast_exp2(fmaf(S[i], a.sl2, -mq));
        pf[1] = fast_exp2(fmaf(S[i + 1], a.sl2, -mq));
        const bf16x2 pb = __builtin_convertvector(pf, bf16x2);
        P[i / 2] = __builtin_bit_cast(unsigned, pb);
        if (i & 2) s1 = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, s1, false);
        else s0 = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, s0, false);
      }
      ls = s0 + s1;
    };
    weights(m);
    if (__builtin_expect(__any(!(ls <= kSumLimit)), 0)) {
      // Move the running maximum up to this tile's maximum and redo.  (The
      // empty volatile statement keeps this rare path a real branch.)
      asm volatile("" ::: "memory");
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, S[i]);
      const float mn = fmaxf(m, pair_max(mx) * a.sl2);
      const float alpha = fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int b = 0; b < D / 32; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[b][i] *= alpha;
      m = mn;
      weights(mn);
    }
    l += ls;
    __builtin_amdgcn_sched_barrier(0);

    // O^T += V^T P^T.  V^T operand for k-step k2 (keys 16k2..16k2+15) and
    // column block b, read transposed: lane L gets keys 16k2 + 4*(L/32) + j
    // (j < 4) and 16k2 + 8 + 4*(L/32) + (j-4) (j >= 4) of column 32b + L%32,
    // the key order of the P^T registers 4*k2 .. 4*k2+3.
    if constexpr (D == 64) {
      s16x4 vr[2][2][2];  // [k2][b][row0/row1]
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        vr[0][b][0] = ds_read_tr16<SOFF>(voff[b][0]);
        vr[0][b][1] = ds_read_tr16<SOFF>(voff[b][1]);
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        vr[1][b][0] = ds_read_tr16<SOFF + 16 * RB>(voff[b][0]);
        vr[1][b][1] = ds_read_tr16<SOFF + 16 * RB>(voff[b][1]);
      }
      lgkm_wait(vr[0][0][0], vr[0][0][1], vr[0][1][0], vr[0][1][1],
                vr[1][0][0], vr[1][0][1], vr[1][1][0], vr[1][1][1]);
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const uint4 pu = make_uint4(P[4 * k2], P[4 * k2 + 1], P[4 * k2 + 2], P[4 * k2 + 3]);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const bf16x8 va = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(vr[k2][b][0], vr[k2][b][1], 0, 1, 2, 3, 4, 5, 6, 7));
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, __builtin_bit_cast(bf16x8, pu),
                                                           acc[b], 0, 0, 0);
        }
      }
    } else {
      // D = 128: one 16-key k-step at a time (fewer live V operands).
      auto pv = [&](auto k2c) {
        constexpr int k2 = decltype(k2c)::value;
        s16x4 vr[4][2];  // [b][row0/row1]
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          vr[b][0] = ds_read_tr16<SOFF + 16 * RB * k2>(voff[b][0]);
          vr[b][1] = ds_read_tr16<SOFF + 16 * RB * k2>(voff[b][1]);
        }
        lgkm_wait(vr[0][0], vr[0][1], vr[1][0], vr[1][1], vr[2][0], vr[2][1], vr[3][0], vr[3][1]);
        const uint4 pu = make_uint4(P[4 * k2], P[4 * k2 + 1], P[4 * k2 + 2], P[4 * k2 + 3]);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const bf16x8 va = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(vr[b][0], vr[b][1], 0, 1, 2, 3, 4, 5, 6, 7));
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, __builtin_bit_cast(bf16x8, pu),
                                                           acc[b], 0, 0, 0);
        }
      };
      pv(std::integral_constant<int, 0>{});
      pv(std::integral_constant<int, 1>{});
    }
  };

  // One step: bit x (= j - j0) of the flags, tile tile_of(j) in stage SG
  // (= j % 2).  This wave's loads of step j done, then every wave's; then the
  // next step's loads into the other stage (after the last step they load
  // real rows nobody reads; the epilogue waits for them before reusing LDS).
  const unsigned short* kn = Kp + kt0 + (size_t)kh * tstep;  // last issued band step (KS = 2)
  const unsigned short* vn = Vp + kt0 + (size_t)kh * tstep;
  auto step = [&](const int j, const int x, auto stage) {
    constexpr int SG = decltype(stage)::value;
    wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
    if constexpr (KS == 1) {
      const size_t row0 = kt0 + (size_t)tile_of(j + 1) * tstep;
      kn = Kp + row0;
      vn = Vp + row0;
    } else {
      kn += KS * tstep;
      vn += KS * tstep;
    }
    if ((nfast_m >> x) & 1)
      issue_band(kn, vn, (1 - SG) * kStageBytes);
    else
      issue(j + 1, (1 - SG) * kStageBytes);
    if ((act_m >> x) & 1) score(j, stage, ((fast_m >> x) & 1) != 0);
  };

  // Steps in pairs (stage 0 then stage 1), flags refreshed every 64 steps.
  // In a launch whose workgroups all run at once, a wavefront's issue
  // priority falls as its steps run out (s_setprio 3 .. 0): the hardware
  // otherwise favours the oldest wavefronts, which finish first and leave the
  // youngest to run on a part-empty compute unit at the end.
  for (int j0 = 0; j0 < n_steps; j0 += 64) {
    flags(j0);
    const int j1 = min(n_steps, j0 + 64);
    for (int j = j0; j < j1; j += 2) {
      if (a.lrf) {
        const int rem = n_steps - j;
        if (rem > 6) __builtin_amdgcn_s_setprio(3);
        else if (rem > 3) __builtin_amdgcn_s_setprio(2);
        else if (rem > 1) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
      }
      step(j, j - j0, std::integral_constant<int, 0>{});
      if (j + 1 < j1) step(j + 1, j + 1 - j0, std::integral_constant<int, 1>{});
    }
  }

  // The loads issued in the last step land before the ring is reused.
  wait_vm_lgkm0<0>();

  // Merge the second key half's state into the first through LDS (the ring
  // is free: every load was waited for in the last step).
  if constexpr (KS == 2) {
    constexpr int PER = 2 + D / 2;
    static_assert((size_t)2 * 64 * PER * 4 <= sizeof(sm.st), "merge area");
    __syncthreads();
    float* mine = (float*)sm.st + ((size_t)qblk * 64 + lane) * PER;
    if (kh == 1 && live) {
      mine[0] = m;
      mine[1] = l;
#pragma unroll
      for (int b = 0; b < D / 32; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) mine[2 + 16 * b + i] = acc[b][i];
    }
    __syncthreads();
    // (Every wave of a global-row item goes on to the arrival count below.)
    if (!gi && (kh == 1 || !live)) return;
    if (kh == 0 && live) {
    const float m1 = mine[0], l1 = mine[1];
    const float mn = fmaxf(m, m1);
    const float a0 = fast_exp2(m - mn), a1 = fast_exp2(m1 - mn);
    l = l * a0 + l1 * a1;
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[b][i] = acc[b][i] * a0 + mine[2 + 16 * b + i] * a1;
    m = mn;
    }
  }

  const float lt = pair_sum(l);
  // Lane-derived values again, from a lane id the compiler cannot fold into
  // the one computed at entry (so that nothing lane-dependent is kept live
  // across the loop only for the stores).
  const int lid = lane_id();
  const int ehi = lid >> 5, el32 = lid & 31;
  const int eu = ua + el32;
  if (gi) {
    // Partial record of this global row for this key chunk (the waves that
    // hold a merged state for live rows).
    float* const set_part = a.part + ((size_t)w.bh * a.n_sets + w.r) * a.n_chunks * ROWS * (D + 4);
    const bool fuse = a.gcount != nullptr;
    if (live && (KS == 1 || kh == 0) && eu < n_rows) {
      float* rec = set_part + ((size_t)w.t0 * ROWS + 32 * qblk + el32) * (D + 4);
      if (fuse) {
        if (ehi == 0) store_agent(rec, m, lt);
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            float* p = rec + 4 + 32 * b + 8 * g4 + 4 * ehi;
            store_agent(p, acc[b][4 * g4], acc[b][4 * g4 + 1]);
            store_agent(p + 2, acc[b][4 * g4 + 2], acc[b][4 * g4 + 3]);
          }
      } else {
        // A separate merge kernel reads these after the launch ends.
        if (ehi == 0) {
          rec[0] = m;
          rec[1] = lt;
        }
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            *(float4*)(rec + 4 + 32 * b + 8 * g4 + 4 * ehi) = make_float4(
                acc[b][4 * g4], acc[b][4 * g4 + 1], acc[b][4 * g4 + 2], acc[b][4 * g4 + 3]);
      }
    }
    if (!fuse) return;
    // Arrival: once every wave's records are complete at the device level,
    // one thread counts this chunk in; the workgroup that brings the count
    // to the number of chunks merges the set's records into O (and resets
    // the count for the next call).
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    wait_vm_lgkm0<0>();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (tid == 0) {
      unsigned* cnt = a.gcount + (size_t)w.bh * a.n_sets + w.r;
      const unsigned before =
          __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = before + 1 == (unsigned)a.n_chunks;
      if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sm.last = last;
    }
    __syncthreads();
    if (!sm.last) return;
    merge_global_set<D, ROWS>(a, w, set_part, tid);
    return;
  }
  if (eu >= n_rows) return;
  const int row = r + d * eu;
  if (sm.rowg[32 * qblk + el32]) return;
  // Natural log-sum-exp of the row's scaled scores (m and the weights are in
  // base 2 of scores times scale * log2(e)).
  if (a.lse && ehi == 0) a.lse[(size_t)w.bh * N + row] = (m + __log2f(lt)) * 0.6931471805599453f;
  const float inv = 1.0f / lt;
  unsigned short* Op = (unsigned short*)a.O + base + (size_t)row * D;
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      bf16x4 o;
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = (__bf16)(acc[b][4 * g4 + c] * inv);
      *(bf16x4*)(Op + 32 * b + 8 * g4 + 4 * ehi) = o;
    }
}

// The band launch: one work item per workgroup.
template <int D, int KS, bool CHUNK>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(B32<D, KS>::WPE, B32<D, KS>::WPE)))
void band32_kernel(const BandWork* __restrict__ work, BandArgs a) {
  __shared__ __attribute__((aligned(16))) BandSmem<D, KS> sm;
  const BandWork w = work[blockIdx.x];
  if constexpr (global_ks<D, KS>() != KS) {
    if (w.dil == 0) {
      band_item<D, global_ks<D, KS>(), CHUNK>(a, w, sm);
      return;
    }
  }
  band_item<D, KS, CHUNK>(a, w, sm);
}

}  // namespace

// Rows per set of the global-row items of a bf16 launch with the given band
// rows per workgroup.
int global_set_rows(int D, int band_rows) { return D == 64 ? 64 : band_rows; }

int band_workgroups_per_cu(int dtype, int D) {
  return dtype == 1 ? (D == 64 ? B32<64, 2>::WPE : B32<128, 2>::WPE) : 2;
}

bool band_takes_global_items(int dtype, int D) { return dtype == 1 && (D == 64 || D == 128); }

hipError_t launch_band_bf16(int D, const BandArgs& a, int n_wg, hipStream_t s, const Timing& t) {
  if (n_wg <= 0) return hipSuccess;
  if (a.n_glob > kGlobCap) return hipErrorInvalidValue;
  const dim3 grid(n_wg), block(256);
  const bool wide = a.rows_per_wg == 128;  // one tile stream for four row blocks
  if (!wide && a.rows_per_wg != 64) return hipErrorInvalidValue;
  if (a.chunk > 0) {
    if (D == 64)
      return launch_kernel(wide ? band32_kernel<64, 1, true> : band32_kernel<64, 2, true>, grid,
                           block, s, a, t);
    if (D == 128)
      return launch_kernel(wide ? band32_kernel<128, 1, true> : band32_kernel<128, 2, true>,
                           grid, block, s, a, t);
    return hipErrorInvalidValue;
  }
  if (D == 64)
    return launch_kernel(wide ? band32_kernel<64, 1, false> : band32_kernel<64, 2, false>, grid,
                         block, s, a, t);
  if (D == 128)
    return launch_kernel(wide ? band32_kernel<128, 1, false> : band32_kernel<128, 2, false>,
                         grid, block, s, a, t);
  return hipErrorInvalidValue;
}

}  // namespace lfattn

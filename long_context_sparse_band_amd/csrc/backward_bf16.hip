// bf16 backward pass for gfx950 (MI355X): dQ, dK, dV of band + global
// attention, D = 64 or 128, for every pattern the forward takes (band,
// dilated, causal, per-batch global sets, chunked attention with a memory
// prefix).
//
// With P = softmax over the row's key set of z = scale * q.k (recomputed from
// the forward's per-row log-sum-exp, no running maximum needed) and the
// upstream gradient dO, the chain rule through the row softmax (Eq. (1) of the
// Unlimiformer page, section 2.3) gives, for every scored pair (i, j):
//   dP_ij = dO_i . V_j,   dS_ij = P_ij (dP_ij - Delta_i),   Delta_i = dO_i . O_i
//   dQ_i = scale sum_j dS_ij K_j,  dK_j = scale sum_i dS_ij Q_i,  dV_j = sum_i P_ij dO_i.
//
// Three launches:
//  - bwd_rows_kernel (row side, like the forward): a workgroup takes 128 (or
//    64) rows of one (batch, head, residue) and walks the 32-key tiles of
//    their band,
//    then the gathered global keys (and Delta = dO . O of its rows, written
//    for the key side): S^T = K Q^T and dP^T = V dO^T on MFMA,
//    dS on the vector unit, dQ^T += K^T dS^T on MFMA (K^T read from the
//    row-major tile with ds_read_b64_tr_b16).  Global-row items (a set of
//    global rows against a chunk of keys) write partial dQ per chunk.
//  - bwd_keys_kernel (key side, the roles of queries and keys swapped): a
//    workgroup takes 128 (or 64) keys and walks the 32-row tiles of the rows whose
//    band holds them, then the gathered global rows: S = Q K^T, dP = dO V^T,
//    dV^T += dO^T P and dK^T += Q^T dS.  Global-key items (a set of global
//    keys against a chunk of rows) write partial dK, dV per chunk.
//  - bwd_merge_kernel: the global rows' dQ and the global keys' dK, dV as
//    the sums of their chunks' partials (no atomics: deterministic).
// Tiles go global -> LDS directly (global_load_lds_dwordx4) through a
// two-stage ring, one barrier per step; the same 16-byte-chunk swizzle as
// the forward keeps the MFMA operand reads free of bank conflicts.
#include "lfattn_internal.h"

namespace lfattn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
#define LDS_AS __attribute__((address_space(3)))

// Per head dimension D: bytes per row, bytes per 32-row tile, 16-byte
// chunks per row.
template <int D>
struct BwdDim {
  static constexpr int RB = 2 * D;
  static constexpr int TILE = 32 * RB;
  static constexpr int CPR = RB / 16;
};
constexpr int kGCap = kMaxGlobalBf16;
constexpr int kOutOfClass = 0x40000000;
constexpr float kLog2e = 1.4426950408889634f;

// Row of register i (0..15) of a 32x32 MFMA result block for lane half hi.
__device__ __forceinline__ constexpr int brow(int i, int hi) {
  return 8 * (i >> 2) + 4 * hi + (i & 3);
}

// Physical 16-byte chunk of logical chunk c in row `row` of a tile (the
// forward's swizzles for 64 LDS banks: the 16 rows a row read serves at a
// time, and the 4 rows x 4 chunks a transposed read serves, each touch
// distinct banks).  D = 64 (128-byte rows): a bijection of row/2 moves the
// 4-chunk block of row pairs 2 apart; D = 128 (256-byte rows): the block bits
// differ over any 4 consecutive rows.
template <int D>
__device__ __forceinline__ int swz(int row, int c) {
  if constexpr (D == 64) {
    const int j = (row >> 1) & 7;
    return c ^ (((j & 1) << 2) | ((j >> 1) & 3));
  } else {
    return c ^ (((row & 3) << 2) | ((row >> 2) & 3));
  }
}

// ds_read_b64_tr_b16 at an LDS byte address (lane transpose of 4x4 blocks of
// 16-bit values); results are used after tr_wait().
__device__ __forceinline__ s16x4 tr_read(unsigned lds_addr) {
  s16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(lds_addr));
  return r;
}
__device__ __forceinline__ void tr_wait(s16x4& a0, s16x4& a1, s16x4& a2, s16x4& a3,
                                        s16x4& a4, s16x4& a5, s16x4& a6, s16x4& a7) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7));
}

// 16-byte direct global -> LDS load: lane i's 16 bytes land at LDS byte
// address M0 + 16 i (M0 = the wave-uniform lds).  Inline assembly, so the
// compiler does not drain outstanding loads before every LDS read; the
// ring's explicit wait orders the accesses.
__device__ __forceinline__ void dma16(const void* gaddr, unsigned lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds), "v"(gaddr)
               : "memory", "m0");
}
// The same from a wave-uniform base address plus a per-lane 32-bit byte
// offset (no per-lane 64-bit address arithmetic).
__device__ __forceinline__ void dma16_s(const void* sbase, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(sbase)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4_s(const void* sbase, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(sbase)
               : "memory", "m0");
}
// 4-byte direct global -> LDS load: lane i's 4 bytes land at M0 + 4 i.
__device__ __forceinline__ void dma4(const void* gaddr, unsigned lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
               :
               : "s"(lds), "v"(gaddr)
               : "memory", "m0");
}
// s_waitcnt vmcnt(0) (gfx9-family encoding; expcnt and lgkmcnt left open).
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// The tile ring: two stages of up to two tiles (one per key split); after
// the loop its first 32 KB hold the key splits' partial sums.
template <int D>
struct BwdSmem {
  unsigned char x[2][2][BwdDim<D>::TILE];  // row side: K tiles; key side: Q tiles
  unsigned char y[2][2][BwdDim<D>::TILE];  // row side: V tiles; key side: dO tiles
  // Key side: per tile row, -lse / scale (-inf for a global row of a band
  // tile, which takes no part there: its weights are exp2(-inf) = 0) and
  // -Delta, the initial values of the score and dP accumulators, loaded
  // straight from the row side's per-row terms.
  float nls[2][2][32];
  float ndl[2][2][32];
  int gpos[kGCap];             // the batch element's global positions
  int gsp[kGCap];              // their place in the residue's subsequence
};

// Row interval [lo(u), hi(u)] of subsequence positions a row u scores (band:
// u - hl .. u + hr; chunked: its chunk, rows before cb being the memory).
struct Pattern {
  int hl, hr, cC, cb;
  __device__ int lo(int u) const { return cC == 0 ? u - hl : (u < cb ? u : cb + (u - cb) / cC * cC); }
  __device__ int hi(int u) const {
    return cC == 0 ? u + hr : (u < cb ? u : cb + (u - cb) / cC * cC + cC - 1);
  }
  // Rows whose interval holds key k: [rlo(k), rhi(k)] (empty before cb when chunked).
  __device__ int rlo(int k) const { return cC == 0 ? k - hr : (k < cb ? 1 : cb + (k - cb) / cC * cC); }
  __device__ int rhi(int k) const {
    return cC == 0 ? k + hl : (k < cb ? 0 : cb + (k - cb) / cC * cC + cC - 1);
  }
};

// The K^T (row side) or Q^T / dO^T (key side) operand for column block b and
// k-step k2 of a 32-row tile at LDS address base: lane L gets rows
// 16k2 + 4(L/32) + j (j < 4) and 16k2 + 8 + 4(L/32) + (j - 4) of column
// 32b + L%32, the row order of the packed weight registers 4k2 .. 4k2+3.
template <int D>
struct TrAddr {
  unsigned off[D / 32][2];
  __device__ void init(int lane) {
    const int g16 = lane >> 4, t16 = lane & 15;
#pragma unroll
    for (int b = 0; b < D / 32; ++b) {
      const int dcol = 32 * b + 16 * (g16 & 1) + 4 * (t16 & 3);
      const int c = dcol >> 3, half = (dcol >> 2) & 1;
      const int row0 = 4 * (g16 >> 1) + (t16 >> 2), row1 = row0 + 8;
      off[b][0] = row0 * BwdDim<D>::RB + 16 * swz<D>(row0, c) + 8 * half;
      off[b][1] = row1 * BwdDim<D>::RB + 16 * swz<D>(row1, c) + 8 * half;
    }
  }
};

// acc[b] += (tile at base)^T . W, W = the packed weights w[0..7] (bf16 pairs),
// over the tile's 32 rows in two k-steps (D = 128: one k-step's eight reads
// at a time, fewer live operands).
template <int D>
__device__ __forceinline__ void tr_mfma(unsigned base, const TrAddr<D>& ta, const unsigned* w,
                                        f32x16* acc) {
  constexpr int NB = D / 32, RB = BwdDim<D>::RB;
  if constexpr (D == 64) {
    s16x4 r[2][2][2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        r[k2][b][0] = tr_read(base + ta.off[b][0] + 16 * RB * k2);
        r[k2][b][1] = tr_read(base + ta.off[b][1] + 16 * RB * k2);
      }
    tr_wait(r[0][0][0], r[0][0][1], r[0][1][0], r[0][1][1], r[1][0][0], r[1][0][1], r[1][1][0],
            r[1][1][1]);
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const uint4 wu = make_uint4(w[4 * k2], w[4 * k2 + 1], w[4 * k2 + 2], w[4 * k2 + 3]);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(r[k2][b][0], r[k2][b][1], 0, 1, 2, 3, 4, 5, 6, 7));
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, wu),
                                                         acc[b], 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      s16x4 r[NB][2];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        r[b][0] = tr_read(base + ta.off[b][0] + 16 * RB * k2);
        r[b][1] = tr_read(base + ta.off[b][1] + 16 * RB * k2);
      }
      tr_wait(r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]);
      const uint4 wu = make_uint4(w[4 * k2], w[4 * k2 + 1], w[4 * k2 + 2], w[4 * k2 + 3]);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(r[b][0], r[b][1], 0, 1, 2, 3, 4, 5, 6, 7));
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, wu),
                                                         acc[b], 0, 0, 0);
      }
    }
  }
}

// s + sum_ks A_ks . B_ks with A from the 32 rows of the tile at LDS pointer t
// (lane: row L%32, columns 16ks + 8(L/32) .. +7) and B in registers.
template <int D>
__device__ __forceinline__ f32x16 rows_mfma(const unsigned char* t, int l32, int hi,
                                            const bf16x8* bop, f32x16 s = f32x16{}) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const bf16x8 a = *(const LDS_AS bf16x8*)(const LDS_AS unsigned char*)
        (t + l32 * BwdDim<D>::RB + 16 * swz<D>(l32, 2 * ks + hi));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop[ks], s, 0, 0, 0);
  }
  return s;
}

// Both products of the key side at once: s += (tile x)·kb and dp += (tile y)·vb
// over the head dimension, one k-step at a time with the two tiles' reads of
// that k-step in flight together (two independent MFMA chains).  Used at
// D = 128 (key side -3%); at D = 64 the four extra registers spill.
template <int D>
__device__ __forceinline__ void rows_mfma2(const unsigned char* tx, const unsigned char* ty,
                                           int l32, int hi, const bf16x8* kb, const bf16x8* vb,
                                           f32x16& s, f32x16& dp) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const int off = l32 * BwdDim<D>::RB + 16 * swz<D>(l32, 2 * ks + hi);
    const bf16x8 a = *(const LDS_AS bf16x8*)(const LDS_AS unsigned char*)(tx + off);
    const bf16x8 b = *(const LDS_AS bf16x8*)(const LDS_AS unsigned char*)(ty + off);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kb[ks], s, 0, 0, 0);
    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, vb[ks], dp, 0, 0, 0);
  }
}

// Pack two fp32 weights to a bf16 pair (round to nearest even).
__device__ __forceinline__ unsigned pack2(float a, float b) {
  f32x2 f = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

// Stage the batch element's global positions (and their subsequence
// positions in residue r of dilation d) in LDS.
template <class SM>
__device__ __forceinline__ void stage_globals(SM& sm, const int* gl, int ng, int r, int d) {
  for (int x = threadIdx.x; x < ng; x += blockDim.x) {
    const int g = gl[x], off = g - r;
    sm.gpos[x] = g;
    sm.gsp[x] = d == 1 ? off : ((off >= 0 && off % d == 0) ? off / d : kOutOfClass);
  }
}

// ---------------------------------------------------------------------------
// Row side: dQ.
// ---------------------------------------------------------------------------
// KS = 1: four waves of 32 rows (128 per workgroup) share one stream of key
// tiles.  KS = 2: two waves of 32 rows (64 per workgroup) take the even
// tiles, the other two the odd ones, and the two partial dQ add up through
// LDS at the end (twice the workgroups, half the tiles per wave).
// Wavefronts per SIMD of the backward kernels: D = 64 fits 168 registers
// (3), D = 128 256 (2).
template <int D>
constexpr int bwd_wpe() { return D == 64 ? 3 : 2; }

// The query side takes WPE wavefronts per SIMD: bwd_wpe, or 4 at D = 64 (128
// registers), where it recomputes its per-lane load and transposed-read
// offsets each step from a thread index the compiler cannot carry across the
// loop, instead of holding them (which would spill inside the loop).
template <int D, int KS, int WPE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void bwd_rows_kernel(const BandWork* __restrict__ work, BwdArgs a) {
  constexpr bool kLean = WPE > bwd_wpe<D>();
  constexpr int RB = 4 / KS, IR = 32 * RB;  // row blocks, rows per item
  constexpr int kBD = D, TILE = BwdDim<D>::TILE, CPR = BwdDim<D>::CPR;
  __shared__ __attribute__((aligned(16))) BwdSmem<D> sm;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rb = wave % RB, kq = wave / RB;
  const int lane = tid & 63, hi = lane >> 5, l32 = lane & 31;
  const BandWork w = work[blockIdx.x];
  const bool gi = w.dil == 0;
  const int d = gi ? 1 : w.dil, r = gi ? 0 : w.r, N = a.N;
  const int Lr = d == 1 ? N - r : (N - r + d - 1) / d;
  const size_t base = (size_t)w.bh * N * kBD;
  // Global-row items attend with the global rows' projections.
  const unsigned short* Qp = (const unsigned short*)(gi ? a.Qg : a.Q) + base;
  const unsigned short* Kp = (const unsigned short*)(gi ? a.Kg : a.K) + base;
  const unsigned short* Vp = (const unsigned short*)(gi ? a.Vg : a.V) + base;
  const unsigned short* dOp = (const unsigned short*)a.dO + base;
  const unsigned short* Op = (const unsigned short*)a.O + base;
  const int* gl = a.glob + w.g0;
  const int ng = w.ng;
  const unsigned char* isg = a.is_glob + (long long)w.b * a.isg_stride;
  const Pattern pat{a.hw, a.hr, a.chunk, a.cbase};

  stage_globals(sm, gl, ng, r, d);
  __syncthreads();

  // This wave's rows: band item, subsequence positions u = ua + l32 (< Lr);
  // global-row item, slots of the global list.
  const int n_rows = gi ? ng : Lr;
  const int ua = (gi ? IR * w.r : w.t0) + 32 * rb;
  const int u = ua + l32;
  const bool row_ok = u < n_rows;
  const int pos_u = !row_ok ? 0 : (gi ? sm.gpos[u] : r + d * u);
  const int lo_u = gi ? 0 : pat.lo(u);
  const unsigned span_u = gi ? 0u : (unsigned)(pat.hi(u) - lo_u);

  // Keys: band item, subsequence positions s_lo .. s_hi then the global
  // keys; global-row item, plain positions c0 .. c1-1.
  const int t0 = w.t0;
  const int c0 = gi ? t0 * a.chunk_keys : 0, c1 = gi ? min(N, c0 + a.chunk_keys) : 0;
  const int s_lo = gi ? 0 : max(0, pat.lo(t0));
  const int s_hi = gi ? -1 : min(Lr - 1, pat.hi(min(t0 + IR - 1, Lr - 1)));
  const int n_band = gi ? (c1 - c0 + 31) / 32 : (s_hi - s_lo) / 32 + 1;
  const int n_tiles = n_band + (gi ? 0 : (ng + 31) / 32);

  // Key position of row rr of tile t; a row past the end of the tile's keys
  // takes the last one (its weights are masked).
  auto key_pos = [&](int t, int rr) -> int {
    if (gi) return min(c0 + 32 * t + rr, c1 - 1);
    if (t < n_band) return r + d * min(s_lo + 32 * t + rr, s_hi);
    return sm.gpos[min(32 * (t - n_band) + rr, ng - 1)];
  };
  // One thread's share of a tile's loads: tile rows tid/CPR + 256/CPR e,
  // physical 16-byte chunk tid%CPR (the 1 KB a wave's direct load fills are
  // bytes 1024 (w + 4e) .. of the tile).  Step j holds tiles KS j .. KS j +
  // KS - 1 in stage j % 2.
  constexpr int NL = TILE / 4096;  // direct loads per matrix and thread
  const int ld_row = tid / CPR, ld_c = swz<D>(ld_row, tid % CPR);
  const unsigned xl = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(LDS_AS void*)&sm.x[0][0][0] + 1024u * wave);
  const unsigned yl = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(LDS_AS void*)&sm.y[0][0][0] + 1024u * wave);
  const int n_steps = (n_tiles + KS - 1) / KS;
  auto load = [&](int j) {
#pragma unroll
    for (int q2 = 0; q2 < KS; ++q2) {
      const int t = KS * j + q2;
      if (t < n_tiles) {
        const unsigned so = (unsigned)((j & 1) * 2 + q2) * TILE;
#pragma unroll
        for (int e = 0; e < NL; ++e) {
          int lr = ld_row, lc = ld_c;
          if constexpr (kLean) {
            int tx = (int)threadIdx.x;
            asm volatile("" : "+v"(tx));
            lr = tx / CPR;
            lc = swz<D>(lr, tx % CPR);
          }
          const size_t p = (size_t)key_pos(t, lr + (256 / CPR) * e);
          dma16(Kp + p * kBD + 8 * lc, xl + so + 4096u * e);
          dma16(Vp + p * kBD + 8 * lc, yl + so + 4096u * e);
        }
      }
    }
  };

  // The first tile's loads go out before the rows' operands, so that their
  // latency overlaps the operand loads and Delta instead of following them.
  if (n_steps > 0) load(0);

  // Operands of the rows: Q and dO rows (B of S^T = K Q^T and dP^T = V dO^T),
  // the log-sum-exp (base 2 of scores times scale * log2(e)) and Delta.
  bf16x8 q[kBD / 16], g[kBD / 16];
#pragma unroll
  for (int ks = 0; ks < kBD / 16; ++ks) {
    q[ks] = *(const bf16x8*)(Qp + (size_t)pos_u * kBD + 16 * ks + 8 * hi);
    g[ks] = *(const bf16x8*)(dOp + (size_t)pos_u * kBD + 16 * ks + 8 * hi);
  }
  const float lse2 = a.lse[(size_t)w.bh * N + pos_u] * kLog2e;
  // Delta = dO . O of the row (each lane half holds 32 of its columns); the
  // band items write it, with the row's -lse / scale, for the key side,
  // which runs after this kernel.
  float dlt = 0.0f;
#pragma unroll
  for (int ks = 0; ks < kBD / 16; ++ks) {
    const bf16x8 o8 = *(const bf16x8*)(Op + (size_t)pos_u * kBD + 16 * ks + 8 * hi);
#pragma unroll
    for (int e = 0; e < 8; ++e) dlt = fmaf((float)g[ks][e], (float)o8[e], dlt);
  }
  dlt += __shfl_xor(dlt, 32);
  const float nls = -a.lse[(size_t)w.bh * N + pos_u] / a.scale;

  TrAddr<D> ta;
  ta.init(lane);
  f32x16 acc[D / 32];
#pragma unroll
  for (int b = 0; b < D / 32; ++b) acc[b] = f32x16{};

  wait_vm0();
  __syncthreads();
  for (int j = 0; j < n_steps; ++j) {
    const int st = j & 1, t = KS * j + kq;
    if (j + 1 < n_steps) load(j + 1);
    // Tiles none of this wave's rows score are skipped, and a tile every
    // row of the wave scores completely needs no mask (wave-uniform tests;
    // lo and hi are non-decreasing in the row).  Lanes of rows past the end
    // or of global rows compute values that are never stored.
    bool act = ua < n_rows && t < n_tiles, full = false;
    if (act) {
      if (gi) {
        full = c0 + 32 * t + 31 < c1;
      } else if (t < n_band) {
        const int k0 = s_lo + 32 * t, k1 = min(k0 + 31, s_hi);
        const int ul = min(ua + 31, n_rows - 1);
        act = (k0 <= pat.hi(ul)) && (k1 >= pat.lo(ua));
        full = (k0 + 31 <= s_hi) && (k0 >= pat.lo(ul)) && (k0 + 31 <= pat.hi(ua));
      }
    }
    if (act) {
      const f32x16 s = rows_mfma<D>(sm.x[st][kq], l32, hi, q);
      const f32x16 dp = rows_mfma<D>(sm.y[st][kq], l32, hi, g);
      unsigned dsw[8];
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[i], a.sl2, -lse2));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[i + 1], a.sl2, -lse2));
        dsw[i / 2] = pack2(p0 * (dp[i] - dlt), p1 * (dp[i + 1] - dlt));
      }
      if (!full) {
        // Keys the row does not score keep no weight: their bf16 halves are
        // cleared bitwise (whatever the value was, an infinity or a NaN
        // included), under one branch rather than a test per register.
        unsigned mk[8];
        if (gi || t < n_band) {
          // Key kk of the tile is allowed when mb + kk lies in [0, lim]: a
          // chunk's keys before c1, or band keys within the row's interval
          // and the item's key range.
          int mb = gi ? 32 * t : s_lo + 32 * t - lo_u;
          int lim = gi ? c1 - c0 - 1 : min((int)span_u, s_hi - lo_u);
          if (!row_ok || lim < 0) mb = -64, lim = 0;
          asm volatile("" : "+v"(mb));
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            const bool k0 = (unsigned)(mb + brow(i, hi)) <= (unsigned)lim;
            const bool k1 = (unsigned)(mb + brow(i + 1, hi)) <= (unsigned)lim;
            mk[i / 2] = (k0 ? 0x0000ffffu : 0u) | (k1 ? 0xffff0000u : 0u);
          }
        } else {
          // A global key is scored here unless the row's band already holds it.
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            bool ok[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int slot = 32 * (t - n_band) + brow(i + e, hi);
              ok[e] = row_ok & (slot < ng) &
                      ((unsigned)(sm.gsp[min(slot, kGCap - 1)] - lo_u) > span_u);
            }
            mk[i / 2] = (ok[0] ? 0x0000ffffu : 0u) | (ok[1] ? 0xffff0000u : 0u);
          }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) dsw[i] &= mk[i];
      }
      const unsigned xb = (unsigned)(uintptr_t)(LDS_AS void*)sm.x[st][kq];
      if constexpr (kLean) {
        TrAddr<D> tq;
        int ll = (int)threadIdx.x & 63;
        asm volatile("" : "+v"(ll));
        tq.init(ll);
        tr_mfma<D>(xb, tq, dsw, acc);
      } else {
        tr_mfma<D>(xb, ta, dsw, acc);
      }
    }
    wait_vm0();
    __syncthreads();
  }
  if (KS == 2) {
    // The odd-tile waves hand their sums to the even-tile waves of the
    // same rows (element e of lane L at float (32 rb + e) * 64 + L).
    constexpr int NE = D / 2;  // accumulator elements per lane
    static_assert(2 * NE * 64 * 4 <= sizeof(sm.x), "reduction area");
    float* red = (float*)&sm.x[0][0][0];
    if (kq == 1)
#pragma unroll
      for (int e = 0; e < NE; ++e) red[(NE * rb + e) * 64 + lane] = acc[e >> 4][e & 15];
    __syncthreads();
    if (kq == 1) return;
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e >> 4][e & 15] += red[(NE * rb + e) * 64 + lane];
  }

  if (!row_ok) return;
  // The key side's per-row terms (three planes of [B*H, N], written by the
  // band items, which hold every position): -Delta, -lse / scale, and the
  // same with -inf at global positions (band tiles leave the global rows to
  // the gathered global tiles).
  const bool row_glob = !gi && isg[pos_u];
  if (!gi && hi == 0) {
    const size_t plane = (size_t)a.n_bh * N, at = (size_t)w.bh * N + pos_u;
    a.terms[at] = -dlt;
    a.terms[plane + at] = nls;
    a.terms[2 * plane + at] = row_glob ? -__builtin_inff() : nls;
  }
  // With separate projections a band row has no Qg gradient.
  if (a.proj && !gi) {
    float* dqg = a.dQg + base + (size_t)pos_u * kBD;
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *(float4*)(dqg + 32 * b + 8 * g4 + 4 * hi) = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (row_glob) return;  // a global row: its gradient comes from the global-row items
  // Band row: its dQ.  Global-row item: the chunk's partial dQ of slot u.
  float* dq = gi ? a.gpart + (((size_t)w.bh * a.n_gch + t0) * a.n_glob + u) * kBD
                 : a.dQ + base + (size_t)pos_u * kBD;
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      *(float4*)(dq + 32 * b + 8 * g4 + 4 * hi) =
          make_float4(a.scale * acc[b][4 * g4], a.scale * acc[b][4 * g4 + 1],
                      a.scale * acc[b][4 * g4 + 2], a.scale * acc[b][4 * g4 + 3]);
}

// ---------------------------------------------------------------------------
// Key side: dK, dV.
// ---------------------------------------------------------------------------
// KS as on the row side: 32 (KS = 2) or 128 (KS = 1) keys per workgroup, and
// with KS = 2 the even and odd row tiles split between two pairs of waves.
// PROJ: the global rows take their own projections (a separate
// instantiation: a second pass over the gathered global rows).
template <int D, int KS, bool PROJ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(bwd_wpe<D>(), bwd_wpe<D>())))
void bwd_keys_kernel(const BandWork* __restrict__ work, BwdArgs a) {
  constexpr int RB = 4 / KS, IK = 32 * RB;  // key blocks, keys per item
  constexpr int kBD = D, TILE = BwdDim<D>::TILE, CPR = BwdDim<D>::CPR;
  __shared__ __attribute__((aligned(16))) BwdSmem<D> sm;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rb = wave % RB, kq = wave / RB;
  const int lane = tid & 63, hi = lane >> 5, l32 = lane & 31;
  const BandWork w = work[blockIdx.x];
  const bool gk = w.dil == 0;
  const int d = gk ? 1 : w.dil, r = gk ? 0 : w.r, N = a.N;
  const int Lr = d == 1 ? N - r : (N - r + d - 1) / d;
  const size_t base = (size_t)w.bh * N * kBD;
  const unsigned short* Qp = (const unsigned short*)a.Q + base;
  const unsigned short* dOp = (const unsigned short*)a.dO + base;
  // Planes of the row side's per-row terms: -Delta, -lse / scale, and the
  // same with -inf at global positions.
  const size_t mplane = (size_t)a.n_bh * N;
  const int* gl = a.glob + w.g0;
  const int ng = w.ng;
  const unsigned char* isg = a.is_glob + (long long)w.b * a.isg_stride;
  const Pattern pat{a.hw, a.hr, a.chunk, a.cbase};

  stage_globals(sm, gl, ng, r, d);
  __syncthreads();

  // This wave's keys: band item, subsequence positions k = ka + l32 (< Lr);
  // global-key item, slots of the global list.
  const int n_keys = gk ? ng : Lr;
  const int ka = (gk ? IK * w.r : w.t0) + 32 * rb;
  const int k = ka + l32;
  const bool key_ok = k < n_keys;
  const int pos_k = !key_ok ? 0 : (gk ? sm.gpos[k] : r + d * k);
  // A global key (band item) is left to the global-key items: its lane's
  // sums are computed but not stored.
  const bool key_band = key_ok && (gk || !isg[pos_k]);
  const int rlo_k = gk ? 0 : pat.rlo(k);

  // Query rows: band item, subsequence positions q_lo .. q_hi (the rows whose
  // interval holds one of the item's keys) then the global rows; global-key
  // item, plain positions c0 .. c1-1.
  const int t0 = w.t0;
  const int c0 = gk ? t0 * a.chunk_keys : 0, c1 = gk ? min(N, c0 + a.chunk_keys) : 0;
  const int kfirst = (a.chunk > 0) ? max(t0, a.cbase) : t0;
  const int klast = min(t0 + IK - 1, Lr - 1);
  const int q_lo = gk ? 0 : max(0, pat.rlo(kfirst));
  const int q_hi = gk ? -1 : min(Lr - 1, pat.rhi(klast));
  const int n_band = gk ? (c1 - c0 + 31) / 32 : (q_hi >= q_lo ? (q_hi - q_lo) / 32 + 1 : 0);
  const int n_tiles = n_band + (gk ? 0 : (ng + 31) / 32);
  // Rows of the key's interval that the item's tiles hold (rows past q_hi
  // are padding: the last band tile repeats row q_hi).
  const unsigned rspan_k = gk ? 0u : (unsigned)(min(pat.rhi(k), q_hi) - rlo_k);

  // Operands of the keys: K and V rows (B of S = Q K^T and dP = dO V^T).
  bf16x8 kr[kBD / 16], vr[kBD / 16];
  auto load_keys = [&](const void* Ksrc, const void* Vsrc) {
    const unsigned short* Kp = (const unsigned short*)Ksrc + base;
    const unsigned short* Vp = (const unsigned short*)Vsrc + base;
#pragma unroll
    for (int ks = 0; ks < kBD / 16; ++ks) {
      kr[ks] = *(const bf16x8*)(Kp + (size_t)pos_k * kBD + 16 * ks + 8 * hi);
      vr[ks] = *(const bf16x8*)(Vp + (size_t)pos_k * kBD + 16 * ks + 8 * hi);
    }
  };
  load_keys(a.K, a.V);

  // Query position of row rr of tile t and whether it takes part (a global
  // row of a band tile is left to the gathered global rows, and with separate
  // projections a global row of a global-key item's chunk to those too; a row
  // past the end of the tile's rows takes the last one and no part).
  auto row_pos = [&](int t, int rr, bool& part) -> int {
    if (gk) {
      const int p = c0 + 32 * t + rr;
      part = p < c1;
      const int pc = min(p, c1 - 1);
      if (PROJ) part = part && !isg[pc];
      return pc;
    }
    if (t < n_band) {
      const int uq = q_lo + 32 * t + rr;
      const int p = r + d * min(uq, q_hi);
      part = uq <= q_hi && !isg[p];
      return p;
    }
    const int slot = 32 * (t - n_band) + rr;
    part = slot < ng;
    return sm.gpos[min(slot, ng - 1)];
  };
  // Tile loads as on the row side.  The rows' -lse / scale and -Delta go to
  // LDS with direct loads too (wavefronts 0 and 1, lane L: row L%32 of the
  // step's tile L/32, KS = 1: both lane halves the one tile, the second slot
  // unused): band tiles take the terms with -inf at global rows, gathered
  // global rows (and the chunks of global-key items, shared projections)
  // the plain ones.  Padding rows repeat a real row; the masks drop them.
  constexpr int NL = TILE / 4096;  // direct loads per matrix and thread
  const int ld_row = tid / CPR, ld_c = swz<D>(ld_row, tid % CPR);
  const unsigned xl = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(LDS_AS void*)&sm.x[0][0][0] + 1024u * wave);
  const unsigned yl = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(LDS_AS void*)&sm.y[0][0][0] + 1024u * wave);
  const unsigned ml = __builtin_amdgcn_readfirstlane(
      wave == 0 ? (unsigned)(uintptr_t)(LDS_AS void*)&sm.nls[0][0][0]
                : (unsigned)(uintptr_t)(LDS_AS void*)&sm.ndl[0][0][0]);
  // A band tile whose 32 rows all lie before q_hi is loaded from its first
  // row's address (wave-uniform) plus per-lane offsets (rows d apart).
  unsigned boff[NL];
#pragma unroll
  for (int e = 0; e < NL; ++e)
    boff[e] = (unsigned)((d * (ld_row + (256 / CPR) * e)) * kBD + 8 * ld_c) * 2u;
  const unsigned moff = (unsigned)(d * (KS == 2 ? lane : (lane & 31))) * 4u;
  // D = 128 (256 registers at two wavefronts per SIMD) recomputes these
  // per-lane offsets where they are used, from a thread index the compiler
  // cannot carry across the loop, instead of holding them (it would spill an
  // MFMA operand, whose reload waits for the step's tile loads).
  auto opaque_tid = [&]() {
    int x = (int)threadIdx.x;
    asm volatile("" : "+v"(x));
    return x;
  };
  // Tiles tb .. te-1 of this item; step j holds tiles tb + KS j .. + KS - 1.
  int tb = 0, te = n_tiles;
  auto fast_tile = [&](int t) { return !gk && t < n_band && q_lo + 32 * t + 31 <= q_hi; };
  auto load = [&](int j) {
#pragma unroll
    for (int q2 = 0; q2 < KS; ++q2) {
      const int t = tb + KS * j + q2;
      if (t < te) {
        const unsigned so = (unsigned)((j & 1) * 2 + q2) * TILE;
        if (fast_tile(t)) {
          const size_t row0 = (size_t)(r + d * (q_lo + 32 * t)) * kBD;
          if constexpr (D == 128) {
            const int tx = opaque_tid(), lr = tx / CPR, lc = swz<D>(lr, tx % CPR);
#pragma unroll
            for (int e = 0; e < NL; ++e) {
              const unsigned bo = (unsigned)((d * (lr + (256 / CPR) * e)) * kBD + 8 * lc) * 2u;
              dma16_s(Qp + row0, bo, xl + so + 4096u * e);
              dma16_s(dOp + row0, bo, yl + so + 4096u * e);
            }
          } else {
#pragma unroll
            for (int e = 0; e < NL; ++e) {
              dma16_s(Qp + row0, boff[e], xl + so + 4096u * e);
              dma16_s(dOp + row0, boff[e], yl + so + 4096u * e);
            }
          }
        } else {
          if constexpr (D == 128) {
            const int tx = opaque_tid(), lr = tx / CPR, lc = swz<D>(lr, tx % CPR);
#pragma unroll
            for (int e = 0; e < NL; ++e) {
              bool part;
              const int p = row_pos(t, lr + (256 / CPR) * e, part);
              dma16(Qp + (size_t)p * kBD + 8 * lc, xl + so + 4096u * e);
              dma16(dOp + (size_t)p * kBD + 8 * lc, yl + so + 4096u * e);
            }
          } else {
#pragma unroll
            for (int e = 0; e < NL; ++e) {
              bool part;
              const int p = row_pos(t, ld_row + (256 / CPR) * e, part);
              dma16(Qp + (size_t)p * kBD + 8 * ld_c, xl + so + 4096u * e);
              dma16(dOp + (size_t)p * kBD + 8 * ld_c, yl + so + 4096u * e);
            }
          }
        }
      }
    }
    if (wave < 2) {
      // Plane 0 (-Delta) for wavefront 1; wavefront 0: plane 2 (-inf at
      // global rows) or 1.  (An index rather than a choice among pointers:
      // the compiler kept the latter in vector registers and spilled.)
      const int t0s = tb + KS * j;
      const unsigned lds = ml + (unsigned)(j & 1) * (2 * 32 * 4);
      if (fast_tile(t0s + KS - 1) && t0s + KS - 1 < te) {
        const int pl = wave == 1 ? 0 : 2;
        if constexpr (D == 128) {
          const unsigned mo = (unsigned)(d * (opaque_tid() & (KS == 2 ? 63 : 31))) * 4u;
          dma4_s(a.terms + ((size_t)pl * mplane + (size_t)w.bh * N + r + d * (q_lo + 32 * t0s)),
                 mo, lds);
        } else {
          dma4_s(a.terms + ((size_t)pl * mplane + (size_t)w.bh * N + r + d * (q_lo + 32 * t0s)),
                 moff, lds);
        }
      } else {
        const int t = min(t0s + (KS == 2 ? lane >> 5 : 0), te - 1);
        bool part;
        const int p = row_pos(t, lane & 31, part);
        const int pl = wave == 1 ? 0 : ((!gk && t < n_band) || (gk && PROJ) ? 2 : 1);
        dma4(a.terms + ((size_t)pl * mplane + (size_t)w.bh * N + p), lds);
      }
    }
  };

  TrAddr<D> ta;
  ta.init(lane);
  f32x16 accK[D / 32], accV[D / 32];

  // The sums over tiles tb .. te-1 in accK, accV (KS = 2: in the even-tile
  // waves, the odd-tile waves' halves added through LDS).
  auto run = [&]() {
#pragma unroll
    for (int b = 0; b < D / 32; ++b) accK[b] = accV[b] = f32x16{};
    const int n_steps = (te - tb + KS - 1) / KS;
    if (n_steps > 0) load(0);
    wait_vm0();
    __syncthreads();
    for (int j = 0; j < n_steps; ++j) {
      const int st = j & 1, t = tb + KS * j + kq;
      if (j + 1 < n_steps) load(j + 1);
      // The tile's rows reach one of this wave's keys; a band tile whose rows
      // all score all of them needs no mask (rlo and rhi are non-decreasing;
      // rows taking no part carry lse +inf, gathered global rows score every
      // key, and keys before the first chunk are global: their lanes are not
      // stored).
      // Other tiles: rows at or past glim are padding.
      const bool band_tile = !gk && t < n_band;
      bool act = ka < n_keys && t < te, full = true;
      int glim = 32;
      if (band_tile) {
        const int u0 = q_lo + 32 * t, u1 = min(u0 + 31, q_hi);
        const int kb = min(ka + 31, n_keys - 1), kf = ka > kfirst ? ka : kfirst;
        act = act && (u0 <= pat.rhi(kb)) && (u1 >= pat.rlo(kf));
        full = (u0 >= pat.rlo(kb)) && (u1 <= pat.rhi(kf)) && (u0 + 31 <= q_hi);
      } else {
        glim = gk ? c1 - c0 - 32 * t : ng - 32 * (t - n_band);
        full = glim >= 32;
      }
      if (act) {
        // Rows 8j + 4hi .. +3 of a result block sit in registers 4j .. 4j+3:
        // the accumulators start at -lse / scale and -Delta of their rows, so
        // s = q.k - lse / scale and dp = dO.v - Delta.
        f32x16 s0, d0;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const float4 l4 = *(const float4*)&sm.nls[st][kq][8 * i4 + 4 * hi];
          const float4 d4 = *(const float4*)&sm.ndl[st][kq][8 * i4 + 4 * hi];
          s0[4 * i4] = l4.x; s0[4 * i4 + 1] = l4.y; s0[4 * i4 + 2] = l4.z; s0[4 * i4 + 3] = l4.w;
          d0[4 * i4] = d4.x; d0[4 * i4 + 1] = d4.y; d0[4 * i4 + 2] = d4.z; d0[4 * i4 + 3] = d4.w;
        }
        f32x16 s, dp;
        if constexpr (D == 128) {
          s = s0;
          dp = d0;
          rows_mfma2<D>(sm.x[st][kq], sm.y[st][kq], l32, hi, kr, vr, s, dp);
        } else {
          s = rows_mfma<D>(sm.x[st][kq], l32, hi, kr, s0);
          dp = rows_mfma<D>(sm.y[st][kq], l32, hi, vr, d0);
        }
        unsigned pw[8], dsw[8];
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float p0 = __builtin_amdgcn_exp2f(s[i] * a.sl2);
          const float p1 = __builtin_amdgcn_exp2f(s[i + 1] * a.sl2);
          pw[i / 2] = pack2(p0, p1);
          dsw[i / 2] = pack2(p0 * dp[i], p1 * dp[i + 1]);
        }
        if (!full) {
          // Pairs outside the key's rows (or padding rows) keep no weight:
          // their bf16 halves are cleared bitwise (whatever the weight was,
          // an infinity or a NaN included).  The lane's row offset is opaque
          // so that the sixteen per-register offsets are formed here, not
          // kept live through the loop.
          int mb = band_tile ? q_lo + 32 * t - rlo_k : 0;
          asm volatile("" : "+v"(mb));
          const unsigned ms = band_tile ? rspan_k : (unsigned)(glim - 1);
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            const bool k0 = (unsigned)(mb + brow(i, hi)) <= ms;
            const bool k1 = (unsigned)(mb + brow(i + 1, hi)) <= ms;
            const unsigned m = (k0 ? 0x0000ffffu : 0u) | (k1 ? 0xffff0000u : 0u);
            pw[i / 2] &= m;
            dsw[i / 2] &= m;
          }
        }
        const unsigned xb = (unsigned)(uintptr_t)(LDS_AS void*)sm.x[st][kq];
        const unsigned yb = (unsigned)(uintptr_t)(LDS_AS void*)sm.y[st][kq];
        if constexpr (D == 128) {
          TrAddr<D> tq;
          tq.init(opaque_tid() & 63);
          tr_mfma<D>(yb, tq, pw, accV);   // dV^T += dO^T P
          tr_mfma<D>(xb, tq, dsw, accK);  // dK^T += Q^T dS
        } else {
          tr_mfma<D>(yb, ta, pw, accV);
          tr_mfma<D>(xb, ta, dsw, accK);
        }
      }
      wait_vm0();
      __syncthreads();
    }
    if constexpr (KS == 2) {
      // As on the row side, for dK (in the x half of the ring) and dV (y).
      constexpr int NE = D / 2;  // accumulator elements per lane
      static_assert(2 * NE * 64 * 4 <= sizeof(sm.x), "reduction area");
      float* rk = (float*)&sm.x[0][0][0];
      float* rv = (float*)&sm.y[0][0][0];
      if (kq == 1)
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          rk[(NE * rb + e) * 64 + lane] = accK[e >> 4][e & 15];
          rv[(NE * rb + e) * 64 + lane] = accV[e >> 4][e & 15];
        }
      __syncthreads();
      if (kq == 0)
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          accK[e >> 4][e & 15] += rk[(NE * rb + e) * 64 + lane];
          accV[e >> 4][e & 15] += rv[(NE * rb + e) * 64 + lane];
        }
      __syncthreads();  // the ring is free again
    }
  };
  // Key lane's dK (scaled) and dV rows at dk and dv.
  auto store = [&](float* dk, float* dv) {
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int c = 32 * b + 8 * g4 + 4 * hi;
        const float4 kv = make_float4(a.scale * accK[b][4 * g4], a.scale * accK[b][4 * g4 + 1],
                                      a.scale * accK[b][4 * g4 + 2], a.scale * accK[b][4 * g4 + 3]);
        const float4 vv = make_float4(accV[b][4 * g4], accV[b][4 * g4 + 1], accV[b][4 * g4 + 2],
                                      accV[b][4 * g4 + 3]);
        *(float4*)(dk + c) = kv;
        *(float4*)(dv + c) = vv;
      }
  };
  const bool holder = KS == 1 || kq == 0;  // holds the item's sums after run()

  // Shared projections: band rows and gathered global rows together.  With
  // separate projections: band rows first (dK, dV), then the gathered global
  // rows with Qg and the keys' Kg, Vg (dKg, dVg of every key of the item).
  if (PROJ && !gk) te = n_band;
  run();
  if (holder && key_band) {
    // Band key: its dK, dV.  Global-key item: the chunk's partials of slot k.
    const size_t plane = (size_t)a.n_bh * a.n_gch * a.n_glob * kBD;
    float* dk = gk ? a.gpart + plane + (((size_t)w.bh * a.n_gch + t0) * a.n_glob + k) * kBD
                   : a.dK + base + (size_t)pos_k * kBD;
    float* dv = gk ? dk + plane : a.dV + base + (size_t)pos_k * kBD;
    store(dk, dv);
  }
  if constexpr (PROJ) {
    if (!gk) {
      tb = n_band;
      te = n_tiles;
      Qp = (const unsigned short*)a.Qg + base;
      load_keys(a.Kg, a.Vg);
      run();
      if (holder && key_ok)
        store(a.dKg + base + (size_t)pos_k * kBD, a.dVg + base + (size_t)pos_k * kBD);
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Global rows and keys: the sums of the chunks' partial gradients.
// ---------------------------------------------------------------------------
// One workgroup per (b*h, global slot), 3 D threads: plane (dQ, dK, dV) and
// column; each adds the slot's partials over the chunks (in chunk order) and
// writes the row.  The partials' base and geometry and the per-batch list
// extents come ahead of the argument block as scalars the build preloads into
// SGPRs, so that the partial loads and the list-extent load go out before any
// argument load returns (a slot past the end of its batch element's list
// reads partials that exist but hold nothing, and stores none).
template <int D>
__global__ __launch_bounds__(3 * D) void bwd_merge_kernel(const float* __restrict__ gpart,
                                                         const int2* __restrict__ gsel,
                                                         int n_glob, int n_gch, int n_bh, int H,
                                                         BwdArgs a) {
  constexpr int kBD = D;
  constexpr int kFirst = 16;  // chunks loaded before the list extent is read
  const int bh = blockIdx.x / n_glob, g = blockIdx.x % n_glob;
  const int pl = threadIdx.x / D, col = threadIdx.x % D;
  const size_t plane = (size_t)n_bh * n_gch * n_glob * kBD;
  const size_t step = (size_t)n_glob * kBD;
  const float* src = gpart + pl * plane + ((size_t)bh * n_gch * n_glob + g) * kBD + col;
  // (Addresses clamped to the last chunk, the values past it dropped in the
  // sum: no branches between the loads.)
  float v[kFirst];
#pragma unroll
  for (int ch = 0; ch < kFirst; ++ch) v[ch] = src[(size_t)min(ch, n_gch - 1) * step];
  const int2 gs = gsel[bh / H];
  // The sum starts from a value this statement defines, after the list
  // extent has arrived: the extent's load is then in flight with the
  // partials' loads instead of being sunk to the end.
  float sum = 0.0f;
  asm volatile("" : "+v"(sum) : "s"(gs.x), "s"(gs.y) : "memory");
  // In chunk order (the trailing zeros of a shorter list add nothing: the
  // sum is never -0).
#pragma unroll
  for (int ch = 0; ch < kFirst; ++ch) sum += ch < n_gch ? v[ch] : 0.0f;
#pragma unroll 8
  for (int ch = kFirst; ch < n_gch; ++ch) sum += src[ch * step];
  if (g >= gs.y) return;
  // The global rows' dQ partials: their Qg gradient with separate
  // projections (and no Q gradient).
  float* dst = pl == 0 ? (a.proj ? a.dQg : a.dQ) : (pl == 1 ? a.dK : a.dV);
  const size_t at = ((size_t)bh * a.N + a.glob[gs.x + g]) * kBD + col;
  dst[at] = sum;
  if (pl == 0 && a.proj) a.dQ[at] = 0.0f;
}

template <int D>
static hipError_t launch_backward_d(const BwdArgs& rows, const BwdArgs& keys, int n_rows_wg,
                                   int n_keys_wg, hipStream_t s, const Timing* t) {
  constexpr int W = bwd_wpe<D>();
  auto rk = rows.ks == 2 ? bwd_rows_kernel<D, 2, W> : bwd_rows_kernel<D, 1, W>;
  if constexpr (D == 64)
    if (rows.rows_wpe == 4) rk = rows.ks == 2 ? bwd_rows_kernel<D, 2, 4> : bwd_rows_kernel<D, 1, 4>;
  hipError_t e = launch_kernel(rk, dim3(n_rows_wg), dim3(256), s, rows, t[0]);
  if (e != hipSuccess) return e;
  auto kk = keys.proj ? (keys.ks == 2 ? bwd_keys_kernel<D, 2, true> : bwd_keys_kernel<D, 1, true>)
                      : (keys.ks == 2 ? bwd_keys_kernel<D, 2, false> : bwd_keys_kernel<D, 1, false>);
  e = launch_kernel(kk, dim3(n_keys_wg), dim3(256), s, keys, t[1]);
  if (e != hipSuccess || keys.n_glob <= 0) return e;
  const float* gpart = keys.gpart;
  int n_glob = keys.n_glob, n_gch = keys.n_gch, n_bh = keys.n_bh, H = keys.H;
  if (n_gch <= 0 || H <= 0) return hipErrorInvalidValue;
  const int2* gsel = keys.gsel;
  void* args[] = {const_cast<float**>(&gpart), const_cast<int2**>(&gsel), &n_glob, &n_gch,
                  &n_bh, &H, const_cast<BwdArgs*>(&keys)};
  return hipExtLaunchKernel(reinterpret_cast<const void*>(bwd_merge_kernel<D>),
                            dim3((unsigned)(n_bh * n_glob)), dim3(3 * D), args, 0, s,
                            t[2].start, t[2].stop, 0);
}

hipError_t launch_backward_bf16(const BwdArgs& rows, const BwdArgs& keys, int n_rows_wg,
                                int n_keys_wg, hipStream_t s, const Timing* t) {
  for (const BwdArgs* a : {&rows, &keys})
    if ((a->D != 64 && a->D != 128) || a->D != rows.D || a->n_glob > kGCap ||
        (a->ks != 1 && a->ks != 2))
      return hipErrorInvalidValue;
  if (n_rows_wg <= 0 || n_keys_wg <= 0) return hipSuccess;
  return rows.D == 64 ? launch_backward_d<64>(rows, keys, n_rows_wg, n_keys_wg, s, t)
                      : launch_backward_d<128>(rows, keys, n_rows_wg, n_keys_wg, s, t);
}

}  // namespace lfattn

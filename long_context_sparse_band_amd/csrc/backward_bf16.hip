// bf16 backward pass for gfx950 (MI355X): dQ, dK, dV of band + global
// attention, D = 64, for every pattern the forward takes (band, dilated,
// causal, per-batch global sets, chunked attention with a memory prefix).
//
// With P = softmax over the row's key set of z = scale * q.k (recomputed from
// the forward's per-row log-sum-exp, no running maximum needed) and the
// upstream gradient dO, the chain rule through the row softmax (Eq. (1) of the
// Unlimiformer page, section 2.3) gives, for every scored pair (i, j):
//   dP_ij = dO_i . V_j,   dS_ij = P_ij (dP_ij - Delta_i),   Delta_i = dO_i . O_i
//   dQ_i = scale sum_j dS_ij K_j,  dK_j = scale sum_i dS_ij Q_i,  dV_j = sum_i P_ij dO_i.
//
// Three launches:
//  - bwd_prep_kernel: Delta for every row; zeroes dQ at the global rows and dK,
//    dV at the global keys (which receive atomic sums below).
//  - bwd_rows_kernel (row side, like the forward): a workgroup takes 128 rows
//    of one (batch, head, residue) and walks the 32-key tiles of their band,
//    then the gathered global keys: S^T = K Q^T and dP^T = V dO^T on MFMA,
//    dS on the vector unit, dQ^T += K^T dS^T on MFMA (K^T read from the
//    row-major tile with ds_read_b64_tr_b16).  Global-row items (128 global
//    rows against a 512-key chunk) add their dQ with atomics.
//  - bwd_keys_kernel (key side, the roles of queries and keys swapped): a
//    workgroup takes 128 keys and walks the 32-row tiles of the rows whose
//    band holds them, then the gathered global rows: S = Q K^T, dP = dO V^T,
//    dV^T += dO^T P and dK^T += Q^T dS.  Global-key items (128 global keys
//    against a 512-row chunk) add dK, dV with atomics.
// Tiles go global -> registers -> LDS through a two-stage ring, one barrier
// per step; the same 16-byte-chunk swizzle as the forward keeps the MFMA
// operand reads free of bank conflicts.
#include "lfattn_internal.h"

namespace lfattn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
#define LDS_AS __attribute__((address_space(3)))

constexpr int kBD = 64;          // head dimension
constexpr int kRB = 2 * kBD;     // bytes per row
constexpr int kTileB = 32 * kRB; // bytes per 32-row tile
constexpr int kItemRows = 128;   // rows (row side) or keys (key side) per workgroup
constexpr int kGCap = kMaxGlobalBf16;
constexpr int kOutOfClass = 0x40000000;
constexpr float kLog2e = 1.4426950408889634f;

// Row of register i (0..15) of a 32x32 MFMA result block for lane half hi.
__device__ __forceinline__ constexpr int brow(int i, int hi) {
  return 8 * (i >> 2) + 4 * hi + (i & 3);
}

// Physical 16-byte chunk of logical chunk c in row `row` of a tile with
// 128-byte rows (the forward's swizzle for 64 LDS banks: the 16 rows a
// row read serves at a time, and the 4 rows x 4 chunks a transposed read
// serves, each touch distinct banks).
__device__ __forceinline__ int swz(int row, int c) {
  const int j = (row >> 1) & 7;
  return c ^ (((j & 1) << 2) | ((j >> 1) & 3));
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
// s_waitcnt vmcnt(0) (gfx9-family encoding; expcnt and lgkmcnt left open).
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

struct BwdSmem {
  unsigned char x[2][kTileB];  // row side: K tiles; key side: Q tiles
  unsigned char y[2][kTileB];  // row side: V tiles; key side: dO tiles
  // Key side: per tile row, -lse / scale (-inf for a row that takes no
  // part: its weights are exp2(-inf) = 0) and -Delta, the initial values of
  // the score and dP accumulators.
  float nls[2][32];
  float ndl[2][32];
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
struct TrAddr {
  unsigned off[2][2];
  __device__ void init(int lane) {
    const int g16 = lane >> 4, t16 = lane & 15;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int dcol = 32 * b + 16 * (g16 & 1) + 4 * (t16 & 3);
      const int c = dcol >> 3, half = (dcol >> 2) & 1;
      const int row0 = 4 * (g16 >> 1) + (t16 >> 2), row1 = row0 + 8;
      off[b][0] = row0 * kRB + 16 * swz(row0, c) + 8 * half;
      off[b][1] = row1 * kRB + 16 * swz(row1, c) + 8 * half;
    }
  }
};

// acc[b] += (tile at base)^T . W, W = the packed weights w[0..7] (bf16 pairs),
// over the tile's 32 rows in two k-steps.
__device__ __forceinline__ void tr_mfma(unsigned base, const TrAddr& ta, const unsigned* w,
                                        f32x16* acc) {
  s16x4 r[2][2][2];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      r[k2][b][0] = tr_read(base + ta.off[b][0] + 16 * kRB * k2);
      r[k2][b][1] = tr_read(base + ta.off[b][1] + 16 * kRB * k2);
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
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, wu), acc[b],
                                                       0, 0, 0);
    }
  }
}

// s + sum_ks A_ks . B_ks with A from the 32 rows of the tile at LDS pointer t
// (lane: row L%32, columns 16ks + 8(L/32) .. +7) and B in registers.
__device__ __forceinline__ f32x16 rows_mfma(const unsigned char* t, int l32, int hi,
                                            const bf16x8* bop, f32x16 s = f32x16{}) {
#pragma unroll
  for (int ks = 0; ks < kBD / 16; ++ks) {
    const bf16x8 a = *(const LDS_AS bf16x8*)(const LDS_AS unsigned char*)
        (t + l32 * kRB + 16 * swz(l32, 2 * ks + hi));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop[ks], s, 0, 0, 0);
  }
  return s;
}

// Pack two fp32 weights to a bf16 pair (round to nearest even).
__device__ __forceinline__ unsigned pack2(float a, float b) {
  f32x2 f = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

// Stage the batch element's global positions (and their subsequence
// positions in residue r of dilation d) in LDS.
__device__ __forceinline__ void stage_globals(BwdSmem& sm, const int* gl, int ng, int r, int d) {
  for (int x = threadIdx.x; x < ng; x += blockDim.x) {
    const int g = gl[x], off = g - r;
    sm.gpos[x] = g;
    sm.gsp[x] = d == 1 ? off : ((off >= 0 && off % d == 0) ? off / d : kOutOfClass);
  }
}

// ---------------------------------------------------------------------------
// Delta and zeroing.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
  const long long row = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long n_rows = (long long)a.n_bh * a.N;
  if (row >= n_rows) return;
  const int bh = (int)(row / a.N), pos = (int)(row % a.N), b = bh / a.H;
  const unsigned short* o = (const unsigned short*)a.O + row * kBD;
  const unsigned short* g = (const unsigned short*)a.dO + row * kBD;
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kBD; c += 8) {
    const bf16x8 ov = *(const bf16x8*)(o + c), gv = *(const bf16x8*)(g + c);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += (float)ov[e] * (float)gv[e];
  }
  a.delta[row] = s;
  if (a.is_glob[(long long)b * a.isg_stride + pos]) {
    float4* q = (float4*)(a.dQ + row * kBD);
    float4* k = (float4*)(a.dK + row * kBD);
    float4* v = (float4*)(a.dV + row * kBD);
#pragma unroll
    for (int c = 0; c < kBD / 4; ++c) {
      q[c] = make_float4(0.f, 0.f, 0.f, 0.f);
      k[c] = make_float4(0.f, 0.f, 0.f, 0.f);
      v[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

// ---------------------------------------------------------------------------
// Row side: dQ.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
void bwd_rows_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) BwdSmem sm;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hi = lane >> 5, l32 = lane & 31;
  const BandWork w = a.work[blockIdx.x];
  const bool gi = w.dil == 0;
  const int d = gi ? 1 : w.dil, r = gi ? 0 : w.r, N = a.N;
  const int Lr = d == 1 ? N - r : (N - r + d - 1) / d;
  const size_t base = (size_t)w.bh * N * kBD;
  const unsigned short* Qp = (const unsigned short*)a.Q + base;
  const unsigned short* Kp = (const unsigned short*)a.K + base;
  const unsigned short* Vp = (const unsigned short*)a.V + base;
  const unsigned short* dOp = (const unsigned short*)a.dO + base;
  const int* gl = a.glob + w.g0;
  const int ng = w.ng;
  const unsigned char* isg = a.is_glob + (long long)w.b * a.isg_stride;
  const Pattern pat{a.hw, a.hr, a.chunk, a.cbase};

  stage_globals(sm, gl, ng, r, d);
  __syncthreads();

  // This wave's rows: band item, subsequence positions u = ua + l32 (< Lr);
  // global-row item, slots of the global list.
  const int n_rows = gi ? ng : Lr;
  const int ua = (gi ? kItemRows * w.r : w.t0) + 32 * wave;
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
  const int s_hi = gi ? -1 : min(Lr - 1, pat.hi(min(t0 + kItemRows - 1, Lr - 1)));
  const int n_band = gi ? (c1 - c0 + 31) / 32 : (s_hi - s_lo) / 32 + 1;
  const int n_tiles = n_band + (gi ? 0 : (ng + 31) / 32);

  // Operands of the rows: Q and dO rows (B of S^T = K Q^T and dP^T = V dO^T),
  // the log-sum-exp (base 2 of scores times scale * log2(e)) and Delta.
  bf16x8 q[kBD / 16], g[kBD / 16];
#pragma unroll
  for (int ks = 0; ks < kBD / 16; ++ks) {
    q[ks] = *(const bf16x8*)(Qp + (size_t)pos_u * kBD + 16 * ks + 8 * hi);
    g[ks] = *(const bf16x8*)(dOp + (size_t)pos_u * kBD + 16 * ks + 8 * hi);
  }
  const float lse2 = a.lse[(size_t)w.bh * N + pos_u] * kLog2e;
  const float dlt = a.delta[(size_t)w.bh * N + pos_u];

  // Key position of row rr of tile t; a row past the end of the tile's keys
  // takes the last one (its weights are masked).
  auto key_pos = [&](int t, int rr) -> int {
    if (gi) return min(c0 + 32 * t + rr, c1 - 1);
    if (t < n_band) return r + d * min(s_lo + 32 * t + rr, s_hi);
    return sm.gpos[min(32 * (t - n_band) + rr, ng - 1)];
  };
  // One thread's share of tile t's loads: tile row tid/8, physical 16-byte
  // chunk tid%8 (wave w fills bytes 1024 w .. 1024 w + 1023 of the tile).
  const int ld_row = tid >> 3, ld_c = swz(ld_row, tid & 7);
  const unsigned xl = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(LDS_AS void*)sm.x[0] + 1024u * wave);
  const unsigned yl = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(LDS_AS void*)sm.y[0] + 1024u * wave);
  auto load = [&](int t) {
    const size_t p = (size_t)key_pos(t, ld_row);
    const unsigned so = (unsigned)(t & 1) * kTileB;
    dma16(Kp + p * kBD + 8 * ld_c, xl + so);
    dma16(Vp + p * kBD + 8 * ld_c, yl + so);
  };

  TrAddr ta;
  ta.init(lane);
  f32x16 acc[2] = {f32x16{}, f32x16{}};

  if (n_tiles > 0) load(0);
  wait_vm0();
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int st = t & 1;
    if (t + 1 < n_tiles) load(t + 1);
    // Tiles none of this wave's rows score are skipped, and a tile every
    // row of the wave scores completely needs no mask (wave-uniform tests;
    // lo and hi are non-decreasing in the row).  Lanes of rows past the end
    // or of global rows compute values that are never stored.
    bool act = ua < n_rows, full = false;
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
      const f32x16 s = rows_mfma(sm.x[st], l32, hi, q);
      const f32x16 dp = rows_mfma(sm.y[st], l32, hi, g);
      unsigned dsw[8];
      if (full) {
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[i], a.sl2, -lse2));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[i + 1], a.sl2, -lse2));
          dsw[i / 2] = pack2(p0 * (dp[i] - dlt), p1 * (dp[i + 1] - dlt));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          float ds2[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int kk = brow(i + e, hi);
            bool ok = row_ok;
            if (gi) {
              ok &= c0 + 32 * t + kk < c1;
            } else if (t < n_band) {
              const int k = s_lo + 32 * t + kk;
              ok &= (k <= s_hi) & ((unsigned)(k - lo_u) <= span_u);
            } else {
              const int slot = 32 * (t - n_band) + kk;
              ok &= (slot < ng) && ((unsigned)(sm.gsp[min(slot, kGCap - 1)] - lo_u) > span_u);
            }
            const float p = ok ? __builtin_amdgcn_exp2f(fmaf(s[i + e], a.sl2, -lse2)) : 0.0f;
            ds2[e] = p * (dp[i + e] - dlt);
          }
          dsw[i / 2] = pack2(ds2[0], ds2[1]);
        }
      }
      const unsigned xb = (unsigned)(uintptr_t)(LDS_AS void*)sm.x[st];
      tr_mfma(xb, ta, dsw, acc);
    }
    wait_vm0();
    __syncthreads();
  }

  if (!row_ok) return;
  if (!gi && isg[pos_u]) return;  // a global row: its dQ comes from the global-row items
  float* dq = a.dQ + base + (size_t)pos_u * kBD;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      float* p = dq + 32 * b + 8 * g4 + 4 * hi;
      const float v0 = a.scale * acc[b][4 * g4], v1 = a.scale * acc[b][4 * g4 + 1];
      const float v2 = a.scale * acc[b][4 * g4 + 2], v3 = a.scale * acc[b][4 * g4 + 3];
      if (gi) {
        unsafeAtomicAdd(p, v0);
        unsafeAtomicAdd(p + 1, v1);
        unsafeAtomicAdd(p + 2, v2);
        unsafeAtomicAdd(p + 3, v3);
      } else {
        *(float4*)p = make_float4(v0, v1, v2, v3);
      }
    }
}

// ---------------------------------------------------------------------------
// Key side: dK, dV.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
void bwd_keys_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) BwdSmem sm;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hi = lane >> 5, l32 = lane & 31;
  const BandWork w = a.work[blockIdx.x];
  const bool gk = w.dil == 0;
  const int d = gk ? 1 : w.dil, r = gk ? 0 : w.r, N = a.N;
  const int Lr = d == 1 ? N - r : (N - r + d - 1) / d;
  const size_t base = (size_t)w.bh * N * kBD;
  const unsigned short* Qp = (const unsigned short*)a.Q + base;
  const unsigned short* Kp = (const unsigned short*)a.K + base;
  const unsigned short* Vp = (const unsigned short*)a.V + base;
  const unsigned short* dOp = (const unsigned short*)a.dO + base;
  const float* lsep = a.lse + (size_t)w.bh * N;
  const float* dlp = a.delta + (size_t)w.bh * N;
  const int* gl = a.glob + w.g0;
  const int ng = w.ng;
  const unsigned char* isg = a.is_glob + (long long)w.b * a.isg_stride;
  const Pattern pat{a.hw, a.hr, a.chunk, a.cbase};

  stage_globals(sm, gl, ng, r, d);
  __syncthreads();

  // This wave's keys: band item, subsequence positions k = ka + l32 (< Lr);
  // global-key item, slots of the global list.
  const int n_keys = gk ? ng : Lr;
  const int ka = (gk ? kItemRows * w.r : w.t0) + 32 * wave;
  const int k = ka + l32;
  const bool key_ok = k < n_keys;
  const int pos_k = !key_ok ? 0 : (gk ? sm.gpos[k] : r + d * k);
  // A global key (band item) is left to the global-key items: its lane's
  // sums are computed but not stored.
  const bool key_band = key_ok && (gk || !isg[pos_k]);
  const int rlo_k = gk ? 0 : pat.rlo(k);
  const unsigned rspan_k = gk ? 0u : (unsigned)(pat.rhi(k) - rlo_k);

  // Query rows: band item, subsequence positions q_lo .. q_hi (the rows whose
  // interval holds one of the item's keys) then the global rows; global-key
  // item, plain positions c0 .. c1-1.
  const int t0 = w.t0;
  const int c0 = gk ? t0 * a.chunk_keys : 0, c1 = gk ? min(N, c0 + a.chunk_keys) : 0;
  const int kfirst = (a.chunk > 0) ? max(t0, a.cbase) : t0;
  const int klast = min(t0 + kItemRows - 1, Lr - 1);
  const int q_lo = gk ? 0 : max(0, pat.rlo(kfirst));
  const int q_hi = gk ? -1 : min(Lr - 1, pat.rhi(klast));
  const int n_band = gk ? (c1 - c0 + 31) / 32 : (q_hi >= q_lo ? (q_hi - q_lo) / 32 + 1 : 0);
  const int n_tiles = n_band + (gk ? 0 : (ng + 31) / 32);

  // Operands of the keys: K and V rows (B of S = Q K^T and dP = dO V^T).
  bf16x8 kr[kBD / 16], vr[kBD / 16];
#pragma unroll
  for (int ks = 0; ks < kBD / 16; ++ks) {
    kr[ks] = *(const bf16x8*)(Kp + (size_t)pos_k * kBD + 16 * ks + 8 * hi);
    vr[ks] = *(const bf16x8*)(Vp + (size_t)pos_k * kBD + 16 * ks + 8 * hi);
  }

  // Query position of row rr of tile t and whether it takes part (a global
  // row of a band tile is left to the gathered global rows; a row past the
  // end of the tile's rows takes the last one and no part).
  auto row_pos = [&](int t, int rr, bool& part) -> int {
    if (gk) {
      const int p = c0 + 32 * t + rr;
      part = p < c1;
      return min(p, c1 - 1);
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
  // Tile loads as on the row side; the thread of chunk 0 of a row also
  // fetches the row's -lse / scale and -Delta.
  const int ld_row = tid >> 3, ld_c = swz(ld_row, tid & 7);
  const bool ld_meta = (tid & 7) == 0;
  const unsigned xl = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(LDS_AS void*)sm.x[0] + 1024u * wave);
  const unsigned yl = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(LDS_AS void*)sm.y[0] + 1024u * wave);
  float m_lse = 0.0f, m_dlt = 0.0f;
  auto load = [&](int t) {
    bool part;
    const int p = row_pos(t, ld_row, part);
    const unsigned so = (unsigned)(t & 1) * kTileB;
    dma16(Qp + (size_t)p * kBD + 8 * ld_c, xl + so);
    dma16(dOp + (size_t)p * kBD + 8 * ld_c, yl + so);
    if (ld_meta) {
      m_lse = part ? -lsep[p] / a.scale : -__builtin_inff();
      m_dlt = -dlp[p];
    }
  };
  auto store_meta = [&](int st) {
    if (ld_meta) {
      sm.nls[st][ld_row] = m_lse;
      sm.ndl[st][ld_row] = m_dlt;
    }
  };

  TrAddr ta;
  ta.init(lane);
  f32x16 accK[2] = {f32x16{}, f32x16{}}, accV[2] = {f32x16{}, f32x16{}};

  if (n_tiles > 0) {
    load(0);
    store_meta(0);
  }
  wait_vm0();
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int st = t & 1;
    if (t + 1 < n_tiles) load(t + 1);
    // The tile's rows reach one of this wave's keys; a band tile whose rows
    // all score all of them needs no mask (rlo and rhi are non-decreasing;
    // rows taking no part carry lse +inf, gathered global rows score every
    // key, and keys before the first chunk are global: their lanes are not
    // stored).
    bool act = ka < n_keys, full = true;
    if (!gk && t < n_band) {
      const int u0 = q_lo + 32 * t, u1 = min(u0 + 31, q_hi);
      const int kb = min(ka + 31, n_keys - 1), kf = ka > kfirst ? ka : kfirst;
      act = act && (u0 <= pat.rhi(kb)) && (u1 >= pat.rlo(kf));
      full = (u0 >= pat.rlo(kb)) && (u1 <= pat.rhi(kf));
    }
    if (act) {
      // Rows 8j + 4hi .. +3 of a result block sit in registers 4j .. 4j+3:
      // the accumulators start at -lse / scale and -Delta of their rows, so
      // s = q.k - lse / scale and dp = dO.v - Delta.
      f32x16 s0, d0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 l4 = *(const float4*)&sm.nls[st][8 * j + 4 * hi];
        const float4 d4 = *(const float4*)&sm.ndl[st][8 * j + 4 * hi];
        s0[4 * j] = l4.x; s0[4 * j + 1] = l4.y; s0[4 * j + 2] = l4.z; s0[4 * j + 3] = l4.w;
        d0[4 * j] = d4.x; d0[4 * j + 1] = d4.y; d0[4 * j + 2] = d4.z; d0[4 * j + 3] = d4.w;
      }
      const f32x16 s = rows_mfma(sm.x[st], l32, hi, kr, s0);
      const f32x16 dp = rows_mfma(sm.y[st], l32, hi, vr, d0);
      unsigned pw[8], dsw[8];
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        float p2[2], ds2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          float p = __builtin_amdgcn_exp2f(s[i + e] * a.sl2);
          if (!full) {
            const int qq = brow(i + e, hi);
            p = (unsigned)(q_lo + 32 * t + qq - rlo_k) <= rspan_k ? p : 0.0f;
          }
          p2[e] = p;
          ds2[e] = p * dp[i + e];
        }
        pw[i / 2] = pack2(p2[0], p2[1]);
        dsw[i / 2] = pack2(ds2[0], ds2[1]);
      }
      const unsigned xb = (unsigned)(uintptr_t)(LDS_AS void*)sm.x[st];
      const unsigned yb = (unsigned)(uintptr_t)(LDS_AS void*)sm.y[st];
      tr_mfma(yb, ta, pw, accV);   // dV^T += dO^T P
      tr_mfma(xb, ta, dsw, accK);  // dK^T += Q^T dS
    }
    if (t + 1 < n_tiles) store_meta(1 - st);
    wait_vm0();
    __syncthreads();
  }

  if (!key_band) return;
  float* dk = a.dK + base + (size_t)pos_k * kBD;
  float* dv = a.dV + base + (size_t)pos_k * kBD;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int c = 32 * b + 8 * g4 + 4 * hi;
      const float4 kv = make_float4(a.scale * accK[b][4 * g4], a.scale * accK[b][4 * g4 + 1],
                                    a.scale * accK[b][4 * g4 + 2], a.scale * accK[b][4 * g4 + 3]);
      const float4 vv = make_float4(accV[b][4 * g4], accV[b][4 * g4 + 1], accV[b][4 * g4 + 2],
                                    accV[b][4 * g4 + 3]);
      if (gk) {
        unsafeAtomicAdd(dk + c, kv.x);
        unsafeAtomicAdd(dk + c + 1, kv.y);
        unsafeAtomicAdd(dk + c + 2, kv.z);
        unsafeAtomicAdd(dk + c + 3, kv.w);
        unsafeAtomicAdd(dv + c, vv.x);
        unsafeAtomicAdd(dv + c + 1, vv.y);
        unsafeAtomicAdd(dv + c + 2, vv.z);
        unsafeAtomicAdd(dv + c + 3, vv.w);
      } else {
        *(float4*)(dk + c) = kv;
        *(float4*)(dv + c) = vv;
      }
    }
}

}  // namespace

hipError_t launch_backward_bf16(const BwdArgs& a, int n_wg, hipStream_t s, const Timing* t) {
  if (a.D != kBD) return hipErrorInvalidValue;
  if (a.n_glob > kGCap) return hipErrorInvalidValue;
  const long long n_rows = (long long)a.n_bh * a.N;
  hipError_t e = launch_kernel(bwd_prep_kernel, dim3((unsigned)((n_rows + 255) / 256)), dim3(256),
                               s, a, t[0]);
  if (e != hipSuccess || n_wg <= 0) return e;
  e = launch_kernel(bwd_rows_kernel, dim3(n_wg), dim3(256), s, a, t[1]);
  if (e != hipSuccess) return e;
  return launch_kernel(bwd_keys_kernel, dim3(n_wg), dim3(256), s, a, t[2]);
}

}  // namespace lfattn

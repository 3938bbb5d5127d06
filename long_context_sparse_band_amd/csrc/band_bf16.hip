// bf16 band kernel for gfx950 (MI355X).
//
// One workgroup (4 wavefronts) takes 128*QB consecutive query rows of one
// (batch, head, dilation residue) and walks the 64-key tiles of their band,
// then the tiles of gathered global keys.  Each wavefront owns 32*QB rows
// (QB blocks of 32, one 32x32 MFMA column block each).
//
// Memory path: K and V tiles go global -> LDS with direct loads
// (global_load_lds_dwordx4) into a ring of NS stages, NS-1 tiles ahead of the
// one being computed; nothing is staged in registers.  Rows are 16-byte-chunk
// swizzled so that the MFMA operand reads of 16 consecutive rows hit distinct
// LDS banks.  V stays row-major: the A operand of O^T += V^T P^T is read with
// ds_read_b64_tr_b16, whose lane transpose delivers the 8 keys of one value
// column that a lane feeds to a 32x32x16 k-step.
//
// Per tile and wavefront: S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys on
// the MFMA rows, queries across lanes, so a lane holds 16 keys of one query);
// weights exp2(s*scale*log2e - m) against the running maximum m; P rounded to
// bf16 is already the B operand of the P.V MFMA, and its row sum is taken with
// v_dot2_f32_bf16 on the packed pairs (the same rounded weights as the
// numerator).  The maximum is not computed in the common case: a tile whose
// weights sum past 2^8 on any lane (which includes the first tile, where m
// starts at -1e30, and any overflow to infinity) is redone against its true
// maximum, rescaling the accumulators.  That is exact because softmax ignores
// a constant added to all its inputs (Unlimiformer, section 2.3, footnote 3).
// 32-key halves of a tile that no row of the wave may score are skipped
// (no MFMA, no exp); only tiles cut by a band edge evaluate the band predicate.
//
// The math is Eq. (1) of the Unlimiformer page (section 2.3) over the pattern
// of the Ultralytics glossary page "Longformer" (section on how the attention
// works): band |i-j| <= window//2 (dilated: j = i + d*k), global rows and
// columns, a global key inside a row's band counted once.
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

constexpr int TK = 64;
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

// Key of register i (0..15) of a 32x32 MFMA result block for lane half hi.
__device__ __forceinline__ constexpr int block_row(int i, int hi) {
  return 8 * (i >> 2) + 4 * hi + (i & 3);
}

// Tile geometry for head dimension D.
template <int D>
struct Geo {
  static constexpr int RB = 2 * D;          // bytes per key row
  static constexpr int CPR = RB / 16;       // 16-byte chunks per row
  static constexpr int RPI = 1024 / RB;     // rows one wave-wide direct load fills
  static constexpr int NI = TK / RPI / 4;   // direct loads per wave per matrix and tile
  static constexpr int MAT = TK * RB;       // bytes of one K (or V) tile
  // Physical chunk of logical chunk c in row `row` (an involution).
  static __device__ __forceinline__ int swz(int row, int c) {
    if constexpr (D == 64) return c ^ ((row >> 1) & 7);
    else return c ^ (row & 15);
  }
};

template <int D, int NS>
struct Smem {
  unsigned char st[NS][2 * Geo<D>::MAT];
  int gsub[NS][TK];
};

template <int D, int QB, int NS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void band_bf16_kernel(BandArgs a) {
  using G = Geo<D>;
  __shared__ __attribute__((aligned(16))) Smem<D, NS> sm;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hi = lane >> 5, l32 = lane & 31;
  const BandWork w = a.work[blockIdx.x];
  const int h = w.bh % a.H;
  const int d = a.dil[h];
  const int r = w.r, t0 = w.t0, hw = a.hw, N = a.N;
  const int Lr = (N - r + d - 1) / d;
  const size_t base = (size_t)w.bh * N * D;
  const unsigned short* Qp = (const unsigned short*)a.Q + base;
  const unsigned short* Kp = (const unsigned short*)a.K + base;
  const unsigned short* Vp = (const unsigned short*)a.V + base;
  constexpr int BM = 128 * QB;

  // Rows of this wave: subsequence positions ua .. ub.
  const int ua = t0 + 32 * QB * wave;
  const int ub = min(ua + 32 * QB - 1, Lr - 1);
  const bool live = ua < Lr;

  // Q operand (B of S^T = K Q^T): Q[row][16ks + 8hi + 0..7].
  bf16x8 q[QB][D / 16];
  int u[QB], lo[QB];
  unsigned rng[QB];
  const int s_lo = max(0, t0 - hw);
  const int s_hi = min(Lr - 1, t0 + BM - 1 + hw);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    u[qb] = ua + 32 * qb + l32;
    const bool ok = u[qb] < Lr;
    const size_t row = (size_t)(r + d * (ok ? u[qb] : 0));
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      q[qb][ks] = *(const bf16x8*)(Qp + row * D + 16 * ks + 8 * hi);
      if (!ok) q[qb][ks] = bf16x8{};
    }
    // Band keys this row may score, as an interval [lo, lo + rng] of
    // subsequence positions; rows past the end get an empty interval.
    int l0 = max(u[qb] - hw, 0), h0 = min(u[qb] + hw, s_hi);
    if (!ok || h0 < l0) { l0 = 0x3fffffff; h0 = l0; }
    lo[qb] = l0;
    rng[qb] = (unsigned)(h0 - l0);
  }

  f32x16 acc[QB][D / 32];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int b = 0; b < D / 32; ++b) acc[qb][b] = f32x16{};
    m[qb] = kNegInit;
    l[qb] = 0.0f;
  }

  const int n_band = (s_hi - s_lo) / TK + 1;
  const int n_gt = (a.n_glob + TK - 1) / TK;
  const int n_tiles = n_band + n_gt;

  // Issue the direct loads of tile j into stage sidx.
  auto issue = [&](int j, int sidx) {
    LDS_AS unsigned char* st = (LDS_AS unsigned char*)sm.st[sidx];
    const bool band = j < n_band;
    const int s0 = s_lo + TK * j, g0 = TK * (j - n_band);
#pragma unroll
    for (int e = 0; e < G::NI; ++e) {
      const int qd = wave + 4 * e;
      const int row = G::RPI * qd + lane / G::CPR;
      const int c = G::swz(row, lane % G::CPR);
      int grow;
      if (band) {
        const int s = min(s0 + row, s_hi);  // rows past the band end repeat a real row
        grow = r + d * s;
      } else {
        const int slot = min(g0 + row, a.n_glob - 1);
        grow = a.glob[slot];
      }
      const size_t off = (size_t)grow * D + 8 * c;
      __builtin_amdgcn_global_load_lds((const void*)(Kp + off), (LDS_AS void*)(st + 1024 * qd), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(Vp + off), (LDS_AS void*)(st + G::MAT + 1024 * qd), 16, 0, 0);
    }
    if (!band && tid < TK) {
      // Subsequence position of each global key in this residue class (or a
      // value no band reaches).
      const int slot = g0 + tid;
      int sp = kNotInClass;
      if (slot < a.n_glob) {
        const int off = a.glob[slot] - r;
        if (off >= 0 && off % d == 0) sp = off / d;
      }
      sm.gsub[sidx][tid] = sp;
    }
  };

  // Prologue: tiles 0 .. NS-2.
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < n_tiles) issue(j, j);

  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  for (int t = 0; t < n_tiles; ++t) {
    // Wait for this wave's loads of tile t (the loads of up to NS-2 later
    // tiles may stay in flight), then for every wave's.
    if (t + NS - 2 < n_tiles) wait_vm_lgkm0<2 * G::NI * (NS - 2)>();
    else wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
    if (t + NS - 1 < n_tiles) issue(t + NS - 1, (t + NS - 1) % NS);

    if (!live) continue;
    const int sidx = t % NS;
    const LDS_AS unsigned char* st = (const LDS_AS unsigned char*)sm.st[sidx];
    const bool band = t < n_band;

    // Which 32-key halves of the tile any row of this wave scores, and which
    // of them need the per-pair predicate.
    bool act[2], edge[2];
    unsigned keep[QB][2];
    if (band) {
      const int s0 = s_lo + TK * t;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int k0 = s0 + 32 * kb, k1 = min(k0 + 31, s_hi);
        act[kb] = k0 <= s_hi && k0 <= ub + hw && k1 >= ua - hw;
        edge[kb] = !(k1 == k0 + 31 && k1 - ua <= hw && ub - k0 <= hw);
      }
    } else {
      const int g0 = TK * (t - n_band);
      const int nvalid = min(TK, a.n_glob - g0);
      const unsigned span = 2u * (unsigned)hw;
      bool any[2] = {false, false};
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          unsigned bits = 0;
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int kk0 = 32 * kb + 8 * g4 + 4 * hi;
            const i32x4 sp = *(const LDS_AS i32x4*)&sm.gsub[sidx][kk0];
            const int spv[4] = {sp[0], sp[1], sp[2], sp[3]};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const bool k = (kk0 + c < nvalid) && u[qb] < Lr &&
                             (unsigned)(spv[c] - u[qb] + hw) > span;
              bits |= (unsigned)k << (4 * g4 + c);
            }
          }
          keep[qb][kb] = bits;
          any[kb] |= bits != 0;
        }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        act[kb] = __any(any[kb]);
        edge[kb] = true;
      }
    }
    if (!act[0] && !act[1]) continue;

    // S^T = K Q^T for the active halves (each K read serves all QB blocks).
    f32x16 S[QB][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (!act[kb]) continue;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) S[qb][kb] = f32x16{};
      const int kk = 32 * kb + l32;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 kv = *(const LDS_AS bf16x8*)(st + kk * G::RB + 16 * G::swz(kk, 2 * ks + hi));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          S[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, q[qb][ks], S[qb][kb], 0, 0, 0);
      }
    }

    // Masks.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (!act[kb] || !edge[kb]) continue;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (band) {
          const int basek = s_lo + TK * t + 32 * kb + 4 * hi - lo[qb];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const unsigned x = (unsigned)(basek + block_row(i, 0));
            S[qb][kb][i] = x > rng[qb] ? -INFINITY : S[qb][kb][i];
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            S[qb][kb][i] = ((keep[qb][kb] >> i) & 1u) ? S[qb][kb][i] : -INFINITY;
        }
      }
    }

    // Weights, packed to bf16 (the B operand of P.V), and their row sums.
    unsigned P[QB][2][8];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      auto weights = [&](float mq) {
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (!act[kb]) continue;
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            f32x2 pf;
            pf[0] = fast_exp2(fmaf(S[qb][kb][i], a.sl2, -mq));
            pf[1] = fast_exp2(fmaf(S[qb][kb][i + 1], a.sl2, -mq));
            const bf16x2 pb = __builtin_convertvector(pf, bf16x2);
            P[qb][kb][i / 2] = __builtin_bit_cast(unsigned, pb);
            if (i & 2) s1 = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, s1, false);
            else s0 = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, s0, false);
          }
        }
        return s0 + s1;
      };
      float ls = weights(m[qb]);
      if (__any(!(ls <= kSumLimit))) {
        // Move the running maximum to this tile's maximum and redo it.
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (!act[kb]) continue;
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, S[qb][kb][i]);
        }
        const float mn = fmaxf(m[qb], pair_max(mx) * a.sl2);
        const float alpha = fast_exp2(m[qb] - mn);
        l[qb] *= alpha;
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[qb][b][i] *= alpha;
        m[qb] = mn;
        ls = weights(mn);
      }
      l[qb] += ls;
    }

    // O^T += V^T P^T.  V^T operand for k-step ks (keys 16ks..16ks+15) and
    // column block b, read transposed: lane L gets keys 16ks + 4*(L/32) + j
    // (j < 4) and 16ks + 8 + 4*(L/32) + (j-4) (j >= 4) of column 32b + L%32,
    // the same key order as the P^T registers 8*(ks%2) .. +7.
    const int g16 = lane >> 4, t16 = lane & 15;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (!act[kb]) continue;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const int ks = 2 * kb + k2;
        const int row0 = 16 * ks + 4 * (g16 >> 1) + (t16 >> 2);
#pragma unroll
        for (int b = 0; b < D / 32; ++b) {
          const int dcol = 32 * b + 16 * (g16 & 1) + 4 * (t16 & 3);
          const int c = dcol >> 3, half = (dcol >> 2) & 1;
          const LDS_AS unsigned char* vb = st + G::MAT;
          const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (LDS_AS s16x4*)(vb + row0 * G::RB + 16 * G::swz(row0, c) + 8 * half));
          const int row1 = row0 + 8;
          const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (LDS_AS s16x4*)(vb + row1 * G::RB + 16 * G::swz(row1, c) + 8 * half));
          const bf16x8 va = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const unsigned* pp = &P[qb][kb][4 * k2];
            const uint4 pu = make_uint4(pp[0], pp[1], pp[2], pp[3]);
            const bf16x8 pbv = __builtin_bit_cast(bf16x8, pu);
            acc[qb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pbv, acc[qb][b], 0, 0, 0);
          }
        }
      }
    }
  }

  if (!live) return;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = pair_sum(l[qb]);
    if (u[qb] >= Lr) continue;
    const int row = r + d * u[qb];
    if (a.is_glob[row]) continue;
    const float inv = 1.0f / lt;
    unsigned short* Op = (unsigned short*)a.O + base + (size_t)row * D;
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 o;
#pragma unroll
        for (int c = 0; c < 4; ++c) o[c] = (__bf16)(acc[qb][b][4 * g4 + c] * inv);
        *(bf16x4*)(Op + 32 * b + 8 * g4 + 4 * hi) = o;
      }
  }
}

}  // namespace

int band_bf16_rows_per_wg(int D) { return D == 64 ? 128 : 128; }

hipError_t launch_band_bf16(int D, const BandArgs& a, int n_wg, hipStream_t s) {
  if (n_wg <= 0) return hipSuccess;
  dim3 grid(n_wg), block(256);
  if (D == 64) hipLaunchKernelGGL((band_bf16_kernel<64, 1, 3>), grid, block, 0, s, a);
  else if (D == 128) hipLaunchKernelGGL((band_bf16_kernel<128, 1, 2>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lfattn

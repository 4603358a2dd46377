// The LoRA-augmented MFMA GEMM core: a 256x256 output tile per workgroup of
// eight waves (two per SIMD), laid out 4 x 2: wave (wm, wn) owns rows
// 64 wm .. 64 wm + 63 and columns 128 wn .. 128 wn + 127, i.e. 4 x 8 MFMA
// blocks of 16 x 16.
//
//   acc  = Z_tile . Bop_tile                       (K-loop, bf16 or fp32 MFMA)
//   side = Z_tile . Sop^T                          (same K-loop, same A fragments:
//                                                   the rank-r product, <= 3 adapters)
//   acc += [s_1 T_1 | s_2 T_2 | ...] . [F_1 ; F_2 ; ...]   (the fold: extra K steps)
//
// The side product rides along the base GEMM's K-loop: its operand rows sit
// in LDS right after the B tile and reuse the A fragments already in
// registers, so X (or H, or dG|dU) is read once for both.  Each wave does the
// side MFMAs on one of the two 32-wide K sub-steps of a tile (bf16), which
// splits that work evenly across the wave-row; the halves are summed through
// LDS after the loop.  Two waves per SIMD hide LDS and barrier latency, and a
// 4 x 8 wave tile keeps the accumulators (128 + 16 per adapter) in AGPRs.
//
// Operands reach LDS in two ways.  K-contiguous operands (activations, and
// the forward's weight rows) go straight from global memory into LDS with
// 16-byte direct loads (no staging registers); the swizzle is applied by
// choosing which global chunk each lane fetches.  The backward's weights,
// stored [K][N], are register-staged and transposed on the way in.
//
// LDS during the K-loop: two stages of [A 256 rows | B 256 rows | side 48 rows]
// x 128 bytes.  After the loop the same memory holds: Ts (float side products,
// [3][256][16]), the fold A tile and the fold B tile; epilogues reuse the fold
// tiles for cross-wave reductions.
#pragma once

#include "common.h"

namespace lora {

constexpr int kGemmThreads = 512;                          // 8 waves
constexpr int kMB = 4;                                     // MFMA row blocks per wave
constexpr int kARows = kBM;
constexpr int kBRows = kBN + kSlot * kMaxSide;
constexpr int kABytes = kARows * kRowBytes;
constexpr int kBBytes = kBRows * kRowBytes;
constexpr int kStage = kABytes + kBBytes;
constexpr int kGemmLds = 2 * kStage;                       // 143360 bytes

constexpr int kTsOff = 0;
constexpr int kTsBytes = kMaxSide * kBM * kSlot * 4;       // 49152
constexpr int kFAOff = kTsBytes;
constexpr int kFBOff = kFAOff + kBM * kRowBytes;
constexpr int kRedOff = kFAOff;                            // epilogue scratch (fold tiles are dead)
constexpr int kRedBytes = 2 * kBM * kRowBytes;             // 65536
static_assert(kFBOff + kBN * kRowBytes <= kGemmLds, "post-loop LDS layout overflows");
// One extra Ts-sized slot past the K-loop stages (kernels that declare
// kGemmLdsX): holds a side product across a second K-loop phase.
constexpr int kFlushOff = kGemmLds;
constexpr int kGemmLdsX = kGemmLds + kBM * kSlot * 4;      // 159744 <= 160 KB

struct WaveId {
  int tid, lane, w, wm, wn, g, r16;
};
__device__ __forceinline__ WaveId wave_id() {
  WaveId q;
  q.tid = threadIdx.x;
  q.lane = q.tid & 63;
  q.w = q.tid >> 6;
  q.wm = q.w >> 1;
  q.wn = q.w & 1;
  q.g = q.lane >> 4;
  q.r16 = q.lane & 15;
  return q;
}
// Output row (within the tile) of C-layout element j of block mb.
__device__ __forceinline__ int acc_row(const WaveId& q, int mb, int j) { return q.wm * 64 + mb * 16 + 4 * q.g + j; }

__device__ __forceinline__ float* ts_ptr(char* smem) { return reinterpret_cast<float*>(smem + kTsOff); }
__device__ __forceinline__ int ts_idx(int slot, int row, int t) { return (slot * kBM + row) * kSlot + t; }

// ---------------------------------------------------------------------------
// Direct global -> LDS loads (gfx950 global_load_lds_dwordx4): lane l of a
// wave writes 16 bytes at LDS base + 16 l, so a 1 KB block = 8 tile rows.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void g2lds16(const void* g, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Logical chunk a lane must fetch so that, written at physical chunk
// (lane & 7) of row 8*blk + (lane >> 3), the tile obeys lds_off's swizzle.
__device__ __forceinline__ int direct_chunk(int lane, int) { return (lane & 7) ^ (lane >> 3); }
// 1 KB block `it` of this wave (wave w fills blocks w + 8 it, it = 0..3).
__device__ __forceinline__ int direct_blk(int it) { return (int)(threadIdx.x >> 6) + 8 * it; }
// Tile row this lane fills in its direct block it.
__device__ __forceinline__ int direct_row(int it) { return 8 * direct_blk(it) + (int)((threadIdx.x & 63) >> 3); }

// ---------------------------------------------------------------------------
// K-loop.  Loader interface:
//   issue(kt, As, Bs)        direct global -> LDS loads for K tile kt
//   load(kt)                 register-staged global loads for K tile kt
//   store(As, Bs)            registers -> LDS stage (A rows, B rows, side rows)
//   side_mask(kt)            bit sb set when side block sb has data in tile kt
// ---------------------------------------------------------------------------
// K tiles kt0 .. nkt-1 (stage buffers restart at stage 0).
template <class T, int NSIDE, class Loader>
__device__ __forceinline__ void kloop(char* smem, int nkt, Loader& ld, f32x4 (&acc)[kMB][8],
                                      f32x4 (&sacc)[NSIDE > 0 ? NSIDE : 1][kMB], int kt0 = 0) {
  constexpr int KSUB = ET<T>::KSUB;
  const WaveId q = wave_id();
  if (nkt <= kt0) return;
  ld.issue(kt0, smem, smem + kABytes);
  ld.load(kt0);
  ld.store(smem, smem + kABytes);
  wait_vmem();
  __syncthreads();
  for (int kt = kt0; kt < nkt; ++kt) {
    const char* As = smem + ((kt - kt0) & 1) * kStage;
    const char* Bs = As + kABytes;
    char* An = smem + ((kt - kt0 + 1) & 1) * kStage;
    const bool more = kt + 1 < nkt;
    if (more) {
      ld.issue(kt + 1, An, An + kABytes);
      ld.load(kt + 1);
    }
    unsigned smask = 0u;
    if constexpr (NSIDE > 0) smask = ld.side_mask(kt);
#pragma unroll
    for (int ks = 0; ks < KSUB; ++ks) {
      Frag<T> af[kMB];
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) af[mb] = lds_frag<T>(As, q.wm * 64 + mb * 16 + q.r16, ks, q.g);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const Frag<T> bfr = lds_frag<T>(Bs, q.wn * 128 + nb * 16 + q.r16, ks, q.g);
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) acc[mb][nb] = mma(acc[mb][nb], af[mb], bfr);
      }
      if constexpr (NSIDE > 0) {
        const bool mine = (KSUB == 2) ? (ks == q.wn) : (q.wn == 0);
        if (mine) {
#pragma unroll
          for (int sb = 0; sb < NSIDE; ++sb) {
            if ((smask >> sb) & 1u) {
              const Frag<T> bfr = lds_frag<T>(Bs, kBN + sb * 16 + q.r16, ks, q.g);
#pragma unroll
              for (int mb = 0; mb < kMB; ++mb) sacc[sb][mb] = mma(sacc[sb][mb], af[mb], bfr);
            }
          }
        }
      }
    }
    if (more) ld.store(An, An + kABytes);
    wait_vmem();
    __syncthreads();
  }
}

__device__ __forceinline__ void zero_acc(f32x4 (&acc)[kMB][8]) {
#pragma unroll
  for (int i = 0; i < kMB; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
}
template <int NS>
__device__ __forceinline__ void zero_side(f32x4 (&sacc)[NS][kMB]) {
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) sacc[s][mb] = (f32x4){0.f, 0.f, 0.f, 0.f};
}

// Sum the per-wave side products into Ts[sb][row][t] (float, raw Z.Sop^T).
// Must follow the K-loop's final barrier.  The fold reads only slots < NSIDE.
template <class T, int NSIDE>
__device__ __forceinline__ void side_reduce(char* smem, f32x4 (&sacc)[NSIDE > 0 ? NSIDE : 1][kMB], int slot0 = 0) {
  const WaveId q = wave_id();
  float* Ts = ts_ptr(smem) + slot0 * kBM * kSlot;
  constexpr bool two = ET<T>::KSUB == 2;
  if (q.wn == 0) {
#pragma unroll
    for (int sb = 0; sb < NSIDE; ++sb)
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) Ts[ts_idx(sb, acc_row(q, mb, j), q.r16)] = sacc[sb][mb][j];
  }
  __syncthreads();
  if (two && q.wn == 1) {
#pragma unroll
    for (int sb = 0; sb < NSIDE; ++sb)
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) Ts[ts_idx(sb, acc_row(q, mb, j), q.r16)] += sacc[sb][mb][j];
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Fold: acc += FA . FB^T with FA[m][16 s + t] = fscale[s] * Ts[s][m][t] and
// FB[n][16 s + t] supplied by the kernel (adapter s's fold operand for output
// column n).  One fold tile holds BK / 16 slots (4 for bf16, 2 for fp32).
// FB functor: fb(R, slot, t0, v) fills v[0..VEC) for LDS row R (a permuted
// output column), adapter slot `slot`, ranks t0..t0+VEC-1; v is pre-zeroed.
// Threads 0..255 build FA rows, threads 256..511 build FB rows.
// ---------------------------------------------------------------------------
template <class T, class FB>
__device__ __forceinline__ void fold(char* smem, f32x4 (&acc)[kMB][8], int nslot, const float (&fscale)[kMaxSide],
                                     FB& fb) {
  constexpr int VEC = ET<T>::VEC, BK = ET<T>::BK, KSUB = ET<T>::KSUB;
  const WaveId q = wave_id();
  if (nslot <= 0) return;
  const int nft = (nslot * kSlot + BK - 1) / BK;
  const float* Ts = ts_ptr(smem);
  char* FA = smem + kFAOff;
  char* FBt = smem + kFBOff;
  const bool build_a = q.tid < kBM;
  const int m = q.tid & (kBM - 1);
  for (int ft = 0; ft < nft; ++ft) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int kk = ft * BK + c * VEC;
      const int slot = kk / kSlot, t0 = kk % kSlot;
      float v[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[e] = 0.f;
      if (slot < nslot) {
        if (build_a) {
          float s = fscale[0];
          if (slot == 1) s = fscale[1];
          if (slot == 2) s = fscale[2];
#pragma unroll
          for (int e = 0; e < VEC; ++e) v[e] = s * Ts[ts_idx(slot, m, t0 + e)];
        } else {
          fb(m, slot, t0, v);
        }
      }
      *reinterpret_cast<u32x4*>((build_a ? FA : FBt) + lds_off(m, c)) = pack(v);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KSUB; ++ks) {
      Frag<T> af[kMB];
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) af[mb] = lds_frag<T>(FA, q.wm * 64 + mb * 16 + q.r16, ks, q.g);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const Frag<T> bfr = lds_frag<T>(FBt, q.wn * 128 + nb * 16 + q.r16, ks, q.g);
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) acc[mb][nb] = mma(acc[mb][nb], af[mb], bfr);
      }
    }
    __syncthreads();
  }
}

// Output column (within the tile) of LDS B row R.
__device__ __forceinline__ int lds_row_col(int lg, int R) { return (R >> 7) * 128 + perm_col(lg, R & 15, (R >> 4) & 7); }
// LDS B row of tile column n.
__device__ __forceinline__ int col_lds_row(int lg, int n) { return (n >> 7) * 128 + perm_row(lg, n & 127); }

// ---------------------------------------------------------------------------
// Loaders.
// ---------------------------------------------------------------------------

// A operand, register-staged: rows of a row-major matrix, optionally split
// along K into [A0 | A1] (A0 has K0 columns, A1 has K1; both row stride ld).
// Thread t stages chunk (t & 7) of rows (t >> 3) + 64 qq, qq = 0..3.
template <class T>
struct RowsA {
  static constexpr bool kDirect = false;
  const T* b0;
  const T* b1;
  long ld, K0, K1;
  int avail;        // rows available from this thread's first row
  bool vec;
  __device__ __forceinline__ void init(const T* A0, const T* A1, long Kd0, long Kd1, long lda, long M, long m0,
                                       bool v) {
    const int r0 = threadIdx.x >> 3;
    ld = lda; K0 = Kd0; K1 = Kd1; vec = v;
    avail = (int)min((long)(1 << 30), M - m0 - r0);
    b0 = (avail > 0) ? A0 + (m0 + r0) * lda : nullptr;
    b1 = (avail > 0 && A1) ? A1 + (m0 + r0) * lda : nullptr;
  }
  __device__ __forceinline__ u32x4 get(int qq, long k) const {
    constexpr int VEC = ET<T>::VEC;
    if (64 * qq >= avail) return zero4();
    const T* r0p = b0 + (long)(64 * qq) * ld;
    if (k + VEC <= K0 || b1 == nullptr) return gload<T>(r0p, k, K0, vec);
    const T* r1p = b1 + (long)(64 * qq) * ld;
    if (k >= K0) return gload<T>(r1p, k - K0, K1, vec);
    float v[VEC];   // a chunk straddling the seam
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const long kk = k + e;
      v[e] = (kk < K0) ? to_f<T>(r0p[kk]) : ((kk - K0 < K1) ? to_f<T>(r1p[kk - K0]) : 0.f);
    }
    return pack(v);
  }
  __device__ __forceinline__ void issue(int, char*) const {}
};

// A operand, direct to LDS.  Requires K0 % BK == 0 (each K tile inside one
// segment), 16-byte aligned rows, and every K tile full.  Rows past M are
// clamped to row M-1 (finite values; those rows are never stored and every
// row reduction masks them).
template <class T>
struct DirectA {
  static constexpr bool kDirect = true;
  const T* b0;
  const T* b1;
  long K0;
  int off[4];
  __device__ __forceinline__ void init(const T* A0, const T* A1, long Kd0, long, long lda, long M, long m0, bool) {
    b0 = A0; b1 = A1 ? A1 : A0; K0 = A1 ? Kd0 : (1L << 40);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      long row = m0 + direct_row(it);
      if (row > M - 1) row = M - 1;
      off[it] = (int)(row * lda);
    }
  }
  __device__ __forceinline__ u32x4 get(int, long) const { return zero4(); }
  __device__ __forceinline__ void issue(int kt, char* As) const {
    const int L = threadIdx.x & 63;
    long k = (long)kt * ET<T>::BK;
    const T* b = b0;
    if (k >= K0) { b = b1; k -= K0; }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int blk = direct_blk(it);
      g2lds16(b + off[it] + k + direct_chunk(L, blk) * ET<T>::VEC, As + blk * 1024);
    }
  }
};

// NK loader: A rows + B rows (output columns, row-major [n][K]) + side rows
// (adapter A_p rows [t][K]), all K-contiguous.  B row pointers are resolved
// once per tile by the kernel for the rows row_of(qq), qq = 0..3, of this
// thread.  With a direct A operand (AOp::kDirect) the B rows are also loaded
// straight into LDS; a nullptr B row then falls back to `bfallback` (a valid
// row whose output columns are never stored).  Side rows (one chunk per
// thread for threads < 128 * NSIDE) are register-staged and zero-filled past
// the rank.
template <class T, class AOp, int NSIDE>
struct NKLoader {
  static constexpr bool DIRECT = AOp::kDirect;
  AOp a;
  const T* brow[4];
  const T* bfallback;
  const T* srow;
  long K;
  bool vecB, vecS;
  unsigned smask;
  u32x4 ra[DIRECT ? 1 : 4], rb[DIRECT ? 1 : 4], rs;
  __device__ static __forceinline__ int row_of(int qq) {
    return DIRECT ? direct_row(qq) : (int)(threadIdx.x >> 3) + 64 * qq;
  }
  // Side row this thread stages (>= 16 * NSIDE: none).
  __device__ static __forceinline__ int side_row() { return (int)(threadIdx.x >> 3); }
  __device__ __forceinline__ void issue(int kt, char* As, char* Bs) const {
    if constexpr (DIRECT) {
      a.issue(kt, As);
      const int L = threadIdx.x & 63;
      const long k = (long)kt * ET<T>::BK;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int blk = direct_blk(it);
        const T* p = brow[it] ? brow[it] : bfallback;
        g2lds16(p + k + direct_chunk(L, blk) * ET<T>::VEC, Bs + blk * 1024);
      }
    }
  }
  __device__ __forceinline__ void load(int kt) {
    const long k = (long)kt * ET<T>::BK + (threadIdx.x & 7) * ET<T>::VEC;
    if constexpr (!DIRECT) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) ra[qq] = a.get(qq, k);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) rb[qq] = gload<T>(brow[qq], k, K, vecB);
    }
    if constexpr (NSIDE > 0) rs = gload<T>(srow, k, K, vecS);
  }
  __device__ __forceinline__ void store(char* As, char* Bs) const {
    const int c = threadIdx.x & 7, r0 = threadIdx.x >> 3;
    if constexpr (!DIRECT) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) *reinterpret_cast<u32x4*>(As + lds_off(r0 + 64 * qq, c)) = ra[qq];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) *reinterpret_cast<u32x4*>(Bs + lds_off(r0 + 64 * qq, c)) = rb[qq];
    }
    if constexpr (NSIDE > 0)
      if (r0 < NSIDE * 16) *reinterpret_cast<u32x4*>(Bs + lds_off(kBN + r0, c)) = rs;
  }
  __device__ __forceinline__ unsigned side_mask(int) const { return smask; }
};

// Transpose helpers: 4 rows x 8 bf16 -> 8 columns x 4 rows (u32x2 each), and 4x4 fp32.
__device__ __forceinline__ void transpose4x8_bf16(const u32x4 (&in)[4], u32x2 (&out)[8]) {
  const unsigned* w = reinterpret_cast<const unsigned*>(in);   // w[k*4 + n/2]
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const unsigned a0 = w[0 * 4 + n / 2], a1 = w[1 * 4 + n / 2], a2 = w[2 * 4 + n / 2], a3 = w[3 * 4 + n / 2];
    if (n & 1) {
      out[n].x = (a0 >> 16) | (a1 & 0xffff0000u);
      out[n].y = (a2 >> 16) | (a3 & 0xffff0000u);
    } else {
      out[n].x = (a0 & 0xffffu) | (a1 << 16);
      out[n].y = (a2 & 0xffffu) | (a3 << 16);
    }
  }
}
__device__ __forceinline__ void transpose4x4_f32(const u32x4 (&in)[4], u32x4 (&out)[4]) {
  out[0] = (u32x4){in[0].x, in[1].x, in[2].x, in[3].x};
  out[1] = (u32x4){in[0].y, in[1].y, in[2].y, in[3].y};
  out[2] = (u32x4){in[0].z, in[1].z, in[2].z, in[3].z};
  out[3] = (u32x4){in[0].w, in[1].w, in[2].w, in[3].w};
}

// KN loader: A rows (token-major) + B stored [K][N] (N contiguous, e.g. W_d
// for dH = dY W_d) transposed into LDS rows while staging, + optional side
// operands stored [K][r] (e.g. B_g for dT_g = dG B_g).
//   krow(k)        -> pointer to row k of the B matrix (nullptr past K)
//   srow(sb, k)    -> pointer to row k of side operand sb (nullptr if inactive)
//   smask_of(kt)   -> active side blocks in tile kt
// Output columns n0 .. n0+255 (bounded by N) go to LDS rows col_lds_row(0, n).
// Each thread stages a 4 (k) x 8 (n) bf16 block (4 x 4 for fp32).
template <class T, class AOp, int NSIDE, class KRow, class SRow, class SMask>
struct KNLoader {
  static constexpr bool DIRECT = AOp::kDirect;
  static constexpr int VEC = ET<T>::VEC, BK = ET<T>::BK;
  AOp a;
  KRow krow;
  SRow srow;
  SMask smask_of;
  long n0, N;
  bool vecB;
  int r;            // adapter rank (side columns beyond r are zero)
  bool vecS;
  u32x4 ra[DIRECT ? 1 : 4];
  u32x4 rb[4];
  u32x4 rs;
  __device__ __forceinline__ void issue(int kt, char* As, char*) const {
    if constexpr (DIRECT) a.issue(kt, As);
  }
  __device__ __forceinline__ void load(int kt) {
    const int tid = threadIdx.x;
    const long k = (long)kt * BK + (tid & 7) * VEC;
    if constexpr (!DIRECT) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) ra[qq] = a.get(qq, k);
    }
    if constexpr (sizeof(T) == 2) {
      const int ng = tid & 31, kg = tid >> 5;              // 8 columns, rows 4 kg .. 4 kg + 3
#pragma unroll
      for (int i = 0; i < 4; ++i) rb[i] = gload<T>(krow((long)kt * BK + kg * 4 + i), n0 + ng * 8, N, vecB);
    } else {
      const int ng = tid & 63, kg = tid >> 6;              // 4 columns, rows 4 kg .. 4 kg + 3
#pragma unroll
      for (int i = 0; i < 4; ++i) rb[i] = gload<T>(krow((long)kt * BK + kg * 4 + i), n0 + ng * 4, N, vecB);
    }
    if constexpr (NSIDE > 0) {
      // side block sb is staged by threads [128 sb, 128 sb + 128)
      const int sb = tid >> 7, tt = tid & 127;
      rs = zero4();
      if (sb < NSIDE) {
        if constexpr (sizeof(T) == 2) rs = gload<T>(srow(sb, (long)kt * BK + (tt >> 1)), (tt & 1) * 8, r, vecS);
        else rs = gload<T>(srow(sb, (long)kt * BK + (tt >> 2)), (tt & 3) * 4, r, vecS);
      }
    }
  }
  __device__ __forceinline__ void store(char* As, char* Bs) const {
    const int tid = threadIdx.x;
    const int c = tid & 7, r0 = tid >> 3;
    if constexpr (!DIRECT) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) *reinterpret_cast<u32x4*>(As + lds_off(r0 + 64 * qq, c)) = ra[qq];
    }
    if constexpr (sizeof(T) == 2) {
      const int ng = tid & 31, kg = tid >> 5;
      u32x2 cols[8];
      transpose4x8_bf16(rb, cols);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<u32x2*>(Bs + lds_off(col_lds_row(0, ng * 8 + i), kg >> 1) + (kg & 1) * 8) = cols[i];
    } else {
      const int ng = tid & 63, kg = tid >> 6;
      u32x4 cols[4];
      transpose4x4_f32(rb, cols);
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(Bs + lds_off(col_lds_row(0, ng * 4 + i), kg)) = cols[i];
    }
    if constexpr (NSIDE > 0) {
      const int sb = tid >> 7, tt = tid & 127;
      if (sb < NSIDE) {
        // rs holds ranks t0 .. t0+VEC-1 of one k: scatter into rows kBN + 16 sb + t.
        const unsigned* wv = reinterpret_cast<const unsigned*>(&rs);
        if constexpr (sizeof(T) == 2) {
          const int kk = tt >> 1, t0 = (tt & 1) * 8;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const unsigned short h = (e & 1) ? (unsigned short)(wv[e >> 1] >> 16) : (unsigned short)(wv[e >> 1] & 0xffffu);
            *reinterpret_cast<unsigned short*>(Bs + lds_off(kBN + sb * 16 + t0 + e, kk >> 3) + (kk & 7) * 2) = h;
          }
        } else {
          const int kk = tt >> 2, t0 = (tt & 3) * 4;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            *reinterpret_cast<unsigned*>(Bs + lds_off(kBN + sb * 16 + t0 + e, kk >> 2) + (kk & 3) * 4) = wv[e];
        }
      }
    }
  }
  __device__ __forceinline__ unsigned side_mask(int kt) const { return smask_of(kt); }
};

// Store 8 consecutive values of one row (16-byte bf16 store, or 2 x 16 bytes fp32).
template <class T>
__device__ __forceinline__ void store_row8(T* p, const float (&v)[8], int n, bool vec) {
  if constexpr (sizeof(T) == 2) {
    gstore<T, 8>(p, v, n, vec);
  } else {
    const float lo[4] = {v[0], v[1], v[2], v[3]};
    const float hi[4] = {v[4], v[5], v[6], v[7]};
    gstore<T, 4>(p, lo, min(n, 4), vec);
    gstore<T, 4>(p + 4, hi, n - 4, vec);
  }
}

// Load 8 consecutive values of one row as floats (zero past len).
template <class T>
__device__ __forceinline__ void load_row8(const T* row, long c0, long len, bool vec, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    unpack(gload<T>(row, c0, len, vec), v);
  } else {
    float t4[4];
    unpack(gload<T>(row, c0, len, vec), t4);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = t4[e];
    unpack(gload<T>(row, c0 + 4, len, vec), t4);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 + e] = t4[e];
  }
}

// Row maps for KN loaders (default-constructible functors).
template <class T>
struct KRow1 {                // rows of one [K][ld] matrix
  const T* W; long K, ld;
  __device__ __forceinline__ const T* operator()(long k) const { return (k < K) ? W + k * ld : nullptr; }
};
template <class T>
struct KRow2 {                // [W0; W1] stacked along K
  const T* W0; const T* W1; long K0, K1, ld;
  __device__ __forceinline__ const T* operator()(long k) const {
    return (k < K0) ? W0 + k * ld : ((k < K0 + K1) ? W1 + (k - K0) * ld : nullptr);
  }
};
template <class T>
struct KRow3 {                // [W0; W1; W2] stacked along K, boundaries o1 < o2 < o3
  const T* W0; const T* W1; const T* W2; long o1, o2, o3, ld;
  __device__ __forceinline__ const T* operator()(long k) const {
    if (k < o1) return W0 + k * ld;
    if (k < o2) return W1 + (k - o1) * ld;
    if (k < o3) return W2 + (k - o2) * ld;
    return nullptr;
  }
};
template <class T>
struct SRowNone {
  __device__ __forceinline__ const T* operator()(int, long) const { return nullptr; }
};
template <class T>
struct SRow2 {                // side block b: rows k - lo[b] of B[b] for lo[b] <= k < hi[b]
  const T* B0; const T* B1; long lo0, hi0, lo1, hi1, ld;
  __device__ __forceinline__ const T* operator()(int sb, long k) const {
    if (sb == 0) return (k >= lo0 && k < hi0) ? B0 + (k - lo0) * ld : nullptr;
    return (k >= lo1 && k < hi1) ? B1 + (k - lo1) * ld : nullptr;
  }
};
struct SMaskNone {
  __device__ __forceinline__ unsigned operator()(int) const { return 0u; }
};
struct SMask2 {               // block 0 active while the tile overlaps [0, K0), block 1 beyond
  long K0; int BK;
  __device__ __forceinline__ unsigned operator()(int kt) const {
    return (((long)kt * BK < K0) ? 1u : 0u) | (((long)(kt + 1) * BK > K0) ? 2u : 0u);
  }
};

// ---------------------------------------------------------------------------
// Epilogue helper: per-wave partial P[t][col] = sum over the wave's 64 rows
// of Aop[row][t] * V[row][col], as MFMAs with K = rows.  The A fragment of
// row pair (mb, mb+1) takes rows 16mb+4g+j and 16(mb+1)+4g+j (j = 0..3) as
// its 8 K slots, which is exactly what a lane holds of V in C layout, so V
// needs no shuffles.  Results stay in C layout: lane holds P[4g+j][col(r16, nb)].
// ---------------------------------------------------------------------------
template <class T>
__device__ __forceinline__ Frag<T> ts_frag(const float* Ts, int slot, float scale, const WaveId& q, int mp) {
  float v[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = scale * Ts[ts_idx(slot, acc_row(q, 2 * mp, j), q.r16)];
    v[4 + j] = scale * Ts[ts_idx(slot, acc_row(q, 2 * mp + 1, j), q.r16)];
  }
  return make_frag<T>(v);
}

// Sum of NOUT partial tiles [16 t][128 cols] over the four wave-rows (fixed
// order wm = 3, 2, 1, 0) and store of the row-block partial to
// part[o] + col * 16 + t (cols bounded by ncols).  Lane column layout: G = 1
// (tile column wn*128 + 8*r16 + nb).
template <int NOUT>
__device__ __forceinline__ void reduce_store_partials(char* smem, f32x4 (&pacc)[NOUT][8], float* const (&part)[NOUT],
                                                      long n0, long ncols) {
  const WaveId q = wave_id();
  float* red = reinterpret_cast<float*>(smem + kRedOff);
  static_assert(NOUT * 2 * 128 * 16 * 4 <= kRedBytes, "reduction scratch too small");
  auto slot = [&](int o, int nb) -> f32x4* {
    return reinterpret_cast<f32x4*>(red + ((o * 2 + q.wn) * 128 + perm_col(0, q.r16, nb)) * 16 + 4 * q.g);
  };
  __syncthreads();
  if (q.wm == 3) {
#pragma unroll
    for (int o = 0; o < NOUT; ++o)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) *slot(o, nb) = pacc[o][nb];
  }
#pragma unroll
  for (int step = 2; step >= 1; --step) {
    __syncthreads();
    if (q.wm == step) {
#pragma unroll
      for (int o = 0; o < NOUT; ++o)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) *slot(o, nb) = *slot(o, nb) + pacc[o][nb];
    }
  }
  __syncthreads();
  if (q.wm == 0) {
#pragma unroll
    for (int o = 0; o < NOUT; ++o)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const f32x4 v = *slot(o, nb) + pacc[o][nb];
        const long col = n0 + q.wn * 128 + perm_col(0, q.r16, nb);
        if (col < ncols) *reinterpret_cast<f32x4*>(part[o] + col * 16 + 4 * q.g) = v;
      }
  }
}

}  // namespace lora

// The LoRA-augmented MFMA GEMM core: a 256x256 output tile per workgroup of
// four waves (2 x 2, each wave 128 x 128 = 8 x 8 MFMA blocks of 16 x 16).
//
//   acc  = Z_tile . Bop_tile                       (K-loop, bf16 or fp32 MFMA)
//   side = Z_tile . Sop^T                          (same K-loop, same A fragments:
//                                                   the rank-r product, <= 3 adapters)
//   acc += [s_1 T_1 | s_2 T_2 | ...] . [F_1 ; F_2 ; ...]   (the fold: extra K steps)
//
// The side product rides along the base GEMM's K-loop: its operand rows sit
// in LDS right after the B tile and reuse the A fragments already in
// registers, so X (or H, or dG|dU) is read once for both.  Each wave of a
// wave-row computes the side product on one of the two 32-wide K sub-steps of
// a tile (bf16), which splits that work evenly; the two halves are summed
// through LDS after the loop.
//
// LDS during the K-loop: two stages of [A 256 rows | B 256 rows | side 48 rows]
// x 128 bytes.  After the loop the same memory holds: Ts (float side products,
// [3][256][16]), the fold A tile and the fold B tile; epilogues reuse the fold
// tiles for cross-wave reductions.
#pragma once

#include "common.h"

namespace lora {

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

__device__ __forceinline__ float* ts_ptr(char* smem) { return reinterpret_cast<float*>(smem + kTsOff); }
__device__ __forceinline__ int ts_idx(int slot, int row, int t) { return (slot * kBM + row) * kSlot + t; }

// ---------------------------------------------------------------------------
// K-loop.  Loader interface:
//   load(kt)                 global -> registers for K tile kt
//   store(As, Bs)            registers -> LDS stage (A rows, B rows, side rows)
//   side_mask(kt)            bit sb set when side block sb has data in tile kt
// ---------------------------------------------------------------------------
template <class T, int NSIDE, class Loader>
__device__ __forceinline__ void kloop(char* smem, int nkt, Loader& ld, f32x4 (&acc)[8][8],
                                      f32x4 (&sacc)[NSIDE > 0 ? NSIDE : 1][8]) {
  constexpr int KSUB = ET<T>::KSUB;
  const WaveId q = wave_id();
  if (nkt <= 0) return;
  ld.load(0);
  ld.store(smem, smem + kABytes);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const char* As = smem + (kt & 1) * kStage;
    const char* Bs = As + kABytes;
    const bool more = kt + 1 < nkt;
    if (more) ld.load(kt + 1);
    unsigned smask = 0u;
    if constexpr (NSIDE > 0) smask = ld.side_mask(kt);
#pragma unroll
    for (int ks = 0; ks < KSUB; ++ks) {
      Frag<T> af[8];
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) af[mb] = lds_frag<T>(As, q.wm * 128 + mb * 16 + q.r16, ks, q.g);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const Frag<T> bfr = lds_frag<T>(Bs, q.wn * 128 + nb * 16 + q.r16, ks, q.g);
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) acc[mb][nb] = mma(acc[mb][nb], af[mb], bfr);
      }
      if constexpr (NSIDE > 0) {
        const bool mine = (KSUB == 2) ? (ks == q.wn) : (q.wn == 0);
        if (mine) {
#pragma unroll
          for (int sb = 0; sb < NSIDE; ++sb) {
            if ((smask >> sb) & 1u) {
              const Frag<T> bfr = lds_frag<T>(Bs, kBN + sb * 16 + q.r16, ks, q.g);
#pragma unroll
              for (int mb = 0; mb < 8; ++mb) sacc[sb][mb] = mma(sacc[sb][mb], af[mb], bfr);
            }
          }
        }
      }
    }
    if (more) {
      char* An = smem + ((kt + 1) & 1) * kStage;
      ld.store(An, An + kABytes);
    }
    __syncthreads();
  }
}

__device__ __forceinline__ void zero_acc(f32x4 (&acc)[8][8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
}

// Sum the per-wave side products into Ts[sb][row][t] (float, raw Z.Sop^T).
// Must follow the K-loop's final barrier.  The fold reads only slots < NSIDE.
template <class T, int NSIDE>
__device__ __forceinline__ void side_reduce(char* smem, f32x4 (&sacc)[NSIDE > 0 ? NSIDE : 1][8]) {
  const WaveId q = wave_id();
  float* Ts = ts_ptr(smem);
  constexpr bool two = ET<T>::KSUB == 2;
  if (q.wn == 0) {
#pragma unroll
    for (int sb = 0; sb < NSIDE; ++sb)
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          Ts[ts_idx(sb, q.wm * 128 + mb * 16 + 4 * q.g + j, q.r16)] = sacc[sb][mb][j];
  }
  __syncthreads();
  if (two && q.wn == 1) {
#pragma unroll
    for (int sb = 0; sb < NSIDE; ++sb)
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          Ts[ts_idx(sb, q.wm * 128 + mb * 16 + 4 * q.g + j, q.r16)] += sacc[sb][mb][j];
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Fold: acc += FA . FB^T with FA[m][16 s + t] = fscale[s] * Ts[s][m][t] and
// FB[n][16 s + t] supplied by the kernel (adapter s's fold operand for output
// column n).  One fold tile holds BK / 16 slots (4 for bf16, 2 for fp32).
// FB functor: fb(R, slot, t0, v) fills v[0..VEC) for LDS row R (a permuted
// output column), adapter slot `slot`, ranks t0..t0+VEC-1; v is pre-zeroed.
// ---------------------------------------------------------------------------
template <class T, class FB>
__device__ __forceinline__ void fold(char* smem, f32x4 (&acc)[8][8], int nslot, const float (&fscale)[kMaxSide],
                                     FB& fb) {
  constexpr int VEC = ET<T>::VEC, BK = ET<T>::BK, KSUB = ET<T>::KSUB;
  const WaveId q = wave_id();
  if (nslot <= 0) return;
  const int nft = (nslot * kSlot + BK - 1) / BK;
  const float* Ts = ts_ptr(smem);
  char* FA = smem + kFAOff;
  char* FBt = smem + kFBOff;
  for (int ft = 0; ft < nft; ++ft) {
    const int m = q.tid;   // one tile row per thread
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int kk = ft * BK + c * VEC;
      const int slot = kk / kSlot, t0 = kk % kSlot;
      float va[VEC], vb[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) { va[e] = 0.f; vb[e] = 0.f; }
      if (slot < nslot) {
        float s = fscale[0];
        if (slot == 1) s = fscale[1];
        if (slot == 2) s = fscale[2];
#pragma unroll
        for (int e = 0; e < VEC; ++e) va[e] = s * Ts[ts_idx(slot, m, t0 + e)];
        fb(m, slot, t0, vb);
      }
      *reinterpret_cast<u32x4*>(FA + lds_off(m, c)) = pack(va);
      *reinterpret_cast<u32x4*>(FBt + lds_off(m, c)) = pack(vb);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KSUB; ++ks) {
      Frag<T> af[8];
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) af[mb] = lds_frag<T>(FA, q.wm * 128 + mb * 16 + q.r16, ks, q.g);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const Frag<T> bfr = lds_frag<T>(FBt, q.wn * 128 + nb * 16 + q.r16, ks, q.g);
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) acc[mb][nb] = mma(acc[mb][nb], af[mb], bfr);
      }
    }
    __syncthreads();
  }
}

// Output column (within the 256-wide tile) held by lane column r16 in block nb.
__device__ __forceinline__ int tile_col(int lg, int wn, int r16, int nb) { return wn * 128 + perm_col(lg, r16, nb); }
// Output column (within the tile) of LDS B row R.
__device__ __forceinline__ int lds_row_col(int lg, int R) { return (R >> 7) * 128 + perm_col(lg, R & 15, (R >> 4) & 7); }
// LDS B row of tile column n.
__device__ __forceinline__ int col_lds_row(int lg, int n) { return (n >> 7) * 128 + perm_row(lg, n & 127); }

// ---------------------------------------------------------------------------
// Loaders.
// ---------------------------------------------------------------------------

// A operand rows: a row-major [M, K] matrix; tile rows m0 .. m0+255.
template <class T>
struct RowsA {
  const T* base;    // row (m0 + (tid >> 3)), or nullptr when past M
  long ld;
  int avail;        // rows available from base (M - m0 - (tid >> 3))
  long K;
  bool vec;
  __device__ __forceinline__ void init(const T* A, long lda, long M, long m0, long Kdim, bool v) {
    const int r0 = threadIdx.x >> 3;
    ld = lda;
    K = Kdim;
    vec = v;
    avail = (int)min((long)(1 << 30), M - m0 - r0);
    base = (avail > 0) ? A + (m0 + r0) * lda : nullptr;
  }
  __device__ __forceinline__ u32x4 get(int qq, long k) const {
    return gload<T>((32 * qq < avail) ? base + (long)(32 * qq) * ld : nullptr, k, K, vec);
  }
};

// A operand = [A0 | A1] concatenated along K (A0 has K0 columns, A1 has K1).
template <class T>
struct SplitRowsA {
  const T* b0;
  const T* b1;
  long ld0, ld1;
  int avail;
  long K0, K1;
  bool vec;
  __device__ __forceinline__ void init(const T* A0, long lda0, long Kd0, const T* A1, long lda1, long Kd1, long M,
                                       long m0, bool v) {
    const int r0 = threadIdx.x >> 3;
    ld0 = lda0; ld1 = lda1; K0 = Kd0; K1 = Kd1; vec = v;
    avail = (int)min((long)(1 << 30), M - m0 - r0);
    b0 = (avail > 0) ? A0 + (m0 + r0) * lda0 : nullptr;
    b1 = (avail > 0) ? A1 + (m0 + r0) * lda1 : nullptr;
  }
  __device__ __forceinline__ u32x4 get(int qq, long k) const {
    constexpr int VEC = ET<T>::VEC;
    if (32 * qq >= avail) return zero4();
    const T* r0p = b0 + (long)(32 * qq) * ld0;
    const T* r1p = b1 + (long)(32 * qq) * ld1;
    if (k + VEC <= K0) return gload<T>(r0p, k, K0, vec);
    if (k >= K0) return gload<T>(r1p, k - K0, K1, vec);
    float v[VEC];   // a chunk straddling the seam
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const long kk = k + e;
      v[e] = (kk < K0) ? to_f<T>(r0p[kk]) : ((kk - K0 < K1) ? to_f<T>(r1p[kk - K0]) : 0.f);
    }
    return pack(v);
  }
};

// NK loader: A rows + B rows (output columns, row-major [n][K]) + side rows
// (adapter A_p rows [t][K]), all K-contiguous.  B and side row pointers are
// resolved once per tile by the kernel.
template <class T, class AOp, int NSIDE>
struct NKLoader {
  static constexpr int NSQ = (NSIDE * 16 * 8 + kThreads - 1) / kThreads;   // side chunks per thread
  AOp a;
  const T* brow[8];
  const T* srow[NSQ > 0 ? NSQ : 1];
  long K;
  bool vecB, vecS;
  unsigned smask;
  u32x4 ra[8], rb[8], rs[NSQ > 0 ? NSQ : 1];
  __device__ __forceinline__ void load(int kt) {
    const long k = (long)kt * ET<T>::BK + (threadIdx.x & 7) * ET<T>::VEC;
#pragma unroll
    for (int qq = 0; qq < 8; ++qq) ra[qq] = a.get(qq, k);
#pragma unroll
    for (int qq = 0; qq < 8; ++qq) rb[qq] = gload<T>(brow[qq], k, K, vecB);
#pragma unroll
    for (int qq = 0; qq < NSQ; ++qq) rs[qq] = gload<T>(srow[qq], k, K, vecS);
  }
  __device__ __forceinline__ void store(char* As, char* Bs) const {
    const int c = threadIdx.x & 7, r0 = threadIdx.x >> 3;
#pragma unroll
    for (int qq = 0; qq < 8; ++qq) *reinterpret_cast<u32x4*>(As + lds_off(r0 + 32 * qq, c)) = ra[qq];
#pragma unroll
    for (int qq = 0; qq < 8; ++qq) *reinterpret_cast<u32x4*>(Bs + lds_off(r0 + 32 * qq, c)) = rb[qq];
#pragma unroll
    for (int qq = 0; qq < NSQ; ++qq) {
      const int sr = r0 + 32 * qq;
      if (sr < NSIDE * 16) *reinterpret_cast<u32x4*>(Bs + lds_off(kBN + sr, c)) = rs[qq];
    }
  }
  __device__ __forceinline__ unsigned side_mask(int) const { return smask; }
};

// Transpose helpers for KN tiles: 8x8 bf16 (rows k, columns n) -> 8 column chunks.
__device__ __forceinline__ void transpose8x8_bf16(const u32x4 (&in)[8], u32x4 (&out)[8]) {
  const unsigned* w = reinterpret_cast<const unsigned*>(in);   // w[k*4 + n/2]
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    unsigned d[4];
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const unsigned a = w[(2 * qd) * 4 + n / 2], b = w[(2 * qd + 1) * 4 + n / 2];
      d[qd] = (n & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    out[n] = (u32x4){d[0], d[1], d[2], d[3]};
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
template <class T, class AOp, int NSIDE, class KRow, class SRow, class SMask>
struct KNLoader {
  static constexpr int VEC = ET<T>::VEC, BK = ET<T>::BK;
  static constexpr int NB = (sizeof(T) == 2) ? 1 : 2;     // transpose blocks per thread
  static constexpr int BR = (sizeof(T) == 2) ? 8 : 4;     // rows (k) per block
  AOp a;
  KRow krow;
  SRow srow;
  SMask smask_of;
  long n0, N;
  bool vecB;
  int r;            // adapter rank (side columns beyond r are zero)
  bool vecS;
  u32x4 ra[8];
  u32x4 rb[NB][BR];
  u32x4 rs[NSIDE > 0 ? NSIDE : 1];
  int kt_cur;
  __device__ __forceinline__ void load(int kt) {
    const int tid = threadIdx.x;
    kt_cur = kt;
    const long k = (long)kt * BK + (tid & 7) * VEC;
#pragma unroll
    for (int qq = 0; qq < 8; ++qq) ra[qq] = a.get(qq, k);
    if constexpr (sizeof(T) == 2) {
      const int ng = tid & 31, kg = tid >> 5;
#pragma unroll
      for (int i = 0; i < 8; ++i) rb[0][i] = gload<T>(krow((long)kt * BK + kg * 8 + i), n0 + ng * 8, N, vecB);
    } else {
      const int ng = tid & 63;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int kg = (tid >> 6) + 4 * b;
#pragma unroll
        for (int i = 0; i < 4; ++i) rb[b][i] = gload<T>(krow((long)kt * BK + kg * 4 + i), n0 + ng * 4, N, vecB);
      }
    }
    if constexpr (NSIDE > 0) {
      // side block sb uses threads [128*(sb&1), +128) ; sb = 2 shares with sb = 0 (second pass)
#pragma unroll
      for (int sb = 0; sb < NSIDE; ++sb) {
        const int tt = tid - 128 * (sb & 1);
        rs[sb] = zero4();
        if (tt >= 0 && tt < 128) {
          if constexpr (sizeof(T) == 2) {
            const long kk = (long)kt * BK + (tt >> 1);
            rs[sb] = gload<T>(srow(sb, kk), (tt & 1) * 8, r, vecS);
          } else {
            const long kk = (long)kt * BK + (tt >> 2);
            rs[sb] = gload<T>(srow(sb, kk), (tt & 3) * 4, r, vecS);
          }
        }
      }
    }
  }
  __device__ __forceinline__ void store(char* As, char* Bs) const {
    const int tid = threadIdx.x;
    const int c = tid & 7, r0 = tid >> 3;
#pragma unroll
    for (int qq = 0; qq < 8; ++qq) *reinterpret_cast<u32x4*>(As + lds_off(r0 + 32 * qq, c)) = ra[qq];
    if constexpr (sizeof(T) == 2) {
      const int ng = tid & 31, kg = tid >> 5;
      u32x4 cols[8];
      transpose8x8_bf16(rb[0], cols);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<u32x4*>(Bs + lds_off(col_lds_row(0, ng * 8 + i), kg)) = cols[i];
    } else {
      const int ng = tid & 63;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int kg = (tid >> 6) + 4 * b;
        u32x4 cols[4];
        transpose4x4_f32(rb[b], cols);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<u32x4*>(Bs + lds_off(col_lds_row(0, ng * 4 + i), kg)) = cols[i];
      }
    }
    if constexpr (NSIDE > 0) {
#pragma unroll
      for (int sb = 0; sb < NSIDE; ++sb) {
        const int tt = tid - 128 * (sb & 1);
        if (tt >= 0 && tt < 128) {
          // rs[sb] holds ranks t0 .. t0+VEC-1 of one k: scatter into rows kBN + 16 sb + t.
          const unsigned* wv = reinterpret_cast<const unsigned*>(&rs[sb]);
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
struct SRow2 {                // side block 0: B0 rows for k < K0; block 1: B1 rows for K0 <= k < K0+K1
  const T* B0; const T* B1; long K0, K1, ld;
  __device__ __forceinline__ const T* operator()(int sb, long k) const {
    if (sb == 0) return (k < K0) ? B0 + k * ld : nullptr;
    return (k >= K0 && k < K0 + K1) ? B1 + (k - K0) * ld : nullptr;
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
// Epilogue helper: per-wave partial P[t][col] = sum over the wave's 128 rows
// of Aop[row][t] * V[row][col], as MFMAs with K = rows.  The A fragment of
// row pair (mb, mb+1) takes rows 16mb+4g+j and 16(mb+1)+4g+j (j = 0..3) as
// its 8 K slots, which is exactly what a lane holds of V in C layout, so V
// needs no shuffles.  Results stay in C layout: lane holds P[4g+j][col(r16, nb)].
// ---------------------------------------------------------------------------
template <class T>
__device__ __forceinline__ Frag<T> ts_frag(const float* Ts, int slot, float scale, int wm, int mp, int g, int r16) {
  float v[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = scale * Ts[ts_idx(slot, wm * 128 + (2 * mp) * 16 + 4 * g + j, r16)];
    v[4 + j] = scale * Ts[ts_idx(slot, wm * 128 + (2 * mp + 1) * 16 + 4 * g + j, r16)];
  }
  return make_frag<T>(v);
}

// Cross-wave (wm = 0, 1) sum of NOUT partial tiles [16 t][128 cols] and store
// of the row-block partial to part[o] + col * 16 + t (cols bounded by ncols).
// Lane column layout: G = 1 (tile column wn*128 + 8*r16 + nb).
template <int NOUT>
__device__ __forceinline__ void reduce_store_partials(char* smem, f32x4 (&pacc)[NOUT][8], float* const (&part)[NOUT],
                                                      long n0, long ncols) {
  const WaveId q = wave_id();
  float* red = reinterpret_cast<float*>(smem + kRedOff);
  static_assert(NOUT * 2 * 128 * 16 * 4 <= kRedBytes, "reduction scratch too small");
  __syncthreads();
  if (q.wm == 1) {
#pragma unroll
    for (int o = 0; o < NOUT; ++o)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int wc = perm_col(0, q.r16, nb);
        *reinterpret_cast<f32x4*>(red + ((o * 2 + q.wn) * 128 + wc) * 16 + 4 * q.g) = pacc[o][nb];
      }
  }
  __syncthreads();
  if (q.wm == 0) {
#pragma unroll
    for (int o = 0; o < NOUT; ++o)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int wc = perm_col(0, q.r16, nb);
        const f32x4 other = *reinterpret_cast<const f32x4*>(red + ((o * 2 + q.wn) * 128 + wc) * 16 + 4 * q.g);
        const f32x4 v = pacc[o][nb] + other;
        const long col = n0 + q.wn * 128 + wc;
        if (col < ncols) *reinterpret_cast<f32x4*>(part[o] + col * 16 + 4 * q.g) = v;
      }
  }
}

}  // namespace lora

// Backward kernels (base weights frozen: no dW anywhere).
//
// LoRA linear backward for the loss <dY, Y> (Opake "Model Patches and
// Kernels", "Fused LoRA operations"; frozen weights get no gradient per
// "Fused linear cross-entropy", key design decisions):
//   dT = s dY B,  dB = s dY^T T,  dA = dT^T Z,  dZ = dY W + dT A.
// GLU backward ("Activation functions": reads dH, G, U; writes dG, dU):
//   dG = dH * U * phi'(G),  dU = dH * phi(G).
// RoPE backward: the adjoint rotation R^T (rotation by -angle) applied to dQ, dK.
//
// Kernels:
//   k_bwd_prologue  one pass over the upstream gradient P (dY, or dQ/dK/dV
//                   un-rotated and un-split into token-major dP):
//                   dT_p = s_p P_p B_p (partials over column ranges) and
//                   dB_p = s_p P_p^T T_p (partials over row blocks), MFMA.
//   k_down_bwd      dH = dY W_d + dT_d A_d (K = h), GLU backward in the
//                   epilogue, plus row-block partials of dA_d, dB_g, dB_u.
//   k_mlp_dx_bwd    dX = [dG|dU] [W_g; W_u] + dT_g A_g + dT_u A_u (K = 2i);
//                   dT_g, dT_u ride the K-loop; partials of dA_g, dA_u.
//   k_proj_dx_bwd   dX = dP [W_q; W_k; W_v] + sum_p dT_p A_p (or one LoRA linear's
//                   dX = dY W + dT A); partials of dA_p.
//   k_reduce        fixed-order sum of partials -> dA / dB in the call dtype.
#pragma once

#include <type_traits>

#include "gemm.h"

namespace lora {

// ===========================================================================
// Prologue
// ===========================================================================
struct ProArgs {
  int qkv;                      // 0: P = dY [N][O];  1: P gathered from dQ/dK/dV
  const void* P;
  const void* src[3];           // dQ, dK, dV as [B][heads][S][d]
  const float* cs; const float* sn;
  int S, d;
  int nh[3];
  void* dP;                     // qkv: token-major dP [N][O]
  const void* Bp[3];            // [O_p][r]
  const float* Tp[3];           // saved T_p [N][r]
  float s[3];
  int off[4];                   // adapter column ranges
  int nadp;
  float* dT_part;               // [NCR][3][N][16]
  float* dB_part;               // [R][O][16]
  long N; int O, r;
  int NCH, CPC, NCR;
  int vecP, vecB;
};

// The prologue's LDS tiles use 128-byte rows (64 bf16 / 32 fp32 along K),
// eight 16-byte chunks XOR-swizzled with row & 7, and MFMA K-steps of 32 bf16
// (two per row) or 8 x 4 fp32: its chunking of the column range is
// independent of the GEMM core's.
constexpr int kPRowBytes = 128;
template <class T> struct PT;
template <> struct PT<bf16> { static constexpr int VEC = 8, BK = 64, KSUB = 2; };
template <> struct PT<float> { static constexpr int VEC = 4, BK = 32, KSUB = 1; };
__device__ __forceinline__ int p_off(int row, int chunk) { return row * kPRowBytes + ((chunk ^ (row & 7)) << 4); }
template <class T> struct PFrag;
template <> struct PFrag<bf16> { u32x4 v; };
template <> struct PFrag<float> { u32x4 v0, v1; };
template <class T> __device__ __forceinline__ PFrag<T> p_frag(const char* buf, int row, int ks, int g);
template <> __device__ __forceinline__ PFrag<bf16> p_frag<bf16>(const char* buf, int row, int ks, int g) {
  PFrag<bf16> f;
  f.v = *reinterpret_cast<const u32x4*>(buf + p_off(row, ks * 4 + g));
  return f;
}
template <> __device__ __forceinline__ PFrag<float> p_frag<float>(const char* buf, int row, int, int g) {
  PFrag<float> f;
  f.v0 = *reinterpret_cast<const u32x4*>(buf + p_off(row, 2 * g));
  f.v1 = *reinterpret_cast<const u32x4*>(buf + p_off(row, 2 * g + 1));
  return f;
}
__device__ __forceinline__ f32x4 p_mma(f32x4 c, const PFrag<bf16>& a, const PFrag<bf16>& b) {
  Frag<bf16> fa, fb;
  fa.v = a.v;
  fb.v = b.v;
  return mma(c, fa, fb);
}
__device__ __forceinline__ f32x4 p_mma(f32x4 c, const PFrag<float>& a, const PFrag<float>& b) {
  Frag<float> f0, f1, g0, g1;
  f0.v = a.v0; f1.v = a.v1; g0.v = b.v0; g1.v = b.v1;
  return mma(mma(c, f0, g0), f1, g1);
}

__device__ __forceinline__ void transpose4x4_f32(const u32x4 (&in)[4], u32x4 (&out)[4]) {
  out[0] = (u32x4){in[0].x, in[1].x, in[2].x, in[3].x};
  out[1] = (u32x4){in[0].y, in[1].y, in[2].y, in[3].y};
  out[2] = (u32x4){in[0].z, in[1].z, in[2].z, in[3].z};
  out[3] = (u32x4){in[0].w, in[1].w, in[2].w, in[3].w};
}

constexpr int kProPr = 0;                       // [256 rows][BK]   row-major P tile
constexpr int kProPc = 32768;                   // tiles [BK cols][BK tokens] x (256 / BK)
constexpr int kProBt = 65536;                   // [16 t][BK]       B_p^T chunk
constexpr int kProTT = 65536 + 2048;            // per adapter tiles [16 t][BK tokens] x (256/BK)
constexpr int kProLds = kProTT + 3 * 16384;     // 116736
// Layout of the buffer-load prologue (no column-major copy; bf16 T^T tiles of
// 8 KB): 58 KB.
constexpr int kProBtBuf = 32768;
constexpr int kProTTBuf = kProBtBuf + 2048;
constexpr int kProLdsBuf = kProTTBuf + 3 * 8192;   // 59392

// Register-staged prologue (fp32, or bf16 calls the buffer-load version
// below cannot take).
template <class T>
__global__ __launch_bounds__(kThreads, 1) void k_bwd_prologue(ProArgs a) {
  constexpr int VEC = PT<T>::VEC, BK = PT<T>::BK, KSUB = PT<T>::KSUB, HW = BK / 2;
  constexpr int NKB = kBM / BK;                 // token tiles per 256 rows
  constexpr int TTB = 16 * kPRowBytes * NKB;     // bytes of one adapter's T^T
  __shared__ __align__(16) char smem[kProLds];
  const WaveId q = wave_id();
  const int rb = blockIdx.x, cr = blockIdx.y;
  const long m0 = (long)rb * kBM;
  char* Pr = smem + kProPr;
  char* Pc = smem + kProPc;
  char* Bt = smem + kProBt;
  char* TT = smem + kProTT;

  // (s_p T_p)^T for this row block, once: TT_p tile kb, row t, element row % BK.
  for (int p = 0; p < a.nadp; ++p) {
    const int row = q.tid;
    const long n = m0 + row;
    float v[16];
    load_rank<float, 16>(a.Tp[p] + min(n, a.N - 1) * a.r, 1, 0, a.r, v);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      char* dst = TT + p * TTB + (row / BK) * (16 * kPRowBytes) + p_off(t, (row % BK) / VEC) + (row % VEC) * ET<T>::BYTES;
      *reinterpret_cast<T*>(dst) = from_f<T>(n < a.N ? a.s[p] * v[t] : 0.f);
    }
  }

  f32x4 dT[3][4];
#pragma unroll
  for (int p = 0; p < 3; ++p)
#pragma unroll
    for (int i = 0; i < 4; ++i) dT[p][i] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int pc = q.tid & 3, rg4 = q.tid >> 2;   // chunk pair (pc, pc+4), rows 4*rg4 .. +3
  const int ch_beg = cr * a.CPC, ch_end = min(a.NCH, (cr + 1) * a.CPC);

  // Column map of chunk ch: kk < HW -> base_lo + kk, kk >= HW -> base_hi + kk - HW.
  struct CMap {
    int p, hd;
    long base_lo, base_hi;
  };
  auto cmap = [&](int ch) {
    CMap m;
    m.p = 0;
    m.hd = 0;
    if (a.qkv) {
      const int cph = a.d / BK;                 // chunks per head
      const int gh = ch / cph, qq = ch % cph;
      m.p = (gh < a.nh[0]) ? 0 : ((gh < a.nh[0] + a.nh[1]) ? 1 : 2);
      m.hd = gh - ((m.p == 0) ? 0 : ((m.p == 1) ? a.nh[0] : a.nh[0] + a.nh[1]));
      m.base_lo = a.off[m.p] + (long)m.hd * a.d + qq * HW;
      m.base_hi = m.base_lo + a.d / 2;
    } else {
      m.base_lo = (long)ch * BK;
      m.base_hi = m.base_lo + HW;
      // Adapter of this chunk by column range (ranges are whole chunks).
      m.p = (a.nadp > 1 && m.base_lo >= a.off[1]) ? ((a.nadp > 2 && m.base_lo >= a.off[2]) ? 2 : 1) : 0;
    }
    return m;
  };

  // Steps 2-5 of a chunk whose P tile rows (4 rows x chunks pc, pc + 4) the
  // thread holds in lo / hi.
  // B_p^T chunk operand: thread tid < 128 supplies elements t0 .. t0+VEC-1 of
  // row kk (tpr threads per kk).
  constexpr int tpr = (sizeof(T) == 2) ? 2 : 4;
  const int bkk = q.tid / tpr, bt0 = (q.tid % tpr) * VEC;
  auto bload = [&](const CMap& m) -> u32x4 {
    const int p = m.p;
    const T* Bsrc = static_cast<const T*>(a.Bp[p]);
    const long col = (bkk < HW) ? m.base_lo + bkk : m.base_hi + (bkk - HW);
    const long lim = (long)a.off[p + 1];
    const T* brow = (col < lim) ? Bsrc + (col - a.off[p]) * a.r : nullptr;
    return gload<T>(brow, bt0, a.r, a.vecB);
  };
  auto process = [&](const CMap& m, const u32x4 (&lo)[4], const u32x4 (&hi)[4], const u32x4& bv) {
    const int p = m.p;
    // 2. Row-major copy for dT, column-major copy for dB.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(Pr + p_off(4 * rg4 + i, pc)) = lo[i];
      *reinterpret_cast<u32x4*>(Pr + p_off(4 * rg4 + i, pc + 4)) = hi[i];
    }
    {
      const int r0 = 4 * rg4;                     // 4 tokens: tile kb, chunk (r0 % BK) / VEC
      char* tile = Pc + (r0 / BK) * (BK * kPRowBytes);
      const int kc = (r0 % BK) / VEC, sub = (r0 % VEC) * ET<T>::BYTES;
      if constexpr (sizeof(T) == 2) {
        const unsigned* wl = reinterpret_cast<const unsigned*>(lo);
        const unsigned* wh = reinterpret_cast<const unsigned*>(hi);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int sh = (c & 1) * 16;
          const unsigned l0 = (wl[0 * 4 + c / 2] >> sh) & 0xffffu, l1 = (wl[1 * 4 + c / 2] >> sh) & 0xffffu;
          const unsigned l2 = (wl[2 * 4 + c / 2] >> sh) & 0xffffu, l3 = (wl[3 * 4 + c / 2] >> sh) & 0xffffu;
          const unsigned h0 = (wh[0 * 4 + c / 2] >> sh) & 0xffffu, h1 = (wh[1 * 4 + c / 2] >> sh) & 0xffffu;
          const unsigned h2 = (wh[2 * 4 + c / 2] >> sh) & 0xffffu, h3 = (wh[3 * 4 + c / 2] >> sh) & 0xffffu;
          *reinterpret_cast<u32x2*>(tile + p_off(pc * VEC + c, kc) + sub) = (u32x2){l0 | (l1 << 16), l2 | (l3 << 16)};
          *reinterpret_cast<u32x2*>(tile + p_off(HW + pc * VEC + c, kc) + sub) = (u32x2){h0 | (h1 << 16), h2 | (h3 << 16)};
        }
      } else {
        u32x4 tl[4], th[4];
        transpose4x4_f32(lo, tl);
        transpose4x4_f32(hi, th);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          *reinterpret_cast<u32x4*>(tile + p_off(pc * VEC + c, kc)) = tl[c];
          *reinterpret_cast<u32x4*>(tile + p_off(HW + pc * VEC + c, kc)) = th[c];
        }
      }
    }
    // 3. B_p^T chunk: row t, element kk = B_p[col(kk) - off_p][t].
    if (q.tid < 128) {
      const int kk = bkk, t0 = bt0;
      const unsigned* wv = reinterpret_cast<const unsigned*>(&bv);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        char* dst = Bt + p_off(t0 + e, kk / VEC) + (kk % VEC) * ET<T>::BYTES;
        if constexpr (sizeof(T) == 2)
          *reinterpret_cast<unsigned short*>(dst) = (unsigned short)((e & 1) ? (wv[e >> 1] >> 16) : (wv[e >> 1] & 0xffffu));
        else
          *reinterpret_cast<unsigned*>(dst) = wv[e];
      }
    }
    __syncthreads();

    // 4. dT_p[rows][t] += P[rows][chunk] . B_p[chunk][t]   (wave w: rows 64w .. 64w+63)
#pragma unroll
    for (int ks = 0; ks < KSUB; ++ks) {
      const PFrag<T> bf = p_frag<T>(Bt, q.r16, ks, q.g);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const PFrag<T> af = p_frag<T>(Pr, (4 * q.w + i) * 16 + q.r16, ks, q.g);
        if (p == 0) dT[0][i] = p_mma(dT[0][i], af, bf);
        else if (p == 1) dT[1][i] = p_mma(dT[1][i], af, bf);
        else dT[2][i] = p_mma(dT[2][i], af, bf);
      }
    }
    // 5. dB_p[col][t] (row-block partial) = P[rows][col]^T . (s_p T_p)[rows][t]
    if (q.w * 16 < BK) {
      f32x4 db = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int ks = 0; ks < KSUB; ++ks) {
          const PFrag<T> af = p_frag<T>(Pc + kb * (BK * kPRowBytes), q.w * 16 + q.r16, ks, q.g);
          const PFrag<T> bf = p_frag<T>(TT + p * TTB + kb * (16 * kPRowBytes), q.r16, ks, q.g);
          db = p_mma(db, af, bf);
        }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kk = q.w * 16 + 4 * q.g + j;
        const long col = (kk < HW) ? m.base_lo + kk : m.base_hi + (kk - HW);
        if (col < a.O) a.dB_part[((long)rb * a.O + col) * 16 + q.r16] = db[j];
      }
    }
    __syncthreads();
  };

  for (int ch = ch_beg; ch < ch_end; ++ch) {
    const CMap m = cmap(ch);
    const int p = m.p, hd = m.hd;
    // 1. P tile: 4 rows x (chunk pc, chunk pc+4) per thread.
    u32x4 lo[4], hi[4];
    const long clo = m.base_lo + pc * VEC, chi = m.base_hi + pc * VEC;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const long n = m0 + 4 * rg4 + i;
      if (n >= a.N) { lo[i] = zero4(); hi[i] = zero4(); continue; }
      if (a.qkv) {
        const int s = (int)(n % a.S);
        const long b = n / a.S;
        const int jlo = (int)(clo - a.off[p] - (long)hd * a.d);   // index within the head, < d/2
        const T* src = static_cast<const T*>(a.src[p]) + ((b * a.nh[p] + hd) * a.S + s) * (long)a.d;
        const u32x4 xl = gload<T>(src, jlo, a.d, a.vecP);
        const u32x4 xh = gload<T>(src, jlo + a.d / 2, a.d, a.vecP);
        if (p < 2) {
          float vl[VEC], vh[VEC], yl[VEC], yh[VEC];
          unpack(xl, vl);
          unpack(xh, vh);
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const float c = a.cs[(long)s * (a.d / 2) + jlo + e], sn = a.sn[(long)s * (a.d / 2) + jlo + e];
            yl[e] = vl[e] * c + vh[e] * sn;      // R^T: rotate by -angle
            yh[e] = vh[e] * c - vl[e] * sn;
          }
          lo[i] = pack(yl);
          hi[i] = pack(yh);
        } else {
          lo[i] = xl;
          hi[i] = xh;
        }
        T* dp = static_cast<T*>(a.dP) + n * a.O;
        *reinterpret_cast<u32x4*>(dp + clo) = lo[i];
        *reinterpret_cast<u32x4*>(dp + chi) = hi[i];
      } else {
        const T* row = static_cast<const T*>(a.P) + n * a.O;
        lo[i] = gload<T>(row, clo, a.O, a.vecP);
        hi[i] = gload<T>(row, chi, a.O, a.vecP);
      }
    }
    const u32x4 bv = q.tid < 128 ? bload(m) : zero4();
    process(m, lo, hi, bv);
  }

  // dT partial of this column range for the call's adapters (zeros for
  // adapters it did not touch).
#pragma unroll
  for (int p = 0; p < 3; ++p)
    if (p < a.nadp)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const long n = m0 + (4 * q.w + i) * 16 + 4 * q.g + j;
          if (n < a.N) a.dT_part[(((long)cr * 3 + p) * a.N + n) * 16 + q.r16] = a.s[p] * dT[p][i][j];
        }
}

// The bf16 buffer-load prologue with eight waves (512 threads): a thread
// holds 2 of a chunk's 256 rows (16-byte pieces pc and pc + 4 of each), so
// twice as many waves keep loads in flight and each does half the per-row
// work; the rows' (sequence, position) split is computed once.  After the
// chunk is in LDS, waves 0-3 form dT (4 m-blocks each) while waves 4-7 form
// the dB partial (one 16-column block each), both with the transpose reads
// of the four-wave version.  Same arguments, grid and results as
// k_bwd_prologue<bf16, true>.
template <class T>
__global__ __launch_bounds__(512, 1) void k_bwd_prologue8(ProArgs a) {
  static_assert(sizeof(T) == 2, "bf16");
  constexpr int VEC = 8, BK = 64, HW = 32, NKB = kBM / BK, TTB = 8192;
  __shared__ __align__(16) char smem[kProLdsBuf];
  const WaveId q = wave_id();
  const int w = __builtin_amdgcn_readfirstlane(q.w);
  const int rb = blockIdx.x, cr = blockIdx.y;
  const long m0 = (long)rb * kBM;
  char* Pr = smem + kProPr;
  char* Bt = smem + kProBtBuf;
  char* TT = smem + kProTTBuf;

  // (s_p T_p)^T for this row block, once (threads 0..255: one row each).
  if (q.tid < kBM) {
    for (int p = 0; p < a.nadp; ++p) {
      const int row = q.tid;
      const long n = m0 + row;
      float v[16];
      load_rank<float, 16>(a.Tp[p] + min(n, a.N - 1) * a.r, 1, 0, a.r, v);
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        char* dst = TT + p * TTB + (row / BK) * (16 * kPRowBytes) + p_off(t, (row % BK) / VEC) + (row % VEC) * 2;
        *reinterpret_cast<T*>(dst) = from_f<T>(n < a.N ? a.s[p] * v[t] : 0.f);
      }
    }
  }

  f32x4 dT[3][4];
#pragma unroll
  for (int p = 0; p < 3; ++p)
#pragma unroll
    for (int i = 0; i < 4; ++i) dT[p][i] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int pc = q.tid & 3, rg = q.tid >> 2;    // pieces (pc, pc + 4) of rows 2 rg, 2 rg + 1
  const int ch_beg = cr * a.CPC, ch_end = min(a.NCH, (cr + 1) * a.CPC);
  // qkv: (batch, position) of the thread's rows.
  long rbat[2];
  int rpos[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const long n = m0 + 2 * rg + i;
    const long nn = (a.qkv && n < a.N) ? n : 0;
    rpos[i] = a.qkv ? (int)(nn % a.S) : 0;
    rbat[i] = a.qkv ? nn / a.S : 0;
  }

  struct CMap {
    int p, hd;
    long base_lo, base_hi;
  };
  auto cmap = [&](int ch) {
    CMap m;
    m.p = 0;
    m.hd = 0;
    if (a.qkv) {
      const int cph = a.d / BK;
      const int gh = ch / cph, qq = ch % cph;
      m.p = (gh < a.nh[0]) ? 0 : ((gh < a.nh[0] + a.nh[1]) ? 1 : 2);
      m.hd = gh - ((m.p == 0) ? 0 : ((m.p == 1) ? a.nh[0] : a.nh[0] + a.nh[1]));
      m.base_lo = a.off[m.p] + (long)m.hd * a.d + qq * HW;
      m.base_hi = m.base_lo + a.d / 2;
    } else {
      m.base_lo = (long)ch * BK;
      m.base_hi = m.base_lo + HW;
      m.p = (a.nadp > 1 && m.base_lo >= a.off[1]) ? ((a.nadp > 2 && m.base_lo >= a.off[2]) ? 2 : 1) : 0;
    }
    return m;
  };
  // B_p chunk rows: thread tid < 128 supplies ranks bt0 .. bt0+7 of row bkk.
  const int bkk = q.tid >> 1, bt0 = (q.tid & 1) * VEC;

  struct Raw {
    u32x4 xl[2], xh[2];
    u32x4 bv;
  };
  struct Rot {
    f32x4 c[2][2], sn[2][2];
  };
  auto fetch = [&](const CMap& m, Raw& r) {
    const int p = m.p;
    {
      const long col = (bkk < HW) ? m.base_lo + bkk : m.base_hi + (bkk - HW);
      const long rows = (long)a.off[p + 1] - a.off[p];
      const __amdgpu_buffer_rsrc_t rb2 = buf_rsrc(a.Bp[p], (unsigned)(rows * a.r * 2));
      const bool ok = q.tid < 128 && col < a.off[p + 1] && bt0 < a.r;
      r.bv = buf_load16(rb2, ok ? (unsigned)(((col - a.off[p]) * a.r + bt0) * 2) : kBufOut);
    }
    if (a.qkv) {
      const __amdgpu_buffer_rsrc_t rs = buf_rsrc(a.src[p], (unsigned)(a.N * a.nh[p] * a.d * 2));
      const int jlo = (int)(m.base_lo + pc * VEC - a.off[p] - (long)m.hd * a.d);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const long n = m0 + 2 * rg + i;
        const long e0 = ((rbat[i] * a.nh[p] + m.hd) * a.S + rpos[i]) * (long)a.d + jlo;
        const unsigned off = n < a.N ? (unsigned)(e0 * 2) : kBufOut;
        r.xl[i] = buf_load16(rs, off);
        r.xh[i] = buf_load16(rs, off + (unsigned)a.d);
      }
    } else {
      const __amdgpu_buffer_rsrc_t rs = buf_rsrc(a.P, (unsigned)(a.N * a.O * 2));
      const long clo = m.base_lo + pc * VEC, chi = m.base_hi + pc * VEC;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const long n = m0 + 2 * rg + i;
        const bool live = n < a.N;
        r.xl[i] = buf_load16(rs, (live && clo < a.O) ? (unsigned)((n * a.O + clo) * 2) : kBufOut);
        r.xh[i] = buf_load16(rs, (live && chi < a.O) ? (unsigned)((n * a.O + chi) * 2) : kBufOut);
      }
    }
  };
  auto fetch_rot = [&](const CMap& m, Rot& r) {
    if (!a.qkv || m.p >= 2) return;
    const int jlo = (int)(m.base_lo + pc * VEC - a.off[m.p] - (long)m.hd * a.d);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const f32x4* cs4 = reinterpret_cast<const f32x4*>(a.cs + (long)rpos[i] * (a.d / 2) + jlo);
      const f32x4* sn4 = reinterpret_cast<const f32x4*>(a.sn + (long)rpos[i] * (a.d / 2) + jlo);
      r.c[i][0] = cs4[0];
      r.c[i][1] = cs4[1];
      r.sn[i][0] = sn4[0];
      r.sn[i][1] = sn4[1];
    }
  };

  auto process = [&](const CMap& m, const u32x4 (&lo)[2], const u32x4 (&hi)[2], const u32x4& bv) {
    const int p = m.p;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *reinterpret_cast<u32x4*>(Pr + p_off(2 * rg + i, pc)) = lo[i];
      *reinterpret_cast<u32x4*>(Pr + p_off(2 * rg + i, pc + 4)) = hi[i];
    }
    if (q.tid < 128) *reinterpret_cast<u32x4*>(Bt + bkk * 32 + bt0 * 2) = bv;
    __syncthreads();
    const int sl = q.r16, g = q.g;
    if (w < 4) {
      // dT_p[rows][t] += P[rows][chunk] . B_p[chunk][t]; wave w: m-blocks 4w .. 4w+3.
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int kr = ks * 32 + 8 * g + (sl >> 2);
        u32x2 b0 = tr16(lds_addr(Bt + kr * 32 + 8 * (sl & 3)));
        u32x2 b1 = tr16(lds_addr(Bt + (kr + 4) * 32 + 8 * (sl & 3)));
        lgkm_tie0(b0, b1);
        PFrag<bf16> bf;
        bf.v = (u32x4){b0.x, b0.y, b1.x, b1.y};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const PFrag<bf16> af = p_frag<bf16>(Pr, (4 * w + i) * 16 + q.r16, ks, q.g);
          if (p == 0) dT[0][i] = p_mma(dT[0][i], af, bf);
          else if (p == 1) dT[1][i] = p_mma(dT[1][i], af, bf);
          else dT[2][i] = p_mma(dT[2][i], af, bf);
        }
      }
    } else {
      // dB_p[col][t] = P[rows][col]^T . (s_p T_p)[rows][t]; wave w: columns
      // 16 (w - 4) .. +15.
      f32x4 db = (f32x4){0.f, 0.f, 0.f, 0.f};
      const int col = (w - 4) * 16 + 4 * (sl & 3);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int row = kb * 64 + ks * 32 + 8 * g + (sl >> 2);
          u32x2 a0 = tr16(lds_addr(Pr + p_off(row, col >> 3) + (col & 7) * 2));
          u32x2 a1 = tr16(lds_addr(Pr + p_off(row + 4, col >> 3) + (col & 7) * 2));
          lgkm_tie0(a0, a1);
          PFrag<bf16> af;
          af.v = (u32x4){a0.x, a0.y, a1.x, a1.y};
          const PFrag<bf16> bf = p_frag<bf16>(TT + p * TTB + kb * (16 * kPRowBytes), q.r16, ks, q.g);
          db = p_mma(db, af, bf);
        }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kk = (w - 4) * 16 + 4 * q.g + j;
        const long c = (kk < HW) ? m.base_lo + kk : m.base_hi + (kk - HW);
        if (c < a.O) a.dB_part[((long)rb * a.O + c) * 16 + q.r16] = db[j];
      }
    }
    __syncthreads();
  };

  // One chunk in flight while one is processed; the rotation of a q/k chunk
  // is fetched one chunk ahead.
  Raw nx;
  Rot rot;
  if (ch_beg < ch_end) {
    fetch(cmap(ch_beg), nx);
    fetch_rot(cmap(ch_beg), rot);
  }
  for (int ch = ch_beg; ch < ch_end; ++ch) {
    const CMap m = cmap(ch);
    u32x4 lo[2], hi[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      lo[i] = nx.xl[i];
      hi[i] = nx.xh[i];
    }
    if (a.qkv) {
      if (m.p < 2) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          float vl[VEC], vh[VEC], yl[VEC], yh[VEC];
          unpack(nx.xl[i], vl);
          unpack(nx.xh[i], vh);
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const float c = rot.c[i][e >> 2][e & 3], sv = rot.sn[i][e >> 2][e & 3];
            yl[e] = vl[e] * c + vh[e] * sv;      // R^T: rotate by -angle
            yh[e] = vh[e] * c - vl[e] * sv;
          }
          lo[i] = pack(yl);
          hi[i] = pack(yh);
        }
      }
      const long clo = m.base_lo + pc * VEC, chi = m.base_hi + pc * VEC;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const long n = m0 + 2 * rg + i;
        if (n < a.N) {
          T* dp = static_cast<T*>(a.dP) + n * a.O;
          *reinterpret_cast<u32x4*>(dp + clo) = lo[i];
          *reinterpret_cast<u32x4*>(dp + chi) = hi[i];
        }
      }
    }
    const u32x4 bv = nx.bv;
    if (ch + 1 < ch_end) {
      const CMap mn = cmap(ch + 1);
      fetch(mn, nx);
      fetch_rot(mn, rot);
    }
    process(m, lo, hi, bv);
  }

  // dT partial of this column range for the call's adapters (waves 0-3).
  if (w < 4) {
#pragma unroll
    for (int p = 0; p < 3; ++p)
      if (p < a.nadp)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const long n = m0 + (4 * w + i) * 16 + 4 * q.g + j;
            if (n < a.N) a.dT_part[(((long)cr * 3 + p) * a.N + n) * 16 + q.r16] = a.s[p] * dT[p][i][j];
          }
  }
}

// Direct buffer -> LDS load (gfx950 buffer_load_dwordx4 ... lds): lane l
// writes 16 bytes at LDS base + 16 l; an offset at or past the resource's
// end writes zeros and never faults.
__device__ __forceinline__ void buf2lds16(__amdgpu_buffer_rsrc_t r, unsigned off, char* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16, off, 0, 0,
                                           0);
}
// Barrier after this wave's LDS traffic has completed, as one asm statement
// (the compiler adds no wait for the direct loads still in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The bf16 backward prologue over a token-major P (dY of the MLP down
// projection or of one LoRA linear) as a ring of LDS stages filled by direct
// buffer loads, NS - 1 chunks in flight.  The waves split the work:
//   waves 0-3  issue every direct load (the 256 x 64 P tile of a chunk and
//              its B_p rows), wait for them, and form dT = P . B_p;
//   waves 4-7  build (s_p T_p)^T once and form the dB partials.
// Same arguments, grid and results (up to the order of the dT sums) as
// k_bwd_prologue8 with qkv = 0.  (The QKV prologue, which also un-rotates and
// stores dP, stays on k_bwd_prologue8: ring forms of it, with the rotation
// on either half of the waves, measured slower.)
constexpr int kPrStage = 32768 + 2048;             // P tile [256][128 B] + B_p chunk [64 kk][16 t]
template <int NS>
constexpr int pr_lds_bytes() { return NS * kPrStage + 3 * 8192; }

template <class T, int NS>
__global__ __launch_bounds__(512, 1) void k_bwd_prologue_ring(ProArgs a) {
  static_assert(sizeof(T) == 2, "bf16");
  static_assert(NS >= 2 && NS <= 4, "ring depth");
  constexpr int HW = 32, NKB = kBM / 64, TTB = 8192, LPC = 9;   // LPC: direct loads per chunk and loader wave
  __shared__ __align__(16) char smem[pr_lds_bytes<NS>()];
  const WaveId q = wave_id();
  const int w = __builtin_amdgcn_readfirstlane(q.w);
  const int L = q.lane;
  const int rb = blockIdx.x, cr = blockIdx.y;
  const long m0 = (long)rb * kBM;
  char* TT = smem + NS * kPrStage;
  const int cb = cr * a.CPC, ce = min(a.NCH, (cr + 1) * a.CPC);
  const int nch = max(0, ce - cb);
  // Adapter of chunk ch by column range (ranges are whole chunks).
  auto adapter = [&](int ch) {
    const int base = ch * 64;
    return (a.nadp > 1 && base >= a.off[1]) ? ((a.nadp > 2 && base >= a.off[2]) ? 2 : 1) : 0;
  };

  // (s_p T_p)^T for this row block, once (waves 4-7: one row each), before
  // any direct load is in flight.
  if (w >= 4) {
    const int row = q.tid - 256;
    const long n = m0 + row;
    for (int p = 0; p < a.nadp; ++p) {
      float v[16];
      load_rank<float, 16>(a.Tp[p] + min(n, a.N - 1) * a.r, 1, 0, a.r, v);
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        char* dst = TT + p * TTB + (row / 64) * (16 * kPRowBytes) + p_off(t, (row % 64) / 8) + (row % 8) * 2;
        *reinterpret_cast<T*>(dst) = from_f<T>(n < a.N ? a.s[p] * v[t] : 0.f);
      }
    }
  }

  // Loader waves: rows 8 (w + 4 it) + L / 8 of the tile, 16-byte piece lc
  // (the LDS rows are 128 bytes, pieces XOR-swizzled with row & 7).
  const int lc = (L & 7) ^ (L >> 3);
  int lrow[8];                                     // n * O of a live row, -1 past N
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const long n = m0 + 8 * ((w & 3) + 4 * it) + (L >> 3);
    lrow[it] = n < a.N ? (int)(n * a.O) : -1;
  }
  const __amdgpu_buffer_rsrc_t prs = buf_rsrc(a.P, (unsigned)(a.N * a.O * 2));
  auto issue = [&](int c, char* S) {
    const int ch = cb + c, p = adapter(ch), base = ch * 64;
    {
      // B_p chunk: lanes < 32 of the loader waves, rank entries bt0 .. bt0+7 of chunk column bkk.
      const int tid = w * 32 + L, bkk = tid >> 1, bt0 = (tid & 1) * 8;
      const int col = base + bkk;
      const int rows = a.off[p + 1] - a.off[p];
      const __amdgpu_buffer_rsrc_t rs = buf_rsrc(a.Bp[p], (unsigned)(rows * a.r * 2));
      const bool ok = col < a.off[p + 1] && bt0 < a.r;
      if (L < 32) buf2lds16(rs, ok ? (unsigned)(((col - a.off[p]) * a.r + bt0) * 2) : kBufOut, S + 32768 + w * 512);
    }
    const int col = base + lc * 8;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const bool ok = lrow[it] >= 0 && col < a.O;
      buf2lds16(prs, ok ? (unsigned)((lrow[it] + col) * 2) : kBufOut, S + ((w & 3) + 4 * it) * 1024);
    }
  };

  f32x4 dT[3][4];
#pragma unroll
  for (int p = 0; p < 3; ++p)
#pragma unroll
    for (int i = 0; i < 4; ++i) dT[p][i] = (f32x4){0.f, 0.f, 0.f, 0.f};

  if (w < 4) {
#pragma unroll
    for (int j = 0; j < NS - 1; ++j)
      if (j < nch) issue(j, smem + j * kPrStage);
  }
  int st = 0;                                      // stage of chunk c
  for (int c = 0; c < nch; ++c) {
    char* const S = smem + st * kPrStage;
    if (w < 4) {
      // Chunk c has landed once at most the later chunks' loads are outstanding.
      const int later = min(nch - 1 - c, NS - 2);
      if constexpr (NS >= 4) {
        if (later >= 2) vm_wait<2 * LPC>();
        else if (later == 1) vm_wait<LPC>();
        else vm_wait<0>();
      } else if constexpr (NS == 3) {
        if (later >= 1) vm_wait<LPC>();
        else vm_wait<0>();
      } else {
        vm_wait<0>();
      }
    }
    lds_barrier();
    // The stage refilled here was read in the previous iteration, before the barrier.
    const int st_next = (st + NS - 1) % NS;
    if (w < 4 && c + NS - 1 < nch) issue(c + NS - 1, smem + st_next * kPrStage);
    const int ch = cb + c, p = adapter(ch), base = ch * 64;
    const int sl = q.r16, g = q.g;
    if (w < 4) {
      // dT_p[rows][t] += P[rows][chunk] . B_p[chunk][t]; wave w: m-blocks 4w .. 4w+3.
      const char* Bt = S + 32768;
      u32x2 b0[2], b1[2];
      u32x4 av[2][4];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int kr = ks * 32 + 8 * g + (sl >> 2);
        b0[ks] = tr16(lds_addr(Bt + kr * 32 + 8 * (sl & 3)));
        b1[ks] = tr16(lds_addr(Bt + (kr + 4) * 32 + 8 * (sl & 3)));
#pragma unroll
        for (int i = 0; i < 4; ++i) av[ks][i] = rd128(S + p_off((4 * w + i) * 16 + sl, ks * 4 + g));
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        lgkm_tie0(b0[ks], b1[ks]);
#pragma unroll
        for (int i = 0; i < 4; ++i) tie<0>(av[ks][i]);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        PFrag<bf16> bf;
        bf.v = (u32x4){b0[ks].x, b0[ks].y, b1[ks].x, b1[ks].y};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          PFrag<bf16> af;
          af.v = av[ks][i];
          if (p == 0) dT[0][i] = p_mma(dT[0][i], af, bf);
          else if (p == 1) dT[1][i] = p_mma(dT[1][i], af, bf);
          else dT[2][i] = p_mma(dT[2][i], af, bf);
        }
      }
    } else {
      // dB_p[col][t] = P[rows][col]^T . (s_p T_p)[rows][t]; wave w: columns
      // 16 (w - 4) .. +15.
      f32x4 db = (f32x4){0.f, 0.f, 0.f, 0.f};
      const int col = (w - 4) * 16 + 4 * (sl & 3);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        u32x2 a0[2], a1[2];
        u32x4 tv[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int row = kb * 64 + ks * 32 + 8 * g + (sl >> 2);
          a0[ks] = tr16(lds_addr(S + p_off(row, col >> 3) + (col & 7) * 2));
          a1[ks] = tr16(lds_addr(S + p_off(row + 4, col >> 3) + (col & 7) * 2));
          tv[ks] = rd128(TT + p * TTB + kb * (16 * kPRowBytes) + p_off(sl, ks * 4 + g));
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          lgkm_tie0(a0[ks], a1[ks]);
          tie<0>(tv[ks]);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          PFrag<bf16> af, bf;
          af.v = (u32x4){a0[ks].x, a0[ks].y, a1[ks].x, a1[ks].y};
          bf.v = tv[ks];
          db = p_mma(db, af, bf);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int cc = base + (w - 4) * 16 + 4 * g + j;
        if (cc < a.O) a.dB_part[((long)rb * a.O + cc) * 16 + sl] = db[j];
      }
    }
    st = (st + 1 == NS) ? 0 : st + 1;
  }

  // dT partial of this column range for the call's adapters (waves 0-3).
  if (w < 4) {
#pragma unroll
    for (int p = 0; p < 3; ++p)
      if (p < a.nadp)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const long n = m0 + (4 * w + i) * 16 + 4 * q.g + j;
            if (n < a.N) a.dT_part[(((long)cr * 3 + p) * a.N + n) * 16 + q.r16] = a.s[p] * dT[p][i][j];
          }
  }
}

// ===========================================================================
// q/k norm backward: dP (token-major [N][O]) from dQ/dK/dV.  For q and k heads
// g = R^T dQ is pulled back through the per-head RMSNorm,
//   dP = rinv * (w g - xhat * mean(w g xhat)),  xhat = Pn * rinv,
// with Pn and rinv saved by the forward; v heads are copied.  One group of
// TPH lanes per (token, head); each lane holds E elements of the head's first
// half and the E matching elements of its second half (the RoPE pairs).
// ===========================================================================
struct NormBwdArgs {
  const void* src[3];           // dQ, dK, dV as [B][heads][S][d]
  const void* Pn;               // [N][off[2]]
  const float* rinv;            // [N][nh[0] + nh[1]]
  const void* nw[2];            // q_norm / k_norm weights [d]
  const float* cs; const float* sn;
  void* dP;                     // [N][O]
  long N; int S, d;
  int nh[3];
  int off[4];
};

template <class T, int TPH>
__global__ __launch_bounds__(256) void k_qk_norm_bwd(NormBwdArgs a) {
  constexpr int E = ET<T>::VEC;                  // 8 bf16 or 4 fp32: one 16-byte chunk
  constexpr int IPB = 256 / TPH;                 // (token, head) items per block
  const int gh = blockIdx.y;                     // head over q | k | v
  const int p = (gh < a.nh[0]) ? 0 : ((gh < a.nh[0] + a.nh[1]) ? 1 : 2);
  const int hd = gh - ((p == 0) ? 0 : ((p == 1) ? a.nh[0] : a.nh[0] + a.nh[1]));
  const long n = (long)blockIdx.x * IPB + threadIdx.x / TPH;
  const int t = threadIdx.x % TPH;
  const int half = a.d >> 1;
  const int jl = t * E;                          // < d/2
  const bool live = n < a.N;                     // whole lane groups share n
  const long nn = live ? n : 0;
  const int s = (int)(nn % a.S);
  const long b = nn / a.S;
  const T* src = static_cast<const T*>(a.src[p]) + ((b * a.nh[p] + hd) * a.S + s) * (long)a.d;
  float gl[E], gh2[E];
  unpack(*reinterpret_cast<const u32x4*>(src + jl), gl);
  unpack(*reinterpret_cast<const u32x4*>(src + jl + half), gh2);
  T* dst = static_cast<T*>(a.dP) + nn * (long)a.off[3] + a.off[p] + (long)hd * a.d;
  if (p < 2) {
    const float* __restrict__ cs = a.cs + (long)s * half + jl;
    const float* __restrict__ sn = a.sn + (long)s * half + jl;
    const T* pn = static_cast<const T*>(a.Pn) + nn * (long)a.off[2] + a.off[p] + (long)hd * a.d;
    const T* w = static_cast<const T*>(a.nw[p]);
    float xl[E], xh[E], wl[E], wh[E];
    unpack(*reinterpret_cast<const u32x4*>(pn + jl), xl);
    unpack(*reinterpret_cast<const u32x4*>(pn + jl + half), xh);
    unpack(*reinterpret_cast<const u32x4*>(w + jl), wl);
    unpack(*reinterpret_cast<const u32x4*>(w + jl + half), wh);
    const float ri = a.rinv[nn * (a.nh[0] + a.nh[1]) + (p == 0 ? 0 : a.nh[0]) + hd];
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float c = cs[e], sv = sn[e];
      const float ul = gl[e] * c + gh2[e] * sv;  // R^T: rotate by -angle
      const float uh = gh2[e] * c - gl[e] * sv;
      gl[e] = ul * wl[e];                        // w g
      gh2[e] = uh * wh[e];
      xl[e] *= ri;                               // xhat
      xh[e] *= ri;
      dot += gl[e] * xl[e] + gh2[e] * xh[e];
    }
    const float m = lane_group_sum<TPH>(dot) / (float)a.d;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      gl[e] = ri * (gl[e] - xl[e] * m);
      gh2[e] = ri * (gh2[e] - xh[e] * m);
    }
  }
  if (live) {
    *reinterpret_cast<u32x4*>(dst + jl) = pack(gl);
    *reinterpret_cast<u32x4*>(dst + jl + half) = pack(gh2);
  }
}

// dT[p][n][t] = sum over the prologue's column ranges c (fixed order) of its
// partials [NCR][3][N][16], for the adapters p < nadp.  One float4 per thread.
static __global__ __launch_bounds__(256) void k_dt_sum(const float* part, float* dT, int NCR, long N) {
  const int p = blockIdx.y;
  const long e4 = (long)blockIdx.x * blockDim.x + threadIdx.x;   // float4 index within [N][16]
  if (e4 >= N * 4) return;
  // Partials are added in column-range order; they are loaded eight at a
  // time so the loads overlap (the sums, and so the result, are unchanged).
  const f32x4* src = reinterpret_cast<const f32x4*>(part + (long)p * N * 16) + e4;
  const long stride = 3 * N * 4;                                  // float4s between column ranges
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  int c = 0;
  for (; c + 8 <= NCR; c += 8) {
    f32x4 b[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) b[u] = src[(long)(c + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) v += b[u];
  }
  for (; c < NCR; ++c) v += src[(long)c * stride];
  reinterpret_cast<f32x4*>(dT + (long)p * N * 16)[e4] = v;
}

// Fill Ts[slot][m][t] (slots < nslot) with the rows m0 .. m0+255 of dT [3][N][16].
__device__ __forceinline__ void load_dT(char* smem, const float* dT, long N, long m0, int nslot) {
  f32x4* Ts = reinterpret_cast<f32x4*>(ts_ptr(smem));
  for (int sl = 0; sl < nslot; ++sl)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = threadIdx.x + kGemmThreads * i;        // float4 index within the slot: row e / 4
      const long n = m0 + (e >> 2);
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (n < N) v = reinterpret_cast<const f32x4*>(dT + ((long)sl * N + n) * 16)[e & 3];
      Ts[sl * kBM * 4 + e] = v;
    }
  __syncthreads();
}

// ===========================================================================
// Down projection backward + GLU backward
// ===========================================================================
struct DownBwdArgs {
  const void* dY; const void* Wd; const void* Ad;
  const void* G; const void* U;
  const float* Tg; const float* Tu;
  const float* dT;              // [3][N][16], summed prologue partials
  float sg, su;
  void* dG; void* dU;
  float* pA_d; float* pB_g; float* pB_u;     // [R][i][16]
  long N; int h, i, r;
  int vecA, vecW, vecO;
  int R, NC;
};

// The whole dH tile is parked (bf16) before the GLU backward: 16 KB per wave
// (its 64 rows x 128 columns) after Ts slot 0, the only side slot this kernel
// uses.  That frees the accumulators for the GLU backward and the partials.
constexpr int kDownParkOff = kBM * kSlot * 4;

// ---------------------------------------------------------------------------
// GLU backward of a whole tile (bf16; N and i multiples of 256).
//
// G and U are staged through LDS by direct loads, one m-block at a time (a
// wave's 16 rows x 128 columns of each, 8 KB) in a wave-private ring of two
// buffers: the next m-block's loads are in flight while one is processed,
// nothing in flight occupies registers, and no workgroup barrier is needed.
// A lane reads its four rows of a column with ds_read_b64_tr_b16, i.e. in the
// accumulator layout, so dH stays where the K-loop left it (rounded to bf16,
// packed in registers), and H, dG, dU are formed per column and go straight
// into the partials' MFMAs as B operands (K = rows).  dG and dU are written
// back over the consumed G and U rows and leave as 16-byte row stores.
//
// Buffer rows are 256 bytes (128 columns); their 32-byte segments are
// XOR-swizzled by row (segment nb ^ (row & 7)), so the transpose reads of 16
// rows and the column writes spread over the banks.  The A operands (dT_d,
// s_g T_g, s_u T_u of the block's rows) sit in LDS as bf16 [row][16], read
// the same way.
//
// Vector memory operations of a wave complete in issue order; the waits
// below count the operations issued after the m-block being waited for.
// ---------------------------------------------------------------------------
constexpr int kGluRing = 0;                         // wave w at + w * 16 KB: two buffers of 8 KB
constexpr int kGluT = 128 * 1024;                   // bf16 [3][256][16]: dT_d, s_g T_g, s_u T_u
constexpr int kGluLds = kGluT + 3 * kBM * 32;       // 155648
static_assert(kGluT >= kGluRing + 8 * 16384, "GLU ring layout");

constexpr int kDownBwdLds = kGluLds > kDownParkOff + 8 * 16384 ? kGluLds : kDownParkOff + 8 * 16384;
static_assert(kDownBwdLds >= kGemmLds && kDownBwdLds <= 163840, "k_down_bwd LDS");

// Ring buffer b of a wave: G rows at b * 8 KB, U rows 4 KB after.  Row r
// (0..15) of 256 bytes holds columns c (0..127) at
// 256 r + 32 ((c / 16) ^ (r & 7)) + 2 (c % 16).
template <int ACT>
__device__ __forceinline__ void glu_bwd_full(char* smem, f32x4 (&acc)[kMB][8], const DownBwdArgs& a, long m0, long n0,
                                             int rb) {
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = w >> 1, wn = w & 1;
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));             // keep lane-derived values after the K-loop
  const int s = lane & 15, g = lane >> 4;
  const long ni = a.i;

  // dH rounded to bf16, packed (rows j0 j1 | j2 j3 of each column): frees the
  // accumulators.
  u32x2 dh[kMB][8];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
      dh[mb][nb] = (u32x2){pack_bf2(acc[mb][nb][0], acc[mb][nb][1]), pack_bf2(acc[mb][nb][2], acc[mb][nb][3])};

  // Direct loads of m-block mb's G and U rows into buffer mb & 1: lane l
  // fills the 16 bytes of row 4 it + l / 16 at chunk l % 16.
  const long wrow = (m0 + wm * 64) * ni + n0 + wn * 128;
  const bf16* Gw = static_cast<const bf16*>(a.G) + wrow;
  const bf16* Uw = static_cast<const bf16*>(a.U) + wrow;
  bf16* dGw = static_cast<bf16*>(a.dG) + wrow;
  bf16* dUw = static_cast<bf16*>(a.dU) + wrow;
  int eoff[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int R = 4 * it + g, c = s;
    eoff[it] = R * (int)ni + 16 * ((c >> 1) ^ (R & 7)) + 8 * (c & 1);
  }
  char* const ringw = smem + kGluRing + w * 16384;
  auto issue = [&](int mb) {
    char* buf = ringw + (mb & 1) * 8192;
    const int mo = mb * 16 * (int)ni;
#pragma unroll
    for (int it = 0; it < 4; ++it) g2lds16(Gw + mo + eoff[it], buf + it * 1024);
#pragma unroll
    for (int it = 0; it < 4; ++it) g2lds16(Uw + mo + eoff[it], buf + 4096 + it * 1024);
  };

  // The A operands of the wave's 64 rows (lane l stages row wm*64 + l), one
  // array at a time; asm writes (see above).
  const long trow = m0 + wm * 64 + lane;
  char* const Tl = smem + kGluT;
  const unsigned tw = lds_addr(Tl + (wm * 64 + lane) * 32);
  auto stage_t = [&](auto Oc, const float (&v)[16]) {
    constexpr int o = decltype(Oc)::value;
    u32x4 lo, hi;
    lo.x = pack_bf2(v[0], v[1]); lo.y = pack_bf2(v[2], v[3]);
    lo.z = pack_bf2(v[4], v[5]); lo.w = pack_bf2(v[6], v[7]);
    hi.x = pack_bf2(v[8], v[9]); hi.y = pack_bf2(v[10], v[11]);
    hi.z = pack_bf2(v[12], v[13]); hi.w = pack_bf2(v[14], v[15]);
    ds_w128_at<o * kBM * 32>(tw, lo);
    ds_w128_at<o * kBM * 32 + 16>(tw, hi);
  };
  {
    float v[16];
    const f32x4* d4 = reinterpret_cast<const f32x4*>(a.dT + trow * 16);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 x = d4[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * c + e] = x[e];
    }
    stage_t(std::integral_constant<int, 0>{}, v);
    load_rank<float, 16>(a.Tg + trow * a.r, 1, 0, a.r, v);
#pragma unroll
    for (int t = 0; t < 16; ++t) v[t] *= a.sg;
    stage_t(std::integral_constant<int, 1>{}, v);
    load_rank<float, 16>(a.Tu + trow * a.r, 1, 0, a.r, v);
#pragma unroll
    for (int t = 0; t < 16; ++t) v[t] *= a.su;
    stage_t(std::integral_constant<int, 2>{}, v);
  }
  issue(0);
  issue(1);

  f32x4 pacc[3][8];
#pragma unroll
  for (int o = 0; o < 3; ++o)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) pacc[o][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // Per-lane bases.  Transpose reads: this lane addresses row Rr, columns
  // 16 nb + 4 (s % 4) .. +3 (one base per nb).  Column writes of row 4g + j:
  // the swizzle 32 ((nb ^ j) ^ 4 x), x = g & 1, is 32 (nb ^ j) + 128 x or
  // - 128 x by bit 7 of 32 (nb ^ j).  Row reads: 16 bytes at 16 lane.
  const int Rr = 4 * g + (s >> 2);
  const unsigned rbase = lds_addr(ringw);
  unsigned trb[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) trb[nb] = rbase + Rr * 256 + 32 * (nb ^ (Rr & 7)) + 8 * (s & 3);
  const int x = g & 1;
  const unsigned wlane = rbase + 4 * g * 256 + 2 * s;
  const unsigned wplus = wlane + 128 * x, wminus = wlane - 128 * x;
  const unsigned rowb = rbase + 16 * lane;
  const unsigned tab = lds_addr(Tl + (wm * 64 + Rr) * 32 + 8 * (s & 3));

  static_for<kMB>([&](auto MBc) {
    constexpr int mb = decltype(MBc)::value;
    constexpr int B = (mb & 1) * 8192;
    // Operations issued after m-block mb's loads: mb 0: L1; 1: L2, S0;
    // 2: S0, L3, S1; 3: S1, S2 (8 each).
    vm_wait<mb == 0 ? 8 : (mb == 2 ? 24 : 16)>();
    Frag4<bf16> aD, aG, aU;
    aD.v = tr16_at<0 * kBM * 32 + mb * 512>(tab);
    aG.v = tr16_at<1 * kBM * 32 + mb * 512>(tab);
    aU.v = tr16_at<2 * kBM * 32 + mb * 512>(tab);
    lgkm_tie0(aD.v, aG.v);
    lgkm_tie0(aU.v);
    static_for<2>([&](auto Hc) {           // two halves of 4 column blocks
      constexpr int h0 = decltype(Hc)::value * 4;
      u32x2 gv[4], uv[4];
      static_for<4>([&](auto Kc) {
        constexpr int k = decltype(Kc)::value;
        gv[k] = tr16_at<B>(trb[h0 + k]);
        uv[k] = tr16_at<B + 4096>(trb[h0 + k]);
      });
#pragma unroll
      for (int k = 0; k < 4; ++k) lgkm_tie0(gv[k], uv[k]);
      static_for<4>([&](auto Kc) {
        constexpr int k = decltype(Kc)::value, nb = h0 + k;
        const float dH4[4] = {bf_lo(dh[mb][nb].x), bf_hi(dh[mb][nb].x), bf_lo(dh[mb][nb].y), bf_hi(dh[mb][nb].y)};
        const float G4[4] = {bf_lo(gv[k].x), bf_hi(gv[k].x), bf_lo(gv[k].y), bf_hi(gv[k].y)};
        const float U4[4] = {bf_lo(uv[k].x), bf_hi(uv[k].x), bf_lo(uv[k].y), bf_hi(uv[k].y)};
        float h4[4], g4[4], u4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float ph, dph;
          act_both<ACT>(G4[j], ph, dph);
          g4[j] = dH4[j] * U4[j] * dph;
          u4[j] = dH4[j] * ph;
          h4[j] = ph * U4[j];
        }
        const Frag4<bf16> fh = make_frag4<bf16>(h4), fg = make_frag4<bf16>(g4), fu = make_frag4<bf16>(u4);
        pacc[0][nb] = mma4(pacc[0][nb], aD, fh);
        pacc[1][nb] = mma4(pacc[1][nb], aG, fg);
        pacc[2][nb] = mma4(pacc[2][nb], aU, fu);
        // dG, dU over G, U: rows 4g + j, column 16 nb + s.
        static_for<4>([&](auto Jc) {
          constexpr int j = decltype(Jc)::value;
          constexpr int A = 32 * (nb ^ j);
          constexpr int off = B + j * 256 + A;
          const unsigned base = (A & 128) ? wminus : wplus;
          const unsigned vg = (j < 2) ? fg.v.x : fg.v.y, vu = (j < 2) ? fu.v.x : fu.v.y;
          if constexpr (j & 1) {
            ds_w16_hi_at<off>(base, vg);
            ds_w16_hi_at<off + 4096>(base, vu);
          } else {
            ds_w16_lo_at<off>(base, vg);
            ds_w16_lo_at<off + 4096>(base, vu);
          }
        });
      });
    });
    // Rows back out: the 16-byte chunks the loads brought in.
    u32x4 og[4], ou[4];
    static_for<4>([&](auto Ic) {
      constexpr int it = decltype(Ic)::value;
      og[it] = rd128_at<B + it * 1024>(rowb);
      ou[it] = rd128_at<B + 4096 + it * 1024>(rowb);
    });
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      tie<0>(og[it]);
      tie<0>(ou[it]);
    }
    // The buffer is free: next-but-one m-block's loads, then this one's stores.
    if constexpr (mb + 2 < kMB) issue(mb + 2);
    asm volatile("" ::: "memory");
    const int mo = mb * 16 * (int)ni;
#pragma unroll
    for (int it = 0; it < 4; ++it) *reinterpret_cast<u32x4*>(dGw + mo + eoff[it]) = og[it];
#pragma unroll
    for (int it = 0; it < 4; ++it) *reinterpret_cast<u32x4*>(dUw + mo + eoff[it]) = ou[it];
    asm volatile("" ::: "memory");
  });
  float* const parts[3] = {a.pA_d + (long)rb * ni * 16, a.pB_g + (long)rb * ni * 16, a.pB_u + (long)rb * ni * 16};
  reduce_store_partials<3, 3>(smem, pacc, parts, n0, ni);
}

template <class T, int ACT, bool FAST, bool FULL = false>
__global__ __launch_bounds__(kGemmThreads, 1) void k_down_bwd(DownBwdArgs a) {
  constexpr bool TR = sizeof(T) == 2;   // bf16: transpose-read K-loop, natural column order
  __shared__ __align__(16) char smem[kDownBwdLds];
  const WaveId q = wave_id();
  int rb, cb;
  tile_coords(a.R * a.NC, a.R, a.NC, 8, rb, cb);
  const long m0 = (long)rb * kBM;
  const long n0 = (long)cb * kBN;
  const T* dY = static_cast<const T*>(a.dY);
  const T* Wd = static_cast<const T*>(a.Wd);
  const long h = a.h, ni = a.i;

  f32x4 acc[kMB][8];
  f32x4 sacc[1][kMB];
  zero_acc(acc);
  const int nkt = (a.h + ET<T>::BK - 1) / ET<T>::BK;
  if constexpr (FAST) {
    static_assert(TR, "the fast path is bf16");
    KRow1<bf16> kr;                                       // h % 64 == 0
    kr.W = Wd; kr.K = h; kr.ld = ni;
    kloop2tr_pp(smem, (int)(h / 64), dY, nullptr, h, kr, h, a.N, m0, ni, n0, ni, acc);
  } else if constexpr (TR) {
    KNTrLoader<RowsA<T>, KRow1<T>, SRowNone<T>, SMaskNone, 0> ld;
    ld.a.init(dY, nullptr, h, 0, h, a.N, m0, a.vecA);
    ld.krow.W = Wd; ld.krow.K = h; ld.krow.ld = ni;
    ld.n0 = n0; ld.N = ni; ld.vecB = a.vecW; ld.r = a.r; ld.vecS = false;
    kloop<T, 0>(smem, nkt, ld, acc, sacc);
  } else {
    KNLoader32<KRow1<T>, SRowNone<T>, SMaskNone, 0> ld;
    ld.a.init(dY, nullptr, h, 0, h, a.N, m0, a.vecA);
    ld.krow.W = Wd; ld.krow.K = h; ld.krow.ld = ni;
    ld.n0 = n0; ld.N = ni; ld.vecB = a.vecW; ld.r = a.r; ld.vecS = false;
    kloop<T, 0>(smem, nkt, ld, acc, sacc);
  }

  load_dT(smem, a.dT, a.N, m0, 1);
  const T* Ad = static_cast<const T*>(a.Ad);
  auto fb = [&](int R, int slot, int t0, float* v) {
    const long n = n0 + (TR ? R : lds_row_col(0, R));
    if (slot != 0 || n >= ni) return;
    load_rank<T, ET<T>::VEC>(Ad + n, ni, t0, a.r, v);
  };
  const float fs[kMaxSide] = {1.f, 0.f, 0.f};
  fold<T>(smem, acc, 1, fs, fb);
  if constexpr (FULL) {
    static_assert(FAST, "whole-tile GLU backward is part of the bf16 fast path");
    glu_bwd_full<ACT>(smem, acc, a, m0, n0, rb);
    return;
  }

  // Epilogue: the lane's view of a row is the 8 consecutive columns c0 .. c0+7.
  char* wpark = smem + kDownParkOff + q.w * 16384;
  if constexpr (TR) {
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) park_mb(wpark + 4096 * mb, acc, mb, q);
  }
  const T* Gs = static_cast<const T*>(a.G);
  const T* Us = static_cast<const T*>(a.U);
  T* dGo = static_cast<T*>(a.dG);
  T* dUo = static_cast<T*>(a.dU);
  const float* Ts = ts_ptr(smem);
  const long c0 = n0 + q.wn * 128 + 8 * q.r16;
  const int nvalid = (int)min(8L, ni - c0);
  f32x4 pacc[3][8];
#pragma unroll
  for (int o = 0; o < 3; ++o)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) pacc[o][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // Per m-block inputs of the GLU backward: G and U for the lane's 8 columns
  // of its four rows, and (s T_g), (s T_u) of those rows for its rank r16.
  // They are fetched as one batch per m-block (four rows in flight at once
  // instead of one); fetching further ahead does not fit the registers.
  struct MbIn {
    Row8<T> g[4], u[4];
    float tg[4], tu[4];
  };
  auto fetch = [&](int mb, MbIn& in) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long row = m0 + acc_row(q, mb, j);
      const bool live = row < a.N && nvalid > 0;
      in.g[j] = fetch_row8<T>(live ? Gs + row * ni : nullptr, c0, ni, a.vecO);
      in.u[j] = fetch_row8<T>(live ? Us + row * ni : nullptr, c0, ni, a.vecO);
      const bool ok = row < a.N && q.r16 < a.r;
      in.tg[j] = ok ? a.sg * a.Tg[row * a.r + q.r16] : 0.f;
      in.tu[j] = ok ? a.su * a.Tu[row * a.r + q.r16] : 0.f;
    }
  };
  // GLU backward of m-block mb (H, dG, dU for the lane's 8 columns of each
  // row; stores dG, dU), then the row-block partials: dA_d^T from dT_d
  // (Ts slot 0) and H; dB_g, dB_u from (s T_g), (s T_u) and dG, dU, as MFMAs
  // whose K runs over the block's rows (a lane's K slots are its rows j).
  auto glu_row = [&](int mb, int j, const MbIn& in, float (&h8)[8], float (&g8)[8], float (&u8)[8]) {
    const long row = m0 + acc_row(q, mb, j);
    const bool live = row < a.N && nvalid > 0;
    float G8[8], U8[8], dH8[8];
    unpack_row8<T>(in.g[j], G8);
    unpack_row8<T>(in.u[j], U8);
    if constexpr (TR) {
      park_row(wpark + 4096 * mb, j, q, dH8);
    } else {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) dH8[nb] = acc[mb][nb][j];
    }
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      float ph, dph;
      act_both<ACT>(G8[nb], ph, dph);
      g8[nb] = dH8[nb] * U8[nb] * dph;
      u8[nb] = dH8[nb] * ph;
      h8[nb] = ph * U8[nb];
    }
    if (live) {
      store_row8<T>(dGo + row * ni + c0, g8, nvalid, a.vecO);
      store_row8<T>(dUo + row * ni + c0, u8, nvalid, a.vecO);
    }
  };
  auto process = [&](int mb, const MbIn& in) {
    const Frag4<T> adT = ts_frag4<T>(Ts, 0, 1.f, q, mb);
    const Frag4<T> aTg = make_frag4<T>(in.tg);
    const Frag4<T> aTu = make_frag4<T>(in.tu);
    if constexpr (sizeof(T) == 2) {
      // bf16: rows (2 jp, 2 jp + 1) go straight into packed fragment dwords.
      u32x2 fh[8], fg[8], fu[8];
#pragma unroll
      for (int jp = 0; jp < 2; ++jp) {
        float h0[8], g0[8], u0[8], h1[8], g1[8], u1[8];
        glu_row(mb, 2 * jp, in, h0, g0, u0);
        glu_row(mb, 2 * jp + 1, in, h1, g1, u1);
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          fh[nb][jp] = pack_bf2(h0[nb], h1[nb]);
          fg[nb][jp] = pack_bf2(g0[nb], g1[nb]);
          fu[nb][jp] = pack_bf2(u0[nb], u1[nb]);
        }
      }
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        Frag4<T> b0, b1, b2;
        b0.v = fh[nb];
        b1.v = fg[nb];
        b2.v = fu[nb];
        pacc[0][nb] = mma4(pacc[0][nb], adT, b0);
        pacc[1][nb] = mma4(pacc[1][nb], aTg, b1);
        pacc[2][nb] = mma4(pacc[2][nb], aTu, b2);
      }
    } else {
      float hv[4][8], gv[4][8], uv[4][8];    // [j][nb]
#pragma unroll
      for (int j = 0; j < 4; ++j) glu_row(mb, j, in, hv[j], gv[j], uv[j]);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const float b0[4] = {hv[0][nb], hv[1][nb], hv[2][nb], hv[3][nb]};
        const float b1[4] = {gv[0][nb], gv[1][nb], gv[2][nb], gv[3][nb]};
        const float b2[4] = {uv[0][nb], uv[1][nb], uv[2][nb], uv[3][nb]};
        pacc[0][nb] = mma4(pacc[0][nb], adT, make_frag4<T>(b0));
        pacc[1][nb] = mma4(pacc[1][nb], aTg, make_frag4<T>(b1));
        pacc[2][nb] = mma4(pacc[2][nb], aTu, make_frag4<T>(b2));
      }
    }
  };
  constexpr int PD = 0;                      // fetch distance in m-blocks
  MbIn in[kMB];
#pragma unroll
  for (int mb = 0; mb < PD; ++mb) fetch(mb, in[mb]);
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) {
    if (mb + PD < kMB) fetch(mb + PD, in[mb + PD]);
    process(mb, in[mb]);
    asm volatile("" ::: "memory");   // keep later fetches from being hoisted (register pressure)
  }
  float* const parts[3] = {a.pA_d + (long)rb * ni * 16, a.pB_g + (long)rb * ni * 16, a.pB_u + (long)rb * ni * 16};
  reduce_store_partials<3>(smem, pacc, parts, n0, ni);
}

// ===========================================================================
// Shared dX epilogue: store dX, then dA_p partials = (scale_p Ts_p)^T . X.
// TR: the accumulators are in natural column order and go through a 4 KB
// per-wave park (after the three Ts slots) one m-block at a time.
// ===========================================================================
constexpr int kParkOff = kTsBytes;

// BUFX (bf16; X rows aligned, X at most 2 GB): X rows come by raw buffer
// loads, branch-free, so a fetch stays in flight across the previous block.
template <class T, int NA, bool TR, bool BUFX = false>
__device__ __forceinline__ void dx_epilogue(char* smem, f32x4 (&acc)[kMB][8], const float (&escale)[kMaxSide],
                                            const T* X, T* dX, float* const (&parts)[NA], long N, long h, long m0,
                                            long n0, bool vecO) {
  const WaveId q = wave_id();
  const float* Ts = ts_ptr(smem);
  const long c0 = n0 + q.wn * 128 + 8 * q.r16;
  const int nvalid = (int)min(8L, h - c0);
  char* wpark = smem + kParkOff + q.w * 4096;
  f32x4 pacc[NA][8];
#pragma unroll
  for (int o = 0; o < NA; ++o)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) pacc[o][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // X rows of m-block mb (the B operand of the dA partials), fetched as one
  // batch per m-block and, with at most two adapters (registers allow), one
  // m-block ahead so the loads overlap the previous block's work.
  auto fetch = [&](int mb, Row8<T> (&x)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long row = m0 + acc_row(q, mb, j);
      const bool live = row < N && nvalid > 0;
      if constexpr (BUFX) {
        static_assert(sizeof(T) == 2, "buffer-load X fetch is bf16");
        x[j].c[0] = buf_load16(buf_rsrc(X, (unsigned)(N * h * 2)), live ? (unsigned)((row * h + c0) * 2) : kBufOut);
      } else {
        x[j] = fetch_row8<T>(live ? X + row * h : nullptr, c0, h, vecO);
      }
    }
  };
  constexpr int PD = NA <= 2 ? 1 : 0;
  Row8<T> xin[kMB][4];
#pragma unroll
  for (int mb = 0; mb < PD; ++mb) fetch(mb, xin[mb]);
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) {
    if (mb + PD < kMB) fetch(mb + PD, xin[mb + PD]);
    if constexpr (TR) park_mb(wpark, acc, mb, q);
    float xv[4][8];   // [j][nb]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long row = m0 + acc_row(q, mb, j);
      if (row < N && nvalid > 0) {
        float v[8];
        if constexpr (TR) {
          park_row(wpark, j, q, v);
        } else {
#pragma unroll
          for (int nb = 0; nb < 8; ++nb) v[nb] = acc[mb][nb][j];
        }
        store_row8<T>(dX + row * h + c0, v, nvalid, vecO);
      }
      unpack_row8<T>(xin[mb][j], xv[j]);
    }
    Frag4<T> adT[NA];
#pragma unroll
    for (int o = 0; o < NA; ++o) adT[o] = ts_frag4<T>(Ts, o, escale[o], q, mb);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const float b[4] = {xv[0][nb], xv[1][nb], xv[2][nb], xv[3][nb]};
      const Frag4<T> bf = make_frag4<T>(b);
#pragma unroll
      for (int o = 0; o < NA; ++o) pacc[o][nb] = mma4(pacc[o][nb], adT[o], bf);
    }
    asm volatile("" ::: "memory");   // keep later fetches from being hoisted (register pressure)
  }
  reduce_store_partials<NA>(smem, pacc, parts, n0, h);
}

// ===========================================================================
// MLP dX
// ===========================================================================
struct MlpDxArgs {
  const void* dG; const void* dU;
  const void* Wg; const void* Wu;
  const void* Bg; const void* Bu;
  const void* Ag; const void* Au;
  const void* X;
  float sg, su;
  void* dX;
  float* pA_g; float* pA_u;       // [R][h][16]
  long N; int h, i, r;
  int vecA, vecW, vecS, vecO;
  int R, NC;
  SplitK sk;                      // fast path only; sk.S == 1: no split
  const float* dT;                // k_mlp_dx_pp: [2][N][16] dT_g, dT_u (summed k_mlp_dt partials)
};

// SPLIT (fast path only): the K range is split over a.sk.S workgroups per
// tile; a separate instantiation, so the merge costs the unsplit kernel no
// registers.
template <class T, bool FAST, bool SPLIT = false>
__global__ __launch_bounds__(kGemmThreads, 1) void k_mlp_dx_bwd(MlpDxArgs a) {
  constexpr bool TR = sizeof(T) == 2;
  static_assert(FAST || !SPLIT, "split K on the fast path only");
  __shared__ __align__(16) char smem[FAST ? kGemmLdsX : kGemmLds];
  const int S = SPLIT ? a.sk.S : 1;
  const bool merge = SPLIT && a.sk.pass == 1;      // split K: merge pass (grid = tiles)
  const int tile = merge ? (int)blockIdx.x : (int)blockIdx.x / S, split = merge ? 0 : (int)blockIdx.x % S;
  int rb, cb;
  tile_coords_at(tile, a.R * a.NC, a.R, a.NC, 8, rb, cb);
  const long m0 = (long)rb * kBM;
  const long n0 = (long)cb * kBN;
  const long h = a.h, ni = a.i, r = a.r;
  const T* Wg = static_cast<const T*>(a.Wg);
  const T* Wu = static_cast<const T*>(a.Wu);
  const T* Bg = static_cast<const T*>(a.Bg);
  const T* Bu = static_cast<const T*>(a.Bu);
  const T* dG = static_cast<const T*>(a.dG);
  const T* dU = static_cast<const T*>(a.dU);
  constexpr int BK = ET<T>::BK;

  f32x4 acc[kMB][8];
  zero_acc(acc);
  const int nkt = (int)((2 * ni + BK - 1) / BK);
  if constexpr (FAST) {
    // bf16, i % 64 == 0, r == 16: the dG tiles carry only dT_g, the dU tiles
    // only dT_u.  Two K-loop phases with one side accumulator; dT_g parks in
    // the flush slot.
    f32x4 sacc[1][kMB];
    if (merge) {
      split_load<1>(a.sk, tile, acc, sacc, reinterpret_cast<float*>(smem + kFlushOff));
    } else {
      KNPairLoader<KRow2<bf16>, SRowLin<bf16>, 1> ld;
      ld.krow.W0 = Wg; ld.krow.W1 = Wu; ld.krow.K0 = ni; ld.krow.K1 = ni; ld.krow.ld = h;
      ld.srow.B = Bg; ld.srow.kb = 0; ld.srow.ld = r;          // phase 1: B_g rows
      ld.init(dG, dU, ni, ni, a.N, m0, h, n0, h, r);
      zero_side(sacc);
      const int nk0 = (int)(ni / 64);
      int kb, ke;                                      // this split's K tiles over both phases
      split_range(2 * nk0, S, split, kb, ke);
      kloop2tr<1>(smem, min(ke, nk0), ld, acc, sacc, kb);
      {
        const WaveId q = wave_id();
        float* fl = reinterpret_cast<float*>(smem + kFlushOff);
        if (q.wn == 0)
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j) fl[acc_row(q, mb, j) * kSlot + q.r16] = sacc[0][mb][j];
        __syncthreads();
        if (q.wn == 1)
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j) fl[acc_row(q, mb, j) * kSlot + q.r16] += sacc[0][mb][j];
      }
      zero_side(sacc);
      ld.srow.B = Bu;                                  // phase 2: B_u rows
      ld.srow.kb = ni;
      kloop2tr<1>(smem, ke, ld, acc, sacc, max(kb, nk0));
      if constexpr (SPLIT) {
        split_store<1>(a.sk, tile, split, acc, sacc, reinterpret_cast<const float*>(smem + kFlushOff));
        return;
      }
    }
    side_reduce<T, 1>(smem, sacc, 1);                // dT_u -> slot 1
    {
      float* Ts = ts_ptr(smem);
      const float* fl = reinterpret_cast<const float*>(smem + kFlushOff);
      for (int e = threadIdx.x; e < kBM * kSlot; e += kGemmThreads) Ts[e] = fl[e];   // dT_g -> slot 0
      __syncthreads();
    }
  } else if constexpr (TR) {
    KNTrLoader<RowsA<T>, KRow2<T>, SRow2<T>, SMask2, 2> ld;
    ld.a.init(dG, dU, ni, ni, ni, a.N, m0, a.vecA);
    ld.krow.W0 = Wg; ld.krow.W1 = Wu; ld.krow.K0 = ni; ld.krow.K1 = ni; ld.krow.ld = h;
    ld.srow.B0 = Bg; ld.srow.lo0 = 0; ld.srow.hi0 = ni;
    ld.srow.B1 = Bu; ld.srow.lo1 = ni; ld.srow.hi1 = 2 * ni;
    ld.srow.ld = r;
    ld.smask_of.K0 = ni; ld.smask_of.BK = BK;
    ld.n0 = n0; ld.N = h; ld.vecB = a.vecW; ld.r = a.r; ld.vecS = a.vecS;
    f32x4 sacc[2][kMB];
    zero_side(sacc);
    kloop<T, 2>(smem, nkt, ld, acc, sacc);
    side_reduce<T, 2>(smem, sacc);
  } else {
    KNLoader32<KRow2<T>, SRow2<T>, SMask2, 2> ld;
    ld.a.init(dG, dU, ni, ni, ni, a.N, m0, a.vecA);
    ld.krow.W0 = Wg; ld.krow.W1 = Wu; ld.krow.K0 = ni; ld.krow.K1 = ni; ld.krow.ld = h;
    ld.srow.B0 = Bg; ld.srow.lo0 = 0; ld.srow.hi0 = ni;
    ld.srow.B1 = Bu; ld.srow.lo1 = ni; ld.srow.hi1 = 2 * ni;
    ld.srow.ld = r;
    ld.smask_of.K0 = ni; ld.smask_of.BK = BK;
    ld.n0 = n0; ld.N = h; ld.vecB = a.vecW; ld.r = a.r; ld.vecS = a.vecS;
    f32x4 sacc[2][kMB];
    zero_side(sacc);
    kloop<T, 2>(smem, nkt, ld, acc, sacc);
    side_reduce<T, 2>(smem, sacc);
  }

  const T* Ag = static_cast<const T*>(a.Ag);
  const T* Au = static_cast<const T*>(a.Au);
  auto fb = [&](int R, int slot, int t0, float* v) {
    const long n = n0 + (TR ? R : lds_row_col(0, R));
    if (n >= h) return;
    const T* src = (slot == 0) ? Ag : Au;
    load_rank<T, ET<T>::VEC>(src + n, h, t0, a.r, v);
  };
  const float fs[kMaxSide] = {a.sg, a.su, 0.f};
  fold<T>(smem, acc, 2, fs, fb);

  float* const parts[2] = {a.pA_g + (long)rb * h * 16, a.pA_u + (long)rb * h * 16};
  dx_epilogue<T, 2, TR, FAST>(smem, acc, fs, static_cast<const T*>(a.X), static_cast<T*>(a.dX), parts, a.N, h, m0, n0,
                        a.vecO);
}

// dT_g = dG B_g and dT_u = dU B_u ([N][16] each) on their own: a streaming
// pass over [dG | dU] (K = 2i in chunks of 64 columns, grid row blocks x KS
// K splits), so that the dX GEMM needs no side product.  Each workgroup
// keeps three chunks in flight in a ring of four LDS stages (direct loads:
// the token rows in the GEMM's 128-byte layout, the 64 B rows of the chunk
// as [64 k][16 t]); wave w multiplies rows 32 w .. 32 w + 31.  Partials
// [KS][3][N][16] (slots 0, 1), summed in a fixed order by k_dt_sum.  A
// workgroup walks its K range from the top down: k_down_bwd writes each row
// group's column tiles in ascending order, so the highest columns of a range
// are the most recently written and the likeliest to be still in the 256 MB
// MALL; read first, they are read before this pass's own misses evict them.
struct MlpDtArgs {
  const void* dG; const void* dU;  // [N][i]
  const void* Bg; const void* Bu;  // [i][16]
  float* part;                     // [KS][3][N][16]
  long N; int i, KS;
};
constexpr int kDtStage = kStage2A + 64 * 32;
constexpr int kDtStages = 4;

template <class T>
__global__ __launch_bounds__(kGemmThreads, 1) void k_mlp_dt(MlpDtArgs a) {
  static_assert(sizeof(T) == 2, "bf16, i % 64 == 0, r == 16");
  __shared__ __align__(16) char smem[kDtStages * kDtStage];
  const WaveId q = wave_id();
  const int L = q.lane, w = __builtin_amdgcn_readfirstlane(q.w);
  const long m0 = (long)blockIdx.x * kBM;
  const int nk0 = a.i / 64;
  int cb, ce;
  split_range(2 * nk0, a.KS, (int)blockIdx.y, cb, ce);
  const bf16* dG = static_cast<const bf16*>(a.dG);
  const bf16* dU = static_cast<const bf16*>(a.dU);
  const bf16* Bg = static_cast<const bf16*>(a.Bg);
  const bf16* Bu = static_cast<const bf16*>(a.Bu);
  int aoff[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    long row = m0 + direct2_row(it);
    if (row > a.N - 1) row = a.N - 1;
    aoff[it] = (int)(row * a.i) + direct2_chunk(L) * 8;
  }
  const int ci = 16 * w + L;                       // B chunk (lanes < 16): k row ci / 2, half ci % 2
  const int soff = (ci >> 1) * 16 + 8 * (ci & 1);
  auto issue = [&](int c) {
    char* S = smem + (c & (kDtStages - 1)) * kDtStage;
    const int cid = cb + ce - 1 - c;
    const bool up = cid >= nk0;
    const long k = (long)(cid - (up ? nk0 : 0)) * 64;
    const bf16* A = (up ? dU : dG) + k;
#pragma unroll
    for (int it = 0; it < 4; ++it) g2lds16(A + aoff[it], S + direct_blk(it) * 1024);
    if (L < 16) g2lds16((up ? Bu : Bg) + k * 16 + soff, S + kStage2A + 256 * w);
  };
  f32x4 acc[2][2];
#pragma unroll
  for (int sl = 0; sl < 2; ++sl)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) acc[sl][mb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kDtStages - 1; ++j)
    if (cb + j < ce) issue(cb + j);
  for (int c = cb; c < ce; ++c) {
    // Chunk c has landed once at most the later chunks' loads (5 per chunk
    // and wave, retired in order) are outstanding.
    if (c + 2 < ce) vm_wait<10>();
    else if (c + 1 < ce) vm_wait<5>();
    else vm_wait<0>();
    asm volatile("s_barrier" ::: "memory");
    // The stage refilled here was read in the previous iteration by every
    // wave, before the barrier.
    if (c + kDtStages - 1 < ce) issue(c + kDtStages - 1);
    const char* S = smem + (c & (kDtStages - 1)) * kDtStage;
    u32x4 av[2][2];
    u32x2 lo[2], hi[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) av[ks][mb] = rd128(S + lds_off2(32 * w + 16 * mb + q.r16, ks * 4 + q.g));
      tr_side_issue(S + kStage2A + ks * 1024, q, lo[ks], hi[ks]);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) tie<0>(av[ks][mb]);
      lgkm_tie0(lo[ks], hi[ks]);
    }
    const bool up = (cb + ce - 1 - c) >= nk0;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const Frag<bf16> bfr = tr_make(lo[ks], hi[ks]);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        Frag<bf16> af;
        af.v = av[ks][mb];
        if (up) acc[1][mb] = mma(acc[1][mb], af, bfr);
        else acc[0][mb] = mma(acc[0][mb], af, bfr);
      }
    }
  }
  // C layout: lane (t = r16, g) holds rows 4 g + j of each m-block.
#pragma unroll
  for (int sl = 0; sl < 2; ++sl)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const long row = m0 + 32 * w + 16 * mb + 4 * q.g + j;
        if (row < a.N) a.part[(((long)blockIdx.y * 3 + sl) * a.N + row) * 16 + q.r16] = acc[sl][mb][j];
      }
}

// Fast path without split K when dT_g, dT_u come precomputed (k_mlp_dt):
// the ping-pong K-loop over [dG | dU] [W_g; W_u] without side work, then the
// fold and the dX epilogue as in k_mlp_dx_bwd.
template <class T>
__global__ __launch_bounds__(kGemmThreads, 1) void k_mlp_dx_pp(MlpDxArgs a) {
  static_assert(sizeof(T) == 2, "bf16 fast path");
  __shared__ __align__(16) char smem[kGemmLds];
  int rb, cb;
  tile_coords(a.R * a.NC, a.R, a.NC, 8, rb, cb);
  const long m0 = (long)rb * kBM;
  const long n0 = (long)cb * kBN;
  const long h = a.h, ni = a.i;
  f32x4 acc[kMB][8];
  zero_acc(acc);
  KRow2<bf16> kr;
  kr.W0 = static_cast<const bf16*>(a.Wg); kr.W1 = static_cast<const bf16*>(a.Wu);
  kr.K0 = ni; kr.K1 = ni; kr.ld = h;
  kloop2tr_pp(smem, (int)(2 * ni / 64), static_cast<const bf16*>(a.dG), static_cast<const bf16*>(a.dU), ni, kr, ni,
              a.N, m0, h, n0, h, acc);
  load_dT(smem, a.dT, a.N, m0, 2);
  const bf16* Ag = static_cast<const bf16*>(a.Ag);
  const bf16* Au = static_cast<const bf16*>(a.Au);
  auto fb = [&](int R, int slot, int t0, float* v) {
    const long n = n0 + R;
    if (n >= h) return;
    load_rank<bf16, 8>((slot == 0 ? Ag : Au) + n, h, t0, a.r, v);
  };
  const float fs[kMaxSide] = {a.sg, a.su, 0.f};
  fold<bf16>(smem, acc, 2, fs, fb);
  float* const parts[2] = {a.pA_g + (long)rb * h * 16, a.pA_u + (long)rb * h * 16};
  dx_epilogue<bf16, 2, true, true>(smem, acc, fs, static_cast<const bf16*>(a.X), static_cast<bf16*>(a.dX), parts,
                                   a.N, h, m0, n0, a.vecO);
}

// ===========================================================================
// Projection dX over NP projections stacked along K (QKV: NP = 3; one LoRA
// linear: NP = 1): dX = dP [W_1; ...; W_NP] + sum_p dT_p A_p; partials of dA_p.
// ===========================================================================
struct ProjDxArgs {
  const void* dP;                 // [N][O], projection p in columns off[p] .. off[p+1]
  const void* W[3]; const void* A[3];
  const float* dT;                // [3][N][16]
  const void* X;
  void* dX;
  float* pA[3];                   // [R][h][16]
  long N; int h, O, r;
  int off[4];
  int vecA, vecW, vecO;
  int R, NC;
};

template <class T, bool FAST, int NP>
__global__ __launch_bounds__(kGemmThreads, 1) void k_proj_dx_bwd(ProjDxArgs a) {
  constexpr bool TR = sizeof(T) == 2;
  __shared__ __align__(16) char smem[kGemmLds];
  int rb, cb;
  tile_coords(a.R * a.NC, a.R, a.NC, 8, rb, cb);
  const long m0 = (long)rb * kBM;
  const long n0 = (long)cb * kBN;
  const long h = a.h;
  const T* dP = static_cast<const T*>(a.dP);
  KRow3<T> kr;
  kr.W0 = static_cast<const T*>(a.W[0]);
  kr.W1 = static_cast<const T*>(a.W[NP > 1 ? 1 : 0]);
  kr.W2 = static_cast<const T*>(a.W[NP > 2 ? 2 : 0]);
  kr.o1 = a.off[1]; kr.o2 = a.off[2]; kr.o3 = a.off[3]; kr.ld = h;

  f32x4 acc[kMB][8];
  f32x4 sacc[1][kMB];
  zero_acc(acc);
  const int nkt = (a.O + ET<T>::BK - 1) / ET<T>::BK;
  if constexpr (FAST) {
    static_assert(TR, "the fast path is bf16");
    // O % 64 == 0
    kloop2tr_pp(smem, a.O / 64, reinterpret_cast<const bf16*>(dP), nullptr, a.O, kr, a.O, a.N, m0, h, n0, h, acc);
  } else if constexpr (TR) {
    KNTrLoader<RowsA<T>, KRow3<T>, SRowNone<T>, SMaskNone, 0> ld;
    ld.a.init(dP, nullptr, a.O, 0, a.O, a.N, m0, a.vecA);
    ld.krow = kr;
    ld.n0 = n0; ld.N = h; ld.vecB = a.vecW; ld.r = a.r; ld.vecS = false;
    kloop<T, 0>(smem, nkt, ld, acc, sacc);
  } else {
    KNLoader32<KRow3<T>, SRowNone<T>, SMaskNone, 0> ld;
    ld.a.init(dP, nullptr, a.O, 0, a.O, a.N, m0, a.vecA);
    ld.krow = kr;
    ld.n0 = n0; ld.N = h; ld.vecB = a.vecW; ld.r = a.r; ld.vecS = false;
    kloop<T, 0>(smem, nkt, ld, acc, sacc);
  }

  load_dT(smem, a.dT, a.N, m0, NP);
  auto fb = [&](int R, int slot, int t0, float* v) {
    const long n = n0 + (TR ? R : lds_row_col(0, R));
    if (n >= h) return;
    const T* src = static_cast<const T*>(a.A[slot < NP ? slot : 0]);
    load_rank<T, ET<T>::VEC>(src + n, h, t0, a.r, v);
  };
  const float fs[kMaxSide] = {1.f, 1.f, 1.f};
  fold<T>(smem, acc, NP, fs, fb);

  const long po = (long)rb * h * 16;
  if constexpr (NP == 1) {
    float* const parts[1] = {a.pA[0] + po};
    dx_epilogue<T, 1, TR, FAST>(smem, acc, fs, static_cast<const T*>(a.X), static_cast<T*>(a.dX), parts, a.N, h, m0, n0,
                          a.vecO);
  } else {
    static_assert(NP == 3, "one or three stacked projections");
    float* const parts[3] = {a.pA[0] + po, a.pA[1] + po, a.pA[2] + po};
    dx_epilogue<T, 3, TR, FAST>(smem, acc, fs, static_cast<const T*>(a.X), static_cast<T*>(a.dX), parts, a.N, h, m0, n0,
                          a.vecO);
  }
}

// ===========================================================================
// Fixed-order reduction of [nslice][cols][16] partials.
//   transpose = 1: out[t][col] (dA, [r, cols]);  0: out[col][t] (dB, [cols, r]).
// ===========================================================================
struct RedJob {
  const float* part;
  long stride;                   // elements between consecutive slices
  long count;                    // elements per slice (cols * 16)
  int nslice;
  int cols;
  int transpose;
  void* out;
};
struct RedArgs {
  RedJob job[6];
  int njobs;
  int r;
};

template <class T>
__global__ __launch_bounds__(256) void k_reduce(RedArgs a) {
  const RedJob& jb = a.job[blockIdx.y];
  const long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= jb.count) return;
  const int t = (int)(e & 15);
  const long col = e >> 4;
  if (t >= a.r) return;
  // Row-block partials are added in row-block order, loaded eight at a time
  // so the loads overlap (the sum is unchanged).
  const float* src = jb.part + e;
  float v = 0.f;
  int x = 0;
  for (; x + 8 <= jb.nslice; x += 8) {
    float b[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) b[u] = src[(long)(x + u) * jb.stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) v += b[u];
  }
  for (; x < jb.nslice; ++x) v += src[(long)x * jb.stride];
  T* out = static_cast<T*>(jb.out);
  if (jb.transpose) out[(long)t * jb.cols + col] = from_f<T>(v);
  else out[col * a.r + t] = from_f<T>(v);
}

}  // namespace lora

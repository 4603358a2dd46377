// Forward kernels: LoRA gate/up + GLU, LoRA down, LoRA QKV + RoPE + GQA split,
// and the RoPE angle table.
//
// Math (Opake "Model Patches and Kernels": "Fused LoRA operations",
// "Activation functions", "Rotary position embeddings (RoPE)"):
//   G = X W_g^T + s_g (X A_g^T) B_g^T,  U likewise,  H = phi(G) * U,
//   Y = H W_d^T + s_d (H A_d^T) B_d^T,
//   P_p = X W_p^T + s_p (X A_p^T) B_p^T for p in {q, k, v}; Q, K rotated.
#pragma once

#include <type_traits>

#include "gemm.h"

namespace lora {

// ===========================================================================
// gate/up: one tile = 256 tokens x (128 gate columns + the same 128 up columns)
// ===========================================================================
struct GateUpArgs {
  const void* X; const void* Wg; const void* Ag; const void* Bg;
  const void* Wu; const void* Au; const void* Bu;
  float sg, su;
  void* G; void* U; void* H;
  float* Tg; float* Tu;
  long N; int h, i, r;
  int vecA, vecW, vecS, vecO;
  int R, NC;
  int L, RPB, nruns;   // run kernel: run length, runs per row block, runs
};

// LDS row R of the B tile -> (is_up, intermediate column index j).
__device__ __forceinline__ void gateup_row(int R, int j0, int& is_up, int& j) {
  const int w = perm_col(1, R & 15, (R >> 4) & 7);   // G = 2: [gate 64 | up 64] per wave window
  is_up = w >> 6;
  j = j0 + (R >> 7) * 64 + (w & 63);
}

template <class T, int ACT, bool FAST>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gateup_fwd(GateUpArgs a) {
  __shared__ __align__(16) char smem[kGemmLds];
  const WaveId q = wave_id();
  int rb, cb;
  tile_coords(a.R * a.NC, a.R, a.NC, 8, rb, cb);
  const long m0 = (long)rb * kBM;
  const int j0 = cb * 128;
  const T* X = static_cast<const T*>(a.X);
  const T* Wg = static_cast<const T*>(a.Wg);
  const T* Wu = static_cast<const T*>(a.Wu);
  const T* Ag = static_cast<const T*>(a.Ag);
  const T* Au = static_cast<const T*>(a.Au);

  auto brow_of = [&](int R) -> const T* {
    int up, j;
    gateup_row(R, j0, up, j);
    return (j < a.i) ? (up ? Wu : Wg) + (long)j * a.h : nullptr;
  };
  auto side_base = [&](int sb) -> const T* { return sb == 0 ? Ag : Au; };   // side rows: A_g, then A_u

  f32x4 acc[kMB][8];
  f32x4 sacc[2][kMB];
  zero_acc(acc);
  zero_side(sacc);
  if constexpr (FAST) {
    NKPairLoader<2> ld;
    ld.init_a(X, a.h, a.N, m0);
    ld.bfallback = Wg;
    ld.smask = 3u;
#pragma unroll
    for (int it = 0; it < 4; ++it) ld.brow[it] = brow_of(ld.row_of(it));
    ld.srow = Ag;
    const int sr = ld.side_row();
    if (sr >= 0) ld.srow = ld.side_ptr(side_base(sr >> 4), sr & 15, a.r, a.h, Ag);
    kloop2<2>(smem, a.h / 64, ld, acc, sacc);
  } else {
    NKLoader<T, RowsA<T>, 2> ld;
    ld.a.init(X, nullptr, a.h, 0, a.h, a.N, m0, a.vecA);
    ld.bfallback = Wg;
    ld.K = a.h;
    ld.vecB = a.vecW;
    ld.vecS = a.vecS;
    ld.smask = 3u;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) ld.brow[qq] = brow_of(ld.row_of(qq));
    ld.srow = nullptr;
    const int sr = ld.side_row();
    if (sr >= 0) ld.srow = decltype(ld)::side_ptr(side_base(sr >> 4), sr & 15, a.r, a.h, Ag);
    kloop<T, 2>(smem, (a.h + ET<T>::BK - 1) / ET<T>::BK, ld, acc, sacc);
  }
  side_reduce<T, 2>(smem, sacc);

  // The row block's T_g, T_u are saved once (by column block 0).
  if (cb == 0 && q.tid < kBM) {
    const float* Ts = ts_ptr(smem);
    const long row = m0 + q.tid;
    if (row < a.N)
      for (int t = 0; t < a.r; ++t) {
        a.Tg[row * a.r + t] = Ts[ts_idx(0, q.tid, t)];
        a.Tu[row * a.r + t] = Ts[ts_idx(1, q.tid, t)];
      }
  }

  const T* Bg = static_cast<const T*>(a.Bg);
  const T* Bu = static_cast<const T*>(a.Bu);
  auto fb = [&](int R, int slot, int t0, float* v) {
    int up, j;
    gateup_row(R, j0, up, j);
    if (slot != up || j >= a.i) return;
    const T* src = (up ? Bu : Bg) + (long)j * a.r;
    load_rank<T, ET<T>::VEC>(src, 1, t0, a.r, v);
  };
  const float fs[kMaxSide] = {a.sg, a.su, 0.f};
  fold<T>(smem, acc, 2, fs, fb);

  // GLU epilogue: lane holds gate (blocks 0..3) and up (blocks 4..7) of the
  // same 4 consecutive intermediate columns.
  T* Go = static_cast<T*>(a.G);
  T* Uo = static_cast<T*>(a.U);
  T* Ho = static_cast<T*>(a.H);
  const int jj = j0 + q.wn * 64 + 4 * q.r16;
  const int nvalid = min(4, a.i - jj);
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long row = m0 + acc_row(q, mb, j);
      if (row >= a.N || nvalid <= 0) continue;
      float gv[4], uv[4], hv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gv[e] = acc[mb][e][j];
        uv[e] = acc[mb][4 + e][j];
        hv[e] = act_fwd<ACT>(gv[e]) * uv[e];
      }
      const long off = row * a.i + jj;
      gstore_nt<T, 4>(Go + off, gv, nvalid, a.vecO);     // G, U: read again only by the backward
      gstore_nt<T, 4>(Uo + off, uv, nvalid, a.vecO);
      gstore<T, 4>(Ho + off, hv, nvalid, a.vecO);
    }
}


// Fast path (bf16, h % 64 == 0) as runs of column tiles: the side products
// T_g, T_u of the row block are computed in the run's first tile only (the
// later tiles skip the side loads and MFMAs) and folded into every tile from
// the run's fold operand in LDS.
// B rows of a gate/up tile for nk_kloop_pp: block wl + 4 it holds LDS rows
// 8 (wl + 4 it) + L / 8, by gateup_row up for it % 4 >= 2 and intermediate
// column j0 + 64 [it >= 4] + 4 c + ((b0 + 2 (it & 1)) & 3) with x = 8 wl +
// L / 8, c = x % 16, b0 = x / 16: two lane offsets, the rest uniform.
struct GateUpPP {
  const bf16* Wg0; const bf16* Wu0; long half;
  int off[2];
  __device__ __forceinline__ GateUpPP(const bf16* Wg, const bf16* Wu, long h, int j0, int wl, int L) {
    Wg0 = Wg + (long)j0 * h;
    Wu0 = Wu + (long)j0 * h;
    half = 64 * h;
    const int x = 8 * wl + (L >> 3), chunk = direct2_chunk(L);
#pragma unroll
    for (int p = 0; p < 2; ++p) off[p] = (4 * (x & 15) + (((x >> 4) + 2 * p) & 3)) * (int)h + chunk * 8;
  }
  __device__ __forceinline__ const bf16* base(int it) const { return ((it & 3) >= 2 ? Wu0 : Wg0) + (it >= 4 ? half : 0); }
  __device__ __forceinline__ static int sel(int it) { return it & 1; }
};

template <int ACT>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gateup_run(GateUpArgs a) {
  __shared__ __align__(16) char smem[kRunLds];
  int rb, cb0, cb1;
  run_coords(a.nruns, a.RPB, a.L, a.NC, rb, cb0, cb1);
  const long m0 = (long)rb * kBM;
  const bf16* X = static_cast<const bf16*>(a.X);
  const bf16* Wg = static_cast<const bf16*>(a.Wg);
  const bf16* Wu = static_cast<const bf16*>(a.Wu);
  const bf16* Ag = static_cast<const bf16*>(a.Ag);
  const bf16* Au = static_cast<const bf16*>(a.Au);
  const bf16* Bg = static_cast<const bf16*>(a.Bg);
  const bf16* Bu = static_cast<const bf16*>(a.Bu);

  // The loader of a kloop2 tile (X rows, B rows of column block cb, side
  // rows when smask != 0); built where it is used, so nothing of it lives
  // through the ping-pong tiles.
  auto make_ld = [&](int cb, unsigned smask) {
    NKPairLoader<2> ld;
    ld.init_a(X, a.h, a.N, m0);
    ld.bfallback = Wg;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      int up, j;
      gateup_row(ld.row_of(it), cb * 128, up, j);
      ld.brow[it] = (j < a.i) ? (up ? Wu : Wg) + (long)j * a.h : nullptr;
    }
    ld.smask = smask;
    ld.srow = Ag;
    const int sr = ld.side_row();
    if (sr >= 0) ld.srow = ld.side_ptr((sr >> 4) == 0 ? Ag : Au, sr & 15, a.r, a.h, Ag);
    return ld;
  };
  const float fs[kMaxSide] = {a.sg, a.su, 0.f};
  char* FA = smem + kRunFAOff;
  bf16* Go = static_cast<bf16*>(a.G);
  bf16* Uo = static_cast<bf16*>(a.U);
  bf16* Ho = static_cast<bf16*>(a.H);
  const int nkt = a.h / 64;

  // Fold and the GLU epilogue (registers only) of the tile at column block
  // cb: the lane holds gate (blocks 0..3) and up (blocks 4..7) of the same 4
  // consecutive intermediate columns.
  auto finish = [&](int cb, f32x4 (&acc)[kMB][8]) {
    const WaveId q = wave_id_opaque();   // everything after the K-loop derives from this
    const int j0 = cb * 128;
    auto fb = [&](int R, int slot, int t0, float* v) {
      int up, j;
      gateup_row(R, j0, up, j);
      if (slot != up || j >= a.i) return;
      const bf16* src = (up ? Bu : Bg) + (long)j * a.r;
      load_rank<bf16, 8>(src, 1, t0, a.r, v);
    };
    fold_run(FA, smem + kRunFBOff, acc, fb);
    const int jj = j0 + q.wn * 64 + 4 * q.r16;
    const int nvalid = min(4, a.i - jj);
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const long row = m0 + acc_row(q, mb, j);
        if (row >= a.N || nvalid <= 0) continue;
        float gv[4], uv[4], hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gv[e] = acc[mb][e][j];
          uv[e] = acc[mb][4 + e][j];
          hv[e] = act_fwd<ACT>(gv[e]) * uv[e];
        }
        const long off = row * a.i + jj;
        gstore_nt<bf16, 4>(Go + off, gv, nvalid, a.vecO);   // G, U: read again only by the backward
        gstore_nt<bf16, 4>(Uo + off, uv, nvalid, a.vecO);
        gstore<bf16, 4>(Ho + off, hv, nvalid, a.vecO);
      }
  };

  {
    // First tile: T_g, T_u ride the K-loop.
    f32x4 acc[kMB][8];
    f32x4 sacc[2][kMB];
    zero_acc(acc);
    zero_side(sacc);
    {
      const NKPairLoader<2> ld = make_ld(cb0, 3u);
      kloop2<2>(smem, nkt, ld, acc, sacc, 0, false);
    }
    const WaveId q = wave_id_opaque();
    side_reduce<bf16, 2>(smem + kRunTsOff, sacc);
    const float* Ts = ts_ptr(smem + kRunTsOff);
    if (cb0 == 0 && q.tid < kBM) {      // T_g, T_u are saved once per row block
      const long row = m0 + q.tid;
      if (row < a.N)
        for (int t = 0; t < a.r; ++t) {
          a.Tg[row * a.r + t] = Ts[ts_idx(0, q.tid, t)];
          a.Tu[row * a.r + t] = Ts[ts_idx(1, q.tid, t)];
        }
    }
    build_fold_a(FA, Ts, 2, fs);
    finish(cb0, acc);
  }
  // Later tiles carry no side product: whole tiles take the ping-pong loop,
  // a ragged last tile the plain loop without side work.
  for (int cb = cb0 + 1; cb < cb1; ++cb) {
    const int j0 = cb * 128;
    f32x4 acc[kMB][8];
    zero_acc(acc);
    if (j0 + 128 <= a.i) {
      const WaveId qo = wave_id_opaque();
      const GateUpPP bp(Wg, Wu, a.h, j0, __builtin_amdgcn_readfirstlane(qo.w) & 3, qo.lane);
      nk_kloop_pp(smem, nkt, X, a.h, a.N, m0, bp, acc);
    } else {
      const NKPairLoader<2> ld = make_ld(cb, 0u);
      f32x4 snone[1][kMB];
      kloop2<0>(smem, nkt, ld, acc, snone, 0, false);
    }
    finish(cb, acc);
  }
}

// ===========================================================================
// Plain LoRA linear with a row-major output (down projection: Y = L_d(H)).
// ===========================================================================
struct LinearArgs {
  const void* Z; const void* W; const void* A; const void* B;
  const void* bias;    // frozen base bias [O] or nullptr
  float s;
  void* Y; float* T;
  long N; int K, O, r;
  int vecA, vecW, vecS, vecO;
  int R, NC;
  SplitK sk;           // fast path only; sk.S == 1: no split
  int L, RPB, nruns;   // run kernel: run length, runs per row block, runs
};

template <class T, bool FAST>
__global__ __launch_bounds__(kGemmThreads, 1) void k_linear_fwd(LinearArgs a) {
  __shared__ __align__(16) char smem[kGemmLds];
  const WaveId q = wave_id();
  const int S = FAST ? a.sk.S : 1;
  const bool merge = S > 1 && a.sk.pass == 1;      // split K: merge pass (grid = tiles)
  const int tile = merge ? (int)blockIdx.x : (int)blockIdx.x / S, split = merge ? 0 : (int)blockIdx.x % S;
  int rb, cb;
  tile_coords_at(tile, a.R * a.NC, a.R, a.NC, 8, rb, cb);
  const long m0 = (long)rb * kBM;
  const long n0 = (long)cb * kBN;
  const T* Z = static_cast<const T*>(a.Z);
  const T* W = static_cast<const T*>(a.W);
  const T* A = static_cast<const T*>(a.A);

  auto brow_of = [&](int R) -> const T* {
    const long n = n0 + lds_row_col(0, R);
    return (n < a.O) ? W + n * a.K : nullptr;
  };

  f32x4 acc[kMB][8];
  f32x4 sacc[1][kMB];
  zero_acc(acc);
  zero_side(sacc);
  if constexpr (FAST) {
    if (merge) {
      split_load<1>(a.sk, tile, acc, sacc, nullptr);
    } else {
      NKPairLoader<1> ld;
      ld.init_a(Z, a.K, a.N, m0);
      ld.bfallback = W;
      ld.smask = 1u;
#pragma unroll
      for (int it = 0; it < 4; ++it) ld.brow[it] = brow_of(ld.row_of(it));
      ld.srow = A;
      const int sr = ld.side_row();
      if (sr >= 0) ld.srow = ld.side_ptr(A, sr, a.r, a.K, A);
      int kb, ke;
      split_range(a.K / 64, S, split, kb, ke);
      kloop2<1>(smem, ke, ld, acc, sacc, kb);
      if (S > 1) {
        split_store<1>(a.sk, tile, split, acc, sacc, nullptr);
        return;
      }
    }
  } else {
    NKLoader<T, RowsA<T>, 1> ld;
    ld.a.init(Z, nullptr, a.K, 0, a.K, a.N, m0, a.vecA);
    ld.bfallback = W;
    ld.K = a.K;
    ld.vecB = a.vecW;
    ld.vecS = a.vecS;
    ld.smask = 1u;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) ld.brow[qq] = brow_of(ld.row_of(qq));
    ld.srow = nullptr;
    const int sr = ld.side_row();
    if (sr >= 0) ld.srow = decltype(ld)::side_ptr(A, sr, a.r, a.K, A);
    kloop<T, 1>(smem, (a.K + ET<T>::BK - 1) / ET<T>::BK, ld, acc, sacc);
  }
  side_reduce<T, 1>(smem, sacc);

  if (cb == 0 && q.tid < kBM) {
    const float* Ts = ts_ptr(smem);
    const long row = m0 + q.tid;
    if (row < a.N)
      for (int t = 0; t < a.r; ++t) a.T[row * a.r + t] = Ts[ts_idx(0, q.tid, t)];
  }

  const T* B = static_cast<const T*>(a.B);
  auto fb = [&](int R, int slot, int t0, float* v) {
    const long n = n0 + lds_row_col(0, R);
    if (slot != 0 || n >= a.O) return;
    load_rank<T, ET<T>::VEC>(B + n * a.r, 1, t0, a.r, v);
  };
  const float fs[kMaxSide] = {a.s, 0.f, 0.f};
  fold<T>(smem, acc, 1, fs, fb);

  T* Y = static_cast<T*>(a.Y);
  const long c0 = n0 + q.wn * 128 + 8 * q.r16;
  const int nvalid = (int)min(8L, a.O - c0);
  float bv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (a.bias) {
    const T* bp = static_cast<const T*>(a.bias) + c0;
    for (int nb = 0; nb < nvalid; ++nb) bv[nb] = to_f<T>(bp[nb]);
  }
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long row = m0 + acc_row(q, mb, j);
      if (row >= a.N || nvalid <= 0) continue;
      float v[8];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) v[nb] = acc[mb][nb][j] + bv[nb];
      store_row8<T>(Y + row * a.O + c0, v, nvalid, a.vecO);
    }
}

// B rows of a linear tile for nk_kloop_pp (columns in perm_col(0, ..)
// order): block wl + 4 it holds output column n0 + 128 (it / 4) + 2 (it % 4)
// + 8 (x % 16) + x / 16 with x = 8 wl + L / 8: one lane offset.
struct LinearPP {
  const bf16* W0; long K;
  int off[2];
  __device__ __forceinline__ LinearPP(const bf16* W, long Kd, long n0, int wl, int L) {
    W0 = W + n0 * Kd;
    K = Kd;
    const int x = 8 * wl + (L >> 3);
    off[0] = off[1] = (8 * (x & 15) + (x >> 4)) * (int)Kd + direct2_chunk(L) * 8;
  }
  __device__ __forceinline__ const bf16* base(int it) const { return W0 + (128 * (it >> 2) + 2 * (it & 3)) * K; }
  __device__ __forceinline__ static int sel(int) { return 0; }
};

// Fast path without split K as runs of column tiles (k_gateup_run's layout
// and LDS): the run's first tile computes T = Z A^T in its K-loop and builds
// the fold operand s T (bf16); whole later tiles take the ping-pong K-loop,
// a ragged last one the plain loop, neither with side work.
template <class T>
__global__ __launch_bounds__(kGemmThreads, 1) void k_linear_run(LinearArgs a) {
  static_assert(sizeof(T) == 2, "the run kernel is bf16");
  __shared__ __align__(16) char smem[kRunLds];
  int rb, cb0, cb1;
  run_coords(a.nruns, a.RPB, a.L, a.NC, rb, cb0, cb1);
  const long m0 = (long)rb * kBM;
  const bf16* Z = static_cast<const bf16*>(a.Z);
  const bf16* W = static_cast<const bf16*>(a.W);
  const bf16* A = static_cast<const bf16*>(a.A);
  const bf16* B = static_cast<const bf16*>(a.B);
  char* FA = smem + kRunFAOff;
  const float fs[kMaxSide] = {a.s, 0.f, 0.f};
  const int nkt = a.K / 64;

  // The kloop2 loader of the tile at n0 (side rows when smask != 0).
  auto make_ld = [&](long n0, unsigned smask) {
    NKPairLoader<1> ld;
    ld.init_a(Z, a.K, a.N, m0);
    ld.bfallback = W;
    ld.smask = smask;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const long n = n0 + lds_row_col(0, ld.row_of(it));
      ld.brow[it] = (n < a.O) ? W + n * a.K : nullptr;
    }
    ld.srow = A;
    const int sr = ld.side_row();
    if (sr >= 0) ld.srow = ld.side_ptr(A, sr, a.r, a.K, A);
    return ld;
  };

  // Fold and store the tile at column n0 (bias added).
  auto finish = [&](long n0, f32x4 (&acc)[kMB][8]) {
    const WaveId q = wave_id_opaque();   // everything after the K-loop derives from this
    auto fb = [&](int R, int slot, int t0, float* v) {
      const long n = n0 + lds_row_col(0, R);
      if (slot != 0 || n >= a.O) return;
      load_rank<bf16, 8>(B + n * a.r, 1, t0, a.r, v);
    };
    fold_run(FA, smem + kRunFBOff, acc, fb);
    bf16* Y = static_cast<bf16*>(a.Y);
    const long c0 = n0 + q.wn * 128 + 8 * q.r16;
    const int nvalid = (int)min(8L, a.O - c0);
    float bv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (a.bias) {
      const bf16* bp = static_cast<const bf16*>(a.bias) + c0;
      for (int nb = 0; nb < nvalid; ++nb) bv[nb] = to_f<bf16>(bp[nb]);
    }
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const long row = m0 + acc_row(q, mb, j);
        if (row >= a.N || nvalid <= 0) continue;
        float v[8];
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) v[nb] = acc[mb][nb][j] + bv[nb];
        store_row8<bf16>(Y + row * a.O + c0, v, nvalid, a.vecO);
      }
  };

  {
    // First tile: T rides the K-loop.
    const long n0 = (long)cb0 * kBN;
    f32x4 acc[kMB][8];
    f32x4 sacc[1][kMB];
    zero_acc(acc);
    zero_side(sacc);
    {
      const NKPairLoader<1> ld = make_ld(n0, 1u);
      kloop2<1>(smem, nkt, ld, acc, sacc, 0, false);
    }
    const WaveId q = wave_id_opaque();
    side_reduce<bf16, 1>(smem + kRunTsOff, sacc);
    const float* Ts = ts_ptr(smem + kRunTsOff);
    if (cb0 == 0 && q.tid < kBM) {      // T is saved once per row block
      const long row = m0 + q.tid;
      if (row < a.N)
        for (int t = 0; t < a.r; ++t) a.T[row * a.r + t] = Ts[ts_idx(0, q.tid, t)];
    }
    build_fold_a(FA, Ts, 1, fs);
    finish(n0, acc);
  }
  for (int cb = cb0 + 1; cb < cb1; ++cb) {
    const long n0 = (long)cb * kBN;
    f32x4 acc[kMB][8];
    zero_acc(acc);
    if (n0 + kBN <= a.O) {
      const WaveId qo = wave_id_opaque();
      const LinearPP bp(W, a.K, n0, __builtin_amdgcn_readfirstlane(qo.w) & 3, qo.lane);
      nk_kloop_pp(smem, nkt, Z, a.K, a.N, m0, bp, acc);
    } else {
      const NKPairLoader<1> ld = make_ld(n0, 0u);
      f32x4 snone[1][kMB];
      kloop2<0>(smem, nkt, ld, acc, snone, 0, false);
    }
    finish(n0, acc);
  }
}

// ===========================================================================
// RoPE angle table: cos/sin of s * theta^(-2j/d), evaluated in double.
// ===========================================================================
static __global__ void k_rope_table(float* cs, float* sn, int S, int half, double theta) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)S * half) return;
  const int s = (int)(idx / half), j = (int)(idx % half);
  const double ang = (double)s * pow(theta, -2.0 * (double)j / (double)(2 * half));
  cs[idx] = (float)cos(ang);
  sn[idx] = (float)sin(ang);
}

// ===========================================================================
// QKV: [P_q | P_k | P_v] tile = X . [W_q; W_k; W_v]^T + fold, then RoPE on
// q/k columns and the head split into [B, heads, S, d].
// ===========================================================================
struct QKVFwdArgs {
  const void* X;
  const void* W[3]; const void* A[3]; const void* B[3];
  const void* bias[3]; // frozen base biases [O_p] or nullptr, added before RoPE
  const void* nw[2];   // q_norm / k_norm weights [d] (used when norm != 0)
  void* Pn;            // norm: pre-norm q|k projections [N][off[2]]
  float* rinv;         // norm: inverse RMS per token and q/k head [N][nh[0] + nh[1]]
  float eps;
  int norm;
  int vecN;
  float s[3];
  void* out[3];        // Q, K, V
  float* T[3];
  const float* cs; const float* sn;
  long N; int h, S, d, r;
  int nh[3];           // heads per projection
  int off[4];          // column offsets: 0, Oq, Oq+Ok, O
  int vecA, vecW, vecS, vecO;
  int R, NC;
  int L, RPB, nruns;   // run kernel: run length, runs per row block, runs
};

// LG = log2(256 / head_dim): 1 for d = 128, 2 for d = 64 (RoPE pairs share a lane).
// NS = the most projections any 256-column tile overlaps (side blocks held).
// Fast-path loader of the head_dim-64 QKV forward (the interface of
// NKPairLoader): every lane's X, W and adapter row pointers are derived afresh
// in each issue() from an opaque thread id and the uniform arguments, so none
// of them lives through the K-loop.  Kept there, they were spilled in these
// variants, and each scratch reload's vmcnt wait serialised the tile's loads
// (k_qkv_fwd took twice as long as at head_dim 128).  At head_dim 128 the
// pointers fit and the stored-pointer loader is faster.
template <int NSIDE, int LG>
struct QKVRowLoader {
  // Named fields, no arrays: a runtime index into a member array would put
  // the whole loader in scratch memory.
  const bf16* X;
  const bf16 *W0, *W1, *W2;       // base weights of q, k, v
  const bf16 *S0, *S1, *S2;       // adapter rows of side blocks 0..2 (nullptr past the tile's projections)
  const bf16* afall;
  long N, m0;
  int h, n0, r;
  int off1, off2, off3;           // projection column boundaries (off0 = 0)
  unsigned smask;
  __device__ __forceinline__ void issue(int kt, char* As, char* Bs) const {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int L = tid & 63, w = tid >> 6;
    const long k = (long)kt * 64 + ((L & 7) ^ (L >> 3)) * 8;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      long row = m0 + 8 * (w + 8 * it) + (L >> 3);
      if (row > N - 1) row = N - 1;
      g2lds16(X + row * h + k, As + (w + 8 * it) * 1024);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int o = n0 + lds_row_col(LG, 8 * (w + 8 * it) + (L >> 3));
      const bf16* p = W0;
      if (o < off3) {
        if (o < off1) p = W0 + (long)o * h;
        else if (o < off2) p = W1 + (long)(o - off1) * h;
        else p = W2 + (long)(o - off2) * h;
      }
      g2lds16(p + k, Bs + (w + 8 * it) * 1024);
    }
    if constexpr (NSIDE > 0) {
      if (L < 16 * NSIDE) {
        const int ci = w * 16 * NSIDE + L, sr = ci >> 3;
        const int chunk = (ci & 7) ^ (sr & 7);
        const int sl = sr >> 4;
        // Opaque copies: a select among the members themselves is turned into
        // a load from a selected member address, which keeps the loader in
        // scratch memory.
        unsigned long b0 = (unsigned long)S0, b1 = (unsigned long)S1, b2 = (unsigned long)S2;
        asm volatile("" : "+v"(b0), "+v"(b1), "+v"(b2));
        const bf16* base = reinterpret_cast<const bf16*>((sl == 0) ? b0 : ((sl == 1) ? b1 : b2));
        const bf16* srow = base ? base + (long)min(sr & 15, r - 1) * h : afall;
        g2lds16(srow + (long)kt * 64 + chunk * 8, Bs + kBN * kRow2 + w * 256 * NSIDE);
      }
    }
  }
};

// The cos / sin rows of a tile's 256 token rows ([256][d/2] fp32 each, cos
// then sin, 2 KB x d/2 in all) into LDS by direct loads, all issued before
// the tile's first output store and waited for once: a wave's loads and
// stores share one completion counter, so a table load issued between the
// stores of one m-block and the next would also wait for those stores.  Rows
// past N take row N - 1's position (their outputs are not stored).
static_assert(2 * kBM * 64 * 4 <= kGemmLds && 2 * kBM * 64 * 4 <= kRunFAOff, "RoPE slab (head_dim 128) in LDS");
__device__ __forceinline__ void stage_rope_slab(char* slab, const float* cs, const float* sn, long m0, long N, int S,
                                                int half) {
  const int w = (int)(threadIdx.x >> 6), L = (int)(threadIdx.x & 63);
  const int ppr = half >> 2;                       // 16-byte pieces per row
  const int rpi = 64 / ppr;                        // rows per 1 KB load (4 or 8)
  const int nins = kBM / rpi;
  const int lr = L / ppr, lp = L - (L / ppr) * ppr;
  const int r0 = (int)m0 + lr, rmax = (int)N - 1;  // token rows fit 31 bits
  for (int i = w; i < nins; i += 8) {
    const int e = (min(r0 + i * rpi, rmax) % S) * half + lp * 4;
    g2lds16(cs + e, slab + i * 1024);
    g2lds16(sn + e, slab + kBM * half * 4 + i * 1024);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// RoPE + split of a QKV tile after its fold (rows m0.., columns n0..): the
// bias, the optional q/k RMSNorm, the rotation of q and k, and the stores
// into the [B][heads][S][d] outputs.  qe: the wave id after the K-loop;
// slab: the tile's cos / sin rows in LDS (stage_rope_slab).
template <class T, int LG>
__device__ __forceinline__ void qkv_rope_store(QKVFwdArgs a, f32x4 (&acc)[kMB][8], long m0, int n0,
                                               const WaveId& qe, const char* slab) {
  const int O = a.off[3];
  auto proj_of = [&](int o) { return (o < a.off[1]) ? 0 : ((o < a.off[2]) ? 1 : 2); };
  // RoPE + split.  Groups alternate first half / second half of a head, so
  // block b (first half) pairs with block b + cw in the same lane.  Per
  // m-block the lane first reads the cos / sin of its four rows (cw
  // consecutive entries each, one LDS read), then rotates and stores.
  constexpr int cw = 8 >> LG;
  constexpr int NG = 8 / (2 * cw);                    // head-half pair groups per lane
  const int half = a.d >> 1;
  const float* cs = reinterpret_cast<const float*>(slab);
  const float* sn = cs + kBM * half;
  auto load_cw = [&](const float* ptr, float (&v)[cw]) {
    if constexpr (cw == 4) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(ptr);
      v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    } else {
      typedef float f32x2 __attribute__((ext_vector_type(2)));
      const f32x2 t = *reinterpret_cast<const f32x2*>(ptr);
      v[0] = t.x; v[1] = t.y;
    }
  };
  // Bias (x1, x2 halves) and q/k norm weights of the lane's columns (the same
  // for every row).  Two forms of the same loads: per-lane branches at head
  // dim 128, unconditional loads under uniform guards at head dim 64 (each
  // form makes the other variant's register allocation spill about 200 bytes
  // per lane).
  float b1v[NG][cw], b2v[NG][cw];
  float w1v[NG][cw], w2v[NG][cw];
  if constexpr (LG == 1) {
    // Bias of the lane's columns (the same for every row): pair halves x1, x2.
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const int o1 = n0 + qe.wn * 128 + perm_col(LG, qe.r16, 2 * cw * gi);
      const T* bp = nullptr;
      int oo = 0;
      if (o1 < O) {
        const int p = proj_of(o1);
        bp = static_cast<const T*>(p == 0 ? a.bias[0] : (p == 1 ? a.bias[1] : a.bias[2]));
        oo = o1 - a.off[p];
      }
#pragma unroll
      for (int e = 0; e < cw; ++e) {
        b1v[gi][e] = bp ? to_f<T>(bp[oo + e]) : 0.f;
        b2v[gi][e] = bp ? to_f<T>(bp[oo + half + e]) : 0.f;
      }
    }
    // q/k norm weights of the lane's columns (index within the head).
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const int o1 = n0 + qe.wn * 128 + perm_col(LG, qe.r16, 2 * cw * gi);
      const T* wp = nullptr;
      int jj = 0;
      if (a.norm && o1 < a.off[2]) {
        const int p = proj_of(o1);
        wp = static_cast<const T*>(p == 0 ? a.nw[0] : a.nw[1]);
        jj = (o1 - a.off[p]) % a.d;
      }
#pragma unroll
      for (int e = 0; e < cw; ++e) {
        w1v[gi][e] = wp ? to_f<T>(wp[jj + e]) : 1.f;
        w2v[gi][e] = wp ? to_f<T>(wp[jj + half + e]) : 1.f;
      }
    }
  } else {
    // Loads below are issued unconditionally from a valid address (a lane with
    // nothing to read points at W_q and discards the value), so they go out
    // together instead of one branch and one wait each.
    const T* const dummy = static_cast<const T*>(a.W[0]);
    // Bias of the lane's columns (the same for every row): pair halves x1, x2.
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
      for (int e = 0; e < cw; ++e) b1v[gi][e] = b2v[gi][e] = 0.f;
    const bool anyb = a.bias[0] != nullptr || a.bias[1] != nullptr || a.bias[2] != nullptr;
#pragma unroll
    for (int gi = 0; gi < NG && anyb; ++gi) {
      const int o1 = n0 + qe.wn * 128 + perm_col(LG, qe.r16, 2 * cw * gi);
      const int o1c = min(o1, O - 1);
      const int p = proj_of(o1c);
      const T* bp = static_cast<const T*>(p == 0 ? a.bias[0] : (p == 1 ? a.bias[1] : a.bias[2]));
      const bool use = bp != nullptr && o1 < O;
      const T* src = use ? bp + (o1c - a.off[p]) : dummy;
      T v1[cw], v2[cw];
#pragma unroll
      for (int e = 0; e < cw; ++e) {
        v1[e] = src[e];
        v2[e] = src[half + e];
      }
#pragma unroll
      for (int e = 0; e < cw; ++e) {
        b1v[gi][e] = use ? to_f<T>(v1[e]) : 0.f;
        b2v[gi][e] = use ? to_f<T>(v2[e]) : 0.f;
      }
    }
    // q/k norm weights of the lane's columns (index within the head).
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
      for (int e = 0; e < cw; ++e) w1v[gi][e] = w2v[gi][e] = 1.f;
#pragma unroll
    for (int gi = 0; gi < NG && a.norm; ++gi) {
      const int o1 = n0 + qe.wn * 128 + perm_col(LG, qe.r16, 2 * cw * gi);
      const int o1c = min(o1, O - 1);
      const int p = proj_of(o1c);
      const bool use = a.norm && o1 < a.off[2];
      const T* src = use ? static_cast<const T*>(p == 0 ? a.nw[0] : a.nw[1]) + (o1c - a.off[p]) % a.d : dummy;
      T v1[cw], v2[cw];
#pragma unroll
      for (int e = 0; e < cw; ++e) {
        v1[e] = src[e];
        v2[e] = src[half + e];
      }
#pragma unroll
      for (int e = 0; e < cw; ++e) {
        w1v[gi][e] = use ? to_f<T>(v1[e]) : 1.f;
        w2v[gi][e] = use ? to_f<T>(v2[e]) : 1.f;
      }
    }
  }
  const float inv_d = 1.0f / (float)a.d;
  const int nhqk = a.nh[0] + a.nh[1];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) {
    asm volatile("" ::: "memory");   // keep later blocks' table loads from being hoisted (registers)
    float cc[4][NG][cw], ss[4][NG][cw];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rl = acc_row(qe, mb, j);            // tile row: slab row
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        const int o1 = n0 + qe.wn * 128 + perm_col(LG, qe.r16, 2 * cw * gi);
        // Every lane reads (clamped to a valid entry); the values are used
        // only for rows < N, columns < O of q and k, as below.
        const int o1c = min(o1, O - 1);
        const int jj = min((o1c - a.off[proj_of(o1c)]) % a.d, half - cw);
        load_cw(cs + rl * half + jj, cc[j][gi]);
        load_cw(sn + rl * half + jj, ss[j][gi]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long row = m0 + acc_row(qe, mb, j);
      if (row >= a.N) continue;
      const int s = (int)(row % a.S);
      const long bidx = row / a.S;
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        const int b1 = 2 * cw * gi;                  // first block of the pair group
        const int o1 = n0 + qe.wn * 128 + perm_col(LG, qe.r16, b1);
        if (o1 >= O) continue;
        const int p = proj_of(o1);
        const int oo = o1 - a.off[p];
        const int hd = oo / a.d, jj = oo % a.d;      // jj < d/2, jj .. jj+cw-1 consecutive
        float x1[cw], x2[cw];
#pragma unroll
        for (int e = 0; e < cw; ++e) {
          x1[e] = acc[mb][b1 + e][j] + b1v[gi][e];
          x2[e] = acc[mb][b1 + cw + e][j] + b2v[gi][e];
        }
        if (a.norm && p < 2) {
          // Per-head RMSNorm: the head's d columns of this row sit in the 16
          // lanes that share the row (cw pairs per lane), so the sum of
          // squares is one 16-lane reduction.  The whole group takes this
          // branch together: row, projection and head are the same for all.
          float sq = 0.f;
#pragma unroll
          for (int e = 0; e < cw; ++e) sq += x1[e] * x1[e] + x2[e] * x2[e];
          sq = lane_group_sum<16>(sq);
          const float ri = rsqrtf(sq * inv_d + a.eps);
          T* pn = static_cast<T*>(a.Pn) + row * (long)a.off[2] + o1;
          gstore<T, cw>(pn, x1, cw, a.vecN);
          gstore<T, cw>(pn + half, x2, cw, a.vecN);
          if (qe.r16 == 0) a.rinv[row * nhqk + (p == 0 ? 0 : a.nh[0]) + hd] = ri;
#pragma unroll
          for (int e = 0; e < cw; ++e) {
            x1[e] *= ri * w1v[gi][e];
            x2[e] *= ri * w2v[gi][e];
          }
        }
        float y1[cw], y2[cw];
#pragma unroll
        for (int e = 0; e < cw; ++e) {
          if (p < 2) {
            y1[e] = x1[e] * cc[j][gi][e] - x2[e] * ss[j][gi][e];
            y2[e] = x2[e] * cc[j][gi][e] + x1[e] * ss[j][gi][e];
          } else {
            y1[e] = x1[e];
            y2[e] = x2[e];
          }
        }
        T* dst = static_cast<T*>(a.out[p]) + ((bidx * a.nh[p] + hd) * a.S + s) * (long)a.d + jj;
        gstore<T, cw>(dst, y1, cw, a.vecO);
        gstore<T, cw>(dst + half, y2, cw, a.vecO);
      }
    }
  }
}

template <class T, int LG, bool FAST, int NS>
__global__ __launch_bounds__(kGemmThreads, 1) void k_qkv_fwd(QKVFwdArgs a) {
  __shared__ __align__(16) char smem[kGemmLds];
  const WaveId q = wave_id();
  int rb, cb;
  tile_coords(a.R * a.NC, a.R, a.NC, 8, rb, cb);
  const long m0 = (long)rb * kBM;
  const int n0 = cb * kBN;
  const int O = a.off[3];
  const T* X = static_cast<const T*>(a.X);

  // Projections overlapping this tile -> fold / side slots.  The projections
  // are contiguous column ranges, so the tile overlaps a contiguous run of
  // them: slot sl holds projection pfirst + sl, sl < nslot (plain arithmetic,
  // no runtime-indexed array, which would live in scratch memory).
  const int hi = min(n0 + kBN, O);
  const int ov0 = (a.off[0] < hi && a.off[1] > n0) ? 1 : 0;
  const int ov1 = (a.off[1] < hi && a.off[2] > n0) ? 1 : 0;
  const int ov2 = (a.off[2] < hi && a.off[3] > n0) ? 1 : 0;
  const int nslot = ov0 + ov1 + ov2;
  const int pfirst = ov0 ? 0 : (ov1 ? 1 : 2);
  auto proj_of = [&](int o) { return (o < a.off[1]) ? 0 : ((o < a.off[2]) ? 1 : 2); };
  auto slot_of = [&](int p) { return p - pfirst; };

  auto brow_of = [&](int R) -> const T* {
    const int o = n0 + lds_row_col(LG, R);
    if (o >= O) return nullptr;
    const int p = proj_of(o);
    return static_cast<const T*>(a.W[p]) + (long)(o - a.off[p]) * a.h;
  };
  auto side_base = [&](int sl) -> const T* {        // side block sl: adapter of projection pfirst + sl
    if (sl >= nslot) return nullptr;
    const int pj = pfirst + sl;
    return static_cast<const T*>(pj == 0 ? a.A[0] : (pj == 1 ? a.A[1] : a.A[2]));
  };
  const T* afall = static_cast<const T*>(pfirst == 0 ? a.A[0] : (pfirst == 1 ? a.A[1] : a.A[2]));

  f32x4 acc[kMB][8];
  f32x4 sacc[NS][kMB];
  zero_acc(acc);
  zero_side(sacc);
  if constexpr (FAST && LG == 1) {
    // head_dim 128: the per-lane row pointers fit in registers through the loop.
    NKPairLoader<NS> ld;
    ld.init_a(X, a.h, a.N, m0);
    ld.bfallback = static_cast<const T*>(a.W[0]);
    ld.smask = (1u << nslot) - 1u;
#pragma unroll
    for (int it = 0; it < 4; ++it) ld.brow[it] = brow_of(ld.row_of(it));
    ld.srow = afall;
    const int sr = ld.side_row();              // side row: slot sr/16, rank sr%16
    if (sr >= 0) ld.srow = ld.side_ptr(side_base(sr >> 4), sr & 15, a.r, a.h, afall);
    kloop2<NS>(smem, a.h / 64, ld, acc, sacc);
  } else if constexpr (FAST) {
    // head_dim 64: the row pointers are derived inside the loop.
    QKVRowLoader<NS, LG> ld;
    ld.X = X;
    ld.W0 = static_cast<const T*>(a.W[0]);
    ld.W1 = static_cast<const T*>(a.W[1]);
    ld.W2 = static_cast<const T*>(a.W[2]);
    ld.S0 = side_base(0);
    ld.S1 = side_base(1);
    ld.S2 = side_base(2);
    ld.afall = afall;
    ld.N = a.N; ld.m0 = m0; ld.h = a.h; ld.n0 = n0; ld.r = a.r;
    ld.off1 = a.off[1]; ld.off2 = a.off[2]; ld.off3 = a.off[3];
    ld.smask = (1u << nslot) - 1u;
    kloop2<NS>(smem, a.h / 64, ld, acc, sacc);
  } else {
    NKLoader<T, RowsA<T>, NS> ld;
    ld.a.init(X, nullptr, a.h, 0, a.h, a.N, m0, a.vecA);
    ld.bfallback = static_cast<const T*>(a.W[0]);
    ld.K = a.h;
    ld.vecB = a.vecW;
    ld.vecS = a.vecS;
    ld.smask = (1u << nslot) - 1u;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) ld.brow[qq] = brow_of(ld.row_of(qq));
    ld.srow = nullptr;
    const int sr = ld.side_row();
    if (sr >= 0) ld.srow = decltype(ld)::side_ptr(side_base(sr >> 4), sr & 15, a.r, a.h, afall);
    kloop<T, NS>(smem, (a.h + ET<T>::BK - 1) / ET<T>::BK, ld, acc, sacc);
  }
  side_reduce<T, NS>(smem, sacc);
  // A fresh (opaque) wave id for everything after the K-loop: the one above
  // dies with the loader set-up instead of staying live through the loop.
  const WaveId qe = wave_id();

  // T_p is saved by the tile holding projection p's first column.
  if (qe.tid < kBM) {
    const float* Ts = ts_ptr(smem);
    const long row = m0 + qe.tid;
    for (int sl = 0; sl < nslot; ++sl) {
      const int p = pfirst + sl;
      if (a.off[p] >= n0 && a.off[p] < n0 + kBN && row < a.N)
        for (int t = 0; t < a.r; ++t) a.T[p][row * a.r + t] = Ts[ts_idx(sl, qe.tid, t)];
    }
  }

  auto fb = [&](int R, int slot, int t0, float* v) {
    const int o = n0 + lds_row_col(LG, R);
    if (o >= O) return;
    const int p = proj_of(o);
    if (slot_of(p) != slot) return;
    const T* src = static_cast<const T*>(a.B[p]) + (long)(o - a.off[p]) * a.r;
    load_rank<T, ET<T>::VEC>(src, 1, t0, a.r, v);
  };
  float fs[kMaxSide];
#pragma unroll
  for (int sl = 0; sl < kMaxSide; ++sl) {
    const int p = min(pfirst + sl, 2);
    fs[sl] = (p == 0) ? a.s[0] : ((p == 1) ? a.s[1] : a.s[2]);
  }
  fold<T>(smem, acc, nslot, fs, fb);                // (ends with a barrier: LDS free)

  stage_rope_slab(smem, a.cs, a.sn, m0, a.N, a.S, a.d >> 1);
  qkv_rope_store<T, LG>(a, acc, m0, n0, qe, smem);
}

// B rows of a head_dim-128 QKV tile inside one projection p for
// nk_kloop_pp (columns in perm_col(1, ..) order): block wl + 4 it holds tile
// column 128 (it / 4) + 64 ((it / 2) % 2) + 2 (it % 2) + 4 (x % 16) + x / 16
// with x = 8 wl + L / 8: one lane offset.
struct QkvPP {
  const bf16* W0; long h;
  int off[2];
  __device__ __forceinline__ QkvPP(const bf16* Wp, long hd, long c0, int wl, int L) {
    W0 = Wp + c0 * hd;
    h = hd;
    const int x = 8 * wl + (L >> 3);
    off[0] = off[1] = (4 * (x & 15) + (x >> 4)) * (int)hd + direct2_chunk(L) * 8;
  }
  __device__ __forceinline__ const bf16* base(int it) const {
    return W0 + (128 * (it >> 2) + 64 * ((it >> 1) & 1) + 2 * (it & 1)) * h;
  }
  __device__ __forceinline__ static int sel(int) { return 0; }
};

// head_dim 128, bf16 fast path, as runs of column tiles (k_gateup_run's
// layout and LDS), for calls whose every run overlaps at most two
// projections: the run's first tile computes T_p of those projections in its
// K-loop and builds the fold operand (s_p T_p, bf16); later tiles inside one
// projection take the ping-pong K-loop, others the plain loop, neither with
// side work.  T_p is saved by the run holding projection p's first column.
template <class T>
__global__ __launch_bounds__(kGemmThreads, 1) void k_qkv_run(QKVFwdArgs a) {
  static_assert(sizeof(T) == 2, "the run kernel is bf16");
  constexpr int LG = 1;
  __shared__ __align__(16) char smem[kRunLds];
  int rb, cb0, cb1;
  run_coords(a.nruns, a.RPB, a.L, a.NC, rb, cb0, cb1);
  const long m0 = (long)rb * kBM;
  const int O = a.off[3];
  const bf16* X = static_cast<const bf16*>(a.X);
  char* FA = smem + kRunFAOff;
  const int nkt = a.h / 64;
  auto proj_of = [&](int o) { return (o < a.off[1]) ? 0 : ((o < a.off[2]) ? 1 : 2); };
  auto wp = [&](int p) { return static_cast<const bf16*>(p == 0 ? a.W[0] : (p == 1 ? a.W[1] : a.W[2])); };
  // Projections overlapping the run's columns: slots 0 .. rns - 1 hold
  // projection rpf + slot.
  const int lo = cb0 * kBN, hi = min(cb1 * kBN, O);
  const int ov0 = (a.off[0] < hi && a.off[1] > lo) ? 1 : 0;
  const int ov1 = (a.off[1] < hi && a.off[2] > lo) ? 1 : 0;
  const int ov2 = (a.off[2] < hi && a.off[3] > lo) ? 1 : 0;
  const int rns = ov0 + ov1 + ov2;
  const int rpf = ov0 ? 0 : (ov1 ? 1 : 2);

  // The kloop2 loader of the tile at n0 (side rows when smask != 0).
  auto make_ld = [&](int n0, unsigned smask) {
    NKPairLoader<2> ld;
    ld.init_a(X, a.h, a.N, m0);
    ld.bfallback = wp(0);
    ld.smask = smask;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int o = n0 + lds_row_col(LG, ld.row_of(it));
      const int p = proj_of(min(o, O - 1));
      ld.brow[it] = (o < O) ? wp(p) + (long)(o - a.off[p]) * a.h : nullptr;
    }
    const bf16* afall = static_cast<const bf16*>(rpf == 0 ? a.A[0] : (rpf == 1 ? a.A[1] : a.A[2]));
    ld.srow = afall;
    const int sr = ld.side_row();              // side row: slot sr / 16, rank sr % 16
    if (sr >= 0) {
      const int sl = sr >> 4, pj = rpf + sl;
      const bf16* base = (sl < rns) ? static_cast<const bf16*>(pj == 0 ? a.A[0] : (pj == 1 ? a.A[1] : a.A[2]))
                                    : nullptr;
      ld.srow = ld.side_ptr(base, sr & 15, a.r, a.h, afall);
    }
    return ld;
  };

  // Fold with the run's operand, then RoPE, split and stores.
  auto finish = [&](int n0, f32x4 (&acc)[kMB][8]) {
    const WaveId qe = wave_id_opaque();
    auto fb = [&](int R, int slot, int t0, float* v) {
      const int o = n0 + lds_row_col(LG, R);
      if (o >= O) return;
      const int p = proj_of(o);
      if (p - rpf != slot) return;
      const bf16* src = static_cast<const bf16*>(p == 0 ? a.B[0] : (p == 1 ? a.B[1] : a.B[2])) +
                        (long)(o - a.off[p]) * a.r;
      load_rank<bf16, 8>(src, 1, t0, a.r, v);
    };
    fold_run(FA, smem + kRunFBOff, acc, fb);
    // The slab covers the stages, the side products and the fold B tile
    // (not the run's fold A operand): after every wave's fold reads, and
    // read by all before the next tile's loads refill stage 0.
    __syncthreads();
    stage_rope_slab(smem, a.cs, a.sn, m0, a.N, a.S, a.d >> 1);
    qkv_rope_store<bf16, LG>(a, acc, m0, n0, qe, smem);
    __syncthreads();
  };

  {
    // First tile: the run's T_p ride the K-loop.
    const int n0 = cb0 * kBN;
    f32x4 acc[kMB][8];
    f32x4 sacc[2][kMB];
    zero_acc(acc);
    zero_side(sacc);
    {
      const NKPairLoader<2> ld = make_ld(n0, (1u << rns) - 1u);
      kloop2<2>(smem, nkt, ld, acc, sacc, 0, false);
    }
    const WaveId q = wave_id_opaque();
    side_reduce<bf16, 2>(smem + kRunTsOff, sacc);
    const float* Ts = ts_ptr(smem + kRunTsOff);
    if (q.tid < kBM) {
      const long row = m0 + q.tid;
      for (int sl = 0; sl < rns; ++sl) {
        const int p = rpf + sl;
        if (a.off[p] >= lo && a.off[p] < hi && row < a.N)
          for (int t = 0; t < a.r; ++t) a.T[p][row * a.r + t] = Ts[ts_idx(sl, q.tid, t)];
      }
    }
    const float fs[kMaxSide] = {rpf == 0 ? a.s[0] : (rpf == 1 ? a.s[1] : a.s[2]),
                                rpf == 0 ? a.s[1] : a.s[2], 0.f};
    build_fold_a(FA, Ts, rns, fs);
    finish(n0, acc);
  }
  for (int cb = cb0 + 1; cb < cb1; ++cb) {
    const int n0 = cb * kBN;
    f32x4 acc[kMB][8];
    zero_acc(acc);
    const int p = proj_of(n0);
    if (n0 + kBN <= a.off[p + 1]) {
      const WaveId qo = wave_id_opaque();
      const QkvPP bp(wp(p), a.h, n0 - a.off[p], __builtin_amdgcn_readfirstlane(qo.w) & 3, qo.lane);
      nk_kloop_pp(smem, nkt, X, a.h, a.N, m0, bp, acc);
    } else {
      const NKPairLoader<2> ld = make_ld(n0, 0u);
      f32x4 snone[1][kMB];
      kloop2<0>(smem, nkt, ld, acc, snone, 0, false);
    }
    finish(n0, acc);
  }
}

}  // namespace lora

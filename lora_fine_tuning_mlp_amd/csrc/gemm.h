// The LoRA-augmented MFMA GEMM core: a 256x256 output tile per workgroup of
// eight waves (two per SIMD), laid out 4 x 2: wave (wm, wn) owns rows
// 64 wm .. 64 wm + 63 and columns 128 wn .. 128 wn + 127, i.e. 4 x 8 MFMA
// blocks of 16 x 16.
//
//   acc  = Z_tile . Bop_tile                       (K-loop, bf16 or fp32 MFMA)
//   side = Z_tile . Sop                            (same K-loop, same A fragments:
//                                                   the rank-r product, <= 3 adapters)
//   acc += [s_1 T_1 | s_2 T_2 | ...] . [F_1 ; F_2 ; ...]   (the fold: extra K steps)
//
// The side product rides along the base GEMM's K-loop: its operand sits in
// LDS right after the B tile and reuses the A fragments already in
// registers, so X (or H, or dG|dU) is read once for both.  The two waves that
// share a row range take alternate K sub-steps (or tiles) of the side work;
// their halves are summed through LDS after the loop.
//
// K-loops.  Fast path (bf16, 16-byte aligned rows, K % 64 == 0): two LDS
// stages of K tiles of 64 in 128-byte rows, every operand loaded straight
// from global memory into LDS (no staging registers); tile kt + 1 is issued
// at the top of iteration kt and has landed by its end (kloop2 for weights
// stored [N][K], kloop2tr for [K][N]).  Staged path (fp32, unaligned or
// ragged shapes): register-staged, masked loads one K tile (32 bf16 / 16
// fp32, 64-byte rows) ahead (kloop).
//
// B operands: weights stored [N][K] (forward) are rows of the tile like A;
// weights stored [K][N] (backward, bf16) keep that layout in LDS and are read
// as MFMA fragments with ds_read_b64_tr_b16, which leaves the accumulators in
// natural column order; the epilogue turns them through LDS ("park") where it
// needs 8 consecutive columns per lane.  fp32 [K][N] tiles are transposed
// while register-staged.
//
// LDS after the K-loop: Ts (float side products, [3][256][16]), the fold A
// tile and the fold B tile; epilogues reuse the fold area for reductions.
#pragma once

#include "common.h"

#include <type_traits>
#include <utility>

namespace lora {

constexpr int kGemmThreads = 512;                          // 8 waves
constexpr int kMB = 4;                                     // MFMA row blocks per wave
constexpr int kARows = kBM;
constexpr int kBRows = kBN + kSlot * kMaxSide;
constexpr int kABytes = kARows * kRowBytes;                // 16384
constexpr int kBBytes = kBRows * kRowBytes;                // 19456
constexpr int kSideOff = kBN * kRowBytes;                  // side operand inside the B region
constexpr int kStage = kABytes + kBBytes;                  // 35840
// LDS of a GEMM workgroup: two fast-path stages of 71680 bytes (the staged
// loop uses two stages of kStage).
constexpr int kGemmLds = 143360;
static_assert(2 * kStage <= kGemmLds, "two staged-loop stages");

constexpr int kTsOff = 0;
constexpr int kTsBytes = kMaxSide * kBM * kSlot * 4;       // 49152
constexpr int kFAOff = kTsBytes;
constexpr int kFBOff = kFAOff + kBM * kRowBytes;
constexpr int kRedOff = kFAOff;                            // epilogue scratch (fold tiles are dead)
constexpr int kRedBytes = 65536;
static_assert(kRedOff + kRedBytes <= kGemmLds, "reduction scratch overflows");
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
// The same from an opaque copy of the thread id: nothing derived from it can
// be hoisted above a K-loop (where every register is taken) by a compiler
// that sees the same values are needed after it.
__device__ __forceinline__ WaveId wave_id_opaque() {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  WaveId q;
  q.tid = tid;
  q.lane = tid & 63;
  q.w = tid >> 6;
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
// wave writes 16 bytes at LDS base + 16 l, i.e. one 1 KB block per
// instruction.  Lanes switched off by the exec mask write nothing.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void g2lds16(const void* g, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}
// 1 KB block `it` of this wave (wave w fills blocks w + 8 it).
__device__ __forceinline__ int direct_blk(int it) { return (int)(threadIdx.x >> 6) + 8 * it; }

// ---------------------------------------------------------------------------
// [K][N] bf16 B tiles in their natural layout (32 rows k x 256 columns, 512
// bytes a row), read as MFMA B fragments with ds_read_b64_tr_b16.  Within
// each 16-lane group that instruction hands lane i the 4 elements
// M[4j + i/4][i % 4] (j = 0..3), M[s] being the 8 bytes lane s addressed.  So
// lane s addresses row kb + s/4, columns nb0 + 4 (s % 4) .. +3, and lane i
// receives column nb0 + i at rows kb .. kb+3; two reads give the 8 K slots.
// 16-byte segments are XOR-swizzled per row (kn_off) so the 8 rows one read
// touches hit distinct bank groups.
// ---------------------------------------------------------------------------
//
// The transpose reads are issued as inline asm: the compiler's wait-count
// pass treats the ds_read_tr intrinsic as possibly aliasing the direct loads
// still in flight and would wait for all of them, which empties the
// pipeline.  Their results become valid through lgkm_tie(), an explicit
// lgkmcnt wait that names the destination registers (LDS operations of a
// wave complete in order, so "at most N outstanding" means everything but
// the last N issued has landed; the compiler's own lgkmcnt waits only get
// more conservative from the extra operations).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int ftr(int k) { return ((k & 3) | (((k >> 3) & 1) << 2)) << 1; }
__device__ __forceinline__ int kn_off(int k, int col) {   // byte offset of (k, col) in the tile
  return k * 512 + ((((col >> 3) ^ ftr(k))) << 4) + ((col & 7) << 1);
}
__device__ __forceinline__ unsigned lds_addr(const char* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
__device__ __forceinline__ u32x2 tr16(unsigned addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}
// LDS writes as inline asm, for code that must not let the compiler see an
// LDS access while direct loads are in flight (it would wait for all of them).
__device__ __forceinline__ void ds_w16_lo(unsigned addr, unsigned v) {
  asm volatile("ds_write_b16 %0, %1" : : "v"(addr), "v"(v));
}
__device__ __forceinline__ void ds_w16_hi(unsigned addr, unsigned v) {
  asm volatile("ds_write_b16_d16_hi %0, %1" : : "v"(addr), "v"(v));
}
__device__ __forceinline__ void ds_w128(unsigned addr, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(v));
}
// The same with an immediate byte offset (the DS offset field), so unrolled
// code addresses many locations from one base register.
template <int OFF>
__device__ __forceinline__ void ds_w16_lo_at(unsigned base, unsigned v) {
  asm volatile("ds_write_b16 %0, %1 offset:%2" : : "v"(base), "v"(v), "n"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_w16_hi_at(unsigned base, unsigned v) {
  asm volatile("ds_write_b16_d16_hi %0, %1 offset:%2" : : "v"(base), "v"(v), "n"(OFF));
}
template <int OFF>
__device__ __forceinline__ u32x2 tr16_at(unsigned base) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(base), "n"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x4 rd128_at(unsigned base) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(base), "n"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ void ds_w128_at(unsigned base, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1 offset:%2" : : "v"(base), "v"(v), "n"(OFF));
}
// Compile-time loop: f(std::integral_constant<int, 0>{}) ... f(<N - 1>), so
// the body can form immediate offsets from the index.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
// At most N of this wave's vector memory operations outstanding (they
// complete in issue order).
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void lgkm_tie(u32x2& a, u32x2& b, u32x2& c, u32x2& d, u32x2& e, u32x2& f, u32x2& g,
                                         u32x2& h) {
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e), "+v"(f), "+v"(g), "+v"(h)
               : "n"(N));
}
// (a and b must be distinct: the same variable named twice would be copied
// into a second register before the wait.)
__device__ __forceinline__ void lgkm_tie0(u32x2& a, u32x2& b) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void lgkm_tie0(u32x2& a) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a));
}
// The two reads of B fragment nb (K slots 0..3 and 4..7 of the lane).
__device__ __forceinline__ void tr_issue(const char* Bs, int nb, const WaveId& q, u32x2& lo, u32x2& hi) {
  const int s = q.r16;
  const int col = q.wn * 128 + nb * 16 + 4 * (s & 3);
  const int k1 = 8 * q.g + (s >> 2);
  lo = tr16(lds_addr(Bs + kn_off(k1, col)));
  hi = tr16(lds_addr(Bs + kn_off(k1 + 4, col)));
}
// Side operand stored [K][r] (r = 16): a [32 k][16 t] tile of 32-byte rows.
__device__ __forceinline__ void tr_side_issue(const char* S, const WaveId& q, u32x2& lo, u32x2& hi) {
  const int s = q.r16;
  const int off = (8 * q.g + (s >> 2)) * 32 + 8 * (s & 3);
  lo = tr16(lds_addr(S + off));
  hi = tr16(lds_addr(S + off + 128));
}
__device__ __forceinline__ Frag<bf16> tr_make(u32x2 lo, u32x2 hi) {
  Frag<bf16> f;
  f.v = (u32x4){lo.x, lo.y, hi.x, hi.y};
  return f;
}

// Fragment reads issued as inline asm like the transpose reads: the compiler
// then tracks no LDS read of the K-loop itself and cannot fall back to
// lgkmcnt(0) before the first MFMA; each fragment is made valid by an
// explicit wait that names it (at most N of this wave's LDS reads still
// outstanding; they complete in issue order).
__device__ __forceinline__ u32x4 rd128(const char* p) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(lds_addr(p)));
  return r;
}
template <int N>
__device__ __forceinline__ void tie(u32x4& a) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(N));
}
template <int N>
__device__ __forceinline__ void tie(u32x2& a, u32x2& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}

// ---------------------------------------------------------------------------
// End of a K iteration: wait for this wave's direct loads and LDS traffic,
// then barrier.  Written as one asm statement so the compiler neither adds
// the fence of __syncthreads() nor moves memory accesses across it.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void sync_stage() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------
// Staged K-loop (fp32, unaligned or ragged shapes).  Loader interface:
//   kBTr                     B (and side) fragments by transpose reads
//   load(kt)                 register-staged global loads for K tile kt
//   store(As, Bs)            registers -> LDS stage
//   side_mask(kt)            bit sb set when side block sb has data in tile kt
// K tiles kt0 .. nkt-1; the loads of tile kt + 1 are in flight while tile kt
// is computed.
// ---------------------------------------------------------------------------
template <class T, int NSIDE, class Loader>
__device__ __forceinline__ void kloop(char* smem, int nkt, Loader& ld, f32x4 (&acc)[kMB][8],
                                      f32x4 (&sacc)[NSIDE > 0 ? NSIDE : 1][kMB], int kt0 = 0) {
  const WaveId q = wave_id();
  if (nkt <= kt0) return;
  auto stage = [&](int kt) { return smem + ((kt - kt0) & 1) * kStage; };
  ld.load(kt0);
  ld.store(stage(kt0), stage(kt0) + kABytes);
  sync_stage();
  for (int kt = kt0; kt < nkt; ++kt) {
    const char* As = stage(kt);
    const char* Bs = As + kABytes;
    const bool more = kt + 1 < nkt;
    char* Sn = stage(kt + 1);
    if (more) ld.load(kt + 1);
    Frag<T> af[kMB];
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) af[mb] = lds_frag<T>(As, q.wm * 64 + mb * 16 + q.r16, q.g);
    if constexpr (Loader::kBTr) {
      u32x2 lo[8], hi[8];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) tr_issue(Bs, nb, q, lo[nb], hi[nb]);
      lgkm_tie<8>(lo[0], hi[0], lo[1], hi[1], lo[2], hi[2], lo[3], hi[3]);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const Frag<T> bfr = tr_make(lo[nb], hi[nb]);
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) acc[mb][nb] = mma(acc[mb][nb], af[mb], bfr);
      }
      lgkm_tie<0>(lo[4], hi[4], lo[5], hi[5], lo[6], hi[6], lo[7], hi[7]);
#pragma unroll
      for (int nb = 4; nb < 8; ++nb) {
        const Frag<T> bfr = tr_make(lo[nb], hi[nb]);
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) acc[mb][nb] = mma(acc[mb][nb], af[mb], bfr);
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const Frag<T> bfr = lds_frag<T>(Bs, q.wn * 128 + nb * 16 + q.r16, q.g);
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) acc[mb][nb] = mma(acc[mb][nb], af[mb], bfr);
      }
    }
    if constexpr (NSIDE > 0) {
      if ((kt & 1) == q.wn) {
        const unsigned smask = ld.side_mask(kt);
#pragma unroll
        for (int sb = 0; sb < NSIDE; ++sb) {
          if ((smask >> sb) & 1u) {
            Frag<T> bfr;
            if constexpr (Loader::kBTr) {
              u32x2 lo, hi;
              tr_side_issue(Bs + kSideOff + sb * 1024, q, lo, hi);
              lgkm_tie0(lo, hi);
              bfr = tr_make(lo, hi);
            } else {
              bfr = lds_frag<T>(Bs, kBN + sb * 16 + q.r16, q.g);
            }
#pragma unroll
            for (int mb = 0; mb < kMB; ++mb) sacc[sb][mb] = mma(sacc[sb][mb], af[mb], bfr);
          }
        }
      }
    }
    if (more) ld.store(Sn, Sn + kABytes);
    sync_stage();
  }
}

// ---------------------------------------------------------------------------
// Forward fast path (bf16, weights stored [N][K]): K tiles of 64 in
// 128-byte LDS rows (eight chunks swizzled with row & 7), two stages.  With
// K-contiguous operands every direct load then requests whole 128-byte cache
// lines; 64-byte rows would split each line over two tiles and double the
// L1 -> L2 requests.  The price is one tile of loads in flight instead of
// three, which these kernels, with both operands K-contiguous, can afford.
// ---------------------------------------------------------------------------
constexpr int kRow2 = 128;
constexpr int kStage2A = kBM * kRow2;                                 // 32768
constexpr int kStage2 = (kBM + kBN + kSlot * kMaxSide) * kRow2;      // 71680
static_assert(2 * kStage2 == kGemmLds, "two 128-byte-row stages");
__device__ __forceinline__ int lds_off2(int row, int chunk) { return row * kRow2 + ((chunk ^ (row & 7)) << 4); }
__device__ __forceinline__ Frag<bf16> lds_frag2(const char* buf, int row, int ks, int g) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const u32x4*>(buf + lds_off2(row, ks * 4 + g));
  return f;
}
// A 1 KB direct block is 8 rows of 128 bytes: lane l writes physical chunk
// l & 7 of row 8 blk + (l >> 3), so it fetches logical chunk (l & 7) ^ (l >> 3).
__device__ __forceinline__ int direct2_chunk(int lane) { return (lane & 7) ^ (lane >> 3); }
__device__ __forceinline__ int direct2_row(int it) { return 8 * direct_blk(it) + (int)((threadIdx.x & 63) >> 3); }

// All operands direct: A rows (tokens), B rows (output columns, resolved by
// the kernel for rows row_of(it), it = 0..3; nullptr -> bfallback) and side
// rows (lanes 0 .. 16 NSIDE - 1 of each wave; ranks past r clamped as in
// NKLoader).  Requires K % 64 == 0, 16-byte aligned rows, 32-bit A offsets.
template <int NSIDE>
struct NKPairLoader {
  const bf16* A;
  int aoff[4];
  const bf16* brow[4];
  const bf16* bfallback;
  const bf16* srow;
  unsigned smask;
  __device__ static __forceinline__ int row_of(int it) { return direct2_row(it); }
  __device__ static __forceinline__ int side_row() {
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    return (l < 16 * NSIDE) ? (w * 16 * NSIDE + l) >> 3 : -1;
  }
  __device__ static __forceinline__ const bf16* side_ptr(const bf16* base, int t, int r, long Kd,
                                                         const bf16* fallback) {
    return base ? base + (long)min(t, r - 1) * Kd : fallback;
  }
  __device__ __forceinline__ void init_a(const bf16* A0, long lda, long M, long m0) {
    A = A0;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      long row = m0 + direct2_row(it);
      if (row > M - 1) row = M - 1;
      aoff[it] = (int)(row * lda);
    }
  }
  __device__ __forceinline__ void issue(int kt, char* As, char* Bs) const {
    const int L = threadIdx.x & 63;
    const long k = (long)kt * 64 + direct2_chunk(L) * 8;
#pragma unroll
    for (int it = 0; it < 4; ++it) g2lds16(A + aoff[it] + k, As + direct_blk(it) * 1024);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const bf16* p = brow[it] ? brow[it] : bfallback;
      g2lds16(p + k, Bs + direct_blk(it) * 1024);
    }
    if constexpr (NSIDE > 0) {
      if (L < 16 * NSIDE && smask != 0u) {
        const int w = threadIdx.x >> 6;
        const int ci = w * 16 * NSIDE + L, sr = ci >> 3;
        const int chunk = (ci & 7) ^ (sr & 7);
        g2lds16(srow + (long)kt * 64 + chunk * 8, Bs + kBN * kRow2 + w * 256 * NSIDE);
      }
    }
  }
};

// prefetched: the caller already issued tile kt0 into stage 0 (a workgroup
// walking several output tiles issues the next tile's first K tile before its
// fold and epilogue); the loop then only waits for it.
template <int NSIDE, class Loader>
__device__ __forceinline__ void kloop2(char* smem, int nkt, const Loader& ld, f32x4 (&acc)[kMB][8],
                                       f32x4 (&sacc)[NSIDE > 0 ? NSIDE : 1][kMB], int kt0 = 0,
                                       bool prefetched = false) {
  const WaveId q = wave_id();
  if (nkt <= kt0) return;
  auto stage = [&](int kt) { return smem + ((kt - kt0) & 1) * kStage2; };
  if (!prefetched) ld.issue(kt0, stage(kt0), stage(kt0) + kStage2A);
  sync_stage();
  for (int kt = kt0; kt < nkt; ++kt) {
    const char* As = stage(kt);
    const char* Bs = As + kStage2A;
    if (kt + 1 < nkt) {
      char* An = stage(kt + 1);
      ld.issue(kt + 1, An, An + kStage2A);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // Reads: side (this wave's turn), A 0..3, B 0..7; the waits count
      // from the end, so they do not depend on the side read.
      const bool side = NSIDE > 0 && ks == q.wn;
      u32x4 sv[NSIDE > 0 ? NSIDE : 1];
      if constexpr (NSIDE > 0) {
        if (side) {
#pragma unroll
          for (int sb = 0; sb < NSIDE; ++sb)
            if ((ld.smask >> sb) & 1u) sv[sb] = rd128(Bs + lds_off2(kBN + sb * 16 + q.r16, ks * 4 + q.g));
        }
      }
      u32x4 av[kMB], bv[8];
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) av[mb] = rd128(As + lds_off2(q.wm * 64 + mb * 16 + q.r16, ks * 4 + q.g));
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) bv[nb] = rd128(Bs + lds_off2(q.wn * 128 + nb * 16 + q.r16, ks * 4 + q.g));
      Frag<bf16> af[kMB];
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        tie<8>(av[mb]);
        af[mb].v = av[mb];
      }
#define LORA_FWD_NB(NB, N)                                                    \
      {                                                                       \
        tie<N>(bv[NB]);                                                       \
        Frag<bf16> bfr;                                                       \
        bfr.v = bv[NB];                                                       \
        _Pragma("unroll") for (int mb = 0; mb < kMB; ++mb) acc[mb][NB] = mma(acc[mb][NB], af[mb], bfr); \
        __builtin_amdgcn_sched_barrier(0);                                    \
      }
      LORA_FWD_NB(0, 7) LORA_FWD_NB(1, 6) LORA_FWD_NB(2, 5) LORA_FWD_NB(3, 4)
      LORA_FWD_NB(4, 3) LORA_FWD_NB(5, 2) LORA_FWD_NB(6, 1) LORA_FWD_NB(7, 0)
#undef LORA_FWD_NB
      if constexpr (NSIDE > 0) {
        if (side) {
#pragma unroll
          for (int sb = 0; sb < NSIDE; ++sb) {
            if ((ld.smask >> sb) & 1u) {
              tie<0>(sv[sb]);
              Frag<bf16> bfr;
              bfr.v = sv[sb];
#pragma unroll
              for (int mb = 0; mb < kMB; ++mb) sacc[sb][mb] = mma(sacc[sb][mb], af[mb], bfr);
            }
          }
        }
      }
    }
    sync_stage();
  }
}

// ---------------------------------------------------------------------------
// Backward fast path (bf16, weights stored [K][N]): K tiles of 64, two
// stages.  The A rows (tokens) take the forward's 128-byte layout, so every
// direct load requests whole cache lines; the [K][N] tile is 64 rows of 512
// bytes in the transpose-read layout (kn_off; its swizzle repeats every 16
// rows) and the optional side tile ([K][r], r = 16) is 64 rows of 32 bytes.
// ---------------------------------------------------------------------------
constexpr int kStage2TrB = 64 * 512;                                  // 32768
constexpr int kStage2TrS = 64 * 32;                                   // 2048
constexpr int kStage2Tr = kStage2A + kStage2TrB + kStage2TrS;         // 67584
static_assert(2 * kStage2Tr <= kGemmLds, "two transpose-read stages");

// A: rows of [A0 | A1] split along K at K0 (K0 % 64 == 0); B: krow(k) -> row k
// of the [K][N] matrix (row stride ldb), columns n0 .. n0+255 (clamped to the
// last chunk, never stored); side: srow(0, k) -> the 16 ranks of row k (row
// stride lds).  Every K tile full and inside one segment of krow / srow, N %
// 8 == 0, 16-byte aligned rows, 32-bit offsets.  Row pointers are resolved
// once per tile from the (uniform) tile start; each lane keeps only 32-bit
// offsets, so the loader's state stays small across the K-loop.
template <class KRow, class SRow, int NSIDE>
struct KNPairLoader {
  static_assert(NSIDE <= 1, "one direct side block");
  const bf16* A0;
  const bf16* A1;
  long K0;
  int aoff[4], boff[4], soff;
  KRow krow;
  SRow srow;
  __device__ __forceinline__ void init(const bf16* a0, const bf16* a1, long k0, long lda, long M, long m0, long ldb,
                                       long n0, long N, long lds) {
    const int L = threadIdx.x & 63, w = threadIdx.x >> 6;
    A0 = a0;
    A1 = a1 ? a1 : a0;
    K0 = a1 ? k0 : (1L << 40);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      long row = m0 + direct2_row(it);
      if (row > M - 1) row = M - 1;
      aoff[it] = (int)(row * lda) + direct2_chunk(L) * 8;
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {              // block = 2 k rows of 512 bytes
      const int row = 2 * direct_blk(it) + (L >> 5);
      const int lseg = (L & 31) ^ ftr(row);
      boff[it] = (int)(row * ldb + min(n0 + lseg * 8, N - 8));
    }
    const int ci = 16 * w + L;                    // side chunk (lanes < 16): row ci / 2
    soff = (int)((ci >> 1) * lds) + 8 * (ci & 1);
  }
  __device__ __forceinline__ void issue(int kt, char* As, char* Bs) const {
    const long k = (long)kt * 64;
    const bf16* ab = (k >= K0) ? A1 + (k - K0) : A0 + k;
#pragma unroll
    for (int it = 0; it < 4; ++it) g2lds16(ab + aoff[it], As + direct_blk(it) * 1024);
    const bf16* bb = krow(k);
#pragma unroll
    for (int it = 0; it < 4; ++it) g2lds16(bb + boff[it], Bs + direct_blk(it) * 1024);
    if constexpr (NSIDE > 0) {
      if ((threadIdx.x & 63) < 16) g2lds16(srow(0, k) + soff, Bs + kStage2TrB + 256 * (threadIdx.x >> 6));
    }
  }
};

// Tile kt + 1 is issued at the top of iteration kt and has landed by its end.
template <int NSIDE, class Loader>
__device__ __forceinline__ void kloop2tr(char* smem, int nkt, const Loader& ld, f32x4 (&acc)[kMB][8],
                                         f32x4 (&sacc)[NSIDE > 0 ? NSIDE : 1][kMB], int kt0 = 0) {
  const WaveId q = wave_id();
  if (nkt <= kt0) return;
  auto stage = [&](int kt) { return smem + ((kt - kt0) & 1) * kStage2Tr; };
  ld.issue(kt0, stage(kt0), stage(kt0) + kStage2A);
  sync_stage();
  for (int kt = kt0; kt < nkt; ++kt) {
    const char* As = stage(kt);
    const char* Bs = As + kStage2A;
    if (kt + 1 < nkt) {
      char* An = stage(kt + 1);
      ld.issue(kt + 1, An, An + kStage2A);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // Reads: side (this wave's turn), A 0..3, then the two transpose reads
      // of each B fragment; waits count from the end.
      const bool side = NSIDE > 0 && ks == q.wn;
      u32x2 slo, shi;
      if (side) tr_side_issue(Bs + kStage2TrB + ks * 1024, q, slo, shi);
      u32x4 av[kMB];
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) av[mb] = rd128(As + lds_off2(q.wm * 64 + mb * 16 + q.r16, ks * 4 + q.g));
      const char* Bk = Bs + ks * 32 * 512;
      u32x2 lo[8], hi[8];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) tr_issue(Bk, nb, q, lo[nb], hi[nb]);
      Frag<bf16> af[kMB];
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        // 16 transpose reads follow the A reads and the counter holds at most
        // 15 outstanding operations, so A has landed: this only ties the
        // registers (lgkmcnt is a 4-bit field).
        tie<15>(av[mb]);
        af[mb].v = av[mb];
      }
#define LORA_TR_NB(NB, N)                                                     \
      {                                                                       \
        tie<N>(lo[NB], hi[NB]);                                               \
        const Frag<bf16> bfr = tr_make(lo[NB], hi[NB]);                       \
        _Pragma("unroll") for (int mb = 0; mb < kMB; ++mb) acc[mb][NB] = mma(acc[mb][NB], af[mb], bfr); \
        __builtin_amdgcn_sched_barrier(0);                                    \
      }
      LORA_TR_NB(0, 14) LORA_TR_NB(1, 12) LORA_TR_NB(2, 10) LORA_TR_NB(3, 8)
      LORA_TR_NB(4, 6) LORA_TR_NB(5, 4) LORA_TR_NB(6, 2) LORA_TR_NB(7, 0)
#undef LORA_TR_NB
      if constexpr (NSIDE > 0) {
        if (side) {
          tie<0>(slo, shi);
          const Frag<bf16> bfr = tr_make(slo, shi);
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb) sacc[0][mb] = mma(sacc[0][mb], af[mb], bfr);
        }
      }
    }
    sync_stage();
  }
}



// Whole-tile ping-pong K-loop over [N][K] operands (the kloop2 layout)
// without side rows.  Wave groups 0-3 (rows 0-127) and 4-7 (rows 128-255)
// run one phase apart: in its read phase a group reads all 24 fragments of
// the K tile (and issues the global loads of the next one: each group its
// 128 A rows, group 0 all 256 B rows); in its MFMA phase it issues the
// tile's 64 MFMAs while the other group reads.  Barriers separate the
// phases; group 1 starts one barrier late and group 0 ends one barrier late,
// so every wave passes the same number.  B block wl + 4 it (it = 0..7, LDS
// rows 8 (wl + 4 it) + L / 8) comes from bp.base(it) + bp.off[bp.sel(it)]:
// a uniform pointer plus one of the lane's two offsets (whole B rows only).
template <class BP>
__device__ __forceinline__ void nk_kloop_pp(char* smem, int nkt, const bf16* X, long lda, long M, long m0,
                                            const BP& bp, f32x4 (&acc)[kMB][8]) {
  const WaveId q = wave_id_opaque();
  const int w = __builtin_amdgcn_readfirstlane(q.w);
  const int grp = w >> 2, wl = w & 3;
  const int L = q.lane;
  int aoff[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    long row = m0 + 8 * (grp * 16 + wl + 4 * it) + (L >> 3);
    if (row > M - 1) row = M - 1;
    aoff[it] = (int)(row * lda) + direct2_chunk(L) * 8;
  }
  // The lane offsets pass through an empty asm at each use, so no 64-bit
  // address is hoisted out of the loop (it would be spilled).
  auto issue = [&](int kt, char* S) {
    const int k = kt * 64;
    int ao[4] = {aoff[0], aoff[1], aoff[2], aoff[3]};
    asm volatile("" : "+v"(ao[0]), "+v"(ao[1]), "+v"(ao[2]), "+v"(ao[3]));
#pragma unroll
    for (int it = 0; it < 4; ++it) g2lds16(X + ao[it] + k, S + (grp * 16 + wl + 4 * it) * 1024);
    if (grp == 0) {
      int bo[2] = {bp.off[0], bp.off[1]};
      asm volatile("" : "+v"(bo[0]), "+v"(bo[1]));
#pragma unroll
      for (int it = 0; it < 8; ++it) g2lds16(bp.base(it) + bo[bp.sel(it)] + k, S + kStage2A + (wl + 4 * it) * 1024);
    }
  };
  auto bar = [] { asm volatile("s_barrier" ::: "memory"); };
  auto stage = [&](int kt) { return smem + (kt & 1) * kStage2; };
  if (nkt <= 0) return;
  issue(0, stage(0));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  bar();
  if (grp == 1) bar();
  __builtin_amdgcn_sched_barrier(0);
  for (int kt = 0; kt < nkt; ++kt) {
    const char* S = stage(kt);
    if (kt + 1 < nkt) issue(kt + 1, stage(kt + 1));
    u32x4 av[2][kMB], bv[2][8];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) av[ks][mb] = rd128(S + lds_off2(q.wm * 64 + mb * 16 + q.r16, ks * 4 + q.g));
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) bv[ks][nb] = rd128(S + kStage2A + lds_off2(q.wn * 128 + nb * 16 + q.r16, ks * 4 + q.g));
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) tie<0>(av[ks][mb]);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) tie<0>(bv[ks][nb]);
    }
    __builtin_amdgcn_sched_barrier(0);
    bar();
    __builtin_amdgcn_sched_barrier(0);
    // MFMA phase, A fragment outer: eight MFMAs in a row share their A
    // operand (measured a little faster under the power limit than sharing
    // the B operand four at a time; each accumulator's sum is unchanged).
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        Frag<bf16> af;
        af.v = av[ks][mb];
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          Frag<bf16> bfr;
          bfr.v = bv[ks][nb];
          acc[mb][nb] = mma(acc[mb][nb], af, bfr);
        }
      }
    if (kt + 1 < nkt) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    bar();
    __builtin_amdgcn_sched_barrier(0);
  }
  if (grp == 0) bar();
}

// Whole-tile ping-pong form of kloop2tr without side block.  Wave groups
// 0-3 (rows 0-127) and 4-7 (rows 128-255) run one phase apart: in its read
// phase a group reads every fragment of the K tile it needs (8 A reads, 32
// transpose reads) and issues the next tile's loads (each group its own 128
// A rows, group 0 the whole B tile); in its MFMA phase it issues the tile's
// 64 MFMAs while the other group reads.  Barriers separate the phases; group
// 1 starts one barrier late and group 0 ends one barrier late, so every wave
// passes the same number.  Operands and stages as kloop2tr (A split along K
// at K0, krow(k) the B row of K row k, every K tile inside one segment).
template <class KRow>
__device__ __forceinline__ void kloop2tr_pp(char* smem, int nkt, const bf16* A0, const bf16* A1, long K0,
                                            const KRow& krow, long lda, long M, long m0, long ldb, long n0,
                                            long N, f32x4 (&acc)[kMB][8]) {
  // Lane values from an opaque thread id: nothing is shared with (or kept
  // live from) code around the loop, e.g. the tiles of a run.
  const WaveId q = wave_id_opaque();
  const int w = __builtin_amdgcn_readfirstlane(q.w);
  const int grp = w >> 2, wl = w & 3;
  const int L = q.lane;
  if (A1 == nullptr) { A1 = A0; K0 = 1L << 40; }
  int aoff[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    long row = m0 + 8 * (grp * 16 + wl + 4 * it) + (L >> 3);
    if (row > M - 1) row = M - 1;
    aoff[it] = (int)(row * lda) + direct2_chunk(L) * 8;
  }
  // B block wl + 4 it holds K rows 8 it + r0 (r0 = 2 wl + L / 32); its
  // swizzle depends on it only through it & 1, so a lane keeps two offsets.
  const int r0 = 2 * wl + (L >> 5);
  int boff[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int lseg = (L & 31) ^ ftr(8 * p + r0);
    boff[p] = (int)(r0 * ldb + min(n0 + lseg * 8, N - 8));
  }
  // The lane offsets pass through an empty asm at each use, so no 64-bit
  // address is hoisted out of the loop (it would be spilled).
  auto issue = [&](int kt, char* S) {
    const long k = (long)kt * 64;
    const bf16* ab = (k >= K0) ? A1 + (k - K0) : A0 + k;
    int ao[4] = {aoff[0], aoff[1], aoff[2], aoff[3]};
    asm volatile("" : "+v"(ao[0]), "+v"(ao[1]), "+v"(ao[2]), "+v"(ao[3]));
#pragma unroll
    for (int it = 0; it < 4; ++it) g2lds16(ab + ao[it], S + (grp * 16 + wl + 4 * it) * 1024);
    if (grp == 0) {
      const bf16* bb = krow(k);
      int bo[2] = {boff[0], boff[1]};
      asm volatile("" : "+v"(bo[0]), "+v"(bo[1]));
#pragma unroll
      for (int it = 0; it < 8; ++it) g2lds16(bb + 8 * it * ldb + bo[it & 1], S + kStage2A + (wl + 4 * it) * 1024);
    }
  };
  auto bar = [] { asm volatile("s_barrier" ::: "memory"); };
  auto stage = [&](int kt) { return smem + (kt & 1) * kStage2Tr; };
  if (nkt <= 0) return;
  issue(0, stage(0));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  bar();
  if (grp == 1) bar();
  __builtin_amdgcn_sched_barrier(0);
  for (int kt = 0; kt < nkt; ++kt) {
    const char* S = stage(kt);
    if (kt + 1 < nkt) issue(kt + 1, stage(kt + 1));
    u32x4 av[2][kMB];
    u32x2 lo[2][8], hi[2][8];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) av[ks][mb] = rd128(S + lds_off2(q.wm * 64 + mb * 16 + q.r16, ks * 4 + q.g));
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) tr_issue(S + kStage2A + ks * 32 * 512, nb, q, lo[ks][nb], hi[ks][nb]);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) tie<0>(av[ks][mb]);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) lgkm_tie0(lo[ks][nb], hi[ks][nb]);
    }
    __builtin_amdgcn_sched_barrier(0);
    bar();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        Frag<bf16> af;
        af.v = av[ks][mb];
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const Frag<bf16> bfr = tr_make(lo[ks][nb], hi[ks][nb]);
          acc[mb][nb] = mma(acc[mb][nb], af, bfr);
        }
      }
    if (kt + 1 < nkt) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    bar();
    __builtin_amdgcn_sched_barrier(0);
  }
  if (grp == 0) bar();
}

// ---------------------------------------------------------------------------
// Split K.  When a call has fewer output tiles than the chip has CUs, each
// tile's K range is cut into S pieces, in two launches of the same kernel.
// The partial pass (grid tiles x S, blockIdx.x = tile * S + split) runs each
// piece's K-loop and writes its fp32 accumulators, side accumulators and
// (optionally) a parked side product to the workspace.  The merge pass (grid
// tiles) sums the S partials in split order, so the result does not depend
// on timing, and runs the epilogue.  The launch boundary orders the two
// passes: no workgroup waits for another, and no cache maintenance is needed
// inside a kernel (a device-scope release per workgroup, with the L2 write-
// back it implies, cost more than the K-loop at these sizes).
// ---------------------------------------------------------------------------
struct SplitK {
  float* part;     // [tiles][S][kSplitFloats]
  int S;           // 1: no split
  int pass;        // with S > 1: 0 = partial pass, 1 = merge pass
};
constexpr int kSplitAcc = kMB * 8;                         // f32x4 accumulators per thread
constexpr int kSplitSide = kMaxSide * kMB;                 // f32x4 side accumulators per thread
constexpr int kSplitFlush = kBM * kSlot;                   // floats of one parked side product
constexpr long kSplitFloats = (long)(kSplitAcc + kSplitSide) * 4 * kGemmThreads + kSplitFlush;

// K tiles [kb, ke) of split `split` out of S over nkt tiles.
__device__ __forceinline__ void split_range(int nkt, int S, int split, int& kb, int& ke) {
  kb = (int)((long)split * nkt / S);
  ke = (int)((long)(split + 1) * nkt / S);
}

// Partial pass: this piece's accumulators (and the parked side product in
// LDS at `flush`, if any) to the workspace.
template <int NS>
__device__ __forceinline__ void split_store(const SplitK& sk, int tile, int split, f32x4 (&acc)[kMB][8],
                                            f32x4 (&sacc)[NS > 0 ? NS : 1][kMB], const float* flush) {
  // An opaque copy of the thread id: nothing derived from it (the partial's
  // addresses) can be hoisted above the K-loop, where every register is taken.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  f32x4* mine = reinterpret_cast<f32x4*>(sk.part + ((long)tile * sk.S + split) * kSplitFloats);
#pragma unroll
  for (int i = 0; i < kSplitAcc; ++i) mine[i * kGemmThreads + tid] = acc[i >> 3][i & 7];
#pragma unroll
  for (int sb = 0; sb < NS; ++sb)
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) mine[(kSplitAcc + sb * kMB + mb) * kGemmThreads + tid] = sacc[sb][mb];
  if (flush) {
    __syncthreads();                             // the flush area was written by other threads
    float* myflush = reinterpret_cast<float*>(mine + (kSplitAcc + kSplitSide) * kGemmThreads);
    for (int e = tid; e < kSplitFlush; e += kGemmThreads) myflush[e] = flush[e];
  }
}

// Merge pass: acc, sacc (and the parked side product into LDS at `flush`)
// as the sum of the tile's S partials, in split order.
template <int NS>
__device__ __forceinline__ void split_load(const SplitK& sk, int tile, f32x4 (&acc)[kMB][8],
                                           f32x4 (&sacc)[NS > 0 ? NS : 1][kMB], float* flush) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kMB; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sb = 0; sb < NS; ++sb)
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) sacc[sb][mb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  if (flush)
    for (int e = tid; e < kSplitFlush; e += kGemmThreads) flush[e] = 0.f;
  // Accumulators: four at a time from up to four partials at once (16 loads
  // in flight), added in split order.
  const f32x4* p0 = reinterpret_cast<const f32x4*>(sk.part + (long)tile * sk.S * kSplitFloats);
  for (int sp0 = 0; sp0 < sk.S; sp0 += 4) {
#pragma unroll
    for (int i0 = 0; i0 < kSplitAcc; i0 += 4) {
      f32x4 t[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k)   // (past the last partial: reload it, discarded below)
          t[u][k] = p0[min(sp0 + u, sk.S - 1) * (kSplitFloats / 4) + (i0 + k) * kGemmThreads + tid];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (sp0 + u < sk.S) acc[(i0 + k) >> 3][(i0 + k) & 7] += t[u][k];
    }
  }
  for (int sp = 0; sp < sk.S; ++sp) {
    const f32x4* pp = reinterpret_cast<const f32x4*>(sk.part + ((long)tile * sk.S + sp) * kSplitFloats);
#pragma unroll
    for (int sb = 0; sb < NS; ++sb)
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) sacc[sb][mb] += pp[(kSplitAcc + sb * kMB + mb) * kGemmThreads + tid];
    if (flush) {
      const float* pf = reinterpret_cast<const float*>(pp + (kSplitAcc + kSplitSide) * kGemmThreads);
      for (int e = tid; e < kSplitFlush; e += kGemmThreads) flush[e] += pf[e];
    }
  }
  __syncthreads();
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

// Sum the two per-wave halves of the side products into Ts[sb][row][t]
// (float, raw Z.Sop).  Must follow the K-loop's final barrier.
template <class T, int NSIDE>
__device__ __forceinline__ void side_reduce(char* smem, f32x4 (&sacc)[NSIDE > 0 ? NSIDE : 1][kMB], int slot0 = 0) {
  const WaveId q = wave_id();
  float* Ts = ts_ptr(smem) + slot0 * kBM * kSlot;
  if (q.wn == 0) {
#pragma unroll
    for (int sb = 0; sb < NSIDE; ++sb)
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) Ts[ts_idx(sb, acc_row(q, mb, j), q.r16)] = sacc[sb][mb][j];
  }
  __syncthreads();
  if (q.wn == 1) {
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
// column n).  One fold tile holds BK / 16 slots (2 for bf16, 1 for fp32).
// FB functor: fb(R, slot, t0, v) fills v[0..VEC) for FB row R (the output
// column the B fragments of row R feed), adapter slot `slot`, ranks
// t0..t0+VEC-1; v is pre-zeroed.  Threads 0..255 build FA rows, threads
// 256..511 build FB rows.
// ---------------------------------------------------------------------------
template <class T, class FB>
__device__ __forceinline__ void fold(char* smem, f32x4 (&acc)[kMB][8], int nslot, const float (&fscale)[kMaxSide],
                                     FB& fb) {
  constexpr int VEC = ET<T>::VEC, BK = ET<T>::BK;
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
    for (int c = 0; c < 4; ++c) {
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
    Frag<T> af[kMB];
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) af[mb] = lds_frag<T>(FA, q.wm * 64 + mb * 16 + q.r16, q.g);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const Frag<T> bfr = lds_frag<T>(FBt, q.wn * 128 + nb * 16 + q.r16, q.g);
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) acc[mb][nb] = mma(acc[mb][nb], af[mb], bfr);
    }
    __syncthreads();
  }
}

// Output column (within the tile) of LDS B row R.
__device__ __forceinline__ int lds_row_col(int lg, int R) { return (R >> 7) * 128 + perm_col(lg, R & 15, (R >> 4) & 7); }
// LDS B row of tile column n.
__device__ __forceinline__ int col_lds_row(int lg, int n) { return (n >> 7) * 128 + perm_row(lg, n & 127); }

// ---------------------------------------------------------------------------
// A operands.
// ---------------------------------------------------------------------------

// Register-staged: rows of a row-major matrix, optionally split along K into
// [A0 | A1] (A0 has K0 columns, A1 has K1; both row stride ld).  Thread t
// stages chunk (t & 3) of rows (t >> 2) + 128 qq, qq = 0, 1.
template <class T>
struct RowsA {
  const T* b0;
  const T* b1;
  long ld, K0, K1;
  int avail;        // rows available from this thread's first row
  bool vec;
  __device__ __forceinline__ void init(const T* A0, const T* A1, long Kd0, long Kd1, long lda, long M, long m0,
                                       bool v) {
    const int r0 = threadIdx.x >> 2;
    ld = lda; K0 = Kd0; K1 = Kd1; vec = v;
    avail = (int)min((long)(1 << 30), M - m0 - r0);
    b0 = (avail > 0) ? A0 + (m0 + r0) * lda : nullptr;
    b1 = (avail > 0 && A1) ? A1 + (m0 + r0) * lda : nullptr;
  }
  __device__ __forceinline__ u32x4 get(int qq, long k) const {
    constexpr int VEC = ET<T>::VEC;
    if (128 * qq >= avail) return zero4();
    const T* r0p = b0 + (long)(128 * qq) * ld;
    if (k + VEC <= K0 || b1 == nullptr) return gload<T>(r0p, k, K0, vec);
    const T* r1p = b1 + (long)(128 * qq) * ld;
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

// ---------------------------------------------------------------------------
// NK loader (staged): A rows + B rows (output columns, row-major [n][K]) +
// side rows (adapter A_p rows [t][K]), all K-contiguous, in registers one K
// tile ahead; zero-filled past K and past the rank.  The kernel resolves the
// B row pointers once for the rows row_of(qq), qq = 0, 1, of this thread, and
// the side row pointer for side_row() (see side_ptr).
// ---------------------------------------------------------------------------
template <class T, class AOp, int NSIDE>
struct NKLoader {
  static constexpr bool kBTr = false;
  AOp a;
  const T* brow[2];
  const T* bfallback;
  const T* srow;
  long K;
  bool vecB, vecS;
  unsigned smask;
  u32x4 ra[2], rb[2], rs;
  __device__ static __forceinline__ int row_of(int qq) { return (int)(threadIdx.x >> 2) + 128 * qq; }
  // Side row (16 sb + t) this thread loads, or -1.
  __device__ static __forceinline__ int side_row() {
    const int r = threadIdx.x >> 2;
    return (r < 16 * NSIDE) ? r : -1;
  }
  // Pointer for side row t of an adapter whose rows start at `base` (nullptr:
  // no adapter in this block); ranks past r load nothing.
  __device__ static __forceinline__ const T* side_ptr(const T* base, int t, int r, long Kd, const T*) {
    return (base && t < r) ? base + (long)t * Kd : nullptr;
  }
  __device__ __forceinline__ void load(int kt) {
    const long k = (long)kt * ET<T>::BK + (threadIdx.x & 3) * ET<T>::VEC;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) ra[qq] = a.get(qq, k);
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) rb[qq] = gload<T>(brow[qq], k, K, vecB);
    if constexpr (NSIDE > 0) {
      rs = zero4();
      if ((int)(threadIdx.x >> 2) < 16 * NSIDE) rs = gload<T>(srow, k, K, vecS);
    }
  }
  __device__ __forceinline__ void store(char* As, char* Bs) const {
    const int c = threadIdx.x & 3, r0 = threadIdx.x >> 2;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) *reinterpret_cast<u32x4*>(As + lds_off(r0 + 128 * qq, c)) = ra[qq];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) *reinterpret_cast<u32x4*>(Bs + lds_off(r0 + 128 * qq, c)) = rb[qq];
    if constexpr (NSIDE > 0)
      if (r0 < NSIDE * 16) *reinterpret_cast<u32x4*>(Bs + lds_off(kBN + r0, c)) = rs;
  }
  __device__ __forceinline__ unsigned side_mask(int) const { return smask; }
};

// ---------------------------------------------------------------------------
// KN loaders: B stored [K][N] (N contiguous, e.g. W_d for dH = dY W_d) plus
// optional side operands stored [K][r] (e.g. B_g for dT_g = dG B_g).
//   krow(k)        -> pointer to row k of the B matrix (nullptr past K)
//   srow(sb, k)    -> pointer to row k of side operand sb (nullptr if inactive)
//   smask_of(kt)   -> active side blocks in tile kt
// ---------------------------------------------------------------------------

// bf16 (staged): the B tile keeps the [k][n] layout (kn_off) and is read
// with transpose reads; output column (within the tile) = wn*128 + 16 nb +
// r16.  The side tile of block sb is [32 k][16 t] at kSideOff + 1024 sb.  Two
// chunks of B and two of A per thread, zero-filled past K and N.
template <class AOp, class KRow, class SRow, class SMask, int NSIDE>
struct KNTrLoader {
  static constexpr bool kBTr = true;
  AOp a;
  KRow krow;
  SRow srow;
  SMask smask_of;
  long n0, N;
  int r;
  bool vecB, vecS;
  u32x4 ra[2], rb[2], rs;
  __device__ __forceinline__ void load(int kt) {
    const int tid = threadIdx.x;
    const long ka = (long)kt * 32 + (tid & 3) * 8;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) ra[qq] = a.get(qq, ka);
    const int seg = tid & 31, kr = tid >> 5;           // k rows kr, kr + 16
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) rb[qq] = gload<bf16>(krow((long)kt * 32 + kr + 16 * qq), n0 + seg * 8, N, vecB);
    if constexpr (NSIDE > 0) {
      const int sb = tid >> 6, e = tid & 63;
      rs = zero4();
      if (sb < NSIDE) rs = gload<bf16>(srow(sb, (long)kt * 32 + (e >> 1)), (e & 1) * 8, r, vecS);
    }
  }
  __device__ __forceinline__ void store(char* As, char* Bs) const {
    const int tid = threadIdx.x;
    const int c = tid & 3, r0 = tid >> 2;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) *reinterpret_cast<u32x4*>(As + lds_off(r0 + 128 * qq, c)) = ra[qq];
    const int seg = tid & 31, kr = tid >> 5;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) *reinterpret_cast<u32x4*>(Bs + kn_off(kr + 16 * qq, seg * 8)) = rb[qq];
    if constexpr (NSIDE > 0) {
      const int sb = tid >> 6, e = tid & 63;
      if (sb < NSIDE) *reinterpret_cast<u32x4*>(Bs + kSideOff + sb * 1024 + 16 * e) = rs;
    }
  }
  __device__ __forceinline__ unsigned side_mask(int kt) const { return smask_of(kt); }
};

// fp32: register-staged, transposed into B rows (output columns, LDS row
// col_lds_row(0, n), G = 1 order) and side rows [t][k].  Thread t stages a
// 4 (k) x 2 (n) block of B.
template <class KRow, class SRow, class SMask, int NSIDE>
struct KNLoader32 {
  static constexpr bool kBTr = false;
  RowsA<float> a;
  KRow krow;
  SRow srow;
  SMask smask_of;
  long n0, N;
  int r;
  bool vecB, vecS;
  u32x4 ra[2];
  float rb[4][2];
  float rs;
  __device__ __forceinline__ void load(int kt) {
    const int tid = threadIdx.x;
    const long ka = (long)kt * 16 + (tid & 3) * 4;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) ra[qq] = a.get(qq, ka);
    const int ng = tid & 127, kg = tid >> 7;              // columns 2 ng, 2 ng + 1; rows 4 kg .. 4 kg + 3
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float* row = krow((long)kt * 16 + 4 * kg + i);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const long n = n0 + 2 * ng + c;
        rb[i][c] = (row && n < N) ? row[n] : 0.f;
      }
    }
    if constexpr (NSIDE > 0) {
      const int sb = tid >> 8, e = tid & 255;               // k = e >> 4, t = e & 15
      rs = 0.f;
      if (sb < NSIDE) {
        const float* row = srow(sb, (long)kt * 16 + (e >> 4));
        if (row && (e & 15) < r) rs = row[e & 15];
      }
    }
  }
  __device__ __forceinline__ void store(char* As, char* Bs) const {
    const int tid = threadIdx.x;
    const int c = tid & 3, r0 = tid >> 2;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) *reinterpret_cast<u32x4*>(As + lds_off(r0 + 128 * qq, c)) = ra[qq];
    const int ng = tid & 127, kg = tid >> 7;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const float v[4] = {rb[0][cc], rb[1][cc], rb[2][cc], rb[3][cc]};
      *reinterpret_cast<u32x4*>(Bs + lds_off(col_lds_row(0, 2 * ng + cc), kg)) = pack(v);
    }
    if constexpr (NSIDE > 0) {
      const int sb = tid >> 8, e = tid & 255, k = e >> 4, t = e & 15;
      if (sb < NSIDE) *reinterpret_cast<float*>(Bs + lds_off(kBN + 16 * sb + t, k >> 2) + (k & 3) * 4) = rs;
    }
  }
  __device__ __forceinline__ unsigned side_mask(int kt) const { return smask_of(kt); }
};

// Raw buffer loads: a resource over `bytes` bytes at `base`; a load whose
// offset is at or past the end reads zero and never faults, so masked lanes
// need no branch (kBufOut is past the end of every buffer of at most 2 GB).
constexpr unsigned kBufOut = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Rank entries t0 .. t0+NV-1 of one adapter row or column (element t at
// src[t * stride]), zero past r.  Every load is issued, with its index
// clamped to r - 1 (r >= 1), so they go out back to back rather than one
// branch and one wait each.
template <class T, int NV>
__device__ __forceinline__ void load_rank(const T* src, long stride, int t0, int r, float* v) {
  T x[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) x[e] = src[(long)min(t0 + e, r - 1) * stride];
#pragma unroll
  for (int e = 0; e < NV; ++e) v[e] = (t0 + e < r) ? to_f<T>(x[e]) : 0.f;
}

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

// 8 consecutive values of one row, still packed as loaded (one 16-byte
// chunk for bf16, two for fp32), so a fetch can be issued well before use.
template <class T> struct Row8 { u32x4 c[sizeof(T) / 2]; };
template <class T>
__device__ __forceinline__ Row8<T> fetch_row8(const T* row, long c0, long len, bool vec) {
  Row8<T> r;
  r.c[0] = gload<T>(row, c0, len, vec);
  if constexpr (sizeof(T) == 4) r.c[1] = gload<T>(row, c0 + 4, len, vec);
  return r;
}
template <class T>
__device__ __forceinline__ void unpack_row8(const Row8<T>& r, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    unpack(r.c[0], v);
  } else {
    float t4[4];
    unpack(r.c[0], t4);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = t4[e];
    unpack(r.c[1], t4);
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
template <class T>
struct SRowLin {              // one side block: row k - kb of B (caller keeps k in range)
  const T* B; long kb, ld;
  __device__ __forceinline__ const T* operator()(int, long k) const { return B + (k - kb) * ld; }
};
struct SMaskNone {
  __device__ __forceinline__ unsigned operator()(int) const { return 0u; }
};
struct SMaskOne {
  __device__ __forceinline__ unsigned operator()(int) const { return 1u; }
};
struct SMask2 {               // block 0 active while the tile overlaps [0, K0), block 1 beyond
  long K0; int BK;
  __device__ __forceinline__ unsigned operator()(int kt) const {
    return (((long)kt * BK < K0) ? 1u : 0u) | (((long)(kt + 1) * BK > K0) ? 2u : 0u);
  }
};

// ---------------------------------------------------------------------------
// Epilogue helpers.
//
// ts_frag4: the A operand (scale * Ts[slot]) of an adapter partial
// P[t][col] = sum over the wave's rows of Aop[row][t] * V[row][col], one
// m-block (16 rows, K = 16) per MFMA: a lane's K slots are its rows j = 0..3,
// exactly what it holds of V in C layout, so V needs no shuffles.
// ---------------------------------------------------------------------------
template <class T>
__device__ __forceinline__ Frag4<T> ts_frag4(const float* Ts, int slot, float scale, const WaveId& q, int mb) {
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = scale * Ts[ts_idx(slot, acc_row(q, mb, j), q.r16)];
  return make_frag4<T>(v);
}

// Park: after a transpose-read K-loop a lane holds columns wn*128 + 16 nb +
// r16 of its rows.  park_mb() writes one m-block of the wave's accumulators
// (bf16) into a wave-private 4 KB area; park_row() then returns 8
// consecutive columns wn*128 + 8 r16 .. +7 of row (mb, j), the layout the
// epilogue's 16-byte loads and stores use.  No barrier: only this wave
// touches its area.
__device__ __forceinline__ int park_off(int row, int colbyte) {   // row 0..15, byte 0..255
  return row * 256 + ((((colbyte >> 5) ^ (((row >> 2) & 3) << 1))) << 5) + (colbyte & 31);
}
__device__ __forceinline__ void park_mb(char* base, const f32x4 (&acc)[kMB][8], int mb, const WaveId& q) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
      *reinterpret_cast<bf16*>(base + park_off(4 * q.g + j, (16 * nb + q.r16) * 2)) = (bf16)acc[mb][nb][j];
}
__device__ __forceinline__ void park_row(const char* base, int j, const WaveId& q, float (&v)[8]) {
  unpack(*reinterpret_cast<const u32x4*>(base + park_off(4 * q.g + j, 16 * q.r16)), v);
}

// Sum of NOUT partial tiles [16 t][128 cols] over the four wave-rows (fixed
// order wm = 3, 2, 1, 0) and store of the row-block partial to
// part[o] + col * 16 + t (cols bounded by ncols).  Lane column layout
// perm_col(LG, r16, nb): LG = 0 gives tile column wn*128 + 8*r16 + nb, LG = 3
// the natural order wn*128 + 16*nb + r16.
template <int NOUT, int LG = 0>
__device__ __forceinline__ void reduce_store_partials(char* smem, f32x4 (&pacc)[NOUT][8], float* const (&part)[NOUT],
                                                      long n0, long ncols) {
  const WaveId q = wave_id();
  float* red = reinterpret_cast<float*>(smem + kRedOff);
  static_assert(NOUT * 2 * 128 * 16 * 4 <= kRedBytes, "reduction scratch too small");
  auto slot = [&](int o, int nb) -> f32x4* {
    return reinterpret_cast<f32x4*>(red + ((o * 2 + q.wn) * 128 + perm_col(LG, q.r16, nb)) * 16 + 4 * q.g);
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
        const long col = n0 + q.wn * 128 + perm_col(LG, q.r16, nb);
        if (col < ncols) *reinterpret_cast<f32x4*>(part[o] + col * 16 + 4 * q.g) = v;
      }
  }
}


// ---------------------------------------------------------------------------
// Runs.  A workgroup walks a run of L consecutive column tiles of one row
// block (the last run of a row block may be shorter).  The rank-r side
// product of the row block is computed in the run's first tile only and its
// fold operand stays in LDS for the rest of the run; the next tile's first K
// tile is issued before the current tile's fold and epilogue.  Runs are
// numbered row block by row block and handed to the 8 XCDs in contiguous
// ranges (consecutive blockIdx go round-robin to the XCDs), so the workgroups
// of one XCD share a few row blocks, and at any moment every XCD reads the
// same few weight column blocks.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void run_coords(int nruns, int RPB, int L, int NC, int& rb, int& cb0, int& cb1) {
  const int b = blockIdx.x;
  const int per = nruns >> 3, rem = nruns & 7, x = b & 7, i = b >> 3;
  const int u = (x < rem) ? x * (per + 1) + i : rem * (per + 1) + (x - rem) * per + i;
  rb = u / RPB;
  cb0 = (u % RPB) * L;
  cb1 = min(NC, cb0 + L);
}

// LDS of a run workgroup: the two K-loop stages, then the run's fold A operand
// (scale * T in bf16, [256 rows][32 K], 64-byte rows).  It starts inside stage
// 1's side-row area, which only the run's first tile loads (before the
// operand is built).  After a K-loop, stage 1 holds the side products (fp32)
// and the fold B tile while stage 0 takes the next tile's first K tile.
constexpr int kRunFAOff = kStage2 + kStage2A + kBN * kRow2;      // stage 1's side rows
constexpr int kRunLds = kRunFAOff + kBM * kRowBytes;
static_assert(kRunLds <= 163840, "run workgroup LDS");
constexpr int kRunTsOff = kStage2;                                // side products, fp32 [3][256][16]
constexpr int kRunFBOff = kStage2 + kTsBytes;                     // fold B tile [256][32 K]
static_assert(kRunFBOff + kBN * kRowBytes <= kRunFAOff, "fold B tile overlaps the fold A operand");

// Build the fold A operand FA[m][16 s + t] = fscale[s] * Ts[s][m][t] (bf16)
// for nslot <= 2 adapters from the side products at `ts`.
__device__ __forceinline__ void build_fold_a(char* FA, const float* ts, int nslot, const float (&fscale)[kMaxSide]) {
  for (int e = threadIdx.x; e < kBM * 4; e += kGemmThreads) {
    const int m = e >> 2, c = e & 3;
    const int slot = (c * 8) / kSlot, t0 = (c * 8) % kSlot;
    float v[8];
    const float sc = slot == 0 ? fscale[0] : fscale[1];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = (slot < nslot) ? sc * ts[ts_idx(slot, m, t0 + u)] : 0.f;
    *reinterpret_cast<u32x4*>(FA + lds_off(m, c)) = pack(v);
  }
}

// acc += FA . FB^T over one fold tile (K = 32) with FB rows built by fb.
template <class FB>
__device__ __forceinline__ void fold_run(const char* FA, char* FBt, f32x4 (&acc)[kMB][8], FB& fb) {
  const WaveId q = wave_id_opaque();
  for (int e = threadIdx.x; e < kBN * 4; e += kGemmThreads) {
    const int R = e >> 2, c = e & 3;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    fb(R, (c * 8) / kSlot, (c * 8) % kSlot, v);
    *reinterpret_cast<u32x4*>(FBt + lds_off(R, c)) = pack(v);
  }
  __syncthreads();
  Frag<bf16> af[kMB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) af[mb] = lds_frag<bf16>(FA, q.wm * 64 + mb * 16 + q.r16, q.g);
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const Frag<bf16> bfr = lds_frag<bf16>(FBt, q.wn * 128 + nb * 16 + q.r16, q.g);
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) acc[mb][nb] = mma(acc[mb][nb], af[mb], bfr);
  }
}

}  // namespace lora

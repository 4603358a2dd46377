// Device-side building blocks shared by every kernel of the LoRA library
// (gfx950 / CDNA4, wave64).
//
// GEMM tiles live in LDS as rows of 64 bytes (32 bf16 or 16 fp32 along K),
// split into four 16-byte chunks; the chunk index is XOR-swizzled with
// (row >> 1) & 3.  Two rows share one 128-byte bank line, and the swizzle
// spreads the 16 consecutive rows an MFMA fragment read touches over all
// bank groups: measured on gfx950 that read runs within 5% of a linear 1 KB
// read, whereas the unswizzled layout (or one keyed on row & 3) runs ~1.5x
// slower.
//
// MFMA: v_mfma_f32_16x16x32_bf16 for bf16 and 4 x v_mfma_f32_16x16x4_f32 for
// fp32.  A "fragment" is one 16-byte chunk of K values of one row (A operand)
// or one column (B operand) held by a lane: lane l covers row/column (l & 15)
// and K slots VEC*(l>>4) .. VEC*(l>>4)+VEC-1.  Because A and B use the same
// slot <-> K map, the products pair up correctly whatever order the hardware
// sums the slots in.  The 16x16 fp32 result is held as C[4*(l>>4) + j][l & 15],
// j = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lora {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;       // 4 waves of 64
constexpr int kBM = 256;            // tile rows (tokens)
constexpr int kBN = 256;            // tile columns
constexpr int kRowBytes = 64;       // one LDS tile row (four 16-byte chunks)
constexpr int kMaxSide = 3;         // adapters whose rank-r product a GEMM carries
constexpr int kSlot = 16;           // K width reserved per adapter in a fold (rank <= 16)

template <class T> struct ET;
template <> struct ET<bf16> {
  static constexpr int VEC = 8;     // elements per 16-byte chunk
  static constexpr int BK = 32;     // K per LDS tile row (one MFMA K-step)
  static constexpr int BYTES = 2;
};
template <> struct ET<float> {
  static constexpr int VEC = 4;
  static constexpr int BK = 16;
  static constexpr int BYTES = 4;
};

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 3; }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ swz(row)) << 4);
}

__device__ __forceinline__ u32x4 zero4() { u32x4 z = {0u, 0u, 0u, 0u}; return z; }

// ---- bf16 <-> fp32 ---------------------------------------------------------
__device__ __forceinline__ float bf_lo(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(unsigned u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ unsigned pack_bf2(float lo, float hi) {
  bf16x2 v;
  v.x = (bf16)lo;   // round to nearest even (v_cvt_pk_bf16_f32)
  v.y = (bf16)hi;
  return __builtin_bit_cast(unsigned, v);
}

// A 16-byte chunk as VEC floats and back.
__device__ __forceinline__ void unpack(u32x4 c, float (&v)[8]) {
  v[0] = bf_lo(c.x); v[1] = bf_hi(c.x); v[2] = bf_lo(c.y); v[3] = bf_hi(c.y);
  v[4] = bf_lo(c.z); v[5] = bf_hi(c.z); v[6] = bf_lo(c.w); v[7] = bf_hi(c.w);
}
__device__ __forceinline__ void unpack(u32x4 c, float (&v)[4]) {
  v[0] = __uint_as_float(c.x); v[1] = __uint_as_float(c.y);
  v[2] = __uint_as_float(c.z); v[3] = __uint_as_float(c.w);
}
__device__ __forceinline__ u32x4 pack(const float (&v)[8]) {
  u32x4 c;
  c.x = pack_bf2(v[0], v[1]); c.y = pack_bf2(v[2], v[3]);
  c.z = pack_bf2(v[4], v[5]); c.w = pack_bf2(v[6], v[7]);
  return c;
}
__device__ __forceinline__ u32x4 pack(const float (&v)[4]) {
  u32x4 c;
  c.x = __float_as_uint(v[0]); c.y = __float_as_uint(v[1]);
  c.z = __float_as_uint(v[2]); c.w = __float_as_uint(v[3]);
  return c;
}

template <class T> __device__ __forceinline__ float to_f(T x);
template <> __device__ __forceinline__ float to_f<bf16>(bf16 x) { return (float)x; }
template <> __device__ __forceinline__ float to_f<float>(float x) { return x; }
template <class T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }

// ---- global 16-byte chunk loads with bounds --------------------------------
// Elements [k, k+VEC) of a row; zero past `len` or when row == nullptr.
// `vec` means the row is 16-byte aligned and len % VEC == 0.
template <class T>
__device__ __forceinline__ u32x4 gload(const T* row, long k, long len, bool vec) {
  constexpr int VEC = ET<T>::VEC;
  if (row == nullptr || k >= len) return zero4();
  if (vec) return *reinterpret_cast<const u32x4*>(row + k);
  float v[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) v[e] = (k + e < len) ? to_f<T>(row[k + e]) : 0.0f;
  return pack(v);
}

// Store `n` (<= VEC) leading elements of v at p (vector store when full and aligned).
template <class T, int NV>
__device__ __forceinline__ void gstore(T* p, const float (&v)[NV], int n, bool vec) {
  if (n <= 0) return;
  if (vec && n == NV) {
    if constexpr (sizeof(T) * NV == 16) {
      *reinterpret_cast<u32x4*>(p) = pack(v);
      return;
    } else if constexpr (sizeof(T) * NV == 8) {
      u32x2 c;
      if constexpr (sizeof(T) == 2) { c.x = pack_bf2(v[0], v[1]); c.y = pack_bf2(v[2], v[3]); }
      else { c.x = __float_as_uint(v[0]); c.y = __float_as_uint(v[1]); }
      *reinterpret_cast<u32x2*>(p) = c;
      return;
    } else if constexpr (sizeof(T) * NV == 4) {
      if constexpr (sizeof(T) == 2) *reinterpret_cast<unsigned*>(p) = pack_bf2(v[0], v[1]);
      else *reinterpret_cast<unsigned*>(p) = __float_as_uint(v[0]);
      return;
    }
  }
#pragma unroll
  for (int e = 0; e < NV; ++e)
    if (e < n) p[e] = from_f<T>(v[e]);
}

// gstore with non-temporal vector stores: for outputs no kernel of the same
// call reads again, so they displace less of the L2 and MALL contents that
// the next kernel does read.
template <class T, int NV>
__device__ __forceinline__ void gstore_nt(T* p, const float (&v)[NV], int n, bool vec) {
  if constexpr (sizeof(T) == 2 && NV == 4) {
    if (vec && n == NV) {
      u32x2 c;
      c.x = pack_bf2(v[0], v[1]);
      c.y = pack_bf2(v[2], v[3]);
      __builtin_nontemporal_store(c, reinterpret_cast<u32x2*>(p));
      return;
    }
  }
  gstore<T, NV>(p, v, n, vec);
}

// ---- MFMA fragments ----------------------------------------------------------
// Main-loop fragment: one 16-byte chunk (8 bf16 or 4 fp32 K slots per lane).
template <class T> struct Frag { u32x4 v; };

__device__ __forceinline__ f32x4 mma(f32x4 c, const Frag<bf16>& a, const Frag<bf16>& b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                 __builtin_bit_cast(bf16x8, b.v), c, 0, 0, 0);
}
// fp32: MFMA j takes K slot j of every lane group, so the four of them cover
// all 16 K values of the fragment.
__device__ __forceinline__ f32x4 mma(f32x4 c, const Frag<float>& a, const Frag<float>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.v.x), __uint_as_float(b.v.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.v.y), __uint_as_float(b.v.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.v.z), __uint_as_float(b.v.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.v.w), __uint_as_float(b.v.w), c, 0, 0, 0);
  return c;
}

// Fragment of LDS tile row `row` for lane group g (= lane >> 4): chunk g.
template <class T> __device__ __forceinline__ Frag<T> lds_frag(const char* buf, int row, int g) {
  Frag<T> f;
  f.v = *reinterpret_cast<const u32x4*>(buf + lds_off(row, g));
  return f;
}

// Epilogue fragment with four K slots per lane: lane l holds K slots
// 4*(l>>4) .. 4*(l>>4)+3, so in C layout a lane's four rows j = 0..3 of one
// m-block are exactly its K slots (v_mfma_f32_16x16x16_bf16, or four
// 16x16x4 fp32 MFMAs).
template <class T> struct Frag4;
template <> struct Frag4<bf16> { u32x2 v; };
template <> struct Frag4<float> { u32x4 v; };
template <class T> __device__ __forceinline__ Frag4<T> make_frag4(const float (&v)[4]);
template <> __device__ __forceinline__ Frag4<bf16> make_frag4<bf16>(const float (&v)[4]) {
  Frag4<bf16> f;
  f.v = (u32x2){pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
  return f;
}
template <> __device__ __forceinline__ Frag4<float> make_frag4<float>(const float (&v)[4]) {
  Frag4<float> f;
  f.v = pack(v);
  return f;
}
__device__ __forceinline__ f32x4 mma4(f32x4 c, const Frag4<bf16>& a, const Frag4<bf16>& b) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a.v), __builtin_bit_cast(i16x4, b.v), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ f32x4 mma4(f32x4 c, const Frag4<float>& a, const Frag4<float>& b) {
  Frag<float> fa, fb;
  fa.v = a.v;
  fb.v = b.v;
  return mma(c, fa, fb);
}

// ---- column permutation of a 128-column wave window ---------------------------
// A wave owns 8 MFMA column blocks of 16.  Loading B rows into LDS in a
// permuted order decides which output column each lane holds: with G groups,
// lane c holds, in block b = gg*(8/G) + e, window column gg*(128/G) + c*(8/G) + e.
// G = 1 gives every lane 8 consecutive columns (16-byte stores); G = 2 puts
// columns w and w+64 in the same lane (GLU gate/up pairs, RoPE pairs for
// head_dim 128); G = 4 pairs w and w+32 (RoPE, head_dim 64).
__device__ __forceinline__ int perm_col(int lg, int c, int b) {   // lg = log2(G)
  const int cw = 8 >> lg, gw = 128 >> lg;
  return (b / cw) * gw + c * cw + (b % cw);
}
__device__ __forceinline__ int perm_row(int lg, int w) {
  const int cw = 8 >> lg, gw = 128 >> lg;
  const int gg = w / gw, rem = w % gw;
  return ((gg * cw + rem % cw) << 4) + rem / cw;
}

// ---- lane-group sums (DPP, within one 16-lane row) -----------------------------
template <int CTRL> __device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum over aligned groups of N lanes (N = 4, 8 or 16); every lane of a group
// gets the group's sum.  All lanes of the group must be active.
template <int N> __device__ __forceinline__ float lane_group_sum(float v) {
  static_assert(N == 4 || N == 8 || N == 16, "groups of 4, 8 or 16 lanes");
  v += dpp_f<0xB1>(v);                           // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);                           // quad_perm [2,3,0,1]
  if constexpr (N >= 8) v += dpp_f<0x141>(v);    // row_half_mirror: lane i <- 7 - i
  if constexpr (N >= 16) v += dpp_f<0x140>(v);   // row_mirror: lane i <- 15 - i
  return v;
}

// ---- activations (fp32) --------------------------------------------------------
#define LORA_ACT_SWIGLU 0
#define LORA_ACT_GEGLU_TANH 1
#define LORA_ACT_GEGLU_ERF 2

// The activations use the hardware exponential (v_exp_f32, 2^x) and
// reciprocal (v_rcp_f32), each within about one ulp, instead of the
// range-reduced expf and the IEEE division sequence: the GLU epilogues
// evaluate them for every element of G while no MFMA runs.  Limits hold:
// e^x -> inf gives rcp -> 0, e^x -> 0 gives rcp(1) = 1.
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float sigmoidf_(float x) { return rcp_hw(1.0f + exp_hw(-x)); }
// tanh(y) = 1 - 2 / (1 + e^(2y)).
__device__ __forceinline__ float tanh_hw(float y) { return 1.0f - 2.0f * rcp_hw(1.0f + exp_hw(2.0f * y)); }

template <int ACT> __device__ __forceinline__ float act_fwd(float g) {
  if constexpr (ACT == LORA_ACT_SWIGLU) {
    return g * sigmoidf_(g);
  } else if constexpr (ACT == LORA_ACT_GEGLU_TANH) {
    const float k0 = 0.7978845608028654f, k1 = 0.044715f;   // sqrt(2/pi), cubic coefficient
    return 0.5f * g * (1.0f + tanh_hw(k0 * (g + k1 * g * g * g)));
  } else {
    return 0.5f * g * (1.0f + erff(g * 0.7071067811865476f));   // exact GELU: g * Phi(g)
  }
}
// phi(g) and phi'(g) together.
template <int ACT> __device__ __forceinline__ void act_both(float g, float& phi, float& dphi) {
  if constexpr (ACT == LORA_ACT_SWIGLU) {
    const float s = sigmoidf_(g);
    phi = g * s;
    dphi = s * (1.0f + g * (1.0f - s));
  } else if constexpr (ACT == LORA_ACT_GEGLU_TANH) {
    const float k0 = 0.7978845608028654f, k1 = 0.044715f;
    const float t = tanh_hw(k0 * (g + k1 * g * g * g));
    phi = 0.5f * g * (1.0f + t);
    dphi = 0.5f * (1.0f + t) + 0.5f * g * (1.0f - t * t) * k0 * (1.0f + 3.0f * k1 * g * g);
  } else {
    // Phi(g) = (1 + erf(g / sqrt 2)) / 2; phi'(g) = Phi(g) + g * exp(-g^2/2) / sqrt(2 pi).
    const float cdf = 0.5f * (1.0f + erff(g * 0.7071067811865476f));
    phi = g * cdf;
    dphi = cdf + g * 0.3989422804014327f * exp_hw(-0.5f * g * g);
  }
}

// ---- tile scheduling -------------------------------------------------------------
// blockIdx.x -> (row block, column block).  Consecutive blocks go round-robin
// to the 8 XCDs; remap so each XCD gets a contiguous range of logical tiles,
// then walk that range in groups of `gm` row blocks so CTAs resident on one
// XCD share A row blocks and B column tiles in its L2.
__device__ __forceinline__ void tile_coords_at(int b, int ntiles, int R, int NC, int gm, int& rb, int& cb) {
  const int per = ntiles >> 3, rem = ntiles & 7, x = b & 7, i = b >> 3;
  const int L = (x < rem) ? x * (per + 1) + i : rem * (per + 1) + (x - rem) * per + i;
  const int gsz = gm * NC;
  const int grp = L / gsz;
  const int first = grp * gm;
  const int g = min(gm, R - first);
  const int w = L - grp * gsz;
  rb = first + w % g;
  cb = w / g;
}
__device__ __forceinline__ void tile_coords(int ntiles, int R, int NC, int gm, int& rb, int& cb) {
  tile_coords_at(blockIdx.x, ntiles, R, NC, gm, rb, cb);
}

}  // namespace lora

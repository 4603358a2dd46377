// Host orchestration and C ABI of the fused LoRA MLP / QKV library (gfx950).
//
// Each entry point validates its arguments on the host (nothing is enqueued
// on an error), carves the caller's workspace, and enqueues its kernels on
// the caller's stream.  No allocation, no synchronisation, no global state
// besides the optional timing recorder and the thread-local error message.
#include "lora_mi355x.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "kernels_bwd.h"
#include "kernels_fwd.h"

using namespace lora;

namespace lora {
// Defined in kernels_default_sched.hip (a translation unit of its own,
// compiled with the default instruction scheduling).
hipError_t launch_mlp_dx_split_bf16(const MlpDxArgs& a, hipStream_t st);
hipError_t launch_linear_run_bf16(const LinearArgs& a, hipStream_t st);
hipError_t launch_qkv_run_bf16(const QKVFwdArgs& a, hipStream_t st);
template <class T>
hipError_t launch_linear_fwd(bool fast, const LinearArgs& a, dim3 grid, hipStream_t st);
template <class T>
hipError_t launch_qkv_fwd(bool fast, int head_dim, int ns, const QKVFwdArgs& a, dim3 grid, hipStream_t st);

// gate/up: the fast path runs as column-tile runs (k_gateup_run).
template <class T, int ACT>
hipError_t launch_gateup(bool fast, const GateUpArgs& a, dim3 grid, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    if (fast) {
      hipLaunchKernelGGL((k_gateup_run<ACT>), grid, dim3(kGemmThreads), 0, st, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((k_gateup_fwd<T, ACT, false>), grid, dim3(kGemmThreads), 0, st, a);
  return hipGetLastError();
}
}  // namespace lora

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}
int ok() {
  g_err[0] = '\0';
  return LORA_OK;
}

// ---- timing ---------------------------------------------------------------
const char* kNames[] = {"k_gateup_fwd",  "k_linear_fwd", "k_rope_table", "k_qkv_fwd",
                        "k_bwd_prologue", "k_down_bwd",   "k_mlp_dx_bwd", "k_proj_dx_bwd",
                        "k_reduce",       "k_dt_sum",     "k_qk_norm_bwd", "k_mlp_dt",
                        "k_bwd_prologue_ring"};
constexpr int kNumNames = sizeof(kNames) / sizeof(kNames[0]);

struct Rec {
  int kernel;
  hipEvent_t e0, e1;
};
std::mutex g_tm;
bool g_timing = false;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

int kernel_id(const char* name) {
  for (int i = 0; i < kNumNames; ++i)
    if (strcmp(kNames[i], name) == 0) return i;
  return -1;
}

template <class Kern, class... Args>
int launch(int kid, Kern kern, dim3 grid, dim3 block, hipStream_t st, Args... args) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return LORA_OK;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  bool timed = false;
  {
    std::lock_guard<std::mutex> lk(g_tm);
    if (g_timing) {
      e0 = take_event();
      e1 = take_event();
      timed = e0 && e1;
      if (!timed) {                      // keep whichever event was made for later
        if (e0) g_pool.push_back(e0);
        if (e1) g_pool.push_back(e1);
      }
    }
  }
  if (timed) (void)hipEventRecord(e0, st);
  hipLaunchKernelGGL(kern, grid, block, 0, st, args...);
  const hipError_t err = hipGetLastError();
  if (timed) {
    (void)hipEventRecord(e1, st);
    std::lock_guard<std::mutex> lk(g_tm);
    g_recs.push_back(Rec{kid, e0, e1});
  }
  if (err != hipSuccess) return fail(LORA_ERR_HIP, "%s launch failed: %s", kNames[kid], hipGetErrorString(err));
  return LORA_OK;
}

// Timed launch through a callable that enqueues one kernel and returns the
// launch status (for kernels compiled in another translation unit).
template <class F>
int launch_call(int kid, hipStream_t st, F enqueue) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  bool timed = false;
  {
    std::lock_guard<std::mutex> lk(g_tm);
    if (g_timing) {
      e0 = take_event();
      e1 = take_event();
      timed = e0 && e1;
      if (!timed) {
        if (e0) g_pool.push_back(e0);
        if (e1) g_pool.push_back(e1);
      }
    }
  }
  if (timed) (void)hipEventRecord(e0, st);
  const hipError_t err = enqueue();
  if (timed) {
    (void)hipEventRecord(e1, st);
    std::lock_guard<std::mutex> lk(g_tm);
    g_recs.push_back(Rec{kid, e0, e1});
  }
  if (err != hipSuccess) return fail(LORA_ERR_HIP, "%s launch failed: %s", kNames[kid], hipGetErrorString(err));
  return LORA_OK;
}

// ---- helpers ----------------------------------------------------------------
bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int vecw(int dtype) { return dtype == LORA_BF16 ? 8 : 4; }
size_t esz(int dtype) { return dtype == LORA_BF16 ? 2 : 4; }
size_t up256(size_t x) { return (x + 255) & ~size_t(255); }
long cdiv(long a, long b) { return (a + b - 1) / b; }

// Launch Fast<true> when allowed (bf16 only), else Fast<false>.
#define LORA_LAUNCH_FAST(kid, FAST_COND, KERN_TRUE, KERN_FALSE, grid, block, st, args)                   \
  ([&]() -> int {                                                                                        \
    if constexpr (sizeof(T) == 2) {                                                                      \
      if (FAST_COND) return launch(kid, KERN_TRUE, grid, block, st, args);                               \
    }                                                                                                    \
    return launch(kid, KERN_FALSE, grid, block, st, args);                                               \
  }())

// Direct global->LDS loads need full bf16 K tiles, 16-byte aligned rows and
// 32-bit row offsets (each call adds what its other operands need); other
// calls take the register-staged (masked) loaders.
bool fast_ok(int dtype, long K, long rows, std::initializer_list<const void*> ptrs) {
  if (dtype != LORA_BF16 || K % ET<bf16>::BK != 0 || rows * K >= (1L << 31)) return false;
  for (const void* p : ptrs)
    if (!al16(p)) return false;
  return true;
}

// dX epilogues of the fast paths read X rows by raw buffer loads: aligned
// rows and X at most 2 GB.
bool x_buf_ok(int vecO, long N, long h) { return vecO && N * h * 2 <= (1L << 31); }

struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class P> P* take(size_t bytes) {
    P* p = reinterpret_cast<P*>(base ? base + off : nullptr);
    off += up256(bytes);
    return p;
  }
};

// Splits of a GEMM's K range when the call has fewer output tiles than the
// chip has CUs (256 on MI355X).  S splits cost about nkt * c_k / S for the
// partial pass and c_m * S for the merge pass (one workgroup per tile reads
// the S partial tiles).  Measured on MI355X: c_k ~ 2.1 us per K tile of 64
// at these sizes; c_m ~ 5 us per 376 KB partial.  So S ~ sqrt(c_k nkt /
// c_m), at most one workgroup per CU and 16 splits.  Shape-only, so the
// workspace queries and the launches agree; used on the bf16 fast paths
// (K % 64 == 0).
constexpr int kCUs = 256;
int split_count(long tiles, long nkt) {
  if (tiles <= 0 || tiles >= kCUs || nkt <= 0) return 1;
  long S = (long)(std::sqrt(2.1 * (double)nkt / 5.0) + 0.5);
  if (S > kCUs / tiles) S = kCUs / tiles;
  if (S > 16) S = 16;
  return S < 1 ? 1 : (int)S;
}
// Runs of column tiles (kernels that walk several tiles of one row block):
// run length L = ceil(tiles / CUs), so the runs fill the chip about once.
void run_layout(long R, long NC, int& L, int& RPB, int& nruns) {
  const long tiles = R * NC;
  L = (int)std::max(1L, cdiv(tiles, kCUs));
  RPB = (int)cdiv(NC, L);
  nruns = (int)(R * RPB);
}
struct SplitWs {
  float* part = nullptr;
  int S = 1;
  long tiles = 0;
};
template <class C>
SplitWs take_split(C& c, bool eligible, long tiles, long nkt) {
  SplitWs sw;
  sw.S = eligible ? split_count(tiles, nkt) : 1;
  sw.tiles = tiles;
  if (sw.S > 1) sw.part = c.template take<float>((size_t)tiles * sw.S * kSplitFloats * 4);
  return sw;
}
// The kernels' SplitK argument (partial pass first).
void split_setup(const SplitWs& sw, SplitK& sk) {
  sk.part = sw.part;
  sk.S = sw.S;
  sk.pass = 0;
}
// Both passes of a split linear forward, or the one launch of an unsplit one.
template <class T>
hipError_t launch_linear_fwd_passes(bool fast, const LinearArgs& a, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    if (fast && a.sk.S == 1) {                   // runs of column tiles
      LinearArgs r = a;
      run_layout(r.R, r.NC, r.L, r.RPB, r.nruns);
      return launch_linear_run_bf16(r, st);
    }
  }
  hipError_t e = launch_linear_fwd<T>(fast, a, dim3(a.R * a.NC * a.sk.S), st);
  if (e == hipSuccess && a.sk.S > 1) {
    LinearArgs m = a;
    m.sk.pass = 1;
    e = launch_linear_fwd<T>(fast, m, dim3(a.R * a.NC), st);
  }
  return e;
}

// Column ranges of the backward prologue (grid R x NCR, CPC chunks of BK
// columns each): at least 8, more when there are few row blocks, so that the
// grid still covers the CUs (a small call has R = 16 row blocks or fewer);
// ranges that would get no chunk are dropped.  (Twice as many ranges, two
// workgroups per CU, measured slower on MI355X: every range adds a dT
// partial of N x 16 floats per adapter.)
void prologue_ranges(long NCH, long R, int& NCR, int& CPC) {
  if (NCH <= 0) {
    NCR = 0;
    CPC = 0;
    return;
  }
  long want = std::max(8L, cdiv(kCUs, std::max(1L, R)));
  if (want > NCH) want = NCH;
  CPC = (int)cdiv(NCH, want);
  NCR = (int)cdiv(NCH, CPC);
}

// MLP workspace.
struct MlpWs {
  void* H;
  void *dG, *dU;
  float *dT_part, *dT, *pA_d, *pB_g, *pB_u, *pA_g, *pA_u, *pB_d;
  SplitWs split;    // forward: down projection; backward: MLP dX
  int NCR, NCH, CPC;
  int KS;           // backward: K splits of k_mlp_dt
  size_t bytes;
};
MlpWs mlp_ws(const lora_mlp_desc_t& d, int pass, void* base) {
  MlpWs w{};
  Carver c(base);
  const long N = d.n_tokens, h = d.hidden, i = d.inter;
  const long R = cdiv(N, kBM);
  const size_t es = esz(d.dtype);
  const int BK = d.dtype == LORA_BF16 ? PT<bf16>::BK : PT<float>::BK;   // prologue column chunk
  w.NCH = (int)cdiv(h, BK);
  prologue_ranges(w.NCH, R, w.NCR, w.CPC);
  const bool bf = d.dtype == LORA_BF16;
  if (pass == 0) {
    w.H = c.take<void>(N * i * es);
    w.split = take_split(c, bf && i % 64 == 0, R * cdiv(h, kBN), i / 64);
  } else {
    w.split = take_split(c, bf && i % 64 == 0 && d.rank == 16, R * cdiv(h, kBN), 2 * i / 64);
    w.dG = c.take<void>(N * i * es);
    w.dU = c.take<void>(N * i * es);
    // k_mlp_dt: about one workgroup per CU over the row blocks x K splits.
    w.KS = (int)std::max(1L, std::min(cdiv(kCUs, std::max(1L, R)), std::max(1L, 2 * i / 64)));
    w.dT_part = c.take<float>((size_t)std::max(w.NCR, w.KS) * 3 * N * 16 * 4);
    w.dT = c.take<float>((size_t)3 * N * 16 * 4);
    w.pA_d = c.take<float>(R * i * 16 * 4);
    w.pB_g = c.take<float>(R * i * 16 * 4);
    w.pB_u = c.take<float>(R * i * 16 * 4);
    w.pA_g = c.take<float>(R * h * 16 * 4);
    w.pA_u = c.take<float>(R * h * 16 * 4);
    w.pB_d = c.take<float>(R * h * 16 * 4);
  }
  w.bytes = c.off;
  return w;
}

struct QkvWs {
  float *cs, *sn;
  void* dP;
  float *dT_part, *dT, *pA[3], *dB_part;
  int NCR, NCH, CPC;
  size_t bytes;
};
QkvWs qkv_ws(const lora_qkv_desc_t& d, int pass, void* base) {
  QkvWs w{};
  Carver c(base);
  const long N = (long)d.batch * d.seq, h = d.hidden;
  const long O = (long)(d.n_q + 2 * d.n_kv) * d.head_dim;
  const long R = cdiv(N, kBM);
  const size_t es = esz(d.dtype);
  const int BK = d.dtype == LORA_BF16 ? PT<bf16>::BK : PT<float>::BK;   // prologue column chunk
  w.cs = c.take<float>((size_t)d.seq * (d.head_dim / 2) * 4);
  w.sn = c.take<float>((size_t)d.seq * (d.head_dim / 2) * 4);
  w.NCH = (int)(O / BK);
  prologue_ranges(w.NCH, R, w.NCR, w.CPC);
  if (pass == 1) {
    w.dP = c.take<void>(N * O * es);
    w.dT_part = c.take<float>((size_t)w.NCR * 3 * N * 16 * 4);
    w.dT = c.take<float>((size_t)3 * N * 16 * 4);
    for (int p = 0; p < 3; ++p) w.pA[p] = c.take<float>(R * h * 16 * 4);
    w.dB_part = c.take<float>(R * O * 16 * 4);
  }
  w.bytes = c.off;
  return w;
}

// LoRA linear workspace (backward only).
struct LinWs {
  float *dT_part, *dT, *pA, *dB_part;
  SplitWs split;    // forward
  int NCR, NCH, CPC;
  size_t bytes;
};
LinWs lin_ws(const lora_linear_desc_t& d, int pass, void* base) {
  LinWs w{};
  Carver c(base);
  const long N = d.n_tokens, in = d.in_features, out = d.out_features;
  const long R = cdiv(N, kBM);
  const int BK = d.dtype == LORA_BF16 ? PT<bf16>::BK : PT<float>::BK;   // prologue column chunk
  w.NCH = (int)cdiv(out, BK);
  prologue_ranges(w.NCH, R, w.NCR, w.CPC);
  if (pass == 0) w.split = take_split(c, d.dtype == LORA_BF16 && in % 64 == 0, R * cdiv(out, kBN), in / 64);
  if (pass == 1) {
    w.dT_part = c.take<float>((size_t)w.NCR * 3 * N * 16 * 4);
    w.dT = c.take<float>((size_t)3 * N * 16 * 4);
    w.pA = c.take<float>(R * in * 16 * 4);
    w.dB_part = c.take<float>(R * out * 16 * 4);
  }
  w.bytes = c.off;
  return w;
}

// ---- validation ---------------------------------------------------------------
int check_mlp(const lora_mlp_desc_t* d) {
  if (!d) return fail(LORA_ERR_NULL, "desc is NULL");
  if (d->n_tokens < 0 || d->hidden <= 0 || d->inter <= 0 || d->rank <= 0)
    return fail(LORA_ERR_SHAPE, "sizes must be positive, n_tokens >= 0 (n_tokens=%lld hidden=%d inter=%d rank=%d)",
                (long long)d->n_tokens, d->hidden, d->inter, d->rank);
  if (d->reserved != 0) return fail(LORA_ERR_SHAPE, "reserved field must be 0");
  if (d->dtype != LORA_F32 && d->dtype != LORA_BF16) return fail(LORA_ERR_UNSUPPORTED, "unsupported dtype %d", d->dtype);
  if (d->act != LORA_SWIGLU && d->act != LORA_GEGLU_TANH && d->act != LORA_GEGLU_ERF)
    return fail(LORA_ERR_UNSUPPORTED, "unsupported activation %d", d->act);
  if (d->rank > LORA_MAX_RANK) return fail(LORA_ERR_UNSUPPORTED, "rank %d above LORA_MAX_RANK", d->rank);
  if (d->n_tokens > (1L << 30) || (long)d->hidden * d->inter > (1L << 31))
    return fail(LORA_ERR_UNSUPPORTED, "sizes beyond the 32-bit tile index range");
  return LORA_OK;
}
int check_proj(const lora_proj_t* p, const char* name) {
  if (!p || !p->W || !p->A || !p->B) return fail(LORA_ERR_NULL, "projection %s has a NULL pointer", name);
  return LORA_OK;
}
int check_proj_nobias(const lora_proj_t* p, const char* name) {
  const int rc = check_proj(p, name);
  if (rc) return rc;
  if (p->bias) return fail(LORA_ERR_UNSUPPORTED, "projection %s has a bias; the fused MLP is bias-free", name);
  return LORA_OK;
}
int check_qkv(const lora_qkv_desc_t* d) {
  if (!d) return fail(LORA_ERR_NULL, "desc is NULL");
  if (d->batch < 0 || d->seq <= 0 || d->hidden <= 0 || d->n_q <= 0 || d->n_kv <= 0 || d->head_dim <= 0 ||
      d->rank <= 0)
    return fail(LORA_ERR_SHAPE, "sizes must be positive");
  if (d->head_dim % 2) return fail(LORA_ERR_SHAPE, "head_dim %d is odd", d->head_dim);
  if (d->n_q % d->n_kv) return fail(LORA_ERR_SHAPE, "n_q %% n_kv != 0 (%d, %d)", d->n_q, d->n_kv);
  if (!(d->rope_theta > 0.0)) return fail(LORA_ERR_SHAPE, "rope_theta must be > 0");
  if (d->dtype != LORA_F32 && d->dtype != LORA_BF16) return fail(LORA_ERR_UNSUPPORTED, "unsupported dtype %d", d->dtype);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(LORA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", d->head_dim);
  if (d->rank > LORA_MAX_RANK) return fail(LORA_ERR_UNSUPPORTED, "rank %d above LORA_MAX_RANK", d->rank);
  if ((long)d->batch * d->seq > (1L << 30)) return fail(LORA_ERR_UNSUPPORTED, "too many tokens");
  return LORA_OK;
}

int check_linear(const lora_linear_desc_t* d) {
  if (!d) return fail(LORA_ERR_NULL, "desc is NULL");
  if (d->n_tokens < 0 || d->in_features <= 0 || d->out_features <= 0 || d->rank <= 0)
    return fail(LORA_ERR_SHAPE, "sizes must be positive, n_tokens >= 0 (n_tokens=%lld in=%d out=%d rank=%d)",
                (long long)d->n_tokens, d->in_features, d->out_features, d->rank);
  if (d->dtype != LORA_F32 && d->dtype != LORA_BF16) return fail(LORA_ERR_UNSUPPORTED, "unsupported dtype %d", d->dtype);
  if (d->rank > LORA_MAX_RANK) return fail(LORA_ERR_UNSUPPORTED, "rank %d above LORA_MAX_RANK", d->rank);
  if (d->n_tokens > (1L << 30) || (long)d->in_features * d->out_features > (1L << 31))
    return fail(LORA_ERR_UNSUPPORTED, "sizes beyond the 32-bit tile index range");
  return LORA_OK;
}

template <class T>
struct DT;
template <>
struct DT<float> {
  static constexpr int code = LORA_F32;
};
template <>
struct DT<bf16> {
  static constexpr int code = LORA_BF16;
};

// ---- MLP ----------------------------------------------------------------------
template <class T, int ACT>
int mlp_fwd_impl(const lora_mlp_desc_t& d, const void* X, const lora_proj_t& g, const lora_proj_t& u,
                 const lora_proj_t& dn, void* Y, void* G, void* U, void* Tsv, const MlpWs& w, hipStream_t st) {
  const long N = d.n_tokens;
  if (N == 0) return ok();                         // empty batch: nothing to compute
  const int h = d.hidden, i = d.inter, r = d.rank, V = vecw(DT<T>::code);
  const int R = (int)cdiv(N, kBM);
  float* T3 = static_cast<float*>(Tsv);
  {
    GateUpArgs a{};
    a.X = X; a.Wg = g.W; a.Ag = g.A; a.Bg = g.B; a.Wu = u.W; a.Au = u.A; a.Bu = u.B;
    a.sg = g.scale; a.su = u.scale;
    a.G = G; a.U = U; a.H = w.H;
    a.Tg = T3; a.Tu = T3 + N * r;
    a.N = N; a.h = h; a.i = i; a.r = r;
    a.vecA = (h % V == 0) && al16(X);
    a.vecW = (h % V == 0) && al16(g.W) && al16(u.W);
    a.vecS = (h % V == 0) && al16(g.A) && al16(u.A);
    a.vecO = (i % 4 == 0) && al16(G) && al16(U) && al16(w.H);
    a.R = R; a.NC = (int)cdiv(i, 128);
    const bool fast = fast_ok(DT<T>::code, h, N, {X, g.W, u.W, g.A, u.A}) && h % 64 == 0;
    run_layout(a.R, a.NC, a.L, a.RPB, a.nruns);
    const dim3 grid(fast && sizeof(T) == 2 ? a.nruns : a.R * a.NC);
    const int rc = grid.x == 0 ? LORA_OK
                               : launch_call(0, st, [&]() { return launch_gateup<T, ACT>(fast, a, grid, st); });
    if (rc) return rc;
  }
  {
    LinearArgs a{};
    a.Z = w.H; a.W = dn.W; a.A = dn.A; a.B = dn.B; a.s = dn.scale;
    a.Y = Y; a.T = T3 + 2 * N * r;
    a.N = N; a.K = i; a.O = h; a.r = r;
    a.vecA = (i % V == 0) && al16(w.H);
    a.vecW = (i % V == 0) && al16(dn.W);
    a.vecS = (i % V == 0) && al16(dn.A);
    a.vecO = (h % 8 == 0) && al16(Y);
    a.R = R; a.NC = (int)cdiv(h, kBN);
    const bool fast = fast_ok(DT<T>::code, i, N, {w.H, dn.W, dn.A}) && i % 64 == 0;
    a.sk.S = 1;
    if (sizeof(T) == 2 && fast) split_setup(w.split, a.sk);
    const int rc = launch_call(1, st, [&]() { return launch_linear_fwd_passes<T>(fast, a, st); });
    if (rc) return rc;
  }
  return ok();
}

// The backward prologue with raw buffer loads (bf16, aligned rows, whole
// 16-byte chunks of B rows (r % 8 == 0), every source it reads at most 2 GB,
// so one 32-bit offset past the end reads zero).
template <class T>
int launch_prologue(const ProArgs& a, dim3 grid, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    const long lim = 1L << 31;
    bool buf = a.vecP != 0 && a.vecB != 0;
    if (a.qkv) {
      for (int p = 0; p < 3; ++p) buf = buf && a.N * a.nh[p] * (long)a.d * 2 <= lim;
    } else {
      buf = buf && a.N * (long)a.O * 2 <= lim;
    }
    if (buf) {
      if (a.qkv) return launch(4, k_bwd_prologue8<T>, grid, dim3(512), st, a);
      return launch(12, k_bwd_prologue_ring<T, 3>, grid, dim3(512), st, a);
    }
  }
  return launch(4, k_bwd_prologue<T>, grid, dim3(kThreads), st, a);
}

template <class T, int ACT>
int mlp_bwd_impl(const lora_mlp_desc_t& d, const void* dY, const void* X, const void* G, const void* U,
                 const void* Tsv, const lora_proj_t& g, const lora_proj_t& u, const lora_proj_t& dn, void* dX,
                 void* dAg, void* dBg, void* dAu, void* dBu, void* dAd, void* dBd, const MlpWs& w, hipStream_t st) {
  const long N = d.n_tokens;
  const int h = d.hidden, i = d.inter, r = d.rank, V = vecw(DT<T>::code);
  const int R = (int)cdiv(N, kBM);
  const float* T3 = static_cast<const float*>(Tsv);
  // No tokens: the adapter gradients are empty sums; only the reduction
  // runs (over zero row blocks), writing zeros.
  if (N > 0) {
    {
      ProArgs a{};
      a.qkv = 0;
      a.P = dY;
      a.Bp[0] = dn.B; a.Tp[0] = T3 + 2 * N * r; a.s[0] = dn.scale;
      a.off[0] = 0; a.off[1] = h; a.off[2] = h; a.off[3] = h;
      a.nadp = 1;
      a.dT_part = w.dT_part; a.dB_part = w.pB_d;
      a.N = N; a.O = h; a.r = r;
      a.NCH = w.NCH; a.CPC = w.CPC; a.NCR = w.NCR;
      a.vecP = (h % V == 0) && al16(dY);
      a.vecB = (r % V == 0) && al16(dn.B);
      int rc = launch_prologue<T>(a, dim3(R, w.NCR), st);
      if (rc) return rc;
      rc = launch(9, k_dt_sum, dim3((unsigned)cdiv(N * 4, 256), 1), dim3(256), st, (const float*)w.dT_part, w.dT,
                  w.NCR, N);
      if (rc) return rc;
    }
    {
      DownBwdArgs a{};
      a.dY = dY; a.Wd = dn.W; a.Ad = dn.A; a.G = G; a.U = U;
      a.Tg = T3; a.Tu = T3 + N * r;
      a.dT = w.dT;
      a.sg = g.scale; a.su = u.scale;
      a.dG = w.dG; a.dU = w.dU;
      a.pA_d = w.pA_d; a.pB_g = w.pB_g; a.pB_u = w.pB_u;
      a.N = N; a.h = h; a.i = i; a.r = r;
      a.vecA = (h % V == 0) && al16(dY);
      a.vecW = (i % V == 0) && al16(dn.W);
      a.vecO = (i % 8 == 0) && al16(G) && al16(U) && al16(w.dG) && al16(w.dU);
      a.R = R; a.NC = (int)cdiv(i, kBN);
      const bool fast = fast_ok(DT<T>::code, h, N, {dY, dn.W}) && i % 8 == 0 && h % 64 == 0;
      // Whole tiles only: the GLU backward stages G, U through LDS (no masks).
      const bool full = fast && a.vecO && N % kBM == 0 && i % kBN == 0 && N * (long)i < (1L << 31);
      int rc;
      if constexpr (sizeof(T) == 2) {
        if (full) {
          rc = launch(5, k_down_bwd<T, ACT, true, true>, dim3(a.R * a.NC), dim3(kGemmThreads), st, a);
          if (rc) return rc;
        }
      }
      if (!full)
        rc = LORA_LAUNCH_FAST(5, fast, (k_down_bwd<T, ACT, true>), (k_down_bwd<T, ACT, false>),
                              dim3(a.R * a.NC), dim3(kGemmThreads), st, a);
      if (rc) return rc;
    }
    {
      MlpDxArgs a{};
      a.dG = w.dG; a.dU = w.dU; a.Wg = g.W; a.Wu = u.W; a.Bg = g.B; a.Bu = u.B; a.Ag = g.A; a.Au = u.A;
      a.X = X; a.sg = g.scale; a.su = u.scale;
      a.dX = dX; a.pA_g = w.pA_g; a.pA_u = w.pA_u;
      a.N = N; a.h = h; a.i = i; a.r = r;
      a.vecA = (i % V == 0) && al16(w.dG) && al16(w.dU);
      a.vecW = (h % V == 0) && al16(g.W) && al16(u.W);
      a.vecS = (r % V == 0) && al16(g.B) && al16(u.B);
      a.vecO = (h % 8 == 0) && al16(dX) && al16(X);
      a.R = R; a.NC = (int)cdiv(h, kBN);
      const bool fast = fast_ok(DT<T>::code, i, N, {w.dG, w.dU, g.W, u.W, g.B, u.B}) && h % 8 == 0 && r == 16 &&
                        i % 64 == 0 && x_buf_ok(a.vecO, N, h);
      a.sk.S = 1;
      if (sizeof(T) == 2 && fast) split_setup(w.split, a.sk);
      int rc = LORA_OK;
      bool done = false;
      if constexpr (sizeof(T) == 2) {
        if (a.sk.S > 1) {                          // set only on the bf16 fast path
          rc = launch_call(6, st, [&]() { return launch_mlp_dx_split_bf16(a, st); });
          done = true;
        } else if (fast) {
          // dT_g, dT_u by a streaming pass of their own, then the dX GEMM
          // without side work.
          MlpDtArgs t{};
          t.dG = w.dG; t.dU = w.dU; t.Bg = g.B; t.Bu = u.B;
          t.part = w.dT_part;
          t.N = N; t.i = i; t.KS = w.KS;
          rc = launch(11, k_mlp_dt<T>, dim3(R, w.KS), dim3(kGemmThreads), st, t);
          if (rc) return rc;
          rc = launch(9, k_dt_sum, dim3((unsigned)cdiv(N * 4, 256), 2), dim3(256), st, (const float*)w.dT_part, w.dT,
                      w.KS, N);
          if (rc) return rc;
          a.dT = w.dT;
          rc = launch(6, k_mlp_dx_pp<T>, dim3(a.R * a.NC), dim3(kGemmThreads), st, a);
          done = true;
        }
      }
      if (!done)
        rc = LORA_LAUNCH_FAST(6, fast, (k_mlp_dx_bwd<T, true>), (k_mlp_dx_bwd<T, false>), dim3(a.R * a.NC),
                              dim3(kGemmThreads), st, a);
      if (rc) return rc;
    }
  }
  {
    RedArgs a{};
    a.r = r;
    a.njobs = 6;
    const long si = (long)i * 16, sh = (long)h * 16;
    a.job[0] = RedJob{w.pA_d, si, si, R, i, 1, dAd};
    a.job[1] = RedJob{w.pB_g, si, si, R, i, 0, dBg};
    a.job[2] = RedJob{w.pB_u, si, si, R, i, 0, dBu};
    a.job[3] = RedJob{w.pA_g, sh, sh, R, h, 1, dAg};
    a.job[4] = RedJob{w.pA_u, sh, sh, R, h, 1, dAu};
    a.job[5] = RedJob{w.pB_d, sh, sh, R, h, 0, dBd};
    const long mx = si > sh ? si : sh;
    const int rc = launch(8, k_reduce<T>, dim3((unsigned)cdiv(mx, 256), 6), dim3(256), st, a);
    if (rc) return rc;
  }
  return ok();
}

// ---- QKV -----------------------------------------------------------------------
void qkv_offsets(const lora_qkv_desc_t& d, int (&off)[4], int (&nh)[3]) {
  nh[0] = d.n_q; nh[1] = d.n_kv; nh[2] = d.n_kv;
  off[0] = 0;
  off[1] = d.n_q * d.head_dim;
  off[2] = off[1] + d.n_kv * d.head_dim;
  off[3] = off[2] + d.n_kv * d.head_dim;
}

int rope_table(const lora_qkv_desc_t& d, const QkvWs& w, hipStream_t st) {
  const long n = (long)d.seq * (d.head_dim / 2);
  return launch(2, k_rope_table, dim3((unsigned)cdiv(n, 256)), dim3(256), st, w.cs, w.sn, d.seq, d.head_dim / 2,
                d.rope_theta);
}

// q/k norm: the weights and what the forward saves for the backward.
struct NormIo {
  const void* w[2];
  float eps;
  void* Pn;        // [N][Oq + Ok], call dtype
  float* rinv;     // [N][n_q + n_kv]
};

template <class T>
int qkv_fwd_impl(const lora_qkv_desc_t& d, const void* X, const lora_proj_t* const (&pr)[3], void* const (&out)[3],
                 void* Tsv, const QkvWs& w, hipStream_t st, const NormIo* nio = nullptr) {
  const long N = (long)d.batch * d.seq;
  if (N == 0) return ok();
  const int h = d.hidden, r = d.rank, V = vecw(DT<T>::code);
  int rc = rope_table(d, w, st);
  if (rc) return rc;
  QKVFwdArgs a{};
  a.X = X;
  bool wal = true, aal = true, oal = true;
  for (int p = 0; p < 3; ++p) {
    a.W[p] = pr[p]->W; a.A[p] = pr[p]->A; a.B[p] = pr[p]->B; a.s[p] = pr[p]->scale; a.bias[p] = pr[p]->bias;
    a.out[p] = out[p];
    a.T[p] = static_cast<float*>(Tsv) + p * N * r;
    wal = wal && al16(pr[p]->W);
    aal = aal && al16(pr[p]->A);
    oal = oal && al16(out[p]);
  }
  a.cs = w.cs; a.sn = w.sn;
  a.N = N; a.h = h; a.S = d.seq; a.d = d.head_dim; a.r = r;
  qkv_offsets(d, a.off, a.nh);
  a.vecA = (h % V == 0) && al16(X);
  a.vecW = (h % V == 0) && wal;
  a.vecS = (h % V == 0) && aal;
  a.vecO = oal;
  if (nio) {
    a.norm = 1;
    a.nw[0] = nio->w[0]; a.nw[1] = nio->w[1];
    a.eps = nio->eps;
    a.Pn = nio->Pn; a.rinv = nio->rinv;
    a.vecN = al16(nio->Pn);
  }
  a.R = (int)cdiv(N, kBM);
  a.NC = (int)cdiv(a.off[3], kBN);
  const bool fast = fast_ok(DT<T>::code, h, N, {X, pr[0]->W, pr[1]->W, pr[2]->W, pr[0]->A, pr[1]->A, pr[2]->A}) &&
                    h % 64 == 0;
  // Most projections any 256-column tile overlaps: 1, 2 or 3 side blocks.
  int ns = 1;
  for (int cb = 0; cb < a.NC; ++cb) {
    int c = 0;
    for (int p = 0; p < 3; ++p)
      if (a.off[p] < std::min((cb + 1) * kBN, a.off[3]) && a.off[p + 1] > cb * kBN) ++c;
    ns = std::max(ns, c);
  }
  if constexpr (sizeof(T) == 2) {
    // Runs of column tiles (head_dim 128, more tiles than CUs, every run
    // over at most two projections).
    run_layout(a.R, a.NC, a.L, a.RPB, a.nruns);
    bool runs = fast && d.head_dim == 128 && a.L > 1;
    for (int u = 0; runs && u < a.RPB; ++u) {
      const int lo = u * a.L * kBN, hi = std::min((u + 1) * a.L * kBN, a.off[3]);
      int c = 0;
      for (int p = 0; p < 3; ++p)
        if (a.off[p] < hi && a.off[p + 1] > lo) ++c;
      runs = c <= 2;
    }
    if (runs) {
      rc = launch_call(3, st, [&]() { return launch_qkv_run_bf16(a, st); });
      if (rc) return rc;
      return ok();
    }
  }
  const dim3 grid(a.R * a.NC);
  rc = launch_call(3, st, [&]() { return launch_qkv_fwd<T>(fast, d.head_dim, ns, a, grid, st); });
  if (rc) return rc;
  return ok();
}

template <class T>
int qkv_bwd_impl(const lora_qkv_desc_t& d, const void* const (&dO)[3], const void* X, const void* Tsv,
                 const lora_proj_t* const (&pr)[3], void* dX, void* const (&dA)[3], void* const (&dB)[3],
                 const QkvWs& w, hipStream_t st, const NormIo* nio = nullptr) {
  const long N = (long)d.batch * d.seq;
  const int h = d.hidden, r = d.rank, V = vecw(DT<T>::code);
  const int R = (int)cdiv(N, kBM);
  int off[4], nh[3];
  qkv_offsets(d, off, nh);
  const int O = off[3];
  // No tokens: the adapter gradients are empty sums; only the reduction
  // runs (over zero row blocks), writing zeros.
  if (N > 0) {
    int rc = rope_table(d, w, st);
    if (rc) return rc;
    if (nio) {
      // dP through RoPE^T and the per-head norm, then the prologue reads it as a
      // plain token-major upstream gradient over the three adapters.
      NormBwdArgs a{};
      for (int p = 0; p < 3; ++p) { a.src[p] = dO[p]; a.nh[p] = nh[p]; }
      a.Pn = nio->Pn; a.rinv = nio->rinv;
      a.nw[0] = nio->w[0]; a.nw[1] = nio->w[1];
      a.cs = w.cs; a.sn = w.sn;
      a.dP = w.dP;
      a.N = N; a.S = d.seq; a.d = d.head_dim;
      for (int k = 0; k < 4; ++k) a.off[k] = off[k];
      constexpr int E = ET<T>::VEC;
      const int tph = d.head_dim / 2 / E;
      const dim3 blk(256);
      const unsigned gy = (unsigned)(nh[0] + nh[1] + nh[2]);
      if (tph == 4) rc = launch(10, k_qk_norm_bwd<T, 4>, dim3((unsigned)cdiv(N, 64), gy), blk, st, a);
      else if (tph == 8) rc = launch(10, k_qk_norm_bwd<T, 8>, dim3((unsigned)cdiv(N, 32), gy), blk, st, a);
      else rc = launch(10, k_qk_norm_bwd<T, 16>, dim3((unsigned)cdiv(N, 16), gy), blk, st, a);
      if (rc) return rc;
    }
    {
      ProArgs a{};
      a.qkv = nio ? 0 : 1;
      a.P = w.dP;
      bool sal = true, bal = true;
      for (int p = 0; p < 3; ++p) {
        a.src[p] = dO[p];
        a.nh[p] = nh[p];
        a.Bp[p] = pr[p]->B;
        a.Tp[p] = static_cast<const float*>(Tsv) + p * N * r;
        a.s[p] = pr[p]->scale;
        sal = sal && al16(dO[p]);
        bal = bal && al16(pr[p]->B);
      }
      a.cs = w.cs; a.sn = w.sn; a.S = d.seq; a.d = d.head_dim;
      a.dP = w.dP;
      for (int k = 0; k < 4; ++k) a.off[k] = off[k];
      a.nadp = 3;
      a.dT_part = w.dT_part; a.dB_part = w.dB_part;
      a.N = N; a.O = O; a.r = r;
      a.NCH = w.NCH; a.CPC = w.CPC; a.NCR = w.NCR;
      a.vecP = nio ? true : sal;
      a.vecB = (r % V == 0) && bal;
      rc = launch_prologue<T>(a, dim3(R, w.NCR), st);
      if (rc) return rc;
      rc = launch(9, k_dt_sum, dim3((unsigned)cdiv(N * 4, 256), 3), dim3(256), st, (const float*)w.dT_part, w.dT,
                  w.NCR, N);
      if (rc) return rc;
    }
    {
      ProjDxArgs a{};
      a.dP = w.dP;
      bool wal = true;
      for (int p = 0; p < 3; ++p) {
        a.W[p] = pr[p]->W; a.A[p] = pr[p]->A; a.pA[p] = w.pA[p];
        wal = wal && al16(pr[p]->W);
      }
      a.dT = w.dT;
      a.X = X; a.dX = dX;
      a.N = N; a.h = h; a.O = O; a.r = r;
      for (int k = 0; k < 4; ++k) a.off[k] = off[k];
      a.vecA = (O % V == 0);
      a.vecW = (h % V == 0) && wal;
      a.vecO = (h % 8 == 0) && al16(dX) && al16(X);
      a.R = R; a.NC = (int)cdiv(h, kBN);
      const bool fast = fast_ok(DT<T>::code, O, N, {w.dP, pr[0]->W, pr[1]->W, pr[2]->W}) && h % 8 == 0 &&
                        O % 64 == 0 && x_buf_ok(a.vecO, N, h);
      rc = LORA_LAUNCH_FAST(7, fast, (k_proj_dx_bwd<T, true, 3>), (k_proj_dx_bwd<T, false, 3>), dim3(a.R * a.NC),
                            dim3(kGemmThreads), st, a);
      if (rc) return rc;
    }
  }
  {
    RedArgs a{};
    a.r = r;
    a.njobs = 6;
    const long sh = (long)h * 16, so = (long)O * 16;
    long mx = sh;
    for (int p = 0; p < 3; ++p) {
      a.job[p] = RedJob{w.pA[p], sh, sh, R, h, 1, dA[p]};
      const long cnt = (long)(off[p + 1] - off[p]) * 16;
      a.job[3 + p] = RedJob{w.dB_part + (long)off[p] * 16, so, cnt, R, off[p + 1] - off[p], 0, dB[p]};
      if (cnt > mx) mx = cnt;
    }
    const int rc = launch(8, k_reduce<T>, dim3((unsigned)cdiv(mx, 256), 6), dim3(256), st, a);
    if (rc) return rc;
  }
  return ok();
}

// ---- LoRA linear ----------------------------------------------------------------
template <class T>
int linear_fwd_impl(const lora_linear_desc_t& d, const void* X, const lora_proj_t& p, void* Y, void* Tsv,
                    const LinWs& w, hipStream_t st) {
  const long N = d.n_tokens;
  if (N == 0) return ok();
  const int in = d.in_features, out = d.out_features, r = d.rank, V = vecw(DT<T>::code);
  LinearArgs a{};
  a.Z = X; a.W = p.W; a.A = p.A; a.B = p.B; a.bias = p.bias; a.s = p.scale;
  a.Y = Y; a.T = static_cast<float*>(Tsv);
  a.N = N; a.K = in; a.O = out; a.r = r;
  a.vecA = (in % V == 0) && al16(X);
  a.vecW = (in % V == 0) && al16(p.W);
  a.vecS = (in % V == 0) && al16(p.A);
  a.vecO = (out % 8 == 0) && al16(Y);
  a.R = (int)cdiv(N, kBM); a.NC = (int)cdiv(out, kBN);
  const bool fast = fast_ok(DT<T>::code, in, N, {X, p.W, p.A}) && in % 64 == 0;
  a.sk.S = 1;
  if (sizeof(T) == 2 && fast) split_setup(w.split, a.sk);
  const int rc = launch_call(1, st, [&]() { return launch_linear_fwd_passes<T>(fast, a, st); });
  if (rc) return rc;
  return ok();
}

template <class T>
int linear_bwd_impl(const lora_linear_desc_t& d, const void* dY, const void* X, const void* Tsv,
                    const lora_proj_t& p, void* dX, void* dA, void* dB, const LinWs& w, hipStream_t st) {
  const long N = d.n_tokens;
  const int in = d.in_features, out = d.out_features, r = d.rank, V = vecw(DT<T>::code);
  const int R = (int)cdiv(N, kBM);
  // No tokens: the adapter gradients are empty sums; only the reduction
  // runs (over zero row blocks), writing zeros.
  if (N > 0) {
    {
      ProArgs a{};
      a.qkv = 0;
      a.P = dY;
      a.Bp[0] = p.B; a.Tp[0] = static_cast<const float*>(Tsv); a.s[0] = p.scale;
      a.off[0] = 0; a.off[1] = out; a.off[2] = out; a.off[3] = out;
      a.nadp = 1;
      a.dT_part = w.dT_part; a.dB_part = w.dB_part;
      a.N = N; a.O = out; a.r = r;
      a.NCH = w.NCH; a.CPC = w.CPC; a.NCR = w.NCR;
      a.vecP = (out % V == 0) && al16(dY);
      a.vecB = (r % V == 0) && al16(p.B);
      int rc = launch_prologue<T>(a, dim3(R, w.NCR), st);
      if (rc) return rc;
      rc = launch(9, k_dt_sum, dim3((unsigned)cdiv(N * 4, 256), 1), dim3(256), st, (const float*)w.dT_part, w.dT,
                  w.NCR, N);
      if (rc) return rc;
    }
    {
      ProjDxArgs a{};
      a.dP = dY;
      a.W[0] = a.W[1] = a.W[2] = p.W;
      a.A[0] = a.A[1] = a.A[2] = p.A;
      a.pA[0] = a.pA[1] = a.pA[2] = w.pA;
      a.dT = w.dT;
      a.X = X; a.dX = dX;
      a.N = N; a.h = in; a.O = out; a.r = r;
      a.off[0] = 0; a.off[1] = out; a.off[2] = out; a.off[3] = out;
      a.vecA = (out % V == 0) && al16(dY);
      a.vecW = (in % V == 0) && al16(p.W);
      a.vecO = (in % 8 == 0) && al16(dX) && al16(X);
      a.R = R; a.NC = (int)cdiv(in, kBN);
      const bool fast = fast_ok(DT<T>::code, out, N, {dY, p.W}) && in % 8 == 0 && out % 64 == 0 &&
                        x_buf_ok(a.vecO, N, in);
      const int rc = LORA_LAUNCH_FAST(7, fast, (k_proj_dx_bwd<T, true, 1>), (k_proj_dx_bwd<T, false, 1>),
                                      dim3(a.R * a.NC), dim3(kGemmThreads), st, a);
      if (rc) return rc;
    }
  }
  {
    RedArgs a{};
    a.r = r;
    a.njobs = 2;
    const long si = (long)in * 16, so = (long)out * 16;
    a.job[0] = RedJob{w.pA, si, si, R, in, 1, dA};
    a.job[1] = RedJob{w.dB_part, so, so, R, out, 0, dB};
    const int rc = launch(8, k_reduce<T>, dim3((unsigned)cdiv(si > so ? si : so, 256), 2), dim3(256), st, a);
    if (rc) return rc;
  }
  return ok();
}

}  // namespace

// =============================================================================
// C ABI
// =============================================================================
namespace {
int check_norm(const lora_qkv_desc_t* desc, const lora_qk_norm_t* norm, const void* Pn, const float* rinv,
               std::initializer_list<const void*> vec_ptrs, NormIo& nio) {
  if (!norm || !norm->q_weight || !norm->k_weight || (desc->batch > 0 && (!Pn || !rinv)))
    return fail(LORA_ERR_NULL, "q/k norm weights, Pn or rinv is NULL");
  if (!(norm->eps >= 0.f)) return fail(LORA_ERR_SHAPE, "norm eps must be >= 0");
  for (const void* p : vec_ptrs)
    if (!al16(p)) return fail(LORA_ERR_UNSUPPORTED, "the q/k norm path needs 16-byte aligned tensors");
  nio.w[0] = norm->q_weight; nio.w[1] = norm->k_weight;
  nio.eps = norm->eps;
  nio.Pn = const_cast<void*>(Pn);
  nio.rinv = const_cast<float*>(rinv);
  return LORA_OK;
}
}  // namespace

// ---- allocation-free variant: a file-scope device scratch array -------------
// Callers that cannot allocate (code under graph capture, tight serving loops)
// use lora_qkv_fwd_noalloc, which keeps its scratch (the RoPE cos / sin table)
// in this array instead of a workspace argument.  Each GPU the library runs on
// holds its own copy until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: only the address hipGetSymbolAddress
// returns for the current device is ever handed to a kernel.
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_dev[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up once per device.
int scratch_for_current_device(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(LORA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(LORA_ERR_HIP, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(LORA_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_dev[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_dev[dev];
  return LORA_OK;
}
}  // namespace

extern "C" {

size_t lora_mlp_workspace_bytes(const lora_mlp_desc_t* desc, int pass) {
  if (check_mlp(desc) != LORA_OK || (pass != 0 && pass != 1)) return 0;
  return mlp_ws(*desc, pass, nullptr).bytes;
}

size_t lora_qkv_workspace_bytes(const lora_qkv_desc_t* desc, int pass) {
  if (check_qkv(desc) != LORA_OK || (pass != 0 && pass != 1)) return 0;
  return qkv_ws(*desc, pass, nullptr).bytes;
}

size_t lora_linear_workspace_bytes(const lora_linear_desc_t* desc, int pass) {
  if (check_linear(desc) != LORA_OK || (pass != 0 && pass != 1)) return 0;
  return lin_ws(*desc, pass, nullptr).bytes;
}

int lora_mlp_fwd(const lora_mlp_desc_t* desc, const void* X, const lora_proj_t* gate, const lora_proj_t* up,
                 const lora_proj_t* down, void* Y, void* G, void* U, void* T, void* workspace,
                 size_t workspace_bytes, void* hip_stream) {
  int rc = check_mlp(desc);
  if (rc) return rc;
  if ((rc = check_proj_nobias(gate, "gate")) || (rc = check_proj_nobias(up, "up")) ||
      (rc = check_proj_nobias(down, "down")))
    return rc;
  if (desc->n_tokens > 0 && (!X || !Y || !G || !U || !T)) return fail(LORA_ERR_NULL, "a tensor pointer is NULL");
  const MlpWs probe = mlp_ws(*desc, 0, nullptr);
  if (probe.bytes > 0 && (!workspace || workspace_bytes < probe.bytes))
    return fail(LORA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, probe.bytes);
  const MlpWs w = mlp_ws(*desc, 0, workspace);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
#define LORA_MLP_FWD(TT, AA) return mlp_fwd_impl<TT, AA>(*desc, X, *gate, *up, *down, Y, G, U, T, w, st)
  if (desc->dtype == LORA_BF16) {
    if (desc->act == LORA_SWIGLU) LORA_MLP_FWD(bf16, LORA_ACT_SWIGLU);
    if (desc->act == LORA_GEGLU_TANH) LORA_MLP_FWD(bf16, LORA_ACT_GEGLU_TANH);
    LORA_MLP_FWD(bf16, LORA_ACT_GEGLU_ERF);
  }
  if (desc->act == LORA_SWIGLU) LORA_MLP_FWD(float, LORA_ACT_SWIGLU);
  if (desc->act == LORA_GEGLU_TANH) LORA_MLP_FWD(float, LORA_ACT_GEGLU_TANH);
  LORA_MLP_FWD(float, LORA_ACT_GEGLU_ERF);
#undef LORA_MLP_FWD
}

int lora_mlp_bwd(const lora_mlp_desc_t* desc, const void* dY, const void* X, const void* G, const void* U,
                 const void* T, const lora_proj_t* gate, const lora_proj_t* up, const lora_proj_t* down, void* dX,
                 void* dA_gate, void* dB_gate, void* dA_up, void* dB_up, void* dA_down, void* dB_down,
                 void* workspace, size_t workspace_bytes, void* hip_stream) {
  int rc = check_mlp(desc);
  if (rc) return rc;
  if ((rc = check_proj_nobias(gate, "gate")) || (rc = check_proj_nobias(up, "up")) ||
      (rc = check_proj_nobias(down, "down")))
    return rc;
  if (!dA_gate || !dB_gate || !dA_up || !dB_up || !dA_down || !dB_down ||
      (desc->n_tokens > 0 && (!dY || !X || !G || !U || !T || !dX)))
    return fail(LORA_ERR_NULL, "a tensor pointer is NULL");
  const MlpWs probe = mlp_ws(*desc, 1, nullptr);
  if (probe.bytes > 0 && (!workspace || workspace_bytes < probe.bytes))
    return fail(LORA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, probe.bytes);
  const MlpWs w = mlp_ws(*desc, 1, workspace);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
#define LORA_MLP_BWD(TT, AA)                                                                                    \
  return mlp_bwd_impl<TT, AA>(*desc, dY, X, G, U, T, *gate, *up, *down, dX, dA_gate, dB_gate, dA_up, dB_up, \
                              dA_down, dB_down, w, st)
  if (desc->dtype == LORA_BF16) {
    if (desc->act == LORA_SWIGLU) LORA_MLP_BWD(bf16, LORA_ACT_SWIGLU);
    if (desc->act == LORA_GEGLU_TANH) LORA_MLP_BWD(bf16, LORA_ACT_GEGLU_TANH);
    LORA_MLP_BWD(bf16, LORA_ACT_GEGLU_ERF);
  }
  if (desc->act == LORA_SWIGLU) LORA_MLP_BWD(float, LORA_ACT_SWIGLU);
  if (desc->act == LORA_GEGLU_TANH) LORA_MLP_BWD(float, LORA_ACT_GEGLU_TANH);
  LORA_MLP_BWD(float, LORA_ACT_GEGLU_ERF);
#undef LORA_MLP_BWD
}

int lora_qkv_fwd(const lora_qkv_desc_t* desc, const void* X, const lora_proj_t* q, const lora_proj_t* k,
                 const lora_proj_t* v, void* Q, void* K, void* V, void* T, void* workspace, size_t workspace_bytes,
                 void* hip_stream) {
  int rc = check_qkv(desc);
  if (rc) return rc;
  if ((rc = check_proj(q, "q")) || (rc = check_proj(k, "k")) || (rc = check_proj(v, "v"))) return rc;
  if (desc->batch > 0 && (!X || !Q || !K || !V || !T)) return fail(LORA_ERR_NULL, "a tensor pointer is NULL");
  const QkvWs probe = qkv_ws(*desc, 0, nullptr);
  if (probe.bytes > 0 && (!workspace || workspace_bytes < probe.bytes))
    return fail(LORA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, probe.bytes);
  const QkvWs w = qkv_ws(*desc, 0, workspace);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const lora_proj_t* const pr[3] = {q, k, v};
  void* const out[3] = {Q, K, V};
  if (desc->dtype == LORA_BF16) return qkv_fwd_impl<bf16>(*desc, X, pr, out, T, w, st);
  return qkv_fwd_impl<float>(*desc, X, pr, out, T, w, st);
}

size_t lora_qkv_fwd_noalloc_max_scratch_bytes(void) { return kNoAllocScratchBytes; }

int lora_qkv_fwd_noalloc(const lora_qkv_desc_t* desc, const void* X, const lora_proj_t* q, const lora_proj_t* k,
                         const lora_proj_t* v, void* Q, void* K, void* V, void* T, void* hip_stream) {
  int rc = check_qkv(desc);
  if (rc) return rc;
  if ((rc = check_proj(q, "q")) || (rc = check_proj(k, "k")) || (rc = check_proj(v, "v"))) return rc;
  if (desc->batch > 0 && (!X || !Q || !K || !V || !T)) return fail(LORA_ERR_NULL, "a tensor pointer is NULL");
  const QkvWs probe = qkv_ws(*desc, 0, nullptr);
  if (probe.bytes > kNoAllocScratchBytes)
    return fail(LORA_ERR_WORKSPACE,
                "the allocation-free QKV forward needs %zu bytes of scratch (RoPE table of seq %d x head_dim %d), "
                "its static buffer holds %zu: use lora_qkv_fwd with a workspace",
                probe.bytes, desc->seq, desc->head_dim, kNoAllocScratchBytes);
  if (desc->batch == 0) return ok();                 // nothing to compute, no device call
  char* base = nullptr;
  if ((rc = scratch_for_current_device(&base))) return rc;
  const QkvWs w = qkv_ws(*desc, 0, base);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const lora_proj_t* const pr[3] = {q, k, v};
  void* const out[3] = {Q, K, V};
  if (desc->dtype == LORA_BF16) return qkv_fwd_impl<bf16>(*desc, X, pr, out, T, w, st);
  return qkv_fwd_impl<float>(*desc, X, pr, out, T, w, st);
}

int lora_qkv_bwd(const lora_qkv_desc_t* desc, const void* dQ, const void* dK, const void* dV, const void* X,
                 const void* T, const lora_proj_t* q, const lora_proj_t* k, const lora_proj_t* v, void* dX,
                 void* dA_q, void* dB_q, void* dA_k, void* dB_k, void* dA_v, void* dB_v, void* workspace,
                 size_t workspace_bytes, void* hip_stream) {
  int rc = check_qkv(desc);
  if (rc) return rc;
  if ((rc = check_proj(q, "q")) || (rc = check_proj(k, "k")) || (rc = check_proj(v, "v"))) return rc;
  if (!dA_q || !dB_q || !dA_k || !dB_k || !dA_v || !dB_v ||
      (desc->batch > 0 && (!dQ || !dK || !dV || !X || !T || !dX)))
    return fail(LORA_ERR_NULL, "a tensor pointer is NULL");
  const QkvWs probe = qkv_ws(*desc, 1, nullptr);
  if (probe.bytes > 0 && (!workspace || workspace_bytes < probe.bytes))
    return fail(LORA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, probe.bytes);
  const QkvWs w = qkv_ws(*desc, 1, workspace);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const lora_proj_t* const pr[3] = {q, k, v};
  const void* const dO[3] = {dQ, dK, dV};
  void* const dA[3] = {dA_q, dA_k, dA_v};
  void* const dB[3] = {dB_q, dB_k, dB_v};
  if (desc->dtype == LORA_BF16) return qkv_bwd_impl<bf16>(*desc, dO, X, T, pr, dX, dA, dB, w, st);
  return qkv_bwd_impl<float>(*desc, dO, X, T, pr, dX, dA, dB, w, st);
}

int lora_qkv_norm_fwd(const lora_qkv_desc_t* desc, const void* X, const lora_proj_t* q, const lora_proj_t* k,
                      const lora_proj_t* v, const lora_qk_norm_t* norm, void* Q, void* K, void* V, void* T, void* Pn,
                      float* rinv, void* workspace, size_t workspace_bytes, void* hip_stream) {
  int rc = check_qkv(desc);
  if (rc) return rc;
  if ((rc = check_proj(q, "q")) || (rc = check_proj(k, "k")) || (rc = check_proj(v, "v"))) return rc;
  if (desc->batch > 0 && (!X || !Q || !K || !V || !T)) return fail(LORA_ERR_NULL, "a tensor pointer is NULL");
  NormIo nio{};
  if ((rc = check_norm(desc, norm, Pn, rinv, {norm ? norm->q_weight : nullptr, norm ? norm->k_weight : nullptr, Pn},
                       nio)))
    return rc;
  const QkvWs probe = qkv_ws(*desc, 0, nullptr);
  if (probe.bytes > 0 && (!workspace || workspace_bytes < probe.bytes))
    return fail(LORA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, probe.bytes);
  const QkvWs w = qkv_ws(*desc, 0, workspace);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const lora_proj_t* const pr[3] = {q, k, v};
  void* const out[3] = {Q, K, V};
  if (desc->dtype == LORA_BF16) return qkv_fwd_impl<bf16>(*desc, X, pr, out, T, w, st, &nio);
  return qkv_fwd_impl<float>(*desc, X, pr, out, T, w, st, &nio);
}

int lora_qkv_norm_bwd(const lora_qkv_desc_t* desc, const void* dQ, const void* dK, const void* dV, const void* X,
                      const void* T, const void* Pn, const float* rinv, const lora_proj_t* q, const lora_proj_t* k,
                      const lora_proj_t* v, const lora_qk_norm_t* norm, void* dX, void* dA_q, void* dB_q,
                      void* dA_k, void* dB_k, void* dA_v, void* dB_v, void* workspace, size_t workspace_bytes,
                      void* hip_stream) {
  int rc = check_qkv(desc);
  if (rc) return rc;
  if ((rc = check_proj(q, "q")) || (rc = check_proj(k, "k")) || (rc = check_proj(v, "v"))) return rc;
  if (!dA_q || !dB_q || !dA_k || !dB_k || !dA_v || !dB_v ||
      (desc->batch > 0 && (!dQ || !dK || !dV || !X || !T || !dX)))
    return fail(LORA_ERR_NULL, "a tensor pointer is NULL");
  NormIo nio{};
  if ((rc = check_norm(desc, norm, Pn, rinv,
                       {norm ? norm->q_weight : nullptr, norm ? norm->k_weight : nullptr, Pn, dQ, dK, dV}, nio)))
    return rc;
  const QkvWs probe = qkv_ws(*desc, 1, nullptr);
  if (probe.bytes > 0 && (!workspace || workspace_bytes < probe.bytes))
    return fail(LORA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, probe.bytes);
  const QkvWs w = qkv_ws(*desc, 1, workspace);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const lora_proj_t* const pr[3] = {q, k, v};
  const void* const dO[3] = {dQ, dK, dV};
  void* const dA[3] = {dA_q, dA_k, dA_v};
  void* const dB[3] = {dB_q, dB_k, dB_v};
  if (desc->dtype == LORA_BF16) return qkv_bwd_impl<bf16>(*desc, dO, X, T, pr, dX, dA, dB, w, st, &nio);
  return qkv_bwd_impl<float>(*desc, dO, X, T, pr, dX, dA, dB, w, st, &nio);
}

int lora_linear_fwd(const lora_linear_desc_t* desc, const void* X, const lora_proj_t* proj, void* Y, void* T,
                    void* workspace, size_t workspace_bytes, void* hip_stream) {
  int rc = check_linear(desc);
  if (rc) return rc;
  if ((rc = check_proj(proj, "proj"))) return rc;
  if (desc->n_tokens > 0 && (!X || !Y || !T)) return fail(LORA_ERR_NULL, "a tensor pointer is NULL");
  const LinWs probe = lin_ws(*desc, 0, nullptr);
  if (probe.bytes > 0 && (!workspace || workspace_bytes < probe.bytes))
    return fail(LORA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, probe.bytes);
  const LinWs w = lin_ws(*desc, 0, workspace);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (desc->dtype == LORA_BF16) return linear_fwd_impl<bf16>(*desc, X, *proj, Y, T, w, st);
  return linear_fwd_impl<float>(*desc, X, *proj, Y, T, w, st);
}

int lora_linear_bwd(const lora_linear_desc_t* desc, const void* dY, const void* X, const void* T,
                    const lora_proj_t* proj, void* dX, void* dA, void* dB, void* workspace, size_t workspace_bytes,
                    void* hip_stream) {
  int rc = check_linear(desc);
  if (rc) return rc;
  if ((rc = check_proj(proj, "proj"))) return rc;
  if (!dA || !dB || (desc->n_tokens > 0 && (!dY || !X || !T || !dX)))
    return fail(LORA_ERR_NULL, "a tensor pointer is NULL");
  const LinWs probe = lin_ws(*desc, 1, nullptr);
  if (probe.bytes > 0 && (!workspace || workspace_bytes < probe.bytes))
    return fail(LORA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, probe.bytes);
  const LinWs w = lin_ws(*desc, 1, workspace);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (desc->dtype == LORA_BF16) return linear_bwd_impl<bf16>(*desc, dY, X, T, *proj, dX, dA, dB, w, st);
  return linear_bwd_impl<float>(*desc, dY, X, T, *proj, dX, dA, dB, w, st);
}

const char* lora_status_string(int status) {
  switch (status) {
    case LORA_OK: return "ok";
    case LORA_ERR_NULL: return "null pointer";
    case LORA_ERR_SHAPE: return "bad shape";
    case LORA_ERR_UNSUPPORTED: return "unsupported configuration";
    case LORA_ERR_WORKSPACE: return "workspace too small";
    case LORA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* lora_last_error_message(void) { return g_err; }

const char* lora_version(void) { return "lora_mi355x 0.1 (gfx950)"; }

int lora_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_tm);
  g_timing = on != 0;
  return LORA_OK;
}

int lora_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_tm);
  for (auto& r : g_recs) {
    g_pool.push_back(r.e0);
    g_pool.push_back(r.e1);
  }
  g_recs.clear();
  return LORA_OK;
}

int lora_timing_query(const char* kernel, double* total_ms, int* launches) {
  if (!kernel || !total_ms || !launches) return fail(LORA_ERR_NULL, "NULL argument");
  const int kid = kernel_id(kernel);
  if (kid < 0) return fail(LORA_ERR_SHAPE, "unknown kernel name %s", kernel);
  std::lock_guard<std::mutex> lk(g_tm);
  double tot = 0.0;
  int n = 0;
  for (auto& r : g_recs) {
    if (r.kernel != kid) continue;
    if (hipEventSynchronize(r.e1) != hipSuccess) return fail(LORA_ERR_HIP, "event synchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.e0, r.e1) != hipSuccess) return fail(LORA_ERR_HIP, "event elapsed failed");
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return ok();
}

const char* lora_kernel_names(void) {
  static std::string s;
  static std::once_flag once;
  std::call_once(once, [] {
    for (int i = 0; i < kNumNames; ++i) {
      if (i) s += ",";
      s += kNames[i];
    }
  });
  return s.c_str();
}

}  // extern "C"

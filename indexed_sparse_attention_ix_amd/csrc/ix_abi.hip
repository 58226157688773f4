#include <algorithm>
// C ABI of libix: argument validation, workspace sizing, dispatch, error reporting,
// and the IndexShare group driver ("IndexShare: Amortizing the Indexer" in "GLM 5.2:
// How Four Co-Designed Mechanisms Beat Raw Scale", Part II: the selection runs once
// per block of layers and is shared across the block).
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <mutex>
#include <string>

#include "ix_internal.h"

// Scratch of indexshare_group_fwd_noalloc: device memory the library owns instead of a
// caller workspace.  Each GPU the library runs on holds its own copy of this array until
// the process ends; host code uses the per-device address from hipGetSymbolAddress, never
// the array's name (which in host code is only a stand-in).
static __device__ __align__(256) unsigned char scratch[IX_NOALLOC_SCRATCH_BYTES];

// Debug status block (ix_debug_enable / ix_debug_read), one per GPU, reached the same way.
static __device__ __align__(64) unsigned long long debug_words[ix::kDbgWords];
static_assert(sizeof(ix_debug_status) == sizeof(unsigned long long) * ix::kDbgWords,
              "ix_debug_status holds the debug words in order");

// Launches go through IX_LAUNCH.  A test build (-DIX_TEST_HOOKS) adds an exported hook that
// makes them return a chosen HIP error without launching, so the IX_ERR_HIP path and its
// message are exercised on a machine without a GPU; the release library has no hook.
#ifdef IX_TEST_HOOKS
static std::atomic<int> g_test_launch_error{0};
extern "C" __attribute__((visibility("default"))) void ix_test_fail_launches(int32_t hip_error) {
  g_test_launch_error.store(hip_error);
}
#define IX_LAUNCH(call) \
  (g_test_launch_error.load() ? static_cast<hipError_t>(g_test_launch_error.load()) : (call))
#else
#define IX_LAUNCH(call) (call)
#endif

namespace {

thread_local std::string g_err;

ix_status fail(ix_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ix_status fail(ix_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

ix_status ok() {
  g_err.clear();
  return IX_OK;
}

ix_status hip_fail(hipError_t e, const char* what) {
  return fail(IX_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// A launch gives its grid in blocks, but the dispatch counts work-items in 32 bits.  The
// kernels run 256-thread blocks over at most one block per query row (and KV head), and
// the element-wise kernels at most 256 threads per row.  So one call covers fewer than
// 2^24 rows, and an element-wise launch at most kMaxBlocks full blocks.
constexpr int64_t kMaxBlocks = (int64_t)0xFFFFFFFF / 256;  // 2^24 - 1
bool items_fit(int64_t threads) { return threads >= 0 && (threads + 255) / 256 <= kMaxBlocks; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Returns IX_OK and sets *empty when B*T == 0.
ix_status check_indexer(const ix_indexer_args* a, bool* empty) {
  if (!a) return fail(IX_ERR_INVALID, "indexer args pointer is NULL");
  if (a->B < 0 || a->T < 0 || a->S_max < 0 || a->H_I < 0 || a->d_I < 0)
    return fail(IX_ERR_INVALID, "negative size (B=%d T=%d S_max=%d H_I=%d d_I=%d)", a->B, a->T,
                a->S_max, a->H_I, a->d_I);
  if (a->d_I != 64 && a->d_I != 128)
    return fail(IX_ERR_UNSUPPORTED, "d_I=%d unsupported (64 or 128)", a->d_I);
  if (a->H_I < 4 || a->H_I > 64 || a->H_I % 4 != 0)
    return fail(IX_ERR_UNSUPPORTED, "H_I=%d unsupported (multiple of 4 in [4,64])", a->H_I);
  *empty = (a->B == 0 || a->T == 0);
  if (*empty) return IX_OK;
  if (a->S_max < 1) return fail(IX_ERR_INVALID, "S_max=%d must be >= 1", a->S_max);
  if (!a->q || !a->k || !a->w || !a->q_pos0 || !a->kv_len)
    return fail(IX_ERR_INVALID, "NULL indexer tensor pointer");
  if (!aligned16(a->q) || !aligned16(a->k))
    return fail(IX_ERR_INVALID, "FP8 q/k base pointers must be 16-byte aligned");
  const double k_bytes = (double)a->B * a->S_max * a->d_I;
  const double q_bytes = (double)a->B * a->T * a->H_I * a->d_I;
  if (k_bytes > 9.0e18 || q_bytes > 9.0e18) return fail(IX_ERR_INVALID, "tensor too large");
  if ((int64_t)a->S_max * a->d_I >= ((int64_t)1 << 31))
    return fail(IX_ERR_UNSUPPORTED, "S_max*d_I=%lld: one sequence's indexer keys must stay below 2 GiB",
                (long long)a->S_max * a->d_I);
  if ((int64_t)a->B * a->T > kMaxBlocks)
    return fail(IX_ERR_UNSUPPORTED, "B*T=%lld query rows: one launch holds at most %lld",
                (long long)((int64_t)a->B * a->T), (long long)kMaxBlocks);
  return IX_OK;
}

ix_status check_k(int32_t k) {
  if (k < 1 || k > 2048) return fail(IX_ERR_UNSUPPORTED, "k=%d unsupported (1..2048)", k);
  return IX_OK;
}

ix_status check_attn_shape(int32_t B, int32_t T, int32_t S_max, int32_t H_q, int32_t H_kv,
                           int32_t d, int32_t k, bool* empty) {
  if (B < 0 || T < 0 || S_max < 0 || H_q < 0 || H_kv < 0 || d < 0)
    return fail(IX_ERR_INVALID, "negative size (B=%d T=%d S_max=%d H_q=%d H_kv=%d d=%d)", B, T,
                S_max, H_q, H_kv, d);
  if (d != 64 && d != 128) return fail(IX_ERR_UNSUPPORTED, "d=%d unsupported (64 or 128)", d);
  if (H_kv < 1 || H_q < 1 || H_q % H_kv != 0 || H_q / H_kv > 16)
    return fail(IX_ERR_UNSUPPORTED, "H_q=%d H_kv=%d unsupported (H_q multiple of H_kv, ratio <= 16)",
                H_q, H_kv);
  ix_status st = check_k(k);
  if (st != IX_OK) return st;
  *empty = (B == 0 || T == 0);
  if (*empty) return IX_OK;
  if (S_max < 1) return fail(IX_ERR_INVALID, "S_max=%d must be >= 1", S_max);
  if ((int64_t)B * T * H_kv > kMaxBlocks)
    return fail(IX_ERR_UNSUPPORTED, "B*T*H_kv=%lld query rows: one launch holds at most %lld",
                (long long)((int64_t)B * T * H_kv), (long long)kMaxBlocks);
  if ((int64_t)S_max * H_kv * d * 2 > ((int64_t)1 << 31))
    return fail(IX_ERR_UNSUPPORTED,
                "S_max*H_kv*d=%lld: one sequence's K (or V) cache must stay within 2 GiB",
                (long long)S_max * H_kv * d);
  return IX_OK;
}

bool pool_ok(int32_t pool) { return pool == 1 || pool == 2 || pool == 4 || pool == 8 || pool == 16; }

bool pair_rows_valid(int32_t pair_rows) {
  return pair_rows == IX_PAIR_ROWS_BF16 || pair_rows == IX_PAIR_ROWS_FP32;
}

ix_status check_pair_rows(int32_t pair_rows) {
  if (!pair_rows_valid(pair_rows))
    return fail(IX_ERR_INVALID, "pair_rows=%d: IX_PAIR_ROWS_BF16 (0) or IX_PAIR_ROWS_FP32 (1)",
                pair_rows);
  return IX_OK;
}

// Bytes of one kept pair's gradient rows in the atomic-free backward forms: the attention's
// dV | dK rows (H_kv heads of 2 d) and the indexer's dk_I row (d_I).
size_t attn_pair_row_bytes(int32_t H_kv, int32_t d, int32_t pair_rows) {
  return (size_t)H_kv * 2 * d * (pair_rows == IX_PAIR_ROWS_FP32 ? 4 : 2);
}

size_t indexer_pair_row_bytes(int32_t d_I, int32_t pair_rows) {
  return (size_t)d_I * (pair_rows == IX_PAIR_ROWS_FP32 ? 4 : 2);
}

// The indexer arguments as the top-k sees them under IndexPool: one key row per block.
ix_indexer_args pooled_args(const ix_indexer_args& a, int32_t pool) {
  ix_indexer_args u = a;
  u.S_max = a.S_max < 0 ? a.S_max : (a.S_max + pool - 1) / pool;
  return u;
}

size_t pooled_blocks_bytes(const ix_indexer_args& u, int32_t k_blocks) {
  return ((size_t)u.B * u.T * k_blocks * sizeof(int32_t) + 255) / 256 * 256;
}

ix_status check_attn_ptrs(const void* q, const void* kc, const void* vc, const int32_t* idx,
                          const void* out) {
  if (!q || !kc || !vc || !idx || !out) return fail(IX_ERR_INVALID, "NULL attention tensor pointer");
  if (!aligned16(q) || !aligned16(kc) || !aligned16(vc))
    return fail(IX_ERR_INVALID, "bf16 q/kc/vc base pointers must be 16-byte aligned");
  return IX_OK;
}

// Address of this device's copy of a library-owned device array (`scratch`,
// `debug_words`): looked up once per device, with that device current, and kept in `table`.
// The device is the stream's (the current one for the NULL stream).
constexpr int kMaxDevices = 64;
std::mutex g_symbol_mu;
void* g_scratch_ptr[kMaxDevices] = {};
void* g_debug_ptr[kMaxDevices] = {};

hipError_t device_symbol(const void* symbol, void** table, hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_symbol_mu);
  if (!table[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, symbol);
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    table[dev] = p;
  }
  *out = table[dev];
  return hipSuccess;
}

hipError_t device_scratch(hipStream_t stream, void** out) {
  return device_symbol(HIP_SYMBOL(scratch), g_scratch_ptr, stream, out);
}

// The debug status: off unless ix_debug_enable(1).  debug_ptr gives the stream's GPU's
// status block while it is on, else NULL (the kernels then count nothing).
std::atomic<bool> g_debug{false};

hipError_t debug_ptr(hipStream_t stream, unsigned long long** out) {
  *out = nullptr;
  if (!g_debug.load()) return hipSuccess;
  void* p = nullptr;
  const hipError_t e = device_symbol(HIP_SYMBOL(debug_words), g_debug_ptr, stream, &p);
  if (e == hipSuccess) *out = static_cast<unsigned long long*>(p);
  return e;
}

// With the debug status on: count the caller's selection entries that name no key.
ix_status debug_check_idx(const int32_t* idx, const int32_t* kv_len, int32_t B, int32_t T,
                          int32_t S_max, int32_t k, hipStream_t stream) {
  if (!g_debug.load()) return IX_OK;
  unsigned long long* dbg = nullptr;
  hipError_t e = IX_LAUNCH(debug_ptr(stream, &dbg));
  if (e == hipSuccess && dbg) e = IX_LAUNCH(ix::launch_idx_check(idx, kv_len, B, T, S_max, k, dbg, stream));
  return e == hipSuccess ? IX_OK : hip_fail(e, "debug check of idx");
}

// The debug status block for a launch (NULL while off).
ix_status debug_words_for(hipStream_t stream, unsigned long long** dbg) {
  const hipError_t e = IX_LAUNCH(debug_ptr(stream, dbg));
  return e == hipSuccess ? IX_OK : hip_fail(e, "debug status address");
}

// indexshare_group_fwd, with the caller's workspace or (use_scratch) the library's scratch.
ix_status group_fwd(const ix_indexer_args* a, int32_t k, int32_t n_layers, const void* const* q,
                    const void* const* kc, const void* const* vc, void* const* out,
                    float* const* lse, int32_t H_q, int32_t H_kv, int32_t d, float sm_scale,
                    int32_t* idx, void* ws, size_t ws_bytes, bool use_scratch, hipStream_t stream) {
  bool empty = false, empty2 = false;
  ix_status st = check_indexer(a, &empty);
  if (st != IX_OK) return st;
  if ((st = check_k(k)) != IX_OK) return st;
  if ((st = check_attn_shape(a->B, a->T, a->S_max, H_q, H_kv, d, k, &empty2)) != IX_OK) return st;
  if (n_layers < 1) return fail(IX_ERR_INVALID, "n_layers=%d must be >= 1", n_layers);
  if (empty) return ok();
  if (!idx) return fail(IX_ERR_INVALID, "idx pointer is NULL");
  if (!q || !kc || !vc || !out) return fail(IX_ERR_INVALID, "NULL per-layer pointer array");
  for (int l = 0; l < n_layers; ++l) {
    if ((st = check_attn_ptrs(q[l], kc[l], vc[l], idx, out[l])) != IX_OK) return st;
  }
  if (!(sm_scale == sm_scale) || sm_scale == __builtin_inff() || sm_scale == -__builtin_inff())
    return fail(IX_ERR_INVALID, "sm_scale must be finite");
  const ix::TopkPlan tp = ix::make_topk_plan(*a, k);
  const ix::AttnPlan ap = ix::make_attn_plan(a->B, a->T, H_q, H_kv, d, k, n_layers);
  const size_t attn_need = ap.ws_bytes;
  const size_t need = tp.ws_bytes > attn_need ? tp.ws_bytes : attn_need;
  if (use_scratch) {
    if (need > IX_NOALLOC_SCRATCH_BYTES)
      return fail(IX_ERR_WORKSPACE,
                  "this call needs %zu bytes of scratch; the no-allocation entry point holds %zu",
                  need, (size_t)IX_NOALLOC_SCRATCH_BYTES);
    const hipError_t es = IX_LAUNCH(device_scratch(stream, &ws));
    if (es != hipSuccess) return hip_fail(es, "no-allocation scratch address");
    ws_bytes = IX_NOALLOC_SCRATCH_BYTES;
  }
  if (!ws || ws_bytes < need)
    return fail(IX_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws ? ws_bytes : (size_t)0, need);
  unsigned long long* dbg = nullptr;
  if ((st = debug_words_for(stream, &dbg)) != IX_OK) return st;
  hipError_t e = IX_LAUNCH(ix::launch_ix_topk(*a, k, tp, idx, nullptr, ws, stream, 1, dbg));
  if (e != hipSuccess) return hip_fail(e, "indexshare selection launch");
  e = IX_LAUNCH(ix::launch_sparse_attn_layers(n_layers, q, kc, vc, idx, a->kv_len, a->B, a->T, a->S_max,
                                    H_q, H_kv, d, k, sm_scale, out, lse, ap, ws, stream));
  if (e != hipSuccess) return hip_fail(e, "indexshare attention launch");
  return ok();
}

}  // namespace

extern "C" {

int32_t ix_abi_version(void) { return IX_ABI_VERSION; }

const char* ix_last_error(void) { return g_err.c_str(); }

ix_status ix_score(const ix_indexer_args* a, int32_t t_begin, int32_t t_end, float* scores,
                   hipStream_t stream) {
  bool empty = false;
  ix_status st = check_indexer(a, &empty);
  if (st != IX_OK) return st;
  if (t_begin < 0 || t_end < t_begin || t_end > a->T)
    return fail(IX_ERR_INVALID, "row range [%d,%d) outside [0,%d)", t_begin, t_end, a->T);
  if (empty || t_end == t_begin) return ok();
  if (!scores) return fail(IX_ERR_INVALID, "scores pointer is NULL");
  hipError_t e = IX_LAUNCH(ix::launch_ix_score(*a, t_begin, t_end, scores, stream));
  if (e != hipSuccess) return hip_fail(e, "ix_score launch");
  return ok();
}

size_t ix_topk_workspace_bytes(const ix_indexer_args* a, int32_t k) {
  bool empty = false;
  if (check_indexer(a, &empty) != IX_OK || check_k(k) != IX_OK) return 0;
  if (empty) return 0;
  return ix::make_topk_plan(*a, k).ws_bytes;
}

ix_status ix_topk(const ix_indexer_args* a, int32_t k, int32_t* idx, float* sel_scores, void* ws,
                  size_t ws_bytes, hipStream_t stream) {
  bool empty = false;
  ix_status st = check_indexer(a, &empty);
  if (st != IX_OK) return st;
  if ((st = check_k(k)) != IX_OK) return st;
  if (empty) return ok();
  if (!idx) return fail(IX_ERR_INVALID, "idx pointer is NULL");
  const ix::TopkPlan plan = ix::make_topk_plan(*a, k);
  if (!ws || ws_bytes < plan.ws_bytes)
    return fail(IX_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws ? ws_bytes : (size_t)0,
                plan.ws_bytes);
  unsigned long long* dbg = nullptr;
  if ((st = debug_words_for(stream, &dbg)) != IX_OK) return st;
  hipError_t e = IX_LAUNCH(ix::launch_ix_topk(*a, k, plan, idx, sel_scores, ws, stream, 1, dbg));
  if (e != hipSuccess) return hip_fail(e, "ix_topk launch");
  return ok();
}

size_t sparse_attn_workspace_bytes(int32_t B, int32_t T, int32_t H_q, int32_t H_kv, int32_t d,
                                   int32_t k) {
  bool empty = false;
  if (check_attn_shape(B, T, 1, H_q, H_kv, d, k, &empty) != IX_OK || empty) return 0;
  return ix::make_attn_plan(B, T, H_q, H_kv, d, k, 1).ws_bytes;
}

ix_status sparse_attn_fwd(const void* q, const void* kc, const void* vc, const int32_t* idx,
                          const int32_t* kv_len, int32_t B, int32_t T, int32_t S_max, int32_t H_q,
                          int32_t H_kv, int32_t d, int32_t k, float sm_scale, void* out,
                          float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  bool empty = false;
  ix_status st = check_attn_shape(B, T, S_max, H_q, H_kv, d, k, &empty);
  if (st != IX_OK) return st;
  if (empty) return ok();
  if ((st = check_attn_ptrs(q, kc, vc, idx, out)) != IX_OK) return st;
  if (!(sm_scale == sm_scale) || sm_scale == __builtin_inff() || sm_scale == -__builtin_inff())
    return fail(IX_ERR_INVALID, "sm_scale must be finite");
  const ix::AttnPlan plan = ix::make_attn_plan(B, T, H_q, H_kv, d, k, 1);
  if (plan.ws_bytes && (!ws || ws_bytes < plan.ws_bytes))
    return fail(IX_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws ? ws_bytes : (size_t)0,
                plan.ws_bytes);
  if ((st = debug_check_idx(idx, kv_len, B, T, S_max, k, stream)) != IX_OK) return st;
  hipError_t e = IX_LAUNCH(ix::launch_sparse_attn(q, kc, vc, idx, kv_len, B, T, S_max, H_q, H_kv, d, k,
                                        sm_scale, out, lse, plan, ws, stream));
  if (e != hipSuccess) return hip_fail(e, "sparse_attn_fwd launch");
  return ok();
}

size_t sparse_attn_group_workspace_bytes(int32_t B, int32_t T, int32_t H_q, int32_t H_kv,
                                         int32_t d, int32_t k, int32_t n_layers) {
  bool empty = false;
  if (n_layers < 1 || check_attn_shape(B, T, 1, H_q, H_kv, d, k, &empty) != IX_OK || empty) return 0;
  return ix::make_attn_plan(B, T, H_q, H_kv, d, k, n_layers).ws_bytes;
}

ix_status sparse_attn_group_fwd(int32_t n_layers, const void* const* q, const void* const* kc,
                                const void* const* vc, void* const* out, float* const* lse,
                                const int32_t* idx, const int32_t* kv_len, int32_t B, int32_t T,
                                int32_t S_max, int32_t H_q, int32_t H_kv, int32_t d, int32_t k,
                                float sm_scale, void* ws, size_t ws_bytes, hipStream_t stream) {
  bool empty = false;
  ix_status st = check_attn_shape(B, T, S_max, H_q, H_kv, d, k, &empty);
  if (st != IX_OK) return st;
  if (n_layers < 1) return fail(IX_ERR_INVALID, "n_layers=%d must be >= 1", n_layers);
  if (empty) return ok();
  if (!q || !kc || !vc || !out) return fail(IX_ERR_INVALID, "NULL per-layer pointer array");
  for (int l = 0; l < n_layers; ++l) {
    if ((st = check_attn_ptrs(q[l], kc[l], vc[l], idx, out[l])) != IX_OK) return st;
  }
  if (!(sm_scale == sm_scale) || sm_scale == __builtin_inff() || sm_scale == -__builtin_inff())
    return fail(IX_ERR_INVALID, "sm_scale must be finite");
  const ix::AttnPlan ap = ix::make_attn_plan(B, T, H_q, H_kv, d, k, n_layers);
  if (ap.ws_bytes && (!ws || ws_bytes < ap.ws_bytes))
    return fail(IX_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws ? ws_bytes : (size_t)0,
                ap.ws_bytes);
  if ((st = debug_check_idx(idx, kv_len, B, T, S_max, k, stream)) != IX_OK) return st;
  hipError_t e = IX_LAUNCH(ix::launch_sparse_attn_layers(n_layers, q, kc, vc, idx, kv_len, B, T, S_max, H_q,
                                               H_kv, d, k, sm_scale, out, lse, ap, ws, stream));
  if (e != hipSuccess) return hip_fail(e, "sparse_attn_group_fwd launch");
  return ok();
}

size_t indexshare_workspace_bytes(const ix_indexer_args* a, int32_t k, int32_t H_q, int32_t H_kv,
                                  int32_t d) {
  bool empty = false, empty2 = false;
  if (check_indexer(a, &empty) != IX_OK || check_k(k) != IX_OK) return 0;
  if (check_attn_shape(a->B, a->T, a->S_max, H_q, H_kv, d, k, &empty2) != IX_OK) return 0;
  if (empty) return 0;
  const size_t t = ix::make_topk_plan(*a, k).ws_bytes;
  // the selection, then the attention of the layers (split partials of up to 8 layers per
  // launch), one after the other on the same stream
  const size_t s = ix::attn_group_ws_bytes(a->B, a->T, H_q, H_kv, d, k);
  return t > s ? t : s;
}

ix_status indexshare_group_fwd(const ix_indexer_args* a, int32_t k, int32_t n_layers,
                               const void* const* q, const void* const* kc, const void* const* vc,
                               void* const* out, float* const* lse, int32_t H_q, int32_t H_kv,
                               int32_t d, float sm_scale, int32_t* idx, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  return group_fwd(a, k, n_layers, q, kc, vc, out, lse, H_q, H_kv, d, sm_scale, idx, ws, ws_bytes,
                   false, stream);
}

ix_status indexshare_group_fwd_noalloc(const ix_indexer_args* a, int32_t k, int32_t n_layers,
                                       const void* const* q, const void* const* kc,
                                       const void* const* vc, void* const* out,
                                       float* const* lse, int32_t H_q, int32_t H_kv, int32_t d,
                                       float sm_scale, int32_t* idx, hipStream_t stream) {
  return group_fwd(a, k, n_layers, q, kc, vc, out, lse, H_q, H_kv, d, sm_scale, idx, nullptr, 0,
                   true, stream);
}

ix_status ix_append_kv(const float* k_I_new, const void* K_new, const void* V_new,
                       const int32_t* pos0, int32_t B, int32_t T_new, int32_t S_max, int32_t d_I,
                       int32_t H_kv, int32_t d, uint8_t* k_I_cache, void* K_cache, void* V_cache,
                       hipStream_t stream) {
  if (B < 0 || T_new < 0 || S_max < 0)
    return fail(IX_ERR_INVALID, "negative size (B=%d T_new=%d S_max=%d)", B, T_new, S_max);
  if (!k_I_new != !k_I_cache)
    return fail(IX_ERR_INVALID, "k_I_new and k_I_cache must both be given or both be NULL");
  if (!K_new != !K_cache || !V_new != !V_cache)
    return fail(IX_ERR_INVALID, "each of K/V needs both its new rows and its cache, or neither");
  if (k_I_new && d_I != 64 && d_I != 128)
    return fail(IX_ERR_UNSUPPORTED, "d_I=%d unsupported (64 or 128)", d_I);
  if (K_new || V_new) {
    if (d != 64 && d != 128) return fail(IX_ERR_UNSUPPORTED, "d=%d unsupported (64 or 128)", d);
    if (H_kv < 1 || H_kv > 16) return fail(IX_ERR_UNSUPPORTED, "H_kv=%d unsupported (1..16)", H_kv);
  }
  if (B == 0 || T_new == 0 || (!k_I_new && !K_new && !V_new)) return ok();
  if (S_max < 1) return fail(IX_ERR_INVALID, "S_max=%d must be >= 1", S_max);
  if (!pos0) return fail(IX_ERR_INVALID, "pos0 pointer is NULL");
  if ((k_I_new && (!aligned16(k_I_new) || (reinterpret_cast<uintptr_t>(k_I_cache) & 7u))) ||
      (K_new && (!aligned16(K_new) || !aligned16(K_cache))) ||
      (V_new && (!aligned16(V_new) || !aligned16(V_cache))))
    return fail(IX_ERR_INVALID,
                "k_I_new, K/V rows and caches must be 16-byte aligned (k_I_cache 8-byte)");
  if ((int64_t)B * T_new > kMaxBlocks)
    return fail(IX_ERR_UNSUPPORTED, "B*T_new=%lld rows: one launch holds at most %lld",
                (long long)((int64_t)B * T_new), (long long)kMaxBlocks);
  hipError_t e = IX_LAUNCH(ix::launch_append_kv(k_I_new, K_new, V_new, pos0, B, T_new, S_max, d_I, H_kv, d,
                                      k_I_cache, K_cache, V_cache, stream));
  if (e != hipSuccess) return hip_fail(e, "ix_append_kv launch");
  return ok();
}

ix_status ix_pool_keys(const uint8_t* k_I, const int32_t* kv_len, int32_t B, int32_t S_max,
                       int32_t d_I, int32_t pool, uint8_t* k_pooled, hipStream_t stream) {
  if (B < 0 || S_max < 0) return fail(IX_ERR_INVALID, "negative size (B=%d S_max=%d)", B, S_max);
  if (d_I != 64 && d_I != 128) return fail(IX_ERR_UNSUPPORTED, "d_I=%d unsupported (64 or 128)", d_I);
  if (!pool_ok(pool)) return fail(IX_ERR_UNSUPPORTED, "pool=%d unsupported (1, 2, 4, 8 or 16)", pool);
  if (B == 0 || S_max == 0) return ok();
  if (!k_I || !k_pooled) return fail(IX_ERR_INVALID, "NULL key pointer");
  if ((reinterpret_cast<uintptr_t>(k_I) | reinterpret_cast<uintptr_t>(k_pooled)) & 7u)
    return fail(IX_ERR_INVALID, "key arrays must be 8-byte aligned");
  const int64_t pieces_per_row = d_I / 8;
  const int64_t block_rows = (int64_t)B * ((S_max + pool - 1) / pool);
  if (block_rows > ((int64_t)1 << 40) || !items_fit(block_rows * pieces_per_row))
    return fail(IX_ERR_UNSUPPORTED, "B*ceil(S_max/pool)=%lld block keys: too many for one launch",
                (long long)block_rows);
  hipError_t e = IX_LAUNCH(ix::launch_pool_keys(k_I, kv_len, B, S_max, d_I, pool, k_pooled, stream));
  if (e != hipSuccess) return hip_fail(e, "ix_pool_keys launch");
  return ok();
}

size_t ix_topk_pooled_workspace_bytes(const ix_indexer_args* a, int32_t pool, int32_t k_blocks) {
  bool empty = false;
  if (!a || !pool_ok(pool) || check_k(k_blocks) != IX_OK) return 0;
  const ix_indexer_args u = pooled_args(*a, pool);
  if (check_indexer(&u, &empty) != IX_OK || empty) return 0;
  if (!items_fit((int64_t)a->B * a->T * k_blocks * pool)) return 0;
  const ix::TopkPlan plan = ix::make_topk_plan(u, k_blocks);
  return plan.ws_bytes + pooled_blocks_bytes(u, k_blocks);
}

ix_status ix_topk_pooled(const ix_indexer_args* a, int32_t pool, int32_t k_blocks, int32_t* idx,
                         void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!a) return fail(IX_ERR_INVALID, "indexer args pointer is NULL");
  if (!pool_ok(pool)) return fail(IX_ERR_UNSUPPORTED, "pool=%d unsupported (1, 2, 4, 8 or 16)", pool);
  ix_status st = check_k(k_blocks);
  if (st != IX_OK) return st;
  bool empty = false;
  const ix_indexer_args u = pooled_args(*a, pool);
  if ((st = check_indexer(&u, &empty)) != IX_OK) return st;
  if (empty) return ok();
  if (!idx) return fail(IX_ERR_INVALID, "idx pointer is NULL");
  if (!items_fit((int64_t)a->B * a->T * k_blocks * pool))
    return fail(IX_ERR_UNSUPPORTED, "B*T*k_blocks*pool=%lld entries: too many for one launch",
                (long long)((int64_t)a->B * a->T * k_blocks * pool));
  const ix::TopkPlan plan = ix::make_topk_plan(u, k_blocks);
  const size_t need = plan.ws_bytes + pooled_blocks_bytes(u, k_blocks);
  if (!ws || ws_bytes < need)
    return fail(IX_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws ? ws_bytes : (size_t)0, need);
  int32_t* blocks = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + plan.ws_bytes);
  unsigned long long* dbg = nullptr;
  if ((st = debug_words_for(stream, &dbg)) != IX_OK) return st;
  hipError_t e = IX_LAUNCH(ix::launch_ix_topk(u, k_blocks, plan, blocks, nullptr, ws, stream, pool, dbg));
  if (e != hipSuccess) return hip_fail(e, "ix_topk_pooled launch");
  e = IX_LAUNCH(ix::launch_expand_blocks(blocks, a->q_pos0, a->kv_len, a->B, a->T, a->S_max, k_blocks, pool,
                               idx, stream));
  if (e != hipSuccess) return hip_fail(e, "ix_topk_pooled expansion launch");
  return ok();
}

size_t sparse_attn_bwd_workspace_bytes(int32_t B, int32_t T, int32_t S_max, int32_t H_kv,
                                       int32_t d, int32_t k, int32_t rows_per_pass,
                                       int32_t pair_rows) {
  bool empty = false;
  if (check_attn_shape(B, T, S_max, H_kv, H_kv, d, k, &empty) != IX_OK || empty) return 0;
  if (rows_per_pass < 1 || !pair_rows_valid(pair_rows)) return 0;
  const int64_t rows = std::min<int64_t>(rows_per_pass, (int64_t)B * T);
  if (rows * k > ((int64_t)1 << 31)) return 0;
  return ix::pair_layout(B, S_max, k, rows, attn_pair_row_bytes(H_kv, d, pair_rows)).total;
}

ix_status sparse_attn_bwd(const void* q, const void* kc, const void* vc, const int32_t* idx,
                          const int32_t* kv_len, const void* out, const float* lse,
                          const void* dout, int32_t B, int32_t T, int32_t S_max, int32_t H_q,
                          int32_t H_kv, int32_t d, int32_t k, float sm_scale, float* dq,
                          float* dkc, float* dvc, int32_t pair_rows, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  bool empty = false;
  ix_status st = check_attn_shape(B, T, S_max, H_q, H_kv, d, k, &empty);
  if (st != IX_OK) return st;
  if ((st = check_pair_rows(pair_rows)) != IX_OK) return st;
  if (empty) return ok();
  if ((st = check_attn_ptrs(q, kc, vc, idx, out)) != IX_OK) return st;
  if (!lse || !dout || !dq || !dkc || !dvc)
    return fail(IX_ERR_INVALID, "NULL lse, dout or gradient pointer");
  if (!aligned16(out) || !aligned16(dout))
    return fail(IX_ERR_INVALID, "bf16 out/dout base pointers must be 16-byte aligned");
  if (!aligned4(lse) || !aligned4(dq) || !aligned4(dkc) || !aligned4(dvc))
    return fail(IX_ERR_INVALID, "fp32 lse and gradient pointers must be 4-byte aligned");
  if (!(sm_scale == sm_scale) || sm_scale == __builtin_inff() || sm_scale == -__builtin_inff())
    return fail(IX_ERR_INVALID, "sm_scale must be finite");
  if (ws) {
    if (!aligned16(ws)) return fail(IX_ERR_INVALID, "workspace must be 16-byte aligned");
    const size_t row_bytes = attn_pair_row_bytes(H_kv, d, pair_rows);
    if (ix::pair_rows_per_pass(B, T, S_max, k, row_bytes, ws_bytes) < 1)
      return fail(IX_ERR_WORKSPACE, "workspace of %zu bytes is below one query row's need (%zu)",
                  ws_bytes, ix::pair_layout(B, S_max, k, 1, row_bytes).total);
  } else if (ws_bytes != 0) {
    return fail(IX_ERR_WORKSPACE, "ws_bytes given without a workspace");
  }
  if ((st = debug_check_idx(idx, kv_len, B, T, S_max, k, stream)) != IX_OK) return st;
  hipError_t e = IX_LAUNCH(ix::launch_sparse_attn_bwd(q, kc, vc, idx, kv_len, out, lse, dout, B, T, S_max,
                                            H_q, H_kv, d, k, sm_scale, dq, dkc, dvc,
                                            pair_rows == IX_PAIR_ROWS_FP32, ws, ws_bytes, stream));
  if (e != hipSuccess) return hip_fail(e, "sparse_attn_bwd launch");
  return ok();
}

ix_status indexshare_group_bwd(const int32_t* idx, const int32_t* kv_len, int32_t n_layers,
                               const void* const* q, const void* const* kc, const void* const* vc,
                               const void* const* out, const float* const* lse,
                               const void* const* dout, int32_t B, int32_t T, int32_t S_max,
                               int32_t H_q, int32_t H_kv, int32_t d, int32_t k, float sm_scale,
                               float* const* dq, float* const* dkc, float* const* dvc,
                               int32_t pair_rows, void* ws, size_t ws_bytes, hipStream_t stream) {
  bool empty = false;
  ix_status st = check_attn_shape(B, T, S_max, H_q, H_kv, d, k, &empty);
  if (st != IX_OK) return st;
  if (n_layers < 1) return fail(IX_ERR_INVALID, "n_layers=%d must be >= 1", n_layers);
  if ((st = check_pair_rows(pair_rows)) != IX_OK) return st;
  if (empty) return ok();
  if (!q || !kc || !vc || !out || !lse || !dout || !dq || !dkc || !dvc)
    return fail(IX_ERR_INVALID, "NULL per-layer pointer array");
  for (int l = 0; l < n_layers; ++l) {
    if ((st = check_attn_ptrs(q[l], kc[l], vc[l], idx, out[l])) != IX_OK) return st;
    if (!lse[l] || !dout[l] || !dq[l] || !dkc[l] || !dvc[l])
      return fail(IX_ERR_INVALID, "layer %d: NULL lse, dout or gradient pointer", l);
    if (!aligned16(dout[l])) return fail(IX_ERR_INVALID, "layer %d: dout must be 16-byte aligned", l);
    if (!aligned16(out[l])) return fail(IX_ERR_INVALID, "layer %d: out must be 16-byte aligned", l);
    if (!aligned4(lse[l]) || !aligned4(dq[l]) || !aligned4(dkc[l]) || !aligned4(dvc[l]))
      return fail(IX_ERR_INVALID, "layer %d: fp32 lse and gradients must be 4-byte aligned", l);
  }
  if (!(sm_scale == sm_scale) || sm_scale == __builtin_inff() || sm_scale == -__builtin_inff())
    return fail(IX_ERR_INVALID, "sm_scale must be finite");
  if (!ws) return fail(IX_ERR_WORKSPACE, "the group backward needs a workspace");
  if (!aligned16(ws)) return fail(IX_ERR_INVALID, "workspace must be 16-byte aligned");
  const size_t row_bytes = attn_pair_row_bytes(H_kv, d, pair_rows);
  if (ix::pair_rows_per_pass(B, T, S_max, k, row_bytes, ws_bytes) < 1)
    return fail(IX_ERR_WORKSPACE, "workspace of %zu bytes is below one query row's need (%zu)",
                ws_bytes, ix::pair_layout(B, S_max, k, 1, row_bytes).total);
  if ((st = debug_check_idx(idx, kv_len, B, T, S_max, k, stream)) != IX_OK) return st;
  hipError_t e = IX_LAUNCH(ix::launch_sparse_attn_bwd_layers(n_layers, q, kc, vc, idx, kv_len, out, lse, dout,
                                                   B, T, S_max, H_q, H_kv, d, k, sm_scale, dq, dkc,
                                                   dvc, pair_rows == IX_PAIR_ROWS_FP32, ws,
                                                   ws_bytes, stream));
  if (e != hipSuccess) return hip_fail(e, "indexshare_group_bwd launch");
  return ok();
}

ix_status ix_indexer_kl(const void* q, const void* kc, const int32_t* idx, const int32_t* kv_len,
                        const float* lse, const float* sel_scores, int32_t B, int32_t T,
                        int32_t S_max, int32_t H_q, int32_t H_kv, int32_t d, int32_t k,
                        float sm_scale, float* loss, float* dscores, hipStream_t stream) {
  bool empty = false;
  ix_status st = check_attn_shape(B, T, S_max, H_q, H_kv, d, k, &empty);
  if (st != IX_OK) return st;
  if (empty) return ok();
  if (!q || !kc || !idx || !lse || !sel_scores || !loss || !dscores)
    return fail(IX_ERR_INVALID, "NULL q, kc, idx, lse, sel_scores, loss or dscores pointer");
  if (!aligned16(q) || !aligned16(kc))
    return fail(IX_ERR_INVALID, "bf16 q/kc base pointers must be 16-byte aligned");
  if (!(sm_scale == sm_scale) || sm_scale == __builtin_inff() || sm_scale == -__builtin_inff())
    return fail(IX_ERR_INVALID, "sm_scale must be finite");
  if ((st = debug_check_idx(idx, kv_len, B, T, S_max, k, stream)) != IX_OK) return st;
  hipError_t e = IX_LAUNCH(ix::launch_indexer_kl(q, kc, idx, kv_len, lse, sel_scores, B, T, S_max, H_q, H_kv,
                                       d, k, sm_scale, loss, dscores, stream));
  if (e != hipSuccess) return hip_fail(e, "ix_indexer_kl launch");
  return ok();
}

size_t ix_indexer_bwd_workspace_bytes(const ix_indexer_args* a, int32_t k, int32_t rows_per_pass,
                                      int32_t pair_rows) {
  bool empty = false;
  if (check_indexer(a, &empty) != IX_OK || empty || check_k(k) != IX_OK) return 0;
  if (rows_per_pass < 1 || !pair_rows_valid(pair_rows)) return 0;
  const int64_t rows = std::min<int64_t>(rows_per_pass, (int64_t)a->B * a->T);
  if (rows * k > ((int64_t)1 << 31)) return 0;
  return ix::pair_layout(a->B, a->S_max, k, rows, indexer_pair_row_bytes(a->d_I, pair_rows)).total;
}

ix_status ix_indexer_bwd(const ix_indexer_args* a, int32_t k, const int32_t* idx,
                         const float* dscores, float* dq_I, float* dw, float* dk_I,
                         int32_t pair_rows, void* ws, size_t ws_bytes, hipStream_t stream) {
  bool empty = false;
  ix_status st = check_indexer(a, &empty);
  if (st != IX_OK) return st;
  st = check_k(k);
  if (st != IX_OK) return st;
  if ((st = check_pair_rows(pair_rows)) != IX_OK) return st;
  if (empty) return ok();
  if (!idx || !dscores || !dq_I || !dw || !dk_I)
    return fail(IX_ERR_INVALID, "NULL idx, dscores, dq_I, dw or dk_I pointer");
  if (!aligned4(a->w) || !aligned4(idx) || !aligned4(dscores) || !aligned4(dq_I) || !aligned4(dw) ||
      !aligned4(dk_I))
    return fail(IX_ERR_INVALID, "w, idx, dscores and gradient pointers must be 4-byte aligned");
  if (ws) {
    if (!aligned16(ws)) return fail(IX_ERR_INVALID, "workspace must be 16-byte aligned");
    const size_t row_bytes = indexer_pair_row_bytes(a->d_I, pair_rows);
    if (ix::pair_rows_per_pass(a->B, a->T, a->S_max, k, row_bytes, ws_bytes) < 1)
      return fail(IX_ERR_WORKSPACE, "workspace of %zu bytes is below one query row's need (%zu)",
                  ws_bytes, ix::pair_layout(a->B, a->S_max, k, 1, row_bytes).total);
  } else if (ws_bytes != 0) {
    return fail(IX_ERR_WORKSPACE, "ws_bytes given without a workspace");
  }
  if ((st = debug_check_idx(idx, a->kv_len, a->B, a->T, a->S_max, k, stream)) != IX_OK) return st;
  hipError_t e = IX_LAUNCH(ix::launch_indexer_bwd(a->q, a->k, a->w, a->kv_len, idx, dscores, a->B, a->T,
                                        a->S_max, a->H_I, a->d_I, k, dq_I, dw, dk_I,
                                        pair_rows == IX_PAIR_ROWS_FP32, ws, ws_bytes, stream));
  if (e != hipSuccess) return hip_fail(e, "ix_indexer_bwd launch");
  return ok();
}

ix_status ix_debug_enable(int32_t on) {
  if (on != 0 && on != 1) return fail(IX_ERR_INVALID, "on=%d: 0 or 1", on);
  g_debug.store(on == 1);
  return ok();
}

ix_status ix_debug_read(ix_debug_status* status, int32_t reset, hipStream_t stream) {
  if (!status) return fail(IX_ERR_INVALID, "NULL status pointer");
  void* p = nullptr;
  hipError_t e = IX_LAUNCH(device_symbol(HIP_SYMBOL(debug_words), g_debug_ptr, stream, &p));
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  unsigned long long w[ix::kDbgWords] = {};
  if (e == hipSuccess) e = hipMemcpy(w, p, sizeof(w), hipMemcpyDeviceToHost);
  if (e == hipSuccess && reset) {
    const unsigned long long zero[ix::kDbgWords] = {};
    e = hipMemcpy(p, zero, sizeof(zero), hipMemcpyHostToDevice);
  }
  if (e != hipSuccess) return hip_fail(e, "ix_debug_read");
  status->idx_out_of_range = w[ix::kDbgIdxOutOfRange];
  status->topk_compactions = w[ix::kDbgTopkCompactions];
  status->topk_resweeps = w[ix::kDbgTopkResweeps];
  status->topk_split_recomputes = w[ix::kDbgTopkSplitRecomputes];
  status->topk_overflow = w[ix::kDbgTopkOverflow];
  return ok();
}

}  // extern "C"

#ifdef IX_TEST_HOOKS
// Test build only: the launch plans, for host tests of their invariants (no GPU needed).
// out[]: the plan's fields in the order listed; returns the number written.
extern "C" __attribute__((visibility("default"))) int32_t ix_test_attn_plan(
    int32_t B, int32_t T, int32_t H_q, int32_t H_kv, int32_t d, int32_t k, int32_t n_layers,
    int64_t* out) {
  const ix::AttnPlan p = ix::make_attn_plan(B, T, H_q, H_kv, d, k, n_layers);
  const int64_t v[] = {p.layers, p.n_splits, p.light ? 1 : 0, p.chunks, p.chunks_per_split,
                       (int64_t)p.part_bytes, (int64_t)p.ws_bytes};
  for (int i = 0; i < 7; ++i) out[i] = v[i];
  return 7;
}

extern "C" __attribute__((visibility("default"))) int32_t ix_test_topk_plan(
    const ix_indexer_args* a, int32_t k, int64_t* out) {
  const ix::TopkPlan p = ix::make_topk_plan(*a, k);
  const int64_t v[] = {p.qc, p.hc, p.g, p.gmax, p.qgroups, p.n_splits, p.split_len, p.cap,
                       p.ksplit, p.fb_cap, p.samp_tiles, p.fb_samp_tiles, p.units,
                       (int64_t)p.ws_bytes};
  for (int i = 0; i < 14; ++i) out[i] = v[i];
  return 14;
}
#endif

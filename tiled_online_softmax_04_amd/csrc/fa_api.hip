// C ABI of libfa.so: argument checks, dispatch, error reporting.  See include/fa.h.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include "../../include/fa.h"
#include "fa_launch.h"

namespace {

thread_local char g_last_error[512] = "";

fa_status fail(fa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

fa_status hip_fail(hipError_t e, const char* what) {
  return fail(FA_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool supported_head_dim(int d) { return d == 64 || d == 128; }

// One head's Q, K or V spans fewer than 2^31 bytes: the kernels address a head
// through a buffer descriptor with 32-bit byte offsets, and the few rows they
// read before a head's first valid row give negative offsets that must wrap
// past 2^31 and so fall outside the buffer (reading zeros).
constexpr long long kMaxHeadBytes = 1LL << 31;

}  // namespace

extern "C" {

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FA_ERR_WORKSPACE: return "workspace too small";
    case FA_ERR_HIP: return "HIP runtime error";
    default: break;
  }
  return "unknown status";
}

const char* fa_last_error(void) { return g_last_error; }

// Checks shared by fa_fwd and fa_fwd_partial.  Returns FA_OK with *empty set
// when there is nothing to compute.
static fa_status check_fwd(fa_dtype dt, const void* q, const void* k, const void* v,
                           const void* o, int batch, int heads_q, int heads_kv, int n, int m,
                           int d, int dv, float scale, int causal, const int32_t* seq_lens,
                           bool* empty, long long in_bytes) {
  *empty = false;
  if (dt != FA_DTYPE_F32 && dt != FA_DTYPE_F16 && dt != FA_DTYPE_BF16)
    return fail(FA_ERR_INVALID, "unknown dtype %d", (int)dt);
  if (batch < 0 || heads_q < 0 || heads_kv < 0 || n < 0 || m < 0 || d <= 0 || dv <= 0)
    return fail(FA_ERR_INVALID, "negative or zero size (batch=%d heads_q=%d heads_kv=%d n=%d "
                "m=%d d=%d dv=%d)", batch, heads_q, heads_kv, n, m, d, dv);
  if (heads_kv == 0 && heads_q != 0) return fail(FA_ERR_INVALID, "heads_kv is 0");
  if (heads_kv != 0 && heads_q % heads_kv != 0)
    return fail(FA_ERR_INVALID, "heads_q (%d) is not a multiple of heads_kv (%d)", heads_q,
                heads_kv);
  if (causal && n != m) return fail(FA_ERR_INVALID, "causal needs n == m (n=%d m=%d)", n, m);
  if (seq_lens && n != m)
    return fail(FA_ERR_INVALID, "seq_lens (left padding) needs n == m (n=%d m=%d)", n, m);
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(FA_ERR_INVALID, "scale must be finite and > 0 (got %g)", (double)scale);
  if ((long long)n * d * in_bytes >= kMaxHeadBytes || (long long)m * d * in_bytes >= kMaxHeadBytes ||
      (long long)m * dv * in_bytes >= kMaxHeadBytes)
    return fail(FA_ERR_INVALID, "one head of q, k or v spans 2^31 bytes or more");
  if (!supported_head_dim(d) || dv != d)
    return fail(FA_ERR_UNSUPPORTED, "head dims d=%d dv=%d (need d == dv in {64, 128})", d, dv);
  if (batch == 0 || heads_q == 0 || n == 0) {
    *empty = true;
    return FA_OK;
  }
  if (!q || !o) return fail(FA_ERR_INVALID, "null q or output");
  if (m > 0 && (!k || !v)) return fail(FA_ERR_INVALID, "null k or v");
  if (!aligned16(q) || !aligned16(o) || (m > 0 && (!aligned16(k) || !aligned16(v))))
    return fail(FA_ERR_INVALID, "tensor pointers must be 16-byte aligned");
  const long long grid = fa::fwd_grid_size((int)dt, batch, heads_q, n);
  if (grid >= (1LL << 31)) return fail(FA_ERR_INVALID, "grid too large (%lld)", grid);
  return FA_OK;
}

fa_status fa_fwd(fa_dtype dt, const void* q, const void* k, const void* v, void* o, int batch,
                 int heads_q, int heads_kv, int n, int m, int d, int dv, float scale, int causal,
                 const int32_t* seq_lens, void* stream) {
  g_last_error[0] = '\0';
  bool empty;
  const fa_status s = check_fwd(dt, q, k, v, o, batch, heads_q, heads_kv, n, m, d, dv, scale,
                                causal, seq_lens, &empty, dt == FA_DTYPE_F32 ? 4 : 2);
  if (s != FA_OK || empty) return s;
  fa::FwdArgs a{(int)dt, q, k, v, o, batch, heads_q, heads_kv, n, m, d, scale, causal ? 1 : 0,
                seq_lens, stream, 0, m, 0, nullptr, nullptr, 0, nullptr, 0, 0, 0};
  const hipError_t e = fa::launch_fwd(a);
  if (e != hipSuccess) return hip_fail(e, "fa_fwd launch");
  return FA_OK;
}

fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, fa_dtype out_dtype,
                     int batch, int heads_q, int heads_kv, int n, int m, int d, int dv,
                     float scale, float q_descale, float k_descale, float v_descale, int causal,
                     const int32_t* seq_lens, void* stream) {
  g_last_error[0] = '\0';
  // Shape, pointer and scale checks as fa_fwd (the bf16 kernel's row counts
  // stand in for the element size, which the checks do not use).
  bool empty;
  fa_status s = check_fwd(out_dtype, q, k, v, o, batch, heads_q, heads_kv, n, m, d, dv, scale,
                          causal, seq_lens, &empty, 1);
  if (s != FA_OK) return s;
  const float ds[3] = {q_descale, k_descale, v_descale};
  for (float x : ds)
    if (!(x > 0.f) || !isfinite(x))
      return fail(FA_ERR_INVALID, "descales must be finite and > 0 (got %g, %g, %g)",
                  (double)q_descale, (double)k_descale, (double)v_descale);
  const double c = (double)scale * q_descale * k_descale * 1.4426950408889634;
  if (!(c >= 1.1754943508222875e-38) || !(c < 3.4e38))
    return fail(FA_ERR_INVALID, "scale * q_descale * k_descale out of float32 range (%g)", c);
  if (empty) return FA_OK;
  const long long grid = fa::fwd_fp8_grid_size(batch, heads_q, n);
  if (grid >= (1LL << 31)) return fail(FA_ERR_INVALID, "grid too large (%lld)", grid);
  fa::Fp8Args a{(int)out_dtype, q, k, v, o, batch, heads_q, heads_kv, n, m, d, scale,
                q_descale, k_descale, v_descale, causal ? 1 : 0, seq_lens, stream};
  const hipError_t e = fa::launch_fwd_fp8(a);
  if (e != hipSuccess) return hip_fail(e, "fa_fwd_fp8 launch");
  return FA_OK;
}

fa_status fa_fwd_partial(fa_dtype dt, const void* q, const void* k, const void* v, float* o,
                         float* lse, int batch, int heads_q, int heads_kv, int n, int m, int d,
                         int dv, float scale, int causal, const int32_t* seq_lens,
                         int key_begin, int key_end, void* stream) {
  g_last_error[0] = '\0';
  bool empty;
  const fa_status s = check_fwd(dt, q, k, v, o, batch, heads_q, heads_kv, n, m, d, dv, scale,
                                causal, seq_lens, &empty, dt == FA_DTYPE_F32 ? 4 : 2);
  if (s != FA_OK) return s;
  if (key_begin < 0 || key_end < key_begin || key_end > m)
    return fail(FA_ERR_INVALID, "key range [%d, %d) outside [0, m = %d]", key_begin, key_end, m);
  if (empty) return FA_OK;
  if (!lse) return fail(FA_ERR_INVALID, "null lse");
  if (((uintptr_t)lse & 3u) != 0) return fail(FA_ERR_INVALID, "lse must be 4-byte aligned");
  fa::FwdArgs a{(int)dt, q, k, v, nullptr, batch, heads_q, heads_kv, n, m, d, scale,
                causal ? 1 : 0, seq_lens, stream, key_begin, key_end, 1, o, lse, 0, nullptr, 0,
                0, 0};
  const hipError_t e = fa::launch_fwd(a);
  if (e != hipSuccess) return hip_fail(e, "fa_fwd_partial launch");
  return FA_OK;
}

static fa_status check_decode_sizes(int num_seqs, int heads_q, int heads_kv, int d, int dv,
                                    int max_blocks_per_seq, int block_size);

fa_status fa_paged_prefill(fa_dtype dt, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const int32_t* seq_lens, int block_size,
                           int num_seqs, int heads_q, int heads_kv, int n, int d, int dv,
                           int num_blocks, int max_blocks_per_seq, float scale, int causal,
                           void* o, void* stream) {
  g_last_error[0] = '\0';
  if (dt != FA_DTYPE_F32 && dt != FA_DTYPE_F16 && dt != FA_DTYPE_BF16)
    return fail(FA_ERR_INVALID, "unknown dtype %d", (int)dt);
  fa_status s = check_decode_sizes(num_seqs, heads_q, heads_kv, d, dv, max_blocks_per_seq,
                                   block_size);
  if (s != FA_OK) return s;
  if (n < 0) return fail(FA_ERR_INVALID, "negative chunk length %d", n);
  if (num_blocks <= 0) return fail(FA_ERR_INVALID, "num_blocks must be > 0");
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(FA_ERR_INVALID, "scale must be finite and > 0 (got %g)", (double)scale);
  if ((long long)n * d * 2 >= kMaxHeadBytes) return fail(FA_ERR_INVALID, "chunk too long");
  if (dt == FA_DTYPE_F32) return fail(FA_ERR_UNSUPPORTED, "paged prefill supports f16 and bf16");
  if (max_blocks_per_seq > fa::max_paged_blocks())
    return fail(FA_ERR_UNSUPPORTED, "max_blocks_per_seq above %d", fa::max_paged_blocks());
  if (num_seqs == 0 || heads_q == 0 || n == 0) return FA_OK;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !o)
    return fail(FA_ERR_INVALID, "null pointer argument");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return fail(FA_ERR_INVALID, "tensor pointers must be 16-byte aligned");
  const long long grid = fa::fwd_grid_size((int)dt, num_seqs, heads_q, n);
  if (grid >= (1LL << 31)) return fail(FA_ERR_INVALID, "grid too large (%lld)", grid);
  fa::FwdArgs a{(int)dt, q, k_cache, v_cache, o, num_seqs, heads_q, heads_kv, n,
                max_blocks_per_seq * block_size, d, scale, causal ? 1 : 0, seq_lens, stream, 0,
                0, 0, nullptr, nullptr, 1, block_table, block_size, max_blocks_per_seq,
                num_blocks};
  const hipError_t e = fa::launch_fwd(a);
  if (e != hipSuccess) return hip_fail(e, "fa_paged_prefill launch");
  return FA_OK;
}

fa_status fa_merge(fa_dtype out_dtype, const float* o_parts, const float* lse_parts, int parts,
                   long long rows, int dv, void* o, float* lse_out, void* stream) {
  g_last_error[0] = '\0';
  if (out_dtype != FA_DTYPE_F32 && out_dtype != FA_DTYPE_F16 && out_dtype != FA_DTYPE_BF16)
    return fail(FA_ERR_INVALID, "unknown dtype %d", (int)out_dtype);
  if (parts <= 0 || rows < 0 || dv <= 0)
    return fail(FA_ERR_INVALID, "bad sizes (parts=%d rows=%lld dv=%d)", parts, rows, dv);
  if (dv % 4 != 0 || dv > 1024)
    return fail(FA_ERR_UNSUPPORTED, "dv must be a multiple of 4 up to 1024 (got %d)", dv);
  if (rows >= (1LL << 31)) return fail(FA_ERR_INVALID, "rows at or above 2^31");
  if (rows == 0) return FA_OK;
  if (!o_parts || !lse_parts || !o) return fail(FA_ERR_INVALID, "null pointer argument");
  if (!aligned16(o_parts) || !aligned16(o))
    return fail(FA_ERR_INVALID, "o_parts and o must be 16-byte aligned");
  if (((uintptr_t)lse_parts & 3u) != 0 || ((uintptr_t)lse_out & 3u) != 0)
    return fail(FA_ERR_INVALID, "lse arrays must be 4-byte aligned");
  fa::MergeArgs a{(int)out_dtype, o_parts, lse_parts, parts, rows, dv, o, lse_out, stream};
  const hipError_t e = fa::launch_merge(a);
  if (e != hipSuccess) return hip_fail(e, "fa_merge launch");
  return FA_OK;
}

static fa_status check_decode_sizes(int num_seqs, int heads_q, int heads_kv, int d, int dv,
                                    int max_blocks_per_seq, int block_size) {
  if (num_seqs < 0 || heads_q < 0 || heads_kv <= 0 || d <= 0 || dv <= 0)
    return fail(FA_ERR_INVALID, "bad sizes (num_seqs=%d heads_q=%d heads_kv=%d d=%d dv=%d)",
                num_seqs, heads_q, heads_kv, d, dv);
  if (block_size <= 0 || max_blocks_per_seq <= 0)
    return fail(FA_ERR_INVALID, "block_size (%d) and max_blocks_per_seq (%d) must be > 0",
                block_size, max_blocks_per_seq);
  if (heads_q % heads_kv != 0)
    return fail(FA_ERR_INVALID, "heads_q (%d) is not a multiple of heads_kv (%d)", heads_q,
                heads_kv);
  if (num_seqs > 65535) return fail(FA_ERR_INVALID, "num_seqs above 65535");
  if ((long long)max_blocks_per_seq * block_size >= (1LL << 31))
    return fail(FA_ERR_INVALID, "max_blocks_per_seq * block_size overflows int32");
  if (!supported_head_dim(d) || dv != d)
    return fail(FA_ERR_UNSUPPORTED, "head dims d=%d dv=%d (need d == dv in {64, 128})", d, dv);
  return FA_OK;
}

size_t fa_paged_decode_workspace_size(int num_seqs, int heads_q, int heads_kv, int dv,
                                      int max_blocks_per_seq, int block_size) {
  if (check_decode_sizes(num_seqs, heads_q, heads_kv, dv, dv, max_blocks_per_seq, block_size) !=
      FA_OK)
    return 0;
  const fa::DecodePlan p =
      fa::decode_plan(num_seqs, heads_q, heads_kv, max_blocks_per_seq, block_size);
  return fa::decode_workspace_bytes(p, num_seqs, heads_q, dv);
}

// Checks shared by fa_paged_decode and fa_paged_decode_noalloc.  Returns FA_OK
// with *empty set when there is nothing to compute, else FA_OK with the plan's
// workspace size in *need.
static fa_status check_decode(fa_dtype dt, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_table,
                              const int32_t* seq_lens, int block_size, int num_seqs, int heads_q,
                              int heads_kv, int d, int dv, int num_blocks,
                              int max_blocks_per_seq, float scale, const void* o, bool* empty,
                              size_t* need) {
  *empty = false;
  *need = 0;
  if (dt != FA_DTYPE_F32 && dt != FA_DTYPE_F16 && dt != FA_DTYPE_BF16)
    return fail(FA_ERR_INVALID, "unknown dtype %d", (int)dt);
  fa_status s = check_decode_sizes(num_seqs, heads_q, heads_kv, d, dv, max_blocks_per_seq,
                                   block_size);
  if (s != FA_OK) return s;
  if (num_blocks <= 0) return fail(FA_ERR_INVALID, "num_blocks must be > 0");
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(FA_ERR_INVALID, "scale must be finite and > 0 (got %g)", (double)scale);
  if ((long long)num_blocks * block_size * heads_kv * d >= (1LL << 40))
    return fail(FA_ERR_INVALID, "cache larger than 2^40 elements");
  if ((long long)num_blocks * block_size >= (1LL << 32))
    return fail(FA_ERR_INVALID, "cache holds 2^32 or more token rows");
  if (dt == FA_DTYPE_F32) return fail(FA_ERR_UNSUPPORTED, "paged decode supports f16 and bf16");
  if (num_seqs == 0 || heads_q == 0) {
    *empty = true;
    return FA_OK;
  }
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !o)
    return fail(FA_ERR_INVALID, "null pointer argument");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return fail(FA_ERR_INVALID, "tensor pointers must be 16-byte aligned");
  const fa::DecodePlan p =
      fa::decode_plan(num_seqs, heads_q, heads_kv, max_blocks_per_seq, block_size);
  if (p.max_splits > 65535)
    return fail(FA_ERR_UNSUPPORTED,
                "max_blocks_per_seq * block_size = %lld keys need %d splits of %d, above the "
                "65535 a launch grid holds",
                (long long)max_blocks_per_seq * block_size, p.max_splits, p.split_tokens);
  *need = fa::decode_workspace_bytes(p, num_seqs, heads_q, dv);
  return FA_OK;
}

fa_status fa_paged_decode(fa_dtype dt, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, const int32_t* seq_lens, int block_size,
                          int num_seqs, int heads_q, int heads_kv, int d, int dv, int num_blocks,
                          int max_blocks_per_seq, float scale, void* o, void* workspace,
                          size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  bool empty;
  size_t need;
  const fa_status s = check_decode(dt, q, k_cache, v_cache, block_table, seq_lens, block_size,
                                   num_seqs, heads_q, heads_kv, d, dv, num_blocks,
                                   max_blocks_per_seq, scale, o, &empty, &need);
  if (s != FA_OK || empty) return s;
  if (!workspace || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes,
                need);
  if (!aligned16(workspace)) return fail(FA_ERR_INVALID, "workspace must be 16-byte aligned");

  fa::DecodeArgs a{(int)dt, q,        k_cache,  v_cache,    block_table,        seq_lens,
                   block_size, num_seqs, heads_q, heads_kv, d, num_blocks, max_blocks_per_seq,
                   scale, o, workspace, stream};
  const hipError_t e = fa::launch_decode(a);
  if (e != hipSuccess) return hip_fail(e, "fa_paged_decode launch");
  return FA_OK;
}

fa_status fa_paged_decode_noalloc(fa_dtype dt, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, int block_size, int num_seqs,
                                  int heads_q, int heads_kv, int d, int dv, int num_blocks,
                                  int max_blocks_per_seq, float scale, void* o, void* stream) {
  g_last_error[0] = '\0';
  bool empty;
  size_t need;
  const fa_status s = check_decode(dt, q, k_cache, v_cache, block_table, seq_lens, block_size,
                                   num_seqs, heads_q, heads_kv, d, dv, num_blocks,
                                   max_blocks_per_seq, scale, o, &empty, &need);
  if (s != FA_OK || empty) return s;
  if (need > (size_t)FA_NOALLOC_SCRATCH_BYTES)
    return fail(FA_ERR_WORKSPACE,
                "these sizes need %zu bytes of split states, above the %zu-byte static scratch "
                "of fa_paged_decode_noalloc (use fa_paged_decode with a workspace)",
                need, (size_t)FA_NOALLOC_SCRATCH_BYTES);
  void* scratch = nullptr;
  hipError_t e = fa::decode_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "fa_paged_decode_noalloc scratch lookup");
  fa::DecodeArgs a{(int)dt, q,        k_cache,  v_cache,    block_table,        seq_lens,
                   block_size, num_seqs, heads_q, heads_kv, d, num_blocks, max_blocks_per_seq,
                   scale, o, scratch, stream};
  e = fa::launch_decode(a);
  if (e != hipSuccess) return hip_fail(e, "fa_paged_decode_noalloc launch");
  return FA_OK;
}

}  // extern "C"

// Internal interface between the C ABI (fa_api.hip) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

namespace fa {

struct FwdArgs {
  int dtype;  // 0 f32, 1 f16, 2 bf16 (fa_dtype values)
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int batch, heads_q, heads_kv, n, m, d;
  float scale;
  int causal;
  const int32_t* seq_lens;
  void* stream;
  // Key range [key_begin, key_end) (0 and m for a full call).  With partial,
  // the result goes to o_f32 (float32, normalised over the range) and lse
  // (natural log of the range's softmax denominator) instead of o.
  int key_begin, key_end;
  int partial;
  float* o_f32;
  float* lse;
  // Paged chunk (f16 / bf16): k and v are caches [num_blocks, block_size,
  // heads_kv, d] reached through block_table [batch, max_blocks]; seq_lens
  // holds the total lengths; the n query rows are each sequence's last n
  // tokens.
  int paged;
  const int32_t* block_table;
  int block_size, max_blocks, num_blocks;
};

// FP8 prefill: q, k, v are E4M3 codes [batch, heads, rows, d] with one
// descale factor each; o is out_dtype (0 f32, 1 f16, 2 bf16).
struct Fp8Args {
  int out_dtype;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int batch, heads_q, heads_kv, n, m, d;
  float scale, q_descale, k_descale, v_descale;
  int causal;
  const int32_t* seq_lens;
  void* stream;
};
long long fwd_fp8_grid_size(int batch, int heads_q, int n);
hipError_t launch_fwd_fp8(const Fp8Args& a);

// Merge of key-range pieces: o_parts [parts, rows, dv] and lse_parts
// [parts, rows] (float32) into o [rows, dv] of out_dtype and, if non-null,
// lse_out [rows].
struct MergeArgs {
  int out_dtype;
  const float* o_parts;
  const float* lse_parts;
  int parts;
  long long rows;
  int dv;
  void* o;
  float* lse_out;
  void* stream;
};
hipError_t launch_merge(const MergeArgs& a);

struct DecodeArgs {
  int dtype;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int block_size, num_seqs, heads_q, heads_kv, d, num_blocks, max_blocks_per_seq;
  float scale;
  void* o;
  void* workspace;
  void* stream;
};

// Number of workgroups fa_fwd launches (the host checks it fits a grid).
long long fwd_grid_size(int dtype, int batch, int heads_q, int n);
// Longest block table a paged prefill can stage (entries per sequence).
int max_paged_blocks();
hipError_t launch_fwd(const FwdArgs& a);

// Split size (tokens) and split count of the paged decode, from sizes only.
struct DecodePlan {
  int split_tokens;  // keys per split workgroup
  int max_splits;    // splits per sequence at max_blocks_per_seq * block_size keys
  int heads_per_wg;  // query heads of one KV group handled by one workgroup
  int subgroups;     // workgroups per (sequence, KV head, split)
};
DecodePlan decode_plan(int num_seqs, int heads_q, int heads_kv, int max_blocks_per_seq,
                       int block_size);
size_t decode_workspace_bytes(const DecodePlan& p, int num_seqs, int heads_q, int dv);
hipError_t launch_decode(const DecodeArgs& a);
// Device address of the calling thread's current device's copy of the static
// scratch array that fa_paged_decode_noalloc uses as its workspace (looked up
// once per device).
hipError_t decode_scratch(void** ptr);

// Compute units of the current device, rounded down to a multiple of the 8
// XCDs (so that workgroup i and its units i + grid, ... share an XCD); 0 if
// unknown.
inline int persistent_grid() {
  static std::mutex mu;
  static int cus[64] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    cus[dev] = n >= 8 ? n / 8 * 8 : -1;
  }
  return cus[dev] > 0 ? cus[dev] : 0;
}

}  // namespace fa

// Launch-side parameter blocks and launchers of the HIP kernels. Validation
// happens in the C-ABI layer before any of these is called; the launchers
// assume sizes and pointers are already checked.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkva {

enum Status { kOk = 0, kEinval = 1, kEunsupported = 2, kEworkspace = 3, kEhip = 4 };

// log2(e): the kernels run the softmax as exp2((s - m) * scale * log2(e)).
constexpr float kLog2eHost = 1.4426950408889634f;

struct DecodeParams {
  const void* q;              // [batch, n_heads, D]
  const void* k;              // contiguous [batch, cap, Hkv, D] or pool [nb, bs, Hkv, D]
  const void* v;
  void* o;                    // [batch, n_heads, D]
  const int32_t* seq_lens;    // [batch]
  const int32_t* block_table; // [batch, max_blocks_per_seq] (paged)
  float* ws_o;                // [n_ranges + batch, n_heads, D] partial outputs, slot = range + seq
  float* ws_ml;               // [n_ranges + batch, n_heads, 2] (m * scale * log2e, l)
  int* ws_cum;                // [batch + 2]: exclusive prefix of lengths, total, tokens per range
  int batch, n_heads, n_kv_heads, group;
  int kvs;                    // KV heads per workgroup slab
  int nslab;                  // n_kv_heads / kvs
  int n_ranges;               // equal token ranges the sequences are cut into
  int min_tokens_per_range;
  int max_seq_len;
  int max_blocks_per_seq, block_shift, num_blocks;
  int kv_capacity;
  float scale_log2;           // attention_scale * log2(e)
  // The arms of one layer (ext only): keys wider than values, sliding window,
  // logit softcap, ALiBi slopes, sink logits.
  bool ext;
  int v_head_dim;             // value width (ext; the key width is head_dim)
  int window;                 // > 0: keys within the last `window` positions
  float scale;                // attention_scale
  float softcap, inv_softcap; // softcap > 0: logit -> softcap * tanh(logit / softcap)
  const float* alibi;         // [n_heads] slopes or null
  const float* sinks;         // [n_heads] sink logits or null
};

int decode_max_ranges();
int decode_min_tokens_per_range();
int decode_heads_per_slab_max();
bool decode_supported(bool bf16, int head_dim);
bool decode_ext_supported(bool bf16, int head_dim, int v_head_dim);
int decode_lanes_per_row(bool bf16, int head_dim);
int launch_decode(bool bf16, bool paged, int head_dim, int gmax, const DecodeParams& p,
                  hipStream_t stream);
// The static scratch array of the allocation-free decode: its size, and the
// current device's address of it (null if the lookup fails).
size_t decode_scratch_bytes();
void* decode_scratch();

struct PrefillParams {
  const void* q;              // [batch, seq_q, n_heads, D]
  const void* k;              // contiguous [batch, cap, Hkv, D] or pool [nb, bs, Hkv, D]
  const void* v;
  void* o;                    // [batch, seq_q, n_heads, D]
  const int32_t* block_table; // [batch, max_blocks_per_seq] (paged)
  int batch, n_heads, n_kv_heads, group;
  int seq_q, seq_kv, position_offset;
  int max_blocks_per_seq, block_shift, num_blocks;
  int kv_capacity;
  int q_tiles;                // ceil(seq_q / BLOCK_M)
  float scale_log2;
  // Ragged batch (null cu_q: every sequence has seq_q, seq_kv, position_offset):
  const int32_t* cu_q;        // [batch + 1] first query row of each sequence in q and o
  const int32_t* kv_lens;     // [batch] keys of each sequence (its chunk is the last rows)
  int total_q;                // rows of q and o; seq_q is then the host bound on a chunk
};

bool prefill_supported(bool bf16, int head_dim);
int prefill_block_m();
int launch_prefill(bool bf16, bool paged, int head_dim, const PrefillParams& p, hipStream_t stream);

struct MlaParams {
  const void* q;              // [batch, n_heads, R + P]
  const void* latent;         // [batch, cap, R + P]
  void* o;                    // [batch, n_heads, R]
  const int32_t* seq_lens;
  __bf16* ws_o;               // [batch, nsplit, n_heads, R] O / l of each split (nsplit > 1 only)
  float* ws_ml;               // [batch, nsplit, n_heads, 2] (m * scale * log2e, l)
  int batch, n_heads, kv_capacity, max_seq_len;
  int nsplit, split_tokens;   // context split: nsplit pieces of split_tokens tokens
  float scale_log2;
  // Paged latent (null block_table: contiguous [batch, kv_capacity, R + P]):
  const int32_t* block_table; // [batch, max_blocks_per_seq]; latent is [num_blocks, bs, R + P]
  int max_blocks_per_seq, block_shift, num_blocks;
};

bool mla_supported(bool bf16, int kv_lora_rank, int rope_dim, int n_heads);
int mla_heads_per_group(int n_heads);   // heads served by one workgroup
int mla_tile_tokens();
int launch_mla(const MlaParams& p, hipStream_t stream);

// The push into a KV cache (contiguous when block_table is null, else a pool).
struct AppendParams {
  const void* k_new;          // [batch, n_new, row] new rows (K)
  const void* v_new;          // [batch, n_new, row] new rows (V); unused by the latent push
  void* k;                    // contiguous [batch, cap, row] or pool [nb, bs, row]
  void* v;
  const int32_t* positions;   // [batch] rows held before the push
  const int32_t* block_table; // [batch, max_blocks_per_seq] or null
  int batch, n_new;
  int64_t row_bytes;          // bytes of one token row
  int max_blocks_per_seq, block_shift, num_blocks;
  int kv_capacity;
};

struct MlaAppendParams {
  AppendParams rows;          // k = the latent cache or pool, n_new = 1
  const void* c_new;          // [batch, kv_lora_rank]
  const void* k_rot_new;      // [batch, rope_dim], not yet rotated
  int kv_lora_rank, rope_dim;
  double theta;               // <= 0: no rotation
};

// Batched per-head GEMM Y[b, h, :n] = W[h] (n x k) X[b, h, :k], bf16 in and
// out, fp32 accumulation; optionally copies copy_len elements of each X row
// (from element copy_src) to Y after the n outputs.
struct MlaProjParams {
  const void* x;              // X rows: element (b, h, i) at b * x_stride_b + h * x_stride_h + i
  const void* w;              // [n_heads, n, k]
  void* y;                    // element (b, h, j) at b * y_stride_b + h * y_stride_h + j
  int batch, n_heads, n, k;
  int64_t x_stride_b, x_stride_h, y_stride_b, y_stride_h;
  int copy_len, copy_src;
};

int launch_mla_proj(const MlaProjParams& p, hipStream_t stream);

int launch_kv_append(const AppendParams& p, hipStream_t stream);
int launch_mla_append(const MlaAppendParams& p, bool bf16, hipStream_t stream);

}  // namespace pkva

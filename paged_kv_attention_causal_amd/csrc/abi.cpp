// C-ABI entry points: argument validation, workspace sizing and kernel
// dispatch. Every check runs on the host before the first HIP call, so a
// rejected call enqueues nothing (and the checks run without a GPU).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <climits>
#include <cmath>
#include <cstdint>

#include "../../include/pkvattn.h"
#include "kernels.hpp"

namespace {

constexpr int kPrefillThreads = 256;
constexpr int kDecodeGroupMax = 8;        // largest n_heads / n_kv_heads the decode kernel packs
constexpr int kMlaTargetGroups = 256;     // workgroups that fill the 256 compute units
constexpr int64_t kMaxGrid = INT_MAX;

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool scale_ok(float s) { return std::isfinite(s) && s >= 0.0f; }

// The softmax multiplier the kernels use: exp2((s - m) * c) with
// c = attention_scale * log2(e). Every kernel masks a score by making it
// -inf and starts its running max at -inf, which needs c > 0 (-inf * 0 is
// NaN). A zero scale makes every visible score 0, i.e. uniform weights; the
// smallest normal float gives the same weights, exp2 of a product that
// small being exactly 1.
float scale_log2(float attention_scale) {
  return std::max(attention_scale * pkva::kLog2eHost, FLT_MIN);
}

bool heads_ok(int n_heads, int n_kv_heads, int head_dim) {
  return n_heads >= 1 && n_kv_heads >= 1 && head_dim >= 1 && n_heads % n_kv_heads == 0;
}

bool dtype_known(int dtype) { return dtype == PKVA_F32 || dtype == PKVA_BF16; }

// Largest power of two that divides n.
int pow2_divisor(int n) { return n & (-n); }

struct DecodeShape {
  int gmax, kvs, nslab, n_ranges;
  size_t ws_bytes;
};

// Upper bound on the equal token ranges the sequences are cut into (the
// launcher lowers it to the resident workgroup slots); sizes the workspace.
int decode_ranges(int batch, int max_seq_len) {
  const int64_t by_tokens = ceil_div((int64_t)batch * max_seq_len, pkva::decode_min_tokens_per_range());
  return (int)std::min<int64_t>(pkva::decode_max_ranges(), std::max<int64_t>(1, by_tokens));
}

size_t decode_ws_bytes(int batch, int n_heads, int head_dim, int max_seq_len) {
  const int64_t slots = (int64_t)decode_ranges(batch, max_seq_len) + batch;
  return (size_t)(slots * n_heads * (head_dim + 2) * (int64_t)sizeof(float) +
                  (int64_t)(batch + 2) * (int64_t)sizeof(int32_t));
}

int decode_shape(int dtype, int batch, int n_heads, int n_kv_heads, int head_dim, int max_seq_len,
                 DecodeShape* out) {
  const int group = n_heads / n_kv_heads;
  if (group > kDecodeGroupMax) return PKVA_EUNSUPPORTED;
  out->gmax = next_pow2(group);
  const int lanes = pkva::decode_lanes_per_row(dtype == PKVA_BF16, head_dim);
  const int ngroups = kPrefillThreads / lanes;
  int kvs = pow2_divisor(n_kv_heads);
  if (kvs > ngroups) kvs = ngroups;
  while (kvs * out->gmax > pkva::decode_heads_per_slab_max()) kvs /= 2;
  out->kvs = kvs;
  out->nslab = n_kv_heads / kvs;
  out->n_ranges = decode_ranges(batch, max_seq_len);
  out->ws_bytes = decode_ws_bytes(batch, n_heads, head_dim, max_seq_len);
  if (out->nslab > 65535) return PKVA_EINVAL;
  return PKVA_OK;
}

struct MlaShape {
  int nsplit, split_tokens;
  size_t ws_bytes;
};

MlaShape mla_shape(int batch, int n_heads, int kv_lora_rank, int max_seq_len) {
  MlaShape s;
  const int tile = pkva::mla_tile_tokens();
  const int64_t items = (int64_t)batch * (n_heads / pkva::mla_heads_per_group(n_heads));
  int64_t nsplit = items >= kMlaTargetGroups ? 1 : ceil_div(kMlaTargetGroups, items);
  const int64_t max_split = ceil_div(max_seq_len, tile);
  if (nsplit > max_split) nsplit = max_split;
  if (nsplit < 1) nsplit = 1;
  const int64_t per = ceil_div(ceil_div(max_seq_len, nsplit), tile) * tile;
  s.split_tokens = (int)per;
  s.nsplit = (int)ceil_div(max_seq_len, per);
  // per split and head: kv_lora_rank bf16 (O / l), then m and l in fp32
  s.ws_bytes = s.nsplit > 1
                   ? (size_t)((int64_t)batch * s.nsplit * n_heads * (kv_lora_rank * 2 + 2 * 4))
                   : 0;
  return s;
}

}  // namespace

extern "C" {

const char* pkva_status_string(int status) {
  switch (status) {
    case PKVA_OK: return "ok";
    case PKVA_EINVAL: return "invalid argument";
    case PKVA_EUNSUPPORTED: return "unsupported dtype or size";
    case PKVA_EWORKSPACE: return "workspace missing or too small";
    case PKVA_EHIP: return "HIP launch failed";
    case PKVA_ESCRATCH: return "sizes exceed the static scratch of the allocation-free call";
    default: return "unknown status";
  }
}

const char* pkva_version(void) { return "pkvattn 0.1.0 gfx950"; }

int attn_prefill(int dtype, const void* q, const void* k, const void* v, void* o, int batch,
                 int n_heads, int n_kv_heads, int head_dim, int seq_q, int seq_kv,
                 int position_offset, float attention_scale, const int32_t* block_table,
                 int max_blocks_per_seq, int block_size, int num_blocks, int kv_capacity,
                 void* stream) {
  if (!dtype_known(dtype)) return PKVA_EUNSUPPORTED;
  if (!q || !k || !v || !o) return PKVA_EINVAL;
  if (batch < 1 || !heads_ok(n_heads, n_kv_heads, head_dim)) return PKVA_EINVAL;
  if (seq_q < 1 || seq_kv < 1 || position_offset < 0) return PKVA_EINVAL;
  if ((int64_t)position_offset + seq_q > INT_MAX / 2) return PKVA_EINVAL;
  if (!scale_ok(attention_scale)) return PKVA_EINVAL;
  const bool paged = block_table != nullptr;
  if (paged) {
    if (!is_pow2(block_size) || max_blocks_per_seq < 1 || num_blocks < 1) return PKVA_EINVAL;
    if ((int64_t)max_blocks_per_seq * block_size < seq_kv) return PKVA_EINVAL;
    if ((int64_t)num_blocks * block_size > INT_MAX) return PKVA_EINVAL;   // pool rows index in 31 bits
  } else {
    if (kv_capacity < seq_kv) return PKVA_EINVAL;
    if ((int64_t)batch * kv_capacity > INT_MAX) return PKVA_EINVAL;       // cache rows index in 31 bits
  }
  const bool bf16 = dtype == PKVA_BF16;
  if (!pkva::prefill_supported(bf16, head_dim)) return PKVA_EUNSUPPORTED;
  const int64_t q_tiles = ceil_div(seq_q, pkva::prefill_block_m());
  if (q_tiles * batch * n_heads > kMaxGrid) return PKVA_EINVAL;

  pkva::PrefillParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o;
  p.block_table = block_table;
  p.batch = batch; p.n_heads = n_heads; p.n_kv_heads = n_kv_heads;
  p.group = n_heads / n_kv_heads;
  p.seq_q = seq_q; p.seq_kv = seq_kv; p.position_offset = position_offset;
  p.max_blocks_per_seq = paged ? max_blocks_per_seq : 0;
  p.block_shift = paged ? log2i(block_size) : 0;
  p.num_blocks = paged ? num_blocks : 0;
  p.kv_capacity = paged ? 0 : kv_capacity;
  p.q_tiles = (int)q_tiles;
  p.scale_log2 = scale_log2(attention_scale);
  const int rc = pkva::launch_prefill(bf16, paged, head_dim, p, (hipStream_t)stream);
  return rc == pkva::kOk ? PKVA_OK : (rc == pkva::kEunsupported ? PKVA_EUNSUPPORTED : PKVA_EHIP);
}

int attn_prefill_varlen(int dtype, const void* q, const void* k, const void* v, void* o,
                        int batch, int n_heads, int n_kv_heads, int head_dim,
                        const int32_t* cu_seqlens_q, const int32_t* seq_kv, int total_q,
                        int max_seq_q, float attention_scale, const int32_t* block_table,
                        int max_blocks_per_seq, int block_size, int num_blocks, int kv_capacity,
                        void* stream) {
  if (!dtype_known(dtype)) return PKVA_EUNSUPPORTED;
  if (!q || !k || !v || !o || !cu_seqlens_q || !seq_kv) return PKVA_EINVAL;
  if (batch < 1 || !heads_ok(n_heads, n_kv_heads, head_dim)) return PKVA_EINVAL;
  if (total_q < 1 || max_seq_q < 1) return PKVA_EINVAL;
  if (!scale_ok(attention_scale)) return PKVA_EINVAL;
  const bool paged = block_table != nullptr;
  if (paged) {
    if (!is_pow2(block_size) || max_blocks_per_seq < 1 || num_blocks < 1) return PKVA_EINVAL;
    if ((int64_t)max_blocks_per_seq * block_size > INT_MAX / 2) return PKVA_EINVAL;
    if ((int64_t)num_blocks * block_size > INT_MAX) return PKVA_EINVAL;   // pool rows index in 31 bits
  } else {
    if (kv_capacity < 1 || kv_capacity > INT_MAX / 2) return PKVA_EINVAL;
    if ((int64_t)batch * kv_capacity > INT_MAX) return PKVA_EINVAL;       // cache rows index in 31 bits
  }
  const bool bf16 = dtype == PKVA_BF16;
  if (!pkva::prefill_supported(bf16, head_dim)) return PKVA_EUNSUPPORTED;
  const int64_t q_tiles = ceil_div(max_seq_q, pkva::prefill_block_m());
  if (q_tiles * batch * n_heads > kMaxGrid) return PKVA_EINVAL;

  pkva::PrefillParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o;
  p.block_table = block_table;
  p.batch = batch; p.n_heads = n_heads; p.n_kv_heads = n_kv_heads;
  p.group = n_heads / n_kv_heads;
  p.seq_q = max_seq_q; p.seq_kv = 0; p.position_offset = 0;
  p.max_blocks_per_seq = paged ? max_blocks_per_seq : 0;
  p.block_shift = paged ? log2i(block_size) : 0;
  p.num_blocks = paged ? num_blocks : 0;
  p.kv_capacity = paged ? 0 : kv_capacity;
  p.q_tiles = (int)q_tiles;
  p.scale_log2 = scale_log2(attention_scale);
  p.cu_q = cu_seqlens_q; p.kv_lens = seq_kv; p.total_q = total_q;
  const int rc = pkva::launch_prefill(bf16, paged, head_dim, p, (hipStream_t)stream);
  return rc == pkva::kOk ? PKVA_OK : (rc == pkva::kEunsupported ? PKVA_EUNSUPPORTED : PKVA_EHIP);
}

size_t attn_decode_workspace_size(int batch, int n_heads, int n_kv_heads, int head_dim,
                                  int max_seq_len) {
  if (batch < 1 || !heads_ok(n_heads, n_kv_heads, head_dim) || max_seq_len < 1) return 0;
  return decode_ws_bytes(batch, n_heads, head_dim, max_seq_len);
}

static int decode_common(int dtype, bool paged, const void* q, const void* k, const void* v,
                         void* o, int batch, int n_heads, int n_kv_heads, int head_dim,
                         const int32_t* block_table, int max_blocks_per_seq, int block_size,
                         int num_blocks, const int32_t* seq_lens, int kv_capacity,
                         int max_seq_len, float attention_scale, void* workspace,
                         size_t workspace_bytes, void* stream, bool use_scratch = false,
                         const pkva_arms* arms = nullptr) {
  if (!dtype_known(dtype)) return PKVA_EUNSUPPORTED;
  if (!q || !k || !v || !o || !seq_lens) return PKVA_EINVAL;
  if (batch < 1 || !heads_ok(n_heads, n_kv_heads, head_dim) || max_seq_len < 1) return PKVA_EINVAL;
  if (!scale_ok(attention_scale)) return PKVA_EINVAL;
  if (paged) {
    if (!block_table) return PKVA_EINVAL;
    if (!is_pow2(block_size) || max_blocks_per_seq < 1 || num_blocks < 1) return PKVA_EINVAL;
    if ((int64_t)max_blocks_per_seq * block_size < max_seq_len) return PKVA_EINVAL;
    if ((int64_t)num_blocks * block_size > INT_MAX) return PKVA_EINVAL;   // pool rows index in 31 bits
  } else {
    if (kv_capacity < max_seq_len) return PKVA_EINVAL;
    if ((int64_t)batch * kv_capacity > INT_MAX) return PKVA_EINVAL;       // cache rows index in 31 bits
  }
  const bool bf16 = dtype == PKVA_BF16;
  // The value width sets the lane layout and the partials (the keys may be wider).
  int dv = head_dim;
  if (arms) {
    if (arms->v_head_dim < 0 || arms->window < 0) return PKVA_EINVAL;
    if (!std::isfinite(arms->softcap) || arms->softcap < 0.0f) return PKVA_EINVAL;
    if (arms->v_head_dim > 0) dv = arms->v_head_dim;
    if (!pkva::decode_ext_supported(bf16, head_dim, dv)) return PKVA_EUNSUPPORTED;
  } else {
    if (!pkva::decode_supported(bf16, head_dim)) return PKVA_EUNSUPPORTED;
  }
  DecodeShape sh;
  const int rc0 = decode_shape(dtype, batch, n_heads, n_kv_heads, dv, max_seq_len, &sh);
  if (rc0 != PKVA_OK) return rc0;
  if (use_scratch) {
    // Only now a HIP call (the symbol lookup, once per device); it enqueues nothing.
    if (sh.ws_bytes > pkva::decode_scratch_bytes()) return PKVA_ESCRATCH;
    workspace = pkva::decode_scratch();
    workspace_bytes = pkva::decode_scratch_bytes();
    if (!workspace) return PKVA_EHIP;
  }
  if (!workspace || workspace_bytes < sh.ws_bytes) return PKVA_EWORKSPACE;
  if (((uintptr_t)workspace & 15u) != 0) return PKVA_EWORKSPACE;

  pkva::DecodeParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o;
  p.seq_lens = seq_lens;
  p.block_table = block_table;
  const int64_t slots = (int64_t)sh.n_ranges + batch;
  p.ws_o = (float*)workspace;
  p.ws_ml = p.ws_o + slots * n_heads * dv;
  p.ws_cum = (int*)(p.ws_ml + slots * n_heads * 2);
  p.batch = batch; p.n_heads = n_heads; p.n_kv_heads = n_kv_heads;
  p.group = n_heads / n_kv_heads;
  p.kvs = sh.kvs; p.nslab = sh.nslab; p.n_ranges = sh.n_ranges;
  p.min_tokens_per_range = pkva::decode_min_tokens_per_range();
  p.max_seq_len = max_seq_len;
  p.max_blocks_per_seq = paged ? max_blocks_per_seq : 0;
  p.block_shift = paged ? log2i(block_size) : 0;
  p.num_blocks = paged ? num_blocks : 0;
  p.kv_capacity = paged ? 0 : kv_capacity;
  p.scale_log2 = scale_log2(attention_scale);
  if (arms) {
    p.ext = true;
    p.v_head_dim = dv;
    p.window = arms->window;
    p.scale = attention_scale;
    p.softcap = arms->softcap;
    p.inv_softcap = arms->softcap > 0.0f ? 1.0f / arms->softcap : 0.0f;
    p.alibi = arms->alibi_slopes;
    p.sinks = arms->sinks;
  }
  const int rc = pkva::launch_decode(bf16, paged, head_dim, sh.gmax, p, (hipStream_t)stream);
  return rc == pkva::kOk ? PKVA_OK : (rc == pkva::kEunsupported ? PKVA_EUNSUPPORTED : PKVA_EHIP);
}

int attn_decode_contig(int dtype, const void* q, const void* k_cache, const void* v_cache, void* o,
                       int batch, int n_heads, int n_kv_heads, int head_dim,
                       const int32_t* seq_lens, int kv_capacity, int max_seq_len,
                       float attention_scale, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return decode_common(dtype, false, q, k_cache, v_cache, o, batch, n_heads, n_kv_heads, head_dim,
                       nullptr, 0, 0, 0, seq_lens, kv_capacity, max_seq_len, attention_scale,
                       workspace, workspace_bytes, stream);
}

int attn_decode_paged(int dtype, const void* q, const void* k_pool, const void* v_pool, void* o,
                      int batch, int n_heads, int n_kv_heads, int head_dim,
                      const int32_t* block_table, int max_blocks_per_seq, int block_size,
                      int num_blocks, const int32_t* seq_lens, int max_seq_len,
                      float attention_scale, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return decode_common(dtype, true, q, k_pool, v_pool, o, batch, n_heads, n_kv_heads, head_dim,
                       block_table, max_blocks_per_seq, block_size, num_blocks, seq_lens, 0,
                       max_seq_len, attention_scale, workspace, workspace_bytes, stream);
}

int attn_decode_contig_ext(int dtype, const void* q, const void* k_cache, const void* v_cache,
                           void* o, int batch, int n_heads, int n_kv_heads, int head_dim,
                           const int32_t* seq_lens, int kv_capacity, int max_seq_len,
                           float attention_scale, const pkva_arms* arms, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!arms) return PKVA_EINVAL;
  return decode_common(dtype, false, q, k_cache, v_cache, o, batch, n_heads, n_kv_heads, head_dim,
                       nullptr, 0, 0, 0, seq_lens, kv_capacity, max_seq_len, attention_scale,
                       workspace, workspace_bytes, stream, false, arms);
}

int attn_decode_paged_ext(int dtype, const void* q, const void* k_pool, const void* v_pool, void* o,
                          int batch, int n_heads, int n_kv_heads, int head_dim,
                          const int32_t* block_table, int max_blocks_per_seq, int block_size,
                          int num_blocks, const int32_t* seq_lens, int max_seq_len,
                          float attention_scale, const pkva_arms* arms, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!arms) return PKVA_EINVAL;
  return decode_common(dtype, true, q, k_pool, v_pool, o, batch, n_heads, n_kv_heads, head_dim,
                       block_table, max_blocks_per_seq, block_size, num_blocks, seq_lens, 0,
                       max_seq_len, attention_scale, workspace, workspace_bytes, stream, false,
                       arms);
}

int attn_decode_paged_noalloc(int dtype, const void* q, const void* k_pool, const void* v_pool,
                              void* o, int batch, int n_heads, int n_kv_heads, int head_dim,
                              const int32_t* block_table, int max_blocks_per_seq, int block_size,
                              int num_blocks, const int32_t* seq_lens, int max_seq_len,
                              float attention_scale, void* stream) {
  return decode_common(dtype, true, q, k_pool, v_pool, o, batch, n_heads, n_kv_heads, head_dim,
                       block_table, max_blocks_per_seq, block_size, num_blocks, seq_lens, 0,
                       max_seq_len, attention_scale, nullptr, 0, stream, /*use_scratch=*/true);
}

int kv_append(int dtype, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
              int batch, int n_kv_heads, int head_dim, int n_new, const int32_t* positions,
              const int32_t* block_table, int max_blocks_per_seq, int block_size, int num_blocks,
              int kv_capacity, void* stream) {
  if (!dtype_known(dtype)) return PKVA_EUNSUPPORTED;
  if (!k_new || !v_new || !k_cache || !v_cache || !positions) return PKVA_EINVAL;
  if (batch < 1 || n_kv_heads < 1 || head_dim < 1 || n_new < 1) return PKVA_EINVAL;
  const bool paged = block_table != nullptr;
  if (paged) {
    if (!is_pow2(block_size) || max_blocks_per_seq < 1 || num_blocks < 1) return PKVA_EINVAL;
  } else {
    if (kv_capacity < 1) return PKVA_EINVAL;
  }
  pkva::AppendParams p{};
  p.k_new = k_new; p.v_new = v_new; p.k = k_cache; p.v = v_cache;
  p.positions = positions; p.block_table = block_table;
  p.batch = batch; p.n_new = n_new;
  p.row_bytes = (int64_t)n_kv_heads * head_dim * (dtype == PKVA_BF16 ? 2 : 4);
  p.max_blocks_per_seq = paged ? max_blocks_per_seq : 0;
  p.block_shift = paged ? log2i(block_size) : 0;
  p.num_blocks = paged ? num_blocks : 0;
  p.kv_capacity = paged ? 0 : kv_capacity;
  const int rc = pkva::launch_kv_append(p, (hipStream_t)stream);
  return rc == pkva::kOk ? PKVA_OK : (rc == pkva::kEinval ? PKVA_EINVAL : PKVA_EHIP);
}

int mla_append_latent(int dtype, const void* c_new, const void* k_rot_new, void* latent, int batch,
                      int kv_lora_rank, int qk_rope_head_dim, const int32_t* positions,
                      float rope_theta, const int32_t* block_table, int max_blocks_per_seq,
                      int block_size, int num_blocks, int kv_capacity, void* stream) {
  if (!dtype_known(dtype)) return PKVA_EUNSUPPORTED;
  if (!c_new || !latent || !positions) return PKVA_EINVAL;
  if (qk_rope_head_dim > 0 && !k_rot_new) return PKVA_EINVAL;
  if (batch < 1 || kv_lora_rank < 1 || qk_rope_head_dim < 0 || qk_rope_head_dim % 2 != 0)
    return PKVA_EINVAL;
  if (!std::isfinite(rope_theta)) return PKVA_EINVAL;
  const bool paged = block_table != nullptr;
  if (paged) {
    if (!is_pow2(block_size) || max_blocks_per_seq < 1 || num_blocks < 1) return PKVA_EINVAL;
  } else {
    if (kv_capacity < 1) return PKVA_EINVAL;
  }
  pkva::MlaAppendParams p{};
  p.rows.k = latent;
  p.rows.positions = positions; p.rows.block_table = block_table;
  p.rows.batch = batch; p.rows.n_new = 1;
  p.rows.row_bytes = (int64_t)(kv_lora_rank + qk_rope_head_dim) * (dtype == PKVA_BF16 ? 2 : 4);
  p.rows.max_blocks_per_seq = paged ? max_blocks_per_seq : 0;
  p.rows.block_shift = paged ? log2i(block_size) : 0;
  p.rows.num_blocks = paged ? num_blocks : 0;
  p.rows.kv_capacity = paged ? 0 : kv_capacity;
  p.c_new = c_new; p.k_rot_new = k_rot_new;
  p.kv_lora_rank = kv_lora_rank; p.rope_dim = qk_rope_head_dim;
  p.theta = rope_theta;
  const int rc = pkva::launch_mla_append(p, dtype == PKVA_BF16, (hipStream_t)stream);
  return rc == pkva::kOk ? PKVA_OK : PKVA_EHIP;
}

int mla_absorb_q(int dtype, const void* q, const void* k_b, void* q_abs, int batch, int n_heads,
                 int qk_nope_head_dim, int qk_rope_head_dim, int kv_lora_rank, void* stream) {
  if (!dtype_known(dtype)) return PKVA_EUNSUPPORTED;
  if (!q || !k_b || !q_abs) return PKVA_EINVAL;
  if (batch < 1 || n_heads < 1 || qk_nope_head_dim < 1 || qk_rope_head_dim < 0 ||
      kv_lora_rank < 1)
    return PKVA_EINVAL;
  // bf16, 16-byte rows pieces: k steps of 16, outputs in tiles of 32, the rope
  // part in 16-byte chunks.
  if (dtype != PKVA_BF16 || qk_nope_head_dim % 16 != 0 || kv_lora_rank % 32 != 0 ||
      qk_rope_head_dim % 8 != 0)
    return PKVA_EUNSUPPORTED;
  if ((((uintptr_t)q | (uintptr_t)k_b | (uintptr_t)q_abs) & 15u) != 0) return PKVA_EINVAL;
  pkva::MlaProjParams p{};
  p.x = q; p.w = k_b; p.y = q_abs;
  p.batch = batch; p.n_heads = n_heads; p.n = kv_lora_rank; p.k = qk_nope_head_dim;
  const int64_t qw = qk_nope_head_dim + qk_rope_head_dim, aw = kv_lora_rank + qk_rope_head_dim;
  p.x_stride_b = n_heads * qw; p.x_stride_h = qw;
  p.y_stride_b = n_heads * aw; p.y_stride_h = aw;
  p.copy_len = qk_rope_head_dim; p.copy_src = qk_nope_head_dim;
  const int rc = pkva::launch_mla_proj(p, (hipStream_t)stream);
  return rc == pkva::kOk ? PKVA_OK : (rc == pkva::kEinval ? PKVA_EINVAL : PKVA_EHIP);
}

int mla_up_proj(int dtype, const void* o_lat, const void* v_b, void* out, int batch, int n_heads,
                int kv_lora_rank, int v_head_dim, void* stream) {
  if (!dtype_known(dtype)) return PKVA_EUNSUPPORTED;
  if (!o_lat || !v_b || !out) return PKVA_EINVAL;
  if (batch < 1 || n_heads < 1 || kv_lora_rank < 1 || v_head_dim < 1) return PKVA_EINVAL;
  if (dtype != PKVA_BF16 || kv_lora_rank % 16 != 0 || v_head_dim % 32 != 0)
    return PKVA_EUNSUPPORTED;
  if ((((uintptr_t)o_lat | (uintptr_t)v_b | (uintptr_t)out) & 15u) != 0) return PKVA_EINVAL;
  pkva::MlaProjParams p{};
  p.x = o_lat; p.w = v_b; p.y = out;
  p.batch = batch; p.n_heads = n_heads; p.n = v_head_dim; p.k = kv_lora_rank;
  p.x_stride_b = (int64_t)n_heads * kv_lora_rank; p.x_stride_h = kv_lora_rank;
  p.y_stride_b = (int64_t)n_heads * v_head_dim; p.y_stride_h = v_head_dim;
  p.copy_len = 0; p.copy_src = 0;
  const int rc = pkva::launch_mla_proj(p, (hipStream_t)stream);
  return rc == pkva::kOk ? PKVA_OK : (rc == pkva::kEinval ? PKVA_EINVAL : PKVA_EHIP);
}

size_t mla_decode_workspace_size(int batch, int n_heads, int kv_lora_rank, int max_seq_len) {
  if (batch < 1 || n_heads < 1 || kv_lora_rank < 1 || max_seq_len < 1) return 0;
  if (!pkva::mla_supported(true, kv_lora_rank, 64, n_heads)) return 0;
  return mla_shape(batch, n_heads, kv_lora_rank, max_seq_len).ws_bytes;
}

static int mla_common(int dtype, const void* q_abs, const void* latent, void* o_lat, int batch,
                      int n_heads, int kv_lora_rank, int qk_rope_head_dim,
                      const int32_t* block_table, int max_blocks_per_seq, int block_size,
                      int num_blocks, const int32_t* seq_lens, int kv_capacity, int max_seq_len,
                      float attention_scale, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (!dtype_known(dtype)) return PKVA_EUNSUPPORTED;
  if (!q_abs || !latent || !o_lat || !seq_lens) return PKVA_EINVAL;
  if (batch < 1 || n_heads < 1 || kv_lora_rank < 1 || qk_rope_head_dim < 0) return PKVA_EINVAL;
  if (max_seq_len < 1) return PKVA_EINVAL;
  const bool paged = block_table != nullptr;
  if (paged) {
    if (!is_pow2(block_size) || max_blocks_per_seq < 1 || num_blocks < 1) return PKVA_EINVAL;
    if ((int64_t)max_blocks_per_seq * block_size < max_seq_len) return PKVA_EINVAL;
    if ((int64_t)num_blocks * block_size > INT_MAX) return PKVA_EINVAL;   // pool rows index in 31 bits
  } else {
    if (kv_capacity < max_seq_len) return PKVA_EINVAL;
  }
  if (!scale_ok(attention_scale)) return PKVA_EINVAL;
  if (!pkva::mla_supported(dtype == PKVA_BF16, kv_lora_rank, qk_rope_head_dim, n_heads))
    return PKVA_EUNSUPPORTED;
  const MlaShape sh = mla_shape(batch, n_heads, kv_lora_rank, max_seq_len);
  if ((int64_t)batch * (n_heads / pkva::mla_heads_per_group(n_heads)) * sh.nsplit > kMaxGrid)
    return PKVA_EINVAL;
  if (sh.ws_bytes > 0) {
    if (!workspace || workspace_bytes < sh.ws_bytes) return PKVA_EWORKSPACE;
    if (((uintptr_t)workspace & 15u) != 0) return PKVA_EWORKSPACE;
  }

  pkva::MlaParams p{};
  p.q = q_abs; p.latent = latent; p.o = o_lat; p.seq_lens = seq_lens;
  p.ws_o = (__bf16*)workspace;
  p.ws_ml = sh.ws_bytes > 0 ? (float*)(p.ws_o + (int64_t)batch * sh.nsplit * n_heads * kv_lora_rank)
                            : nullptr;
  p.batch = batch; p.n_heads = n_heads; p.kv_capacity = paged ? 0 : kv_capacity;
  p.max_seq_len = max_seq_len;
  p.nsplit = sh.nsplit; p.split_tokens = sh.split_tokens;
  p.scale_log2 = scale_log2(attention_scale);
  p.block_table = block_table;
  p.max_blocks_per_seq = paged ? max_blocks_per_seq : 0;
  p.block_shift = paged ? log2i(block_size) : 0;
  p.num_blocks = paged ? num_blocks : 0;
  const int rc = pkva::launch_mla(p, (hipStream_t)stream);
  return rc == pkva::kOk ? PKVA_OK : PKVA_EHIP;
}

int mla_decode_latent(int dtype, const void* q_abs, const void* latent, void* o_lat, int batch,
                      int n_heads, int kv_lora_rank, int qk_rope_head_dim,
                      const int32_t* seq_lens, int kv_capacity, int max_seq_len,
                      float attention_scale, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return mla_common(dtype, q_abs, latent, o_lat, batch, n_heads, kv_lora_rank, qk_rope_head_dim,
                    nullptr, 0, 0, 0, seq_lens, kv_capacity, max_seq_len, attention_scale,
                    workspace, workspace_bytes, stream);
}

int mla_decode_latent_paged(int dtype, const void* q_abs, const void* latent_pool, void* o_lat,
                            int batch, int n_heads, int kv_lora_rank, int qk_rope_head_dim,
                            const int32_t* block_table, int max_blocks_per_seq, int block_size,
                            int num_blocks, const int32_t* seq_lens, int max_seq_len,
                            float attention_scale, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (!block_table) return PKVA_EINVAL;
  return mla_common(dtype, q_abs, latent_pool, o_lat, batch, n_heads, kv_lora_rank,
                    qk_rope_head_dim, block_table, max_blocks_per_seq, block_size, num_blocks,
                    seq_lens, 0, max_seq_len, attention_scale, workspace, workspace_bytes, stream);
}

}  // extern "C"

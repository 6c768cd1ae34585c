// The push of push-then-attend: this step's K/V rows, or this token's MLA
// latent row, written into the cache through the block table before the
// attention reads it (frink-models 0.38.0 src/decoder/attn_block.rs,
// push_and_attend_row: push to whichever backing, then attend;
// kopitiam-runtime 0.2.4 src/attention.rs, attention_forward appends before
// scoring; frink-models 0.31.0 src/mla/mod.rs, mla_forward_token and
// absorbed_attention: the latent row is c followed by k_rot, which is
// rotated once, before every head shares it).
//
// Row i of sequence b becomes token t = positions[b] + i, at cache row
// (b, t) of a contiguous cache or at row t % block_size of block
// block_table[b][t / block_size] of a pool. A token row ([Hkv, D] for K/V,
// [R + P] for the latent) is contiguous at both ends, so the copy moves
// whole 16-byte chunks, one per thread, with coalesced loads and stores.
// A row whose target lies outside the cache (negative position, past the
// capacity or the table, a block id outside the pool) is not written.
//
// The rotary embedding turns pair (x[2i], x[2i+1]) of k_rot by
// position * theta^(-2i/P) (interleaved pairs). It is computed in double
// precision and rounded once to the storage type, so the stored value is
// the correctly rounded rotation whatever the position.
#include "common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace pkva {

namespace {

constexpr int kThreads = 256;

// Cache row index of token t of sequence b, or -1 when it lies outside.
__device__ __forceinline__ int64_t target_row(const AppendParams& p, int b, int64_t t) {
  if (t < 0) return -1;
  if (p.block_table == nullptr) {
    return t < p.kv_capacity ? (int64_t)b * p.kv_capacity + t : -1;
  }
  const int64_t blk = t >> p.block_shift;
  if (blk >= p.max_blocks_per_seq) return -1;
  const int id = p.block_table[(int64_t)b * p.max_blocks_per_seq + blk];
  if (id < 0 || id >= p.num_blocks) return -1;
  return ((int64_t)id << p.block_shift) + (t & ((1 << p.block_shift) - 1));
}

// One thread per CHUNK-byte piece of a token row, for K and V together.
template <int CHUNK>
__global__ __launch_bounds__(kThreads) void kv_append_kernel(AppendParams p) {
  using V = typename std::conditional<CHUNK == 16, uint4,
            typename std::conditional<CHUNK == 8, uint2,
            typename std::conditional<CHUNK == 4, uint32_t, uint16_t>::type>::type>::type;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t per_row = p.row_bytes / CHUNK;
  if (idx >= (int64_t)p.batch * p.n_new * per_row) return;
  const int64_t r = idx / per_row;          // (b, i) row of the new rows
  const int64_t ch = idx % per_row;
  const int b = (int)(r / p.n_new), i = (int)(r % p.n_new);
  const int64_t dst = target_row(p, b, (int64_t)p.positions[b] + i);
  if (dst < 0) return;
  const int64_t so = r * p.row_bytes + ch * CHUNK;
  const int64_t dofs = dst * p.row_bytes + ch * CHUNK;
  const V kx = *(const V*)((const char*)p.k_new + so);
  const V vx = *(const V*)((const char*)p.v_new + so);
  *(V*)((char*)p.k + dofs) = kx;
  *(V*)((char*)p.v + dofs) = vx;
}

// double -> bf16 rounded to nearest even in one step: truncate to float, mark
// an inexact truncation in the lowest bit (round to odd), then round the float
// to bf16; two extra bits of precision make the second rounding exact.
__device__ __forceinline__ __bf16 to_bf16(double x) {
  float f = __double2float_rz(x);
  uint32_t u = __float_as_uint(f);
  if ((double)f != x && (u & 0x7f800000u) != 0x7f800000u) u |= 1u;
  return (__bf16)__uint_as_float(u);
}

// One workgroup per sequence: c is copied in 16-byte chunks (or elements),
// k_rot is rotated pair by pair.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void mla_append_kernel(MlaAppendParams p) {
  using T = typename std::conditional<BF16, __bf16, float>::type;
  const int b = blockIdx.x;
  const int W = p.kv_lora_rank + p.rope_dim;
  const int64_t dst = target_row(p.rows, b, (int64_t)p.rows.positions[b]);
  if (dst < 0) return;
  T* row = (T*)p.rows.k + dst * W;
  const T* c = (const T*)p.c_new + (int64_t)b * p.kv_lora_rank;
  const int cbytes = p.kv_lora_rank * (int)sizeof(T);
  if ((cbytes % 16) == 0 && ((uintptr_t)row % 16) == 0) {
    for (int j = threadIdx.x; j < cbytes / 16; j += kThreads)
      ((uint4*)row)[j] = ((const uint4*)c)[j];
  } else {
    for (int j = threadIdx.x; j < p.kv_lora_rank; j += kThreads) row[j] = c[j];
  }
  const T* kr = (const T*)p.k_rot_new + (int64_t)b * p.rope_dim;
  T* out = row + p.kv_lora_rank;
  const double pos = (double)p.rows.positions[b];
  for (int i = threadIdx.x; i < p.rope_dim / 2; i += kThreads) {
    const double a = (double)(float)kr[2 * i];
    const double bb = (double)(float)kr[2 * i + 1];
    if (p.theta > 0.0) {
      const double ang = pos * pow(p.theta, -2.0 * i / p.rope_dim);
      double s, co;
      sincos(ang, &s, &co);
      const double y0 = a * co - bb * s;
      const double y1 = a * s + bb * co;
      if constexpr (BF16) {
        out[2 * i] = to_bf16(y0);
        out[2 * i + 1] = to_bf16(y1);
      } else {
        out[2 * i] = (float)y0;
        out[2 * i + 1] = (float)y1;
      }
    } else {
      out[2 * i] = kr[2 * i];
      out[2 * i + 1] = kr[2 * i + 1];
    }
  }
}

}  // namespace

int launch_kv_append(const AppendParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.batch * p.n_new;
  auto go = [&](auto kernel, int chunk) {
    const int64_t n = rows * (p.row_bytes / chunk);
    const int64_t grid = (n + kThreads - 1) / kThreads;
    if (grid > INT32_MAX) return kEinval;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError() == hipSuccess ? kOk : kEhip;
  };
  const uintptr_t align = (uintptr_t)p.k_new | (uintptr_t)p.v_new | (uintptr_t)p.k |
                          (uintptr_t)p.v | (uintptr_t)p.row_bytes;
  if ((align & 15u) == 0) return go(kv_append_kernel<16>, 16);
  if ((align & 7u) == 0) return go(kv_append_kernel<8>, 8);
  if ((align & 3u) == 0) return go(kv_append_kernel<4>, 4);
  return go(kv_append_kernel<2>, 2);
}

int launch_mla_append(const MlaAppendParams& p, bool bf16, hipStream_t stream) {
  if (bf16) {
    hipLaunchKernelGGL(mla_append_kernel<true>, dim3(p.rows.batch), dim3(kThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL(mla_append_kernel<false>, dim3(p.rows.batch), dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError() == hipSuccess ? kOk : kEhip;
}

}  // namespace pkva

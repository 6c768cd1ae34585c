// The per-head projections around the absorbed MLA attention (frink-models
// 0.31.0 src/mla/mod.rs, absorbed_attention and the MlaKvB::Split doc):
//   absorb:  q_abs[b, h] = [k_b[h] q_nope[b, h] | q_rot[b, h]],  k_b[h] is [R, qk_nope]
//   up-proj: out[b, h]   = v_b[h] o_lat[b, h],                    v_b[h] is [v_dim, R]
// Both are batched GEMMs with one weight matrix per head: Y[b, h, n] =
// sum_k W[h][n][k] X[b, h, k], the batch as the small dimension. At decode
// batch sizes they read every weight byte once and are bound by HBM.
//
// One wave computes a 32 x 32 tile Y^T[n0 .. n0+31][b0 .. b0+31] of one head
// on 32x32x16 bf16 MFMAs over the whole K: the A operand (W rows, 8
// consecutive k per lane) and the B operand (X rows, likewise) are 16-byte
// loads straight from global memory, with no reuse inside the wave to stage
// through LDS (a weight byte feeds the 32 batch rows of its tile; the X rows
// of a head are shared by its N / 32 tiles through the L2). In the
// accumulator lane l holds batch row b0 + l % 32 and 16 of the 32 outputs,
// in runs of four, so each run leaves as one 8-byte store.
#include "common.hpp"
#include "kernels.hpp"

namespace pkva {

namespace {

constexpr int kWaves = 4;
constexpr int kKB = 8;      // MFMA k-steps whose operands are loaded together

__global__ __launch_bounds__(64 * kWaves) void mla_proj_kernel(MlaProjParams p) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int lr = lane % 32, hf = lane / 32;
  const int n_tiles = p.n / 32, b_tiles = (p.batch + 31) / 32;
  const int64_t tile = (int64_t)blockIdx.x * kWaves + wave;
  if (tile >= (int64_t)p.n_heads * n_tiles * b_tiles) return;
  // Tiles of one head adjacent (they share the head's X rows), N fastest.
  const int nt = (int)(tile % n_tiles);
  const int bt = (int)((tile / n_tiles) % b_tiles);
  const int h = (int)(tile / ((int64_t)n_tiles * b_tiles));
  const int n0 = nt * 32, b0 = bt * 32;
  const int b = b0 + lr;
  const bool live = b < p.batch;

  const __bf16* wrow = (const __bf16*)p.w + ((int64_t)h * p.n + n0 + lr) * p.k + 8 * hf;
  const __bf16* xrow = (const __bf16*)p.x + (int64_t)b * p.x_stride_b + (int64_t)h * p.x_stride_h +
                       8 * hf;
  f32x16_t acc = f32x16_t{};
  const int ksteps = p.k / 16;
  for (int k0 = 0; k0 < ksteps; k0 += kKB) {
    bf16x8_t a[kKB], bb[kKB];
#pragma unroll
    for (int j = 0; j < kKB; ++j) {
      if (k0 + j < ksteps) {
        a[j] = *(const bf16x8_t*)(wrow + 16 * (k0 + j));
        bb[j] = live ? *(const bf16x8_t*)(xrow + 16 * (k0 + j)) : bf16x8_t{};
      }
    }
#pragma unroll
    for (int j = 0; j < kKB; ++j)
      if (k0 + j < ksteps) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], bb[j], acc, 0, 0, 0);
  }
  if (live) {
    __bf16* yrow = (__bf16*)p.y + (int64_t)b * p.y_stride_b + (int64_t)h * p.y_stride_h + n0;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const bf16x4_t v = {(__bf16)acc[4 * g4 + 0], (__bf16)acc[4 * g4 + 1], (__bf16)acc[4 * g4 + 2],
                          (__bf16)acc[4 * g4 + 3]};
      *(bf16x4_t*)(yrow + 8 * g4 + 4 * hf) = v;
    }
    // The absorbed query carries the rope part after the projected part: the
    // head's first N tile copies it (16 bytes per step, two lanes per row).
    if (p.copy_len > 0 && nt == 0) {
      const char* src = (const char*)(xrow - 8 * hf) + (int64_t)p.copy_src * 2;
      char* dst = (char*)(yrow - n0) + (int64_t)p.n * 2;
      for (int c = 16 * hf; c < p.copy_len * 2; c += 32)
        *(uint4*)(dst + c) = *(const uint4*)(src + c);
    }
  }
}

}  // namespace

int launch_mla_proj(const MlaProjParams& p, hipStream_t stream) {
  const int64_t tiles = (int64_t)p.n_heads * (p.n / 32) * ((p.batch + 31) / 32);
  const int64_t grid = (tiles + kWaves - 1) / kWaves;
  if (grid > INT32_MAX) return kEinval;
  hipLaunchKernelGGL(mla_proj_kernel, dim3((unsigned)grid), dim3(64 * kWaves), 0, stream, p);
  return hipGetLastError() == hipSuccess ? kOk : kEhip;
}

}  // namespace pkva

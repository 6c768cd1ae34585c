// The per-head projections around the absorbed MLA attention (frink-models
// 0.31.0 src/mla/mod.rs, absorbed_attention and the MlaKvB::Split doc):
//   absorb:  q_abs[b, h] = [k_b[h] q_nope[b, h] | q_rot[b, h]],  k_b[h] is [R, qk_nope]
//   up-proj: out[b, h]   = v_b[h] o_lat[b, h],                    v_b[h] is [v_dim, R]
// Both are batched GEMMs with one weight matrix per head: Y[b, h, n] =
// sum_k W[h][n][k] X[b, h, k], the batch as the small dimension. At decode
// batch sizes they read every weight byte once and are bound by HBM.
//
// A workgroup (4 waves) owns 32 batch rows of one head and NG x 32 outputs;
// its waves split that as NG output tiles times KS = 4 / NG slices of K, so
// that a narrow N (the up-projection's 128) still spreads its long K over
// four waves. Each wave accumulates a 32 x 32 tile Y^T[n][b] on 32x32x16
// bf16 MFMAs: the A operand (W rows, 8 consecutive k per lane) and the B
// operand (X rows, likewise) are 16-byte loads straight from global memory,
// all of a wave's issued together; a weight byte is read once. The K slices
// are summed through LDS, and the tile goes out through LDS too, so that
// every batch row leaves as whole 16-byte chunks of NG x 64 bytes.
#include "common.hpp"
#include "kernels.hpp"

namespace pkva {

namespace {

constexpr int kWaves = 4;
constexpr int kMaxSteps = 8;     // 16-deep k-steps a wave loads at once

template <int NG>
__global__ __launch_bounds__(64 * kWaves) void mla_proj_kernel(MlaProjParams p) {
  constexpr int KS = kWaves / NG;                 // K slices per output tile
  __shared__ float s_acc[kWaves][16][64];         // accumulators, register-major
  __shared__ __attribute__((aligned(16))) __bf16 s_out[32][NG * 32 + 8];

  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int lr = lane % 32, hf = lane / 32;
  const int n_groups = p.n / (32 * NG), b_tiles = (p.batch + 31) / 32;
  // Workgroups of one head adjacent (they share the head's X rows).
  const int ng = blockIdx.x % n_groups;
  const int bt = (blockIdx.x / n_groups) % b_tiles;
  const int h = blockIdx.x / (n_groups * b_tiles);
  const int nt = wave % NG, ks = wave / NG;
  const int n0 = (ng * NG + nt) * 32, b0 = bt * 32;
  const int b = b0 + lr;
  const bool live = b < p.batch;

  const int ksteps = p.k / 16;
  const int per = (ksteps + KS - 1) / KS;
  const int s_lo = ks * per, s_hi = min(ksteps, s_lo + per);
  const __bf16* wrow = (const __bf16*)p.w + ((int64_t)h * p.n + n0 + lr) * p.k + 8 * hf;
  const __bf16* xrow = (const __bf16*)p.x + (int64_t)b * p.x_stride_b + (int64_t)h * p.x_stride_h +
                       8 * hf;
  f32x16_t acc = f32x16_t{};
  for (int k0 = s_lo; k0 < s_hi; k0 += kMaxSteps) {
    bf16x8_t a[kMaxSteps], bb[kMaxSteps];
#pragma unroll
    for (int j = 0; j < kMaxSteps; ++j) {
      if (k0 + j < s_hi) {
        a[j] = *(const bf16x8_t*)(wrow + 16 * (k0 + j));
        bb[j] = live ? *(const bf16x8_t*)(xrow + 16 * (k0 + j)) : bf16x8_t{};
      }
    }
#pragma unroll
    for (int j = 0; j < kMaxSteps; ++j)
      if (k0 + j < s_hi) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], bb[j], acc, 0, 0, 0);
  }
  // Sum the K slices of each output tile (fixed order: slice 0 first).
  if constexpr (KS > 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s_acc[wave][r][lane] = acc[r];
    __syncthreads();
    if (ks == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = acc[r];
#pragma unroll
        for (int j = 1; j < KS; ++j) v += s_acc[wave + j * NG][r][lane];
        acc[r] = v;
      }
    }
  }
  // Accumulator register r holds Y^T[n0 + 8 (r / 4) + 4 hf + r % 4][b0 + lr].
  if (ks == 0) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const bf16x4_t v = {(__bf16)acc[4 * g4 + 0], (__bf16)acc[4 * g4 + 1],
                          (__bf16)acc[4 * g4 + 2], (__bf16)acc[4 * g4 + 3]};
      *(bf16x4_t*)&s_out[lr][nt * 32 + 8 * g4 + 4 * hf] = v;
    }
  }
  __syncthreads();
  // Rows of the tile: NG * 64 bytes each, in 16-byte chunks.
  constexpr int kChunks = NG * 4;   // per row
  for (int i = threadIdx.x; i < 32 * kChunks; i += 64 * kWaves) {
    const int row = i / kChunks, ch = i % kChunks;
    if (b0 + row < p.batch) {
      __bf16* y = (__bf16*)p.y + (int64_t)(b0 + row) * p.y_stride_b + (int64_t)h * p.y_stride_h +
                  ng * NG * 32 + ch * 8;
      *(uint4*)y = *(const uint4*)&s_out[row][ch * 8];
    }
  }
  // The absorbed query carries the rope part after the projected part: the
  // head's first workgroup of each batch tile copies it, 16 bytes at a time.
  if (p.copy_len > 0 && ng == 0) {
    const int chunks = p.copy_len / 8;
    for (int i = threadIdx.x; i < 32 * chunks; i += 64 * kWaves) {
      const int row = i / chunks, ch = i % chunks;
      if (b0 + row < p.batch) {
        const __bf16* src = (const __bf16*)p.x + (int64_t)(b0 + row) * p.x_stride_b +
                            (int64_t)h * p.x_stride_h + p.copy_src + ch * 8;
        __bf16* dst = (__bf16*)p.y + (int64_t)(b0 + row) * p.y_stride_b +
                      (int64_t)h * p.y_stride_h + p.n + ch * 8;
        *(uint4*)dst = *(const uint4*)src;
      }
    }
  }
}

}  // namespace

int launch_mla_proj(const MlaProjParams& p, hipStream_t stream) {
  // Output tiles per workgroup: four for a short K (each wave one tile), one
  // for a long K (its four waves split K), so both shapes launch about as
  // many waves as there are output tiles times K / 128.
  const int tiles = p.n / 32;
  const int ng = p.k > 256 ? 1 : (tiles % 4 == 0 ? 4 : (tiles % 2 == 0 ? 2 : 1));
  const int64_t grid = (int64_t)p.n_heads * ((p.batch + 31) / 32) * (tiles / ng);
  if (grid > INT32_MAX) return kEinval;
  switch (ng) {
    case 4: hipLaunchKernelGGL(mla_proj_kernel<4>, dim3((unsigned)grid), dim3(64 * kWaves), 0, stream, p); break;
    case 2: hipLaunchKernelGGL(mla_proj_kernel<2>, dim3((unsigned)grid), dim3(64 * kWaves), 0, stream, p); break;
    default: hipLaunchKernelGGL(mla_proj_kernel<1>, dim3((unsigned)grid), dim3(64 * kWaves), 0, stream, p); break;
  }
  return hipGetLastError() == hipSuccess ? kOk : kEhip;
}

}  // namespace pkva

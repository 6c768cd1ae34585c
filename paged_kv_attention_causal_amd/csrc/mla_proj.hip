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
// bf16 MFMAs. Operands reach LDS by global -> LDS copies of whole rows (1 KB
// per op = 4 rows of 128 k, 16-byte chunk c of row r stored at chunk slot
// c ^ (r % 16), which keeps the 16 rows of an operand read on distinct bank
// groups): a direct 16-byte-per-lane load of an MFMA operand would touch 32
// rows with 32 bytes each per instruction. A weight byte is read once. The K
// slices are summed through LDS, and the tile goes out through LDS too, so
// that every batch row leaves as whole 16-byte chunks of NG x 64 bytes.
#include "common.hpp"
#include "kernels.hpp"

namespace pkva {

namespace {

constexpr int kWaves = 4;
constexpr int kPassSteps = 8;           // 16-deep k-steps per pass (128 k, 256-byte rows)
constexpr int kRowB = 16 * kPassSteps * 2;
constexpr int kTileB = 32 * kRowB;      // one 32-row operand tile of a pass (8 KB)

template <int NG>
__global__ __launch_bounds__(64 * kWaves) void mla_proj_kernel(MlaProjParams p) {
  constexpr int KS = kWaves / NG;                 // K slices per output tile
  // Operand tiles of the current pass: [0] W of each wave, [1] X of each K slice.
  // After the MFMAs the same bytes hold the K-slice sums and the output rows.
  __shared__ __attribute__((aligned(1024))) char s_buf[2 * kWaves * kTileB];
  static_assert(sizeof(float) * kWaves * 16 * 64 + 32 * (NG * 32 + 8) * 2 <= 2 * kWaves * kTileB,
                "the epilogue fits in the operand buffer");
  float(*s_acc)[16][64] = (float(*)[16][64])s_buf;
  __bf16(*s_out)[NG * 32 + 8] = (__bf16(*)[NG * 32 + 8])(s_buf + sizeof(float) * kWaves * 16 * 64);

  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int lr = lane % 32, hf = lane / 32;
  const int n_groups = p.n / (32 * NG), b_tiles = (p.batch + 31) / 32;
  // Workgroups of one head adjacent (they share the head's X rows).
  const int ng = blockIdx.x % n_groups;
  const int bt = (blockIdx.x / n_groups) % b_tiles;
  const int h = blockIdx.x / (n_groups * b_tiles);
  const int nt = wave % NG, ks = wave / NG;
  const int n0 = (ng * NG + nt) * 32, b0 = bt * 32;

  const int ksteps = p.k / 16;
  const int per = (ksteps + KS - 1) / KS;
  const int s_lo = ks * per, s_hi = min(ksteps, s_lo + per);
  const char* wbase = (const char*)p.w + ((int64_t)h * p.n + n0) * p.k * 2;
  const char* xbase = (const char*)p.x + (int64_t)h * p.x_stride_h * 2;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(s_buf);
  char* w_tile = s_buf + wave * kTileB;
  char* x_tile = s_buf + (kWaves + ks) * kTileB;
  // Copy op j (0..7) of a 32-row tile: rows 4 j + lane / 16; the lane brings
  // the row's chunk (lane % 16) ^ (row % 16) of the pass, clamped to the
  // slice's last chunk (a clamped chunk feeds no MFMA).
  const int crow_in = lane / 16, cslot = lane % 16;
  auto op_chunk = [&](int row, int k0, int kend) {
    const int c = min(cslot ^ (row % 16), (kend - k0) * 2 - 1);   // 16-byte chunk of the pass
    return (int64_t)k0 * 32 + c * 16;
  };
  f32x16_t acc = f32x16_t{};
  // The same number of passes on every wave (a slice may run out of k-steps
  // before the others: it then only takes part in the barriers).
  const int n_pass = (per + kPassSteps - 1) / kPassSteps;
  for (int ps = 0; ps < n_pass; ++ps) {
    const int k0 = s_lo + ps * kPassSteps;
    const int k1 = min(s_hi, k0 + kPassSteps);
    if (k0 < k1) {   // uniform over the wave (and over the waves of a K slice)
      // This wave's W tile.
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = 4 * j + crow_in;
        dma16_addr(wbase + (int64_t)row * p.k * 2 + op_chunk(row, k0, k1),
                   lds0 + (uint32_t)(wave * kTileB + 1024 * j));
      }
      // The X tile of this K slice: its NG waves share the 8 copies (rows
      // past the batch read the last row; their outputs are not stored).
      for (int j = nt; j < 8; j += NG) {
        const int row = 4 * j + crow_in;
        const int b = min(b0 + row, p.batch - 1);
        dma16_addr(xbase + (int64_t)b * p.x_stride_b * 2 + op_chunk(row, k0, k1),
                   lds0 + (uint32_t)((kWaves + ks) * kTileB + 1024 * j));
      }
    }
    wait_vmcnt<0>();
    __syncthreads();
    // A operand: W row n0 + lr, k-step kk of the pass: chunk 2 kk + hf;
    // B operand: X row b0 + lr, likewise.
#pragma unroll
    for (int kk = 0; kk < kPassSteps; ++kk) {
      if (k0 + kk < k1) {
        const int off = lr * kRowB + 16 * ((2 * kk + hf) ^ (lr % 16));
        const bf16x8_t a = *(const bf16x8_t*)(w_tile + off);
        const bf16x8_t bb = *(const bf16x8_t*)(x_tile + off);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bb, acc, 0, 0, 0);
      }
    }
    __syncthreads();   // the tiles are refilled by the next pass or reused below
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

// Absorbed multi-head latent attention decode (frink-models 0.31.0
// src/mla/mod.rs, absorbed_attention and the MlaKvB doc): every head h
// attends over the sequence's cached latent rows [c | k_rot] (width R + P)
// with its absorbed query q_abs[h]; the value is each row's first R entries.
// It is multi-query attention with one shared KV head, so the latent tile is
// loaded once per workgroup and serves all of its heads.
//
// One workgroup = 4 waves = 16 heads of one sequence over a token range.
// 64-token latent tiles move through a two-stage LDS ring (row-major, padded
// rows): the next tile is loaded into registers while the current one is
// consumed. Per tile:
//   wave w computes S^T = L Q^T for tokens 16w..16w+15 (16x16x32 bf16 MFMA,
//   Q^T in registers) and writes the raw scores to LDS;
//   every wave then reads all 64 scores of its lane's head, runs the same
//   online-softmax update (identical in all four waves), and accumulates its
//   own quarter of the value width, O^T[128w .. 128w+127] += V^T P^T, with
//   the V^T operand read from the row-major tile by ds_read_b64_tr_b16.
// When the batch already fills the chip each workgroup takes a whole
// sequence and writes o_lat directly; otherwise the context is split and
// mla_combine merges the pieces in split order.
#include "common.hpp"
#include "kernels.hpp"

namespace pkva {

namespace {

constexpr int kThreads = 256;
constexpr int kHeads = 16;       // heads per workgroup
constexpr int kTile = 64;        // tokens per LDS tile
constexpr int kR = 512;          // kv_lora_rank
constexpr int kP = 64;           // qk_rope_head_dim
constexpr int kW = kR + kP;      // latent row width
constexpr int kLatStr = kW + 8;  // padded row stride of the row-major tile
constexpr int kSStr = kTile + 4;
constexpr int kKSteps = kW / 32; // MFMA k-steps for the scores (18)
constexpr int kDPerWave = kR / 4;

__device__ __forceinline__ f32x4_t mma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Physical workgroup id -> logical item, so that the items that read the same
// sequence's latent (its head groups and splits) run on one XCD and share its
// L2. Workgroups are dispatched to the 8 XCDs round-robin by id.
__device__ __forceinline__ int xcd_logical(int i, int n) {
  constexpr int kXcd = 8;
  if (n % kXcd != 0) return i;
  return (i % kXcd) * (n / kXcd) + i / kXcd;
}

// Transposed LDS read: four consecutive rows of one 16-bit column per lane.
__device__ __forceinline__ bf16x4_t ds_read_tr16(const void* p) {
  typedef __attribute__((ext_vector_type(4))) short s16x4;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(__attribute__((address_space(3))) char*)(p));
  return __builtin_bit_cast(bf16x4_t, v);
}

__global__ __launch_bounds__(kThreads) void mla_kernel(MlaParams p) {
  constexpr int kRowB = kLatStr * 2;                    // padded row bytes in LDS
  constexpr int kChunks = kTile * (kW / 8);             // 16-byte chunks per tile
  constexpr int kLpt = kChunks / kThreads;              // loads per thread per tile
  static_assert(kChunks % kThreads == 0, "tile must split evenly over the threads");
  __shared__ __attribute__((aligned(16))) __bf16 sLat[2][kTile * kLatStr];
  __shared__ __attribute__((aligned(16))) float sS[kHeads * kSStr];

  const int n_hg = p.n_heads / kHeads;
  const int n_items = p.batch * n_hg * p.nsplit;
  const int item = xcd_logical(blockIdx.x, n_items);
  const int split = item % p.nsplit;
  const int hg = (item / p.nsplit) % n_hg;
  const int b = item / (p.nsplit * n_hg);

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int l16 = lane % 16, quad = lane / 16;
  const int head = hg * kHeads + l16;

  const int L = p.seq_lens[b];
  const bool bad = L < 1 || L > p.max_seq_len;
  const int t_begin = split * p.split_tokens;
  const int t_end = bad ? 0 : min(L, t_begin + p.split_tokens);

  // Q^T as the B operand: lane holds head l16, dims 32*kk + 8*quad .. +7.
  bf16x8_t qB[kKSteps];
  {
    const __bf16* qg = (const __bf16*)p.q + ((int64_t)b * p.n_heads + head) * kW + 8 * quad;
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) qB[kk] = *(const bf16x8_t*)(qg + 32 * kk);
  }

  f32x4_t oacc[kDPerWave / 16];
#pragma unroll
  for (int db = 0; db < kDPerWave / 16; ++db) oacc[db] = f32x4_t{};
  float m_run = -INFINITY;
  float l_run = 0.0f;
  const float c = p.scale_log2;
  const char* lat = (const char*)p.latent + (int64_t)b * p.kv_capacity * (kW * 2);

  // Tile fetch into registers (tokens past t_end read as zero) and stash to LDS.
  uint4 st[kLpt];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int j = 0; j < kLpt; ++j) {
      const int ci = tid + kThreads * j;
      const int row = ci / (kW / 8), cc = ci % (kW / 8);
      const int t = t0 + row;
      st[j] = make_uint4(0, 0, 0, 0);
      if (t < t_end) st[j] = *(const uint4*)(lat + (int64_t)t * (kW * 2) + cc * 16);
    }
  };
  auto stash = [&](int stage) {
#pragma unroll
    for (int j = 0; j < kLpt; ++j) {
      const int ci = tid + kThreads * j;
      const int row = ci / (kW / 8), cc = ci % (kW / 8);
      *(uint4*)((char*)sLat[stage] + row * kRowB + cc * 16) = st[j];
    }
  };

  if (t_begin < t_end) {
    fetch(t_begin);
    stash(0);
    __syncthreads();
  }
  int stage = 0;
  for (int t0 = t_begin; t0 < t_end; t0 += kTile, stage ^= 1) {
    const bool more = t0 + kTile < t_end;
    if (more) fetch(t0 + kTile);
    const char* tile = (const char*)sLat[stage];

    // ---- raw scores for tokens 16*wave .. +15 of the tile
    {
      f32x4_t acc = f32x4_t{};
      const char* lrow = tile + (16 * wave + l16) * kRowB + 16 * quad;
#pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) acc = mma16(*(const bf16x8_t*)(lrow + 64 * kk), qB[kk], acc);
      // accumulator: lane l16 = head, rows = tokens 16*wave + 4*quad + r
      *(f32x4_t*)(sS + l16 * kSStr + 16 * wave + 4 * quad) = acc;
    }
    __syncthreads();

    // ---- online softmax over the tile's 64 tokens (same in every wave)
    float sv[2][8];
    float mx = -INFINITY;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const float* srow = sS + l16 * kSStr + 32 * pp + 8 * quad;
      const f32x4_t a = *(const f32x4_t*)srow;
      const f32x4_t b4 = *(const f32x4_t*)(srow + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sv[pp][j] = a[j];
        sv[pp][4 + j] = b4[j];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = t0 + 32 * pp + 8 * quad + j;
        if (t >= t_end) sv[pp][j] = -INFINITY;
        mx = fmaxf(mx, sv[pp][j]);
      }
    }
    mx = fmaxf(mx, xchg<4>(mx));
    mx = fmaxf(mx, xchg<5>(mx));
    const float m_new = fmaxf(m_run, mx);
    const float mc = m_new * c;   // finite: the tile holds at least one live token
    const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(fmaf(m_run, c, -mc));
    m_run = m_new;
    float psum = 0.0f;
    bf16x8_t pB[2];
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = sv[pp][j];
        const float e = x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(fmaf(x, c, -mc));
        psum += e;
        pB[pp][j] = (__bf16)e;
      }
    l_run = fmaf(l_run, alpha, psum);
#pragma unroll
    for (int db = 0; db < kDPerWave / 16; ++db) oacc[db] *= alpha;

    // ---- O^T[this wave's quarter] += V^T P^T over tokens 32*pp + 8*quad + j.
    // Lane (quad, l16) addresses row k0 + l16/4 at columns 4*(l16%4)..+3 of a
    // 16-column slice and receives column (slice + l16) of rows k0 .. k0+3.
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const int r0 = 32 * pp + 8 * quad + l16 / 4;
#pragma unroll
      for (int db = 0; db < kDPerWave / 16; ++db) {
        const int col = kDPerWave * wave + 16 * db + 4 * (l16 % 4);
        const bf16x4_t lo = ds_read_tr16(tile + r0 * kRowB + col * 2);
        const bf16x4_t hi = ds_read_tr16(tile + (r0 + 4) * kRowB + col * 2);
        const bf16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oacc[db] = mma16(a, pB[pp], oacc[db]);
      }
    }
    if (more) stash(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: the head's sum is spread over the 4 lanes l16 + 16*quad
  float l_tot = l_run + xchg<4>(l_run);
  l_tot = l_tot + xchg<5>(l_tot);
  const int d0 = kDPerWave * wave + 4 * quad;
  if (p.nsplit == 1) {
    __bf16* og = (__bf16*)p.o + ((int64_t)b * p.n_heads + head) * kR;
    if (bad) {
#pragma unroll
      for (int db = 0; db < kDPerWave / 16; ++db) {
        const bf16x4_t w = {(__bf16)__builtin_nanf(""), (__bf16)__builtin_nanf(""),
                            (__bf16)__builtin_nanf(""), (__bf16)__builtin_nanf("")};
        *(bf16x4_t*)(og + d0 + 16 * db) = w;
      }
      return;
    }
    const float inv = 1.0f / l_tot;
#pragma unroll
    for (int db = 0; db < kDPerWave / 16; ++db) {
      const bf16x4_t w = {(__bf16)(oacc[db][0] * inv), (__bf16)(oacc[db][1] * inv),
                          (__bf16)(oacc[db][2] * inv), (__bf16)(oacc[db][3] * inv)};
      *(bf16x4_t*)(og + d0 + 16 * db) = w;
    }
  } else {
    // Partial of this split: unnormalised O, m in the log2 domain, l.
    const int64_t w = ((int64_t)b * p.nsplit + split) * p.n_heads + head;
    float* wo = p.ws_o + w * kR;
#pragma unroll
    for (int db = 0; db < kDPerWave / 16; ++db)
      *(f32x4_t*)(wo + d0 + 16 * db) = oacc[db];
    if (wave == 0 && quad == 0) {
      const bool live = t_begin < t_end;
      p.ws_ml[w * 2 + 0] = live ? m_run * c : -INFINITY;
      p.ws_ml[w * 2 + 1] = live ? l_tot : 0.0f;
    }
  }
}

// Merge the splits of one (sequence, head) in split order.
__global__ __launch_bounds__(kThreads) void mla_combine(MlaParams p) {
  const int b = blockIdx.x / p.n_heads;
  const int h = blockIdx.x % p.n_heads;
  const int L = p.seq_lens[b];
  const bool bad = L < 1 || L > p.max_seq_len;
  const int nsp = bad ? 0 : (L + p.split_tokens - 1) / p.split_tokens;
  float M = -INFINITY;
  for (int s = 0; s < nsp; ++s) M = fmaxf(M, p.ws_ml[(((int64_t)b * p.nsplit + s) * p.n_heads + h) * 2]);
  for (int d = threadIdx.x; d < kR; d += kThreads) {
    float out = __builtin_nanf("");
    if (!bad) {
      float num = 0.0f, den = 0.0f;
      for (int s = 0; s < nsp; ++s) {
        const int64_t w = ((int64_t)b * p.nsplit + s) * p.n_heads + h;
        const float wt = __builtin_amdgcn_exp2f(p.ws_ml[w * 2] - M);
        num = fmaf(wt, p.ws_o[w * kR + d], num);
        den = fmaf(wt, p.ws_ml[w * 2 + 1], den);
      }
      out = num / den;
    }
    ((__bf16*)p.o)[((int64_t)b * p.n_heads + h) * kR + d] = (__bf16)out;
  }
}

}  // namespace

bool mla_supported(bool bf16, int kv_lora_rank, int rope_dim, int n_heads) {
  return bf16 && kv_lora_rank == kR && rope_dim == kP && n_heads % kHeads == 0;
}

int mla_heads_per_group() { return kHeads; }
int mla_tile_tokens() { return kTile; }

int launch_mla(const MlaParams& p, hipStream_t stream) {
  const int n_items = p.batch * (p.n_heads / kHeads) * p.nsplit;
  hipLaunchKernelGGL(mla_kernel, dim3(n_items), dim3(kThreads), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return kEhip;
  if (p.nsplit > 1) {
    hipLaunchKernelGGL(mla_combine, dim3(p.batch * p.n_heads), dim3(kThreads), 0, stream, p);
    if (hipGetLastError() != hipSuccess) return kEhip;
  }
  return kOk;
}

}  // namespace pkva

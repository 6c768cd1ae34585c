// Multi-token causal GQA prefill over a contiguous or block-table paged K/V.
//
// Row i of the query sits at absolute position position_offset + i and
// attends to keys j <= position_offset + i, j < seq_kv (kopitiam-runtime
// 0.2.4 src/attention.rs, causal_mask); query head h reads KV head h / G
// (repeat_kv_heads). The softmax is computed online over key tiles.
//
// One workgroup = 4 waves = 128 query rows of one (sequence, head). Each
// wave owns 32 rows. Per 64-key tile:
//   K tile [64 x D] and V^T tile [D x 64] are staged in LDS;
//   S^T = K Q^T on 32x32 MFMAs (Q^T held in registers as the B operand), so
//     in the accumulator layout every lane holds one query row: lane l owns
//     row l % 32 and 16 of each 32 keys, the other 16 sit in lane l ^ 32;
//   the row max needs one cross-half exchange (v_permlane32_swap); the row
//     sum stays per lane until the end;
//   P (rounded to bf16 for the bf16 instantiation) feeds O^T += V^T P^T
//     straight from the accumulator registers: the accumulator's key order
//     is a fixed permutation that the V^T operand reads follow;
//   O^T keeps each lane's query row in its own registers, so rescaling by
//     exp2(m_old - m_new) and the final 1/l never leave the lane.
// Key tiles wholly above the diagonal are never visited; only tiles that
// cross the diagonal or the end of the keys apply the mask.
#include "common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace pkva {

namespace {

constexpr int kThreads = 256;
constexpr int kBlockM = 128;   // query rows per workgroup (32 per wave)
constexpr int kBlockN = 64;    // keys per tile

template <bool BF16>
struct Mfma;

// bf16 inputs: v_mfma_f32_32x32x16_bf16, 8 bf16 per lane per operand.
template <>
struct Mfma<true> {
  using Elem = __bf16;
  using Op = bf16x8_t;
  static constexpr int K = 16;
  __device__ __forceinline__ static f32x16_t mma(Op a, Op b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

// fp32 inputs: v_mfma_f32_32x32x2_f32, 1 float per lane per operand.
template <>
struct Mfma<false> {
  using Elem = float;
  using Op = float;
  static constexpr int K = 2;
  __device__ __forceinline__ static f32x16_t mma(Op a, Op b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

template <bool PAGED>
struct KeyRow {
  const int32_t* bt;   // this sequence's block table row (paged)
  int64_t seq_base;    // contiguous: element offset of row 0 of this sequence
  __device__ __forceinline__ int64_t operator()(int t, int shift, int64_t row_stride) const {
    if constexpr (PAGED) {
      const int64_t blk = bt[t >> shift];
      return ((blk << shift) + (t & ((1 << shift) - 1))) * row_stride;
    } else {
      return seq_base + (int64_t)t * row_stride;
    }
  }
};

template <bool BF16, int D, bool PAGED>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillParams p) {
  using M = Mfma<BF16>;
  using T = typename M::Elem;
  using Seg = typename std::conditional<BF16, bf16x8_t, f32x4_t>::type;  // one 16-byte segment
  constexpr int ESZ = sizeof(T);
  constexpr int E = 16 / ESZ;                 // elements per 16-byte segment
  constexpr int SEGS = D / E;                 // 16-byte segments per K/V row
  constexpr int DB = (D + 31) / 32;           // 32-row blocks of O^T
  constexpr int KPAD = BF16 ? 8 : 4;
  constexpr int KSTR = D + KPAD;              // sK row stride (elements)
  constexpr int VSTR = kBlockN + (BF16 ? 8 : 4);  // sVt row stride (elements)
  constexpr int KSTEPS = D / M::K;            // MFMAs per 32x32 S^T block
  static_assert(D % E == 0 && D % M::K == 0, "unsupported head size");

  __shared__ __attribute__((aligned(16))) T sK[kBlockN * KSTR];
  __shared__ __attribute__((aligned(16))) T sVt[DB * 32 * VSTR];
  __shared__ int s_bad;

  // Heaviest query tiles first; within a tile level, heads of one sequence.
  const int per_level = p.batch * p.n_heads;
  const int qt = p.q_tiles - 1 - (int)(blockIdx.x / per_level);
  const int rest = blockIdx.x % per_level;
  const int h = rest % p.n_heads;
  const int b = rest / p.n_heads;
  const int kvh = h / p.group;

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int lr = lane % 32, hf = lane / 32;
  const int q0 = qt * kBlockM;
  const int off = p.position_offset;
  const int64_t row_stride = (int64_t)p.n_kv_heads * D;
  const int shift = p.block_shift;

  // Keys this tile can see: 0 .. last_key.
  const int q_last = min(q0 + kBlockM, p.seq_q) - 1;
  const int last_key = min(p.seq_kv - 1, off + q_last);
  const int n_kt = last_key / kBlockN + 1;

  KeyRow<PAGED> row;
  if constexpr (PAGED) {
    row.bt = p.block_table + (int64_t)b * p.max_blocks_per_seq;
    row.seq_base = 0;
    if (tid == 0) s_bad = 0;
    __syncthreads();
    const int nblk = (last_key >> shift) + 1;
    for (int i = tid; i < nblk; i += kThreads) {
      const int id = row.bt[i];
      if (id < 0 || id >= p.num_blocks) s_bad = 1;
    }
    __syncthreads();
    if (s_bad) {
      // A needed block lies outside the pool: NaN rows, no K/V read.
      for (int idx = tid; idx < kBlockM * D; idx += kThreads) {
        const int i = q0 + idx / D;
        if (i < p.seq_q) {
          const int64_t o = (((int64_t)b * p.seq_q + i) * p.n_heads + h) * D + idx % D;
          ((T*)p.o)[o] = (T)__builtin_nanf("");
        }
      }
      return;
    }
  } else {
    row.bt = nullptr;
    row.seq_base = (int64_t)b * p.kv_capacity * row_stride;
  }
  const T* kg = (const T*)p.k + (int64_t)kvh * D;
  const T* vg = (const T*)p.v + (int64_t)kvh * D;

  // Zero the padding rows of V^T once (head sizes below 32).
  if constexpr (DB * 32 > D) {
    for (int i = tid; i < (DB * 32 - D) * VSTR; i += kThreads) sVt[D * VSTR + i] = (T)0.0f;
  }

  // Q^T as the B operand: lane holds query row q0 + 32*wave + lr, dims per k-step.
  const int qrow = q0 + wave * 32 + lr;
  typename M::Op qB[KSTEPS];
  {
    const T* qg = (const T*)p.q + (((int64_t)b * p.seq_q + qrow) * p.n_heads + h) * D;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      if constexpr (BF16) {
        if (qrow < p.seq_q) {
          qB[kk] = *(const bf16x8_t*)(qg + kk * 16 + hf * 8);
        } else {
          qB[kk] = bf16x8_t{};
        }
      } else {
        qB[kk] = qrow < p.seq_q ? qg[kk * 2 + hf] : 0.0f;
      }
    }
  }

  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16_t{};
  float m_run = -INFINITY;   // running max of raw scores for this lane's row
  float l_run = 0.0f;        // this lane's share of the running sum
  const float c = p.scale_log2;
  const int wave_pos_first = off + q0 + wave * 32;     // position of the wave's first row
  const int my_pos = off + qrow;
  const bool wave_live = q0 + wave * 32 < p.seq_q;

  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * kBlockN;
    __syncthreads();
    // ---- stage K [64 x D] and V^T [D x 64] in LDS
    for (int sidx = tid; sidx < kBlockN * SEGS; sidx += kThreads) {
      const int key = sidx / SEGS, seg = sidx % SEGS;
      const int t = k0 + key;
      uint4 w = make_uint4(0, 0, 0, 0);
      // Keys past last_key are masked for every row of the tile: never read
      // (their blocks were not validated).
      if (t <= last_key) w = *(const uint4*)(kg + row(t, shift, row_stride) + seg * E);
      *(uint4*)(sK + key * KSTR + seg * E) = w;
    }
    for (int u = tid; u < (kBlockN / 4) * SEGS; u += kThreads) {
      const int kq = u / SEGS, seg = u % SEGS;
      Seg x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = k0 + kq * 4 + j;
        uint4 w = make_uint4(0, 0, 0, 0);
        if (t <= last_key) w = *(const uint4*)(vg + row(t, shift, row_stride) + seg * E);
        x[j] = __builtin_bit_cast(Seg, w);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        T* dst = sVt + (seg * E + e) * VSTR + kq * 4;
        if constexpr (BF16) {
          bf16x4_t v4 = {x[0][e], x[1][e], x[2][e], x[3][e]};
          *(bf16x4_t*)dst = v4;
        } else {
          *(float4*)dst = make_float4(x[0][e], x[1][e], x[2][e], x[3][e]);
        }
      }
    }
    __syncthreads();

    // The wave's rows see none of this tile's keys: nothing to add.
    if (!wave_live || k0 > wave_pos_first + 31) continue;

    // ---- S^T = K Q^T, two 32-key blocks
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16_t acc = f32x16_t{};
      const T* krow = sK + (kb * 32 + lr) * KSTR;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        typename M::Op a;
        if constexpr (BF16) {
          a = *(const bf16x8_t*)(krow + kk * 16 + hf * 8);
        } else {
          a = krow[kk * 2 + hf];
        }
        acc = M::mma(a, qB[kk], acc);
      }
      s[kb] = acc;
    }

    // ---- causal / length mask on tiles that cross the diagonal or the end
    const bool need_mask = (k0 + kBlockN - 1 > wave_pos_first) || (k0 + kBlockN > p.seq_kv);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
          if (key > my_pos || key >= p.seq_kv) s[kb][r] = -INFINITY;
        }
    }

    // ---- online softmax on this lane's row
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float m_new = fmaxf(m_run, mx);
    // Key 0 is visible to every row, so m_new is finite after the first tile;
    // the guards keep weights exact (0) for masked keys even when scale == 0.
    const float mc = m_new == -INFINITY ? 0.0f : m_new * c;
    const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(fmaf(m_run, c, -mc));
    m_run = m_new;
    float psum = 0.0f;
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float sv = s[kb][r];
          const float x = BF16 ? fmaf(sv, c, -mc) : (sv - m_new) * c;
          const float e = sv == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x);
          s[kb][r] = e;
          psum += e;
        }
    } else if constexpr (BF16) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -mc));
          s[kb][r] = e;
          psum += e;
        }
    } else {
      // fp32: (s - m) * c, so the row maximum weighs exactly 1.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f((s[kb][r] - m_new) * c);
          s[kb][r] = e;
          psum += e;
        }
    }
    l_run = fmaf(l_run, alpha, psum);
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= alpha;

    // ---- O^T += V^T P^T; accumulator register r of key block kb is key
    //      32*kb + 8*(r/4) + 4*hf + r%4, and the V^T reads follow that order.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (BF16) {
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          bf16x8_t pb;
#pragma unroll
          for (int j = 0; j < 8; ++j) pb[j] = (__bf16)s[kb][8 * mm + j];
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const T* vrow = sVt + (db * 32 + lr) * VSTR + kb * 32 + 16 * mm + 4 * hf;
            const bf16x4_t lo = *(const bf16x4_t*)(vrow);
            const bf16x4_t hi = *(const bf16x4_t*)(vrow + 8);
            const bf16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            oacc[db] = M::mma(a, pb, oacc[db]);
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const float a = sVt[(db * 32 + lr) * VSTR + kb * 32 + 8 * (r / 4) + 4 * hf + (r % 4)];
            oacc[db] = M::mma(a, s[kb][r], oacc[db]);
          }
        }
      }
    }
  }

  // ---- epilogue: l = both halves' shares; O^T / l -> o[b, row, h, :]
  const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run),
                                                    false, false);
  const float l_tot = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
  if (qrow < p.seq_q) {
    const float inv = 1.0f / l_tot;
    T* og = (T*)p.o + (((int64_t)b * p.seq_q + qrow) * p.n_heads + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + 8 * g4 + 4 * hf;
        if (d < D) {
          if constexpr (BF16) {
            bf16x4_t w = {(__bf16)(oacc[db][4 * g4 + 0] * inv), (__bf16)(oacc[db][4 * g4 + 1] * inv),
                          (__bf16)(oacc[db][4 * g4 + 2] * inv), (__bf16)(oacc[db][4 * g4 + 3] * inv)};
            *(bf16x4_t*)(og + d) = w;
          } else {
            *(float4*)(og + d) = make_float4(oacc[db][4 * g4 + 0] * inv, oacc[db][4 * g4 + 1] * inv,
                                             oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv);
          }
        }
      }
  }
}

template <bool BF16, int D, bool PAGED>
int launch_t(const PrefillParams& p, hipStream_t stream) {
  const int grid = p.q_tiles * p.batch * p.n_heads;
  hipLaunchKernelGGL((prefill_kernel<BF16, D, PAGED>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? kOk : kEhip;
}

}  // namespace

bool prefill_supported(bool bf16, int head_dim) {
  return (bf16 && head_dim == 128) || (!bf16 && head_dim == 16);
}

int prefill_block_m() { return kBlockM; }

int launch_prefill(bool bf16, bool paged, int head_dim, const PrefillParams& p, hipStream_t stream) {
  if (bf16 && head_dim == 128) {
    return paged ? launch_t<true, 128, true>(p, stream) : launch_t<true, 128, false>(p, stream);
  }
  if (!bf16 && head_dim == 16) {
    return paged ? launch_t<false, 16, true>(p, stream) : launch_t<false, 16, false>(p, stream);
  }
  return kEunsupported;
}

}  // namespace pkva

// Single-token GQA decode over a contiguous or block-table paged KV cache.
//
// The query of sequence b sits at position seq_lens[b] - 1 and attends to
// keys 0 .. seq_lens[b] - 1, its own key included: the row was pushed
// before the attend (frink-models 0.38.0 src/decoder/attn_block.rs,
// push_and_attend_row). Query head h reads KV head h / G (kopitiam-runtime
// 0.2.4 src/attention.rs, repeat_kv_heads).
//
// Split-K over the context. One workgroup owns a chunk of kDecChunk tokens
// of one sequence and a slab of KV heads, with every query head of those KV
// heads, so each K/V byte of the chunk is read from HBM exactly once:
//   pass 1  stream the chunk's K rows; 16-byte lane loads, each lane group
//           covers one (token, KV head) row; dot products with the group's
//           G queries are reduced across the group with DPP exchanges and
//           land in LDS as raw scores;
//   pass 2  per head, exact softmax over the chunk in LDS (chunk max m,
//           exp2, chunk sum l);
//   pass 3  stream the chunk's V rows and accumulate p * v per lane, then
//           reduce the token sub-rows through LDS in a fixed tree order.
// The chunk's (m, l, O) go to the workspace; decode_combine merges the
// chunks of a sequence in chunk order. Contiguous and paged differ only in
// the row address, so their arithmetic, and their results, are identical.
#include "common.hpp"
#include "kernels.hpp"

namespace pkva {

namespace {

constexpr int kThreads = 256;
constexpr int kDecChunk = 256;   // tokens per workgroup (the split-K unit)
constexpr int kHsMax = 32;       // query heads per workgroup
constexpr int kUnroll = 8;       // row loads in flight per lane

template <bool BF16>
struct Lane16 {
  static constexpr int E = BF16 ? 8 : 4;   // elements per 16-byte lane load
};

// Dot products of one 16-byte K chunk with GMAX query chunks.
template <bool BF16, int GMAX>
__device__ __forceinline__ void dot_rows(const uint4 (&q)[GMAX], const uint4 k, float (&s)[GMAX]) {
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    if constexpr (BF16) {
      float acc = dot2_bf16(q[h].x, k.x, 0.0f);
      acc = dot2_bf16(q[h].y, k.y, acc);
      acc = dot2_bf16(q[h].z, k.z, acc);
      acc = dot2_bf16(q[h].w, k.w, acc);
      s[h] = acc;
    } else {
      float acc = __uint_as_float(q[h].x) * __uint_as_float(k.x);
      acc = fmaf(__uint_as_float(q[h].y), __uint_as_float(k.y), acc);
      acc = fmaf(__uint_as_float(q[h].z), __uint_as_float(k.z), acc);
      acc = fmaf(__uint_as_float(q[h].w), __uint_as_float(k.w), acc);
      s[h] = acc;
    }
  }
}

template <bool BF16>
__device__ __forceinline__ void unpack16(const uint4 w, float (&x)[Lane16<BF16>::E]) {
  if constexpr (BF16) {
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
    x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z);
    x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  } else {
    x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
  }
}

// Element offset of row (token t, kv head kvh) of sequence b.
template <bool PAGED>
struct RowAddr {
  const int* s_blk;  // paged: block ids of the chunk, s_blk[i] = block of (blk0 + i)
  int blk0;
  int64_t seq_base;  // contiguous: b * kv_capacity * row_stride
  __device__ __forceinline__ int64_t operator()(int t, int shift, int64_t row_stride) const {
    if constexpr (PAGED) {
      const int bs_mask = (1 << shift) - 1;
      const int64_t blk = s_blk[(t >> shift) - blk0];
      return ((blk << shift) + (t & bs_mask)) * row_stride;
    } else {
      return seq_base + (int64_t)t * row_stride;
    }
  }
};

template <bool BF16, int D, int GMAX, bool PAGED>
__global__ __launch_bounds__(kThreads) void decode_partial(DecodeParams p) {
  constexpr int E = Lane16<BF16>::E;
  constexpr int LG = D / E;          // lanes per (token, kv head) row
  constexpr int NG = kThreads / LG;  // lane groups per workgroup
  constexpr int NV = GMAX > LG ? GMAX / LG : 1;
  constexpr int LPH = LG > GMAX ? LG / GMAX : 1;  // lanes sharing one head sum
  static_assert(D % E == 0 && kThreads % LG == 0, "head size must split into 16-byte lanes");

  __shared__ float s_S[kHsMax * (kDecChunk + 1)];
  __shared__ int s_blk[kDecChunk + 2];
  __shared__ int s_bad;

  const int chunk = blockIdx.x;
  const int b = blockIdx.y / p.nslab;
  const int slab = blockIdx.y % p.nslab;
  const int L = p.seq_lens[b];
  if (L < 1 || L > p.max_seq_len) return;          // combine writes NaN for b
  const int c0 = chunk * kDecChunk;
  if (c0 >= L) return;
  const int nvalid = min(kDecChunk, L - c0);

  const int tid = threadIdx.x;
  const int G = p.group;
  const int kvs = p.kvs;
  const int R = NG / kvs;            // tokens per pass over the workgroup
  const int g = tid / LG, li = tid % LG;
  const int kvl = g % kvs, r = g / kvs;
  const int kvh = slab * kvs + kvl;
  const int HS = kvs * G;
  const int64_t row_stride = (int64_t)p.n_kv_heads * D;
  const int shift = p.block_shift;

  // Block ids of the chunk, checked against the pool once.
  RowAddr<PAGED> addr;
  if constexpr (PAGED) {
    addr.blk0 = c0 >> shift;
    const int nblk = ((c0 + nvalid - 1) >> shift) - addr.blk0 + 1;
    if (tid == 0) s_bad = 0;
    __syncthreads();
    for (int i = tid; i < nblk; i += kThreads) {
      const int id = p.block_table[(int64_t)b * p.max_blocks_per_seq + addr.blk0 + i];
      s_blk[i] = id;
      if (id < 0 || id >= p.num_blocks) s_bad = 1;
    }
    addr.s_blk = s_blk;
    addr.seq_base = 0;
    __syncthreads();
    if (s_bad) {
      // A block outside the pool: poison this chunk's partial, read nothing.
      const int64_t wbase = ((int64_t)(b * p.nslab + slab) * p.max_chunks + chunk) * HS;
      if (tid < HS) {
        p.ws_ml[(wbase + tid) * 2 + 0] = 0.0f;
        p.ws_ml[(wbase + tid) * 2 + 1] = __builtin_nanf("");
      }
      return;
    }
  } else {
    addr.s_blk = nullptr;
    addr.blk0 = 0;
    addr.seq_base = (int64_t)b * p.kv_capacity * row_stride;
  }

  const char* kbase = (const char*)p.k + ((int64_t)kvh * D + li * E) * (BF16 ? 2 : 4);
  const char* vbase = (const char*)p.v + ((int64_t)kvh * D + li * E) * (BF16 ? 2 : 4);
  constexpr int ESZ = BF16 ? 2 : 4;

  // This lane's slice of its group's G query rows.
  uint4 q[GMAX];
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    if (h < G) {
      const int64_t qoff = ((int64_t)b * p.n_heads + (int64_t)kvh * G + h) * D + li * E;
      q[h] = *(const uint4*)((const char*)p.q + qoff * ESZ);
    } else {
      q[h] = make_uint4(0, 0, 0, 0);
    }
  }

  // ---- pass 1: raw scores q . k for every token of the chunk -> s_S[head][t]
  const int step = R * kUnroll;
  for (int base = 0; base < nvalid; base += step) {
    uint4 kb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int tl = base + u * R + r;
      kb[u] = make_uint4(0, 0, 0, 0);
      if (tl < nvalid) kb[u] = *(const uint4*)(kbase + addr(c0 + tl, shift, row_stride) * ESZ);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int tl = base + u * R + r;
      float s[GMAX];
      dot_rows<BF16, GMAX>(q, kb[u], s);
      reduce_scatter<LG, GMAX>(s, li);
      if (tl < nvalid && (li % LPH) == 0) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const int h = (li / LPH) * NV + i;
          if (h < G) s_S[(kvl * G + h) * (kDecChunk + 1) + tl] = s[i];
        }
      }
    }
  }
  __syncthreads();

  // ---- pass 2: per-head softmax over the chunk (log2 domain)
  const int wave = tid / 64, lane = tid % 64;
  const float c = p.scale_log2;
  const int64_t wbase = ((int64_t)(b * p.nslab + slab) * p.max_chunks + chunk) * HS;
  for (int hs = wave; hs < HS; hs += kThreads / 64) {
    float* row = s_S + hs * (kDecChunk + 1);
    float x[kDecChunk / 64];
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < kDecChunk / 64; ++j) {
      const int t = lane + 64 * j;
      x[j] = t < nvalid ? row[t] : -INFINITY;
      m = fmaxf(m, x[j]);
    }
    m = wave_max(m);
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < kDecChunk / 64; ++j) {
      const int t = lane + 64 * j;
      const float e = t < nvalid ? __builtin_amdgcn_exp2f((x[j] - m) * c) : 0.0f;
      row[t] = e;
      sum += e;
    }
    sum = wave_sum(sum);
    if (lane == 0) {
      p.ws_ml[(wbase + hs) * 2 + 0] = m * c;
      p.ws_ml[(wbase + hs) * 2 + 1] = sum;
    }
  }
  __syncthreads();

  // ---- pass 3: O += p * v over this lane's token sub-row
  float acc[GMAX][E];
#pragma unroll
  for (int h = 0; h < GMAX; ++h)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[h][e] = 0.0f;

  for (int base = 0; base < nvalid; base += step) {
    uint4 vb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int tl = base + u * R + r;
      vb[u] = make_uint4(0, 0, 0, 0);
      if (tl < nvalid) vb[u] = *(const uint4*)(vbase + addr(c0 + tl, shift, row_stride) * ESZ);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int tl = base + u * R + r;
      if (tl < nvalid) {
        float x[E];
        unpack16<BF16>(vb[u], x);
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
          if (h < G) {
            const float pw = s_S[(kvl * G + h) * (kDecChunk + 1) + tl];
#pragma unroll
            for (int e = 0; e < E; ++e) acc[h][e] = fmaf(pw, x[e], acc[h][e]);
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- fixed-order tree over the token sub-rows: acc(r) += acc(r + s)
  float* red = s_S;  // reused: (NG / 2) * GMAX * D floats <= kHsMax * (kDecChunk + 1)
  constexpr int SLICE = GMAX * E * LG;  // floats per (sub-row, kv head)
  static_assert((NG / 2) * GMAX * D <= kHsMax * (kDecChunk + 1), "reduction buffer too small");
  for (int s = R / 2; s >= 1; s /= 2) {
    if (r >= s && r < 2 * s) {
      float* dst = red + ((r - s) * kvs + kvl) * SLICE;
#pragma unroll
      for (int h = 0; h < GMAX; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) dst[(h * E + e) * LG + li] = acc[h][e];
    }
    __syncthreads();
    if (r < s) {
      const float* src = red + (r * kvs + kvl) * SLICE;
#pragma unroll
      for (int h = 0; h < GMAX; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] += src[(h * E + e) * LG + li];
    }
    __syncthreads();
  }

  if (r == 0) {
    float* dst = p.ws_o + wbase * D;
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      if (h < G) {
        float* d = dst + (int64_t)(kvl * G + h) * D + li * E;
#pragma unroll
        for (int e = 0; e < E; e += 4)
          *(float4*)(d + e) = make_float4(acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]);
      }
    }
  }
}

// Merge the chunk partials of one (sequence, slab) in chunk order:
//   o = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c,  M = max_c m_c.
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void decode_combine(DecodeParams p) {
  const int b = blockIdx.x / p.nslab;
  const int slab = blockIdx.x % p.nslab;
  const int HS = p.kvs * p.group;
  const int L = p.seq_lens[b];
  const bool bad = L < 1 || L > p.max_seq_len;
  const int nch = bad ? 0 : (L + kDecChunk - 1) / kDecChunk;
  const int64_t wbase = (int64_t)(b * p.nslab + slab) * p.max_chunks * HS;
  for (int idx = threadIdx.x; idx < HS * D; idx += kThreads) {
    const int hs = idx / D, d = idx % D;
    float out;
    if (bad) {
      out = __builtin_nanf("");
    } else {
      float M = -INFINITY;
      for (int ch = 0; ch < nch; ++ch) M = fmaxf(M, p.ws_ml[(wbase + ch * HS + hs) * 2]);
      float num = 0.0f, den = 0.0f;
      for (int ch = 0; ch < nch; ++ch) {
        const int64_t w = wbase + ch * HS + hs;
        const float wt = __builtin_amdgcn_exp2f(p.ws_ml[w * 2] - M);
        num = fmaf(wt, p.ws_o[w * D + d], num);
        den = fmaf(wt, p.ws_ml[w * 2 + 1], den);
      }
      out = num / den;
    }
    const int h = slab * HS + hs;
    const int64_t o = ((int64_t)b * p.n_heads + h) * D + d;
    if constexpr (BF16) {
      ((__bf16*)p.o)[o] = (__bf16)out;
    } else {
      ((float*)p.o)[o] = out;
    }
  }
}

template <bool BF16, int D, int GMAX, bool PAGED>
int launch_one(const DecodeParams& p, hipStream_t stream) {
  dim3 grid(p.max_chunks, p.batch * p.nslab);
  hipLaunchKernelGGL((decode_partial<BF16, D, GMAX, PAGED>), grid, dim3(kThreads), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return kEhip;
  hipLaunchKernelGGL((decode_combine<BF16, D>), dim3(p.batch * p.nslab), dim3(kThreads), 0,
                     stream, p);
  if (hipGetLastError() != hipSuccess) return kEhip;
  return kOk;
}

template <bool BF16, int D, bool PAGED>
int launch_g(const DecodeParams& p, int gmax, hipStream_t stream) {
  switch (gmax) {
    case 1: return launch_one<BF16, D, 1, PAGED>(p, stream);
    case 2: return launch_one<BF16, D, 2, PAGED>(p, stream);
    case 4: return launch_one<BF16, D, 4, PAGED>(p, stream);
    case 8: return launch_one<BF16, D, 8, PAGED>(p, stream);
    default: return kEunsupported;
  }
}

}  // namespace

int decode_chunk_tokens() { return kDecChunk; }
int decode_heads_per_slab_max() { return kHsMax; }

bool decode_supported(bool bf16, int head_dim) {
  return (bf16 && head_dim == 128) || (!bf16 && head_dim == 16);
}

int decode_lanes_per_row(bool bf16, int head_dim) { return head_dim / (bf16 ? 8 : 4); }

int launch_decode(bool bf16, bool paged, int head_dim, int gmax, const DecodeParams& p,
                  hipStream_t stream) {
  if (bf16 && head_dim == 128) {
    return paged ? launch_g<true, 128, true>(p, gmax, stream)
                 : launch_g<true, 128, false>(p, gmax, stream);
  }
  if (!bf16 && head_dim == 16) {
    return paged ? launch_g<false, 16, true>(p, gmax, stream)
                 : launch_g<false, 16, false>(p, gmax, stream);
  }
  return kEunsupported;
}

}  // namespace pkva

// Single-token GQA decode over a contiguous or block-table paged KV cache.
//
// The query of sequence b sits at position seq_lens[b] - 1 and attends to
// keys 0 .. seq_lens[b] - 1, its own key included: the row was pushed
// before the attend (frink-models 0.38.0 src/decoder/attn_block.rs,
// push_and_attend_row). Query head h reads KV head h / G (kopitiam-runtime
// 0.2.4 src/attention.rs, repeat_kv_heads).
//
// Split-K over the context with a balanced partition: all sequences' tokens
// are laid end to end and cut into equal ranges, one per workgroup, so every
// workgroup streams the same number of K/V bytes whatever the length mix.
// A workgroup owns its range for a slab of KV heads, with every query head
// of those KV heads, so each K/V byte is read from HBM exactly once.
//
// Inside a workgroup every aligned group of lanes (16 for bf16 D=128) is an
// independent worker for one KV head and one token stream (every R-th token
// of the piece): it loads the K and V rows of U tokens at once (16 bytes per
// lane), reduces q . k for its G query heads with a DPP butterfly so every
// lane holds every score, and runs the online softmax for the batch in
// registers (one rescale per batch). There is no barrier in the streaming
// loop. At the end of a sequence's piece the token streams are merged
// through LDS in a fixed tree order and the piece's (m, l, O) goes to
// workspace slot (range index + sequence index), which is unique.
// decode_combine merges a sequence's pieces in range order. Contiguous and
// paged differ only in the row address, so their arithmetic, and their
// results, are identical.
#include "common.hpp"
#include "kernels.hpp"

#include <atomic>
#include <mutex>

namespace pkva {

namespace {

constexpr int kThreads = 256;
constexpr int kHsMax = 32;       // query heads per workgroup
// Tokens per batch per lane group (K and V rows in flight) and waves per SIMD
// the kernels of groups of 4 to 7 query heads are built for: the plain
// kernel streams best with more rows in flight at two waves per SIMD, the
// kernel with the arms (more VALU per token) with fewer at three (measured).
#ifndef PKVA_DECODE_UNROLL
#define PKVA_DECODE_UNROLL 4
#endif
#ifndef PKVA_DECODE_WAVES_G4
#define PKVA_DECODE_WAVES_G4 2
#endif
#ifndef PKVA_DECODE_UNROLL_EXT
#define PKVA_DECODE_UNROLL_EXT 2
#endif
#ifndef PKVA_DECODE_WAVES_G4_EXT
#define PKVA_DECODE_WAVES_G4_EXT 3
#endif
constexpr int kUnroll = PKVA_DECODE_UNROLL;
constexpr int kWavesG4 = PKVA_DECODE_WAVES_G4;
constexpr int kUnrollExt = PKVA_DECODE_UNROLL_EXT;
constexpr int kWavesG4Ext = PKVA_DECODE_WAVES_G4_EXT;
#ifndef PKVA_DECODE_SLOTS_PCT
#define PKVA_DECODE_SLOTS_PCT 100
#endif
// Ranges per launch, in percent of the resident workgroup slots: above 100
// the dispatcher hands the later ranges to whichever unit frees a slot first.
constexpr int kSlotsPct = PKVA_DECODE_SLOTS_PCT;
constexpr int kBtWin = 1024;     // block-table entries cached in LDS per sub-piece
constexpr float kLazy = 8.0f;    // log2 headroom before the running max is moved
constexpr float kLog2e = 1.4426950408889634f;

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

// Inclusive scan of one value per thread across the workgroup (256 threads).
__device__ __forceinline__ int block_scan(int x, int* s_tmp) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
#pragma unroll
  for (int d = 1; d < 64; d *= 2) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_tmp[wave] = x;
  __syncthreads();
  int add = 0;
  for (int w = 0; w < wave; ++w) add += s_tmp[w];
  __syncthreads();
  return x + add;
}

// The keys sequence b attends to: tokens start .. start + n - 1 with n its
// valid length (0 for a length outside [1, max_seq_len]) or, with a sliding
// window, the last `window` of them.
template <bool EXT>
__device__ __forceinline__ int span_len(const DecodeParams& p, int b, int* start) {
  const int L = p.seq_lens[b];
  *start = 0;
  if (L < 1 || L > p.max_seq_len) return 0;
  if constexpr (EXT) {
    if (p.window > 0 && L > p.window) {
      *start = L - p.window;
      return p.window;
    }
  }
  return L;
}

// The logit of a score in the exp2 domain with the layer's arms,
//   log2(e) (softcap tanh(scale s / softcap) + slope (t - pos))   (softcap > 0)
//   log2(e) (scale s + slope (t - pos))                            (otherwise),
// with the constant factors folded: a = scale log2(e) (no softcap) or
// 2 log2(e) scale / softcap (the exp2 argument of the tanh), cap = softcap
// log2(e), and alibi = slope log2(e) (t - pos) computed once per token.
struct ArmConst {
  float a, cap;
  bool softcap;
};
__device__ __forceinline__ ArmConst arm_const(const DecodeParams& p) {
  ArmConst k;
  k.softcap = p.softcap > 0.0f;
  k.a = k.softcap ? p.scale * p.inv_softcap * (2.0f * kLog2e) : p.scale * kLog2e;
  k.cap = p.softcap * kLog2e;
  return k;
}
__device__ __forceinline__ float arm_logit(const ArmConst& k, float s, float alibi) {
  if (k.softcap) {
    const float e = __builtin_amdgcn_exp2f(s * k.a);
    // tanh(y) = 1 - 2 / (1 + e^(2y)): exp2 and a reciprocal; it saturates to
    // +-1 for large |y| (e^(2y) -> inf or 0) and loses only absolute
    // precision (about 1e-7) near 0.
    const float t = fmaf(-2.0f, __builtin_amdgcn_rcpf(1.0f + e), 1.0f);
    return fmaf(k.cap, t, alibi);
  }
  return fmaf(s, k.a, alibi);
}

// EXT: the arms (window, softcap, ALiBi, sinks) and keys DX elements wider
// than the values (K rows D + DX wide, V rows D wide). Scores then live in
// the exp2 domain (c = 1) instead of raw dot products.
template <bool BF16, int D, int GMAX, bool PAGED, bool WIDE = false, bool EXT = false, int DX = 0>
__global__ __launch_bounds__(kThreads, GMAX >= 8 ? 2 : (GMAX >= 4 ? (EXT ? kWavesG4Ext : kWavesG4) : 4))
void decode_partial(DecodeParams p) {
  constexpr int E = Lane16<BF16>::E;
  constexpr int LG = D / E;          // lanes per (token, kv head) row
  constexpr int NG = kThreads / LG;  // lane groups per workgroup
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int U = GMAX >= 8 ? 2 : (EXT ? kUnrollExt : kUnroll);  // tokens per batch per lane group
  constexpr int DK = D + DX;         // key width
  constexpr int LX = DX / E;         // lanes that hold a second K chunk
  static_assert(D % E == 0 && kThreads % LG == 0 && LG <= 16 && U % 2 == 0,
                "head size must split into at most 16 lanes of 16 bytes");
  static_assert(DX % E == 0 && LX <= LG && (EXT || DX == 0), "extra key width");
  // Merge buffer: per (sub-row, kv head) slice GMAX*D partial sums + GMAX m and l.
  constexpr int SLICE = GMAX * D + 2 * GMAX;

  __shared__ float s_red[(NG / 2) * SLICE];
  __shared__ int s_blk[kBtWin];
  __shared__ int s_tmp[8];
  __shared__ int s_first, s_first_cum, s_bad;

  const int wg = blockIdx.x;         // token range index
  const int slab = blockIdx.y;
  const int tid = threadIdx.x;

  // ---- total tokens (invalid lengths count as 0), the range, its first sequence
  int total = 0;
  for (int base = 0; base < p.batch; base += kThreads) {
    const int b = base + tid;
    int st;
    const int len = b < p.batch ? span_len<EXT>(p, b, &st) : 0;
    const int incl = block_scan(len, s_tmp);
    if (wg == 0 && slab == 0 && b < p.batch) p.ws_cum[b] = total + incl - len;
    if (tid == kThreads - 1) s_tmp[5] = incl;
    __syncthreads();
    total += s_tmp[5];
    __syncthreads();
  }
  const int per = max(p.min_tokens_per_range, (total + p.n_ranges - 1) / p.n_ranges);
  if (wg == 0 && slab == 0 && tid == 0) {
    p.ws_cum[p.batch] = total;       // the combine pass reads these two
    p.ws_cum[p.batch + 1] = per;
  }
  const int64_t r_begin = (int64_t)wg * per;
  if (r_begin >= total) return;
  const int64_t r_end = min<int64_t>(r_begin + per, total);
  {
    int run = 0;
    for (int base = 0; base < p.batch; base += kThreads) {
      const int b = base + tid;
      int st;
      const int len = b < p.batch ? span_len<EXT>(p, b, &st) : 0;
      const int incl = run + block_scan(len, s_tmp);
      // the one sequence with cum_excl <= r_begin < cum_incl
      if (b < p.batch && len > 0 && incl > r_begin && incl - len <= r_begin) {
        s_first = b;
        s_first_cum = incl - len;
      }
      if (tid == kThreads - 1) s_tmp[5] = incl;
      __syncthreads();
      run = s_tmp[5];
      __syncthreads();
    }
  }

  const int G = p.group;
  const int kvs = p.kvs;
  const int R = NG / kvs;            // token streams per kv head
  const int g = tid / LG, li = tid % LG;
  const int kvl = g % kvs, r = g / kvs;
  const int kvh = slab * kvs + kvl;
  const int HS = kvs * G;
  const uint32_t k_row_bytes = (uint32_t)(p.n_kv_heads * DK * ESZ);
  const uint32_t v_row_bytes = (uint32_t)(p.n_kv_heads * D * ESZ);
  const int shift = p.block_shift;
  const int bs_mask = (1 << shift) - 1;
  const float c = EXT ? 1.0f : p.scale_log2;
  const char* kbase0 = (const char*)p.k + ((int64_t)kvh * DK + li * E) * ESZ;
  const char* kxbase0 = kbase0 + D * ESZ;   // the lane's second K chunk (li < LX)
  const char* vbase0 = (const char*)p.v + ((int64_t)kvh * D + li * E) * ESZ;

  int b = s_first;
  int64_t cum = s_first_cum;
  for (; b < p.batch && cum < r_end; ++b) {
    int start;
    const int L = span_len<EXT>(p, b, &start);
    if (L == 0) continue;
    // the piece's tokens, as absolute positions in the sequence
    const int t_lo = (int)(max<int64_t>(r_begin, cum) - cum) + start;
    const int t_hi = (int)(min<int64_t>(r_end, cum + L) - cum) + start;
    cum += L;
    if (t_hi <= t_lo) continue;
    const int qpos = start + L - 1;   // the query's position

    // This lane's slice of its group's G query rows.
    uint4 q[GMAX], qx[GMAX];
    float slope[GMAX];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      q[h] = make_uint4(0, 0, 0, 0);
      qx[h] = make_uint4(0, 0, 0, 0);
      slope[h] = 0.0f;
      if (h < G) {
        const int head = kvh * G + h;
        const int64_t qoff = ((int64_t)b * p.n_heads + head) * DK + li * E;
        q[h] = *(const uint4*)((const char*)p.q + qoff * ESZ);
        if constexpr (DX > 0) {
          if (li < LX) qx[h] = *(const uint4*)((const char*)p.q + (qoff + D) * ESZ);
        }
        if constexpr (EXT) {
          if (p.alibi != nullptr) slope[h] = p.alibi[head] * kLog2e;   // exp2 domain
        }
      }
    }
    const ArmConst ak = arm_const(p);
    float acc[GMAX][E];
    float m[GMAX], l[GMAX];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] = 0.0f;
    }
    bool bad = false;
    const int seq_row0 = PAGED ? 0 : b * p.kv_capacity;   // first cache row of sequence b

    // Tokens [c0, c1) of the piece, with the block ids they touch in the LDS
    // window (at most kBtWin). Returns false when a block lies outside the
    // pool (then nothing is read).
    auto sub_piece = [&](int c0, int c1) -> bool {
      int blk0 = 0;
      if constexpr (PAGED) {
        blk0 = c0 >> shift;
        const int nblk = ((c1 - 1) >> shift) - blk0 + 1;
        __syncthreads();   // previous readers are done with s_blk
        if (tid == 0) s_bad = 0;
        __syncthreads();
        for (int i = tid; i < nblk; i += kThreads) {
          const int id = p.block_table[(int64_t)b * p.max_blocks_per_seq + blk0 + i];
          s_blk[i] = id;
          if (id < 0 || id >= p.num_blocks) s_bad = 1;
        }
        __syncthreads();
        if (s_bad) return false;
      }

      // Load the K (or V) rows of the batch starting at token t0. Rows past the
      // piece read as zero.
      auto row_of = [&](int t) -> uint64_t {
        // pool (or cache) row index; the host checks that it fits in 31 bits
        return PAGED ? (uint32_t)((s_blk[(t >> shift) - blk0] << shift) + (t & bs_mask))
                     : (uint32_t)(seq_row0 + t);
      };
      // K and V bytes are read exactly once: non-temporal loads keep them from
      // displacing other lines in the caches (and from the write-back of dirty
      // lines they would otherwise force).
      auto load_rows = [&](uint4 (&x)[U], const char* base, uint32_t row_bytes, int t0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int t = t0 + u * R;
          x[u] = make_uint4(0, 0, 0, 0);
          if (t < c1) x[u] = load_nt16(base + row_of(t) * row_bytes);
        }
      };
      // K rows: the lane's chunk, and its second chunk when the keys are wider.
      auto load_k = [&](uint4 (&x)[U], uint4 (&xx)[DX > 0 ? U : 1], int t0) {
        load_rows(x, kbase0, k_row_bytes, t0);
        if constexpr (DX > 0) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int t = t0 + u * R;
            xx[u] = make_uint4(0, 0, 0, 0);
            if (li < LX && t < c1) xx[u] = load_nt16(kxbase0 + row_of(t) * k_row_bytes);
          }
        }
      };
      // Scores, online softmax and p * v for the batch at t0.
      // Scores, online softmax and p * v for the batch at t0; as soon as the
      // K (then V) rows of this batch are consumed, the registers are refilled
      // with the next batch's rows, so a batch is always in flight.
      auto consume = [&](uint4 (&kx)[U], uint4 (&kx2)[DX > 0 ? U : 1], uint4 (&vx)[U], int t0) {
        const int tn = t0 + R * U;   // next batch
        float s[U][GMAX];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          dot_rows<BF16, GMAX>(q, kx[u], s[u]);
          if constexpr (DX > 0) {
            float s2[GMAX];
            dot_rows<BF16, GMAX>(qx, kx2[u], s2);
#pragma unroll
            for (int h = 0; h < GMAX; ++h) s[u][h] += s2[h];
          }
#pragma unroll
          for (int h = 0; h < GMAX; ++h) s[u][h] = group_sum<LG>(s[u][h]);
          if constexpr (EXT) {
#pragma unroll
            for (int h = 0; h < GMAX; ++h)
              s[u][h] = arm_logit(ak, s[u][h], slope[h] * (float)(t0 + u * R - qpos));
          }
        }
        load_k(kx, kx2, tn);
        // Online softmax against a reference max m: rescale only when a score
        // exceeds m by more than 2^kLazy in the exp2 domain (weights stay <= 2^kLazy).
        bool grow = false;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int h = 0; h < GMAX; ++h)
            if (t0 + u * R < c1) grow |= (s[u][h] - m[h]) * c > kLazy;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {   // wave-uniform branch
#pragma unroll
          for (int h = 0; h < GMAX; ++h) {
            float mb = s[0][h];
#pragma unroll
            for (int u = 1; u < U; ++u)
              if (t0 + u * R < c1) mb = fmaxf(mb, s[u][h]);
            const float m_new = fmaxf(m[h], mb);
            const float alpha = m[h] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((m[h] - m_new) * c);
            m[h] = m_new;
            l[h] *= alpha;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[h][e] *= alpha;
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int h = 0; h < GMAX; ++h) {   // the weights overwrite the scores
            s[u][h] = t0 + u * R < c1 ? __builtin_amdgcn_exp2f((s[u][h] - m[h]) * c) : 0.0f;
            l[h] += s[u][h];
          }
        if constexpr (BF16) {
          // p * v over token pairs on v_dot2_f32_bf16: (p_u, p_u+1) . (v_u[e], v_u+1[e])
#pragma unroll
          for (int u = 0; u < U; u += 2) {
            uint32_t vp[E];
            const uint32_t a[4] = {vx[u].x, vx[u].y, vx[u].z, vx[u].w};
            const uint32_t bb[4] = {vx[u + 1].x, vx[u + 1].y, vx[u + 1].z, vx[u + 1].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              vp[2 * i] = __builtin_amdgcn_perm(bb[i], a[i], 0x05040100u);      // low halves
              vp[2 * i + 1] = __builtin_amdgcn_perm(bb[i], a[i], 0x07060302u);  // high halves
            }
#pragma unroll
            for (int h = 0; h < GMAX; ++h) {
              const uint32_t pp = pack_bf16x2(s[u][h], s[u + 1][h]);
#pragma unroll
              for (int e = 0; e < E; ++e) acc[h][e] = dot2_bf16(pp, vp[e], acc[h][e]);
            }
          }
        } else {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            float x[E];
            unpack16<BF16>(vx[u], x);
#pragma unroll
            for (int h = 0; h < GMAX; ++h)
#pragma unroll
              for (int e = 0; e < E; ++e) acc[h][e] = fmaf(s[u][h], x[e], acc[h][e]);
          }
        }
        load_rows(vx, vbase0, v_row_bytes, tn);
      };
      uint4 kx[U], kx2[DX > 0 ? U : 1], vx[U];
      load_k(kx, kx2, c0 + r);
      load_rows(vx, vbase0, v_row_bytes, c0 + r);
      for (int t0 = c0 + r; t0 < c1; t0 += R * U) consume(kx, kx2, vx, t0);
      return true;
    };
    if constexpr (PAGED && WIDE) {
      // Pieces whose blocks may exceed the window: sub-pieces of at most
      // kBtWin - 1 blocks (at most kBtWin block ids once misaligned). The span
      // is a multiple of R * U tokens, so every stream takes the same tokens
      // in the same batches as in one pass over the piece: the arithmetic,
      // and the result, match the contiguous kernel bit for bit.
      // (R * U is a power of two no larger than 128 <= (kBtWin - 1) << shift.)
      const int span = ((kBtWin - 1) << shift) & ~(R * U - 1);
      for (int c0 = t_lo; c0 < t_hi; c0 += span) {
        if (!sub_piece(c0, min(t_hi, c0 + span))) { bad = true; break; }
      }
    } else {
      // The launcher has checked that every piece's blocks fit in the window:
      // no loop here, which keeps the kernel's registers down.
      bad = !sub_piece(t_lo, t_hi);
    }

    const int64_t slot = (int64_t)(wg + b) * p.n_heads + (int64_t)slab * HS;
    if (bad) {
      if (tid < HS) {
        p.ws_ml[(slot + tid) * 2 + 0] = 0.0f;
        p.ws_ml[(slot + tid) * 2 + 1] = __builtin_nanf("");
      }
      __syncthreads();
      continue;
    }
    // ---- fixed-order tree over the token streams: state(r) (+)= state(r + s)
    for (int s2 = R / 2; s2 >= 1; s2 /= 2) {
      __syncthreads();
      if (r >= s2 && r < 2 * s2) {
        float* dst = s_red + ((r - s2) * kvs + kvl) * SLICE;
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
#pragma unroll
          for (int e = 0; e < E; ++e) dst[(h * E + e) * LG + li] = acc[h][e];
          if (li == 0) {
            dst[GMAX * D + h] = m[h];
            dst[GMAX * D + GMAX + h] = l[h];
          }
        }
      }
      __syncthreads();
      if (r < s2) {
        const float* src = s_red + (r * kvs + kvl) * SLICE;
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
          const float mo = src[GMAX * D + h];
          const float M = fmaxf(m[h], mo);
          const float a = m[h] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((m[h] - M) * c);
          const float bo = mo == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((mo - M) * c);
          m[h] = M;
          l[h] = l[h] * a + src[GMAX * D + GMAX + h] * bo;
#pragma unroll
          for (int e = 0; e < E; ++e) acc[h][e] = acc[h][e] * a + src[(h * E + e) * LG + li] * bo;
        }
      }
    }
    if (r == 0) {
#pragma unroll
      for (int h = 0; h < GMAX; ++h) {
        if (h < G) {
          float* d = p.ws_o + (slot + kvl * G + h) * D + li * E;
#pragma unroll
          for (int e = 0; e < E; e += 4) {
            const f32x4_t w = {acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]};
            store_nt((f32x4_t*)(d + e), w);
          }
          if (li == 0) {
            store_nt(p.ws_ml + (slot + kvl * G + h) * 2 + 0, m[h] * c);
            store_nt(p.ws_ml + (slot + kvl * G + h) * 2 + 1, l[h]);
          }
        }
      }
    }
    __syncthreads();
  }
}

// Merge the pieces of one sequence in range order, one thread per output:
//   o = sum_w 2^(m_w - M) O_w / sum_w 2^(m_w - M) l_w,  M = max_w m_w,
// computed with a running maximum (EXT: a head's sink logit joins the
// denominator at the end, with no value). The loads of up to kCombineBatch
// pieces are issued together, so a typical sequence costs one memory round trip.
constexpr int kCombineBatch = 16;

template <bool BF16, int D, bool EXT>
__global__ __launch_bounds__(kThreads) void decode_combine(DecodeParams p) {
  constexpr int HPW = kThreads / D > 0 ? kThreads / D : 1;  // heads per workgroup
  const int hgroups = (p.n_heads + HPW - 1) / HPW;
  const int b = blockIdx.x / hgroups;
  const int h = (blockIdx.x % hgroups) * HPW + threadIdx.x / D;
  const int d = threadIdx.x % D;
  if (h >= p.n_heads) return;
  int start;
  const int L = span_len<EXT>(p, b, &start);
  float out = __builtin_nanf("");
  if (L > 0) {
    const int per = p.ws_cum[p.batch + 1];
    const int cb = p.ws_cum[b];
    const int w0 = cb / per, w1 = (cb + L - 1) / per;
    float M = -INFINITY, num = 0.0f, den = 0.0f;
    for (int w = w0; w <= w1; w += kCombineBatch) {
      float mm[kCombineBatch], ll[kCombineBatch], oo[kCombineBatch];
#pragma unroll
      for (int j = 0; j < kCombineBatch; ++j) {
        const int64_t s = (int64_t)(w + j + b) * p.n_heads + h;
        const bool ok = w + j <= w1;
        mm[j] = ok ? p.ws_ml[s * 2] : -INFINITY;
        ll[j] = ok ? p.ws_ml[s * 2 + 1] : 0.0f;
        oo[j] = ok ? p.ws_o[s * D + d] : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < kCombineBatch; ++j) {
        if (w + j <= w1) {
          const float Mn = fmaxf(M, mm[j]);
          const float a = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
          const float wt = __builtin_amdgcn_exp2f(mm[j] - Mn);
          num = fmaf(wt, oo[j], num * a);
          den = fmaf(wt, ll[j], den * a);
          M = Mn;
        }
      }
    }
    if constexpr (EXT) {
      if (p.sinks != nullptr) {
        const float sk = p.sinks[h] * kLog2e;
        const float Mn = fmaxf(M, sk);
        const float a = __builtin_amdgcn_exp2f(M - Mn);
        num *= a;
        den = den * a + __builtin_amdgcn_exp2f(sk - Mn);
      }
    }
    out = num / den;
  }
  const int64_t o = ((int64_t)b * p.n_heads + h) * D + d;
  if constexpr (BF16) {
    store_nt((__bf16*)p.o + o, (__bf16)out);
  } else {
    store_nt((float*)p.o + o, out);
  }
}

// Per-device facts the launcher needs on every call, looked up once per
// device (compute units, and the resident workgroups per unit of each
// kernel instantiation): the runtime queries cost microseconds per call.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];   // 0 = not looked up yet

// Token ranges for one launch: one per workgroup slot the device can keep
// resident (compute units x workgroups per unit), never more than the
// workspace holds or than min-size ranges the batch can fill. The slot count
// is the smaller of the contiguous and paged kernels' occupancy, so the two
// entry points always cut the same ranges and stay bitwise equal.
template <bool BF16, int D, int GMAX, bool EXT, int DX>
int resident_ranges(const DecodeParams& p) {
  static std::atomic<int> slots_per_cu[kMaxDevices];   // per instantiation; 0 = not yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  int cus = g_cus[dev].load(std::memory_order_relaxed);
  int occ = slots_per_cu[dev].load(std::memory_order_relaxed);
  if (cus <= 0 || occ <= 0) {
    int occ_c = 0, occ_p = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &occ_c, decode_partial<BF16, D, GMAX, false, false, EXT, DX>, kThreads, 0) != hipSuccess)
      return -1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &occ_p, decode_partial<BF16, D, GMAX, true, false, EXT, DX>, kThreads, 0) != hipSuccess)
      return -1;
    occ = max(1, min(occ_c, occ_p));
    // Two threads may both look it up; they store the same values.
    g_cus[dev].store(cus, std::memory_order_relaxed);
    slots_per_cu[dev].store(occ, std::memory_order_relaxed);
  }
  const int slots = (int)((int64_t)cus * occ * kSlotsPct / 100 / p.nslab);
  return max(1, min(p.n_ranges, slots));
}

template <bool BF16, int D, int GMAX, bool PAGED, bool EXT, int DX>
int launch_one(DecodeParams p, hipStream_t stream) {
  p.n_ranges = resident_ranges<BF16, D, GMAX, EXT, DX>(p);
  if (p.n_ranges < 1) return kEhip;
  dim3 grid(p.n_ranges, p.nslab);
  // A piece holds at most `per` tokens, per <= max(min range, ceil(B * max_len / ranges)),
  // so it touches at most per / block_size + 2 blocks.
  const int64_t by_len = ((int64_t)p.batch * p.max_seq_len + p.n_ranges - 1) / p.n_ranges;
  const int64_t per_max = by_len > p.min_tokens_per_range ? by_len : p.min_tokens_per_range;
  const bool wide = PAGED && (per_max >> p.block_shift) + 2 > kBtWin;
  if (wide) {
    hipLaunchKernelGGL((decode_partial<BF16, D, GMAX, PAGED, true, EXT, DX>), grid, dim3(kThreads),
                       0, stream, p);
  } else {
    hipLaunchKernelGGL((decode_partial<BF16, D, GMAX, PAGED, false, EXT, DX>), grid, dim3(kThreads),
                       0, stream, p);
  }
  if (hipGetLastError() != hipSuccess) return kEhip;
  constexpr int HPW = kThreads / D > 0 ? kThreads / D : 1;
  const int cgrid = p.batch * ((p.n_heads + HPW - 1) / HPW);
  hipLaunchKernelGGL((decode_combine<BF16, D, EXT>), dim3(cgrid), dim3(kThreads), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return kEhip;
  return kOk;
}

template <bool BF16, int D, bool PAGED, bool EXT, int DX>
int launch_g(const DecodeParams& p, int gmax, hipStream_t stream) {
  switch (gmax) {
    case 1: return launch_one<BF16, D, 1, PAGED, EXT, DX>(p, stream);
    case 2: return launch_one<BF16, D, 2, PAGED, EXT, DX>(p, stream);
    case 4: return launch_one<BF16, D, 4, PAGED, EXT, DX>(p, stream);
    case 8: return launch_one<BF16, D, 8, PAGED, EXT, DX>(p, stream);
    default: return kEunsupported;
  }
}

template <bool BF16, int D, bool EXT, int DX>
int launch_p(bool paged, const DecodeParams& p, int gmax, hipStream_t stream) {
  return paged ? launch_g<BF16, D, true, EXT, DX>(p, gmax, stream)
               : launch_g<BF16, D, false, EXT, DX>(p, gmax, stream);
}

}  // namespace

// ---- scratch of attn_decode_paged_noalloc
// The split partials, maxima, sums and prefix sums of one call, in the layout
// of the caller-provided workspace, in a fixed device array: each device
// that runs the library holds its own copy until the process ends. Calls
// that overlap on one device share it and race; nothing in it has to start
// at zero (every slot a call reads was written earlier in the same call).
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

namespace {
std::atomic<void*> g_scratch[kMaxDevices];   // device address of each device's copy
std::mutex g_scratch_mu;
}  // namespace

size_t decode_scratch_bytes() { return kScratchBytes; }

// The current device's address of the scratch array, looked up once per
// device with that device current (the array's name in host code is only a
// stand-in for the symbol, never a device address). Null on failure.
void* decode_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr != nullptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ptr = g_scratch[dev].load(std::memory_order_relaxed);
  if (ptr == nullptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

int decode_max_ranges() { return 2048; }          // 256 CUs x 8 resident workgroups
int decode_min_tokens_per_range() { return 64; }
int decode_heads_per_slab_max() { return kHsMax; }

bool decode_supported(bool bf16, int head_dim) {
  return (bf16 && head_dim == 128) || (!bf16 && head_dim == 16);
}

bool decode_ext_supported(bool bf16, int head_dim, int v_head_dim) {
  return bf16 ? (v_head_dim == 128 && (head_dim == 128 || head_dim == 192))
              : (head_dim == 16 && v_head_dim == 16);
}

int decode_lanes_per_row(bool bf16, int head_dim) { return head_dim / (bf16 ? 8 : 4); }

int launch_decode(bool bf16, bool paged, int head_dim, int gmax, const DecodeParams& p,
                  hipStream_t stream) {
  if (p.ext) {
    if (bf16 && p.v_head_dim == 128 && head_dim == 128)
      return launch_p<true, 128, true, 0>(paged, p, gmax, stream);
    if (bf16 && p.v_head_dim == 128 && head_dim == 192)
      return launch_p<true, 128, true, 64>(paged, p, gmax, stream);
    if (!bf16 && head_dim == 16 && p.v_head_dim == 16)
      return launch_p<false, 16, true, 0>(paged, p, gmax, stream);
    return kEunsupported;
  }
  if (bf16 && head_dim == 128) return launch_p<true, 128, false, 0>(paged, p, gmax, stream);
  if (!bf16 && head_dim == 16) return launch_p<false, 16, false, 0>(paged, p, gmax, stream);
  return kEunsupported;
}

}  // namespace pkva

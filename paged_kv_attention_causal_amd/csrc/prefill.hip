// Multi-token causal GQA prefill over a contiguous or block-table paged K/V.
//
// Row i of the query sits at absolute position position_offset + i and
// attends to keys j <= position_offset + i, j < seq_kv (kopitiam-runtime
// 0.2.4 src/attention.rs, causal_mask); query head h reads KV head h / G
// (repeat_kv_heads). The softmax is computed online over key tiles.
//
// One workgroup = 8 waves = 256 query rows of one (sequence, head); each
// wave owns 32 rows, and a compute unit holds one workgroup (two waves per
// SIMD), so that the last workgroups of a launch still keep every SIMD
// busy with two waves, and one copy of each key tile serves 256 rows. Key
// tiles of 64 rows reach LDS by global -> LDS copies (no staging
// registers) into two rings, K one tile ahead of V, so that one step
// overlaps MFMAs with the VALU softmax:
//   step t (bf16): copy K(t+2), V(t+1); S(t+1) = K(t+1) Q^T; O^T += V(t)^T
//   P(t)^T while the VALU makes P(t+1) = exp2(S(t+1) - m) in bf16 and its
//   row sums; the row max of S(t+1) is taken only when a row sum shows that
//   m could move (and P(t+1) is made again in the rare step that moves it);
//   one barrier. P, not S, is what crosses the barrier.
//   step t (fp32): copy K(t+2), V(t+1); S(t+1) = K(t+1) Q^T while P(t) =
//   exp2(S(t) - m); O^T += V(t)^T P(t)^T; row max of S(t+1); one barrier.
// The LDS image of a tile spreads rows over the banks so that the operand
// reads are free of bank conflicts with lane-base-plus-immediate addresses:
//   S^T = K Q^T on 32x32 MFMAs (Q^T in registers as the B operand): in the
//     accumulator layout lane l owns query row l % 32 and 16 of each 32 keys,
//     the other 16 sit in lane l ^ 32; the row max needs one cross-half
//     exchange (v_permlane32_swap), the row sum stays per lane until the end;
//   O^T += V^T P^T takes P straight from the accumulator registers (bf16
//     for the bf16 instantiation); the V^T operand comes from the row-major
//     V tile through ds_read_b64_tr_b16, which hands each lane one column of
//     four consecutive rows, in the accumulator's key order;
//   the running max moves only when a row's max grows by more than 2^8 in
//     the exp2 domain (then O and l are rescaled), so most tiles skip it.
// Key tiles wholly above the diagonal are never visited; only tiles that
// cross the diagonal or the end of the keys apply the mask.
#include "common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace pkva {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kBlockM = 32 * kWaves;   // query rows per workgroup (32 per wave)
constexpr int kBlockN = 64;    // keys per tile
constexpr int kBtWin = 256;    // block-table entries cached in LDS
constexpr int kXcds = 8;       // accelerator complex dies, each with its own L2
constexpr float kLazy = 8.0f;  // log2 headroom before the running max moves
constexpr float kNoMaxSum = 128.0f;   // 2^(kLazy - 1)
constexpr int kSortMax = 128;  // ragged batches with up to this many (sequence, tile) pairs are
                               // dispatched in work order

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

// Transposed LDS read: four consecutive rows of one 16-bit column per lane.
__device__ __forceinline__ bf16x4_t ds_read_tr16(const void* p) {
  typedef __attribute__((ext_vector_type(4))) short s16x4;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(__attribute__((address_space(3))) char*)(p));
  return __builtin_bit_cast(bf16x4_t, v);
}

template <bool BF16, int D, bool PAGED, bool VARLEN>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillParams p) {
  using M = Mfma<BF16>;
  using T = typename M::Elem;
  constexpr int ESZ = sizeof(T);
  constexpr int E = 16 / ESZ;                 // elements per 16-byte chunk
  constexpr int ROWB = D * ESZ;               // bytes per K/V row
  constexpr int CPR = ROWB / 16;              // chunks per row
  // LDS image of a key tile, filled by global -> LDS copies of 1 KB (64 lanes
  // x 16 bytes, back to back in LDS). bf16 (256-byte rows): copy x holds rows
  // x, x + 16, x + 32, x + 48 and sits at sigma(x) * 1040 bytes with
  // sigma(4u + j) = 4j + u. The 16 rows of a K-operand read then start in 16
  // different 16-byte bank groups, the 4 rows x 4 chunks of a transposed V
  // read are disjoint, and every address is a lane base plus an immediate.
  // fp32 (64-byte rows, the small head size): rows back to back.
  constexpr int NCH = kBlockN * CPR;          // chunks per tile
  constexpr int kCopies = NCH / 64;           // 1 KB copies per tile
  constexpr int kCopiesW = (kCopies + kWaves - 1) / kWaves;   // per wave (at most)
  constexpr int TILEB = BF16 ? 15 * 1040 + 1024 : kBlockN * ROWB;
  constexpr int DB = (D + 31) / 32;           // 32-row blocks of O^T
  constexpr int KSTEPS = D / M::K;            // MFMAs per 32x32 S^T block
  static_assert(D % E == 0 && D % M::K == 0, "unsupported head size");
  static_assert(!BF16 || CPR == 16, "the bf16 path is laid out for 256-byte rows");
  static_assert(NCH % 64 == 0, "whole copies");
  constexpr int OROW = ROWB + 16;             // padded LDS row of the output tile
  constexpr int LDSB = 4 * TILEB > kBlockM * OROW ? 4 * TILEB : kBlockM * OROW;

  // [0][slot] = K ring, [1][slot] = V ring. K runs one tile ahead of V.
  __shared__ __attribute__((aligned(16))) char s_lds[LDSB];
  // ring(0, slot) = K slot, ring(1, slot) = V slot. K runs one tile ahead of V.
  auto ring = [&](int kv, int slot) -> char* { return s_lds + (kv * 2 + slot) * TILEB; };
  __shared__ int s_bt[PAGED ? kBtWin : 1];
  __shared__ int s_bad;

  // Work order: heaviest query tiles first; within a tile level, sequence,
  // then head (the heads of one KV head adjacent). Workgroups are handed to
  // the 8 XCDs round robin (XCD = id % 8), and each XCD has its own L2: so
  // in every run of 8 x group ids, XCD x takes the group heads that share
  // one KV head, which then read the same key tiles at the same time.
  int work = blockIdx.x;
  {
    const int span = kXcds * p.group;
    if ((int)(blockIdx.x / span + 1) * span <= (int)gridDim.x) {
      const int g = blockIdx.x / span, x = blockIdx.x % kXcds, j = (blockIdx.x / kXcds) % p.group;
      work = g * span + x * p.group + j;
    }
  }
  const int per_level = p.batch * p.n_heads;
  int level = work / per_level;
  const int rest = work % per_level;
  int h = rest % p.n_heads;
  int b = rest / p.n_heads;

  // The sequence's query rows, keys and offset: shared by the batch, or
  // (ragged batch) its own, with its query rows packed after the previous
  // sequence's and the chunk being the last seq_q of its seq_kv tokens.
  int seq_q = p.seq_q, seq_kv = p.seq_kv, off = p.position_offset;
  int64_t q_row0 = (int64_t)b * p.seq_q;   // the sequence's first row of q and o
  int qt;                                    // query tile of this work item
  bool poisoned = false;                     // bad sizes or block ids: NaN rows
  if constexpr (VARLEN) {
    // Ragged batches: the (sequence, tile level) pairs go out heaviest first
    // by their key-tile steps (longest processing time first), so that a
    // light tile of a short history does not hold a slot while heavier ones
    // of other sequences wait. Workgroup w takes pair number w / n_heads of
    // that order, head w % n_heads; the pairs are those of the level order
    // (level l: the sequence's tile tiles - 1 - l). Every thread ranks one
    // candidate pair against all others (up to kSortMax pairs; larger
    // batches keep the level order).
    const int n_cand = p.batch * p.q_tiles;
    if (n_cand <= kSortMax) {
      __shared__ int s_steps[kSortMax];
      __shared__ int s_sel;
      const int t = threadIdx.x;
      int steps = -1;
      if (t < n_cand) {
        const int cb = t / p.q_tiles, cl = t % p.q_tiles;
        const int c0 = p.cu_q[cb], c1 = p.cu_q[cb + 1];
        const int cq = (c1 - c0 + kBlockM - 1) / kBlockM - 1 - cl;   // its query tile
        if (c0 >= 0 && c1 >= c0 && c1 <= p.total_q && cq >= 0) {
          const int rows = min(kBlockM, c1 - c0 - cq * kBlockM);
          const int64_t last = (int64_t)p.kv_lens[cb] - (c1 - c0) + (int64_t)cq * kBlockM + rows - 1;
          const int64_t st = last < 0 ? 0 : last / kBlockN + 1;
          steps = st > (1 << 30) ? (1 << 30) : (int)st;
        }
      }
      if (t < kSortMax) s_steps[t] = steps;
      if (t == 0) s_sel = -1;
      __syncthreads();
      if (steps >= 0) {
        int rank = 0;
        for (int u = 0; u < n_cand; ++u) {
          const int su = s_steps[u];
          rank += su > steps || (su == steps && u < t);
        }
        if (rank == work / p.n_heads) s_sel = t;
      }
      __syncthreads();
      if (s_sel < 0) return;   // uniform: no pair of this rank
      b = s_sel / p.q_tiles;
      level = s_sel % p.q_tiles;
      h = work % p.n_heads;
    }
  }
  const int kvh = h / p.group;

  if constexpr (VARLEN) {
    const int s0 = p.cu_q[b], s1 = p.cu_q[b + 1];
    // Rows outside [0, total_q): nothing of this sequence can be written.
    if (s0 < 0 || s1 < s0 || s1 > p.total_q) return;
    seq_q = s1 - s0;
    q_row0 = s0;
    seq_kv = p.kv_lens[b];
    off = seq_kv - seq_q;
    // Tile levels count from each sequence's last (heaviest) tile.
    qt = (seq_q + kBlockM - 1) / kBlockM - 1 - level;
    if (qt < 0) return;   // uniform over the workgroup
    const int64_t cap = PAGED ? (int64_t)p.max_blocks_per_seq << p.block_shift : p.kv_capacity;
    poisoned = off < 0 || seq_kv > cap || seq_q > p.seq_q;
  } else {
    qt = p.q_tiles - 1 - level;
  }

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int lr = lane % 32, hf = lane / 32;
  const int q0 = qt * kBlockM;
  const uint32_t row_bytes = (uint32_t)(p.n_kv_heads * ROWB);
  const int shift = p.block_shift;
  const int bs_mask = (1 << shift) - 1;

  // Keys this tile can see: 0 .. last_key.
  const int q_last = min(q0 + kBlockM, seq_q) - 1;
  const int last_key = min(seq_kv - 1, off + q_last);
  const int n_kt = last_key / kBlockN + 1;

  const char* kg = (const char*)p.k + (int64_t)kvh * ROWB;
  const char* vg = (const char*)p.v + (int64_t)kvh * ROWB;
  const int32_t* bt_row = PAGED ? p.block_table + (int64_t)b * p.max_blocks_per_seq : nullptr;
  const int seq_row0 = PAGED ? 0 : b * p.kv_capacity;
  int win0 = 0, win_end = 0;   // block-table window [win0, win_end) held in s_bt
  if (tid == 0) s_bad = 0;

  // (Re)load the block-table window so it starts at block blk; validates ids.
  auto load_window = [&](int blk) {
    __syncthreads();
    win0 = blk;
    win_end = min(blk + kBtWin, (last_key >> shift) + 1);
    for (int i = tid; i < win_end - win0; i += kThreads) {
      const int id = bt_row[win0 + i];
      s_bt[i] = id;
      if (id < 0 || id >= p.num_blocks) s_bad = 1;
    }
    __syncthreads();
  };
  // Make sure the window holds every block of key tiles lo .. hi (lo's first
  // block is where a reload starts). False on a bad block id.
  auto cover = [&](int lo, int hi) -> bool {
    if constexpr (PAGED) {
      const int last = min(last_key, hi * kBlockN + kBlockN - 1) >> shift;
      if (last >= win_end) {   // uniform: every thread holds the same window
        load_window((lo * kBlockN) >> shift);
        if (s_bad) return false;
      }
    }
    return true;
  };

  // Byte offset of copy x, and of key row r, inside a tile's LDS image.
  auto copy_off = [](int x) -> int { return BF16 ? (4 * (x % 4) + x / 4) * 1040 : 1024 * x; };
  auto row_off = [&](int r) -> int { return BF16 ? copy_off(r % 16) + 256 * (r / 16) : r * ROWB; };

  // Copy the K (or V) rows of key tile kt into the LDS image at slot: this
  // wave's share of the copies, 16 bytes per lane. Rows past last_key copy
  // row last_key instead (finite data; the mask and P = 0 discard them), so
  // every wave always issues kCopiesW copies.
  // A whole tile (no row past last_key) takes a fixed lane offset per copy.
  uint32_t whole_off[kCopiesW];
#pragma unroll
  for (int jj = 0; jj < kCopiesW; ++jj) {
    const int x = wave + kWaves * jj;
    const int row = BF16 ? x + 16 * (lane / 16) : 16 * x + lane / CPR;
    whole_off[jj] = (uint32_t)row * row_bytes + (lane % CPR) * 16;
  }
  auto issue = [&](const char* g, int kt, char* slot) __attribute__((always_inline)) {
    const int k0 = kt * kBlockN;
    const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(slot);
    if (!PAGED && k0 + kBlockN - 1 <= last_key) {   // uniform
#pragma unroll
      for (int jj = 0; jj < kCopiesW; ++jj) {
        const int x = wave + kWaves * jj;
        if (kCopies % kWaves != 0 && x >= kCopies) break;
        dma16(g + (int64_t)(seq_row0 + k0) * row_bytes, whole_off[jj], lds + copy_off(x));
      }
      return;
    }
#pragma unroll
    for (int jj = 0; jj < kCopiesW; ++jj) {
      const int x = wave + kWaves * jj;
      if (kCopies % kWaves != 0 && x >= kCopies) break;
      const int row = BF16 ? x + 16 * (lane / 16) : 16 * x + lane / CPR;
      const int cc = lane % CPR;
      const int t = min(k0 + row, last_key);
      if constexpr (PAGED) {
        const uint32_t prow = (uint32_t)((s_bt[(t >> shift) - win0] << shift) + (t & bs_mask));
        dma16_addr(g + (uint64_t)prow * row_bytes + cc * 16, lds + copy_off(x));
      } else {
        dma16(g + (int64_t)(seq_row0 + k0) * row_bytes, (uint32_t)(t - k0) * row_bytes + cc * 16,
              lds + copy_off(x));
      }
    }
  };

  if constexpr (PAGED) {
    if (!poisoned) {
      load_window(0);
      poisoned = s_bad != 0;
    }
  }

  if (!poisoned) {
    // Q^T as the B operand: lane holds query row q0 + 32*wave + lr.
    const int qrow = q0 + wave * 32 + lr;
    typename M::Op qB[KSTEPS];
    {
      const T* qgp = (const T*)p.q + ((q_row0 + qrow) * p.n_heads + h) * D;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        if constexpr (BF16) {
          qB[kk] = qrow < seq_q ? *(const bf16x8_t*)(qgp + kk * 16 + hf * 8) : bf16x8_t{};
        } else {
          qB[kk] = qrow < seq_q ? qgp[kk * 2 + hf] : 0.0f;
        }
      }
    }

    f32x16_t oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16_t{};
    float m_ref = -INFINITY;   // reference max of raw scores for this lane's row
    float l_run = 0.0f;        // this lane's share of the running sum
    const float c = p.scale_log2;
    const int wave_pos_first = off + q0 + wave * 32;
    const int my_pos = off + qrow;
    const bool wave_live = q0 + wave * 32 < seq_q;
    // Tiles this wave computes (0 .. n_w - 1), and the first one that needs
    // the mask (crosses the wave's diagonal or the end of the keys).
    const int n_w = wave_live ? min(n_kt, (wave_pos_first + 31) / kBlockN + 1) : 0;
    const int kt_open = min(min((wave_pos_first + 1) / kBlockN, seq_kv / kBlockN), n_w);

    // S^T = K Q^T for the K tile at sK.
    auto qk = [&](const char* sK, f32x16_t (&s)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16_t acc = f32x16_t{};
        const int row = kb * 32 + lr;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          typename M::Op a;
          if constexpr (BF16) {
            a = *(const bf16x8_t*)(sK + row_off(row) + (2 * kk + hf) * 16);
          } else {
            a = *(const float*)(sK + row_off(row) + (kk * 2 + hf) * 4);
          }
          acc = M::mma(a, qB[kk], acc);
        }
        s[kb] = acc;
      }
    };
    // Accumulator register r of key block kb holds key k0 + 32*kb + 8*(r/4) + 4*hf + r%4.
    auto mask = [&](int k0, f32x16_t (&s)[2]) __attribute__((always_inline)) {
      const int lim = min(my_pos, seq_kv - 1) - (k0 + 4 * hf);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * kb + 8 * (r / 4) + (r % 4) > lim) s[kb][r] = -INFINITY;
    };
    // Row max over the tile (this lane's 32 keys, then across the two lane
    // halves); the reference max moves only when it grows by more than
    // 2^kLazy, and then O and l are rescaled. (maximum, not maxnum: no
    // canonicalising moves; scores carry no NaN unless the inputs do, and
    // then the row is NaN either way.)
    auto row_max = [&](const f32x16_t (&s)[2]) __attribute__((always_inline)) -> float {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2)
          mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, s[kb][r]), s[kb][r + 1]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      return __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    };
    // True (and O, l rescaled to the new reference max) if the max moved.
    auto rescale_if_grown = [&](float mx) __attribute__((always_inline)) -> bool {
      if (__builtin_amdgcn_ballot_w64((mx - m_ref) * c > kLazy) == 0) return false;   // wave-uniform
      const float m_new = fmaxf(m_ref, mx);
      const float alpha =
          m_ref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((m_ref - m_new) * c);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      return true;
    };
    auto update_max = [&](const f32x16_t (&s)[2]) __attribute__((always_inline)) {
      rescale_if_grown(row_max(s));
    };
    // fp32: P = 2^((s - m_ref) c) in place, l += row sums of P, O^T += V^T P^T.
    auto exp_pv = [&](f32x16_t (&s)[2], const char* sV) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[kb][r] = __builtin_amdgcn_exp2f((s[kb][r] - m_ref) * c);   // masked: exp2(-inf) = 0
      if constexpr (!BF16) {
        float psum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) psum += s[kb][r];
        l_run += psum;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const int d = db * 32 + lr;
              const float a = d < D ? *(const float*)(sV + row_off(key) + d * 4) : 0.0f;
              oacc[db] = M::mma(a, s[kb][r], oacc[db]);
            }
          }
      }
    };

    // bf16: P of the tile whose P V comes next, made as soon as that tile's
    // scores are known (one step ahead of its P V), so that the scores live
    // only within a step and the exp2 work runs beside the P V MFMAs.
    bf16x8_t pc[2][2];   // [key block][16-key half]
    // P = 2^((s - m_ref) c) into pc; returns this lane's row sum of P.
    auto make_p = [&](const f32x16_t (&s)[2]) __attribute__((always_inline)) -> float {
      float psum = 0.0f;
      if constexpr (BF16) {
        const float mc = m_ref == -INFINITY ? 0.0f : m_ref * c;
        const uint32_t ones = 0x3f803f80u;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int mm = 0; mm < 2; ++mm) {
            bf16x8_t pb;
#pragma unroll
            for (int j = 0; j < 8; ++j)   // masked: exp2(-inf) = 0
              pb[j] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[kb][8 * mm + j], c, -mc));
            const auto w = __builtin_bit_cast(uint4, pb);
            psum = dot2_bf16(w.x, ones, psum);
            psum = dot2_bf16(w.y, ones, psum);
            psum = dot2_bf16(w.z, ones, psum);
            psum = dot2_bf16(w.w, ones, psum);
            pc[kb][mm] = pb;
          }
      }
      return psum;
    };
    // O^T += V^T P^T with the P in pc.
    auto pv = [&](const char* sV) __attribute__((always_inline)) {
      if constexpr (BF16) {
        const int g16 = lane / 16, i16 = lane % 16;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int mm = 0; mm < 2; ++mm) {
            const int lo_row = kb * 32 + 16 * mm + 4 * hf + i16 / 4;
            const int hi_row = lo_row + 8;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const int chunk = 4 * db + 2 * (g16 % 2) + (i16 % 4) / 2;
              const bf16x4_t lo = ds_read_tr16(sV + row_off(lo_row) + chunk * 16 + 8 * (i16 % 2));
              const bf16x4_t hi = ds_read_tr16(sV + row_off(hi_row) + chunk * 16 + 8 * (i16 % 2));
              const bf16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
              oacc[db] = M::mma(a, pc[kb][mm], oacc[db]);
            }
          }
      }
    };
    // bf16 scores of tile t + 1 -> pc, while the P V of tile t (pv, issued
    // before) runs: P is made with the current reference max, which moves
    // rarely, and made again if the tile's max moved it.
    // The row max is needed only when a P could exceed 2^kLazy: every P is at
    // most its lane's row sum, so a sum below 2^(kLazy - 1) (a factor of two
    // covers the bf16 rounding of P and the exp2 error) rules a move of the
    // reference max out, and the max is then skipped. Where the max is
    // taken, the decision is the same as always; the results do not change.
    auto next_p = [&](const f32x16_t (&s)[2]) __attribute__((always_inline)) {
      float psum = make_p(s);
      // P stays here, ahead of the rare branch (else the compiler moves it
      // into both paths, after every MFMA of the step).
      asm volatile("" : "+v"(psum), "+v"(pc[0][0]), "+v"(pc[0][1]), "+v"(pc[1][0]),
                   "+v"(pc[1][1]));
      if (__builtin_amdgcn_ballot_w64(!(psum < kNoMaxSum && m_ref > -INFINITY)) != 0) {
        if (rescale_if_grown(row_max(s))) psum = make_p(s);
      }
      l_run += psum;
    };

    // ---- prologue: K0, V0 and K1 in LDS; S of tile 0.
    issue(kg, 0, ring(0, 0));
    issue(vg, 0, ring(1, 0));
    if (n_kt > 1) {
      poisoned = !cover(1, 1);
      if (!poisoned) issue(kg, 1, ring(0, 1));
    }
    wait_vmcnt<0>();
    __syncthreads();
    f32x16_t sc[2];   // scores of the tile being finished
    if (!poisoned && n_w > 0) {
      qk(ring(0, 0), sc);
      if (kt_open == 0) mask(0, sc);
      update_max(sc);
      if constexpr (BF16) l_run += make_p(sc);
    }
    __syncthreads();   // K slot 0 is refilled in the first step

    // One step t: copies of K(t+2) and V(t+1) into the slots that K(t) and
    // V(t-1) left; S(t+1) = K(t+1) Q^T on MFMA while the VALU turns S(t)
    // into P(t); O += V(t)^T P(t)^T; row max of S(t+1). The copies land
    // before the step's closing barrier.
    auto step = [&](int t, auto steady) -> bool {
      constexpr bool kSteady = decltype(steady)::value;
      const bool more1 = kSteady || t + 1 < n_kt;
      const bool more2 = t + 2 < n_kt;
      if (more1) {
        if (!cover(t + 1, more2 ? t + 2 : t + 1)) return false;
        if (more2) issue(kg, t + 2, ring(0, t & 1));
        issue(vg, t + 1, ring(1, (t + 1) & 1));
      }
      const char* sKn = ring(0, (t + 1) & 1);
      const char* sV = ring(1, t & 1);
      if constexpr (BF16) {
        if (kSteady || t + 1 < n_w) {
          f32x16_t sn[2];
          qk(sKn, sn);
          pv(sV);
          if (!kSteady) mask((t + 1) * kBlockN, sn);
          next_p(sn);
        } else if (t < n_w) {
          pv(sV);
        }
      } else if constexpr (kSteady) {
        f32x16_t sn[2];
        qk(sKn, sn);
        exp_pv(sc, sV);
        update_max(sn);
        sc[0] = sn[0];
        sc[1] = sn[1];
      } else {
        if (t + 1 < n_w) {
          f32x16_t sn[2];
          qk(sKn, sn);
          exp_pv(sc, sV);
          mask((t + 1) * kBlockN, sn);
          update_max(sn);
          sc[0] = sn[0];
          sc[1] = sn[1];
        } else if (t < n_w) {
          exp_pv(sc, sV);
        }
      }
      wait_vmcnt<0>();
      __syncthreads();
      return true;
    };

    // Steps whose next tile is computed by this wave without the mask take a
    // loop of their own (no mask code, no per-step conditions on the compute
    // side); the rest take the general loop. Every step has the same barriers
    // whichever loop runs it, so the switch point may differ between waves.
    int t = 0;
    if (!poisoned) {
      for (; t + 1 < kt_open && !poisoned; ++t) poisoned = !step(t, std::true_type{});
      for (; t < n_kt && !poisoned; ++t) poisoned = !step(t, std::false_type{});
    }

    if (!poisoned) {
      // ---- epilogue: l = both halves' shares; O^T / l -> o[b, row, h, :].
      // The tile goes through LDS so that each row leaves as whole 16-byte
      // chunks, full lines that non-temporal stores write straight to memory.
      const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run),
                                                        __float_as_uint(l_run), false, false);
      const float l_tot = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
      const float inv = 1.0f / l_tot;
      constexpr int ORP = 64 / CPR;            // rows one wave stores per pass
      static_assert(kBlockM * OROW <= LDSB, "output tile fits in the LDS block");
      static_assert(32 % ORP == 0, "a wave's 32 rows split into whole passes");
      // Every step ends on a workgroup barrier, so no wave still reads the
      // rings here and they can take the output tile.
      char* s_out = &s_lds[0] + wave * 32 * OROW;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + 8 * g4 + 4 * hf;
          if (d < D) {
            char* dst = s_out + lr * OROW + d * ESZ;
            if constexpr (BF16) {
              *(bf16x4_t*)dst = bf16x4_t{(__bf16)(oacc[db][4 * g4 + 0] * inv), (__bf16)(oacc[db][4 * g4 + 1] * inv),
                                         (__bf16)(oacc[db][4 * g4 + 2] * inv), (__bf16)(oacc[db][4 * g4 + 3] * inv)};
            } else {
              *(f32x4_t*)dst = f32x4_t{oacc[db][4 * g4 + 0] * inv, oacc[db][4 * g4 + 1] * inv,
                                       oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv};
            }
          }
        }
      // A wave reads back only its own rows, after its own LDS writes (LDS
      // operations of one wave complete in order).
      const int row0 = q0 + wave * 32;       // the wave's first query row (uniform)
      char* og = (char*)p.o + (((q_row0 + row0) * p.n_heads + h) * D) * ESZ;
      const uint32_t ostride = (uint32_t)(p.n_heads * ROWB);   // bytes between query rows
      const int rr0 = lane / CPR, cc = lane % CPR;
#pragma unroll
      for (int r0 = 0; r0 < 32; r0 += ORP) {
        const int rr = r0 + rr0;
        if (row0 + rr < seq_q) {
          const u32x4_t v = *(const u32x4_t*)(s_out + rr * OROW + cc * 16);
          store_nt((u32x4_t*)(og + (uint32_t)rr * ostride + cc * 16), v);
        }
      }
      return;
    }
  }

  // A needed block lies outside the pool: NaN rows for this (sequence, head).
  for (int idx = tid; idx < kBlockM * D; idx += kThreads) {
    const int i = q0 + idx / D;
    if (i < seq_q) {
      const int64_t o = ((q_row0 + i) * p.n_heads + h) * D + idx % D;
      ((T*)p.o)[o] = (T)__builtin_nanf("");
    }
  }
}

template <bool BF16, int D, bool PAGED>
int launch_t(const PrefillParams& p, hipStream_t stream) {
  const int grid = p.q_tiles * p.batch * p.n_heads;
  if (p.cu_q != nullptr) {
    hipLaunchKernelGGL((prefill_kernel<BF16, D, PAGED, true>), dim3(grid), dim3(kThreads), 0,
                       stream, p);
  } else {
    hipLaunchKernelGGL((prefill_kernel<BF16, D, PAGED, false>), dim3(grid), dim3(kThreads), 0,
                       stream, p);
  }
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

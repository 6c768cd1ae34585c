// Absorbed multi-head latent attention decode (frink-models 0.31.0
// src/mla/mod.rs, absorbed_attention and the MlaKvB doc): every head h
// attends over the sequence's cached latent rows [c | k_rot] (width R + P)
// with its absorbed query q_abs[h]; the value is each row's first R entries.
// It is multi-query attention with one shared KV head, so a latent tile is
// staged once per workgroup and serves all of its heads.
//
// One workgroup = 128 heads of one sequence over a range of its context,
// one wave per 32 heads (a smaller head count leaves the heads past the last
// one idle: they compute on a copy of its query and are not stored). A
// latent byte read from LDS by a wave feeds its 32 heads (S^T = L Q^T on
// 32x32x16 MFMAs, Q^T in 144 VGPRs); O^T += V^T P^T is split by value dims
// (each wave owns all 128 heads x 128 of the dims, the 256 AGPRs), so one
// wave per SIMD. The context of a sequence is split over workgroups to fill
// the chip; mla_combine merges the pieces.
//
// 32-token latent tiles (36 KB) are copied global -> LDS by the DMA path
// (global_load_lds_dwordx4) three tiles ahead into a four-stage ring. Rows
// are 1152 bytes with the 16-byte chunks XOR-swizzled by 2*(r%4) + (r/4)%2
// inside each group of 8: a DMA op fills 1 KB of the tile with any
// lane-to-chunk map, and both operand reads stay free of bank conflicts.
//
// Per step a wave hands P of tile i to the others, then runs the 36 MFMAs of
// S^T for tile i + 1 interleaved with the first 24 of the 32 of
// O^T += V^T P^T for tile i, and the last 8 with the softmax of tile i + 1
// between them (so that its VALU work runs beside MFMAs). In the
// accumulator layout lane l owns head l % 32 and 16 of the tile's tokens
// (the other 16 in lane l ^ 32): the max needs one v_permlane32_swap, the
// sum stays per lane until the end; P goes
// from the accumulator registers straight to the B operand, and the V^T
// operand comes from the row-major tile through ds_read_b64_tr_b16. The
// running max moves only when a head's max grows by more than 2^8 in the
// exp2 domain (then O and l are rescaled), and the tile max is taken only
// when a row sum of P shows that it could have.
#include "common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace pkva {

namespace {

constexpr int kHW = 32;           // heads per wave
constexpr int kMaxWaves = 4;      // waves (head groups of 32) per workgroup
constexpr int kTile = 32;         // tokens per tile
constexpr int kStages = 4;
constexpr int kPrefetch = 3;      // tiles in flight ahead of the one consumed
constexpr int kR = 512;           // kv_lora_rank
constexpr int kP = 64;            // qk_rope_head_dim
constexpr int kW = kR + kP;       // latent row width
constexpr int kRowB = kW * 2;     // 1152 bytes
constexpr int kChunks = kW / 8;   // 16-byte chunks per row (72)
constexpr int kTileB = kTile * kRowB;
constexpr int kDmaTile = kTileB / 1024;   // 1 KB DMA ops per tile (36)
constexpr int kKSteps = kW / 16;  // 16-deep MFMA steps of the scores (36)
constexpr int kDB = kR / 32;      // 32-row blocks of O^T (16)
constexpr float kLazy = 8.0f;
constexpr float kNoMaxSum = 128.0f;   // 2^(kLazy - 1)
constexpr int kXcds = 8;          // accelerator complex dies, each with its own L2
constexpr int kAhead = 4;        // MFMA pairs whose operands are read ahead
constexpr int kBtWin = 512;       // block ids of a paged latent held in LDS
static_assert(kTileB % 1024 == 0 && kChunks % 8 == 0, "tile geometry");
static_assert(kKSteps >= 2 * kDB, "value MFMAs interleave with the score MFMAs");

__device__ __forceinline__ f32x16_t mma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The score MFMAs, written so their accumulator lives in VGPRs: the 256 AGPRs
// hold O^T, and with the compiler's choice (AGPR accumulators for every MFMA
// of the kernel) the scores would displace O^T blocks every tile. Dependent
// MFMAs on one accumulator need no wait states; a VALU read of the result
// does (see score_wait).
__device__ __forceinline__ f32x16_t mma_v_first(bf16x8_t a, bf16x8_t b) {
  f32x16_t d;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ void mma_v(f32x16_t& d, bf16x8_t a, bf16x8_t b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// Wait states between the last score MFMA (8 passes) and a VALU access of its
// accumulator, which the compiler cannot see through the inline assembly.
__device__ __forceinline__ void score_wait() { asm volatile("s_nop 15\n\ts_nop 7" ::: "memory"); }

// Transposed LDS read: four consecutive rows of one 16-bit column per lane.
__device__ __forceinline__ bf16x4_t ds_read_tr16(const char* p) {
  typedef __attribute__((ext_vector_type(4))) short s16x4;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(__attribute__((address_space(3))) const char*)(p));
  return __builtin_bit_cast(bf16x4_t, v);
}

// Tile image in LDS: nine 4 KB column blocks; block c8 holds chunks
// 8 c8 .. 8 c8 + 7 (128 bytes) of all 32 rows, and chunk c of row r sits at
// 4096 (c / 8) + 128 r + 16 ((c % 8) ^ swz(r)). Rows r and r + 2 start on the
// same banks (of the 64 4-byte banks, 256 bytes, the LDS serves per clock):
// the eight rows of one parity among 16 consecutive ones take the eight XOR
// values, so a K-fragment read (16 lanes = 16 rows, one chunk) hits 16
// distinct 16-byte bank groups, and rows 4k and 4k + 2 differ in bit 2,
// which keeps the four-chunk groups of a V^T read apart.
__device__ __forceinline__ int swz(int r) {
  const int m = (r >> 1) & 7;
  return 4 * (m & 1) + (m >> 1);
}

// acc *= alpha with acc kept in accumulation registers (read, scale and write
// back in place; plain VALU arithmetic on them makes the compiler move all of
// them through VGPRs on every loop trip). The s_nops cover the MFMA-write to
// v_accvgpr_read and v_accvgpr_write to MFMA wait states.
// Tile t of a wave's O^T covers head block t % HB; alpha[t % HB] is this
// lane's factor for it.
template <int HB>
__device__ __forceinline__ void scale_acc(f32x16_t (&acc)[kDB], const float (&alpha)[HB]) {
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float x = acc[db][i], t;
      asm volatile(
          "v_accvgpr_read_b32 %1, %0\n\t"
          "v_mul_f32 %1, %1, %2\n\t"
          "v_accvgpr_write_b32 %0, %1"
          : "+a"(x), "=&v"(t)
          : "v"(alpha[db % HB]));
      acc[db][i] = x;
    }
  asm volatile("s_nop 7" ::: "memory");
}

// PAGED: the latent rows live in a pool [num_blocks, block_size, R + P];
// token t of sequence b is row t % block_size of block
// block_table[b][t / block_size]. The block ids a piece needs are checked
// up front and held in an LDS window (reloaded, between barriers, when a
// tile's blocks run past it); every copy then takes its row's address.
template <int NW, bool PAGED>
__global__ __launch_bounds__(64 * NW, 1) void mla_kernel(MlaParams p) {
  static_assert(NW == kMaxWaves, "built for four waves of 32 heads");
  static_assert(kDmaTile % NW == 0, "every thread copies the same number of chunks");
  constexpr int kDmaPerThread = kDmaTile / NW;
  // O^T += V^T P^T is split by value dims: a wave owns the O^T tiles of
  // kPvHB head blocks x kPvDB dim blocks (all heads of the workgroup x
  // 512 / NW dims), so each V^T byte is read from LDS by one wave; P^T goes
  // through LDS.
  constexpr int kPvHB = NW;
  constexpr int kPvDB = kDB / kPvHB;
  __shared__ __attribute__((aligned(1024))) char s_lat[kStages * kTileB];
  __shared__ __attribute__((aligned(16))) char s_p[NW * kHW * 64];   // P^T rows, 64 B per head
  __shared__ float s_alpha[NW * kHW];                               // rescale factors
  __shared__ float s_l[NW * kHW];                                   // softmax sums at the end
  __shared__ __attribute__((aligned(16))) int s_flag[4];
  __shared__ int s_bt[PAGED ? kBtWin : 1];
  __shared__ int s_bad;

  // Work item = (sequence, head group, split), split fastest. Workgroups go
  // to the 8 XCDs round robin (XCD = id % 8); a run of consecutive items
  // per XCD keeps the pieces of one sequence on one L2, which then reads the
  // sequence's queries from memory once.
  const int n_hg = (p.n_heads + kHW * NW - 1) / (kHW * NW);
  int item = blockIdx.x;
  if (gridDim.x % kXcds == 0) item = (blockIdx.x % kXcds) * (gridDim.x / kXcds) + blockIdx.x / kXcds;
  const int split = item % p.nsplit;
  const int hg = (item / p.nsplit) % n_hg;
  const int b = item / (p.nsplit * n_hg);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int lr = lane % 32, hf = lane / 32;
  const int head = (hg * NW + wave) * kHW + lr;

  const int L = p.seq_lens[b];
  bool bad = L < 1 || L > p.max_seq_len;
  const int t_begin = split * p.split_tokens;
  int t_end = bad ? 0 : min(L, t_begin + p.split_tokens);
  const char* lat = (const char*)p.latent + (PAGED ? 0 : (int64_t)b * p.kv_capacity * kRowB);

  // Paged: check every block id the piece needs, then fill the window.
  const int shift = p.block_shift;
  const int32_t* bt_row = PAGED ? p.block_table + (int64_t)b * p.max_blocks_per_seq : nullptr;
  int win0 = 0, win_end = 0;   // block ids [win0, win_end) of the sequence held in s_bt
  auto load_window = [&](int blk) __attribute__((always_inline)) {
    __syncthreads();   // no wave still reads the old window
    win0 = blk;
    win_end = min(blk + kBtWin, ((t_end - 1) >> shift) + 1);
    for (int i = tid; i < win_end - win0; i += 64 * NW) s_bt[i] = bt_row[win0 + i];
    __syncthreads();
  };
  if constexpr (PAGED) {
    if (t_end > t_begin) {
      if (tid == 0) s_bad = 0;
      __syncthreads();
      for (int i = (t_begin >> shift) + tid; i <= ((t_end - 1) >> shift); i += 64 * NW) {
        const int id = bt_row[i];
        if (id < 0 || id >= p.num_blocks) s_bad = 1;
      }
      __syncthreads();
      if (s_bad) {   // a needed block lies outside the pool: NaN for the sequence
        bad = true;
        t_end = 0;
      } else {
        load_window(t_begin >> shift);
      }
    }
  }
  const int n_t = t_end > t_begin ? (t_end - t_begin + kTile - 1) / kTile : 0;

  // Copy tile i (tokens t_begin + 32 i ..) into its stage. DMA op J of a
  // tile (1 KB, LDS bytes [1024 J, +1024)) covers column block J / 4, rows
  // 8 u .. 8 u + 7 with u = J % 4: lane l brings row 8 u + l / 8, chunk
  // 8 (J / 4) + ((l % 8) ^ swz(row)), which lies at byte
  // dlane[u % 2] + 8 u kRowB + 128 (J / 4) of the tile's rows (swz has period
  // 16, so the lane part depends on u % 2 only). This wave issues ops
  // J = wave + NW j. Rows past t_end copy row t_end - 1 instead (their
  // scores are masked; a NaN beyond the context must not reach P * V), so
  // every thread issues the same number of copies per tile and the counted
  // waits hold.
  const int drow = lane / 8;
  uint32_t dlane[2];
#pragma unroll
  for (int u2 = 0; u2 < 2; ++u2)
    dlane[u2] = (uint32_t)(drow * kRowB + 16 * ((lane % 8) ^ swz(8 * u2 + drow)));
  // issue_prep(i) runs on every wave at the same point (a paged window reload
  // takes barriers); issue_op(i, j) then issues DMA op j of tile i, so the
  // ops of a tile can be spread between the MFMAs of a step.
  auto issue_prep = [&](int i) __attribute__((always_inline)) {
    if constexpr (PAGED) {
      const int t0 = t_begin + kTile * i;
      const int last = min(t_end - 1 - t0, kTile - 1);   // last live row of the tile
      if (((t0 + last) >> shift) >= win_end) load_window(t0 >> shift);   // uniform
    }
  };
  // MODE 1: a whole contiguous tile (one lane offset, the rest uniform);
  // MODE 2: the last, partial tile of a contiguous range, or a paged tile.
  auto issue_op = [&](int i, int j, auto mode) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode)::value;
    const int J = wave + NW * j, u = J % 4, c8 = J / 4;
    const uint32_t st = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(s_lat) +
                        (uint32_t)((i % kStages) * kTileB) + 1024u * J;
    const int t0 = t_begin + kTile * i;
    if constexpr (PAGED) {
      const int last = min(t_end - 1 - t0, kTile - 1);
      const int bs_mask = (1 << shift) - 1;
      const int t = t0 + min(8 * u + drow, last);
      const uint32_t prow = (uint32_t)((s_bt[(t >> shift) - win0] << shift) + (t & bs_mask));
      dma16_addr(lat + (uint64_t)prow * kRowB + (dlane[u & 1] - drow * kRowB) + 128 * c8, st);
      return;
    }
    if constexpr (MODE == 1) {
      dma16(lat + (int64_t)(t0 + 8 * u) * kRowB + 128 * c8, dlane[u & 1], st);
    } else {
      // The lane's row is clamped to the last live one; the offset (which
      // the instruction takes as unsigned) stays relative to the tile start.
      const int last = min(t_end - 1 - t0, kTile - 1);   // last live row of the tile
      const int row = 8 * u + drow;
      dma16(lat + (int64_t)t0 * kRowB + 128 * c8,
            dlane[u & 1] + (uint32_t)((8 * u - (row - min(row, last))) * kRowB), st);
    }
  };
  auto issue = [&](int i) __attribute__((always_inline)) {
    issue_prep(i);
#pragma unroll
    for (int j = 0; j < kDmaPerThread; ++j) issue_op(i, j, std::integral_constant<int, 2>{});
  };
  // publish(i) runs when the tiles up to min(i + kPrefetch - 2, n_t - 1) are
  // issued: wait until at most the later tiles' copies are in flight (vmcnt
  // counts in issue order), then the barrier publishes tile i to every wave.
  // The same barrier retires every read of the stage the next copy reuses:
  // a wave reads tile j's stage in steps j - 1 (its keys) and j (its
  // values), and the copy of tile j + 4 into that stage is issued only after
  // publish(j + 2), which no wave passes before it has finished step j.
  auto publish = [&](int i) __attribute__((always_inline)) {
    const int later = max(0, min(i + kPrefetch - 2, n_t - 1) - i);
    static_assert(kPrefetch - 2 <= 1, "extend the wait cases");
    // (vmcnt holds at most 63: waiting for fewer in flight is also correct.)
    constexpr int kOne = kDmaPerThread < 63 ? kDmaPerThread : 63;
    if (later == 0) {
      wait_vmcnt<0>();
    } else {
      wait_vmcnt<kOne>();
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Per-lane LDS offsets inside a tile (the rest is an immediate):
  //   K fragment of S^T (A operand): row lr, chunk 2 kk + hf, in column block
  //   kk / 4: one base per kk % 4;
  //   V^T fragment: lane (g16, i16) reads row 16 mm + 4 hf + i16 / 4 (+8 for
  //   the upper half), chunk 4 db + 2 (g16 % 2) + (i16 % 4) / 2, half
  //   i16 % 2, in column block db / 2: one base per (db parity, half).
  const int g16 = lane / 16, i16 = lane % 16;
  int k_base[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) k_base[j] = 128 * lr + 16 * ((2 * j + hf) ^ swz(lr));
  int v_base[2][2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 4 * hf + i16 / 4 + 8 * h;
      const int cl = 2 * (g16 % 2) + (i16 % 4) / 2;
      v_base[par][h] = 128 * r + 16 * ((4 * par + cl) ^ swz(r)) + 8 * (i16 % 2);
    }

  bf16x8_t qB[kKSteps];   // Q^T as the B operand: head lr, dims 16*kk + 8*hf .. +7
  f32x16_t oacc[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) oacc[db] = f32x16_t{};
  float m_ref = -INFINITY, l_run = 0.0f;
  const float c = p.scale_log2;
  bf16x8_t pb[2];   // P of this wave's heads for the latest softmax, [k-step]

  // Operand reads run kAhead MFMAs ahead through register rings; the
  // scheduling barriers keep the compiler from hoisting all of them (which
  // would not fit in registers).
  auto read_k = [&](const char* sk, int kk) __attribute__((always_inline)) {
    return *(const bf16x8_t*)(sk + k_base[kk % 4] + 4096 * (kk / 4));
  };
  auto read_v = [&](const char* sv, int mm, int db) __attribute__((always_inline)) {
    const char* vb = sv + 4096 * (db / 2) + 2048 * mm;
    const bf16x4_t lo = ds_read_tr16(vb + v_base[db & 1][0]);
    const bf16x4_t hi = ds_read_tr16(vb + v_base[db & 1][1]);
    return bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  // P^T fragment of head block hb, k-step ks: lane (lr, hf) reads the
  // 16 bytes lane (lr, hf) of the owning wave wrote as its pb[ks]. Rows are
  // 64 bytes with the chunk XOR-swizzled by (lr / 4) % 4: the 16 lanes of a
  // read or write then cover 16 distinct 16-byte bank groups.
  auto p_addr = [&](int ks, int hb) __attribute__((always_inline)) {
    return s_p + (hb * kHW + lr) * 64 + 16 * ((2 * ks + hf) ^ ((lr >> 2) & 3));
  };
  auto read_p = [&](int ks, int hb) __attribute__((always_inline)) {
    return *(const bf16x8_t*)p_addr(ks, hb);
  };
  auto head_block = [&](int hbi) __attribute__((always_inline)) { return hbi; };
  auto dim_block = [&](int dbi) __attribute__((always_inline)) { return kPvDB * wave + dbi; };
  // The 32 value MFMAs in the order idx = 16 ks + kPvHB dbi + hbi: V^T
  // group G = idx / kPvHB (k-step G / kPvDB, dim block G % kPvDB) serves
  // kPvHB MFMAs in a row; the P^T fragments of a k-step stay in registers.
  // V^T groups are read kAhead MFMAs ahead through a ring; the P^T
  // fragments of k-step 1 replace those of k-step 0 right after their last
  // use (three MFMAs ahead).
  constexpr int kV0 = (kAhead + kPvHB - 1) / kPvHB;   // V^T groups read before the loop
  constexpr int kVS = kV0 + 1;                        // V^T ring slots
  constexpr int kPS = kPvHB;                          // P^T slots
  auto v_group = [&](const char* sv, int G) __attribute__((always_inline)) {
    return read_v(sv, G / kPvDB, dim_block(G % kPvDB));
  };
  // When dma_tile >= 0, the copies of that tile are issued one every
  // kDmaStride MFMA steps: an op that has to wait for room in the memory
  // queues then stalls a wave for part of an MFMA's latency, not all at once.
  constexpr int kDmaStride = kKSteps / kDmaPerThread;
  static_assert(kKSteps % kDmaPerThread == 0, "DMA ops spread evenly over the score steps");
  // S^T of the tile in stage `stage` alone (36 dependent MFMAs): the first
  // tile of a range.
  auto scores = [&](f32x16_t& s, int stage) __attribute__((always_inline)) {
    const char* sk = s_lat + stage * kTileB;
    bf16x8_t kr[kAhead + 1];
#pragma unroll
    for (int j = 0; j < kAhead; ++j) kr[j] = read_k(sk, j);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) {
      if (kk + kAhead < kKSteps) kr[(kk + kAhead) % (kAhead + 1)] = read_k(sk, kk + kAhead);
      if (kk == 0) {
        s = mma_v_first(kr[0], qB[0]);
      } else {
        mma_v(s, kr[kk % (kAhead + 1)], qB[kk]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // O^T += V^T P^T alone (the last tile of the range).
  auto values = [&](int pv_stage) __attribute__((always_inline)) {
    const char* sv = s_lat + pv_stage * kTileB;
    bf16x8_t vr[kVS], pr[kPS];
#pragma unroll
    for (int G = 0; G < kV0; ++G) vr[G % kVS] = v_group(sv, G);
#pragma unroll
    for (int j = 0; j < kPS; ++j) pr[j] = read_p(j / kPvHB, head_block(j % kPvHB));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int idx = 0; idx < 2 * kDB; ++idx) {
      if ((idx + kAhead) % kPvHB == 0) {
        const int G = (idx + kAhead) / kPvHB;
        if (G >= kV0 && G < 2 * kPvDB) vr[G % kVS] = v_group(sv, G);
      }
      const int hbi = idx % kPvHB, t = (idx % 16 / kPvHB) * kPvHB + hbi;
      oacc[t] = mma(vr[(idx / kPvHB) % kVS], pr[hbi], oacc[t]);
      if (idx >= 16 - kPvHB && idx < 16) pr[hbi] = read_p(1, head_block(hbi));
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Softmax of tile i (scores in s): mask tokens past t_end, lazy max,
  // P in bf16 (pb) and the row sum of the same rounded values. Accumulator
  // register r holds token 32 i + 8*(r/4) + 4*hf + r%4 of the range.
  const uint32_t ones = 0x3f803f80u;
  bool resc = false;        // this wave's heads need O^T rescaled (wave-uniform)
  float alpha_own = 1.0f;   // the factor of head lr when resc
  // The softmax of a tile in three parts, so that the pairs can run between
  // the value MFMAs of the step that computed the tile's scores:
  // sm_begin masks tokens past t_end; sm_pair(k) makes P of the lane's
  // scores 2k and 2k + 1 with the current reference max (bf16, into pb) and
  // adds them to the row sum; sm_end takes the max only when a P could
  // exceed 2^kLazy (every P is at most its lane's row sum, so a sum below
  // 2^(kLazy - 1) rules a move out; a factor of two covers the bf16
  // rounding of P and the exp2 error), moves the reference max when it grew
  // by more than that, and then makes P again.
  float sm_mc = 0.0f, sm_ps = 0.0f;
  auto sm_begin = [&](f32x16_t& s, int i) __attribute__((always_inline)) {
    score_wait();
    const int t0 = t_begin + kTile * i;
    if (t0 + kTile > t_end) {
      const int lim = t_end - 1 - (t0 + 4 * hf);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r / 4) + (r % 4) > lim) s[r] = -INFINITY;
    }
    sm_mc = m_ref * c;
    sm_ps = 0.0f;
    resc = false;
  };
  auto sm_pair = [&](const f32x16_t& s, int k) __attribute__((always_inline)) {
    const int mm = k / 4, j = 2 * (k % 4);
    const bf16x2_t two = {(__bf16)__builtin_amdgcn_exp2f(fmaf(s[8 * mm + j], c, -sm_mc)),
                          (__bf16)__builtin_amdgcn_exp2f(fmaf(s[8 * mm + j + 1], c, -sm_mc))};
    pb[mm][j] = two[0];
    pb[mm][j + 1] = two[1];
    sm_ps = dot2_bf16(__builtin_bit_cast(uint32_t, two), ones, sm_ps);
  };
  auto sm_end = [&](f32x16_t& s) __attribute__((always_inline)) {
    float ps = sm_ps;
    asm volatile("" : "+v"(ps), "+v"(pb[0]), "+v"(pb[1]));
    if (__builtin_amdgcn_ballot_w64(!(ps < kNoMaxSum && m_ref > -INFINITY)) != 0) {
      float m = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; r += 2)
        m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m, s[r]), s[r + 1]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m),
                                                       false, false);
      m = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      // Token t0 is live for every head, so m is finite. A rescale of O^T
      // is recorded here and applied by every wave to its tiles of these
      // heads once the factors are published (see rescale).
      if (__builtin_amdgcn_ballot_w64((m - m_ref) * c > kLazy) != 0) {
        const float m_new = fmaxf(m_ref, m);
        alpha_own = m_ref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((m_ref - m_new) * c);
        m_ref = m_new;
        l_run *= alpha_own;
        resc = true;
        sm_mc = m_ref * c;
        sm_ps = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) sm_pair(s, k);
        ps = sm_ps;
      }
    }
    l_run += ps;
  };
  auto softmax = [&](f32x16_t& s, int i) __attribute__((always_inline)) {
    sm_begin(s, i);
#pragma unroll
    for (int k = 0; k < 8; ++k) sm_pair(s, k);
    sm_end(s);
  };

  // One value MFMA (index idx of 32) with its V^T read-ahead and P^T reload.
  auto value_step = [&](const char* sv, bf16x8_t (&vr)[kVS], bf16x8_t (&pr)[kPS], int idx)
      __attribute__((always_inline)) {
    if ((idx + kAhead) % kPvHB == 0) {
      const int G = (idx + kAhead) / kPvHB;
      if (G >= kV0 && G < 2 * kPvDB) vr[G % kVS] = v_group(sv, G);
    }
    const int hbi = idx % kPvHB, t = (idx % 16 / kPvHB) * kPvHB + hbi;
    oacc[t] = mma(vr[(idx / kPvHB) % kVS], pr[hbi], oacc[t]);
    if (idx >= 16 - kPvHB && idx < 16) pr[hbi] = read_p(1, head_block(hbi));
  };
  // A steady step's MFMAs: the 36 score MFMAs of the next tile with the
  // first 32 - kTail value MFMAs of this one between them, then the last
  // kTail value MFMAs with the next tile's softmax between them (its VALU
  // work then runs beside MFMAs instead of after them).
  constexpr int kTail = 8;   // one softmax pair per value MFMA (16 measured slightly slower)
  static_assert(kTail % 8 == 0 && kTail <= 2 * kDB, "softmax pairs spread evenly");
  // After the publish barrier: scale this wave's O^T tiles of every head
  // whose owner recorded a rescale. Before the first values O^T is zero.
  auto rescale_with = [&](const int4 fl, int i) __attribute__((always_inline)) {
    const int any = fl.x | fl.y | fl.z | fl.w;
    if (__builtin_expect(any != 0, 0) && i > 0) {
      float a[kPvHB];
#pragma unroll
      for (int hbi = 0; hbi < kPvHB; ++hbi) {
        const int hb = head_block(hbi);
        a[hbi] = s_flag[hb] ? s_alpha[hb * kHW + lr] : 1.0f;
      }
      scale_acc(oacc, a);
    }
  };
  auto rescale = [&](int i) __attribute__((always_inline)) {
    rescale_with(*(const int4*)s_flag, i);
  };

  // The value MFMAs start after kShift score MFMAs, so that the rescale
  // flags (read from LDS at the section's start) have arrived when a
  // pending rescale must be applied, before the first of them.
  constexpr int kShift = 4;
  auto section = [&](f32x16_t& s, int stage, int pv_stage, int dma_tile, auto dma_mode,
                     int sm_tile) __attribute__((always_inline)) {
    constexpr int DMA = decltype(dma_mode)::value;   // 0: no copies, else issue_op's MODE
    const char* sk = s_lat + stage * kTileB;
    const char* sv = s_lat + pv_stage * kTileB;
    bf16x8_t kr[kAhead + 1], vr[kVS], pr[kPS];
#pragma unroll
    for (int j = 0; j < kAhead; ++j) kr[j] = read_k(sk, j);
#pragma unroll
    for (int G = 0; G < kV0; ++G) vr[G % kVS] = v_group(sv, G);
#pragma unroll
    for (int j = 0; j < kPS; ++j) pr[j] = read_p(j / kPvHB, head_block(j % kPvHB));
    const int4 fl = *(const int4*)s_flag;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) {
      if (kk + kAhead < kKSteps) kr[(kk + kAhead) % (kAhead + 1)] = read_k(sk, kk + kAhead);
      if (kk == 0) {
        s = mma_v_first(kr[0], qB[0]);
      } else {
        mma_v(s, kr[kk % (kAhead + 1)], qB[kk]);
      }
      if (kk == kShift) {
        // The tile's rescale (if any): its flags were read while the first
        // score MFMAs issued.
        rescale_with(fl, sm_tile - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kk >= kShift && kk < 2 * kDB - kTail + kShift) value_step(sv, vr, pr, kk - kShift);
      if (DMA != 0 && kk % kDmaStride == 0) issue_op(dma_tile, kk / kDmaStride, dma_mode);
      __builtin_amdgcn_sched_barrier(0);
    }
    sm_begin(s, sm_tile);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int idx = 2 * kDB - kTail; idx < 2 * kDB; ++idx) {
      value_step(sv, vr, pr, idx);
      constexpr int kEvery = kTail / 8;
      if ((idx - (2 * kDB - kTail)) % kEvery == kEvery - 1) sm_pair(s, (idx - (2 * kDB - kTail)) / kEvery);
      __builtin_amdgcn_sched_barrier(0);
    }
    sm_end(s);
  };
  // Hand P (and a pending rescale) of this wave's heads to the others:
  // the barrier first, because every wave reads the buffer during the
  // previous step's values; the next barrier (publish) makes the writes
  // visible.
  auto exchange = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) *(bf16x8_t*)p_addr(mm, wave) = pb[mm];
    if (resc && hf == 0) s_alpha[wave * kHW + lr] = alpha_own;
    if (lane == 0) s_flag[wave] = resc ? 1 : 0;
  };
  if (n_t > 0) {
    // Prologue. Q^T first: each wave copies its 32 heads' rows (36 KB,
    // contiguous in q_abs) into its own stage of the ring with 1 KB DMA ops
    // in the tile layout, waits for its own copies and reads Q^T from there
    // with the K-fragment pattern (lane (lr, hf) gets row lr, chunk
    // 2 kk + hf: the B operand). Loading it straight into registers would
    // touch 32 rows with 32 bytes each per instruction. Then tiles 0 .. 2;
    // tile 0 published, its scores.
    // While Q^T is in flight, one dword of every 128-byte line of tiles
    // 0 .. 2 (of tile 0 for a paged latent) is loaded and dropped: the lines
    // are then in the caches when those tiles are copied after the barrier,
    // instead of every workgroup asking for its first tiles from memory at
    // the same moment. (Measured: with a paged latent, touching tile 0 alone
    // is ~2 us faster per call than three tiles; no difference otherwise.)
    constexpr int kPfTiles = PAGED ? 1 : kPrefetch;
    constexpr int kPfLines = kPfTiles * kTile * (kRowB / 128);
    constexpr int kPf = (kPfLines + 64 * NW - 1) / (64 * NW);   // loads per thread
    uint32_t touched = 0;
    {
      // Heads past the last one (a head count that leaves part of the
      // group idle) copy the last head's row: their results are computed
      // from real data and never stored.
      const int h0 = (hg * NW + wave) * kHW;   // this wave's first head
      const char* qb = (const char*)p.q + (int64_t)b * p.n_heads * kRowB;
      const uint32_t qst = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(s_lat) +
                           (uint32_t)(wave * kTileB);
#pragma unroll
      for (int J = 0; J < kDmaTile; ++J)
      {
        const int hq = min(h0 + 8 * (J % 4) + drow, p.n_heads - 1);
        dma16(qb + 128 * (J / 4), (uint32_t)(hq * kRowB) + (dlane[J % 2] - (uint32_t)(drow * kRowB)),
              qst + 1024u * J);
      }
      const int rows = min(t_end - t_begin, kPfTiles * kTile);
#pragma unroll
      for (int k = 0; k < kPf; ++k) {
        const int l = min(tid + 64 * NW * k, kPfLines - 1);
        const int t = t_begin + min(l / (kRowB / 128), rows - 1);
        const int col = l % (kRowB / 128);
        int64_t row;
        if constexpr (PAGED) {
          row = ((int64_t)s_bt[(t >> shift) - win0] << shift) + (t & ((1 << shift) - 1));
        } else {
          row = t;
        }
        touched ^= *(const uint32_t*)(lat + row * kRowB + 128 * col);
      }
      // Wait for everything: a counted wait would assume that the copies to
      // LDS and the loads to registers complete in issue order.
      wait_vmcnt<0>();
      asm volatile("" ::: "memory");
      const char* sq = s_lat + wave * kTileB;
#pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) qB[kk] = read_k(sq, kk);
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): Q^T is in registers
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();         // every wave is done with the ring
      asm volatile("" ::: "memory");
    }
    for (int i = 0; i < kPrefetch && i < n_t; ++i) issue(i);
    {   // publish tile 0 with the copies of tiles 1 .. min(2, n_t - 1) still in flight
      constexpr int kOne = kDmaPerThread < 63 ? kDmaPerThread : 63;
      constexpr int kTwo = 2 * kDmaPerThread < 63 ? 2 * kDmaPerThread : 63;
      static_assert(kPrefetch == 3, "the first wait counts two later tiles");
      if (n_t >= 3) {
        wait_vmcnt<kTwo>();
      } else if (n_t == 2) {
        wait_vmcnt<kOne>();
      } else {
        wait_vmcnt<0>();
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    if (p.nsplit < 0) s_bad = (int)touched;   // never true: keeps the touching loads
    // One score tile is enough: the softmax turns it into P (pb) before the
    // next tile's scores are computed into the same registers (in a step,
    // the next tile's softmax follows its score MFMAs).
    f32x16_t sc;
    scores(sc, 0);
    softmax(sc, 0);

    // Step i: P of tile i to the others; publish tile i + 1; scores of tile
    // i + 1 together with the values of tile i and then the softmax of tile
    // i + 1, with the copies of tile
    // i + kPrefetch spread between them (into the stage tile i - 1 left:
    // every wave is past step i - 1 once the barrier opens). The steps run
    // in three loops by what they copy (whole contiguous tiles, with one lane
    // offset per op; partial or paged tiles; nothing), and the last tile is
    // peeled off (no next tile): a branch between variants inside one loop
    // makes the compiler move O^T between register sets.
    static_assert(kPrefetch == kStages - 1, "the copy reuses the stage of tile i - 1");
    auto step = [&](int i, auto mode) __attribute__((always_inline)) {
      exchange();
      publish(i + 1);
      constexpr int MODE = decltype(mode)::value;
      if constexpr (MODE != 0) issue_prep(i + kPrefetch);
      section(sc, (i + 1) % kStages, i % kStages, MODE != 0 ? i + kPrefetch : -1, mode, i + 1);
    };
    const int n_whole = PAGED ? 0 : (t_end - t_begin) / kTile;   // tiles 0 .. n_whole-1 are whole
    int i = 0;
    for (; i + 1 < n_t && i + kPrefetch < n_whole; ++i) step(i, std::integral_constant<int, 1>{});
    for (; i + 1 < n_t && i + kPrefetch < n_t; ++i) step(i, std::integral_constant<int, 2>{});
    for (; i + 1 < n_t; ++i) step(i, std::integral_constant<int, 0>{});
    exchange();
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    rescale(n_t - 1);
    values((n_t - 1) % kStages);
  }

  // ---- epilogue: l = both halves' shares, published per head. The scaled
  // O^T tiles go through LDS (free once every wave is past its last tile)
  // so that every store writes one head's 1 KB row: row h of the workgroup
  // at byte h * kOutRow (padded: the 32 heads written at once spread over
  // the banks).
  const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run),
                                                    false, false);
  const float l_tot = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
  if (hf == 0) s_l[wave * kHW + lr] = l_tot;
  __bf16* dst;   // the workgroup's first row (head hg * 32 * NW)
  if (p.nsplit == 1) {
    dst = (__bf16*)p.o + ((int64_t)b * p.n_heads + hg * kHW * NW) * kR;
  } else {
    // Partial of this split: O / l in bf16 (half the traffic of the fp32
    // numerator, one more rounding of the size of the output's own), then
    // m in the log2 domain and l in fp32.
    // A piece with a block outside the pool leaves a NaN sum, which makes
    // the merged row NaN.
    const int64_t w = ((int64_t)b * p.nsplit + split) * p.n_heads + head;
    dst = p.ws_o + (((int64_t)b * p.nsplit + split) * p.n_heads + hg * kHW * NW) * kR;
    if (hf == 0 && head < p.n_heads) {
      store_nt(p.ws_ml + w * 2 + 0, n_t > 0 ? m_ref * c : -INFINITY);
      store_nt(p.ws_ml + w * 2 + 1, n_t > 0 ? l_tot : (bad ? __builtin_nanf("") : 0.0f));
    }
  }
  constexpr int kOutRow = kR * 2 + 8;
  static_assert(kHW * kMaxWaves * kOutRow <= kStages * kTileB, "output rows fit in the ring");
  __syncthreads();   // every wave is done with the latent tiles; every sum is published
  // Tile t covers head block head_block(t % kPvHB) and dim block
  // dim_block(t / kPvHB); register r holds dim 32 db + 8 (r/4) + 4 hf + r%4
  // of head lr of the block.
#pragma unroll
  for (int t = 0; t < kDB; ++t) {
    const int hrow = head_block(t % kPvHB) * kHW + lr, db = dim_block(t / kPvHB);
    const float l_h = s_l[hrow];
    const float inv = p.nsplit == 1 ? (bad ? __builtin_nanf("") : 1.0f / l_h)
                                    : (n_t > 0 ? 1.0f / l_h : 0.0f);
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const bf16x4_t v = {(__bf16)(oacc[t][4 * g4 + 0] * inv), (__bf16)(oacc[t][4 * g4 + 1] * inv),
                          (__bf16)(oacc[t][4 * g4 + 2] * inv), (__bf16)(oacc[t][4 * g4 + 3] * inv)};
      *(bf16x4_t*)(s_lat + hrow * kOutRow + 2 * (32 * db + 8 * g4 + 4 * hf)) = v;
    }
  }
  __syncthreads();   // every wave's slice of every row is written
  char* my_rows = s_lat + (wave * kHW) * kOutRow;
  __bf16* my_dst = dst + (int64_t)(wave * kHW) * kR;
  const int live_rows = min(kHW, p.n_heads - (hg * NW + wave) * kHW);   // heads that exist
#pragma unroll 4
  for (int r = 0; r < kHW; ++r) {
    if (r < live_rows) {
      const u32x4_t v = *(const u32x4_t*)(my_rows + r * kOutRow + 16 * lane);
      store_nt((u32x4_t*)(my_dst + (int64_t)r * kR + 8 * lane), v);
    }
  }
}

// Merge the splits of each (sequence, head) in split order: one wave per
// head, eight values per lane. Split s contributes 2^(m_s - M) l_s times its
// normalised partial, with a running maximum M; the loads of up to
// kCombineBatch splits are issued together, so a sequence costs one memory
// round trip per batch.
constexpr int kCombineThreads = 256;
constexpr int kCombineHeads = kCombineThreads / (kR / 8);   // heads per workgroup
constexpr int kCombineBatch = 8;
__global__ __launch_bounds__(kCombineThreads) void mla_combine(MlaParams p) {
  const int hh = threadIdx.x / (kR / 8);
  const int d = 8 * (threadIdx.x % (kR / 8));
  const int bh = blockIdx.x * kCombineHeads + hh;   // b * n_heads + h
  if (bh >= p.batch * p.n_heads) return;            // (whole waves)
  const int b = bh / p.n_heads, h = bh % p.n_heads;
  const int L = p.seq_lens[b];
  const bool bad = L < 1 || L > p.max_seq_len;
  const int nsp = bad ? 0 : (L + p.split_tokens - 1) / p.split_tokens;
  const int64_t w0 = (int64_t)b * p.nsplit * p.n_heads + h;   // split s: w0 + s * n_heads
  float M = -INFINITY, den = 0.0f;
  float num[8] = {};
  for (int s0 = 0; s0 < nsp; s0 += kCombineBatch) {
    float mm[kCombineBatch], ll[kCombineBatch];
    bf16x8_t oo[kCombineBatch];
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) {
      const bool ok = s0 + j < nsp;
      const int64_t w = w0 + (int64_t)(s0 + j) * p.n_heads;
      mm[j] = ok ? p.ws_ml[w * 2] : -INFINITY;
      ll[j] = ok ? p.ws_ml[w * 2 + 1] : 0.0f;
      oo[j] = ok ? *(const bf16x8_t*)(p.ws_o + w * kR + d) : bf16x8_t{};
    }
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) {
      if (s0 + j < nsp) {
        const float Mn = fmaxf(M, mm[j]);
        const float a = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
        // Every split below nsp holds tokens, so its m is finite, unless a
        // block outside the pool poisoned it (m = -inf, l = NaN): then wl is
        // NaN and so is the row.
        const float wl = __builtin_amdgcn_exp2f(mm[j] - Mn) * ll[j];
        den = fmaf(den, a, wl);
#pragma unroll
        for (int e = 0; e < 8; ++e) num[e] = fmaf(wl, (float)oo[j][e], num[e] * a);
        M = Mn;
      }
    }
  }
  const float inv = bad ? __builtin_nanf("") : 1.0f / den;
  bf16x8_t out;
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = (__bf16)(num[e] * inv);
  store_nt((bf16x8_t*)((__bf16*)p.o + (int64_t)bh * kR + d), out);
}

template <int NW>
int launch_nw(const MlaParams& p, hipStream_t stream) {
  const int n_items = p.batch * ((p.n_heads + kHW * NW - 1) / (kHW * NW)) * p.nsplit;
  if (p.block_table != nullptr) {
    hipLaunchKernelGGL((mla_kernel<NW, true>), dim3(n_items), dim3(64 * NW), 0, stream, p);
  } else {
    hipLaunchKernelGGL((mla_kernel<NW, false>), dim3(n_items), dim3(64 * NW), 0, stream, p);
  }
  return hipGetLastError() == hipSuccess ? kOk : kEhip;
}

}  // namespace

bool mla_supported(bool bf16, int kv_lora_rank, int rope_dim, int n_heads) {
  return bf16 && kv_lora_rank == kR && rope_dim == kP && n_heads >= 1 &&
         (n_heads <= kHW * kMaxWaves || n_heads % (kHW * kMaxWaves) == 0);
}

int mla_heads_per_group(int n_heads) { return min(n_heads, kHW * kMaxWaves); }
int mla_tile_tokens() { return kTile; }

int launch_mla(const MlaParams& p, hipStream_t stream) {
  // Every head count runs the four-wave workgroup of 128 heads: with fewer
  // heads the idle ones compute on a copy of the last head's query and are
  // not stored. (A workgroup of fewer waves would leave SIMDs of its compute
  // unit idle, as the 144 KB tile ring allows one workgroup per unit.)
  const int rc = launch_nw<kMaxWaves>(p, stream);
  if (rc != kOk) return rc;
  if (p.nsplit > 1) {
    const int64_t bh = (int64_t)p.batch * p.n_heads;
    hipLaunchKernelGGL(mla_combine, dim3((unsigned)((bh + kCombineHeads - 1) / kCombineHeads)),
                       dim3(kCombineThreads), 0, stream, p);
    if (hipGetLastError() != hipSuccess) return kEhip;
  }
  return kOk;
}

}  // namespace pkva

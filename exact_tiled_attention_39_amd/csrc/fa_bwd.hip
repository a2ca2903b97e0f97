// FlashAttention backward kernels for gfx950 (CDNA4): dQ, dK, dV of softmax(scale Q K^T) V,
// recomputing the scores and probabilities tile by tile instead of storing them (the "Flash
// Attention" notes, 14cs17, Common Pitfalls, Pitfall 3; FromZero2AI "FlashAttention: GPU
// Memory-Bound Speedups ...", section "Core Mechanisms", mechanism 3). With the forward's
// log-sum-exp L_i, P_ij = exp(s_ij - L_i) needs no running maximum, and the gradient of the
// loss sum(O * dO) is
//
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),   D_i = rowsum(dO * O)_i,
//     dQ = scale dS K,   dK = scale dS^T Q.
//
// Three launches on the caller's stream:
//  * fa_bwd_delta_kernel: D = rowsum(dO * O) in fp32, and -log2(e) L, into the caller's delta
//    workspace (two arrays of batch x heads_q x seqlen floats).
//  * fa_bwd_dkdv_kernel: one workgroup per 128 keys of a (batch entry or sequence, kv head).
//    Each SIMD runs a dV wave and a dK wave for the same 32 keys, with K (dV wave) or V (dK
//    wave) resident in registers as MFMA B operands and dV^T or dK^T accumulating in fp32.
//    64-query tiles of Q and dO (of every query head that shares the kv head) stream through a
//    three-stage LDS ring. The two waves of a SIMD alternate between matrix and element-wise
//    phases: the dV wave forms S = Q K^T and P of a tile, hands P to the dK wave through LDS
//    and accumulates dV^T += dO^T P; the dK wave, one phase behind, forms dP = dO V^T,
//    dS = P (dP - D) and accumulates dK^T += Q^T dS.
//  * fa_bwd_dq_kernel: one workgroup per 256 queries of a (batch entry or sequence, query
//    head). Its 8 waves own 32 queries each, with Q^T and dO^T resident, and dQ^T
//    accumulating. 64-key tiles of K and V stream through a three-stage LDS ring. The two
//    waves of a SIMD alternate between matrix phases (S^T = K Q^T and dP^T = V dO^T of a tile,
//    lane = query, with dQ^T += K^T dS^T of the tile before) and element-wise phases (dS^T).
//  * Q and dO (dK/dV) and K (dQ) are read both as operands of a contraction over head-dims and,
//    transposed, of a contraction over the tile's rows; each tile is stored once in LDS, in a
//    swizzled layout that serves both reads without bank conflicts.
// Splitting dQ from dK/dV recomputes S and dP once more, but every gradient accumulates in
// one workgroup's registers: no atomics, and the result is deterministic.
// All MFMAs are v_mfma_f32_32x32x16_{bf16,f16}; P and dS are rounded to the input type (round
// to nearest even) as MFMA operands; gradients accumulate in fp32 and are stored rounded to
// the input type.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <utility>

#include "fa.h"
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

using namespace dev;

constexpr int kTileRows = 32;    // rows of the streamed side per step

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  float* delta;       // D, the first array of the caller's workspace
  float* nlse;        // -log2(e) L, the second array
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  const int32_t* cu_seqlens;
  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int64_t do_sb, do_sh, do_sn;
  int64_t dq_sb, dq_sh, dq_sn;
  int64_t dk_sb, dk_sh, dk_sn;
  int64_t dv_sb, dv_sh, dv_sn;
  int32_t seqlen;     // tokens per batch entry (packed total for varlen)
  int32_t heads_q;
  int32_t heads_kv;
  int32_t group;      // heads_q / heads_kv
  int32_t n_kblocks;  // 128-key blocks per (batch entry or sequence)
  int32_t n_qblocks;  // 256-query blocks per (batch entry or sequence)
  int32_t rows_delta; // batch * heads_q * seqlen
  float c;            // |scale| * log2(e), or log2(e) when scale == 0
  uint32_t s_and;     // 0 when scale == 0, else all ones (applied to the resident operand)
  uint32_t s_xor;     // 0x80008000 when scale < 0 (negates the resident operand exactly)
  float scale;        // the signed scale: dQ = scale dS K, dK = scale dS^T Q
};

constexpr float kLog2e = 1.4426950408889634f;

// Single-copy layout of a 32-row tile (rows are queries or keys, head-dim contiguous in device
// memory), for a tensor that is read both ways: as the operand of a contraction over head-dims
// and, through ds_read_b64_tr_b16, as the A operand of a contraction over rows. Block s (1 KB)
// holds head-dims 16 s .. 16 s + 15 of the 32 rows as 64 chunks of 16 bytes; chunk (r, c) is
// row r, head-dims 16 s + 8 c .. + 7, and sits at chunk position
//     16 (r / 16 + 2 c) + r % 4 + 4 ((r / 4 + c + 2 (s % 2)) % 4).
// The rotation of the 4-row group index by c and by the block parity spreads both read
// patterns over all LDS banks: 16 lanes of an operand read hit 16 distinct 16-byte slots of a
// 256-byte bank row, and 32 lanes of a transposing read hit 32 distinct 8-byte slots.
struct SwizzledTile {
  // The chunk that lane L of a direct-to-LDS load into block s receives (its position is L).
  static __device__ __forceinline__ void row_col(int s, int lane, int& row, int& col) {
    const int hi = lane >> 4, lo = lane & 15;
    const int c = hi >> 1;
    row = 16 * (hi & 1) + 4 * (((lo >> 2) - c - 2 * (s & 1)) & 3) + (lo & 3);
    col = 16 * s + 8 * c;
  }
  // Operand read: lane L takes chunk (L % 32, L / 32) of block s at byte s * 1024 + this
  // offset (sp = s % 2).
  static __device__ __forceinline__ int operand_offset(int lane, int sp) {
    const int r = lane & 31, c = lane >> 5;
    return 16 * (16 * ((r >> 4) + 2 * c) + (r & 3) + 4 * (((r >> 2) + c + 2 * sp) & 3));
  }
  // Transposing reads of the A operand for head-dims 32 j .. 32 j + 31 and rows 16 t .. 16 t +
  // 15: the read for rows {4 g .. 4 g + 3} (part 0) or {8 + 4 g .. 8 + 4 g + 3} (part 1) of
  // half-wave g sits at byte 2048 j + 256 t + this offset. Lane L supplies 4 head-dims of one
  // row: row 8 part + 4 (L / 32) + (L % 16) / 4 of the step, head-dims 32 j + 16 ((L / 16) % 2)
  // + 4 (L % 4) .. + 3.
  static __device__ __forceinline__ int transpose_offset(int lane, int part) {
    const int g16 = lane >> 4, i = lane & 15;
    const int c = (i >> 1) & 1, sp = g16 & 1;
    return 1024 * sp + 512 * c + 16 * (i >> 2) + 64 * ((2 * part + (g16 >> 1) + c + 2 * sp) & 3) +
           8 * (i & 1);
  }
};

// ---------------------------------------------------------------------------------------
// D = rowsum(dO * O), fp32. 16 lanes per row, 8 (d = 128) or 4 (d = 64) elements per lane.
// The same pass writes -log2(e) L of every row, the offset the dK/dV kernel adds to c S: one
// multiply per row here instead of one per score there.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void fa_bwd_delta_kernel(const BwdArgs p) {
  using E = Elem<BF16>;
  constexpr int kPer = D / 16;
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int part = threadIdx.x & 15;
  float acc = 0.f;
  if (row < p.rows_delta) {
    const int n = row % p.seqlen;
    const int bh = row / p.seqlen;
    const int h = bh % p.heads_q, b = bh / p.heads_q;
    const uint16_t* orow = p.o + b * p.o_sb + h * p.o_sh + int64_t(n) * p.o_sn + part * kPer;
    const uint16_t* drow = p.dout + b * p.do_sb + h * p.do_sh + int64_t(n) * p.do_sn + part * kPer;
#pragma unroll
    for (int e = 0; e < kPer; ++e) acc += E::to_f32(orow[e]) * E::to_f32(drow[e]);
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
  if (part == 0 && row < p.rows_delta) p.delta[row] = acc;
  if (part == 1 && row < p.rows_delta) p.nlse[row] = p.lse[row] * -kLog2e;
}

// ---------------------------------------------------------------------------------------
// Shared pieces of the two main kernels.

template <int D>
struct BwdGeo {
  static constexpr int kSteps = D / 16;       // head-dim steps of a contraction over D
  static constexpr int kOBlocks = D / 32;     // 32-wide head-dim blocks
  static constexpr int kBlocks = kTileRows * D / 512;  // 1 KB blocks per tile per layout
  static constexpr int kTileBytes = kBlocks * 1024;
};

// Workgroup order: (batch entry or sequence, head) pairs in plain order, block index heaviest
// first where `desc` (causal work grows with the block index when desc, shrinks otherwise).
struct Item {
  int blk, b, h;
};
__device__ __forceinline__ Item item_of(int pairs, int heads, int n_blocks, bool desc) {
  const int t = blockIdx.x / pairs;
  const int bh = blockIdx.x - t * pairs;
  Item it;
  it.blk = desc ? n_blocks - 1 - t : t;
  it.b = bh / heads;
  it.h = bh - it.b * heads;
  return it;
}

// The 16 row entries of a 32x32 accumulator held by lane (half = lane / 32): entry i is row
// 8 (i / 4) + 4 half + i % 4. Rows [row0, row0 + 32) of a 64-row tile: 4 runs of 4 floats.
__device__ __forceinline__ void read_rows16(const float* lds_rows, int half, float out[16]) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(lds_rows + 8 * g + 4 * half);
    out[4 * g + 0] = x[0];
    out[4 * g + 1] = x[1];
    out[4 * g + 2] = x[2];
    out[4 * g + 3] = x[3];
  }
}

// Store a transposed 32-row x D accumulator set (lane = row, entries = head-dims) as rows of
// the output: entry 4 g + r of block j is head-dim 32 j + 8 g + 4 half + r.
template <int D, bool BF16>
__device__ __forceinline__ void store_rows(uint16_t* row_ptr, const f32x16* acc, float mul,
                                           int half) {
  using E = Elem<BF16>;
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = j * 32 + 8 * g + 4 * half;
      u32x2 w;
      w[0] = E::pack(acc[j][4 * g + 0] * mul, acc[j][4 * g + 1] * mul);
      w[1] = E::pack(acc[j][4 * g + 2] * mul, acc[j][4 * g + 3] * mul);
      *reinterpret_cast<u32x2*>(row_ptr + d0) = w;
    }
  }
}

// Resident B operands of a wave's 32 rows: lane L holds row r0 + L % 32, head-dims
// 16 s + 8 (L / 32) .. + 7 for every step s (rows outside [0, nrows) read as zero).
template <int D>
__device__ __forceinline__ void load_resident(const uint16_t* base, int64_t sn, int r0, int nrows,
                                              int lane, u32x4* out) {
  const int rows = min(max(nrows - r0, 0), 32);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(base + int64_t(max(r0, 0)) * sn), (short)0,
      rows > 0 ? int((rows - 1) * sn * 2) + D * 2 : 0, 0x00020000);
  const int off = int((lane & 31) * sn * 2) + (lane >> 5) * 16;
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    out[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + s * 32,
                                                                             0, 0));
}

// ---------------------------------------------------------------------------------------
// Both main kernels run 8 waves, two per SIMD, each wave within 256 registers, so that the
// SIMD overlaps one wave's element-wise phase with the other's matrix phase. A tile of 64 rows
// of the streamed side moves through a three-stage LDS ring per step.

constexpr int kWaves = 8;
constexpr int kThreads8 = 64 * kWaves;

// ---------------------------------------------------------------------------------------
// dK, dV: one workgroup per 128 keys. Waves 0-3 (one per SIMD) accumulate dV for 32 keys
// each, waves 4-7 dK for the same keys; a SIMD holds one of each, and the two alternate, one
// barrier-delimited phase apart, between matrix work (M phase) and element-wise work (V
// phase), so that each SIMD overlaps one wave's exponentials or products with the other's
// MFMAs. Query tiles of 64 rows (of one query head; the tiles of every query head that
// shares the kv head follow each other) are processed as two 32-row halves. For tile t:
//   slot A_t: dV wave M: S(t) = Q(t) K^T interleaved with dV^T += dO(t-1)^T P(t-1);
//             dK wave V: dS(t-1) = P(t-1) (dP(t-1) - D(t-1)), rounded as the B operand;
//   slot B_t: dV wave V: P(t) = exp2(c S(t) - log2(e) L) (masked), stored in fp32 for the dK
//             wave and rounded as its own B operand;
//             dK wave M: dP(t) = dO(t) V^T interleaved with dK^T += Q(t-1)^T dS(t-1).
// P(t) is written in B_t and read in A_{t+1}, so one LDS slot holds it. Q and dO tiles, with
// the tile's L and D, stream through a three-stage LDS ring by direct-to-LDS loads issued one
// tile ahead; each is stored once, in the swizzled layout that serves both its operand and its
// transposing reads.
template <int D, bool BF16, bool CAUSAL, bool VARLEN>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads8, kThreads8),
                          amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dkdv_kernel(const BwdArgs p) {
  using E = Elem<BF16>;
  using G = BwdGeo<D>;
  constexpr int kSteps = G::kSteps;
  constexpr int kOBlocks = G::kOBlocks;
  constexpr int kRowsT = 2 * kTileRows;        // query rows per tile
  constexpr int kHalfBytes = G::kTileBytes;    // one 32-row half of a tile
  constexpr int kTBytes = 2 * G::kTileBytes;   // a 64-row tile of one tensor
  constexpr int kPer = 2 * G::kBlocks / 4;     // 1 KB blocks of its tensor a wave loads per tile
  constexpr int kRing = 3;
  // Ring stage x of each tensor: Q tile at kQ + x kTBytes, dO tile at kDo + x kTBytes, 64
  // values -log2(e) L at kRows + 2048 x and 64 D 1 KB after them (each a 1 KB direct-to-LDS
  // load); each region spans less than 64 KB, so a per-lane base plus an immediate reaches
  // every stage.
  constexpr int kQ = 0, kDo = kRing * kTBytes, kRows = 2 * kRing * kTBytes;
  constexpr int kPbuf = kRows + kRing * 2048;  // P of each key group: 64 rows x 32 keys fp32
  constexpr int kPwave = 2 * 4096;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kPbuf + 4 * kPwave];
  const uint32_t lds0 = lds_address(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = wave >> 2;  // 0: dV, 1: dK
  const int half = lane >> 5;

  const int pairs = gridDim.x / p.n_kblocks;
  const Item it = item_of(pairs, p.heads_kv, p.n_kblocks, false);
  const int hk = it.h;
  int seq0 = 0, slen = p.seqlen, bidx = it.b;
  if (VARLEN) {
    seq0 = p.cu_seqlens[it.b];
    slen = p.cu_seqlens[it.b + 1] - seq0;
    bidx = 0;
  }
  const int k0 = it.blk * 128;
  if (k0 >= slen) return;  // uniform across the workgroup
  const int kw0 = k0 + 32 * (wave & 3);  // first key of this wave
  const int key = kw0 + (lane & 31);     // key of this lane (accumulator column)

  const int t_first = CAUSAL ? k0 / kRowsT : 0;
  const int n_qt = (slen + kRowsT - 1) / kRowsT;
  const int per_head = n_qt - t_first;
  const int n_steps = per_head * p.group;

  // DMA: waves 0-3 load the Q blocks of a tile, waves 4-7 the dO blocks, kPer each (block b is
  // block b % kSteps of half b / kSteps); waves 0 and 1 also load the tile's 64 -log2(e) L and
  // 64 D values (lanes 0..15 carry them, the rest read 0).
  const bool is_do = role;
  const int64_t lay_sn = is_do ? p.do_sn : p.q_sn;
  const int64_t lay_sh = is_do ? p.do_sh : p.q_sh;
  int ld_off[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = (wave & 3) * kPer + i;
    int row, col;
    SwizzledTile::row_col(b % kSteps, lane, row, col);
    ld_off[i] = int((row + kTileRows * (b / kSteps)) * lay_sn * 2) + col * 2;
  }
  // The next tile to issue, carried from tile to tile (tile x is query tile t_first +
  // x % per_head of query head it.h * group + x / per_head): its tile index, row pointer and
  // LSE/D row; a change of head adds the jump to the next head's first tile.
  const int hq0 = it.h * p.group;
  const uint16_t* iss_src = (is_do ? p.dout + bidx * p.do_sb : p.q + bidx * p.q_sb) +
                            hq0 * lay_sh + int64_t(seq0 + t_first * kRowsT) * lay_sn;
  const int64_t src_step = int64_t(kRowsT) * lay_sn;
  const int64_t src_jump = lay_sh - int64_t(per_head) * src_step;
  int64_t iss_lrow = (int64_t(bidx) * p.heads_q + hq0) * p.seqlen + seq0 + t_first * kRowsT;
  const int64_t lrow_jump = p.seqlen - int64_t(per_head) * kRowsT;
  int iss_t = t_first;
  auto issue = [&](int stage) __attribute__((always_inline)) {
    const int rows = min(slen - iss_t * kRowsT, kRowsT);
    const u32x4 rs = make_rsrc(iss_src, int((rows - 1) * lay_sn * 2) + D * 2);
    const uint32_t base = lds0 + (is_do ? kDo : kQ) + stage * kTBytes + (wave & 3) * kPer * 1024;
#pragma unroll
    for (int i = 0; i < kPer; ++i) dma16(rs, base + i * 1024, ld_off[i]);
    if (wave < 2) {
      const float* lsrc = wave == 0 ? p.nlse + iss_lrow : p.delta + iss_lrow;
      dma16(make_rsrc(lsrc, rows * 4), lds0 + kRows + stage * 2048 + wave * 1024, lane * 16);
    }
    iss_src += src_step;
    iss_lrow += kRowsT;
    if (++iss_t == n_qt) {
      iss_t = t_first;
      iss_src += src_jump;
      iss_lrow += lrow_jump;
    }
  };
  // phase boundary: a workgroup barrier that orders the P hand-off through LDS (a fence on
  // both sides) and that the instruction scheduler may not move work across
  auto phase_sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };

  // per-lane LDS read offsets, each with its region's start folded in and hidden from the
  // compiler, so that it addresses every stage of a region as this base plus an immediate
  // instead of keeping one address register per stage
  auto lane_base = [](int off) __attribute__((always_inline)) {
    asm volatile("" : "+v"(off));
    return off;
  };
  const int q_op0 = lane_base(kQ + SwizzledTile::operand_offset(lane, 0));
  const int q_op1 = lane_base(kQ + SwizzledTile::operand_offset(lane, 1));
  const int q_tr0 = lane_base(kQ + SwizzledTile::transpose_offset(lane, 0));
  const int q_tr1 = lane_base(kQ + SwizzledTile::transpose_offset(lane, 1));
  const int do_op0 = lane_base(kDo + SwizzledTile::operand_offset(lane, 0));
  const int do_op1 = lane_base(kDo + SwizzledTile::operand_offset(lane, 1));
  const int do_tr0 = lane_base(kDo + SwizzledTile::transpose_offset(lane, 0));
  const int do_tr1 = lane_base(kDo + SwizzledTile::transpose_offset(lane, 1));
  const int rows_rd = lane_base(kRows + 16 * half);
  // P hand-off: entries 4 g .. 4 g + 3 of half hf, lane L at byte 4096 hf + 1024 g + 16 L of
  // the wave's 8 KB
  unsigned char* const pbuf = smem + lane_base(kPbuf + (wave & 3) * kPwave + lane * 16);

  // resident B operand: K^T (sign of the scale applied) for the dV wave, V^T for the dK wave
  u32x4 rf[kSteps];
  if (role) {
    load_resident<D>(p.v + bidx * p.v_sb + hk * p.v_sh + int64_t(seq0) * p.v_sn, p.v_sn, kw0,
                     slen, lane, rf);
  } else {
    load_resident<D>(p.k + bidx * p.k_sb + hk * p.k_sh + int64_t(seq0) * p.k_sn, p.k_sn, kw0,
                     slen, lane, rf);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) rf[s] = (rf[s] & p.s_and) ^ p.s_xor;
  }
  f32x16 acc[kOBlocks];  // dV^T or dK^T: lane holds head-dims of its key column
#pragma unroll
  for (int j = 0; j < kOBlocks; ++j) acc[j] = f32x16{};
  f32x16 xacc[2];  // S (dV wave) or dP (dK wave) of each half of the tile between its phases
  xacc[0] = xacc[1] = f32x16{};
  u32x4 pb[4];     // P (dV wave) or dS (dK wave), rounded: B operands of the row chain
#pragma unroll
  for (int u = 0; u < 4; ++u) pb[u] = u32x4{0, 0, 0, 0};

  // M phase: the chains over head-dims of the two halves (xacc[hf] = rows of half hf of the
  // tile in stage xs (operand reads) . rf) and the chain over rows (acc[j] += (head-dims of
  // block j of the tile in stage ys, transposing reads) . pb), interleaved one to one, each
  // LDS operand read kAheadM MFMAs before its MFMA.
  constexpr int kMfma = 4 * kSteps;
  static_assert(4 * kOBlocks == 2 * kSteps, "one row-chain MFMA per d-chain MFMA");
  constexpr int kAheadM = 8;
  // At d = 64 the dV wave reads its tile's -log2(e) L rows in its M phase, which is half as
  // long as its V phase there (measured 3-4 % faster; at d = 128 the M phase is the tight one).
  float nl_r[2][16];
  auto phase_m = [&](auto dk_c, int xs, int ys) __attribute__((always_inline)) {
    constexpr bool DK = decltype(dk_c)::value;  // d chain over dO, row chain over Q
    if constexpr (!DK && D == 64) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        read_rows16(reinterpret_cast<const float*>(smem + rows_rd + xs * 2048 + 128 * hf), 0,
                    nl_r[hf]);
    }
    const int x0 = (DK ? do_op0 : q_op0) + xs * kTBytes;
    const int x1 = (DK ? do_op1 : q_op1) + xs * kTBytes;
    const int y0 = (DK ? q_tr0 : do_tr0) + ys * kTBytes;
    const int y1 = (DK ? q_tr1 : do_tr1) + ys * kTBytes;
    u32x4 opnd[kMfma];
    // MFMA n: even n is d-chain step s = n / 4 of half (n / 2) % 2; odd n is row-chain MFMA
    // m = n / 2, head-dim block m % kOBlocks, 16-row step u = m / kOBlocks (half u / 2)
    auto fetch = [&](auto nn) __attribute__((always_inline)) {
      constexpr int n = decltype(nn)::value;
      if constexpr (n % 2 == 0) {
        constexpr int hf = (n / 2) % 2, s = n / 4;
        opnd[n] = *reinterpret_cast<const u32x4*>(smem + ((s & 1) ? x1 : x0) + hf * kHalfBytes +
                                                  s * 1024);
      } else {
        constexpr int m = n / 2, j = m % kOBlocks, u = m / kOBlocks;
        constexpr int off = (u / 2) * kHalfBytes + 2048 * j + 256 * (u % 2);
        const u32x2 lo = E::read_tr(smem + y0 + off);
        const u32x2 hi = E::read_tr(smem + y1 + off);
        opnd[n] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    };
    auto mfma = [&](auto nn) __attribute__((always_inline)) {
      constexpr int n = decltype(nn)::value;
      if constexpr (n % 2 == 0) {
        constexpr int hf = (n / 2) % 2, s = n / 4;
        xacc[hf] = E::mfma(opnd[n], rf[s], s == 0 ? f32x16{} : xacc[hf]);
      } else {
        constexpr int m = n / 2, j = m % kOBlocks, u = m / kOBlocks;
        acc[j] = E::mfma(opnd[n], pb[u], acc[j]);
      }
    };
    [&]<int... n>(std::integer_sequence<int, n...>) {
      (fetch(Int<n>{}), ...);
    }(std::make_integer_sequence<int, kAheadM>{});
    [&]<int... n>(std::integer_sequence<int, n...>) {
      ((
           [&] {
             if constexpr (n + kAheadM < kMfma) fetch(Int<n + kAheadM>{});
             mfma(Int<n>{});
             __builtin_amdgcn_sched_barrier(0);
           }()),
       ...);
    }(std::make_integer_sequence<int, kMfma>{});
  };

  // dV wave's V phase for the tile in stage `stage`: P = exp2(c S - log2(e) L), masked where
  // the key is past the end or above the diagonal; stored for the dK wave, rounded into pb.
  int cur_t = t_first;  // query tile of the next V phase (advanced like the issue's)
  auto phase_v_dv = [&](int stage) __attribute__((always_inline)) {
    const int r0t = cur_t * kRowsT;
    if (++cur_t == n_qt) cur_t = t_first;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int r0 = r0t + kTileRows * hf;
      // entry i is query row r0 + 4 half + off_i, off_i = 8 (i / 4) + i % 4
      float nl[16], pv[16];
      if constexpr (D == 64) {
#pragma unroll
        for (int i = 0; i < 16; ++i) nl[i] = nl_r[hf][i];
      } else {
        read_rows16(reinterpret_cast<const float*>(smem + rows_rd + stage * 2048 + 128 * hf), 0,
                    nl);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) pv[i] = fmaf(xacc[hf][i], p.c, nl[i]);
      if ((r0 + kTileRows > slen) || (CAUSAL && r0 < kw0 + 31)) {
        // the entry is visible when lo <= off_i <= hi (no row of a key past the end is)
        const int rbase = r0 + 4 * half;
        const int hi = slen - 1 - rbase;
        const int lo = key < slen ? (CAUSAL ? key - rbase : -kTileRows) : kTileRows;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = 8 * (i >> 2) + (i & 3);
          pv[i] = (off >= lo && off <= hi) ? pv[i] : -INFINITY;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) pv[i] = __builtin_amdgcn_exp2f(pv[i]);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(pbuf + 4096 * hf + g * 1024) =
            f32x4{pv[4 * g], pv[4 * g + 1], pv[4 * g + 2], pv[4 * g + 3]};
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int w = 0; w < 4; ++w)
          pb[2 * hf + tt][w] = E::pack(pv[8 * tt + 2 * w], pv[8 * tt + 2 * w + 1]);
    }
  };
  // dK wave's V phase for the tile in stage `stage`: dS = P (dP - D), rounded into pb.
  auto phase_v_dk = [&](int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      float del[16];
      read_rows16(reinterpret_cast<const float*>(smem + rows_rd + stage * 2048 + 1024 + 128 * hf),
                  0, del);
      float ds[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 pv = *reinterpret_cast<const f32x4*>(pbuf + 4096 * hf + g * 1024);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          ds[4 * g + r] = pv[r] * (xacc[hf][4 * g + r] - del[4 * g + r]);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int w = 0; w < 4; ++w)
          pb[2 * hf + tt][w] = E::pack(ds[8 * tt + 2 * w], ds[8 * tt + 2 * w + 1]);
    }
  };

  // Slots A_t and B_t, with the ring stage of tile t a loop variable. Tile t + 1 is issued in
  // A_t into the stage of tile t - 2, whose last reader (the dK wave's Q^T in B_{t-1}) finished
  // before B_{t-1}'s closing barrier; B_t's closing barrier waits for it (A_{t+1} reads it).
  // The loop runs t = 0 .. n_steps, every phase unconditional: in A_0 and B_0 the products
  // with tile -1 meet zeros (stage kRing - 1, P and the B operands start at 0); in A_{n_steps}
  // and B_{n_steps} the d chains read a stale stage and their results, like P(n_steps), are
  // never used. Both waves run every barrier.
  auto run = [&](auto role_c) __attribute__((always_inline)) {
    constexpr bool DK = decltype(role_c)::value;
    int st = 0, st_prev = kRing - 1, st_next = 1;
    for (int t = 0; t <= n_steps; ++t) {
      if (t + 1 < n_steps) issue(st_next);
      if constexpr (!DK)
        phase_m(role_c, st, st_prev);
      else
        phase_v_dk(st_prev);
      phase_sync();
      if constexpr (!DK)
        phase_v_dv(st);
      else
        phase_m(role_c, st, st_prev);
      if (t + 1 < n_steps) wait_vmcnt<0>();  // tile t + 1
      phase_sync();
      st_prev = st;
      st = st_next;
      st_next = st_next == kRing - 1 ? 0 : st_next + 1;
    }
  };

  if (n_steps > 0) {
    {
      // Stage kRing - 1 (Q, dO, L and D) and P stand in for tile -1 until tile kRing - 1 lands
      // there: zeros, so that dS(-1) = 0 and every product with tile -1 adds 0.
      const u32x4 zero = u32x4{0, 0, 0, 0};
      for (int off = tid * 16; off < kTBytes; off += kThreads8 * 16) {
        *reinterpret_cast<u32x4*>(smem + kQ + (kRing - 1) * kTBytes + off) = zero;
        *reinterpret_cast<u32x4*>(smem + kDo + (kRing - 1) * kTBytes + off) = zero;
      }
      for (int off = tid * 16; off < 4 * kPwave; off += kThreads8 * 16)
        *reinterpret_cast<u32x4*>(smem + kPbuf + off) = zero;
      if (tid < 128)
        *reinterpret_cast<u32x4*>(smem + kRows + (kRing - 1) * 2048 + tid * 16) = zero;
    }
    issue(0);
    // Tile 0 and the resident operand are complete from here on: passing the operand through
    // an empty asm makes the compiler's own load tracking agree, so that it adds no memory
    // waits inside the loop (where they would also wait for the tile in flight).
    wait_vmcnt<0>();
#pragma unroll
    for (int s = 0; s < kSteps; ++s) asm volatile("" : "+v"(rf[s]));
    __syncthreads();
    if (role)
      run(std::true_type{});
    else
      run(std::false_type{});
  }
  if (key < slen) {
    if (role)
      store_rows<D, BF16>(p.dk + bidx * p.dk_sb + hk * p.dk_sh + int64_t(seq0 + key) * p.dk_sn,
                          acc, p.scale, half);
    else
      store_rows<D, BF16>(p.dv + bidx * p.dv_sb + hk * p.dv_sh + int64_t(seq0 + key) * p.dv_sn,
                          acc, 1.f, half);
  }
}

// ---------------------------------------------------------------------------------------
// dQ: one workgroup per 256 queries, 8 waves of 32 queries, Q^T and dO^T resident and dQ^T
// accumulating in each. Key tiles of 64 keys are processed as two 32-key halves. The waves of
// a SIMD (w and w + 4, groups 0 and 1) alternate, one barrier-delimited phase apart, between
// an M phase, M(t): S^T(t) = K(t) Q^T and dP^T(t) = V(t) dO^T interleaved with
// dQ^T += K(t-1)^T dS^T(t-1), and a V phase, V(t): dS^T(t) = P^T(t) (dP^T(t) - D) with
// P^T(t) = exp2(c S^T(t) - log2(e) L) (masked), rounded as the next M phase's B operand.
// Step t: group 0 runs M(t), then V(t); group 1 runs V(t-1), then M(t). A barrier ends each
// step; at d = 64 a second one between the halves holds the groups in opposite phases (slot
// 2t: M(t) beside V(t-1); slot 2t+1: V(t) beside M(t)), while at d = 128 the groups may drift
// within a step (1-3 % faster there, slower at d = 64, the same bits).
// K and V tiles stream through a three-stage LDS ring by direct-to-LDS loads issued one tile
// ahead; each is stored once, in the swizzled layout (K serves both its operand and its
// transposing reads).
template <int D, bool BF16, bool CAUSAL, bool VARLEN>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads8, kThreads8),
                          amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dq_kernel(const BwdArgs p) {
  using E = Elem<BF16>;
  using G = BwdGeo<D>;
  constexpr int kSteps = G::kSteps;
  constexpr int kOBlocks = G::kOBlocks;
  constexpr int kKeysT = 2 * kTileRows;       // keys per tile
  constexpr int kHalfBytes = G::kTileBytes;   // one 32-key half of a tile
  constexpr int kTBytes = 2 * G::kTileBytes;  // a 64-key tile of one tensor
  constexpr int kPer = 2 * G::kBlocks / 4;    // 1 KB blocks of its tensor a wave loads per tile
  constexpr int kRing = 3;
  // ring stage x: K tile at kK + x kTBytes, V tile at kV + x kTBytes
  constexpr int kK = 0, kV = kRing * kTBytes;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kRing * kTBytes];
  const uint32_t lds0 = lds_address(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int half = lane >> 5;

  const int pairs = gridDim.x / p.n_qblocks;
  const Item it = item_of(pairs, p.heads_q, p.n_qblocks, CAUSAL);
  const int h = it.h;
  const int hk = h / p.group;
  int seq0 = 0, slen = p.seqlen, bidx = it.b;
  if (VARLEN) {
    seq0 = p.cu_seqlens[it.b];
    slen = p.cu_seqlens[it.b + 1] - seq0;
    bidx = 0;
  }
  const int q0 = it.blk * 256;
  if (q0 >= slen) return;  // uniform across the workgroup
  // The waves of a SIMD take neighbouring 32-query slices, so both reach the causal diagonal
  // at nearly the same tile.
  const int qw0 = q0 + 32 * (2 * (wave & 3) + grp);  // first query of this wave
  const int qrow = qw0 + (lane & 31);                 // query of this lane (accumulator column)

  u32x4 qf[kSteps], dof[kSteps];
  load_resident<D>(p.q + bidx * p.q_sb + h * p.q_sh + int64_t(seq0) * p.q_sn, p.q_sn, qw0, slen,
                   lane, qf);
  load_resident<D>(p.dout + bidx * p.do_sb + h * p.do_sh + int64_t(seq0) * p.do_sn, p.do_sn, qw0,
                   slen, lane, dof);
  float nlse = 0.f, del = 0.f;  // -log2e LSE and D of this lane's query
  if (qrow < slen) {
    const int64_t r = (int64_t(bidx) * p.heads_q + h) * p.seqlen + seq0 + qrow;
    nlse = p.nlse[r];
    del = p.delta[r];
  }
  f32x16 dqacc[kOBlocks];
#pragma unroll
  for (int j = 0; j < kOBlocks; ++j) dqacc[j] = f32x16{};

  const int kv_end = CAUSAL ? min(slen, q0 + 256) : slen;
  const int n_tiles = (kv_end + kKeysT - 1) / kKeysT;

  // DMA: waves 0-3 load the K blocks of a tile, waves 4-7 the V blocks, kPer each (block b is
  // block b % kSteps of half b / kSteps)
  const int64_t lay_sn = grp ? p.v_sn : p.k_sn;
  int ld_off[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = (wave & 3) * kPer + i;
    int row, col;
    SwizzledTile::row_col(b % kSteps, lane, row, col);
    ld_off[i] = int((row + kTileRows * (b / kSteps)) * lay_sn * 2) + col * 2;
  }
  // rows of the next tile to issue, carried from tile to tile
  const uint16_t* iss_src = grp ? p.v + bidx * p.v_sb + hk * p.v_sh + int64_t(seq0) * p.v_sn
                                : p.k + bidx * p.k_sb + hk * p.k_sh + int64_t(seq0) * p.k_sn;
  const int64_t src_step = int64_t(kKeysT) * lay_sn;
  int iss_r0 = 0;
  auto issue = [&](int stage) __attribute__((always_inline)) {
    const int rows = min(slen - iss_r0, kKeysT);
    const u32x4 rs = make_rsrc(iss_src, int((rows - 1) * lay_sn * 2) + D * 2);
    const uint32_t base = lds0 + (grp ? kV : kK) + stage * kTBytes + (wave & 3) * kPer * 1024;
#pragma unroll
    for (int i = 0; i < kPer; ++i) dma16(rs, base + i * 1024, ld_off[i]);
    iss_src += src_step;
    iss_r0 += kKeysT;
  };
  auto phase_sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };

  // per-lane LDS read offsets (region start folded in, hidden from the compiler so that every
  // stage is this base plus an immediate)
  auto lane_base = [](int off) __attribute__((always_inline)) {
    asm volatile("" : "+v"(off));
    return off;
  };
  const int k_op0 = lane_base(kK + SwizzledTile::operand_offset(lane, 0));
  const int k_op1 = lane_base(kK + SwizzledTile::operand_offset(lane, 1));
  const int k_tr0 = lane_base(kK + SwizzledTile::transpose_offset(lane, 0));
  const int k_tr1 = lane_base(kK + SwizzledTile::transpose_offset(lane, 1));
  const int v_op0 = lane_base(kV + SwizzledTile::operand_offset(lane, 0));
  const int v_op1 = lane_base(kV + SwizzledTile::operand_offset(lane, 1));

  f32x16 sacc[2], dpacc[2];  // S^T and dP^T of each half of the tile between its phases
  sacc[0] = sacc[1] = dpacc[0] = dpacc[1] = f32x16{};
  u32x4 pb[4];               // dS^T of the previous tile, rounded (B operands)
#pragma unroll
  for (int u = 0; u < 4; ++u) pb[u] = u32x4{0, 0, 0, 0};

  // M phase on the tile in stage xs (S^T and dP^T chains of both halves) and the previous tile
  // in stage ys (dQ^T chain): MFMA n is, by n % 3, S, dP (step s = n / 6 of half (n / 3) % 2)
  // or dQ (MFMA n / 3: head-dim block % kOBlocks, 16-key step / kOBlocks); each LDS operand
  // is read kAheadM MFMAs before its MFMA.
  constexpr int kMfma = 6 * kSteps;
  static_assert(4 * kOBlocks == 2 * kSteps, "one dQ MFMA per S MFMA");
  constexpr int kAheadM = 4;
  auto phase_m = [&](int xs, int ys) __attribute__((always_inline)) {
    const int xo = xs * kTBytes, yo = ys * kTBytes;
    const int ko0 = k_op0 + xo, ko1 = k_op1 + xo, vo0 = v_op0 + xo, vo1 = v_op1 + xo;
    const int kt0 = k_tr0 + yo, kt1 = k_tr1 + yo;
    u32x4 opnd[kMfma];
    auto fetch = [&](auto nn) __attribute__((always_inline)) {
      constexpr int n = decltype(nn)::value, g = n / 3, hf = g % 2, s = g / 2;
      if constexpr (n % 3 == 0) {
        opnd[n] = *reinterpret_cast<const u32x4*>(smem + ((s & 1) ? ko1 : ko0) +
                                                  hf * kHalfBytes + s * 1024);
      } else if constexpr (n % 3 == 1) {
        opnd[n] = *reinterpret_cast<const u32x4*>(smem + ((s & 1) ? vo1 : vo0) +
                                                  hf * kHalfBytes + s * 1024);
      } else {
        constexpr int j = g % kOBlocks, u = g / kOBlocks;
        constexpr int off = (u / 2) * kHalfBytes + 2048 * j + 256 * (u % 2);
        const u32x2 lo = E::read_tr(smem + kt0 + off);
        const u32x2 hi = E::read_tr(smem + kt1 + off);
        opnd[n] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    };
    auto mfma = [&](auto nn) __attribute__((always_inline)) {
      constexpr int n = decltype(nn)::value, g = n / 3, hf = g % 2, s = g / 2;
      if constexpr (n % 3 == 0) {
        sacc[hf] = E::mfma(opnd[n], qf[s], s == 0 ? f32x16{} : sacc[hf]);
      } else if constexpr (n % 3 == 1) {
        dpacc[hf] = E::mfma(opnd[n], dof[s], s == 0 ? f32x16{} : dpacc[hf]);
      } else {
        constexpr int j = g % kOBlocks, u = g / kOBlocks;
        dqacc[j] = E::mfma(opnd[n], pb[u], dqacc[j]);
      }
    };
    [&]<int... n>(std::integer_sequence<int, n...>) {
      (fetch(Int<n>{}), ...);
    }(std::make_integer_sequence<int, kAheadM>{});
    [&]<int... n>(std::integer_sequence<int, n...>) {
      ((
           [&] {
             if constexpr (n + kAheadM < kMfma) fetch(Int<n + kAheadM>{});
             mfma(Int<n>{});
             __builtin_amdgcn_sched_barrier(0);
           }()),
       ...);
    }(std::make_integer_sequence<int, kMfma>{});
  };

  // V phase of key tile `tile`: dS^T = P^T (dP^T - D), P^T = exp2(c S^T - log2(e) L), with
  // P = 0 where the key is past the end or above the diagonal; rounded into pb.
  auto phase_v = [&](int tile) __attribute__((always_inline)) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int r0 = tile * kKeysT + kTileRows * hf;
      // entry i is key r0 + 4 half + off_i, off_i = 8 (i / 4) + i % 4
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = fmaf(sacc[hf][i], p.c, nlse);
      if ((r0 + kTileRows > slen) || (CAUSAL && r0 + kTileRows - 1 > qw0)) {
        // visible while off_i <= lim
        const int lim = (CAUSAL ? min(slen - 1, qrow) : slen - 1) - r0 - 4 * half;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = 8 * (i >> 2) + (i & 3);
          x[i] = off <= lim ? x[i] : -INFINITY;
        }
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int i = 8 * tt + 2 * w;
          const float d0 = __builtin_amdgcn_exp2f(x[i]) * (dpacc[hf][i] - del);
          const float d1 = __builtin_amdgcn_exp2f(x[i + 1]) * (dpacc[hf][i + 1] - del);
          pb[2 * hf + tt][w] = E::pack(d0, d1);
        }
    }
  };

  // Step t starts by issuing tile t + 1 (into the stage of tile t - 2, last read by the M(t-1)
  // of both groups in step t - 1) and ends by waiting for it (step t + 1 reads it); no wave
  // reads another's data, so the ring needs only the barrier that ends each step. The ring
  // stage is a loop variable. The loop runs t = 0 .. n_tiles: M(0) of either group adds
  // K(-1)^T dS^T(-1) = 0 (the stand-in stage is zero, pb starts at 0); M(n_tiles) of either
  // group only adds dQ(n_tiles - 1) (its S and dP chains read a stale stage and are not used).
  auto run = [&](auto grp_c) __attribute__((always_inline)) {
    constexpr bool G1 = decltype(grp_c)::value;
    int st = 0, st_prev = kRing - 1, st_next = 1;  // stages of tiles t, t - 1, t + 1
    for (int t = 0; t <= n_tiles; ++t) {
      if (t + 1 < n_tiles) issue(st_next);
      if constexpr (!G1) {
        phase_m(st, st_prev);
      } else {
        if (t >= 1) phase_v(t - 1);
      }
      if constexpr (D == 64) phase_sync();  // the two halves of a step (see above)
      if constexpr (!G1) {
        if (t < n_tiles) phase_v(t);
      } else {
        phase_m(st, st_prev);
      }
      if (t + 1 < n_tiles) wait_vmcnt<0>();  // tile t + 1
      phase_sync();
      st_prev = st;
      st = st_next;
      st_next = st_next == kRing - 1 ? 0 : st_next + 1;
    }
  };

  {
    // The K stage kRing - 1 stands in for tile -1 until tile kRing - 1 lands there: zeros, so
    // that dQ^T += K(-1)^T dS^T(-1) with dS^T(-1) = 0 adds 0.
    const u32x4 zero = u32x4{0, 0, 0, 0};
    for (int off = tid * 16; off < kTBytes; off += kThreads8 * 16)
      *reinterpret_cast<u32x4*>(smem + kK + (kRing - 1) * kTBytes + off) = zero;
  }
  if (n_tiles > 0) issue(0);
  // tile 0 and the resident operands complete; the empty asm makes the compiler's own load
  // tracking agree, so that it adds no memory waits inside the loop
  wait_vmcnt<0>();
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    qf[s] = (qf[s] & p.s_and) ^ p.s_xor;
    asm volatile("" : "+v"(qf[s]), "+v"(dof[s]));
  }
  __syncthreads();
  if (grp)
    run(std::true_type{});
  else
    run(std::false_type{});

  if (qrow < slen) {
    uint16_t* dqrow = p.dq + bidx * p.dq_sb + h * p.dq_sh + int64_t(seq0 + qrow) * p.dq_sn;
    store_rows<D, BF16>(dqrow, dqacc, p.scale, half);
  }
}

// ---------------------------------------------------------------------------------------
template <int D, bool BF16, bool CAUSAL, bool VARLEN>
hipError_t launch_bwd_typed(const BwdArgs& a, int groups, hipStream_t stream) {
  const int64_t rows = a.rows_delta;
  hipLaunchKernelGGL((fa_bwd_delta_kernel<D, BF16>), dim3(int((rows + 15) / 16)), dim3(256), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, BF16, CAUSAL, VARLEN>),
                     dim3(a.n_kblocks * a.heads_kv * groups), dim3(kThreads8), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fa_bwd_dq_kernel<D, BF16, CAUSAL, VARLEN>),
                     dim3(a.n_qblocks * a.heads_q * groups), dim3(kThreads8), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_bwd_mode(const BwdArgs& a, int groups, bool causal, bool varlen,
                           hipStream_t s) {
  if (causal)
    return varlen ? launch_bwd_typed<D, BF16, true, true>(a, groups, s)
                  : launch_bwd_typed<D, BF16, true, false>(a, groups, s);
  return varlen ? launch_bwd_typed<D, BF16, false, true>(a, groups, s)
                : launch_bwd_typed<D, BF16, false, false>(a, groups, s);
}

}  // namespace

fa_status launch_backward(const fa_bwd_params& p, void* stream, const char** hip_error) {
  BwdArgs a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.v = static_cast<const uint16_t*>(p.v);
  a.o = static_cast<const uint16_t*>(p.o);
  a.dout = static_cast<const uint16_t*>(p.dout);
  a.lse = p.lse;
  a.delta = p.delta;
  a.dq = static_cast<uint16_t*>(p.dq);
  a.dk = static_cast<uint16_t*>(p.dk);
  a.dv = static_cast<uint16_t*>(p.dv);
  a.cu_seqlens = p.cu_seqlens;
  a.q_sb = p.q_stride[0]; a.q_sh = p.q_stride[1]; a.q_sn = p.q_stride[2];
  a.k_sb = p.k_stride[0]; a.k_sh = p.k_stride[1]; a.k_sn = p.k_stride[2];
  a.v_sb = p.v_stride[0]; a.v_sh = p.v_stride[1]; a.v_sn = p.v_stride[2];
  a.o_sb = p.o_stride[0]; a.o_sh = p.o_stride[1]; a.o_sn = p.o_stride[2];
  a.do_sb = p.do_stride[0]; a.do_sh = p.do_stride[1]; a.do_sn = p.do_stride[2];
  a.dq_sb = p.dq_stride[0]; a.dq_sh = p.dq_stride[1]; a.dq_sn = p.dq_stride[2];
  a.dk_sb = p.dk_stride[0]; a.dk_sh = p.dk_stride[1]; a.dk_sn = p.dk_stride[2];
  a.dv_sb = p.dv_stride[0]; a.dv_sh = p.dv_stride[1]; a.dv_sn = p.dv_stride[2];
  a.seqlen = p.seqlen;
  a.heads_q = p.heads_q;
  a.heads_kv = p.heads_kv;
  a.group = p.heads_q / p.heads_kv;
  const bool varlen = p.cu_seqlens != nullptr;
  const int rows = varlen ? p.max_seqlen : p.seqlen;
  a.n_kblocks = (rows + 127) / 128;
  a.n_qblocks = (rows + 255) / 256;
  a.rows_delta = p.batch * p.heads_q * p.seqlen;
  a.nlse = p.delta + int64_t(a.rows_delta);
  a.c = float((p.scale == 0.f ? 1.0 : std::fabs(double(p.scale))) * 1.4426950408889634);
  a.s_and = p.scale == 0.f ? 0u : 0xFFFFFFFFu;
  a.s_xor = p.scale < 0.f ? 0x80008000u : 0u;
  a.scale = p.scale;
  const int groups = varlen ? p.num_seqs : p.batch;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool causal = p.causal != 0;
  hipError_t e;
  if (p.head_dim == 128)
    e = p.dtype == FA_BF16 ? launch_bwd_mode<128, true>(a, groups, causal, varlen, s)
                           : launch_bwd_mode<128, false>(a, groups, causal, varlen, s);
  else
    e = p.dtype == FA_BF16 ? launch_bwd_mode<64, true>(a, groups, causal, varlen, s)
                           : launch_bwd_mode<64, false>(a, groups, causal, varlen, s);
  if (e != hipSuccess) {
    *hip_error = hipGetErrorString(e);
    return FA_ERR_LAUNCH;
  }
  return FA_OK;
}

}  // namespace fa

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
//  * fa_bwd_delta_kernel: D = rowsum(dO * O) in fp32 (into the caller's delta buffer).
//  * fa_bwd_dkdv_kernel: one workgroup per 128 keys of a (batch entry or sequence, kv head).
//    Its 4 waves own 32 keys each, with K and V resident in registers as MFMA B operands and
//    dK^T, dV^T accumulating in fp32. 64-query tiles of Q and dO (of every query head that
//    shares the kv head) stream through double-buffered LDS. Per tile and wave:
//    S = Q K^T and dP = dO V^T (lane = key, as B operand), P and dS in registers, then
//    dV^T += dO^T P and dK^T += Q^T dS with dO^T, Q^T from transposing LDS reads.
//  * fa_bwd_dq_kernel: one workgroup per 128 queries of a (batch entry or sequence, query
//    head). Its 4 waves own 32 queries each, with Q^T and dO^T resident, and dQ^T
//    accumulating. 64-key tiles of K and V stream through LDS. Per tile and wave:
//    S^T = K Q^T and dP^T = V dO^T (lane = query), dS^T, then dQ^T += K^T dS^T.
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

constexpr int kOwn = 128;        // rows a workgroup owns: 4 waves x 32
constexpr int kTileRows = 64;    // rows of the streamed side per step
constexpr int kBwdThreads = 256;

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  float* delta;
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
  int32_t n_blocks;   // 128-row blocks per (batch entry or sequence)
  int32_t rows_delta; // batch * heads_q * seqlen
  float c;            // |scale| * log2(e), or log2(e) when scale == 0
  uint32_t s_and;     // 0 when scale == 0, else all ones (applied to the resident operand)
  uint32_t s_xor;     // 0x80008000 when scale < 0 (negates the resident operand exactly)
  float scale;        // the signed scale: dQ = scale dS K, dK = scale dS^T Q
};

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------------------
// D = rowsum(dO * O), fp32. 16 lanes per row, 8 (d = 128) or 4 (d = 64) elements per lane.
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
}

// ---------------------------------------------------------------------------------------
// Shared pieces of the two main kernels.

template <int D>
struct BwdGeo {
  static constexpr int kSteps = D / 16;       // head-dim steps of a contraction over D
  static constexpr int kOBlocks = D / 32;     // 32-wide head-dim blocks
  static constexpr int kBlocks = D / 8;       // 1 KB blocks per 64-row tile per layout
  static constexpr int kTileBytes = kBlocks * 1024;
  static constexpr int kPerWave = kBlocks / 4;  // blocks of one layout issued per wave
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
// dK, dV: one workgroup per 128 keys.
template <int D, bool BF16, bool CAUSAL, bool VARLEN>
__global__ __attribute__((amdgpu_flat_work_group_size(kBwdThreads, kBwdThreads),
                          amdgpu_waves_per_eu(1, 1)))
void fa_bwd_dkdv_kernel(const BwdArgs p) {
  using E = Elem<BF16>;
  using G = BwdGeo<D>;
  constexpr int kSteps = G::kSteps;
  constexpr int kOBlocks = G::kOBlocks;
  constexpr int kPer = G::kPerWave;
  // stage: Q operand | Q transposing | dO operand | dO transposing | LSE rows | D rows
  constexpr int kQop = 0, kQtr = G::kTileBytes, kDop = 2 * G::kTileBytes,
                kDtr = 3 * G::kTileBytes, kLse = 4 * G::kTileBytes, kDel = kLse + 1024;
  constexpr int kStage = kDel + 1024;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kStage];
  const uint32_t lds0 = lds_address(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;

  const int pairs = gridDim.x / p.n_blocks;
  const Item it = item_of(pairs, p.heads_kv, p.n_blocks, false);
  const int hk = it.h;
  int seq0 = 0, slen = p.seqlen, bidx = it.b;
  if (VARLEN) {
    seq0 = p.cu_seqlens[it.b];
    slen = p.cu_seqlens[it.b + 1] - seq0;
    bidx = 0;
  }
  const int k0 = it.blk * kOwn;
  if (k0 >= slen) return;  // uniform across the workgroup
  const int kw0 = k0 + 32 * wave;  // first key of this wave
  const int key = kw0 + (lane & 31);  // key of this lane (accumulator column)

  // resident K^T and V^T operands (K scaled by the sign of the scale, or zeroed for scale 0)
  u32x4 kf[kSteps], vf[kSteps];
  load_resident<D>(p.k + bidx * p.k_sb + hk * p.k_sh + int64_t(seq0) * p.k_sn, p.k_sn, kw0, slen,
                   lane, kf);
  load_resident<D>(p.v + bidx * p.v_sb + hk * p.v_sh + int64_t(seq0) * p.v_sn, p.v_sn, kw0, slen,
                   lane, vf);
#pragma unroll
  for (int s = 0; s < kSteps; ++s) kf[s] = (kf[s] & p.s_and) ^ p.s_xor;

  f32x16 dkacc[kOBlocks], dvacc[kOBlocks];
#pragma unroll
  for (int j = 0; j < kOBlocks; ++j) dkacc[j] = dvacc[j] = f32x16{};

  // query tiles: causal keys k0.. are seen by queries >= k0 only
  const int t_first = CAUSAL ? k0 / kTileRows : 0;
  const int n_qt = (slen + kTileRows - 1) / kTileRows;
  const int per_head = n_qt - t_first;
  const int n_steps = per_head * p.group;

  // per-lane source offsets of this wave's DMA blocks (rows of the tile, bytes)
  int op_off[kPer], tr_off[kPer], dop_off[kPer], dtr_off[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    int row, col;
    OperandLayout::row_col(wave * kPer + i, lane, kSteps, row, col);
    op_off[i] = int(row * p.q_sn * 2) + col * 2;
    dop_off[i] = int(row * p.do_sn * 2) + col * 2;
    TransposeLayout::row_col(wave * kPer + i, lane, kOBlocks, row, col);
    tr_off[i] = int(row * p.q_sn * 2) + col * 2;
    dtr_off[i] = int(row * p.do_sn * 2) + col * 2;
  }

  auto step_head = [&](int st) { return it.h * p.group + st / per_head; };
  auto step_tile = [&](int st) { return t_first + st % per_head; };

  // issue the loads of step st into stage ST
  auto issue = [&](auto stage, int st) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage)::value;
    const int h = step_head(st);
    const int r0 = step_tile(st) * kTileRows;
    const int rows = min(slen - r0, kTileRows);
    const uint16_t* qb = p.q + bidx * p.q_sb + h * p.q_sh + int64_t(seq0 + r0) * p.q_sn;
    const uint16_t* db = p.dout + bidx * p.do_sb + h * p.do_sh + int64_t(seq0 + r0) * p.do_sn;
    const u32x4 rq = make_rsrc(qb, int((rows - 1) * p.q_sn * 2) + D * 2);
    const u32x4 rd = make_rsrc(db, int((rows - 1) * p.do_sn * 2) + D * 2);
    const uint32_t base = lds0 + ST * kStage + wave * kPer * 1024;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      dma16(rq, base + kQop + i * 1024, op_off[i]);
      dma16(rq, base + kQtr + i * 1024, tr_off[i]);
      dma16(rd, base + kDop + i * 1024, dop_off[i]);
      dma16(rd, base + kDtr + i * 1024, dtr_off[i]);
    }
    if (wave < 2) {
      // 64 fp32 rows of LSE (wave 0) or D (wave 1): lanes 0..15 carry them, the rest read 0
      const int64_t row0 = (int64_t(bidx) * p.heads_q + h) * p.seqlen + seq0 + r0;
      const float* src = wave == 0 ? p.lse + row0 : p.delta + row0;
      dma16(make_rsrc(src, rows * 4), lds0 + ST * kStage + (wave == 0 ? kLse : kDel),
            lane * 16);
    }
  };

  auto compute = [&](auto stage, int st) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage)::value;
    const unsigned char* sb = smem + ST * kStage;
    const int r0 = step_tile(st) * kTileRows;
    // S = Q K^T and dP = dO V^T for the two 32-query halves of the tile
    f32x16 sacc[2], dpacc[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      sacc[qb] = f32x16{};
      dpacc[qb] = f32x16{};
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(sb + kQop + (qb * kSteps + s) * 1024 +
                                                        lane * 16);
        sacc[qb] = E::mfma(a, kf[s], sacc[qb]);
        const u32x4 g = *reinterpret_cast<const u32x4*>(sb + kDop + (qb * kSteps + s) * 1024 +
                                                        lane * 16);
        dpacc[qb] = E::mfma(g, vf[s], dpacc[qb]);
      }
    }
    // P = exp2(c S - log2e L) and dS = P (dP - D); entry i of half qb is query row
    // r0 + 32 qb + 8 (i / 4) + 4 half + i % 4
    u32x4 pp[2][2], pds[2][2];
    const bool edge = (r0 + kTileRows > slen) || (CAUSAL && r0 < kw0 + 31);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float lse[16], del[16];
      read_rows16(reinterpret_cast<const float*>(sb + kLse) + 32 * qb, half, lse);
      read_rows16(reinterpret_cast<const float*>(sb + kDel) + 32 * qb, half, del);
      float pv[16], dsv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qrow = r0 + 32 * qb + 8 * (i >> 2) + 4 * half + (i & 3);
        float x = fmaf(sacc[qb][i], p.c, -lse[i] * kLog2e);
        if (edge) {
          const bool ok = qrow < slen && key < slen && (!CAUSAL || key <= qrow);
          x = ok ? x : -INFINITY;
        }
        pv[i] = __builtin_amdgcn_exp2f(x);
        dsv[i] = pv[i] * (dpacc[qb][i] - del[i]);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pp[qb][tt][e] = E::pack(pv[8 * tt + 2 * e], pv[8 * tt + 2 * e + 1]);
          pds[qb][tt][e] = E::pack(dsv[8 * tt + 2 * e], dsv[8 * tt + 2 * e + 1]);
        }
    }
    // dV^T += dO^T P and dK^T += Q^T dS, contracting over the tile's 64 queries
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int j = 0; j < kOBlocks; ++j) {
          const int blk = ((2 * qb + tt) * kOBlocks + j) * 1024;
          const u32x2 dlo = E::read_tr(sb + kDtr + blk + lane * 8);
          const u32x2 dhi = E::read_tr(sb + kDtr + blk + 512 + lane * 8);
          dvacc[j] = E::mfma(u32x4{dlo[0], dlo[1], dhi[0], dhi[1]}, pp[qb][tt], dvacc[j]);
          const u32x2 qlo = E::read_tr(sb + kQtr + blk + lane * 8);
          const u32x2 qhi = E::read_tr(sb + kQtr + blk + 512 + lane * 8);
          dkacc[j] = E::mfma(u32x4{qlo[0], qlo[1], qhi[0], qhi[1]}, pds[qb][tt], dkacc[j]);
        }
  };

  auto sync = [&]() __attribute__((always_inline)) {
    wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __syncthreads();
  };

  if (n_steps > 0) {
    issue(Int<0>{}, 0);
    sync();
    for (int st = 0; st < n_steps; st += 2) {
      if (st + 1 < n_steps) issue(Int<1>{}, st + 1);
      compute(Int<0>{}, st);
      sync();
      if (st + 1 < n_steps) {
        if (st + 2 < n_steps) issue(Int<0>{}, st + 2);
        compute(Int<1>{}, st + 1);
        sync();
      }
    }
  }

  if (key < slen) {
    uint16_t* dkrow = p.dk + bidx * p.dk_sb + hk * p.dk_sh + int64_t(seq0 + key) * p.dk_sn;
    uint16_t* dvrow = p.dv + bidx * p.dv_sb + hk * p.dv_sh + int64_t(seq0 + key) * p.dv_sn;
    store_rows<D, BF16>(dkrow, dkacc, p.scale, half);
    store_rows<D, BF16>(dvrow, dvacc, 1.f, half);
  }
}

// ---------------------------------------------------------------------------------------
// dQ: one workgroup per 128 queries.
template <int D, bool BF16, bool CAUSAL, bool VARLEN>
__global__ __attribute__((amdgpu_flat_work_group_size(kBwdThreads, kBwdThreads),
                          amdgpu_waves_per_eu(1, 1)))
void fa_bwd_dq_kernel(const BwdArgs p) {
  using E = Elem<BF16>;
  using G = BwdGeo<D>;
  constexpr int kSteps = G::kSteps;
  constexpr int kOBlocks = G::kOBlocks;
  constexpr int kPer = G::kPerWave;
  // stage: K operand | K transposing | V operand
  constexpr int kKop = 0, kKtr = G::kTileBytes, kVop = 2 * G::kTileBytes;
  constexpr int kStage = 3 * G::kTileBytes;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kStage];
  const uint32_t lds0 = lds_address(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;

  const int pairs = gridDim.x / p.n_blocks;
  const Item it = item_of(pairs, p.heads_q, p.n_blocks, CAUSAL);
  const int h = it.h;
  const int hk = h / p.group;
  int seq0 = 0, slen = p.seqlen, bidx = it.b;
  if (VARLEN) {
    seq0 = p.cu_seqlens[it.b];
    slen = p.cu_seqlens[it.b + 1] - seq0;
    bidx = 0;
  }
  const int q0 = it.blk * kOwn;
  if (q0 >= slen) return;  // uniform across the workgroup
  const int qw0 = q0 + 32 * wave;     // first query of this wave
  const int qrow = qw0 + (lane & 31);  // query of this lane (accumulator column)

  // resident Q^T (sign and zero of the scale applied) and dO^T operands
  u32x4 qf[kSteps], dof[kSteps];
  load_resident<D>(p.q + bidx * p.q_sb + h * p.q_sh + int64_t(seq0) * p.q_sn, p.q_sn, qw0, slen,
                   lane, qf);
  load_resident<D>(p.dout + bidx * p.do_sb + h * p.do_sh + int64_t(seq0) * p.do_sn, p.do_sn, qw0,
                   slen, lane, dof);
#pragma unroll
  for (int s = 0; s < kSteps; ++s) qf[s] = (qf[s] & p.s_and) ^ p.s_xor;
  float lse2 = 0.f, del = 0.f;
  if (qrow < slen) {
    const int64_t r = (int64_t(bidx) * p.heads_q + h) * p.seqlen + seq0 + qrow;
    lse2 = p.lse[r] * kLog2e;
    del = p.delta[r];
  }

  f32x16 dqacc[kOBlocks];
#pragma unroll
  for (int j = 0; j < kOBlocks; ++j) dqacc[j] = f32x16{};

  const int kv_end = CAUSAL ? min(slen, q0 + kOwn) : slen;
  const int n_tiles = (kv_end + kTileRows - 1) / kTileRows;

  int op_off_k[kPer], tr_off_k[kPer], op_off_v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    int row, col;
    OperandLayout::row_col(wave * kPer + i, lane, kSteps, row, col);
    op_off_k[i] = int(row * p.k_sn * 2) + col * 2;
    op_off_v[i] = int(row * p.v_sn * 2) + col * 2;
    TransposeLayout::row_col(wave * kPer + i, lane, kOBlocks, row, col);
    tr_off_k[i] = int(row * p.k_sn * 2) + col * 2;
  }
  const uint16_t* kbase = p.k + bidx * p.k_sb + hk * p.k_sh + int64_t(seq0) * p.k_sn;
  const uint16_t* vbase = p.v + bidx * p.v_sb + hk * p.v_sh + int64_t(seq0) * p.v_sn;

  auto issue = [&](auto stage, int tile) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage)::value;
    const int r0 = tile * kTileRows;
    const int rows = min(slen - r0, kTileRows);
    const u32x4 rk = make_rsrc(kbase + int64_t(r0) * p.k_sn, int((rows - 1) * p.k_sn * 2) + D * 2);
    const u32x4 rv = make_rsrc(vbase + int64_t(r0) * p.v_sn, int((rows - 1) * p.v_sn * 2) + D * 2);
    const uint32_t base = lds0 + ST * kStage + wave * kPer * 1024;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      dma16(rk, base + kKop + i * 1024, op_off_k[i]);
      dma16(rk, base + kKtr + i * 1024, tr_off_k[i]);
      dma16(rv, base + kVop + i * 1024, op_off_v[i]);
    }
  };

  auto compute = [&](auto stage, int tile) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage)::value;
    const unsigned char* sb = smem + ST * kStage;
    const int r0 = tile * kTileRows;
    // S^T = K Q^T and dP^T = V dO^T for the two 32-key halves of the tile
    f32x16 sacc[2], dpacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
      dpacc[kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(sb + kKop + (kb * kSteps + s) * 1024 +
                                                        lane * 16);
        sacc[kb] = E::mfma(a, qf[s], sacc[kb]);
        const u32x4 g = *reinterpret_cast<const u32x4*>(sb + kVop + (kb * kSteps + s) * 1024 +
                                                        lane * 16);
        dpacc[kb] = E::mfma(g, dof[s], dpacc[kb]);
      }
    }
    // entry i of key half kb is key r0 + 32 kb + 8 (i / 4) + 4 half + i % 4
    const bool edge = (r0 + kTileRows > slen) || (CAUSAL && r0 + kTileRows - 1 > qw0);
    u32x4 pds[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float dsv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = r0 + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
        float x = fmaf(sacc[kb][i], p.c, -lse2);
        if (edge) {
          const bool ok = key < slen && (!CAUSAL || key <= qrow);
          x = ok ? x : -INFINITY;
        }
        dsv[i] = __builtin_amdgcn_exp2f(x) * (dpacc[kb][i] - del);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pds[kb][tt][e] = E::pack(dsv[8 * tt + 2 * e], dsv[8 * tt + 2 * e + 1]);
    }
    // dQ^T += K^T dS^T, contracting over the tile's 64 keys
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int j = 0; j < kOBlocks; ++j) {
          const int blk = ((2 * kb + tt) * kOBlocks + j) * 1024;
          const u32x2 lo = E::read_tr(sb + kKtr + blk + lane * 8);
          const u32x2 hi = E::read_tr(sb + kKtr + blk + 512 + lane * 8);
          dqacc[j] = E::mfma(u32x4{lo[0], lo[1], hi[0], hi[1]}, pds[kb][tt], dqacc[j]);
        }
  };

  auto sync = [&]() __attribute__((always_inline)) {
    wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __syncthreads();
  };

  issue(Int<0>{}, 0);
  sync();
  for (int t = 0; t < n_tiles; t += 2) {
    if (t + 1 < n_tiles) issue(Int<1>{}, t + 1);
    compute(Int<0>{}, t);
    sync();
    if (t + 1 < n_tiles) {
      if (t + 2 < n_tiles) issue(Int<0>{}, t + 2);
      compute(Int<1>{}, t + 1);
      sync();
    }
  }

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
                     dim3(a.n_blocks * a.heads_kv * groups), dim3(kBwdThreads), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fa_bwd_dq_kernel<D, BF16, CAUSAL, VARLEN>),
                     dim3(a.n_blocks * a.heads_q * groups), dim3(kBwdThreads), 0, stream, a);
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
  a.n_blocks = (rows + kOwn - 1) / kOwn;
  a.rows_delta = p.batch * p.heads_q * p.seqlen;
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

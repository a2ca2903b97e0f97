// FlashAttention forward kernels for gfx950 (CDNA4): exact softmax(scale * Q K^T) V with
// online-softmax rescaling; the N x N scores and probabilities never leave registers.
//
// Algorithm: "Flash Attention" notes (14cs17), section "Flash Attention Algorithm" (for each
// query block: load Q_i, start O_i = 0, l_i = 0, m_i = -inf, stream K_j/V_j blocks through
// on-chip memory, form S_ij = Q_i K_j^T, update (m_i, l_i, O_i) by the online softmax of
// Theorem 2, write O_i), with FlashAttention-2's choices from the section "Flash Attention 2
// Improvements": the grid runs over query blocks, and O is normalised by l once at the end.
//
// Mapping onto the hardware (one workgroup = one 128-row query block of one head):
//  * 4 waves of 64 lanes; wave w owns query rows [32w, 32w + 32) of the block, so waves never
//    reduce across each other.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_{bf16,f16}: the
//    A operand is 32 keys x 16 head-dims read from LDS, the B operand is Q^T held in VGPRs for
//    the whole kernel. In the 32x32 accumulator lane L holds query column L % 32 and 16 keys,
//    so the row maximum and row sum are in-lane plus one exchange between the two half-waves,
//    and the rescale of O by exp2(m_old - m_new) is a per-lane multiply.
//  * The exponentiated scores, rounded to the input type, are used directly as the B operand
//    of O^T += V^T P^T; the matching V^T operand comes from row-major V tiles in LDS through
//    the gfx950 transposing read ds_read_b64_tr_b16, with the key order permuted to match the
//    accumulator layout (keys {4h..4h+3, 8+4h..8+4h+3} of each 16-key step for half-wave h).
//  * K and V tiles of 64 keys are double-buffered in LDS, filled from buffer loads whose
//    out-of-range part reads as zero (ragged tails need no branches). Rows are padded so both
//    the 128-bit K reads and the transposing V reads are free of bank conflicts, and every LDS
//    address in the loop is a per-lane base plus an immediate.
//  * The reference maximum of the online softmax is raised lazily (only when a tile's maximum
//    exceeds it by more than 2^8), so the rescale of O is rare after the first tiles.
//  * exp is exp2 with scale * log2(e) folded into one FMA per score.
//  * Causal blocks stop at the diagonal; only diagonal and ragged-tail tiles are masked; a
//    wave whose rows are all above a tile skips that tile.
//  * The workgroup index is remapped so that the blocks of one head run on one XCD (its L2
//    serves the K/V re-reads), heaviest causal blocks first.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "fa.h"
#include "fa_launch.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __fp16 f16x4_tr __attribute__((__vector_size__(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T) __attribute__((address_space(3))) T*

constexpr int kBlockM = 256;  // query rows per workgroup (B_r): 8 waves x 32 rows
constexpr int kBlockN = 64;   // keys per K/V tile (B_c)
constexpr int kThreads = 512;

struct KernelArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int32_t* cu_seqlens;
  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int32_t seqlen;     // tokens per batch entry (packed total for varlen)
  int32_t heads_q;
  int32_t group;      // heads_q / heads_kv
  int32_t n_qblocks;  // query blocks per (batch entry or sequence, head)
  float c;            // |scale| * log2(e), or log2(e) when scale == 0
  uint32_t q_and;     // 0 when scale == 0 (all scores are exactly 0), else all ones
  uint32_t q_xor;     // 0x80008000 when scale < 0: Q is negated exactly and c stays positive
  int32_t xcd_group;  // 1: keep the blocks of a head on one XCD
};

template <bool BF16>
struct Elem;

template <>
struct Elem<true> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ u32x2 read_tr(const uint16_t* lds) {
    bf16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_PTR(bf16x4))(lds));
    return __builtin_bit_cast(u32x2, r);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
  }
};

template <>
struct Elem<false> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ u32x2 read_tr(const uint16_t* lds) {
    f16x4_tr r = __builtin_amdgcn_ds_read_tr16_b64_v4f16((LDS_PTR(f16x4_tr))(lds));
    return __builtin_bit_cast(u32x2, r);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
  }
};

// LDS tile geometry. Rows are padded instead of swizzled so that every LDS address in the
// loop is a per-lane base plus a compile-time immediate:
//  * K rows are read as 16-byte chunks by 32 consecutive rows (the MFMA A operand); a skew of
//    16 bytes per row puts 16 consecutive rows in 16 distinct 16-byte bank groups;
//  * V rows are read by the transposing read, 4 consecutive rows x 64 bytes per 32 lanes; a
//    skew of 64 bytes per row spreads those 4 rows over all four 64-byte bank groups.
template <int D>
struct Tile {
  static constexpr int kPitchK = D + 8;    // elements
  static constexpr int kPitchV = D + 32;   // elements
  static constexpr int kBytesK = kBlockN * kPitchK * 2;
  static constexpr int kBytesV = kBlockN * kPitchV * 2;
  static constexpr int kLdsBytes = 2 * (kBytesK + kBytesV);  // two stages of K and V
};

// Raw buffer resource over [base, base + bytes): loads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

template <int N>
using Int = std::integral_constant<int, N>;

// Running maxima grow lazily: O and l are rescaled only when some row's tile maximum exceeds
// the reference maximum by more than this many powers of two. Any reference maximum gives the
// same O = O~ / l and LSE = m + log2(l); this bound keeps exp2(s - m) <= 2^8.
constexpr float kLazyRescale = 8.0f;

template <int D, bool BF16, bool CAUSAL, bool VARLEN>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(2, 2)))
void fa_fwd_kernel(const KernelArgs p) {
  using E = Elem<BF16>;
  using T = Tile<D>;
  constexpr int kChunks = D / 8;                        // 16-byte chunks per row
  constexpr int kSteps = D / 16;                        // k-steps of the S^T product
  constexpr int kOBlocks = D / 32;                      // 32-wide head-dim blocks of O^T
  constexpr int kGroupThreads = kThreads / 2;           // one wave group stages one tensor
  constexpr int kLoads = kBlockN * kChunks / kGroupThreads;  // 16-byte loads per thread
  constexpr int kRowsPerPass = kGroupThreads / kChunks;

  __shared__ __attribute__((aligned(16))) unsigned char smem[T::kLdsBytes];
  unsigned char* lds_k = smem;                     // stage s at s * kBytesK
  unsigned char* lds_v = smem + 2 * T::kBytesK;    // stage s at s * kBytesV

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int grp = wave >> 2;   // wave group: 0 stages K tiles, 1 stages V tiles
  const int half = lane >> 5;  // which 8-element half of each 16-wide k step this lane feeds
  const int lq = lane & 31;    // query column owned by this lane

  // ---- work item: (query block, head, batch entry / sequence) -------------------------
  const int total = gridDim.x;
  int item = blockIdx.x;
  if (p.xcd_group && (total & 7) == 0) {
    // Workgroups are dealt to the 8 XCDs round-robin; give XCD x a contiguous range.
    item = (item & 7) * (total >> 3) + (item >> 3);
  }
  int bh, t;
  if (VARLEN) {
    // Heaviest blocks first across all sequences and heads (lengths differ per sequence).
    const int pairs = total / p.n_qblocks;
    t = item / pairs;
    bh = item - t * pairs;
  } else {
    bh = item / p.n_qblocks;
    t = item - bh * p.n_qblocks;
  }
  const int qblock = CAUSAL ? (p.n_qblocks - 1 - t) : t;
  const int b = bh / p.heads_q;
  const int h = bh - b * p.heads_q;
  int seq0 = 0, slen = p.seqlen, bidx = b;
  if (VARLEN) {
    seq0 = p.cu_seqlens[b];
    slen = p.cu_seqlens[b + 1] - seq0;
    bidx = 0;
  }
  const int q0 = qblock * kBlockM;
  if (q0 >= slen) return;  // uniform across the workgroup, before any barrier
  const int hk = h / p.group;

  const uint16_t* qb = p.q + bidx * p.q_sb + h * p.q_sh + int64_t(seq0) * p.q_sn;
  const uint16_t* kbase = p.k + bidx * p.k_sb + hk * p.k_sh + int64_t(seq0) * p.k_sn;
  const uint16_t* vbase = p.v + bidx * p.v_sb + hk * p.v_sh + int64_t(seq0) * p.v_sn;

  const int kv_end = CAUSAL ? min(slen, q0 + kBlockM) : slen;
  const int n_tiles = (kv_end + kBlockN - 1) / kBlockN;

  // ---- Q^T fragments (B operand), resident for the whole kernel -----------------------
  // The two waves sharing a SIMD (w and w + 4) take neighbouring 32-row slices, so both
  // groups reach the causal diagonal at nearly the same tile.
  const int wrow0 = q0 + 32 * (2 * (wave & 3) + grp);  // first query row of this wave
  const int qrow = wrow0 + lq;                          // query row of this lane
  u32x4 qf[kSteps];
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    if (qrow < slen) {
      qf[s] = *reinterpret_cast<const u32x4*>(qb + int64_t(qrow) * p.q_sn + s * 16 + half * 8);
      qf[s] = (qf[s] & p.q_and) ^ p.q_xor;
    } else {
      qf[s] = u32x4{0, 0, 0, 0};
    }
  }

  // ---- K/V staging: group 0 stages K tiles, group 1 stages V tiles ----------------------
  // buffer loads (zero past the sequence end) -> registers -> LDS (padded rows)
  const int gt = tid & (kGroupThreads - 1);
  const int ld_row = gt / kChunks;
  const int ld_ch = gt % kChunks;
  const uint16_t* ld_base = grp ? vbase : kbase;
  const int64_t ld_sn = grp ? p.v_sn : p.k_sn;
  int ld_voff[kLoads];
#pragma unroll
  for (int r = 0; r < kLoads; ++r)
    ld_voff[r] = int((ld_row + r * kRowsPerPass) * ld_sn * 2) + ld_ch * 16;
  unsigned char* st_base = grp ? lds_v + ld_row * T::kPitchV * 2 + ld_ch * 16
                               : lds_k + ld_row * T::kPitchK * 2 + ld_ch * 16;
  const int st_pass = (grp ? T::kPitchV : T::kPitchK) * 2 * kRowsPerPass;
  const int st_stage = grp ? T::kBytesV : T::kBytesK;

  u32x4 stg[kLoads];
  // issue the loads of tile `tile` of this group's tensor
  auto gload = [&](int tile) __attribute__((always_inline)) {
    const int key0 = tile * kBlockN;
    const int rows = min(slen - key0, kBlockN);  // rows of this tile inside the sequence
    const int bytes = int((rows - 1) * ld_sn * 2) + D * 2;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(ld_base + int64_t(key0) * ld_sn, bytes);
#pragma unroll
    for (int r = 0; r < kLoads; ++r)
      stg[r] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, ld_voff[r], 0, 0);
  };
  // write the staged tile into its LDS stage
  auto lds_put = [&](int tile) __attribute__((always_inline)) {
    unsigned char* dst = st_base + (tile & 1) * st_stage;
#pragma unroll
    for (int r = 0; r < kLoads; ++r) *reinterpret_cast<u32x4*>(dst + r * st_pass) = stg[r];
  };

  // Per-lane LDS read bases; everything else in the M phase is an immediate offset.
  //  K (A operand of S^T): row lq of each 32-key half, 16-byte chunk (2s + half).
  const unsigned char* rd_k = lds_k + lq * T::kPitchK * 2 + half * 16;
  //  V (transposing read): the 16 lanes of a group cover 4 consecutive keys x 16 head-dims.
  const int sub = lane & 15;
  const unsigned char* rd_v = lds_v + (4 * half + (sub >> 2)) * T::kPitchV * 2 +
                              (16 * ((lane >> 4) & 1) + 4 * (sub & 3)) * 2;

  float m_run = -INFINITY;  // reference maximum of scaled scores, log2 units (Theorem 2's m)
  float l_run = 0.f;        // running sum of this half-wave's keys (Theorem 2's l)
  f32x16 oacc[kOBlocks];    // unnormalised O^T: lane holds head-dims of its query column
#pragma unroll
  for (int j = 0; j < kOBlocks; ++j) oacc[j] = f32x16{};
  f32x16 sacc[2];           // S^T of the tile between its M and V phases
  u32x4 pb[2][2];           // P^T of the previous tile, in the input type (B operands)
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) pb[kb][tt] = u32x4{0, 0, 0, 0};

  // S^T = K Q^T, two 32-key halves (A: K rows from LDS stage KS).
  auto s_mfma = [&](auto ks, int kb, int s) __attribute__((always_inline)) {
    constexpr int KS = decltype(ks)::value;
    const u32x4 a = *reinterpret_cast<const u32x4*>(rd_k + KS * T::kBytesK +
                                                   kb * 32 * T::kPitchK * 2 + s * 32);
    sacc[kb] = E::mfma(a, qf[s], s == 0 ? f32x16{} : sacc[kb]);
  };
  // O^T += V^T P^T for head-dim block j, key half kb, 16-key step tt (V from stage VS).
  // The 16 lanes of a group receive head-dim column (lane % 32) of four consecutive keys per
  // transposing read; keys {16t+4h+0..3, 16t+8+4h+0..3} form the 8-element k slice of
  // half-wave h, matching the accumulator rows of P^T.
  auto pv_mfma = [&](auto vs, int j, int kb, int tt) __attribute__((always_inline)) {
    constexpr int VS = decltype(vs)::value;
    const unsigned char* base =
        rd_v + VS * T::kBytesV + (kb * 32 + 16 * tt) * T::kPitchV * 2 + j * 64;
    const u32x2 lo = E::read_tr(reinterpret_cast<const uint16_t*>(base));
    const u32x2 hi = E::read_tr(reinterpret_cast<const uint16_t*>(base + 8 * T::kPitchV * 2));
    oacc[j] = E::mfma(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb[kb][tt], oacc[j]);
  };

  // M phase (matrix cores), straight-line: S of tile p from K stage KS, and P V of tile p - 1
  // from V stage 1 - KS. Before the first tile P is zero and V stage 1 holds zeros; after the
  // last tile the S result is never used.
  auto phase_m = [&](auto ks) __attribute__((always_inline)) {
    constexpr int KS = decltype(ks)::value;
    constexpr int kS = 2 * kSteps;     // S MFMAs per tile
    constexpr int kPv = 4 * kOBlocks;  // PV MFMAs per tile
    __builtin_amdgcn_s_setprio(1);  // the wave feeding the matrix cores issues first
#pragma unroll
    for (int i = 0; i < (kS > kPv ? kS : kPv); ++i) {
      if (i < kS) s_mfma(Int<KS>{}, i / kSteps, i % kSteps);
      if (i < kPv) pv_mfma(Int<1 - KS>{}, i / 4, (i / 2) & 1, i & 1);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // V phase (vector units): online softmax of S_p (Theorem 2) into P_p, plus this group's
  // share of the K/V staging: write tile p + 1 into LDS, start loading tile p + 2.
  // Keys this wave cannot see (past the sequence end, above the diagonal) get P = 0.
  auto phase_v = [&](int tile) __attribute__((always_inline)) {
    if (tile >= 0 && tile < n_tiles) {
      const int key0 = tile * kBlockN;
      const bool edge = (key0 + kBlockN > slen) || (CAUSAL && key0 + kBlockN - 1 > wrow0);
      if (edge) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
            const bool ok = key < slen && (!CAUSAL || key <= qrow);
            sacc[kb][i] = ok ? sacc[kb][i] : -INFINITY;
          }
        }
      }
      float mx = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      if (__builtin_amdgcn_ballot_w64(mx * p.c > m_run + kLazyRescale)) {
        const float m_new = fmaxf(m_run, fmaxf(mx, __shfl_xor(mx, 32)) * p.c);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first tile
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int j = 0; j < kOBlocks; ++j) oacc[j] *= alpha;
      }
      const float neg_m = -m_run;
      float rsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], p.c, neg_m));
          sacc[kb][i] = e;
          rsum += e;
        }
      l_run += rsum;
      // B operand of step tt of key half kb is accumulator entries 8tt .. 8tt+7.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pb[kb][tt][e] = E::pack(sacc[kb][8 * tt + 2 * e], sacc[kb][8 * tt + 2 * e + 1]);
    }
    if (tile + 1 < n_tiles) lds_put(tile + 1);
    if (tile + 2 < n_tiles) gload(tile + 2);
  };

  // Phase boundary: a workgroup barrier that the instruction scheduler may not move
  // register-only work across (a plain barrier orders memory operations only).
  auto phase_sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- ping-pong schedule --------------------------------------------------------------
  // Slot 2p:   group 0 runs M(p),   group 1 runs V(p - 1)
  // Slot 2p+1: group 0 runs V(p),   group 1 runs M(p)
  // so on every SIMD one wave feeds the matrix cores while the other runs the softmax.
  // K_p is read in slots 2p and 2p+1 (stage p & 1) and written by group 0 in slot 2p - 1;
  // V_p is read in slots 2p+2 and 2p+3 (stage p & 1) and written by group 1 in slot 2p.
  // Both groups execute 2 (n_tiles + 1) barriers after the prologue's one.
  {
    // stage 1 of K and V starts as zeros (it is read before it is first written)
    const u32x4 zero = u32x4{0, 0, 0, 0};
    for (int off = tid * 16; off < T::kBytesK; off += kThreads * 16)
      *reinterpret_cast<u32x4*>(lds_k + T::kBytesK + off) = zero;
    for (int off = tid * 16; off < T::kBytesV; off += kThreads * 16)
      *reinterpret_cast<u32x4*>(lds_v + T::kBytesV + off) = zero;
  }
  gload(0);
  if (grp == 0) {
    lds_put(0);
    if (n_tiles > 1) gload(1);
  }
  __syncthreads();
  if (grp == 0) {
    for (int tile = 0; tile <= n_tiles; tile += 2) {
      phase_m(Int<0>{});
      phase_sync();
      phase_v(tile);
      phase_sync();
      if (tile + 1 <= n_tiles) {
        phase_m(Int<1>{});
        phase_sync();
        phase_v(tile + 1);
        phase_sync();
      }
    }
  } else {
    for (int tile = 0; tile <= n_tiles; tile += 2) {
      phase_v(tile - 1);
      phase_sync();
      phase_m(Int<0>{});
      phase_sync();
      if (tile + 1 <= n_tiles) {
        phase_v(tile);
        phase_sync();
        phase_m(Int<1>{});
        phase_sync();
      }
    }
  }

  // ---- epilogue: O = O~ / l, LSE = ln(l) + m; both half-waves hold partial sums --------
  if (wrow0 >= slen) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qrow < slen) {
    const float inv = 1.f / l_tot;
    uint16_t* orow = p.o + bidx * p.o_sb + h * p.o_sh + int64_t(seq0 + qrow) * p.o_sn;
#pragma unroll
    for (int j = 0; j < kOBlocks; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = j * 32 + 8 * g + 4 * half;
        u32x2 w;
        w[0] = E::pack(oacc[j][4 * g + 0] * inv, oacc[j][4 * g + 1] * inv);
        w[1] = E::pack(oacc[j][4 * g + 2] * inv, oacc[j][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
    }
    if (half == 0) {
      const float lse2 = m_run + __builtin_amdgcn_logf(l_tot);  // log2 units
      p.lse[(int64_t(bidx) * p.heads_q + h) * p.seqlen + seq0 + qrow] = lse2 * 0.69314718055994531f;
    }
  }
}

template <int D, bool BF16, bool CAUSAL, bool VARLEN>
hipError_t launch_typed(const KernelArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((fa_fwd_kernel<D, BF16, CAUSAL, VARLEN>), dim3(grid), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_mode(const KernelArgs& a, int grid, bool causal, bool varlen,
                       hipStream_t s) {
  if (causal)
    return varlen ? launch_typed<D, BF16, true, true>(a, grid, s)
                  : launch_typed<D, BF16, true, false>(a, grid, s);
  return varlen ? launch_typed<D, BF16, false, true>(a, grid, s)
                : launch_typed<D, BF16, false, false>(a, grid, s);
}

}  // namespace

fa_status launch_forward(const fa_fwd_params& p, void* stream, const char** hip_error) {
  KernelArgs a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.v = static_cast<const uint16_t*>(p.v);
  a.o = static_cast<uint16_t*>(p.o);
  a.lse = p.lse;
  a.cu_seqlens = p.cu_seqlens;
  a.q_sb = p.q_stride[0]; a.q_sh = p.q_stride[1]; a.q_sn = p.q_stride[2];
  a.k_sb = p.k_stride[0]; a.k_sh = p.k_stride[1]; a.k_sn = p.k_stride[2];
  a.v_sb = p.v_stride[0]; a.v_sh = p.v_stride[1]; a.v_sn = p.v_stride[2];
  a.o_sb = p.o_stride[0]; a.o_sh = p.o_stride[1]; a.o_sn = p.o_stride[2];
  a.seqlen = p.seqlen;
  a.heads_q = p.heads_q;
  a.group = p.heads_q / p.heads_kv;
  const bool varlen = p.cu_seqlens != nullptr;
  const int rows = varlen ? p.max_seqlen : p.seqlen;
  a.n_qblocks = (rows + kBlockM - 1) / kBlockM;
  const double c = (p.scale == 0.f ? 1.0 : std::fabs(double(p.scale))) * 1.4426950408889634;
  a.c = float(c);
  a.q_and = p.scale == 0.f ? 0u : 0xFFFFFFFFu;
  a.q_xor = p.scale < 0.f ? 0x80008000u : 0u;
  a.xcd_group = varlen ? 0 : 1;
  const int groups = varlen ? p.num_seqs : p.batch;
  const int grid = a.n_qblocks * p.heads_q * groups;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool causal = p.causal != 0;
  hipError_t e;
  if (p.head_dim == 128)
    e = p.dtype == FA_BF16 ? launch_mode<128, true>(a, grid, causal, varlen, s)
                           : launch_mode<128, false>(a, grid, causal, varlen, s);
  else
    e = p.dtype == FA_BF16 ? launch_mode<64, true>(a, grid, causal, varlen, s)
                           : launch_mode<64, false>(a, grid, causal, varlen, s);
  if (e != hipSuccess) {
    *hip_error = hipGetErrorString(e);
    return FA_ERR_LAUNCH;
  }
  return FA_OK;
}

}  // namespace fa

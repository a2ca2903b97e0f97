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
//  * K and V tiles of 64 keys are double-buffered in LDS. Rows are 16-byte-chunk XOR swizzled
//    so that both the 128-bit K reads and the transposing V reads spread over the banks.
//  * exp is exp2 with scale * log2(e) folded into one FMA per score.
//  * Causal blocks stop at the diagonal; only diagonal and ragged-tail tiles are masked; a
//    wave whose rows are all above a tile skips that tile.
//  * The workgroup index is remapped so that the blocks of one head run on one XCD (its L2
//    serves the K/V re-reads), heaviest causal blocks first.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

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

constexpr int kBlockM = 128;  // query rows per workgroup (B_r)
constexpr int kBlockN = 64;   // keys per K/V tile (B_c)
constexpr int kThreads = 256;

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

// Physical 16-byte chunk of logical chunk `ch` in LDS row `row`.
template <int D>
__device__ __forceinline__ int swizzle(int row, int ch) {
  if constexpr (D == 128) {
    return ch ^ (((row & 3) << 2) | ((row >> 2) & 3));
  } else {
    return ch ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
  }
}

template <int D>
__device__ __forceinline__ int lds_offset(int row, int col) {  // in elements
  return row * D + (swizzle<D>(row, col >> 3) << 3) + (col & 7);
}

template <int D, bool BF16, bool CAUSAL, bool VARLEN>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(2, 2)))
void fa_fwd_kernel(const KernelArgs p) {
  using E = Elem<BF16>;
  constexpr int kChunks = D / 8;                       // 16-byte chunks per row
  constexpr int kSteps = D / 16;                       // k-steps of the S^T product
  constexpr int kOBlocks = D / 32;                     // 32-wide head-dim blocks of O^T
  constexpr int kLoads = kBlockN * kChunks / kThreads; // 16-byte loads per thread per tensor
  constexpr int kTile = kBlockN * D;                   // elements per K (or V) tile

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
  const int wrow0 = q0 + wave * 32;  // first query row of this wave
  const int qrow = wrow0 + lq;       // query row of this lane
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

  // ---- K/V tile staging: global -> registers -> LDS (swizzled) ------------------------
  u32x4 kr[kLoads], vr[kLoads];
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int id = r * kThreads + tid;
      const int row = id / kChunks, ch = id % kChunks;
      const int key = tile * kBlockN + row;
      if (key < slen) {
        kr[r] = *reinterpret_cast<const u32x4*>(kbase + int64_t(key) * p.k_sn + ch * 8);
        vr[r] = *reinterpret_cast<const u32x4*>(vbase + int64_t(key) * p.v_sn + ch * 8);
      } else {
        kr[r] = u32x4{0, 0, 0, 0};  // zero rows: masked scores, and no NaN from stale V
        vr[r] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* ks = smem + buf * 2 * kTile;
    uint16_t* vs = ks + kTile;
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int id = r * kThreads + tid;
      const int row = id / kChunks, ch = id % kChunks;
      const int off = row * D + (swizzle<D>(row, ch) << 3);
      *reinterpret_cast<u32x4*>(ks + off) = kr[r];
      *reinterpret_cast<u32x4*>(vs + off) = vr[r];
    }
  };

  float m_run = -INFINITY;  // running max of scaled scores, log2 units (Theorem 2's m)
  float l_run = 0.f;        // running sum of this half-wave's keys (Theorem 2's l)
  f32x16 oacc[kOBlocks];    // unnormalised O^T: lane holds head-dims of its query column
#pragma unroll
  for (int j = 0; j < kOBlocks; ++j) oacc[j] = f32x16{};

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int tile = 0; tile < n_tiles; ++tile) {
    const int buf = tile & 1;
    const bool has_next = tile + 1 < n_tiles;
    if (has_next) load_tile(tile + 1);  // in flight while this tile is consumed

    const int key0 = tile * kBlockN;
    const bool wave_live = wrow0 < slen && !(CAUSAL && key0 > wrow0 + 31);
    if (wave_live) {
      const uint16_t* ks = smem + buf * 2 * kTile;
      const uint16_t* vs = ks + kTile;

      // S^T = K Q^T for two 32-key halves of the tile.
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16{};
        const int row = kb * 32 + lq;
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
          const u32x4 a =
              *reinterpret_cast<const u32x4*>(ks + lds_offset<D>(row, s * 16 + half * 8));
          sacc[kb] = E::mfma(a, qf[s], sacc[kb]);
        }
      }

      // Mask keys past the sequence end, and above the diagonal when causal.
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

      // Online softmax (Theorem 2): new running max, rescale factor, exponentials.
      float mx = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * p.c);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_new;
      const float neg_m = -m_use;
      float rsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], p.c, neg_m));
          sacc[kb][i] = e;
          rsum += e;
        }
      l_run = l_run * alpha + rsum;
#pragma unroll
      for (int j = 0; j < kOBlocks; ++j) oacc[j] *= alpha;

      // P^T fragments in the input type: B operand of step t of key half kb is
      // accumulator entries 8t .. 8t+7.
      u32x4 pb[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pb[kb][tt][e] = E::pack(sacc[kb][8 * tt + 2 * e], sacc[kb][8 * tt + 2 * e + 1]);

      // O^T += V^T P^T. Lane reads 4 head-dim columns x 4 keys per transposing read; the
      // 16 lanes of a group together receive column (lane % 32) of 4 consecutive keys.
      const int sub = lane & 15;
      const int col_in = 16 * ((lane >> 4) & 1) + 4 * (sub & 3);
#pragma unroll
      for (int j = 0; j < kOBlocks; ++j) {
        const int col = j * 32 + col_in;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const int r0 = kb * 32 + 16 * tt + 4 * half + (sub >> 2);
            const u32x2 lo = E::read_tr(vs + lds_offset<D>(r0, col));
            const u32x2 hi = E::read_tr(vs + lds_offset<D>(r0 + 8, col));
            const u32x4 a = u32x4{lo[0], lo[1], hi[0], hi[1]};
            oacc[j] = E::mfma(a, pb[kb][tt], oacc[j]);
          }
        }
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
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

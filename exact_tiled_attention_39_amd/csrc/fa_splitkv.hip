// Split-KV forward for short query chunks on gfx950: token-by-token decode, or a few new tokens,
// against a long key/value context.
//
// The result is the forward pass of fa_fwd.hip (exact softmax(scale * Q K^T) V with its
// log-sum-exp), organised for the case the forward kernel serves badly: with one query per
// sequence its 256-row query blocks are almost all padding, and its grid of batch x heads
// workgroups is far too small to keep HBM busy while the K/V context streams in.
//
//  * Packed rows: the query rows of all heads that share a kv head are one block of 32 rows
//    (row r = token (r / group), query head group * kv_head + r % group), so every K/V tile is
//    read once for the whole head group (the GQA layout of the "Flash Attention" notes,
//    section "Flash Attention 2 Improvements").
//  * Split keys: the key tiles of each (sequence, kv head, row block) are divided into
//    `splits` contiguous ranges, one workgroup each; packed sequences (up to 64) are taken
//    longest first, so that short ranges fill in behind the long ones. A split runs the
//    online softmax of the notes' Theorem 2 over its range and writes its normalised partial
//    output O_z and its log-sum-exp L_z (log2 units) to the caller's workspace. The merge
//    kernel then applies the same rescaling rule once more across splits: M = max_z L_z,
//    w_z = 2^(L_z - M), O = sum_z w_z O_z / sum_z w_z, LSE = M + log2(sum_z w_z). With one
//    split the first kernel writes O and LSE itself.
//  * One wave per workgroup with a private three-stage ring of 32-key K/V tiles in LDS, filled
//    by direct-to-LDS loads two tiles ahead: no barriers, and the three workgroups an LDS of
//    160 KB holds per CU keep about 100 KB of loads in flight per CU.
//  * The tile arithmetic is the forward kernel's: S^T = K Q^T on v_mfma_f32_32x32x16 with Q^T
//    resident, P rounded to the input type as the B operand of O^T += V^T P^T, V^T from the
//    transposing LDS read, scores in log2 units via one FMA with |scale| * log2(e).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "fa.h"
#include "fa_device.h"
#include "fa_launch.h"

// Split partials of fa_fwd_splitkv_noalloc, for callers that cannot allocate device memory.
// Every GPU the library runs on holds its own copy of this array until the process ends, and
// every call on that GPU reuses it. In host code `scratch` is only a stand-in for the symbol:
// its device address comes from hipGetSymbolAddress (noalloc_scratch below).
static __device__ __align__(256) float scratch[FA_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace fa {
namespace {

using namespace dev;

constexpr int kTileKeys = kSplitTileKeys;    // keys per K/V tile
constexpr int kBlockRows = kSplitBlockRows;  // packed query rows per workgroup
constexpr int kRing = 3;        // LDS ring stages per wave
constexpr int kMergeWaves = 4;  // rows merged per workgroup of the merge kernel

struct SplitArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  float* ws_o;    // [splits][rows_total][D] normalised partial outputs
  float* ws_lse;  // [splits][rows_total] partial log-sum-exp, log2 units (-inf: no key)
  const int32_t* cu_seqlens;
  const int32_t* cu_seqlens_k;
  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int64_t rows_total;  // batch * heads_q * seqlen: rows of LSE (and of each partial)
  int32_t seqlen;
  int32_t seqlen_k;
  int32_t heads_q;
  int32_t heads_kv;
  int32_t group;        // heads_q / heads_kv
  int32_t n_rowblocks;  // 32-row blocks per (sequence, kv head)
  int32_t splits;
  int32_t items;        // splits * heads_kv * (batch or sequences)
  int32_t num_seqs;     // packed sequences (with cu_seqlens)
  float c;              // |scale| * log2(e), or log2(e) when scale == 0
  uint32_t q_and;       // 0 when scale == 0, else all ones
  uint32_t q_xor;       // 0x80008000 when scale < 0 (Q negated exactly)
  const float* rope_cos;  // RoPE tables [rope_rows, D / 2], or NULL: Q is not rotated
  const float* rope_sin;
  int32_t rope_rows;
  int32_t rope_interleaved;
};

template <int D>
struct SplitGeo {
  static constexpr int kSteps = D / 16;            // k-steps of the S^T product
  static constexpr int kOBlocks = D / 32;          // 32-wide head-dim blocks of O^T
  static constexpr int kKBlocks = kSteps;          // 1 KB operand blocks per 32-key K tile
  static constexpr int kVBlocks = 2 * kOBlocks;    // 1 KB transposing blocks per V tile
  static constexpr int kDma = kKBlocks + kVBlocks;  // direct-to-LDS loads per tile
  static constexpr int kStageBytes = kDma * 1024;
  static_assert((kRing - 1) * kDma < 64, "outstanding loads fit the vmcnt counter");
};

template <int D, bool BF16, bool CAUSAL, bool VARLEN>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64)))
void fa_splitkv_kernel(const SplitArgs p) {
  using E = Elem<BF16>;
  using G = SplitGeo<D>;
  constexpr int kSteps = G::kSteps;
  constexpr int kOBlocks = G::kOBlocks;
  constexpr int kDma = G::kDma;

  __shared__ __attribute__((aligned(1024))) unsigned char smem[kRing * G::kStageBytes];
  const uint32_t lds_ring = lds_address(smem);
  const int lane = threadIdx.x;
  const int half = lane >> 5;
  const int lq = lane & 31;

  // ---- work item --------------------------------------------------------------------
  // Workgroups go to the 8 XCDs round-robin; the row blocks of one (split, kv head, sequence)
  // item read the same K/V range, so they are given the same XCD (blockIdx % 8).
  const int r8 = blockIdx.x >> 3;
  const int rb = r8 % p.n_rowblocks;
  const int item = (r8 / p.n_rowblocks) * 8 + int(blockIdx.x & 7);
  if (item >= p.items) return;
  const int z = item % p.splits;
  const int gb = item / p.splits;
  const int g = gb % p.heads_kv;
  int b = gb / p.heads_kv;
  if (VARLEN && p.num_seqs <= 64 && p.splits > 1) {
    // Packed sequences of unequal lengths: item block b runs the sequence with the b-th most
    // keys (ties by index), so the longest ranges start first and the short ones fill in
    // behind them. Lane s holds sequence s's key count and counts the sequences ahead of it.
    const int len = lane < p.num_seqs ? p.cu_seqlens_k[lane + 1] - p.cu_seqlens_k[lane] : -1;
    int rank = 0;
    for (int j = 0; j < p.num_seqs; ++j) {
      const int lj = __shfl(len, j);
      rank += (lj > len || (lj == len && j < lane)) ? 1 : 0;
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < p.num_seqs && rank == b);
    b = __builtin_amdgcn_readfirstlane(int(__builtin_ctzll(hit)));
  }

  int seq0 = 0, slen = p.seqlen, kseq0 = 0, klen = p.seqlen_k, bidx = b;
  if (VARLEN) {
    seq0 = p.cu_seqlens[b];
    slen = p.cu_seqlens[b + 1] - seq0;
    kseq0 = p.cu_seqlens_k[b];
    klen = p.cu_seqlens_k[b + 1] - kseq0;
    bidx = 0;
  }
  const int row0 = rb * kBlockRows;
  if (row0 >= slen * p.group) return;  // this sequence has fewer rows
  // queries are the last slen of the klen key positions: token t sees keys j <= t + shift
  const int shift = klen - slen;
  const int t_last = min(slen - 1, (row0 + kBlockRows - 1) / p.group);
  const int kv_end = CAUSAL ? min(klen, t_last + shift + 1) : klen;
  const int n_all = kv_end > 0 ? (kv_end + kTileKeys - 1) / kTileKeys : 0;
  // split z takes tiles [t_begin, t_end): the n_all tiles dealt as evenly as possible
  const int t_begin = int(int64_t(z) * n_all / p.splits);
  const int t_end = int(int64_t(z + 1) * n_all / p.splits);
  const int n = t_end - t_begin;

  // ---- Q^T of the lane's packed row (B operand), resident ------------------------------
  const int prow = row0 + lq;
  const int tq = prow / p.group;  // query token within the sequence
  const int hq = g * p.group + (prow - tq * p.group);
  const bool row_ok = tq < slen;
  u32x4 qf[kSteps];
  if (row_ok) {
    const uint16_t* qr =
        p.q + bidx * p.q_sb + hq * p.q_sh + int64_t(seq0 + tq) * p.q_sn + half * 8;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) qf[s] = *reinterpret_cast<const u32x4*>(qr + 16 * s);
  } else {
#pragma unroll
    for (int s = 0; s < kSteps; ++s) qf[s] = u32x4{0, 0, 0, 0};
  }
  if (p.rope_cos != nullptr) {
    // RoPE: query token tq sits at key position tq + shift (clamped into the tables)
    const int pos = min(max(tq + shift, 0), p.rope_rows - 1);
    rope_rotate_fragments<BF16, kSteps>(qf, p.rope_cos + int64_t(pos) * (D / 2),
                                        p.rope_sin + int64_t(pos) * (D / 2),
                                        p.rope_interleaved != 0, half);
  }
#pragma unroll
  for (int s = 0; s < kSteps; ++s) qf[s] = (qf[s] & p.q_and) ^ p.q_xor;

  // ---- direct-to-LDS staging of the split's tiles ---------------------------------------
  // Stage layout: kKBlocks operand blocks of K (block s: lane L's 16 bytes are key L % 32,
  // head-dims 16 s + 8 (L / 32) ..), then kVBlocks transposing blocks of V (block tt, j).
  const uint16_t* kbase = p.k + bidx * p.k_sb + g * p.k_sh + int64_t(kseq0) * p.k_sn;
  const uint16_t* vbase = p.v + bidx * p.v_sb + g * p.v_sh + int64_t(kseq0) * p.v_sn;
  int k_voff[G::kKBlocks];
  int v_voff[G::kVBlocks];
#pragma unroll
  for (int i = 0; i < G::kKBlocks; ++i) {
    int row, col;
    OperandLayout::row_col(i, lane, kSteps, row, col);
    k_voff[i] = int(row * p.k_sn * 2) + col * 2;
  }
#pragma unroll
  for (int i = 0; i < G::kVBlocks; ++i) {
    int row, col;
    TransposeLayout::row_col(i, lane, kOBlocks, row, col);
    v_voff[i] = int(row * p.v_sn * 2) + col * 2;
  }
  auto dma_tile = [&](int i, int stage) __attribute__((always_inline)) {
    const int key0 = (t_begin + i) * kTileKeys;
    const int rows = min(klen - key0, kTileKeys);  // >= 1: key0 < kv_end <= klen
    const u32x4 kr = make_rsrc(kbase + int64_t(key0) * p.k_sn, int((rows - 1) * p.k_sn * 2) + D * 2);
    const u32x4 vr = make_rsrc(vbase + int64_t(key0) * p.v_sn, int((rows - 1) * p.v_sn * 2) + D * 2);
    const uint32_t dst = lds_ring + stage * G::kStageBytes;
#pragma unroll
    for (int j = 0; j < G::kKBlocks; ++j) dma16(kr, dst + j * 1024, k_voff[j]);
#pragma unroll
    for (int j = 0; j < G::kVBlocks; ++j) dma16(vr, dst + (G::kKBlocks + j) * 1024, v_voff[j]);
  };

  const unsigned char* rd_k = smem + lane * 16;
  const unsigned char* rd_v = smem + G::kKBlocks * 1024 + lane * 8;
  // the lane's last visible key (its row's causal limit or the sequence end)
  const int row_lim = CAUSAL ? min(klen - 1, tq + shift) : klen - 1;
  const int t_first = row0 / p.group;  // smallest token of the block

  float m_run = -INFINITY;  // running maximum of scaled scores, log2 units
  float l_run = 0.f;        // this half-wave's running sum (for the log-sum-exp)
  float lr_run = 0.f;       // the same of P~ rounded to the input type (O's normaliser)
  f32x16 oacc[kOBlocks];
#pragma unroll
  for (int j = 0; j < kOBlocks; ++j) oacc[j] = f32x16{};

  for (int i = 0; i < kRing - 1 && i < n; ++i) dma_tile(i, i);
  int stage = 0;
  for (int i = 0; i < n; ++i) {
    // the stage of tile i - 1 is free: its LDS reads completed at the end of the last step
    if (i + kRing - 1 < n) dma_tile(i + kRing - 1, (stage + kRing - 1) % kRing);
    const int after = min(n - 1 - i, kRing - 1);  // tiles issued after tile i
    if (after >= 2)
      wait_vmcnt<2 * kDma>();
    else if (after == 1)
      wait_vmcnt<kDma>();
    else
      wait_vmcnt<0>();
    const int so = stage * G::kStageBytes;

    // S^T = K Q^T in two accumulation chains
    f32x16 sa = f32x16{}, sb = f32x16{};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(rd_k + so + s * 1024);
      if (s & 1)
        sb = E::mfma(a, qf[s], sb);
      else
        sa = E::mfma(a, qf[s], sa);
    }
    f32x16 sacc = sa + sb;

    // mask: entry e holds key key0 + 8 (e / 4) + 4 half + e % 4
    const int key0 = (t_begin + i) * kTileKeys;
    if (key0 + kTileKeys > klen || (CAUSAL && key0 + kTileKeys - 1 > t_first + shift)) {
      const int lim = row_lim - key0 - 4 * half;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        sacc[e] = 8 * (e >> 2) + (e & 3) <= lim ? sacc[e] : -INFINITY;
    }

    // online softmax (Theorem 2): exact tile maximum, rescale of l and O
    float mx = sacc[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sacc[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * p.c);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;  // a row with no key yet
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float ex[16];
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      ex[e] = __builtin_amdgcn_exp2f(fmaf(sacc[e], p.c, -m_use));
      sum += ex[e];
    }
    l_run = l_run * alpha + sum;
    lr_run *= alpha;
    m_run = m_new;
#pragma unroll
    for (int j = 0; j < kOBlocks; ++j) oacc[j] *= alpha;

    // O^T += V^T P^T; the B operand of 16-key step tt is entries 8 tt .. 8 tt + 7
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      u32x4 pb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pb[e] = E::pack(ex[8 * tt + 2 * e], ex[8 * tt + 2 * e + 1]);
        lr_run = E::add_pair(pb[e], lr_run);
      }
#pragma unroll
      for (int j = 0; j < kOBlocks; ++j) {
        const unsigned char* base = rd_v + so + (tt * kOBlocks + j) * 1024;
        const u32x2 lo = E::read_tr(base);
        const u32x2 hi = E::read_tr(base + 512);
        oacc[j] = E::mfma(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb, oacc[j]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this stage's LDS reads are done
    __builtin_amdgcn_sched_barrier(0);
    stage = stage + 1 == kRing ? 0 : stage + 1;
  }

  // ---- epilogue -----------------------------------------------------------------------
  // O~ is normalised by the sum of the rounded weights it was built from (an exact convex
  // combination of V rows); the log-sum-exp takes the fp32 sum
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float lr_tot = lr_run + __shfl_xor(lr_run, 32);
  if (!row_ok) return;
  // no key of this split is visible to the row
  const bool empty = n == 0 || t_begin * kTileKeys > row_lim;
  const int64_t ridx = (int64_t(bidx) * p.heads_q + hq) * p.seqlen + seq0 + tq;
  const float inv = empty ? 0.f : 1.f / lr_tot;
  const float lse2 = m_run + __builtin_amdgcn_logf(l_tot);  // log2 units
  if (p.splits == 1) {
    uint16_t* orow = p.o + bidx * p.o_sb + hq * p.o_sh + int64_t(seq0 + tq) * p.o_sn;
#pragma unroll
    for (int j = 0; j < kOBlocks; ++j) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = j * 32 + 8 * q4 + 4 * half;
        u32x2 w;
        w[0] = empty ? 0u : E::pack(oacc[j][4 * q4 + 0] * inv, oacc[j][4 * q4 + 1] * inv);
        w[1] = empty ? 0u : E::pack(oacc[j][4 * q4 + 2] * inv, oacc[j][4 * q4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
    }
    if (half == 0) p.lse[ridx] = empty ? -INFINITY : lse2 * 0.69314718055994531f;
    return;
  }
  const int64_t widx = int64_t(z) * p.rows_total + ridx;
  if (half == 0) p.ws_lse[widx] = empty ? -INFINITY : lse2;
  if (empty) return;  // the merge skips splits with L_z = -inf
  float* wo = p.ws_o + widx * D;
#pragma unroll
  for (int j = 0; j < kOBlocks; ++j) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = j * 32 + 8 * q4 + 4 * half;
      *reinterpret_cast<f32x4*>(wo + d0) =
          f32x4{oacc[j][4 * q4 + 0] * inv, oacc[j][4 * q4 + 1] * inv,
                oacc[j][4 * q4 + 2] * inv, oacc[j][4 * q4 + 3] * inv};
    }
  }
}

// Merge of the splits of one output row per wave: M = max_z L_z, w_z = 2^(L_z - M),
// O = sum_z w_z O_z / sum_z w_z, LSE = (M + log2 sum_z w_z) ln 2. A row no split saw gets O = 0
// and LSE = -inf.
template <int D, bool BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kMergeWaves, 64 * kMergeWaves)))
void fa_splitkv_merge_kernel(const SplitArgs p) {
  using E = Elem<BF16>;
  constexpr int kPer = D / 64;  // head-dims per lane
  const int lane = threadIdx.x & 63;
  const int64_t ridx = int64_t(blockIdx.x) * kMergeWaves + (threadIdx.x >> 6);
  if (ridx >= p.rows_total) return;
  const int64_t bh = ridx / p.seqlen;
  const int tok = int(ridx - bh * p.seqlen);
  const int b = int(bh / p.heads_q);
  const int h = int(bh - int64_t(b) * p.heads_q);

  // The row's maximum L_z: lane l reads splits l, l + 64, ...
  float m = -INFINITY;
  for (int z = lane; z < p.splits; z += 64)
    m = fmaxf(m, p.ws_lse[int64_t(z) * p.rows_total + ridx]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  float acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (m != -INFINITY) {
    for (int z0 = 0; z0 < p.splits; z0 += 64) {
      // lane l holds the weight of split z0 + l (0 for a split that saw no key: its O_z was
      // never written, so it is selected away rather than multiplied)
      const int zl = z0 + lane;
      const float lz = zl < p.splits ? p.ws_lse[int64_t(zl) * p.rows_total + ridx] : -INFINITY;
      const float wl = lz == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(lz - m);
      const int cnt = min(64, p.splits - z0);
      // independent loads, issued back to back
#pragma unroll 8
      for (int j = 0; j < cnt; ++j) {
        const float w = __shfl(wl, j);
        const float* src = p.ws_o + (int64_t(z0 + j) * p.rows_total + ridx) * D + lane * kPer;
        wsum += w;
#pragma unroll
        for (int e = 0; e < kPer; ++e) acc[e] += w != 0.f ? w * src[e] : 0.f;
      }
    }
  }
  const bool none = m == -INFINITY;
  const float inv = none ? 0.f : 1.f / wsum;
  uint16_t* orow = p.o + int64_t(b) * p.o_sb + h * p.o_sh + int64_t(tok) * p.o_sn + lane * kPer;
  if constexpr (kPer == 2) {
    *reinterpret_cast<uint32_t*>(orow) = none ? 0u : E::pack(acc[0] * inv, acc[1] * inv);
  } else {
    const uint32_t w = none ? 0u : E::pack(acc[0] * inv, 0.f);
    *orow = uint16_t(w & 0xFFFFu);
  }
  if (lane == 0)
    p.lse[ridx] = none ? -INFINITY : (m + __builtin_amdgcn_logf(wsum)) * 0.69314718055994531f;
}

template <int D, bool BF16, bool CAUSAL, bool VARLEN>
hipError_t launch_split_typed(const SplitArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((fa_splitkv_kernel<D, BF16, CAUSAL, VARLEN>), dim3(grid), dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  const int64_t merge_grid = (a.rows_total + kMergeWaves - 1) / kMergeWaves;
  hipLaunchKernelGGL((fa_splitkv_merge_kernel<D, BF16>), dim3(unsigned(merge_grid)),
                     dim3(64 * kMergeWaves), 0, s, a);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_split_mode(const SplitArgs& a, int grid, bool causal, bool varlen,
                             hipStream_t s) {
  if (causal)
    return varlen ? launch_split_typed<D, BF16, true, true>(a, grid, s)
                  : launch_split_typed<D, BF16, true, false>(a, grid, s);
  return varlen ? launch_split_typed<D, BF16, false, true>(a, grid, s)
                : launch_split_typed<D, BF16, false, false>(a, grid, s);
}

}  // namespace

void* noalloc_scratch(const char** hip_error) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *hip_error = hipGetErrorString(e);
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *hip_error = "device index beyond the 64 the split-KV scratch table holds";
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    // once per device, with that device current: this device's copy of the array
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      *hip_error = e != hipSuccess ? hipGetErrorString(e) : "hipGetSymbolAddress returned NULL";
      return nullptr;
    }
    addr[dev] = ptr;
  }
  return addr[dev];
}

fa_status launch_forward_splitkv(const fa_fwd_params& p, const SplitPlan& plan, void* workspace,
                                 void* stream, const char** hip_error) {
  if (p.rope_cos != nullptr && p.k_rot != nullptr) {
    const fa_status st = launch_rope_keys(p, stream, hip_error);
    if (st != FA_OK) return st;
  }
  SplitArgs a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.v = static_cast<const uint16_t*>(p.v);
  a.o = static_cast<uint16_t*>(p.o);
  a.lse = p.lse;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_lse = a.ws_o == nullptr ? nullptr
                               : a.ws_o + int64_t(plan.splits) * plan.rows_total * p.head_dim;
  a.cu_seqlens = p.cu_seqlens;
  a.cu_seqlens_k = p.cu_seqlens_k != nullptr ? p.cu_seqlens_k : p.cu_seqlens;
  a.q_sb = p.q_stride[0]; a.q_sh = p.q_stride[1]; a.q_sn = p.q_stride[2];
  a.k_sb = p.k_stride[0]; a.k_sh = p.k_stride[1]; a.k_sn = p.k_stride[2];
  a.v_sb = p.v_stride[0]; a.v_sh = p.v_stride[1]; a.v_sn = p.v_stride[2];
  a.o_sb = p.o_stride[0]; a.o_sh = p.o_stride[1]; a.o_sn = p.o_stride[2];
  if (p.rope_cos != nullptr && p.k_rot != nullptr) {  // attention reads the rotated keys
    a.k = static_cast<const uint16_t*>(p.k_rot);
    a.k_sb = p.k_rot_stride[0]; a.k_sh = p.k_rot_stride[1]; a.k_sn = p.k_rot_stride[2];
  }
  a.rope_cos = p.rope_cos;
  a.rope_sin = p.rope_sin;
  a.rope_rows = p.rope_rows;
  a.rope_interleaved = p.rope_interleaved;
  a.rows_total = plan.rows_total;
  a.seqlen = p.seqlen;
  a.seqlen_k = p.seqlen_k;
  a.heads_q = p.heads_q;
  a.heads_kv = p.heads_kv;
  a.group = p.heads_q / p.heads_kv;
  a.n_rowblocks = int32_t(plan.rowblocks);
  a.splits = plan.splits;
  a.items = int32_t(plan.items);
  a.num_seqs = p.cu_seqlens != nullptr ? p.num_seqs : 0;
  const double c = (p.scale == 0.f ? 1.0 : std::fabs(double(p.scale))) * 1.4426950408889634;
  a.c = float(c);
  a.q_and = p.scale == 0.f ? 0u : 0xFFFFFFFFu;
  a.q_xor = p.scale < 0.f ? 0x80008000u : 0u;
  const bool varlen = p.cu_seqlens != nullptr;
  const bool causal = p.causal != 0;
  const int grid = int(plan.grid);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (p.head_dim == 128)
    e = p.dtype == FA_BF16 ? launch_split_mode<128, true>(a, grid, causal, varlen, s)
                           : launch_split_mode<128, false>(a, grid, causal, varlen, s);
  else
    e = p.dtype == FA_BF16 ? launch_split_mode<64, true>(a, grid, causal, varlen, s)
                           : launch_split_mode<64, false>(a, grid, causal, varlen, s);
  if (e != hipSuccess) {
    *hip_error = hipGetErrorString(e);
    return FA_ERR_LAUNCH;
  }
  return FA_OK;
}

}  // namespace fa

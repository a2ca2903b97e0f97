// FlashAttention forward kernels for gfx950 (CDNA4): exact softmax(scale * Q K^T) V with
// online-softmax rescaling; the N x N scores and probabilities never leave registers.
//
// Algorithm: "Flash Attention" notes (14cs17), section "Flash Attention Algorithm" (for each
// query block: load Q_i, start O_i = 0, l_i = 0, m_i = -inf, stream K_j/V_j blocks through
// on-chip memory, form S_ij = Q_i K_j^T, update (m_i, l_i, O_i) by the online softmax of
// Theorem 2, write O_i), with FlashAttention-2's choices from the section "Flash Attention 2
// Improvements": the grid runs over query blocks, and O is normalised by l once at the end.
//
// Mapping onto the hardware (one workgroup = one 256-row query block of one head):
//  * 8 waves of 64 lanes in two groups of four; wave w owns 32 query rows of the block, so
//    waves never reduce across each other.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_{bf16,f16}: the
//    A operand is 32 keys x 16 head-dims read from LDS, the B operand is Q^T held in VGPRs for
//    the whole kernel. In the 32x32 accumulator lane L holds query column L % 32 and 16 keys,
//    so row statistics are in-lane plus one exchange between the two half-waves, and the
//    rescale of O by exp2(m_old - m_new) is a per-lane multiply.
//  * The exponentiated scores, rounded to the input type, are used directly as the B operand
//    of O^T += V^T P^T; the matching V^T operand comes from V through the gfx950 transposing
//    read ds_read_b64_tr_b16, with the key order permuted to match the accumulator layout
//    (keys {4h..4h+3, 8+4h..8+4h+3} of each 16-key step for half-wave h).
//  * Ping-pong: the two wave groups alternate, one barrier-delimited phase apart, between an
//    M phase (the S MFMAs of tile p and the P V MFMAs of tile p - 1) and a V phase (the online
//    softmax of tile p), so each SIMD overlaps one wave's softmax with the other's matrix work.
//    At d = 64, where the softmax is the longer phase, the softmax wave runs at the higher
//    issue priority; at d = 128 the matrix wave does (measured the faster choice for each).
//  * K and V tiles of 64 keys stream into four-stage LDS rings by direct-to-LDS buffer loads
//    (no staging registers, no LDS store instructions), issued two to three tiles ahead.
//    Each tile is stored fragment-major: every 1 KB block holds exactly one MFMA operand in
//    lane order, so every LDS read in the loop is contiguous (free of bank conflicts) and is a
//    per-lane base plus an immediate. Out-of-range rows read as zero (ragged tails).
//  * Running maxima are raised lazily: the first tile's maximum is the reference; a later tile
//    is exponentiated against the current reference and only if some lane's sum exceeds 2^15
//    (a score that far above the reference) is the tile maximum formed and O, l rescaled. Any reference maximum
//    gives the same O = O~ / l and LSE = m + log2(l); the bound keeps each exp2 <= 2^15.
//  * Two row sums: l of the fp32 exponentials gives the LSE, and l~ of the same values rounded
//    to the input type (the weights the P V product actually uses) normalises O, so the output
//    is an exact convex combination of V rows. With a lazily raised reference the dominant
//    weight is rarely exactly 1, and normalising by l would leave its rounding error in O.
//  * exp is exp2 with scale * log2(e) folded into one FMA per score.
//  * Causal blocks stop at the diagonal; only diagonal and ragged-tail tiles are masked.
//    Causal blocks are aligned to the sequence end, so a partial block is the cheapest one.
//  * The workgroup index is remapped so that the blocks of one head run on one XCD (its L2
//    serves the K/V re-reads), heaviest causal blocks first.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>
#include <utility>

#include "fa.h"
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

using namespace dev;

constexpr int kBlockM = 256;  // query rows per workgroup (B_r): 8 waves x 32 rows
constexpr int kBlockN = 64;   // keys per K/V tile (B_c)
constexpr int kThreads = 512;
constexpr int kStages = 4;    // depth of the K and V rings in LDS

struct KernelArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int32_t* cu_seqlens;
  const int32_t* cu_seqlens_k;  // key ranges of the packed sequences (== cu_seqlens by default)
  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int32_t seqlen;     // query tokens per batch entry (packed total for varlen)
  int32_t seqlen_k;   // key tokens per batch entry (unused for varlen)
  int32_t heads_q;
  int32_t group;      // heads_q / heads_kv
  int32_t n_qblocks;  // query blocks per (batch entry or sequence, head)
  float c;            // |scale| * log2(e), or log2(e) when scale == 0
  uint32_t q_and;     // 0 when scale == 0 (all scores are exactly 0), else all ones
  uint32_t q_xor;     // 0x80008000 when scale < 0: Q is negated exactly and c stays positive
  int32_t xcd_group;  // 0: plain order; 1: (batch, head) pairs in 8 contiguous runs, one per
                      // XCD; 2: kv heads dealt to the 8 XCDs in turn (heads_kv % 8 == 0)
  const float* rope_cos;  // RoPE tables [rope_rows, D / 2], or NULL: Q is not rotated
  const float* rope_sin;
  int32_t rope_rows;
  int32_t rope_interleaved;
};

// Fragment-major tile geometry. A K tile is kKBlocks blocks of 1 KB, block (kb, s) holding
// the A operand of the S^T MFMA for key half kb and k-step s in lane order (lane L: 16 bytes
// of key row 32 kb + L % 32, head-dims 16 s + 8 (L / 32) .. + 7). A V tile is kVBlocks blocks,
// block (kb, tt, j) holding the two transposing reads of the P V MFMA for key half kb, 16-key
// step tt and head-dim block j: bytes [0, 512) serve keys 16 tt + 0..7 of the half, bytes
// [512, 1024) keys 16 tt + 8..15, 8 bytes per lane in lane order.
template <int D>
struct Geo {
  static constexpr int kSteps = D / 16;            // k-steps of the S^T product
  static constexpr int kOBlocks = D / 32;          // 32-wide head-dim blocks of O^T
  static constexpr int kKBlocks = 2 * kSteps;      // blocks per K tile
  static constexpr int kVBlocks = 4 * kOBlocks;    // blocks per V tile
  static constexpr int kKBytes = kKBlocks * 1024;  // = 64 keys x D x 2 bytes
  static constexpr int kVBytes = kVBlocks * 1024;
  static constexpr int kDmaPerWave = kKBlocks / 4;  // 1 KB loads per staging wave per tile
  static constexpr int kLdsBytes = kStages * (kKBytes + kVBytes);
  static_assert(kKBlocks == kVBlocks, "K and V tiles have the same size");
};

// A tile is rescaled (its maximum formed) only when some lane's sum of exp2 exceeds this.
constexpr float kLazyBound = 32768.0f;

template <int D, bool BF16, bool CAUSAL, bool VARLEN>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(2, 2)))
void fa_fwd_kernel(const KernelArgs p) {
  using E = Elem<BF16>;
  using G = Geo<D>;
  constexpr int kSteps = G::kSteps;
  constexpr int kOBlocks = G::kOBlocks;
  constexpr int kDma = G::kDmaPerWave;

  __shared__ __attribute__((aligned(1024))) unsigned char smem[G::kLdsBytes];
  unsigned char* const lds_k = smem;                          // stage s at s * kKBytes
  unsigned char* const lds_v = smem + kStages * G::kKBytes;   // stage s at s * kVBytes
  // LDS byte address of smem (the value M0 takes for a direct-to-LDS load into it)
  const uint32_t lds_ring = lds_address(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int grp = wave >> 2;   // wave group: 0 stages K tiles, 1 stages V tiles
  const int gw = wave & 3;     // wave within its group
  const int half = lane >> 5;  // which 8-element half of each 16-wide k step this lane feeds
  const int lq = lane & 31;    // query column owned by this lane

  // ---- work item: (query block t, head, batch entry / sequence) -----------------------
  // Workgroups are dealt to the 8 XCDs round-robin (XCD = blockIdx % 8). With xcd_group the
  // blocks of one (batch, head) pair, and of the query heads sharing its kv head, all land on
  // one XCD, whose L2 then serves their K/V re-reads; mode 2 gives every XCD an equal share of
  // the heads of every batch entry, which also balances sequences of unequal length. Within
  // an XCD, t runs 0, 1, ... over query blocks n_qblocks - 1 - t, heaviest causal block
  // first, so the tail of the launch is made of the lightest blocks.
  const int pairs = gridDim.x / p.n_qblocks;
  int t, b, h;
  if (p.xcd_group == 2) {
    const int per = pairs >> 3;      // (batch, head) pairs per XCD
    const int hpx = p.heads_q >> 3;  // query heads per XCD per batch entry
    const int r = blockIdx.x >> 3;
    t = r / per;
    const int j = r - t * per;
    b = j / hpx;
    const int hh = j - b * hpx;
    const int kvl = hh / p.group, gq = hh - kvl * p.group;
    h = ((kvl << 3) + int(blockIdx.x & 7)) * p.group + gq;
  } else {
    int bh;
    if (p.xcd_group == 1 && (pairs & 7) == 0) {
      const int per = pairs >> 3;
      const int r = blockIdx.x >> 3;
      t = r / per;
      bh = (blockIdx.x & 7) * per + (r - t * per);
    } else {
      t = blockIdx.x / pairs;
      bh = blockIdx.x - t * pairs;
    }
    b = bh / p.heads_q;
    h = bh - b * p.heads_q;
  }
  int seq0 = 0, slen = p.seqlen, kseq0 = 0, klen = p.seqlen_k, bidx = b;
  if (VARLEN) {
    seq0 = p.cu_seqlens[b];
    slen = p.cu_seqlens[b + 1] - seq0;
    kseq0 = p.cu_seqlens_k[b];
    klen = p.cu_seqlens_k[b + 1] - kseq0;
    bidx = 0;
  }
  // The queries are the last slen of the klen key positions: causal query i sees keys
  // j <= i + shift (shift = 0 for self-attention).
  const int shift = klen - slen;
  // Causal blocks are aligned to the sequence end (shifted down by pad rows), so a partial
  // block is block 0, which sees the fewest keys (its rows below 0 are idle); block u then
  // sees 4 u + ceil((256 - pad) / 64) key tiles, and the order stays heaviest first.
  const int qblock = CAUSAL ? (p.n_qblocks - 1 - t) : t;
  const int pad = CAUSAL ? (-slen) & (kBlockM - 1) : 0;
  const int q0 = kBlockM * qblock - pad;
  if (q0 >= slen) return;  // uniform across the workgroup, before any barrier
  const int hk = h / p.group;

  const uint16_t* qb = p.q + bidx * p.q_sb + h * p.q_sh + int64_t(seq0) * p.q_sn;
  const uint16_t* kbase = p.k + bidx * p.k_sb + hk * p.k_sh + int64_t(kseq0) * p.k_sn;
  const uint16_t* vbase = p.v + bidx * p.v_sb + hk * p.v_sh + int64_t(kseq0) * p.v_sn;

  // keys [0, kv_end) are visible to some row of the block (none when kv_end <= 0)
  const int kv_end = CAUSAL ? min(klen, q0 + kBlockM + shift) : klen;
  const int n_tiles = kv_end > 0 ? (kv_end + kBlockN - 1) / kBlockN : 0;

  // ---- Q^T fragments (B operand), resident for the whole kernel -----------------------
  // The two waves sharing a SIMD (w and w + 4) take neighbouring 32-row slices, so both
  // groups reach the causal diagonal at nearly the same tile.
  const int wrow0 = q0 + 32 * (2 * gw + grp);  // first query row of this wave
  const int qrow = wrow0 + lq;                  // query row of this lane
  // buffer loads over this wave's rows inside [0, slen): rows outside read as zero
  u32x4 qf[kSteps];
  {
    const int lo = max(wrow0, 0);
    const int rows = max(min(slen, wrow0 + 32) - lo, 0);
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(qb + int64_t(lo) * p.q_sn), (short)0,
        rows > 0 ? int((rows - 1) * p.q_sn * 2) + D * 2 : 0, 0x00020000);
    // a lane below row 0 reads far past the end of the range
    const int qoff = qrow >= 0 ? int((qrow - lo) * p.q_sn * 2) + half * 16 : 0x40000000;
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
      qf[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qr, qoff + s * 32,
                                                                              0, 0));
    if (p.rope_cos != nullptr) {
      // RoPE: the lane's query row sits at key position qrow + shift (rows outside the
      // sequence hold zeros; their position is clamped only to stay inside the tables)
      const int pos = min(max(qrow + shift, 0), p.rope_rows - 1);
      rope_rotate_fragments<BF16, kSteps>(qf, p.rope_cos + int64_t(pos) * (D / 2),
                                          p.rope_sin + int64_t(pos) * (D / 2),
                                          p.rope_interleaved != 0, half);
    }
#pragma unroll
    for (int s = 0; s < kSteps; ++s) qf[s] = (qf[s] & p.q_and) ^ p.q_xor;
  }

  // ---- direct-to-LDS staging: group 0 streams K tiles, group 1 streams V tiles ----------
  // Staging wave gw fills blocks [gw * kDma, (gw + 1) * kDma) of each tile; lane L of a load
  // writes bytes [16 L, 16 L + 16) of its block, so it fetches the 16 source bytes that the
  // fragment-major layout puts there.
  const uint16_t* ld_base = grp ? vbase : kbase;
  const int64_t ld_sn = grp ? p.v_sn : p.k_sn;
  int ld_voff[kDma];
#pragma unroll
  for (int i = 0; i < kDma; ++i) {
    const int blk = gw * kDma + i;
    int row, col;
    if (grp == 0)
      OperandLayout::row_col(blk, lane, kSteps, row, col);  // K block (kb, s)
    else
      TransposeLayout::row_col(blk, lane, kOBlocks, row, col);  // V block (kb, tt, j)
    ld_voff[i] = int(row * ld_sn * 2) + col * 2;
  }
  // issue the loads of tile `tile` into ring stage ST of this group's tensor
  auto dma = [&](auto st, int tile) __attribute__((always_inline)) {
    constexpr int ST = decltype(st)::value;
    const int key0 = tile * kBlockN;
    const int rows = min(klen - key0, kBlockN);  // rows of this tile inside the sequence
    const int bytes = int((rows - 1) * ld_sn * 2) + D * 2;
    const u32x4 rsrc = make_rsrc(ld_base + int64_t(key0) * ld_sn, bytes);
    const uint32_t dst = lds_ring + (grp ? kStages * G::kKBytes + ST * G::kVBytes
                                         : ST * G::kKBytes) + gw * kDma * 1024;
#pragma unroll
    for (int i = 0; i < kDma; ++i) dma16(rsrc, dst + i * 1024, ld_voff[i]);
  };
  // wait until the loads of the tile issued `after` tiles before the most recent are in LDS
  // (after = number of this wave's tiles issued later, 0..2)
  auto dma_wait = [&](int after) __attribute__((always_inline)) {
    if (after >= 2)
      wait_vmcnt<2 * kDma>();
    else if (after == 1)
      wait_vmcnt<kDma>();
    else
      wait_vmcnt<0>();
  };

  // Per-lane LDS read bases; everything else in the M phase is an immediate offset.
  const unsigned char* rd_k = lds_k + lane * 16;
  const unsigned char* rd_v = lds_v + lane * 8;

  float m_run = -INFINITY;  // reference maximum of scaled scores, log2 units (Theorem 2's m)
  float l_run = 0.f;        // running sum of this half-wave's keys (Theorem 2's l), for the LSE
  float lr_run[4] = {0.f, 0.f, 0.f, 0.f};  // the same sum of the rounded P~, O's normaliser
  f32x16 oacc[kOBlocks];    // unnormalised O^T: lane holds head-dims of its query column
#pragma unroll
  for (int j = 0; j < kOBlocks; ++j) oacc[j] = f32x16{};
  f32x16 sacc[2];           // S^T of the tile between its M and V phases
  u32x4 pb[2][2];           // P^T of the previous tile, in the input type (B operands)
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) pb[kb][tt] = u32x4{0, 0, 0, 0};

  constexpr bool kMidBarrier = D == 64;  // see the schedule below

  // M phase (matrix cores), straight-line: S of tile p from K stage KS, and P V of tile p - 1
  // from V stage VS. Before the first tile P is zero and the V stage holds zeros; after the
  // last tile the S result is never used.
  // The 2 kSteps S MFMAs and 4 kOBlocks P V MFMAs go in groups of eight: four S MFMAs (k-steps
  // 2g and 2g + 1 of both key halves, so each Q^T operand feeds two in a row) then four P V
  // MFMAs (P V index 4g .. 4g + 3, which for d = 128 share one P^T operand). Consecutive MFMAs
  // into one accumulator are at least two apart. The LDS operand of MFMA n + kAhead is read
  // before MFMA n issues, and each step is pinned in place, so the read latency hides behind
  // kAhead matrix operations.
  constexpr int kMfma = 2 * (2 * kSteps);
  static_assert(2 * kSteps == 4 * kOBlocks, "S and P V MFMAs pair up");
  static_assert(kMfma % 8 == 0, "groups of four S and four P V MFMAs");
  constexpr int kAhead = 8;
  // MFMA n of the phase: an S MFMA (index 2 s + kb) or a P V MFMA (index i, head-dim block
  // i % kOBlocks, 16-key step i / kOBlocks)
  constexpr auto is_s = [](int n) constexpr { return (n & 7) < 4; };
  constexpr auto s_idx = [](int n) constexpr { return 4 * (n >> 3) + (n & 7); };
  constexpr auto pv_idx = [](int n) constexpr { return 4 * (n >> 3) + (n & 7) - 4; };
  auto phase_m = [&](auto ks, auto vs) __attribute__((always_inline)) {
    constexpr int KS = decltype(ks)::value;
    constexpr int VS = decltype(vs)::value;
    if constexpr (!kMidBarrier) __builtin_amdgcn_s_setprio(1);  // see the softmax's priority
    u32x4 opnd[kMfma];
    auto fetch = [&](auto nn) __attribute__((always_inline)) {
      constexpr int n = decltype(nn)::value;
      if constexpr (is_s(n)) {
        constexpr int kb = s_idx(n) & 1, s = s_idx(n) >> 1;  // S(kb, s)
        opnd[n] = *reinterpret_cast<const u32x4*>(rd_k + KS * G::kKBytes +
                                                  (kb * kSteps + s) * 1024);
      } else {
        constexpr int i = pv_idx(n), j = i % kOBlocks, kbtt = i / kOBlocks;  // PV(j, kb, tt)
        const unsigned char* base = rd_v + VS * G::kVBytes + (kbtt * kOBlocks + j) * 1024;
        const u32x2 lo = E::read_tr(base);
        const u32x2 hi = E::read_tr(base + 512);
        opnd[n] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    };
    auto issue = [&](auto nn) __attribute__((always_inline)) {
      constexpr int n = decltype(nn)::value;
      if constexpr (is_s(n)) {
        constexpr int kb = s_idx(n) & 1, s = s_idx(n) >> 1;
        sacc[kb] = E::mfma(opnd[n], qf[s], s == 0 ? f32x16{} : sacc[kb]);
      } else {
        constexpr int i = pv_idx(n), j = i % kOBlocks, kbtt = i / kOBlocks;
        oacc[j] = E::mfma(opnd[n], pb[kbtt >> 1][kbtt & 1], oacc[j]);
      }
    };
    [&]<int... n>(std::integer_sequence<int, n...>) {
      (fetch(Int<n>{}), ...);
    }(std::make_integer_sequence<int, kAhead>{});
    [&]<int... n>(std::integer_sequence<int, n...>) {
      ((
           [&] {
             if constexpr (n + kAhead < kMfma) fetch(Int<n + kAhead>{});
             issue(Int<n>{});
             __builtin_amdgcn_sched_barrier(0);
           }()),
       ...);
    }(std::make_integer_sequence<int, kMfma>{});
    if constexpr (!kMidBarrier) __builtin_amdgcn_s_setprio(0);
  };

  // Online softmax of S_tile (Theorem 2) into P_tile. Keys this wave cannot see (past the
  // sequence end, above the diagonal) get P = 0.
  // Issue priority: with two barriers per step (d = 64) the softmax wave issues ahead of the
  // matrix wave on its SIMD, as the V phase is the longer of the two; with one barrier per
  // step (d = 128) the matrix wave does (measured 0.3-0.6 % faster than either of the others).
  auto softmax = [&](int tile) __attribute__((always_inline)) {
    if constexpr (kMidBarrier) __builtin_amdgcn_s_setprio(1);
    const int key0 = tile * kBlockN;
    const bool edge = (key0 + kBlockN > klen) || (CAUSAL && key0 + kBlockN - 1 > wrow0 + shift);
    if (edge) {
      // entry i of key half kb is key key0 + off + 4 half; it is visible while off <= lim
      const int lim = (CAUSAL ? min(klen - 1, qrow + shift) : klen - 1) - key0 - 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = kb * 32 + 8 * (i >> 2) + (i & 3);
          sacc[kb][i] = off <= lim ? sacc[kb][i] : -INFINITY;
        }
      }
    }
    f32x16 ex[2];
    float part[4];
    auto expo = [&](float m_ref) __attribute__((always_inline)) {
      const float neg_m = -m_ref;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          ex[kb][i] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], p.c, neg_m));
          if (kb == 0 && i < 4)
            part[i] = ex[kb][i];
          else
            part[i & 3] += ex[kb][i];
        }
    };
    auto tile_max = [&]() __attribute__((always_inline)) {
      float mx = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      return fmaxf(mx, __shfl_xor(mx, 32)) * p.c;
    };
    // First tile: its own maximum is the reference (O and the sums are still zero). Every row
    // that sees any key sees one in the first tile of its sequence, so a row whose reference
    // stays -inf sees no key at all; its NaN sums take the rare path and are never stored.
    if (tile == 0) {
      if constexpr (D == 64) {
        // the same maximum, formed in the opposite order: the compiler then keeps the rare
        // path's first steps inside it instead of hoisting them into every tile
        float mx = sacc[1][15];
#pragma unroll
        for (int kb = 1; kb >= 0; --kb)
#pragma unroll
          for (int i = 15; i >= 0; --i) mx = fmaxf(mx, sacc[kb][i]);
        m_run = fmaxf(mx, __shfl_xor(mx, 32)) * p.c;
      } else {
        m_run = tile_max();
      }
    }
    expo(m_run);
    float rsum = (part[0] + part[1]) + (part[2] + part[3]);
    // Rare path: a score far above the reference. NaN sums also land here; they propagate to
    // the output either way.
    if (__builtin_amdgcn_ballot_w64(!(rsum <= kLazyBound))) {
      const float m_new = fmaxf(m_run, tile_max());
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int e = 0; e < 4; ++e) lr_run[e] *= alpha;
#pragma unroll
      for (int j = 0; j < kOBlocks; ++j) oacc[j] *= alpha;
      expo(m_run);
      rsum = (part[0] + part[1]) + (part[2] + part[3]);
    }
    l_run += rsum;
    // B operand of step tt of key half kb is accumulator entries 8tt .. 8tt+7.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pb[kb][tt][e] = E::pack(ex[kb][8 * tt + 2 * e], ex[kb][8 * tt + 2 * e + 1]);
          lr_run[e] = E::add_pair(pb[kb][tt][e], lr_run[e]);
        }
    if constexpr (kMidBarrier) __builtin_amdgcn_s_setprio(0);
  };

  // Phase boundary: this wave's LDS reads are complete, then a workgroup barrier that the
  // instruction scheduler may not move register-only work across.
  auto phase_sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- ping-pong schedule over ring stages ---------------------------------------------
  // Step p: group 0 runs M(p), then V(p); group 1 runs V(p - 1), then M(p). Each step ends
  // with a barrier; at d = 64 a second barrier between the two halves keeps the groups in
  // opposite phases (slot 2p: M(p) beside V(p - 1); slot 2p + 1: V(p) beside M(p)). At
  // d = 128 the groups drift within a step, which measured slightly faster on causal shapes
  // and 4 % slower at d = 64; the ring needs only the barrier that ends each step.
  // M(p) reads K_p (stage p % 4) and V_{p-1} (stage (p - 1) % 4).
  // K_p is read in step p (the M(p) of both groups); group 0 issues K_{p+3} after its M(p),
  // into the stage of K_{p-1}, whose readers (the M(p - 1) of both groups) ended before step
  // p began, and has waited for K_{p+1} before step p's closing barrier.
  // V_p is read in step p + 1; group 1 issues V_{p+2} at the start of step p, into the stage
  // of V_{p-2}, whose readers (the M(p - 1) of both groups) ended before step p began, and
  // has waited for V_p before step p's closing barrier.
  // Both groups execute the same barriers: n_tiles + 1 steps after the prologue's one (two
  // per step at d = 64). A block whose rows see no key at all (n_tiles == 0, only possible
  // when keys are fewer than queries) skips the loop as a whole workgroup.
  if (n_tiles > 0) {
    {
      // V stage 3 is read (with P = 0) before any tile lands there: it must hold finite data.
      const u32x4 zero = u32x4{0, 0, 0, 0};
      for (int off = tid * 16; off < G::kVBytes; off += kThreads * 16)
        *reinterpret_cast<u32x4*>(lds_v + 3 * G::kVBytes + off) = zero;
    }
    if (grp == 0) {
      dma(Int<0>{}, 0);
      if (n_tiles > 1) dma(Int<1>{}, 1);
      if (n_tiles > 2) dma(Int<2>{}, 2);
      dma_wait(min(n_tiles - 1, 2));  // K_0 in LDS
    } else {
      dma(Int<0>{}, 0);
      if (n_tiles > 1) dma(Int<1>{}, 1);
    }
    __syncthreads();

    // one ring step of each group; ST = p % 4
    auto step_g0 = [&](auto st, int tile) __attribute__((always_inline)) {
      constexpr int ST = decltype(st)::value;
      phase_m(Int<ST>{}, Int<(ST + 3) & 3>{});
      if constexpr (kMidBarrier) phase_sync();
      if (tile < n_tiles) softmax(tile);
      if (tile + 3 < n_tiles) dma(Int<(ST + 3) & 3>{}, tile + 3);
      if (tile + 1 < n_tiles) dma_wait(min(n_tiles - 2 - tile, 2));  // K_{tile+1} in LDS
      phase_sync();
    };
    auto step_g1 = [&](auto st, int tile) __attribute__((always_inline)) {
      constexpr int ST = decltype(st)::value;
      if (tile >= 1) softmax(tile - 1);
      if (tile + 2 < n_tiles) dma(Int<(ST + 2) & 3>{}, tile + 2);
      if constexpr (kMidBarrier) phase_sync();
      phase_m(Int<ST>{}, Int<(ST + 3) & 3>{});
      if (tile < n_tiles) dma_wait(min(n_tiles - 1 - tile, 2));  // V_tile in LDS
      phase_sync();
    };
    if (grp == 0) {
      for (int tile = 0; tile <= n_tiles; tile += 4) {
        step_g0(Int<0>{}, tile);
        if (tile + 1 <= n_tiles) step_g0(Int<1>{}, tile + 1);
        if (tile + 2 <= n_tiles) step_g0(Int<2>{}, tile + 2);
        if (tile + 3 <= n_tiles) step_g0(Int<3>{}, tile + 3);
      }
    } else {
      for (int tile = 0; tile <= n_tiles; tile += 4) {
        step_g1(Int<0>{}, tile);
        if (tile + 1 <= n_tiles) step_g1(Int<1>{}, tile + 1);
        if (tile + 2 <= n_tiles) step_g1(Int<2>{}, tile + 2);
        if (tile + 3 <= n_tiles) step_g1(Int<3>{}, tile + 3);
      }
    }
  }

  // ---- epilogue: O = O~ / l~, LSE = ln(l) + m; both half-waves hold partial sums -------
  if (wrow0 >= slen || wrow0 + 32 <= 0) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float lr_half = (lr_run[0] + lr_run[1]) + (lr_run[2] + lr_run[3]);
  const float lr_tot = lr_half + __shfl_xor(lr_half, 32);
  if (qrow >= 0 && qrow < slen) {
    // a row that sees no key: O = 0, LSE = -inf (its sums are 0 or NaN and are not used)
    const bool empty = (CAUSAL ? min(klen, qrow + shift + 1) : klen) <= 0;
    const float inv = empty ? 0.f : 1.f / lr_tot;
    uint16_t* orow = p.o + bidx * p.o_sb + h * p.o_sh + int64_t(seq0 + qrow) * p.o_sn;
#pragma unroll
    for (int j = 0; j < kOBlocks; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = j * 32 + 8 * g + 4 * half;
        u32x2 w;
        w[0] = empty ? 0u : E::pack(oacc[j][4 * g + 0] * inv, oacc[j][4 * g + 1] * inv);
        w[1] = empty ? 0u : E::pack(oacc[j][4 * g + 2] * inv, oacc[j][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
    }
    if (half == 0) {
      const float lse2 = m_run + __builtin_amdgcn_logf(l_tot);  // log2 units
      p.lse[(int64_t(bidx) * p.heads_q + h) * p.seqlen + seq0 + qrow] =
          empty ? -INFINITY : lse2 * 0.69314718055994531f;
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
  if (p.rope_cos != nullptr && p.k_rot != nullptr) {
    const fa_status st = launch_rope_keys(p, stream, hip_error);
    if (st != FA_OK) return st;
  }
  KernelArgs a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.v = static_cast<const uint16_t*>(p.v);
  a.o = static_cast<uint16_t*>(p.o);
  a.lse = p.lse;
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
  a.seqlen = p.seqlen;
  a.seqlen_k = p.seqlen_k;
  a.heads_q = p.heads_q;
  a.group = p.heads_q / p.heads_kv;
  const bool varlen = p.cu_seqlens != nullptr;
  const int rows = varlen ? p.max_seqlen : p.seqlen;
  a.n_qblocks = (rows + kBlockM - 1) / kBlockM;
  const double c = (p.scale == 0.f ? 1.0 : std::fabs(double(p.scale))) * 1.4426950408889634;
  a.c = float(c);
  a.q_and = p.scale == 0.f ? 0u : 0xFFFFFFFFu;
  a.q_xor = p.scale < 0.f ? 0x80008000u : 0u;
  a.xcd_group = p.heads_kv % 8 == 0 ? 2 : (varlen ? 0 : 1);
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

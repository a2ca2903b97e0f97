// FP8 forward kernel for gfx950: exact tiled attention on E4M3 (OCP) Q, K, V with per-(batch,
// head) descale factors, on the 32x32x64 FP8 matrix instructions (twice the 16-bit rate).
//
// FP8 matrix cores are FlashAttention-3's second lever (xspy page "FlashAttention and chunked
// prefill mechanics", section 1). The algorithm is the forward kernel's (fa_fwd.hip): one
// workgroup per 256-row query block, 8 waves in two ping-pong groups, S^T = K Q^T with Q^T
// resident, the online softmax of the "Flash Attention" notes' Theorem 2, O^T += V^T P^T,
// four-stage direct-to-LDS rings, end-aligned causal blocks and the XCD-aware block order.
// What changes for 8-bit operands:
//  * Each MFMA contracts 64 elements: a lane holds 32 bytes of its row (bytes 32 (L / 32) ..
//    + 31 of the 64). A K tile is stored as 1 KB blocks (key half kb, k-step s, byte half hb),
//    lane L's 16 bytes at 16 L, so each operand is two conflict-free 16-byte LDS reads.
//  * The P V product contracts over the 64 keys of a tile in one MFMA per 32 head-dims. Lane
//    (n, h) of P^T carries the 32 probabilities its S^T accumulators hold, for keys
//    key(h, j) = 32 (j / 16) + 8 ((j % 16) / 4) + 4 h + j % 4, j = 0..31. The V^T operand
//    must carry V[key(h, j)][m] in byte j: it comes from four ds_read_b64_tr_b8 per MFMA over
//    512-byte blocks laid out so that every direct-to-LDS lane still fetches 16 contiguous
//    bytes of one V row (see TrBlock below).
//  * Probabilities are rounded to E4M3 before the P V product. The running maximum is raised
//    lazily, as in the 16-bit kernel (the exact tile maximum, a serial reduction and a
//    cross-lane exchange ahead of every exponential, measured 18 % of the kernel's time), so a
//    probability may exceed E4M3's 448. The MFMA's E8M0 block scales take care of that: the
//    64 keys of a tile form two scale blocks of 32 (key half kb, both lane halves of a query
//    column), each scaled by its own power of two, lane n giving block 0's and lane n + 32
//    block 1's. Each block is divided by 2^k before rounding, k = max(0, e - 7) for a block sum
//    in [2^e, 2^(e+1)), so no value exceeds 2^8, and the MFMA multiplies 2^k back exactly.
//    Exponentials carry a shift of 8 (2^(s c - m + 8)) so that small probabilities keep
//    E4M3's normal range. The row sum keeps the unrounded values.
//  * Scores are scaled by c = |scale * descale_q * descale_k| log2(e) (a negative product
//    negates Q's sign bits), and O is multiplied by descale_v / l and stored as bf16.
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

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short v2s __attribute__((ext_vector_type(2)));

constexpr int kBlockM = 256;
constexpr int kBlockN = 64;
constexpr int kThreads = 512;
constexpr int kStages = 4;

struct Fp8Args {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  uint16_t* o;  // bf16
  float* lse;
  const float* q_descale;  // [batch, heads_q], or NULL for 1
  const float* k_descale;  // [batch, heads_kv]
  const float* v_descale;  // [batch, heads_kv]
  const int32_t* cu_seqlens;
  const int32_t* cu_seqlens_k;
  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int32_t seqlen;
  int32_t seqlen_k;
  int32_t heads_q;
  int32_t heads_kv;
  int32_t group;
  int32_t n_qblocks;
  float scale;
  int32_t xcd_group;
};

template <int D>
struct Geo8 {
  static constexpr int kSteps = D / 64;          // 64-wide k-steps of the S^T product
  static constexpr int kOBlocks = D / 32;        // 32-wide head-dim blocks of O^T
  static constexpr int kKBlocks = 4 * kSteps;    // 1 KB blocks per K tile: (kb, s, hb)
  static constexpr int kVBlocks = 2 * kOBlocks;  // 1 KB blocks per V tile: two TrBlocks each
  static constexpr int kKBytes = kKBlocks * 1024;  // = 64 keys x D bytes
  static constexpr int kVBytes = kVBlocks * 1024;
  static constexpr int kDmaPerWave = kKBlocks / 4;
  static constexpr int kLdsBytes = kStages * (kKBytes + kVBytes);
  static_assert(kKBlocks == kVBlocks, "K and V tiles have the same size");
};

// Sum and maximum of a value over lanes L and L ^ 32 with v_permlane32_swap (a VALU exchange;
// __shfl_xor goes through the LDS permute unit and its latency). The instruction swaps lanes
// 32..63 of its first operand with lanes 0..31 of its second, so swapping x with a copy of
// itself leaves lanes 0..31's values in the first register and lanes 32..63's in the second,
// in every lane. It is written as inline assembly with both registers as read-write operands:
// the compiler builtin's second result was folded into the first (r[0] + r[1] became 2 r[0]).
// The s_nop pairs give the wait states around a permlane that the compiler would otherwise
// insert itself.
__device__ __forceinline__ void halves_of(float x, float& lo, float& hi) {
  uint32_t a = __builtin_bit_cast(uint32_t, x);
  uint32_t b = a;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  lo = __builtin_bit_cast(float, a);
  hi = __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float sum_halves(float x) {
  float lo, hi;
  halves_of(x, lo, hi);
  return lo + hi;
}
__device__ __forceinline__ float max_halves(float x) {
  float lo, hi;
  halves_of(x, lo, hi);
  return fmaxf(lo, hi);
}

// The key carried in byte j (0..31) of a P^T / V^T operand lane of half h.
__host__ __device__ constexpr int key_of_byte(int h, int j) {
  return 32 * (j >> 4) + 8 * ((j & 15) >> 2) + 4 * h + (j & 3);
}

// V tile layout: TrBlock t = 4 jb + r (512 bytes) serves the 8 operand bytes j = 8 r .. 8 r + 7
// of the V^T operand of head-dim block jb through one ds_read_b64_tr_b8 (lane L reading 8
// bytes at 8 L). That instruction hands lane i of each 16-lane group g byte (i % 8) of the
// group's lane 2 b + i / 8 as its byte b, i.e. byte 128 g + 16 b + i of the block. So the
// 16 bytes at 16 (8 g + b) must be V[key(g / 2, 8 r + b)][32 jb + 16 (g % 2) .. + 15]: one
// row, 16 contiguous head-dims, which is what a direct-to-LDS lane fetches.
__device__ __forceinline__ void v_row_col(int blk, int lane, int& row, int& col) {
  const int t = 2 * blk + (lane >> 5);  // TrBlock written by this lane
  const int jb = t >> 2, r = t & 3;
  const int l = lane & 31;
  const int g = l >> 3, b = l & 7;
  row = key_of_byte(g >> 1, 8 * r + b);
  col = 32 * jb + 16 * (g & 1);
}

// K tile layout: block (kb, s, hb) = (kb * kSteps + s) * 2 + hb holds bytes 16 hb .. 16 hb + 15
// of the S^T A operand of key half kb and k-step s: lane L's 16 bytes are key 32 kb + L % 32,
// head-dims 64 s + 32 (L / 32) + 16 hb .. + 15.
template <int kSteps>
__device__ __forceinline__ void k_row_col(int blk, int lane, int& row, int& col) {
  const int hb = blk & 1, ks = blk >> 1;
  const int kb = ks / kSteps, s = ks % kSteps;
  row = 32 * kb + (lane & 31);
  col = 64 * s + 32 * (lane >> 5) + 16 * hb;
}

__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
  // E4M3 x E4M3 (format 0 for both operands), unit block scales (E8M0 127 = 2^0)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// The same with a per-lane E8M0 scale for the B operand: bytes 0..15 of lanes n and n + 32 (K
// block 0) take lane n's scale, bytes 16..31 of both (K block 1) lane n + 32's.
__device__ __forceinline__ f32x16 mfma8_bscaled(i32x8 a, i32x8 b, f32x16 c, int b_scale) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, b_scale);
}

// A tile is rescaled (its maximum formed) only when some lane's sum of shifted exponentials
// exceeds this (2^15 relative to the reference maximum, times the shift 2^8).
constexpr float kLazyBound8 = 8388608.0f;

template <int D, bool CAUSAL, bool VARLEN>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(2, 2)))
void fa_fwd_fp8_kernel(const Fp8Args p) {
  using G = Geo8<D>;
  constexpr int kSteps = G::kSteps;
  constexpr int kOBlocks = G::kOBlocks;
  constexpr int kDma = G::kDmaPerWave;

  __shared__ __attribute__((aligned(1024))) unsigned char smem[G::kLdsBytes];
  unsigned char* const lds_k = smem;
  unsigned char* const lds_v = smem + kStages * G::kKBytes;
  const uint32_t lds_ring = lds_address(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int gw = wave & 3;
  const int half = lane >> 5;
  const int lq = lane & 31;

  // ---- work item (the forward kernel's order) -----------------------------------------
  const int pairs = gridDim.x / p.n_qblocks;
  int t, b, h;
  if (p.xcd_group == 2) {
    const int per = pairs >> 3;
    const int hpx = p.heads_q >> 3;
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
  const int shift = klen - slen;
  const int qblock = CAUSAL ? (p.n_qblocks - 1 - t) : t;
  const int pad = CAUSAL ? (-slen) & (kBlockM - 1) : 0;
  const int q0 = kBlockM * qblock - pad;
  if (q0 >= slen) return;
  const int hk = h / p.group;

  // per-(batch, head) descales: scores scale by scale * dq * dk, the output by dv
  const float dq = p.q_descale ? p.q_descale[bidx * p.heads_q + h] : 1.f;
  const float dk = p.k_descale ? p.k_descale[bidx * p.heads_kv + hk] : 1.f;
  const float dv = p.v_descale ? p.v_descale[bidx * p.heads_kv + hk] : 1.f;
  const float sprod = p.scale * dq * dk;
  const float c = (sprod == 0.f ? 1.f : fabsf(sprod)) * 1.44269504088896341f;
  const uint32_t q_and = sprod == 0.f ? 0u : 0xFFFFFFFFu;
  const uint32_t q_xor = sprod < 0.f ? 0x80808080u : 0u;

  const uint8_t* qb = p.q + bidx * p.q_sb + h * p.q_sh + int64_t(seq0) * p.q_sn;
  const uint8_t* kbase = p.k + bidx * p.k_sb + hk * p.k_sh + int64_t(kseq0) * p.k_sn;
  const uint8_t* vbase = p.v + bidx * p.v_sb + hk * p.v_sh + int64_t(kseq0) * p.v_sn;

  const int kv_end = CAUSAL ? min(klen, q0 + kBlockM + shift) : klen;
  const int n_tiles = kv_end > 0 ? (kv_end + kBlockN - 1) / kBlockN : 0;

  // ---- Q^T fragments: 32 bytes per k-step, resident ------------------------------------
  const int wrow0 = q0 + 32 * (2 * gw + grp);
  const int qrow = wrow0 + lq;
  i32x8 qf[kSteps];
  {
    const int lo = max(wrow0, 0);
    const int rows = max(min(slen, wrow0 + 32) - lo, 0);
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(qb + int64_t(lo) * p.q_sn), (short)0,
        rows > 0 ? int((rows - 1) * p.q_sn) + D : 0, 0x00020000);
    const int qoff = qrow >= 0 ? int((qrow - lo) * p.q_sn) + half * 32 : 0x40000000;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const u32x4 lo16 = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(qr, qoff + s * 64, 0, 0));
      const u32x4 hi16 = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(qr, qoff + s * 64 + 16, 0, 0));
      i32x8 f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        f[w] = int((lo16[w] & q_and) ^ q_xor);
        f[4 + w] = int((hi16[w] & q_and) ^ q_xor);
      }
      qf[s] = f;
    }
  }

  // ---- direct-to-LDS staging: group 0 streams K tiles, group 1 V tiles -----------------
  const uint8_t* ld_base = grp ? vbase : kbase;
  const int64_t ld_sn = grp ? p.v_sn : p.k_sn;
  int ld_voff[kDma];
#pragma unroll
  for (int i = 0; i < kDma; ++i) {
    const int blk = gw * kDma + i;
    int row, col;
    if (grp == 0)
      k_row_col<kSteps>(blk, lane, row, col);
    else
      v_row_col(blk, lane, row, col);
    ld_voff[i] = int(row * ld_sn) + col;
  }
  auto dma = [&](auto st, int tile) __attribute__((always_inline)) {
    constexpr int ST = decltype(st)::value;
    const int key0 = tile * kBlockN;
    const int rows = min(klen - key0, kBlockN);
    const int bytes = int((rows - 1) * ld_sn) + D;
    const u32x4 rsrc = make_rsrc(ld_base + int64_t(key0) * ld_sn, bytes);
    const uint32_t dst = lds_ring + (grp ? kStages * G::kKBytes + ST * G::kVBytes
                                         : ST * G::kKBytes) + gw * kDma * 1024;
#pragma unroll
    for (int i = 0; i < kDma; ++i) dma16(rsrc, dst + i * 1024, ld_voff[i]);
  };

  const unsigned char* rd_k = lds_k + lane * 16;
  const unsigned char* rd_v = lds_v + lane * 8;

  float m_run = -INFINITY;  // running maximum of scaled scores, log2 units
  float l_run = 0.f;        // this half-wave's running sum of shifted exponentials
  f32x16 oacc[kOBlocks];
#pragma unroll
  for (int j = 0; j < kOBlocks; ++j) oacc[j] = f32x16{};
  f32x16 sacc[2];
  i32x8 pb = i32x8{0, 0, 0, 0, 0, 0, 0, 0};  // P^T of the previous tile, E4M3
  int pscale = 127;                           // its E8M0 block scale (this lane's block)

  // M phase: the 2 kSteps S MFMAs of tile p (K stage KS) and the kOBlocks P V MFMAs of tile
  // p - 1 (V stage VS), alternating in pairs, each operand read kAhead MFMAs ahead.
  constexpr int kS = 2 * kSteps;
  constexpr int kMfma = kS + kOBlocks;
  constexpr int kAhead = 4;
  // MFMA n: S MFMAs are n = 4 g, 4 g + 1 (index 2 g + {0,1}); P V MFMAs n = 4 g + 2, 4 g + 3
  constexpr auto is_s = [](int n) constexpr { return (n & 3) < 2; };
  constexpr auto s_idx = [](int n) constexpr { return 2 * (n >> 2) + (n & 1); };
  constexpr auto pv_idx = [](int n) constexpr { return 2 * (n >> 2) + (n & 1); };
  static_assert(kS == kOBlocks, "S and P V MFMAs pair up");
  auto phase_m = [&](auto ks, auto vs) __attribute__((always_inline)) {
    constexpr int KS = decltype(ks)::value;
    constexpr int VS = decltype(vs)::value;
    i32x8 opnd[kMfma];
    auto fetch = [&](auto nn) __attribute__((always_inline)) {
      constexpr int n = decltype(nn)::value;
      if constexpr (is_s(n)) {
        constexpr int i = s_idx(n), kb = i & 1, s = i >> 1;  // S(kb, s)
        const unsigned char* base = rd_k + KS * G::kKBytes + ((kb * kSteps + s) * 2) * 1024;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(base);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(base + 1024);
        opnd[n] = i32x8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]),
                        int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
      } else {
        constexpr int jb = pv_idx(n);
        const unsigned char* base = rd_v + VS * G::kVBytes + (4 * jb) * 512;
        i32x8 a;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (FA_LDS_PTR(i32x2))(base + r * 512));
          a[2 * r] = x[0];
          a[2 * r + 1] = x[1];
        }
        opnd[n] = a;
      }
    };
    auto issue = [&](auto nn) __attribute__((always_inline)) {
      constexpr int n = decltype(nn)::value;
      if constexpr (is_s(n)) {
        constexpr int i = s_idx(n), kb = i & 1, s = i >> 1;
        sacc[kb] = mfma8(opnd[n], qf[s], s == 0 ? f32x16{} : sacc[kb]);
      } else {
        constexpr int jb = pv_idx(n);
        oacc[jb] = mfma8_bscaled(opnd[n], pb, oacc[jb], pscale);
      }
    };
    [&]<int... n>(std::integer_sequence<int, n...>) {
      (fetch(Int<n>{}), ...);
    }(std::make_integer_sequence<int, (kAhead < kMfma ? kAhead : kMfma)>{});
    [&]<int... n>(std::integer_sequence<int, n...>) {
      ((
           [&] {
             if constexpr (n + kAhead < kMfma) fetch(Int<n + kAhead>{});
             issue(Int<n>{});
             __builtin_amdgcn_sched_barrier(0);
           }()),
       ...);
    }(std::make_integer_sequence<int, kMfma>{});
  };

  // Online softmax of a tile (Theorem 2) with a lazily raised reference maximum; P rounded to
  // E4M3 under per-block power-of-two scales.
  auto softmax = [&](int tile) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    const int key0 = tile * kBlockN;
    const bool edge = (key0 + kBlockN > klen) || (CAUSAL && key0 + kBlockN - 1 > wrow0 + shift);
    if (edge) {
      const int lim = (CAUSAL ? min(klen - 1, qrow + shift) : klen - 1) - key0 - 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = kb * 32 + 8 * (i >> 2) + (i & 3);
          sacc[kb][i] = off <= lim ? sacc[kb][i] : -INFINITY;
        }
    }
    float ex[2][16];
    float part[2][2];  // per key half, two interleaved partial sums
    auto expo = [&]() __attribute__((always_inline)) {
      const float off = 8.f - m_run;  // shifted by 2^8; +inf before the first tile
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          ex[kb][i] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], c, off));
          if (i < 2)
            part[kb][i] = ex[kb][i];
          else
            part[kb][i & 1] += ex[kb][i];
        }
    };
    expo();
    float s0 = part[0][0] + part[0][1];
    float s1 = part[1][0] + part[1][1];
    // Rare path: the first tile (no reference yet), or a score far above the reference; NaN
    // sums land here too and propagate either way.
    if (__builtin_amdgcn_ballot_w64(!(s0 + s1 <= kLazyBound8))) {
      float mx = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      const float m_new = fmaxf(m_run, max_halves(mx) * c);
      const float alpha = m_new == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int j = 0; j < kOBlocks; ++j) oacc[j] *= alpha;
      if (m_run == -INFINITY) m_run = 0.f;  // nothing visible yet: any reference will do
      expo();
      s0 = part[0][0] + part[0][1];
      s1 = part[1][0] + part[1][1];
    }
    l_run += s0 + s1;
    // block sums over both lane halves of this query column; 2^k with k = max(0, e - 7)
    const float b0 = sum_halves(s0);
    const float b1 = sum_halves(s1);
    const int k0 = max(int((__builtin_bit_cast(uint32_t, b0) >> 23) & 0xFF) - 127 - 7, 0);
    const int k1 = max(int((__builtin_bit_cast(uint32_t, b1) >> 23) & 0xFF) - 127 - 7, 0);
    const float d0 = __builtin_bit_cast(float, uint32_t(127 + k0) << 23);  // 2^k0
    const float d1 = __builtin_bit_cast(float, uint32_t(127 + k1) << 23);
    pscale = 127 + (half ? k1 : k0);
    // byte j of P^T is entry j % 16 of key half j / 16; v_cvt_scalef32_pk_fp8_f32 rounds
    // value / 2^k to E4M3 (nearest even) in one instruction per pair
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int kb = w >> 2, i = 4 * (w & 3);
      const float d = kb ? d1 : d0;
      v2s x = v2s{0, 0};
      x = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(x, ex[kb][i], ex[kb][i + 1], d, false);
      x = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(x, ex[kb][i + 2], ex[kb][i + 3], d, true);
      pb[w] = __builtin_bit_cast(int, x);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  auto phase_sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- ping-pong schedule --------------------------------------------------------------
  // Step p: group 0 runs M(p), then V(p); group 1 runs V(p - 1), then M(p). Two steps share
  // one barrier (double step p, p even, runs tiles p and p + 1). The matrix phase is much the
  // shorter here; with fewer barriers the two groups drift and their softmax phases overlap:
  // one barrier per step measured 5-7 % faster than two, and one per two steps another 1 %
  // at d = 128 and 12 % at d = 64, with the same results.
  // Ring: double step p reads K_p, K_{p+1} and V_{p-1}, V_p (stages p % 4 and p % 4 + 1, and
  // (p - 1) % 4 and p % 4), and loads the next double step's K_{p+2}, K_{p+3} (group 0) and
  // V_{p+1}, V_{p+2} (group 1) into the stages the previous double step read; each group
  // waits for its own loads before the closing barrier.
  if (n_tiles > 0) {
    {
      const u32x4 zero = u32x4{0, 0, 0, 0};
      for (int off = tid * 16; off < G::kVBytes; off += kThreads * 16)
        *reinterpret_cast<u32x4*>(lds_v + 3 * G::kVBytes + off) = zero;
    }
    // K_0, K_1 and V_0 are ready at the start of double step 0 (V stage 3 stands in for V_{-1})
    if (grp == 0) {
      dma(Int<0>{}, 0);
      if (n_tiles > 1) dma(Int<1>{}, 1);
    } else {
      dma(Int<0>{}, 0);
    }
    wait_vmcnt<0>();
    __syncthreads();

    auto dstep_g0 = [&](auto st0, int p) __attribute__((always_inline)) {
      constexpr int S0 = decltype(st0)::value;
      phase_m(Int<S0>{}, Int<(S0 + 3) & 3>{});
      if (p < n_tiles) softmax(p);
      if (p + 2 < n_tiles) dma(Int<(S0 + 2) & 3>{}, p + 2);
      if (p + 1 <= n_tiles) {
        phase_m(Int<S0 + 1>{}, Int<S0>{});
        if (p + 1 < n_tiles) softmax(p + 1);
        if (p + 3 < n_tiles) dma(Int<(S0 + 3) & 3>{}, p + 3);
      }
      wait_vmcnt<0>();
      phase_sync();
    };
    auto dstep_g1 = [&](auto st0, int p) __attribute__((always_inline)) {
      constexpr int S0 = decltype(st0)::value;
      if (p >= 1) softmax(p - 1);
      if (p + 1 < n_tiles) dma(Int<(S0 + 1) & 3>{}, p + 1);
      phase_m(Int<S0>{}, Int<(S0 + 3) & 3>{});
      if (p + 1 <= n_tiles) {
        softmax(p);
        if (p + 2 < n_tiles) dma(Int<(S0 + 2) & 3>{}, p + 2);
        phase_m(Int<S0 + 1>{}, Int<S0>{});
      }
      wait_vmcnt<0>();
      phase_sync();
    };
    if (grp == 0) {
      for (int p = 0; p <= n_tiles; p += 4) {
        dstep_g0(Int<0>{}, p);
        if (p + 2 <= n_tiles) dstep_g0(Int<2>{}, p + 2);
      }
    } else {
      for (int p = 0; p <= n_tiles; p += 4) {
        dstep_g1(Int<0>{}, p);
        if (p + 2 <= n_tiles) dstep_g1(Int<2>{}, p + 2);
      }
    }
  }

  // ---- epilogue: O = dv O~ / l (bf16), LSE = (m + log2 l - 8) ln 2 ----------------------
  if (wrow0 >= slen || wrow0 + 32 <= 0) return;
  const float l_tot = sum_halves(l_run);
  if (qrow >= 0 && qrow < slen) {
    const bool empty = (CAUSAL ? min(klen, qrow + shift + 1) : klen) <= 0;
    const float inv = empty ? 0.f : dv / l_tot;
    uint16_t* orow = p.o + bidx * p.o_sb + h * p.o_sh + int64_t(seq0 + qrow) * p.o_sn;
#pragma unroll
    for (int j = 0; j < kOBlocks; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = j * 32 + 8 * g + 4 * half;
        u32x2 w;
        w[0] = empty ? 0u
                     : Elem<true>::pack(oacc[j][4 * g + 0] * inv, oacc[j][4 * g + 1] * inv);
        w[1] = empty ? 0u
                     : Elem<true>::pack(oacc[j][4 * g + 2] * inv, oacc[j][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
    }
    if (half == 0) {
      const float lse2 = m_run + __builtin_amdgcn_logf(l_tot) - 8.f;
      p.lse[(int64_t(bidx) * p.heads_q + h) * p.seqlen + seq0 + qrow] =
          empty ? -INFINITY : lse2 * 0.69314718055994531f;
    }
  }
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_fp8_typed(const Fp8Args& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((fa_fwd_fp8_kernel<D, CAUSAL, VARLEN>), dim3(grid), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fp8_mode(const Fp8Args& a, int grid, bool causal, bool varlen, hipStream_t s) {
  if (causal)
    return varlen ? launch_fp8_typed<D, true, true>(a, grid, s)
                  : launch_fp8_typed<D, true, false>(a, grid, s);
  return varlen ? launch_fp8_typed<D, false, true>(a, grid, s)
                : launch_fp8_typed<D, false, false>(a, grid, s);
}

}  // namespace

fa_status launch_forward_fp8(const fa_fwd_params& p, void* stream, const char** hip_error) {
  Fp8Args a;
  a.q = static_cast<const uint8_t*>(p.q);
  a.k = static_cast<const uint8_t*>(p.k);
  a.v = static_cast<const uint8_t*>(p.v);
  a.o = static_cast<uint16_t*>(p.o);
  a.lse = p.lse;
  a.q_descale = p.q_descale;
  a.k_descale = p.k_descale;
  a.v_descale = p.v_descale;
  a.cu_seqlens = p.cu_seqlens;
  a.cu_seqlens_k = p.cu_seqlens_k != nullptr ? p.cu_seqlens_k : p.cu_seqlens;
  a.q_sb = p.q_stride[0]; a.q_sh = p.q_stride[1]; a.q_sn = p.q_stride[2];
  a.k_sb = p.k_stride[0]; a.k_sh = p.k_stride[1]; a.k_sn = p.k_stride[2];
  a.v_sb = p.v_stride[0]; a.v_sh = p.v_stride[1]; a.v_sn = p.v_stride[2];
  a.o_sb = p.o_stride[0]; a.o_sh = p.o_stride[1]; a.o_sn = p.o_stride[2];
  a.seqlen = p.seqlen;
  a.seqlen_k = p.seqlen_k;
  a.heads_q = p.heads_q;
  a.heads_kv = p.heads_kv;
  a.group = p.heads_q / p.heads_kv;
  const bool varlen = p.cu_seqlens != nullptr;
  const int rows = varlen ? p.max_seqlen : p.seqlen;
  a.n_qblocks = (rows + kBlockM - 1) / kBlockM;
  a.scale = p.scale;
  a.xcd_group = p.heads_kv % 8 == 0 ? 2 : (varlen ? 0 : 1);
  const int groups = varlen ? p.num_seqs : p.batch;
  const int grid = a.n_qblocks * p.heads_q * groups;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool causal = p.causal != 0;
  const hipError_t e = p.head_dim == 128 ? launch_fp8_mode<128>(a, grid, causal, varlen, s)
                                         : launch_fp8_mode<64>(a, grid, causal, varlen, s);
  if (e != hipSuccess) {
    *hip_error = hipGetErrorString(e);
    return FA_ERR_LAUNCH;
  }
  return FA_OK;
}

}  // namespace fa

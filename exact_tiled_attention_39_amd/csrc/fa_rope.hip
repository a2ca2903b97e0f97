// RoPE of the keys for gfx950: one streaming pass that rotates K into k_rot before attention.
//
// The forward kernels rotate Q as they load it (once per workgroup). K cannot be treated the
// same way: every key tile is read by every query block of its head, so rotating it where it
// is loaded would repeat the same work up to N / 256 times inside a kernel whose vector ALU is
// already busy with the softmax. A separate pass rotates each key once and costs one extra
// read and write of K; its output is exactly what a cache of rotated keys holds.
//
// Rotation (the RoPE of the "Flash Attention" notes' FlashAttention-2 feature list): pair i of
// the key at position p, (a, b) -> (a c - b s, a s + b c) with the caller's fp32 table entries
// c = cos[p][i], s = sin[p][i]; each product and the sum or difference rounded to fp32 on its
// own, then rounded to the input type. Positions count from each sequence's first key.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fa.h"
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

using namespace dev;

constexpr int kRopeThreads = 256;

struct RopeArgs {
  const uint16_t* k;
  uint16_t* out;
  const float* cos;
  const float* sin;
  const int32_t* cu_seqlens_k;
  int64_t k_sb, k_sh, k_sn;
  int64_t o_sb, o_sh, o_sn;
  int64_t rows;      // batch * heads_kv * seqlen_k
  int32_t seqlen_k;  // keys per batch entry (packed total with cu_seqlens_k)
  int32_t heads_kv;
  int32_t num_seqs;
  int32_t rope_rows;
};

// D / 16 threads per key row; thread u rotates the 8 pairs of frequencies 8 u .. 8 u + 7: with
// interleaved pairs the 16 elements 16 u .. 16 u + 15, otherwise elements 8 u .. 8 u + 7 with
// their partners D/2 further on. It reads both 16-byte pieces before writing them, so k_rot may
// be k itself.
template <int D, bool BF16, bool INTERLEAVED, bool VARLEN>
__global__ __launch_bounds__(kRopeThreads) void fa_rope_keys_kernel(const RopeArgs a) {
  using E = Elem<BF16>;
  constexpr int kUnits = D / 16;
  const int64_t row = int64_t(blockIdx.x) * (kRopeThreads / kUnits) + threadIdx.x / kUnits;
  const int u = threadIdx.x % kUnits;
  if (row >= a.rows) return;
  const int64_t bh = row / a.seqlen_k;
  const int j = int(row - bh * a.seqlen_k);
  const int b = int(bh / a.heads_kv);
  const int h = int(bh - int64_t(b) * a.heads_kv);
  int pos = j;
  if (VARLEN) {
    // the sequence holding packed key j: the last s with cu_seqlens_k[s] <= j
    int lo = 0, hi = a.num_seqs;  // invariant: cu[lo] <= j < cu[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.cu_seqlens_k[mid] <= j)
        lo = mid;
      else
        hi = mid;
    }
    pos = j - a.cu_seqlens_k[lo];
  }
  pos = min(pos, a.rope_rows - 1);
  const int col_a = INTERLEAVED ? 16 * u : 8 * u;
  const int col_b = INTERLEAVED ? 16 * u + 8 : 8 * u + D / 2;
  const uint16_t* src = a.k + b * a.k_sb + h * a.k_sh + int64_t(j) * a.k_sn;
  uint16_t* dst = a.out + b * a.o_sb + h * a.o_sh + int64_t(j) * a.o_sn;
  const u32x4 va = *reinterpret_cast<const u32x4*>(src + col_a);
  const u32x4 vb = *reinterpret_cast<const u32x4*>(src + col_b);
  const float* cs = a.cos + int64_t(pos) * (D / 2) + 8 * u;
  const float* sn = a.sin + int64_t(pos) * (D / 2) + 8 * u;
  const f32x4 c0 = *reinterpret_cast<const f32x4*>(cs);
  const f32x4 c1 = *reinterpret_cast<const f32x4*>(cs + 4);
  const f32x4 s0 = *reinterpret_cast<const f32x4*>(sn);
  const f32x4 s1 = *reinterpret_cast<const f32x4*>(sn + 4);
  const float c[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
  const float s[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
  float x[16];  // interleaved: elements col_a .. col_a + 15; else a-half then b-half
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    x[2 * w] = E::to_f32(uint16_t(va[w] & 0xFFFFu));
    x[2 * w + 1] = E::to_f32(uint16_t(va[w] >> 16));
    x[8 + 2 * w] = E::to_f32(uint16_t(vb[w] & 0xFFFFu));
    x[8 + 2 * w + 1] = E::to_f32(uint16_t(vb[w] >> 16));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (INTERLEAVED)
      rope_pair(x[2 * i], x[2 * i + 1], c[i], s[i], x[2 * i], x[2 * i + 1]);
    else
      rope_pair(x[i], x[8 + i], c[i], s[i], x[i], x[8 + i]);
  }
  u32x4 ra, rb;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    ra[w] = E::pack(x[2 * w], x[2 * w + 1]);
    rb[w] = E::pack(x[8 + 2 * w], x[8 + 2 * w + 1]);
  }
  *reinterpret_cast<u32x4*>(dst + col_a) = ra;
  *reinterpret_cast<u32x4*>(dst + col_b) = rb;
}

template <int D, bool BF16>
hipError_t launch_rope_typed(const RopeArgs& a, bool interleaved, bool varlen, hipStream_t s) {
  constexpr int kRowsPerBlock = kRopeThreads / (D / 16);
  const int64_t grid = (a.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (interleaved) {
    if (varlen)
      hipLaunchKernelGGL((fa_rope_keys_kernel<D, BF16, true, true>), dim3(unsigned(grid)),
                         dim3(kRopeThreads), 0, s, a);
    else
      hipLaunchKernelGGL((fa_rope_keys_kernel<D, BF16, true, false>), dim3(unsigned(grid)),
                         dim3(kRopeThreads), 0, s, a);
  } else {
    if (varlen)
      hipLaunchKernelGGL((fa_rope_keys_kernel<D, BF16, false, true>), dim3(unsigned(grid)),
                         dim3(kRopeThreads), 0, s, a);
    else
      hipLaunchKernelGGL((fa_rope_keys_kernel<D, BF16, false, false>), dim3(unsigned(grid)),
                         dim3(kRopeThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

fa_status launch_rope_keys(const fa_fwd_params& p, void* stream, const char** hip_error) {
  RopeArgs a;
  a.k = static_cast<const uint16_t*>(p.k);
  a.out = static_cast<uint16_t*>(p.k_rot);
  a.cos = p.rope_cos;
  a.sin = p.rope_sin;
  a.cu_seqlens_k = p.cu_seqlens_k != nullptr ? p.cu_seqlens_k : p.cu_seqlens;
  a.k_sb = p.k_stride[0]; a.k_sh = p.k_stride[1]; a.k_sn = p.k_stride[2];
  a.o_sb = p.k_rot_stride[0]; a.o_sh = p.k_rot_stride[1]; a.o_sn = p.k_rot_stride[2];
  a.rows = int64_t(p.batch) * p.heads_kv * p.seqlen_k;
  a.seqlen_k = p.seqlen_k;
  a.heads_kv = p.heads_kv;
  a.num_seqs = p.cu_seqlens != nullptr ? p.num_seqs : 0;
  a.rope_rows = p.rope_rows;
  if (a.rows == 0) return FA_OK;
  const bool varlen = p.cu_seqlens != nullptr;
  const bool inter = p.rope_interleaved != 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (p.head_dim == 128)
    e = p.dtype == FA_BF16 ? launch_rope_typed<128, true>(a, inter, varlen, s)
                           : launch_rope_typed<128, false>(a, inter, varlen, s);
  else
    e = p.dtype == FA_BF16 ? launch_rope_typed<64, true>(a, inter, varlen, s)
                           : launch_rope_typed<64, false>(a, inter, varlen, s);
  if (e != hipSuccess) {
    *hip_error = hipGetErrorString(e);
    return FA_ERR_LAUNCH;
  }
  return FA_OK;
}

}  // namespace fa

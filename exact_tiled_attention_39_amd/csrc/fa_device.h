// Device-side building blocks shared by the forward and backward kernels of libfa (gfx950):
// operand types, the 32x32x16 MFMA and the transposing LDS read per input type, raw buffer
// descriptors, the direct-to-LDS load, and the two fragment-major LDS tile layouts.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

namespace fa {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __fp16 f16x4_tr __attribute__((__vector_size__(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS_PTR(T) __attribute__((address_space(3))) T*

template <int N>
using Int = std::integral_constant<int, N>;

// Per input type: v_mfma_f32_32x32x16 on 8-element operands, ds_read_b64_tr_b16, the
// round-to-nearest-even pack of two fp32 values, and the sum of a packed pair added to an fp32
// value (v_dot2c_f32_{bf16,f16} against (1, 1): both products are exact).
template <bool BF16>
struct Elem;

template <>
struct Elem<true> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ u32x2 read_tr(const unsigned char* lds) {
    bf16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((FA_LDS_PTR(bf16x4))(lds));
    return __builtin_bit_cast(u32x2, r);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
  }
  static __device__ __forceinline__ float to_f32(uint16_t bits) {
    return __builtin_bit_cast(float, uint32_t(bits) << 16);
  }
  static __device__ __forceinline__ float add_pair(uint32_t pair, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair),
                                           __builtin_bit_cast(bf16x2, 0x3F803F80u), acc, false);
  }
};

template <>
struct Elem<false> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ u32x2 read_tr(const unsigned char* lds) {
    f16x4_tr r = __builtin_amdgcn_ds_read_tr16_b64_v4f16((FA_LDS_PTR(f16x4_tr))(lds));
    return __builtin_bit_cast(u32x2, r);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
  }
  static __device__ __forceinline__ float to_f32(uint16_t bits) {
    return float(__builtin_bit_cast(_Float16, bits));
  }
  static __device__ __forceinline__ float add_pair(uint32_t pair, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair),
                                  __builtin_bit_cast(f16x2, 0x3C003C00u), acc, false);
  }
};

// Raw buffer descriptor over [base, base + bytes) in scalar registers: loads past the end
// return zeros. (base and bytes are wave-uniform.)
__device__ __forceinline__ u32x4 make_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(uint32_t(a));
  r[1] = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32) & 0xFFFFu);
  r[2] = __builtin_amdgcn_readfirstlane(uint32_t(bytes));
  r[3] = 0x00020000u;
  return r;
}

// One 16-byte-per-lane direct-to-LDS load: lane L's 16 bytes at byte offset voff of the
// buffer land at LDS byte lds_addr + 16 L. Written as one asm statement so that the compiler's
// memory-counter bookkeeping does not treat every later LDS read as dependent on it; the
// kernels wait for these loads explicitly (wait_vmcnt) before the barrier that publishes them.
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t lds_addr, int voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_addr), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}

// s_waitcnt on outstanding vector-memory operations only (lgkm and exp counters left at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS byte address of a shared-memory pointer (the value M0 takes for a direct-to-LDS load).
__device__ __forceinline__ uint32_t lds_address(unsigned char* p) {
  return __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((FA_LDS_PTR(unsigned char))(p))));
}

// The two fragment-major layouts of a tile of 64 rows x D head-dims (rows are keys or queries,
// row-major in device memory with the head-dim contiguous). Both are 1 KB blocks, each holding
// one MFMA operand in lane order, so every read is contiguous and free of bank conflicts.
//
// Operand layout: block (h, s), h = 32-row half, s = 16-wide head-dim step, holds the A (or B)
// operand of a 32x32x16 MFMA contracting over head-dims: lane L has the 16 bytes of row
// 32 h + L % 32, head-dims 16 s + 8 (L / 32) .. + 7. Block index h * (D / 16) + s.
struct OperandLayout {
  static __device__ __forceinline__ void row_col(int blk, int lane, int steps, int& row,
                                                 int& col) {
    const int h = blk / steps, s = blk % steps;
    row = 32 * h + (lane & 31);
    col = 16 * s + 8 * (lane >> 5);
  }
};

// Transposing layout: block (h, t, j), h = 32-row half, t = 16-row step, j = 32-wide head-dim
// block, holds the two ds_read_b64_tr_b16 of the A operand of an MFMA contracting over rows
// (head-dims of block j as the M dimension). Bytes [0, 512) serve rows 16 t + 0..7 of the half,
// bytes [512, 1024) rows 16 t + 8..15; within each, lane L's 8 bytes sit at 8 L. The rows of
// each 16-row step come permuted to match the 32x32 accumulator: half-wave g of the MFMA
// reads rows {4g .. 4g + 3, 8 + 4g .. 8 + 4g + 3}. Block index (2 h + t) * (D / 32) + j.
struct TransposeLayout {
  static __device__ __forceinline__ void row_col(int blk, int lane, int oblocks, int& row,
                                                 int& col) {
    const int ht = blk / oblocks, j = blk % oblocks;
    const int part = lane >> 5;
    const int m = 2 * (lane & 31);
    row = 16 * ht + 8 * part + 4 * (m >> 5) + ((m & 15) >> 2);
    col = 32 * j + 16 * ((m >> 4) & 1) + 4 * (m & 3);
  }
};

// RoPE rotation of one pair by (c, s): (a c - b s, a s + b c), each product and the sum or
// difference rounded to fp32 on its own (no fused multiply-add), as the library documents.
__device__ __forceinline__ void rope_pair(float a, float b, float c, float s, float& ra,
                                          float& rb) {
#pragma clang fp contract(off)
  const float ac = a * c;
  const float bs = b * s;
  const float as = a * s;
  const float bc = b * c;
  ra = ac - bs;
  rb = as + bc;
}

// Rotates one row held as MFMA operand fragments in place: fragment t holds the 8 elements at
// head-dims 16 t + 8 half .. + 7 (the operand layout of the Q^T B operand). cs and sn point at
// the fp32 table row of the row's position. Interleaved pairs (2i, 2i + 1) lie inside one
// fragment; half-split pairs (i, i + D/2) are fragments t and t + kSteps / 2 of the same lane.
template <bool BF16, int kSteps>
__device__ __forceinline__ void rope_rotate_fragments(u32x4 (&x)[kSteps], const float* cs,
                                                      const float* sn, bool interleaved,
                                                      int half) {
  using E = Elem<BF16>;
  auto unpack = [](u32x4 v, float (&f)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      f[2 * w] = E::to_f32(uint16_t(v[w] & 0xFFFFu));
      f[2 * w + 1] = E::to_f32(uint16_t(v[w] >> 16));
    }
  };
  auto pack = [](const float (&f)[8]) __attribute__((always_inline)) {
    u32x4 v;
#pragma unroll
    for (int w = 0; w < 4; ++w) v[w] = E::pack(f[2 * w], f[2 * w + 1]);
    return v;
  };
  if (interleaved) {
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
      const int f0 = 8 * t + 4 * half;  // frequencies of the fragment's 4 pairs
      const f32x4 c = *reinterpret_cast<const f32x4*>(cs + f0);
      const f32x4 s = *reinterpret_cast<const f32x4*>(sn + f0);
      float e[8];
      unpack(x[t], e);
#pragma unroll
      for (int i = 0; i < 4; ++i) rope_pair(e[2 * i], e[2 * i + 1], c[i], s[i], e[2 * i], e[2 * i + 1]);
      x[t] = pack(e);
    }
  } else {
#pragma unroll
    for (int t = 0; t < kSteps / 2; ++t) {
      const int f0 = 16 * t + 8 * half;  // frequencies of the fragment's 8 elements
      const f32x4 c0 = *reinterpret_cast<const f32x4*>(cs + f0);
      const f32x4 c1 = *reinterpret_cast<const f32x4*>(cs + f0 + 4);
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(sn + f0);
      const f32x4 s1 = *reinterpret_cast<const f32x4*>(sn + f0 + 4);
      float a[8], b[8];
      unpack(x[t], a);
      unpack(x[t + kSteps / 2], b);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        rope_pair(a[i], b[i], i < 4 ? c0[i] : c1[i - 4], i < 4 ? s0[i] : s1[i - 4], a[i], b[i]);
      x[t] = pack(a);
      x[t + kSteps / 2] = pack(b);
    }
  }
}

}  // namespace dev
}  // namespace fa

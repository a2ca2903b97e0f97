// The C-ABI argument validation and split planning of libfa, on the host under ASan/UBSan.
// Every entry point is called with the documented error cases and then with a seeded sweep of
// parameter blocks drawn from edge values (zero, negative, just past each limit, INT32/INT64
// extremes, misaligned and NULL pointers). Kernel launches are the stand-ins of
// launch_stubs.cpp; no pointer is dereferenced on the host. Exits non-zero on any failed check
// (a sanitizer finding aborts the program by itself).
#include <cinttypes>
#include <cstdlib>
#include <climits>
#include <cstdio>
#include <cstring>
#include <random>

#include "fa.h"

extern int g_stub_launches;

namespace {

int g_failures = 0;
#define CHECK(cond)                                                          \
  do {                                                                       \
    if (!(cond)) {                                                           \
      std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);            \
      ++g_failures;                                                          \
    }                                                                        \
  } while (0)

void* fake(uintptr_t addr) { return reinterpret_cast<void*>(addr); }

const uintptr_t kBase = uintptr_t(1) << 32;  // 16-byte aligned stand-in device addresses

void set3(int64_t* s, int64_t b, int64_t h, int64_t n) { s[0] = b; s[1] = h; s[2] = n; }

fa_fwd_params good_fwd() {
  fa_fwd_params p;
  std::memset(&p, 0, sizeof(p));
  p.struct_size = sizeof(fa_fwd_params);
  p.dtype = FA_BF16;
  p.q = fake(kBase);
  p.k = fake(kBase + 0x100000);
  p.v = fake(kBase + 0x200000);
  p.o = fake(kBase + 0x300000);
  p.lse = static_cast<float*>(fake(kBase + 0x400000));
  p.batch = 2; p.heads_q = 8; p.heads_kv = 2; p.seqlen = 300; p.seqlen_k = 300;
  p.head_dim = 128; p.causal = 1; p.scale = 0.088f;
  set3(p.q_stride, 8 * 300 * 128, 300 * 128, 128);
  set3(p.o_stride, 8 * 300 * 128, 300 * 128, 128);
  set3(p.k_stride, 2 * 300 * 128, 300 * 128, 128);
  set3(p.v_stride, 2 * 300 * 128, 300 * 128, 128);
  return p;
}

fa_bwd_params good_bwd() {
  fa_bwd_params p;
  std::memset(&p, 0, sizeof(p));
  p.struct_size = sizeof(fa_bwd_params);
  p.dtype = FA_F16;
  p.q = fake(kBase); p.k = fake(kBase + 0x100000); p.v = fake(kBase + 0x200000);
  p.o = fake(kBase + 0x300000); p.dout = fake(kBase + 0x400000);
  p.lse = static_cast<const float*>(fake(kBase + 0x500000));
  p.delta = static_cast<float*>(fake(kBase + 0x600000));
  p.dq = fake(kBase + 0x700000); p.dk = fake(kBase + 0x800000); p.dv = fake(kBase + 0x900000);
  p.batch = 1; p.heads_q = 4; p.heads_kv = 4; p.seqlen = 257; p.head_dim = 64;
  p.causal = 1; p.scale = 0.125f;
  for (int64_t* s : {p.q_stride, p.k_stride, p.v_stride, p.o_stride, p.do_stride, p.dq_stride,
                     p.dk_stride, p.dv_stride})
    set3(s, 4 * 257 * 64, 257 * 64, 64);
  return p;
}

void documented_cases() {
  fa_fwd_params p = good_fwd();
  CHECK(fa_check_args(&p) == FA_OK);
  int before = g_stub_launches;
  CHECK(fa_fwd(&p, nullptr) == FA_OK && g_stub_launches == before + 1);
  CHECK(fa_check_args(nullptr) == FA_ERR_NULL);
  { fa_fwd_params b = p; b.struct_size -= 8; CHECK(fa_check_args(&b) == FA_ERR_ABI); }
  { fa_fwd_params b = p; b.head_dim = 96; CHECK(fa_check_args(&b) == FA_ERR_UNSUPPORTED); }
  { fa_fwd_params b = p; b.dtype = 7; CHECK(fa_check_args(&b) == FA_ERR_UNSUPPORTED); }
  { fa_fwd_params b = p; b.scale = 1.0f / 0.0f; CHECK(fa_check_args(&b) == FA_ERR_UNSUPPORTED); }
  { fa_fwd_params b = p; b.heads_kv = 3; CHECK(fa_check_args(&b) == FA_ERR_GQA); }
  { fa_fwd_params b = p; b.q = fake(kBase + 4); CHECK(fa_check_args(&b) == FA_ERR_ALIGN); }
  { fa_fwd_params b = p; b.q_stride[2] = 64; CHECK(fa_check_args(&b) == FA_ERR_ALIGN); }
  { fa_fwd_params b = p; b.k_stride[2] = (int64_t(1) << 23) + 8; CHECK(fa_check_args(&b) == FA_ERR_ALIGN); }
  { fa_fwd_params b = p; b.o = nullptr; CHECK(fa_check_args(&b) == FA_ERR_NULL); }
  { fa_fwd_params b = p; b.reserved0 = 1; CHECK(fa_check_args(&b) == FA_ERR_SHAPE); }
  { fa_fwd_params b = p; b.cu_seqlens = static_cast<const int32_t*>(fake(kBase + 0xA00000));
    CHECK(fa_check_args(&b) == FA_ERR_VARLEN); }  // batch 2 with packed sequences
  { fa_fwd_params b = p; b.seqlen = 0; before = g_stub_launches;
    CHECK(fa_fwd(&b, nullptr) == FA_OK && g_stub_launches == before); }
  // split-KV plan and workspace checks, and the allocation-free variant's scratch limit
  int32_t splits = 0;
  uint64_t bytes = 0;
  CHECK(fa_splitkv_plan(&p, 0, &splits, &bytes) == FA_OK && splits >= 1 && splits <= 256);
  CHECK(fa_splitkv_plan(&p, 257, &splits, &bytes) == FA_ERR_SHAPE);
  CHECK(fa_splitkv_plan(&p, 4, &splits, &bytes) == FA_OK && splits == 4 &&
        bytes == uint64_t(4) * 2 * 8 * 300 * 129 * 4);
  CHECK(fa_fwd_splitkv(&p, 4, nullptr, bytes, nullptr) == FA_ERR_NULL);
  CHECK(fa_fwd_splitkv(&p, 4, fake(kBase + 8), bytes, nullptr) == FA_ERR_ALIGN);
  CHECK(fa_fwd_splitkv(&p, 4, fake(kBase), bytes - 1, nullptr) == FA_ERR_SHAPE);
  CHECK(fa_fwd_splitkv(&p, 4, fake(kBase), bytes, nullptr) == FA_OK);
  CHECK(fa_fwd_splitkv_noalloc(&p, 4, nullptr) == FA_OK);
  CHECK(fa_fwd_splitkv_noalloc(&p, 256, nullptr) == FA_ERR_SCRATCH);
  // backward
  fa_bwd_params g = good_bwd();
  CHECK(fa_bwd_check_args(&g) == FA_OK);
  before = g_stub_launches;
  CHECK(fa_bwd(&g, nullptr) == FA_OK && g_stub_launches == before + 1);
  { fa_bwd_params b = g; b.delta = nullptr; CHECK(fa_bwd_check_args(&b) == FA_ERR_NULL); }
  { fa_bwd_params b = g; b.dq_stride[1] = 3; CHECK(fa_bwd_check_args(&b) == FA_ERR_ALIGN); }
  for (int s = -3; s < 12; ++s) CHECK(fa_status_string(s) != nullptr);
}

// Edge values for the sweep.
const int32_t kI32[] = {0, 1, 2, 3, 7, 8, 31, 32, 64, 65, 127, 128, 255, 256, 300, 4096, 65536,
                        (1 << 23), (1 << 23) + 1, INT32_MAX / 2, INT32_MAX - 1, INT32_MAX, -1,
                        -2, INT32_MIN};
const int64_t kI64[] = {0, 8, 16, 64, 128, 136, 4096, int64_t(1) << 23, (int64_t(1) << 23) + 8,
                        int64_t(1) << 31, int64_t(1) << 40, INT64_MAX / 2, INT64_MAX, -8, 3};

template <class R>
int32_t pick32(R& rng) { return kI32[rng() % (sizeof(kI32) / sizeof(kI32[0]))]; }
template <class R>
int64_t pick64(R& rng) { return kI64[rng() % (sizeof(kI64) / sizeof(kI64[0]))]; }
template <class R>
void* pickptr(R& rng, uintptr_t base) {
  switch (rng() % 8) {
    case 0: return nullptr;
    case 1: return fake(base + 4);
    case 2: return fake(base + 2);
    default: return fake(base);
  }
}

void sweep_forward(int rounds) {
  std::mt19937_64 rng(12345);
  for (int r = 0; r < rounds; ++r) {
    fa_fwd_params p = good_fwd();
    // change a random subset of the fields
    const int edits = 1 + int(rng() % 6);
    for (int e = 0; e < edits; ++e) {
      switch (rng() % 20) {
        case 0: p.batch = pick32(rng); break;
        case 1: p.heads_q = pick32(rng); break;
        case 2: p.heads_kv = pick32(rng); break;
        case 3: p.seqlen = pick32(rng); break;
        case 4: p.seqlen_k = pick32(rng); break;
        case 5: p.head_dim = pick32(rng); break;
        case 6: p.num_seqs = pick32(rng); p.cu_seqlens =
                    static_cast<const int32_t*>(pickptr(rng, kBase + 0xB00000)); break;
        case 7: p.max_seqlen = pick32(rng); break;
        case 8: p.q_stride[rng() % 3] = pick64(rng); break;
        case 9: p.k_stride[rng() % 3] = pick64(rng); break;
        case 10: p.v_stride[rng() % 3] = pick64(rng); break;
        case 11: p.o_stride[rng() % 3] = pick64(rng); break;
        case 12: p.q = pickptr(rng, kBase); break;
        case 13: p.lse = static_cast<float*>(pickptr(rng, kBase + 0x400000)); break;
        case 14: p.dtype = int32_t(rng() % 4) - (rng() % 5 == 0 ? 3 : 0); break;
        case 15: p.cu_seqlens_k = static_cast<const int32_t*>(pickptr(rng, kBase + 0xC00000)); break;
        case 16: p.rope_cos = static_cast<const float*>(pickptr(rng, kBase + 0xD00000));
                 p.rope_sin = static_cast<const float*>(pickptr(rng, kBase + 0xE00000));
                 p.rope_rows = pick32(rng); break;
        case 17: p.k_rot = pickptr(rng, kBase + 0xF00000); p.k_rot_stride[rng() % 3] = pick64(rng);
                 break;
        case 18: p.scale = (rng() % 2) ? -0.0f : 1e30f; break;
        case 19: p.causal = int32_t(rng() % 3); break;
      }
    }
    const fa_status st = fa_check_args(&p);
    CHECK(st >= FA_OK && st <= FA_ERR_SCRATCH);
    int before = g_stub_launches;
    const fa_status fs = fa_fwd(&p, nullptr);
    CHECK(fs == st);
    if (st != FA_OK) CHECK(g_stub_launches == before);
    int32_t splits = -1;
    uint64_t bytes = 0;
    const int32_t want = int32_t(rng() % 300) - 20;
    const fa_status ps = fa_splitkv_plan(&p, want, &splits, &bytes);
    if (st != FA_OK) CHECK(ps == st);
    if (ps == FA_OK) {
      CHECK(splits >= 1 && splits <= FA_MAX_SPLITS);
      CHECK(want == 0 || splits == want);
      CHECK(fa_fwd_splitkv(&p, want, bytes ? fake(kBase) : nullptr, bytes, nullptr) == FA_OK);
      const fa_status ns = fa_fwd_splitkv_noalloc(&p, want, nullptr);
      CHECK(ns == (bytes > FA_NOALLOC_SCRATCH_BYTES ? FA_ERR_SCRATCH : FA_OK));
    }
    CHECK(fa_status_string(st) != nullptr);
  }
}

void sweep_backward(int rounds) {
  std::mt19937_64 rng(777);
  for (int r = 0; r < rounds; ++r) {
    fa_bwd_params p = good_bwd();
    const int edits = 1 + int(rng() % 5);
    for (int e = 0; e < edits; ++e) {
      switch (rng() % 12) {
        case 0: p.batch = pick32(rng); break;
        case 1: p.heads_q = pick32(rng); break;
        case 2: p.heads_kv = pick32(rng); break;
        case 3: p.seqlen = pick32(rng); break;
        case 4: p.head_dim = pick32(rng); break;
        case 5: p.num_seqs = pick32(rng); p.cu_seqlens =
                    static_cast<const int32_t*>(pickptr(rng, kBase + 0xB00000)); break;
        case 6: p.max_seqlen = pick32(rng); break;
        case 7: p.dq_stride[rng() % 3] = pick64(rng); break;
        case 8: p.do_stride[rng() % 3] = pick64(rng); break;
        case 9: p.dk = pickptr(rng, kBase + 0x800000); break;
        case 10: p.delta = static_cast<float*>(pickptr(rng, kBase + 0x600000)); break;
        case 11: p.dtype = int32_t(rng() % 4); break;
      }
    }
    const fa_status st = fa_bwd_check_args(&p);
    const int before = g_stub_launches;
    CHECK(fa_bwd(&p, nullptr) == st);
    if (st != FA_OK) CHECK(g_stub_launches == before);
  }
}

}  // namespace

int main(int argc, char** argv) {
  const int rounds = argc > 1 ? std::atoi(argv[1]) : 200000;
  documented_cases();
  sweep_forward(rounds);
  sweep_backward(rounds / 2);
  std::printf("%d checks failed; %d stub launches\n", g_failures, g_stub_launches);
  return g_failures == 0 ? 0 : 1;
}

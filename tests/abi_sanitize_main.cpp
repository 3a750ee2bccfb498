// Host-side driver for the sanitizer run of the C ABI (tests/test_abi_sanitize_cpu.py).
//
// It links the ABI's host code, built with AddressSanitizer and UndefinedBehavior-
// Sanitizer, and calls every entry point with one argument defect at a time (each
// must give its documented status), then once more with well-formed arguments.  On
// a machine without a GPU those last calls reach the launch code and must fail with
// QSA_E_HIP; with a GPU present they are skipped, because their device pointers are
// placeholders.  Exit status 0 when every status matched; the sanitizers abort on
// the first error they find.
#include "qsa.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

namespace {

int g_fail = 0;

void expect(const char* what, int got, int want) {
  if (got != want) {
    std::printf("FAIL %s: status %d (%s), expected %d (%s)\n", what, got, qsa_status_string(got),
                want, qsa_status_string(want));
    ++g_fail;
  } else {
    std::printf("ok   %s: %s\n", what, qsa_status_string(got));
  }
}

qsa_dims good_dims() {
  qsa_dims d;
  d.num_q_heads = 16;
  d.num_kv_heads = 2;
  d.head_dim = 256;
  d.idx_heads = 4;
  d.idx_dim = 128;
  d.page_size = 64;
  d.rope_theta = 1e7f;
  d.sm_scale = 0.0625f;
  return d;
}

// Placeholder device addresses: never dereferenced on the host, and never passed to a
// kernel (the launch-path calls run only where no GPU exists).
template <class T>
T* fake(uintptr_t a) {
  return reinterpret_cast<T*>(a);
}

}  // namespace

int main() {
  int ndev = 0;
  const bool have_gpu = hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0;

  for (int s = -2; s <= 8; ++s) {
    const char* str = qsa_status_string(s);
    if (str == nullptr || std::strlen(str) == 0) {
      std::printf("FAIL status string %d\n", s);
      ++g_fail;
    }
  }

  const qsa_dims dims = good_dims();
  qsa_dims bad = good_dims();
  bad.num_q_heads = 8;
  qsa_dims bad_page = good_dims();
  bad_page.page_size = 24;

  // ---- workspace sizes
  if (qsa_workspace_bytes(nullptr, QSA_OP_INDEX_TOPK, 4, 4096, 0) != 0) ++g_fail;
  if (qsa_workspace_bytes(&dims, 99, 4, 4096, 0) != 0) ++g_fail;
  if (qsa_workspace_bytes(&dims, QSA_OP_INDEX_TOPK, 4, 0, 0) != 0) ++g_fail;
  if (qsa_workspace_bytes(&dims, QSA_OP_INDEX_TOPK, 4, QSA_MAX_CONTEXT + 1, 0) != 0) ++g_fail;
  const size_t ws_index = qsa_workspace_bytes(&dims, QSA_OP_INDEX_TOPK, 4, 8192, 0);
  const size_t ws_dec = qsa_workspace_bytes(&dims, QSA_OP_GQA_DECODE, 4, 0, 4);
  const size_t ws_pre = qsa_workspace_bytes(&dims, QSA_OP_GQA_PREFILL, 64, 0, 0);
  std::printf("workspaces: index %zu, decode %zu, prefill %zu\n", ws_index, ws_dec, ws_pre);
  if (ws_index == 0) ++g_fail;

  // ---- profiling events
  void* ev[18] = {};
  expect("profile events: 0 cancels", qsa_profile_kernel_events(nullptr, 0), QSA_OK);
  expect("profile events: odd count", qsa_profile_kernel_events(ev, 3), QSA_E_SHAPE);
  expect("profile events: too many", qsa_profile_kernel_events(ev, 18), QSA_E_SHAPE);
  expect("profile events: NULL handle", qsa_profile_kernel_events(ev, 2), QSA_E_NULL);
  expect("profile events: NULL array", qsa_profile_kernel_events(nullptr, 2), QSA_E_NULL);

  // ---- placeholders
  auto u16 = fake<uint16_t>(0x100000);
  auto cu16 = fake<const uint16_t>(0x100000);
  auto i32 = fake<int32_t>(0x200000);
  auto ci32 = fake<const int32_t>(0x200000);
  auto f32 = fake<float>(0x300000);
  auto cf32 = fake<const float>(0x300000);
  auto cu8 = fake<const uint8_t>(0x400000);
  auto i32b = fake<int32_t>(0x500000);
  std::vector<uint8_t> axis(64, 0);
  void* ws = fake<void>(0x600000);
  const int B = 4, PT = 256, SEL = QSA_MAX_SEL + 1;   // a multiple of 4

  // ---- builder
  expect("build: NULL dims",
         qsa_build_index_keys(nullptr, B, cu16, ci32, ci32, 4, 1, ci32, PT, u16, u16, nullptr),
         QSA_E_NULL);
  expect("build: unsupported dims",
         qsa_build_index_keys(&bad, B, cu16, ci32, ci32, 4, 1, ci32, PT, u16, u16, nullptr),
         QSA_E_UNSUPPORTED);
  expect("build: page size",
         qsa_build_index_keys(&bad_page, B, cu16, ci32, ci32, 4, 1, ci32, PT, u16, u16, nullptr),
         QSA_E_UNSUPPORTED);
  expect("build: batch 0 is a no-op",
         qsa_build_index_keys(&dims, 0, cu16, ci32, ci32, 4, 1, ci32, PT, u16, u16, nullptr),
         QSA_OK);
  expect("build: negative batch",
         qsa_build_index_keys(&dims, -1, cu16, ci32, ci32, 4, 1, ci32, PT, u16, u16, nullptr),
         QSA_E_SHAPE);
  expect("build: NULL ring",
         qsa_build_index_keys(&dims, B, cu16, ci32, ci32, 4, 1, ci32, PT, nullptr, u16, nullptr),
         QSA_E_NULL);
  expect("build mrope: NULL axis",
         qsa_build_index_keys_mrope(&dims, B, cu16, ci32, ci32, ci32, 4, 1, ci32, PT, nullptr, u16,
                                    i32, u16, nullptr),
         QSA_E_NULL);

  // ---- indexer
  expect("index: NULL idx_q",
         qsa_index_topk(&dims, B, B, nullptr, cf32, ci32, ci32, 8192, ci32, PT, cu16, i32, i32b,
                        SEL, i32, ws, ws_index, nullptr),
         QSA_E_NULL);
  expect("index: max_pos beyond the context",
         qsa_index_topk(&dims, B, B, cu16, cf32, ci32, ci32, QSA_MAX_CONTEXT + 1, ci32, PT, cu16,
                        i32, i32b, SEL, i32, ws, ws_index, nullptr),
         QSA_E_SHAPE);
  expect("index: sel_stride not a multiple of 4",
         qsa_index_topk(&dims, B, B, cu16, cf32, ci32, ci32, 8192, ci32, PT, cu16, i32, i32b,
                        QSA_MAX_SEL, i32, ws, ws_index, nullptr),
         QSA_E_SHAPE);
  expect("index: sel_stride below the expansion",
         qsa_index_topk(&dims, B, B, cu16, cf32, ci32, ci32, 8192, ci32, PT, cu16, i32, i32b, 100,
                        i32, ws, ws_index, nullptr),
         QSA_E_SHAPE);
  expect("index: small workspace",
         qsa_index_topk(&dims, B, B, cu16, cf32, ci32, ci32, 8192, ci32, PT, cu16, i32, i32b, SEL,
                        i32, ws, ws_index - 1, nullptr),
         QSA_E_WORKSPACE);
  expect("decode build+index: NULL ring",
         qsa_decode_build_index_topk(&dims, B, cu16, ci32, 8192, ci32, PT, nullptr, u16, cu16, cf32,
                                     i32, i32b, SEL, i32, ws, ws_index, nullptr),
         QSA_E_NULL);
  expect("decode build+index mrope: NULL positions",
         qsa_decode_build_index_topk_mrope(&dims, B, cu16, nullptr, ci32, 8192, ci32, PT,
                                           axis.data(), u16, i32, u16, cu16, cf32, i32, i32b, SEL,
                                           i32, ws, ws_index, nullptr),
         QSA_E_NULL);

  // ---- sparse GQA
  expect("gqa decode: n_extra beyond the limit",
         qsa_sparse_gqa_decode(&dims, B, cu16, cu16, cu16, ci32, PT, ci32, ci32, SEL, ci32,
                               QSA_MAX_EXTRA + 1, u16, f32, ws, ws_dec, nullptr),
         QSA_E_SHAPE);
  expect("gqa decode: NULL out",
         qsa_sparse_gqa_decode(&dims, B, cu16, cu16, cu16, ci32, PT, ci32, ci32, SEL, nullptr, 0,
                               nullptr, f32, ws, ws_dec, nullptr),
         QSA_E_NULL);
  if (ws_dec > 0)
    expect("gqa decode: small workspace",
           qsa_sparse_gqa_decode(&dims, B, cu16, cu16, cu16, ci32, PT, ci32, ci32, SEL, nullptr, 0,
                                 u16, f32, ws, ws_dec - 1, nullptr),
           QSA_E_WORKSPACE);
  expect("gqa decode noalloc: n_extra beyond the limit",
         qsa_sparse_gqa_decode_noalloc(&dims, B, cu16, cu16, cu16, ci32, PT, ci32, ci32, SEL, ci32,
                                       QSA_MAX_EXTRA + 1, u16, f32, nullptr),
         QSA_E_SHAPE);
  expect("gqa decode noalloc: NULL extra_pos with n_extra",
         qsa_sparse_gqa_decode_noalloc(&dims, B, cu16, cu16, cu16, ci32, PT, ci32, ci32, SEL,
                                       nullptr, 2, u16, f32, nullptr),
         QSA_E_NULL);
  expect("gqa prefill: NULL q_req",
         qsa_sparse_gqa_prefill(&dims, 64, cu16, nullptr, cu16, cu16, ci32, PT, ci32, ci32, SEL,
                                u16, f32, ws, ws_pre, nullptr),
         QSA_E_NULL);
  expect("gqa decode fp8: non-positive scale",
         qsa_sparse_gqa_decode_fp8(&dims, B, cu16, cu8, cu8, 0.f, 1.f, ci32, PT, ci32, ci32, SEL,
                                   nullptr, 0, u16, f32, ws, ws_dec, nullptr),
         QSA_E_SHAPE);
  expect("gqa prefill fp8: unsupported dims",
         qsa_sparse_gqa_prefill_fp8(&bad, 64, cu16, ci32, cu8, cu8, 1.f, 1.f, ci32, PT, ci32, ci32,
                                    SEL, u16, f32, ws, ws_pre, nullptr),
         QSA_E_UNSUPPORTED);

  // ---- well-formed calls: they reach the launch code
  if (have_gpu) {
    std::printf("a GPU is present: the launch-path calls (placeholder pointers) are skipped\n");
  } else {
    expect("build: launch without a device",
           qsa_build_index_keys(&dims, B, cu16, ci32, ci32, 4, 1, ci32, PT, u16, u16, nullptr),
           QSA_E_HIP);
    expect("index: launch without a device",
           qsa_index_topk(&dims, B, B, cu16, cf32, ci32, ci32, 8192, ci32, PT, cu16, i32, i32b, SEL,
                          i32, ws, ws_index, nullptr),
           QSA_E_HIP);
    expect("decode build+index: launch without a device",
           qsa_decode_build_index_topk(&dims, B, cu16, ci32, 8192, ci32, PT, u16, u16, cu16, cf32,
                                       i32, i32b, SEL, i32, ws, ws_index, nullptr),
           QSA_E_HIP);
    expect("gqa decode: launch without a device",
           qsa_sparse_gqa_decode(&dims, B, cu16, cu16, cu16, ci32, PT, ci32, ci32, SEL, ci32, 4, u16,
                                 f32, ws, ws_dec, nullptr),
           QSA_E_HIP);
    expect("gqa decode noalloc: launch without a device",
           qsa_sparse_gqa_decode_noalloc(&dims, B, cu16, cu16, cu16, ci32, PT, ci32, ci32, SEL,
                                         nullptr, 0, u16, f32, nullptr),
           QSA_E_HIP);
    expect("gqa prefill: launch without a device",
           qsa_sparse_gqa_prefill(&dims, 64, cu16, ci32, cu16, cu16, ci32, PT, ci32, ci32, SEL, u16,
                                  f32, ws, ws_pre, nullptr),
           QSA_E_HIP);
  }
  std::printf("%s: %d mismatches\n", g_fail ? "FAILED" : "PASSED", g_fail);
  return g_fail ? 1 : 0;
}

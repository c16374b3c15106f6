/*
 * Host-side paths of the C ABI, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host code by tests/test_host_sanitized.py
 * and run without a GPU: argument validation of every entry point (each call
 * below fails before anything is enqueued, or is a T = 0 / n = 0 no-op),
 * workspace sizing, the GEMM tile and GEMV row queries, the 4-bit code books
 * and the status strings. Pointers are host addresses standing in for device
 * buffers; no call reaches a launch.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "llmint8.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static _Alignas(256) unsigned char buf[4096];

int main(void) {
  void* p = buf;
  void* mis = buf + 2;  /* 2-byte aligned only */
  void* odd = buf + 1;
  const int INVALID = LLMINT8_ERR_INVALID_ARG, UNSUP = LLMINT8_ERR_UNSUPPORTED;

  /* weight quantization */
  EXPECT(llmint8_quantize_weight(NULL, 16, 64, p, p, NULL) == INVALID);
  EXPECT(llmint8_quantize_weight(p, 16, 72, p, p, NULL) == UNSUP);
  EXPECT(llmint8_quantize_weight(mis, 16, 64, p, p, NULL) == INVALID);
  EXPECT(llmint8_quantize_weight_ex(p, 7, 16, 64, p, p, NULL) == INVALID);

  /* forward: validation and the T = 0 no-op */
  EXPECT(llmint8_workspace_bytes(16, 1024, 1024) == 0); /* fused decode route: no workspace */
  EXPECT(llmint8_workspace_bytes_path(16, 1024, 1024, LLMINT8_PATH_GEMV) == 0);
  EXPECT(llmint8_workspace_bytes_path(16, 1024, 1024, LLMINT8_PATH_GEMM) > 16 * 1024);
  EXPECT(llmint8_workspace_bytes_path(16, 1024, 1024, LLMINT8_PATH_GEMM) < llmint8_workspace_bytes(64, 1024, 1024));
  EXPECT(llmint8_workspace_bytes_path(16, 1024, 1024, LLMINT8_PATH_GEMM_352x256) ==
         llmint8_workspace_bytes_path(16, 1024, 1024, LLMINT8_PATH_GEMM));
  EXPECT(llmint8_workspace_bytes_path(16, 1024, 1024, 3) == 0); /* unknown path */
  const size_t need = llmint8_workspace_bytes(64, 1024, 1024);
  EXPECT(need > 64 * 1024);
  EXPECT(llmint8_linear(NULL, 64, 1024, p, p, 1024, 6.0f, p, p, need, NULL) == INVALID);
  EXPECT(llmint8_linear(p, 64, 1024, p, p, 1024, NAN, p, p, need, NULL) == INVALID);
  EXPECT(llmint8_linear(p, 64, 1024, p, p, 1024, -1.0f, p, p, need, NULL) == INVALID);
  EXPECT(llmint8_linear(p, 64, 1024, p, p, 1024, 6.0f, p, p, need - 256, NULL) == LLMINT8_ERR_WORKSPACE);
  EXPECT(llmint8_linear(p, 64, 1024, p, p, 1024, 6.0f, NULL, p, need, NULL) == INVALID);
  EXPECT(llmint8_linear(p, 64, 1024, p, p, 1024, 6.0f, p, NULL, need, NULL) == INVALID);
  EXPECT(llmint8_linear(p, 64, 1024, p, p, 1024, 6.0f, p, (char*)p + 16, need, NULL) == INVALID);
  EXPECT(llmint8_linear(p, 64, 1000, p, p, 1024, 6.0f, p, p, need, NULL) == UNSUP);
  EXPECT(llmint8_linear(p, 0, 1024, p, p, 1024, 6.0f, p, p, need, NULL) == LLMINT8_OK);
  EXPECT(llmint8_linear_ex(p, 9, 64, 1024, p, p, 1024, 6.0f, NULL, p, p, need, NULL) == INVALID);
  EXPECT(llmint8_linear_ex(p, LLMINT8_DTYPE_BF16, 64, 1024, p, p, 1024, 6.0f, odd, p, p, need, NULL) ==
         INVALID);
  for (int path = -1; path < 25; ++path) /* an unknown path, or else the misaligned Xq copy */
    EXPECT(llmint8_linear_debug(p, 64, 1024, p, p, 1024, 6.0f, p, p, need, NULL, path, NULL, NULL, NULL,
                                mis, NULL, NULL) == INVALID);
  void* ev[4] = {p, p, p, p};
  int nk = -1;
  EXPECT(llmint8_linear_timed(p, 64, 1024, p, p, 1024, 6.0f, p, p, need, NULL, LLMINT8_PATH_GEMM, ev, 2,
                              &nk) == INVALID);

  /* workspace sizes grow with every dimension and cover the largest shapes */
  EXPECT(llmint8_workspace_bytes(2048, 4096, 11008) < llmint8_workspace_bytes(4096, 4096, 11008));
  EXPECT(llmint8_workspace_bytes(2048, 4096, 11008) < llmint8_workspace_bytes(2048, 8192, 11008));
  EXPECT(llmint8_workspace_bytes(2048, 4096, 11008) < llmint8_workspace_bytes(2048, 4096, 28672));
  EXPECT(llmint8_workspace_bytes(32767, 65536, 32767) > (size_t)32767 * 65536);
  /* bounded: the int8 activations plus 512 outlier columns of 16-bit operands */
  EXPECT(llmint8_workspace_bytes(2048, 4096, 11008) < (size_t)2048 * 4096 + (size_t)2 * 512 * (2048 + 11008) + (1 << 20));
  EXPECT(llmint8_workspace_bytes(2048, 4096, 11008) > (size_t)2048 * 4096 + (size_t)2 * 512 * (2048 + 11008));
  EXPECT(llmint8_backward_workspace_bytes(2048, 4096, 11008) == 0); /* dequantized on the fly */

  /* backward, codecs, 4-bit */
  EXPECT(llmint8_linear_backward_input(NULL, 16, 64, p, p, 64, p, p, 1 << 20, NULL) == INVALID);
  EXPECT(llmint8_dequantize_weight_t(NULL, p, 64, 64, p, NULL) == INVALID);
  EXPECT(llmint8_quantize_blockwise(p, 0, 17, 64, p, p, NULL) == UNSUP);
  EXPECT(llmint8_quantize_blockwise(p, 0, 64, 100, p, p, NULL) == UNSUP);
  EXPECT(llmint8_quantize_blockwise(p, 0, 0, 64, p, p, NULL) == LLMINT8_OK);
  EXPECT(llmint8_quantize_4bit(p, 0, 64, 48, LLMINT8_QUANT_NF4, p, p, NULL) != LLMINT8_OK);
  EXPECT(llmint8_quantize_4bit(p, 0, 64, 64, 5, p, p, NULL) == INVALID);
  EXPECT(llmint8_linear_4bit(p, 0, 1, 100, p, p, 64, LLMINT8_QUANT_NF4, 8, NULL, p, NULL) == UNSUP);
  EXPECT(llmint8_linear_4bit(p, 0, 0, 128, p, p, 64, LLMINT8_QUANT_NF4, 8, NULL, p, NULL) == LLMINT8_OK);

  /* 4-bit code books: 16 values in [-1, 1], both ends reached, repeatable */
  for (int q = 0; q < 2; ++q) {
    float v[16], w[16];
    EXPECT(llmint8_code_book_4bit(q, v) == LLMINT8_OK);
    EXPECT(llmint8_code_book_4bit(q, w) == LLMINT8_OK);
    float lo = 2.0f, hi = -2.0f;
    for (int c = 0; c < 16; ++c) {
      EXPECT(v[c] == w[c] && v[c] >= -1.0f && v[c] <= 1.0f);
      lo = v[c] < lo ? v[c] : lo;
      hi = v[c] > hi ? v[c] : hi;
    }
    EXPECT(lo == -1.0f && hi == 1.0f);
  }
  float v[16];
  EXPECT(llmint8_code_book_4bit(2, v) == INVALID);
  EXPECT(llmint8_code_book_4bit(0, NULL) == INVALID);

  /* queries */
  int prev = 1 << 30;
  for (int64_t K = 16; K <= 65536; K += 16) {
    const int r = llmint8_gemv_max_rows(K);
    EXPECT(r >= 0 && r <= 16 && r <= prev);
    prev = r;
  }
  EXPECT(llmint8_gemv_max_rows(15) == 0 && llmint8_gemv_max_rows(65552) == 0);
  for (int64_t T = 1; T <= 8192; T = T * 3 + 1)
    for (int64_t N = 1; N <= 65536; N = N * 5 + 3) {
      const int t = llmint8_gemm_tile(T, N);
      EXPECT(t >= LLMINT8_PATH_GEMM_256x256 && t <= LLMINT8_PATH_GEMM_352x256);
    }
  EXPECT(llmint8_gemm_tile(2048, 11008) == LLMINT8_PATH_GEMM_352x256);
  for (int s = -6; s <= 1; ++s) EXPECT(llmint8_status_string(s) != NULL);

  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("host check ok\n");
  return 0;
}

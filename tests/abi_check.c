/* Compiled with gcc as plain C99 against include/qr.h and linked with
 * libquarot_hip.so by tests/test_abi.py: the header is usable from C, every
 * entry point links, and the host-side validation answers as documented.
 * Only calls that return before any launch are made (no GPU is needed). */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "qr.h"

static int failures = 0;

#define EXPECT(cond)                                                 \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "%s:%d: failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                    \
    }                                                                \
  } while (0)

int main(void) {
  /* a fake, 16-byte-aligned non-null device address: never dereferenced */
  void* const A = (void*)(uintptr_t)(1u << 20);
  const hipStream_t st = NULL;
  int32_t n = -1, m = -1;

  EXPECT(qr_abi_version() == QR_ABI_VERSION);
  for (int code = QR_OK; code <= QR_ERR_SCRATCH; ++code)
    EXPECT(qr_status_str(code) != NULL && strncmp(qr_status_str(code), "QR_", 3) == 0);
  EXPECT(qr_status_str(1234) != NULL);

  EXPECT(qr_hadamard_factor(11008, &n, &m) == QR_OK && n == 6 && m == 172);
  EXPECT(qr_hadamard_factor(28672, &n, &m) == QR_OK && n == 10 && m == 28);
  EXPECT(qr_hadamard_factor(8192, &n, &m) == QR_OK && n == 13 && m == 1);
  EXPECT(qr_hadamard_factor(4097, &n, &m) == QR_ERR_UNSUPPORTED);
  EXPECT(qr_hadamard_factor(4096, NULL, NULL) == QR_ERR_NULL);

  /* empty work: QR_OK without a launch */
  EXPECT(qr_hadamard_quant(A, 0, 8192, 8192, QR_ROT_HADAMARD, NULL, 1.0f, A, A, NULL, st) == QR_OK);
  EXPECT(qr_hadamard(A, 0, 4096, 4096, NULL, A, 1, st) == QR_OK);
  EXPECT(qr_w4a4_gemm(A, A, 0, A, A, 16, 4096, A, NULL, st) == QR_OK);
  EXPECT(qr_kv_rotate_quant(A, 2, 0, 8, 128, 1024, QR_ROT_HADAMARD, NULL, 128, 0.95f, A, A, 10, 0,
                            NULL, st) == QR_OK);
  EXPECT(qr_kv_rotate_quant_bits(A, 2, 0, 8, 128, 1024, QR_ROT_NONE, NULL, 128, 0.95f, 3, A, A, 10,
                                 0, NULL, st) == QR_OK);
  EXPECT(qr_rmsnorm_quant(A, 0, 8192, 8192, 1e-5f, 1.0f, A, A, NULL, st) == QR_OK);
  EXPECT(qr_hadamard_heads_quant(A, 0, 64, 128, 8192, 1.0f, A, A, NULL, st) == QR_OK);
  EXPECT(qr_hadamard_quant_i8(A, 0, 28672, 28672, QR_ROT_HADAMARD, NULL, 1.0f, 8, A, A, NULL, st) ==
         QR_OK);
  EXPECT(qr_rmsnorm_quant_i8(A, 0, 4096, 4096, 1e-5f, 1.0f, 6, A, A, NULL, st) == QR_OK);
  EXPECT(qr_hadamard_heads_quant_i8(A, 0, 32, 128, 4096, 1.0f, 8, A, A, NULL, st) == QR_OK);
  EXPECT(qr_w8a8_gemm(A, A, 16, A, A, 0, 4096, A, NULL, st) == QR_OK);
  EXPECT(qr_kv_decode_workspace_bytes(0, 64, 8, 128, 2098) == 0);
  EXPECT(qr_kv_decode_attention(A, 0, 64, 8, 128, A, A, A, A, 2098, 2098, 128, 0.088f, A, A, 0,
                                st) == QR_OK);

  /* rejected before any launch */
  EXPECT(qr_hadamard_quant(A, 4, 4100, 4104, QR_ROT_HADAMARD, NULL, 1.0f, A, A, NULL, st) ==
         QR_ERR_UNSUPPORTED);
  EXPECT(qr_hadamard_quant(A, 4, 8192, 8192, QR_ROT_HADAMARD, NULL, 2.0f, A, A, NULL, st) ==
         QR_ERR_ARG);
  EXPECT(qr_w4a4_gemm(A, A, 16, A, A, 16, 4100, A, NULL, st) == QR_ERR_UNSUPPORTED);
  EXPECT(qr_w8a8_gemm(NULL, A, 16, A, A, 16, 4096, A, NULL, st) == QR_ERR_NULL);
  EXPECT(qr_rmsnorm_quant(A, 4, 8192, 8192, -1.0f, 1.0f, A, A, NULL, st) == QR_ERR_ARG);
  EXPECT(qr_hadamard_heads_quant(A, 4, 48, 128, 6144, 1.0f, A, A, NULL, st) == QR_ERR_UNSUPPORTED);
  EXPECT(qr_kv_rotate_quant_bits(A, 2, 3, 8, 128, 1024, QR_ROT_NONE, NULL, 128, 0.95f, 5, A, A, 10,
                                 0, NULL, st) == QR_ERR_ARG);
  EXPECT(qr_hadamard_quant_i8(A, 4, 8192, 8192, QR_ROT_HADAMARD, NULL, 1.0f, 8,
                              (char*)A + 4, A, NULL, st) == QR_ERR_ALIGN);
  EXPECT(qr_calibrate_mfma_i8(A, 0, 100, (int32_t*)A, NULL, st) == QR_ERR_SHAPE);
  EXPECT(qr_calibrate_mfma_i8(A, 8, 0, (int32_t*)A, NULL, st) == QR_ERR_SHAPE);
  EXPECT(qr_calibrate_mfma_i8(NULL, 8, 100, (int32_t*)A, NULL, st) == QR_ERR_NULL);
  EXPECT(qr_calibrate_mfma_i8((char*)A + 4, 8, 100, (int32_t*)A, NULL, st) == QR_ERR_ALIGN);
  EXPECT(qr_calibrate_stream(A, 0, A, 8, st) == QR_OK);
  EXPECT(qr_calibrate_stream(A, -1, A, 8, st) == QR_ERR_SHAPE);
  EXPECT(qr_calibrate_stream(A, 16, A, 0, st) == QR_ERR_SHAPE);
  EXPECT(qr_calibrate_stream(NULL, 16, A, 8, st) == QR_ERR_NULL);
  EXPECT(qr_calibrate_stream((char*)A + 4, 16, A, 8, st) == QR_ERR_ALIGN);

  if (failures) return 1;
  printf("abi_check: ok\n");
  return 0;
}

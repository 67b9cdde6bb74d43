/* Calls the entry points of include/qgguf.h (all but moe_qgemv_q4_k_noalloc,
 * whose source holds device memory and so cannot be built for the host
 * alone; it shares the MoE call's checks) with invalid arguments (null,
 * out-of-range and misaligned pointers and sizes, sizes at the limits) and
 * with valid-looking ones on a machine without a GPU, in a build of the
 * argument checks under AddressSanitizer / UndefinedBehaviorSanitizer.  The
 * pointers are never dereferenced by the checks.  Each call must return the
 * documented status; exit status 0 = all as documented, no sanitizer report. */
#include <stdint.h>
#include <stdio.h>

#include "../../include/qgguf.h"

static int fails = 0;
#define EXPECT(call, want)                                                                 \
  do {                                                                                     \
    qg_status got_ = (call);                                                               \
    if (got_ != (want)) {                                                                  \
      printf("%s:%d: %s -> %d (%s), want %d\n", __FILE__, __LINE__, #call, (int)got_,     \
             qg_status_str(got_), (int)(want));                                            \
      ++fails;                                                                             \
    }                                                                                      \
  } while (0)

int main(void) {
  void *A = (void *)(uintptr_t)0x100000;   /* 256-byte aligned, never dereferenced */
  void *B = (void *)(uintptr_t)0x200000;
  float *Y = (float *)(uintptr_t)0x300000;
  int32_t *I = (int32_t *)(uintptr_t)0x400000;
  void *M2 = (void *)(uintptr_t)0x100002;  /* 2-byte aligned */
  const int64_t big = (int64_t)1 << 40;
  /* quantize */
  EXPECT(quantize_q8_1(NULL, B, 1, 32, 0), QG_ERR_NULL);
  EXPECT(quantize_q8_1(Y, B, 1, 31, 0), QG_ERR_SHAPE);
  EXPECT(quantize_q8_1(Y, B, -1, 32, 0), QG_ERR_SHAPE);
  EXPECT(quantize_q8_1(Y, B, big, big, 0), QG_ERR_SHAPE);
  EXPECT(quantize_q8_1((float *)M2, B, 1, 32, 0), QG_ERR_ALIGN);
  EXPECT(quantize_q8_1(Y, B, 0, 32, 0), QG_OK);
  EXPECT(quantize_q8_1(Y, B, 1, 32, 0), QG_ERR_NO_DEVICE);
  /* GEMVs */
  qg_status (*gemv[])(const void *, const void *, float *, int64_t, int64_t, hipStream_t) = {
      qgemv_q8_0, qgemv_q4_k, qgemv_q6_k, qgemv_q5_k, qgemv_q4_0, qgemv_q5_0};
  for (int f = 0; f < 6; ++f) {
    EXPECT(gemv[f](NULL, B, Y, 1, 256, 0), QG_ERR_NULL);
    EXPECT(gemv[f](A, B, Y, 1, 250, 0), QG_ERR_SHAPE);
    EXPECT(gemv[f](A, B, Y, -3, 256, 0), QG_ERR_SHAPE);
    EXPECT(gemv[f](A, B, Y, (int64_t)1 << 31, 256, 0), QG_ERR_SHAPE);
    EXPECT(gemv[f](A, B, Y, 1, ((int64_t)1 << 24) + 256, 0), QG_ERR_SHAPE);
    EXPECT(gemv[f](M2, B, Y, 1, 256, 0), QG_ERR_ALIGN);
    EXPECT(gemv[f](A, B, Y, 0, 256, 0), QG_OK);
    EXPECT(gemv[f](A, B, Y, 5, 256, 0), QG_ERR_NO_DEVICE);
  }
  /* small-batch */
  qg_status (*gb[])(const void *, const void *, float *, int64_t, int64_t, int64_t, hipStream_t) = {
      qgemv_q8_0_batch, qgemv_q4_k_batch, qgemv_q6_k_batch};
  qg_status (*gbd[])(const void *, const void *, int32_t *, int64_t, int64_t, int64_t, hipStream_t) = {
      qg_blockdots_q8_0_batch, qg_blockdots_q4_k_batch, qg_blockdots_q6_k_batch};
  for (int f = 0; f < 3; ++f) {
    EXPECT(gb[f](A, B, Y, 9, 4, 256, 0), QG_ERR_SHAPE);
    EXPECT(gb[f](A, B, Y, 8, ((int64_t)1 << 31) - 1, 256, 0), QG_ERR_SHAPE);
    EXPECT(gb[f](A, B, NULL, 2, 4, 256, 0), QG_ERR_NULL);
    EXPECT(gb[f](A, B, Y, 0, 4, 256, 0), QG_OK);
    EXPECT(gb[f](A, B, Y, 3, 4, 256, 0), QG_ERR_NO_DEVICE);
    EXPECT(gbd[f](A, B, I, 8, (int64_t)1 << 30, 4096, 0), QG_ERR_SHAPE);
    EXPECT(gbd[f](A, B, I, 2, 4, 256, 0), QG_ERR_NO_DEVICE);
  }
  /* mmq */
  qg_status (*mm[])(const void *, const void *, float *, int64_t, int64_t, int64_t, hipStream_t) = {
      qgemm_q4_k_mmq, qgemm_q6_k_mmq, qgemm_q8_0_mmq, qgemm_q5_k_mmq, qgemm_q4_0_mmq, qgemm_q5_0_mmq};
  qg_status (*mmd[])(const void *, const void *, int32_t *, int64_t, int64_t, int64_t, hipStream_t) = {
      qg_blockdots_q4_k_mmq, qg_blockdots_q6_k_mmq, qg_blockdots_q8_0_mmq, qg_blockdots_q5_k_mmq,
      qg_blockdots_q4_0_mmq, qg_blockdots_q5_0_mmq};
  for (int f = 0; f < 6; ++f) {
    EXPECT(mm[f](A, B, Y, ((int64_t)1 << 31) - 1, ((int64_t)1 << 31) - 1, 256, 0), QG_ERR_SHAPE);
    EXPECT(mm[f](A, B, Y, -1, 4, 256, 0), QG_ERR_SHAPE);
    EXPECT(mm[f](A, M2, Y, 4, 4, 256, 0), QG_ERR_ALIGN);
    EXPECT(mm[f](A, B, Y, 0, 4, 256, 0), QG_OK);
    EXPECT(mm[f](A, B, Y, 4, 4, 256, 0), QG_ERR_NO_DEVICE);
    EXPECT(mmd[f](A, B, I, (int64_t)1 << 20, (int64_t)1 << 20, 4096, 0), QG_ERR_SHAPE);
  }
  /* block dots */
  EXPECT(qg_blockdots_q4_k(A, B, I, NULL, 4, 256, 0), QG_ERR_NULL);
  EXPECT(qg_blockdots_q5_k(A, B, I, (int32_t *)M2, 4, 256, 0), QG_ERR_ALIGN);
  EXPECT(qg_blockdots_q6_k(A, B, I, 4, 256, 0), QG_ERR_NO_DEVICE);
  EXPECT(qg_blockdots_q8_0(A, B, I, 4, 32, 0), QG_ERR_NO_DEVICE);
  EXPECT(qg_blockdots_q4_0(A, B, I, 4, 64, 0), QG_ERR_NO_DEVICE);
  EXPECT(qg_blockdots_q5_0(A, B, I, 4, 96, 0), QG_ERR_SHAPE);
  /* rmsnorm */
  EXPECT(rmsnorm_quantize_q8_1(Y, Y, -1.0f, B, NULL, 1, 32, 0), QG_ERR_SHAPE);
  EXPECT(rmsnorm_quantize_q8_1(Y, Y, 1.0f / 0.0f, B, NULL, 1, 32, 0), QG_ERR_SHAPE);
  EXPECT(rmsnorm_quantize_q8_1(Y, Y, 1e-5f, B, (float *)M2, 1, 32, 0), QG_ERR_ALIGN);
  EXPECT(rmsnorm_quantize_q8_1(Y, Y, 1e-5f, B, NULL, 2, 64, 0), QG_ERR_NO_DEVICE);
  /* router */
  EXPECT(moe_router_topk(Y, Y, I, Y, Y, 4, 257, 64, 8, 0), QG_ERR_SHAPE);
  EXPECT(moe_router_topk(Y, Y, I, Y, Y, 4, 8, 64, 9, 0), QG_ERR_SHAPE);
  EXPECT(moe_router_topk(Y, NULL, NULL, NULL, NULL, 0, 8, 64, 2, 0), QG_OK);
  EXPECT(moe_router_topk(Y, Y, I, Y, Y, 4, 8, 64, 2, 0), QG_ERR_NO_DEVICE);
  /* MoE */
  const size_t ws = moe_qgemv_q4_k_workspace_size(16, 8, 128, 768, 2048);
  if (ws == 0 || ws % 256) { printf("workspace size %zu\n", ws); ++fails; }
  if (moe_qgemv_q4_k_workspace_size(-1, 8, 128, 768, 2048) != 0) { printf("negative size\n"); ++fails; }
  EXPECT(moe_qgemv_q4_k(A, A, B, I, Y, Y, 16, 8, 128, 768, 2048, A, ws - 1, 0), QG_ERR_WORKSPACE);
  EXPECT(moe_qgemv_q4_k(A, A, B, I, Y, Y, 16, 8, 128, 768, 2048, M2, ws, 0), QG_ERR_ALIGN);
  EXPECT(moe_qgemv_q4_k(A, A, B, I, Y, Y, 16, 65, 128, 768, 2048, A, ws, 0), QG_ERR_SHAPE);
  EXPECT(moe_qgemv_q4_k(A, A, B, I, Y, Y, 16, 8, 128, 700, 2048, A, ws, 0), QG_ERR_SHAPE);
  EXPECT(moe_qgemv_q4_k(A, A, B, I, Y, Y, (int64_t)1 << 20, 8, 128, 768, 2048, A, ws, 0), QG_ERR_SHAPE);
  EXPECT(moe_qgemv_q4_k(A, A, B, I, Y, NULL, 16, 8, 128, 768, 2048, A, ws, 0), QG_ERR_NULL);
  EXPECT(moe_qgemv_q4_k(A, A, B, I, Y, Y, 16, 8, 128, 768, 2048, A, ws, 0), QG_ERR_NO_DEVICE);
  EXPECT(qg_blockdots_moe_q4_k(A, A, B, I, Y, 16, 8, 128, 768, 2048, A, ws, I, NULL, 0), QG_ERR_NULL);
  EXPECT(qg_blockdots_moe_q4_k(A, A, B, I, Y, 4096, 8, 128, 768, 2048, A, (size_t)1 << 40, I, I, 0), QG_ERR_SHAPE);
  if (qg_moe_q4_k_launches(16, 8, 128, 700, 2048) != 0) { printf("launches of an invalid shape\n"); ++fails; }
  /* measurement references */
  EXPECT(qg_peak_read(A, 1000, (uint32_t *)I, 64, 64, 256, 4, 1, 0), QG_ERR_SHAPE);
  EXPECT(qg_peak_read(A, 1024, (uint32_t *)I, 63, 64, 256, 4, 1, 0), QG_ERR_SHAPE);
  EXPECT(qg_peak_read(A, 1024, (uint32_t *)I, 64, 64, 256, 5, 1, 0), QG_ERR_SHAPE);
  EXPECT(qg_peak_read(A, 1024, (uint32_t *)I, 64, 64, 256, 8, 0, 0), QG_ERR_NO_DEVICE);
  int64_t ops = 0;
  EXPECT(qg_peak_mfma_i8(I, 1 << 16, 0, &ops, 0), QG_ERR_SHAPE);
  EXPECT(qg_peak_mfma_i8(I, 1 << 16, 10, NULL, 0), QG_ERR_NULL);
  for (int s = 0; s <= 8; ++s)
    if (!qg_status_str((qg_status)s)) ++fails;
  printf(fails ? "api driver: %d unexpected statuses\n" : "api driver: all statuses as documented%.0d\n", fails);
  return fails != 0;
}

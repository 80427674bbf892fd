/*
 * A plain C caller of the KDA C ABI (include/kda.h): no Python, no torch.
 *
 *   kda_capi_check DIR B T H DK DV CHUNK
 *
 * Reads from DIR the bfloat16 inputs q, k, v, g, beta of a prefill ([B,T,H,*], raw
 * little-endian bfloat16 bits, files q.bin ...) and its float32 initial state s0.bin
 * ([B,H,DK,DV]); runs kda_chunk_fwd (float32 output, the library's own segmentation
 * with a workspace of the size it asks for) and then one kda_recurrent_step that feeds
 * each sequence's last token again to the final states; writes o.bin, s.bin (after the
 * prefill), od.bin and sd.bin (after the step), all float32.  Exit status 0 on success;
 * a failing call prints its status string and exits 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kda.h"

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(2); }
  void* p = malloc(bytes);
  if (!p || fread(p, 1, bytes, f) != bytes) { fprintf(stderr, "short read %s\n", path); exit(2); }
  fclose(f);
  return p;
}

static void write_file(const char* dir, const char* name, const void* p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(p, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(2); }
  fclose(f);
}

static void* to_device(const void* h, size_t bytes) {
  void* d = NULL;
  if (hipMalloc(&d, bytes) != hipSuccess || hipMemcpy(d, h, bytes, hipMemcpyHostToDevice) != hipSuccess) {
    fprintf(stderr, "device copy failed\n");
    exit(2);
  }
  return d;
}

static void check(kda_status_t st, const char* what) {
  if (st != KDA_OK) {
    fprintf(stderr, "%s: %s\n", what, kda_status_str(st));
    exit(1);
  }
}

int main(int argc, char** argv) {
  if (argc != 8) {
    fprintf(stderr, "usage: %s DIR B T H DK DV CHUNK\n", argv[0]);
    return 2;
  }
  const char* dir = argv[1];
  const int64_t B = atoll(argv[2]), T = atoll(argv[3]), H = atoll(argv[4]);
  const int dk = atoi(argv[5]), dv = atoi(argv[6]), chunk = atoi(argv[7]);
  const size_t ntok = (size_t)(B * T * H);
  const size_t nstate = (size_t)(B * H) * (size_t)dk * (size_t)dv;

  void* q = to_device(read_file(dir, "q.bin", ntok * dk * 2), ntok * dk * 2);
  void* k = to_device(read_file(dir, "k.bin", ntok * dk * 2), ntok * dk * 2);
  void* v = to_device(read_file(dir, "v.bin", ntok * dv * 2), ntok * dv * 2);
  void* g = to_device(read_file(dir, "g.bin", ntok * dk * 2), ntok * dk * 2);
  void* beta = to_device(read_file(dir, "beta.bin", ntok * 2), ntok * 2);
  float* s0 = (float*)to_device(read_file(dir, "s0.bin", nstate * 4), nstate * 4);

  float *o = NULL, *s = NULL;
  void* ws = NULL;
  const size_t ws_bytes = kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, KDA_BF16);
  if (hipMalloc((void**)&o, ntok * dv * 4) != hipSuccess || hipMalloc((void**)&s, nstate * 4) != hipSuccess ||
      (ws_bytes && hipMalloc(&ws, ws_bytes) != hipSuccess)) {
    fprintf(stderr, "allocation failed\n");
    return 2;
  }
  check(kda_chunk_fwd(q, k, v, g, beta, s0, o, s, NULL, 0, B, T, H, dk, dv, chunk, KDA_BF16,
                      KDA_F32, ws, ws_bytes, NULL),
        "kda_chunk_fwd");
  if (hipDeviceSynchronize() != hipSuccess) { fprintf(stderr, "prefill failed\n"); return 2; }
  float* ho = (float*)malloc(ntok * dv * 4);
  float* hs = (float*)malloc(nstate * 4);
  hipMemcpy(ho, o, ntok * dv * 4, hipMemcpyDeviceToHost);
  hipMemcpy(hs, s, nstate * 4, hipMemcpyDeviceToHost);
  write_file(dir, "o.bin", ho, ntok * dv * 4);
  write_file(dir, "s.bin", hs, nstate * 4);

  /* one decode step: N = B sequences, each fed its last token again ([B,T,H,d] rows T-1) */
  const size_t nh = (size_t)(B * H);
  void *dq, *dk_, *dv_, *dg, *db;
  float* od = NULL;
  if (hipMalloc(&dq, nh * dk * 2) != hipSuccess || hipMalloc(&dk_, nh * dk * 2) != hipSuccess ||
      hipMalloc(&dv_, nh * dv * 2) != hipSuccess || hipMalloc(&dg, nh * dk * 2) != hipSuccess ||
      hipMalloc(&db, nh * 2) != hipSuccess || hipMalloc((void**)&od, nh * dv * 4) != hipSuccess) {
    fprintf(stderr, "allocation failed\n");
    return 2;
  }
  for (int64_t b = 0; b < B; ++b) {
    const size_t row = (size_t)((b * T + (T - 1)) * H);  /* token T-1 of sequence b */
    hipMemcpy((char*)dq + b * H * dk * 2, (char*)q + row * dk * 2, H * dk * 2, hipMemcpyDeviceToDevice);
    hipMemcpy((char*)dk_ + b * H * dk * 2, (char*)k + row * dk * 2, H * dk * 2, hipMemcpyDeviceToDevice);
    hipMemcpy((char*)dv_ + b * H * dv * 2, (char*)v + row * dv * 2, H * dv * 2, hipMemcpyDeviceToDevice);
    hipMemcpy((char*)dg + b * H * dk * 2, (char*)g + row * dk * 2, H * dk * 2, hipMemcpyDeviceToDevice);
    hipMemcpy((char*)db + b * H * 2, (char*)beta + row * 2, H * 2, hipMemcpyDeviceToDevice);
  }
  check(kda_recurrent_step(dq, dk_, dv_, dg, db, s, od, B, H, dk, dv, KDA_BF16, KDA_F32, NULL),
        "kda_recurrent_step");
  if (hipDeviceSynchronize() != hipSuccess) { fprintf(stderr, "decode failed\n"); return 2; }
  float* hod = (float*)malloc(nh * dv * 4);
  hipMemcpy(hod, od, nh * dv * 4, hipMemcpyDeviceToHost);
  hipMemcpy(hs, s, nstate * 4, hipMemcpyDeviceToHost);
  write_file(dir, "od.bin", hod, nh * dv * 4);
  write_file(dir, "sd.bin", hs, nstate * 4);
  printf("ok B%lld T%lld H%lld dk%d dv%d chunk %d, workspace %zu bytes\n", (long long)B,
         (long long)T, (long long)H, dk, dv, chunk, ws_bytes);
  return 0;
}

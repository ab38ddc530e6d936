/* The layer's forward driven from C alone (no Python, no PyTorch in the process):
 *   c_forward <dir> T d N Z K I
 * reads <dir>/x.bin (bf16 [T][d]), w_router.bin (fp32 [N+Z][d]), bias.bin (fp32 [N+Z]),
 * w_gate.bin and w_up.bin (bf16 [N][I][d]), w_down.bin (bf16 [N][d][I]); allocates device
 * buffers and the workspace with hipMalloc, runs lc_moe_forward on the null stream and
 * writes y.bin (bf16 [T][d]), idx.bin (int32 [T][K]), gate.bin (fp32 [T][K]) and
 * load.bin (int32 [N+Z]).  Exit status 0 on success. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "lc_moe.h"

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* p = malloc(bytes ? bytes : 1);
  if (p && fread(p, 1, bytes, f) != bytes) {
    free(p);
    p = NULL;
  }
  fclose(f);
  return p;
}

static int write_file(const char* dir, const char* name, const void* p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return 1;
  const int bad = fwrite(p, 1, bytes, f) != bytes;
  return fclose(f) != 0 || bad;
}

/* host bytes -> new device buffer */
static void* upload(const void* host, size_t bytes) {
  void* d = NULL;
  if (hipMalloc(&d, bytes) != hipSuccess) return NULL;
  if (hipMemcpy(d, host, bytes, hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return d;
}

int main(int argc, char** argv) {
  if (argc != 8) {
    fprintf(stderr, "usage: %s dir T d N Z K I\n", argv[0]);
    return 2;
  }
  const char* dir = argv[1];
  lc_moe_shape s;
  s.T = atoi(argv[2]);
  s.d = atoi(argv[3]);
  s.N = atoi(argv[4]);
  s.Z = atoi(argv[5]);
  s.K = atoi(argv[6]);
  s.I = atoi(argv[7]);
  s.dtype = LC_MOE_BF16;
  const size_t T = s.T, d = s.d, N = s.N, E = (size_t)s.N + s.Z, K = s.K, I = s.I;
  const size_t b_x = T * d * 2, b_wr = E * d * 4, b_b = E * 4, b_w = N * I * d * 2;
  void* hx = read_file(dir, "x.bin", b_x);
  void* hwr = read_file(dir, "w_router.bin", b_wr);
  void* hb = read_file(dir, "bias.bin", b_b);
  void* hg = read_file(dir, "w_gate.bin", b_w);
  void* hu = read_file(dir, "w_up.bin", b_w);
  void* hd = read_file(dir, "w_down.bin", b_w);
  if (!hx || !hwr || !hb || !hg || !hu || !hd) {
    fprintf(stderr, "input files missing or short\n");
    return 3;
  }
  const size_t ws_bytes = lc_moe_workspace_size(&s);
  if (ws_bytes == 0) {
    fprintf(stderr, "shape outside the limits\n");
    return 4;
  }
  lc_moe_weights w;
  memset(&w, 0, sizeof w);
  void* x = upload(hx, b_x);
  w.w_router = (const float*)upload(hwr, b_wr);
  w.bias = (const float*)upload(hb, b_b);
  w.w_gate = upload(hg, b_w);
  w.w_up = upload(hu, b_w);
  w.w_down = upload(hd, b_w);
  void *y = NULL, *idx = NULL, *gate = NULL, *load = NULL, *ws = NULL;
  if (!x || !w.w_router || !w.bias || !w.w_gate || !w.w_up || !w.w_down || hipMalloc(&y, b_x) != hipSuccess ||
      hipMalloc(&idx, T * K * 4) != hipSuccess || hipMalloc(&gate, T * K * 4) != hipSuccess ||
      hipMalloc(&load, E * 4) != hipSuccess || hipMalloc(&ws, ws_bytes) != hipSuccess) {
    fprintf(stderr, "device allocation or upload failed\n");
    return 5;
  }
  const lc_moe_status st = lc_moe_forward(&s, x, &w, y, (int32_t*)idx, (float*)gate, (int32_t*)load, ws, ws_bytes, 0);
  if (st != LC_MOE_OK) {
    fprintf(stderr, "lc_moe_forward: %s\n", lc_moe_status_str(st));
    return 6;
  }
  if (hipDeviceSynchronize() != hipSuccess) {
    fprintf(stderr, "device error\n");
    return 7;
  }
  void* hy = malloc(b_x);
  void* hidx = malloc(T * K * 4);
  void* hgate = malloc(T * K * 4);
  void* hload = malloc(E * 4);
  if (!hy || !hidx || !hgate || !hload || hipMemcpy(hy, y, b_x, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(hidx, idx, T * K * 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(hgate, gate, T * K * 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(hload, load, E * 4, hipMemcpyDeviceToHost) != hipSuccess) {
    fprintf(stderr, "download failed\n");
    return 8;
  }
  if (write_file(dir, "y.bin", hy, b_x) || write_file(dir, "idx.bin", hidx, T * K * 4) ||
      write_file(dir, "gate.bin", hgate, T * K * 4) || write_file(dir, "load.bin", hload, E * 4)) {
    fprintf(stderr, "writing outputs failed\n");
    return 9;
  }
  printf("c_forward ok\n");
  return 0;
}

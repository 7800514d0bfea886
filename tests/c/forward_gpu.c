/* A plain C caller of the whole block on the GPU: reads one layer's inputs
 * from raw files, copies them to device memory it allocates itself, runs
 * moe_forward on the default stream with a workspace of moe_workspace_size
 * bytes, and writes the output back to a file.
 *
 *   forward_gpu DIR
 *
 * DIR/meta.txt holds "N H E top_k I I_shared norm_topk_prob dtype"
 * (dtype: 0 float32, 1 bfloat16); DIR/x.bin, router_w.bin, w_gate_up.bin,
 * w_down.bin (and shared_w_gate_up.bin, shared_w_down.bin, shared_gate.bin
 * when I_shared > 0) hold the row-major tensors as raw elements.  The
 * output goes to DIR/out.bin.  Exit status 0 on success. */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_mi355x.h"

static const char* g_dir;

static int check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 1;
  }
  return 0;
}

/* Reads DIR/name (exactly `bytes` bytes) into new device memory. */
static void* load(const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", g_dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path);
    return NULL;
  }
  void* host = malloc(bytes ? bytes : 1);
  const size_t got = host ? fread(host, 1, bytes, f) : 0;
  const int extra = fgetc(f) != EOF;
  fclose(f);
  void* dev = NULL;
  if (!host || got != bytes || extra) {
    fprintf(stderr, "%s: expected %zu bytes\n", path, bytes);
  } else if (check_hip(hipMalloc(&dev, bytes ? bytes : 1), "hipMalloc") ||
             check_hip(hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice), "hipMemcpy")) {
    dev = NULL;
  }
  free(host);
  return dev;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s DIR\n", argv[0]);
    return 2;
  }
  g_dir = argv[1];
  char path[4096];
  snprintf(path, sizeof path, "%s/meta.txt", g_dir);
  FILE* f = fopen(path, "r");
  long long N, H, E, k, I, Is;
  int norm, dtype;
  if (!f || fscanf(f, "%lld %lld %lld %lld %lld %lld %d %d", &N, &H, &E, &k, &I, &Is, &norm, &dtype) != 8) {
    fprintf(stderr, "cannot read %s\n", path);
    return 2;
  }
  fclose(f);

  moe_problem p;
  memset(&p, 0, sizeof p);
  p.num_tokens = N;
  p.hidden = H;
  p.num_experts = E;
  p.top_k = k;
  p.inter = I;
  p.shared_inter = Is;
  p.dtype = dtype;
  p.norm_topk_prob = norm;
  const size_t es = dtype == MOE_BF16 ? 2 : 4;

  void* x = load("x.bin", (size_t)(N * H) * es);
  void* router_w = load("router_w.bin", (size_t)(E * H) * es);
  void* w_gate_up = load("w_gate_up.bin", (size_t)(E * 2 * I * H) * es);
  void* w_down = load("w_down.bin", (size_t)(E * H * I) * es);
  void *s_gate_up = NULL, *s_down = NULL, *s_gate = NULL;
  if (Is > 0) {
    s_gate_up = load("shared_w_gate_up.bin", (size_t)(2 * Is * H) * es);
    s_down = load("shared_w_down.bin", (size_t)(H * Is) * es);
    s_gate = load("shared_gate.bin", (size_t)H * es);
    if (!s_gate_up || !s_down || !s_gate) return 1;
  }
  if (!x || !router_w || !w_gate_up || !w_down) return 1;

  size_t ws_bytes = 0;
  if (moe_workspace_size(&p, &ws_bytes) != MOE_OK) {
    fprintf(stderr, "moe_workspace_size: %s\n", moe_last_error());
    return 1;
  }
  const size_t out_bytes = (size_t)(N * H) * es;
  void *workspace = NULL, *out = NULL;
  if (check_hip(hipMalloc(&workspace, ws_bytes ? ws_bytes : 1), "hipMalloc") ||
      check_hip(hipMalloc(&out, out_bytes ? out_bytes : 1), "hipMalloc"))
    return 1;
  const int rc = moe_forward(&p, x, router_w, w_gate_up, w_down, s_gate_up, s_down, s_gate, out, workspace,
                             ws_bytes, NULL);
  if (rc != MOE_OK) {
    fprintf(stderr, "moe_forward: %d %s\n", rc, moe_last_error());
    return 1;
  }
  void* host = malloc(out_bytes ? out_bytes : 1);
  if (!host || check_hip(hipDeviceSynchronize(), "hipDeviceSynchronize") ||
      check_hip(hipMemcpy(host, out, out_bytes, hipMemcpyDeviceToHost), "hipMemcpy"))
    return 1;
  snprintf(path, sizeof path, "%s/out.bin", g_dir);
  f = fopen(path, "wb");
  if (!f || fwrite(host, 1, out_bytes, f) != out_bytes) {
    fprintf(stderr, "cannot write %s\n", path);
    return 1;
  }
  fclose(f);
  free(host);
  void* bufs[] = {x, router_w, w_gate_up, w_down, s_gate_up, s_down, s_gate, workspace, out};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i)
    if (bufs[i]) hipFree(bufs[i]);
  printf("forward_gpu: N=%lld H=%lld E=%lld k=%lld I=%lld I_shared=%lld workspace %zu bytes\n", N, H, E, k, I, Is,
         ws_bytes);
  return 0;
}

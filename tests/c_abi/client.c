/* A plain C client of libgqa: no Python, no torch. It reads a prefill and a decode case
 * from a raw file, moves them to the GPU with the HIP runtime, calls gqa_prefill and
 * gqa_decode (with the K/V append), and writes both outputs and the appended cache row back
 * to a raw file for the test to compare with the oracle.
 *
 * Input file (little endian): int32 B, T, H, G, d, S (decode cache rows per sequence),
 * then bf16 arrays: prefill q [B*T, H, d], k [B*T, G, d], v [B*T, G, d], gamma_q [d],
 * gamma_k [d]; decode q [B, H, d], k_new [B, G, d], v_new [B, G, d], k_cache and v_cache
 * [B, S, G, d]; int32 seq_lens [B] (counting the new token).
 * Output file: bf16 prefill out [B*T, H, d], decode out [B, H, d], then k_cache and
 * v_cache after the call. Exit status 0 on success, 1 with a message otherwise. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "gqa.h"

#define CHECK_HIP(x)                                                     \
  do {                                                                   \
    hipError_t e_ = (x);                                                 \
    if (e_ != hipSuccess) {                                              \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));     \
      exit(1);                                                           \
    }                                                                    \
  } while (0)
#define CHECK_GQA(x)                                                     \
  do {                                                                   \
    gqa_status s_ = (x);                                                 \
    if (s_ != GQA_OK) {                                                  \
      fprintf(stderr, "%s failed: %s\n", #x, gqa_status_str(s_));        \
      exit(1);                                                           \
    }                                                                    \
  } while (0)

static void* read_exact(FILE* f, size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p || fread(p, 1, n, f) != n) {
    fprintf(stderr, "short input\n");
    exit(1);
  }
  return p;
}

static void* to_device(const void* h, size_t n) {
  void* d = NULL;
  CHECK_HIP(hipMalloc(&d, n ? n : 1));
  CHECK_HIP(hipMemcpy(d, h, n, hipMemcpyHostToDevice));
  return d;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s input output\n", argv[0]);
    return 1;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) {
    fprintf(stderr, "cannot open %s\n", argv[1]);
    return 1;
  }
  int32_t hdr[6];
  if (fread(hdr, sizeof(int32_t), 6, in) != 6) {
    fprintf(stderr, "short header\n");
    return 1;
  }
  const int B = hdr[0], T = hdr[1], H = hdr[2], G = hdr[3], d = hdr[4], S = hdr[5];
  const size_t N = (size_t)B * T, e = 2;
  const size_t nq = N * H * d * e, nk = N * G * d * e, ng = (size_t)d * e;
  const size_t dq = (size_t)B * H * d * e, dk = (size_t)B * G * d * e;
  const size_t nc = (size_t)B * S * G * d * e;
  void* h_q = read_exact(in, nq);
  void* h_k = read_exact(in, nk);
  void* h_v = read_exact(in, nk);
  void* h_gq = read_exact(in, ng);
  void* h_gk = read_exact(in, ng);
  void* h_dq = read_exact(in, dq);
  void* h_kn = read_exact(in, dk);
  void* h_vn = read_exact(in, dk);
  void* h_kc = read_exact(in, nc);
  void* h_vc = read_exact(in, nc);
  int32_t* h_len = (int32_t*)read_exact(in, (size_t)B * 4);
  fclose(in);

  void *q = to_device(h_q, nq), *k = to_device(h_k, nk), *v = to_device(h_v, nk);
  void *gq = to_device(h_gq, ng), *gk = to_device(h_gk, ng);
  void *out = NULL, *dout = NULL;
  CHECK_HIP(hipMalloc(&out, nq));
  CHECK_HIP(hipMalloc(&dout, dq));

  gqa_params p;
  gqa_params_init(&p);
  p.q_norm_w = gq;
  p.k_norm_w = gk;
  size_t ws_bytes = gqa_workspace_bytes(GQA_OP_PREFILL, B, T, H, G, d, GQA_BF16);
  const size_t ws_dec = gqa_workspace_bytes(GQA_OP_DECODE, B, S, H, G, d, GQA_BF16);
  if (ws_dec > ws_bytes) ws_bytes = ws_dec;
  void* ws = NULL;
  CHECK_HIP(hipMalloc(&ws, ws_bytes));
  p.workspace = ws;
  p.workspace_bytes = ws_bytes;
  CHECK_GQA(gqa_prefill(q, k, v, NULL, out, B, T, H, G, d, 1, &p));

  void *dqd = to_device(h_dq, dq), *kn = to_device(h_kn, dk), *vn = to_device(h_vn, dk);
  void *kc = to_device(h_kc, nc), *vc = to_device(h_vc, nc);
  int32_t* lens = (int32_t*)to_device(h_len, (size_t)B * 4);
  p.k_new = kn;
  p.v_new = vn;
  CHECK_GQA(gqa_decode(dqd, kc, vc, lens, dout, B, H, G, d, S, &p));
  CHECK_HIP(hipDeviceSynchronize());

  void* h_out = malloc(nq);
  void* h_dout = malloc(dq);
  if (!h_out || !h_dout) return 1;
  CHECK_HIP(hipMemcpy(h_out, out, nq, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(h_dout, dout, dq, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(h_kc, kc, nc, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(h_vc, vc, nc, hipMemcpyDeviceToHost));
  FILE* o = fopen(argv[2], "wb");
  if (!o || fwrite(h_out, 1, nq, o) != nq || fwrite(h_dout, 1, dq, o) != dq ||
      fwrite(h_kc, 1, nc, o) != nc || fwrite(h_vc, 1, nc, o) != nc) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 1;
  }
  fclose(o);
  return 0;
}

// A C++ program that uses the library through its C-ABI alone (include/lwm_attn.h, no Python):
// it reads bf16 Q, K, V, dO and int32 segment ids from files, builds the block table, runs the
// forward (FINAL) and the backward on one stream, and writes O, LSE, dQ, dK, dV to files.
// Test infrastructure and a usage example; tests/test_gpu_capi.py builds the inputs, runs it
// as a child process and compares its outputs with the float64 oracle.
//
// usage: capi_example B H S DIR   (DIR holds q.bin k.bin v.bin do.bin seg.bin; outputs are
//        written there as o.bin lse.bin dq.bin dk.bin dv.bin)
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "lwm_attn.h"

namespace {

bool read_file(const std::string& path, void* dst, size_t bytes) {
  FILE* f = std::fopen(path.c_str(), "rb");
  if (!f) return false;
  const size_t n = std::fread(dst, 1, bytes, f);
  std::fclose(f);
  return n == bytes;
}

bool write_file(const std::string& path, const void* src, size_t bytes) {
  FILE* f = std::fopen(path.c_str(), "wb");
  if (!f) return false;
  const size_t n = std::fwrite(src, 1, bytes, f);
  std::fclose(f);
  return n == bytes;
}

#define HIP_OK(x)                                                                \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));        \
      return 1;                                                                  \
    }                                                                            \
  } while (0)

#define LWM_OK_OR_FAIL(x)                                                        \
  do {                                                                           \
    int rc_ = (x);                                                               \
    if (rc_ != LWM_OK) {                                                         \
      std::fprintf(stderr, "%s failed: %s\n", #x, lwm_attn_status_string(rc_));  \
      return 1;                                                                  \
    }                                                                            \
  } while (0)

}  // namespace

int main(int argc, char** argv) {
  if (argc != 5) {
    std::fprintf(stderr, "usage: %s B H S DIR\n", argv[0]);
    return 2;
  }
  const int B = std::atoi(argv[1]), H = std::atoi(argv[2]), S = std::atoi(argv[3]), D = 128;
  const std::string dir = argv[4];
  if (B <= 0 || H <= 0 || S <= 0) return 2;

  lwm_attn_desc d = {};
  d.B = B;
  d.H = H;
  d.Sq = S;
  d.Sk = S;
  d.D = D;
  d.scale = 1.0f / std::sqrt(float(D));
  d.causal = 1;
  d.block_q = 64;
  d.block_k = 64;
  d.dtype = LWM_BF16;

  const size_t elems = size_t(B) * H * S * D, rows = size_t(B) * H * S;
  std::vector<uint16_t> host(elems);
  std::vector<int32_t> seg(size_t(B) * S);
  void *q, *k, *v, *dO, *o, *dq, *dk, *dv, *table, *ws;
  int32_t* segd;
  float* lse;
  void** tensors[] = {&q, &k, &v, &dO, &o, &dq, &dk, &dv};
  for (void** t : tensors) HIP_OK(hipMalloc(t, elems * 2));
  HIP_OK(hipMalloc(&segd, seg.size() * 4));
  HIP_OK(hipMalloc(&lse, rows * 4));
  const char* names[] = {"q", "k", "v", "do"};
  void* inputs[] = {q, k, v, dO};
  for (int i = 0; i < 4; ++i) {
    if (!read_file(dir + "/" + names[i] + ".bin", host.data(), elems * 2)) {
      std::fprintf(stderr, "cannot read %s.bin\n", names[i]);
      return 1;
    }
    HIP_OK(hipMemcpy(inputs[i], host.data(), elems * 2, hipMemcpyHostToDevice));
  }
  if (!read_file(dir + "/seg.bin", seg.data(), seg.size() * 4)) return 1;
  HIP_OK(hipMemcpy(segd, seg.data(), seg.size() * 4, hipMemcpyHostToDevice));

  const size_t table_bytes = lwm_attn_block_table_bytes(&d);
  const size_t ws_bytes = lwm_attn_bwd_workspace_bytes(&d);
  if (table_bytes == 0 || ws_bytes == 0) {
    std::fprintf(stderr, "size queries rejected the descriptor\n");
    return 1;
  }
  HIP_OK(hipMalloc(&table, table_bytes));
  HIP_OK(hipMalloc(&ws, ws_bytes));
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));

  LWM_OK_OR_FAIL(lwm_attn_build_block_table(&d, segd, segd, table, stream));
  LWM_OK_OR_FAIL(lwm_attn_fwd(&d, LWM_OUT_FINAL, q, k, v, segd, segd, table, o, lse, nullptr,
                              nullptr, nullptr, stream));
  LWM_OK_OR_FAIL(lwm_attn_bwd(&d, q, k, v, o, dO, lse, segd, segd, table, dq, dk, dv, ws, ws_bytes,
                              stream));
  // a call the library must refuse: a workspace one byte short
  if (lwm_attn_bwd(&d, q, k, v, o, dO, lse, segd, segd, table, dq, dk, dv, ws, ws_bytes - 1,
                   stream) != LWM_ERR_WORKSPACE) {
    std::fprintf(stderr, "a short workspace was not refused\n");
    return 1;
  }
  HIP_OK(hipStreamSynchronize(stream));

  const char* outs[] = {"o", "dq", "dk", "dv"};
  void* outd[] = {o, dq, dk, dv};
  for (int i = 0; i < 4; ++i) {
    HIP_OK(hipMemcpy(host.data(), outd[i], elems * 2, hipMemcpyDeviceToHost));
    if (!write_file(dir + "/" + outs[i] + ".bin", host.data(), elems * 2)) return 1;
  }
  std::vector<float> lse_h(rows);
  HIP_OK(hipMemcpy(lse_h.data(), lse, rows * 4, hipMemcpyDeviceToHost));
  if (!write_file(dir + "/lse.bin", lse_h.data(), rows * 4)) return 1;

  HIP_OK(hipStreamDestroy(stream));
  for (void** t : tensors) HIP_OK(hipFree(*t));
  HIP_OK(hipFree(segd));
  HIP_OK(hipFree(lse));
  HIP_OK(hipFree(table));
  HIP_OK(hipFree(ws));
  std::printf("capi_example: B=%d H=%d S=%d done\n", B, H, S);
  return 0;
}

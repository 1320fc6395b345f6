// A plain C++ caller of the decode library: HIP runtime calls and the C header
// only (no Python, no torch).  Test infrastructure: the GPU test writes a
// seeded workload into a folder, runs this program on it and compares the
// outputs with the float64 oracle.
//
// usage: mla_c_caller DIR
//   DIR/meta.txt : batch heads q_len page_size num_pages bt_stride max_seq_len causal bmm1 bmm2
//   DIR/q.bin    : bf16 [batch * q_len * heads * 576]
//   DIR/kv.bin   : bf16 [num_pages * page_size * 576]
//   DIR/bt.bin   : int32 [batch * bt_stride]
//   DIR/lens.bin : int32 [batch]
// writes DIR/out.bin (bf16 [batch * q_len * heads * 512]) and DIR/lse.bin
// (float32 [batch * q_len * heads]); exits with the library's status code, or
// 100 + n for an I/O or runtime failure.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "mla_decode.h"

namespace {

template <typename T>
bool read_file(const std::string& path, std::vector<T>& v, size_t n) {
  FILE* f = std::fopen(path.c_str(), "rb");
  if (f == nullptr) return false;
  v.resize(n);
  const size_t got = std::fread(v.data(), sizeof(T), n, f);
  std::fclose(f);
  return got == n;
}

template <typename T>
bool write_file(const std::string& path, const std::vector<T>& v) {
  FILE* f = std::fopen(path.c_str(), "wb");
  if (f == nullptr) return false;
  const size_t put = std::fwrite(v.data(), sizeof(T), v.size(), f);
  std::fclose(f);
  return put == v.size();
}

template <typename T>
T* to_device(const std::vector<T>& v) {
  void* p = nullptr;
  if (hipMalloc(&p, v.size() * sizeof(T)) != hipSuccess) return nullptr;
  if (hipMemcpy(p, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess) return nullptr;
  return static_cast<T*>(p);
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) {
    std::fprintf(stderr, "usage: %s DIR\n", argv[0]);
    return 101;
  }
  const std::string dir = argv[1];
  int B, H, SQ, PS, BTW, max_len, causal;
  long long num_pages;
  float bmm1, bmm2;
  FILE* m = std::fopen((dir + "/meta.txt").c_str(), "r");
  if (m == nullptr) return 102;
  const int nread = std::fscanf(m, "%d %d %d %d %lld %d %d %d %f %f", &B, &H, &SQ, &PS, &num_pages, &BTW, &max_len,
                                &causal, &bmm1, &bmm2);
  std::fclose(m);
  if (nread != 10) return 102;

  const size_t rows = (size_t)B * SQ;
  std::vector<uint16_t> q, kv;
  std::vector<int32_t> bt, lens;
  if (!read_file(dir + "/q.bin", q, rows * H * 576) || !read_file(dir + "/kv.bin", kv, (size_t)num_pages * PS * 576) ||
      !read_file(dir + "/bt.bin", bt, (size_t)B * BTW) || !read_file(dir + "/lens.bin", lens, (size_t)B))
    return 103;

  mla_decode_dims_t dims{};
  dims.batch = B;
  dims.num_heads = H;
  dims.q_len_fixed = SQ;
  dims.total_q = (int32_t)rows;
  dims.page_size = PS;
  dims.num_pages = num_pages;
  dims.block_table_stride = BTW;
  dims.kv_dtype = MLA_KV_BF16;
  dims.kv_lora_rank = 512;
  dims.qk_rope_head_dim = 64;

  const size_t ws_bytes = mla_decode_paged_workspace_size(&dims, max_len, SQ, 1);
  if (ws_bytes == 0) return 104;
  uint16_t* d_q = to_device(q);
  uint16_t* d_kv = to_device(kv);
  int32_t* d_bt = to_device(bt);
  int32_t* d_lens = to_device(lens);
  void *d_out = nullptr, *d_lse = nullptr, *d_ws = nullptr;
  if (!d_q || !d_kv || !d_bt || !d_lens || hipMalloc(&d_out, rows * H * 512 * 2) != hipSuccess ||
      hipMalloc(&d_lse, rows * H * 4) != hipSuccess || hipMalloc(&d_ws, ws_bytes) != hipSuccess)
    return 105;
  hipStream_t stream;
  if (hipStreamCreate(&stream) != hipSuccess) return 106;

  const int rc = mla_decode_paged(d_q, d_kv, d_bt, d_lens, nullptr, max_len, SQ, bmm1, bmm2, causal, d_out,
                                  static_cast<float*>(d_lse), d_ws, ws_bytes, &dims, stream);
  if (rc != MLA_OK) {
    std::fprintf(stderr, "mla_decode_paged: %s\n", mla_status_string(rc));
    return rc;
  }
  if (hipStreamSynchronize(stream) != hipSuccess) return 107;

  std::vector<uint16_t> out(rows * H * 512);
  std::vector<float> lse(rows * H);
  if (hipMemcpy(out.data(), d_out, out.size() * 2, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(lse.data(), d_lse, lse.size() * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return 108;
  if (!write_file(dir + "/out.bin", out) || !write_file(dir + "/lse.bin", lse)) return 109;
  (void)hipStreamDestroy(stream);
  (void)hipFree(d_q);
  (void)hipFree(d_kv);
  (void)hipFree(d_bt);
  (void)hipFree(d_lens);
  (void)hipFree(d_out);
  (void)hipFree(d_lse);
  (void)hipFree(d_ws);
  std::printf("mla_c_caller: ok (%zu rows x %d heads, workspace %zu bytes)\n", rows, H, ws_bytes);
  return 0;
}

// One CSA decode step driven through the C ABI alone (no Python, no torch):
// reads a workload file, runs csa_index_scores -> csa_topk -> csa_decode_attn
// on a HIP stream of its own, and writes top-k indices, outputs and lse.
//
//   decode_step <input file> <output file>
//
// Input file: 16 int32 (B, H, D_nope, D_rope, H_I, D_I, k, W, m, page_size,
// num_pages, max_pages, 0, 0, 0, 0), 8 float32 (q_idx_scale, k_idx_scale,
// lat_scale, swa_scale, softmax_scale, 0, 0, 0), then the arrays in this
// order, each contiguous: q_idx u8 [B][H_I][D_I], w f32 [B][H_I],
// k_idx u8 [P][ps][D_I], lat_nope u8 [P][ps][D_nope], lat_rope u16
// [P][ps][D_rope], page_table i32 [B][max_pages], n_comp i32 [B], q_pos i32
// [B], q u16 [B][H][D], sink f32 [H], swa_nope u8 [B][W][D_nope], swa_rope
// u16 [B][W][D_rope], swa_pos i32 [B][W].
// Output file: topk i32 [B][k], out u16 [B][H][D], lse f32 [B][H].
// Exit status: 0 on success, 1 on a file error, 2 on a HIP error, 3 on a
// library status other than CSA_OK.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "csa.h"

namespace {

FILE* g_in = nullptr;

void* read_to_device(size_t bytes) {
  std::vector<unsigned char> host(bytes);
  if (bytes && fread(host.data(), 1, bytes, g_in) != bytes) {
    fprintf(stderr, "decode_step: short input file\n");
    exit(1);
  }
  void* dev = nullptr;
  if (hipMalloc(&dev, bytes ? bytes : 16) != hipSuccess) {
    fprintf(stderr, "decode_step: hipMalloc of %zu bytes failed\n", bytes);
    exit(2);
  }
  if (bytes && hipMemcpy(dev, host.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) exit(2);
  return dev;
}

void* device_buffer(size_t bytes) {
  void* dev = nullptr;
  if (hipMalloc(&dev, bytes ? bytes : 16) != hipSuccess) exit(2);
  return dev;
}

void check(const char* what, int rc) {
  if (rc != CSA_OK) {
    fprintf(stderr, "decode_step: %s returned %d (%s)\n", what, rc, csa_status_string(rc));
    exit(3);
  }
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: decode_step <input> <output>\n");
    return 1;
  }
  g_in = fopen(argv[1], "rb");
  if (!g_in) return 1;
  int32_t hdr[16];
  float fh[8];
  if (fread(hdr, sizeof(int32_t), 16, g_in) != 16 || fread(fh, sizeof(float), 8, g_in) != 8) return 1;
  const int B = hdr[0], H = hdr[1], Dn = hdr[2], Dr = hdr[3], HI = hdr[4], DI = hdr[5], k = hdr[6], W = hdr[7];
  const int m = hdr[8], ps = hdr[9], P = hdr[10], maxp = hdr[11];
  const int D = Dn + Dr;
  printf("decode_step: B=%d H=%d D=%d+%d indexer %dx%d k=%d W=%d m=%d pages %d x %d (library %d)\n", B, H, Dn, Dr,
         HI, DI, k, W, m, P, ps, csa_version());

  auto* q_idx = static_cast<uint8_t*>(read_to_device((size_t)B * HI * DI));
  auto* w = static_cast<float*>(read_to_device((size_t)B * HI * 4));
  auto* k_idx = static_cast<uint8_t*>(read_to_device((size_t)P * ps * DI));
  auto* lat_nope = static_cast<uint8_t*>(read_to_device((size_t)P * ps * Dn));
  auto* lat_rope = static_cast<uint16_t*>(read_to_device((size_t)P * ps * Dr * 2));
  auto* page_table = static_cast<int32_t*>(read_to_device((size_t)B * maxp * 4));
  auto* n_comp = static_cast<int32_t*>(read_to_device((size_t)B * 4));
  auto* q_pos = static_cast<int32_t*>(read_to_device((size_t)B * 4));
  auto* q = static_cast<uint16_t*>(read_to_device((size_t)B * H * D * 2));
  auto* sink = static_cast<float*>(read_to_device((size_t)H * 4));
  auto* swa_nope = static_cast<uint8_t*>(read_to_device((size_t)B * W * Dn));
  auto* swa_rope = static_cast<uint16_t*>(read_to_device((size_t)B * W * Dr * 2));
  auto* swa_pos = static_cast<int32_t*>(read_to_device((size_t)B * W * 4));
  fclose(g_in);

  const int64_t ld = ((int64_t)maxp * ps + 15) / 16 * 16;
  auto* scores = static_cast<float*>(device_buffer((size_t)B * ld * 4));
  auto* n_vis = static_cast<int32_t*>(device_buffer((size_t)B * 4));
  auto* topk = static_cast<int32_t*>(device_buffer((size_t)B * k * 4));
  auto* out = static_cast<uint16_t*>(device_buffer((size_t)B * H * D * 2));
  auto* lse = static_cast<float*>(device_buffer((size_t)B * H * 4));
  const size_t tws = csa_topk_workspace_size(B, ld, k);
  const size_t aws = csa_attn_workspace_size(B, H, Dn, Dr, k + W);
  if (tws == CSA_WORKSPACE_UNSUPPORTED || aws == CSA_WORKSPACE_UNSUPPORTED) {
    fprintf(stderr, "workspace query: unsupported shape\n");
    return 2;
  }
  void* topk_ws = tws ? device_buffer(tws) : nullptr;
  void* attn_ws = aws ? device_buffer(aws) : nullptr;

  hipStream_t stream;
  if (hipStreamCreateWithFlags(&stream, hipStreamNonBlocking) != hipSuccess) return 2;
  csa_latent_cache cache{lat_nope, lat_rope, fh[2], page_table, n_comp, B, P, ps, maxp, Dn, Dr, m};
  csa_swa_ring ring{swa_nope, swa_rope, fh[3], swa_pos, W};
  check("csa_index_scores", csa_index_scores(q_idx, fh[0], w, k_idx, fh[1], page_table, n_comp, P, ps, maxp, B, q_pos,
                                             nullptr, B, HI, DI, m, scores, ld, n_vis, stream));
  check("csa_topk", csa_topk(scores, ld, n_vis, B, k, topk, topk_ws, tws, stream));
  check("csa_decode_attn", csa_decode_attn(q, (int64_t)H * D, &cache, topk, k, &ring, q_pos, sink, fh[4], 0.0f, B, H,
                                           out, lse, attn_ws, aws, stream));
  if (hipStreamSynchronize(stream) != hipSuccess) return 2;

  std::vector<int32_t> h_topk((size_t)B * k);
  std::vector<uint16_t> h_out((size_t)B * H * D);
  std::vector<float> h_lse((size_t)B * H);
  if (hipMemcpy(h_topk.data(), topk, h_topk.size() * 4, hipMemcpyDeviceToHost) != hipSuccess) return 2;
  if (hipMemcpy(h_out.data(), out, h_out.size() * 2, hipMemcpyDeviceToHost) != hipSuccess) return 2;
  if (hipMemcpy(h_lse.data(), lse, h_lse.size() * 4, hipMemcpyDeviceToHost) != hipSuccess) return 2;
  FILE* fo = fopen(argv[2], "wb");
  if (!fo) return 1;
  fwrite(h_topk.data(), 4, h_topk.size(), fo);
  fwrite(h_out.data(), 2, h_out.size(), fo);
  fwrite(h_lse.data(), 4, h_lse.size(), fo);
  fclose(fo);
  (void)hipStreamDestroy(stream);
  printf("decode_step: ok\n");
  return 0;
}

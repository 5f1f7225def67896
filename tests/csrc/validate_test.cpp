// Host-only test of the C-ABI argument validation (no HIP calls): every error
// path returns its status before any memory is touched.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "validate.hpp"

static int failures = 0;
#define EXPECT_EQ(a, b)                                                                   \
  do {                                                                                    \
    long long _a = (a), _b = (b);                                                         \
    if (_a != _b) {                                                                       \
      std::fprintf(stderr, "%s:%d: %s = %lld, expected %lld\n", __FILE__, __LINE__, #a, _a, _b); \
      ++failures;                                                                         \
    }                                                                                     \
  } while (0)

int main() {
  using namespace wan;
  alignas(16) static unsigned char buf[1 << 20];
  void* qkv = buf;                 // 1 MB fake "device" region (never dereferenced)
  void* g1 = buf + 4096;  // inside the 196 KB packed buffer of the first call
  void* g2 = buf + 8192;
  Sizes z;
  // norm + rope
  EXPECT_EQ(validate_qknorm_rope(qkv, g1, g2, 1, 2, 8, 8, 2, 128, 1e-6f, 1e4f, &z), WAN_E_ALIAS);  // gammas inside qkv range
  static unsigned char other[8192] __attribute__((aligned(16)));
  g1 = other;
  g2 = other + 1024;
  EXPECT_EQ(validate_qknorm_rope(qkv, g1, g2, 1, 2, 8, 8, 2, 128, 1e-6f, 1e4f, &z), WAN_OK);
  EXPECT_EQ(z.S, 128);
  EXPECT_EQ(z.D, 256);
  EXPECT_EQ(validate_qknorm_rope(nullptr, g1, g2, 1, 2, 8, 8, 2, 128, 1e-6f, 1e4f, &z), WAN_E_NULL);
  EXPECT_EQ(validate_qknorm_rope(qkv, nullptr, g2, 1, 2, 8, 8, 2, 128, 1e-6f, 1e4f, &z), WAN_E_NULL);
  EXPECT_EQ(validate_qknorm_rope(qkv, g1, g2, 1, 2, 8, 8, 2, 64, 1e-6f, 1e4f, &z), WAN_E_UNSUPPORTED);
  EXPECT_EQ(validate_qknorm_rope(qkv, g1, g2, 1, 2, 8, 8, 0, 128, 1e-6f, 1e4f, &z), WAN_E_SHAPE);
  EXPECT_EQ(validate_qknorm_rope(qkv, g1, g2, 1, 2, 8, 8, 257, 128, 1e-6f, 1e4f, &z), WAN_E_UNSUPPORTED);
  EXPECT_EQ(validate_qknorm_rope(qkv, g1, g2, -1, 2, 8, 8, 2, 128, 1e-6f, 1e4f, &z), WAN_E_SHAPE);
  EXPECT_EQ(validate_qknorm_rope(qkv, g1, g2, 1, -2, 8, 8, 2, 128, 1e-6f, 1e4f, &z), WAN_E_SHAPE);
  EXPECT_EQ(validate_qknorm_rope(qkv, g1, g2, 1, 2, 8, 8, 2, 128, -1.f, 1e4f, &z), WAN_E_VALUE);
  EXPECT_EQ(validate_qknorm_rope(qkv, g1, g2, 1, 2, 8, 8, 2, 128, 1e-6f, 0.f, &z), WAN_E_VALUE);
  EXPECT_EQ(validate_qknorm_rope(qkv, g1, g2, 1, 2, 8, 8, 2, 128, NAN, 1e4f, &z), WAN_E_VALUE);
  EXPECT_EQ(validate_qknorm_rope(buf + 2, g1, g2, 1, 2, 8, 8, 2, 128, 1e-6f, 1e4f, &z), WAN_E_ALIGN);
  EXPECT_EQ(validate_qknorm_rope(qkv, other + 8, g2, 1, 2, 8, 8, 2, 128, 1e-6f, 1e4f, &z), WAN_E_ALIGN);
  // empty: OK without looking at pointers
  EXPECT_EQ(validate_qknorm_rope(nullptr, nullptr, nullptr, 0, 2, 8, 8, 2, 128, 1e-6f, 1e4f, &z), WAN_OK);
  EXPECT_EQ(z.empty, 1);
  EXPECT_EQ(validate_qknorm_rope(nullptr, nullptr, nullptr, 1, 0, 8, 8, 2, 128, 1e-6f, 1e4f, &z), WAN_OK);
  // overflow: S beyond 2^31-1, and B*S*3D beyond int64
  EXPECT_EQ(validate_qknorm_rope(qkv, g1, g2, 1, 1 << 20, 1 << 12, 1, 2, 128, 1e-6f, 1e4f, &z), WAN_E_OVERFLOW);
  EXPECT_EQ(validate_qknorm_rope(qkv, g1, g2, 1, INT64_MAX / 2, 4, 1, 2, 128, 1e-6f, 1e4f, &z), WAN_E_OVERFLOW);
  EXPECT_EQ(validate_qknorm_rope(qkv, g1, g2, INT64_MAX / 1000, 1000, 1000, 1, 2, 128, 1e-6f, 1e4f, &z), WAN_E_OVERFLOW);

  // attention
  alignas(16) static unsigned char outb[1 << 16];
  alignas(16) static float lseb[1024];
  EXPECT_EQ(validate_attn(qkv, outb, lseb, 1, 16, 2, 128, 0.088f, 2, &z), WAN_OK);
  EXPECT_EQ(validate_attn(qkv, outb, nullptr, 1, 16, 2, 128, 0.088f, 2, &z), WAN_OK);
  EXPECT_EQ(validate_attn(qkv, nullptr, nullptr, 1, 16, 2, 128, 0.088f, 2, &z), WAN_E_NULL);
  EXPECT_EQ(validate_attn(qkv, buf + 4096, nullptr, 1, 16, 2, 128, 0.088f, 2, &z), WAN_E_ALIAS);
  EXPECT_EQ(validate_attn(qkv, outb, reinterpret_cast<float*>(outb + 16), 1, 16, 2, 128, 0.088f, 2, &z), WAN_E_ALIAS);
  EXPECT_EQ(validate_attn(qkv, outb, reinterpret_cast<float*>(buf + 64), 1, 16, 2, 128, 0.088f, 2, &z), WAN_E_ALIAS);
  EXPECT_EQ(validate_attn(qkv, outb + 8, nullptr, 1, 16, 2, 128, 0.088f, 2, &z), WAN_E_ALIGN);
  EXPECT_EQ(validate_attn(qkv, outb, reinterpret_cast<float*>(reinterpret_cast<char*>(lseb) + 2), 1, 16, 2, 128, 0.088f, 2, &z), WAN_E_ALIGN);
  EXPECT_EQ(validate_attn(qkv, outb, nullptr, 1, 16, 2, 96, 0.088f, 2, &z), WAN_E_UNSUPPORTED);
  EXPECT_EQ(validate_attn(qkv, outb, nullptr, 1, 16, 2, 128, 0.f, 2, &z), WAN_E_VALUE);
  EXPECT_EQ(validate_attn(qkv, outb, nullptr, 1, 16, 2, 128, INFINITY, 2, &z), WAN_E_VALUE);
  EXPECT_EQ(validate_attn(nullptr, nullptr, nullptr, 3, 0, 2, 128, 0.088f, 2, &z), WAN_OK);
  EXPECT_EQ(validate_attn(qkv, outb, nullptr, 1, (int64_t)INT32_MAX + 1, 2, 128, 0.088f, 2, &z), WAN_E_OVERFLOW);
  EXPECT_EQ(validate_attn(qkv, outb, nullptr, -2, 16, 2, 128, 0.088f, 2, &z), WAN_E_SHAPE);

  // chunk + merge
  alignas(16) static float of32[1 << 14];
  alignas(16) static float lsea[256], lsec[256];
  alignas(16) static float of32b[1 << 14];
  EXPECT_EQ(validate_attn_chunk(qkv, qkv, of32, lsea, 1, 16, 16, 2, 128, 0.088f, &z), WAN_OK);
  EXPECT_EQ(validate_attn_chunk(qkv, qkv, of32, nullptr, 1, 16, 16, 2, 128, 0.088f, &z), WAN_E_NULL);
  EXPECT_EQ(validate_attn_chunk(qkv, qkv, of32, lsea, 1, 16, 0, 2, 128, 0.088f, &z), WAN_E_SHAPE);
  EXPECT_EQ(validate_attn_chunk(qkv, qkv, of32, lsea, 1, 0, 0, 2, 128, 0.088f, &z), WAN_OK);
  EXPECT_EQ(validate_attn_chunk(qkv, qkv, buf + 1024, lsea, 1, 16, 16, 2, 128, 0.088f, &z), WAN_E_ALIAS);
  EXPECT_EQ(validate_attn_chunk(qkv, qkv, of32, of32 + 4, 1, 16, 16, 2, 128, 0.088f, &z), WAN_E_ALIAS);
  EXPECT_EQ(validate_attn_chunk(qkv, qkv, of32, lsea, 1, 16, -1, 2, 128, 0.088f, &z), WAN_E_SHAPE);
  EXPECT_EQ(validate_attn_merge(of32, lsea, of32b, lsec, nullptr, 1, 16, 2, 128, &z), WAN_OK);
  EXPECT_EQ(validate_attn_merge(of32, lsea, of32b, lsec, outb, 1, 16, 2, 128, &z), WAN_OK);
  EXPECT_EQ(validate_attn_merge(of32, lsea, of32, lsec, nullptr, 1, 16, 2, 128, &z), WAN_E_ALIAS);
  EXPECT_EQ(validate_attn_merge(of32, lsea, of32b, lsea, nullptr, 1, 16, 2, 128, &z), WAN_E_ALIAS);
  EXPECT_EQ(validate_attn_merge(of32, lsea, of32b, nullptr, nullptr, 1, 16, 2, 128, &z), WAN_E_NULL);
  EXPECT_EQ(validate_attn_merge(of32 + 1, lsea, of32b, lsec, nullptr, 1, 16, 2, 128, &z), WAN_E_ALIGN);

  // one ring round folded into the accumulator
  EXPECT_EQ(validate_attn_chunk_fold(qkv, qkv, of32, lsea, outb, 1, 16, 16, 2, 128, 0.088f, &z), WAN_OK);
  EXPECT_EQ(validate_attn_chunk_fold(qkv, qkv, of32, lsea, nullptr, 1, 16, 16, 2, 128, 0.088f, &z), WAN_OK);
  EXPECT_EQ(validate_attn_chunk_fold(qkv, qkv, of32, lsea, buf + 512, 1, 16, 16, 2, 128, 0.088f, &z), WAN_E_ALIAS);
  EXPECT_EQ(validate_attn_chunk_fold(qkv, qkv, of32, lsea, of32 + 64, 1, 16, 16, 2, 128, 0.088f, &z), WAN_E_ALIAS);
  EXPECT_EQ(validate_attn_chunk_fold(qkv, qkv, of32, lsea, outb + 8, 1, 16, 16, 2, 128, 0.088f, &z), WAN_E_ALIGN);
  EXPECT_EQ(validate_attn_chunk_fold(qkv, qkv, of32, nullptr, outb, 1, 16, 16, 2, 128, 0.088f, &z), WAN_E_NULL);
  EXPECT_EQ(validate_attn_chunk_fold(qkv, qkv, of32, lsea, outb, 1, 16, 0, 2, 128, 0.088f, &z), WAN_E_SHAPE);

  // QKV projection: x [1,16,256], w [768,256], out [1,16,768]
  EXPECT_EQ(validate_qkv_proj(buf, buf + 16384, nullptr, outb, 1, 16, 2, 128, &z), WAN_OK);
  EXPECT_EQ(validate_qkv_proj(buf, buf + 16384, buf + 600000, outb, 1, 16, 2, 128, &z), WAN_OK);
  EXPECT_EQ(validate_qkv_proj(buf, buf + 16384, nullptr, buf + 8192, 1, 16, 2, 128, &z), WAN_E_ALIAS);
  EXPECT_EQ(validate_qkv_proj(buf, buf + 16384, outb + 64, outb, 1, 16, 2, 128, &z), WAN_E_ALIAS);
  EXPECT_EQ(validate_qkv_proj(buf, nullptr, nullptr, outb, 1, 16, 2, 128, &z), WAN_E_NULL);
  EXPECT_EQ(validate_qkv_proj(buf + 8, buf + 16384, nullptr, outb, 1, 16, 2, 128, &z), WAN_E_ALIGN);
  EXPECT_EQ(validate_qkv_proj(buf, buf + 16384, nullptr, outb, 1, 16, 2, 64, &z), WAN_E_UNSUPPORTED);
  EXPECT_EQ(validate_qkv_proj(nullptr, nullptr, nullptr, nullptr, 0, 16, 2, 128, &z), WAN_OK);
  // B * S token rows past 2^31 - 257 do not fit the GEMM's 32-bit row indices
  EXPECT_EQ(validate_qkv_proj(buf, buf + 16384, nullptr, outb, 2, 1 << 30, 2, 128, &z), WAN_E_OVERFLOW);
  EXPECT_EQ(validate_qkv_proj(buf, buf + 16384, nullptr, outb, 1, (1LL << 31) - 300, 2, 128, &z), WAN_E_ALIAS);

  // Projection + norm + RoPE: x [1,16,256] at buf, w [768,256] at buf + 16384
  // (393 KB), out [1,16,768] at outb, gammas in `other`, workspace separate.
  // Workspace: 256 control bytes + 256 (one token block) + 16 tokens x 4 x 8 bytes.
  FusedWorkspace fw;
  EXPECT_EQ(fused_workspace(16, 2, &fw), 1);
  EXPECT_EQ(fw.arrive_off, 256);
  EXPECT_EQ(fw.partial_off, 512);
  EXPECT_EQ(fw.bytes, 512 + 16 * 2 * 2 * 8);
  EXPECT_EQ(fused_workspace(257, 2, &fw), 1);  // two token blocks: the counts still fit 256 bytes
  EXPECT_EQ(fw.partial_off, 512);
  EXPECT_EQ(fused_workspace(256 * 33, 1, &fw), 1);  // 33 token blocks: 264 bytes of counts
  EXPECT_EQ(fw.partial_off, 256 + 512);
  EXPECT_EQ(fused_workspace(INT64_MAX / 4, 256, &fw), 0);
  alignas(16) static unsigned char wsb[4096];
  const int64_t wsn = 512 + 16 * 32;
  unsigned char* gq2 = other;
  unsigned char* gk2 = other + 1024;
  EXPECT_EQ(validate_qkv_proj_norm_rope(buf, buf + 16384, nullptr, gq2, gk2, outb, wsb, wsn, 1, 1, 4, 4, 2, 128, 1e-6f,
                                        1e4f, &z), WAN_OK);
  EXPECT_EQ(validate_qkv_proj_norm_rope(buf, buf + 16384, nullptr, gq2, gk2, outb, wsb, wsn - 1, 1, 1, 4, 4, 2, 128,
                                        1e-6f, 1e4f, &z), WAN_E_SHAPE);
  EXPECT_EQ(validate_qkv_proj_norm_rope(buf, buf + 16384, nullptr, gq2, gk2, outb, nullptr, wsn, 1, 1, 4, 4, 2, 128,
                                        1e-6f, 1e4f, &z), WAN_E_NULL);
  EXPECT_EQ(validate_qkv_proj_norm_rope(buf, buf + 16384, nullptr, gq2, gk2, outb, wsb + 8, wsn, 1, 1, 4, 4, 2, 128,
                                        1e-6f, 1e4f, &z), WAN_E_ALIGN);
  EXPECT_EQ(validate_qkv_proj_norm_rope(buf, buf + 16384, nullptr, gq2, gk2, outb, outb + 1024, wsn, 1, 1, 4, 4, 2,
                                        128, 1e-6f, 1e4f, &z), WAN_E_ALIAS);  // workspace inside the output
  EXPECT_EQ(validate_qkv_proj_norm_rope(buf, buf + 16384, nullptr, gq2, gk2, outb, buf + 32, wsn, 1, 1, 4, 4, 2, 128,
                                        1e-6f, 1e4f, &z), WAN_E_ALIAS);  // ... inside x
  EXPECT_EQ(validate_qkv_proj_norm_rope(buf, buf + 16384, nullptr, gq2, gk2, outb, gq2, wsn, 1, 1, 4, 4, 2, 128, 1e-6f,
                                        1e4f, &z), WAN_E_ALIAS);  // ... on a gamma
  EXPECT_EQ(validate_qkv_proj_norm_rope(buf, buf + 16384, nullptr, outb + 64, gk2, outb, wsb, wsn, 1, 1, 4, 4, 2, 128,
                                        1e-6f, 1e4f, &z), WAN_E_ALIAS);  // a gamma inside the output
  EXPECT_EQ(validate_qkv_proj_norm_rope(buf, buf + 16384, nullptr, gq2, gk2, outb, wsb, wsn, 1, 1, 4, 4, 2, 128, std::nanf(""),
                                        1e4f, &z), WAN_E_VALUE);
  EXPECT_EQ(validate_qkv_proj_norm_rope(buf, buf + 16384, nullptr, gq2, gk2, outb, wsb, wsn, 1, 1, 4, 4, 2, 128, 1e-6f,
                                        -1.f, &z), WAN_E_VALUE);
  EXPECT_EQ(validate_qkv_proj_norm_rope(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0, 1, 4, 4,
                                        2, 128, 1e-6f, 1e4f, &z), WAN_OK);  // no tokens: nothing is touched
  EXPECT_EQ(validate_qkv_proj_norm_rope(buf, buf + 16384, nullptr, gq2, gk2, outb, wsb, wsn, 1, 1, 4, 4, 2, 96, 1e-6f,
                                        1e4f, &z), WAN_E_UNSUPPORTED);

  // fp8 quantisation and attention
  alignas(16) static unsigned char qk8[1 << 16], vt8[1 << 16];
  alignas(16) static float sc[4], am[4];
  EXPECT_EQ(validate_quant_fp8(qkv, qk8, vt8, sc, am, 1, 16, 2, 128, &z), WAN_OK);
  EXPECT_EQ(validate_quant_fp8(qkv, qk8, vt8, sc, sc, 1, 16, 2, 128, &z), WAN_E_ALIAS);
  EXPECT_EQ(validate_quant_fp8(qkv, qk8, qk8 + 16, sc, am, 1, 16, 2, 128, &z), WAN_E_ALIAS);
  EXPECT_EQ(validate_quant_fp8(qkv, buf + 512, vt8, sc, am, 1, 16, 2, 128, &z), WAN_E_ALIAS);
  EXPECT_EQ(validate_quant_fp8(qkv, qk8, vt8, sc, am, 70000, 16, 2, 128, &z), WAN_E_OVERFLOW);
  EXPECT_EQ(validate_quant_fp8(qkv, qk8, nullptr, sc, am, 1, 16, 2, 128, &z), WAN_E_NULL);
  EXPECT_EQ(validate_attn_fp8(qk8, vt8, sc, outb, lsea, 1, 16, 2, 128, 0.088f, &z), WAN_OK);
  EXPECT_EQ(validate_attn_fp8(qk8, vt8, sc, qk8 + 64, nullptr, 1, 16, 2, 128, 0.088f, &z), WAN_E_ALIAS);
  EXPECT_EQ(validate_attn_fp8(qk8, vt8, nullptr, outb, nullptr, 1, 16, 2, 128, 0.088f, &z), WAN_E_NULL);
  EXPECT_EQ(validate_attn_fp8(qk8, vt8, sc, outb, nullptr, 1, 16, 2, 128, -2.f, &z), WAN_E_VALUE);
  // fused norm + quantisation: both sets of checks, and no gamma inside an fp8 output
  EXPECT_EQ(validate_qknorm_rope_fp8(qkv, g1, g2, 1, 2, 8, 8, 2, 128, 1e-6f, 1e4f, qk8, vt8, sc, am, &z), WAN_OK);
  EXPECT_EQ(validate_qknorm_rope_fp8(qkv, qk8 + 256, g2, 1, 2, 8, 8, 2, 128, 1e-6f, 1e4f, qk8, vt8, sc, am, &z),
            WAN_E_ALIAS);
  EXPECT_EQ(validate_qknorm_rope_fp8(qkv, g1, vt8, 1, 2, 8, 8, 2, 128, 1e-6f, 1e4f, qk8, vt8, sc, am, &z),
            WAN_E_ALIAS);
  EXPECT_EQ(validate_qknorm_rope_fp8(qkv, g1, g2, 1, 2, 8, 8, 2, 128, 1e-6f, 1e4f, qk8, vt8, sc, sc, &z),
            WAN_E_ALIAS);
  EXPECT_EQ(validate_qknorm_rope_fp8(qkv, g1, g2, 1, 2, 8, 8, 2, 128, 1e-6f, 1e4f, buf + 512, vt8, sc, am, &z),
            WAN_E_ALIAS);
  EXPECT_EQ(validate_qknorm_rope_fp8(qkv, g1, g2, 1, 2, 8, 8, 2, 128, 1e-6f, 1e4f, qk8, nullptr, sc, am, &z),
            WAN_E_NULL);
  EXPECT_EQ(validate_qknorm_rope_fp8(qkv, nullptr, g2, 1, 2, 8, 8, 2, 128, 1e-6f, 1e4f, qk8, vt8, sc, am, &z),
            WAN_E_NULL);
  EXPECT_EQ(validate_qknorm_rope_fp8(qkv, g1, g2, 1, 2, 8, 8, 2, 128, -1.f, 1e4f, qk8, vt8, sc, am, &z), WAN_E_VALUE);
  EXPECT_EQ(validate_qknorm_rope_fp8(qkv, g1, g2, 70000, 2, 8, 8, 2, 128, 1e-6f, 1e4f, qk8, vt8, sc, am, &z),
            WAN_E_OVERFLOW);
  EXPECT_EQ(validate_qknorm_rope_fp8(nullptr, nullptr, nullptr, 1, 0, 8, 8, 2, 128, 1e-6f, 1e4f, nullptr, nullptr,
                                     nullptr, nullptr, &z),
            WAN_OK);
  // size products that overflow int64 are reported, never computed: an empty
  // call with a huge batch, a huge batch times a huge chunk, a huge batch
  // times the widest head count
  EXPECT_EQ(validate_attn(nullptr, nullptr, nullptr, INT64_MAX, 0, 256, 128, 0.088f, 2, &z), WAN_OK);
  EXPECT_EQ(validate_attn(qkv, outb, lseb, INT64_MAX / 256, 1, 256, 128, 0.088f, 2, &z), WAN_E_OVERFLOW);
  EXPECT_EQ(validate_attn_chunk(qkv, qkv, of32, lsea, 1LL << 40, 1, INT32_MAX, 1, 128, 0.088f, &z), WAN_E_OVERFLOW);
  EXPECT_EQ(validate_attn_chunk_fold(qkv, qkv, of32, lsea, outb, 1LL << 40, 1, INT32_MAX, 1, 128, 0.088f, &z),
            WAN_E_OVERFLOW);
  EXPECT_EQ(validate_attn_chunk(qkv, qkv, of32, lsea, INT64_MAX / 384, 1, 2, 1, 128, 0.088f, &z), WAN_E_OVERFLOW);
  EXPECT_EQ(validate_attn_fp8(qk8, vt8, sc, outb, nullptr, INT64_MAX / 256, 1, 256, 128, 0.088f, &z), WAN_E_OVERFLOW);
  int64_t big = 0;
  EXPECT_EQ(fp8_vt_bytes(1, INT64_MAX, 1, &big), 0);
  EXPECT_EQ(fp8_vt_bytes(INT64_MAX / 128, 256, 1, &big), 0);
  // NaN scalars are rejected (the check reads the bit pattern, so it also
  // holds in code compiled with finite-math assumptions)
  volatile float nan = NAN;
  EXPECT_EQ(validate_attn(qkv, outb, nullptr, 1, 16, 2, 128, nan, 2, &z), WAN_E_VALUE);
  EXPECT_EQ(validate_attn(nullptr, nullptr, nullptr, 0, 16, 2, 128, nan, 2, &z), WAN_E_VALUE);
  EXPECT_EQ(validate_qknorm_rope(qkv, g1, g2, 1, 2, 8, 8, 2, 128, 1e-6f, nan, &z), WAN_E_VALUE);
  EXPECT_EQ(validate_attn_chunk(qkv, qkv, of32, lsea, 1, 16, 16, 2, 128, nan, &z), WAN_E_VALUE);
  EXPECT_EQ(validate_attn_fp8(qk8, vt8, sc, outb, nullptr, 1, 16, 2, 128, nan, &z), WAN_E_VALUE);
  EXPECT_EQ(finite(-INFINITY), 0);
  EXPECT_EQ(finite(3.0e38f), 1);

  // Skip-Softmax: the attention checks, a finite threshold >= 0, and a
  // decision map distinct from the other buffers
  alignas(16) static unsigned char mapb[4096];
  EXPECT_EQ(validate_attn_skip(qkv, outb, lseb, mapb, 1, 16, 2, 128, 0.088f, 0.02f, &z), WAN_OK);
  EXPECT_EQ(validate_attn_skip(qkv, outb, nullptr, nullptr, 1, 16, 2, 128, 0.088f, 0.f, &z), WAN_OK);
  EXPECT_EQ(validate_attn_skip(qkv, outb, nullptr, nullptr, 1, 16, 2, 128, 0.088f, -1e-3f, &z), WAN_E_VALUE);
  EXPECT_EQ(validate_attn_skip(qkv, outb, nullptr, nullptr, 1, 16, 2, 128, 0.088f, nan, &z), WAN_E_VALUE);
  EXPECT_EQ(validate_attn_skip(qkv, outb, nullptr, nullptr, 1, 16, 2, 128, 0.088f, INFINITY, &z), WAN_E_VALUE);
  EXPECT_EQ(validate_attn_skip(qkv, outb, nullptr, buf + 100, 1, 16, 2, 128, 0.088f, 0.02f, &z), WAN_E_ALIAS);
  EXPECT_EQ(validate_attn_skip(qkv, outb, nullptr, outb + 7, 1, 16, 2, 128, 0.088f, 0.02f, &z), WAN_E_ALIAS);
  EXPECT_EQ(validate_attn_skip(qkv, outb, lseb, reinterpret_cast<unsigned char*>(lseb) + 1, 1, 16, 2, 128, 0.088f,
                               0.02f, &z), WAN_E_ALIAS);
  EXPECT_EQ(validate_attn_skip(nullptr, nullptr, nullptr, nullptr, 0, 16, 2, 128, 0.088f, 0.02f, &z), WAN_OK);
  int64_t mb = 0;
  EXPECT_EQ(skip_map_bytes(2, 100, 3, &mb), 1);
  EXPECT_EQ(mb, 2 * 3 * 3 * 2);  // ceil(100/48) = 3 query blocks, ceil(100/64) = 2 key blocks
  EXPECT_EQ(skip_map_bytes(INT64_MAX / 2, 1000, 256, &mb), 0);

  int64_t vtb = 0;
  EXPECT_EQ(fp8_vt_bytes(2, 129, 3, &vtb), 1);
  EXPECT_EQ(vtb, 2 * 3 * 128 * 256);

  if (failures) {
    std::fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  std::printf("validate_test: all checks passed\n");
  return 0;
}

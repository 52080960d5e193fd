// Drives the host half of libtq (the C ABI's size queries, parameter-image
// builder and every argument check) under AddressSanitizer and
// UndefinedBehaviorSanitizer on the CPU.  The kernel launchers and the two
// HIP runtime calls the host half makes are replaced by stubs that report
// failure, so no call here reaches a GPU; device pointers are aligned
// addresses that the host code must never dereference.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "tq.h"
#include "tq_internal.h"

namespace tq {
hipError_t launch_quantize(const QuantArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_decode(const DecodeArgs&, hipStream_t) { return hipErrorNotSupported; }
bool decode_mfma_applies(int k_codec, int v_codec, int group) {
  return v_codec == POLAR && group <= kMaxGroup && (k_codec == POLAR || k_codec == POLAR_QJL || k_codec == Q8_BLOCK32);
}
hipError_t launch_decode_mfma(const DecodeArgs&, hipStream_t) { return hipErrorNotSupported; }
bool decode_reg_applies(int k_codec, int v_codec, int group) {
  return v_codec == POLAR && group <= kMaxGroup && (k_codec == POLAR || k_codec == POLAR_QJL);
}
hipError_t launch_decode_reg(const DecodeArgs&, hipStream_t) { return hipErrorNotSupported; }
bool decode_q8_applies(int k_codec, int v_codec, int group, int v_bits) {
  return k_codec == Q8_BLOCK32 && v_codec == POLAR && group > 4 &&
         ((group + 3) / 4 == 2 ? (v_bits >= 2 && v_bits <= 4) : ((group + 3) / 4 == 3 && v_bits == 2));
}
hipError_t launch_decode_q8(const DecodeArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_dequantize(const DequantArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_quantize_tree(const QuantArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_stream_read(const void*, uint64_t, uint32_t*, hipStream_t) { return hipErrorNotSupported; }
hipError_t scratch_workspace(void**, hipStream_t) { return hipErrorNotSupported; }
}  // namespace tq

extern "C" hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) {
  return hipErrorNotSupported;
}
extern "C" hipError_t hipStreamSynchronize(hipStream_t) { return hipErrorNotSupported; }

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #cond);  \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static tq_config base(int kc, int kb, int vc, int vb) {
  tq_config c{};
  c.abi_version = TQ_ABI_VERSION;
  c.head_dim = 128;
  c.n_q_heads = 32;
  c.n_kv_heads = 8;
  c.batch = 2;
  c.max_ctx = 1000;
  c.k_codec = kc;
  c.k_bits = kb;
  c.qjl_m = kc == TQ_CODEC_POLAR_QJL ? 128 : 0;
  c.v_codec = vc;
  c.v_bits = vb;
  c.seed = 42;
  c.layer = 3;
  return c;
}

int main() {
  for (int s = 0; s <= 6; ++s) EXPECT(tq_status_string(static_cast<tq_status>(s)) != nullptr);
  const int pairs[][4] = {
      {TQ_CODEC_POLAR_QJL, 2, TQ_CODEC_POLAR, 2}, {TQ_CODEC_POLAR_QJL, 3, TQ_CODEC_POLAR, 3},
      {TQ_CODEC_POLAR_QJL, 4, TQ_CODEC_POLAR, 4}, {TQ_CODEC_POLAR, 3, TQ_CODEC_RAW_F32, 32},
      {TQ_CODEC_Q8_BLOCK32, 8, TQ_CODEC_POLAR, 2}, {TQ_CODEC_RAW_F32, 32, TQ_CODEC_RAW_F32, 32},
      {TQ_CODEC_POLAR_TREE, 3, TQ_CODEC_POLAR_TREE, 2}, {TQ_CODEC_POLAR_TREE, 4, TQ_CODEC_POLAR, 4}};
  // fake, 256-byte aligned device addresses: argument checks only look at them
  void* dev = reinterpret_cast<void*>(uintptr_t{1} << 20);
  void* odd = reinterpret_cast<void*>((uintptr_t{1} << 20) + 2);
  const int32_t* lens = static_cast<const int32_t*>(dev);
  float* fdev = static_cast<float*>(dev);
  for (const auto& p : pairs) {
    tq_config c = base(p[0], p[1], p[2], p[3]);
    uint64_t kb = 0, vb = 0, pb = 0, wb = 0, wb2 = 0;
    EXPECT(tq_cache_bytes(&c, &kb, &vb) == TQ_OK && kb > 0 && vb > 0);
    EXPECT(tq_params_bytes(&c, &pb) == TQ_OK && pb > 0);
    std::vector<uint8_t> img(pb);
    EXPECT(tq_params_host(&c, img.data(), pb) == TQ_OK);
    EXPECT(tq_params_host(&c, img.data(), pb - 1) == TQ_EWORKSPACE);
    EXPECT(tq_params_host(&c, nullptr, pb) == TQ_EINVAL);
    for (int n : {0, 1, 127, 128, 129, 999, 1000}) {
      EXPECT(tq_decode_workspace_bytes(&c, n, &wb) == TQ_OK && wb > 0);
      EXPECT(tq_decode_workspace_bytes(&c, 1000, &wb2) == TQ_OK && wb2 >= wb);
    }
    EXPECT(tq_decode_workspace_bytes(&c, 1001, &wb) == TQ_EINVAL);
    EXPECT(tq_decode_workspace_bytes(&c, -1, &wb) == TQ_EINVAL);
    // the copy to the device fails in the stub: reported, not thrown
    EXPECT(tq_init_params(&c, dev, pb, nullptr) == TQ_EDEVICE);
    EXPECT(tq_init_params(&c, odd, pb, nullptr) == TQ_EINVAL);
    // append: argument checks, then the (stubbed) launch
    EXPECT(tq_quantize_append(&c, dev, dev, dev, lens, 0, dev, dev, TQ_BF16, 0, nullptr) == TQ_OK);
    EXPECT(tq_quantize_append(&c, dev, dev, dev, lens, 999, dev, dev, TQ_BF16, 2, nullptr) == TQ_ECAPACITY);
    EXPECT(tq_quantize_append(&c, dev, dev, dev, lens, 0, dev, dev, 7, 1, nullptr) == TQ_EINVAL);
    EXPECT(tq_quantize_append(&c, dev, nullptr, dev, lens, 0, dev, dev, TQ_BF16, 1, nullptr) == TQ_EINVAL);
    EXPECT(tq_quantize_append(&c, odd, dev, dev, lens, 0, dev, dev, TQ_BF16, 1, nullptr) == TQ_EINVAL);
    EXPECT(tq_quantize_append(&c, dev, dev, dev, lens, 0, dev, dev, TQ_BF16, 5, nullptr) == TQ_EDEVICE);
    // decode
    uint64_t need = 0;
    EXPECT(tq_decode_workspace_bytes(&c, 700, &need) == TQ_OK);
    EXPECT(tq_decode_attention(&c, dev, dev, dev, lens, 700, fdev, fdev, nullptr, dev, need - 1, nullptr) ==
           TQ_EWORKSPACE);
    EXPECT(tq_decode_attention(&c, dev, dev, dev, lens, 1001, fdev, fdev, nullptr, dev, need, nullptr) == TQ_EINVAL);
    EXPECT(tq_decode_attention(&c, dev, dev, dev, lens, 700, nullptr, fdev, nullptr, dev, need, nullptr) ==
           TQ_EINVAL);
    EXPECT(tq_decode_attention(&c, dev, dev, dev, lens, 700, fdev, fdev, nullptr, dev, need, nullptr) == TQ_EDEVICE);
    EXPECT(tq_decode_attention_noalloc(&c, dev, dev, dev, lens, 700, fdev, fdev, nullptr, nullptr) == TQ_EDEVICE);
    EXPECT(tq_decode_attention_noalloc(&c, dev, dev, dev, lens, 1001, fdev, fdev, nullptr, nullptr) == TQ_EINVAL);
    EXPECT(tq_append_decode(&c, dev, dev, dev, lens, 1000, dev, dev, TQ_BF16, fdev, fdev, nullptr, dev, need,
                            nullptr) == TQ_ECAPACITY);
    // dequantize
    EXPECT(tq_dequantize(&c, dev, dev, dev, 0, 0, 0, fdev, fdev, 0, nullptr) == TQ_OK);
    EXPECT(tq_dequantize(&c, dev, dev, dev, 2, 0, 1, fdev, fdev, 0, nullptr) == TQ_EINVAL);
    EXPECT(tq_dequantize(&c, dev, dev, dev, 0, 990, 11, fdev, fdev, 0, nullptr) == TQ_EINVAL);
    EXPECT(tq_dequantize(&c, dev, dev, dev, 0, 0, 1, fdev, fdev, 2u, nullptr) == TQ_EINVAL);
    EXPECT(tq_dequantize(&c, dev, dev, dev, 0, 0, 8, fdev, fdev, 0, nullptr) == TQ_EDEVICE);
  }
  // malformed configurations
  tq_config c = base(TQ_CODEC_POLAR_QJL, 3, TQ_CODEC_POLAR, 2);
  uint64_t kb = 0, vb = 0;
  tq_config bad = c;
  bad.abi_version = 99;
  EXPECT(tq_cache_bytes(&bad, &kb, &vb) != TQ_OK);
  bad = c;
  bad.head_dim = 64;
  EXPECT(tq_cache_bytes(&bad, &kb, &vb) == TQ_EUNSUPPORTED);
  bad = c;
  bad.n_q_heads = 33;
  EXPECT(tq_cache_bytes(&bad, &kb, &vb) == TQ_EINVAL);
  bad = c;
  bad.k_bits = 9;
  EXPECT(tq_cache_bytes(&bad, &kb, &vb) != TQ_OK);
  bad = c;
  bad.batch = -1;
  EXPECT(tq_cache_bytes(&bad, &kb, &vb) == TQ_EINVAL);
  bad = c;
  bad.decode_chunk = 100;
  EXPECT(tq_cache_bytes(&bad, &kb, &vb) == TQ_EINVAL);
  EXPECT(tq_cache_bytes(nullptr, &kb, &vb) == TQ_EINVAL);
  EXPECT(tq_cache_bytes(&c, nullptr, &vb) == TQ_EINVAL);
  // the measurement helper's checks
  uint32_t* sink = static_cast<uint32_t*>(dev);
  EXPECT(tq_stream_read(dev, 0, sink, nullptr) == TQ_OK);
  EXPECT(tq_stream_read(dev, 17, sink, nullptr) == TQ_EINVAL);
  EXPECT(tq_stream_read(nullptr, 16, sink, nullptr) == TQ_EINVAL);
  EXPECT(tq_stream_read(dev, 16, sink, nullptr) == TQ_EDEVICE);
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("host ABI checks clean\n");
  return 0;
}

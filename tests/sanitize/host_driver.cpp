// Drives the host-side code of libhkv (format set-up and validation, the
// decode planner through hkv_decode_workspace_bytes, and every entry point's
// argument checks) with no GPU, for runs under AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_sanitize.py).  Every call here
// returns before anything is enqueued.  Exits non-zero on an unexpected
// status.
#include <cstdio>
#include <cstring>

#include "hkv.h"

static int fails = 0;
static void expect(bool ok, const char* what) {
  if (!ok) {
    std::printf("unexpected: %s (%s)\n", what, hkv_last_error());
    ++fails;
  }
}

int main() {
  const char* names[] = {"q4_0", "q8_0", "octave_k3v4", "octave_k3v3", "octave_k3v3_compact"};
  const int heads[] = {64, 128, 192, 256, 320, 96};
  for (const char* n : names)
    for (int d : heads)
      for (int rope : {0, 64, 128, 32})
        for (int ps : {1, 16, 64, 1024, 0}) {
          hkv_format f;
          std::memset(&f, 0, sizeof(f));
          if (hkv_format_init(&f, n, d, rope, ps) != HKV_OK) continue;
          for (int hq : {1, 8, 16, 32})
            for (int hkv : {1, 2, 4, 3})
              for (int nqs : {1, 4, 8, 16, 17})
                for (int klen : {0, 1, 255, 4096, 131072})
                  (void)hkv_decode_workspace_bytes(&f, 4 * nqs, hq, hkv, klen, nqs);
          // argument checks: all of these fail before any HIP call
          float dummy[4];
          uint8_t* cache = reinterpret_cast<uint8_t*>(dummy) + 1;  // misaligned
          expect(hkv_quantize_append(&f, dummy, dummy, HKV_F32, 4, 2, nullptr, nullptr, nullptr) ==
                     HKV_ERR_INVALID_ARG, "quantize_append null pointers");
          expect(hkv_quantize_append(&f, dummy, dummy, 7, 4, 2, nullptr, nullptr,
                                     nullptr) == HKV_ERR_INVALID_ARG, "quantize_append dtype");
          expect(hkv_dequantize(&f, cache, 2, reinterpret_cast<int64_t*>(dummy), 1, 0, dummy,
                                dummy, nullptr) == HKV_ERR_INVALID_ARG, "dequantize alignment");
          expect(hkv_decode_attention(&f, dummy, HKV_F32, 2, 16, 3, nullptr, nullptr, 1, nullptr,
                                      nullptr, 64, 1, 0.1f, 0, nullptr, nullptr, 0, nullptr) ==
                     HKV_ERR_INVALID_ARG, "decode head ratio");
          expect(hkv_decode_attention(&f, dummy, HKV_F32, 3, 16, 2, nullptr, nullptr, 1, nullptr,
                                      nullptr, 64, 2, 0.1f, 0, nullptr, nullptr, 0, nullptr) ==
                     HKV_ERR_INVALID_ARG, "decode queries_per_seq");
          expect(hkv_decode_attention(&f, dummy, HKV_F32, 2, 16, 2, nullptr, nullptr, 1, nullptr,
                                      nullptr, 64, 1, 0.1f, 8u, nullptr, nullptr, 0, nullptr) ==
                     HKV_ERR_INVALID_ARG, "decode flags");
          expect(hkv_decode_attention_noalloc(&f, dummy, HKV_F32, 2, 16, 3, nullptr, nullptr, 1,
                                              nullptr, nullptr, 64, 1, 0.1f, 0, nullptr,
                                              nullptr) == HKV_ERR_INVALID_ARG,
                 "decode_noalloc head ratio");
          hkv_format g = f;
          g.slot_bytes += 1;
          expect(hkv_quantize_append(&g, dummy, dummy, HKV_F32, 1, 1, nullptr, nullptr, nullptr) ==
                     HKV_ERR_INVALID_ARG, "inconsistent descriptor");
        }
  expect(hkv_format_init(nullptr, "q4_0", 256, 0, 16) == HKV_ERR_INVALID_ARG, "null format");
  expect(hkv_hadamard(nullptr, HKV_F32, nullptr, 4, 100, 64, nullptr, 0, nullptr) ==
             HKV_ERR_INVALID_ARG, "hadamard n");
  expect(std::strlen(hkv_version()) > 0, "version");
  std::printf(fails ? "host driver: FAILED\n" : "host driver: ok\n");
  return fails ? 1 : 0;
}

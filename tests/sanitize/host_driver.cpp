// Host-side exercise of the encoder and the blob validator for a build with
// AddressSanitizer and UndefinedBehaviorSanitizer: every format over several
// geometries and value distributions (random, constant, one rare symbol), the
// blob validated, then validated again after truncations and byte flips.
// Any memory or undefined-behaviour error aborts the run; prints "ok".
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "../../include/dgt.h"

namespace {

struct Case {
  uint32_t fmt, n, k, tn, tk, lanes, pb;
};

int fail(const char* what, const Case& c, int rc) {
  std::fprintf(stderr, "%s: fmt %u %ux%u tile %ux%u R %u: rc %d\n", what, c.fmt, c.n, c.k, c.tn,
               c.tk, c.lanes, rc);
  return 1;
}

bool wide(uint32_t fmt) {
  return fmt == DGT_FMT_BF16_SPLIT || fmt == DGT_FMT_BF16_EXP || fmt == DGT_FMT_BF16_PAIR ||
         fmt == DGT_FMT_BF16_WORD;
}

// weights of a case: mode 0 random in the format's range, 1 constant, 2 one rare value
std::vector<uint8_t> weights(const Case& c, int mode, std::mt19937& g) {
  const size_t nk = (size_t)c.n * c.k;
  std::vector<uint8_t> w(nk * (wide(c.fmt) ? 2 : 1));
  std::normal_distribution<float> nd(0.f, 1.f);
  for (size_t i = 0; i < nk; ++i) {
    uint32_t v;
    if (c.fmt == DGT_FMT_INT4 || c.fmt == DGT_FMT_INT4_PAIR) {
      const float x = 8.f + 1.2f * nd(g);
      v = (uint32_t)std::min(15.f, std::max(0.f, x + 0.5f));
      if (mode == 1) v = 7;
      if (mode == 2) v = (i == 77) ? 15 : 8;
    } else if (wide(c.fmt)) {
      float x = 0.02f * nd(g);
      uint32_t b;
      std::memcpy(&b, &x, 4);
      v = b >> 16;  // truncation is enough for a distribution
      if ((v & 0x7F80u) == 0x7F80u) v = 0x3F80;  // no inf / nan patterns
      if (mode == 1) v = 0x3F80;
      if (mode == 2) v = (i == 77) ? 0xC2F0 : 0x3C24;
    } else {
      const float x = 8.f * nd(g);
      v = (uint32_t)(int32_t)std::min(127.f, std::max(-127.f, x)) & 0xFFu;
      if (c.fmt == DGT_FMT_FP8_E4M3 && (v & 0x7F) == 0x7F) v = 0x38;  // no nan codes
      if (mode == 1) v = 3;
      if (mode == 2) v = (i == 77) ? 0x21 : 0x05;
    }
    if (wide(c.fmt)) {
      w[2 * i] = (uint8_t)(v & 0xFF);
      w[2 * i + 1] = (uint8_t)(v >> 8);
    } else {
      w[i] = (uint8_t)v;
    }
  }
  return w;
}

}  // namespace

int main() {
  const Case cases[] = {
      {DGT_FMT_INT8, 256, 64, 128, 32, 32, 12},       {DGT_FMT_INT8, 128, 128, 128, 64, 64, 12},
      {DGT_FMT_INT4, 256, 256, 128, 64, 64, 12},      {DGT_FMT_INT4, 256, 256, 128, 64, 128, 12},
      {DGT_FMT_FP8_E4M3, 512, 128, 256, 64, 64, 12},  {DGT_FMT_BF16_SPLIT, 256, 128, 128, 64, 64, 12},
      {DGT_FMT_BF16_SPLIT, 256, 64, 256, 32, 64, 12}, {DGT_FMT_INT4_PAIR, 256, 256, 128, 64, 64, 12},
      {DGT_FMT_BF16_EXP, 256, 128, 128, 64, 64, 12},  {DGT_FMT_BF16_PAIR, 256, 128, 128, 64, 64, 12},
      {DGT_FMT_BF16_PAIR, 128, 128, 128, 32, 32, 12}, {DGT_FMT_BF16_WORD, 256, 128, 128, 64, 64, 16},
      {DGT_FMT_BF16_WORD, 256, 256, 256, 64, 64, 16},
  };
  std::mt19937 g(1234);
  int n_blobs = 0, n_rejected = 0;
  for (const Case& c : cases) {
    for (int mode = 0; mode < 3; ++mode) {
      const std::vector<uint8_t> w = weights(c, mode, g);
      dgt_params p{c.fmt, c.n, c.k, c.tn, c.tk, c.lanes, c.pb, 0};
      const size_t cap = dgt_compress_bound(&p);
      if (cap == 0) return fail("compress_bound", c, 0);
      std::vector<uint8_t> blob(cap);
      size_t size = 0;
      int rc = dgt_compress_layer(&p, w.data(), blob.data(), cap, &size);
      if (rc != DGT_OK) return fail("compress", c, rc);
      blob.resize(size);
      dgt_info info;
      rc = dgt_layer_info(blob.data(), blob.size(), &info);
      if (rc != DGT_OK || info.total_bytes != size) return fail("layer_info", c, rc);
      ++n_blobs;
      // a buffer one byte short is refused
      std::vector<uint8_t> small(size - 1);
      size_t s2 = 0;
      rc = dgt_compress_layer(&p, w.data(), small.data(), small.size(), &s2);
      if (rc != DGT_E_BUFSIZE) return fail("short buffer", c, rc);
      // truncations and byte flips: any status, no memory error
      std::uniform_int_distribution<size_t> pos(0, size - 1);
      for (int t = 0; t < 64; ++t) {
        std::vector<uint8_t> bad = blob;
        size_t len = size;
        if (t < 16) {
          len = pos(g);
        } else {
          for (int f = 0; f < 1 + t % 4; ++f) bad[pos(g)] ^= (uint8_t)(1u << (t % 8));
        }
        dgt_info bi;
        if (dgt_layer_info(bad.data(), len, &bi) != DGT_OK) ++n_rejected;
      }
    }
  }
  // argument errors
  dgt_params bad{DGT_FMT_INT8, 100, 64, 128, 64, 64, 12, 0};
  if (dgt_compress_bound(&bad) != 0) return 1;
  if (dgt_layer_info(nullptr, 0, nullptr) == DGT_OK) return 1;
  std::printf("ok: %d blobs, %d corrupted copies rejected\n", n_blobs, n_rejected);
  return 0;
}

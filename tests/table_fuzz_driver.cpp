// Host driver for the table builders (asv_seg_table_build,
// asv_block_table_build) under AddressSanitizer and UndefinedBehaviorSanitizer:
// random valid rounds (size query, exact blob, a blob one byte short) and
// malformed ones, each with its expected return code. Built and run by
// tests/test_table_sanitized.py with g++ (host code only, no GPU).

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "asv.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what, int iter) {
  if (!ok) {
    std::fprintf(stderr, "FAIL %s (iteration %d)\n", what, iter);
    ++failures;
  }
}

typedef int (*BuildFn)(const asv_stream_desc*, int32_t, const void* const*, int32_t, const void* const*,
                       const void* const*, int32_t, void*, size_t, asv_table_info*);

// Fake, non-overlapping, 16-byte aligned device addresses for every layer and stream.
struct Ptrs {
  std::vector<const void*> conv, k, v;
};

Ptrs make_ptrs(const std::vector<asv_stream_desc>& s, int n_conv, int n_attn) {
  Ptrs p;
  uintptr_t next = uintptr_t(1) << 40;
  for (int l = 0; l < n_conv; ++l)
    for (size_t i = 0; i < s.size(); ++i) {
      p.conv.push_back(reinterpret_cast<const void*>(next));
      next += 2 * 2048 * 2;
    }
  for (int l = 0; l < n_attn; ++l)
    for (size_t i = 0; i < s.size(); ++i) {
      const uintptr_t bytes = uintptr_t(8) * uintptr_t(s[i].kv_capacity) * 64 * 2;
      p.k.push_back(reinterpret_cast<const void*>(next));
      next += bytes;
      p.v.push_back(reinterpret_cast<const void*>(next));
      next += bytes;
    }
  return p;
}

int build(BuildFn fn, const std::vector<asv_stream_desc>& s, const Ptrs& p, int n_conv, int n_attn,
          std::vector<unsigned char>* blob, asv_table_info* info, long shrink) {
  asv_table_info q;
  std::memset(&q, 0, sizeof(q));
  const int rc = fn(s.data(), int32_t(s.size()), p.conv.data(), n_conv, p.k.data(), p.v.data(), n_attn,
                    nullptr, 0, &q);
  if (rc != ASV_OK) return rc;
  const size_t bytes = size_t(q.blob_bytes) - size_t(shrink);
  blob->assign(bytes == 0 ? 1 : bytes, 0xAB);
  return fn(s.data(), int32_t(s.size()), p.conv.data(), n_conv, p.k.data(), p.v.data(), n_attn,
            blob->data(), bytes, info);
}

}  // namespace

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 400;
  std::mt19937 rng(12345);
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  for (int it = 0; it < iters; ++it) {
    const BuildFn fn = (it & 1) ? asv_block_table_build : asv_seg_table_build;
    // a valid round: windows of 1..40 rows (up to 2,048 in all), keys up to 131,072
    std::vector<asv_stream_desc> s;
    int rows = 0;
    const int n = uni(1, 60);
    for (int i = 0; i < n; ++i) {
      const int w = uni(0, 3) == 0 ? uni(17, 40) : uni(1, 16);
      if (rows + w > ASV_MAX_ROWS) break;
      const int lo = w, hi = uni(0, 4) == 0 ? ASV_MAX_KEYS : 40000;
      const int k = uni(lo, hi < lo ? lo : hi);
      int cap = (k + 31) / 32 * 32 + 32 * uni(0, 3);
      if (cap > ASV_MAX_KEYS) cap = (k + 31) / 32 * 32;
      s.push_back(asv_stream_desc{w, k, cap});
      rows += w;
    }
    const int n_conv = uni(0, 3), n_attn = uni(0, 3);
    const Ptrs p = make_ptrs(s, n_conv, n_attn);
    std::vector<unsigned char> blob;
    asv_table_info info;
    std::memset(&info, 0, sizeof(info));
    int rc = build(fn, s, p, n_conv, n_attn, &blob, &info, 0);
    expect(rc == ASV_OK, "valid round builds", it);
    if (rc == ASV_OK) {
      expect(info.n_rows == rows && info.n_streams == int32_t(s.size()), "row and stream counts", it);
      expect(info.n_work >= 1 && info.partial_count >= info.n_rows * 32, "work and partial counts", it);
      expect(size_t(info.blob_bytes) == blob.size(), "blob size", it);
    }
    rc = build(fn, s, p, n_conv, n_attn, &blob, &info, 1);
    expect(rc == ASV_E_CAPACITY, "a blob one byte short is refused", it);

    // malformed rounds, one fault each
    std::vector<asv_stream_desc> bad = s;
    const int j = uni(0, int(bad.size()) - 1);
    switch (it % 5) {
      case 0: bad[j].rows = 0; break;
      case 1: bad[j].key_count = bad[j].rows - 1; break;
      case 2: bad[j].kv_capacity = (bad[j].key_count + 31) / 32 * 32 + 16; break;   // not a multiple of 32
      case 3: bad[j].kv_capacity = ASV_MAX_KEYS + 32; bad[j].key_count = ASV_MAX_KEYS + 1; break;
      default: bad.push_back(asv_stream_desc{ASV_MAX_ROWS, ASV_MAX_ROWS, ASV_MAX_ROWS}); break;
    }
    const Ptrs pb = make_ptrs(bad, n_conv, n_attn);
    asv_table_info q;
    std::memset(&q, 0, sizeof(q));
    rc = fn(bad.data(), int32_t(bad.size()), pb.conv.data(), n_conv, pb.k.data(), pb.v.data(), n_attn,
            nullptr, 0, &q);
    expect(rc == ASV_E_SHAPE, "a malformed round is refused by shape", it);

    // aliasing: two streams given the same K cache in a layer
    if (n_attn > 0 && s.size() >= 2) {
      Ptrs pa = p;
      pa.k[1] = pa.k[0];
      rc = fn(s.data(), int32_t(s.size()), pa.conv.data(), n_conv, pa.k.data(), pa.v.data(), n_attn,
              nullptr, 0, &q);
      expect(rc == ASV_E_ARG, "aliasing caches are refused", it);
    }
  }
  std::printf("table fuzz: %d iterations, %d failures\n", iters, failures);
  return failures == 0 ? 0 : 1;
}

// Host-side memory-safety harness for libtria, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on its host code (tests/test_asan_host.py builds and
// runs it on the CPU).  No GPU work is done: every call either reads and writes
// host memory only (the stats-file functions) or is rejected by the C ABI's
// validation before anything is launched.
//
//   1. A seeded byte-mutation fuzz of tria_stats_parse: valid files of every
//      version are encoded, then mutated (bit flips, random bytes, truncation,
//      extension, header fields set to boundary values) and parsed into output
//      arrays of exactly the size the parsed header implies, each a heap block of
//      its own so that any read or write past a buffer is caught.
//   2. Argument validation of every device entry point with invalid arguments:
//      the status must be an error, and nothing may be read past the host arrays
//      the call is given (the offsets array is sized exactly n_offsets).
//
// The random numbers come from SplitMix64 (Steele, Lea and Flood, "Fast
// splittable pseudorandom number generators", OOPSLA 2014).
#include "tria.h"

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <vector>

namespace {

uint64_t g_state = 1;

uint64_t next_u64() {
  uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

uint32_t below(uint32_t n) { return n ? (uint32_t)(next_u64() % n) : 0; }

int g_fail = 0;

void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "FAIL: %s (%s)\n", what, tria_last_error());
    ++g_fail;
  }
}

// A heap copy of exactly n bytes (a distinct block even for n == 0).
std::unique_ptr<unsigned char[]> exact_copy(const std::vector<unsigned char>& v, size_t n) {
  std::unique_ptr<unsigned char[]> p(new unsigned char[n ? n : 1]);
  if (n) std::memcpy(p.get(), v.data(), n);
  return p;
}

struct Base {
  std::vector<unsigned char> bytes;
  tria_stats_info info;
  std::vector<float> re, im, ab, mrl, scales;
};

Base make_base(uint32_t version, bool scales, uint32_t L, uint32_t H, uint32_t Hkv, uint32_t fc) {
  Base b;
  b.info = tria_stats_info{version, L, H, Hkv, fc, 2 * fc, scales ? 1 : 0, version >= 2 ? 1 : 0};
  const size_t n = (size_t)L * H * fc;
  for (auto* v : {&b.re, &b.im, &b.ab, &b.mrl}) {
    v->resize(n);
    for (float& x : *v) x = (float)((double)(next_u64() >> 11) * 0x1.0p-53 * 4.0 - 2.0);
  }
  b.scales.resize(L);
  for (float& x : b.scales) x = 0.5f + (float)below(100) / 50.0f;
  const size_t need = tria_stats_encode(&b.info, b.re.data(), b.im.data(), b.ab.data(), b.mrl.data(),
                                        scales ? b.scales.data() : nullptr, nullptr, 0);
  expect(need > 0, "encode size");
  b.bytes.resize(need);
  const size_t got = tria_stats_encode(&b.info, b.re.data(), b.im.data(), b.ab.data(), b.mrl.data(),
                                       scales ? b.scales.data() : nullptr, b.bytes.data(), need);
  expect(got == need, "encode");
  return b;
}

void put_u32(std::vector<unsigned char>& v, size_t off, uint32_t x) {
  if (off + 4 > v.size()) return;
  for (int i = 0; i < 4; ++i) v[off + i] = (unsigned char)(x >> (8 * i));
}

void mutate(std::vector<unsigned char>& v) {
  static const uint32_t special[] = {0u, 1u, 2u, 3u, 4u, 7u, 4096u, 4097u, 65536u, 65537u,
                                     0x7fffffffu, 0x80000000u, 0xffffffffu, 0x54524941u};
  switch (below(7)) {
    case 0:  // flip a bit
      if (!v.empty()) v[below((uint32_t)v.size())] ^= (unsigned char)(1u << below(8));
      break;
    case 1:  // a random byte
      if (!v.empty()) v[below((uint32_t)v.size())] = (unsigned char)next_u64();
      break;
    case 2:  // truncate
      v.resize(below((uint32_t)v.size() + 1));
      break;
    case 3:  // extend
      for (uint32_t i = 0, k = 1 + below(64); i < k; ++i) v.push_back((unsigned char)next_u64());
      break;
    case 4:  // a header field (magic .. flags) set to a boundary value
      put_u32(v, 4 * below(8), special[below(sizeof special / sizeof special[0])]);
      break;
    case 5:  // a header field set to a random value
      put_u32(v, 4 * below(8), (uint32_t)next_u64());
      break;
    default:  // the size the header implies after a change of fc, kept consistent
      put_u32(v, 20, 1 + below(8));
      break;
  }
}

// Parses a buffer of exactly n bytes: the header first, then into arrays of the
// exact size the header gives.  Returns whether the file was accepted.
bool parse_exact(const std::vector<unsigned char>& v, size_t n) {
  auto buf = exact_copy(v, n);
  tria_stats_info info{};
  tria_status st = tria_stats_parse(buf.get(), n, &info, nullptr, nullptr, nullptr, nullptr, nullptr);
  if (st != TRIA_OK) {
    expect(st == TRIA_EINVAL || st == TRIA_ESHAPE, "parse status is EINVAL or ESHAPE");
    expect(std::strlen(tria_last_error()) > 0, "a rejected file leaves a message");
    return false;
  }
  const size_t cnt = (size_t)info.n_layers * info.n_heads * info.fc;
  std::unique_ptr<float[]> re(new float[cnt]), im(new float[cnt]), ab(new float[cnt]), mrl(new float[cnt]),
      sc(new float[info.n_layers]);
  tria_stats_info again{};
  st = tria_stats_parse(buf.get(), n, &again, re.get(), im.get(), ab.get(), mrl.get(), sc.get());
  expect(st == TRIA_OK, "a header that parses parses with its arrays");
  expect(std::memcmp(&again, &info, sizeof info) == 0, "the same header both times");
  // re-encoding what was read gives the same bytes
  const size_t need = tria_stats_encode(&info, re.get(), im.get(), ab.get(), mrl.get(),
                                        info.has_budget_scales ? sc.get() : nullptr, nullptr, 0);
  expect(need == n, "the parsed header implies the file's size");
  if (need == n) {
    std::unique_ptr<unsigned char[]> out(new unsigned char[need]);
    tria_stats_encode(&info, re.get(), im.get(), ab.get(), mrl.get(), info.has_budget_scales ? sc.get() : nullptr,
                      out.get(), need);
    expect(std::memcmp(out.get(), buf.get(), n) == 0, "encode(parse(file)) == file");
  }
  return true;
}

void fuzz_stats(int iters) {
  std::vector<Base> bases;
  const uint32_t shapes[][4] = {{1, 1, 1, 1}, {2, 4, 2, 4}, {3, 8, 2, 16}, {1, 6, 3, 64}};
  for (uint32_t version = 1; version <= 3; ++version)
    for (int sc = 0; sc < (version == 3 ? 2 : 1); ++sc)
      for (const auto& s : shapes) bases.push_back(make_base(version, sc != 0, s[0], s[1], s[2], s[3]));
  // every base file round-trips
  for (const Base& b : bases) {
    const size_t cnt = b.re.size();
    std::unique_ptr<float[]> re(new float[cnt]), im(new float[cnt]), ab(new float[cnt]), mrl(new float[cnt]),
        sc(new float[b.info.n_layers]);
    auto buf = exact_copy(b.bytes, b.bytes.size());
    tria_stats_info info{};
    expect(tria_stats_parse(buf.get(), b.bytes.size(), &info, re.get(), im.get(), ab.get(), mrl.get(), sc.get()) ==
               TRIA_OK,
           "a base file parses");
    expect(std::memcmp(re.get(), b.re.data(), cnt * 4) == 0 && std::memcmp(im.get(), b.im.data(), cnt * 4) == 0 &&
               std::memcmp(ab.get(), b.ab.data(), cnt * 4) == 0,
           "the statistics round-trip");
    expect(info.version < 2 || std::memcmp(mrl.get(), b.mrl.data(), cnt * 4) == 0, "mrl round-trips");
    for (uint32_t l = 0; l < b.info.n_layers; ++l)
      expect(sc[l] == (b.info.has_budget_scales ? b.scales[l] : 1.0f), "layer scales (1.0 when absent)");
  }
  int accepted = 0;
  for (int i = 0; i < iters; ++i) {
    std::vector<unsigned char> v = bases[below((uint32_t)bases.size())].bytes;
    for (uint32_t k = 0, nm = 1 + below(6); k < nm; ++k) mutate(v);
    accepted += parse_exact(v, v.size()) ? 1 : 0;
  }
  // NULL arguments
  tria_stats_info info{};
  expect(tria_stats_parse(nullptr, 0, &info, nullptr, nullptr, nullptr, nullptr, nullptr) == TRIA_EINVAL,
         "NULL bytes");
  expect(tria_stats_parse(bases[0].bytes.data(), bases[0].bytes.size(), nullptr, nullptr, nullptr, nullptr, nullptr,
                          nullptr) == TRIA_EINVAL,
         "NULL info");
  std::printf("stats fuzz: %d mutated files, %d accepted\n", iters, accepted);
}

void scalings() {
  // band mask and per-layer budgets on exact-size arrays, including rejected inputs
  const int rows = 3, fc = 5;
  std::unique_ptr<float[]> re(new float[rows * fc]), im(new float[rows * fc]), ab(new float[rows * fc]),
      mask(new float[fc]);
  for (int i = 0; i < rows * fc; ++i) re[i] = 1.0f, im[i] = -0.5f, ab[i] = 2.0f;
  for (int f = 0; f < fc; ++f) mask[f] = 0.25f * f;
  expect(tria_stats_band_mask(rows, fc, mask.get(), re.get(), im.get(), ab.get()) == TRIA_OK, "band mask");
  mask[2] = NAN;
  expect(tria_stats_band_mask(rows, fc, mask.get(), re.get(), im.get(), ab.get()) == TRIA_EINVAL, "NaN mask");
  mask[2] = -1.0f;
  expect(tria_stats_band_mask(rows, fc, mask.get(), re.get(), im.get(), ab.get()) == TRIA_EINVAL, "negative mask");
  std::unique_ptr<int32_t[]> ul(new int32_t[4]), out(new int32_t[4]);
  std::unique_ptr<float[]> sc(new float[2]);
  sc[0] = 1.0f, sc[1] = 0.5f;
  for (int u = 0; u < 4; ++u) ul[u] = u % 2;
  expect(tria_stats_layer_budgets(4, ul.get(), 2, sc.get(), 1001, out.get()) == TRIA_OK && out[0] == 1001 &&
             out[1] == 501,
         "layer budgets, round half up");
  ul[3] = 2;
  expect(tria_stats_layer_budgets(4, ul.get(), 2, sc.get(), 1001, out.get()) == TRIA_EINVAL, "layer out of range");
  sc[1] = INFINITY;
  ul[3] = 1;
  expect(tria_stats_layer_budgets(4, ul.get(), 2, sc.get(), 1001, out.get()) == TRIA_EINVAL, "infinite scale");
}

// Valid host structures for the validation calls; the device pointers are never
// dereferenced (each call is rejected first).
struct Fixture {
  std::unique_ptr<int64_t[]> offs;
  tria_params p;
  tria_kv_view k, v;
  Fixture(int n_off) : offs(new int64_t[n_off]) {
    for (int i = 0; i < n_off; ++i) offs[i] = (int64_t)1 << i;
    p = tria_params{128, 8, 4, 2, TRIA_PAIR_NEOX, TRIA_AGG_MAX, 1e6, offs.get(), n_off, 4, 128, TRIA_OFFSETS_MEAN};
    void* base = reinterpret_cast<void*>(uintptr_t(1) << 40);
    k = tria_kv_view{base, 8 * 4096 * 128, 4096 * 128, 128, nullptr, 0, 0, 0};
    v = k;
    v.base = reinterpret_cast<void*>((uintptr_t(1) << 40) + (uintptr_t(1) << 32));
  }
};

void validation() {
  int32_t* dev = reinterpret_cast<int32_t*>(uintptr_t(1) << 41);
  float* fdev = reinterpret_cast<float*>(uintptr_t(1) << 41);
  void* ws = reinterpret_cast<void*>(uintptr_t(1) << 42);
  for (int trial = 0; trial < 400; ++trial) {
    Fixture f(1 + (int)below(17));
    tria_params p = f.p;
    tria_kv_view k = f.k, v = f.v;
    // one invalid field per call
    switch (trial % 12) {
      case 0: p.head_dim = (int)below(300) | 1; break;
      case 1: p.group = 9 + (int)below(100); break;
      case 2: p.pairing = 2 + (int)below(5); break;
      case 3: p.agg = -1 - (int)below(5); break;
      case 4: p.rope_base = trial % 2 ? NAN : 0.5; break;
      case 5: p.n_offsets = 0; break;
      case 6: p.offsets = nullptr; break;
      case 7: f.offs[below((uint32_t)p.n_offsets)] = -1 - (int64_t)below(9); break;
      case 8: p.offset_reduce = 2 + (int)below(3); break;
      case 9: k.base = reinterpret_cast<void*>((uintptr_t(1) << 40) + 8); break;
      case 10: k.stride_slot = 100; break;
      default: p.sink = -1; break;
    }
    const bool bad_view = trial % 12 == 9 || trial % 12 == 10;
    if (!bad_view) expect(tria_workspace_size(&p, 4, 4096) == 0, "workspace size of invalid params is 0");
    expect(tria_score(&p, &k, 4, 4096, dev, dev, dev, fdev, fdev, fdev, nullptr, fdev, ws, size_t(1) << 40,
                      nullptr) != TRIA_OK,
           "tria_score rejects");
    if (!bad_view) {
      expect(tria_select(&p, 4, 4096, 2048, dev, dev, fdev, dev, dev, ws, size_t(1) << 40, nullptr) != TRIA_OK,
             "tria_select rejects");
      expect(tria_calibrate(&p, ws, 0, 4096 * 128, 128, 4096, fdev, fdev, fdev, nullptr, nullptr, ws,
                            size_t(1) << 40, nullptr) != TRIA_OK,
             "tria_calibrate rejects");
    }
    expect(tria_compact(&p, &k, &v, dev, 1, 4, 4096, 2048, dev, dev, dev, &f.k, &f.v, dev, nullptr) != TRIA_OK,
           "tria_compact rejects");
    expect(tria_append(&p, &k, &v, dev, 4, 4096, dev, dev, 128, ws, ws, dev, ws, nullptr) != TRIA_OK,
           "tria_append rejects");
    expect(tria_compact_inplace(&p, &k, &v, dev, 4, 4096, 2048, dev, dev, dev, ws, nullptr) != TRIA_OK,
           "tria_compact_inplace rejects");
  }
  // NULL structures
  expect(tria_score(nullptr, nullptr, 1, 16, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                    nullptr, 0, nullptr) == TRIA_EINVAL,
         "NULL params");
  expect(tria_workspace_size(nullptr, 1, 16) == 0, "NULL params: no workspace");
  for (int s = TRIA_OK; s <= TRIA_ELAUNCH; ++s)
    expect(std::strlen(tria_strerror((tria_status)s)) > 0, "every status has a name");
}

}  // namespace

int main(int argc, char** argv) {
  g_state = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
  const int iters = argc > 2 ? std::atoi(argv[2]) : 20000;
  fuzz_stats(iters);
  scalings();
  validation();
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}

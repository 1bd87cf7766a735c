// Test driver for the host runtime pieces that need no GPU: repacking a
// canonical expert blob into the device layout, unpacking it again, and the
// host expert path.  Built by tests/test_host_sanitized.py with the address
// and undefined-behaviour sanitizers; the test compares what it writes with
// the oracle.
//
//   host_check <fmt> <hidden> <inter> <rows> <threads> <dir>
// reads <dir>/blob.bin (canonical blob), <dir>/x.bin (bf16 [rows][hidden]),
// <dir>/w.bin (fp32 [rows]); writes <dir>/mats.bin (fp64: gate [I][H], up
// [I][H], down [H][I], decoded from the device layout) and <dir>/p.bin (bf16
// [rows][hidden], the host expert's weighted rows).
//
//   host_check decode <fmt> <hidden> <inter> <dir>
// reads <dir>/blob.bin and writes <dir>/dec.bin: fp32 gate, up, down as the
// host FFN decodes them lane by lane, in [rows][cols] order.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "layout.h"

static std::vector<unsigned char> slurp(const std::string& path) {
  std::vector<unsigned char> v;
  FILE* f = std::fopen(path.c_str(), "rb");
  if (!f) return v;
  unsigned char buf[1 << 16];
  size_t n;
  while ((n = std::fread(buf, 1, sizeof(buf), f)) > 0) v.insert(v.end(), buf, buf + n);
  std::fclose(f);
  return v;
}

static bool spill(const std::string& path, const void* p, size_t n) {
  FILE* f = std::fopen(path.c_str(), "wb");
  if (!f) return false;
  const bool ok = std::fwrite(p, 1, n, f) == n;
  return std::fclose(f) == 0 && ok;
}

static int decode_mode(int argc, char** argv) {
  if (argc != 6) return 2;
  const int fmt = std::atoi(argv[2]), H = std::atoi(argv[3]), I = std::atoi(argv[4]);
  const std::string dir = argv[5];
  const std::vector<unsigned char> blob = slurp(dir + "/blob.bin");
  if (int64_t(blob.size()) != ftmoe::canonical_bytes(fmt, H, I)) return 2;
  const ftmoe::ExpertLayout L = ftmoe::make_layout(fmt, H, I);
  std::vector<uint8_t> dev(size_t(L.bytes));
  ftmoe::repack_expert(L, blob.data(), dev.data());
  std::vector<float> out;
  for (int m = 0; m < 3; ++m) {
    const int R = L.m[m].rows, K = L.m[m].cols, nkb = K / ftmoe::kTileK;
    std::vector<float> mat(size_t(R) * K);
    float w[32];
    for (int rb = 0; rb < R / ftmoe::kTileRows; ++rb)
      for (int kb = 0; kb < nkb; ++kb)
        for (int lane = 0; lane < 64; ++lane) {
          ftmoe::host_decode_lane(L, dev.data(), m, int64_t(rb) * nkb + kb, lane, w);
          const int r = rb * ftmoe::kTileRows + (lane & 15), k0 = kb * ftmoe::kTileK + 32 * (lane >> 4);
          std::memcpy(&mat[size_t(r) * K + k0], w, sizeof(w));
        }
    out.insert(out.end(), mat.begin(), mat.end());
  }
  return spill(dir + "/dec.bin", out.data(), out.size() * 4) ? 0 : 3;
}

int main(int argc, char** argv) {
  if (argc >= 2 && std::string(argv[1]) == "decode") return decode_mode(argc, argv);
  if (argc != 7) {
    std::fprintf(stderr, "usage: host_check fmt hidden inter rows threads dir\n");
    return 2;
  }
  const int fmt = std::atoi(argv[1]), H = std::atoi(argv[2]), I = std::atoi(argv[3]), rows = std::atoi(argv[4]),
            threads = std::atoi(argv[5]);
  const std::string dir = argv[6];
  const std::vector<unsigned char> blob = slurp(dir + "/blob.bin"), xb = slurp(dir + "/x.bin"),
                                   wb = slurp(dir + "/w.bin");
  if (int64_t(blob.size()) != ftmoe::canonical_bytes(fmt, H, I) || xb.size() != size_t(rows) * H * 2 ||
      wb.size() != size_t(rows) * 4) {
    std::fprintf(stderr, "input sizes do not match the shape\n");
    return 2;
  }
  const ftmoe::ExpertLayout L = ftmoe::make_layout(fmt, H, I);
  std::vector<uint8_t> dev(size_t(L.bytes));
  ftmoe::repack_expert(L, blob.data(), dev.data());
  std::vector<double> mats;
  for (int m = 0; m < 3; ++m) {
    std::vector<double> row(size_t(L.m[m].cols));
    for (int r = 0; r < L.m[m].rows; ++r) {
      ftmoe::unpack_row_f64(L, dev.data(), m, r, row.data());
      mats.insert(mats.end(), row.begin(), row.end());
    }
  }
  std::vector<uint16_t> x(size_t(rows) * H), out(size_t(rows) * H);
  std::vector<float> w(static_cast<size_t>(rows));
  std::memcpy(x.data(), xb.data(), xb.size());
  std::memcpy(w.data(), wb.data(), wb.size());
  ftmoe::host_expert(L, dev.data(), x.data(), w.data(), rows, out.data(), threads);
  if (!spill(dir + "/mats.bin", mats.data(), mats.size() * 8) || !spill(dir + "/p.bin", out.data(), out.size() * 2))
    return 3;
  return 0;
}

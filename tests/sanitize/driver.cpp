// Sanitizer driver for the host half of the library (dfh_host.cpp) and the
// CPU oracle (oracle.c), built with AddressSanitizer and UndefinedBehavior-
// Sanitizer by tests/test_sanitizers.py.  It runs every host entry point on
// edge-size inputs of all three kinds, cross-checks the library's sections
// with the oracle's, decodes them with the oracle (serially and over tile
// ranges on threads), round-trips container files, and loads damaged files.
// Exit status 0 when every check holds; the sanitizers abort on the first
// memory or undefined-behaviour error.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "dfh.h"

extern "C" {
typedef struct {
  uint64_t n, total_bits, n_threads, n_tiles, bitstream_bytes, gaps_bytes, tile_out_entries, sm_bytes,
      max_tile_elems;
} oracle_layout_t;
int oracle_histogram(int kind, const void *src, uint64_t n, uint64_t *hist);
int oracle_code_lengths(const uint64_t *hist, int max_len, uint8_t *lengths);
int oracle_layout(int kind, const void *src, uint64_t n, const uint8_t *lengths, oracle_layout_t *out);
int oracle_encode(int kind, const void *src, uint64_t n, const uint8_t *lengths, oracle_layout_t *lay,
                  uint8_t *bitstream, uint8_t *gaps, uint64_t *tile_out, uint8_t *sm);
int oracle_build_lut(const uint8_t *lengths, uint16_t *lut, int cap, int *n_luts);
int oracle_decode_serial(int kind, const uint8_t *lengths, const uint8_t *stream, uint64_t stream_bytes,
                         uint64_t n, const uint8_t *sm, void *dst);
int oracle_decode_tiles(int kind, const uint8_t *lengths, const uint8_t *stream, uint64_t stream_bytes,
                        const uint8_t *gaps, const uint64_t *tile_out, uint64_t n_tiles, uint64_t n_threads,
                        const uint8_t *sm, void *dst, int cpu_threads);
int oracle_pack_u4(const uint8_t *syms, uint64_t n, uint8_t *out);
}

static int failures = 0;
#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      failures++;                                                     \
    }                                                                 \
  } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {  // xorshift64*
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 0x2545F4914F6CDD1Dull;
}
// a bell-shaped small integer: the sum of four uniform bytes
static int bell() {
  const uint64_t r = next_u64();
  return (int)((r & 255) + ((r >> 8) & 255) + ((r >> 16) & 255) + ((r >> 24) & 255));
}

// n elements of one kind as the raw input bytes (uint4: packed)
static std::vector<uint8_t> make_input(int kind, uint64_t n, int shape) {
  std::vector<uint8_t> b;
  if (kind == DF_KIND_BF16) {
    b.resize(2 * n);
    for (uint64_t i = 0; i < n; i++) {
      uint16_t u;
      if (shape == 0) u = (uint16_t)(0x3C00 + (bell() - 510) * 3);  // exponents near 120
      else if (shape == 1) u = (uint16_t)next_u64();                 // every pattern
      else u = 0xBC00;                                                // one symbol
      std::memcpy(&b[2 * i], &u, 2);
    }
  } else if (kind == DF_KIND_U8) {
    b.resize(n);
    for (uint64_t i = 0; i < n; i++)
      b[i] = shape == 0 ? (uint8_t)(bell() / 4) : shape == 1 ? (uint8_t)next_u64() : (uint8_t)77;
  } else {
    std::vector<uint8_t> s(n);
    for (uint64_t i = 0; i < n; i++)
      s[i] = shape == 0 ? (uint8_t)(bell() / 64) : shape == 1 ? (uint8_t)(next_u64() & 15) : (uint8_t)5;
    b.resize((n + 1) / 2);
    oracle_pack_u4(s.data(), n, b.data());
  }
  return b;
}

static std::vector<uint8_t> section(const df_container *c, df_section s) {
  uint64_t nb = 0;
  const uint8_t *p = (const uint8_t *)df_container_section(c, s, &nb);
  return p ? std::vector<uint8_t>(p, p + nb) : std::vector<uint8_t>();
}

static void round_trip(int kind, uint64_t n, int shape, const std::string &tmp) {
  const std::vector<uint8_t> src = make_input(kind, n, shape);
  const void *sp = src.empty() ? nullptr : src.data();
  uint64_t hist[256], ohist[256];
  CHECK(df_histogram((df_kind)kind, sp, n, hist) == DF_OK);
  CHECK(oracle_histogram(kind, sp, n, ohist) == 0);
  CHECK(std::memcmp(hist, ohist, sizeof hist) == 0);
  uint8_t len[256], olen[256];
  CHECK(df_build_codebook(hist, 32, len) == DF_OK);
  CHECK(oracle_code_lengths(ohist, 32, olen) >= 0);
  CHECK(std::memcmp(len, olen, 256) == 0);
  df_container *c = nullptr;
  CHECK(df_encode((df_kind)kind, sp, n, len, &c) == DF_OK);
  if (!c) return;
  CHECK(df_container_validate(c) == DF_OK);
  df_info inf;
  CHECK(df_container_info(c, &inf) == DF_OK);

  // the oracle's encoding of the same input with the same lengths
  oracle_layout_t lay;
  CHECK(oracle_layout(kind, sp, n, len, &lay) == 0);
  std::vector<uint8_t> bs(lay.bitstream_bytes), gp(lay.gaps_bytes), sm(lay.sm_bytes);
  std::vector<uint64_t> to(lay.tile_out_entries);
  CHECK(oracle_encode(kind, sp, n, len, &lay, bs.data(), gp.data(), to.data(),
                      kind == DF_KIND_BF16 ? sm.data() : nullptr) == 0);
  CHECK(section(c, DF_SEC_BITSTREAM) == bs);
  CHECK(section(c, DF_SEC_GAPS) == gp);
  const std::vector<uint8_t> lto = section(c, DF_SEC_TILE_OUT);
  CHECK(lto.size() == 8 * to.size() && std::memcmp(lto.data(), to.data(), lto.size()) == 0);
  if (kind == DF_KIND_BF16) CHECK(section(c, DF_SEC_SIGN_MANTISSA) == sm);
  std::vector<uint16_t> lut(64 * 256);
  int nl = 0;
  CHECK(oracle_build_lut(len, lut.data(), 64, &nl) == 0);
  const std::vector<uint8_t> llut = section(c, DF_SEC_LUT);
  CHECK(llut.size() == 512u * (unsigned)nl && std::memcmp(llut.data(), lut.data(), llut.size()) == 0);

  // the oracle decodes the library's container
  if (n) {
    const std::vector<uint8_t> sbs = section(c, DF_SEC_BITSTREAM), sgp = section(c, DF_SEC_GAPS),
                               ssm = section(c, DF_SEC_SIGN_MANTISSA);
    const size_t esz = kind == DF_KIND_BF16 ? 2 : 1;
    std::vector<uint8_t> out(n * esz), out2(n * esz);
    CHECK(oracle_decode_tiles(kind, len, sbs.data(), sbs.size(), sgp.data(), (const uint64_t *)lto.data(),
                              inf.n_tiles, inf.n_threads, ssm.empty() ? nullptr : ssm.data(), out.data(), 3) == 0);
    CHECK(oracle_decode_serial(kind, len, sbs.data(), sbs.size(), n, ssm.empty() ? nullptr : ssm.data(),
                               out2.data()) == 0);
    CHECK(out == out2);
    if (kind == DF_KIND_U4) {
      std::vector<uint8_t> packed((n + 1) / 2);
      oracle_pack_u4(out.data(), n, packed.data());
      CHECK(packed == src);
    } else {
      CHECK(out == src);
    }
  }

  // device-encoder host helpers agree with the container
  if (n) {
    df_info lay2;
    uint8_t last = 0;
    if (kind == DF_KIND_BF16) last = (uint8_t)((((const uint16_t *)src.data())[n - 1] >> 7) & 0xFF);
    else if (kind == DF_KIND_U8) last = src[n - 1];
    else last = (uint8_t)((src[(n - 1) / 2] >> (4 * ((n - 1) & 1))) & 15);
    CHECK(df_encode_layout((df_kind)kind, n, hist, last, len, &lay2) == DF_OK);
    CHECK(lay2.total_bits == inf.total_bits && lay2.n_tiles == inf.n_tiles && lay2.n_threads == inf.n_threads);
    std::vector<uint16_t> lut2(64 * 256);
    std::vector<uint64_t> dtab(DF_DTAB_BYTES_U8 / 8 + 4096);
    uint32_t nl2 = 0;
    CHECK(df_build_tables((df_kind)kind, len, lut2.data(), 64, &nl2, dtab.data()) == DF_OK);
    CHECK(nl2 == (uint32_t)nl);
    const std::vector<uint8_t> ldt = section(c, DF_SEC_DTAB);
    CHECK(std::memcmp(ldt.data(), dtab.data(), ldt.size()) == 0);
  }

  // file round trip, then damaged copies of the file
  CHECK(df_container_save(c, tmp.c_str()) == DF_OK);
  df_container *d = nullptr;
  CHECK(df_container_load(tmp.c_str(), &d) == DF_OK);
  if (d) {
    for (int s = 0; s < DF_SEC_COUNT; s++) CHECK(section(c, (df_section)s) == section(d, (df_section)s));
    df_container_free(d);
  }
  FILE *f = std::fopen(tmp.c_str(), "rb");
  std::vector<uint8_t> file;
  if (f) {
    int ch;
    while ((ch = std::fgetc(f)) != EOF) file.push_back((uint8_t)ch);
    std::fclose(f);
  }
  for (int k = 0; k < 12 && !file.empty(); k++) {
    std::vector<uint8_t> bad = file;
    if (k < 4) bad.resize(bad.size() * (size_t)k / 4);               // truncated
    else bad[(size_t)(next_u64() % bad.size())] ^= (uint8_t)(1u << (k % 8));  // one bit flipped
    FILE *g = std::fopen(tmp.c_str(), "wb");
    if (!g) break;
    std::fwrite(bad.data(), 1, bad.size(), g);
    std::fclose(g);
    df_container *e = nullptr;
    const df_status st = df_container_load(tmp.c_str(), &e);
    if (st == DF_OK) {  // a flip inside the stream or the sign|mantissa plane may load
      CHECK(e != nullptr);
      if (e) {
        CHECK(df_container_validate(e) == DF_OK);
        df_container_free(e);
      }
    }
  }
  df_container_free(c);
}

static void codebook_cases() {
  uint64_t h[256];
  uint8_t len[256];
  std::memset(h, 0, sizeof h);
  CHECK(df_build_codebook(h, 32, len) == DF_OK);  // no symbol
  h[9] = 5;
  CHECK(df_build_codebook(h, 32, len) == DF_OK && len[9] == 1);  // one symbol
  uint64_t a = 1, b = 1;  // Fibonacci counts: plain Huffman is 39 deep
  for (int s = 0; s < 40; s++) {
    h[s] = a;
    const uint64_t t = a + b;
    a = b;
    b = t;
  }
  for (uint32_t L = 6; L <= 32; L++) {
    CHECK(df_build_codebook(h, L, len) == DF_OK);
    uint8_t mx = 0;
    for (int s = 0; s < 256; s++) mx = len[s] > mx ? len[s] : mx;
    CHECK(mx <= L);
  }
  CHECK(df_build_codebook(h, 5, len) == DF_ERR_CODEBOOK);  // 40 symbols need 6 bits
  CHECK(df_build_codebook(h, 0, len) == DF_ERR_ARG);
  CHECK(df_build_codebook(h, 33, len) == DF_ERR_ARG);
  for (int s = 0; s < 256; s++) h[s] = 1 + (next_u64() % 1000000);
  CHECK(df_build_codebook(h, 8, len) == DF_OK);
  for (int s = 0; s < 256; s++) CHECK(len[s] == 8);
}

int main(int argc, char **argv) {
  const std::string tmp = argc > 1 ? argv[1] : "/tmp/dfh_sanitize.dfc";
  codebook_cases();
  const uint64_t sizes[] = {0, 1, 2, 63, 64, 65, 255, 257, 6143, 16384, 16385, 100003};
  for (int kind = 0; kind < 3; kind++)
    for (uint64_t n : sizes)
      for (int shape = 0; shape < 3; shape++) round_trip(kind, n, shape, tmp);
  std::remove(tmp.c_str());
  std::printf("sanitize driver: %s (%d failed checks)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
